// resa_sparse_step: one decode step of one attention layer - tail descriptor
// refresh, group block scores, top-n selection and block sparse attention -
// in a single persistent launch.
//
// "Rectified Sparse Attention" analysis page (paper-graph-ui): §3.4.1
// (Eq 3-5: descriptors, block scores, top-n with the local window; Eq 2:
// attention over the selected blocks), §3.4.3 Algorithm 1 (the block key
// cache is updated as tokens are appended), §3.4.4 (split attention kernel
// with a log-sum-exp merge; kernel time without CPU overhead).
//
// Work units.  The blocks of each (request, KV head) are cut into W slices;
// unit (row, w) is slice w of row = request * H + KV head.  A persistent grid
// of at most one 512-thread workgroup per compute unit takes units
// blockIdx.x, blockIdx.x + gridDim.x, ... and carries each through all of
// its phases.  Thread t of a unit stands for block sb0 + t of its slice.
//
// Phases of unit (row, w):
//  1. Score the slice (score_core.h) and keep its keys in LDS; store three
//     statistics of its candidate keys: minimum, maximum, an upper bound v_w
//     of its c-th largest key (c = ceil(k / W), k = blocks chosen by score)
//     and a lower edge l_w of it, both from a 64-bin histogram of the slice.
//  2. Once all W slices are in: T = max_w v_w and T_lo = the m-th largest
//     l_w, m = ceil(k / c).  At most c - 1 keys of a slice exceed v_w, so at
//     most W (c - 1) < k keys exceed T: they are all among the k highest.
//     The m slices with the largest l_w hold at least c keys >= l_w each, so
//     at least k keys are >= T_lo: no key below T_lo is chosen.  Only the
//     "band" [T_lo, T] needs ranking; each slice stores its band keys.
//  3. Slice W - 1 is the selector: once every slice has stored its band, it
//     finds the exact threshold (the k-th largest key, ties to the lower
//     block id) from the band alone (select_core.h) and publishes it.  The
//     other slices meanwhile attend over their blocks above T.
//  4. With the threshold, every slice attends over the rest of its selected
//     blocks; the selector's own slice is shared out among the other slices,
//     so the selector never holds the critical path up with attention.
//  5. Each unit writes one partial (m, l, o) per query head; once all W are
//     in, every unit merges its share of the row's outputs (decode_core.h)
//     and writes its selected block ids at their place in the ascending
//     list.  The last unit to finish resets the row's words for the next
//     call.
//
// Waits: a unit waits only for events every unit of its row triggers
// without waiting itself at that point (all slices scored, all bands
// stored, the threshold, all partials), the grid never holds more
// workgroups than can be resident at once, and a row's W <= gridDim.x units
// are taken in one sweep of the grid or two adjacent ones, so no wait can
// close a cycle.  Waits are bounded.
//
// Exchange between workgroups: device-scope stores, a wait for their
// completion, then an atomic or a flag store; device-scope loads after the
// atomic or flag is seen (select_core.h).
#include "decode_core.h"
#include "desc_unit.h"
#include "score_core.h"

namespace resa {
namespace {

constexpr int kStepWaves = 8;
constexpr int kStepThreads = 64 * kStepWaves;
constexpr int kStepMaxUnroll = 8;  // passes per slice
constexpr int kLineWords = 32;     // one 128-byte line
// Flag lines per row: arrivals after scoring, arrivals after the band
// stores, state words, arrivals of partials, units done.
constexpr int kCntS = 0, kCntB = 1, kState = 2, kCntM = 3, kCntDone = 4, kFlagLines = 5;
// State words: threshold published, threshold key, last block id taken at
// the threshold, a wait gave up.
constexpr int kReady = 0, kThr = 1, kCut = 2, kTimedOut = 3;
constexpr int kStatWords = 4;  // per slice: ~minimum, maximum, v_w, l_w
constexpr int kCntWords = 4;   // per slice: keys above T, band keys, selected blocks
constexpr int kBandCap = 4096;  // band keys the selector ranks in LDS
constexpr uint32_t kSpinLimit = 1u << 20;  // about a second of polling

// blocks per pass of the scoring workgroup: kStepThreads / lanes per descriptor
inline int step_bpp(int dtype, int D) {
  const int ch = 2 * D * (dtype == 0 ? 2 : 4) / 32;
  return kStepThreads / ch;
}

// Thread 0 polls `word` until it is at least `want` (bounded); every thread
// gets the outcome.  Contains a workgroup barrier.
__device__ __forceinline__ bool wait_at_least(const uint32_t* word, uint32_t want, int* s_ok) {
  if (threadIdx.x == 0) {
    bool ok = false;
    for (uint32_t it = 0; it < kSpinLimit; ++it) {
      if (load_agent(word) >= want) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    *s_ok = ok ? 1 : 0;
  }
  __syncthreads();
  return *s_ok != 0;
}

// Eq 5 count and the per-row quantities every phase needs.  (Fields are
// passed one by one: a reference to the kernel argument would make the
// compiler copy the whole argument block to scratch memory.)
struct RowInfo {
  int L, M, nl, C, n, k;
  __device__ __forceinline__ RowInfo(int seq_len, int max_blocks, int budget_num, int budget_den, int min_blocks,
                                     int local_blocks) {
    L = clampi(seq_len, 0, max_blocks * kBlock);
    M = (L + kBlock - 1) / kBlock;
    nl = local_blocks < M ? local_blocks : M;
    C = M - nl;
    n = 0;
    if (M > 0) {
      long long nn = ((long long)M * budget_num + budget_den - 1) / budget_den;
      if (nn < min_blocks) nn = min_blocks;
      if (nn < local_blocks) nn = local_blocks;
      if (nn > M) nn = M;
      n = (int)nn;
    }
    k = n - nl;
  }
};

struct StepBandLds {
  __align__(16) uint32_t key[kBandCap];  // band keys, ascending block order
  int id[kBandCap];                       // their block ids
};

template <typename T, int D>
union StepLds {
  struct {
    SelectLds<kStepThreads> sl;
    StepBandLds bl;
  } sel;
  MergeLds<kStepWaves, D> ml;
};

// Attends over list positions [0, n) split evenly over the wavefronts.
template <typename T, int D, class IdAt>
__device__ __forceinline__ void attend_list(WaveAttn<T, D>& st, IdAt id_at, int n, const typename Frag<T, D>::Q& qf,
                                            const T* k_pool, const T* v_pool, const int32_t* tab, int H, int i, int L,
                                            int max_blocks, int num_pool_blocks, float scale_log2) {
  const int wave = threadIdx.x >> 6;
  const int per = (n + kStepWaves - 1) / kStepWaves;
  const int p0 = min(n, wave * per), p1 = min(n, p0 + per);
  st.run(id_at, p0, p1, p1, qf, k_pool, v_pool, tab, H, i, L, max_blocks, num_pool_blocks, scale_log2);
}

template <typename T, int D, int MAXG, int KPT>
__global__ __launch_bounds__(kStepThreads) void step_kernel(const StepArgs a) {
  using SS = SliceScore<T, D, MAXG, kStepThreads, kStepMaxUnroll>;
  using F = Frag<T, D>;
  constexpr int NT = kStepThreads;
  constexpr int SBMAX = SS::BPP * kStepMaxUnroll;
  static_assert(SBMAX <= NT, "one slice block per thread");
  constexpr int KPB = kBandCap / NT;  // band keys per thread in the selector
  __shared__ __align__(16) float s_coef[2 * D];
  __shared__ uint2 s_mm[kStepWaves];
  __shared__ uint32_t s_thi[kStepWaves];
  __shared__ uint32_t s_hist[64];
  __shared__ WaveSlots<int, kStepWaves> s_scan;
  __shared__ int s_i[4];
  __shared__ uint32_t s_u[4];
  __shared__ __align__(16) uint32_t s_lw[NT];
  __shared__ uint32_t s_key[SBMAX];
  __shared__ int s_list[SBMAX];
  __shared__ int s_list2[SBMAX];
  __shared__ uint32_t s_okey[SBMAX];
  __shared__ int s_pre[NT];
  __shared__ StepLds<T, D> lds;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int H = a.H;
  const int W = a.nslices;
  const int U = a.unroll;
  const int SB = U * SS::BPP;
  const int units = a.R * H * W;
  const T* k_pool = static_cast<const T*>(a.k_pool);
  const T* v_pool = static_cast<const T*>(a.v_pool);

  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int row = unit / W;
    const int w = unit % W;
    const int r = row / H;
    const int i = row % H;
    const RowInfo ri(a.seq_lens[r], a.max_blocks, a.budget_num, a.budget_den, a.min_blocks, a.local_blocks);
    const int32_t* tab = a.table + (size_t)r * a.max_blocks;
    uint32_t* key_row = a.keys + (size_t)row * a.key_stride;
    uint32_t* flags = a.flags + (size_t)row * kFlagLines * kLineWords;
    uint32_t* state = flags + kState * kLineWords;
    uint32_t* stats = a.stats + (size_t)row * W * kStatWords;
    uint32_t* cnts = a.cnts + (size_t)row * W * kCntWords;
    uint32_t* band = a.band + (size_t)row * a.band_stride * 2;  // (key, block id) pairs
    const int sb0 = w * SB;
    const bool need_sel = ri.k > 0 && ri.k < ri.C;  // uniform over the row
    const bool selector = need_sel && w == W - 1;
    const bool orphan = selector && W > 1;  // the other slices attend over this slice
    int scan_use = 0;
    bool ok = true;

    // ------------------------------------------------------------ 1. scoring
    SS ss;
    ss.run(static_cast<const T*>(a.q) + (size_t)row * a.G * D, static_cast<const T*>(a.desc_pool), tab, ri.M,
           ri.C, sb0, U, H, i, a.G, a.mode, a.max_blocks, a.num_pool_blocks, key_row, nullptr, s_coef);
    // Tail refresh: the slice holding the row's last block recomputes its
    // descriptor (its own loads of that descriptor are complete; the block is
    // always selected, so its score never matters).
    if (a.refresh_tail && wave == 0 && ri.M > 0 && ri.M - 1 >= sb0 && ri.M - 1 < sb0 + SB) {
      const int p = clampi(tab[ri.M - 1], 0, a.num_pool_blocks - 1);
      descriptor_unit<T, D>(static_cast<const T*>(a.k_pool) + ((size_t)p * H + i) * kBlock * D,
                            static_cast<T*>(a.desc_pool) + ((size_t)p * H + i) * 2 * D, ri.L - (ri.M - 1) * kBlock);
    }
    const int lg = t % SS::CH;
    if (lg == 0) {
#pragma unroll
      for (int u = 0; u < kStepMaxUnroll; ++u)
        if (u < U) s_key[u * SS::BPP + t / SS::CH] = ss.key[u];
    }
    uint32_t kmin = ss.kmin, kmax = ss.kmax;
    wave_min_max(kmin, kmax);
    if (lane == 0) s_mm[wave] = make_uint2(kmin, kmax);
    if (t < 64) s_hist[t] = 0u;
    __syncthreads();
    if (need_sel) {
      uint32_t smin = 0xffffffffu, smax = 0u;
#pragma unroll
      for (int v = 0; v < kStepWaves; ++v) {
        smin = min(smin, s_mm[v].x);
        smax = max(smax, s_mm[v].y);
      }
      // v_w and l_w: the edges of the histogram bin holding the slice's c-th
      // largest candidate key
      const int cand = max(0, min(ri.C, sb0 + SB) - sb0);
      const int c = (ri.k + W - 1) / W;
      uint32_t v_w = smax, l_w = 0u;
      if (cand >= c) {  // uniform
        const uint32_t d = smax - smin;
        const int nb = d ? 32 - __clz(d) : 0;
        const int shift = nb > 6 ? nb - 6 : 0;  // at most 64 bins of width 2^shift
#pragma unroll
        for (int u = 0; u < kStepMaxUnroll; ++u)
          if (u < U && lg == 0 && ss.blk[u] < ri.C) atomicAdd(&s_hist[(ss.key[u] - smin) >> shift], 1u);
        __syncthreads();
        if (wave == 0) {
          // bins from the top: lane l holds bin 63 - l
          const int h = (int)s_hist[63 - lane];
          const int incl = wave_incl_sum(h);
          const uint64_t hit = __ballot(incl >= c);  // the slice has >= c candidates: some lane reaches c
          const int bin = 63 - __builtin_ctzll(hit);
          const uint64_t top = (uint64_t)smin + ((uint64_t)(bin + 1) << shift) - 1u;
          v_w = top < (uint64_t)smax ? (uint32_t)top : smax;
          l_w = smin + ((uint32_t)bin << shift);
        }
      }
      if (t == 0) {  // (thread 0 is in wave 0, which holds v_w and l_w)
        store_agent(stats + (size_t)w * kStatWords, ~smin);
        store_agent(stats + (size_t)w * kStatWords + 1, smax);
        store_agent(stats + (size_t)w * kStatWords + 2, v_w);
        store_agent(stats + (size_t)w * kStatWords + 3, l_w);
      }
      wait_vm_all();  // key and statistics stores complete
      __syncthreads();
      if (t == 0)
        __hip_atomic_fetch_add(flags + kCntS * kLineWords, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ------------------------------------------------------------ 2. bounds
    uint32_t thi = 0u, tlo = 0u, mn = 0u, mx = 0u;
    uint32_t okey = 0u;  // key of block t of the selector's slice
    const int bo = (W - 1) * SB + t;
    if (need_sel) {
      ok = wait_at_least(flags + kCntS * kLineWords, (uint32_t)W, &s_i[1]) && ok;
      if (!selector && t < SB && bo < ri.C) okey = load_agent(key_row + bo);
      uint32_t vmax = 0u;
      mn = 0xffffffffu;
      for (int s2 = t; s2 < W; s2 += NT) {
        mn = min(mn, ~load_agent(stats + (size_t)s2 * kStatWords));
        mx = max(mx, load_agent(stats + (size_t)s2 * kStatWords + 1));
        vmax = max(vmax, load_agent(stats + (size_t)s2 * kStatWords + 2));
      }
      const int c = (ri.k + W - 1) / W;
      const int m = (ri.k + c - 1) / c;
      s_lw[t] = t < W ? load_agent(stats + (size_t)t * kStatWords + 3) : 0u;
      wave_min_max(mn, mx);
      uint32_t dummy = 0xffffffffu;
      wave_min_max(dummy, vmax);
      if (lane == 0) {
        s_mm[wave] = make_uint2(mn, mx);
        s_thi[wave] = vmax;
      }
      if (t == 0) s_u[0] = 0u;
      __syncthreads();
      mn = 0xffffffffu;
      mx = 0u;
#pragma unroll
      for (int v = 0; v < kStepWaves; ++v) {
        mn = min(mn, s_mm[v].x);
        mx = max(mx, s_mm[v].y);
        thi = max(thi, s_thi[v]);
      }
      if (t < W) {
        // place of x in descending order, ties by slice; sixteen entries per
        // step, read as four 16-byte words (entries past W are 0 and never count)
        const uint32_t x = s_lw[t];
        int rank = 0;
        for (int s0 = 0; s0 < W; s0 += 16) {
          uint4 y4[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) y4[v] = *reinterpret_cast<const uint4*>(&s_lw[s0 + 4 * v]);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint32_t y[4] = {y4[v].x, y4[v].y, y4[v].z, y4[v].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int s2 = s0 + 4 * v + e;
              rank += (y[e] > x || (y[e] == x && s2 < t)) ? 1 : 0;
            }
          }
        }
        if (rank == m - 1) s_u[0] = x;
      }
      __syncthreads();
      tlo = s_u[0];
      thi = (uint32_t)__builtin_amdgcn_readfirstlane((int)thi);
      tlo = (uint32_t)__builtin_amdgcn_readfirstlane((int)tlo);
      mn = (uint32_t)__builtin_amdgcn_readfirstlane((int)mn);
      mx = (uint32_t)__builtin_amdgcn_readfirstlane((int)mx);
    }

    // ------------------------------------------------------------ classify the slice
    // (re-read from LDS where needed, so nothing of it stays in registers
    // through the attention loops)
    const int b = sb0 + t;
    const bool in_slice = t < SB && b < ri.M;
    const bool cand = in_slice && b < ri.C;
    // selected whatever the exact threshold: the recent blocks, every
    // candidate when all are taken, keys above T
    auto certain = [&](uint32_t key) {
      return in_slice && (b >= ri.C || ri.k >= ri.C || (need_sel && key > thi));
    };
    if (need_sel) {
      const uint32_t key = t < SB ? s_key[t] : 0u;
      const bool inband = cand && key >= tlo && key <= thi;
      int tot_a, tot_b;
      block_exclusive_scan<NT>(cand && key > thi ? 1 : 0, s_scan, scan_use, tot_a);
      const int pos = block_exclusive_scan<NT>(inband ? 1 : 0, s_scan, scan_use, tot_b);
      if (inband) {
        uint32_t* e = band + 2 * ((size_t)sb0 + pos);
        store_agent(e, key);
        store_agent(e + 1, (uint32_t)b);
      }
      if (t == 0) {
        store_agent(cnts + (size_t)w * kCntWords, (uint32_t)tot_a);
        store_agent(cnts + (size_t)w * kCntWords + 1, (uint32_t)tot_b);
      }
      wait_vm_all();  // band and count stores complete
      __syncthreads();
      if (t == 0)
        __hip_atomic_fetch_add(flags + kCntB * kLineWords, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ------------------------------------------------------------ 3. the selector
    uint32_t thr = 0u;
    int cut = 0x7fffffff;
    if (selector) {
      ok = wait_at_least(flags + kCntB * kLineWords, (uint32_t)W, &s_i[1]) && ok;
      const int na = t < W ? (int)load_agent(cnts + (size_t)t * kCntWords) : 0;
      const int nbs = t < W ? (int)load_agent(cnts + (size_t)t * kCntWords + 1) : 0;
      int NA, NB;
      block_exclusive_scan<NT>(na, s_scan, scan_use, NA);
      const int pre = block_exclusive_scan<NT>(nbs, s_scan, scan_use, NB);
      if (t < W) s_pre[t] = pre;
      const int k2 = ri.k - NA;  // keys to take from the band
      SelectLds<NT>& sl = lds.sel.sl;
      for (int q = t; q <= kBins; q += NT) {
        sl.hist2[0][q] = 0u;
        sl.hist2[1][q] = 0u;
      }
      if (t == 0) sl.packed = 0;
      __syncthreads();
      int sel_use = 0;
      if (tlo > 0u && NB <= kBandCap && k2 >= 1 && k2 <= NB) {  // uniform
        // the band in ascending block order: slice by slice
        // (all loads of a thread issued before any is used)
        uint32_t gk[KPB], gi[KPB];
#pragma unroll
        for (int j = 0; j < KPB; ++j) {
          const int e = t + j * NT;
          gk[j] = 0u;
          gi[j] = 0u;
          if (e < NB) {
            int lo = 0, hi = W - 1;  // the last slice whose band starts at or before e
            while (lo < hi) {
              const int mid = (lo + hi + 1) >> 1;
              if (s_pre[mid] <= e) lo = mid;
              else hi = mid - 1;
            }
            const uint32_t* src = band + 2 * ((size_t)lo * SB + (e - s_pre[lo]));
            gk[j] = load_agent(src);
            gi[j] = load_agent(src + 1);
          }
        }
#pragma unroll
        for (int j = 0; j < KPB; ++j) {
          const int e = t + j * NT;
          if (e < NB) {
            lds.sel.bl.key[e] = gk[j];
            lds.sel.bl.id[e] = (int)gi[j];
          }
        }
        __syncthreads();
        KeyRuns<NT, KPB> kb;
        kb.load_lds(lds.sel.bl.key);
        kb.set_count(NB);
        const Threshold th = select_threshold<NT, KPB>(sl, kb, NB, k2, tlo, thi, sel_use);
        thr = th.thr;
        if (th.take_eq < th.n_eq) cut = lds.sel.bl.id[cut_position<NT, KPB>(sl, kb, thr, th.take_eq, sel_use)];
      } else {
        // no usable band: every candidate of the row
        KeyRuns<NT, KPT> kr;
        kr.template prefetch<true>(key_row, a.key_stride);
        kr.set_count(ri.C);
        const Threshold th = select_threshold<NT, KPT>(sl, kr, ri.C, ri.k, mn, mx, sel_use);
        thr = th.thr;
        if (th.take_eq < th.n_eq) cut = cut_position<NT, KPT>(sl, kr, thr, th.take_eq, sel_use);
      }
      thr = (uint32_t)__builtin_amdgcn_readfirstlane((int)thr);
      cut = __builtin_amdgcn_readfirstlane(cut);
      if (t == 0) {
        store_agent(state + kThr, thr);
        store_agent(state + kCut, (uint32_t)cut);
        wait_vm_all();
        store_agent(state + kReady, 1u);
      }
    }

    // ------------------------------------------------------------ 4. attention
    typename F::Q qf;
    F::load_q(qf, static_cast<const T*>(a.q) + (size_t)row * a.G * D, lane & 15, lane >> 4, a.G);
    WaveAttn<T, D> st;
    st.init();
    if (!orphan) {  // the blocks above T while the selector works
      const bool cert = certain(t < SB ? s_key[t] : 0u);
      int n1;
      const int pos = block_exclusive_scan<NT>(cert ? 1 : 0, s_scan, scan_use, n1);
      if (cert) s_list[pos] = b;
      __syncthreads();
      attend_list<T, D>(st, [&](int p) { return s_list[p]; }, n1, qf, k_pool, v_pool, tab, H, i, ri.L,
                        a.max_blocks, a.num_pool_blocks, a.scale_log2);
    }
    if (need_sel && !selector && t < SB) s_okey[t] = okey;  // long since loaded
    // selected, not certain (needs the threshold)
    auto rest_of = [&](uint32_t key) {
      return need_sel && cand && !certain(key) && (key > thr || (key == thr && b <= cut));
    };
    if (need_sel) {
      if (!selector) {
        ok = wait_at_least(state + kReady, 1u, &s_i[2]) && ok;
        thr = (uint32_t)__builtin_amdgcn_readfirstlane((int)load_agent(state + kThr));
        cut = __builtin_amdgcn_readfirstlane((int)load_agent(state + kCut));
      }
      const bool rest = rest_of(t < SB ? s_key[t] : 0u);
      int n2 = 0, q0 = 0, q1 = 0;
      if (!orphan) {
        const int pos = block_exclusive_scan<NT>(rest ? 1 : 0, s_scan, scan_use, n2);
        if (rest) s_list[pos] = b;
      }
      if (!selector && W > 1) {
        // this slice's share of the selector's slice
        const bool oin = t < SB && bo < ri.M;
        const uint32_t ok2 = t < SB ? s_okey[t] : 0u;
        const bool osel = oin && (bo >= ri.C || ok2 > thr || (ok2 == thr && bo <= cut));
        int no;
        const int pos = block_exclusive_scan<NT>(osel ? 1 : 0, s_scan, scan_use, no);
        if (osel) s_list2[pos] = bo;
        q0 = (int)((long long)w * no / (W - 1));
        q1 = (int)((long long)(w + 1) * no / (W - 1));
      }
      __syncthreads();
      attend_list<T, D>(st, [&](int p) { return p < n2 ? s_list[p] : s_list2[q0 + p - n2]; }, n2 + q1 - q0, qf,
                        k_pool, v_pool, tab, H, i, ri.L, a.max_blocks, a.num_pool_blocks, a.scale_log2);
    }

    // this unit's partial and its count of selected blocks, then count in
    const size_t prow = (size_t)row * W + w;
    wg_merge_store<T, D, kStepWaves, true>(st, lds.ml, a.G, a.part_o + prow * a.G * D, a.part_ml + prow * a.G * 2);
    const uint32_t key = t < SB ? s_key[t] : 0u;
    const bool mine = certain(key) || rest_of(key);
    int nsel;
    const int spos = block_exclusive_scan<NT>(mine ? 1 : 0, s_scan, scan_use, nsel);
    if (t == 0) store_agent(cnts + (size_t)w * kCntWords + 2, (uint32_t)nsel);
    wait_vm_all();
    __syncthreads();
    if (t == 0)
      __hip_atomic_fetch_add(flags + kCntM * kLineWords, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // ------------------------------------------------------------ 5. merge and output
    // Once all W partials of the row are in, unit w merges its share of the
    // row's output float4s (sixteen lanes per float4, each lane reading every
    // sixteenth partial).
    ok = wait_at_least(flags + kCntM * kLineWords, (uint32_t)W, &s_i[1]) && ok;
    {
      const AgentPartials pp(a.part_o + (size_t)row * W * a.G * D, a.part_ml + (size_t)row * W * a.G * 2,
                             (uint32_t)((size_t)W * a.G * D * 4), (uint32_t)((size_t)W * a.G * 2 * 4));
      constexpr int C4 = D / 4;
      const int nout = a.G * C4;  // output float4s of the row
      const int o0 = (int)((long long)w * nout / W), o1 = (int)((long long)(w + 1) * nout / W);
      for (int g = o0 * kMergeParts + t; g < o1 * kMergeParts; g += NT) {  // uniform per DPP row
        const int part = g % kMergeParts;
        const int o = g / kMergeParts;
        const int c4 = o % C4;
        const int j = o / C4;
        const floatx4_t v = merge_float4<D>(pp, 0, W, a.G, j, c4, part);
        if (part == 0) *reinterpret_cast<floatx4_t*>(a.out + ((size_t)row * a.G + j) * D + 4 * c4) = v;
      }
    }
    // the slice's selected ids at their place in the ascending list
    {
      int off;
      block_exclusive_scan<NT>(t < w ? (int)load_agent(cnts + (size_t)t * kCntWords + 2) : 0, s_scan, scan_use,
                               off);
      int32_t* out = a.sel_idx + (size_t)row * a.max_sel;
      if (mine && off + spos < a.max_sel) out[off + spos] = b;
      if (w == W - 1)
        for (int j = ri.n + t; j < a.max_sel; j += NT) out[j] = -1;
      if (w == 0 && t == 0) a.sel_cnt[row] = ri.n;
    }
    __syncthreads();
    if (t == 0) {
      if (!ok) store_agent(state + kTimedOut, 1u);
      const uint32_t old = __hip_atomic_fetch_add(flags + kCntDone * kLineWords, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      if (old == (uint32_t)(W - 1)) {
        // every unit of the row is past all of its waits: reset for the next call
        store_agent(flags + kCntS * kLineWords, 0u);
        store_agent(flags + kCntB * kLineWords, 0u);
        store_agent(state + kReady, 0u);
        store_agent(state + kThr, 0u);
        store_agent(state + kCut, 0u);
        store_agent(flags + kCntM * kLineWords, 0u);
        store_agent(flags + kCntDone * kLineWords, 0u);
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const StepArgs& a, hipStream_t stream) {
  const int cand_max = a.key_stride;
  dim3 grid((unsigned)a.grid);
#define RESA_STEP_LAUNCH(MAXG, KPT) \
  hipLaunchKernelGGL((step_kernel<T, D, MAXG, KPT>), grid, dim3(kStepThreads), 0, stream, a)
#define RESA_STEP_KPT(MAXG)                                             \
  do {                                                                  \
    if (cand_max <= 8 * kStepThreads) RESA_STEP_LAUNCH(MAXG, 8);        \
    else if (cand_max <= 16 * kStepThreads) RESA_STEP_LAUNCH(MAXG, 16); \
    else if (cand_max <= 32 * kStepThreads) RESA_STEP_LAUNCH(MAXG, 32); \
    else RESA_STEP_LAUNCH(MAXG, 0);                                     \
  } while (0)
  if (a.G <= 8) RESA_STEP_KPT(8);
  else RESA_STEP_KPT(16);
#undef RESA_STEP_KPT
#undef RESA_STEP_LAUNCH
  return hipGetLastError();
}

}  // namespace

void step_geometry(int dtype, int D, int R, int H, int max_blocks, int* unroll, int* nslices) {
  const int bpp = step_bpp(dtype, D);
  const long long rows = (long long)R * H;
  int U = kStepMaxUnroll;
  while (U > 1 && rows * ((max_blocks + bpp * U - 1) / (bpp * U)) < 256) U /= 2;
  *unroll = U;
  *nslices = (max_blocks + bpp * U - 1) / (bpp * U);
}

void step_workspace_parts(int dtype, int D, int R, int H, int G, int max_blocks, int max_sel,
                          size_t parts[kStepParts]) {
  (void)max_sel;
  int U, W;
  step_geometry(dtype, D, R, H, max_blocks, &U, &W);
  const size_t rows = (size_t)R * H;
  parts[0] = rows * kFlagLines * kLineWords * sizeof(uint32_t);
  parts[1] = rows * W * kStatWords * sizeof(uint32_t);
  parts[2] = rows * W * kCntWords * sizeof(uint32_t);
  parts[3] = rows * key_stride_for(max_blocks) * sizeof(uint32_t);
  parts[4] = rows * step_band_stride(dtype, D, R, H, max_blocks) * 2 * sizeof(uint32_t);
  parts[5] = rows * W * G * D * sizeof(float);
  parts[6] = rows * W * G * 2 * sizeof(float);
}

int step_band_stride(int dtype, int D, int R, int H, int max_blocks) {
  int U, W;
  step_geometry(dtype, D, R, H, max_blocks, &U, &W);
  return W * U * step_bpp(dtype, D);
}

hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
  if (a.dtype == 0) return a.D == 128 ? launch_t<bf16_t, 128>(a, stream) : launch_t<bf16_t, 64>(a, stream);
  return a.D == 128 ? launch_t<float, 128>(a, stream) : launch_t<float, 64>(a, stream);
}

}  // namespace resa
