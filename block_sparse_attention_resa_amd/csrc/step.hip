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
// blockIdx.x, blockIdx.x + gridDim.x, ..., first all of its scoring phases,
// then all of its attention phases, then all of its merge phases.  No
// workgroup waits during scoring, so every row's scores complete; later waits
// are for events that workgroups already running trigger, and a workgroup
// waits in a phase only after finishing the earlier phases of all of its
// units, so the grid (never more workgroups than can be resident at once)
// cannot deadlock.  Waits are bounded.
//
// Scoring phase of unit (row, w).  Score the slice (score_core.h), store the
// keys, and store three statistics of the slice's candidate keys: minimum,
// maximum, and an upper bound v_w of its c-th largest key, c = ceil(k / W)
// (k = blocks chosen by score), from a 64-bin histogram of the slice.  Then
// count in with one atomic add.  The last arrival of a row computes
// T = max_w v_w and publishes it, then runs the exact selection
// (select_core.h), writes sel_idx / sel_cnt and the list of selected blocks
// whose key is at most T, and publishes that list.
//
// Why T helps.  At most c - 1 keys of a slice exceed v_w, so at most
// W (c - 1) < k keys exceed T: every block whose key exceeds T is among the
// k highest, whatever the exact threshold.  Such blocks (and the forced
// local blocks) are "certain" as soon as T is known.
//
// Attention phase of unit (row, w) (units claimed in order from a counter).
// Wait for T; attend over the certain
// blocks of slice w (about half of the selection on the measured workloads)
// while the exact selection is still running; wait for the selection; attend
// over chunk w of the remaining selected blocks; write one partial (m, l, o)
// per query head and count in.
//
// Merge phase of unit (row, w).  Wait until all W partials of the row are in,
// then merge (decode_core.h) unit w's share of the row's outputs, so the
// merge is spread over the row's workgroups; the last unit to finish resets
// the row's counters and state words to zero for the next call.
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
// Flag lines per row: arrival counter of the scoring phase, state words,
// arrival counter of the attention phase, count of merged shares.
constexpr int kCntS = 0, kState = 1, kCntM = 2, kCntDone = 3, kFlagLines = 4;
// State words: T published, T, selection published, length of the
// remaining-blocks list, attention phase waited in vain.
constexpr int kArrived = 0, kThi = 1, kReady = 2, kNunc = 3, kTimedOut = 4;
constexpr int kStatWords = 4;  // per slice: ~minimum, maximum, v_w, l_w
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

template <typename T, int D>
union StepLds {
  struct {
    SelectLds<kStepThreads> sl;
    BandLds bl;
  } sel;
  MergeLds<kStepWaves, D> ml;
};

template <typename T, int D, int MAXG, int KPT>
__global__ __launch_bounds__(kStepThreads) void step_kernel(const StepArgs a) {
  using SS = SliceScore<T, D, MAXG, kStepThreads, kStepMaxUnroll>;
  using F = Frag<T, D>;
  constexpr int SBMAX = SS::BPP * kStepMaxUnroll;
  __shared__ __align__(16) float s_coef[2 * D];
  __shared__ uint2 s_mm[kStepWaves];
  __shared__ uint32_t s_hist[64];
  __shared__ int s_cnt[kStepWaves];
  __shared__ int s_list[SBMAX];
  __shared__ int s_i[4];
  __shared__ uint32_t s_u[4];
  __shared__ uint32_t s_lw[kStepThreads];
  __shared__ StepLds<T, D> lds;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int H = a.H;
  const int W = a.nslices;
  const int U = a.unroll;
  const int SB = U * SS::BPP;
  const int units = a.R * H * W;

  // ------------------------------------------------------------ scoring
  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int row = unit / W;
    const int w = unit % W;
    const int r = row / H;
    const int i = row % H;
    const RowInfo ri(a.seq_lens[r], a.max_blocks, a.budget_num, a.budget_den, a.min_blocks, a.local_blocks);
    const int32_t* tab = a.table + (size_t)r * a.max_blocks;
    uint32_t* key_row = a.keys + (size_t)row * a.key_stride;
    uint32_t* flags = a.flags + (1 + (size_t)row * kFlagLines) * kLineWords;
    uint32_t* stats = a.stats + (size_t)row * W * kStatWords;
    const int sb0 = w * SB;
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
    // slice key range
    uint32_t kmin = ss.kmin, kmax = ss.kmax;
    wave_min_max(kmin, kmax);
    if (lane == 0) s_mm[wave] = make_uint2(kmin, kmax);
    if (t < 64) s_hist[t] = 0u;
    __syncthreads();
    uint32_t smin = 0xffffffffu, smax = 0u;
#pragma unroll
    for (int v = 0; v < kStepWaves; ++v) {
      smin = min(smin, s_mm[v].x);
      smax = max(smax, s_mm[v].y);
    }
    // v_w: an upper bound of the slice's c-th largest candidate key
    const int cand = max(0, min(ri.C, sb0 + SB) - sb0);
    const int c = ri.k > 0 ? (ri.k + W - 1) / W : 1;
    const bool hist_needed = ri.k > 0 && ri.k < ri.C && cand >= c;  // uniform
    uint32_t v_w = 0u, l_w = 0u;
    if (hist_needed) {
      const uint32_t d = smax - smin;
      const int nb = d ? 32 - __clz(d) : 0;
      const int shift = nb > 6 ? nb - 6 : 0;  // at most 64 bins of width 2^shift
      const int lg = t % SS::CH;
#pragma unroll
      for (int u = 0; u < kStepMaxUnroll; ++u)
        if (u < U && lg == 0 && ss.blk[u] < ri.C) atomicAdd(&s_hist[(ss.key[u] - smin) >> shift], 1u);
      __syncthreads();
      if (wave == 0) {
        // bins from the top: lane l holds bin 63 - l
        const int h = (int)s_hist[63 - lane];
        const int incl = wave_incl_sum(h);
        const uint64_t hit = __ballot(incl >= c);  // some lane reaches c: the slice has >= c candidates
        if (hit == 0u) {
          v_w = smax;
        } else {
          // the c-th largest key lies in `bin`: its upper edge bounds it from
          // above, its lower edge from below
          const int bin = 63 - __builtin_ctzll(hit);
          const uint64_t top = (uint64_t)smin + ((uint64_t)(bin + 1) << shift) - 1u;
          v_w = top < (uint64_t)smax ? (uint32_t)top : smax;
          l_w = smin + ((uint32_t)bin << shift);
        }
      }
    }
    wait_vm_all();  // key stores complete
    __syncthreads();
    if (t == 0) {
      store_agent(stats + (size_t)w * kStatWords, ~smin);
      store_agent(stats + (size_t)w * kStatWords + 1, smax);
      store_agent(stats + (size_t)w * kStatWords + 2, v_w);
      store_agent(stats + (size_t)w * kStatWords + 3, l_w);
      wait_vm_all();
      const uint32_t old = __hip_atomic_fetch_add(flags + kCntS * kLineWords, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      const bool last = old == (uint32_t)(W - 1);
      if (last) store_agent(flags + kCntS * kLineWords, 0u);  // every slice of the row is in: reset
      s_i[0] = last ? 1 : 0;
    }
    __syncthreads();
    if (s_i[0] == 0) continue;

    // ---- last slice of the row: T, then the exact selection
    uint32_t mn = 0xffffffffu, mx = 0u, thi = 0u;
    for (int s2 = t; s2 < W; s2 += kStepThreads) {
      mn = min(mn, ~load_agent(stats + (size_t)s2 * kStatWords));
      mx = max(mx, load_agent(stats + (size_t)s2 * kStatWords + 1));
      thi = max(thi, load_agent(stats + (size_t)s2 * kStatWords + 2));
    }
    wave_min_max(mn, mx);
    uint32_t dummy = 0xffffffffu;
    wave_min_max(dummy, thi);
    if (lane == 0) {
      s_mm[wave] = make_uint2(mn, mx);
      s_hist[wave] = thi;
    }
    __syncthreads();
    mn = 0xffffffffu;
    mx = 0u;
    thi = 0u;
#pragma unroll
    for (int v = 0; v < kStepWaves; ++v) {
      mn = min(mn, s_mm[v].x);
      mx = max(mx, s_mm[v].y);
      thi = max(thi, s_hist[v]);
    }
    // T_lo: the m-th largest l_w, m = ceil(k / c).  The m slices with the
    // largest l_w hold at least c keys >= l_w each, so at least m c >= k keys
    // are >= T_lo and the threshold is >= T_lo.  (0, no bound, for rows with
    // more slices than threads.)
    uint32_t tlo = 0u;
    if (ri.k > 0 && ri.k < ri.C && W <= kStepThreads) {
      const int m = (ri.k + c - 1) / c;
      if (t < W) s_lw[t] = load_agent(stats + (size_t)t * kStatWords + 3);
      if (t == 0) s_u[0] = 0u;
      __syncthreads();
      if (t < W) {
        const uint32_t x = s_lw[t];
        int rank = 0;
        for (int s2 = 0; s2 < W; ++s2) {
          const uint32_t y = s_lw[s2];
          rank += (y > x || (y == x && s2 < t)) ? 1 : 0;
        }
        if (rank == m - 1) s_u[0] = x;
      }
      __syncthreads();
      tlo = s_u[0];
    }
    uint32_t* state = flags + kState * kLineWords;
    if (t == 0) {
      store_agent(state + kThi, thi);
      wait_vm_all();
      store_agent(state + kArrived, 1u);
    }
    int32_t* out = a.sel_idx + (size_t)row * a.max_sel;
    for (int j = t; j < a.max_sel; j += kStepThreads) {
      if (j >= ri.n) out[j] = -1;
      else if (j >= ri.k) out[j] = ri.C + (j - ri.k);  // forced recent blocks close the ascending list
    }
    if (t == 0) a.sel_cnt[row] = ri.n;
    int n_unc = 0;
    if (ri.k == ri.C) {
      for (int j = t; j < ri.C; j += kStepThreads) out[j] = j;
    } else if (ri.k > 0) {
      KeyRuns<kStepThreads, KPT> kr;
      kr.prefetch(key_row, a.key_stride);
      kr.set_count(ri.C);
      auto clear = [&]() {
        for (int b = t; b <= kBins; b += kStepThreads) {
          lds.sel.sl.hist2[0][b] = 0u;
          lds.sel.sl.hist2[1][b] = 0u;
        }
        if (t == 0) lds.sel.sl.packed = 0;
      };
      clear();
      n_unc = -1;
      if constexpr (KPT > 0) {
        // only the keys in [T_lo, T] need ranking (the rest when the band is too wide)
        if (tlo > 0u) n_unc = select_band<kStepThreads, KPT>(lds.sel.sl, lds.sel.bl, kr, ri.k, tlo, thi, out,
                                                              a.unc + (size_t)row * a.max_sel);
      }
      if (n_unc < 0) {
        __syncthreads();
        clear();
        __syncthreads();
        n_unc = select_top<kStepThreads, KPT>(lds.sel.sl, kr, ri.C, ri.k, mn, mx, out, thi,
                                               a.unc + (size_t)row * a.max_sel);
      }
    }
    wait_vm_all();  // the list of remaining blocks is complete
    __syncthreads();
    if (t == 0) {
      store_agent(state + kNunc, (uint32_t)n_unc);
      wait_vm_all();
      store_agent(state + kReady, 1u);
    }
  }

  // ------------------------------------------------------------ attention
  // Units are claimed in order from a counter, so a workgroup busy with a
  // selection takes fewer of them.
  uint32_t* const gline = a.flags;  // [0] units claimed, [1] workgroups finished
  for (;;) {
    if (t == 0) s_i[0] = (int)__hip_atomic_fetch_add(gline, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int unit = s_i[0];
    if (unit >= units) break;
    const int row = unit / W;
    const int w = unit % W;
    const int r = row / H;
    const int i = row % H;
    const RowInfo ri(a.seq_lens[r], a.max_blocks, a.budget_num, a.budget_den, a.min_blocks, a.local_blocks);
    const int32_t* tab = a.table + (size_t)r * a.max_blocks;
    const uint32_t* key_row = a.keys + (size_t)row * a.key_stride;
    uint32_t* flags = a.flags + (1 + (size_t)row * kFlagLines) * kLineWords;
    uint32_t* state = flags + kState * kLineWords;
    const int sb0 = w * SB;
    const T* k_pool = static_cast<const T*>(a.k_pool);
    const T* v_pool = static_cast<const T*>(a.v_pool);

    typename F::Q qf;
    F::load_q(qf, static_cast<const T*>(a.q) + (size_t)row * a.G * D, lane & 15, lane >> 4, a.G);
    WaveAttn<T, D> st;
    st.init();

    // certain blocks of this slice, once T is known
    const bool ok1 = wait_at_least(state + kArrived, 1u, &s_i[1]);
    const uint32_t thi = load_agent(state + kThi);
    bool cert = false;
    const int b = sb0 + t;
    if (t < SB && b < ri.M) {
      if (b >= ri.C || ri.k == ri.C) cert = true;
      else if (ri.k > 0) cert = load_agent(key_row + b) > thi;
    }
    const uint64_t bal = __ballot(cert);
    if (lane == 0) s_cnt[wave] = __popcll(bal);
    __syncthreads();
    int before = 0, n1 = 0;
#pragma unroll
    for (int v = 0; v < kStepWaves; ++v) {
      before += v < wave ? s_cnt[v] : 0;
      n1 += s_cnt[v];
    }
    if (cert) s_list[before + __popcll(bal & ((1ull << lane) - 1ull))] = b;
    __syncthreads();
    {
      const int per = (n1 + kStepWaves - 1) / kStepWaves;
      const int p0 = min(n1, wave * per), p1 = min(n1, p0 + per);
      st.run([&](int p) { return s_list[p]; }, p0, p1, p1, qf, k_pool, v_pool, tab, H, i, ri.L, a.max_blocks,
             a.num_pool_blocks, a.scale_log2);
    }

    // the rest of the selection, once it is known: chunk w of the list
    const bool ok2 = wait_at_least(state + kReady, 1u, &s_i[2]);
    const int n_unc = clampi((int)load_agent(state + kNunc), 0, a.max_sel);
    {
      const int q0 = (int)((long long)w * n_unc / W), q1 = (int)((long long)(w + 1) * n_unc / W);
      const int per = (q1 - q0 + kStepWaves - 1) / kStepWaves;
      const int p0 = min(q1, q0 + wave * per), p1 = min(q1, p0 + per);
      const uint32_t* unc_row = a.unc + (size_t)row * a.max_sel;
      st.run([&](int p) { return (int)load_agent(unc_row + p); }, p0, p1, p1, qf, k_pool, v_pool, tab, H, i, ri.L,
             a.max_blocks, a.num_pool_blocks, a.scale_log2);
    }
    if (t == 0 && !(ok1 && ok2)) store_agent(state + kTimedOut, 1u);

    // this unit's partial, then count in
    const size_t prow = (size_t)row * W + w;
    wg_merge_store<T, D, kStepWaves, true>(st, lds.ml, a.G, a.part_o + prow * a.G * D, a.part_ml + prow * a.G * 2);
    wait_vm_all();
    __syncthreads();
    if (t == 0)
      __hip_atomic_fetch_add(flags + kCntM * kLineWords, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ------------------------------------------------------------ merge
  // Once all W partials of a row are in, unit w merges its share of the
  // row's output float4s (sixteen lanes per float4, each lane reading every
  // sixteenth partial), so the merge is spread over the row's workgroups.
  // These waits come after this workgroup's own arrivals, so no workgroup
  // waits for itself.
  for (int unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int row = unit / W;
    const int w = unit % W;
    uint32_t* flags = a.flags + (1 + (size_t)row * kFlagLines) * kLineWords;
    uint32_t* state = flags + kState * kLineWords;
    const bool ok3 = wait_at_least(flags + kCntM * kLineWords, (uint32_t)W, &s_i[1]);
    const AgentPartials pp(a.part_o + (size_t)row * W * a.G * D, a.part_ml + (size_t)row * W * a.G * 2,
                           (uint32_t)((size_t)W * a.G * D * 4), (uint32_t)((size_t)W * a.G * 2 * 4));
    constexpr int C4 = D / 4;
    const int nout = a.G * C4;  // output float4s of the row
    const int o0 = (int)((long long)w * nout / W), o1 = (int)((long long)(w + 1) * nout / W);
    for (int g = o0 * kMergeParts + t; g < o1 * kMergeParts; g += kStepThreads) {  // uniform per DPP row
      const int part = g % kMergeParts;
      const int o = g / kMergeParts;
      const int c4 = o % C4;
      const int j = o / C4;
      const floatx4_t v = merge_float4<D>(pp, 0, W, a.G, j, c4, part);
      if (part == 0) *reinterpret_cast<floatx4_t*>(a.out + ((size_t)row * a.G + j) * D + 4 * c4) = v;
    }
    __syncthreads();
    if (t == 0) {
      if (!ok3) store_agent(state + kTimedOut, 1u);
      const uint32_t old = __hip_atomic_fetch_add(flags + kCntDone * kLineWords, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      if (old == (uint32_t)(W - 1)) {
        // every unit of the row is past all of its waits: reset for the next call
        store_agent(state + kArrived, 0u);
        store_agent(state + kThi, 0u);
        store_agent(state + kReady, 0u);
        store_agent(state + kNunc, 0u);
        store_agent(flags + kCntM * kLineWords, 0u);
        store_agent(flags + kCntDone * kLineWords, 0u);
      }
    }
  }
  // the last workgroup to finish (every claim is made by then) resets the claim counter
  if (t == 0) {
    const uint32_t old = __hip_atomic_fetch_add(gline + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == gridDim.x - 1) {
      store_agent(gline, 0u);
      store_agent(gline + 1, 0u);
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const StepArgs& a, hipStream_t stream) {
  const int cand_max = a.key_stride;
  dim3 grid((unsigned)a.grid);
#define RESA_STEP_LAUNCH(MAXG, KPT) \
  hipLaunchKernelGGL((step_kernel<T, D, MAXG, KPT>), grid, dim3(kStepThreads), 0, stream, a)
#define RESA_STEP_KPT(MAXG)                                         \
  do {                                                              \
    if (cand_max <= 8 * kStepThreads) RESA_STEP_LAUNCH(MAXG, 8);        \
    else if (cand_max <= 16 * kStepThreads) RESA_STEP_LAUNCH(MAXG, 16); \
    else if (cand_max <= 32 * kStepThreads) RESA_STEP_LAUNCH(MAXG, 32); \
    else RESA_STEP_LAUNCH(MAXG, 0);                                 \
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

void step_workspace_parts(int dtype, int D, int R, int H, int G, int max_blocks, int max_sel, size_t parts[6]) {
  int U, W;
  step_geometry(dtype, D, R, H, max_blocks, &U, &W);
  const size_t rows = (size_t)R * H;
  parts[0] = (1 + rows * kFlagLines) * kLineWords * sizeof(uint32_t);
  parts[1] = rows * W * kStatWords * sizeof(uint32_t);
  parts[2] = rows * key_stride_for(max_blocks) * sizeof(uint32_t);
  parts[3] = rows * max_sel * sizeof(uint32_t);
  parts[4] = rows * W * G * D * sizeof(float);
  parts[5] = rows * W * G * 2 * sizeof(float);
}

hipError_t launch_step(const StepArgs& a, hipStream_t stream) {
  if (a.dtype == 0) return a.D == 128 ? launch_t<bf16_t, 128>(a, stream) : launch_t<bf16_t, 64>(a, stream);
  return a.D == 128 ? launch_t<float, 128>(a, stream) : launch_t<float, 64>(a, stream);
}

}  // namespace resa
