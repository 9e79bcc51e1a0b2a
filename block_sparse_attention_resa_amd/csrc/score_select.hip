// resa_score_select: group block scores (Eq 4) and top-n block selection
// (Eq 5 with the forced local window) of the "Rectified Sparse Attention"
// analysis page (paper-graph-ui), §3.4.1, in two launches.
//
// Scoring.  A workgroup scores a run of consecutive blocks for a group of KV
// heads of one request: thread -> (block, head, 32-byte descriptor chunk) is
// fixed, so one table entry per block serves all heads of the group and the
// heads' descriptors of a block, adjacent in the pool, are read together.
// Each thread folds its share of the group's queries into the coefficients
// (N, P) (score_core.h) once, then streams its descriptor chunks with one
// fused multiply-add per stored value; CH lanes combine a descriptor with
// DPP row rotations.  Scores are written as order-preserving 32-bit keys.
// One extra workgroup per request refreshes the tail block's descriptor of
// every KV head when asked (the block the newest token was appended to; it
// is always selected, so the score read for it concurrently never matters).
//
// Selection.  One 1024-thread workgroup per (request, KV head) runs the
// histogram select of select_core.h over that row's keys (sixteen
// wavefronts: the selection is latency-bound on one CU, and more resident
// wavefronts hide more of it than fewer, longer ones).  A second launch
// rather than a last-arriving scoring workgroup: keeping the selection's
// registers and LDS out of the scoring workgroups lets several of them share
// a CU, and the fused form measured slower on every workload.
#include "desc_unit.h"
#include "score_core.h"
#include "select_core.h"

namespace resa {
namespace {

constexpr int kScoreFill = 256;     // scoring workgroups that keep the 256 CUs busy
constexpr long long kScoreFill8 = 640;  // scoring workgroups at eight passes from which eight are used
constexpr int kScoreThreads = 256;  // threads of a scoring workgroup, at most
constexpr int kSelectThreads = 1024;
constexpr int kSelectSmall = 512;  // threads of the selection of rows of up to 4096 keys

// U: blocks per thread (passes), 4, or 2 or 1 for grids too small to give
// every CU a workgroup at 4, or 8 for grids large at 8 too.
template <typename T, int D, int MODE, int MAXG, int U>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    const T* __restrict__ q, const T* desc, const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens,
    uint32_t* __restrict__ keys, float* __restrict__ scores, int H, int HW, int G, int max_blocks,
    int num_pool_blocks, const T* __restrict__ k_pool, T* desc_tail, int score_wgs, int key_stride) {
  using CL = ChunkLoad<T>;
  constexpr int VPL = CL::kVals;
  constexpr int CH = 2 * D / VPL;  // lanes per descriptor
  constexpr int HALF = CH / 2;     // lanes per descriptor row
  extern __shared__ float s_coef[];  // [HW][2][D]: N (min row) then P (max row)

  const int r = blockIdx.y;
  const int h0 = blockIdx.z * HW;  // this workgroup's KV heads: [h0, h0 + HW)
  const int t = threadIdx.x;
  if ((int)blockIdx.x >= score_wgs) {
    // tail refresh of the group's heads, one wavefront per head
    const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
    const int M = (L + kBlock - 1) / kBlock;
    if (M == 0) return;
    const int p = clampi(table[(size_t)r * max_blocks + M - 1], 0, num_pool_blocks - 1);
    for (int i = h0 + (t >> 6); i < min(H, h0 + HW); i += (int)(blockDim.x >> 6))
      descriptor_unit<T, D>(k_pool + ((size_t)p * H + i) * kBlock * D, desc_tail + ((size_t)p * H + i) * 2 * D,
                            L - (M - 1) * kBlock);
    return;
  }
  const int lane = t & 63;
  const int grp = t / CH;
  const int lg = t % CH;
  const int part = lg / HALF;  // 0: min row, 1: max row
  const int c0 = (lg % HALF) * VPL;
  const int hl = grp % HW;  // head within the group
  const int head = h0 + hl;
  const bool head_ok = head < H;
  const int bsub = grp / HW;
  const int bpi = blockDim.x / (CH * HW);  // blocks per pass
  const int wg_blocks = bpi * U;
  const int wg_b0 = blockIdx.x * wg_blocks;
  uint32_t* key_row = keys + ((size_t)r * H + (head_ok ? head : 0)) * key_stride;
  float* score_row = scores ? scores + ((size_t)r * H + (head_ok ? head : 0)) * max_blocks : nullptr;

  // The request length (a scalar load) and the physical ids of this
  // workgroup's blocks (one coalesced load per wavefront, handed to the lanes
  // with a shuffle) are in flight together; the descriptor loads need both,
  // so skipping blocks past the sequence end costs no extra wait and no
  // descriptor past it is read (in a ragged batch the table is sized for the
  // longest request).  Load order matters: the in-order vector-memory
  // counter makes a wait for a load also wait for every load issued before
  // it, so the table entries go out first, then the queries, then the
  // descriptors.
  const int seq_len = seq_lens[r];
  int my_pid = 0;
  if (lane < wg_blocks && wg_b0 + lane < max_blocks) my_pid = table[(size_t)r * max_blocks + wg_b0 + lane];
  // Every thread folds channel pairs of the group's queries into (N, P); all
  // G rows are loaded before any is used (rows past G re-read row G - 1 and
  // are ignored).  This thread's first pair is loaded here; further pairs
  // (only when the heads' channel pairs outnumber the threads) are folded
  // after the descriptor loads are issued.
  using Pair = typename CL::Pair;
  const int nheads = min(HW, H - h0);
  const int npairs = nheads * D / 2;
  const int nthr = blockDim.x;
  Pair qv[MAXG];
  {
    // branch-free (a thread past the last pair re-reads it), so no wait is
    // placed at a join before the descriptor loads
    const int v0 = t < npairs ? t : npairs - 1;
    const T* qh = q + ((size_t)r * H * G + (size_t)(h0 + v0 / (D / 2)) * G) * D + (v0 % (D / 2)) * 2;
#pragma unroll
    for (int j = 0; j < MAXG; ++j) qv[j] = *reinterpret_cast<const Pair*>(qh + (size_t)min(j, G - 1) * D);
  }
  const int L = clampi(seq_len, 0, max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  uint4 buf[U][2];
  int bl[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int bo = u * bpi + bsub;
    const int b = wg_b0 + bo;
    bl[u] = b;
    const int p = clampi(__shfl(my_pid, bo), 0, num_pool_blocks - 1);
    if (b < M && head_ok) {
      const uint4* src = reinterpret_cast<const uint4*>(desc + (((size_t)p * H + head) * 2 + part) * D + c0);
      buf[u][0] = src[0];
      buf[u][1] = src[1];
    } else {
      buf[u][0] = make_uint4(0, 0, 0, 0);
      buf[u][1] = make_uint4(0, 0, 0, 0);
    }
  }
  for (int v = t; v < npairs; v += nthr) {
    const int hh = v / (D / 2);
    const int c = (v % (D / 2)) * 2;
    if (v != t) {  // rare: more channel pairs than threads
      const T* qh = q + ((size_t)r * H * G + (size_t)(h0 + hh) * G) * D + c;
#pragma unroll
      for (int j = 0; j < MAXG; ++j) qv[j] = *reinterpret_cast<const Pair*>(qh + (size_t)min(j, G - 1) * D);
    }
    float p0 = 0.f, p1 = 0.f, n0 = 0.f, n1 = 0.f;
#pragma unroll
    for (int j = 0; j < MAXG; ++j) {
      float x0, x1;
      CL::unpack_pair(qv[j], x0, x1);
      x0 = j < G ? x0 : 0.f;
      x1 = j < G ? x1 : 0.f;
      if constexpr (MODE == 0) {
        p0 += fmaxf(x0, 0.f);
        p1 += fmaxf(x1, 0.f);
        n0 += fminf(x0, 0.f);
        n1 += fminf(x1, 0.f);
      } else {
        p0 += x0;
        p1 += x1;
      }
    }
    if constexpr (MODE != 0) {
      const float m0 = p0 / (float)G, m1 = p1 / (float)G;
      p0 = fmaxf(m0, 0.f);
      p1 = fmaxf(m1, 0.f);
      n0 = fminf(m0, 0.f);
      n1 = fminf(m1, 0.f);
    }
    s_coef[(hh * 2 + 0) * D + c] = n0;
    s_coef[(hh * 2 + 0) * D + c + 1] = n1;
    s_coef[(hh * 2 + 1) * D + c] = p0;
    s_coef[(hh * 2 + 1) * D + c + 1] = p1;
  }
  __syncthreads();
  float coef[VPL];
  const int hc = head_ok ? hl : 0;
#pragma unroll
  for (int v = 0; v < VPL; v += 4) {
    const floatx4_t c4 = *reinterpret_cast<const floatx4_t*>(&s_coef[(hc * 2 + part) * D + c0 + v]);
    coef[v] = c4[0];
    coef[v + 1] = c4[1];
    coef[v + 2] = c4[2];
    coef[v + 3] = c4[3];
  }

#pragma unroll
  for (int u = 0; u < U; ++u) {
    float vals[VPL];
    CL::unpack(buf[u][0], buf[u][1], vals);
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) acc = fmaf(coef[v], vals[v], acc);
    acc = group_sum<CH>(acc);
    if (lg == 0 && head_ok && bl[u] < M) {
      key_row[bl[u]] = f32_order_key(acc);
      if (score_row) score_row[bl[u]] = acc;
    }
  }
}

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void select_kernel(const uint32_t* __restrict__ keys,
                                                    const int32_t* __restrict__ seq_lens,
                                                    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt,
                                                    int H, int max_blocks, int max_sel, int budget_num,
                                                    int budget_den, int min_blocks, int local_blocks,
                                                    int key_stride) {
  __shared__ SelectLds<NT> sl;
  const int i = blockIdx.x;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  KeyRuns<NT, KPT> kr;
  kr.prefetch(keys + ((size_t)r * H + i) * key_stride, key_stride);  // in flight with seq_lens
  const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  int32_t* out = sel_idx + ((size_t)r * H + i) * max_sel;

  int n = 0, nl = 0;
  if (M > 0) {
    long long nn = ((long long)M * budget_num + budget_den - 1) / budget_den;
    if (nn < min_blocks) nn = min_blocks;
    if (nn < local_blocks) nn = local_blocks;
    if (nn > M) nn = M;
    n = (int)nn;
    nl = local_blocks < M ? local_blocks : M;
  }
  const int k = n - nl;  // blocks chosen by score
  const int C = M - nl;  // candidates: blocks [0, C)
  for (int j = tid; j < max_sel; j += NT) {
    if (j >= n) out[j] = -1;
    else if (j >= k) out[j] = C + (j - k);  // forced recent blocks close the ascending list
  }
  if (tid == 0) sel_cnt[(size_t)r * H + i] = n;
  if (k == 0) return;
  if (k == C) {
    for (int j = tid; j < C; j += NT) out[j] = j;
    return;
  }
  kr.set_count(C);
  for (int b = tid; b <= kBins; b += NT) {  // published by the barrier of block_min_max
    sl.hist2[0][b] = 0u;
    sl.hist2[1][b] = 0u;
  }
  if (tid == 0) sl.packed = 0;
  // key range of the candidates
  uint32_t mn = 0xffffffffu, mx = 0u;
  RESA_FOR_KEYS({
    const uint32_t x = kr.key(j);
    mn = in ? min(mn, x) : mn;
    mx = in ? max(mx, x) : mx;
  });
  int mm_use = 1;  // the slot set the selection's first range pass does not use
  block_min_max<NT>(mn, mx, sl.mm_slots, mm_use);
  select_top<NT, KPT>(sl, kr, C, k, mn, mx, out);
}

template <typename T, int D>
hipError_t launch_scores_t(const ScoreArgs& a, hipStream_t stream) {
  constexpr int VPL = ChunkLoad<T>::kVals;
  constexpr int CH = 2 * D / VPL;
  // heads per workgroup: all of them when whole wavefronts of blocks of all
  // heads fit in kScoreThreads threads, else the largest power of two of
  // heads whose blocks do
  auto min_blocks_per_pass = [](int unit) {
    int m = 1;
    while ((unit * m) % 64 != 0) ++m;
    return m;
  };
  int HW = a.H;
  if (CH * HW * min_blocks_per_pass(CH * HW) > kScoreThreads) {
    HW = 1;
    while (CH * HW * 2 <= kScoreThreads) HW *= 2;
  }
  const int unit = CH * HW;  // threads per block of all the group's heads
  int m = min_blocks_per_pass(unit);
  while (unit * m * 2 <= kScoreThreads && m * 2 * 4 <= 64) m *= 2;
  const int threads = unit * m;  // <= kScoreThreads
  const int bpi = m;
  // Four passes per thread, unless the grid would then leave CUs idle (short
  // rows, few requests): fewer passes and more workgroups there.  Large
  // grids (long rows of several requests) take eight: each workgroup's fixed
  // cost (table entries, query fold, barrier) is then spread over twice the
  // descriptors (per layer-step: ragged 8 x 32-64K 44.3 -> 43.5 us, 4 x 131K
  // 51.2 -> 50.9, 128 x 2K 42.8 -> 42.1; sixteen passes were slower, and
  // grids below kScoreFill8 at eight passes, such as one 256K request or 64
  // requests of 4K, gain nothing).
  const long long groups = (long long)a.R * ((a.H + HW - 1) / HW);
  int U = 4;
  if (bpi * 8 <= 64 && groups * ((a.max_blocks + bpi * 8 - 1) / (bpi * 8)) >= kScoreFill8) U = 8;
  while (U > 1 && groups * ((a.max_blocks + bpi * U - 1) / (bpi * U)) < kScoreFill) U /= 2;
  const int blocks_per_wg = bpi * U;  // <= 64: one table entry per lane
  const int wgs = (a.max_blocks + blocks_per_wg - 1) / blocks_per_wg;
  const size_t lds = (size_t)HW * 2 * D * sizeof(float);
  dim3 grid((unsigned)(wgs + (a.refresh_tail ? 1 : 0)), (unsigned)a.R, (unsigned)((a.H + HW - 1) / HW));
#define RESA_SCORE_LAUNCH_U(MODE, MAXG, UU)                                                                  \
  hipLaunchKernelGGL((score_kernel<T, D, MODE, MAXG, UU>), grid, dim3(threads), lds, stream,                 \
                     static_cast<const T*>(a.q), static_cast<const T*>(a.desc_pool), a.table, a.seq_lens, a.keys, \
                     a.scores, a.H, HW, a.G, a.max_blocks, a.num_pool_blocks, static_cast<const T*>(a.k_pool), \
                     static_cast<T*>(const_cast<void*>(a.desc_pool)), wgs, a.key_stride)
#define RESA_SCORE_LAUNCH(MODE, MAXG)                      \
  do {                                                     \
    if (U == 8) RESA_SCORE_LAUNCH_U(MODE, MAXG, 8);        \
    else if (U == 4) RESA_SCORE_LAUNCH_U(MODE, MAXG, 4);   \
    else if (U == 2) RESA_SCORE_LAUNCH_U(MODE, MAXG, 2);   \
    else RESA_SCORE_LAUNCH_U(MODE, MAXG, 1);               \
  } while (0)
  if (a.G <= 8) {
    if (a.mode == 0) RESA_SCORE_LAUNCH(0, 8);
    else RESA_SCORE_LAUNCH(1, 8);
  } else {
    if (a.mode == 0) RESA_SCORE_LAUNCH(0, 16);
    else RESA_SCORE_LAUNCH(1, 16);
  }
#undef RESA_SCORE_LAUNCH
#undef RESA_SCORE_LAUNCH_U
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const ScoreArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)a.H, (unsigned)a.R);
  const long long cand_max = a.key_stride;
#define RESA_SELECT_LAUNCH(NT, KPT)                                                                           \
  hipLaunchKernelGGL((select_kernel<NT, KPT>), grid, dim3(NT), 0, stream, a.keys, a.seq_lens, a.sel_idx, a.sel_cnt, \
                     a.H, a.max_blocks, a.max_sel, a.budget_num, a.budget_den, a.min_blocks, a.local_blocks,   \
                     a.key_stride)
  // rows of up to 4096 keys: half the threads (every barrier waits for half
  // the wavefronts)
  if (cand_max <= 4LL * kSelectSmall) RESA_SELECT_LAUNCH(kSelectSmall, 4);
  else if (cand_max <= 8LL * kSelectSmall) RESA_SELECT_LAUNCH(kSelectSmall, 8);
  else if (cand_max <= 8LL * kSelectThreads) RESA_SELECT_LAUNCH(kSelectThreads, 8);
  else if (cand_max <= 16LL * kSelectThreads) RESA_SELECT_LAUNCH(kSelectThreads, 16);
  else if (cand_max <= 32LL * kSelectThreads) RESA_SELECT_LAUNCH(kSelectThreads, 32);
  else RESA_SELECT_LAUNCH(kSelectThreads, 0);
#undef RESA_SELECT_LAUNCH
  return hipGetLastError();
}

hipError_t launch_scores(const ScoreArgs& a, hipStream_t stream) {
  if (a.dtype == 0)
    return a.D == 128 ? launch_scores_t<bf16_t, 128>(a, stream) : launch_scores_t<bf16_t, 64>(a, stream);
  return a.D == 128 ? launch_scores_t<float, 128>(a, stream) : launch_scores_t<float, 64>(a, stream);
}

hipError_t launch_score_select(const ScoreArgs& a, hipStream_t stream) {
  const hipError_t e = launch_scores(a, stream);
  if (e != hipSuccess) return e;
  return launch_select(a, stream);
}

}  // namespace resa
