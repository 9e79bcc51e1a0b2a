// resa_score_select in one launch: group block scores (Eq 4) and top-n
// block selection (Eq 5 with the forced local window) of the "Rectified
// Sparse Attention" analysis page (paper-graph-ui), §3.4.1.
//
// A 1024-thread workgroup scores one slice of consecutive blocks of one
// (request, KV head) (score_core.h), writes the scores as order-preserving
// keys, stores the slice's candidate key range in its own slot and counts
// itself in with one atomic add.  The workgroup that arrives last for a
// (request, KV head) - every key of the row is written by then - runs the
// selection (select_core.h) with its 1024 threads while the others have
// exited, so the selection costs no launch of its own.  The last workgroup
// resets the counter to zero for the next call.  One extra workgroup per
// (request, KV head) refreshes the tail block's descriptor when asked.
#include "desc_unit.h"
#include "score_core.h"

namespace resa {
namespace {

constexpr int kNT = 1024;      // threads of a scoring / selection workgroup
constexpr int kMaxUnroll = 4;  // passes of a scoring workgroup over its slice

// Exchange records in the workspace.  Per (request, KV head): an arrival
// counter, zero between calls, alone in a 128-byte line (counters of
// different heads on one line slow each other's atomics down); then per
// slice the complement of its smallest candidate key and its largest
// candidate key (complement and value of an empty slice: 0).
constexpr int kSyncWords = 32;
constexpr int kMinSliceBlocks = 32;  // blocks of the smallest slice (fp32, d = 128, one pass)
inline int max_slices(int max_blocks) { return (max_blocks + kMinSliceBlocks - 1) / kMinSliceBlocks; }

template <typename T, int D, int MAXG, int KPT>
__global__ __launch_bounds__(kNT) void score_select_kernel(const ScoreArgs a) {
  using SS = SliceScore<T, D, MAXG, kNT, kMaxUnroll>;
  __shared__ __align__(16) float s_coef[2 * D];  // N (min row), then P (max row)
  __shared__ uint2 s_mm[kNT / 64];
  __shared__ int s_last;
  __shared__ SelectLds<kNT> sl;

  const int slice = blockIdx.x;
  const int i = blockIdx.y;
  const int r = blockIdx.z;
  const int t = threadIdx.x;
  const int H = a.H;
  const int32_t* tab = a.table + (size_t)r * a.max_blocks;
  if (slice >= a.nslices) {
    // Tail refresh: one wavefront recomputes the descriptor of the head's last
    // block (the block the newest token was appended to).  That block is
    // always selected, so the score the scoring workgroups read for it
    // concurrently is never used.
    if (t >= 64) return;
    const int L = clampi(a.seq_lens[r], 0, a.max_blocks * kBlock);
    const int M = (L + kBlock - 1) / kBlock;
    if (M == 0) return;
    const int p = clampi(tab[M - 1], 0, a.num_pool_blocks - 1);
    descriptor_unit<T, D>(static_cast<const T*>(a.k_pool) + ((size_t)p * H + i) * kBlock * D,
                          static_cast<T*>(const_cast<void*>(a.desc_pool)) + ((size_t)p * H + i) * 2 * D,
                          L - (M - 1) * kBlock);
    return;
  }
  const int lane = t & 63;
  const int wave = t >> 6;
  const int L = clampi(a.seq_lens[r], 0, a.max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  const int nl = a.local_blocks < M ? a.local_blocks : M;
  const int C = M - nl;  // candidates: blocks [0, C)
  uint32_t* key_row = a.keys + ((size_t)r * H + i) * a.key_stride;
  float* score_row = a.scores ? a.scores + ((size_t)r * H + i) * a.max_blocks : nullptr;
  SS ss;
  ss.run(static_cast<const T*>(a.q) + ((size_t)r * H + i) * a.G * D, static_cast<const T*>(a.desc_pool), tab, M, C,
         slice * a.unroll * SS::BPP, a.unroll, H, i, a.G, a.mode, a.max_blocks, a.num_pool_blocks, key_row,
         score_row, s_coef);

  // This slice's candidate key range goes to its own slot; then the
  // workgroup counts itself in.  Every key and range store has completed
  // (device scope) before the arrival atomic is issued.
  uint32_t kmin = ss.kmin, kmax = ss.kmax;
  wave_min_max(kmin, kmax);
  if (lane == 0) s_mm[wave] = make_uint2(kmin, kmax);
  __syncthreads();
  uint32_t* counter = a.sync + ((size_t)r * H + i) * kSyncWords;
  uint32_t* ranges = a.ranges + ((size_t)r * H + i) * a.range_stride;
  if (t == 0) {
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int w = 0; w < kNT / 64; ++w) {
      mn = min(mn, s_mm[w].x);
      mx = max(mx, s_mm[w].y);
    }
    store_agent(ranges + 2 * slice, ~mn);
    store_agent(ranges + 2 * slice + 1, mx);
  }
  wait_vm_all();  // this thread's key (and range) stores are complete
  __syncthreads();
  if (t == 0) {
    const uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == (uint32_t)(a.nslices - 1);
    if (last) store_agent(counter, 0u);  // every workgroup of the row has arrived: reset for the next call
    s_last = last ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;

  // ---- the last workgroup of (r, i): the selection
  int n = 0;
  if (M > 0) {
    long long nn = ((long long)M * a.budget_num + a.budget_den - 1) / a.budget_den;
    if (nn < a.min_blocks) nn = a.min_blocks;
    if (nn < a.local_blocks) nn = a.local_blocks;
    if (nn > M) nn = M;
    n = (int)nn;
  }
  const int k = n - nl;  // blocks chosen by score
  int32_t* out = a.sel_idx + ((size_t)r * H + i) * a.max_sel;
  for (int j = t; j < a.max_sel; j += kNT) {
    if (j >= n) out[j] = -1;
    else if (j >= k) out[j] = C + (j - k);  // forced recent blocks close the ascending list
  }
  if (t == 0) a.sel_cnt[(size_t)r * H + i] = n;
  if (k == 0) return;
  if (k == C) {
    for (int j = t; j < C; j += kNT) out[j] = j;
    return;
  }
  // keys and slice ranges in flight together
  KeyRuns<kNT, KPT> kr;
  kr.prefetch(key_row, a.key_stride);
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int s2 = t; s2 < a.nslices; s2 += kNT) {
    mn = min(mn, ~load_agent(ranges + 2 * s2));
    mx = max(mx, load_agent(ranges + 2 * s2 + 1));
  }
  kr.set_count(C);
  wave_min_max(mn, mx);
  if (lane == 0) s_mm[wave] = make_uint2(mn, mx);
  for (int b = t; b <= kBins; b += kNT) {
    sl.hist2[0][b] = 0u;
    sl.hist2[1][b] = 0u;
  }
  if (t == 0) sl.packed = 0;
  __syncthreads();
  mn = 0xffffffffu;
  mx = 0u;
#pragma unroll
  for (int w = 0; w < kNT / 64; ++w) {
    mn = min(mn, s_mm[w].x);
    mx = max(mx, s_mm[w].y);
  }
  select_top<kNT, KPT>(sl, kr, C, k, mn, mx, out);
}

template <typename T, int D>
hipError_t launch_t(const ScoreArgs& a0, hipStream_t stream) {
  constexpr int BPP = SliceScore<T, D, 8, kNT, kMaxUnroll>::BPP;
  ScoreArgs a = a0;
  a.range_stride = 2 * max_slices(a.max_blocks);
  // Slices of up to four passes, fewer while that leaves the launch short of
  // about one workgroup per compute unit.
  const long long units = (long long)a.R * a.H;
  int U = kMaxUnroll;
  while (U > 1 && units * ((a.max_blocks + BPP * U - 1) / (BPP * U)) < 256) U /= 2;
  a.unroll = U;
  a.nslices = (a.max_blocks + BPP * U - 1) / (BPP * U);
  dim3 grid((unsigned)(a.nslices + (a.refresh_tail ? 1 : 0)), (unsigned)a.H, (unsigned)a.R);
  const int cand_max = a.key_stride;
#define RESA_SS_LAUNCH(MAXG, KPT) \
  hipLaunchKernelGGL((score_select_kernel<T, D, MAXG, KPT>), grid, dim3(kNT), 0, stream, a)
#define RESA_SS_KPT(MAXG)                              \
  do {                                                 \
    if (cand_max <= 8 * kNT) RESA_SS_LAUNCH(MAXG, 8);   \
    else if (cand_max <= 16 * kNT) RESA_SS_LAUNCH(MAXG, 16); \
    else if (cand_max <= 32 * kNT) RESA_SS_LAUNCH(MAXG, 32); \
    else RESA_SS_LAUNCH(MAXG, 0);                      \
  } while (0)
  if (a.G <= 8) RESA_SS_KPT(8);
  else RESA_SS_KPT(16);
#undef RESA_SS_KPT
#undef RESA_SS_LAUNCH
  return hipGetLastError();
}

}  // namespace

size_t score_select_sync_bytes(int R, int H) { return (size_t)R * H * kSyncWords * sizeof(uint32_t); }
size_t score_select_range_bytes(int R, int H, int max_blocks) {
  return (size_t)R * H * 2 * max_slices(max_blocks) * sizeof(uint32_t);
}

hipError_t launch_score_select(const ScoreArgs& a, hipStream_t stream) {
  if (a.dtype == 0) return a.D == 128 ? launch_t<bf16_t, 128>(a, stream) : launch_t<bf16_t, 64>(a, stream);
  return a.D == 128 ? launch_t<float, 128>(a, stream) : launch_t<float, 64>(a, stream);
}

}  // namespace resa
