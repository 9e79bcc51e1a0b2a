// resa_sparse_step: one decode step of one attention layer - tail descriptor
// refresh, group block scores, top-n selection and block sparse attention -
// in three launches: scoring, selection fused with the split attention, and
// the log-sum-exp merge.
//
// "Rectified Sparse Attention" analysis page (paper-graph-ui): §3.4.1
// (Eq 3-5: descriptors, block scores, top-n with the local window; Eq 2:
// attention over the selected blocks), §3.4.3 Algorithm 1 (the block key
// cache is updated as tokens are appended), §3.4.4 (split attention kernel
// with a log-sum-exp merge; kernel time without CPU overhead).
//
// Selection inside the attention launch.  Grid (splits, KV heads, requests),
// as resa_sparse_decode.  Split s of a row attends over positions
// [s bps, (s + 1) bps) of the row's ascending selected list.  Instead of
// waiting for a selection launch to write that list, every one of the row's
// split workgroups reads the row's score keys (written by the scoring
// launch; at most 32 KB, served mostly from the L2 after the first
// workgroup of an XCD) and finds the row's threshold itself with the
// histogram select of select_core.h.  The selection is deterministic, so
// every split finds the same threshold; one scan of the per-thread taken
// counts then places each selected id, and the split keeps the ids of its
// own positions in LDS and writes them to sel_idx.  No workgroup waits for
// another: the cost is the selection's latency inside each workgroup, in
// place of a selection launch (its ramp, its key loads from memory, its
// ordered output) between scoring and attention.
//
// Where the redundancy costs more than the launch it removes, the step runs
// the selection launch and the decode launch instead: rows of more than
// 8192 keys (16 per thread; at 16384 keys the 256 workgroups' key reads
// alone take about 4 us and the selection another 6 in every workgroup,
// against 8.9 us for the whole selection launch on four CUs), grids of more
// than 256 workgroups (they run in rounds, each repeating the selection's
// latency), fp32 caches, and lists longer than the LDS list holds.  Every path gives the same
// sel_idx and sel_cnt.
#include "decode_core.h"

namespace resa {
namespace {

constexpr int kStepNW = kDecodeWaves;  // wavefronts of a select+attend workgroup
constexpr int kStepNT = 64 * kStepNW;
constexpr int kListCap = 2 * (kBins + 4);  // list entries the two selection histograms' LDS holds
constexpr long long kStepFusedMaxWgs = 256;  // the fused grid's workgroups, at most: one per CU

template <int NT, int NW, int D>
struct SelDecodeLds {
  SelectLds<NT> sl;  // hist2 holds the split's id list once the threshold is known
  MergeLds<NW, D> mls;
};

template <typename T, int D, int NW, int KPT>
__global__ __launch_bounds__(64 * NW) void select_decode_kernel(
    const uint32_t* __restrict__ keys, int key_stride, const T* __restrict__ q, const T* __restrict__ k_pool,
    const T* __restrict__ v_pool, const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens,
    int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt, int max_sel, float* __restrict__ part_o,
    float* __restrict__ part_ml, float* __restrict__ out, int H, int G, int max_blocks, int num_pool_blocks, int S,
    float scale_log2,
    int budget_num, int budget_den, int min_blocks, int local_blocks) {
  constexpr int NT = 64 * NW;
  using F = Frag<T, D>;
  __shared__ SelDecodeLds<NT, NW, D> lds;
  SelectLds<NT>& sl = lds.sl;
  int32_t* list = reinterpret_cast<int32_t*>(&sl.hist2[0][0]);

  const int s = blockIdx.x;
  const int i = blockIdx.y;
  const int r = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int quad = lane >> 4;
  const size_t row = (size_t)r * H + i;

  // the row's keys and the group's queries are in flight together
  KeyRuns<NT, KPT> kr;
  kr.prefetch(keys + row * key_stride, key_stride);
  typename F::Q qf;
  F::load_q(qf, q + row * G * D, col, quad, G);

  const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  int n = 0, nl = 0;
  if (M > 0) {
    long long nn = ((long long)M * budget_num + budget_den - 1) / budget_den;
    if (nn < min_blocks) nn = min_blocks;
    if (nn < local_blocks) nn = local_blocks;
    if (nn > M) nn = M;
    n = (int)nn;
    nl = local_blocks < M ? local_blocks : M;
  }
  const int k = n - nl;  // blocks chosen by score, from the candidates [0, C)
  const int C = M - nl;  // list positions >= k hold the forced recent blocks C, C + 1, ...
  const int bps = (max_sel + S - 1) / S;  // list positions per split
  const int beg = s * bps;

  if (k > 0 && k < C) {
    kr.set_count(C);
    for (int b = tid; b <= kBins; b += NT) {  // published by the barrier of block_min_max
      sl.hist2[0][b] = 0u;
      sl.hist2[1][b] = 0u;
    }
    if (tid == 0) sl.packed = 0;
    uint32_t mn = 0xffffffffu, mx = 0u;
    RESA_FOR_KEYS({
      const uint32_t x = kr.key(j);
      mn = in ? min(mn, x) : mn;
      mx = in ? max(mx, x) : mx;
    });
    int mm_use = 1;  // the slot set the selection's first range pass does not use
    block_min_max<NT>(mn, mx, sl.mm_slots, mm_use);
    int scan_use = 0;
    const Threshold th = select_threshold<NT, KPT>(sl, kr, C, k, mn, mx, scan_use);
    uint32_t take;
    int pos;
    // its barriers also order every histogram read before the list writes below
    select_take<NT, KPT>(sl, kr, th, scan_use, take, pos);
    if (pos < beg + bps && pos + __popc(take) > beg) {
      const int first = tid * KPT;
      for (uint32_t m = take; m != 0u; m &= m - 1u, ++pos)
        if (pos >= beg && pos < beg + bps) list[pos - beg] = first + __builtin_ctz(m);
    }
  }
  for (int j = tid; j < bps; j += NT) {
    const int p = beg + j;
    if (p >= n) list[j] = 0;           // past the list: never attended
    else if (p >= k) list[j] = C + (p - k);  // forced recent blocks (all positions when k == C)
    else if (k == C) list[j] = p;      // every candidate is selected
  }
  __syncthreads();
  int32_t* out_row = sel_idx + row * max_sel;
  for (int j = tid; j < bps && beg + j < max_sel; j += NT) out_row[beg + j] = beg + j < n ? list[j] : -1;
  if (s == 0 && tid == 0) sel_cnt[row] = n;

  // attention over this split's positions, as the sparse decode kernel
  const int per = (bps + NW - 1) / NW;
  const int wb = beg + wave * per;
  const int we_cap = min(min(beg + bps, max_sel), wb + per);
  const int we = min(we_cap, n);
  WaveAttn<T, D> st;
  st.init();
  st.run([&](int p) { return list[p - beg]; }, wb, we_cap, we, qf, k_pool, v_pool, table + (size_t)r * max_blocks,
         H, i, L, max_blocks, num_pool_blocks, scale_log2);
  const size_t prow = row * S + s;
  wg_merge_store<T, D, NW>(st, lds.mls, G, part_o + prow * G * D, part_ml + prow * G * 2,
                           S == 1 ? out + row * G * D : nullptr);  // one split: the output itself
}

// Keys per thread of the fused kernel for rows of `key_stride` keys, or 0
// for rows the step leaves to the selection launch.
int step_kpt(int key_stride) {
  if (key_stride <= 4 * kStepNT) return 4;
  if (key_stride <= 8 * kStepNT) return 8;
  if (key_stride <= 16 * kStepNT) return 16;
  return 0;
}

template <typename T, int D>
hipError_t launch_select_decode_t(const ScoreArgs& sa, const DecodeArgs& da, int kpt, hipStream_t stream) {
  dim3 grid((unsigned)da.splits, (unsigned)da.H, (unsigned)da.R);
#define RESA_SELDEC_LAUNCH(KPT)                                                                                  \
  hipLaunchKernelGGL((select_decode_kernel<T, D, kStepNW, KPT>), grid, dim3(kStepNT), 0, stream, sa.keys,        \
                     sa.key_stride, static_cast<const T*>(da.q), static_cast<const T*>(da.k_pool),                \
                     static_cast<const T*>(da.v_pool), da.table, da.seq_lens, sa.sel_idx, sa.sel_cnt, sa.max_sel, \
                     da.part_o, da.part_ml, da.out, da.H, da.G, da.max_blocks, da.num_pool_blocks, da.splits,     \
                     da.scale_log2, sa.budget_num, sa.budget_den, sa.min_blocks, sa.local_blocks)
  switch (kpt) {
    case 4: RESA_SELDEC_LAUNCH(4); break;
    case 8: RESA_SELDEC_LAUNCH(8); break;
    default: RESA_SELDEC_LAUNCH(16); break;
  }
#undef RESA_SELDEC_LAUNCH
  return hipGetLastError();
}

}  // namespace

bool step_fused(int dtype, int key_stride, int max_sel, int splits, long long rows) {
  const int bps = (max_sel + splits - 1) / splits;
  // The fused grid must fit one round of workgroups (one per CU): in a second
  // round every workgroup's selection would sit on the critical path again
  // (batch 128 x 2K: 45.0 against 42.8 us for the separate launches).
  return dtype == 0 && step_kpt(key_stride) > 0 && bps <= kListCap && rows * splits <= kStepFusedMaxWgs;
}

hipError_t launch_step(const ScoreArgs& sa, const DecodeArgs& da, hipStream_t stream) {
  hipError_t e = launch_scores(sa, stream);
  if (e != hipSuccess) return e;
  if (!step_fused(sa.dtype, sa.key_stride, sa.max_sel, da.splits, (long long)da.R * da.H)) {
    e = launch_select(sa, stream);
    if (e != hipSuccess) return e;
    return launch_decode(da, stream);
  }
  const int kpt = step_kpt(sa.key_stride);
  e = da.D == 128 ? launch_select_decode_t<bf16_t, 128>(sa, da, kpt, stream)
                  : launch_select_decode_t<bf16_t, 64>(sa, da, kpt, stream);
  if (e != hipSuccess || da.splits == 1) return e;  // one split: the attention wrote the output
  return launch_merge(da.part_o, da.part_ml, da.out, da.R, da.H, da.G, da.D, da.splits, da.G, 1, stream);
}

}  // namespace resa
