// Split-K flash decode over a block list: group block sparse attention
// (selected blocks) and dense attention (all blocks), and the log-sum-exp
// merge of split partials.
//
// "Rectified Sparse Attention" analysis page (paper-graph-ui): §3.4.1 Eq 1
// and Eq 2, §3.4.4 (split execution with partial log-sum-exp results
// combined afterwards).
//
// Work decomposition.  Grid (splits, KV heads, requests).  The block list of
// one (request, KV head) is cut into `splits` equal ranges, one per workgroup
// of 8 wavefronts (about one workgroup per CU); the wavefronts take
// consecutive sub-ranges and each keeps its own online-softmax state
// (decode_core.h), merged through LDS into one partial (m, l, o) per query
// head.  A second kernel merges the splits' partials with their log-sum-exp
// weights; with one split per row (large batches) the workgroup normalises
// and writes the output itself and no merge is launched.
#include "decode_core.h"
#include "resa_internal.h"

namespace resa {
namespace {

template <typename T, int D, bool SPARSE, int NW>
__global__ __launch_bounds__(64 * NW) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k_pool, const T* __restrict__ v_pool,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_cnt, int max_sel, float* __restrict__ part_o, float* __restrict__ part_ml,
    float* __restrict__ out, int H, int G, int max_blocks, int num_pool_blocks, int S, float scale_log2) {
  using F = Frag<T, D>;
  __shared__ MergeLds<NW, D> mls;

  const int s = blockIdx.x;
  const int i = blockIdx.y;
  const int r = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int quad = lane >> 4;

  const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  int n, bps;
  if (SPARSE) {
    n = clampi(sel_cnt[(size_t)r * H + i], 0, max_sel < M ? max_sel : M);
    bps = (max_sel + S - 1) / S;
  } else {
    n = M;
    bps = (max_blocks + S - 1) / S;
  }
  // The split and wavefront ranges depend only on the list capacity, so the
  // block-id loads do not wait for sel_cnt; n only trims the range.
  const int beg = s * bps;
  const int per = (bps + NW - 1) / NW;
  const int cap = SPARSE ? max_sel : max_blocks;
  const int wb = beg + wave * per;
  const int we_cap = min(min(beg + bps, cap), wb + per);  // positions readable without n
  const int we = min(we_cap, n);

  typename F::Q qf;
  F::load_q(qf, q + ((size_t)r * H + i) * G * D, col, quad, G);
  WaveAttn<T, D> st;
  st.init();
  const int32_t* tab_row = table + (size_t)r * max_blocks;
  if constexpr (SPARSE) {
    const int32_t* sel_row = sel_idx + ((size_t)r * H + i) * max_sel;
    st.run([&](int p) { return sel_row[p]; }, wb, we_cap, we, qf, k_pool, v_pool, tab_row, H, i, L, max_blocks,
           num_pool_blocks, scale_log2);
  } else {
    st.run([&](int p) { return p; }, wb, we_cap, we, qf, k_pool, v_pool, tab_row, H, i, L, max_blocks,
           num_pool_blocks, scale_log2);
  }
  const size_t prow = ((size_t)r * H + i) * S + s;  // partial row of this workgroup
  // a row's only split writes the output itself (no merge launch follows)
  wg_merge_store<T, D, NW>(st, mls, G, part_o + prow * G * D, part_ml + prow * G * 2,
                           S == 1 ? out + ((size_t)r * H + i) * G * D : nullptr);
}

// One wavefront per merge workgroup while the grid is small: the decode
// merges are latency-bound, and small workgroups spread their loads over
// more CUs (0.2-0.5 us per layer-step against 256-thread workgroups at every
// decode size measured).  Merges of more than kMergeSmallMaxWgs wavefronts
// (the rectification's) fill the chip either way and run 256-thread
// workgroups.
constexpr int kMergeSmallThreads = 64;
constexpr int kMergeLargeThreads = 256;
constexpr long long kMergeSmallMaxWgs = 2048;
constexpr long long kMergeMaxGrid = 1 << 20;  // workgroups of one merge launch
constexpr unsigned kXcds = 8;  // MI355X: 8 XCDs, each with its own L2; workgroups are dealt to them in turn

// Log-sum-exp merge of split partials (decode_core.h), one output float4 per
// P lanes.  64-bit thread index; the grid strides over the rows when it is
// capped (rows * C4 * P may exceed 2^31).  The stride is a multiple of P, so
// the P lanes of a group always share one row and leave the loop together.
template <int D, int P, int NTH>
__global__ __launch_bounds__(NTH) void merge_kernel(const float* __restrict__ part_o,
                                                              const float* __restrict__ part_ml,
                                                              float* __restrict__ out, int H, int G, int S,
                                                              int rows_per_head, int row_stride_out,
                                                              long long total_rows) {
  constexpr int C4 = D / 4;  // float4 per output row
  const PlainPartials pp{part_o, part_ml};
  // XCD-aware order: workgroup b runs on XCD b mod 8, so logical workgroups
  // are numbered XCD by XCD (a bijection on the first 8 * (grid / 8)
  // workgroups; the rest keep their index).  Neighbouring workgroups share
  // 128-byte lines of the partials and the (m, l) pairs of their rows; on
  // one XCD they fetch them from HBM once instead of once per L2.
  const unsigned nwg = gridDim.x;
  const unsigned full = nwg - nwg % kXcds;
  const unsigned wg =
      blockIdx.x < full ? (blockIdx.x % kXcds) * (full / kXcds) + blockIdx.x / kXcds : blockIdx.x;
  const long long stride = (long long)nwg * NTH;
  for (long long g = (long long)wg * NTH + threadIdx.x; g < total_rows * C4 * P; g += stride) {
    const int part = (int)(g % P);
    const int c4 = (int)((g / P) % C4);
    const long long grow = g / (P * C4);  // (r, i, row) flattened
    const int row = (int)(grow % rows_per_head);
    const long long ri = grow / rows_per_head;  // r * H + i
    const floatx4_t v = merge_float4<D, P>(pp, (size_t)ri * S, S, rows_per_head, row, c4, part);
    if (part == 0) {
      const long long r = ri / H;
      const int i = (int)(ri % H);
      const int j = row % G;
      const int t = row / G;
      float* dst = out + (((size_t)r * row_stride_out + t) * H * G + (size_t)i * G + j) * D + 4 * c4;
      *reinterpret_cast<floatx4_t*>(dst) = v;
    }
  }
}

template <int D, int P>
hipError_t launch_merge_t(const float* part_o, const float* part_ml, float* out, int H, int G, int S,
                          int rows_per_head, int row_stride_out, long long rows, hipStream_t stream) {
  const long long threads = rows * (D / 4) * P;
  long long wgs = (threads + kMergeSmallThreads - 1) / kMergeSmallThreads;
  if (wgs <= kMergeSmallMaxWgs) {
    hipLaunchKernelGGL((merge_kernel<D, P, kMergeSmallThreads>), dim3((unsigned)wgs), dim3(kMergeSmallThreads), 0,
                       stream, part_o, part_ml, out, H, G, S, rows_per_head, row_stride_out, rows);
    return hipGetLastError();
  }
  wgs = (threads + kMergeLargeThreads - 1) / kMergeLargeThreads;
  if (wgs > kMergeMaxGrid) wgs = kMergeMaxGrid;  // larger merges stride over the rows
  hipLaunchKernelGGL((merge_kernel<D, P, kMergeLargeThreads>), dim3((unsigned)wgs), dim3(kMergeLargeThreads), 0,
                     stream, part_o, part_ml, out, H, G, S, rows_per_head, row_stride_out, rows);
  return hipGetLastError();
}

template <int D>
hipError_t launch_merge_d(const float* part_o, const float* part_ml, float* out, int H, int G, int S,
                          int rows_per_head, int row_stride_out, long long rows, hipStream_t stream) {
  // lanes per float4: the fewest that take every partial in one batch of loads
  if (S <= 1 * kMergeBatch)
    return launch_merge_t<D, 1>(part_o, part_ml, out, H, G, S, rows_per_head, row_stride_out, rows, stream);
  if (S <= 2 * kMergeBatch)
    return launch_merge_t<D, 2>(part_o, part_ml, out, H, G, S, rows_per_head, row_stride_out, rows, stream);
  if (S <= 4 * kMergeBatch)
    return launch_merge_t<D, 4>(part_o, part_ml, out, H, G, S, rows_per_head, row_stride_out, rows, stream);
  if (S <= 8 * kMergeBatch)
    return launch_merge_t<D, 8>(part_o, part_ml, out, H, G, S, rows_per_head, row_stride_out, rows, stream);
  return launch_merge_t<D, kMergeMaxParts>(part_o, part_ml, out, H, G, S, rows_per_head, row_stride_out, rows,
                                           stream);
}

template <typename T, int D, int NW>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)a.splits, (unsigned)a.H, (unsigned)a.R);
  dim3 block(64 * NW);
  if (a.sel_idx) {
    hipLaunchKernelGGL((decode_kernel<T, D, true, NW>), grid, block, 0, stream, static_cast<const T*>(a.q),
                       static_cast<const T*>(a.k_pool), static_cast<const T*>(a.v_pool), a.table, a.seq_lens,
                       a.sel_idx, a.sel_cnt, a.max_sel, a.part_o, a.part_ml, a.out, a.H, a.G, a.max_blocks,
                       a.num_pool_blocks, a.splits, a.scale_log2);
  } else {
    hipLaunchKernelGGL((decode_kernel<T, D, false, NW>), grid, block, 0, stream, static_cast<const T*>(a.q),
                       static_cast<const T*>(a.k_pool), static_cast<const T*>(a.v_pool), a.table, a.seq_lens,
                       nullptr, nullptr, 0, a.part_o, a.part_ml, a.out, a.H, a.G, a.max_blocks, a.num_pool_blocks,
                       a.splits, a.scale_log2);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;  // one split: the decode wrote the output
  return launch_merge(a.part_o, a.part_ml, a.out, a.R, a.H, a.G, a.D, a.splits, a.G, 1, stream);
}

}  // namespace

hipError_t launch_merge(const float* part_o, const float* part_ml, float* out, int R, int H, int G, int D, int S,
                        int rows_per_head, int row_stride_out, hipStream_t stream) {
  const long long rows = (long long)R * H * rows_per_head;
  if (D == 128)
    return launch_merge_d<128>(part_o, part_ml, out, H, G, S, rows_per_head, row_stride_out, rows, stream);
  return launch_merge_d<64>(part_o, part_ml, out, H, G, S, rows_per_head, row_stride_out, rows, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  // fp32 fragments need twice the registers: 4 wavefronts per workgroup keeps them spill-free
  if (a.dtype == 0)
    return a.D == 128 ? launch_decode_t<bf16_t, 128, kDecodeWaves>(a, stream)
                      : launch_decode_t<bf16_t, 64, kDecodeWaves>(a, stream);
  return a.D == 128 ? launch_decode_t<float, 128, 4>(a, stream) : launch_decode_t<float, 64, 4>(a, stream);
}

}  // namespace resa
