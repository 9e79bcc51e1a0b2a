// Block descriptors: element-wise min / max of each 16-token key block.
//
// "Rectified Sparse Attention" analysis page (paper-graph-ui), §3.4.1 Eq 3
// (block descriptors) and §3.4.3 Algorithm 1 (the block key cache is updated
// as tokens are appended and recomputed for the blocks a rectification
// rewrites).
//
// One wavefront handles one (block, KV head) unit: the 16 x d key tile is
// 4 KiB for bf16 / d = 128.  Lane l reads 16-byte chunk (l % CPR) of rows
// l / CPR, l / CPR + 64 / CPR, ... so every load instruction covers whole
// rows and the wavefront reads the tile once, fully coalesced.  Values are
// compared through order-preserving integer keys (-0 < +0), so the result is
// a bit-exact copy of one stored key value per channel.  The lanes sharing a
// chunk then combine their partial min / max with cross-lane shuffles.
#include "desc_unit.h"
#include "resa_internal.h"

namespace resa {
namespace {

// Block range [b0, b1) of request r, see resa_build_descriptors.
__device__ __forceinline__ void block_range(int M, int L, const int32_t* first_block, int num_blocks,
                                            int window, int r, int& b0, int& b1) {
  if (window > 0) {
    b0 = L >= window ? (L - window) / kBlock : M;
    b1 = M;
  } else if (first_block == nullptr) {
    b0 = num_blocks <= 0 ? 0 : (M > num_blocks ? M - num_blocks : 0);
    b1 = M;
  } else {
    const long long f = first_block[r];
    const long long n = num_blocks > 0 ? num_blocks : M;
    long long lo = f < 0 ? 0 : (f > M ? M : f);
    long long hi = f + n;
    hi = hi < lo ? lo : (hi > M ? M : hi);
    b0 = (int)lo;
    b1 = (int)hi;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void descriptor_kernel(const T* __restrict__ k_pool, T* __restrict__ desc,
                                                        const int32_t* __restrict__ table,
                                                        const int32_t* __restrict__ seq_lens,
                                                        const int32_t* __restrict__ first_block, int num_blocks,
                                                        int window, int H, int max_blocks, int num_pool_blocks) {
  const int r = blockIdx.y;
  const int wave = threadIdx.x >> 6;
  const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  int b0, b1;
  block_range(M, L, first_block, num_blocks, window, r, b0, b1);
  const int units = (b1 - b0) * H;
  for (int u = blockIdx.x * 4 + wave; u < units; u += gridDim.x * 4) {
    const int b = b0 + u / H;
    const int i = u % H;
    const int p = clampi(table[(size_t)r * max_blocks + b], 0, num_pool_blocks - 1);
    descriptor_unit<T, D>(k_pool + ((size_t)p * H + i) * kBlock * D, desc + ((size_t)p * H + i) * 2 * D,
                          L - b * kBlock);
  }
}

template <typename T, int D>
hipError_t launch_t(const DescArgs& a, hipStream_t stream) {
  long long span;  // upper bound of blocks per request in the range
  if (a.window > 0)
    span = a.window / kBlock + 2;
  else if (a.num_blocks > 0)
    span = a.num_blocks;
  else
    span = a.max_blocks;
  if (span > a.max_blocks) span = a.max_blocks;
  long long wgs = (span * a.H + 3) / 4;
  if (wgs < 1) wgs = 1;
  if (wgs > 16384) wgs = 16384;
  dim3 grid((unsigned)wgs, (unsigned)a.R);
  hipLaunchKernelGGL((descriptor_kernel<T, D>), grid, dim3(256), 0, stream,
                     static_cast<const T*>(a.k_pool), static_cast<T*>(a.desc_pool), a.table, a.seq_lens,
                     a.first_block, a.num_blocks, a.window, a.H, a.max_blocks, a.num_pool_blocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_descriptors(const DescArgs& a, hipStream_t stream) {
  if (a.dtype == 0) return a.D == 128 ? launch_t<bf16_t, 128>(a, stream) : launch_t<bf16_t, 64>(a, stream);
  return a.D == 128 ? launch_t<float, 128>(a, stream) : launch_t<float, 64>(a, stream);
}

}  // namespace resa
