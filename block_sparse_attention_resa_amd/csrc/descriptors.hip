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
#include "resa_internal.h"

namespace resa {
namespace {

template <typename T>
struct KeyTraits;

template <>
struct KeyTraits<bf16_t> {
  static constexpr int kValsPerChunk = 8;
  __device__ static void to_keys(const uint4& v, uint32_t* k) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      k[2 * e] = bf16_order_key(w[e] & 0xffffu);
      k[2 * e + 1] = bf16_order_key(w[e] >> 16);
    }
  }
  __device__ static uint4 from_keys(const uint32_t* k) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = bf16_from_order_key(k[2 * e]) | (bf16_from_order_key(k[2 * e + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

template <>
struct KeyTraits<float> {
  static constexpr int kValsPerChunk = 4;
  __device__ static void to_keys(const uint4& v, uint32_t* k) {
    k[0] = u32_order_key(v.x);
    k[1] = u32_order_key(v.y);
    k[2] = u32_order_key(v.z);
    k[3] = u32_order_key(v.w);
  }
  __device__ static uint4 from_keys(const uint32_t* k) {
    return make_uint4(u32_from_order_key(k[0]), u32_from_order_key(k[1]), u32_from_order_key(k[2]),
                      u32_from_order_key(k[3]));
  }
};

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
  using KT = KeyTraits<T>;
  constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;                 // rows per load instruction
  constexpr int NLD = kBlock / RPI;             // load instructions per tile
  constexpr int VPC = KT::kValsPerChunk;

  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  int b0, b1;
  block_range(M, L, first_block, num_blocks, window, r, b0, b1);
  const int units = (b1 - b0) * H;
  const int chunk = lane % CPR;
  const int row0 = lane / CPR;

  for (int u = blockIdx.x * 4 + wave; u < units; u += gridDim.x * 4) {
    const int b = b0 + u / H;
    const int i = u % H;
    const int p = clampi(table[(size_t)r * max_blocks + b], 0, num_pool_blocks - 1);
    const T* src = k_pool + ((size_t)p * H + i) * kBlock * D;
    uint4 v[NLD];
#pragma unroll
    for (int k = 0; k < NLD; ++k)
      v[k] = *reinterpret_cast<const uint4*>(src + (size_t)(row0 + k * RPI) * D + chunk * VPC);

    uint32_t lo[VPC], hi[VPC];
#pragma unroll
    for (int e = 0; e < VPC; ++e) {
      lo[e] = 0xffffffffu;
      hi[e] = 0u;
    }
    const int valid_rows = L - b * kBlock;  // >= 1
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      if (row0 + k * RPI < valid_rows) {
        uint32_t kk[VPC];
        KT::to_keys(v[k], kk);
#pragma unroll
        for (int e = 0; e < VPC; ++e) {
          lo[e] = min(lo[e], kk[e]);
          hi[e] = max(hi[e], kk[e]);
        }
      }
    }
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1) {
#pragma unroll
      for (int e = 0; e < VPC; ++e) {
        lo[e] = min(lo[e], (uint32_t)__shfl_xor((int)lo[e], off));
        hi[e] = max(hi[e], (uint32_t)__shfl_xor((int)hi[e], off));
      }
    }
    if (row0 == 0) {
      T* dst = desc + ((size_t)p * H + i) * 2 * D + chunk * VPC;
      *reinterpret_cast<uint4*>(dst) = KT::from_keys(lo);
      *reinterpret_cast<uint4*>(dst + D) = KT::from_keys(hi);
    }
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
