// Min / max descriptor of one (block, KV head) key tile, computed by one
// wavefront (Eq 3 of the "Rectified Sparse Attention" analysis page,
// §3.4.1).  Lane l reads 16-byte chunk (l % CPR) of rows l / CPR,
// l / CPR + 64 / CPR, ...; rows at or past `valid_rows` are ignored.  Values
// are compared through order-preserving integer keys (-0 < +0), so every
// result is a bit-exact copy of a stored key value.  Shared by the
// descriptor kernel and the tail refresh of resa_score_select.
#pragma once

#include "resa_internal.h"

namespace resa {

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

template <typename T, int D>
__device__ __forceinline__ void descriptor_unit(const T* __restrict__ src, T* __restrict__ dst, int valid_rows) {
  using KT = KeyTraits<T>;
  constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per key row
  constexpr int RPI = 64 / CPR;                 // rows per load instruction
  constexpr int NLD = kBlock / RPI;             // load instructions per tile
  constexpr int VPC = KT::kValsPerChunk;
  const int lane = threadIdx.x & 63;
  const int chunk = lane % CPR;
  const int row0 = lane / CPR;
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
    *reinterpret_cast<uint4*>(dst + chunk * VPC) = KT::from_keys(lo);
    *reinterpret_cast<uint4*>(dst + D + chunk * VPC) = KT::from_keys(hi);
  }
}

}  // namespace resa
