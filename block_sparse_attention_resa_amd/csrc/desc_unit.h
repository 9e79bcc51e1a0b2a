// Min / max descriptor of one (block, KV head) key tile, computed by one
// wavefront (Eq 3 of the "Rectified Sparse Attention" analysis page,
// §3.4.1).  Lane l reads 16-byte chunk (l % CPR) of rows l / CPR,
// l / CPR + 64 / CPR, ...; rows at or past `valid_rows` are ignored.  Values
// are compared through order-preserving integer keys (-0 < +0), so every
// result is a bit-exact copy of a stored key value.  Shared by the
// descriptor kernel and the tail refresh of resa_score_select.
#pragma once

#include <type_traits>

#include "resa_internal.h"

namespace resa {

typedef __attribute__((ext_vector_type(2))) unsigned short ushort2_t;
typedef __attribute__((ext_vector_type(2))) short short2_t;

// Order-preserving 16-bit keys of two bf16 values in one word (the same map
// as bf16_order_key, with -0 < +0): negative values are complemented, others
// get the sign bit set.
__device__ __forceinline__ ushort2_t bf16x2_order_key(uint32_t w) {
  const short2_t s = __builtin_bit_cast(short2_t, w) >> (short)15;  // -1 for negative values
  return __builtin_bit_cast(ushort2_t, w) ^ (__builtin_bit_cast(ushort2_t, s) | (unsigned short)0x8000);
}
__device__ __forceinline__ uint32_t bf16x2_from_order_key(ushort2_t k) {
  const short2_t s = __builtin_bit_cast(short2_t, k) >> (short)15;  // -1 for keys of non-negative values
  return __builtin_bit_cast(uint32_t, k ^ (~__builtin_bit_cast(ushort2_t, s) | (unsigned short)0x8000));
}

// Packed 16-bit min / max of two words.  The lane-swap results go through
// these 32-bit helpers: written directly as vector min / max of the two
// swap results, the operation was dropped from the generated code.
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(ushort2_t, a),
                                                                __builtin_bit_cast(ushort2_t, b)));
}
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(ushort2_t, a),
                                                                __builtin_bit_cast(ushort2_t, b)));
}

// Packed min / max over the lanes l, l ^ cpr, l ^ 2 cpr, ... (cpr = 8 or 16):
// row rotation by 8 within 16-lane rows, then the 16- and 32-lane swaps (each
// leaves the two partners' values in the two results).
template <bool MIN>
__device__ __forceinline__ uint32_t rows_reduce(uint32_t u, int cpr) {
  if (cpr <= 8) {
    const uint32_t r = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xf, 0xf, false);  // row_ror:8
    u = MIN ? pk_min_u16(u, r) : pk_max_u16(u, r);
  }
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  u = MIN ? pk_min_u16(a[0], a[1]) : pk_max_u16(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return MIN ? pk_min_u16(b[0], b[1]) : pk_max_u16(b[0], b[1]);
}

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

// Geometry of one wavefront's pass over a 16 x D key tile.
template <typename T, int D>
struct DescTile {
  static constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per key row
  static constexpr int RPI = 64 / CPR;                 // rows per load instruction
  static constexpr int NLD = kBlock / RPI;             // load instructions per tile
  static constexpr int VPC = KeyTraits<T>::kValsPerChunk;
};

// The lane's share of a key tile: chunk (lane % CPR) of rows lane / CPR + k RPI.
template <typename T, int D>
__device__ __forceinline__ void descriptor_load(const T* __restrict__ src, uint4 (&v)[DescTile<T, D>::NLD]) {
  using DT = DescTile<T, D>;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 0; k < DT::NLD; ++k)
    v[k] = *reinterpret_cast<const uint4*>(src + (size_t)(lane / DT::CPR + k * DT::RPI) * D +
                                           (lane % DT::CPR) * DT::VPC);
}

// Min / max of the loaded tile over its first valid_rows rows, written to dst
// (min row, then max row).
template <typename T, int D>
__device__ __forceinline__ void descriptor_reduce(const uint4 (&v)[DescTile<T, D>::NLD], T* __restrict__ dst,
                                                  int valid_rows) {
  using KT = KeyTraits<T>;
  using DT = DescTile<T, D>;
  constexpr int VPC = DT::VPC;
  const int lane = threadIdx.x & 63;
  const int chunk = lane % DT::CPR;
  const int row0 = lane / DT::CPR;
  if constexpr (std::is_same<T, bf16_t>::value) {
    // Two channels per 32-bit word: packed 16-bit order keys and packed
    // 16-bit min / max, then lane swaps across the rows of a chunk.
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = 0xffffffffu;
      hi[e] = 0u;
    }
#pragma unroll
    for (int k = 0; k < DT::NLD; ++k) {
      if (row0 + k * DT::RPI < valid_rows) {
        const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t kk = __builtin_bit_cast(uint32_t, bf16x2_order_key(w[e]));
          lo[e] = pk_min_u16(lo[e], kk);
          hi[e] = pk_max_u16(hi[e], kk);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = rows_reduce<true>(lo[e], DT::CPR);
      hi[e] = rows_reduce<false>(hi[e], DT::CPR);
    }
    if (row0 == 0) {
      uint32_t wl[4], wh[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wl[e] = bf16x2_from_order_key(__builtin_bit_cast(ushort2_t, lo[e]));
        wh[e] = bf16x2_from_order_key(__builtin_bit_cast(ushort2_t, hi[e]));
      }
      *reinterpret_cast<uint4*>(dst + chunk * VPC) = make_uint4(wl[0], wl[1], wl[2], wl[3]);
      *reinterpret_cast<uint4*>(dst + D + chunk * VPC) = make_uint4(wh[0], wh[1], wh[2], wh[3]);
    }
  } else {
    uint32_t lo[VPC], hi[VPC];
#pragma unroll
    for (int e = 0; e < VPC; ++e) {
      lo[e] = 0xffffffffu;
      hi[e] = 0u;
    }
#pragma unroll
    for (int k = 0; k < DT::NLD; ++k) {
      if (row0 + k * DT::RPI < valid_rows) {
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
    for (int off = DT::CPR; off < 64; off <<= 1) {
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
}

template <typename T, int D>
__device__ __forceinline__ void descriptor_unit(const T* __restrict__ src, T* __restrict__ dst, int valid_rows) {
  uint4 v[DescTile<T, D>::NLD];
  descriptor_load<T, D>(src, v);
  descriptor_reduce<T, D>(v, dst, valid_rows);
}

}  // namespace resa
