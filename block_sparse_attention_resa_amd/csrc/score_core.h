// Group block scores (Eq 4 of the "Rectified Sparse Attention" analysis
// page, paper-graph-ui, §3.4.1): descriptor chunk loads and the DPP group
// sums of the scoring kernel.
//
// For one GQA group the score of block b sums, over the group's query heads
// j and channels c, max(q_jc * lo_bc, q_jc * hi_bc).  Because hi >= lo this
// equals sum_c P_c * hi_bc + N_c * lo_bc with P_c = sum_j max(q_jc, 0) and
// N_c = sum_j min(q_jc, 0) (mean-pooled query: the positive / negative part
// of the mean), so 2 d threads fold the group's queries into (N, P) once and
// every lane then streams its chunk of the descriptors with one fused
// multiply-add per stored value.  A descriptor (2 x d values) is split into
// 32-byte chunks; CH consecutive lanes own one descriptor and combine their
// partial sums with DPP row rotations.  All descriptor loads of the slice
// are in flight at once.
#pragma once

#include "resa_internal.h"

namespace resa {


template <typename T>
struct ChunkLoad;

template <>
struct ChunkLoad<bf16_t> {
  static constexpr int kVals = 16;  // bf16 values per 32-byte chunk
  using Pair = uint32_t;            // two consecutive channels
  __device__ static void unpack_pair(uint32_t w, float& a, float& b) {
    a = bf16_lo_f32(w);
    b = bf16_hi_f32(w);
  }
  __device__ static void unpack(const uint4& a, const uint4& b, float* f) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f[2 * e] = bf16_lo_f32(w[e]);
      f[2 * e + 1] = bf16_hi_f32(w[e]);
    }
  }
};

template <>
struct ChunkLoad<float> {
  static constexpr int kVals = 8;
  using Pair = uint2;
  __device__ static void unpack_pair(uint2 w, float& a, float& b) {
    a = __uint_as_float(w.x);
    b = __uint_as_float(w.y);
  }
  __device__ static void unpack(const uint4& a, const uint4& b, float* f) {
    f[0] = __uint_as_float(a.x);
    f[1] = __uint_as_float(a.y);
    f[2] = __uint_as_float(a.z);
    f[3] = __uint_as_float(a.w);
    f[4] = __uint_as_float(b.x);
    f[5] = __uint_as_float(b.y);
    f[6] = __uint_as_float(b.z);
    f[7] = __uint_as_float(b.w);
  }
};


__device__ __forceinline__ float to_f32(const bf16_t& x) { return __uint_as_float((uint32_t)x.bits << 16); }
__device__ __forceinline__ float to_f32(const float& x) { return x; }

// Sum over aligned groups of N lanes, the result in every lane of the group.
// N = 16 (a whole DPP row) and 32 use row rotations (and one 16-lane swap),
// which stay in the vector ALU; other N use lane shuffles.
template <int N>
__device__ __forceinline__ float row_rot_add(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));  // row_ror:8
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));  // row_ror:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));  // row_ror:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));  // row_ror:1
  return x;
}
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N == 16) {
    return row_rot_add<16>(x);
  } else if constexpr (N == 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return row_rot_add<16>(__uint_as_float(a[0]) + __uint_as_float(a[1]));
  } else {
#pragma unroll
    for (int off = N / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
  }
}

}  // namespace resa
