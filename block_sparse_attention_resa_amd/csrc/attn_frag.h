// MFMA operand fragments for one 16-token KV block, shared by the decode
// and rectification kernels.
//
// Score tile: S^T (16 tokens x 16 query columns) = K . Q^T.
//   A = K     : lane l holds token l%16 and a slice of channels;
//   B = Q^T   : lane l holds query column l%16 and the same channel slice
//               (the contraction index is permuted identically in A and B,
//               which leaves the product unchanged);
//   C = S^T   : lane l holds tokens 4*(l/16)+e, e = 0..3, of column l%16.
// Output tile: O^T (16 channels x 16 query columns) += V^T . P^T.
//   A = V^T   : lane l holds channel 16*t + l%16, tokens 4*(l/16)+e, read as
//               one 8-byte (bf16) or 16-byte (fp32) load from the
//               channel-major value block;
//   B = P^T   : lane l holds tokens 4*(l/16)+e of column l%16, i.e. exactly
//               the C layout of the score tile, so P stays in registers;
//   C = O^T   : lane l holds channels 16*t + 4*(l/16)+e of column l%16.
// bf16 uses v_mfma_f32_16x16x32_bf16 for scores and
// v_mfma_f32_16x16x16_bf16 for the output (P split into a bf16 high part
// and a bf16 residual); fp32 uses v_mfma_f32_16x16x4_f32 for both.
#pragma once

#include "resa_internal.h"

namespace resa {

typedef __attribute__((ext_vector_type(2))) float float2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;


// Maximum over the four lanes of a score-tile column (lanes l, l ^ 16,
// l ^ 32, l ^ 48) with the lane-swap instructions: after a swap of the two
// 32-lane halves (then of neighbouring 16-lane rows) between two copies of
// the value, each lane holds its own value in one copy and its partner's in
// the other.
__device__ __forceinline__ float quad_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <typename T, int D>
struct Frag;

template <int D>
struct Frag<bf16_t, D> {
  static constexpr int KK = D / 32;  // QK^T instructions per block
  static constexpr int NT = D / 16;  // output channel tiles
  struct Q {
    uint4 v[KK];
  };
  struct KV {
    uint4 k[KK];
    uint2 v[NT];
  };
  // Q^T operand for heads < G (zeros for padding columns).
  __device__ static void load_q(Q& q, const bf16_t* qg, int col, int quad, int G) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      q.v[kk] = col < G ? *reinterpret_cast<const uint4*>(qg + (size_t)col * D + quad * 8 * KK + 8 * kk)
                        : make_uint4(0, 0, 0, 0);
  }
  // Q^T operand from an explicit query row pointer (zeros when !valid).
  __device__ static void load_q_row(Q& q, const bf16_t* row, int quad, bool valid) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      q.v[kk] = valid ? *reinterpret_cast<const uint4*>(row + quad * 8 * KK + 8 * kk) : make_uint4(0, 0, 0, 0);
  }
  __device__ static void load_kv(KV& f, const bf16_t* kb, const bf16_t* vb, int col, int quad) {
    const uint4* kp = reinterpret_cast<const uint4*>(kb + (size_t)col * D + quad * 8 * KK);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) f.k[kk] = kp[kk];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      f.v[t] = *reinterpret_cast<const uint2*>(vb + (size_t)(16 * t + col) * kBlock + 4 * quad);
  }
  __device__ static floatx4_t qk(const KV& f, const Q& q) {
    floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f.k[kk]),
                                                  __builtin_bit_cast(bf16x8_t, q.v[kk]), s, 0, 0, 0);
    return s;
  }
  // Zero the value operand entries of tokens e with bit e of `keep` clear.
  __device__ static void mask_v(KV& f, unsigned keep) {
    const uint32_t m0 = (keep & 1u ? 0xffffu : 0u) | (keep & 2u ? 0xffff0000u : 0u);
    const uint32_t m1 = (keep & 4u ? 0xffffu : 0u) | (keep & 8u ? 0xffff0000u : 0u);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f.v[t].x &= m0;
      f.v[t].y &= m1;
    }
  }
  __device__ static void pv(floatx4_t* acc, const KV& f, const float* p) {
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // bf16 high parts and the bf16 of the residuals, two per instruction
      const bf16x2_t hi = __builtin_convertvector(float2_t{p[2 * h], p[2 * h + 1]}, bf16x2_t);
      const float2_t hf = __builtin_convertvector(hi, float2_t);
      const bf16x2_t lo = __builtin_convertvector(float2_t{p[2 * h] - hf.x, p[2 * h + 1] - hf.y}, bf16x2_t);
      hw[h] = __builtin_bit_cast(uint32_t, hi);
      lw[h] = __builtin_bit_cast(uint32_t, lo);
    }
    const uint2 ph = make_uint2(hw[0], hw[1]);
    const uint2 pl = make_uint2(lw[0], lw[1]);
    const short4_t bh = __builtin_bit_cast(short4_t, ph);
    const short4_t bl = __builtin_bit_cast(short4_t, pl);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const short4_t a = __builtin_bit_cast(short4_t, f.v[t]);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bh, acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bl, acc[t], 0, 0, 0);
    }
  }
};

template <int D>
struct Frag<float, D> {
  static constexpr int KK = D / 4;
  static constexpr int NT = D / 16;
  struct Q {
    float v[KK];
  };
  struct KV {
    float k[KK];
    uint4 v[NT];
  };
  __device__ static void load_q(Q& q, const float* qg, int col, int quad, int G) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) q.v[kk] = col < G ? qg[(size_t)col * D + quad * KK + kk] : 0.f;
  }
  __device__ static void load_q_row(Q& q, const float* row, int quad, bool valid) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) q.v[kk] = valid ? row[quad * KK + kk] : 0.f;
  }
  __device__ static void load_kv(KV& f, const float* kb, const float* vb, int col, int quad) {
    const uint4* kp = reinterpret_cast<const uint4*>(kb + (size_t)col * D + quad * KK);
#pragma unroll
    for (int c = 0; c < KK / 4; ++c) {
      const uint4 x = kp[c];
      f.k[4 * c] = __uint_as_float(x.x);
      f.k[4 * c + 1] = __uint_as_float(x.y);
      f.k[4 * c + 2] = __uint_as_float(x.z);
      f.k[4 * c + 3] = __uint_as_float(x.w);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
      f.v[t] = *reinterpret_cast<const uint4*>(vb + (size_t)(16 * t + col) * kBlock + 4 * quad);
  }
  __device__ static floatx4_t qk(const KV& f, const Q& q) {
    floatx4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) s = __builtin_amdgcn_mfma_f32_16x16x4f32(f.k[kk], q.v[kk], s, 0, 0, 0);
    return s;
  }
  __device__ static void mask_v(KV& f, unsigned keep) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f.v[t].x = keep & 1u ? f.v[t].x : 0u;
      f.v[t].y = keep & 2u ? f.v[t].y : 0u;
      f.v[t].z = keep & 4u ? f.v[t].z : 0u;
      f.v[t].w = keep & 8u ? f.v[t].w : 0u;
    }
  }
  __device__ static void pv(floatx4_t* acc, const KV& f, const float* p) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.v[t].x), p[0], acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.v[t].y), p[1], acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.v[t].z), p[2], acc[t], 0, 0, 0);
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.v[t].w), p[3], acc[t], 0, 0, 0);
    }
  }
};

}  // namespace resa
