// Group block scores (Eq 4 of the "Rectified Sparse Attention" analysis
// page, paper-graph-ui, §3.4.1): descriptor chunk loads, the DPP group sums,
// and the scoring of one slice of consecutive blocks by a workgroup.
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

#include "select_core.h"

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

// One slice: blocks sb0 + u * BPP + (thread / CH), u < U, of request r and
// KV head i.  After the call, every lane holds the order key of its group's
// block u in key[u] (blk[u] = the block id; the key is meaningful only for
// blocks below M), the slice's candidate key range folded over the lanes
// into kmin / kmax (candidates: blocks below C), and the keys of blocks below
// M are stored in key_row with device-scope stores (score_row, if not null,
// receives the fp32 scores).  s_coef is 2 d floats of LDS; the call contains
// one workgroup barrier.
template <typename T, int D, int MAXG, int NT, int UMAX>
struct SliceScore {
  static constexpr int VPL = ChunkLoad<T>::kVals;  // values of a lane's 32-byte descriptor chunk
  static constexpr int CH = 2 * D / VPL;           // lanes per descriptor
  static constexpr int HALF = CH / 2;              // lanes per descriptor row
  static constexpr int BPP = NT / CH;              // blocks per pass of the workgroup
  uint32_t key[UMAX];
  int blk[UMAX];
  uint32_t kmin, kmax;

  __device__ __forceinline__ void run(const T* __restrict__ q_group, const T* desc, const int32_t* __restrict__ tab_row,
                                      int M, int C, int sb0, int U, int H, int i, int G, int mode, int max_blocks,
                                      int num_pool_blocks, uint32_t* key_row, float* score_row, float* s_coef) {
    static_assert(2 * D <= NT, "one folding thread per coefficient");
    const int t = threadIdx.x;
    const int grp = t / CH;
    const int lg = t % CH;
    const int part = lg / HALF;  // 0: min row, 1: max row
    const int c0 = (lg % HALF) * VPL;
    // Load order matters: the in-order vector-memory counter makes a wait for
    // a load also wait for every load issued before it.  The table entries
    // (for the descriptor addresses) go out first, then the group's queries,
    // then the descriptor loads; no descriptor at or past M is read.
    int pid[UMAX];
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
      blk[u] = sb0 + u * BPP + grp;
      pid[u] = (u < U && blk[u] < max_blocks) ? tab_row[blk[u]] : 0;
    }
    // Thread t < 2 d folds channel t % d of the group's queries into one
    // coefficient (row t / d: N for the min row, P for the max row); all G
    // values are loaded before any is used (rows past G re-read row G - 1 and
    // are ignored).
    const bool folder = t < 2 * D;
    const int fc = t % D;
    const int frow = t / D;
    float qv[MAXG];
#pragma unroll
    for (int j = 0; j < MAXG; ++j) qv[j] = folder ? to_f32(q_group[(size_t)min(j, G - 1) * D + fc]) : 0.f;
    uint4 buf[UMAX][2];
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
      if (u < U && blk[u] < M) {
        const int p = clampi(pid[u], 0, num_pool_blocks - 1);
        const uint4* src = reinterpret_cast<const uint4*>(desc + (((size_t)p * H + i) * 2 + part) * D + c0);
        buf[u][0] = src[0];
        buf[u][1] = src[1];
      } else {
        buf[u][0] = make_uint4(0u, 0u, 0u, 0u);
        buf[u][1] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (folder) {
      // sum over the group's heads in head order
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < MAXG; ++j) {
        if (j < G) {
          if (mode == 0) acc += frow ? fmaxf(qv[j], 0.f) : fminf(qv[j], 0.f);
          else acc += qv[j];
        }
      }
      if (mode != 0) {
        const float m = acc / (float)G;
        acc = frow ? fmaxf(m, 0.f) : fminf(m, 0.f);
      }
      s_coef[t] = acc;
    }
    __syncthreads();
    float coef[VPL];
#pragma unroll
    for (int v = 0; v < VPL; v += 4) {
      const floatx4_t c4 = *reinterpret_cast<const floatx4_t*>(&s_coef[part * D + c0 + v]);
      coef[v] = c4[0];
      coef[v + 1] = c4[1];
      coef[v + 2] = c4[2];
      coef[v + 3] = c4[3];
    }
    kmin = 0xffffffffu;
    kmax = 0u;
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
      key[u] = 0u;
      if (u < U) {  // uniform
        float vals[VPL];
        ChunkLoad<T>::unpack(buf[u][0], buf[u][1], vals);
        float acc = 0.f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) acc = fmaf(coef[v], vals[v], acc);
        acc = group_sum<CH>(acc);
        key[u] = f32_order_key(acc);
        if (lg == 0 && blk[u] < M) {
          store_agent(key_row + blk[u], key[u]);
          if (score_row) score_row[blk[u]] = acc;
        }
        if (blk[u] < C) {
          kmin = min(kmin, key[u]);
          kmax = max(kmax, key[u]);
        }
      }
    }
  }
};

}  // namespace resa
