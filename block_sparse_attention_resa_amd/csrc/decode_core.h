// Split-K decode attention over a list of KV blocks: the per-wavefront
// online-softmax loop, the merge of a workgroup's wavefronts into one
// partial (m, l, o) per query head, and the log-sum-exp merge of partials.
//
// "Rectified Sparse Attention" analysis page (paper-graph-ui): §3.4.1 Eq 1
// (GQA attention) and Eq 2 (attention restricted to the selected blocks,
// masked positions excluded from the softmax), §3.4.4 (split execution with
// partial log-sum-exp results combined afterwards, one load of each KV block
// per GQA group shared by all of its query heads).
//
// Matrix cores.  Per 16-token block a wavefront computes the transposed score
// tile S^T (16 tokens x 16 query-head columns, g <= 16 of them used) as
// K . Q^T with v_mfma_f32_16x16x32_bf16 (16x16x4_f32 for fp32 caches), then
// O^T (channels x heads) += V^T . P^T with v_mfma_f32_16x16x16_bf16
// (attn_frag.h).  The S^T accumulator layout is exactly the B-operand layout
// of the second product, so P never leaves registers, and P enters the
// product as a bf16 high part plus a bf16 residual.
//
// Data movement.  Every byte of K and V is used by exactly one wavefront, so
// operands go from HBM straight into VGPRs in MFMA layout; the next pair of
// blocks is requested before the current pair is computed.  Block ids and
// physical ids for up to 64 list positions are fetched with one vector load
// each and broadcast with readlane.  Rows past the sequence end are masked
// (score -> -inf, value -> 0), so any bit pattern there is harmless.
#pragma once

#include "attn_frag.h"
#include "select_core.h"

namespace resa {

constexpr int kChunk = 2;  // blocks per pipelined chunk

template <typename T, int D>
struct Chunk {
  typename Frag<T, D>::KV f[kChunk];
  int blk[kChunk];  // logical block id, -1 = empty slot
};

// Online-softmax state of one wavefront over the 16 query columns of one KV
// head: running maximum (log2 units), running sum and O^T accumulators.
template <typename T, int D>
struct WaveAttn {
  using F = Frag<T, D>;
  static constexpr int NT = F::NT;
  float m_run, l_run;
  floatx4_t acc[NT];

  __device__ __forceinline__ void init() {
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Folds the blocks at list positions [p0, p_end) into the state.  Positions
  // [p0, p_cap) may be read before p_end is known (p_end <= p_cap), so the id
  // loads need not wait for the list length.  id_at(pos) returns the logical
  // block id at a position; it is clamped into [0, max_blocks).
  template <class IdAt>
  __device__ __forceinline__ void run(IdAt id_at, int p0, int p_cap, int p_end, const typename F::Q& qf,
                                      const T* __restrict__ k_pool, const T* __restrict__ v_pool,
                                      const int32_t* __restrict__ tab_row, int H, int i, int L, int max_blocks,
                                      int num_pool_blocks, float scale_log2) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;
    const int quad = lane >> 4;
    const size_t head_stride = (size_t)kBlock * D;  // elements per (block, head) tile
    for (int g0 = p0; g0 < p_cap; g0 += 64) {
      int my_blk = 0, my_pid = 0;
      if (g0 + lane < p_cap) {
        my_blk = clampi(id_at(g0 + lane), 0, max_blocks - 1);
        my_pid = clampi(tab_row[my_blk], 0, num_pool_blocks - 1);
      }
      if (g0 >= p_end) break;
      const int gn = min(64, p_end - g0);

      auto load_chunk = [&](Chunk<T, D>& c, int at) {
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
          if (at + j < gn) {
            const int b = __builtin_amdgcn_readlane(my_blk, at + j);
            const int p = __builtin_amdgcn_readlane(my_pid, at + j);
            const size_t tile = ((size_t)p * H + i) * head_stride;
            F::load_kv(c.f[j], k_pool + tile, v_pool + tile, col, quad);
            c.blk[j] = b;
          } else {
            c.blk[j] = -1;
          }
        }
      };

      auto compute_chunk = [&](Chunk<T, D>& c) {
        floatx4_t sv[kChunk];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
          if (c.blk[j] >= 0) {
            sv[j] = F::qk(c.f[j], qf);
            const int tok0 = c.blk[j] * kBlock + 4 * quad;
            const bool partial = c.blk[j] * kBlock + kBlock > L;
            unsigned keep = 0xfu;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bool ok = !partial || tok0 + e < L;
              sv[j][e] = ok ? sv[j][e] * scale_log2 : -INFINITY;
              keep &= ok ? 0xfu : ~(1u << e);
              mx = fmaxf(mx, sv[j][e]);
            }
            if (partial) F::mask_v(c.f[j], keep);
          } else {
            sv[j] = floatx4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
          }
        }
        mx = quad_max(mx);
        const float m_new = fmaxf(m_run, mx);
        // With nothing valid seen yet (m_new = -inf) keep the state unchanged;
        // otherwise alpha = 0 on the first chunk (m_run = -inf).
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] *= alpha;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) {
          if (c.blk[j] >= 0) {
            float p[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              p[e] = __builtin_amdgcn_exp2f(sv[j][e] - m_use);
              l_run += p[e];
            }
            F::pv(acc, c.f[j], p);
          }
        }
      };

      Chunk<T, D> cur;
      load_chunk(cur, 0);
      for (int at = 0; at < gn; at += kChunk) {
        Chunk<T, D> nxt;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) nxt.blk[j] = -1;
        if (at + kChunk < gn) load_chunk(nxt, at + kChunk);
        compute_chunk(cur);
        cur = nxt;
      }
    }
  }
};

// LDS of the merge of NW wavefronts (query columns merged per pass: 8 for up
// to 8 wavefronts, 4 beyond).
template <int NW, int D>
struct MergeLds {
  static constexpr int kCols = NW <= 8 ? 8 : 4;
  float acc[NW][kCols][D + 4];
  float m[NW][16];
  float l[NW][16];
};

// Merges the NW wavefronts' states into one partial per query column j < G:
// part_o[j * D + c] = sum_w 2^(m_w - m) o_w[c], part_ml[2 j] = m = max_w m_w,
// part_ml[2 j + 1] = sum_w 2^(m_w - m) l_w.  With `out` not null (the row's
// only split) it writes the normalised output out[j * D + c] = part_o / l
// instead, the same operations as the merge of a single partial.  Contains
// workgroup barriers.
template <typename T, int D, int NW>
__device__ __forceinline__ void wg_merge_store(WaveAttn<T, D>& st, MergeLds<NW, D>& ml, int G,
                                               float* __restrict__ part_o, float* __restrict__ part_ml,
                                               float* __restrict__ out = nullptr) {
  constexpr int NT = WaveAttn<T, D>::NT;
  constexpr int CG = MergeLds<NW, D>::kCols;
  constexpr int NTH = 64 * NW;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int quad = lane >> 4;
  float l_run = st.l_run;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (quad == 0) {
    ml.m[wave][col] = st.m_run;
    ml.l[wave][col] = l_run;
  }
  for (int c0 = 0; c0 < G; c0 += CG) {
    if (col >= c0 && col < c0 + CG) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<floatx4_t*>(&ml.acc[wave][col - c0][16 * t + 4 * quad]) = st.acc[t];
    }
    __syncthreads();
    const int ncols = min(CG, G - c0);
    for (int idx = threadIdx.x; idx < ncols * D; idx += NTH) {
      const int jl = idx / D;
      const int j = c0 + jl;
      const int c = idx % D;
      float mw = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) mw = fmaxf(mw, ml.m[w][j]);
      float o = 0.f, l = 0.f;
      if (mw != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float wt = exp2f(ml.m[w][j] - mw);
          o += wt * ml.acc[w][jl][c];
          l += wt * ml.l[w][j];
        }
      }
      if (out) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        out[j * D + c] = o * inv;
      } else {
        part_o[j * D + c] = o;
        if (c == 0) {
          part_ml[j * 2] = mw;
          part_ml[j * 2 + 1] = l;
        }
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------- partial merge
//
//   out[c] = sum_s 2^(m_s - m) o_s[c] / sum_s 2^(m_s - m) l_s,  m = max_s m_s.
// P consecutive lanes (P = 1, 2, 4, 8 or 16, within one DPP row) share one
// output float4: lane part p folds partials p, p + P, p + 2 P, ..., a batch
// of kMergeBatch at a time with all loads issued first, each batch weighted
// against its own maximum (independent exponentials rather than a chain).
// The launcher picks the smallest P whose lanes take all S partials in one
// batch (16 beyond that).  The P lanes then agree on the group maximum by
// DPP exchanges, scale their sums once, and add them by DPP exchanges
// (partners at xor 1 and 2, then the half-row and row mirrors, which pair
// lanes of groups already holding equal values).  Floating-point addition
// is commutative, so both partners of an exchange form the same value; with
// no barrier, no LDS and a fixed order of every sum, the result is
// deterministic.
constexpr int kMergeMaxParts = 16;  // lanes per output float4, at most
constexpr int kMergeBatch = 4;      // partials per lane per batch of loads

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Maximum over the P lanes of an aligned group, in every lane of it.
template <int P>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (P >= 2) x = fmaxf(x, dpp_f32<0xb1>(x));   // quad_perm [1,0,3,2]
  if constexpr (P >= 4) x = fmaxf(x, dpp_f32<0x4e>(x));   // quad_perm [2,3,0,1]
  if constexpr (P >= 8) x = fmaxf(x, dpp_f32<0x141>(x));  // row_half_mirror
  if constexpr (P >= 16) x = fmaxf(x, dpp_f32<0x140>(x)); // row_mirror
  return x;
}
template <int CTRL>
__device__ __forceinline__ void group_add_step(float& l, floatx4_t& o) {
  l += dpp_f32<CTRL>(l);
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] += dpp_f32<CTRL>(o[e]);
}

// Partials read with ordinary loads.
struct PlainPartials {
  const float* __restrict__ o;
  const float* __restrict__ ml;
  __device__ float2 load_ml(size_t row) const { return *reinterpret_cast<const float2*>(ml + row * 2); }
  __device__ floatx4_t load_o(size_t off) const { return *reinterpret_cast<const floatx4_t*>(o + off); }
};

// One output float4 (lane group of P): S partials of partial row `row` in
// the rows-per-partial layout (partial s, row: s * rows + row), channels
// [4 c4, 4 c4 + 4).  Returns the merged float4 (in every lane of the group).
template <int D, int P, class Parts>
__device__ __forceinline__ floatx4_t merge_float4(const Parts& pp, size_t base, int S, int rows, int row, int c4,
                                                  int part) {
  float m_run = -INFINITY, l_run = 0.f;
  floatx4_t o_run = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = part; s0 < S; s0 += P * kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch];
    floatx4_t ov[kMergeBatch];
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
      const int sp = s0 + b * P;
      const bool ok = sp < S;
      const size_t pr = (base + (ok ? sp : 0)) * rows + row;
      const float2 ml = pp.load_ml(pr);
      mv[b] = ok ? ml.x : -INFINITY;
      lv[b] = ok ? ml.y : 0.f;
      ov[b] = pp.load_o(pr * D + 4 * c4);
    }
    float m_new = m_run;
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) m_new = fmaxf(m_new, mv[b]);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;  // nothing seen yet: every weight is 0
    const float a = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_use);
    l_run *= a;
    o_run *= a;
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
      const float w = mv[b] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv[b] - m_use);
      l_run = fmaf(w, lv[b], l_run);
      o_run += w * ov[b];
    }
    m_run = m_new;
  }
  const float m_all = group_max<P>(m_run);
  const float m_use = m_all == -INFINITY ? 0.f : m_all;
  const float w = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_use);
  float l_sum = l_run * w;
  floatx4_t o_sum = o_run * w;
  if constexpr (P >= 2) group_add_step<0xb1>(l_sum, o_sum);
  if constexpr (P >= 4) group_add_step<0x4e>(l_sum, o_sum);
  if constexpr (P >= 8) group_add_step<0x141>(l_sum, o_sum);
  if constexpr (P >= 16) group_add_step<0x140>(l_sum, o_sum);
  const float inv = l_sum > 0.f ? 1.f / l_sum : 0.f;
  return o_sum * inv;
}

}  // namespace resa
