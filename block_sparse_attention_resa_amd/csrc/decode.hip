// Split-K flash decode over a block list: group block sparse attention
// (selected blocks) and dense attention (all blocks).
//
// "Rectified Sparse Attention" analysis page (paper-graph-ui): §3.4.1 Eq 1
// (GQA attention) and Eq 2 (attention restricted to the selected blocks,
// masked positions excluded from the softmax), §3.4.4 (split execution over
// the GPU with partial log-sum-exp results combined afterwards, and one load
// of each KV block per GQA group shared by all of its query heads).
//
// Work decomposition.  Grid (splits, KV heads, requests).  The block list of
// one (request, KV head) is cut into `splits` equal ranges, one per workgroup
// of 8 wavefronts (about one workgroup per CU); the wavefronts take
// consecutive sub-ranges and each keeps its own online-softmax state, merged
// through LDS into one partial (m, l, o) per query head.  A second kernel
// merges the splits' partials with their log-sum-exp weights.
//
// Matrix cores.  Per 16-token block a wavefront computes the transposed score
// tile S^T (16 tokens x 16 query-head columns, g <= 16 of them used) as
// K . Q^T with v_mfma_f32_16x16x32_bf16 (16x16x4_f32 for fp32 caches), then
// O^T (channels x heads) += V^T . P^T with v_mfma_f32_16x16x16_bf16.  The S^T
// accumulator layout (lane l: tokens 4*(l/16)+e, column l%16) is exactly the
// B-operand layout of the second product, so P never leaves registers.  The
// value pool stores each block channel-major ([d][16]), which makes the
// V^T A-operand four consecutive tokens of one channel: one 8-byte load.
// Keys are token-major, and a lane's four 16-byte K loads are contiguous
// because the contraction index is permuted identically in K and Q.
//
// P is split into a bf16 high part and a bf16 residual (p - hi) and both are
// multiplied by V, so the probabilities enter the matrix product with about
// 16 significant bits; a plain bf16 P would contribute a relative error of
// about 1e-3 to the output on its own.
//
// Data movement.  Every byte of K and V is used by exactly one wavefront, so
// operands go from HBM straight into VGPRs in MFMA layout; the next chunk's
// loads are issued before the current chunk is computed.  Block ids and
// physical ids for up to 64 positions are fetched with one vector load each
// and broadcast with readlane.  Rows past the sequence end are masked by
// selection (score -> -inf, value -> 0), so any bit pattern there is harmless.
#include "attn_frag.h"
#include "resa_internal.h"

namespace resa {
namespace {

constexpr int kChunk = 2;  // blocks per pipelined chunk

template <typename T, int D>
struct Chunk {
  typename Frag<T, D>::KV f[kChunk];
  int blk[kChunk];  // logical block id, -1 = empty slot
};

// Query columns merged per LDS pass inside a workgroup (LDS stays ~34 KiB).
template <int NW>
struct DecodeShape {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kCols = NW <= 8 ? 8 : 4;
};

template <typename T, int D, bool SPARSE, int NW>
__global__ __launch_bounds__(64 * NW) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k_pool, const T* __restrict__ v_pool,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_cnt, int max_sel, float* __restrict__ part_o, float* __restrict__ part_ml,
    int H, int G, int max_blocks, int num_pool_blocks, int S, float scale_log2) {
  using F = Frag<T, D>;
  using SH = DecodeShape<NW>;
  constexpr int NT = F::NT;
  constexpr int NTH = SH::kThreads;
  constexpr int CG = SH::kCols;
  __shared__ float s_acc[NW][CG][D + 4];
  __shared__ float s_m[NW][16];
  __shared__ float s_l[NW][16];

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
  // block-id loads below do not wait for sel_cnt; n only trims the range.
  const int beg = s * bps;
  const int per = (bps + NW - 1) / NW;
  const int cap = SPARSE ? max_sel : max_blocks;
  const int wb = beg + wave * per;
  const int we_cap = min(min(beg + bps, cap), wb + per);  // positions readable without n
  const int we = min(we_cap, n);

  typename F::Q qf;
  F::load_q(qf, q + ((size_t)r * H + i) * G * D, col, quad, G);

  float m_run = -INFINITY;
  float l_run = 0.f;
  floatx4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int32_t* sel_row = SPARSE ? sel_idx + ((size_t)r * H + i) * max_sel : nullptr;
  const int32_t* tab_row = table + (size_t)r * max_blocks;
  const size_t head_stride = (size_t)kBlock * D;  // elements per (block, head) tile

  for (int g0 = wb; g0 < we_cap; g0 += 64) {
    // Ids and physical blocks of up to 64 positions, fetched before n and L
    // are known (every address stays inside the list and the table); a block
    // id past the sequence end only contributes masked rows.
    int my_blk = 0, my_pid = 0;
    if (g0 + lane < we_cap) {
      my_blk = SPARSE ? clampi(sel_row[g0 + lane], 0, max_blocks - 1) : g0 + lane;
      my_pid = clampi(tab_row[my_blk], 0, num_pool_blocks - 1);
    }
    if (g0 >= we) break;
    const int gn = min(64, we - g0);

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

  // ---- merge the wavefronts of this workgroup into one partial (m, l, o) per column
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (quad == 0) {
    s_m[wave][col] = m_run;
    s_l[wave][col] = l_run;
  }
  const size_t prow = ((size_t)r * H + i) * S + s;  // partial row of this workgroup
  for (int c0 = 0; c0 < G; c0 += CG) {
    if (col >= c0 && col < c0 + CG) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        *reinterpret_cast<floatx4_t*>(&s_acc[wave][col - c0][16 * t + 4 * quad]) = acc[t];
    }
    __syncthreads();
    const int ncols = min(CG, G - c0);
    for (int idx = threadIdx.x; idx < ncols * D; idx += NTH) {
      const int jl = idx / D;
      const int j = c0 + jl;
      const int c = idx % D;
      float mw = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) mw = fmaxf(mw, s_m[w][j]);
      float o = 0.f, l = 0.f;
      if (mw != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float wt = exp2f(s_m[w][j] - mw);
          o += wt * s_acc[w][jl][c];
          l += wt * s_l[w][j];
        }
      }
      part_o[(prow * G + j) * D + c] = o;
      if (c == 0) {
        part_ml[(prow * G + j) * 2] = mw;
        part_ml[(prow * G + j) * 2 + 1] = l;
      }
    }
    __syncthreads();
  }

}

// Log-sum-exp merge of split partials:
//   out[c] = sum_s 2^(m_s - m) o_s[c] / sum_s 2^(m_s - m) l_s,  m = max_s m_s.
// kMergeParts consecutive lanes (one DPP row) share one output float4: lane
// part p folds splits p, p + kMergeParts, p + 2 kMergeParts, ..., a batch of
// kMergeBatch at a time with all loads issued first, each batch weighted
// against its own maximum (independent exponentials rather than a chain).
// The sixteen lanes then agree on the row maximum by DPP exchanges, scale
// their sums once, and add them by DPP exchanges (partners at xor 1 and 2,
// then the half-row and row mirrors, which pair lanes of groups already
// holding equal values).  Floating-point addition is commutative, so both
// partners of an exchange form the same value; with no barrier, no LDS and
// a fixed order of every sum, the result is deterministic.
constexpr int kMergeThreads = 256;
constexpr int kMergeParts = 16;  // lanes per output float4
constexpr int kMergeBatch = 4;   // splits per lane per batch of loads
constexpr long long kMergeMaxGrid = 1 << 20;  // workgroups of one merge launch

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Maximum, then sum, over the sixteen lanes of a DPP row.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<0xb1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f32<0x4e>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f32<0x141>(x));  // row_half_mirror
  return fmaxf(x, dpp_f32<0x140>(x));  // row_mirror
}
template <int CTRL>
__device__ __forceinline__ void row16_add_step(float& l, floatx4_t& o) {
  l += dpp_f32<CTRL>(l);
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] += dpp_f32<CTRL>(o[e]);
}

template <int D>
__device__ __forceinline__ void merge_one(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                                          float* __restrict__ out, int H, int G, int S, int rows_per_head,
                                          int row_stride_out, long long g) {
  constexpr int C4 = D / 4;
  const int part = (int)(g % kMergeParts);
  const int c4 = (int)((g / kMergeParts) % C4);
  const long long grow = g / (kMergeParts * C4);  // (r, i, row) flattened
  const int row = (int)(grow % rows_per_head);
  const long long ri = grow / rows_per_head;  // r * H + i
  const size_t base = (size_t)ri * S;

  float m_run = -INFINITY, l_run = 0.f;
  floatx4_t o_run = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = part; s0 < S; s0 += kMergeParts * kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch];
    floatx4_t ov[kMergeBatch];
#pragma unroll
    for (int b = 0; b < kMergeBatch; ++b) {
      const int sp = s0 + b * kMergeParts;
      const bool ok = sp < S;
      const size_t pr = (base + (ok ? sp : 0)) * rows_per_head + row;
      const float2 ml = *reinterpret_cast<const float2*>(part_ml + pr * 2);
      mv[b] = ok ? ml.x : -INFINITY;
      lv[b] = ok ? ml.y : 0.f;
      ov[b] = *reinterpret_cast<const floatx4_t*>(part_o + pr * D + 4 * c4);
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
  const float m_all = row16_max(m_run);
  const float m_use = m_all == -INFINITY ? 0.f : m_all;
  const float w = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_use);
  float l_sum = l_run * w;
  floatx4_t o_sum = o_run * w;
  row16_add_step<0xb1>(l_sum, o_sum);
  row16_add_step<0x4e>(l_sum, o_sum);
  row16_add_step<0x141>(l_sum, o_sum);
  row16_add_step<0x140>(l_sum, o_sum);
  if (part == 0) {
    const long long r = ri / H;
    const int i = (int)(ri % H);
    const int j = row % G;
    const int t = row / G;
    float* dst = out + (((size_t)r * row_stride_out + t) * H * G + (size_t)i * G + j) * D + 4 * c4;
    const float inv = l_sum > 0.f ? 1.f / l_sum : 0.f;
    *reinterpret_cast<floatx4_t*>(dst) = o_sum * inv;
  }
}

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float* __restrict__ part_o,
                                                              const float* __restrict__ part_ml,
                                                              float* __restrict__ out, int H, int G, int S,
                                                              int rows_per_head, int row_stride_out,
                                                              long long total_rows) {
  constexpr int C4 = D / 4;  // float4 per output row
  // 64-bit thread index; the grid strides over the rows when it is capped
  // (rows * C4 * kMergeParts may exceed 2^31).  The stride is a multiple of
  // kMergeParts, so the sixteen lanes of a DPP row always share one row and
  // leave the loop together.
  const long long stride = (long long)gridDim.x * kMergeThreads;
  for (long long g = (long long)blockIdx.x * kMergeThreads + threadIdx.x; g < total_rows * C4 * kMergeParts;
       g += stride)
    merge_one<D>(part_o, part_ml, out, H, G, S, rows_per_head, row_stride_out, g);
}

template <typename T, int D, int NW>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)a.splits, (unsigned)a.H, (unsigned)a.R);
  dim3 block(64 * NW);
  if (a.sel_idx) {
    hipLaunchKernelGGL((decode_kernel<T, D, true, NW>), grid, block, 0, stream, static_cast<const T*>(a.q),
                       static_cast<const T*>(a.k_pool), static_cast<const T*>(a.v_pool), a.table, a.seq_lens,
                       a.sel_idx, a.sel_cnt, a.max_sel, a.part_o, a.part_ml, a.H, a.G, a.max_blocks,
                       a.num_pool_blocks, a.splits, a.scale_log2);
  } else {
    hipLaunchKernelGGL((decode_kernel<T, D, false, NW>), grid, block, 0, stream, static_cast<const T*>(a.q),
                       static_cast<const T*>(a.k_pool), static_cast<const T*>(a.v_pool), a.table, a.seq_lens,
                       nullptr, nullptr, 0, a.part_o, a.part_ml, a.H, a.G, a.max_blocks, a.num_pool_blocks,
                       a.splits, a.scale_log2);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(a.part_o, a.part_ml, a.out, a.R, a.H, a.G, a.D, a.splits, a.G, 1, stream);
}

}  // namespace

hipError_t launch_merge(const float* part_o, const float* part_ml, float* out, int R, int H, int G, int D, int S,
                        int rows_per_head, int row_stride_out, hipStream_t stream) {
  const long long rows = (long long)R * H * rows_per_head;
  const long long threads = rows * (D / 4) * kMergeParts;
  long long wgs = (threads + kMergeThreads - 1) / kMergeThreads;
  if (wgs > kMergeMaxGrid) wgs = kMergeMaxGrid;  // larger merges stride over the rows
  const dim3 grid((unsigned)wgs);
  if (D == 128)
    hipLaunchKernelGGL((merge_kernel<128>), grid, dim3(kMergeThreads), 0, stream, part_o, part_ml, out, H, G, S,
                       rows_per_head, row_stride_out, rows);
  else
    hipLaunchKernelGGL((merge_kernel<64>), grid, dim3(kMergeThreads), 0, stream, part_o, part_ml, out, H, G, S,
                       rows_per_head, row_stride_out, rows);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  // fp32 fragments need twice the registers: 4 wavefronts per workgroup keeps them spill-free
  if (a.dtype == 0)
    return a.D == 128 ? launch_decode_t<bf16_t, 128, kDecodeWaves>(a, stream)
                      : launch_decode_t<bf16_t, 64, kDecodeWaves>(a, stream);
  return a.D == 128 ? launch_decode_t<float, 128, 4>(a, stream) : launch_decode_t<float, 64, 4>(a, stream);
}

}  // namespace resa
