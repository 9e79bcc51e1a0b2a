// Dense rectification: rewrite the last `chunk` cache positions, refresh the
// descriptors of the blocks they touch, and run causal chunk attention of the
// chunk's queries over the whole rewritten cache.
//
// "Rectified Sparse Attention" analysis page (paper-graph-ui): §3.4.2 (the
// f most recent tokens are re-encoded in one parallel dense pass over the
// entire cache, their cache entries overwritten and the affected block
// descriptors recomputed), §3.4.3 Algorithm 1 (the rectification step of the
// decoding loop) and §3.4.4 (rectification uses a dense attention kernel).
//
// Kernels, in stream order:
//   1. row write: position L - chunk + t of KV head i <- k_new / v_new[r][t][i]
//      (values go into the channel-major value block);
//   2. the descriptor kernel over blocks floor((L - chunk)/16) .. M - 1;
//   3. causal chunk attention.  The chunk's chunk * g query rows of one KV
//      head are the columns of 16-wide MFMA tiles.  bf16 caches: a 512-thread
//      workgroup holds sixteen tiles (256 query rows) and streams one split
//      of the cache through LDS, so every K / V byte is read from HBM once
//      per workgroup.  fp32 caches: a 256-thread workgroup holds four tiles
//      and each wavefront reads its K / V operands directly.  Each query row
//      t masks positions > L - chunk + t; blocks past the workgroup's last
//      visible position are skipped;
//   4. the log-sum-exp merge of the splits (shared with decode).
#include <type_traits>

#include "attn_frag.h"
#include "resa_internal.h"

namespace resa {
namespace {

constexpr int kRectWaves = 4;
constexpr int kRectThreads = 64 * kRectWaves;
constexpr int kRectChunk = 2;

template <typename T>
__global__ void write_rows_kernel(const T* __restrict__ k_new, const T* __restrict__ v_new, T* __restrict__ k_pool,
                                  T* __restrict__ v_pool, const int32_t* __restrict__ table,
                                  const int32_t* __restrict__ seq_lens, int H, int D, int chunk, int max_blocks,
                                  int num_pool_blocks) {
  const int t = blockIdx.x;
  const int r = blockIdx.y;
  const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
  if (L < chunk) return;
  const int pos = L - chunk + t;
  const int row = pos % kBlock;
  const int p = clampi(table[(size_t)r * max_blocks + pos / kBlock], 0, num_pool_blocks - 1);
  for (int idx = threadIdx.x; idx < H * D; idx += blockDim.x) {
    const int i = idx / D;
    const int c = idx % D;
    const size_t src = (((size_t)r * chunk + t) * H + i) * D + c;
    k_pool[(((size_t)p * H + i) * kBlock + row) * D + c] = k_new[src];
    v_pool[(((size_t)p * H + i) * D + c) * kBlock + row] = v_new[src];
  }
}

template <typename T, int D>
struct RChunk {
  typename Frag<T, D>::KV f[kRectChunk];
  int blk[kRectChunk];
};

template <typename T, int D>
__global__ __launch_bounds__(kRectThreads) void rectify_attn_kernel(
    const T* __restrict__ q_chunk, const T* __restrict__ k_pool, const T* __restrict__ v_pool,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens, float* __restrict__ part_o,
    float* __restrict__ part_ml, int H, int G, int chunk, int max_blocks, int num_pool_blocks, int S,
    float scale_log2) {
  using F = Frag<T, D>;
  constexpr int NT = F::NT;
  const int s = blockIdx.x;
  const int rg = blockIdx.y;
  const int r = blockIdx.z / H;
  const int i = blockIdx.z % H;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int quad = lane >> 4;

  const int rows = chunk * G;
  const int qr = (rg * kRectWaves + wave) * 16 + col;  // this lane's query row (tile column)
  const bool row_ok = qr < rows;
  const int t = row_ok ? qr / G : 0;
  const int j = qr % G;

  const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  const int P0 = L - chunk;
  int beg = 0, end = 0;
  if (P0 >= 0) {
    int last = rg * kRectWaves * 16 + kRectWaves * 16 - 1;
    last = last < rows - 1 ? last : rows - 1;
    const int mlim = min(M, (P0 + last / G) / kBlock + 1);
    const int bps = (max_blocks + S - 1) / S;
    beg = s * bps;
    end = min(mlim, beg + bps);
  }
  const int my_lim = P0 + t;  // last visible position of this lane's row

  typename F::Q qf;
  F::load_q_row(qf, q_chunk + (((size_t)r * chunk + t) * H * G + (size_t)i * G + j) * D, quad, row_ok && P0 >= 0);

  float m_run = -INFINITY;
  float l_run = 0.f;
  floatx4_t acc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) acc[tt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const int32_t* tab_row = table + (size_t)r * max_blocks;
  const size_t head_stride = (size_t)kBlock * D;

  for (int g0 = beg; g0 < end; g0 += 64) {
    const int gn = min(64, end - g0);
    int my_pid = 0;
    if (lane < gn) my_pid = clampi(tab_row[g0 + lane], 0, num_pool_blocks - 1);

    auto load_chunk = [&](RChunk<T, D>& c, int at) {
#pragma unroll
      for (int jj = 0; jj < kRectChunk; ++jj) {
        if (at + jj < gn) {
          const int p = __builtin_amdgcn_readlane(my_pid, at + jj);
          const size_t tile = ((size_t)p * H + i) * head_stride;
          F::load_kv(c.f[jj], k_pool + tile, v_pool + tile, col, quad);
          c.blk[jj] = g0 + at + jj;
        } else {
          c.blk[jj] = -1;
        }
      }
    };

    auto compute_chunk = [&](RChunk<T, D>& c) {
      floatx4_t sv[kRectChunk];
      float mx = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < kRectChunk; ++jj) {
        if (c.blk[jj] >= 0) {
          sv[jj] = F::qk(c.f[jj], qf);
          const int tok0 = c.blk[jj] * kBlock + 4 * quad;
          unsigned keep = 0xfu;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool vis = tok0 + e <= my_lim;
            sv[jj][e] = vis ? sv[jj][e] * scale_log2 : -INFINITY;
            keep &= tok0 + e < L ? 0xfu : ~(1u << e);
            mx = fmaxf(mx, sv[jj][e]);
          }
          if (c.blk[jj] * kBlock + kBlock > L) F::mask_v(c.f[jj], keep);
        } else {
          sv[jj] = floatx4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) acc[tt] *= alpha;
#pragma unroll
      for (int jj = 0; jj < kRectChunk; ++jj) {
        if (c.blk[jj] >= 0) {
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = exp2f(sv[jj][e] - m_use);
            l_run += p[e];
          }
          F::pv(acc, c.f[jj], p);
        }
      }
    };

    RChunk<T, D> cur;
    load_chunk(cur, 0);
    for (int at = 0; at < gn; at += kRectChunk) {
      RChunk<T, D> nxt;
#pragma unroll
      for (int jj = 0; jj < kRectChunk; ++jj) nxt.blk[jj] = -1;
      if (at + kRectChunk < gn) load_chunk(nxt, at + kRectChunk);
      compute_chunk(cur);
      cur = nxt;
    }
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (row_ok) {
    const size_t pr = (((size_t)r * H + i) * S + s) * rows + qr;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) *reinterpret_cast<floatx4_t*>(part_o + pr * D + 16 * tt + 4 * quad) = acc[tt];
    if (quad == 0) {
      part_ml[pr * 2] = m_run;
      part_ml[pr * 2 + 1] = l_run;
    }
  }
}

// bf16 chunk attention with K / V streamed through LDS.  A 512-thread
// workgroup owns up to 256 query rows of one KV head (8 wavefronts x two
// 16-column tiles) and walks one split of the cache two blocks (32 tokens)
// per step.  The blocks of the next kRlStages - 1 steps are in flight as
// direct global-to-LDS copies (no registers held), into a ring of LDS
// stages, so each K / V byte leaves HBM once per workgroup and is read from
// LDS by all eight wavefronts.  Both products use v_mfma_f32_16x16x32_bf16:
// S^T = K . Q^T per block, and O^T += V^T . P^T over the two blocks at once,
// the contraction slots of a lane holding tokens 4q..4q+3 of each block in
// both operands.  P enters as a bf16 high part and a bf16 residual, as in
// decode.  Key rows are stored with their 16-byte pieces XOR-swizzled by row
// so the sixteen rows a wavefront reads together fall in different banks.
constexpr int kRlWaves = 8;
constexpr int kRlThreads = 64 * kRlWaves;
constexpr int kRlTiles = 2;                         // 16-column tiles per wavefront
constexpr int kRlRows = kRlWaves * kRlTiles * 16;  // query rows per workgroup
constexpr int kRlStep = 2;                          // blocks per step
constexpr int kRlStages = 6;                        // LDS ring: steps in flight + the one computed
constexpr int kRlPidMax = 2048;                     // blocks per split (physical ids kept in LDS)

template <int D>
struct RectLds {
  static constexpr int CPR = D / 8;                  // 16-byte pieces per key row
  static constexpr int BLK = kBlock * D;             // elements of one K (or V) block
  static constexpr int PIECES = kBlock * CPR;        // 16-byte pieces of one K (or V) block
  static constexpr int KPIECES = kRlStep * PIECES;   // key pieces per step
  static constexpr int STAGE = 2 * kRlStep * BLK;    // elements per stage: keys, then values
  static constexpr int ISSUES = 2 * KPIECES / kRlThreads;  // copies per wavefront per step
  static_assert(2 * KPIECES % kRlThreads == 0, "a step is a whole number of copies per wavefront");
  static_assert(KPIECES % 64 == 0, "a wavefront copies keys or values, not both");
  // piece index of (row, logical piece c) inside a key block
  __device__ static int kpiece(int row, int c) { return row * CPR + (c ^ ((row / (16 / CPR)) % CPR)); }
};

// One 16-byte piece per lane from global memory straight into LDS at
// lds_wave + 16 * lane (lds_wave is the same for the whole wavefront).  The
// copy is written out so that the compiler does not track it: it would
// otherwise wait for every copy in flight before any LDS read from a stage
// it cannot tell apart.  The instruction writes no register; its completion
// is awaited explicitly (vmcnt in ring_sync) before the stage is read.
__device__ __forceinline__ void copy_to_lds16(const bf16_t* src, bf16_t* lds_wave) {
  const uint32_t dst = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16_t*)lds_wave);  // LDS byte offset
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(dst), "v"(src)
               : "memory", "m0");
}

// vmcnt(N) together with lgkmcnt(0), then a workgroup barrier.  The LDS
// copies are tracked by vmcnt; the barrier itself orders nothing, so the
// compiler is told not to move memory accesses across it.
template <int N>
__device__ __forceinline__ void ring_sync() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(kRlThreads) void rectify_attn_lds_kernel(
    const bf16_t* __restrict__ q_chunk, const bf16_t* __restrict__ k_pool, const bf16_t* __restrict__ v_pool,
    const int32_t* __restrict__ table, const int32_t* __restrict__ seq_lens, float* __restrict__ part_o,
    float* __restrict__ part_ml, int H, int G, int chunk, int max_blocks, int num_pool_blocks, int S,
    float scale_log2) {
  using LY = RectLds<D>;
  constexpr int KK = D / 32;  // score MFMAs per block
  constexpr int NT = D / 16;  // output channel tiles
  constexpr int NS = kRlStages;
  __shared__ __align__(16) bf16_t lds[NS * LY::STAGE];
  __shared__ int s_pid[kRlPidMax];

  const int s = blockIdx.x;
  const int rg = blockIdx.y;
  const int r = blockIdx.z / H;
  const int i = blockIdx.z % H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;
  const int quad = lane >> 4;

  const int rows = chunk * G;
  const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  const int P0 = L - chunk;
  int beg = 0, end = 0;
  if (P0 >= 0) {
    const int last = min(rg * kRlRows + kRlRows - 1, rows - 1);
    const int mlim = min(M, (P0 + last / G) / kBlock + 1);  // blocks any row of this workgroup sees
    const int bps = (max_blocks + S - 1) / S;
    beg = s * bps;
    end = min(mlim, beg + bps);
  }
  const int nblk = end > beg ? end - beg : 0;
  const int nsteps = (nblk + kRlStep - 1) / kRlStep;

  // Query rows of this lane (one per tile) and their last visible position.
  uint4 qf[kRlTiles][KK];
  int lim[kRlTiles];
  int qr[kRlTiles];
#pragma unroll
  for (int c = 0; c < kRlTiles; ++c) {
    qr[c] = rg * kRlRows + (wave * kRlTiles + c) * 16 + col;
    const bool ok = qr[c] < rows && P0 >= 0;
    const int t = ok ? qr[c] / G : 0;
    const int j = ok ? qr[c] % G : 0;
    lim[c] = ok ? P0 + t : -1;
    const bf16_t* qrow = q_chunk + (((size_t)r * chunk + t) * H * G + (size_t)i * G + j) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[c][kk] = ok ? *reinterpret_cast<const uint4*>(qrow + quad * 8 * KK + 8 * kk) : make_uint4(0, 0, 0, 0);
  }

  // The query fragments are complete before the loop: the compiler does not
  // track the LDS copies, and a load of its own still pending inside the loop
  // would make it wait for every copy in flight there.
#pragma unroll
  for (int c = 0; c < kRlTiles; ++c)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint4 x = qf[c][kk];
      asm volatile("" ::"v"(x.x), "v"(x.y), "v"(x.z), "v"(x.w));
    }

  float m_ref[kRlTiles], l_run[kRlTiles];
  floatx4_t acc[kRlTiles][NT];
#pragma unroll
  for (int c = 0; c < kRlTiles; ++c) {
    m_ref[c] = -INFINITY;
    l_run[c] = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[c][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }

  // physical ids of the split's blocks (the host keeps a split within kRlPidMax blocks)
  const int32_t* tab_row = table + (size_t)r * max_blocks;
  for (int b = tid; b < nblk; b += kRlThreads) s_pid[b] = clampi(tab_row[beg + b], 0, num_pool_blocks - 1);
  __syncthreads();

  // Copies of one step into one stage: every wavefront moves ISSUES x 64
  // pieces of 16 bytes straight from HBM into LDS.  Blocks past `end` copy an
  // in-range block (the first of the split) and are masked when computed.
  const size_t head_stride = (size_t)kBlock * D;
  auto issue = [&](int step, int stage) {
#pragma unroll
    for (int u = 0; u < LY::ISSUES; ++u) {
      const int p0 = u * kRlThreads + wave * 64;  // first piece of this copy (wavefront-uniform)
      const int piece = p0 + lane;
      const bool is_k = p0 < LY::KPIECES;
      const int pp = is_k ? piece : piece - LY::KPIECES;
      const int b = pp / LY::PIECES;
      const int w = pp % LY::PIECES;
      const int gb = min(step * kRlStep + b, nblk - 1);
      const int pid = clampi(s_pid[max(gb, 0)], 0, num_pool_blocks - 1);
      const size_t tile = ((size_t)pid * H + i) * head_stride;
      const bf16_t* src;
      if (is_k) {
        const int row = w / LY::CPR;
        const int c = (w % LY::CPR) ^ ((row / (16 / LY::CPR)) % LY::CPR);  // logical piece stored here
        src = k_pool + tile + (size_t)row * D + c * 8;
      } else {
        src = v_pool + tile + (size_t)w * 8;
      }
      copy_to_lds16(src, lds + stage * LY::STAGE + p0 * 8);
    }
  };

  // Lowest last-visible position over this wavefront's valid rows (its rows
  // are consecutive, so the first one has the lowest).
  const int first_row = rg * kRlRows + wave * kRlTiles * 16;
  const int lim_lo = first_row < rows && P0 >= 0 ? P0 + first_row / G : -1;

  // One step: scores, online softmax, output update (the hardware exp2, whose
  // results below 2^-126 flush to zero, which changes no sum beyond fp32
  // rounding).  The reference maximum
  // m_ref is raised only when a column's new maximum exceeds it by more than
  // 8 (log2 units), so most steps skip rescaling the accumulators; the
  // probabilities then stay below 2^8, and the merge, which weighs each
  // split by 2^(m - max m), is exact for any reference value.
  auto compute = [&](const bf16_t* kb, const bf16_t* vb, int blk0, auto masked) {
    floatx4_t sv[kRlStep][kRlTiles];
#pragma unroll
    for (int b = 0; b < kRlStep; ++b) {
      uint4 kf[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kf[kk] = *reinterpret_cast<const uint4*>(kb + b * LY::BLK + LY::kpiece(col, quad * KK + kk) * 8);
#pragma unroll
      for (int c = 0; c < kRlTiles; ++c) {
        floatx4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[kk]),
                                                      __builtin_bit_cast(bf16x8_t, qf[c][kk]), x, 0, 0, 0);
        sv[b][c] = x;
      }
    }
    // Value operands of both blocks, shared by every tile: V^T slots 0-3 are
    // block 0 tokens 4q..4q+3, slots 4-7 block 1.  Entries of blocks past the
    // split and of tokens past the sequence end are zeroed: their
    // probability is 0 but the bytes there may be anything.
    bf16x8_t vop[NT];
    {
      uint2 keep[kRlStep];
#pragma unroll
      for (int b = 0; b < kRlStep; ++b) {
        if constexpr (decltype(masked)::value) {
          const int vl = blk0 + b < end ? L - (blk0 + b) * kBlock - 4 * quad : 0;  // valid tokens from 4q on
          keep[b].x = (vl > 0 ? 0xffffu : 0u) | (vl > 1 ? 0xffff0000u : 0u);
          keep[b].y = (vl > 2 ? 0xffffu : 0u) | (vl > 3 ? 0xffff0000u : 0u);
        } else {
          keep[b] = make_uint2(0xffffffffu, 0xffffffffu);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint2 v0 = *reinterpret_cast<const uint2*>(vb + (16 * t + col) * kBlock + 4 * quad);
        uint2 v1 = *reinterpret_cast<const uint2*>(vb + LY::BLK + (16 * t + col) * kBlock + 4 * quad);
        if constexpr (decltype(masked)::value) {
          v0 = make_uint2(v0.x & keep[0].x, v0.y & keep[0].y);
          v1 = make_uint2(v1.x & keep[1].x, v1.y & keep[1].y);
        }
        vop[t] = __builtin_bit_cast(bf16x8_t, make_uint4(v0.x, v0.y, v1.x, v1.y));
      }
    }
#pragma unroll
    for (int c = 0; c < kRlTiles; ++c) {
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < kRlStep; ++b) {
        const int tok0 = (blk0 + b) * kBlock + 4 * quad;
        const bool in_split = blk0 + b < end;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // masked: past the row's last visible position (which also covers
          // the sequence end) or past the split
          if constexpr (decltype(masked)::value)
            sv[b][c][e] = in_split && tok0 + e <= lim[c] ? sv[b][c][e] : -INFINITY;
          mx = fmaxf(mx, sv[b][c][e]);
        }
      }
      mx = quad_max(mx);
      const float m_cand = mx * scale_log2;  // scale > 0: the maximum of the scaled scores
      const bool raise = m_cand > m_ref[c] + 8.f;
      if (__ballot(raise)) {
        const float alpha = raise ? __builtin_amdgcn_exp2f(m_ref[c] - m_cand) : 1.f;  // 0 while m_ref = -inf
        m_ref[c] = raise ? m_cand : m_ref[c];
        l_run[c] *= alpha;
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[c][t] *= alpha;
      }
      const float neg_m = m_ref[c] == -INFINITY ? 0.f : -m_ref[c];
      float p[kRlStep * 4];
#pragma unroll
      for (int b = 0; b < kRlStep; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[4 * b + e] = __builtin_amdgcn_exp2f(fmaf(sv[b][c][e], scale_log2, neg_m));
          l_run[c] += p[4 * b + e];
        }
      // P^T operands, same slot order as V^T: a bf16 high part and the bf16
      // of the residual
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const bf16x2_t hi = __builtin_convertvector(float2_t{p[2 * h], p[2 * h + 1]}, bf16x2_t);
        const float2_t hf = __builtin_convertvector(hi, float2_t);
        const bf16x2_t lo = __builtin_convertvector(float2_t{p[2 * h] - hf.x, p[2 * h + 1] - hf.y}, bf16x2_t);
        hw[h] = __builtin_bit_cast(uint32_t, hi);
        lw[h] = __builtin_bit_cast(uint32_t, lo);
      }
      const bf16x8_t ph = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      // O^T += V^T . P^T over both blocks
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[t], ph, acc[c][t], 0, 0, 0);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[t], pl, acc[c][t], 0, 0, 0);
    }
  };

  // Steps go in pairs, one barrier per pair: pair (s, s + 1) is computed
  // from stages s % NS and (s + 1) % NS while the copies of the next
  // NS - 2 steps are in flight; after the barrier the two stages of the
  // previous pair are free and receive steps s + NS - 2 and s + NS - 1.
  static_assert(NS % 2 == 0 && NS >= 4, "stages come in pairs");
#pragma unroll
  for (int j = 0; j < NS - 2; ++j)
    if (j < nsteps) issue(j, j);
  int stage = 0;
#pragma clang loop unroll(disable)
  for (int step = 0; step < nsteps; step += 2) {
    // this pair's copies are done once at most the next pair's are pending
    if (step + NS - 3 < nsteps) ring_sync<LY::ISSUES * 2>();
    else ring_sync<0>();
    const int freed = stage == 0 ? NS - 2 : stage - 2;  // stages of the previous pair
    if (step + NS - 2 < nsteps) issue(step + NS - 2, freed);
    if (step + NS - 1 < nsteps) issue(step + NS - 1, freed + 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16_t* kb = lds + (stage + h) * LY::STAGE;
      const bf16_t* vb = kb + kRlStep * LY::BLK;
      const int blk0 = beg + (step + h) * kRlStep;
      // Steps wholly inside the split, the sequence and every row's causal
      // window (all but the last few) skip the masking.
      const bool plain = blk0 + kRlStep <= end && (blk0 + kRlStep) * kBlock - 1 <= lim_lo;
      if (plain) compute(kb, vb, blk0, std::integral_constant<bool, false>{});
      else compute(kb, vb, blk0, std::integral_constant<bool, true>{});
      __builtin_amdgcn_sched_barrier(0);  // keep the two steps' live ranges apart
    }
    stage = stage == NS - 2 ? 0 : stage + 2;
  }
  ring_sync<0>();  // no copy may still be writing when the workgroup ends

#pragma unroll
  for (int c = 0; c < kRlTiles; ++c) {
    float l = l_run[c];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (qr[c] < rows) {
      const size_t pr = (((size_t)r * H + i) * S + s) * rows + qr[c];
#pragma unroll
      for (int t = 0; t < NT; ++t) *reinterpret_cast<floatx4_t*>(part_o + pr * D + 16 * t + 4 * quad) = acc[c][t];
      if (quad == 0) {
        part_ml[pr * 2] = m_ref[c];
        part_ml[pr * 2 + 1] = l;
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_rectify_t(const RectifyArgs& a, hipStream_t stream) {
  const int wt = a.H * D < 1024 ? a.H * D : 1024;
  hipLaunchKernelGGL((write_rows_kernel<T>), dim3((unsigned)a.chunk, (unsigned)a.R), dim3(wt), 0, stream,
                     static_cast<const T*>(a.k_new), static_cast<const T*>(a.v_new), static_cast<T*>(a.k_pool),
                     static_cast<T*>(a.v_pool), a.table, a.seq_lens, a.H, D, a.chunk, a.max_blocks,
                     a.num_pool_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  DescArgs d{};
  d.k_pool = a.k_pool;
  d.desc_pool = a.desc_pool;
  d.table = a.table;
  d.seq_lens = a.seq_lens;
  d.first_block = nullptr;
  d.num_blocks = 0;
  d.window = a.chunk;
  d.R = a.R;
  d.H = a.H;
  d.D = D;
  d.dtype = a.dtype;
  d.max_blocks = a.max_blocks;
  d.num_pool_blocks = a.num_pool_blocks;
  e = launch_descriptors(d, stream);
  if (e != hipSuccess) return e;

  const int rows = a.chunk * a.G;
  const int bps = (a.max_blocks + a.splits - 1) / a.splits;
  if (std::is_same<T, bf16_t>::value && bps <= kRlPidMax) {
    const int rgroups = (rows + kRlRows - 1) / kRlRows;
    dim3 grid((unsigned)a.splits, (unsigned)rgroups, (unsigned)(a.R * a.H));
    hipLaunchKernelGGL((rectify_attn_lds_kernel<D>), grid, dim3(kRlThreads), 0, stream,
                       static_cast<const bf16_t*>(a.q_chunk), static_cast<const bf16_t*>(a.k_pool),
                       static_cast<const bf16_t*>(a.v_pool), a.table, a.seq_lens, a.part_o, a.part_ml, a.H, a.G,
                       a.chunk, a.max_blocks, a.num_pool_blocks, a.splits, a.scale_log2);
    // (a split longer than kRlPidMax blocks, i.e. a cache beyond 2^21 blocks, takes the kernel below)
  } else {
    const int rgroups = (rows + kRectWaves * 16 - 1) / (kRectWaves * 16);
    dim3 grid((unsigned)a.splits, (unsigned)rgroups, (unsigned)(a.R * a.H));
    hipLaunchKernelGGL((rectify_attn_kernel<T, D>), grid, dim3(kRectThreads), 0, stream,
                       static_cast<const T*>(a.q_chunk), static_cast<const T*>(a.k_pool),
                       static_cast<const T*>(a.v_pool), a.table, a.seq_lens, a.part_o, a.part_ml, a.H, a.G,
                       a.chunk, a.max_blocks, a.num_pool_blocks, a.splits, a.scale_log2);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(a.part_o, a.part_ml, a.out, a.R, a.H, a.G, D, a.splits, rows, a.chunk, stream);
}

}  // namespace

hipError_t launch_rectify(const RectifyArgs& a, hipStream_t stream) {
  if (a.dtype == 0)
    return a.D == 128 ? launch_rectify_t<bf16_t, 128>(a, stream) : launch_rectify_t<bf16_t, 64>(a, stream);
  return a.D == 128 ? launch_rectify_t<float, 128>(a, stream) : launch_rectify_t<float, 64>(a, stream);
}

}  // namespace resa
