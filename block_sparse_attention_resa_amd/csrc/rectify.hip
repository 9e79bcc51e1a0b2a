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
//      per workgroup.  fp32 caches (and bf16 splits longer than the 2048
//      page ids the LDS kernel keeps): a 256-thread workgroup holds four
//      tiles and each wavefront reads its K / V operands directly.  Each query row
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
// per step.  The blocks of the next steps are in flight as direct
// global-to-LDS copies (no registers held) into a ring of LDS stages, so each
// K / V byte leaves HBM once per workgroup and is read from LDS by all eight
// wavefronts.  Both products use v_mfma_f32_16x16x32_bf16: S^T = K . Q^T as
// two 16-token score tiles per step, and O^T += V^T . P^T over the step's 32
// tokens at once, the contraction slots of a lane holding eight consecutive
// tokens in both operands.  P enters as a bf16 high part and a bf16
// residual, as in decode.  Key and value pieces are XOR-swizzled in LDS so
// that the rows (channels) a wavefront reads together fall in different
// banks.
constexpr int kRlWaves = 8;
constexpr int kRlThreads = 64 * kRlWaves;
constexpr int kRlTiles = 2;                         // 16-column tiles per wavefront
constexpr int kRlRows = kRlWaves * kRlTiles * 16;  // query rows per workgroup
constexpr int kRlStep = 2;                          // blocks per step
constexpr int kRlStages = 8;                        // LDS ring stages (one step each)
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
  static_assert(CPR == 8 || CPR == 16, "head dims 64 and 128");
  // The two score tiles of a step take tokens {8a + e} and {8a + 4 + e}
  // (a < 4, e < 4), so that a lane's eight probabilities cover eight
  // consecutive tokens, which lie in one 16-byte value piece.  Key rows are
  // XOR-swizzled so that the sixteen rows of either tile fall in distinct
  // 16-byte bank groups: with 256-byte rows (d = 128) a row's swizzle takes
  // bits 0-1 and 3-4 of the token, with 128-byte rows (two to a bank row)
  // bits 1 and 3-4.
  __device__ static int kswz(int token) {
    return CPR == 16 ? (token & 3) | ((token >> 1) & 12) : ((token >> 1) & 1) | ((token >> 2) & 6);
  }
  // piece index of (token, logical piece c) inside the keys of a step
  __device__ static int kpiece(int token, int c) { return token * CPR + (c ^ kswz(token)); }
  // piece index of (channel, token half h) inside a value block: the halves
  // swap for channels with bit 3 set, so the sixteen channels a wavefront
  // reads together fall in distinct bank groups
  __device__ static int vpiece(int ch, int h) { return ch * 2 + (h ^ ((ch >> 3) & 1)); }
};

// One 16-byte piece per lane from global memory straight into LDS at
// lds_wave + 16 * lane (lds_wave is the same for the whole wavefront).  The
// copy is written out so that the compiler does not track it: it would
// otherwise wait for every copy in flight before any LDS read from a stage
// it cannot tell apart.  The instruction writes no register; its completion
// is awaited explicitly (vmcnt in ring_sync) before the stage is read.
// The source is a wavefront-uniform base (scalar registers) plus a 32-bit
// byte offset per lane; the destination is an LDS byte address.
__device__ __forceinline__ void copy_to_lds16(const bf16_t* base_ptr, uint32_t voff, uint32_t lds_dst) {
  const uint64_t b = (uint64_t)(uintptr_t)base_ptr;  // uniform; read from the first lane into scalar registers
  // (the builtin returns int: both halves are taken as uint32_t, so the low
  // half is zero-extended)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t base = ((uint64_t)hi << 32) | (uint64_t)lo;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_dst), "v"(voff), "s"(base)
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar address math
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
  // pieces of 16 bytes straight from HBM into LDS.  Which pieces a lane
  // moves is the same for every step: copy u of a wavefront takes keys or
  // values (uniform) of block cb[u] of the step (uniform), at byte offset
  // cvoff[u] of that block's tile.  Blocks past `end` copy an in-range block
  // (the first of the split) and are masked when computed.
  const size_t head_stride = (size_t)kBlock * D;
  const uint32_t lds_base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) bf16_t*)lds);  // LDS byte address
  bool ck[LY::ISSUES];
  int cb[LY::ISSUES];
  uint32_t cvoff[LY::ISSUES];
#pragma unroll
  for (int u = 0; u < LY::ISSUES; ++u) {
    const int p0 = u * kRlThreads + wave * 64;  // first piece of this copy (wavefront-uniform)
    ck[u] = p0 < LY::KPIECES;
    const int pp = (ck[u] ? p0 : p0 - LY::KPIECES) + lane;
    cb[u] = (ck[u] ? p0 : p0 - LY::KPIECES) / LY::PIECES;
    const int w = pp % LY::PIECES;
    if (ck[u]) {
      const int token = pp / LY::CPR;  // token of the step
      const int c = (pp % LY::CPR) ^ LY::kswz(token);  // logical piece stored here
      cvoff[u] = (uint32_t)(((token % kBlock) * D + c * 8) * sizeof(bf16_t));
    } else {
      const int ch = w / 2;
      const int h = (w % 2) ^ ((ch >> 3) & 1);  // token half stored here
      cvoff[u] = (uint32_t)((ch * kBlock + h * 8) * sizeof(bf16_t));
    }
  }
  // The physical ids a step's copies need are read from LDS one pair of
  // steps ahead, so the copies themselves wait for nothing.
  auto read_pids = [&](int step, int (&pid)[LY::ISSUES]) {
#pragma unroll
    for (int u = 0; u < LY::ISSUES; ++u) pid[u] = s_pid[max(min(step * kRlStep + cb[u], nblk - 1), 0)];
  };
  auto issue = [&](int stage, const int (&pids)[LY::ISSUES]) {
#pragma unroll
    for (int u = 0; u < LY::ISSUES; ++u) {
      const int pid = __builtin_amdgcn_readfirstlane(clampi(pids[u], 0, num_pool_blocks - 1));
      const bf16_t* base = (ck[u] ? k_pool : v_pool) + ((size_t)pid * H + i) * head_stride;
      copy_to_lds16(base, cvoff[u],
                    lds_base + (uint32_t)((stage * LY::STAGE + (u * kRlThreads + wave * 64) * 8) * sizeof(bf16_t)));
    }
  };

  // Lowest last-visible position over this wavefront's valid rows (its rows
  // are consecutive, so the first one has the lowest).
  const int first_row = rg * kRlRows + wave * kRlTiles * 16;
  const int lim_lo = first_row < rows && P0 >= 0 ? P0 + first_row / G : -1;

  // The steps are software-pipelined inside each wavefront so that the
  // matrix unit and the vector ALU work at the same time: the scores of step
  // s + 1 (MFMA) are computed beside the exponentials of step s (vector
  // ALU), and the output update of step s (MFMA) beside the conversion of
  // its probabilities to bf16 operands (vector ALU).  The hardware exp2
  // flushes results below 2^-126 to zero, which changes no sum beyond fp32
  // rounding.  Probabilities are taken against a per-column reference m_ref
  // that is raised only when some probability would exceed 2^8, i.e. when a
  // column maximum passes the reference by more than 8 (log2 units); most
  // steps therefore need neither column maxima nor a rescale of the
  // accumulators, and the merge, which weighs each split by 2^(m - max m),
  // is exact for any reference value.
  // Key operands of score tile u: row r holds token 8 (r / 4) + 4 u + r % 4.
  // The swizzle of token t + 4 equals that of t (bit 2 of t is clear), so
  // tile 1 lies 4 rows past tile 0.
  int k_off[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) k_off[kk] = LY::kpiece(8 * (col >> 2) + (col & 3), quad * KK + kk) * 8;
  auto load_k = [&](const bf16_t* kb, uint4 (&kf)[kRlStep][KK]) {
#pragma unroll
    for (int u = 0; u < kRlStep; ++u)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kf[u][kk] = *reinterpret_cast<const uint4*>(kb + k_off[kk] + u * 4 * LY::CPR * 8);
  };
  auto qk = [&](const uint4 (&kf)[kRlStep][KK], floatx4_t (&sv)[kRlStep][kRlTiles]) {
#pragma unroll
    for (int b = 0; b < kRlStep; ++b)
#pragma unroll
      for (int c = 0; c < kRlTiles; ++c) {
        floatx4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
          x = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[b][kk]),
                                                      __builtin_bit_cast(bf16x8_t, qf[c][kk]), x, 0, 0, 0);
        sv[b][c] = x;
      }
  };
  // Value operand of output tile t, shared by every query tile: slot j of a
  // lane in quad q is token 8 q + j of the step (block q / 2), the same
  // order as the probabilities.  On masked steps the entries of blocks past
  // the split and of tokens past the sequence end are zeroed (`keep`): their
  // probability is 0 but the bytes there may be anything.
  // (channel 16 t + c has the swizzle of channel c, so tile t lies 16
  // channels past tile 0)
  const int v_off = (quad >> 1) * LY::BLK + LY::vpiece(col, quad & 1) * 8;
  auto v_operand = [&](const bf16_t* vb, int t) {
    return *reinterpret_cast<const uint4*>(vb + v_off + t * 16 * kBlock);
  };
  auto v_keep = [&](int blk0) {
    const int vl = blk0 + (quad >> 1) < end ? L - blk0 * kBlock - 8 * quad : 0;  // valid tokens from 8q on
    uint4 k;
    k.x = (vl > 0 ? 0xffffu : 0u) | (vl > 1 ? 0xffff0000u : 0u);
    k.y = (vl > 2 ? 0xffffu : 0u) | (vl > 3 ? 0xffff0000u : 0u);
    k.z = (vl > 4 ? 0xffffu : 0u) | (vl > 5 ? 0xffff0000u : 0u);
    k.w = (vl > 6 ? 0xffffu : 0u) | (vl > 7 ? 0xffff0000u : 0u);
    return k;
  };
  // Scores past the row's last visible position (which also covers the
  // sequence end) or past the split are excluded.  Entry e of score tile u
  // in quad q is token 8 q + 4 u + e of the step.
  auto mask_s = [&](int blk0, floatx4_t (&sv)[kRlStep][kRlTiles]) {
    const bool in_split = blk0 + (quad >> 1) < end;
#pragma unroll
    for (int u = 0; u < kRlStep; ++u) {
      const int tok0 = blk0 * kBlock + 8 * quad + 4 * u;
#pragma unroll
      for (int c = 0; c < kRlTiles; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[u][c][e] = in_split && tok0 + e <= lim[c] ? sv[u][c][e] : -INFINITY;
    }
  };
  // Probabilities of a step against the references.
  auto exps = [&](const floatx4_t (&sv)[kRlStep][kRlTiles], float (&p)[kRlTiles][kRlStep * 4]) {
#pragma unroll
    for (int c = 0; c < kRlTiles; ++c) {
      const float neg_m = m_ref[c] == -INFINITY ? 0.f : -m_ref[c];
#pragma unroll
      for (int u = 0; u < kRlStep; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[c][4 * u + e] = __builtin_amdgcn_exp2f(fmaf(sv[u][c][e], scale_log2, neg_m));
    }
  };
  // True in a lane where a score of the step passes its column's reference
  // by more than 8 (log2 units).
  auto passes = [&](const floatx4_t (&sv)[kRlStep][kRlTiles]) {
    bool any = false;
#pragma unroll
    for (int c = 0; c < kRlTiles; ++c) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < kRlStep; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sv[u][c][e]);
      any = any || mx * scale_log2 > m_ref[c] + 8.f;
    }
    return any;
  };
  // Raise the reference of every column whose maximum passes it by more than
  // 8 to that maximum and rescale the column's accumulated output and sum.
  auto raise_ref = [&](const floatx4_t (&sv)[kRlStep][kRlTiles]) {
#pragma unroll
    for (int c = 0; c < kRlTiles; ++c) {
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < kRlStep; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sv[u][c][e]);
      const float m_cand = quad_max(mx) * scale_log2;  // scale > 0: the maximum of the scaled scores
      const bool raise = m_cand > m_ref[c] + 8.f;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_ref[c] - m_cand) : 1.f;  // 0 while m_ref = -inf
      m_ref[c] = raise ? m_cand : m_ref[c];
      l_run[c] *= alpha;
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[c][t] *= alpha;
    }
  };
  // Probabilities of one tile as P^T operands in the V^T slot order: a bf16
  // high part and the bf16 of the residual.
  auto split = [&](const float (&p)[kRlStep * 4], bf16x8_t& ph, bf16x8_t& pl) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const bf16x2_t hi = __builtin_convertvector(float2_t{p[2 * h], p[2 * h + 1]}, bf16x2_t);
      const float2_t hf = __builtin_convertvector(hi, float2_t);
      const bf16x2_t lo = __builtin_convertvector(float2_t{p[2 * h] - hf.x, p[2 * h + 1] - hf.y}, bf16x2_t);
      hw[h] = __builtin_bit_cast(uint32_t, hi);
      lw[h] = __builtin_bit_cast(uint32_t, lo);
    }
    ph = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    pl = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
  };
  // O^T += V^T . P^T over both blocks of a step.
  auto pv = [&](const bf16_t* vb, const bf16x8_t (&ph)[kRlTiles], const bf16x8_t (&pl)[kRlTiles], auto masked,
                int blk0) {
    uint4 keep = make_uint4(~0u, ~0u, ~0u, ~0u);
    if constexpr (decltype(masked)::value) keep = v_keep(blk0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint4 v = v_operand(vb, t);
      if constexpr (decltype(masked)::value) v = make_uint4(v.x & keep.x, v.y & keep.y, v.z & keep.z, v.w & keep.w);
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, v);
#pragma unroll
      for (int c = 0; c < kRlTiles; ++c) {
        acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ph[c], acc[c][t], 0, 0, 0);
        acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl[c], acc[c][t], 0, 0, 0);
      }
    }
  };
  // Steps wholly inside the split, the sequence and every row's causal
  // window (all but the last few) skip the masking.
  auto plain = [&](int s) {
    const int blk0 = beg + s * kRlStep;
    return blk0 + kRlStep <= end && (blk0 + kRlStep) * kBlock - 1 <= lim_lo;
  };

  floatx4_t scur[kRlStep][kRlTiles];  // scores of the step about to be computed
  // Step s: scores of step s + 1 (for the last step, scores of a stage
  // already read, unused), then probabilities and output update of step s.
  // `masked` steps apply the split, sequence and causal masks.
  auto body = [&](int s, auto masked) {
    const bool has_next = s + 1 < nsteps;
    const bf16_t* kb_next = lds + ((has_next ? s + 1 : s) % NS) * LY::STAGE;
    const bf16_t* vb = lds + (s % NS) * LY::STAGE + kRlStep * LY::BLK;
    const int blk0 = beg + s * kRlStep;
    uint4 kf[kRlStep][KK];
    load_k(kb_next, kf);
    floatx4_t snext[kRlStep][kRlTiles];
    qk(kf, snext);
    float p[kRlTiles][kRlStep * 4];
    exps(scur, p);
    if constexpr (decltype(masked)::value) mask_s(blk0 + kRlStep, snext);
    bf16x8_t ph[kRlTiles], pl[kRlTiles];
#pragma unroll
    for (int c = 0; c < kRlTiles; ++c) {
#pragma unroll
      for (int j = 0; j < kRlStep * 4; ++j) l_run[c] += p[c][j];
      split(p[c], ph[c], pl[c]);
    }
    pv(vb, ph, pl, masked, blk0);
    // rare: a column maximum of step s + 1 passes its reference by more than 8
    if (__ballot(has_next && passes(snext))) raise_ref(snext);
#pragma unroll
    for (int u = 0; u < kRlStep; ++u)
#pragma unroll
      for (int c = 0; c < kRlTiles; ++c) scur[u][c] = snext[u][c];
  };

  // Ring protocol, one barrier per pair of steps.  Step s lives in stage
  // s % NS.  Step s reads the values of step s and the keys of step s + 1,
  // so the barrier before pair (s, s + 1) waits until the copies of steps
  // <= s + 2 have landed (those of up to NS - 5 later steps may still be in
  // flight) and then refills the stages of steps s - 2 and s - 1, which no
  // wavefront reads any more, with steps s + NS - 2 and s + NS - 1.
  static_assert(NS % 2 == 0 && NS >= 6 && NS - 5 <= 3, "stages come in pairs; at most three steps pending");
#pragma unroll
  for (int j = 0; j < NS - 2; ++j)
    if (j < nsteps) {
      int pj[LY::ISSUES];
      read_pids(j, pj);
      issue(j, pj);
    }
  int pf0[LY::ISSUES], pf1[LY::ISSUES];  // ids for the next pair's copies
  read_pids(NS - 2, pf0);
  read_pids(NS - 1, pf1);
#pragma clang loop unroll(disable)
  for (int step = 0; step < nsteps; step += 2) {
    const int pending = min(min(step + NS - 3, nsteps - 1) - (step + 2), NS - 5);
    if (pending >= 3) ring_sync<3 * LY::ISSUES>();
    else if (pending == 2) ring_sync<2 * LY::ISSUES>();
    else if (pending == 1) ring_sync<LY::ISSUES>();
    else ring_sync<0>();
    if (step + NS - 2 < nsteps) issue((step + NS - 2) % NS, pf0);
    if (step + NS - 1 < nsteps) issue((step + NS - 1) % NS, pf1);
    read_pids(step + NS, pf0);
    read_pids(step + NS + 1, pf1);
    if (step == 0) {
      uint4 kf[kRlStep][KK];
      load_k(lds, kf);
      qk(kf, scur);
      if (!plain(0)) mask_s(beg, scur);
      if (__ballot(passes(scur))) raise_ref(scur);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int s = step + h;
      if (h == 1 && s >= nsteps) break;
      if (plain(s) && (s + 1 >= nsteps || plain(s + 1))) body(s, std::integral_constant<bool, false>{});
      else body(s, std::integral_constant<bool, true>{});
    }
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
