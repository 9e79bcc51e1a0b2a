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
//      head are the columns of 16-wide MFMA tiles; a 256-thread workgroup
//      holds four tiles (64 query rows, one per wavefront) and walks one
//      split of the cache, so the four wavefronts read the same K / V blocks
//      (served from the CU's L1 / the XCD's L2 after the first).  Each query
//      row t masks positions > L - chunk + t; blocks past the workgroup's
//      last visible position are skipped;
//   4. the log-sum-exp merge of the splits (shared with decode).
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
  const int rgroups = (rows + kRectWaves * 16 - 1) / (kRectWaves * 16);
  dim3 grid((unsigned)a.splits, (unsigned)rgroups, (unsigned)(a.R * a.H));
  hipLaunchKernelGGL((rectify_attn_kernel<T, D>), grid, dim3(kRectThreads), 0, stream,
                     static_cast<const T*>(a.q_chunk), static_cast<const T*>(a.k_pool),
                     static_cast<const T*>(a.v_pool), a.table, a.seq_lens, a.part_o, a.part_ml, a.H, a.G, a.chunk,
                     a.max_blocks, a.num_pool_blocks, a.splits, a.scale_log2);
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
