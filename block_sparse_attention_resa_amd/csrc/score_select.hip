// Group block scoring and top-n block selection.
//
// "Rectified Sparse Attention" analysis page (paper-graph-ui), §3.4.1:
// Eq 4 (block score from the min / max descriptors), Eq 5 (the dynamic count
// n = max(n_min, ceil(M * rho))), the local window (the most recent block is
// always kept) and the GQA-shared pattern (one selection per KV head).
//
// Scoring.  For one GQA group the score of block b sums, over the group's
// query heads j and channels c, max(q_jc * lo_bc, q_jc * hi_bc).  Because
// hi >= lo this equals sum_c P_c * hi_bc + N_c * lo_bc with
// P_c = sum_j max(q_jc, 0) and N_c = sum_j min(q_jc, 0), so each thread folds
// the group's queries into its own slice of (P, N) once and the kernel then
// streams the descriptors with one fused multiply-add per stored value.  A
// descriptor (2 x d values) is split into 32-byte chunks; CH consecutive
// lanes own one descriptor and combine their partial sums with shuffles.
// The thread -> (KV head, chunk) assignment is fixed for the whole kernel so
// the coefficients stay in registers.  Scores are written as order-preserving
// 32-bit keys for the selection kernel.
//
// Selection.  One 1024-thread workgroup per (request, KV head).  Thread t
// owns a contiguous run of candidate blocks, held in registers.  The
// (n - n_local)-th largest key among the older blocks is found by an MSB-first
// radix select over the bits in which the candidates differ, with a 256-bin
// LDS histogram per 8-bit digit; the pass stops early once every key of the
// boundary bucket is needed.  Blocks above the threshold are taken, blocks
// equal to it are taken lowest index first, and a block-wide prefix count
// writes the selected ids in ascending order.
#include "resa_internal.h"

namespace resa {
namespace {

// ------------------------------------------------------------------ scores

template <typename T>
struct ChunkLoad;

template <>
struct ChunkLoad<bf16_t> {
  static constexpr int kVals = 16;  // bf16 values per 32-byte chunk
  __device__ static void unpack(const uint4& a, const uint4& b, float* f) {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f[2 * e] = bf16_lo_f32(w[e]);
      f[2 * e + 1] = bf16_hi_f32(w[e]);
    }
  }
  __device__ static float load_q(const bf16_t* p) { return __uint_as_float((uint32_t)p->bits << 16); }
};

template <>
struct ChunkLoad<float> {
  static constexpr int kVals = 8;
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
  __device__ static float load_q(const float* p) { return *p; }
};

constexpr int kScoreUnroll = 4;

template <typename T, int D>
__global__ __launch_bounds__(1024) void score_kernel(const T* __restrict__ q, const T* __restrict__ desc,
                                                    const int32_t* __restrict__ table,
                                                    const int32_t* __restrict__ seq_lens,
                                                    uint32_t* __restrict__ keys, float* __restrict__ scores, int H,
                                                    int G, int max_blocks, int num_pool_blocks, int mode,
                                                    int blocks_per_wg) {
  using CL = ChunkLoad<T>;
  constexpr int VPL = CL::kVals;
  constexpr int CH = 2 * D / VPL;  // lanes per descriptor
  constexpr int HALF = CH / 2;     // lanes per descriptor row

  const int r = blockIdx.y;
  const int t = threadIdx.x;
  const int grp = t / CH;
  const int lg = t % CH;
  const int part = lg / HALF;  // 0: min row, 1: max row
  const int c0 = (lg % HALF) * VPL;
  const int head = grp % H;
  const int bsub = grp / H;
  const int bpi = blockDim.x / (CH * H);  // blocks per iteration

  // Fold the group's queries into this thread's slice of P (max row) or N (min row).
  float coef[VPL];
  {
    const T* qh = q + ((size_t)r * H * G + (size_t)head * G) * D + c0;
#pragma unroll
    for (int v = 0; v < VPL; ++v) coef[v] = 0.f;
    if (mode == 0) {
      for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          const float x = CL::load_q(qh + (size_t)j * D + v);
          coef[v] += part ? fmaxf(x, 0.f) : fminf(x, 0.f);
        }
      }
    } else {
      for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int v = 0; v < VPL; ++v) coef[v] += CL::load_q(qh + (size_t)j * D + v);
      }
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const float m = coef[v] / (float)G;
        coef[v] = part ? fmaxf(m, 0.f) : fminf(m, 0.f);
      }
    }
  }

  const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  const int wg_b0 = blockIdx.x * blocks_per_wg;
  const int iters = blocks_per_wg / bpi;
  uint32_t* key_row = keys + ((size_t)r * H + head) * max_blocks;
  float* score_row = scores ? scores + ((size_t)r * H + head) * max_blocks : nullptr;

  for (int it0 = 0; it0 < iters; it0 += kScoreUnroll) {
    uint4 buf[kScoreUnroll][2];
    int bl[kScoreUnroll];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int b = wg_b0 + (it0 + u) * bpi + bsub;
      bl[u] = b;
      if (it0 + u < iters && b < M) {
        const int p = clampi(table[(size_t)r * max_blocks + b], 0, num_pool_blocks - 1);
        const uint4* src =
            reinterpret_cast<const uint4*>(desc + (((size_t)p * H + head) * 2 + part) * D + c0);
        buf[u][0] = src[0];
        buf[u][1] = src[1];
      } else {
        buf[u][0] = make_uint4(0, 0, 0, 0);
        buf[u][1] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      float vals[VPL];
      CL::unpack(buf[u][0], buf[u][1], vals);
      float acc = 0.f;
#pragma unroll
      for (int v = 0; v < VPL; ++v) acc = fmaf(coef[v], vals[v], acc);
#pragma unroll
      for (int off = HALF; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
      if (lg == 0 && it0 + u < iters && bl[u] < M) {
        key_row[bl[u]] = f32_order_key(acc);
        if (score_row) score_row[bl[u]] = acc;
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_scores_t(const ScoreArgs& a, hipStream_t stream) {
  constexpr int VPL = ChunkLoad<T>::kVals;
  constexpr int CH = 2 * D / VPL;
  const int unit = CH * a.H;  // threads per block of all heads
  int m = 1;
  while ((unit * m) % 64 != 0) ++m;
  while (unit * m * 2 <= 256) m *= 2;
  const int threads = unit * m;  // <= 1024 checked by the caller
  const int bpi = m;
  const int blocks_per_wg = bpi * kScoreUnroll;
  const int wgs = (a.max_blocks + blocks_per_wg - 1) / blocks_per_wg;
  dim3 grid((unsigned)wgs, (unsigned)a.R);
  hipLaunchKernelGGL((score_kernel<T, D>), grid, dim3(threads), 0, stream, static_cast<const T*>(a.q),
                     static_cast<const T*>(a.desc_pool), a.table, a.seq_lens, a.keys, a.scores, a.H, a.G,
                     a.max_blocks, a.num_pool_blocks, a.mode, blocks_per_wg);
  return hipGetLastError();
}

// ------------------------------------------------------------------ select

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// Exclusive prefix sum over the workgroup (thread order); also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_waves, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int n = __shfl_up(incl, off);
    if (lane >= off) incl += n;
  }
  if (lane == 63) lds_waves[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int x = lds_waves[w];
    before += w < wave ? x : 0;
    total += x;
  }
  __syncthreads();
  return before + incl - v;
}

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(const uint32_t* __restrict__ keys,
                                                            const int32_t* __restrict__ seq_lens,
                                                            int32_t* __restrict__ sel_idx,
                                                            int32_t* __restrict__ sel_cnt, int H, int max_blocks,
                                                            int max_sel, int budget_num, int budget_den,
                                                            int min_blocks, int local_blocks) {
  __shared__ uint32_t hist[256];
  __shared__ int lds_waves[kSelWaves];
  __shared__ uint32_t lds_and[kSelWaves], lds_or[kSelWaves];
  __shared__ int bc[3];

  const int i = blockIdx.x;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  int32_t* out = sel_idx + ((size_t)r * H + i) * max_sel;

  int n = 0, nl = 0;
  if (M > 0) {
    const long long ceil_part = ((long long)M * budget_num + budget_den - 1) / budget_den;
    long long nn = ceil_part;
    if (nn < min_blocks) nn = min_blocks;
    if (nn < local_blocks) nn = local_blocks;
    if (nn > M) nn = M;
    n = (int)nn;
    nl = local_blocks < M ? local_blocks : M;
  }
  const int k = n - nl;  // blocks chosen by score
  const int C = M - nl;  // candidates: blocks [0, C)
  for (int j = tid; j < max_sel; j += kSelThreads) {
    if (j >= n) out[j] = -1;
    else if (j >= k) out[j] = C + (j - k);  // forced recent blocks close the ascending list
  }
  if (tid == 0) sel_cnt[(size_t)r * H + i] = n;
  if (k == 0) return;
  if (k == C) {
    for (int j = tid; j < C; j += kSelThreads) out[j] = j;
    return;
  }

  const uint32_t* kr = keys + ((size_t)r * H + i) * max_blocks;
  const int kpt = (C + kSelThreads - 1) / kSelThreads;
  const int base = tid * kpt;
  const int cnt = base < C ? (C - base < kpt ? C - base : kpt) : 0;

  uint32_t reg[KPT > 0 ? KPT : 1];
  auto key_at = [&](int j) -> uint32_t {
    if constexpr (KPT > 0) {
      return reg[j];
    } else {
      return kr[base + j];
    }
  };
  if constexpr (KPT > 0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) reg[j] = j < cnt ? kr[base + j] : 0u;
  }

  // Bits shared by every candidate key.
  uint32_t a = 0xffffffffu, o = 0u;
  if constexpr (KPT > 0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j < cnt) {
        a &= reg[j];
        o |= reg[j];
      }
  } else {
    for (int j = 0; j < cnt; ++j) {
      const uint32_t x = kr[base + j];
      a &= x;
      o |= x;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    a &= (uint32_t)__shfl_xor((int)a, off);
    o |= (uint32_t)__shfl_xor((int)o, off);
  }
  if (lane == 0) {
    lds_and[wave] = a;
    lds_or[wave] = o;
  }
  __syncthreads();
  a = 0xffffffffu;
  o = 0u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    a &= lds_and[w];
    o |= lds_or[w];
  }
  const uint32_t diff = a ^ o;
  int top = diff ? 31 - __clz(diff) : -1;  // highest bit in which candidates differ
  uint32_t fixed = top >= 31 ? 0u : (top < 0 ? 0xffffffffu : ~((2u << top) - 1u));
  uint32_t prefix = a & fixed;
  int remaining = k;  // keys still to take whose fixed bits equal `prefix`

  while (top >= 0) {
    const int width = top + 1 < 8 ? top + 1 : 8;
    const int shift = top + 1 - width;
    const uint32_t dmask = (1u << width) - 1u;
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    if constexpr (KPT > 0) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const uint32_t x = reg[j];
        if (j < cnt && (x & fixed) == prefix) atomicAdd(&hist[(x >> shift) & dmask], 1u);
      }
    } else {
      for (int j = 0; j < cnt; ++j) {
        const uint32_t x = kr[base + j];
        if ((x & fixed) == prefix) atomicAdd(&hist[(x >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                     h3 = hist[4 * lane + 3];
      const int c = (int)(h0 + h1 + h2 + h3);
      int s = c;  // suffix sum: keys whose digit is >= 4 * lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int x = __shfl_down(s, off);
        if (lane + off < 64) s += x;
      }
      const unsigned long long ball = __ballot(s >= remaining);
      const int lx = 63 - __clzll(ball);
      if (lane == lx) {
        int above = s - c;
        const uint32_t hh[4] = {h0, h1, h2, h3};
        int dsel = 4 * lane;
        int need = remaining - above;
        int cntd = (int)h0;
        for (int e = 3; e >= 0; --e) {
          if (above + (int)hh[e] >= remaining) {
            dsel = 4 * lane + e;
            need = remaining - above;
            cntd = (int)hh[e];
            break;
          }
          above += (int)hh[e];
        }
        bc[0] = dsel;
        bc[1] = need;
        bc[2] = cntd;
      }
    }
    __syncthreads();
    const uint32_t dsel = (uint32_t)bc[0];
    remaining = bc[1];
    const int cntd = bc[2];
    prefix |= dsel << shift;
    fixed |= dmask << shift;
    top = shift - 1;
    if (remaining == cntd) break;  // the whole boundary bucket is taken
  }

  // Keys whose fixed bits exceed `prefix` are taken; of those equal to it, the
  // `remaining` lowest block ids.
  int cgt = 0, ceq = 0;
  for (int j = 0; j < cnt; ++j) {
    const uint32_t x = key_at(j) & fixed;
    cgt += x > prefix;
    ceq += x == prefix;
  }
  int tot;
  const int eq_before = block_exclusive_scan(ceq, lds_waves, tot);
  int eq_quota = remaining - eq_before;
  eq_quota = eq_quota < 0 ? 0 : (eq_quota > ceq ? ceq : eq_quota);
  const int out_before = block_exclusive_scan(cgt + eq_quota, lds_waves, tot);
  int pos = out_before;
  int eq_seen = 0;
  for (int j = 0; j < cnt; ++j) {
    const uint32_t x = key_at(j) & fixed;
    bool take = x > prefix;
    if (x == prefix) {
      take = eq_seen < eq_quota;
      ++eq_seen;
    }
    if (take) out[pos++] = base + j;
  }
}

}  // namespace

hipError_t launch_scores(const ScoreArgs& a, hipStream_t stream) {
  if (a.dtype == 0)
    return a.D == 128 ? launch_scores_t<bf16_t, 128>(a, stream) : launch_scores_t<bf16_t, 64>(a, stream);
  return a.D == 128 ? launch_scores_t<float, 128>(a, stream) : launch_scores_t<float, 64>(a, stream);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)a.H, (unsigned)a.R);
  const long long cand_max = a.max_blocks;
  if (cand_max <= 8LL * kSelThreads) {
    hipLaunchKernelGGL((select_kernel<8>), grid, dim3(kSelThreads), 0, stream, a.keys, a.seq_lens, a.sel_idx,
                       a.sel_cnt, a.H, a.max_blocks, a.max_sel, a.budget_num, a.budget_den, a.min_blocks,
                       a.local_blocks);
  } else if (cand_max <= 32LL * kSelThreads) {
    hipLaunchKernelGGL((select_kernel<32>), grid, dim3(kSelThreads), 0, stream, a.keys, a.seq_lens, a.sel_idx,
                       a.sel_cnt, a.H, a.max_blocks, a.max_sel, a.budget_num, a.budget_den, a.min_blocks,
                       a.local_blocks);
  } else {
    hipLaunchKernelGGL((select_kernel<0>), grid, dim3(kSelThreads), 0, stream, a.keys, a.seq_lens, a.sel_idx,
                       a.sel_cnt, a.H, a.max_blocks, a.max_sel, a.budget_num, a.budget_den, a.min_blocks,
                       a.local_blocks);
  }
  return hipGetLastError();
}

}  // namespace resa
