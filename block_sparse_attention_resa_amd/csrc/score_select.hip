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
// lanes own one descriptor and combine their partial sums with DPP row
// rotations.
// The thread -> (KV head, chunk) assignment is fixed for the whole kernel so
// the coefficients stay in registers.  Scores are written as order-preserving
// 32-bit keys for the selection kernel.
//
// Selection.  One 1024-thread workgroup per (request, KV head); thread t
// owns the consecutive candidate blocks [k t, k t + k) (16-byte loads, kept
// in registers; rows longer than 32768 blocks fall back to blocks t, t +
// 1024, ... re-read from memory).  The (n - n_local)-th largest key among
// the older blocks is found by histogram passes in LDS over monotone bin
// maps: the first pass bins the score range [min, max] into 2048
// equal-width bins, later passes (rarely needed) bin the key offsets inside
// the boundary bucket.  Once the boundary bucket holds at most 256 keys they
// are packed into LDS and ranked in parallel.  Blocks above the threshold
// are taken, blocks equal to it lowest index first, and one scan of the
// per-thread counts places every selected id in ascending order.
// Wave-wide scans and reductions use DPP lane shifts, and wavefronts whose
// keys are all candidates run every per-key loop without masks.
#include "desc_unit.h"
#include "resa_internal.h"

namespace resa {
namespace {

// ------------------------------------------------------------------ scores

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

constexpr int kScoreUnroll = 4;

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

template <typename T, int D, int MODE, int MAXG>
__global__ __launch_bounds__(1024) void score_kernel(const T* __restrict__ q, const T* desc,
                                                    const int32_t* __restrict__ table,
                                                    const int32_t* __restrict__ seq_lens,
                                                    uint32_t* __restrict__ keys, float* __restrict__ scores, int H,
                                                    int G, int max_blocks, int num_pool_blocks,
                                                    const T* __restrict__ k_pool, T* desc_tail, int score_wgs,
                                                    int key_stride) {
  using CL = ChunkLoad<T>;
  constexpr int VPL = CL::kVals;
  constexpr int CH = 2 * D / VPL;  // lanes per descriptor
  constexpr int HALF = CH / 2;     // lanes per descriptor row
  extern __shared__ float s_coef[];  // [H][2][D]: N (min row) then P (max row)

  const int r = blockIdx.y;
  const int t = threadIdx.x;
  if ((int)blockIdx.x >= score_wgs) {
    // Tail refresh: the extra workgroup recomputes the descriptor of each KV
    // head's last block (the block the newest token was appended to).  The
    // last block is always selected, so the score the other workgroups read
    // for it concurrently is never used.
    const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
    const int M = (L + kBlock - 1) / kBlock;
    if (M == 0) return;
    const int p = clampi(table[(size_t)r * max_blocks + M - 1], 0, num_pool_blocks - 1);
    for (int i = t >> 6; i < H; i += (int)(blockDim.x >> 6))
      descriptor_unit<T, D>(k_pool + ((size_t)p * H + i) * kBlock * D, desc_tail + ((size_t)p * H + i) * 2 * D,
                            L - (M - 1) * kBlock);
    return;
  }
  const int lane = t & 63;
  const int grp = t / CH;
  const int lg = t % CH;
  const int part = lg / HALF;  // 0: min row, 1: max row
  const int c0 = (lg % HALF) * VPL;
  const int head = grp % H;
  const int bsub = grp / H;
  const int bpi = blockDim.x / (CH * H);  // blocks per iteration
  const int wg_blocks = bpi * kScoreUnroll;
  const int wg_b0 = blockIdx.x * wg_blocks;
  uint32_t* key_row = keys + ((size_t)r * H + head) * key_stride;
  float* score_row = scores ? scores + ((size_t)r * H + head) * max_blocks : nullptr;

  // The request length (a scalar load) and the physical ids of this
  // workgroup's blocks (one coalesced load per wavefront, handed to the lanes
  // with a shuffle) are in flight together; the descriptor loads need both,
  // so skipping blocks past the sequence end costs no extra wait and no
  // descriptor past it is read (in a ragged batch the table is sized for the
  // longest request).
  const int seq_len = seq_lens[r];  // first used after the query loads are issued
  int my_pid = 0;
  if (lane < wg_blocks && wg_b0 + lane < max_blocks) my_pid = table[(size_t)r * max_blocks + wg_b0 + lane];
  // Load order matters: the in-order vector-memory counter makes a wait for
  // a load also wait for every load issued before it.  The table entries
  // (needed for the descriptor addresses) go out first, then the group's
  // query values, then the descriptor loads.  Every thread folds channel pairs of the
  // queries into P = sum_j max(q_j, 0) and N = sum_j min(q_j, 0) (MODE 0) or
  // the positive / negative part of the mean query (MODE 1); all G rows are
  // loaded before any is used (rows past G re-read row G-1 and are ignored).
  constexpr int kMaxG = MAXG;
  using Pair = typename CL::Pair;
  const int npairs = H * D / 2;
  const int nthr = blockDim.x;
  // This thread's first channel pair is loaded here; further pairs (only when
  // H*D/2 exceeds the workgroup size) are folded after the descriptor loads.
  Pair qv[kMaxG];
  {
    // branch-free (a thread past the last pair re-reads it), so no wait is
    // placed at a join before the descriptor loads
    const int v0 = t < npairs ? t : npairs - 1;
    const T* qh = q + ((size_t)r * H * G + (size_t)(v0 / (D / 2)) * G) * D + (v0 % (D / 2)) * 2;
#pragma unroll
    for (int j = 0; j < kMaxG; ++j) qv[j] = *reinterpret_cast<const Pair*>(qh + (size_t)min(j, G - 1) * D);
  }
  const int L = clampi(seq_len, 0, max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  uint4 buf[kScoreUnroll][2];
  int bl[kScoreUnroll];
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u) {
    const int bo = u * bpi + bsub;
    const int b = wg_b0 + bo;
    bl[u] = b;
    const int p = clampi(__shfl(my_pid, bo), 0, num_pool_blocks - 1);
    if (b < M) {
      const uint4* src = reinterpret_cast<const uint4*>(desc + (((size_t)p * H + head) * 2 + part) * D + c0);
      buf[u][0] = src[0];
      buf[u][1] = src[1];
    } else {
      buf[u][0] = make_uint4(0, 0, 0, 0);
      buf[u][1] = make_uint4(0, 0, 0, 0);
    }
  }
  for (int v = t; v < npairs; v += nthr) {
    const int hh = v / (D / 2);
    const int c = (v % (D / 2)) * 2;
    if (v != t) {  // rare: more channel pairs than threads
      const T* qh = q + ((size_t)r * H * G + (size_t)hh * G) * D + c;
#pragma unroll
      for (int j = 0; j < kMaxG; ++j) qv[j] = *reinterpret_cast<const Pair*>(qh + (size_t)min(j, G - 1) * D);
    }
    float p0 = 0.f, p1 = 0.f, n0 = 0.f, n1 = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxG; ++j) {
      float x0, x1;
      CL::unpack_pair(qv[j], x0, x1);
      x0 = j < G ? x0 : 0.f;
      x1 = j < G ? x1 : 0.f;
      if constexpr (MODE == 0) {
        p0 += fmaxf(x0, 0.f);
        p1 += fmaxf(x1, 0.f);
        n0 += fminf(x0, 0.f);
        n1 += fminf(x1, 0.f);
      } else {
        p0 += x0;
        p1 += x1;
      }
    }
    if constexpr (MODE != 0) {
      const float m0 = p0 / (float)G, m1 = p1 / (float)G;
      p0 = fmaxf(m0, 0.f);
      p1 = fmaxf(m1, 0.f);
      n0 = fminf(m0, 0.f);
      n1 = fminf(m1, 0.f);
    }
    s_coef[(hh * 2 + 0) * D + c] = n0;
    s_coef[(hh * 2 + 0) * D + c + 1] = n1;
    s_coef[(hh * 2 + 1) * D + c] = p0;
    s_coef[(hh * 2 + 1) * D + c + 1] = p1;
  }
  __syncthreads();
  float coef[VPL];
#pragma unroll
  for (int v = 0; v < VPL; v += 4) {
    const floatx4_t c4 = *reinterpret_cast<const floatx4_t*>(&s_coef[(head * 2 + part) * D + c0 + v]);
    coef[v] = c4[0];
    coef[v + 1] = c4[1];
    coef[v + 2] = c4[2];
    coef[v + 3] = c4[3];
  }

#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u) {
    float vals[VPL];
    CL::unpack(buf[u][0], buf[u][1], vals);
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) acc = fmaf(coef[v], vals[v], acc);
    acc = group_sum<CH>(acc);
    if (lg == 0 && bl[u] < M) {
      key_row[bl[u]] = f32_order_key(acc);
      if (score_row) score_row[bl[u]] = acc;
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
  while (unit * m * 2 <= 256 && m * 2 * kScoreUnroll <= 64) m *= 2;
  const int threads = unit * m;  // <= 1024 checked by the caller
  const int bpi = m;
  const int blocks_per_wg = bpi * kScoreUnroll;  // <= 64: one table entry per lane
  const int wgs = (a.max_blocks + blocks_per_wg - 1) / blocks_per_wg;
  const size_t lds = (size_t)a.H * 2 * D * sizeof(float);
  dim3 grid((unsigned)(wgs + (a.refresh_tail ? 1 : 0)), (unsigned)a.R);
#define RESA_SCORE_LAUNCH(MODE, MAXG)                                                                        \
  hipLaunchKernelGGL((score_kernel<T, D, MODE, MAXG>), grid, dim3(threads), lds, stream,                     \
                     static_cast<const T*>(a.q), static_cast<const T*>(a.desc_pool), a.table, a.seq_lens, a.keys, \
                     a.scores, a.H, a.G, a.max_blocks, a.num_pool_blocks, static_cast<const T*>(a.k_pool),  \
                     static_cast<T*>(const_cast<void*>(a.desc_pool)), wgs, a.key_stride)
  if (a.G <= 8) {
    if (a.mode == 0) RESA_SCORE_LAUNCH(0, 8);
    else RESA_SCORE_LAUNCH(1, 8);
  } else {
    if (a.mode == 0) RESA_SCORE_LAUNCH(0, 16);
    else RESA_SCORE_LAUNCH(1, 16);
  }
#undef RESA_SCORE_LAUNCH
  return hipGetLastError();
}

// ------------------------------------------------------------------ select

constexpr int kDigitBits = 11;  // histogram pass: 2048 bins
constexpr int kBins = 1 << kDigitBits;
constexpr int kFinishMax = 256;  // boundary bucket size the ranking finish takes (a multiple of 8)
static_assert(kFinishMax % 8 == 0, "the ranking reads the bucket eight keys at a time");

// Cross-lane steps through DPP (row shifts within 16-lane rows, then the
// row-15 / row-31 broadcasts), which stay in the vector ALU instead of the
// LDS crossbar.  Lanes that have no source receive `id`.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t id, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_sum(int x) {
  uint32_t v = (uint32_t)x;
  v += dpp_u32<0x111>(0u, v);  // row_shr:1
  v += dpp_u32<0x112>(0u, v);  // row_shr:2
  v += dpp_u32<0x114>(0u, v);  // row_shr:4
  v += dpp_u32<0x118>(0u, v);  // row_shr:8
  v += dpp_u32<0x142, 0xa>(0u, v);  // row_bcast:15 into rows 1 and 3
  v += dpp_u32<0x143, 0xc>(0u, v);  // row_bcast:31 into rows 2 and 3
  return (int)v;
}

// Minimum and maximum over the 64 lanes, returned in every lane.
__device__ __forceinline__ void wave_min_max(uint32_t& mn, uint32_t& mx) {
  mn = min(mn, dpp_u32<0x111>(0xffffffffu, mn));
  mx = max(mx, dpp_u32<0x111>(0u, mx));
  mn = min(mn, dpp_u32<0x112>(0xffffffffu, mn));
  mx = max(mx, dpp_u32<0x112>(0u, mx));
  mn = min(mn, dpp_u32<0x114>(0xffffffffu, mn));
  mx = max(mx, dpp_u32<0x114>(0u, mx));
  mn = min(mn, dpp_u32<0x118>(0xffffffffu, mn));
  mx = max(mx, dpp_u32<0x118>(0u, mx));
  mn = min(mn, dpp_u32<0x142, 0xa>(0xffffffffu, mn));
  mx = max(mx, dpp_u32<0x142, 0xa>(0u, mx));
  mn = min(mn, dpp_u32<0x143, 0xc>(0xffffffffu, mn));
  mx = max(mx, dpp_u32<0x143, 0xc>(0u, mx));
  mn = (uint32_t)__builtin_amdgcn_readlane((int)mn, 63);
  mx = (uint32_t)__builtin_amdgcn_readlane((int)mx, 63);
}

// Cross-wavefront exchange slots, two sets used alternately: a call writes
// its set, waits at one barrier and reads it; the next call of the same kind
// writes the other set, and the call after that can rewrite the first only
// after every thread has passed the intervening call's barrier, i.e. after
// every read of the first call.  So one barrier per call suffices.
template <typename V, int NW>
struct WaveSlots {
  V v[2][NW];
};

// Exclusive prefix sum over the workgroup in thread order; `total` gets the sum.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, WaveSlots<int, NT / 64>& slots, int& use, int& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int* lds_waves = slots.v[use];
  use ^= 1;
  const int incl = wave_incl_sum(v);
  if (lane == 63) lds_waves[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = lds_waves[w];
    before += w < wave ? x : 0;
    total += x;
  }
  return before + incl - v;
}

template <int NT>
__device__ __forceinline__ void block_min_max(uint32_t& mn, uint32_t& mx, WaveSlots<uint2, NT / 64>& slots,
                                              int& use) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint2* lds_mm = slots.v[use];
  use ^= 1;
  wave_min_max(mn, mx);
  if (lane == 0) lds_mm[wave] = make_uint2(mn, mx);
  __syncthreads();
  mn = 0xffffffffu;
  mx = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint2 x = lds_mm[w];
    mn = min(mn, x.x);
    mx = max(mx, x.y);
  }
}

// Candidate keys of one (request, KV head).  KPT > 0: thread t owns the KPT
// consecutive blocks [KPT t, KPT t + KPT), read with 16-byte loads before the
// request's length is known (the row is padded to a multiple of 4 entries and
// indices are clamped into it), so that a per-thread count and one scan give
// every selected block its place in the ascending output.  KPT == 0 (any
// size): thread t owns blocks t + NT j and re-reads the row.
template <int NT, int KPT>
struct KeyRuns {
  static_assert(KPT % 4 == 0, "keys are read four at a time");
  static_assert(KPT <= 32, "the member mask holds one bit per key");
  uint32_t reg[KPT > 0 ? KPT : 1];
  const uint32_t* row;
  int C, rounds;
  uint32_t in_mask;  // KPT > 0: bit j set when this thread's key j is a candidate
  bool full;         // KPT > 0, uniform over the wavefront: every key of every lane is a candidate
  bool any;          // KPT > 0, uniform over the wavefront: some lane holds a candidate
  __device__ void prefetch(const uint32_t* kr, int row_stride) {
    row = kr;
    if constexpr (KPT > 0) {
      const uint4* r4 = reinterpret_cast<const uint4*>(kr);
      const int last = row_stride / 4 - 1;
#pragma unroll
      for (int v = 0; v < KPT / 4; ++v) {
        const int idx = (int)threadIdx.x * (KPT / 4) + v;
        const uint4 x = r4[idx < last ? idx : last];
        reg[4 * v] = x.x;
        reg[4 * v + 1] = x.y;
        reg[4 * v + 2] = x.z;
        reg[4 * v + 3] = x.w;
      }
    }
  }
  __device__ void set_count(int c) {
    C = c;
    rounds = (c + NT - 1) / NT;
    if constexpr (KPT > 0) {
      const int mine = min(max(c - (int)threadIdx.x * KPT, 0), KPT);  // candidates among this thread's keys
      in_mask = mine >= 32 ? ~0u : (1u << mine) - 1u;
      full = __all(mine == KPT) != 0;
      any = __any(mine > 0) != 0;
    } else {
      full = false;
      any = true;
    }
  }
  __device__ bool valid(int j) const {
    if constexpr (KPT > 0) return (in_mask >> j) & 1u;
    else return j < rounds && (int)threadIdx.x + j * NT < C;
  }
  __device__ uint32_t key(int j) const {
    if constexpr (KPT > 0) return reg[j];
    else return row[threadIdx.x + j * NT];
  }
  __device__ int nrounds() const { return KPT > 0 ? KPT : rounds; }
};

// Runs the statements in the variadic argument for every round j of `kr`,
// with `in` telling whether the lane's key of that round is a candidate.  In
// wavefronts whose keys are all candidates (all but the last one or two of a
// row) `in` is the constant true, so those run the statements unmasked;
// wavefronts without a candidate skip them (every use is a no-op for a key
// that is not a candidate).  Expects NT, KPT and a KeyRuns `kr` in scope.
#define RESA_FOR_KEYS(...)                                                       \
  do {                                                                           \
    if constexpr (KPT > 0) {                                                     \
      if (kr.full) {                                                             \
        _Pragma("unroll") for (int j = 0; j < KPT; ++j) {                        \
          constexpr bool in = true;                                              \
          __VA_ARGS__                                                            \
        }                                                                        \
      } else if (kr.any) {                                                       \
        /* opaque copy: the per-key conditions are not kept across phases */    \
        uint32_t im_ = kr.in_mask;                                               \
        asm volatile("" : "+v"(im_));                                            \
        _Pragma("unroll") for (int j = 0; j < KPT; ++j) {                        \
          const bool in = (im_ >> j) & 1u;                                       \
          __VA_ARGS__                                                            \
        }                                                                        \
      }                                                                          \
    } else {                                                                     \
      for (int j = 0; j < kr.rounds; ++j) {                                      \
        const bool in = (int)threadIdx.x + j * NT < kr.C;                        \
        __VA_ARGS__                                                              \
      }                                                                          \
    }                                                                            \
  } while (0)

// Monotone map of a key onto kBins histogram bins, built for a bucket whose
// keys lie in [lo, hi] (keys outside are clamped to the end bins).  By value:
// bins of equal width in score, which spreads any finite score distribution
// evenly.  By key: the key offset shifted right, which always separates lo
// from hi and shrinks the range 2^11-fold per pass; over a range inside one
// sign and at most two binades it is within 2x of equal width in score and
// costs fewer instructions, so the first pass uses it there.
struct BinMap {
  bool by_value;
  float fmin, scale;
  uint32_t lo, hi;
  int shift;
  __device__ void init(uint32_t lo_key, uint32_t hi_key, bool allow_value) {
    lo = lo_key;
    hi = hi_key;
    const uint32_t d = hi_key - lo_key;
    const int nb = d ? 32 - __clz(d) : 0;
    shift = nb > kDigitBits ? nb - kDigitBits : 0;
    by_value = false;
    fmin = 0.f;
    scale = 0.f;
    // same sign and exponents at most one apart: key order is near-linear in score
    const bool narrow = ((lo_key ^ hi_key) >> 31) == 0u && ((hi_key >> 23) - (lo_key >> 23)) <= 1u;
    if (allow_value && !narrow) {
      const float a = __uint_as_float(u32_from_order_key(lo_key));
      const float b = __uint_as_float(u32_from_order_key(hi_key));
      const float range = b - a;
      const float s = (float)kBins / range;
      // lo lands in bin 0; hi must land in bin >= 1 so every pass makes progress
      if (__builtin_isfinite(a) && __builtin_isfinite(b) && __builtin_isfinite(range) && range > 0.f &&
          __builtin_isfinite(s) && range * s >= 1.f) {
        by_value = true;
        fmin = a;
        scale = s;
      }
    }
  }
  __device__ int value_bin(uint32_t key) const {
    const float f = __uint_as_float(u32_from_order_key(min(max(key, lo), hi)));
    const int b = (int)((f - fmin) * scale);
    return min(max(b, 0), kBins - 1);
  }
  __device__ int key_bin(uint32_t key) const { return (int)((min(max(key, lo), hi) - lo) >> shift); }
  // The same maps for a key known to lie in [lo, hi] (no clamping on that
  // side); any other key gives an unspecified bin.
  __device__ int value_bin_in(uint32_t key) const {
    const int b = (int)((__uint_as_float(u32_from_order_key(key)) - fmin) * scale);
    return min(b, kBins - 1);
  }
  __device__ int key_bin_in(uint32_t key) const { return (int)((key - lo) >> shift); }
  __device__ int operator()(uint32_t key) const { return by_value ? value_bin(key) : key_bin(key); }
};

// Candidates still in play: keys in [lo, hi] and, after a pass whose range was
// not re-measured, in histogram bin `bin` of `map`.
struct Bucket {
  uint32_t lo, hi;
  BinMap map;
  int bin;  // -1: no bin condition
  __device__ bool has(uint32_t x) const { return x >= lo && x <= hi && (bin < 0 || map(x) == bin); }
};

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void select_kernel(const uint32_t* __restrict__ keys,
                                                   const int32_t* __restrict__ seq_lens,
                                                   int32_t* __restrict__ sel_idx, int32_t* __restrict__ sel_cnt,
                                                   int H, int max_blocks, int max_sel, int budget_num,
                                                   int budget_den, int min_blocks, int local_blocks,
                                                   int key_stride) {
  constexpr int NW = NT / 64;
  constexpr int BPT = kBins / NT;                   // histogram bins per thread in the scan
  constexpr bool kKeepBins = KPT > 0 && KPT <= 16;  // first-pass bins kept in registers (16 bits each)
  static_assert(KPT <= 32, "member masks hold one bit per key");
  __shared__ uint32_t hist2[2][kBins + 1];  // alternating pass histograms; the last slot takes non-members
  __shared__ WaveSlots<int, NW> scan_slots;
  __shared__ WaveSlots<uint2, NW> mm_slots;
  int scan_use = 0, mm_use = 0;  // alternating slot sets, identical in every thread
  __shared__ __align__(16) uint32_t bucket[kFinishMax];
  __shared__ int bc2[2][3];  // boundary record of a pass (bin, rank left, keys), by pass parity
  __shared__ int packed;      // keys of the boundary bucket packed so far

  const int i = blockIdx.x;
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  KeyRuns<NT, KPT> kr;
  kr.prefetch(keys + ((size_t)r * H + i) * key_stride, key_stride);  // in flight with seq_lens
  const int L = clampi(seq_lens[r], 0, max_blocks * kBlock);
  const int M = (L + kBlock - 1) / kBlock;
  int32_t* out = sel_idx + ((size_t)r * H + i) * max_sel;

  int n = 0, nl = 0;
  if (M > 0) {
    long long nn = ((long long)M * budget_num + budget_den - 1) / budget_den;
    if (nn < min_blocks) nn = min_blocks;
    if (nn < local_blocks) nn = local_blocks;
    if (nn > M) nn = M;
    n = (int)nn;
    nl = local_blocks < M ? local_blocks : M;
  }
  const int k = n - nl;  // blocks chosen by score
  const int C = M - nl;  // candidates: blocks [0, C)
  for (int j = tid; j < max_sel; j += NT) {
    if (j >= n) out[j] = -1;
    else if (j >= k) out[j] = C + (j - k);  // forced recent blocks close the ascending list
  }
  if (tid == 0) sel_cnt[(size_t)r * H + i] = n;
  if (k == 0) return;
  if (k == C) {
    for (int j = tid; j < C; j += NT) out[j] = j;
    return;
  }

  kr.set_count(C);
  const int R = kr.nrounds();
  for (int b = tid; b <= kBins; b += NT) {  // published by the next barrier
    hist2[0][b] = 0u;
    hist2[1][b] = 0u;
  }
  if (tid == 0) packed = 0;

  // Key range of all candidates.
  uint32_t mn = 0xffffffffu, mx = 0u;
  RESA_FOR_KEYS({
    const uint32_t x = kr.key(j);
    mn = in ? min(mn, x) : mn;
    mx = in ? max(mx, x) : mx;
  });
  block_min_max<NT>(mn, mx, mm_slots, mm_use);

  Bucket bk;
  bk.lo = mn;
  bk.hi = mx;
  bk.bin = -1;
  bk.map.init(mn, mx, false);
  int remaining = k;  // keys still to take from the bucket
  int bucket_n = C;   // keys in the bucket
  uint32_t bins[kKeepBins ? KPT / 2 : 1];  // first-pass bin of every key, two per register
#pragma unroll
  for (int v = 0; v < (kKeepBins ? KPT / 2 : 1); ++v) bins[v] = (uint32_t)kBins | ((uint32_t)kBins << 16);

  // Histogram passes until the bucket holding the k-th largest key is small.
  int npass = 0;
  while (bucket_n > kFinishMax && remaining < bucket_n && bk.lo != bk.hi) {
    if (bk.bin >= 0) {  // re-measure the range of the previous pass's bucket
      uint32_t a = 0xffffffffu, b = 0u;
      RESA_FOR_KEYS({
        const uint32_t x = kr.key(j);
        const bool m = in && bk.has(x);
        a = m ? min(a, x) : a;
        b = m ? max(b, x) : b;
      });
      block_min_max<NT>(a, b, mm_slots, mm_use);
      bk.lo = a;
      bk.hi = b;
      bk.bin = -1;
      if (a == b) break;
    }
    BinMap map;
    map.init(bk.lo, bk.hi, npass == 0);
    uint32_t* hist = hist2[npass & 1];
    if (npass == 0) {  // every candidate is in the bucket
#define RESA_COUNT_KEY(BIN)                                         \
  {                                                                 \
    const int b = BIN;                                              \
    if (in) atomicAdd(&hist[b], 1u); /* constant in full waves */   \
    if constexpr (kKeepBins) {                                      \
      const uint32_t kept = in ? (uint32_t)b : (uint32_t)kBins;     \
      if (j & 1) bins[j / 2] |= kept << 16;                         \
      else bins[j / 2] = kept;                                      \
    }                                                               \
  }
      // every candidate lies in [min, max] of the candidates; the bins of the
      // others are not used
      if (map.by_value) RESA_FOR_KEYS(RESA_COUNT_KEY(map.value_bin_in(kr.key(j))));
      else RESA_FOR_KEYS(RESA_COUNT_KEY(map.key_bin_in(kr.key(j))));
#undef RESA_COUNT_KEY
    } else {
      RESA_FOR_KEYS({
        const uint32_t x = kr.key(j);
        if (in && bk.has(x)) atomicAdd(&hist[map(x)], 1u);
      });
    }
    __syncthreads();
    // Suffix counts: thread t owns bins [BPT*rt, BPT*rt + BPT) with rt = NT-1-t,
    // so an exclusive scan in thread order counts the keys in higher bins.
    const int rt = NT - 1 - tid;
    uint32_t hb[BPT];
    int c = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      hb[e] = hist[BPT * rt + e];
      c += (int)hb[e];
    }
    int tot;
    const int above0 = block_exclusive_scan<NT>(c, scan_slots, scan_use, tot);
    int* bc = bc2[npass & 1];
    // this pass's histogram is read; clear it for the pass after next
#pragma unroll
    for (int e = 0; e < BPT; ++e) hist[BPT * rt + e] = 0u;
    if (tid < (kBins + 1) - BPT * NT) hist[BPT * NT + tid] = 0u;
    if (above0 < remaining && above0 + c >= remaining) {
      int above = above0;
#pragma unroll
      for (int e = BPT - 1; e >= 0; --e) {
        if (above < remaining && above + (int)hb[e] >= remaining) {
          bc[0] = BPT * rt + e;
          bc[1] = remaining - above;
          bc[2] = (int)hb[e];
        }
        above += (int)hb[e];
      }
    }
    __syncthreads();
    bk.map = map;
    bk.bin = bc[0];
    remaining = bc[1];
    bucket_n = bc[2];
    ++npass;  // the next pass writes the other record, so no barrier is needed here
  }

  // The threshold: the remaining-th largest key of the bucket.  Keys above it
  // are taken; of the n_eq keys equal to it, the `take_eq` lowest block ids.
  uint32_t thr;
  int take_eq, n_eq;
  if (bk.lo == bk.hi) {  // every key in the bucket is equal
    thr = bk.lo;
    take_eq = remaining;
    n_eq = bucket_n;
  } else if (bucket_n <= kFinishMax) {
    // Ranking finish: the bucket's keys are packed into LDS (slots handed out
    // by an LDS counter: their order does not matter), then each member
    // counts the members above and equal to it; the one whose rank range
    // holds `remaining` is the threshold.
    const bool kept = kKeepBins && npass == 1;
    if constexpr (KPT > 0) {
      // members as a bit mask (after one pass, from the kept bins, where
      // non-candidates hold kBins, which is no bucket's bin)
      uint32_t mem = 0;
      bool by_kept = false;
      if constexpr (kKeepBins) by_kept = kept;
      if (by_kept) {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
          mem |= (((bins[j / 2] >> (16 * (j & 1))) & 0xffffu) == (uint32_t)bk.bin ? 1u : 0u) << j;
      } else {
        RESA_FOR_KEYS({ mem |= (in && bk.has(kr.key(j)) ? 1u : 0u) << j; });
      }
      // Slots: one LDS atomic per wavefront that holds members; each lane's
      // members follow those of the lanes before it.  Keys of a round that
      // holds no member in the wavefront are skipped as a whole.
      if (__ballot(mem != 0u)) {
        const int cnt = __popc(mem);
        const int incl = wave_incl_sum(cnt);
        int base = 0;
        if ((tid & 63) == 63) base = atomicAdd(&packed, incl);
        int pos = __builtin_amdgcn_readlane(base, 63) + incl - cnt;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const bool b = (mem >> j) & 1u;
          if (__ballot(b)) {
            if (b && pos < kFinishMax) bucket[pos] = kr.key(j);
            pos += b ? 1 : 0;
          }
        }
      }
    } else {
      RESA_FOR_KEYS({
        if (in && bk.has(kr.key(j))) {
          const int pos = atomicAdd(&packed, 1);
          if (pos < kFinishMax) bucket[pos] = kr.key(j);
        }
      });
    }
    __syncthreads();
    const int nb = bucket_n;  // the members counted by the last pass
    int* bc = bc2[npass & 1];  // the record the last pass did not use
    if (tid < nb) {
      const uint32_t x = bucket[tid];
      int gt = 0, eq = 0;
      // four members per LDS read, two reads in flight (slots past nb are masked)
      const uint4* b4 = reinterpret_cast<const uint4*>(bucket);
      for (int q = 0; q < nb; q += 8) {
        const uint4 ya = b4[q / 4];
        const uint4 yb = b4[q / 4 + 1];  // q + 7 < kFinishMax: kFinishMax is a multiple of 8
        const uint32_t y[8] = {ya.x, ya.y, ya.z, ya.w, yb.x, yb.y, yb.z, yb.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool ok = q + e < nb;
          gt += ok && y[e] > x ? 1 : 0;
          eq += ok && y[e] == x ? 1 : 0;
        }
      }
      if (gt < remaining && remaining <= gt + eq) {  // every writer stores the same values
        bc[0] = (int)x;
        bc[1] = remaining - gt;
        bc[2] = eq;
      }
    }
    __syncthreads();
    thr = (uint32_t)bc[0];
    take_eq = bc[1];
    n_eq = bc[2];
  } else {
    // remaining == bucket_n: the whole bucket is taken; the threshold is its
    // smallest key and every key equal to it lies in the bucket.
    uint32_t a = 0xffffffffu, b = 0u;
    RESA_FOR_KEYS({
      const uint32_t x = kr.key(j);
      a = (in && bk.has(x)) ? min(a, x) : a;
    });
    block_min_max<NT>(a, b, mm_slots, mm_use);
    thr = a;
    take_eq = bucket_n;
    n_eq = bucket_n;
  }

  // Output in ascending block order.  Each thread's keys are consecutive
  // blocks, so one scan of the per-thread counts gives every thread its first
  // output position; ties at the threshold are ranked the same way.
  const bool ties = take_eq < n_eq;
  if constexpr (KPT > 0) {
    uint32_t take = 0;
    if (!ties) {  // every key at or above the threshold
      RESA_FOR_KEYS({ take |= (in && kr.key(j) >= thr ? 1u : 0u) << j; });
    } else {  // of the keys equal to the threshold, the take_eq lowest block ids
      uint32_t equal = 0;
      RESA_FOR_KEYS({
        const uint32_t x = kr.key(j);
        take |= (in && x > thr ? 1u : 0u) << j;
        equal |= (in && x == thr ? 1u : 0u) << j;
      });
      int n_all;
      int room = take_eq - block_exclusive_scan<NT>(__popc(equal), scan_slots, scan_use, n_all);
      for (uint32_t m = equal; m != 0u && room > 0; m &= m - 1u, --room) take |= m & (~m + 1u);
    }
    int tot;
    int pos = block_exclusive_scan<NT>(__popc(take), scan_slots, scan_use, tot);
    const int first = tid * KPT;
    for (uint32_t m = take; m != 0u; m &= m - 1u, ++pos)
      if (pos < k) out[pos] = first + __builtin_ctz(m);
  } else {
    // Any number of rounds: one block scan per round.
    int base_out = 0, base_eq = 0;
    for (int j = 0; j < R; ++j) {
      const bool v = kr.valid(j);
      const uint32_t x = kr.key(j);
      const bool is_eq = v && x == thr;
      int tot_eq;
      const int eq_before = block_exclusive_scan<NT>(is_eq ? 1 : 0, scan_slots, scan_use, tot_eq);
      const bool t = (v && x > thr) || (is_eq && (!ties || base_eq + eq_before < take_eq));
      int tot;
      const int pos = block_exclusive_scan<NT>(t ? 1 : 0, scan_slots, scan_use, tot);
      if (t && base_out + pos < k) out[base_out + pos] = tid + j * NT;
      base_out += tot;
      base_eq += tot_eq;
    }
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
#define RESA_SELECT_LAUNCH(NT, KPT)                                                                          \
  hipLaunchKernelGGL((select_kernel<NT, KPT>), grid, dim3(NT), 0, stream, a.keys, a.seq_lens, a.sel_idx,      \
                     a.sel_cnt, a.H, a.max_blocks, a.max_sel, a.budget_num, a.budget_den, a.min_blocks,      \
                     a.local_blocks, a.key_stride)
  // 16 wavefronts: the select is latency-bound on one CU, and more resident
  // wavefronts hide more of it than fewer, longer ones (measured).
  if (cand_max <= 8LL * 1024) RESA_SELECT_LAUNCH(1024, 8);
  else if (cand_max <= 16LL * 1024) RESA_SELECT_LAUNCH(1024, 16);
  else if (cand_max <= 32LL * 1024) RESA_SELECT_LAUNCH(1024, 32);
  else RESA_SELECT_LAUNCH(1024, 0);
#undef RESA_SELECT_LAUNCH
  return hipGetLastError();
}

}  // namespace resa
