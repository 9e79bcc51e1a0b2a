// Top-n block selection over order-preserving 32-bit score keys, run by one
// workgroup per (request, KV head).
//
// "Rectified Sparse Attention" analysis page (paper-graph-ui), §3.4.1 Eq 5
// (the n - n_local highest-scoring older blocks; ties here go to the lower
// block id).
//
// Thread t owns the consecutive candidate blocks [k t, k t + k) (16-byte
// loads, kept in registers; rows longer than 32 keys per thread fall back to
// blocks t, t + NT, ... re-read from memory).  The k-th largest key is found by
// histogram passes in LDS over monotone bin maps: the first pass bins the
// candidates' range into 4096 equal-width bins, later passes (rarely needed)
// bin the key offsets inside the boundary bucket.  Once the boundary bucket
// holds at most 256 keys they are packed into LDS and each is ranked against
// all of them by one thread.  Blocks above the threshold are taken, blocks equal to it
// lowest index first, and one scan of the per-thread counts places every
// selected id in ascending order.  Wave-wide scans and reductions use DPP
// lane shifts, and wavefronts whose keys are all candidates run every
// per-key loop without masks.
#pragma once

#include "resa_internal.h"

namespace resa {

constexpr int kDigitBits = 12;  // histogram pass: 4096 bins
constexpr int kBins = 1 << kDigitBits;
constexpr int kFinishMax = 256;  // boundary bucket size the ranking finish takes

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
  // The keys were written by an earlier launch (the launch boundary has made
  // them visible), so they are read with plain 16-byte loads.
  __device__ void prefetch(const uint32_t* kr, int row_stride) {
    row = kr;
    if constexpr (KPT > 0) {
      const int last = row_stride / 4 - 1;
#pragma unroll
      for (int v = 0; v < KPT / 4; ++v) {
        const int idx = (int)threadIdx.x * (KPT / 4) + v;
        const int q = idx < last ? idx : last;
        const uint4 x = *reinterpret_cast<const uint4*>(kr + 4 * q);
        reg[4 * v] = x.x;
        reg[4 * v + 1] = x.y;
        reg[4 * v + 2] = x.z;
        reg[4 * v + 3] = x.w;
      }
    }
  }
  // KPT > 0: keys [KPT t, KPT t + KPT) of an LDS array of at least NT * KPT
  // entries (entries past the count are ignored).
  __device__ void load_lds(const uint32_t* keys) {
    static_assert(KPT > 0, "register-held keys only");
    row = keys;
#pragma unroll
    for (int v = 0; v < KPT / 4; ++v) {
      const uint4 x = *reinterpret_cast<const uint4*>(keys + ((int)threadIdx.x * (KPT / 4) + v) * 4);
      reg[4 * v] = x.x;
      reg[4 * v + 1] = x.y;
      reg[4 * v + 2] = x.z;
      reg[4 * v + 3] = x.w;
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

// LDS of the selection by an NT-thread workgroup.
template <int NT>
struct SelectLds {
  // alternating pass histograms; slot kBins takes non-members (rows padded
  // to keep the second one 16-byte aligned for the scan's vector reads)
  __align__(16) uint32_t hist2[2][kBins + 4];
  WaveSlots<int, NT / 64> scan_slots;
  WaveSlots<uint2, NT / 64> mm_slots;
  __align__(16) uint32_t bucket[kFinishMax + 8];  // read eight at a time
  int bc2[2][3];  // boundary record of a pass (bin, rank left, keys), by pass parity
  int packed;     // keys of the boundary bucket packed so far
};

// The k-th largest key `thr` of a row: every key above it is selected, and
// of the n_eq keys equal to it the take_eq lowest block ids.
struct Threshold {
  uint32_t thr;
  int take_eq, n_eq;
};

// Threshold of the top-k of the C candidate keys of one row (k in (0, C))
// held by `kr` (prefetched, count set), whose range [mn, mx] is known.
// Expects the two histograms and `packed` cleared and published by a
// barrier.  `scan_use` carries the parity of the exchange slots to the
// caller's later scans.  Every thread of the workgroup calls it.
template <int NT, int KPT>
__device__ __forceinline__ Threshold select_threshold(SelectLds<NT>& sl, KeyRuns<NT, KPT>& kr, int C, int k,
                                                      uint32_t mn, uint32_t mx, int& scan_use) {
  constexpr int BPT = kBins / NT;                   // histogram bins per thread in the scan (2, 4 or 8)
  constexpr bool kKeepBins = KPT > 0 && KPT * NT <= 16 * 1024;  // first-pass bins kept in registers (16 bits each)
  static_assert(BPT == 2 || BPT == 4 || BPT == 8, "the scan reads two, four or eight bins per thread");
  int mm_use = 0;  // alternating slot sets, identical in every thread
  const int tid = threadIdx.x;

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
      block_min_max<NT>(a, b, sl.mm_slots, mm_use);
      bk.lo = a;
      bk.hi = b;
      bk.bin = -1;
      if (a == b) break;
    }
    BinMap map;
    map.init(bk.lo, bk.hi, npass == 0);
    uint32_t* hist = sl.hist2[npass & 1];
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
      // every candidate lies in [min, max] of the candidates
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
    if constexpr (BPT == 2) {
      const uint2 h2 = *reinterpret_cast<const uint2*>(&hist[BPT * rt]);
      hb[0] = h2.x;
      hb[1] = h2.y;
      c = (int)(h2.x + h2.y);
    } else {
#pragma unroll
      for (int e = 0; e < BPT; e += 4) {
        const uint4 h4 = *reinterpret_cast<const uint4*>(&hist[BPT * rt + e]);
        hb[e] = h4.x;
        hb[e + 1] = h4.y;
        hb[e + 2] = h4.z;
        hb[e + 3] = h4.w;
        c += (int)(h4.x + h4.y + h4.z + h4.w);
      }
    }
    int tot;
    const int above0 = block_exclusive_scan<NT>(c, sl.scan_slots, scan_use, tot);
    int* bc = sl.bc2[npass & 1];
    // this pass's histogram is read; clear it for the pass after next
    if constexpr (BPT == 2) {
      *reinterpret_cast<uint2*>(&hist[BPT * rt]) = make_uint2(0u, 0u);
    } else {
#pragma unroll
      for (int e = 0; e < BPT; e += 4) *reinterpret_cast<uint4*>(&hist[BPT * rt + e]) = make_uint4(0u, 0u, 0u, 0u);
    }
    if (tid == 0) hist[kBins] = 0u;
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
    // Ranking finish: the bucket's keys are packed into LDS (their order does
    // not matter), then thread m ranks
    // member m against all of them; the member whose rank range holds
    // `remaining` is the threshold.
    bool kept = false;
    if constexpr (kKeepBins) kept = npass == 1;
    if constexpr (KPT > 0) {
      // members as a bit mask (after one pass, from the kept bins, where
      // non-candidates hold kBins, which is no bucket's bin); the few lanes
      // that hold members claim slots one by one
      uint32_t mem = 0;
      if (kept) {
        const uint32_t b2 = (uint32_t)bk.bin | ((uint32_t)bk.bin << 16);
#pragma unroll
        for (int j = 0; j < KPT; j += 2) {
          const uint32_t x = bins[j / 2] ^ b2;
          mem |= ((x & 0xffffu) == 0u ? 1u : 0u) << j;
          mem |= ((x >> 16) == 0u ? 2u : 0u) << j;
        }
      } else {
        RESA_FOR_KEYS({ mem |= (in && bk.has(kr.key(j)) ? 1u : 0u) << j; });
      }
      // Slots: one LDS atomic per wavefront that holds members (a lane per
      // member would serialise on the one counter); each lane's members
      // follow those of the lanes before it.  Wavefronts without a member,
      // and rounds without one in the wavefront, are skipped as a whole.
      if (__ballot(mem != 0u)) {
        const int cnt = __popc(mem);
        const int incl = wave_incl_sum(cnt);
        int base = 0;
        if ((tid & 63) == 63) base = atomicAdd(&sl.packed, incl);
        int pos = __builtin_amdgcn_readlane(base, 63) + incl - cnt;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const bool b = (mem >> j) & 1u;
          if (__ballot(b)) {
            if (b && pos < kFinishMax) sl.bucket[pos] = kr.key(j);
            pos += b ? 1 : 0;
          }
        }
      }
    } else {
      RESA_FOR_KEYS({
        if (in && bk.has(kr.key(j))) {
          const int pos = atomicAdd(&sl.packed, 1);
          if (pos < kFinishMax) sl.bucket[pos] = kr.key(j);
        }
      });
    }
    __syncthreads();
    const int nb = bucket_n;  // the members counted by the last pass
    int* bc = sl.bc2[npass & 1];  // the record the last pass did not use
    static_assert(kFinishMax <= NT, "one bucket member per thread");
    if (tid < nb) {
      // member tid against every member, eight per step (two 16-byte reads
      // that every lane makes alike)
      const uint32_t x = sl.bucket[tid];
      int gt = 0, eq = 0;
      for (int s0 = 0; s0 < nb; s0 += 8) {
        const uint4 a = *reinterpret_cast<const uint4*>(&sl.bucket[s0]);
        const uint4 b = *reinterpret_cast<const uint4*>(&sl.bucket[s0 + 4]);
        const uint32_t y[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool in = s0 + e < nb;
          gt += in && y[e] > x ? 1 : 0;
          eq += in && y[e] == x ? 1 : 0;
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
    block_min_max<NT>(a, b, sl.mm_slots, mm_use);
    thr = a;
    take_eq = bucket_n;
    n_eq = bucket_n;
  }
  return Threshold{thr, take_eq, n_eq};
}

// Position, in the key order of `kr`, of the take_eq-th key equal to thr
// (take_eq >= 1 of them exist).  Every thread calls it and gets the result.
template <int NT, int KPT>
__device__ __forceinline__ int cut_position(SelectLds<NT>& sl, KeyRuns<NT, KPT>& kr, uint32_t thr, int take_eq,
                                            int& scan_use) {
  const int tid = threadIdx.x;
  int* res = &sl.bc2[0][0];
  if constexpr (KPT > 0) {
    uint32_t equal = 0;
    RESA_FOR_KEYS({ equal |= (in && kr.key(j) == thr ? 1u : 0u) << j; });
    int n_all;
    const int before = block_exclusive_scan<NT>(__popc(equal), sl.scan_slots, scan_use, n_all);
    if (before < take_eq && take_eq <= before + __popc(equal)) {
      uint32_t m = equal;
      for (int q = before + 1; q < take_eq; ++q) m &= m - 1u;
      *res = tid * KPT + __builtin_ctz(m);
    }
  } else {
    int base = 0;
    for (int j = 0; j < kr.rounds; ++j) {
      const bool e = kr.valid(j) && kr.key(j) == thr;
      int tot;
      const int pos = block_exclusive_scan<NT>(e ? 1 : 0, sl.scan_slots, scan_use, tot);
      if (e && base + pos + 1 == take_eq) *res = tid + j * NT;
      base += tot;
    }
  }
  __syncthreads();
  return *res;
}

// The keys this thread takes of a row's top-k (register-held keys, KPT > 0):
// bit j of `take` is set when block KPT t + j is selected, and `pos` is the
// place of the first of them in the ascending list of the k selected ids
// (the others follow it in bit order).  Each thread's keys are consecutive
// blocks, so one scan of the per-thread counts gives every thread its first
// output position; ties at the threshold are ranked the same way.  Every
// thread of the workgroup calls it.
template <int NT, int KPT>
__device__ __forceinline__ void select_take(SelectLds<NT>& sl, KeyRuns<NT, KPT>& kr, const Threshold& th,
                                            int& scan_use, uint32_t& take, int& pos) {
  static_assert(KPT > 0, "register-held keys only");
  const uint32_t thr = th.thr;
  const bool ties = th.take_eq < th.n_eq;
  take = 0;
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
    int room = th.take_eq - block_exclusive_scan<NT>(__popc(equal), sl.scan_slots, scan_use, n_all);
    for (uint32_t m = equal; m != 0u && room > 0; m &= m - 1u, --room) take |= m & (~m + 1u);
  }
  int tot;
  pos = block_exclusive_scan<NT>(__popc(take), sl.scan_slots, scan_use, tot);
}

// Top-k of the C candidate keys of one row (k in (0, C)) held by `kr`
// (prefetched, count set), whose range [mn, mx] is known: writes the k
// selected block ids, ascending, to out.  Expects the two histograms and
// `packed` cleared and published by a barrier.  Every thread of the
// workgroup calls it.
template <int NT, int KPT>
__device__ __forceinline__ void select_top(SelectLds<NT>& sl, KeyRuns<NT, KPT>& kr, int C, int k, uint32_t mn,
                                           uint32_t mx, int32_t* __restrict__ out) {
  int scan_use = 0;
  const int tid = threadIdx.x;
  const Threshold th = select_threshold<NT, KPT>(sl, kr, C, k, mn, mx, scan_use);

  // Output in ascending block order.
  if constexpr (KPT > 0) {
    uint32_t take;
    int pos;
    select_take<NT, KPT>(sl, kr, th, scan_use, take, pos);
    const int first = tid * KPT;
    for (uint32_t m = take; m != 0u; m &= m - 1u, ++pos)
      if (pos < k) out[pos] = first + __builtin_ctz(m);
  } else {
    // Any number of rounds: one block scan per round.
    const uint32_t thr = th.thr;
    const int take_eq = th.take_eq;
    const bool ties = take_eq < th.n_eq;
    const int R = kr.nrounds();
    int base_out = 0, base_eq = 0;
    for (int j = 0; j < R; ++j) {
      const bool v = kr.valid(j);
      const uint32_t x = kr.key(j);
      const bool is_eq = v && x == thr;
      int tot_eq;
      const int eq_before = block_exclusive_scan<NT>(is_eq ? 1 : 0, sl.scan_slots, scan_use, tot_eq);
      const bool t = (v && x > thr) || (is_eq && (!ties || base_eq + eq_before < take_eq));
      int tot;
      const int pos = block_exclusive_scan<NT>(t ? 1 : 0, sl.scan_slots, scan_use, tot);
      if (t && base_out + pos < k) out[base_out + pos] = tid + j * NT;
      base_out += tot;
      base_eq += tot_eq;
    }
  }
}

}  // namespace resa
