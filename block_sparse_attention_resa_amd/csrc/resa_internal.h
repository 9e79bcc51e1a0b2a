// Internal declarations shared by the libresa translation units: device
// helpers (bf16 handling, order-preserving keys, MFMA operand types) and the
// host-side launchers each kernel file exports to the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace resa {

constexpr int kBlock = 16;       // tokens per KV block
constexpr int kMaxSplits = 1024;  // upper bound on the split count of one call
constexpr int kDecodeWaves = 8;   // wavefronts per decode workgroup

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short short4_t;
typedef __attribute__((ext_vector_type(4))) float floatx4_t;

struct bf16_t {
  uint16_t bits;
};

// ----------------------------------------------------------------- scalars

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__device__ __forceinline__ float bf16_lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Order-preserving maps to unsigned integers: a < b as floats (with -0 < +0)
// iff key(a) < key(b) as unsigned integers.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t u32_order_key(uint32_t u) {
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t u32_from_order_key(uint32_t k) {
  return (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
}
__device__ __forceinline__ uint32_t bf16_order_key(uint32_t h) {  // h: 16-bit pattern
  return (h & 0x8000u) ? (~h & 0xffffu) : (h | 0x8000u);
}
__device__ __forceinline__ uint32_t bf16_from_order_key(uint32_t k) {
  return (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
}

// ----------------------------------------------------------------- launchers
// Each launcher enqueues on `stream` and returns hipGetLastError()'s result.

struct DescArgs {
  const void* k_pool;
  void* desc_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  const int32_t* first_block;  // nullable
  int32_t num_blocks;          // range selector, see resa_build_descriptors
  int32_t window;              // > 0: blocks floor((L-window)/16) .. M-1 (rectify)
  int32_t R, H, D, dtype, max_blocks, num_pool_blocks;
};
hipError_t launch_descriptors(const DescArgs& a, hipStream_t stream);

// Scoring and selection of resa_score_select.
struct ScoreArgs {
  const void* q;
  const void* desc_pool;  // also written (tail block) when refresh_tail
  const void* k_pool;     // read when refresh_tail
  int32_t refresh_tail;
  const int32_t* table;
  const int32_t* seq_lens;
  uint32_t* keys;  // [R][H][key_stride] workspace
  float* scores;   // nullable export [R][H][max_blocks]
  int32_t* sel_idx;
  int32_t* sel_cnt;
  int32_t R, H, G, D, dtype, max_blocks, num_pool_blocks, mode;
  int32_t key_stride;  // key_stride_for(max_blocks)
  int32_t max_sel, budget_num, budget_den, min_blocks, local_blocks;
};
// The scoring launch, then the selection launch.
hipError_t launch_score_select(const ScoreArgs& a, hipStream_t stream);

// Row stride of the score keys: a multiple of 4 entries, so every row starts
// 16-byte aligned and the selection can read its keys with 16-byte loads.
inline int key_stride_for(int max_blocks) { return (max_blocks + 3) & ~3; }

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  const int32_t* sel_idx;  // null for dense
  const int32_t* sel_cnt;  // null for dense
  int32_t max_sel;
  float* out;
  float* part_o;       // [R][H][S][G][D]
  float* part_ml;      // [R][H][S][G][2]
  int32_t R, H, G, D, dtype, max_blocks, num_pool_blocks, splits;
  float scale_log2;  // sm_scale * log2(e)
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// The two launches of resa_score_select on their own.
hipError_t launch_scores(const ScoreArgs& a, hipStream_t stream);
hipError_t launch_select(const ScoreArgs& a, hipStream_t stream);

// One decode step of one layer (resa_sparse_step): the scoring launch, then
// the selection fused with the split attention, then the merge of the
// splits.  `sa` carries the scoring and selection arguments (sel_idx,
// sel_cnt, keys), `da` the attention's (splits, partials, out).  Whether
// the fused launch serves these sizes (else the selection launch and the
// decode launch run in its place):
bool step_fused(int dtype, int key_stride, int max_sel, int splits, long long rows);
hipError_t launch_step(const ScoreArgs& sa, const DecodeArgs& da, hipStream_t stream);

// Log-sum-exp merge of split partials: out row (r, t, i*G + j) from
// part_o / part_ml rows ((r*H + i)*S + s)*rows_per_head + t*G + j.
hipError_t launch_merge(const float* part_o, const float* part_ml, float* out, int R, int H, int G, int D, int S,
                        int rows_per_head, int row_stride_out, hipStream_t stream);

struct RectifyArgs {
  const void* q_chunk;
  const void* k_new;
  const void* v_new;
  void* k_pool;
  void* v_pool;
  void* desc_pool;
  const int32_t* table;
  const int32_t* seq_lens;
  float* out;
  float* part_o;   // [R][H][S][chunk*G][D]
  float* part_ml;  // [R][H][S][chunk*G][2]
  int32_t R, H, G, D, dtype, max_blocks, num_pool_blocks, chunk, splits;
  float scale_log2;
};
hipError_t launch_rectify(const RectifyArgs& a, hipStream_t stream);

}  // namespace resa
