// C ABI of libresa: argument checks, workspace layout, split counts and the
// kernel launch sequence of each call.  Every check runs on the host before
// anything is enqueued; nothing here allocates, synchronises or prints.
#include <math.h>

#include <atomic>
#include <mutex>

#include "../../include/resa.h"
#include "resa_internal.h"

namespace {

using namespace resa;

constexpr size_t kAlign = 256;
constexpr int kMaxChunk = 256;
constexpr int kMaxBlocksLimit = 1 << 26;  // keeps max_blocks * 16 within int32

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

resa_status check_config(const resa_config* c) {
  if (!c) return RESA_ERR_INVALID_ARG;
  if (c->num_kv_heads < 1 || c->group_size < 1 || c->budget_den < 1 || c->budget_num < 1 ||
      c->budget_num > c->budget_den || c->min_blocks < 0 || c->local_blocks < 1 || c->num_splits < 0 ||
      !(c->sm_scale > 0.f) || !isfinite(c->sm_scale))
    return RESA_ERR_INVALID_ARG;
  if (c->dtype != RESA_BF16 && c->dtype != RESA_F32) return RESA_ERR_INVALID_ARG;
  if (c->score_mode != RESA_SCORE_SUM_HEADS && c->score_mode != RESA_SCORE_MEAN_POOL) return RESA_ERR_INVALID_ARG;
  if (c->block_size != kBlock) return RESA_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return RESA_ERR_UNSUPPORTED;
  if (c->group_size > 16) return RESA_ERR_UNSUPPORTED;  // one 16-column MFMA tile per KV head
  if (c->num_kv_heads > 65535) return RESA_ERR_UNSUPPORTED;
  return RESA_OK;
}

resa_status check_kv(const resa_paged_kv* kv, bool need_k, bool need_v, bool need_desc) {
  if (!kv || !kv->block_table || !kv->seq_lens) return RESA_ERR_INVALID_ARG;
  if (kv->num_pool_blocks < 1 || kv->max_blocks < 1) return RESA_ERR_INVALID_ARG;
  if (kv->max_blocks > kMaxBlocksLimit) return RESA_ERR_UNSUPPORTED;
  if (need_k && (!kv->k_pool || !aligned16(kv->k_pool))) return RESA_ERR_INVALID_ARG;
  if (need_v && (!kv->v_pool || !aligned16(kv->v_pool))) return RESA_ERR_INVALID_ARG;
  if (need_desc && (!kv->desc_pool || !aligned16(kv->desc_pool))) return RESA_ERR_INVALID_ARG;
  return RESA_OK;
}

resa_status check_requests(int32_t R) {
  if (R < 0) return RESA_ERR_INVALID_ARG;
  if (R > 65535) return RESA_ERR_UNSUPPORTED;
  return RESA_OK;
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

int selection_count(const resa_config* c, long long M) {
  if (M <= 0) return 0;
  long long n = (M * c->budget_num + c->budget_den - 1) / c->budget_den;
  if (n < c->min_blocks) n = c->min_blocks;
  if (n < c->local_blocks) n = c->local_blocks;
  if (n > M) n = M;
  return (int)n;
}

// Splits per (request, KV head).  The automatic choice aims at about two
// workgroups per compute unit of the 256-CU MI355X for decode, four for the
// rectification kernel, without letting a workgroup's share drop below a few
// blocks per wavefront.  It depends only on the arguments, so results are
// reproducible run to run.
int splits_for(const resa_config* c, int op, int R, int max_blocks, int max_sel, int chunk) {
  const long long units = (long long)R * c->num_kv_heads;
  long long len, target, min_share;
  if (op == RESA_OP_SPARSE_DECODE) {
    len = max_sel;
    target = 256;  // 8-wavefront workgroups: about one per CU
    // at least four list positions per split: on short lists more splits
    // (half a block per wavefront) still shorten the call (16K: 9.3 -> 8.7 us)
    min_share = kDecodeWaves / 2;
  } else if (op == RESA_OP_DENSE_DECODE) {
    len = max_blocks;
    target = 256;
    min_share = 8 * kDecodeWaves;
  } else if (c->dtype == RESA_BF16) {  // rectify, 256 query rows per workgroup: about one per CU
    const long long rg = ceil_div((long long)chunk * c->group_size, 256);
    len = max_blocks;
    target = 256 / (rg > 0 ? rg : 1);
    min_share = 32;
    // a split keeps the physical ids of its blocks in LDS: at most 2048 of them
    const long long units_all = units > 0 ? units : 1;
    if (target < units_all * ceil_div(max_blocks, 2048)) target = units_all * ceil_div(max_blocks, 2048);
  } else {  // rectify, fp32: 64 query rows per workgroup
    const long long rg = ceil_div((long long)chunk * c->group_size, 64);
    len = max_blocks;
    target = 1024 / (rg > 0 ? rg : 1);
    min_share = 32;
  }
  if (len < 1) len = 1;
  long long s;
  if (c->num_splits > 0) {
    s = c->num_splits;
  } else {
    s = units > 0 ? (target + units - 1) / units : 1;
    const long long cap = (len + min_share - 1) / min_share;
    if (s > cap) s = cap;
  }
  if (s > len) s = len;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  return (int)s;
}

size_t partial_bytes(const resa_config* c, int R, int S, long long rows_per_head) {
  const size_t rows = (size_t)R * c->num_kv_heads * S * rows_per_head;
  return align_up(rows * c->head_dim * sizeof(float)) + align_up(rows * 2 * sizeof(float));
}

size_t workspace_bytes(const resa_config* c, int op, int R, int max_blocks, int max_sel, int chunk) {
  switch (op) {
    case RESA_OP_SCORE_SELECT:  // the score keys
      return align_up((size_t)R * c->num_kv_heads * key_stride_for(max_blocks) * sizeof(uint32_t));
    case RESA_OP_SPARSE_DECODE:
    case RESA_OP_DENSE_DECODE: {
      const int S = splits_for(c, op, R, max_blocks, max_sel, chunk);
      return partial_bytes(c, R, S, c->group_size);
    }
    case RESA_OP_DENSE_RECTIFY: {
      const int S = splits_for(c, op, R, max_blocks, max_sel, chunk);
      return partial_bytes(c, R, S, (long long)chunk * c->group_size);
    }
    case RESA_OP_SPARSE_STEP:  // the score keys, then the sparse decode's partials
      return workspace_bytes(c, RESA_OP_SCORE_SELECT, R, max_blocks, max_sel, 0) +
             workspace_bytes(c, RESA_OP_SPARSE_DECODE, R, max_blocks, max_sel, 0);
    default:
      return 0;
  }
}

float scale_log2(const resa_config* c) { return (float)((double)c->sm_scale * 1.4426950408889634); }

resa_status from_hip(hipError_t e) { return e == hipSuccess ? RESA_OK : RESA_ERR_LAUNCH; }

constexpr int kMaxDevices = 64;  // devices whose scratch address is remembered

}  // namespace

// Device memory of resa_sparse_decode_noalloc: every GPU the library runs on
// holds its own copy until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol); it uses the device address looked up by scratch_of_current_device.
static __device__ __align__(256) unsigned char scratch[RESA_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and remembered.
resa_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return RESA_ERR_LAUNCH;
  if (dev >= kMaxDevices) return RESA_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RESA_ERR_LAUNCH;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return RESA_OK;
}

}  // namespace

extern "C" {

int32_t resa_abi_version(void) { return RESA_ABI_VERSION; }

const char* resa_status_string(resa_status s) {
  switch (s) {
    case RESA_OK:
      return "ok";
    case RESA_ERR_INVALID_ARG:
      return "invalid argument";
    case RESA_ERR_UNSUPPORTED:
      return "unsupported configuration";
    case RESA_ERR_WORKSPACE:
      return "workspace missing or too small";
    case RESA_ERR_LAUNCH:
      return "kernel launch failed";
  }
  return "unknown status";
}

resa_status resa_config_init(resa_config* cfg, int32_t num_kv_heads, int32_t group_size, int32_t head_dim,
                             int32_t dtype) {
  if (!cfg || head_dim <= 0) return RESA_ERR_INVALID_ARG;
  cfg->num_kv_heads = num_kv_heads;
  cfg->group_size = group_size;
  cfg->head_dim = head_dim;
  cfg->block_size = kBlock;
  cfg->dtype = dtype;
  cfg->budget_num = 1;
  cfg->budget_den = 10;
  cfg->min_blocks = 16;
  cfg->local_blocks = 1;
  cfg->score_mode = RESA_SCORE_SUM_HEADS;
  cfg->sm_scale = (float)(1.0 / sqrt((double)head_dim));
  cfg->num_splits = 0;
  return check_config(cfg);
}

int32_t resa_selection_count(const resa_config* cfg, int32_t num_blocks) {
  if (check_config(cfg) != RESA_OK || num_blocks < 0) return -1;
  return selection_count(cfg, num_blocks);
}

size_t resa_workspace_bytes(const resa_config* cfg, int32_t op, int32_t num_requests, int32_t max_blocks,
                            int32_t max_sel, int32_t chunk) {
  if (check_config(cfg) != RESA_OK || num_requests < 0 || max_blocks < 1 || max_blocks > kMaxBlocksLimit)
    return 0;
  if ((op == RESA_OP_SPARSE_DECODE || op == RESA_OP_SPARSE_STEP) && max_sel < 1) return 0;
  if (op == RESA_OP_DENSE_RECTIFY && (chunk < 1 || chunk > kMaxChunk)) return 0;
  return workspace_bytes(cfg, op, num_requests, max_blocks, max_sel, chunk);
}

int32_t resa_num_splits(const resa_config* cfg, int32_t op, int32_t num_requests, int32_t max_blocks,
                        int32_t max_sel, int32_t chunk) {
  if (check_config(cfg) != RESA_OK || num_requests < 0 || max_blocks < 1 || max_blocks > kMaxBlocksLimit) return 0;
  if (op != RESA_OP_SPARSE_DECODE && op != RESA_OP_DENSE_DECODE && op != RESA_OP_DENSE_RECTIFY) return 0;
  if (op == RESA_OP_SPARSE_DECODE && max_sel < 1) return 0;
  if (op == RESA_OP_DENSE_RECTIFY && (chunk < 1 || chunk > kMaxChunk)) return 0;
  return splits_for(cfg, op, num_requests, max_blocks, max_sel, chunk);
}

resa_status resa_build_descriptors(const resa_config* cfg, const resa_paged_kv* kv, int32_t num_requests,
                                   const int32_t* first_block, int32_t num_blocks, void* stream) {
  resa_status st = check_config(cfg);
  if (st == RESA_OK) st = check_kv(kv, true, false, true);
  if (st == RESA_OK) st = check_requests(num_requests);
  if (st != RESA_OK) return st;
  if (num_requests == 0) return RESA_OK;
  DescArgs a{};
  a.k_pool = kv->k_pool;
  a.desc_pool = kv->desc_pool;
  a.table = kv->block_table;
  a.seq_lens = kv->seq_lens;
  a.first_block = first_block;
  a.num_blocks = num_blocks;
  a.window = 0;
  a.R = num_requests;
  a.H = cfg->num_kv_heads;
  a.D = cfg->head_dim;
  a.dtype = cfg->dtype;
  a.max_blocks = kv->max_blocks;
  a.num_pool_blocks = kv->num_pool_blocks;
  (void)hipGetLastError();
  return from_hip(launch_descriptors(a, static_cast<hipStream_t>(stream)));
}

resa_status resa_score_select(const resa_config* cfg, const resa_paged_kv* kv, int32_t num_requests, const void* q,
                              int32_t refresh_tail, int32_t* sel_idx, int32_t* sel_cnt, int32_t max_sel,
                              float* scores, void* ws, size_t ws_bytes, void* stream) {
  resa_status st = check_config(cfg);
  if (st == RESA_OK) st = check_kv(kv, refresh_tail != 0, false, true);
  if (st == RESA_OK) st = check_requests(num_requests);
  if (st != RESA_OK) return st;
  if (!q || !aligned16(q) || !sel_idx || !sel_cnt) return RESA_ERR_INVALID_ARG;
  if (max_sel < selection_count(cfg, kv->max_blocks)) return RESA_ERR_INVALID_ARG;
  if (num_requests == 0) return RESA_OK;
  const size_t need = workspace_bytes(cfg, RESA_OP_SCORE_SELECT, num_requests, kv->max_blocks, max_sel, 0);
  if (!ws || ws_bytes < need || !aligned16(ws)) return RESA_ERR_WORKSPACE;

  (void)hipGetLastError();
  ScoreArgs sa{};
  sa.q = q;
  sa.desc_pool = kv->desc_pool;
  sa.k_pool = kv->k_pool;
  sa.refresh_tail = refresh_tail != 0;
  sa.table = kv->block_table;
  sa.seq_lens = kv->seq_lens;
  sa.keys = static_cast<uint32_t*>(ws);
  sa.scores = scores;
  sa.sel_idx = sel_idx;
  sa.sel_cnt = sel_cnt;
  sa.R = num_requests;
  sa.H = cfg->num_kv_heads;
  sa.G = cfg->group_size;
  sa.D = cfg->head_dim;
  sa.dtype = cfg->dtype;
  sa.max_blocks = kv->max_blocks;
  sa.num_pool_blocks = kv->num_pool_blocks;
  sa.mode = cfg->score_mode;
  sa.key_stride = key_stride_for(kv->max_blocks);
  sa.max_sel = max_sel;
  sa.budget_num = cfg->budget_num;
  sa.budget_den = cfg->budget_den;
  sa.min_blocks = cfg->min_blocks;
  sa.local_blocks = cfg->local_blocks;
  return from_hip(launch_score_select(sa, static_cast<hipStream_t>(stream)));
}

static resa_status decode_common(const resa_config* cfg, const resa_paged_kv* kv, int32_t R, const void* q,
                                 const int32_t* sel_idx, const int32_t* sel_cnt, int32_t max_sel, float* out,
                                 void* ws, size_t ws_bytes, void* stream, int op) {
  resa_status st = check_config(cfg);
  if (st == RESA_OK) st = check_kv(kv, true, true, false);
  if (st == RESA_OK) st = check_requests(R);
  if (st != RESA_OK) return st;
  if (!q || !aligned16(q) || !out || !aligned16(out)) return RESA_ERR_INVALID_ARG;
  if (op == RESA_OP_SPARSE_DECODE && (!sel_idx || !sel_cnt || max_sel < 1)) return RESA_ERR_INVALID_ARG;
  if (R == 0) return RESA_OK;
  const int S = splits_for(cfg, op, R, kv->max_blocks, max_sel, 0);
  const size_t need = workspace_bytes(cfg, op, R, kv->max_blocks, max_sel, 0);
  if (!ws || ws_bytes < need || !aligned16(ws)) return RESA_ERR_WORKSPACE;
  const size_t rows = (size_t)R * cfg->num_kv_heads * S * cfg->group_size;
  DecodeArgs a{};
  a.q = q;
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.table = kv->block_table;
  a.seq_lens = kv->seq_lens;
  a.sel_idx = op == RESA_OP_SPARSE_DECODE ? sel_idx : nullptr;
  a.sel_cnt = op == RESA_OP_SPARSE_DECODE ? sel_cnt : nullptr;
  a.max_sel = op == RESA_OP_SPARSE_DECODE ? max_sel : 0;
  a.out = out;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(rows * cfg->head_dim * sizeof(float)));
  a.R = R;
  a.H = cfg->num_kv_heads;
  a.G = cfg->group_size;
  a.D = cfg->head_dim;
  a.dtype = cfg->dtype;
  a.max_blocks = kv->max_blocks;
  a.num_pool_blocks = kv->num_pool_blocks;
  a.splits = S;
  a.scale_log2 = scale_log2(cfg);
  (void)hipGetLastError();
  return from_hip(launch_decode(a, static_cast<hipStream_t>(stream)));
}

resa_status resa_sparse_decode(const resa_config* cfg, const resa_paged_kv* kv, int32_t num_requests, const void* q,
                               const int32_t* sel_idx, const int32_t* sel_cnt, int32_t max_sel, float* out, void* ws,
                               size_t ws_bytes, void* stream) {
  return decode_common(cfg, kv, num_requests, q, sel_idx, sel_cnt, max_sel, out, ws, ws_bytes, stream,
                       RESA_OP_SPARSE_DECODE);
}

resa_status resa_sparse_decode_noalloc(const resa_config* cfg, const resa_paged_kv* kv, int32_t num_requests,
                                       const void* q, const int32_t* sel_idx, const int32_t* sel_cnt,
                                       int32_t max_sel, float* out, void* stream) {
  // The same checks and kernels as resa_sparse_decode; the workspace is this
  // device's static scratch, so a call needing more than its size is refused
  // before anything is looked up or enqueued.
  resa_status st = check_config(cfg);
  if (st == RESA_OK) st = check_kv(kv, true, true, false);
  if (st == RESA_OK) st = check_requests(num_requests);
  if (st != RESA_OK) return st;
  if (max_sel < 1) return RESA_ERR_INVALID_ARG;
  const size_t need = workspace_bytes(cfg, RESA_OP_SPARSE_DECODE, num_requests, kv->max_blocks, max_sel, 0);
  if (need > (size_t)RESA_NOALLOC_SCRATCH_BYTES) return RESA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != RESA_OK) return st;
  return decode_common(cfg, kv, num_requests, q, sel_idx, sel_cnt, max_sel, out, ws,
                       (size_t)RESA_NOALLOC_SCRATCH_BYTES, stream, RESA_OP_SPARSE_DECODE);
}

resa_status resa_sparse_step(const resa_config* cfg, const resa_paged_kv* kv, int32_t num_requests, const void* q,
                             int32_t refresh_tail, int32_t* sel_idx, int32_t* sel_cnt, int32_t max_sel, float* out,
                             void* ws, size_t ws_bytes, void* stream) {
  resa_status st = check_config(cfg);
  if (st == RESA_OK) st = check_kv(kv, true, true, true);
  if (st == RESA_OK) st = check_requests(num_requests);
  if (st != RESA_OK) return st;
  if (!q || !aligned16(q) || !sel_idx || !sel_cnt || !out || !aligned16(out)) return RESA_ERR_INVALID_ARG;
  if (max_sel < selection_count(cfg, kv->max_blocks)) return RESA_ERR_INVALID_ARG;
  if (num_requests == 0) return RESA_OK;
  const size_t need = workspace_bytes(cfg, RESA_OP_SPARSE_STEP, num_requests, kv->max_blocks, max_sel, 0);
  if (!ws || ws_bytes < need || !aligned16(ws)) return RESA_ERR_WORKSPACE;
  const size_t key_bytes = workspace_bytes(cfg, RESA_OP_SCORE_SELECT, num_requests, kv->max_blocks, max_sel, 0);
  char* parts = static_cast<char*>(ws) + key_bytes;  // the decode's partials follow the keys
  const int S = splits_for(cfg, RESA_OP_SPARSE_DECODE, num_requests, kv->max_blocks, max_sel, 0);
  const size_t rows = (size_t)num_requests * cfg->num_kv_heads * S * cfg->group_size;

  ScoreArgs sa{};
  sa.q = q;
  sa.desc_pool = kv->desc_pool;
  sa.k_pool = kv->k_pool;
  sa.refresh_tail = refresh_tail != 0;
  sa.table = kv->block_table;
  sa.seq_lens = kv->seq_lens;
  sa.keys = static_cast<uint32_t*>(ws);
  sa.scores = nullptr;
  sa.sel_idx = sel_idx;
  sa.sel_cnt = sel_cnt;
  sa.R = num_requests;
  sa.H = cfg->num_kv_heads;
  sa.G = cfg->group_size;
  sa.D = cfg->head_dim;
  sa.dtype = cfg->dtype;
  sa.max_blocks = kv->max_blocks;
  sa.num_pool_blocks = kv->num_pool_blocks;
  sa.mode = cfg->score_mode;
  sa.key_stride = key_stride_for(kv->max_blocks);
  sa.max_sel = max_sel;
  sa.budget_num = cfg->budget_num;
  sa.budget_den = cfg->budget_den;
  sa.min_blocks = cfg->min_blocks;
  sa.local_blocks = cfg->local_blocks;

  DecodeArgs da{};
  da.q = q;
  da.k_pool = kv->k_pool;
  da.v_pool = kv->v_pool;
  da.table = kv->block_table;
  da.seq_lens = kv->seq_lens;
  da.sel_idx = sel_idx;
  da.sel_cnt = sel_cnt;
  da.max_sel = max_sel;
  da.out = out;
  da.part_o = reinterpret_cast<float*>(parts);
  da.part_ml = reinterpret_cast<float*>(parts + align_up(rows * cfg->head_dim * sizeof(float)));
  da.R = num_requests;
  da.H = cfg->num_kv_heads;
  da.G = cfg->group_size;
  da.D = cfg->head_dim;
  da.dtype = cfg->dtype;
  da.max_blocks = kv->max_blocks;
  da.num_pool_blocks = kv->num_pool_blocks;
  da.splits = S;
  da.scale_log2 = scale_log2(cfg);
  (void)hipGetLastError();
  return from_hip(launch_step(sa, da, static_cast<hipStream_t>(stream)));
}

resa_status resa_dense_decode(const resa_config* cfg, const resa_paged_kv* kv, int32_t num_requests, const void* q,
                              float* out, void* ws, size_t ws_bytes, void* stream) {
  return decode_common(cfg, kv, num_requests, q, nullptr, nullptr, 0, out, ws, ws_bytes, stream,
                       RESA_OP_DENSE_DECODE);
}

resa_status resa_dense_rectify(const resa_config* cfg, const resa_paged_kv* kv, int32_t num_requests, int32_t chunk,
                               const void* q_chunk, const void* k_new, const void* v_new, float* out, void* ws,
                               size_t ws_bytes, void* stream) {
  resa_status st = check_config(cfg);
  if (st == RESA_OK) st = check_kv(kv, true, true, true);
  if (st == RESA_OK) st = check_requests(num_requests);
  if (st != RESA_OK) return st;
  if (chunk < 1 || chunk > kMaxChunk || (long long)chunk > (long long)kv->max_blocks * kBlock)
    return RESA_ERR_INVALID_ARG;
  if (!q_chunk || !k_new || !v_new || !out || !aligned16(q_chunk) || !aligned16(out)) return RESA_ERR_INVALID_ARG;
  if (num_requests == 0) return RESA_OK;
  const int S = splits_for(cfg, RESA_OP_DENSE_RECTIFY, num_requests, kv->max_blocks, 0, chunk);
  const size_t need = workspace_bytes(cfg, RESA_OP_DENSE_RECTIFY, num_requests, kv->max_blocks, 0, chunk);
  if (!ws || ws_bytes < need || !aligned16(ws)) return RESA_ERR_WORKSPACE;
  const size_t rows = (size_t)num_requests * cfg->num_kv_heads * S * chunk * cfg->group_size;
  RectifyArgs a{};
  a.q_chunk = q_chunk;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_pool = kv->k_pool;
  a.v_pool = kv->v_pool;
  a.desc_pool = kv->desc_pool;
  a.table = kv->block_table;
  a.seq_lens = kv->seq_lens;
  a.out = out;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(rows * cfg->head_dim * sizeof(float)));
  a.R = num_requests;
  a.H = cfg->num_kv_heads;
  a.G = cfg->group_size;
  a.D = cfg->head_dim;
  a.dtype = cfg->dtype;
  a.max_blocks = kv->max_blocks;
  a.num_pool_blocks = kv->num_pool_blocks;
  a.chunk = chunk;
  a.splits = S;
  a.scale_log2 = scale_log2(cfg);
  (void)hipGetLastError();
  return from_hip(launch_rectify(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
