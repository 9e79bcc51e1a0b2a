/*
 * resa.h - C ABI of libresa, the decode-time hot path of Rectified Sparse
 * Attention (ReSA) for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the "Rectified Sparse Attention" analysis page
 * (paper-graph-ui), §3.4.1-§3.4.4:
 *   resa_build_descriptors  per-block min/max key descriptors (Eq 3; the
 *                           incremental block-key-cache update of Algorithm 1)
 *   resa_score_select       group block scores (Eq 4) and top-n selection with
 *                           the forced local window (Eq 5, §3.4.1)
 *   resa_sparse_decode      group block sparse attention over the selected
 *                           blocks (Eq 2), split over the GPU and merged with
 *                           stored log-sum-exp values (§3.4.4)
 *   resa_dense_decode       dense attention (Eq 1), the baseline of §5
 *   resa_dense_rectify      dense rectification (§3.4.2): write the last f
 *                           positions' rows, refresh their descriptors, and
 *                           run causal chunk attention over the whole cache
 *   resa_sparse_step        resa_score_select followed by resa_sparse_decode
 *                           in one launch fewer (the decode step of one layer)
 *
 * Conventions for every call
 * --------------------------
 * - Every pointer except `cfg`, `kv` (the structs themselves) is a DEVICE
 *   pointer on the current HIP device.  `stream` is a hipStream_t (NULL = the
 *   default stream).  Calls only enqueue work on `stream`; none synchronises,
 *   allocates, prints or aborts.
 * - Arguments are checked on the host before anything is enqueued.  A call
 *   that returns an error has enqueued nothing and changed nothing.
 *   RESA_ERR_LAUNCH reports a failed kernel launch (hipGetLastError).
 *   Faults inside kernels surface at the caller's next synchronisation.
 * - The caller owns every buffer.  Outputs must not alias inputs.
 * - Values read from device memory are range-clamped by the kernels so that
 *   no access leaves the buffers described below: a sequence length outside
 *   [0, max_blocks*16] is clamped into it, a block-table entry outside
 *   [0, num_pool_blocks) is clamped into it, a selected block id outside
 *   [0, max_blocks) is clamped into it (rows at or past the sequence length
 *   never contribute).  Such inputs give unspecified results, never an
 *   out-of-bounds access.  Requests with sequence length 0 produce a zero
 *   output and an empty selection.
 * - Rows of the last block at positions >= the sequence length may hold any
 *   bit pattern (NaN included); no result depends on them.
 * - Results are deterministic: the same inputs and configuration give
 *   bitwise-identical outputs (no floating-point atomics).
 *
 * Paged KV cache layout (element type = cfg->dtype, d = cfg->head_dim,
 * H = cfg->num_kv_heads, block size 16):
 *   k_pool    [num_pool_blocks][H][16][d]   keys, token-major within a block
 *   v_pool    [num_pool_blocks][H][d][16]   values, channel-major within a
 *                                           block (16 consecutive tokens of one
 *                                           channel are contiguous)
 *   desc_pool [num_pool_blocks][H][2][d]    descriptor of each block: row 0 is
 *                                           the element-wise minimum of the
 *                                           block's keys, row 1 the maximum
 *   block_table [R][max_blocks] int32       physical block of logical block b
 *                                           of request r (token t lives in
 *                                           logical block t/16, row t%16)
 *   seq_lens  [R] int32                     cached tokens of each request,
 *                                           including the current one
 * Queries q are [R][H*g][d] with query head h = i*g + j belonging to KV head
 * i (GQA group i).  Outputs are float32.
 */
#ifndef RESA_H
#define RESA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RESA_ABI_VERSION 1

typedef enum {
  RESA_OK = 0,
  RESA_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shape */
  RESA_ERR_UNSUPPORTED = 2, /* a configuration the library has no kernel for */
  RESA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  RESA_ERR_LAUNCH = 4       /* a kernel launch failed */
} resa_status;

typedef enum { RESA_BF16 = 0, RESA_F32 = 1 } resa_dtype;

/* How a GQA group's query heads are turned into one block score (Eq 4). */
typedef enum {
  RESA_SCORE_SUM_HEADS = 0, /* sum over the group's heads of Eq 4 */
  RESA_SCORE_MEAN_POOL = 1  /* Eq 4 applied to the mean of the group's heads */
} resa_score_mode;

typedef enum {
  RESA_OP_SCORE_SELECT = 1,
  RESA_OP_SPARSE_DECODE = 2,
  RESA_OP_DENSE_DECODE = 3,
  RESA_OP_DENSE_RECTIFY = 4,
  RESA_OP_SPARSE_STEP = 5
} resa_op;

/* Method configuration, passed by pointer to every call. */
typedef struct resa_config {
  int32_t num_kv_heads; /* H >= 1 */
  int32_t group_size;   /* g: query heads per KV head, 1..16 */
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t block_size;   /* must be 16 */
  int32_t dtype;        /* resa_dtype of q, K, V, descriptors, rectify inputs */
  int32_t budget_num;   /* attended fraction rho = budget_num / budget_den */
  int32_t budget_den;   /*   (0 < num <= den); default 1/10 */
  int32_t min_blocks;   /* n_min >= 0, default 16 (§3.4.5) */
  int32_t local_blocks; /* n_local >= 1 most recent blocks always selected */
  int32_t score_mode;   /* resa_score_mode */
  float sm_scale;       /* softmax scale, > 0; default fp32(1/sqrt(d)) */
  int32_t num_splits;   /* 0 = automatic; else splits per (request, KV head) */
} resa_config;

/* Paged KV cache description (see the layout above).  Pointers are device
 * pointers.  Which of k/v/desc a call reads or writes is stated per call. */
typedef struct resa_paged_kv {
  void* k_pool;
  void* v_pool;
  void* desc_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t num_pool_blocks; /* >= 1 */
  int32_t max_blocks;      /* columns of block_table, >= 1 */
} resa_paged_kv;

int32_t resa_abi_version(void);
const char* resa_status_string(resa_status status);

/* Fills `cfg` with the defaults of §3.4.5 for the given shape: block 16,
 * rho = 1/10, n_min = 16, n_local = 1, sum-over-heads scoring,
 * sm_scale = fp32(1/sqrt(head_dim)), automatic splits. */
resa_status resa_config_init(resa_config* cfg, int32_t num_kv_heads, int32_t group_size,
                             int32_t head_dim, int32_t dtype);

/* Eq 5 with this library's readings: n = min(M, max(n_min, ceil(M*rho), n_local)),
 * with an exact integer ceiling.  Returns -1 on an invalid configuration. */
int32_t resa_selection_count(const resa_config* cfg, int32_t num_blocks);

/* Bytes of workspace `op` needs for `num_requests` requests of up to
 * `max_blocks` blocks; `max_sel` is the sel_idx row capacity (sparse ops) and
 * `chunk` the rectification window (rectify).  Returns 0 on invalid arguments.
 * Calls that share a workspace must be ordered on one stream.  No
 * workspace needs initialisation. */
size_t resa_workspace_bytes(const resa_config* cfg, int32_t op, int32_t num_requests,
                            int32_t max_blocks, int32_t max_sel, int32_t chunk);

/* Splits per (request, KV head) that `op` uses for these sizes (what
 * cfg->num_splits = 0 resolves to).  Returns 0 on invalid arguments. */
int32_t resa_num_splits(const resa_config* cfg, int32_t op, int32_t num_requests,
                        int32_t max_blocks, int32_t max_sel, int32_t chunk);

/*
 * Block descriptors (Eq 3; Algorithm 1's block-key-cache update).
 * For each request r and KV head i, for every block b in the range below,
 * writes desc_pool[block_table[r][b]][i][0][c] = min and [1][c] = max over the
 * block's rows t < seq_lens[r] of k_pool's key component c, using the total
 * order -0 < +0 (the result is bit-identical to the stored key values).
 * Range per request, with M_r = ceil(seq_lens[r]/16):
 *   first_block == NULL, num_blocks <= 0 : all blocks [0, M_r)
 *   first_block == NULL, num_blocks >  0 : the last num_blocks blocks
 *                                          [max(0, M_r - num_blocks), M_r)
 *   first_block != NULL                  : [first_block[r], first_block[r] + n)
 *                                          clipped to [0, M_r), where n =
 *                                          num_blocks, or M_r if num_blocks <= 0
 * first_block is a device array [R].  Reads k_pool; writes desc_pool.
 */
resa_status resa_build_descriptors(const resa_config* cfg, const resa_paged_kv* kv,
                                   int32_t num_requests, const int32_t* first_block,
                                   int32_t num_blocks, void* stream);

/*
 * Group block scoring (Eq 4) and top-n selection (Eq 5 + local window).
 * Per request r and KV head i with M = ceil(seq_lens[r]/16) blocks: scores
 * every block from desc_pool and q (score_mode), then selects
 * n = resa_selection_count(cfg, M) blocks: the local_blocks most recent blocks
 * always, and the highest-scoring older blocks (ties: lower block id first).
 * refresh_tail != 0 also recomputes, from k_pool, the descriptor of block
 * M-1 of every request and KV head (the block the newest token was appended
 * to: Algorithm 1's incremental block-key-cache update) in the same launch;
 * it then equals what resa_build_descriptors(cfg, kv, R, NULL, 1, ...) writes.
 * That block is always selected, so its score does not influence the
 * selection; its exported score is unspecified when refresh_tail != 0.
 *   sel_idx [R][H][max_sel] int32   selected logical block ids, ascending,
 *                                   entries [n, max_sel) set to -1
 *   sel_cnt [R][H] int32            n
 *   scores  [R][H][max_blocks] f32  optional (NULL to skip): every block's
 *                                   score; entries >= M are left untouched
 * Requires max_sel >= resa_selection_count(cfg, kv->max_blocks) and
 * ws_bytes >= resa_workspace_bytes(cfg, RESA_OP_SCORE_SELECT, ...).
 * Reads q, desc_pool, block_table, seq_lens (and k_pool, writing the last
 * block's descriptor in desc_pool, when refresh_tail != 0).
 */
resa_status resa_score_select(const resa_config* cfg, const resa_paged_kv* kv,
                              int32_t num_requests, const void* q, int32_t refresh_tail,
                              int32_t* sel_idx, int32_t* sel_cnt, int32_t max_sel,
                              float* scores, void* ws, size_t ws_bytes, void* stream);

/*
 * Group block sparse attention (Eq 2, masked positions excluded from the
 * softmax).  For each query head h = i*g + j of request r:
 *   out[r][h] = sum_t softmax_t(sm_scale * q[r][h] . K_i[t]) V_i[t]
 * over the rows t < seq_lens[r] of the blocks sel_idx[r][i][0 .. sel_cnt[r][i]).
 * The listed ids must be distinct (any order).  sel_cnt is clamped to
 * [0, min(max_sel, M)].  out is [R][H*g][d] float32.
 * Reads q, k_pool, v_pool, block_table, seq_lens, sel_idx, sel_cnt.
 */
resa_status resa_sparse_decode(const resa_config* cfg, const resa_paged_kv* kv,
                               int32_t num_requests, const void* q, const int32_t* sel_idx,
                               const int32_t* sel_cnt, int32_t max_sel, float* out, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * One decode step of one layer: exactly what resa_score_select(cfg, kv,
 * num_requests, q, refresh_tail, sel_idx, sel_cnt, max_sel, NULL, ...)
 * followed by resa_sparse_decode(cfg, kv, num_requests, q, sel_idx, sel_cnt,
 * max_sel, out, ...) compute - the same sel_idx and sel_cnt, and the same out
 * (the attention is split the same way) - in one launch fewer: the scoring
 * launch, then one launch in which every split workgroup of a (request, KV
 * head) finds the row's selection threshold itself from the score keys and
 * attends over its own share of the selected list, then the merge of the
 * splits (split execution with a log-sum-exp merge: "Rectified Sparse
 * Attention" analysis page, §3.4.4; kernel time without CPU overhead: §5).
 * Rows of more than 8192 blocks (max_blocks), calls whose attention grid
 * (requests x KV heads x splits) exceeds 256 workgroups, fp32 caches and
 * lists whose per-split share exceeds 8200 ids run the separate selection
 * launch and the decode launch instead.
 * Requires max_sel >= resa_selection_count(cfg, kv->max_blocks) and
 * ws_bytes >= resa_workspace_bytes(cfg, RESA_OP_SPARSE_STEP, num_requests,
 * kv->max_blocks, max_sel, 0); the workspace needs no initialisation.
 * Reads q, k_pool, v_pool, desc_pool, block_table, seq_lens (and writes the
 * last block's descriptor when refresh_tail != 0); writes sel_idx, sel_cnt,
 * out [R][H*g][d] float32.
 */
resa_status resa_sparse_step(const resa_config* cfg, const resa_paged_kv* kv, int32_t num_requests,
                             const void* q, int32_t refresh_tail, int32_t* sel_idx, int32_t* sel_cnt,
                             int32_t max_sel, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * resa_sparse_decode without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid allocation.  It computes exactly what
 * resa_sparse_decode computes, with the same kernels and the same argument
 * checks.  Its workspace is a static device array of
 * RESA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it
 * runs on until the process ends; its address is looked up (once per device,
 * with that device current) on the first call on a device.  The call
 * allocates nothing: no hipMalloc, hipFree or allocating library routine.
 * A call whose workspace (resa_workspace_bytes(cfg, RESA_OP_SPARSE_DECODE,
 * num_requests, kv->max_blocks, max_sel, 0)) exceeds that size returns
 * RESA_ERR_WORKSPACE and enqueues nothing.  All calls on one GPU share its
 * array and it keeps the last call's contents (the decode writes every word
 * it reads first, so nothing in it needs clearing): calls that overlap on
 * one GPU (on different streams, or from several threads) race and must be
 * ordered by the caller.  A failed lookup of the array returns
 * RESA_ERR_LAUNCH.
 */
#define RESA_NOALLOC_SCRATCH_BYTES (8u << 20)
resa_status resa_sparse_decode_noalloc(const resa_config* cfg, const resa_paged_kv* kv,
                                       int32_t num_requests, const void* q, const int32_t* sel_idx,
                                       const int32_t* sel_cnt, int32_t max_sel, float* out,
                                       void* stream);

/*
 * Dense decode attention (Eq 1): as resa_sparse_decode with every block
 * [0, M) of every request.  The baseline of §5.  out is [R][H*g][d] float32.
 */
resa_status resa_dense_decode(const resa_config* cfg, const resa_paged_kv* kv,
                              int32_t num_requests, const void* q, float* out, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * Dense rectification (§3.4.2, Algorithm 1).  With L = seq_lens[r] (which
 * already counts the window) and P = L - chunk, per request r:
 *   1. copies k_new[r][t][i][:] / v_new[r][t][i][:] into cache position P + t
 *      of KV head i, t in [0, chunk) (bit-exact);
 *   2. recomputes the descriptors of blocks floor(P/16) .. M-1;
 *   3. out[r][t][h] = causal dense attention of q_chunk[r][t][h] over cache
 *      positions 0 .. P + t of the rewritten cache.
 * q_chunk [R][chunk][H*g][d], k_new / v_new [R][chunk][H][d] (cfg->dtype);
 * out [R][chunk][H*g][d] float32.  Requests with L < chunk are skipped (their
 * out rows are zero and their cache is untouched).  1 <= chunk <= 256.
 * Reads and writes k_pool, v_pool, desc_pool.
 */
resa_status resa_dense_rectify(const resa_config* cfg, const resa_paged_kv* kv,
                               int32_t num_requests, int32_t chunk, const void* q_chunk,
                               const void* k_new, const void* v_new, float* out, void* ws,
                               size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RESA_H */
