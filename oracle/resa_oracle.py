"""Plain CPU oracle of the ReSA decode hot path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
the benchmark's ``cpu_baseline`` leg may import this module.  The library
(`libresa.so` and its Python binding) never calls it, and it shares no code
with the HIP path.

Every function is the plain definition from the pages, written in NumPy,
float64 throughout.  Inputs are the exact fp32 values of the stored operands
(bf16 -> fp32 is exact).  Nothing is blocked, fused or reordered beyond what
the definition states; the only library primitives used as steps are
elementwise arithmetic, ``min``/``max``/``sum`` reductions, ``exp``, matrix
products and a sort.

Sources (titles of the pages as published):

* "Rectified Sparse Attention" analysis (paper-graph-ui), §3.4.1 Eq 1-5,
  §3.4.2 (dense rectification), §3.4.3 Algorithm 1 and Eq 6, §3.4.5 defaults.

Readings taken where the pages are silent or contradict each other (listed
with reasons in the design notes):

* the budget: ``rho = budget_num / budget_den`` is the *selected* fraction
  (0.10 by default) and the count is an integer ceiling;
* the count is capped at the number of blocks that exist;
* the most recent ``local_blocks`` blocks (the tail, possibly partial) are
  always selected and count toward the total;
* ties in the block ranking go to the lower block index;
* masked positions are excluded from the softmax (never multiplied by 0);
* the default group score sums ``max(q.kmin, q.kmax)`` over every query head
  of the GQA group; ``mean_pool`` scores with the group's mean query instead;
* min/max use the total order with -0 < +0, so descriptors are unique bit
  patterns;
* rectification is causal within the chunk and attends to the rows it has
  just written; the window is the last ``f`` positions.
"""

from __future__ import annotations

import numpy as np

BLOCK = 16

SCORE_SUM_HEADS = "sum_heads"
SCORE_MEAN_POOL = "mean_pool"


# ---------------------------------------------------------------------------
# counts


def num_blocks(seq_len: int, block: int = BLOCK) -> int:
    """Number of blocks holding ``seq_len`` tokens (the last one may be partial)."""
    return (int(seq_len) + block - 1) // block


def selection_count(M: int, budget_num: int, budget_den: int, min_blocks: int = 16,
                    local_blocks: int = 1) -> int:
    """Eq 5 (§3.4.1): n = max(n_min, ceil(M * rho)), with rho = num/den as an
    integer ratio, never fewer than the forced local window and never more than
    the M blocks that exist."""
    M = int(M)
    ceil_part = (M * int(budget_num) + int(budget_den) - 1) // int(budget_den)
    return min(M, max(int(min_blocks), ceil_part, int(local_blocks)))


def memory_factor(block: int, p: float, f: int) -> float:
    """Eq 6 (§3.4.3): average memory access per step relative to dense decode,
    1/b + p + 1/f, where p is the fraction of the cache attended."""
    return 1.0 / block + p + 1.0 / f


def touched_blocks(seq_len: int, chunk: int, block: int = BLOCK) -> range:
    """Blocks whose rows a rectification of the last ``chunk`` positions rewrites
    (§3.4.2: the descriptors of every affected block are recomputed)."""
    first = (int(seq_len) - int(chunk)) // block
    return range(first, num_blocks(seq_len, block))


# ---------------------------------------------------------------------------
# Eq 3: block descriptors


def _min_total_order(rows: np.ndarray) -> np.ndarray:
    """Column-wise minimum with -0 < +0."""
    m = rows.min(axis=0)
    neg_zero = np.any((rows == 0) & np.signbit(rows), axis=0)
    return np.where(m == 0, np.where(neg_zero, -0.0, 0.0), m)


def _max_total_order(rows: np.ndarray) -> np.ndarray:
    """Column-wise maximum with -0 < +0."""
    m = rows.max(axis=0)
    pos_zero = np.any((rows == 0) & ~np.signbit(rows), axis=0)
    return np.where(m == 0, np.where(pos_zero, 0.0, -0.0), m)


def descriptors(K: np.ndarray, seq_len: int, block: int = BLOCK):
    """Eq 3 (§3.4.1): for every block of ``block`` consecutive keys, the
    element-wise minimum and maximum over the block's rows.  Only rows below
    ``seq_len`` belong to the cache; the last block may be partial.

    K: [>= seq_len, d] keys of one KV head.  Returns (lo, hi), each [M, d] float64.
    """
    L = int(seq_len)
    K = np.asarray(K, dtype=np.float64)[:L]
    assert np.all(np.isfinite(K)), "keys must be finite"
    M = num_blocks(L, block)
    d = K.shape[1]
    lo = np.empty((M, d))
    hi = np.empty((M, d))
    for b in range(M):
        lo[b], hi[b] = block_descriptor(K, L, b, block)
    return lo, hi


def block_descriptor(K: np.ndarray, seq_len: int, b: int, block: int = BLOCK):
    """Eq 3 for the single block ``b``: (min, max) over its rows below seq_len."""
    L = int(seq_len)
    rows = np.asarray(K, dtype=np.float64)[b * block: min(b * block + block, L)]
    assert rows.shape[0] > 0, "block holds no cached row"
    return _min_total_order(rows), _max_total_order(rows)


# ---------------------------------------------------------------------------
# Eq 4: block scores


def scores(q_group: np.ndarray, lo: np.ndarray, hi: np.ndarray,
           mode: str = SCORE_SUM_HEADS) -> np.ndarray:
    """Eq 4 (§3.4.1): score_b = sum_c max(q_c * kmax_bc, q_c * kmin_bc).

    ``sum_heads`` applies Eq 4 to every query head of the group and adds the
    results; ``mean_pool`` applies it once to the group's mean query (§3.4.1,
    Fig 3).  q_group: [g, d]; lo, hi: [M, d].  Returns [M] float64.
    """
    q = np.asarray(q_group, dtype=np.float64)
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    if mode == SCORE_MEAN_POOL:
        q = q.mean(axis=0, keepdims=True)
    elif mode != SCORE_SUM_HEADS:
        raise ValueError(mode)
    out = np.zeros(lo.shape[0])
    for j in range(q.shape[0]):
        qj = q[j][None, :]
        out += np.maximum(qj * hi, qj * lo).sum(axis=1)
    return out


# ---------------------------------------------------------------------------
# Eq 5 + local window: selection


def select(S: np.ndarray, budget_num: int = 1, budget_den: int = 10, min_blocks: int = 16,
           local_blocks: int = 1) -> np.ndarray:
    """Top-n block selection (§3.4.1, Eq 5 and the local-window rule).

    The ``local_blocks`` most recent blocks are always taken (their score is
    treated as +inf); the remaining ``n - local`` slots go to the highest
    scores among the older blocks, ties to the lower block index.  Returns the
    selected block ids in ascending order.
    """
    S = np.asarray(S, dtype=np.float64)
    M = S.shape[0]
    if M == 0:
        return np.zeros(0, dtype=np.int64)
    n = selection_count(M, budget_num, budget_den, min_blocks, local_blocks)
    nl = min(int(local_blocks), M)
    forced = list(range(M - nl, M))
    cand = np.arange(M - nl)
    # sort by descending score, then ascending index
    order = cand[np.lexsort((cand, -S[: M - nl]))]
    chosen = order[: n - nl].tolist()
    return np.array(sorted(chosen + forced), dtype=np.int64)


# ---------------------------------------------------------------------------
# Eq 1 / Eq 2: attention


def block_rows(blocks, seq_len: int, block: int = BLOCK) -> np.ndarray:
    """Token positions covered by ``blocks`` that lie below ``seq_len``
    (the per-token expansion of the block mask, Eq 2)."""
    L = int(seq_len)
    rows = [np.arange(b * block, min(b * block + block, L)) for b in blocks]
    return np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)


def attend(q_group: np.ndarray, K: np.ndarray, V: np.ndarray, seq_len: int, blocks,
           sm_scale: float, block: int = BLOCK) -> np.ndarray:
    """Eq 2 (§3.4.1), masked positions excluded: for each query head j of the
    group, softmax(sm_scale * q_j . K[t]) over the rows t of the selected blocks,
    then the weighted sum of V[t].  q_group: [g, d]; K, V: [>= seq_len, d].
    Returns [g, d] float64."""
    blocks = [int(b) for b in blocks]
    assert len(set(blocks)) == len(blocks), "blocks must be distinct"
    M = num_blocks(seq_len, block)
    assert all(0 <= b < M for b in blocks)
    rows = block_rows(blocks, seq_len, block)
    assert rows.size > 0
    q = np.asarray(q_group, dtype=np.float64)
    Kr = np.asarray(K, dtype=np.float64)[rows]
    Vr = np.asarray(V, dtype=np.float64)[rows]
    logits = float(sm_scale) * (q @ Kr.T)  # [g, T]
    logits = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ Vr


def dense(q_group: np.ndarray, K: np.ndarray, V: np.ndarray, seq_len: int, sm_scale: float,
          block: int = BLOCK) -> np.ndarray:
    """Eq 1 (§3.4.1): attention over every cached position < seq_len."""
    return attend(q_group, K, V, seq_len, range(num_blocks(seq_len, block)), sm_scale, block)


# ---------------------------------------------------------------------------
# Dense rectification (§3.4.2, Algorithm 1)


def rectify(q_chunk: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, K: np.ndarray,
            V: np.ndarray, seq_len: int, sm_scale: float, block: int = BLOCK):
    """Rectification of one KV head's cache.

    The last f = len(k_new) positions [L - f, L) are overwritten with the freshly
    computed rows; the descriptors of every block those rows touch are
    recomputed; each chunk query t (position L - f + t) attends densely and
    causally to positions 0 .. L - f + t of the rewritten cache.

    q_chunk: [f, g, d]; k_new, v_new: [f, d]; K, V: [>= L, d].
    Returns (out [f, g, d], K', V' (new arrays, [L, d]), touched block ids,
    lo, hi of those blocks).
    """
    L = int(seq_len)
    f = int(np.asarray(k_new).shape[0])
    assert 1 <= f <= L
    P = L - f
    K2 = np.array(np.asarray(K, dtype=np.float64)[:L])
    V2 = np.array(np.asarray(V, dtype=np.float64)[:L])
    K2[P:L] = np.asarray(k_new, dtype=np.float64)
    V2[P:L] = np.asarray(v_new, dtype=np.float64)
    tb = list(touched_blocks(L, f, block))
    desc = [block_descriptor(K2, L, b, block) for b in tb]
    lo = np.stack([x[0] for x in desc])
    hi = np.stack([x[1] for x in desc])
    out = np.stack([dense(q_chunk[t], K2, V2, P + t + 1, sm_scale, block) for t in range(f)])
    return out, K2, V2, tb, lo, hi
