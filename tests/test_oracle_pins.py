"""Pins for the CPU oracle: each test checks it against something other than
itself (numbers the pages print, closed forms, library routines, brute force
on tiny inputs, invariants).  CPU only."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "pages_worked_examples.json")))


# ---------------------------------------------------------------- counts

@pytest.mark.parametrize("case", GOLD["selection_count"], ids=lambda c: f"M{c['M']}")
def test_selection_count_worked_examples(case):
    assert O.selection_count(case["M"], case["budget_num"], case["budget_den"],
                             case["min_blocks"], case["local_blocks"]) == case["expected"]


def test_selection_count_integer_ceiling():
    # 100 * 0.07 is 7.000000000000001 in binary floating point: a float ceiling
    # would select 8 blocks, the exact ceiling of 7 is 7.
    assert math.ceil(100 * 0.07) == 8
    assert O.selection_count(100, 7, 100, 0, 1) == 7
    assert O.selection_count(101, 7, 100, 0, 1) == 8


def test_selection_count_caps_and_floors():
    assert O.selection_count(5, 1, 10, 16, 1) == 5  # never more blocks than exist
    assert O.selection_count(1, 1, 10, 16, 1) == 1
    assert O.selection_count(40, 1, 10, 2, 6) == 6  # local window counts as a floor
    assert O.selection_count(400, 1, 10, 16, 1) == 40


@pytest.mark.parametrize("case", GOLD["memory_factor"], ids=lambda c: str(c["p"]))
def test_memory_factor_worked_examples(case):
    assert O.memory_factor(case["block"], case["p"], case["f"]) == pytest.approx(case["expected"],
                                                                                rel=1e-12)


def test_touched_blocks_worked_example():
    case = GOLD["touched_blocks"][0]
    assert len(O.touched_blocks(case["seq_len"], case["chunk"])) == case["expected_count"]
    # a window that does not start on a block boundary touches one more block
    assert list(O.touched_blocks(70, 32)) == [2, 3, 4]
    assert list(O.touched_blocks(64, 64)) == [0, 1, 2, 3]


def test_descriptor_size_worked_example():
    case = GOLD["descriptor_values_per_block"][0]
    d = case["head_dim"]
    lo, hi = O.descriptors(np.random.default_rng(0).standard_normal((16, d)), 16)
    assert lo.size + hi.size == case["expected_values"]
    # one block caches 16 key rows and 16 value rows of d values each
    assert (2 * 16 * d) // (lo.size + hi.size) == case["expected_ratio_vs_keys_and_values"]


# ---------------------------------------------------------------- descriptors

@pytest.mark.parametrize("seed,L,d", [(0, 1, 4), (1, 16, 8), (2, 17, 8), (3, 70, 16), (4, 255, 64)])
def test_descriptors_bound_and_attained(seed, L, d):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((L + 9, d)).astype(np.float32)
    K[L:] = 1e30  # rows past the cache end must be ignored
    lo, hi = O.descriptors(K, L)
    assert lo.shape == (O.num_blocks(L), d)
    for b in range(lo.shape[0]):
        rows = K[b * 16: min(b * 16 + 16, L)].astype(np.float64)
        assert np.all(lo[b] <= rows) and np.all(rows <= hi[b])
        # every bound is one of the block's own values (no padding, no rounding)
        assert np.all(np.any(rows == lo[b], axis=0))
        assert np.all(np.any(rows == hi[b], axis=0))


def test_block_descriptor_ignores_rows_past_cache_end():
    rng = np.random.default_rng(18)
    K = rng.standard_normal((40, 4))
    K[35:] = 1e30
    lo, hi = O.block_descriptor(K, 35, 2)
    np.testing.assert_array_equal(hi, K[32:35].max(axis=0))
    np.testing.assert_array_equal(lo, K[32:35].min(axis=0))


def test_descriptors_single_row_tail():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((33, 8))
    lo, hi = O.descriptors(K, 33)
    assert lo.shape[0] == 3
    np.testing.assert_array_equal(lo[2], K[32])
    np.testing.assert_array_equal(hi[2], K[32])


def test_descriptors_signed_zero_order():
    K = np.zeros((16, 3))
    K[3, 0] = -0.0
    K[:, 1] = -0.0
    K[5, 1] = 0.0
    K[:, 2] = -0.0
    lo, hi = O.descriptors(K, 16)
    assert np.signbit(lo[0, 0]) and not np.signbit(hi[0, 0])
    assert np.signbit(lo[0, 1]) and not np.signbit(hi[0, 1])
    assert np.signbit(lo[0, 2]) and np.signbit(hi[0, 2])


def test_descriptors_row_order_invariant():
    rng = np.random.default_rng(6)
    K = rng.standard_normal((48, 8))
    K2 = K.copy()
    K2[16:32] = K2[16:32][rng.permutation(16)]
    a, b = O.descriptors(K, 48), O.descriptors(K2, 48)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


# ---------------------------------------------------------------- scores

def _box_max_bruteforce(q, lo, hi):
    """max over every corner x of the box [lo, hi] of q . x."""
    best = -np.inf
    for corner in itertools.product(*[(lo[c], hi[c]) for c in range(len(q))]):
        best = max(best, float(np.dot(q, corner)))
    return best


@pytest.mark.parametrize("mode", [O.SCORE_SUM_HEADS, O.SCORE_MEAN_POOL])
def test_scores_equal_box_maximum(mode):
    rng = np.random.default_rng(7)
    g, d, L = 3, 5, 40
    q = rng.standard_normal((g, d))
    K = rng.standard_normal((L, d))
    lo, hi = O.descriptors(K, L)
    S = O.scores(q, lo, hi, mode)
    heads = q if mode == O.SCORE_SUM_HEADS else q.mean(axis=0, keepdims=True)
    for b in range(lo.shape[0]):
        expect = sum(_box_max_bruteforce(qj, lo[b], hi[b]) for qj in heads)
        assert S[b] == pytest.approx(expect, rel=1e-12, abs=1e-12)


def test_scores_upper_bound_true_maximum():
    rng = np.random.default_rng(8)
    g, d, L = 7, 128, 16 * 50 + 5
    q = rng.standard_normal((g, d))
    K = rng.standard_normal((L, d))
    lo, hi = O.descriptors(K, L)
    S = O.scores(q, lo, hi)
    for b in range(lo.shape[0]):
        rows = K[b * 16: min(b * 16 + 16, L)]
        per_head_max = (q @ rows.T).max(axis=1)  # [g]
        assert S[b] >= per_head_max.sum() - 1e-9
        assert per_head_max.sum() >= (q @ rows.T).sum(axis=0).max() - 1e-9


def test_scores_single_row_block_is_dot_product():
    rng = np.random.default_rng(9)
    g, d = 4, 32
    q = rng.standard_normal((g, d))
    K = rng.standard_normal((17, d))
    lo, hi = O.descriptors(K, 17)
    S = O.scores(q, lo, hi)
    assert S[1] == pytest.approx(float((q @ K[16]).sum()), rel=1e-12)


def test_scores_positive_negative_split_identity():
    # max(q lo, q hi) = relu(q) hi + min(q, 0) lo when hi >= lo
    rng = np.random.default_rng(10)
    q = rng.standard_normal((7, 64))
    K = rng.standard_normal((160, 64))
    lo, hi = O.descriptors(K, 160)
    P = np.maximum(q, 0).sum(axis=0)
    N = np.minimum(q, 0).sum(axis=0)
    np.testing.assert_allclose(O.scores(q, lo, hi), hi @ P + lo @ N, rtol=1e-12)


def test_scores_rank_planted_blocks_first():
    from synth import WORKLOADS, make_layer
    spec = WORKLOADS["tiny_f32_ctx2k"]
    inp = make_layer(spec, seed=3)
    K = inp.keys[0][0].numpy()
    q = inp.q[0].numpy()
    lo, hi = O.descriptors(K, inp.seq_lens[0])
    S = O.scores(q, lo, hi)
    # plausibility of the workload recipe, not a pin: shifting every key of a
    # block by 0.5 * qbar raises its score by 0.5 * sum_j q_j . qbar (about 4
    # standard deviations of the unplanted scores here)
    planted = inp.planted[0][0]
    rest = np.setdiff1d(np.arange(len(S) - 1), planted)
    assert S[planted].mean() > S[rest].mean() + 3 * S[rest].std()
    assert len(set(planted) & set(O.select(S).tolist())) >= 3


# ---------------------------------------------------------------- selection

def _check_selection(S, sel, num, den, nmin, nl):
    M = len(S)
    n = O.selection_count(M, num, den, nmin, nl)
    sel = list(sel)
    assert len(sel) == n and sel == sorted(set(sel))
    forced = set(range(M - min(nl, M), M))
    assert forced <= set(sel)
    chosen = set(sel) - forced
    rest = set(range(M)) - set(sel)
    for a in chosen:
        for b in rest:
            assert S[a] > S[b] or (S[a] == S[b] and a < b)


@pytest.mark.parametrize("seed", range(6))
def test_select_exchange_property_with_ties(seed):
    rng = np.random.default_rng(seed)
    for M in [1, 2, 5, 17, 64, 300]:
        S = rng.integers(0, 4, size=M).astype(np.float64)  # many exact ties
        for (num, den, nmin, nl) in [(1, 10, 16, 1), (1, 10, 2, 1), (3, 10, 0, 2), (1, 2, 1, 1)]:
            _check_selection(S, O.select(S, num, den, nmin, nl), num, den, nmin, nl)


def test_select_bruteforce_subsets():
    rng = np.random.default_rng(11)
    for trial in range(40):
        M = int(rng.integers(1, 10))
        S = rng.integers(0, 3, size=M).astype(np.float64)
        nl = 1
        n = O.selection_count(M, 1, 2, 2, nl)
        cands = list(range(M - nl))
        found = []
        for C in itertools.combinations(cands, n - nl):
            rest = [b for b in cands if b not in C]
            key = lambda b: (S[b], -b)  # noqa: E731
            if not rest or not C or min(map(key, C)) > max(map(key, rest)):
                found.append(sorted(list(C) + list(range(M - nl, M))))
        assert len(found) == 1
        assert O.select(S, 1, 2, 2, nl).tolist() == found[0]


def test_select_takes_all_when_budget_covers():
    S = np.arange(10, dtype=np.float64)[::-1]
    assert O.select(S, 1, 10, 16, 1).tolist() == list(range(10))


def test_select_local_window_forced():
    S = np.array([5.0, 4.0, 3.0, -1e9, -1e9, -1e9])
    assert O.select(S, 1, 2, 0, 3).tolist() == [3, 4, 5]
    assert O.select(S, 2, 3, 0, 1).tolist() == [0, 1, 2, 5]


# ---------------------------------------------------------------- attention

def _sdpa(q, K, V, mask, scale):
    """torch's fp64 CPU scaled_dot_product_attention as an independent routine.
    q: [g, d]; K, V: [T, d]; mask: [g or 1, T] bool (True = attend)."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, :, None, :]
    g = qt.shape[1]
    Kt = torch.from_numpy(np.asarray(K, np.float64))[None, None].expand(1, g, -1, -1)
    Vt = torch.from_numpy(np.asarray(V, np.float64))[None, None].expand(1, g, -1, -1)
    m = torch.from_numpy(np.asarray(mask))[None, :, None, :].expand(1, g, 1, -1)
    return F.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=m, scale=scale)[0, :, 0].numpy()


@pytest.mark.parametrize("seed,L", [(0, 70), (1, 64), (2, 17), (3, 300)])
def test_attend_matches_masked_sdpa(seed, L):
    rng = np.random.default_rng(seed)
    g, d = 3, 16
    q = rng.standard_normal((g, d))
    K = rng.standard_normal((L + 5, d))
    V = rng.standard_normal((L + 5, d))
    M = O.num_blocks(L)
    blocks = sorted(set(rng.choice(M, size=max(1, M // 2), replace=False).tolist()) | {M - 1})
    scale = 0.3
    out = O.attend(q, K, V, L, blocks, scale)
    mask = np.array([(t // 16 in blocks) and t < L for t in range(L + 5)])[None, :]
    np.testing.assert_allclose(out, _sdpa(q, K, V, mask, scale), rtol=1e-12, atol=1e-12)


def test_dense_matches_sdpa():
    rng = np.random.default_rng(12)
    g, d, L = 7, 128, 16 * 20 + 3
    q = rng.standard_normal((g, d))
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    scale = float(np.float32(1 / math.sqrt(d)))
    mask = np.ones((1, L), dtype=bool)
    np.testing.assert_allclose(O.dense(q, K, V, L, scale), _sdpa(q, K, V, mask, scale),
                               rtol=1e-12, atol=1e-12)


def test_attend_large_logits_stable():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((2, 8)) * 50
    K = rng.standard_normal((40, 8)) * 50
    V = rng.standard_normal((40, 8))
    out = O.attend(q, K, V, 40, [0, 2], 1.0)
    mask = np.array([t // 16 in (0, 2) for t in range(40)])[None, :]
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out, _sdpa(q, K, V, mask, 1.0), rtol=1e-10, atol=1e-12)


def test_attend_zero_query_is_mean_of_selected_rows():
    rng = np.random.default_rng(14)
    K = rng.standard_normal((50, 8))
    V = rng.standard_normal((50, 8))
    out = O.attend(np.zeros((2, 8)), K, V, 50, [1, 3], 0.5)
    rows = list(range(16, 32)) + [48, 49]
    np.testing.assert_allclose(out, np.broadcast_to(V[rows].mean(axis=0), (2, 8)), rtol=1e-13)


def test_attend_single_valid_row_returns_it():
    rng = np.random.default_rng(15)
    K = rng.standard_normal((49, 8))
    V = rng.standard_normal((49, 8))
    out = O.attend(rng.standard_normal((3, 8)), K, V, 49, [3], 0.7)
    np.testing.assert_allclose(out, np.broadcast_to(V[48], (3, 8)), rtol=1e-14)


def test_attend_order_of_blocks_irrelevant():
    rng = np.random.default_rng(16)
    q = rng.standard_normal((2, 8))
    K = rng.standard_normal((100, 8))
    V = rng.standard_normal((100, 8))
    a = O.attend(q, K, V, 100, [0, 3, 6], 0.4)
    b = O.attend(q, K, V, 100, [6, 0, 3], 0.4)
    np.testing.assert_allclose(a, b, rtol=1e-13)


def test_attend_all_blocks_is_dense():
    rng = np.random.default_rng(17)
    q = rng.standard_normal((2, 8))
    K = rng.standard_normal((77, 8))
    V = rng.standard_normal((77, 8))
    np.testing.assert_allclose(O.attend(q, K, V, 77, range(5), 0.4), O.dense(q, K, V, 77, 0.4),
                               rtol=1e-14)


# ---------------------------------------------------------------- rectification

def _rect_case(seed, L, f, g=2, d=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((f, g, d)), rng.standard_normal((f, d)), rng.standard_normal((f, d)),
            rng.standard_normal((L, d)), rng.standard_normal((L, d)))


@pytest.mark.parametrize("seed,L,f", [(0, 100, 20), (1, 64, 64), (2, 33, 1), (3, 200, 37)])
def test_rectify_matches_causal_sdpa(seed, L, f):
    qc, kn, vn, K, V = _rect_case(seed, L, f)
    out, K2, V2, tb, lo, hi = O.rectify(qc, kn, vn, K, V, L, 0.35)
    P = L - f
    Kref = K.copy()
    Kref[P:] = kn
    Vref = V.copy()
    Vref[P:] = vn
    for t in range(f):
        mask = (np.arange(L) <= P + t)[None, :]
        np.testing.assert_allclose(out[t], _sdpa(qc[t], Kref, Vref, mask, 0.35),
                                   rtol=1e-12, atol=1e-12)


def test_rectify_rows_and_descriptors():
    L, f = 150, 40
    qc, kn, vn, K, V = _rect_case(4, L, f)
    out, K2, V2, tb, lo, hi = O.rectify(qc, kn, vn, K, V, L, 0.35)
    np.testing.assert_array_equal(K2[L - f:], kn)
    np.testing.assert_array_equal(V2[L - f:], vn)
    np.testing.assert_array_equal(K2[: L - f], K[: L - f])
    assert tb == list(range((L - f) // 16, O.num_blocks(L)))
    full_lo, full_hi = O.descriptors(K2, L)
    np.testing.assert_array_equal(lo, full_lo[tb])
    np.testing.assert_array_equal(hi, full_hi[tb])
    old_lo, _ = O.descriptors(K, L)
    np.testing.assert_array_equal(full_lo[: tb[0]], old_lo[: tb[0]])


def test_rectify_single_row_window_is_dense_decode():
    qc, kn, vn, K, V = _rect_case(5, 90, 1)
    out, K2, V2, *_ = O.rectify(qc, kn, vn, K, V, 90, 0.5)
    np.testing.assert_allclose(out[0], O.dense(qc[0], K2, V2, 90, 0.5), rtol=1e-14)


def test_rectify_is_causal():
    qc, kn, vn, K, V = _rect_case(6, 80, 10)
    out1 = O.rectify(qc, kn, vn, K, V, 80, 0.5)[0]
    kn2, vn2 = kn.copy(), vn.copy()
    kn2[5:] += 3.0
    vn2[5:] -= 2.0
    out2 = O.rectify(qc, kn2, vn2, K, V, 80, 0.5)[0]
    np.testing.assert_array_equal(out1[:5], out2[:5])
    assert not np.allclose(out1[5:], out2[5:])
