"""GPU parity of every library call against the CPU oracle on small seeded
inputs that still span several tiles, splits and a ragged tail, plus the
degenerate cases of the method.  Runs through the C ABI (ctypes binding)."""

import numpy as np
import pytest
import torch

import block_sparse_attention_resa_amd as resa
import oracle as O
from synth import WORKLOADS, make_rectify_inputs, num_blocks
from tests import gpu_common as C

pytestmark = pytest.mark.gpu

BF = WORKLOADS["qwen7b_ctx32k_b1"]

CASES = {
    "tiny_f32_ctx2k": dict(spec=WORKLOADS["tiny_f32_ctx2k"]),
    "bf16_d128_L647": dict(spec=BF.with_(seq_lens=(16 * 40 + 7,))),
    "bf16_ragged_r3_perm_nan": dict(spec=BF.with_(num_requests=3, seq_lens=(1, 17, 16 * 57 + 3)),
                                    permute=True, pad_fill=float("nan")),
    "bf16_d64_h2_g3": dict(spec=BF.with_(num_kv_heads=2, group_size=3, head_dim=64, seq_lens=(5000,),
                                         outlier_channels=4)),
    "f32_d128_h2_g5": dict(spec=WORKLOADS["tiny_f32_ctx2k"].with_(num_kv_heads=2, group_size=5,
                                                                  head_dim=128, seq_lens=(1000,))),
    "bf16_g16_L3000": dict(spec=BF.with_(num_kv_heads=1, group_size=16, seq_lens=(3000,))),
    # 17 KV heads: more heads than one scoring workgroup holds (two head groups)
    "bf16_h17_g2": dict(spec=BF.with_(num_kv_heads=17, group_size=2, seq_lens=(1500,), outlier_channels=4)),
    "bf16_mean_pool": dict(spec=BF.with_(seq_lens=(4000,)), score_mode=resa.RESA_SCORE_MEAN_POOL),
    "bf16_budget3_local3": dict(spec=BF.with_(seq_lens=(2000,), budget_num=3, budget_den=10,
                                              local_blocks=3, min_blocks=4)),
    "bf16_floor_covers_all": dict(spec=BF.with_(seq_lens=(16 * 12 + 5,))),
    "bf16_extra_table_cols": dict(spec=BF.with_(num_requests=2, seq_lens=(700, 1500)), extra_blocks=37),
}


def run_step(case):
    """resa_sparse_step on a case (no tail refresh): (sel_idx, sel_cnt, out)."""
    R, H, HG, d = case.R, case.spec.num_kv_heads, case.spec.num_q_heads, case.spec.head_dim
    ms = C.max_sel_for(case)
    sel_idx = torch.full((R, H, ms), -7, dtype=torch.int32, device="cuda")
    sel_cnt = torch.full((R, H), -7, dtype=torch.int32, device="cuda")
    out = torch.full((R, HG, d), float("nan"), device="cuda")
    ws = resa.alloc_workspace(case.cfg, resa.OP_SPARSE_STEP, R, case.kv.max_blocks, ms)
    resa.sparse_step(case.cfg, case.kv, case.inp.q, sel_idx, sel_cnt, out, ws)
    return sel_idx, sel_cnt, out


def make(name, seed=11):
    kw = dict(CASES[name])
    spec = kw.pop("spec")
    return C.make_case(spec, seed, **kw)


@pytest.fixture(autouse=True)
def _gpu():
    C.require_gpu()


def oracle_scores(case, r, i):
    K = C.keys_of(case, r, i)
    lo, hi = O.descriptors(K, case.inp.seq_lens[r])
    mode = O.SCORE_MEAN_POOL if case.cfg.score_mode == resa.RESA_SCORE_MEAN_POOL else O.SCORE_SUM_HEADS
    return O.scores(C.group_q(case, r, i), lo, hi, mode)


@pytest.mark.parametrize("name", list(CASES))
def test_descriptors_bit_exact(name):
    case = make(name)
    C.run_descriptors(case)
    torch.cuda.synchronize()
    for r in range(case.R):
        for i in range(case.spec.num_kv_heads):
            C.check_descriptors(case, r, i, C.keys_of(case, r, i), case.inp.seq_lens[r])


@pytest.mark.parametrize("name", ["bf16_d128_L647", "bf16_ragged_r3_perm_nan", "tiny_f32_ctx2k"])
def test_descriptor_ranges_tail_and_first_block(name):
    case = make(name)
    C.run_descriptors(case)
    full = case.kv.desc_pool.clone()
    # Spoil every descriptor, then rebuild only the last block of each request.
    case.kv.desc_pool.fill_(3.0)
    C.run_descriptors(case, None, 1)
    torch.cuda.synchronize()
    for r, L in enumerate(case.inp.seq_lens):
        M = num_blocks(L)
        p = int(case.kv.block_table[r, M - 1])
        assert torch.equal(C.desc_bits(case.kv.desc_pool[p]), C.desc_bits(full[p]))
        if M > 1:
            p0 = int(case.kv.block_table[r, 0])
            assert bool((case.kv.desc_pool[p0] == 3.0).all())
    # explicit per-request ranges
    case.kv.desc_pool.fill_(3.0)
    first = torch.tensor([max(0, num_blocks(L) - 3) for L in case.inp.seq_lens], dtype=torch.int32,
                         device="cuda")
    C.run_descriptors(case, first, 2)
    torch.cuda.synchronize()
    for r, L in enumerate(case.inp.seq_lens):
        M = num_blocks(L)
        f = max(0, M - 3)
        for b in range(M):
            p = int(case.kv.block_table[r, b])
            if f <= b < min(M, f + 2):
                assert torch.equal(C.desc_bits(case.kv.desc_pool[p]), C.desc_bits(full[p]))
            else:
                assert bool((case.kv.desc_pool[p] == 3.0).all())


@pytest.mark.parametrize("name", ["bf16_d128_L647", "bf16_ragged_r3_perm_nan", "tiny_f32_ctx2k",
                                  "bf16_budget3_local3"])
def test_score_select_refreshes_tail_descriptor(name):
    case = make(name)
    C.run_descriptors(case)
    full = case.kv.desc_pool.clone()
    sel_ref, cnt_ref, _ = C.run_score_select(case, with_scores=False)
    # spoil the last block's descriptor of every request; the fused refresh restores it
    for r, L in enumerate(case.inp.seq_lens):
        p = int(case.kv.block_table[r, num_blocks(L) - 1])
        case.kv.desc_pool[p] = 7.0
    R, H = case.R, case.spec.num_kv_heads
    ms = C.max_sel_for(case)
    sel_idx = torch.full((R, H, ms), -7, dtype=torch.int32, device="cuda")
    sel_cnt = torch.full((R, H), -7, dtype=torch.int32, device="cuda")
    ws = resa.alloc_workspace(case.cfg, resa.OP_SCORE_SELECT, R, case.kv.max_blocks, ms)
    resa.score_select(case.cfg, case.kv, case.inp.q, sel_idx, sel_cnt, ws, refresh_tail=True)
    torch.cuda.synchronize()
    assert torch.equal(C.desc_bits(case.kv.desc_pool), C.desc_bits(full))
    # the tail block is forced, so its (spoiled) score cannot change the selection
    assert torch.equal(sel_idx, sel_ref) and torch.equal(sel_cnt, cnt_ref)


@pytest.mark.parametrize("name", list(CASES))
def test_score_select_parity(name):
    case = make(name)
    C.run_descriptors(case)
    sel_idx, sel_cnt, scores = C.run_score_select(case)
    sel_idx2, sel_cnt2, _ = C.run_score_select(case, with_scores=False)
    torch.cuda.synchronize()
    assert torch.equal(sel_idx, sel_idx2) and torch.equal(sel_cnt, sel_cnt2), "selection not deterministic"
    lists = C.sel_lists(sel_idx, sel_cnt)
    ms = sel_idx.shape[2]
    for r in range(case.R):
        M = num_blocks(case.inp.seq_lens[r])
        for i in range(case.spec.num_kv_heads):
            S = oracle_scores(case, r, i)
            g = scores[r, i, :M].cpu().numpy().astype(np.float64)
            assert np.all(np.abs(g - S) <= 2e-5 * (np.abs(S) + np.abs(S).mean() + 1e-6)), \
                f"scores differ: {np.abs(g - S).max()}"
            C.check_selection(S, lists[r][i], case.cfg, tag=f"{name} r{r} i{i}")
            tail = sel_idx[r, i, int(sel_cnt[r, i]):].cpu()
            assert bool((tail == -1).all()), "unused sel_idx entries must be -1"
            assert len(lists[r][i]) <= ms


@pytest.mark.parametrize("name", list(CASES))
def test_sparse_decode_parity(name):
    case = make(name)
    C.run_descriptors(case)
    sel_idx, sel_cnt, _ = C.run_score_select(case)
    out = C.run_sparse(case, sel_idx, sel_cnt)
    # the same kernel on the oracle's own selection
    ms = sel_idx.shape[2]
    o_idx = torch.full_like(sel_idx, -1)
    o_cnt = torch.zeros_like(sel_cnt)
    o_sets = {}
    for r in range(case.R):
        for i in range(case.spec.num_kv_heads):
            s = O.select(oracle_scores(case, r, i), case.cfg.budget_num, case.cfg.budget_den,
                         case.cfg.min_blocks, case.cfg.local_blocks).tolist()
            o_sets[r, i] = s
            o_idx[r, i, : len(s)] = torch.tensor(s, dtype=torch.int32)
            o_cnt[r, i] = len(s)
    assert ms >= max(len(s) for s in o_sets.values())
    out_o = C.run_sparse(case, o_idx, o_cnt)
    torch.cuda.synchronize()
    lists = C.sel_lists(sel_idx, sel_cnt)
    g = case.spec.group_size
    scale = C.sm_scale(case.cfg)
    for r in range(case.R):
        L = case.inp.seq_lens[r]
        for i in range(case.spec.num_kv_heads):
            K, V, q = C.keys_of(case, r, i), C.values_of(case, r, i), C.group_q(case, r, i)
            ref_gpu_set = O.attend(q, K, V, L, lists[r][i], scale)
            C.check_out(out[r, i * g:(i + 1) * g].cpu().numpy(), ref_gpu_set, f"{name} r{r} i{i} own set")
            ref_o = O.attend(q, K, V, L, o_sets[r, i], scale)
            C.check_out(out_o[r, i * g:(i + 1) * g].cpu().numpy(), ref_o, f"{name} r{r} i{i} oracle set")


@pytest.mark.parametrize("name", list(CASES))
def test_dense_decode_parity(name):
    case = make(name)
    out = C.run_dense(case)
    torch.cuda.synchronize()
    g = case.spec.group_size
    scale = C.sm_scale(case.cfg)
    for r in range(case.R):
        L = case.inp.seq_lens[r]
        for i in range(case.spec.num_kv_heads):
            ref = O.dense(C.group_q(case, r, i), C.keys_of(case, r, i), C.values_of(case, r, i), L, scale)
            C.check_out(out[r, i * g:(i + 1) * g].cpu().numpy(), ref, f"{name} r{r} i{i}")


@pytest.mark.parametrize("name", ["bf16_d128_L647", "bf16_ragged_r3_perm_nan", "tiny_f32_ctx2k"])
def test_sparse_with_every_block_equals_dense(name):
    case = make(name)
    R, H = case.R, case.spec.num_kv_heads
    mb = case.kv.max_blocks
    idx = torch.full((R, H, mb), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros((R, H), dtype=torch.int32, device="cuda")
    for r, L in enumerate(case.inp.seq_lens):
        M = num_blocks(L)
        perm = torch.randperm(M, generator=torch.Generator().manual_seed(r)).to(torch.int32)
        idx[r, :, :M] = perm.to("cuda")  # any order of the full list
        cnt[r] = M
    sp = C.run_sparse(case, idx, cnt)
    de = C.run_dense(case)
    torch.cuda.synchronize()
    C.check_out(sp.cpu().numpy(), de.cpu().numpy().astype(np.float64), f"{name} all-blocks")


def test_split_count_changes_rounding_only():
    case = make("bf16_d128_L647")
    outs = []
    for S in (1, 2, 7, 41):
        case.cfg.num_splits = S
        outs.append(C.run_dense(case).cpu().numpy())
    for o in outs[1:]:
        C.check_out(o, outs[0].astype(np.float64), "split invariance")
    case.cfg.num_splits = 0
    a = C.run_dense(case)
    b = C.run_dense(case)
    assert torch.equal(a, b), "dense decode not bitwise deterministic"


def test_many_splits_merge_batches():
    """Split counts on both sides of every change of the merge's lanes per
    output float4, one split (the decode writes the output, no merge), and
    more splits than one lane group folds in one batch of loads (64), so the
    merge runs several batches; dense and all-blocks sparse decode against the
    oracle's dense attention."""
    case = make("bf16_d64_h2_g3")  # 5000 rows: 313 blocks
    M = num_blocks(case.inp.seq_lens[0])
    g = case.spec.group_size
    scale = C.sm_scale(case.cfg)
    refs = {}
    for i in range(case.spec.num_kv_heads):
        refs[i] = O.dense(C.group_q(case, 0, i), C.keys_of(case, 0, i), C.values_of(case, 0, i),
                          case.inp.seq_lens[0], scale)
    idx = torch.full((1, case.spec.num_kv_heads, M), -1, dtype=torch.int32, device="cuda")
    idx[0, :, :] = torch.arange(M, dtype=torch.int32, device="cuda")
    cnt = torch.full((1, case.spec.num_kv_heads), M, dtype=torch.int32, device="cuda")
    # every lanes-per-float4 boundary of the merge (1, 2, 4, 8, 16 lanes take
    # up to 4, 8, 16, 32, 64 splits in one batch), one split (no merge), and
    # several batches
    for S in (1, 4, 5, 8, 9, 16, 17, 32, 33, 64, 65, 129, 200, M):
        case.cfg.num_splits = S
        de = C.run_dense(case)
        sp = C.run_sparse(case, idx, cnt)
        torch.cuda.synchronize()
        for i in range(case.spec.num_kv_heads):
            C.check_out(de[0, i * g:(i + 1) * g].cpu().numpy(), refs[i], f"dense S={S} i{i}")
            C.check_out(sp[0, i * g:(i + 1) * g].cpu().numpy(), refs[i], f"sparse all-blocks S={S} i{i}")
    case.cfg.num_splits = 0


def test_zero_length_request():
    spec = BF.with_(num_requests=2, seq_lens=(33, 700))
    case = C.make_case(spec, 5)
    case.kv.seq_lens[0] = 0
    C.run_descriptors(case)
    sel_idx, sel_cnt, _ = C.run_score_select(case)
    sp = C.run_sparse(case, sel_idx, sel_cnt)
    de = C.run_dense(case)
    st_idx, st_cnt, st_out = run_step(case)
    torch.cuda.synchronize()
    assert int(sel_cnt[0].abs().sum()) == 0
    assert bool((sel_idx[0] == -1).all())
    assert float(sp[0].abs().max()) == 0.0 and float(de[0].abs().max()) == 0.0
    # the step call: the same selection, a zero output for the empty request
    assert torch.equal(st_idx, sel_idx) and torch.equal(st_cnt, sel_cnt)
    assert torch.equal(st_out, sp)
    g = spec.group_size
    for i in range(spec.num_kv_heads):
        ref = O.dense(C.group_q(case, 1, i), C.keys_of(case, 1, i), C.values_of(case, 1, i), 700,
                      C.sm_scale(case.cfg))
        C.check_out(de[1, i * g:(i + 1) * g].cpu().numpy(), ref, "second request")


# ---------------------------------------------------------------- rectification

RECT = {
    "bf16_r2_ragged_chunk20_nan": dict(spec=BF.with_(num_kv_heads=2, group_size=3, num_requests=2,
                                                     seq_lens=(300, 259)), chunk=20, pad_fill=float("nan"),
                                       permute=True),
    "bf16_d128_g7_chunk64": dict(spec=BF.with_(seq_lens=(1500,)), chunk=64),
    "f32_whole_cache": dict(spec=WORKLOADS["tiny_f32_ctx2k"].with_(seq_lens=(100,)), chunk=100),
    "bf16_chunk1": dict(spec=BF.with_(num_kv_heads=1, seq_lens=(77,)), chunk=1),
    "bf16_short_request_skipped": dict(spec=BF.with_(num_kv_heads=2, num_requests=2, seq_lens=(10, 400)),
                                       chunk=20),
    "bf16_d64_chunk37": dict(spec=BF.with_(num_kv_heads=2, group_size=2, head_dim=64, seq_lens=(2000,)),
                             chunk=37),
}


@pytest.mark.parametrize("name", list(RECT))
def test_rectify_parity(name):
    kw = dict(RECT[name])
    spec, chunk = kw.pop("spec"), kw.pop("chunk")
    case = C.make_case(spec, 21, **kw)
    C.run_descriptors(case)
    R, H, g, d = spec.num_requests, spec.num_kv_heads, spec.group_size, spec.head_dim
    qc, kn, vn = make_rectify_inputs(spec, 21, chunk, device="cuda")
    K0, V0 = C.logical_cache(case)
    K0 = [k.clone() for k in K0]
    V0 = [v.clone() for v in V0]
    out = torch.full((R, chunk, H * g, d), float("nan"), device="cuda")
    ws = resa.alloc_workspace(case.cfg, resa.OP_DENSE_RECTIFY, R, case.kv.max_blocks, chunk=chunk)
    resa.dense_rectify(case.cfg, case.kv, qc, kn, vn, out, ws)
    torch.cuda.synchronize()
    K1, V1 = C.logical_cache(case)
    scale = C.sm_scale(case.cfg)
    for r in range(R):
        L = case.inp.seq_lens[r]
        if L < chunk:  # skipped: cache untouched, output zero
            assert torch.equal(K1[r], K0[r]) and torch.equal(V1[r], V0[r])
            assert float(out[r].abs().max()) == 0.0
            continue
        P = L - chunk
        for i in range(H):
            # rows: the window is overwritten bit-exactly, everything else untouched
            assert torch.equal(K1[r][i, P:L], kn[r, :, i]) and torch.equal(V1[r][i, P:L], vn[r, :, i])
            assert torch.equal(K1[r][i, :P], K0[r][i, :P]) and torch.equal(V1[r][i, :P], V0[r][i, :P])
            Kr = C.np64(K0[r][i])
            Vr = C.np64(V0[r][i])
            ref, K2, V2, tb, lo, hi = O.rectify(C.np64(qc[r, :, i * g:(i + 1) * g]), C.np64(kn[r, :, i]),
                                                C.np64(vn[r, :, i]), Kr, Vr, L, scale)
            # descriptors of every block equal a rebuild of the rewritten cache
            C.check_descriptors(case, r, i, K2, L)
            C.check_out(out[r, :, i * g:(i + 1) * g].cpu().numpy(), ref, f"{name} r{r} i{i}")


def test_rectify_long_split_fallback_kernel():
    """A caller-forced single split longer than the LDS kernel's page-id list
    (2048 blocks) takes the direct-load kernel; both kernels against the oracle."""
    spec = BF.with_(num_kv_heads=1, seq_lens=(16 * 2100 + 9,))
    chunk = 32
    outs = {}
    for S in (1, 0):
        case = C.make_case(spec, 31)
        case.cfg.num_splits = S
        C.run_descriptors(case)
        qc, kn, vn = make_rectify_inputs(spec, 31, chunk, device="cuda")
        K0, V0 = C.logical_cache(case)
        out = torch.full((1, chunk, spec.group_size * 1, spec.head_dim), float("nan"), device="cuda")
        ws = resa.alloc_workspace(case.cfg, resa.OP_DENSE_RECTIFY, 1, case.kv.max_blocks, chunk=chunk)
        resa.dense_rectify(case.cfg, case.kv, qc, kn, vn, out, ws)
        torch.cuda.synchronize()
        outs[S] = out
        L = case.inp.seq_lens[0]
        ref, K2, V2, tb, lo, hi = O.rectify(C.np64(qc[0]), C.np64(kn[0, :, 0]), C.np64(vn[0, :, 0]),
                                            C.np64(K0[0][0]), C.np64(V0[0][0]), L, C.sm_scale(case.cfg))
        C.check_descriptors(case, 0, 0, K2, L)
        C.check_out(out[0].cpu().numpy(), ref, f"rectify splits={S}")
    assert resa.num_splits(case.cfg, resa.OP_DENSE_RECTIFY, 1, case.kv.max_blocks, 0, chunk) > 1


def test_out_of_range_device_values_are_clamped():
    """Values read from device memory are clamped into range (the conventions
    in include/resa.h): a sequence length past the table's capacity acts as the
    capacity and a negative one as 0, block-table entries outside the pool act
    as the nearest pool block, selected ids outside the table as the nearest
    column and a count past the list as the list.  Each run with out-of-range
    values must equal, bit for bit, the run with the clamped values."""
    import dataclasses

    case = make("bf16_d128_L647")
    C.run_descriptors(case)
    kv = case.kv
    P, mb = int(kv.k_pool.shape[0]), kv.max_blocks

    def with_kv(table=None, seq=None):
        return dataclasses.replace(case, kv=resa.PagedKV(kv.k_pool, kv.v_pool, kv.desc_pool,
                                                          kv.block_table if table is None else table,
                                                          kv.seq_lens if seq is None else seq))

    def all_outputs(c):
        sel, cnt, sc = C.run_score_select(c)
        sp = C.run_sparse(c, sel, cnt)
        de = C.run_dense(c)
        st_sel, st_cnt, st_out = run_step(c)
        torch.cuda.synchronize()
        return [sel, cnt, sc, sp, de, st_sel, st_cnt, st_out]

    def same(a, b, tag):
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), tag

    def seq(v):
        return torch.tensor([v], dtype=torch.int32, device="cuda")

    same(all_outputs(with_kv(seq=seq(2 ** 30))), all_outputs(with_kv(seq=seq(mb * 16))), "long sequence length")
    neg = all_outputs(with_kv(seq=seq(-5)))
    same(neg, all_outputs(with_kv(seq=seq(0))), "negative sequence length")
    assert int(neg[1].abs().sum()) == 0 and float(neg[4].abs().max()) == 0.0

    bad, clamped = kv.block_table.clone(), kv.block_table.clone()
    bad[0, 3], clamped[0, 3] = -7, 0
    bad[0, 5], clamped[0, 5] = P + 1000, P - 1
    same(all_outputs(with_kv(table=bad)), all_outputs(with_kv(table=clamped)), "block-table entries")

    sel, cnt, _ = C.run_score_select(case)
    M = num_blocks(case.inp.seq_lens[0])
    ms = sel.shape[2]
    sel_bad, sel_c = sel.clone(), sel.clone()
    sel_bad[0, 0, 1], sel_c[0, 0, 1] = -4, 0
    sel_bad[0, 0, 2], sel_c[0, 0, 2] = mb + 9, mb - 1
    cnt_bad, cnt_c = cnt.clone(), cnt.clone()
    cnt_bad[0, 1], cnt_c[0, 1] = ms + 50, min(ms, M)
    a = C.run_sparse(case, sel_bad, cnt_bad)
    b = C.run_sparse(case, sel_c, cnt_c)
    torch.cuda.synchronize()
    assert torch.equal(a, b), "selected ids and counts"


def test_large_batch_single_split():
    """64 requests x 4 KV heads: the automatic split count is one, so the
    sparse decode, the dense decode and the step write their outputs from
    the attention workgroups (no merge launch).  All three against the
    oracle, and the sparse decode against a run forced to two splits (merge
    launch) within rounding."""
    import dataclasses

    R = 64
    spec = BF.with_(num_requests=R, seq_lens=tuple(300 + 37 * r for r in range(R)))
    case = C.make_case(spec, 17)
    ms = C.max_sel_for(case)
    assert resa.num_splits(case.cfg, resa.OP_SPARSE_DECODE, R, case.kv.max_blocks, ms) == 1
    assert resa.num_splits(case.cfg, resa.OP_DENSE_DECODE, R, case.kv.max_blocks) == 1
    C.run_descriptors(case)
    sel_idx, sel_cnt, _ = C.run_score_select(case)
    sp = C.run_sparse(case, sel_idx, sel_cnt)
    de = C.run_dense(case)
    st_idx, st_cnt, st_out = run_step(case)
    two = dataclasses.replace(case, cfg=dataclasses.replace(case.cfg, num_splits=2))
    sp2 = C.run_sparse(two, sel_idx, sel_cnt)
    torch.cuda.synchronize()
    assert torch.equal(st_idx, sel_idx) and torch.equal(st_cnt, sel_cnt)
    assert torch.equal(st_out, sp), "step and two calls split the list the same way"
    C.check_out(sp.cpu().numpy(), sp2.cpu().numpy().astype(np.float64), "one split against two")
    lists = C.sel_lists(sel_idx, sel_cnt)
    g = spec.group_size
    scale = C.sm_scale(case.cfg)
    for r in range(0, R, 9):
        L = case.inp.seq_lens[r]
        for i in range(spec.num_kv_heads):
            q, K, V = C.group_q(case, r, i), C.keys_of(case, r, i), C.values_of(case, r, i)
            C.check_out(sp[r, i * g:(i + 1) * g].cpu().numpy(), O.attend(q, K, V, L, lists[r][i], scale),
                        f"sparse r{r} i{i}")
            C.check_out(de[r, i * g:(i + 1) * g].cpu().numpy(), O.dense(q, K, V, L, scale), f"dense r{r} i{i}")
