"""resa_sparse_step (scoring, then the selection fused with the split
attention, then the merge) against the CPU oracle and against the two-call
path (resa_score_select + resa_sparse_decode): the same selection id for id,
the tail descriptor refreshed bit-exactly, and attention outputs within the
output tolerance of the oracle on the selected blocks.  Covers the small
parity cases (ragged, permuted pools, NaN padding, d = 64, fp32, g = 16,
mean-pooled scoring, wider local windows, the n_min floor, extra table
columns), crafted score distributions on both sides of every change of the
fused kernel's keys per thread and of its fallbacks, the full-size
workloads, repeated calls on one workspace and graph replays."""

import numpy as np
import pytest
import torch

import block_sparse_attention_resa_amd as resa
import oracle as O
from synth import WORKLOADS, num_blocks
from tests import gpu_common as C
from tests.test_gpu_parity import CASES, make, oracle_scores
from tests.test_gpu_select import distribution

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    C.require_gpu()


def run_step(case, q=None, refresh_tail=False, ws=None):
    R, H, HG, d = case.R, case.spec.num_kv_heads, case.spec.num_q_heads, case.spec.head_dim
    ms = C.max_sel_for(case)
    sel_idx = torch.full((R, H, ms), -7, dtype=torch.int32, device="cuda")
    sel_cnt = torch.full((R, H), -7, dtype=torch.int32, device="cuda")
    out = torch.full((R, HG, d), float("nan"), device="cuda")
    if ws is None:
        ws = resa.alloc_workspace(case.cfg, resa.OP_SPARSE_STEP, R, case.kv.max_blocks, ms)
    resa.sparse_step(case.cfg, case.kv, case.inp.q if q is None else q, sel_idx, sel_cnt, out, ws,
                     refresh_tail=refresh_tail)
    return sel_idx, sel_cnt, out


def check_step_against_oracle(case, sel_idx, sel_cnt, out, q=None, tag=""):
    lists = C.sel_lists(sel_idx, sel_cnt)
    g = case.spec.group_size
    scale = C.sm_scale(case.cfg)
    qq = case.inp.q if q is None else q
    for r in range(case.R):
        L = case.inp.seq_lens[r]
        for i in range(case.spec.num_kv_heads):
            K, V = C.keys_of(case, r, i), C.values_of(case, r, i)
            qg = C.np64(qq[r, i * g:(i + 1) * g])
            lo, hi = O.descriptors(K, L)
            mode = O.SCORE_MEAN_POOL if case.cfg.score_mode == resa.RESA_SCORE_MEAN_POOL else O.SCORE_SUM_HEADS
            C.check_selection(O.scores(qg, lo, hi, mode), lists[r][i], case.cfg, tag=f"{tag} r{r} i{i}")
            C.check_out(out[r, i * g:(i + 1) * g].cpu().numpy(), O.attend(qg, K, V, L, lists[r][i], scale),
                        f"{tag} step r{r} i{i}")


@pytest.mark.parametrize("name", list(CASES))
def test_step_matches_two_calls_and_oracle(name):
    case = make(name)
    C.run_descriptors(case)
    sel_ref, cnt_ref, _ = C.run_score_select(case, with_scores=False)
    out_ref = C.run_sparse(case, sel_ref, cnt_ref)
    sel_idx, sel_cnt, out = run_step(case)
    torch.cuda.synchronize()
    assert torch.equal(sel_idx, sel_ref) and torch.equal(sel_cnt, cnt_ref), "selection differs from score_select"
    C.check_out(out.cpu().numpy(), out_ref.cpu().numpy().astype(np.float64), f"{name} vs two calls")
    check_step_against_oracle(case, sel_idx, sel_cnt, out, tag=name)


@pytest.mark.parametrize("name", ["bf16_d128_L647", "bf16_ragged_r3_perm_nan", "tiny_f32_ctx2k"])
def test_step_refreshes_tail_descriptor(name):
    case = make(name)
    C.run_descriptors(case)
    full = case.kv.desc_pool.clone()
    for r, L in enumerate(case.inp.seq_lens):
        p = int(case.kv.block_table[r, num_blocks(L) - 1])
        case.kv.desc_pool[p] = 7.0
    sel_idx, sel_cnt, out = run_step(case, refresh_tail=True)
    torch.cuda.synchronize()
    assert torch.equal(C.desc_bits(case.kv.desc_pool), C.desc_bits(full))
    check_step_against_oracle(case, sel_idx, sel_cnt, out, tag=name)


def test_step_repeated_calls_on_one_workspace():
    """Several calls with different queries on one workspace, each checked."""
    case = make("bf16_extra_table_cols")
    C.run_descriptors(case)
    ms = C.max_sel_for(case)
    ws = resa.alloc_workspace(case.cfg, resa.OP_SPARSE_STEP, case.R, case.kv.max_blocks, ms)
    gen = torch.Generator(device="cuda").manual_seed(5)
    for rep in range(3):
        q = torch.randn(case.inp.q.shape, device="cuda", generator=gen).to(case.inp.q.dtype)
        sel_idx, sel_cnt, out = run_step(case, q=q, ws=ws)
        torch.cuda.synchronize()
        check_step_against_oracle(case, sel_idx, sel_cnt, out, q=q, tag=f"rep{rep}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,seed,layer", [("qwen7b_ctx32k_b1", 101, 0), ("qwen7b_ragged_b8", 102, 0),
                                             ("qwen7b_ctx131k_b4_rectify", 103, 0),
                                             ("qwen7b_ctx256k_l28", 2024, 0)])
def test_step_full_size_workloads(name, seed, layer):
    spec = WORKLOADS[name]
    case = C.make_case(spec, seed=seed, layer=layer, permute=name == "qwen7b_ragged_b8")
    C.run_descriptors(case)
    sel_idx, sel_cnt, out = run_step(case, refresh_tail=True)
    sel_ref, cnt_ref, _ = C.run_score_select(case, with_scores=False)
    torch.cuda.synchronize()
    assert torch.equal(sel_idx, sel_ref) and torch.equal(sel_cnt, cnt_ref)
    check_step_against_oracle(case, sel_idx, sel_cnt, out, tag=name)


def test_step_graph_replays_match_oracle():
    """The step of three layers captured in a HIP graph, replayed four times
    with eager work and synchronisations in between; every replay is checked
    against the oracle and is bit-identical to the eager call."""
    spec = WORKLOADS["qwen7b_ctx32k_b1"]
    cases = [C.make_case(spec, seed=400 + l) for l in range(3)]
    R, H, g, d = 1, spec.num_kv_heads, spec.group_size, spec.head_dim
    state = []
    for case in cases:
        C.run_descriptors(case)
        ms = C.max_sel_for(case)
        state.append(dict(case=case, sel_idx=torch.full((R, H, ms), -5, dtype=torch.int32, device="cuda"),
                          sel_cnt=torch.zeros((R, H), dtype=torch.int32, device="cuda"),
                          out=torch.zeros((R, H * g, d), device="cuda"),
                          ws=resa.alloc_workspace(case.cfg, resa.OP_SPARSE_STEP, R, case.kv.max_blocks, ms)))

    def step():
        for st in state:
            c = st["case"]
            resa.sparse_step(c.cfg, c.kv, c.inp.q, st["sel_idx"], st["sel_cnt"], st["out"], st["ws"],
                             refresh_tail=True)

    step()
    torch.cuda.synchronize()
    eager = [(st["sel_idx"].clone(), st["out"].clone()) for st in state]
    for st in state:
        check_step_against_oracle(st["case"], st["sel_idx"], st["sel_cnt"], st["out"], tag="eager")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for st in state:
            st["out"].fill_(float("nan"))
            st["sel_idx"].fill_(-9)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for st, (si, o) in zip(state, eager):
            assert torch.equal(st["sel_idx"], si), f"replay {rep}: selection differs"
            assert torch.equal(st["out"], o), f"replay {rep}: output differs"
            check_step_against_oracle(st["case"], st["sel_idx"], st["sel_cnt"], st["out"], tag=f"replay{rep}")


def run_crafted(dist, M, seed, budget=(1, 10), splits=0):
    """Selection of the step on a crafted bf16 score row: with group size 1,
    a query that is 1 on channel 0 and 0 elsewhere and bf16 descriptors,
    Eq 4's score of block b is exactly hi_0(b) (every other term is an exact
    zero), so the row can hold any bf16 distribution.  Checks sel_idx and
    sel_cnt id for id against the oracle's selection and against
    resa_score_select, and the attention output against the two calls."""
    rng = np.random.default_rng(seed)
    R, H, D = 2, 2, 64
    Ms = [M, max(1, M - 7)]
    mb = M
    P = R * mb
    cfg = resa.Config(num_kv_heads=H, group_size=1, head_dim=D, dtype=resa.RESA_BF16, budget_num=budget[0],
                      budget_den=budget[1], num_splits=splits)
    desc = torch.zeros((P, H, 2, D), dtype=torch.float32)
    S = {}
    for r in range(R):
        for i in range(H):
            s = torch.from_numpy(distribution(dist, rng, Ms[r])).to(torch.bfloat16).float()
            s[s == 0] = 1e-3
            s = s.to(torch.bfloat16).float()
            S[r, i] = s.numpy().astype(np.float64)
            rows = torch.arange(Ms[r]) + r * mb
            desc[rows, i, 0, 0] = s
            desc[rows, i, 1, 0] = s
            desc[rows, i, :, 1:] = torch.from_numpy(rng.normal(0, 1, (Ms[r], 2, D - 1)).astype(np.float32))
    table = (torch.arange(mb, dtype=torch.int32)[None, :] + torch.arange(R, dtype=torch.int32)[:, None] * mb)
    seq = torch.tensor([m * 16 - 3 for m in Ms], dtype=torch.int32)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    kv = resa.PagedKV(torch.randn((P, H, 16, D), device="cuda", generator=gen).to(torch.bfloat16),
                      torch.randn((P, H, D, 16), device="cuda", generator=gen).to(torch.bfloat16),
                      desc.to(torch.bfloat16).cuda(), table.cuda(), seq.cuda())
    q = torch.zeros((R, H, D), dtype=torch.float32)
    q[:, :, 0] = 1.0
    q = q.to(torch.bfloat16).cuda()
    ms = resa.selection_count(cfg, M)
    sel_idx = torch.full((R, H, ms), -7, dtype=torch.int32, device="cuda")
    sel_cnt = torch.zeros((R, H), dtype=torch.int32, device="cuda")
    out = torch.full((R, H, D), float("nan"), device="cuda")
    resa.sparse_step(cfg, kv, q, sel_idx, sel_cnt, out, resa.alloc_workspace(cfg, resa.OP_SPARSE_STEP, R, mb, ms))
    si2 = torch.full_like(sel_idx, -5)
    sc2 = torch.zeros_like(sel_cnt)
    resa.score_select(cfg, kv, q, si2, sc2, resa.alloc_workspace(cfg, resa.OP_SCORE_SELECT, R, mb, ms))
    out2 = torch.full_like(out, float("nan"))
    resa.sparse_decode(cfg, kv, q, si2, sc2, out2, resa.alloc_workspace(cfg, resa.OP_SPARSE_DECODE, R, mb, ms))
    torch.cuda.synchronize()
    assert torch.equal(sel_idx, si2) and torch.equal(sel_cnt, sc2), f"{dist} M={M}: step and score_select differ"
    sel_idx, sel_cnt = sel_idx.cpu(), sel_cnt.cpu()
    for r in range(R):
        for i in range(H):
            ref = O.select(S[r, i], cfg.budget_num, cfg.budget_den, cfg.min_blocks, cfg.local_blocks)
            n = int(sel_cnt[r, i])
            got = sel_idx[r, i, :n].numpy()
            assert n == len(ref), f"{dist} r{r} i{i}: count {n} != {len(ref)}"
            assert np.array_equal(got, ref), \
                f"{dist} M={Ms[r]} r{r} i{i}: first difference at {np.nonzero(got != ref)[0][:3]}"
            assert torch.all(sel_idx[r, i, n:] == -1)
    C.check_out(out.cpu().numpy(), out2.cpu().numpy().astype(np.float64), f"{dist} M={M} vs two calls")


# rows on both sides of every change of the fused kernel's keys per thread
# (2048, 4096 keys) and of its limit (8192 keys; longer rows take the
# selection launch and the decode launch)
@pytest.mark.parametrize("M", [20, 300, 2048, 2052, 4096, 4100, 8192, 8196, 16384, 16388])
@pytest.mark.parametrize("dist", ["normal", "few_levels", "huge_outlier", "clustered_top"])
def test_step_select_sizes(dist, M):
    run_crafted(dist, M, seed=M + 3)


@pytest.mark.parametrize("dist", ["equal", "two_levels", "mixed_sign_wide", "near_float_max", "tiny"])
def test_step_select_distributions_16k(dist):
    run_crafted(dist, 16384, seed=17)


@pytest.mark.parametrize("splits", [1, 2, 7])
@pytest.mark.parametrize("M", [8192, 16384])
def test_step_select_long_lists(M, splits):
    """A 3/5 budget at 8192 blocks: the list (4916 ids) fits the fused
    kernel's LDS list even with one split; at 16384 blocks (9831 ids) every
    split count takes the two-call kernels."""
    run_crafted("normal", M, seed=23 + splits, budget=(3, 5), splits=splits)


@pytest.mark.parametrize("splits", [1, 5, 64])
def test_step_explicit_splits_and_wide_list_rows(splits):
    """An explicit split count and sel_idx rows wider than the selection
    (positions past n must read -1): the step against the two calls, id for
    id and bit for bit (both split the list the same way), and against the
    oracle."""
    case = make("bf16_ragged_r3_perm_nan")
    case.cfg.num_splits = splits
    C.run_descriptors(case)
    R, H, HG, d = case.R, case.spec.num_kv_heads, case.spec.num_q_heads, case.spec.head_dim
    ms = C.max_sel_for(case) + 37
    si = torch.full((R, H, ms), -7, dtype=torch.int32, device="cuda")
    sc = torch.full((R, H), -7, dtype=torch.int32, device="cuda")
    out = torch.full((R, HG, d), float("nan"), device="cuda")
    resa.sparse_step(case.cfg, case.kv, case.inp.q, si, sc, out,
                     resa.alloc_workspace(case.cfg, resa.OP_SPARSE_STEP, R, case.kv.max_blocks, ms))
    si2 = torch.full_like(si, -5)
    sc2 = torch.full_like(sc, -5)
    resa.score_select(case.cfg, case.kv, case.inp.q, si2, sc2,
                      resa.alloc_workspace(case.cfg, resa.OP_SCORE_SELECT, R, case.kv.max_blocks, ms))
    out2 = torch.full_like(out, float("nan"))
    resa.sparse_decode(case.cfg, case.kv, case.inp.q, si2, sc2, out2,
                       resa.alloc_workspace(case.cfg, resa.OP_SPARSE_DECODE, R, case.kv.max_blocks, ms))
    torch.cuda.synchronize()
    assert torch.equal(si, si2) and torch.equal(sc, sc2)
    assert torch.equal(out, out2)
    for r in range(R):
        for i in range(H):
            assert bool((si[r, i, int(sc[r, i]):] == -1).all())
    check_step_against_oracle(case, si, sc, out, tag=f"splits{splits}")
