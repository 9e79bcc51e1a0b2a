"""GPU parity at the full sizes of the five measured workloads, in the launch
configuration bench.py times (automatic split counts), checked against the
CPU oracle on every output the oracle can afford (whole layers for the 32K
and ragged batches, two of the 28 layers at 256K, every rectification row of
one 128K request and sampled rows of the others), the sweep's budgets at
64K, plus HIP-graph replay of the timed step against the oracle."""

import numpy as np
import pytest
import torch

import block_sparse_attention_resa_amd as resa
import oracle as O
from synth import WORKLOADS, make_append_rows, make_rectify_inputs, num_blocks, write_rows
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    C.require_gpu()


def layer_parity(case, check_dense=True, heads=None):
    """Descriptors, scores / selection and sparse + dense outputs of every
    request and (selected) KV head of one layer against the oracle."""
    C.run_descriptors(case)
    sel_idx, sel_cnt, scores = C.run_score_select(case)
    sp = C.run_sparse(case, sel_idx, sel_cnt)
    de = C.run_dense(case) if check_dense else None
    torch.cuda.synchronize()
    lists = C.sel_lists(sel_idx, sel_cnt)
    g = case.spec.group_size
    scale = C.sm_scale(case.cfg)
    swaps = 0
    heads = range(case.spec.num_kv_heads) if heads is None else heads
    for r in range(case.R):
        L = case.inp.seq_lens[r]
        for i in heads:
            K, V, q = C.keys_of(case, r, i), C.values_of(case, r, i), C.group_q(case, r, i)
            C.check_descriptors(case, r, i, K, L)
            lo, hi = O.descriptors(K, L)
            S = O.scores(q, lo, hi)
            swaps += C.check_selection(S, lists[r][i], case.cfg, tag=f"r{r} i{i}")
            C.check_out(sp[r, i * g:(i + 1) * g].cpu().numpy(), O.attend(q, K, V, L, lists[r][i], scale),
                        f"sparse r{r} i{i}")
            if check_dense:
                C.check_out(de[r, i * g:(i + 1) * g].cpu().numpy(), O.dense(q, K, V, L, scale), f"dense r{r} i{i}")
    return swaps


def test_qwen7b_ctx32k_b1():
    case = C.make_case(WORKLOADS["qwen7b_ctx32k_b1"], seed=101)
    swaps = layer_parity(case)
    print(f"near-tie swaps at the selection boundary: {swaps}")


@pytest.mark.timeout(600)
def test_qwen7b_ragged_b8():
    spec = WORKLOADS["qwen7b_ragged_b8"]
    case = C.make_case(spec, seed=102, permute=True)
    assert len(set(case.inp.seq_lens)) > 1
    swaps = layer_parity(case)
    print(f"seq_lens {case.inp.seq_lens}, near-tie swaps: {swaps}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layer", [0, 27])
def test_qwen7b_ctx256k_layer(layer):
    spec = WORKLOADS["qwen7b_ctx256k_l28"]
    case = C.make_case(spec, seed=2024, layer=layer)
    assert case.kv.max_blocks == 16384
    assert C.max_sel_for(case) == 1639
    swaps = layer_parity(case)
    print(f"layer {layer}: near-tie swaps {swaps}")


def step_against_oracle(case, sel_idx, sel_cnt, out, tag):
    """Selection and sparse outputs of one layer-step against the oracle."""
    lists = C.sel_lists(sel_idx, sel_cnt)
    g = case.spec.group_size
    scale = C.sm_scale(case.cfg)
    for r in range(case.R):
        L = case.inp.seq_lens[r]
        for i in range(case.spec.num_kv_heads):
            K, V, q = C.keys_of(case, r, i), C.values_of(case, r, i), C.group_q(case, r, i)
            lo, hi = O.descriptors(K, L)
            C.check_selection(O.scores(q, lo, hi), lists[r][i], case.cfg, tag=f"{tag} r{r} i{i}")
            C.check_out(out[r, i * g:(i + 1) * g].cpu().numpy(), O.attend(q, K, V, L, lists[r][i], scale),
                        f"{tag} r{r} i{i}")


def test_graph_replay_matches_eager():
    """The timed step (score/select with tail refresh + sparse decode over
    several layers) captured in a HIP graph: every replay, with eager work and
    synchronisations in between, reproduces the eager results bit for bit,
    and every replay's selections and outputs match the oracle."""
    graph_replay_case(WORKLOADS["qwen7b_ctx32k_b1"], seeds=(300, 301, 302), reps=4)


@pytest.mark.timeout(900)
def test_graph_replay_matches_eager_256k():
    """The benchmark's own configuration: two layers of the 256K workload
    (16384 blocks per head, the 1024-thread selection and 64 decode splits
    per head), the two calls captured in one HIP graph and replayed twice."""
    graph_replay_case(WORKLOADS["qwen7b_ctx256k_l28"], seeds=(2024, 2025), reps=2)


def graph_replay_case(spec, seeds, reps):
    cases = [C.make_case(spec, seed=sd) for sd in seeds]
    R, H, g, d = 1, spec.num_kv_heads, spec.group_size, spec.head_dim
    state = []
    for case in cases:
        C.run_descriptors(case)
        ms = C.max_sel_for(case)
        st = dict(case=case,
                  sel_idx=torch.full((R, H, ms), -5, dtype=torch.int32, device="cuda"),
                  sel_cnt=torch.zeros((R, H), dtype=torch.int32, device="cuda"),
                  out=torch.zeros((R, H * g, d), device="cuda"),
                  ws_s=resa.alloc_workspace(case.cfg, resa.OP_SCORE_SELECT, R, case.kv.max_blocks, ms),
                  ws_d=resa.alloc_workspace(case.cfg, resa.OP_SPARSE_DECODE, R, case.kv.max_blocks, ms))
        state.append(st)

    def step():
        for st in state:
            c = st["case"]
            resa.score_select(c.cfg, c.kv, c.inp.q, st["sel_idx"], st["sel_cnt"], st["ws_s"], refresh_tail=True)
            resa.sparse_decode(c.cfg, c.kv, c.inp.q, st["sel_idx"], st["sel_cnt"], st["out"], st["ws_d"])

    step()
    torch.cuda.synchronize()
    eager = [(st["sel_idx"].clone(), st["out"].clone()) for st in state]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(reps):
        for st in state:  # eager work between replays
            st["out"].fill_(float("nan"))
            st["sel_idx"].fill_(-9)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for st, (si, o) in zip(state, eager):
            assert torch.equal(st["sel_idx"], si), f"replay {rep}: selection differs"
            assert torch.equal(st["out"], o), f"replay {rep}: output differs"
            step_against_oracle(st["case"], st["sel_idx"], st["sel_cnt"], st["out"], f"replay {rep}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("budget", [(1, 50), (1, 20), (1, 5)])
def test_budget_sweep_64k(budget):
    """The budgets of the context x budget sweep besides 1/10, at 64K
    (4096 blocks per KV head; 82, 205 and 820 of them chosen): score/select +
    sparse decode and the step call, selections and outputs against the
    oracle, and the two paths against each other."""
    num, den = budget
    spec = WORKLOADS["qwen7b_ctx32k_b1"].with_(seq_lens=(65536,), budget_num=num, budget_den=den)
    case = C.make_case(spec, seed=640 + den)
    C.run_descriptors(case)
    sel_idx, sel_cnt, _ = C.run_score_select(case, with_scores=False)
    out = C.run_sparse(case, sel_idx, sel_cnt)
    torch.cuda.synchronize()
    assert int(sel_cnt[0, 0]) == O.selection_count(4096, num, den, spec.min_blocks, spec.local_blocks)
    step_against_oracle(case, sel_idx, sel_cnt, out, f"rho {num}/{den}")
    ms = C.max_sel_for(case)
    si2 = torch.full_like(sel_idx, -3)
    sc2 = torch.full_like(sel_cnt, -3)
    out2 = torch.full_like(out, float("nan"))
    ws = resa.alloc_workspace(case.cfg, resa.OP_SPARSE_STEP, case.R, case.kv.max_blocks, ms)
    resa.sparse_step(case.cfg, case.kv, case.inp.q, si2, sc2, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(si2, sel_idx) and torch.equal(sc2, sel_cnt)
    C.check_out(out2.cpu().numpy(), out.cpu().numpy().astype(np.float64), f"rho {num}/{den} step vs two calls")


@pytest.mark.timeout(900)
def test_qwen7b_ctx131k_b4_sparse_then_rectify():
    """64 sparse decode steps (each appends a token and refreshes the tail
    descriptor inside resa_score_select), then dense rectification of the
    last 64 positions, then one more sparse step on the rectified cache."""
    spec = WORKLOADS["qwen7b_ctx131k_b4_rectify"]
    steps, f = spec.sparse_steps, spec.rectify_chunk
    case = C.make_case(spec, seed=131, spare_blocks=5)
    R, H, g, d = spec.num_requests, spec.num_kv_heads, spec.group_size, spec.head_dim
    scale = C.sm_scale(case.cfg)
    C.run_descriptors(case)
    # logical caches the oracle follows (fp32 copies, grown as tokens are appended)
    K = [[C.keys_of(case, r, i).astype(np.float32) for i in range(H)] for r in range(R)]
    V = [[C.values_of(case, r, i).astype(np.float32) for i in range(H)] for r in range(R)]
    lens = list(case.inp.seq_lens)
    ms = C.max_sel_for(case)
    sel_idx = torch.empty((R, H, ms), dtype=torch.int32, device="cuda")
    sel_cnt = torch.empty((R, H), dtype=torch.int32, device="cuda")
    out = torch.empty((R, H * g, d), device="cuda")
    ws_s = resa.alloc_workspace(case.cfg, resa.OP_SCORE_SELECT, R, case.kv.max_blocks, ms)
    ws_d = resa.alloc_workspace(case.cfg, resa.OP_SPARSE_DECODE, R, case.kv.max_blocks, ms)

    def append(step_id):
        qn, kn, vn = make_append_rows(spec, 131, step_id, case.inp.outliers, device="cuda")
        for r in range(R):
            write_rows(case.paged, r, lens[r], kn[r], vn[r])
            for i in range(H):
                K[r][i] = np.concatenate([K[r][i], kn[r, i][None].float().cpu().numpy()])
                V[r][i] = np.concatenate([V[r][i], vn[r, i][None].float().cpu().numpy()])
            lens[r] += 1
        case.kv.seq_lens.copy_(torch.tensor(lens, dtype=torch.int32))
        return qn

    def sparse_step(qn, check):
        resa.score_select(case.cfg, case.kv, qn, sel_idx, sel_cnt, ws_s, refresh_tail=True)
        resa.sparse_decode(case.cfg, case.kv, qn, sel_idx, sel_cnt, out, ws_d)
        torch.cuda.synchronize()
        if not check:
            return
        lists = C.sel_lists(sel_idx, sel_cnt)
        for r in range(R):
            for i in range(H):
                q = C.np64(qn[r, i * g:(i + 1) * g])
                Kr, Vr = K[r][i].astype(np.float64), V[r][i].astype(np.float64)
                C.check_descriptors(case, r, i, Kr, lens[r])
                lo, hi = O.descriptors(Kr, lens[r])
                C.check_selection(O.scores(q, lo, hi), lists[r][i], case.cfg, tag=f"r{r} i{i}")
                C.check_out(out[r, i * g:(i + 1) * g].cpu().numpy(),
                            O.attend(q, Kr, Vr, lens[r], lists[r][i], scale), f"step r{r} i{i}")

    for st in range(steps):
        qn = append(st)
        sparse_step(qn, check=st in (0, steps - 1))
    assert lens == [131072 + steps] * R

    # rectification of the last f positions
    qc, kn, vn = make_rectify_inputs(spec, 131, f, device="cuda")
    rout = torch.full((R, f, H * g, d), float("nan"), device="cuda")
    ws_r = resa.alloc_workspace(case.cfg, resa.OP_DENSE_RECTIFY, R, case.kv.max_blocks, chunk=f)
    resa.dense_rectify(case.cfg, case.kv, qc, kn, vn, rout, ws_r)
    torch.cuda.synchronize()
    K1, V1 = C.logical_cache(case, lens)
    for r in range(R):
        L = lens[r]
        P = L - f
        for i in range(H):
            assert torch.equal(K1[r][i, P:L], kn[r, :, i]) and torch.equal(V1[r][i, P:L], vn[r, :, i])
            assert torch.equal(K1[r][i, :P].float().cpu(), torch.from_numpy(K[r][i][:P]))
            K[r][i][P:L] = kn[r, :, i].float().cpu().numpy()
            V[r][i][P:L] = vn[r, :, i].float().cpu().numpy()
            Kr, Vr = K[r][i].astype(np.float64), V[r][i].astype(np.float64)
            # descriptors: every block equals a rebuild of the rectified cache
            C.check_descriptors(case, r, i, Kr, L)
            if r == 0:
                # request 0: every chunk row (all 448 query rows of the KV
                # head) against the oracle's rectification, which writes the
                # chunk's rows and attends causally for each of them
                ref, _, _, _, _, _ = O.rectify(C.np64(qc[r, :, i * g:(i + 1) * g]), C.np64(kn[r, :, i]),
                                               C.np64(vn[r, :, i]), Kr, Vr, L, scale)
                for t in range(f):
                    C.check_out(rout[r, t, i * g:(i + 1) * g].cpu().numpy(), ref[t], f"rectify r{r} i{i} t{t}")
                continue
            for t in (0, f // 2 - 1, f - 1):  # sampled chunk rows, all heads of the group
                ref = O.dense(C.np64(qc[r, t, i * g:(i + 1) * g]), Kr, Vr, P + t + 1, scale)
                C.check_out(rout[r, t, i * g:(i + 1) * g].cpu().numpy(), ref, f"rectify r{r} i{i} t{t}")

    # one more sparse step on the rectified cache: the new token opens a 1-row tail block
    qn = append(steps)
    assert all(L % 16 == 1 for L in lens)
    sparse_step(qn, check=True)
