"""resa_sparse_decode_noalloc (the entry point for callers that cannot
allocate) against resa_sparse_decode on the same inputs, through the C ABI:
two calls in a row, the second with a smaller input, each equal to the
workspace call bit for bit and to the oracle within the output tolerance;
and a call needing more than the static scratch is refused."""

import numpy as np
import pytest
import torch

import block_sparse_attention_resa_amd as resa
import oracle as O
from synth import WORKLOADS
from tests import gpu_common as C

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    C.require_gpu()


def run_pair(case):
    C.run_descriptors(case)
    sel_idx, sel_cnt, _ = C.run_score_select(case, with_scores=False)
    ref = C.run_sparse(case, sel_idx, sel_cnt)
    R, HG, d = case.R, case.spec.num_q_heads, case.spec.head_dim
    out = torch.full((R, HG, d), float("nan"), device="cuda")
    resa.sparse_decode_noalloc(case.cfg, case.kv, case.inp.q, sel_idx, sel_cnt, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "no-alloc output differs from the workspace call"
    lists = C.sel_lists(sel_idx, sel_cnt)
    g = case.spec.group_size
    scale = C.sm_scale(case.cfg)
    for r in range(R):
        L = case.inp.seq_lens[r]
        for i in range(case.spec.num_kv_heads):
            K, V, q = C.keys_of(case, r, i), C.values_of(case, r, i), C.group_q(case, r, i)
            C.check_out(out[r, i * g:(i + 1) * g].cpu().numpy(), O.attend(q, K, V, L, lists[r][i], scale),
                        f"noalloc r{r} i{i}")


def test_noalloc_matches_workspace_call_twice_second_smaller():
    big = WORKLOADS["qwen7b_ctx32k_b1"].with_(num_requests=3, seq_lens=(20000, 33000, 9001))
    small = WORKLOADS["qwen7b_ctx32k_b1"].with_(num_requests=1, seq_lens=(3003,))
    run_pair(C.make_case(big, seed=71, permute=True))
    run_pair(C.make_case(small, seed=72))


def test_noalloc_refuses_more_than_its_scratch():
    spec = WORKLOADS["qwen7b_ctx32k_b1"].with_(seq_lens=(640,))
    case = C.make_case(spec, seed=73)
    cfg = resa.Config(num_kv_heads=4, group_size=7, head_dim=128, num_splits=1024)
    need = resa.workspace_bytes(cfg, resa.OP_SPARSE_DECODE, 1, case.kv.max_blocks, 2048)
    assert need > resa.NOALLOC_SCRATCH_BYTES
    sel_idx = torch.zeros((1, 4, 2048), dtype=torch.int32, device="cuda")
    sel_cnt = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    out = torch.zeros((1, 28, 128), device="cuda")
    with pytest.raises(resa.ResaError) as e:
        resa.sparse_decode_noalloc(cfg, case.kv, case.inp.q, sel_idx, sel_cnt, out)
    assert e.value.status == 3
