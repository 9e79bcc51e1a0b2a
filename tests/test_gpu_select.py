"""Top-n selection on crafted score distributions.

With fp32 descriptors and a query that is 1 on channel 0 and 0 elsewhere
(group size 1), Eq 4's group score of block b is exactly hi_0(b): every other
term is an exact zero.  That lets these tests hand the selection any score
distribution — ties, few distinct levels, mixed signs over sixty decades, a
single huge outlier, values near the float range limit — and demand the
oracle's selection (ties to the lower block id) exactly, id for id."""

import numpy as np
import pytest
import torch

import block_sparse_attention_resa_amd as resa
import oracle as O
from tests import gpu_common as C

pytestmark = pytest.mark.gpu

D = 64


@pytest.fixture(autouse=True)
def _gpu():
    C.require_gpu()


def distribution(name: str, rng: np.random.Generator, M: int) -> np.ndarray:
    """Non-zero fp32 scores of one (request, head)."""
    if name == "normal":  # the shape real group scores take (mean ~1900, sd ~65)
        s = rng.normal(1900.0, 65.0, M)
    elif name == "equal":
        s = np.full(M, 3.0)
    elif name == "two_levels":
        s = np.where(rng.random(M) < 0.3, 2.0, 1.0)
    elif name == "few_levels":
        s = np.round(rng.normal(0.0, 1.0, M) * 4.0) / 4.0 + 0.125
    elif name == "mixed_sign_wide":
        s = rng.choice([-1.0, 1.0], M) * 10.0 ** rng.uniform(-30, 30, M)
    elif name == "huge_outlier":
        s = rng.normal(10.0, 1.0, M)
        s[rng.integers(0, M, 2)] = [1e38, -1e38]
    elif name == "near_float_max":
        s = rng.normal(0.0, 1.0, M) + 0.5
        s[rng.integers(0, M, 4)] = [3.3e38, -3.3e38, 3.0e38, -2.9e38]
    elif name == "tiny":
        s = rng.normal(1.0, 0.1, M) * 1e-30
    elif name == "clustered_top":  # many near-equal scores right at the boundary
        s = rng.normal(0.0, 1.0, M)
        hot = rng.random(M) < 0.2  # three adjacent floats 1.5, 1.5 + ulp, 1.5 + 2 ulp
        s[hot] = 1.5 + rng.integers(0, 3, int(hot.sum())) * 2.0 ** -23
    else:
        raise KeyError(name)
    s = s.astype(np.float32)
    s[s == 0] = np.float32(1e-3)
    return s


def run_case(dist: str, M: int, seed: int):
    rng = np.random.default_rng(seed)
    R, H = 2, 2
    Ms = [M, max(1, M - 7)]
    mb = M
    P = R * mb
    cfg = resa.Config(num_kv_heads=H, group_size=1, head_dim=D, dtype=resa.RESA_F32)
    desc = torch.zeros((P, H, 2, D), dtype=torch.float32)
    S = {}
    for r in range(R):
        for i in range(H):
            s = distribution(dist, rng, Ms[r])
            S[r, i] = s
            rows = torch.arange(Ms[r]) + r * mb
            desc[rows, i, 0, 0] = torch.from_numpy(s)  # lo = hi: any finite value works
            desc[rows, i, 1, 0] = torch.from_numpy(s)
            desc[rows, i, :, 1:] = torch.from_numpy(rng.normal(0, 1, (Ms[r], 2, D - 1)).astype(np.float32))
    table = (torch.arange(mb, dtype=torch.int32)[None, :] + torch.arange(R, dtype=torch.int32)[:, None] * mb)
    seq = torch.tensor([m * 16 - 3 for m in Ms], dtype=torch.int32)
    kv = resa.PagedKV(torch.empty((P, H, 16, D), device="cuda"), torch.empty((P, H, D, 16), device="cuda"),
                      desc.cuda(), table.cuda(), seq.cuda())
    q = torch.zeros((R, H, D), dtype=torch.float32)
    q[:, :, 0] = 1.0
    q = q.cuda()
    ms = resa.selection_count(cfg, M)
    sel_idx = torch.full((R, H, ms), -7, dtype=torch.int32, device="cuda")
    sel_cnt = torch.zeros((R, H), dtype=torch.int32, device="cuda")
    scores = torch.zeros((R, H, mb), dtype=torch.float32, device="cuda")
    ws = resa.alloc_workspace(cfg, resa.OP_SCORE_SELECT, R, mb, ms)
    resa.score_select(cfg, kv, q, sel_idx, sel_cnt, ws, scores=scores)
    torch.cuda.synchronize()
    sel_idx, sel_cnt, scores = sel_idx.cpu(), sel_cnt.cpu(), scores.cpu()
    for r in range(R):
        for i in range(H):
            s = S[r, i]
            got_s = scores[r, i, : Ms[r] - 1].numpy()
            assert np.array_equal(got_s, s[:-1]), f"{dist} r{r} i{i}: scores are not hi_0 exactly"
            ref = O.select(s.astype(np.float64), cfg.budget_num, cfg.budget_den, cfg.min_blocks, cfg.local_blocks)
            n = int(sel_cnt[r, i])
            got = sel_idx[r, i, :n].numpy()
            assert n == len(ref), f"{dist} r{r} i{i}: count {n} != {len(ref)}"
            assert np.array_equal(got, ref), \
                f"{dist} M={Ms[r]} r{r} i{i}: first difference at {np.nonzero(got != ref)[0][:3]}"
            assert torch.all(sel_idx[r, i, n:] == -1)


DISTS = ["normal", "equal", "two_levels", "few_levels", "mixed_sign_wide", "huge_outlier", "near_float_max",
         "tiny", "clustered_top"]


@pytest.mark.parametrize("dist", DISTS)
def test_select_distributions_16k(dist):
    run_case(dist, 16384, seed=11)


# sizes on both sides of every change of the selection's thread count and
# keys per thread (rows of up to 2048, 4096, 8192, 16384 and 32768 keys)
@pytest.mark.parametrize("M", [20, 200, 300, 2048, 2052, 4096, 4100, 5000, 8192, 8196, 30000, 40000])
@pytest.mark.parametrize("dist", ["normal", "few_levels", "huge_outlier"])
def test_select_sizes(dist, M):
    run_case(dist, M, seed=M)


# short rows, every distribution: fewer candidates than one histogram pass
# needs, and rows of 1024 to 2048 keys (the 512-thread selection)
@pytest.mark.parametrize("M", [60, 66, 1024, 1025, 2048])
@pytest.mark.parametrize("dist", DISTS)
def test_select_short_rows(dist, M):
    run_case(dist, M, seed=7 * M + 1)
