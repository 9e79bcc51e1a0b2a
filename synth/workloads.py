"""Seeded synthetic workloads shaped like Qwen2.5-7B decode attention.

Head layout and context lengths follow the efficiency setup described on the
Rectified Sparse Attention analysis page (paper-graph-ui), §3.4.5 and §5:
28 query heads over 4 KV heads (group 7), head dimension 128, block size 16,
contexts from 32K to 256K.  The value distributions follow the recipes of the
five workloads this library is measured on:

* keys and values are i.i.d. N(0, 1) draws in fp32, rounded once to the
  storage dtype (bf16 uses round-to-nearest-even, torch's own conversion);
* ``outlier_channels`` distinct channels per (layer, KV head) have their key
  draws scaled by ``outlier_scale`` (8 in the bf16 workloads);
* ``plant_count`` (or ``ceil(plant_frac * M)``) distinct non-tail blocks per
  (request, KV head) get ``plant_alpha * qbar`` added to their keys, where
  ``qbar`` is the mean of the group's (already rounded) query heads;
* queries are N(0, 1).

Nothing here computes descriptors, scores, selections or attention.

Memory layout produced for the library (the C header documents it too):

* ``k_pool``  ``[P][H_kv][16][d]``  token-major rows of one 16-token block;
* ``v_pool``  ``[P][H_kv][d][16]``  channel-major within the block;
* ``desc_pool`` ``[P][H_kv][2][d]`` (row 0 = min, row 1 = max), left empty;
* ``block_table`` ``[R][max_blocks]`` int32 physical block ids, ``-1`` unused;
* ``seq_lens`` ``[R]`` int32.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import torch

BLOCK = 16


def num_blocks(seq_len: int, block: int = BLOCK) -> int:
    """Number of ``block``-token blocks covering ``seq_len`` tokens."""
    return (int(seq_len) + block - 1) // block


def round_bf16(x: torch.Tensor) -> torch.Tensor:
    """fp32 -> bf16 (round to nearest even) -> fp32."""
    return x.to(torch.bfloat16).to(torch.float32)


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    dtype: str  # "bf16" or "f32"
    num_requests: int
    num_kv_heads: int
    group_size: int
    head_dim: int
    seq_lens: Optional[Tuple[int, ...]] = None  # fixed per-request lengths
    ctx_range: Optional[Tuple[int, int]] = None  # else uniform integers in [lo, hi]
    layers: int = 1
    outlier_channels: int = 0
    outlier_scale: float = 8.0
    plant_count: Optional[int] = None
    plant_frac: Optional[float] = None
    plant_alpha: float = 0.5
    budget_num: int = 1
    budget_den: int = 10
    min_blocks: int = 16
    local_blocks: int = 1
    rectify_chunk: int = 0
    sparse_steps: int = 0
    description: str = ""

    @property
    def num_q_heads(self) -> int:
        return self.num_kv_heads * self.group_size

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)

    def draw_seq_lens(self, seed: int) -> List[int]:
        if self.seq_lens is not None:
            assert len(self.seq_lens) == self.num_requests
            return [int(x) for x in self.seq_lens]
        lo, hi = self.ctx_range
        g = torch.Generator().manual_seed(_mix(seed, 0x5E9))
        return [int(x) for x in torch.randint(lo, hi + 1, (self.num_requests,), generator=g)]


WORKLOADS = {
    # Tiny single decode step in fp32, small enough for brute force.
    "tiny_f32_ctx2k": WorkloadSpec(
        name="tiny_f32_ctx2k", dtype="f32", num_requests=1, num_kv_heads=1, group_size=2,
        head_dim=64, seq_lens=(2048,), plant_count=4,
        description="1 request, 1 KV head, group 2, d=64, ctx 2048, fp32, 4 planted blocks"),
    # One Qwen2.5-7B-shaped layer at 32K, batch 1.
    "qwen7b_ctx32k_b1": WorkloadSpec(
        name="qwen7b_ctx32k_b1", dtype="bf16", num_requests=1, num_kv_heads=4, group_size=7,
        head_dim=128, seq_lens=(32768,), outlier_channels=8, plant_frac=0.05,
        description="28 q heads / 4 KV heads, d=128, ctx 32768, bf16, 10% budget"),
    # Ragged batch of 8 requests, contexts uniform in [32K, 64K].
    "qwen7b_ragged_b8": WorkloadSpec(
        name="qwen7b_ragged_b8", dtype="bf16", num_requests=8, num_kv_heads=4, group_size=7,
        head_dim=128, ctx_range=(32768, 65536), outlier_channels=8, plant_frac=0.05,
        description="8 requests, ctx ~ U[32768, 65536], 28/4 heads, d=128, bf16"),
    # 256K context, 28 independent layers (the headline workload).
    "qwen7b_ctx256k_l28": WorkloadSpec(
        name="qwen7b_ctx256k_l28", dtype="bf16", num_requests=1, num_kv_heads=4, group_size=7,
        head_dim=128, seq_lens=(262144,), layers=28, outlier_channels=8, plant_frac=0.05,
        description="1 request, ctx 262144, 28 independent layers, 28/4 heads, d=128, bf16"),
    # 4 requests at 128K: 64 sparse steps, then rectify the last 64 tokens.
    "qwen7b_ctx131k_b4_rectify": WorkloadSpec(
        name="qwen7b_ctx131k_b4_rectify", dtype="bf16", num_requests=4, num_kv_heads=4,
        group_size=7, head_dim=128, seq_lens=(131072,) * 4, outlier_channels=8,
        plant_frac=0.05, rectify_chunk=64, sparse_steps=64,
        description="4 requests at 131072, 64 sparse steps then rectify f=64"),
}


def _mix(*parts: int) -> int:
    """Deterministic 63-bit seed derivation (splitmix64 finaliser)."""
    x = 0x9E3779B97F4A7C15
    for p in parts:
        x = (x ^ (int(p) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        x = (x + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        x = z ^ (z >> 31)
    return x & 0x7FFFFFFFFFFFFFFF


@dataclass
class LayerInputs:
    """Logical (un-paged) inputs of one layer.  All tensors hold values already
    rounded to the storage dtype and are stored in that dtype."""

    spec: WorkloadSpec
    seq_lens: List[int]
    q: torch.Tensor  # [R, H_q, d]
    keys: List[torch.Tensor]  # per request [H_kv, L_r, d]
    values: List[torch.Tensor]  # per request [H_kv, L_r, d]
    outliers: List[List[int]]  # per KV head
    planted: List[List[List[int]]]  # [r][i] -> planted block ids
    seed: int = 0
    layer: int = 0
    extra: dict = field(default_factory=dict)


def _draw_normal(gen: torch.Generator, shape, device) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)


def make_layer(spec: WorkloadSpec, seed: int, layer: int = 0, device="cpu",
               seq_lens: Optional[Sequence[int]] = None) -> LayerInputs:
    """Draw one layer of the workload.  Deterministic in (spec, seed, layer, device)."""
    device = torch.device(device)
    lens = list(seq_lens) if seq_lens is not None else spec.draw_seq_lens(seed)
    R, Hkv, g, d = spec.num_requests, spec.num_kv_heads, spec.group_size, spec.head_dim
    dt = spec.torch_dtype
    small = torch.Generator().manual_seed(_mix(seed, layer, 1))
    big = torch.Generator(device=device).manual_seed(_mix(seed, layer, 2))

    q32 = _draw_normal(big, (R, Hkv * g, d), device)
    q = q32.to(dt)
    qf = q.to(torch.float32)

    outliers = []
    for _ in range(Hkv):
        if spec.outlier_channels:
            outliers.append(sorted(torch.randperm(d, generator=small)[: spec.outlier_channels].tolist()))
        else:
            outliers.append([])

    keys, values, planted = [], [], []
    for r in range(R):
        L = lens[r]
        M = num_blocks(L)
        z = _draw_normal(big, (Hkv, L, d), device)
        for i in range(Hkv):
            if outliers[i]:
                ch = torch.tensor(outliers[i], device=device)
                z[i][:, ch] *= spec.outlier_scale
        plant_r = []
        for i in range(Hkv):
            if spec.plant_count is not None:
                cnt = spec.plant_count
            elif spec.plant_frac is not None:
                cnt = math.ceil(spec.plant_frac * M)
            else:
                cnt = 0
            cnt = max(0, min(cnt, M - 1))
            blocks = sorted(torch.randperm(max(M - 1, 1), generator=small)[:cnt].tolist()) if cnt else []
            if blocks:
                qbar = qf[r, i * g:(i + 1) * g].mean(dim=0)
                bt = torch.tensor(blocks, device=device, dtype=torch.int64)
                rows = (bt[:, None] * BLOCK + torch.arange(BLOCK, device=device)[None, :]).flatten()
                rows = rows[rows < L]
                z[i][rows] += spec.plant_alpha * qbar
            plant_r.append(blocks)
        planted.append(plant_r)
        keys.append(z.to(dt))
        del z
        values.append(_draw_normal(big, (Hkv, L, d), device).to(dt))
    return LayerInputs(spec=spec, seq_lens=lens, q=q, keys=keys, values=values,
                       outliers=outliers, planted=planted, seed=seed, layer=layer)


def make_append_rows(spec: WorkloadSpec, seed: int, step: int, outliers: List[List[int]],
                     device="cpu") -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """One decode step's new (q, k, v) rows: q [R, H_q, d], k/v [R, H_kv, d].
    Keys use the layer's outlier channels; nothing is planted."""
    device = torch.device(device)
    R, Hkv, g, d = spec.num_requests, spec.num_kv_heads, spec.group_size, spec.head_dim
    gen = torch.Generator(device=device).manual_seed(_mix(seed, 77, step))
    q = _draw_normal(gen, (R, Hkv * g, d), device)
    k = _draw_normal(gen, (R, Hkv, d), device)
    for i in range(Hkv):
        if outliers[i]:
            k[:, i, torch.tensor(outliers[i], device=device)] *= spec.outlier_scale
    v = _draw_normal(gen, (R, Hkv, d), device)
    dt = spec.torch_dtype
    return q.to(dt), k.to(dt), v.to(dt)


def make_rectify_inputs(spec: WorkloadSpec, seed: int, chunk: int, device="cpu"):
    """Fresh N(0,1) q_chunk [R, f, H_q, d], k_new / v_new [R, f, H_kv, d]."""
    device = torch.device(device)
    R, Hkv, g, d = spec.num_requests, spec.num_kv_heads, spec.group_size, spec.head_dim
    gen = torch.Generator(device=device).manual_seed(_mix(seed, 99, chunk))
    dt = spec.torch_dtype
    q = _draw_normal(gen, (R, chunk, Hkv * g, d), device).to(dt)
    k = _draw_normal(gen, (R, chunk, Hkv, d), device).to(dt)
    v = _draw_normal(gen, (R, chunk, Hkv, d), device).to(dt)
    return q, k, v


@dataclass
class Paged:
    k_pool: torch.Tensor  # [P, H_kv, 16, d]
    v_pool: torch.Tensor  # [P, H_kv, d, 16]
    desc_pool: torch.Tensor  # [P, H_kv, 2, d]
    block_table: torch.Tensor  # [R, max_blocks] int32
    seq_lens: torch.Tensor  # [R] int32
    max_blocks: int
    num_pool_blocks: int


def make_paged(inp: LayerInputs, max_blocks: Optional[int] = None, device=None,
               permute_seed: Optional[int] = None, pad_fill: float = 0.0,
               spare_blocks: int = 0) -> Paged:
    """Lay the logical caches of ``inp`` out as a paged pool.

    Blocks of one request are contiguous in the pool and requests follow each
    other, unless ``permute_seed`` is given, in which case the physical block
    ids are a seeded random permutation (exercising the indirection).  Rows of
    the tail block beyond the sequence length are filled with ``pad_fill``
    (NaN is allowed: the library must never read them into a result).
    ``spare_blocks`` extra physical blocks per request are reserved after each
    request's blocks (room for appended tokens) and listed in the table.
    """
    spec = inp.spec
    device = torch.device(device) if device is not None else inp.q.device
    R, Hkv, d = spec.num_requests, spec.num_kv_heads, spec.head_dim
    Ms = [num_blocks(L) for L in inp.seq_lens]
    Ms_alloc = [m + spare_blocks for m in Ms]
    mb = max(Ms_alloc) if max_blocks is None else int(max_blocks)
    assert mb >= max(Ms_alloc)
    P = sum(Ms_alloc)
    phys = torch.arange(P, dtype=torch.int64)
    if permute_seed is not None:
        phys = torch.randperm(P, generator=torch.Generator().manual_seed(_mix(permute_seed, 5)))
    table = torch.full((R, mb), -1, dtype=torch.int32)
    dt = spec.torch_dtype
    k_pool = torch.zeros((P, Hkv, BLOCK, d), dtype=dt, device=device)
    v_pool = torch.zeros((P, Hkv, d, BLOCK), dtype=dt, device=device)
    desc = torch.zeros((P, Hkv, 2, d), dtype=dt, device=device)
    base = 0
    for r in range(R):
        L, M = inp.seq_lens[r], Ms[r]
        ids = phys[base: base + Ms_alloc[r]]
        table[r, : Ms_alloc[r]] = ids.to(torch.int32)
        base += Ms_alloc[r]
        kr = inp.keys[r].to(device)
        vr = inp.values[r].to(device)
        pad = M * BLOCK - L
        if pad:
            fill = torch.full((Hkv, pad, d), pad_fill, dtype=dt, device=device)
            kr = torch.cat([kr, fill], dim=1)
            vr = torch.cat([vr, fill], dim=1)
        # [H, M*16, d] -> [M, H, 16, d]
        kb = kr.reshape(Hkv, M, BLOCK, d).permute(1, 0, 2, 3)
        vb = vr.reshape(Hkv, M, BLOCK, d).permute(1, 0, 3, 2)
        idx = ids[:M].to(device)
        k_pool[idx] = kb
        v_pool[idx] = vb
        del kr, vr, kb, vb
    return Paged(k_pool=k_pool, v_pool=v_pool, desc_pool=desc,
                 block_table=table.to(device), seq_lens=torch.tensor(inp.seq_lens, dtype=torch.int32,
                                                                      device=device),
                 max_blocks=mb, num_pool_blocks=P)


def paged_to_logical(k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
                     seq_lens: Sequence[int]):
    """Inverse of :func:`make_paged` for reading caches back: returns per request
    ``K [H_kv, L, d]`` and ``V [H_kv, L, d]`` (same dtype, on the pools' device)."""
    out_k, out_v = [], []
    table = block_table.to(k_pool.device).long()
    for r, L in enumerate(seq_lens):
        M = num_blocks(L)
        ids = table[r, :M]
        kb = k_pool[ids]  # [M, H, 16, d]
        vb = v_pool[ids]  # [M, H, d, 16]
        H, d = kb.shape[1], kb.shape[3]
        K = kb.permute(1, 0, 2, 3).reshape(H, M * BLOCK, d)[:, :L]
        V = vb.permute(1, 0, 3, 2).reshape(H, M * BLOCK, d)[:, :L]
        out_k.append(K)
        out_v.append(V)
    return out_k, out_v


def write_rows(paged: Paged, r: int, pos: int, k_rows: torch.Tensor, v_rows: torch.Tensor) -> None:
    """Store one token's K/V rows ``[H_kv, d]`` of request ``r`` at position ``pos``
    into the paged pools (the cache append a model's attention layer performs)."""
    blk = int(paged.block_table[r, pos // BLOCK].item())
    t = pos % BLOCK
    paged.k_pool[blk, :, t, :] = k_rows.to(paged.k_pool.dtype)
    paged.v_pool[blk, :, :, t] = v_rows.to(paged.v_pool.dtype)
