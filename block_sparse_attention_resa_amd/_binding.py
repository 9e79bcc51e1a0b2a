"""ctypes binding of libresa (include/resa.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks their
dtype / shape / contiguity against the configuration, and passes raw device
pointers plus torch's current HIP stream to the library.  All arithmetic runs
in the library's HIP kernels; if libresa.so is missing or fails to load, every
call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libresa.so")

RESA_OK = 0
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration", 3: "workspace", 4: "launch failed"}

RESA_BF16 = 0
RESA_F32 = 1
RESA_SCORE_SUM_HEADS = 0
RESA_SCORE_MEAN_POOL = 1
OP_SCORE_SELECT = 1
OP_SPARSE_DECODE = 2
OP_DENSE_DECODE = 3
OP_DENSE_RECTIFY = 4
OP_SPARSE_STEP = 5

EXPORTED = (
    "resa_abi_version", "resa_status_string", "resa_config_init", "resa_selection_count",
    "resa_workspace_bytes", "resa_num_splits", "resa_build_descriptors", "resa_score_select",
    "resa_sparse_decode", "resa_dense_decode", "resa_dense_rectify", "resa_sparse_decode_noalloc",
    "resa_sparse_step",
)

NOALLOC_SCRATCH_BYTES = 8 << 20  # RESA_NOALLOC_SCRATCH_BYTES


class ResaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({STATUS.get(status, '?')})")
        self.status = status


class CConfig(ctypes.Structure):
    _fields_ = [
        ("num_kv_heads", ctypes.c_int32), ("group_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32), ("dtype", ctypes.c_int32), ("budget_num", ctypes.c_int32),
        ("budget_den", ctypes.c_int32), ("min_blocks", ctypes.c_int32), ("local_blocks", ctypes.c_int32),
        ("score_mode", ctypes.c_int32), ("sm_scale", ctypes.c_float), ("num_splits", ctypes.c_int32),
    ]


class CPagedKV(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p), ("desc_pool", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("num_pool_blocks", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libresa.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libresa.so not found at {path}; build it with "
                           "`python -m block_sparse_attention_resa_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp, kvp = ctypes.POINTER(CConfig), ctypes.POINTER(CPagedKV)
    sig = {
        "resa_abi_version": (i32, []),
        "resa_status_string": (ctypes.c_char_p, [i32]),
        "resa_config_init": (i32, [cfgp, i32, i32, i32, i32]),
        "resa_selection_count": (i32, [cfgp, i32]),
        "resa_workspace_bytes": (sz, [cfgp, i32, i32, i32, i32, i32]),
        "resa_num_splits": (i32, [cfgp, i32, i32, i32, i32, i32]),
        "resa_build_descriptors": (i32, [cfgp, kvp, i32, vp, i32, vp]),
        "resa_score_select": (i32, [cfgp, kvp, i32, vp, i32, vp, vp, i32, vp, vp, sz, vp]),
        "resa_sparse_decode": (i32, [cfgp, kvp, i32, vp, vp, vp, i32, vp, vp, sz, vp]),
        "resa_sparse_decode_noalloc": (i32, [cfgp, kvp, i32, vp, vp, vp, i32, vp, vp]),
        "resa_sparse_step": (i32, [cfgp, kvp, i32, vp, i32, vp, vp, i32, vp, vp, sz, vp]),
        "resa_dense_decode": (i32, [cfgp, kvp, i32, vp, vp, vp, sz, vp]),
        "resa_dense_rectify": (i32, [cfgp, kvp, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


@dataclass
class Config:
    """Mirror of resa_config.  Defaults follow §3.4.5 of the analysis page."""

    num_kv_heads: int
    group_size: int
    head_dim: int
    dtype: int = RESA_BF16
    block_size: int = 16
    budget_num: int = 1
    budget_den: int = 10
    min_blocks: int = 16
    local_blocks: int = 1
    score_mode: int = RESA_SCORE_SUM_HEADS
    sm_scale: Optional[float] = None
    num_splits: int = 0

    def c(self) -> CConfig:
        scale = self.sm_scale if self.sm_scale is not None else 1.0 / math.sqrt(self.head_dim)
        return CConfig(self.num_kv_heads, self.group_size, self.head_dim, self.block_size, self.dtype,
                       self.budget_num, self.budget_den, self.min_blocks, self.local_blocks,
                       self.score_mode, float(scale), self.num_splits)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == RESA_BF16 else torch.float32


@dataclass
class PagedKV:
    """Device tensors of a paged cache, laid out as include/resa.h states."""

    k_pool: torch.Tensor  # [P, H, 16, d]
    v_pool: torch.Tensor  # [P, H, d, 16]
    desc_pool: torch.Tensor  # [P, H, 2, d]
    block_table: torch.Tensor  # [R, max_blocks] int32
    seq_lens: torch.Tensor  # [R] int32

    def c(self) -> CPagedKV:
        return CPagedKV(self.k_pool.data_ptr(), self.v_pool.data_ptr(), self.desc_pool.data_ptr(),
                        self.block_table.data_ptr(), self.seq_lens.data_ptr(),
                        int(self.k_pool.shape[0]), int(self.block_table.shape[1]))

    @property
    def num_requests(self) -> int:
        return int(self.block_table.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


def _stream_ptr() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_cache(cfg: Config, kv: PagedKV):
    dt = cfg.torch_dtype
    P = kv.k_pool.shape[0]
    H, d = cfg.num_kv_heads, cfg.head_dim
    _need(kv.k_pool, "k_pool", dt, (P, H, 16, d))
    _need(kv.v_pool, "v_pool", dt, (P, H, d, 16))
    _need(kv.desc_pool, "desc_pool", dt, (P, H, 2, d))
    _need(kv.block_table, "block_table", torch.int32)
    _need(kv.seq_lens, "seq_lens", torch.int32, (kv.block_table.shape[0],))


def _call(name: str, *args):
    st = getattr(load_library(), name)(*args)
    if st != RESA_OK:
        raise ResaError(name, st)


def abi_version() -> int:
    return load_library().resa_abi_version()


def selection_count(cfg: Config, num_blocks: int) -> int:
    c = cfg.c()
    return load_library().resa_selection_count(ctypes.byref(c), int(num_blocks))


def workspace_bytes(cfg: Config, op: int, num_requests: int, max_blocks: int, max_sel: int = 0,
                    chunk: int = 0) -> int:
    c = cfg.c()
    return int(load_library().resa_workspace_bytes(ctypes.byref(c), op, num_requests, max_blocks, max_sel,
                                                   chunk))


def num_splits(cfg: Config, op: int, num_requests: int, max_blocks: int, max_sel: int = 0,
               chunk: int = 0) -> int:
    c = cfg.c()
    return int(load_library().resa_num_splits(ctypes.byref(c), op, num_requests, max_blocks, max_sel, chunk))


def alloc_workspace(cfg: Config, op: int, num_requests: int, max_blocks: int, max_sel: int = 0,
                    chunk: int = 0, device="cuda") -> torch.Tensor:
    n = workspace_bytes(cfg, op, num_requests, max_blocks, max_sel, chunk)
    if n == 0:
        raise ValueError("invalid workspace request")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def build_descriptors(cfg: Config, kv: PagedKV, first_block: Optional[torch.Tensor] = None,
                      num_blocks: int = 0) -> None:
    _check_cache(cfg, kv)
    if first_block is not None:
        _need(first_block, "first_block", torch.int32, (kv.num_requests,))
    c, k = cfg.c(), kv.c()
    _call("resa_build_descriptors", ctypes.byref(c), ctypes.byref(k), kv.num_requests, _ptr(first_block),
          int(num_blocks), _stream_ptr())


def score_select(cfg: Config, kv: PagedKV, q: torch.Tensor, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                 workspace: torch.Tensor, scores: Optional[torch.Tensor] = None,
                 refresh_tail: bool = False) -> None:
    _check_cache(cfg, kv)
    R, H, G, d = kv.num_requests, cfg.num_kv_heads, cfg.group_size, cfg.head_dim
    _need(q, "q", cfg.torch_dtype, (R, H * G, d))
    _need(sel_idx, "sel_idx", torch.int32)
    if sel_idx.dim() != 3 or tuple(sel_idx.shape[:2]) != (R, H):
        raise ValueError("sel_idx must be [R, H, max_sel]")
    _need(sel_cnt, "sel_cnt", torch.int32, (R, H))
    _need(workspace, "workspace", torch.uint8)
    if scores is not None:
        _need(scores, "scores", torch.float32, (R, H, kv.max_blocks))
    c, k = cfg.c(), kv.c()
    _call("resa_score_select", ctypes.byref(c), ctypes.byref(k), R, q.data_ptr(), int(bool(refresh_tail)),
          sel_idx.data_ptr(),
          sel_cnt.data_ptr(), int(sel_idx.shape[2]), _ptr(scores), workspace.data_ptr(), workspace.numel(),
          _stream_ptr())


def sparse_decode(cfg: Config, kv: PagedKV, q: torch.Tensor, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                  out: torch.Tensor, workspace: torch.Tensor) -> None:
    _check_cache(cfg, kv)
    R, H, G, d = kv.num_requests, cfg.num_kv_heads, cfg.group_size, cfg.head_dim
    _need(q, "q", cfg.torch_dtype, (R, H * G, d))
    _need(sel_idx, "sel_idx", torch.int32)
    if sel_idx.dim() != 3 or tuple(sel_idx.shape[:2]) != (R, H):
        raise ValueError("sel_idx must be [R, H, max_sel]")
    _need(sel_cnt, "sel_cnt", torch.int32, (R, H))
    _need(out, "out", torch.float32, (R, H * G, d))
    _need(workspace, "workspace", torch.uint8)
    c, k = cfg.c(), kv.c()
    _call("resa_sparse_decode", ctypes.byref(c), ctypes.byref(k), R, q.data_ptr(), sel_idx.data_ptr(),
          sel_cnt.data_ptr(), int(sel_idx.shape[2]), out.data_ptr(), workspace.data_ptr(), workspace.numel(),
          _stream_ptr())


def sparse_step(cfg: Config, kv: PagedKV, q: torch.Tensor, sel_idx: torch.Tensor, sel_cnt: torch.Tensor,
                out: torch.Tensor, workspace: torch.Tensor, refresh_tail: bool = False) -> None:
    """resa_score_select + resa_sparse_decode in one launch fewer (workspace of OP_SPARSE_STEP)."""
    _check_cache(cfg, kv)
    R, H, G, d = kv.num_requests, cfg.num_kv_heads, cfg.group_size, cfg.head_dim
    _need(q, "q", cfg.torch_dtype, (R, H * G, d))
    _need(sel_idx, "sel_idx", torch.int32)
    if sel_idx.dim() != 3 or tuple(sel_idx.shape[:2]) != (R, H):
        raise ValueError("sel_idx must be [R, H, max_sel]")
    _need(sel_cnt, "sel_cnt", torch.int32, (R, H))
    _need(out, "out", torch.float32, (R, H * G, d))
    _need(workspace, "workspace", torch.uint8)
    c, k = cfg.c(), kv.c()
    _call("resa_sparse_step", ctypes.byref(c), ctypes.byref(k), R, q.data_ptr(), int(bool(refresh_tail)),
          sel_idx.data_ptr(), sel_cnt.data_ptr(), int(sel_idx.shape[2]), out.data_ptr(), workspace.data_ptr(),
          workspace.numel(), _stream_ptr())


def sparse_decode_noalloc(cfg: Config, kv: PagedKV, q: torch.Tensor, sel_idx: torch.Tensor,
                          sel_cnt: torch.Tensor, out: torch.Tensor) -> None:
    """resa_sparse_decode on the library's static per-GPU scratch (no workspace)."""
    _check_cache(cfg, kv)
    R, H, G, d = kv.num_requests, cfg.num_kv_heads, cfg.group_size, cfg.head_dim
    _need(q, "q", cfg.torch_dtype, (R, H * G, d))
    _need(sel_idx, "sel_idx", torch.int32)
    if sel_idx.dim() != 3 or tuple(sel_idx.shape[:2]) != (R, H):
        raise ValueError("sel_idx must be [R, H, max_sel]")
    _need(sel_cnt, "sel_cnt", torch.int32, (R, H))
    _need(out, "out", torch.float32, (R, H * G, d))
    c, k = cfg.c(), kv.c()
    _call("resa_sparse_decode_noalloc", ctypes.byref(c), ctypes.byref(k), R, q.data_ptr(), sel_idx.data_ptr(),
          sel_cnt.data_ptr(), int(sel_idx.shape[2]), out.data_ptr(), _stream_ptr())


def dense_decode(cfg: Config, kv: PagedKV, q: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor) -> None:
    _check_cache(cfg, kv)
    R, H, G, d = kv.num_requests, cfg.num_kv_heads, cfg.group_size, cfg.head_dim
    _need(q, "q", cfg.torch_dtype, (R, H * G, d))
    _need(out, "out", torch.float32, (R, H * G, d))
    _need(workspace, "workspace", torch.uint8)
    c, k = cfg.c(), kv.c()
    _call("resa_dense_decode", ctypes.byref(c), ctypes.byref(k), R, q.data_ptr(), out.data_ptr(),
          workspace.data_ptr(), workspace.numel(), _stream_ptr())


def dense_rectify(cfg: Config, kv: PagedKV, q_chunk: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                  out: torch.Tensor, workspace: torch.Tensor) -> None:
    _check_cache(cfg, kv)
    R, H, G, d = kv.num_requests, cfg.num_kv_heads, cfg.group_size, cfg.head_dim
    f = int(q_chunk.shape[1]) if q_chunk.dim() == 4 else -1
    _need(q_chunk, "q_chunk", cfg.torch_dtype, (R, f, H * G, d))
    _need(k_new, "k_new", cfg.torch_dtype, (R, f, H, d))
    _need(v_new, "v_new", cfg.torch_dtype, (R, f, H, d))
    _need(out, "out", torch.float32, (R, f, H * G, d))
    _need(workspace, "workspace", torch.uint8)
    c, k = cfg.c(), kv.c()
    _call("resa_dense_rectify", ctypes.byref(c), ctypes.byref(k), R, f, q_chunk.data_ptr(), k_new.data_ptr(),
          v_new.data_ptr(), out.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream_ptr())
