"""Host-side checks of the C ABI: the library loads, exports every function
include/resa.h declares, and rejects bad arguments before touching the GPU.
No call here reaches a kernel launch, so these run without a GPU."""

import ctypes
import math
import os
import re

import pytest

import oracle as O
from block_sparse_attention_resa_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "resa.h")

FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first
FAKE_ODD = 0x10002


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libresa.so not built")
    return B.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(resa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("resa_build_descriptors", "resa_score_select", "resa_sparse_decode", "resa_dense_rectify",
              "resa_dense_decode"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert sorted(B.EXPORTED) == declared_functions()


def test_abi_version_and_status_strings(lib):
    assert lib.resa_abi_version() == 1
    for s, txt in [(0, b"ok"), (1, b"invalid argument"), (3, b"workspace missing or too small")]:
        assert lib.resa_status_string(s) == txt


def cfg(**kw):
    c = B.CConfig()
    assert B.load_library().resa_config_init(ctypes.byref(c), kw.pop("H", 4), kw.pop("G", 7), kw.pop("d", 128),
                                             kw.pop("dtype", 0)) == 0
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_config_defaults(lib):
    c = cfg()
    assert (c.block_size, c.budget_num, c.budget_den, c.min_blocks, c.local_blocks, c.num_splits) == \
        (16, 1, 10, 16, 1, 0)
    assert c.sm_scale == pytest.approx(1 / math.sqrt(128), rel=1e-7)
    c64 = cfg(d=64)
    assert c64.sm_scale == 0.125


@pytest.mark.parametrize("num,den,nmin,nl", [(1, 10, 16, 1), (7, 100, 0, 1), (9, 10, 0, 1), (1, 3, 4, 5)])
def test_selection_count_matches_oracle(lib, num, den, nmin, nl):
    c = cfg(budget_num=num, budget_den=den, min_blocks=nmin, local_blocks=nl)
    for M in list(range(0, 300)) + [2048, 8196, 16384, 65536]:
        assert lib.resa_selection_count(ctypes.byref(c), M) == O.selection_count(M, num, den, nmin, nl)


def test_workspace_and_splits(lib):
    c = cfg()
    assert lib.resa_workspace_bytes(ctypes.byref(c), B.OP_SCORE_SELECT, 1, 16384, 1639, 0) >= 4 * 16384 * 4
    for op in (B.OP_SPARSE_DECODE, B.OP_DENSE_DECODE):
        S = lib.resa_num_splits(ctypes.byref(c), op, 1, 16384, 1639, 0)
        assert S >= 1
        assert lib.resa_workspace_bytes(ctypes.byref(c), op, 1, 16384, 1639, 0) >= 4 * S * 7 * 130 * 4
    S = lib.resa_num_splits(ctypes.byref(c), B.OP_DENSE_RECTIFY, 4, 8200, 0, 64)
    assert S >= 1
    assert lib.resa_workspace_bytes(ctypes.byref(c), B.OP_DENSE_RECTIFY, 4, 8200, 0, 64) >= \
        4 * 4 * S * 64 * 7 * 130 * 4
    # explicit split counts are honoured (capped by the list length)
    c.num_splits = 3
    assert lib.resa_num_splits(ctypes.byref(c), B.OP_DENSE_DECODE, 1, 100, 0, 0) == 3
    assert lib.resa_num_splits(ctypes.byref(c), B.OP_SPARSE_DECODE, 1, 100, 2, 0) == 2
    # invalid requests give 0
    assert lib.resa_workspace_bytes(ctypes.byref(c), 99, 1, 10, 1, 0) == 0
    assert lib.resa_workspace_bytes(ctypes.byref(c), B.OP_DENSE_RECTIFY, 1, 10, 0, 0) == 0
    assert lib.resa_workspace_bytes(ctypes.byref(c), B.OP_SPARSE_DECODE, 1, 10, 0, 0) == 0


@pytest.mark.parametrize("field,value,status", [
    ("num_kv_heads", 0, 1), ("group_size", 0, 1), ("group_size", 17, 2), ("head_dim", 96, 2),
    ("block_size", 32, 2), ("dtype", 5, 1), ("budget_num", 0, 1), ("budget_num", 11, 1),
    ("budget_den", 0, 1), ("min_blocks", -1, 1), ("local_blocks", 0, 1), ("score_mode", 7, 1),
    ("sm_scale", 0.0, 1), ("sm_scale", float("nan"), 1), ("num_splits", -2, 1), ("num_kv_heads", 65536, 2),
])
def test_bad_config_rejected(lib, field, value, status):
    c = cfg()
    setattr(c, field, value)
    assert lib.resa_selection_count(ctypes.byref(c), 10) == -1
    kv = B.CPagedKV(FAKE, FAKE, FAKE, FAKE, FAKE, 10, 10)
    st = lib.resa_build_descriptors(ctypes.byref(c), ctypes.byref(kv), 1, None, 0, None)
    assert st == status


def kv_ok():
    return B.CPagedKV(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 32)


def test_null_and_misaligned_pointers_rejected(lib):
    c = cfg()
    for field in ("k_pool", "desc_pool", "block_table", "seq_lens"):
        kv = kv_ok()
        setattr(kv, field, None)
        assert lib.resa_build_descriptors(ctypes.byref(c), ctypes.byref(kv), 1, None, 0, None) == 1
    kv = kv_ok()
    kv.k_pool = FAKE_ODD
    assert lib.resa_build_descriptors(ctypes.byref(c), ctypes.byref(kv), 1, None, 0, None) == 1
    assert lib.resa_build_descriptors(None, ctypes.byref(kv_ok()), 1, None, 0, None) == 1
    assert lib.resa_build_descriptors(ctypes.byref(c), None, 1, None, 0, None) == 1
    kv = kv_ok()
    kv.num_pool_blocks = 0
    assert lib.resa_build_descriptors(ctypes.byref(c), ctypes.byref(kv), 1, None, 0, None) == 1
    kv = kv_ok()
    kv.max_blocks = 0
    assert lib.resa_build_descriptors(ctypes.byref(c), ctypes.byref(kv), 1, None, 0, None) == 1
    assert lib.resa_build_descriptors(ctypes.byref(c), ctypes.byref(kv_ok()), -1, None, 0, None) == 1


def test_zero_requests_is_a_no_op(lib):
    c = cfg()
    kv = kv_ok()
    assert lib.resa_build_descriptors(ctypes.byref(c), ctypes.byref(kv), 0, None, 0, None) == 0
    assert lib.resa_dense_decode(ctypes.byref(c), ctypes.byref(kv), 0, FAKE, FAKE, None, 0, None) == 0


def test_score_select_argument_checks(lib):
    c = cfg()
    kv = kv_ok()
    n_full = lib.resa_selection_count(ctypes.byref(c), 32)
    ws = lib.resa_workspace_bytes(ctypes.byref(c), B.OP_SCORE_SELECT, 1, 32, n_full, 0)
    call = lambda q, si, sc, ms, wsp, wsb, rt=0: lib.resa_score_select(  # noqa: E731
        ctypes.byref(c), ctypes.byref(kv), 1, q, rt, si, sc, ms, None, wsp, wsb, None)
    assert call(None, FAKE, FAKE, n_full, FAKE, ws) == 1
    assert call(FAKE_ODD, FAKE, FAKE, n_full, FAKE, ws) == 1
    assert call(FAKE, None, FAKE, n_full, FAKE, ws) == 1
    assert call(FAKE, FAKE, None, n_full, FAKE, ws) == 1
    assert call(FAKE, FAKE, FAKE, n_full - 1, FAKE, ws) == 1  # sel_idx rows too short
    assert call(FAKE, FAKE, FAKE, n_full, None, ws) == 3
    assert call(FAKE, FAKE, FAKE, n_full, FAKE, ws - 1) == 3
    kv.k_pool = None  # the tail refresh reads k_pool
    assert call(FAKE, FAKE, FAKE, n_full, FAKE, ws, 1) == 1


def test_decode_argument_checks(lib):
    c = cfg()
    kv = kv_ok()
    ws = lib.resa_workspace_bytes(ctypes.byref(c), B.OP_SPARSE_DECODE, 1, 32, 16, 0)
    sp = lambda q, si, sc, ms, out, wsp, wsb: lib.resa_sparse_decode(  # noqa: E731
        ctypes.byref(c), ctypes.byref(kv), 1, q, si, sc, ms, out, wsp, wsb, None)
    assert sp(None, FAKE, FAKE, 16, FAKE, FAKE, ws) == 1
    assert sp(FAKE, None, FAKE, 16, FAKE, FAKE, ws) == 1
    assert sp(FAKE, FAKE, FAKE, 0, FAKE, FAKE, ws) == 1
    assert sp(FAKE, FAKE, FAKE, 16, None, FAKE, ws) == 1
    assert sp(FAKE, FAKE, FAKE, 16, FAKE_ODD, FAKE, ws) == 1
    assert sp(FAKE, FAKE, FAKE, 16, FAKE, FAKE, ws - 1) == 3
    kv2 = kv_ok()
    kv2.v_pool = None
    assert lib.resa_dense_decode(ctypes.byref(c), ctypes.byref(kv2), 1, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    wsd = lib.resa_workspace_bytes(ctypes.byref(c), B.OP_DENSE_DECODE, 1, 32, 0, 0)
    assert lib.resa_dense_decode(ctypes.byref(c), ctypes.byref(kv), 1, FAKE, FAKE, None, wsd, None) == 3


def test_rectify_argument_checks(lib):
    c = cfg()
    kv = kv_ok()
    ws = lib.resa_workspace_bytes(ctypes.byref(c), B.OP_DENSE_RECTIFY, 1, 32, 0, 16)
    rc = lambda chunk, q, k, v, out, wsb: lib.resa_dense_rectify(  # noqa: E731
        ctypes.byref(c), ctypes.byref(kv), 1, chunk, q, k, v, out, FAKE, wsb, None)
    assert rc(0, FAKE, FAKE, FAKE, FAKE, ws) == 1
    assert rc(257, FAKE, FAKE, FAKE, FAKE, ws) == 1
    assert rc(16, None, FAKE, FAKE, FAKE, ws) == 1
    assert rc(16, FAKE, None, FAKE, FAKE, ws) == 1
    assert rc(16, FAKE, FAKE, None, FAKE, ws) == 1
    assert rc(16, FAKE, FAKE, FAKE, None, ws) == 1
    assert rc(16, FAKE, FAKE, FAKE, FAKE, ws - 1) == 3
    kv2 = kv_ok()
    kv2.max_blocks = 1
    assert lib.resa_dense_rectify(ctypes.byref(c), ctypes.byref(kv2), 1, 17, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  1 << 30, None) == 1


def test_binding_rejects_cpu_tensors():
    import torch
    cfgp = B.Config(num_kv_heads=1, group_size=2, head_dim=64, dtype=B.RESA_F32)
    t = torch.zeros(4, 1, 16, 64)
    kv = B.PagedKV(t, torch.zeros(4, 1, 64, 16), torch.zeros(4, 1, 2, 64),
                   torch.zeros(1, 4, dtype=torch.int32), torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError):
        B.build_descriptors(cfgp, kv)


def test_noalloc_refuses_more_than_its_scratch_before_any_gpu_call(lib):
    """The no-allocation decode checks its size on the host: a call that
    needs more than the static scratch returns the workspace error without
    looking up the scratch or launching anything (fake pointers here)."""
    c = cfg()
    c.num_splits = 1024
    kv = B.CPagedKV(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 40)
    need = lib.resa_workspace_bytes(ctypes.byref(c), B.OP_SPARSE_DECODE, 1, 40, 2048, 0)
    assert need > B.NOALLOC_SCRATCH_BYTES
    st = lib.resa_sparse_decode_noalloc(ctypes.byref(c), ctypes.byref(kv), 1, FAKE, FAKE, FAKE, 2048, FAKE, None)
    assert st == 3
    assert lib.resa_sparse_decode_noalloc(ctypes.byref(c), ctypes.byref(kv), 1, FAKE, FAKE, FAKE, 0, FAKE, None) == 1
    assert lib.resa_sparse_decode_noalloc(None, ctypes.byref(kv), 1, FAKE, FAKE, FAKE, 16, FAKE, None) == 1


def test_step_workspace_and_argument_checks(lib):
    """resa_sparse_step's workspace holds the score keys and the sparse
    decode's partials (it needs no initialisation), and its host checks
    refuse bad arguments before anything is launched (fake pointers)."""
    c = cfg()
    for R, mb, ms in [(1, 32, 16), (1, 16384, 1639), (8, 4096, 410), (3, 100, 20)]:
        step = lib.resa_workspace_bytes(ctypes.byref(c), B.OP_SPARSE_STEP, R, mb, ms, 0)
        parts = (lib.resa_workspace_bytes(ctypes.byref(c), B.OP_SCORE_SELECT, R, mb, ms, 0) +
                 lib.resa_workspace_bytes(ctypes.byref(c), B.OP_SPARSE_DECODE, R, mb, ms, 0))
        assert step == parts and step > 0
    assert lib.resa_workspace_bytes(ctypes.byref(c), B.OP_SPARSE_STEP, 1, 32, 0, 0) == 0
    kv = kv_ok()
    n_full = lib.resa_selection_count(ctypes.byref(c), 32)
    ws = lib.resa_workspace_bytes(ctypes.byref(c), B.OP_SPARSE_STEP, 1, 32, n_full, 0)
    call = lambda q, si, sc, ms, out, wsp, wsb: lib.resa_sparse_step(  # noqa: E731
        ctypes.byref(c), ctypes.byref(kv), 1, q, 1, si, sc, ms, out, wsp, wsb, None)
    assert call(None, FAKE, FAKE, n_full, FAKE, FAKE, ws) == 1
    assert call(FAKE_ODD, FAKE, FAKE, n_full, FAKE, FAKE, ws) == 1
    assert call(FAKE, None, FAKE, n_full, FAKE, FAKE, ws) == 1
    assert call(FAKE, FAKE, None, n_full, FAKE, FAKE, ws) == 1
    assert call(FAKE, FAKE, FAKE, n_full - 1, FAKE, FAKE, ws) == 1  # sel_idx rows too short
    assert call(FAKE, FAKE, FAKE, n_full, None, FAKE, ws) == 1
    assert call(FAKE, FAKE, FAKE, n_full, FAKE_ODD, FAKE, ws) == 1
    assert call(FAKE, FAKE, FAKE, n_full, FAKE, None, ws) == 3
    assert call(FAKE, FAKE, FAKE, n_full, FAKE, FAKE, ws - 1) == 3
    assert lib.resa_sparse_step(ctypes.byref(c), ctypes.byref(kv), 0, FAKE, 1, FAKE, FAKE, n_full, FAKE, None, 0,
                                None) == 0  # no requests: nothing to do
    kv.v_pool = None  # the attention reads v_pool
    assert call(FAKE, FAKE, FAKE, n_full, FAKE, FAKE, ws) == 1
