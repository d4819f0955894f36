"""Host-side checks of the C ABI (no GPU needed).

The library is loaded (built first if missing; hipcc cross-compiles for gfx950 without a
GPU), every symbol that include/bsg.h declares must be exported with C linkage, and the
host-side argument validation must reject bad calls before anything is launched.  Only
calls that fail validation, or that are pure host queries, are made here.
"""
import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_gqa_pool_amd import _lib
from block_sparse_gqa_pool_amd import build as bld

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsg.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        bld.build()
    return _lib.lib()


def _dims(**kw):
    base = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=64, top_k=8, num_pages=64,
                pt_stride=32, dtype=_lib.BSG_BF16)
    base.update(kw)
    return _lib.BsgDims(**base)


def test_header_declarations_match_exports(L):
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(bsg_[a-z_0-9]+)\s*\(", text))
    assert declared == set(_lib.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (bsg_\w+)$", out, re.M))
    assert declared <= exported, declared - exported
    for name in declared:
        getattr(L, name)


def test_debug_errors_in_release_build(L):
    bits = ctypes.c_uint32(99)
    assert L.bsg_debug_errors(None, 0) == -1
    expect = -3 if os.path.basename(_lib.LIB_PATH) != "libbsg_debug.so" else 0
    assert L.bsg_debug_errors(ctypes.byref(bits), 0) == expect


def test_version_and_status_strings(L):
    assert L.bsg_version() == 10000
    for st, name in _lib.STATUS.items():
        assert L.bsg_status_str(st).decode().startswith(name)
    assert b"unknown" in L.bsg_status_str(7)


BAD = ctypes.c_void_p(0x10)  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("dims,expect", [
    (None, -1),
    (_dims(num_q_heads=6, num_kv_heads=4), -2),
    (_dims(batch=0), -2),
    (_dims(top_k=0), -2),
    (_dims(head_dim=96), -3),
    (_dims(page_size=32), -3),
    (_dims(top_k=65), -3),
    (_dims(dtype=7), -3),
])
def test_validation_of_dims(L, dims, expect):
    dp = None if dims is None else ctypes.byref(dims)
    s = None
    assert L.bsg_block_pool(dp, BAD, BAD, BAD, None, BAD, s) == expect
    assert L.bsg_group_score(dp, BAD, 4, BAD, BAD, BAD, BAD, 32, s) == expect
    assert L.bsg_topk_blocks(dp, BAD, 4, 32, BAD, BAD, s) == expect
    assert L.bsg_group_score_topk(dp, BAD, 4, BAD, BAD, BAD, BAD, BAD, 1 << 30, s) == expect
    assert L.bsg_sparse_attn_prefill(dp, BAD, 4, BAD, BAD, BAD, BAD, BAD, 0.1, BAD, None, s) == expect
    assert L.bsg_sparse_attn_decode(dp, BAD, BAD, BAD, BAD, BAD, BAD, 0.1, BAD, 1 << 30, BAD, None, s) == expect
    assert L.bsg_decode_step(dp, BAD, BAD, BAD, BAD, BAD, BAD, 0.1, BAD, BAD, 1 << 30, BAD, None, s) == expect
    assert L.bsg_sparse_attn_prefill_gated(dp, BAD, 4, BAD, BAD, BAD, BAD, BAD, 0.1, BAD, 0, BAD, BAD, None,
                                           s) == expect
    assert L.bsg_decode_step_gated(dp, BAD, BAD, BAD, BAD, BAD, BAD, 0.1, BAD, BAD, 1 << 30, BAD, 0, BAD, BAD, None,
                                   s) == expect
    if dims is not None and expect != 0:
        assert L.bsg_decode_step_workspace_bytes(dp) == 0
        assert L.bsg_decode_workspace_bytes(dp) == 0
        assert L.bsg_group_score_topk_workspace_bytes(dp, 4) == 0


def test_validation_of_pointers_and_sizes(L):
    d = ctypes.byref(_dims())
    s = None
    assert L.bsg_block_pool(d, None, BAD, BAD, None, BAD, s) == -1
    assert L.bsg_block_pool(d, BAD, BAD, None, None, BAD, s) == -1
    assert L.bsg_group_score(d, BAD, 0, BAD, BAD, BAD, BAD, 32, s) == -2
    assert L.bsg_group_score(d, BAD, 4, BAD, BAD, BAD, None, 32, s) == -1
    assert L.bsg_topk_blocks(d, BAD, 4, 0, BAD, BAD, s) == -2
    assert L.bsg_sparse_attn_prefill(d, BAD, 0, BAD, BAD, BAD, BAD, BAD, 0.1, BAD, None, s) == -2
    assert L.bsg_sparse_attn_prefill(d, BAD, 4, BAD, BAD, BAD, BAD, BAD, 0.1, None, None, s) == -1
    # decode: missing or short workspace
    need = L.bsg_decode_workspace_bytes(d)
    assert need > 0
    assert L.bsg_sparse_attn_decode(d, BAD, BAD, BAD, BAD, BAD, BAD, 0.1, None, need, BAD, None, s) == -4
    assert L.bsg_sparse_attn_decode(d, BAD, BAD, BAD, BAD, BAD, BAD, 0.1, BAD, need - 1, BAD, None, s) == -4
    need2 = L.bsg_decode_step_workspace_bytes(d)
    assert need2 >= need
    assert L.bsg_decode_step(d, BAD, BAD, BAD, BAD, BAD, BAD, 0.1, BAD, BAD, need2 - 1, BAD, None, s) == -4
    assert L.bsg_decode_step(d, BAD, BAD, BAD, BAD, BAD, BAD, 0.1, None, BAD, need2, BAD, None, s) == -1
    # decode with G * D beyond what the split kernel holds
    big = ctypes.byref(_dims(num_q_heads=64, num_kv_heads=2))
    n2 = L.bsg_decode_workspace_bytes(big)
    assert L.bsg_sparse_attn_decode(big, BAD, BAD, BAD, BAD, BAD, BAD, 0.1, BAD, n2, BAD, None, s) == -3


def test_decode_workspace_size_formula(L):
    for B, Hq, Hkv, D, k in [(32, 32, 4, 128, 32), (4, 64, 8, 128, 32), (1, 8, 2, 64, 4), (3, 16, 16, 64, 1)]:
        d = _dims(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, top_k=k)
        n = L.bsg_decode_workspace_bytes(ctypes.byref(d))
        per_split = B * Hkv * (Hq // Hkv) * (D + 2) * 4
        assert n % per_split == 0 and 1 <= n // per_split <= k


def test_validation_of_gated_calls(L):
    d = ctypes.byref(_dims())
    s = None
    pf = lambda gate, per_dim, x: L.bsg_sparse_attn_prefill_gated(d, BAD, 4, BAD, BAD, BAD, BAD, BAD, 0.1, gate,
                                                                  per_dim, x, BAD, None, s)
    assert pf(None, 0, BAD) == -1
    assert pf(BAD, 0, None) == -1
    assert pf(BAD, 2, BAD) == -2
    assert pf(BAD, -1, BAD) == -2
    need = L.bsg_decode_step_workspace_bytes(d)
    ds = lambda gate, per_dim, x, ws=need: L.bsg_decode_step_gated(d, BAD, BAD, BAD, BAD, BAD, BAD, 0.1, BAD, BAD, ws,
                                                                   gate, per_dim, x, BAD, None, s)
    assert ds(None, 0, BAD) == -1
    assert ds(BAD, 0, None) == -1
    assert ds(BAD, 3, BAD) == -2
    assert ds(BAD, 1, BAD, need - 1) == -4


def test_validation_of_fp8_calls(L):
    """The fp8 calls reject a non-bf16 dims, NULL pointers and a short workspace before any
    launch (no device memory is touched: every rejected pointer is a dummy)."""
    s = None
    d = ctypes.byref(_dims())
    df = ctypes.byref(_dims(dtype=_lib.BSG_F32))
    assert L.bsg_quantize_pages_fp8(df, BAD, BAD, BAD, BAD, BAD, s) == -3
    assert L.bsg_quantize_pages_fp8(d, None, BAD, BAD, BAD, BAD, s) == -1
    assert L.bsg_quantize_pages_fp8(d, BAD, BAD, BAD, BAD, None, s) == -1
    assert L.bsg_block_pool_fp8(df, BAD, BAD, BAD, BAD, None, BAD, BAD, s) == -3
    assert L.bsg_block_pool_fp8(d, BAD, None, BAD, BAD, None, BAD, BAD, s) == -1
    need = L.bsg_decode_step_workspace_bytes(d)
    assert need > 0
    step = lambda dd, ws, **nul: L.bsg_decode_step_fp8(
        dd, BAD, BAD, BAD, None if nul.get("rs") else BAD, BAD, BAD, BAD, None if nul.get("vs") else BAD, BAD,
        0.1, BAD, BAD, ws, BAD, None, s)
    assert step(df, need) == -3
    assert step(d, need, rs=True) == -1
    assert step(d, need, vs=True) == -1
    assert step(d, need - 1) == -4
    # outside the matrix-core decode path (G > 16): unsupported
    dg = ctypes.byref(_dims(num_q_heads=34, num_kv_heads=2))
    assert step(dg, 1 << 30) == -3


def test_validation_of_token_calls(L):
    """Token-level calls reject f32 dims, NULL pointers, K < 1 and short workspaces before any
    launch (dummy pointers only)."""
    s = None
    d = ctypes.byref(_dims())
    df = ctypes.byref(_dims(dtype=_lib.BSG_F32))
    need = L.bsg_token_topk_workspace_bytes(d, 0)
    assert need == 2 * 2 * 32 * 64 * 4 and L.bsg_token_topk_workspace_bytes(d, 1) == 2 * 2 * 8 * 64 * 4
    assert L.bsg_token_topk(df, BAD, BAD, BAD, BAD, None, 16, BAD, BAD, need, s) == -3
    assert L.bsg_token_topk(d, None, BAD, BAD, BAD, None, 16, BAD, BAD, need, s) == -1
    assert L.bsg_token_topk(d, BAD, BAD, BAD, BAD, None, 0, BAD, BAD, need, s) == -2
    assert L.bsg_token_topk(d, BAD, BAD, BAD, BAD, None, 16, BAD, BAD, need - 1, s) == -4
    na = L.bsg_decode_tokens_workspace_bytes(d, 2048)
    assert na > 0
    attn = lambda dd, ws, tok=BAD: L.bsg_sparse_attn_decode_tokens(dd, BAD, BAD, BAD, BAD, BAD, tok, 2048, 0.1, BAD,
                                                                   ws, BAD, None, s)
    assert attn(df, na) == -3 and attn(d, na, None) == -1 and attn(d, na - 1) == -4
    dg = ctypes.byref(_dims(num_q_heads=34, num_kv_heads=2))
    assert attn(dg, 1 << 30) == -3
    ns = L.bsg_decode_step_tokens_workspace_bytes(d, 64, 1)
    assert ns > 0 and L.bsg_decode_step_tokens_workspace_bytes(d, 64, 0) > 0
    step = lambda two, ws, bc=BAD: L.bsg_decode_step_tokens(d, BAD, BAD, bc, BAD, BAD, BAD, 64, two, 0.1, BAD, BAD,
                                                            BAD, ws, BAD, None, s)
    assert step(1, ns, None) == -1 and step(1, ns - 1) == -4
