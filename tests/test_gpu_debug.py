"""The debug build (-DBSG_DEBUG, libbsg_debug.so): clean calls record nothing and give the
release library's results bit for bit; out-of-range ids in the caller's tables (page-table
entries, block ids, token ids) are clamped as in the release build, every kernel returns
normally, and each kind is recorded in the error word that bsg_debug_errors reads back."""
import math
import os

import pytest
import torch

import block_sparse_gqa_pool_amd as bsg
from block_sparse_gqa_pool_amd import _lib
from block_sparse_gqa_pool_amd import build as bld
from workloads import SPECS, make_workload

from gpu_util import note

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PAGE, BLOCK, TOKEN = 1, 2, 4


@pytest.fixture
def debug_lib():
    path = bld.lib_path("debug")
    if bld.is_stale("debug"):
        pytest.fail(f"{path} is missing or older than the sources: python -m block_sparse_gqa_pool_amd.build --debug")
    saved = (_lib.LIB_PATH, _lib._lib)
    _lib.LIB_PATH, _lib._lib = path, None
    bsg.debug_errors(reset=True)
    try:
        yield
    finally:
        _lib.LIB_PATH, _lib._lib = saved


def _decode_inputs(seed, **kw):
    spec = SPECS[2].replace(**{**dict(batch=3, ctx_len=64 * 40 + 9, top_k=6), **kw})
    w = make_workload(spec, seed, device=DEV)
    B, Hq, _, D = w.q.shape
    cache = torch.zeros(w.k_cache.shape[0], spec.num_kv_heads, D, dtype=w.k_cache.dtype, device=DEV)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
    return spec, w, cache


def _step(spec, w, cache, page_table):
    B, Hq, _, D = w.q.shape
    idx = torch.empty(B, spec.num_kv_heads, spec.top_k, dtype=torch.int32, device=DEV)
    out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.decode_step(w.q[:, :, 0].contiguous(), w.kv_lens, cache, w.k_cache, w.v_cache, page_table,
                    1.0 / math.sqrt(D), idx, out, lse)
    torch.cuda.synchronize()
    return idx, out, lse


def test_release_build_has_no_error_word():
    with pytest.raises(bsg.BsgError):
        bsg.debug_errors()


def test_clean_step_records_nothing_and_matches_release():
    note("[case] debug build: clean decode step vs the release build")
    spec, w, cache = _decode_inputs(11)
    ref = _step(spec, w, cache, w.page_table)
    path = bld.lib_path("debug")
    if bld.is_stale("debug"):
        pytest.fail(f"{path} is missing or older than the sources: python -m block_sparse_gqa_pool_amd.build --debug")
    saved = (_lib.LIB_PATH, _lib._lib)
    _lib.LIB_PATH, _lib._lib = path, None
    try:
        bsg.debug_errors(reset=True)
        got = _step(spec, w, cache, w.page_table)
        assert bsg.debug_errors() == 0
    finally:
        _lib.LIB_PATH, _lib._lib = saved
    assert torch.equal(ref[0], got[0])
    assert torch.equal(ref[1].view(torch.int16), got[1].view(torch.int16))
    assert torch.equal(ref[2], got[2])


def test_bad_page_ids_are_recorded(debug_lib):
    note("[case] debug build: page-table entries out of range")
    spec, w, cache = _decode_inputs(12)
    pt = w.page_table.clone()
    num_pages = w.k_cache.shape[0]
    pt[0, 3] = num_pages + 7            # a candidate block of sequence 0
    pt[1, 0] = -5                       # block 0 of sequence 1
    idx, out, lse = _step(spec, w, cache, pt)
    assert bsg.debug_errors() & PAGE
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert bsg.debug_errors() == 0      # the previous call reset the word
    _step(spec, w, cache, w.page_table)
    assert bsg.debug_errors() == 0


def test_bad_block_ids_are_recorded(debug_lib):
    note("[case] debug build: block ids at or past pt_stride (decode and prefill attention)")
    spec, w, cache = _decode_inputs(13)
    idx, _, _ = _step(spec, w, cache, w.page_table)
    assert bsg.debug_errors() == 0
    B, Hq, _, D = w.q.shape
    bad = idx.clone()
    bad[0, 0, 0] = w.page_table.shape[1] + 3
    out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
    bsg.sparse_attn_decode(w.q[:, :, 0].contiguous(), w.kv_lens, w.k_cache, w.v_cache, w.page_table, bad,
                           1.0 / math.sqrt(D), out)
    torch.cuda.synchronize()
    assert bsg.debug_errors() & BLOCK
    assert torch.isfinite(out.float()).all()
    # prefill over the last 5 positions of each sequence
    ql = 5
    q = w.q[:, :, :1].expand(B, Hq, ql, D).contiguous()
    bidx = torch.zeros(B, spec.num_kv_heads, ql, spec.top_k, dtype=torch.int32, device=DEV)
    bidx[..., 1:] = -1
    bidx[1, 0, 2, 0] = w.page_table.shape[1] + 9
    outp = torch.empty_like(q)
    bsg.sparse_attn_prefill(q, w.kv_lens, w.k_cache, w.v_cache, w.page_table, bidx, 1.0 / math.sqrt(D), outp)
    torch.cuda.synchronize()
    assert bsg.debug_errors() & BLOCK
    assert torch.isfinite(outp.float()).all()


def test_bad_token_ids_are_recorded(debug_lib):
    note("[case] debug build: token ids past the page table")
    spec, w, cache = _decode_inputs(14)
    B, Hq, _, D = w.q.shape
    K = 64
    tok = torch.arange(K, dtype=torch.int32, device=DEV).view(1, 1, K).repeat(B, spec.num_kv_heads, 1).contiguous()
    tok[2, 1, 5] = w.page_table.shape[1] * spec.page_size + 100
    out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
    bsg.sparse_attn_decode_tokens(w.q[:, :, 0].contiguous(), w.kv_lens, w.k_cache, w.v_cache, w.page_table, tok,
                                  1.0 / math.sqrt(D), out)
    torch.cuda.synchronize()
    assert bsg.debug_errors() & TOKEN
    assert torch.isfinite(out.float()).all()
