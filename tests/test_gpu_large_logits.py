"""GPU parity with large logit gaps: the softmax rescale paths.

The matrix-core prefill kernel subtracts a lazily kept reference maximum and rescales its
accumulated output and sum only when a later sub-block would push a weight past 2^64, i.e.
when a selected key scores more than 64 ln 2 above the row's first attended sub-block.  With
unit-variance data and scale 1/sqrt(D) that never happens, so these cases make it happen:
scale = 1.0 (raw logits), or block offsets large enough that planted blocks outscore the
first block by more than 64 ln 2 at the usual scale.  Each case asserts on the host, from the
oracle's per-sub-block maxima, that a large share of rows takes the rescale path, then
compares outputs and lse with the oracle ("Sparse Attention + Linear Backbones", section 5.5:
exact softmax over the selected keys, whatever their logits).  The output bound is the one of
gpu_util.check_out_peaked: with a sharply peaked softmax the bf16 roundings scale with the
output's magnitude.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_gqa_pool_amd as bsg
import oracle as O
from workloads import SPECS, make_workload

from gpu_util import check_out, check_out_peaked, compare_selection, lazy_max_rescale_rows, note, np_inputs, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LSE_TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    bsg.lib()


def _prefill_on_oracle_selection(w, scale):
    s = w.spec
    q, kp, vp, pt, kv = np_inputs(w)
    cache = O.block_pool(kp, pt, kv, s.dtype)
    sc = O.group_scores(q, cache, pt, kv, s.num_kv_heads, s.page_size)
    idx = O.select_blocks(sc, kv, q.shape[2], s.page_size, s.top_k)
    ref_out, ref_lse = O.sparse_attention(q, kp, vp, pt, kv, idx, scale)
    out = torch.empty_like(w.q)
    lse = torch.empty(w.q.shape[:3], dtype=torch.float32, device=DEV)
    bsg.sparse_attn_prefill(w.q, w.kv_lens, w.k_cache, w.v_cache, w.page_table, torch.from_numpy(idx).to(DEV),
                            scale, out, lse)
    torch.cuda.synchronize()
    return (q, kp, pt, kv, idx), to_np(out), lse.cpu().numpy(), ref_out, ref_lse


# (spec changes, scale: None = 1/sqrt(D)); bf16 cases run the matrix-core kernel
BF16_CASES = [
    (dict(top_k=8), 1.0),                                        # D 128, 64-token blocks
    (dict(top_k=8, offset_std=2.0), None),                       # same, usual scale, large offsets
    (dict(page_size=128, top_k=5), 1.0),                         # 128-token blocks
    (dict(page_size=128, top_k=5, offset_std=2.0), None),
    (dict(head_dim=64, top_k=8, offset_std=2.5), None),          # D 64
    (dict(head_dim=64, page_size=128, top_k=5, offset_std=2.5), None),
    (dict(head_dim=64, top_k=8, offset_std=1.5), 1.0),
    (dict(top_k=8, q_len=500), 1.0),                             # queries over a cached prefix
]


@pytest.mark.parametrize("case,scale", BF16_CASES)
def test_prefill_mfma_rescale_path(case, scale):
    spec = SPECS[1].replace(seq_len=64 * 24 + 13, **case)
    sc = 1.0 / math.sqrt(spec.head_dim) if scale is None else scale
    note(f"[case] prefill rescale bf16 {case} scale={sc:.4f}")
    w = make_workload(spec, 5, tail_fill=float("nan")).to(DEV)
    (q, kp, pt, kv, idx), got, gl, ref, rl = _prefill_on_oracle_selection(w, sc)
    rows = lazy_max_rescale_rows(q, kp, pt, kv, idx, sc, spec.page_size, spec.group_size)
    frac = rows.mean()
    note(f"  rows forced through the rescale path: {int(rows.sum())} of {rows.size} ({frac:.1%})")
    assert frac >= 0.10
    check_out_peaked(got, ref, "out")
    check_out_peaked(got[rows], ref[rows], "out (rescaled rows)")
    err = np.abs(gl - rl)
    note(f"  lse max abs err {err.max():.3e} (rescaled rows {err[rows].max():.3e}); |lse| up to {np.abs(rl).max():.1f}")
    assert err.max() <= LSE_TOL


@pytest.mark.parametrize("case,scale", [(dict(), 1.0), (dict(offset_std=2.5), None), (dict(head_dim=128), 1.0)])
def test_prefill_fp32_large_logits(case, scale):
    """fp32 inputs run the VALU kernel (exact running maximum per key)."""
    spec = SPECS[0].replace(**case)
    sc = 1.0 / math.sqrt(spec.head_dim) if scale is None else scale
    note(f"[case] prefill large logits f32 {case} scale={sc:.4f}")
    w = make_workload(spec, 6, tail_fill=float("nan")).to(DEV)
    (q, kp, pt, kv, idx), got, gl, ref, rl = _prefill_on_oracle_selection(w, sc)
    rows = lazy_max_rescale_rows(q, kp, pt, kv, idx, sc, spec.page_size, spec.group_size)
    note(f"  rows with a gap above 64 ln 2: {int(rows.sum())} of {rows.size}")
    assert rows.sum() > 0
    check_out(got, ref, "f32", "out")
    assert np.abs(gl - rl).max() <= 1e-4 * max(1.0, float(np.abs(rl).max()))


@pytest.mark.parametrize("case,scale", [(dict(), 1.0), (dict(offset_std=2.0), None), (dict(head_dim=64), 1.0),
                                        (dict(page_size=128, top_k=9), 1.0)])
@pytest.mark.parametrize("api", ["attn", "step"])
def test_decode_large_logits(case, scale, api):
    spec = SPECS[2].replace(batch=3, ctx_len=64 * 150 + 11, **case)
    sc = 1.0 / math.sqrt(spec.head_dim) if scale is None else scale
    note(f"[case] decode large logits {case} scale={sc:.4f} api={api}")
    w = make_workload(spec, 19, tail_fill=float("nan")).to(DEV)
    q, kp, vp, pt, kv = np_inputs(w)
    r = O.decode_reference(q, kp, vp, pt, kv, spec.page_size, spec.top_k, spec.dtype, sc)
    B, Hq, _, D = w.q.shape
    out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    q1 = w.q[:, :, 0].contiguous()
    if api == "attn":
        didx = torch.from_numpy(r["block_idx"][:, :, 0]).contiguous().to(DEV)
        bsg.sparse_attn_decode(q1, w.kv_lens, w.k_cache, w.v_cache, w.page_table, didx, sc, out, lse)
    else:
        cache = torch.zeros(w.k_cache.shape[0], spec.num_kv_heads, D, dtype=w.k_cache.dtype, device=DEV)
        bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
        didx = torch.empty(B, spec.num_kv_heads, spec.top_k, dtype=torch.int32, device=DEV)
        bsg.decode_step(q1, w.kv_lens, cache, w.k_cache, w.v_cache, w.page_table, sc, didx, out, lse)
    torch.cuda.synchronize()
    gi = didx.cpu().numpy()[:, :, None]
    bad, exempt = compare_selection(gi, r["block_idx"], r["scores"], spec.top_k)
    assert not bad, bad
    same = np.repeat(~(gi != r["block_idx"]).any(-1)[:, :, 0], spec.group_size, axis=1)
    check_out_peaked(to_np(out)[same], r["out"][:, :, 0][same], "decode out")
    err = np.abs(lse.cpu().numpy()[same] - r["lse"][:, :, 0][same])
    note(f"  lse max abs err {err.max():.3e}; |lse| up to {np.abs(r['lse']).max():.1f}")
    assert err.max() <= LSE_TOL
