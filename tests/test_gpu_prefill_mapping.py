"""The prefill kernel's workgroup -> tile mapping, on the device.

The kernel remaps workgroup ids to tiles so that each XCD gets a balanced set of positions.
There are three forms, chosen by the launch's shape: eight or more (sequence, head) ranges of
at least 512 tiles (ranges rotate over the XCDs), shorter parts cut finer, and the plain
contiguous deal.  One more case takes the kernel's form for a three-stage ring (one barrier
per sub-block instead of pairs).  A mistake in any of them would leave some tiles unwritten or
write others twice.  Each case here starts from NaN-filled outputs and requires every output
and log-sum-exp row to be written with finite values, then compares sampled rows with the
oracle.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_gqa_pool_amd as bsg
import oracle as O
from workloads import SPECS, make_workload

from gpu_util import check_out, compare_selection, note, sample_tokens, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (spec overrides, which mapping form the launch takes)
CASES = [
    # 8 KV heads x 512 tiles of 32 tokens: the rotating form
    (dict(num_q_heads=64, num_kv_heads=8, page_size=128, top_k=16, seq_len=16384), "rotate"),
    # 4 KV heads x 512 tiles: 16 parts would be quarter ranges, so finer parts (4 rounds of 16)
    (dict(num_q_heads=32, num_kv_heads=4, page_size=64, top_k=32, seq_len=16384), "finer"),
    # 3 KV heads x 97 tiles (ragged last tile): the contiguous form
    (dict(num_q_heads=24, num_kv_heads=3, page_size=64, top_k=8, seq_len=32 * 96 + 17), "contiguous"),
    # no GQA sharing (256 tokens per tile) and top-40: the selections take 40 KiB of LDS, so the
    # ring has 3 stages and the kernel runs one barrier per sub-block instead of pairs
    (dict(num_q_heads=4, num_kv_heads=4, page_size=64, top_k=40, seq_len=4096 + 77), "three_stage_ring"),
]


@pytest.mark.parametrize("over,form", CASES, ids=[c[1] for c in CASES])
def test_every_row_written_once(over, form):
    spec = SPECS[1].replace(**over)
    note(f"[case] prefill mapping {form}: {over}")
    w = make_workload(spec, 11, device=DEV)
    B, Hq, S, D = w.q.shape
    Hkv, bs, k = spec.num_kv_heads, spec.page_size, spec.top_k
    cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=DEV)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
    idx = torch.empty(B, Hkv, S, k, dtype=torch.int32, device=DEV)
    bsg.group_score_topk(w.q, w.kv_lens, cache, w.page_table, idx, page_size=bs)
    out = torch.full_like(w.q, float("nan"))
    lse = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=DEV)
    scale = 1.0 / math.sqrt(D)
    bsg.sparse_attn_prefill(w.q, w.kv_lens, w.k_cache, w.v_cache, w.page_table, idx, scale, out, lse)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "some output rows were never written"
    assert torch.isfinite(lse).all(), "some log-sum-exp rows were never written"
    # a second call over the same outputs writes the same bytes (no row depends on another tile)
    out2 = torch.full_like(w.q, float("nan"))
    bsg.sparse_attn_prefill(w.q, w.kv_lens, w.k_cache, w.v_cache, w.page_table, idx, scale, out2, None)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)

    tsel = sample_tokens(S, bs, 48, seed=7)
    kp, vp = to_np(w.k_cache), to_np(w.v_cache)
    pt = w.page_table.cpu().numpy()
    kv = w.kv_lens_host
    ora_cache = O.block_pool(kp, pt, kv, spec.dtype)
    qfull = np.zeros((B, Hq, S, D), np.float32)
    qfull[:, :, tsel] = to_np(w.q[:, :, torch.from_numpy(tsel).to(DEV)])
    sc = O.group_scores(qfull, ora_cache, pt, kv, Hkv, bs, tsel)
    oidx = O.select_blocks(sc, kv, S, bs, k, tsel)
    gi = idx[:, :, torch.from_numpy(tsel).to(DEV)].cpu().numpy()
    bad, _ = compare_selection(gi, oidx, sc, k)
    assert not bad, bad[:5]
    ref, rlse = O.sparse_attention(qfull, kp, vp, pt, kv, oidx, scale, tsel)
    go = to_np(out[:, :, torch.from_numpy(tsel).to(DEV)])
    same = np.repeat(~(gi != oidx).any(-1), spec.group_size, axis=1)
    check_out(go[same], ref[same], spec.dtype, f"{form} sampled out")
    gl = lse[:, :, torch.from_numpy(tsel).to(DEV)].cpu().numpy()
    assert np.abs(gl[same] - rlse[same]).max() <= 2e-3
