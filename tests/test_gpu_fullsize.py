"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The whole path runs on the device at full size; the oracle recomputes sampled outputs
one by one: sampled query tokens for the prefill workloads (with the oracle's own block
cache over every block), sampled sequences for the decode workloads (all of their pages).
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_gqa_pool_amd as bsg
import oracle as O
from workloads import SPECS, make_workload

from gpu_util import check_out, compare_selection, gpu_prefill, mini_pool, note, sample_tokens, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("cfg,n_tok", [(1, 160), (3, 96)])
def test_full_prefill_sampled(cfg, n_tok):
    spec = SPECS[cfg]
    note(f"[case] full prefill {spec.name}")
    w = make_workload(spec, cfg, device=DEV)
    g = gpu_prefill(w, spec.top_k, fused=True)
    S = w.q.shape[2]
    tsel = sample_tokens(S, spec.page_size, n_tok, seed=cfg)
    kp = to_np(w.k_cache)
    vp = to_np(w.v_cache)
    pt = w.page_table.cpu().numpy()
    kv = w.kv_lens_host
    q = to_np(w.q[:, :, torch.from_numpy(tsel).to(DEV)])            # only the sampled queries
    cache = O.block_pool(kp, pt, kv, spec.dtype)
    assert np.array_equal(to_np(g["block_cache"]), cache), "block cache differs"
    # the oracle sees the sampled queries at their true positions: pad q to full length lazily
    qfull = np.zeros((1, spec.num_q_heads, S, spec.head_dim), np.float32)
    qfull[:, :, tsel] = q
    sc = O.group_scores(qfull, cache, pt, kv, spec.num_kv_heads, spec.page_size, tsel)
    idx = O.select_blocks(sc, kv, S, spec.page_size, spec.top_k, tsel)
    gi = g["block_idx"][:, :, torch.from_numpy(tsel).to(DEV)].cpu().numpy()
    bad, exempt = compare_selection(gi, idx, sc, spec.top_k)
    note(f"  sampled rows {gi.shape[1] * gi.shape[2]}, exempt {len(exempt)}, bad {len(bad)}")
    assert not bad, bad[:5]
    out, lse = O.sparse_attention(qfull, kp, vp, pt, kv, idx, 1.0 / math.sqrt(spec.head_dim), tsel)
    go = to_np(g["out"][:, :, torch.from_numpy(tsel).to(DEV)])
    same = np.repeat(~(gi != idx).any(-1), spec.group_size, axis=1)
    check_out(go[same], out[same], spec.dtype, "sampled out")
    gl = g["lse"][:, :, torch.from_numpy(tsel).to(DEV)].cpu().numpy()
    assert np.abs(gl[same] - lse[same]).max() <= 2e-3


@pytest.mark.parametrize("cfg,seqs", [(2, (0, 13, 31)), (4, None)])
def test_full_decode_sampled(cfg, seqs):
    spec = SPECS[cfg]
    note(f"[case] full decode {spec.name}")
    w = make_workload(spec, cfg, device=DEV)
    B, Hq, _, D = w.q.shape
    Hkv, bs, k = spec.num_kv_heads, spec.page_size, spec.top_k
    scale = 1.0 / math.sqrt(D)
    cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=DEV)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
    # the launch configuration bench.py times: the fused decode step
    idx3 = torch.empty(B, Hkv, k, dtype=torch.int32, device=DEV)
    out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.decode_step(w.q[:, :, 0].contiguous(), w.kv_lens, cache, w.k_cache, w.v_cache, w.page_table, scale, idx3,
                    out, lse)
    # and the separate calls must select the same blocks
    idx = torch.empty(B, Hkv, 1, k, dtype=torch.int32, device=DEV)
    bsg.group_score_topk(w.q, w.kv_lens, cache, w.page_table, idx, page_size=bs)
    torch.cuda.synchronize()
    assert torch.equal(idx[:, :, 0], idx3)
    if seqs is None:
        seqs = (int(np.argmin(w.kv_lens_host)),)
    note(f"  sampled sequences {seqs} of lengths {[w.kv_lens_host[b] for b in seqs]}")
    q, kp, vp, ptm, kv = mini_pool(w, seqs)
    r = O.decode_reference(q, kp, vp, ptm, kv, bs, k, spec.dtype, scale)
    sel = list(seqs)
    gi = idx.cpu().numpy()[sel]
    bad, exempt = compare_selection(gi, r["block_idx"], r["scores"], k)
    note(f"  exempt {len(exempt)}, bad {len(bad)}")
    assert not bad, bad
    same = np.repeat(~(gi != r["block_idx"]).any(-1)[:, :, 0], spec.group_size, axis=1)
    check_out(to_np(out)[sel][same], r["out"][:, :, 0][same], spec.dtype, "decode out")
    assert np.abs(lse.cpu().numpy()[sel][same] - r["lse"][:, :, 0][same]).max() <= 2e-3
    # every physical page of the sampled sequences went through the oracle's block pool:
    # compare the device block cache on those pages bit for bit
    pt = w.page_table.cpu().numpy()
    for i, b in enumerate(seqs):
        n = w.kv_lens_host[b] // bs
        dev_reps = to_np(cache[torch.from_numpy(pt[b, :n].astype(np.int64)).to(DEV)])
        assert np.array_equal(dev_reps, r["block_cache"][ptm[i, :n]])
