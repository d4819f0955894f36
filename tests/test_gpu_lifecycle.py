"""GPU tests of the page lifecycle: prefill in chunks over a growing paged prefix, and a
decode loop that appends tokens into their pages and refreshes the block cache whenever a
page completes.

The block cache holds one representative per complete page, indexed like the KV cache
("Art of Focus: Ling 2.0 and the Revolution in Sparse Attention", section "Summarizing the
Breakthrough": representatives are built as the context is prefilled, kept in a page-aware
cache sharing the KV cache's indexing, and used at decode).  So:

* a chunked prefill, which pools each chunk's newly completed pages (`blk_begin`) and then
  selects and attends for the chunk's queries over everything before them, must give the
  same block cache, the same selections and the same outputs as a one-shot prefill --
  bit for bit wherever the chunk is long enough to use the same selection kernel, since no
  step of a row's arithmetic depends on how the queries are tiled;
* a decode loop whose token slots beyond kv_len hold NaN until the token is written must
  match the oracle at every step (block cache bit for bit, selections up to the tie
  window, outputs within the bf16 bounds).
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_gqa_pool_amd as bsg
import oracle as O
from workloads import SPECS, make_workload

from gpu_util import check_out, compare_selection, gpu_prefill, note, sample_tokens, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _chunked_prefill(w, top_k, chunks):
    """Prefill chunk by chunk (batch 1): pool the pages completed by the chunk, select and
    attend for its queries.  Returns (block_cache, block_idx, out, lse) over all queries."""
    s = w.spec
    B, Hq, S, D = w.q.shape
    assert B == 1 and sum(chunks) == S
    bs, Hkv = s.page_size, s.num_kv_heads
    scale = 1.0 / math.sqrt(D)
    cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=DEV)
    idx = torch.empty(B, Hkv, S, top_k, dtype=torch.int32, device=DEV)
    out = torch.empty_like(w.q)
    lse = torch.empty(B, Hq, S, dtype=torch.float32, device=DEV)
    start = 0
    for n in chunks:
        end = start + n
        kv = torch.tensor([end], dtype=torch.int32, device=DEV)
        begin = torch.tensor([start // bs], dtype=torch.int32, device=DEV)   # pages completed since
        bsg.block_pool(w.k_cache, w.page_table, kv, cache, blk_begin=begin)
        qc = w.q[:, :, start:end].contiguous()
        ic = torch.empty(B, Hkv, n, top_k, dtype=torch.int32, device=DEV)
        bsg.group_score_topk(qc, kv, cache, w.page_table, ic, page_size=bs)
        oc = torch.empty_like(qc)
        lc = torch.empty(B, Hq, n, dtype=torch.float32, device=DEV)
        bsg.sparse_attn_prefill(qc, kv, w.k_cache, w.v_cache, w.page_table, ic, scale, oc, lc)
        idx[:, :, start:end] = ic
        out[:, :, start:end] = oc
        lse[:, :, start:end] = lc
        start = end
    torch.cuda.synchronize()
    return cache, idx, out, lse


@pytest.mark.parametrize("spec,chunks", [
    (SPECS[1].replace(seq_len=64 * 40 + 29), (700, 1100, 789)),          # bf16, G 8, bs 64, k 32
    (SPECS[1].replace(seq_len=64 * 24 + 5), (64, 1, 63, 700, 713)),      # page-sized, 1-token, ragged chunks
    (SPECS[3].replace(seq_len=128 * 20 + 3, region=512, num_q_heads=16, num_kv_heads=2), (1000, 1563)),   # bs 128
    (SPECS[0], (300, 300, 424)),                                          # fp32
])
def test_chunked_prefill_matches_one_shot(spec, chunks):
    """Queries of chunks of >= 32 tokens go through the same selection kernel as the one-shot
    prefill and must match it bit for bit (bf16; the fp32 path is one kernel throughout).
    Shorter chunks are selected by the materialised-score path (one query: the decode scan),
    whose fp32 sums are ordered differently, so they are held to the oracle instead."""
    w = make_workload(spec, 21, device=DEV, tail_fill=float("nan"))
    note(f"[case] chunked prefill {spec.name} S={w.q.shape[2]} chunks={chunks}")
    k = spec.top_k
    one = gpu_prefill(w, k)
    cache, idx, out, lse = _chunked_prefill(w, k, chunks)
    if cache.dtype == torch.bfloat16:
        assert torch.equal(cache.view(torch.int16), one["block_cache"].view(torch.int16))
    else:
        assert torch.equal(cache, one["block_cache"])
    S = w.q.shape[2]
    exact = torch.zeros(S, dtype=torch.bool)
    start = 0
    for n in chunks:
        if n >= 32 or spec.dtype == "f32":
            exact[start:start + n] = True
        start += n
    ex = exact.to(DEV)
    assert torch.equal(idx[:, :, ex], one["block_idx"][:, :, ex]), "chunked selection differs from one-shot"
    assert torch.equal(out[:, :, ex], one["out"][:, :, ex]), "chunked output differs from one-shot"
    assert torch.equal(lse[:, :, ex], one["lse"][:, :, ex])
    # sampled queries and every query of a short chunk against the oracle
    tsel = np.union1d(sample_tokens(S, spec.page_size, 48, seed=5), np.nonzero(~exact.numpy())[0])
    q, kp, vp = to_np(w.q), to_np(w.k_cache), to_np(w.v_cache)
    pt, kv = w.page_table.cpu().numpy(), w.kv_lens_host
    r = O.prefill_reference(q, kp, vp, pt, kv, spec.page_size, k, spec.dtype, t_idx=tsel)
    gi = idx[:, :, torch.from_numpy(tsel).to(DEV)].cpu().numpy()
    bad, exempt = compare_selection(gi, r["block_idx"], r["scores"], k)
    note(f"  oracle rows {gi.shape[1] * gi.shape[2]}, exempt {len(exempt)}, bad {len(bad)}")
    assert not bad, bad[:5]
    same = np.repeat(~(gi != r["block_idx"]).any(-1), spec.group_size, axis=1)
    go = to_np(out[:, :, torch.from_numpy(tsel).to(DEV)])
    check_out(go[same], r["out"][same], spec.dtype, "oracle-checked out")


@pytest.mark.parametrize("spec,steps", [
    (SPECS[4].replace(batch=3, ctx_range=(64 * 20 + 50, 64 * 34), num_q_heads=16, num_kv_heads=2), 70),
    (SPECS[2].replace(batch=2, ctx_len=64 * 13 + 3), 10),                  # 826 -> 836 crosses 832
])
def test_decode_loop_with_page_completion(spec, steps):
    """Each step writes the new token's K/V into its page slot (NaN before), refreshes the
    block cache if the token completed its page, and runs one decode step."""
    w = make_workload(spec, 33, device=DEV, tail_fill=float("nan"))
    B, Hq, _, D = w.q.shape
    Hkv, bs, k = spec.num_kv_heads, spec.page_size, spec.top_k
    scale = 1.0 / math.sqrt(D)
    kv_final = np.array(w.kv_lens_host, dtype=np.int64)
    kv0 = kv_final - steps
    note(f"[case] decode loop {spec.name} B={B} kv {list(kv0)} -> {list(kv_final)} steps {steps}")
    pt = w.page_table.cpu().numpy()
    # the tokens the loop appends: save their K/V and blank their slots with NaN
    pages = np.concatenate([pt[b, (np.arange(kv0[b], kv_final[b]) // bs)] for b in range(B)])
    slots = np.concatenate([np.arange(kv0[b], kv_final[b]) % bs for b in range(B)])
    pg = torch.from_numpy(pages.astype(np.int64)).to(DEV)
    sl = torch.from_numpy(slots.astype(np.int64)).to(DEV)
    k_new = w.k_cache[pg, :, sl].clone()          # [B * steps, Hkv, D]
    v_new = w.v_cache[pg, :, sl].clone()
    w.k_cache[pg, :, sl] = float("nan")
    w.v_cache[pg, :, sl] = float("nan")
    kp, vp = to_np(w.k_cache), to_np(w.v_cache)   # host copies kept in step with the device
    kn, vn = to_np(k_new), to_np(v_new)
    gen = torch.Generator(device="cpu").manual_seed(1234)
    qs = (torch.randn(steps, B, Hq, D, generator=gen) * 0.5).to(w.q.dtype)
    cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=DEV)
    kv_dev = torch.from_numpy(kv0.astype(np.int32)).to(DEV)
    bsg.block_pool(w.k_cache, w.page_table, kv_dev, cache)
    idx = torch.empty(B, Hkv, k, dtype=torch.int32, device=DEV)
    out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    refreshed = 0
    for n in range(steps):
        kv = kv0 + n + 1
        # append token kv0 + n of every sequence
        rows = np.array([b * steps + n for b in range(B)])
        rt = torch.from_numpy(rows).to(DEV)
        w.k_cache[pg[rt], :, sl[rt]] = k_new[rt]
        w.v_cache[pg[rt], :, sl[rt]] = v_new[rt]
        kp[pages[rows], :, slots[rows]] = kn[rows]
        vp[pages[rows], :, slots[rows]] = vn[rows]
        kv_dev = torch.from_numpy(kv.astype(np.int32)).to(DEV)
        done = (kv % bs) == 0                       # the token completed its page
        if done.any():
            # a sequence whose page did not complete gets an empty refresh range
            begin = np.where(done, kv // bs - 1, kv // bs).astype(np.int32)
            bsg.block_pool(w.k_cache, w.page_table, kv_dev, cache, blk_begin=torch.from_numpy(begin).to(DEV))
            refreshed += int(done.sum())
        q = qs[n].to(DEV).contiguous()
        bsg.decode_step(q, kv_dev, cache, w.k_cache, w.v_cache, w.page_table, scale, idx, out, lse)
        torch.cuda.synchronize()
        r = O.decode_reference(to_np(q)[:, :, None, :], kp, vp, pt, list(kv), bs, k, spec.dtype, scale)
        dc = to_np(cache)
        for b in range(B):                          # every complete page, bit for bit
            full = pt[b, :kv[b] // bs]
            assert np.array_equal(dc[full], r["block_cache"][full]), f"step {n}: block cache of sequence {b}"
        gi = idx.cpu().numpy()[:, :, None, :]
        bad, exempt = compare_selection(gi, r["block_idx"], r["scores"], k)
        assert not bad, (n, bad)
        same = np.repeat(~(gi != r["block_idx"]).any(-1)[:, :, 0], spec.group_size, axis=1)
        check_out(to_np(out)[same], r["out"][:, :, 0][same], spec.dtype, f"step {n} out")
        assert np.abs(lse.cpu().numpy()[same] - r["lse"][:, :, 0][same]).max() <= 2e-3
    note(f"  pages refreshed during the loop: {refreshed}")
    assert refreshed >= 1
