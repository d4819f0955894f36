"""On-device metamorphic checks: relations that hold between runs of the library itself.

* Page placement: the page table is the only index into the caches ("Art of Focus: Ling 2.0
  and the Revolution in Sparse Attention", section "Summarizing the Breakthrough": the block
  cache shares the KV cache's indexing), so moving the pages of a prefill to other physical
  slots and permuting the table must give bit-identical block cache entries, selections,
  outputs and lse.
* Decode equals prefill: a decode step at kv_len = t + 1 with query row t of a prefill is that
  prefill's row t (the representations built at prefill are the ones decode reads): the same
  blocks (up to the tie window) and the same output within the bf16 bounds.
* Split invariance: decode splits each group's selected pages over workgroups and merges
  partials by log-sum-exp; the split count follows the batch size, so the same sequences run
  alone and inside a larger batch must agree: lse (fp32 sums of fp32 weights) to fp32
  rounding, outputs within the bf16 bounds of each other (each split rounds its weights to
  bf16 against its own running maximum, so the roundings differ with the split).
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import block_sparse_gqa_pool_amd as bsg
import oracle as O
from workloads import SPECS, make_workload

from gpu_util import check_out, compare_selection, gpu_prefill, note, np_inputs, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    bsg.lib()


def _permute_pages(w, seed):
    """The same workload with its pages moved to a random permutation of the physical slots."""
    P = w.k_cache.shape[0]
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(P)).to(DEV)
    k2 = torch.empty_like(w.k_cache)
    v2 = torch.empty_like(w.v_cache)
    k2[perm] = w.k_cache
    v2[perm] = w.v_cache
    pt2 = perm.to(torch.int32)[w.page_table.long()].contiguous()
    return perm, k2, v2, pt2


@pytest.mark.parametrize("case", [
    dict(),                                                     # bf16, 64-token blocks, G 8
    dict(page_size=128, top_k=5, head_dim=64),
    dict(q_len=333),
    dict(batch=2),
    dict(dtype="f32", head_dim=64, num_q_heads=8, num_kv_heads=2, top_k=4),
])
def test_prefill_page_placement_bit_identical(case):
    spec = SPECS[1].replace(**{"seq_len": 64 * 40 + 21, "top_k": 8, **case})
    note(f"[case] page placement {case}")
    w = make_workload(spec, 61, tail_fill=float("nan")).to(DEV)
    a = gpu_prefill(w, spec.top_k)
    perm, k2, v2, pt2 = _permute_pages(w, 3)
    w.k_cache, w.v_cache, w.page_table = k2, v2, pt2
    b = gpu_prefill(w, spec.top_k)
    assert torch.equal(b["block_cache"][perm].view(torch.uint8), a["block_cache"].view(torch.uint8))
    assert torch.equal(b["block_idx"], a["block_idx"])
    assert torch.equal(b["out"].view(torch.uint8), a["out"].view(torch.uint8))
    assert torch.equal(b["lse"].view(torch.int32), a["lse"].view(torch.int32))


@pytest.mark.parametrize("case", [dict(), dict(page_size=128, top_k=5), dict(head_dim=64)])
def test_decode_at_t_plus_one_equals_prefill_row(case):
    spec = SPECS[1].replace(**{"seq_len": 64 * 60 + 37, "top_k": 8, **case})
    note(f"[case] decode(kv_len = t + 1) vs prefill row t {case}")
    w = make_workload(spec, 71).to(DEV)
    bs, Hkv, G, D = spec.page_size, spec.num_kv_heads, spec.group_size, spec.head_dim
    pf = gpu_prefill(w, spec.top_k)
    S = w.q.shape[2]
    rng = np.random.default_rng(0)
    ts = sorted({0, 1, bs - 1, bs, 2 * bs + 5, S - 1, *rng.choice(S, 24, replace=False).tolist()})
    T = len(ts)
    # one decode sequence per sampled t, all reading the prefill's pages and block cache
    kv = torch.tensor([t + 1 for t in ts], dtype=torch.int32, device=DEV)
    pt = w.page_table.expand(T, -1).contiguous()
    q1 = w.q[0][:, ts].transpose(0, 1).contiguous()               # [T, Hq, D]
    idx = torch.empty(T, Hkv, spec.top_k, dtype=torch.int32, device=DEV)
    out = torch.empty(T, spec.num_q_heads, D, dtype=w.q.dtype, device=DEV)
    lse = torch.empty(T, spec.num_q_heads, dtype=torch.float32, device=DEV)
    bsg.decode_step(q1, kv, pf["block_cache"], w.k_cache, w.v_cache, pt, 1.0 / math.sqrt(D), idx, out, lse)
    torch.cuda.synchronize()
    pidx = pf["block_idx"][0][:, ts].transpose(0, 1).cpu().numpy()   # [T, Hkv, k]
    didx = idx.cpu().numpy()
    # selection: equal, or differing only inside the tie window of the oracle's scores
    q, kp, vp, ptn, kvh = np_inputs(w)
    cache = O.block_pool(kp, ptn, kvh, spec.dtype)
    sc = O.group_scores(q, cache, ptn, kvh, Hkv, bs, np.array(ts))     # [1, Hkv, T, nb]
    bad, exempt = compare_selection(didx.transpose(1, 0, 2)[None], pidx.transpose(1, 0, 2)[None], sc, spec.top_k)
    note(f"  rows {T * Hkv}, differing inside the tie window {len(exempt)}")
    assert not bad, bad
    same = np.repeat((didx == pidx).all(-1), G, axis=1)               # [T, Hq]
    pout = to_np(pf["out"][0][:, ts].transpose(0, 1))
    plse = pf["lse"][0][:, ts].transpose(0, 1).cpu().numpy()
    check_out(to_np(out)[same], pout[same].astype(np.float64), "bf16", "decode vs prefill row")
    assert np.abs(lse.cpu().numpy()[same] - plse[same]).max() <= 2e-3


@pytest.mark.parametrize("case", [
    dict(),                                                     # matrix-core path
    dict(page_size=128, top_k=9),
    dict(num_q_heads=80, num_kv_heads=4, head_dim=64),          # G = 20: VALU split path
])
def test_decode_split_count_invariance(case):
    spec = SPECS[2].replace(**{"batch": 3, "ctx_len": 64 * 150 + 11, **case})
    note(f"[case] decode split invariance {case}")
    w = make_workload(spec, 81, tail_fill=float("nan")).to(DEV)
    Hkv, D, k = spec.num_kv_heads, spec.head_dim, spec.top_k
    Hq = spec.num_q_heads
    scale = 1.0 / math.sqrt(D)
    q, kp, vp, pt, kv = np_inputs(w)
    r = O.decode_reference(q, kp, vp, pt, kv, spec.page_size, k, spec.dtype, scale)
    idx_small = torch.from_numpy(r["block_idx"][:, :, 0]).contiguous().to(DEV)
    q1 = w.q[:, :, 0].contiguous()

    def run(B):
        reps = (B + 2) // 3
        qb = q1.repeat(reps, 1, 1)[:B].contiguous()
        kvb = w.kv_lens.repeat(reps)[:B].contiguous()
        ptb = w.page_table.repeat(reps, 1)[:B].contiguous()
        ib = idx_small.repeat(reps, 1, 1)[:B].contiguous()
        d = bsg.dims(w.k_cache, ptb, Hq, k)
        out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
        lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
        bsg.sparse_attn_decode(qb, kvb, w.k_cache, w.v_cache, ptb, ib, scale, out, lse)
        torch.cuda.synchronize()
        return d, out[:3], lse[:3]

    splits = {}
    results = []
    for B in (3, 48, 256):
        d, out, lse = run(B)
        ws = int(bsg.lib().bsg_decode_workspace_bytes(ctypes.byref(d)))
        n = ws // (B * Hq * (D + 2) * 4)                                # partials per (sequence, head)
        splits[B] = n
        results.append((out, lse))
    note(f"  splits per (sequence, group) by batch size: {splits}")
    assert len(set(splits.values())) >= 2
    o0, l0 = results[0]
    for o, l in results[1:]:
        dl = (l - l0).abs().max().item()
        note(f"  lse max diff {dl:.2e}")
        assert dl <= 1e-5 * max(1.0, l0.abs().max().item())
        check_out(to_np(o), to_np(o0).astype(np.float64), spec.dtype, "output vs the other split count")
    check_out(to_np(o0), r["out"][:, :, 0], spec.dtype, "decode out")
