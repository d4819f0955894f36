"""bsg_decode_step_noalloc (workspace in the library's static device scratch) against
bsg_decode_step (caller workspace): bit-identical selections, outputs and lse on two calls in
a row, the second with a smaller input, and a clean rejection of sizes beyond the scratch."""
import math

import pytest
import torch

import block_sparse_gqa_pool_amd as bsg
from workloads import SPECS, make_workload

from gpu_util import note

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _inputs(spec, seed):
    w = make_workload(spec, seed, device=DEV, tail_fill=float("nan"))
    B, Hq, _, D = w.q.shape
    cache = torch.zeros(w.k_cache.shape[0], spec.num_kv_heads, D, dtype=w.k_cache.dtype, device=DEV)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
    return w, cache


def _both(w, cache, spec):
    B, Hq, _, D = w.q.shape
    q1 = w.q[:, :, 0].contiguous()
    scale = 1.0 / math.sqrt(D)
    res = []
    for noalloc in (False, True):
        idx = torch.full((B, spec.num_kv_heads, spec.top_k), -9, dtype=torch.int32, device=DEV)
        out = torch.full((B, Hq, D), float("nan"), dtype=w.q.dtype, device=DEV)
        lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=DEV)
        if noalloc:
            bsg.decode_step_noalloc(q1, w.kv_lens, cache, w.k_cache, w.v_cache, w.page_table, scale, idx, out, lse)
        else:
            bsg.decode_step(q1, w.kv_lens, cache, w.k_cache, w.v_cache, w.page_table, scale, idx, out, lse)
        torch.cuda.synchronize()
        res.append((idx, out, lse))
    return res


@pytest.mark.parametrize("first,second", [
    (dict(batch=32, ctx_len=64 * 2048), dict(batch=5, ctx_len=64 * 300 + 7)),            # 128K x 32, then small
    (dict(batch=4, ctx_len=64 * 900 + 3, num_q_heads=64, num_kv_heads=8, page_size=128, top_k=9),
     dict(batch=2, ctx_len=64 * 40 + 1, num_q_heads=64, num_kv_heads=8, page_size=128, top_k=9)),
    (dict(batch=3, ctx_len=64 * 150 + 11, num_q_heads=80, num_kv_heads=4, head_dim=64),  # G = 20: split path
     dict(batch=2, ctx_len=64 * 20 + 5, num_q_heads=80, num_kv_heads=4, head_dim=64)),
])
def test_decode_step_noalloc_matches_decode_step(first, second):
    assert bsg.noalloc_scratch_bytes() == 8 << 20
    for i, kw in enumerate((first, second)):
        spec = SPECS[2].replace(**kw)
        note(f"[case] decode_step_noalloc call {i}: {kw}")
        w, cache = _inputs(spec, 90 + i)
        (ia, oa, la), (ib, ob, lb) = _both(w, cache, spec)
        assert torch.equal(ia, ib)
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32))
        del w, cache
        torch.cuda.empty_cache()


def test_decode_step_noalloc_rejects_sizes_beyond_scratch():
    """A batch whose workspace exceeds the scratch is refused before anything is enqueued."""
    spec = SPECS[2].replace(batch=64, ctx_len=64 * 64)
    w, cache = _inputs(spec, 3)
    B, Hq, _, D = w.q.shape
    big = torch.zeros(B, w.page_table.shape[1] * 100, dtype=torch.int32, device=DEV)  # a longer page-table row
    big[:, :w.page_table.shape[1]] = w.page_table
    need = bsg.decode_step_workspace_bytes(w.k_cache, big, Hq, spec.top_k)
    note(f"  workspace needed {need} bytes, scratch {bsg.noalloc_scratch_bytes()} bytes")
    assert need > bsg.noalloc_scratch_bytes()
    idx = torch.full((B, spec.num_kv_heads, spec.top_k), -9, dtype=torch.int32, device=DEV)
    out = torch.zeros(B, Hq, D, dtype=w.q.dtype, device=DEV)
    with pytest.raises(bsg.BsgError) as e:
        bsg.decode_step_noalloc(w.q[:, :, 0].contiguous(), w.kv_lens, cache, w.k_cache, w.v_cache, big,
                                1.0 / math.sqrt(D), idx, out)
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert bool((idx == -9).all()) and bool((out == 0).all())
