"""GPU parity of the gated epilogue: out = g * A + (1 - g) * x ("Sparse Attention for
Long-Context LLMs", section 4.3, step 6), with one gate per (head, query) row or per element.

The reference is the oracle's attention output A (float64) passed through the oracle's
gated_fusion; lse must equal the ungated call's bit for bit (the gate does not touch it).
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_gqa_pool_amd as bsg
import oracle as O
from workloads import SPECS, make_workload

from gpu_util import check_out, compare_selection, mini_pool, note, sample_tokens, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gate_and_x(shape, per_dim, dtype, seed):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    gshape = shape if per_dim else shape[:-1]
    gate = (torch.rand(gshape, generator=gen) * 2.0 - 0.5).to(DEV)          # gates in [-0.5, 1.5)
    x = torch.randn(shape, generator=gen).to(dtype).to(DEV)
    return gate.contiguous(), x.contiguous()


@pytest.mark.parametrize("per_dim", [0, 1])
@pytest.mark.parametrize("spec", [SPECS[1].replace(seq_len=2048 + 40), SPECS[0]], ids=["bf16", "f32"])
def test_prefill_gated(spec, per_dim):
    w = make_workload(spec, 41, device=DEV, tail_fill=float("nan"))
    note(f"[case] gated prefill {spec.name} per_dim={per_dim}")
    B, Hq, S, D = w.q.shape
    k, bs = spec.top_k, spec.page_size
    scale = 1.0 / math.sqrt(D)
    cache = torch.zeros(w.k_cache.shape[0], spec.num_kv_heads, D, dtype=w.k_cache.dtype, device=DEV)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
    idx = torch.empty(B, spec.num_kv_heads, S, k, dtype=torch.int32, device=DEV)
    bsg.group_score_topk(w.q, w.kv_lens, cache, w.page_table, idx, page_size=bs)
    gate, x = _gate_and_x(tuple(w.q.shape), per_dim, w.q.dtype, 7 + per_dim)
    out0, lse0 = torch.empty_like(w.q), torch.empty(B, Hq, S, dtype=torch.float32, device=DEV)
    bsg.sparse_attn_prefill(w.q, w.kv_lens, w.k_cache, w.v_cache, w.page_table, idx, scale, out0, lse0)
    out, lse = torch.empty_like(w.q), torch.empty(B, Hq, S, dtype=torch.float32, device=DEV)
    bsg.sparse_attn_prefill_gated(w.q, w.kv_lens, w.k_cache, w.v_cache, w.page_table, idx, scale, gate, x, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse0), "the gate changed lse"
    tsel = sample_tokens(S, bs, 40, seed=3)
    r = O.prefill_reference(to_np(w.q), to_np(w.k_cache), to_np(w.v_cache), w.page_table.cpu().numpy(),
                            w.kv_lens_host, bs, k, spec.dtype, t_idx=tsel)
    ts = torch.from_numpy(tsel).to(DEV)
    gi = idx[:, :, ts].cpu().numpy()
    bad, _ = compare_selection(gi, r["block_idx"], r["scores"], k)
    assert not bad, bad[:5]
    ref = O.gated_fusion(r["out"], to_np(gate[:, :, ts]), to_np(x[:, :, ts]))
    same = np.repeat(~(gi != r["block_idx"]).any(-1), spec.group_size, axis=1)
    check_out(to_np(out[:, :, ts])[same], ref[same], spec.dtype, "gated out")


@pytest.mark.parametrize("per_dim", [0, 1])
@pytest.mark.parametrize("spec", [
    SPECS[2].replace(batch=3, ctx_len=64 * 60 + 9),                                       # fused decode step
    SPECS[2].replace(batch=40, ctx_len=64 * 12 + 9),             # 160 units: one workgroup each, gate in that kernel
    SPECS[2].replace(batch=2, ctx_len=64 * 30 + 1, num_q_heads=40, head_dim=64, num_kv_heads=2),   # G = 20: split path
], ids=["fused", "fused_one_member", "split"])
def test_decode_step_gated(spec, per_dim):
    w = make_workload(spec, 43, device=DEV, tail_fill=float("nan"))
    note(f"[case] gated decode {spec.name} G={spec.group_size} per_dim={per_dim}")
    B, Hq, _, D = w.q.shape
    Hkv, bs, k = spec.num_kv_heads, spec.page_size, spec.top_k
    scale = 1.0 / math.sqrt(D)
    cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=DEV)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
    q = w.q[:, :, 0].contiguous()
    gate, x = _gate_and_x((B, Hq, D), per_dim, w.q.dtype, 11 + per_dim)
    idx0 = torch.empty(B, Hkv, k, dtype=torch.int32, device=DEV)
    out0, lse0 = torch.empty_like(q), torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.decode_step(q, w.kv_lens, cache, w.k_cache, w.v_cache, w.page_table, scale, idx0, out0, lse0)
    idx = torch.empty_like(idx0)
    out, lse = torch.empty_like(q), torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.decode_step_gated(q, w.kv_lens, cache, w.k_cache, w.v_cache, w.page_table, scale, idx, gate, x, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0) and torch.equal(lse, lse0)
    seqs = list(range(B))
    qn, kp, vp, ptm, kv = mini_pool(w, seqs)
    r = O.decode_reference(qn, kp, vp, ptm, kv, bs, k, spec.dtype, scale)
    gi = idx.cpu().numpy()[:, :, None, :]
    bad, _ = compare_selection(gi, r["block_idx"], r["scores"], k)
    assert not bad, bad
    ref = O.gated_fusion(r["out"][:, :, 0], to_np(gate), to_np(x))
    same = np.repeat(~(gi != r["block_idx"]).any(-1)[:, :, 0], spec.group_size, axis=1)
    check_out(to_np(out)[same], ref[same], spec.dtype, "gated decode out")
