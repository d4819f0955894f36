"""GPU parity of token-level and two-level selection for decode.

Token level: every earlier token is scored with the identity indexer (the group-summed query
dotted with the token's key), the top K are kept, attention runs over them.  Two level: the
block top-k first, then the token top-K among the kept blocks' tokens.  The oracle computes
the same from the pages' definitions; selections are compared with the tie window, outputs
within the bf16 bounds.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_gqa_pool_amd as bsg
import oracle as O
from workloads import SPECS, make_workload

from gpu_util import check_out, compare_selection, compare_token_selection, note, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _host(w):
    return (to_np(w.q), to_np(w.k_cache), to_np(w.v_cache), w.page_table.cpu().numpy(), list(w.kv_lens_host))


CASES = [
    (SPECS[2].replace(batch=3, ctx_len=64 * 40 + 9), 256),                                   # G 8, bs 64, D 128
    (SPECS[4].replace(batch=2, ctx_range=(64 * 30 + 1, 64 * 50 - 1)), 512),                   # ragged
    (SPECS[2].replace(batch=2, ctx_len=128 * 12 + 100, page_size=128, head_dim=64, num_q_heads=32,
                      num_kv_heads=2, top_k=5), 300),                                         # bs 128, D 64, G 16
    (SPECS[2].replace(batch=2, ctx_len=64 * 5 + 3), 2048),                                    # K above every length
    (SPECS[2].replace(batch=2, ctx_len=64 * 20), 1),                                          # K = 1
    (SPECS[2].replace(batch=2, ctx_len=64 * 90 + 5), 700),                                    # rows > 4096
    (SPECS[2].replace(batch=2, ctx_len=64 * 700 + 3), 1500),                                  # rows > 32768: parts
]
IDS = ["g8_bs64", "ragged", "bs128_d64_g16", "k_all", "k1", "long_rows", "parts"]


@pytest.mark.parametrize("spec,K", CASES, ids=IDS)
def test_token_level_step_matches_oracle(spec, K):
    w = make_workload(spec, 61, device=DEV, tail_fill=float("nan"))
    note(f"[case] token-level decode {spec.name} K={K}")
    B, Hq, _, D = w.q.shape
    Hkv = spec.num_kv_heads
    scale = 1.0 / math.sqrt(D)
    q1 = w.q[:, :, 0].contiguous()
    tok = torch.full((B, Hkv, K), -7, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q1)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.decode_step_tokens(q1, w.kv_lens, w.k_cache, w.v_cache, w.page_table, scale, tok, out, lse)
    torch.cuda.synchronize()
    q, kp, vp, pt, kv = _host(w)
    r = O.decode_tokens_reference(q, kp, vp, pt, kv, K, scale)
    gi = tok.cpu().numpy()[:, :, None, :]
    bad, exempt = compare_token_selection(gi, r["token_idx"], r["scores"], K)
    note(f"  exempt {len(exempt)}, bad {len(bad)}")
    assert not bad, bad
    same = np.repeat(~(gi != r["token_idx"]).any(-1)[:, :, 0], spec.group_size, axis=1)
    check_out(to_np(out)[same], r["out"][:, :, 0][same], "bf16", "token-level out")
    assert np.abs(lse.cpu().numpy()[same] - r["lse"][:, :, 0][same]).max() <= 2e-3
    # the separate calls give the same result bit for bit
    tok2 = torch.full_like(tok, -7)
    bsg.token_topk(q1, w.kv_lens, w.k_cache, w.page_table, tok2)
    out2 = torch.empty_like(q1)
    lse2 = torch.empty_like(lse)
    bsg.sparse_attn_decode_tokens(q1, w.kv_lens, w.k_cache, w.v_cache, w.page_table, tok2, scale, out2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(tok, tok2) and torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse, lse2)


@pytest.mark.parametrize("spec,K", CASES[:3] + [(SPECS[2].replace(batch=2, ctx_len=64 * 20 + 7, top_k=4), 4096)],
                         ids=IDS[:3] + ["k_all_blocks"])
def test_two_level_step_matches_oracle(spec, K):
    w = make_workload(spec, 62, device=DEV, tail_fill=float("nan"))
    note(f"[case] two-level decode {spec.name} k={spec.top_k} K={K}")
    B, Hq, _, D = w.q.shape
    Hkv, bs, k = spec.num_kv_heads, spec.page_size, spec.top_k
    scale = 1.0 / math.sqrt(D)
    cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=DEV)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
    q1 = w.q[:, :, 0].contiguous()
    bidx = torch.empty(B, Hkv, k, dtype=torch.int32, device=DEV)
    tok = torch.full((B, Hkv, K), -7, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q1)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.decode_step_tokens(q1, w.kv_lens, w.k_cache, w.v_cache, w.page_table, scale, tok, out, lse,
                           block_cache=cache, block_idx=bidx)
    torch.cuda.synchronize()
    q, kp, vp, pt, kv = _host(w)
    r = O.two_level_decode_reference(q, kp, vp, pt, kv, bs, k, K, "bf16", scale)
    gb = bidx.cpu().numpy()[:, :, None, :]
    bad, exempt = compare_selection(gb, r["block_idx"], r["block_scores"], k)
    assert not bad, bad
    blk_same = ~(gb != r["block_idx"]).any(-1)                      # [B, Hkv, 1]
    gi = tok.cpu().numpy()[:, :, None, :]
    tb, te = compare_token_selection(gi, r["token_idx"], r["scores"], K)
    tb = [x for x in tb if blk_same[x]]                              # rows whose block sets agree
    note(f"  block exempt {len(exempt)}, token exempt {len(te)}, token bad {len(tb)}")
    assert not tb, tb
    same = np.repeat((~(gi != r["token_idx"]).any(-1) & blk_same)[:, :, 0], spec.group_size, axis=1)
    check_out(to_np(out)[same], r["out"][:, :, 0][same], "bf16", "two-level out")
    assert np.abs(lse.cpu().numpy()[same] - r["lse"][:, :, 0][same]).max() <= 2e-3


@pytest.mark.parametrize("hq,hkv,D", [(80, 4, 64), (36, 6, 128)], ids=["g20", "hkv6"])
def test_token_selection_other_groupings(hq, hkv, D):
    """Token-level selection alone (bsg_token_topk) at groupings the token attention does not
    take or that leave a score workgroup's last groups empty: with G = 20 each summing thread
    reads its query rows itself (more than the 16 per group staged in LDS); with Hkv = 6 the
    second workgroup of four groups has two."""
    spec = SPECS[2].replace(batch=2, ctx_len=64 * 30 + 5, num_q_heads=hq, num_kv_heads=hkv, head_dim=D)
    w = make_workload(spec, 65, device=DEV, tail_fill=float("nan"))
    note(f"[case] token-level selection Hq={hq} Hkv={hkv} D={D}")
    B, Hq, _, D = w.q.shape
    K = 300
    tok = torch.full((B, hkv, K), -7, dtype=torch.int32, device=DEV)
    bsg.token_topk(w.q[:, :, 0].contiguous(), w.kv_lens, w.k_cache, w.page_table, tok)
    torch.cuda.synchronize()
    q, kp, vp, pt, kv = _host(w)
    r = O.decode_tokens_reference(q, kp, vp, pt, kv, K, 1.0 / math.sqrt(D))
    bad, exempt = compare_token_selection(tok.cpu().numpy()[:, :, None, :], r["token_idx"], r["scores"], K)
    note(f"  exempt {len(exempt)}, bad {len(bad)}")
    assert not bad, bad


@pytest.mark.parametrize("ctx,K", [(64 * 700 + 3, 1500), (64 * 300 + 9, 999)], ids=["parts", "one_pass"])
def test_token_level_ties_keep_lower_tokens(ctx, K):
    """Every key of the cache equal: every candidate scores the same, so the kept tokens must
    be the K lowest positions, exactly; rows past 32768 candidates are selected in parts and
    then over the parts' lists, and the ties must still resolve as in one pass."""
    spec = SPECS[2].replace(batch=2, ctx_len=ctx)
    w = make_workload(spec, 64, device=DEV)
    w.k_cache.copy_(w.k_cache[0, 0, 0].expand_as(w.k_cache))
    B, Hq, _, D = w.q.shape
    tok = torch.full((B, spec.num_kv_heads, K), -7, dtype=torch.int32, device=DEV)
    note(f"[case] token-level ties ctx={ctx} K={K}")
    bsg.token_topk(w.q[:, :, 0].contiguous(), w.kv_lens, w.k_cache, w.page_table, tok)
    torch.cuda.synchronize()
    want = torch.arange(K, dtype=torch.int32, device=DEV).expand_as(tok)
    assert torch.equal(tok, want)


def test_token_attention_on_oracle_lists():
    """Attention over token lists the oracle chose (including -1 padding and tokens of the
    partial last page), compared to the oracle's attention."""
    spec = SPECS[4].replace(batch=3, ctx_range=(64 * 20 + 1, 64 * 30 - 1))
    w = make_workload(spec, 63, device=DEV, tail_fill=float("nan"))
    B, Hq, _, D = w.q.shape
    scale = 1.0 / math.sqrt(D)
    q, kp, vp, pt, kv = _host(w)
    rng = np.random.default_rng(4)
    K = 700
    idx = np.full((B, spec.num_kv_heads, 1, K), -1, np.int32)
    for b in range(B):
        for g in range(spec.num_kv_heads):
            n = int(rng.integers(1, K + 1))
            idx[b, g, 0, :n] = np.sort(rng.choice(kv[b], size=min(n, kv[b]), replace=False))
    ref, rlse = O.token_attention(q, kp, vp, pt, kv, idx, scale)
    out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.sparse_attn_decode_tokens(w.q[:, :, 0].contiguous(), w.kv_lens, w.k_cache, w.v_cache, w.page_table,
                                  torch.from_numpy(idx[:, :, 0]).to(DEV).contiguous(), scale, out, lse)
    torch.cuda.synchronize()
    check_out(to_np(out), ref[:, :, 0], "bf16", "token attention")
    assert np.abs(lse.cpu().numpy() - rlse[:, :, 0]).max() <= 2e-3


@pytest.mark.parametrize("cfg", [2, 4], ids=["ctx128k_b32", "ctx512k_1m_b4"])
def test_token_level_full_size_sampled(cfg):
    """The 128K x 32 decode workload (two sequences) and the ragged ~1M x 4 one (its shortest
    sequence) at K = 2048 tokens, against the oracle."""
    spec = SPECS[cfg]
    w = make_workload(spec, cfg, device=DEV)
    B, Hq, _, D = w.q.shape
    Hkv, K = spec.num_kv_heads, 2048
    scale = 1.0 / math.sqrt(D)
    q1 = w.q[:, :, 0].contiguous()
    tok = torch.empty(B, Hkv, K, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q1)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.decode_step_tokens(q1, w.kv_lens, w.k_cache, w.v_cache, w.page_table, scale, tok, out, lse)
    torch.cuda.synchronize()
    from gpu_util import mini_pool
    seqs = [0, 21] if cfg == 2 else [int(np.argmin(w.kv_lens_host))]
    note(f"[case] token-level full decode {spec.name}: sequences {seqs}")
    qn, kp, vp, ptm, kv = mini_pool(w, seqs)
    r = O.decode_tokens_reference(qn, kp, vp, ptm, kv, K, scale)
    gi = tok.cpu().numpy()[seqs][:, :, None, :]
    bad, exempt = compare_token_selection(gi, r["token_idx"], r["scores"], K)
    note(f"  exempt {len(exempt)}, bad {len(bad)}")
    assert not bad, bad
    same = np.repeat(~(gi != r["token_idx"]).any(-1)[:, :, 0], spec.group_size, axis=1)
    check_out(to_np(out)[seqs][same], r["out"][:, :, 0][same], "bf16", "token-level out")
