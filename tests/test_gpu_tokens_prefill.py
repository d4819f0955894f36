"""GPU parity of token-level and two-level selection for prefill rows.

Every query position of the prompt is a row: token level scores all earlier tokens with the
identity indexer (the group-summed query dotted with each key, the decode definition at
every position), keeps the top K and attends over them; two level first keeps the row's
top-k blocks (the prefill block selection), then the top K of their tokens.  The oracle
computes the same from the pages' definitions; selections are compared with the tie
window, outputs within the bf16 bounds where the selections agree.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_gqa_pool_amd as bsg
import oracle as O
from workloads import SPECS, make_workload

from gpu_util import check_out, compare_selection, compare_token_selection, note, sample_tokens, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu_tokens(w, K, two=False, scale=None):
    s = w.spec
    B, Hq, ql, D = w.q.shape
    Hkv = s.num_kv_heads
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    bidx = None
    if two:
        cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=DEV)
        bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
        bidx = torch.empty(B, Hkv, ql, s.top_k, dtype=torch.int32, device=DEV)
        bsg.group_score_topk(w.q, w.kv_lens, cache, w.page_table, bidx, page_size=s.page_size)
    tok = torch.full((B, Hkv, ql, K), -7, dtype=torch.int32, device=DEV)
    bsg.token_topk_prefill(w.q, w.kv_lens, w.k_cache, w.page_table, tok, block_idx=bidx)
    out = torch.full_like(w.q, float("nan"))
    lse = torch.full((B, Hq, ql), float("nan"), dtype=torch.float32, device=DEV)
    bsg.sparse_attn_prefill_tokens(w.q, w.kv_lens, w.k_cache, w.v_cache, w.page_table, tok, scale, out, lse)
    torch.cuda.synchronize()
    return bidx, tok, out, lse


def _check(w, K, bidx, tok, out, lse, tsel=None, two=False):
    s = w.spec
    B, Hq, ql, D = w.q.shape
    scale = 1.0 / math.sqrt(D)
    kp, vp = to_np(w.k_cache), to_np(w.v_cache)
    pt, kv = w.page_table.cpu().numpy(), list(w.kv_lens_host)
    if tsel is None:
        tsel = np.arange(ql)
        q = to_np(w.q)
    else:
        q = np.zeros((B, Hq, ql, D), np.float32)
        q[:, :, tsel] = to_np(w.q[:, :, torch.from_numpy(tsel).to(DEV)])
    ts = torch.from_numpy(tsel).to(DEV)
    blk_same = True
    ob = None
    if two:
        cache = O.block_pool(kp, pt, kv, s.dtype)
        bsc = O.group_scores(q, cache, pt, kv, s.num_kv_heads, s.page_size, tsel)
        ob = O.select_blocks(bsc, kv, ql, s.page_size, s.top_k, tsel)
        gb = bidx[:, :, ts].cpu().numpy()
        bad, ex = compare_selection(gb, ob, bsc, s.top_k)
        assert not bad, bad[:5]
        blk_same = ~(gb != ob).any(-1)
    sc = O.token_scores(q, kp, pt, kv, tsel, block_idx=ob)
    oi = O.select_tokens(sc, K)
    gi = tok[:, :, ts].cpu().numpy()
    bad, exempt = compare_token_selection(gi, oi, sc, K)
    if two:
        bad = [x for x in bad if blk_same[x]]
    note(f"  rows {gi.shape[0] * gi.shape[1] * gi.shape[2]}, token exempt {len(exempt)}, bad {len(bad)}")
    assert not bad, bad[:5]
    ref, rl = O.token_attention(q, kp, vp, pt, kv, oi, scale, tsel)
    same = np.repeat(~(gi != oi).any(-1) & blk_same, s.group_size, axis=1)
    check_out(to_np(out[:, :, ts])[same], ref[same], "bf16", "prefill token out")
    assert np.abs(lse[:, :, ts].cpu().numpy()[same] - rl[same]).max() <= 2e-3


CASES = [
    (SPECS[1].replace(seq_len=64 * 9 + 17), 128),                                            # 5 tiles, ragged
    (SPECS[1].replace(seq_len=64 * 6 + 5, q_len=200), 64),                                   # queries at the end
    (SPECS[1].replace(seq_len=128 * 5 + 33, page_size=128, head_dim=64, num_q_heads=32, num_kv_heads=2,
                      top_k=4), 100),                                                        # bs 128, D 64, G 16
    (SPECS[1].replace(seq_len=64 * 4 + 9), 1024),                                            # K above every row
    (SPECS[1].replace(seq_len=64 * 4 + 9), 1),                                               # K = 1
    (SPECS[1].replace(batch=2, seq_len=64 * 5 + 3), 77),                                     # two sequences
]
IDS = ["g8_bs64", "q_tail", "bs128_d64_g16", "k_all", "k1", "batch2"]


@pytest.mark.parametrize("spec,K", CASES, ids=IDS)
def test_token_level_prefill_matches_oracle(spec, K):
    w = make_workload(spec, 71, device=DEV, tail_fill=float("nan"))
    note(f"[case] token-level prefill {spec.name} q_len={w.q.shape[2]} K={K}")
    bidx, tok, out, lse = _gpu_tokens(w, K)
    _check(w, K, bidx, tok, out, lse)


def test_token_level_prefill_in_windows():
    """A page table wide enough that one position's scores take 32 MiB: the positions go
    through in windows of 32 rows, each a tile of the matrix-core kernel with 32 valid rows."""
    spec = SPECS[1].replace(seq_len=64 * 9 + 17, num_q_heads=16, num_kv_heads=2)
    w = make_workload(spec, 72, device=DEV, tail_fill=float("nan"))
    wide = torch.zeros(w.page_table.shape[0], 65536, dtype=torch.int32, device=DEV)
    wide[:, :w.page_table.shape[1]] = w.page_table
    w.page_table = wide
    K = 96
    note(f"[case] token-level prefill in windows, pt_stride {wide.shape[1]}")
    bidx, tok, out, lse = _gpu_tokens(w, K)
    w.page_table = wide[:, :(spec.seq_len + 63) // 64].contiguous()
    _check(w, K, bidx, tok, out, lse)


@pytest.mark.parametrize("spec,K", CASES[:3] + [(SPECS[1].replace(seq_len=64 * 7 + 3, top_k=3), 4096)],
                         ids=IDS[:3] + ["k_all_blocks"])
def test_two_level_prefill_matches_oracle(spec, K):
    w = make_workload(spec, 73, device=DEV, tail_fill=float("nan"))
    note(f"[case] two-level prefill {spec.name} q_len={w.q.shape[2]} k={spec.top_k} K={K}")
    bidx, tok, out, lse = _gpu_tokens(w, K, two=True)
    _check(w, K, bidx, tok, out, lse, two=True)


@pytest.mark.parametrize("two,K", [(False, 2048), (True, 512)], ids=["token_level", "two_level"])
def test_prefill_tokens_full_size_sampled(two, K):
    """The 32K prefill workload (32 query heads, 4 KV heads, 64-token blocks, top-32 blocks):
    every position through the device path, sampled positions against the oracle."""
    spec = SPECS[1]
    w = make_workload(spec, 1, device=DEV)
    note(f"[case] {'two-level' if two else 'token-level'} prefill {spec.name} K={K}")
    bidx, tok, out, lse = _gpu_tokens(w, K, two=two)
    tsel = sample_tokens(w.q.shape[2], spec.page_size, 24, seed=5)
    _check(w, K, bidx, tok, out, lse, tsel=tsel, two=two)
