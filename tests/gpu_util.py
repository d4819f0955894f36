"""Helpers for the GPU parity tests: run the library, run the oracle, compare."""
from __future__ import annotations

import math
import sys
from typing import Optional, Sequence

import numpy as np
import torch

import block_sparse_gqa_pool_amd as bsg
import oracle as O

TIE_REL = 1e-4          # selection tie window (relative score gap)
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
F32_MAX = 1e-4


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.dtype in (torch.bfloat16, torch.float16) else t.detach().cpu().numpy()


def np_inputs(w):
    return (to_np(w.q), to_np(w.k_cache), to_np(w.v_cache), w.page_table.cpu().numpy(), list(w.kv_lens_host))


def cache_dtype(w) -> str:
    return w.spec.dtype


def gpu_prefill(w, top_k: int, scale: Optional[float] = None, fused: bool = True, lse: bool = True):
    """block_pool -> selection -> sparse attention on the device; returns torch tensors."""
    s = w.spec
    B, Hq, ql, D = w.q.shape
    dev = w.q.device
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    cache = torch.zeros(w.k_cache.shape[0], s.num_kv_heads, D, dtype=w.k_cache.dtype, device=dev)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
    idx = torch.empty(B, s.num_kv_heads, ql, top_k, dtype=torch.int32, device=dev)
    if fused:
        bsg.group_score_topk(w.q, w.kv_lens, cache, w.page_table, idx, page_size=s.page_size)
    else:
        sc = torch.empty(B, s.num_kv_heads, ql, w.pt_stride, dtype=torch.float32, device=dev)
        bsg.group_score(w.q, w.kv_lens, cache, w.page_table, sc, page_size=s.page_size)
        bsg.topk_blocks(sc, w.kv_lens, idx, page_size=s.page_size)
    out = torch.empty_like(w.q)
    l = torch.empty(B, Hq, ql, dtype=torch.float32, device=dev) if lse else None
    bsg.sparse_attn_prefill(w.q, w.kv_lens, w.k_cache, w.v_cache, w.page_table, idx, scale, out, l)
    torch.cuda.synchronize()
    return dict(block_cache=cache, block_idx=idx, out=out, lse=l)


def sample_tokens(q_len: int, bs: int, n: int, seed: int = 0) -> np.ndarray:
    """Sorted distinct query indices: the first and last few, block edges, random others."""
    rng = np.random.default_rng(seed)
    picks = {0, 1, q_len - 1, q_len - 2, min(bs - 1, q_len - 1), min(bs, q_len - 1)}
    for e in (bs, 2 * bs, q_len // 2):
        for d in (-1, 0, 1):
            if 0 <= e + d < q_len:
                picks.add(e + d)
    picks.update(rng.choice(q_len, size=min(n, q_len), replace=False).tolist())
    return np.array(sorted(picks), dtype=np.int64)


def compare_selection(gpu_idx: np.ndarray, ora_idx: np.ndarray, scores64: np.ndarray, top_k: int):
    """Selection parity with the tie exemption.

    gpu_idx, ora_idx: [B, Hkv, T, k]; scores64: oracle float64 scores [B, Hkv, T, nb].
    A differing row is exempt only if the oracle's last kept and first dropped candidates
    score within TIE_REL of each other and every block in the difference scores within that
    window of the boundary.  Returns (bad_rows, exempt_rows)."""
    bad, exempt = [], []
    diff = np.nonzero((gpu_idx != ora_idx).any(-1))
    for b, g, t in zip(*diff):
        row = scores64[b, g, t]
        gi = [int(x) for x in gpu_idx[b, g, t] if x >= 0]
        oi = [int(x) for x in ora_idx[b, g, t] if x >= 0]
        own = oi[-1]
        ok = (len(gi) == len(oi) and gi == sorted(gi) and len(set(gi)) == len(gi) and gi[-1] == own
              and all(0 <= j < own for j in gi[:-1]))
        m = top_k - 1
        cands = sorted(range(own), key=lambda j: (-np.float32(row[j]), j))
        if ok and len(cands) > m >= 1:
            sa, sb = row[cands[m - 1]], row[cands[m]]
            win = TIE_REL * max(abs(sa), abs(sb))
            ok = abs(sa - sb) < win and all(abs(row[j] - sa) <= win or abs(row[j] - sb) <= win
                                            for j in set(gi) ^ set(oi))
        else:
            ok = False
        (exempt if ok else bad).append((int(b), int(g), int(t)))
    return bad, exempt


def check_out(gpu_out: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    err = np.abs(gpu_out.astype(np.float64) - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    note(f"  {what}: max abs err {mx:.3e}, mean abs err {mean:.3e}")
    assert np.all(np.isfinite(gpu_out)), f"{what}: non-finite outputs"
    if dtype == "bf16":
        assert mx <= BF16_MAX and mean <= BF16_MEAN, f"{what}: max {mx} mean {mean}"
    else:
        assert mx <= F32_MAX, f"{what}: max {mx}"


def check_out_peaked(gpu_out: np.ndarray, ref: np.ndarray, what: str):
    """bf16 outputs of a sharply peaked softmax (large logits): element-wise
    |err| <= BF16_MAX + 2^-7 |ref| and mean-abs <= BF16_MEAN.

    When one weight dominates, the output is close to a single value row, and two bf16
    roundings each cost up to the unit roundoff 2^-8 of its magnitude: the output's own
    rounding, and the rounding of the dominant weight (the weights enter the value product
    in bf16, their sum in fp32).  The absolute bound alone is sized for outputs averaged over
    many keys, whose magnitude is well below 1."""
    err = np.abs(gpu_out.astype(np.float64) - ref)
    lim = BF16_MAX + 2.0 ** -7 * np.abs(ref)
    worst = float((err / lim).max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    note(f"  {what}: max abs err {float(err.max()) if err.size else 0:.3e} (|ref| up to "
         f"{float(np.abs(ref).max()) if err.size else 0:.2f}), worst err / bound {worst:.3f}, mean abs err {mean:.3e}")
    assert np.all(np.isfinite(gpu_out)), f"{what}: non-finite outputs"
    assert worst <= 1.0 and mean <= BF16_MEAN, f"{what}: worst err/bound {worst}, mean {mean}"


def mini_pool(w, seqs: Sequence[int]):
    """Host copies holding only the pages of the given sequences, with a remapped table."""
    pt = w.page_table.cpu().numpy()
    bs = w.spec.page_size
    rows, pages = [], []
    for b in seqs:
        n = (w.kv_lens_host[b] + bs - 1) // bs
        rows.append((len(pages), n))
        pages.extend(pt[b, :n].tolist())
    sel = torch.tensor(pages, dtype=torch.int64, device=w.k_cache.device)
    kp = to_np(w.k_cache.index_select(0, sel))
    vp = to_np(w.v_cache.index_select(0, sel))
    ptm = np.zeros((len(seqs), max(n for _, n in rows)), np.int32)
    for i, (o, n) in enumerate(rows):
        ptm[i, :n] = np.arange(o, o + n, dtype=np.int32)
    q = to_np(w.q[list(seqs)])
    kv = [w.kv_lens_host[b] for b in seqs]
    return q, kp, vp, ptm, kv


def compare_token_selection(gpu_idx: np.ndarray, ora_idx: np.ndarray, scores64: np.ndarray, top_k: int):
    """Token selection parity with the tie exemption (as compare_selection, for token lists).

    gpu_idx, ora_idx: [B, Hkv, T, K] ascending, -1 padded; scores64: oracle float64 scores
    [B, Hkv, T, L] (-inf for non-candidates).  A differing row is exempt only if the
    oracle's K-th and (K+1)-th candidates score within TIE_REL of each other and every token
    in the difference scores within that window of the boundary.  Returns (bad, exempt)."""
    bad, exempt = [], []
    diff = np.nonzero((gpu_idx != ora_idx).any(-1))
    for b, g, t in zip(*diff):
        row = scores64[b, g, t]
        gi = [int(x) for x in gpu_idx[b, g, t] if x >= 0]
        oi = [int(x) for x in ora_idx[b, g, t] if x >= 0]
        cand = np.nonzero(np.isfinite(row))[0]
        ok = (len(gi) == len(oi) and gi == sorted(gi) and len(set(gi)) == len(gi)
              and all(np.isfinite(row[j]) for j in gi) and len(cand) > top_k)
        if ok:
            order = cand[np.lexsort((cand, -row[cand].astype(np.float32)))]
            sa, sb = row[order[top_k - 1]], row[order[top_k]]
            win = TIE_REL * max(abs(sa), abs(sb))
            ok = abs(sa - sb) <= win and all(abs(row[j] - sa) <= win or abs(row[j] - sb) <= win
                                             for j in set(gi) ^ set(oi))
        (exempt if ok else bad).append((int(b), int(g), int(t)))
    return bad, exempt


def lazy_max_rescale_rows(q, kp, pt, kv, idx, scale: float, page_size: int, group_size: int, sub: int = 64):
    """Rows (sequence, query head, query) of a prefill that must move a lazily kept softmax
    reference maximum after their first sub-block.

    The matrix-core prefill kernel keeps, per row, the maximum m of the first 64-key sub-block
    it attends to, and only rescales its accumulated output and sum when a later sub-block
    holds a weight exp(z - m) above 2^64, i.e. a scaled logit z more than 64 ln 2 above m.
    Sub-blocks are visited in ascending key order (selected blocks ascending, the causal keys
    of each).  This returns a bool array [B, Hq, q_len]: True where some later sub-block's
    maximum exceeds the first one's by more than 64 ln 2 + 1, which forces at least one
    rescale of a non-empty accumulator (the first such sub-block triggers unless an earlier
    one already did).  q: [B, Hq, T, D]; kp: [P, Hkv, bs, D]; idx: [B, Hkv, T, k]."""
    B, Hq, T, D = q.shape
    thr = 64.0 * math.log(2.0) + 1.0
    res = np.zeros((B, Hq, T), bool)
    for b in range(B):
        L = kv[b]
        nb = (L + page_size - 1) // page_size
        pos = np.arange(L - T, L)
        for g in range(Hq // group_size):
            keys = kp[pt[b, :nb], g].reshape(nb * page_size, D)[:L].astype(np.float64)
            selm = np.zeros((T, nb), bool)
            for s in range(idx.shape[3]):
                j = idx[b, g, :, s]
                ok = j >= 0
                selm[np.nonzero(ok)[0], j[ok]] = True
            keep = np.repeat(selm, page_size, axis=1)[:, :L] & (np.arange(L)[None, :] <= pos[:, None])
            nsub = (L + sub - 1) // sub
            for h in range(g * group_size, (g + 1) * group_size):
                z = (q[b, h].astype(np.float64) @ keys.T) * scale
                z = np.where(keep, z, -np.inf)
                zp = np.full((T, nsub * sub), -np.inf)
                zp[:, :L] = z
                m = zp.reshape(T, nsub, sub).max(-1)                     # [T, nsub]
                fin = np.isfinite(m)
                first = np.argmax(fin, axis=1)
                m0 = m[np.arange(T), first]
                later = np.where(np.arange(nsub)[None, :] > first[:, None], m, -np.inf).max(1)
                res[b, h] = fin.any(1) & (later - m0 > thr)
    return res
