"""CPU oracle for block-sparse GQA attention over a pooled, page-aware block cache.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain reference that the
GPU library is checked against.  Only the test suite, the package smoke check
and the benchmark's CPU-baseline leg may import it; the library itself never
does, and it shares no code with the library (no kernels, headers, tables or
helpers).  Inputs are numpy arrays (values as float32/float64, tables as
int32); nothing here knows about torch or the GPU.

What is computed, with the passage each step follows:

1. Block representatives ("Art of Focus: Ling 2.0 and the Revolution in Sparse
   Attention", section "Summarizing the Breakthrough": at prefill the tokens of
   a block are aggregated into one representative that lives in a cache keyed
   like the paged KV cache).  The aggregate is the arithmetic mean of the
   block's keys per KV head.  Block size = page size, so the representative of
   a logical block is stored at the block's physical page id.
2. Group scores (same page, same section: the query heads of a GQA group share
   one block selection; "MiniMax Sparse Attention (MSA)" post, second
   paragraph: the index branch scores KV blocks and picks a top-k subset per
   GQA group).  Score of block j for query token t of group g =
   sum over the group's heads h of q[h, t] . rep[j, g]  (unscaled logits).
3. Causal top-k (MSA post, second and third paragraphs: top-k per group,
   ranked without any exponential).  Candidates are the blocks strictly before
   the query's own block; the own block is always kept and counts toward k;
   ranking is by score, higher first, equal scores keep the lower block index;
   the kept list is sorted ascending and padded with -1.
4. Exact attention over the selected blocks ("Sparse Attention + Linear
   Backbones", section 5.5 "Pseudocode Sketch": softmax of q.k/sqrt(d) over the
   selected keys, then times the selected values; "Sparse Attention for
   Long-Context LLMs: Evolution and Practical Deployment", section 4.3: the
   top-k mask restricts the softmax, read here as an additive minus-infinity
   mask, i.e. the unselected keys do not take part).  Inside the own block a
   key takes part only if its position is at most the query's position.
5. Gated fusion (optional; "Sparse Attention for Long-Context LLMs", section
   4.3 "Gating Mechanisms Reduce Risk", step 6: the final output is the gate times the attention output plus
   one minus the gate times the original representation, the gate being a
   scalar or a vector per dimension).  Here the gate and the other tensor are
   caller inputs: out = g * A + (1 - g) * x, in float64.
6. fp8 KV cache and block cache (optional; "Sparse Attention + Linear
   Backbones", section 3, and "Sparse Attention for Long-Context LLMs",
   section 8, list KV-cache quantization as a system-level optimisation to
   combine with sparse attention; neither fixes a format).  Reading taken
   here: OCP E4M3 codes with one power-of-two scale per (page, KV head) tile,
   the smallest power of two 2^e with max|x| <= 448 * 2^e over the tile's
   valid tokens; codes are x / 2^e rounded to nearest, ties to even; slots
   past the sequence length hold code 0.  The fp8 block cache is built from
   the fp8 keys: the float32 sum of the decoded codes in token order, times
   scale / page_size, quantised the same way per (page, head).  Attention and
   scores then run on the decoded values (code value times scale), exactly as
   steps 2-4 on a float cache.
7. Token-level selection (optional; "Sparse Attention + Linear Backbones",
   sections 5.1-5.3 and the pseudocode of 5.5: an indexer scores every
   earlier position, the 2048 highest-scoring positions are kept per query,
   attention runs over those; the indexer uses no positional encoding).  The
   learned indexer is absent, so the index is the identity one: the score of
   token s for the query heads of group g is the sum over the group's heads of
   q . k_s (the block score of step 2 at granularity one).  Candidates are the
   tokens at or before the query's position; the top K are kept by (score,
   lower index first), sorted ascending, padded with -1; attention is exact
   over the kept tokens.
8. Two-level selection (optional; "Sparse Attention for Long-Context LLMs",
   section 8: coarse filtering followed by fine filtering): the block top-k of
   step 3, then the token top-K of step 7 among the tokens of the kept blocks
   (causal inside the own block), then attention over the kept tokens.

Precision: attention and scores are computed in float64.  Two results are
codes decided by floating point, and those decisions are taken in the
library's own precision: the block-cache entry (float32 sum of the block's
keys in token order, times 1/page_size, then rounded to nearest-even into the
cache dtype) and the block ranking (float64 score rounded to float32, then
ordered by (-score, index)).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "bf16_bits", "bf16_value", "round_to_cache", "gather_tokens", "block_pool",
    "query_positions", "group_scores", "select_blocks",
    "sparse_attention", "prefill_reference", "decode_reference", "gated_fusion",
    "e4m3_value", "e4m3_code", "fp8_scale_exp", "quantize_pages_fp8", "fp8_dequant", "block_pool_fp8",
    "token_scores", "select_tokens", "token_attention", "decode_tokens_reference", "two_level_decode_reference",
]


# ----------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even) on the float32 bit pattern
# ----------------------------------------------------------------------------
def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 code (uint16) of float32 values (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """float32 value of bf16 codes."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_cache(x32: np.ndarray, cache_dtype: str) -> np.ndarray:
    """float32 array -> values representable in the cache dtype (as float32)."""
    if cache_dtype == "f32":
        return np.asarray(x32, dtype=np.float32)
    if cache_dtype == "bf16":
        return bf16_value(bf16_bits(x32))
    raise ValueError(cache_dtype)


# ----------------------------------------------------------------------------
# paged layout helpers
# ----------------------------------------------------------------------------
def gather_tokens(pages: np.ndarray, pt_row: np.ndarray, n_tokens: int) -> np.ndarray:
    """Logical tokens [Hkv, n_tokens, D] of one sequence from a paged pool.

    ``pages``: [P, Hkv, bs, D]; logical block j lives in page ``pt_row[j]``.
    """
    P, Hkv, bs, D = pages.shape
    nblk = (n_tokens + bs - 1) // bs
    sel = pages[np.asarray(pt_row[:nblk], dtype=np.int64)]        # [nblk, Hkv, bs, D]
    return sel.transpose(1, 0, 2, 3).reshape(Hkv, nblk * bs, D)[:, :n_tokens]


def query_positions(kv_len: int, q_len: int, t_idx: Optional[Sequence[int]] = None) -> np.ndarray:
    """Position of query t: kv_len - q_len + t (the newest query is last)."""
    t = np.arange(q_len) if t_idx is None else np.asarray(t_idx, dtype=np.int64)
    return kv_len - q_len + t


# ----------------------------------------------------------------------------
# 1. block representatives
# ----------------------------------------------------------------------------
def block_pool(k_pages: np.ndarray, page_table: np.ndarray, kv_lens: Sequence[int],
               cache_dtype: str, blk_begin: Optional[Sequence[int]] = None,
               block_cache: Optional[np.ndarray] = None) -> np.ndarray:
    """Mean of each complete block's keys, per KV head, into the block cache.

    For sequence b and each complete logical block j in [blk_begin[b],
    kv_len[b] // bs): ``cache[page_table[b, j], g, :]`` = round_to_cache(
    (K[tok 0] + K[tok 1] + ... + K[tok bs-1]) * (1/bs)), the sum taken in
    float32 in token order.  Entries of other pages are left as they were
    (zero for a fresh cache).  Returns the block cache [P, Hkv, D] (float32
    values, representable in ``cache_dtype``).
    """
    P, Hkv, bs, D = k_pages.shape
    out = np.zeros((P, Hkv, D), np.float32) if block_cache is None else np.array(block_cache, np.float32)
    inv = np.float32(1.0 / bs)
    for b, L in enumerate(kv_lens):
        begin = 0 if blk_begin is None else int(blk_begin[b])
        end = int(L) // bs
        if end <= begin:
            continue
        phys = np.asarray(page_table[b, begin:end], dtype=np.int64)
        keys = np.asarray(k_pages[phys], dtype=np.float32)            # [n, Hkv, bs, D]
        acc = np.zeros((len(phys), Hkv, D), np.float32)
        for i in range(bs):                                           # token order
            acc = acc + keys[:, :, i, :]
        out[phys] = round_to_cache(acc * inv, cache_dtype)
    return out


# ----------------------------------------------------------------------------
# 2. group scores
# ----------------------------------------------------------------------------
def group_scores(q: np.ndarray, block_cache: np.ndarray, page_table: np.ndarray,
                 kv_lens: Sequence[int], num_kv_heads: int, page_size: int,
                 t_idx: Optional[Sequence[int]] = None) -> np.ndarray:
    """Scores [B, Hkv, T, nb_max] in float64; -inf where j is not a candidate.

    q: [B, Hq, q_len, D].  Candidates of a query at position p are the blocks
    j < p // page_size, i.e. strictly before its own block.
    """
    B, Hq, q_len, D = q.shape
    G = Hq // num_kv_heads
    nb_max = page_table.shape[1]
    T = q_len if t_idx is None else len(t_idx)
    out = np.full((B, num_kv_heads, T, nb_max), -np.inf, np.float64)
    tsel = np.arange(q_len) if t_idx is None else np.asarray(t_idx, dtype=np.int64)
    for b in range(B):
        pos = query_positions(int(kv_lens[b]), q_len, tsel)
        own = pos // page_size
        nb = int(own.max()) if T else 0
        if nb == 0:
            continue
        reps = np.asarray(block_cache[np.asarray(page_table[b, :nb], np.int64)], np.float64)  # [nb, Hkv, D]
        for g in range(num_kv_heads):
            qs = np.asarray(q[b, g * G:(g + 1) * G][:, tsel], np.float64).sum(axis=0)   # [T, D]
            s = qs @ reps[:, g, :].T                                                   # [T, nb]
            cand = np.arange(nb)[None, :] < own[:, None]
            out[b, g, :, :nb] = np.where(cand, s, -np.inf)
    return out


# ----------------------------------------------------------------------------
# 3. causal top-k per group
# ----------------------------------------------------------------------------
def select_blocks(scores: np.ndarray, kv_lens: Sequence[int], q_len: int, page_size: int,
                  top_k: int, t_idx: Optional[Sequence[int]] = None) -> np.ndarray:
    """Selected logical blocks [B, Hkv, T, top_k] (int32, ascending, -1 padded).

    ``scores`` as returned by :func:`group_scores` for the same ``t_idx``.  The
    ranking is decided on the float32 rounding of the scores: order by score
    (higher first), equal scores by block index (lower first); keep the first
    min(top_k - 1, own) candidates, then add the own block.
    """
    B, Hkv, T, nb_max = scores.shape
    s32 = scores.astype(np.float32)
    out = np.full((B, Hkv, T, top_k), -1, np.int32)
    tsel = np.arange(q_len) if t_idx is None else np.asarray(t_idx, dtype=np.int64)
    for b in range(B):
        own = query_positions(int(kv_lens[b]), q_len, tsel) // page_size        # [T]
        # stable sort of -score: descending score, ascending index among equals;
        # non-candidates (-inf) end up last
        order = np.argsort(-s32[b], axis=-1, kind="stable")                     # [Hkv, T, nb]
        m = top_k - 1
        if m > 0:
            top = order[..., :m] if nb_max >= m else np.concatenate(
                [order, np.full(order.shape[:-1] + (m - nb_max,), np.iinfo(np.int64).max)], axis=-1)
            valid = top < own[None, :, None]
            sel = np.where(valid, top, np.iinfo(np.int64).max)
        else:
            sel = np.zeros((Hkv, T, 0), np.int64)
        full = np.concatenate([sel, np.broadcast_to(own[None, :, None], (Hkv, T, 1))], axis=-1)
        full = np.sort(full, axis=-1)
        full = np.where(full == np.iinfo(np.int64).max, -1, full)
        out[b] = full.astype(np.int32)
    return out


# ----------------------------------------------------------------------------
# 4. exact attention over the selected blocks
# ----------------------------------------------------------------------------
def sparse_attention(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray, page_table: np.ndarray,
                     kv_lens: Sequence[int], block_idx: np.ndarray, scale: float,
                     t_idx: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(out [B, Hq, T, D], lse [B, Hq, T]) in float64.

    ``block_idx`` [B, Hkv, T, k] for the same ``t_idx``.  For query head h of
    group g = h // G at position p: z_i = (q . k_i) * scale over the selected
    keys i, out = sum_i softmax(z)_i v_i, lse = max z + log(sum exp(z - max z)).
    Only the pages of the selected blocks are read.
    """
    B, Hq, q_len, D = q.shape
    _, Hkv, bs, _ = k_pages.shape
    G = Hq // Hkv
    tsel = np.arange(q_len) if t_idx is None else np.asarray(t_idx, dtype=np.int64)
    T = len(tsel)
    out = np.zeros((B, Hq, T, D), np.float64)
    lse = np.full((B, Hq, T), -np.inf, np.float64)
    for b in range(B):
        L = int(kv_lens[b])
        pos_all = query_positions(L, q_len, tsel)
        for g in range(Hkv):
            for ti in range(T):
                pos = int(pos_all[ti])
                Ks, Vs = [], []
                for j in block_idx[b, g, ti]:
                    j = int(j)
                    if j < 0:
                        continue
                    n = min(bs, pos - j * bs + 1)          # keys of block j at positions <= pos
                    if n <= 0:
                        continue
                    page = int(page_table[b, j])
                    Ks.append(np.asarray(k_pages[page, g, :n], np.float64))
                    Vs.append(np.asarray(v_pages[page, g, :n], np.float64))
                if not Ks:
                    continue
                K = np.concatenate(Ks)
                V = np.concatenate(Vs)
                qh = np.asarray(q[b, g * G:(g + 1) * G, tsel[ti]], np.float64)   # [G, D]
                z = (qh @ K.T) * scale                                           # [G, n]
                m = z.max(axis=1, keepdims=True)
                w = np.exp(z - m)
                l = w.sum(axis=1, keepdims=True)
                out[b, g * G:(g + 1) * G, ti] = (w @ V) / l
                lse[b, g * G:(g + 1) * G, ti] = (m + np.log(l))[:, 0]
    return out, lse


# ----------------------------------------------------------------------------
# whole path
# ----------------------------------------------------------------------------
def prefill_reference(q, k_pages, v_pages, page_table, kv_lens, page_size, top_k, cache_dtype,
                      scale: Optional[float] = None, t_idx=None):
    """Block pool -> group scores -> top-k -> sparse attention, for the queries
    ``t_idx`` (default all).  Returns dict(block_cache, scores, block_idx, out, lse)."""
    B, Hq, q_len, D = q.shape
    Hkv = k_pages.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    cache = block_pool(k_pages, page_table, kv_lens, cache_dtype)
    sc = group_scores(q, cache, page_table, kv_lens, Hkv, page_size, t_idx)
    idx = select_blocks(sc, kv_lens, q_len, page_size, top_k, t_idx)
    out, lse = sparse_attention(q, k_pages, v_pages, page_table, kv_lens, idx, scale, t_idx)
    return dict(block_cache=cache, scores=sc, block_idx=idx, out=out, lse=lse)


def decode_reference(q, k_pages, v_pages, page_table, kv_lens, page_size, top_k, cache_dtype,
                     scale: Optional[float] = None, block_cache=None):
    """One decode step (q_len = 1).  The block cache holds every complete block
    of each sequence; it is built here unless given."""
    if block_cache is None:
        block_cache = block_pool(k_pages, page_table, kv_lens, cache_dtype)
    B, Hq, q_len, D = q.shape
    Hkv = k_pages.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    sc = group_scores(q, block_cache, page_table, kv_lens, Hkv, page_size)
    idx = select_blocks(sc, kv_lens, q_len, page_size, top_k)
    out, lse = sparse_attention(q, k_pages, v_pages, page_table, kv_lens, idx, scale)
    return dict(block_cache=block_cache, scores=sc, block_idx=idx, out=out, lse=lse)


# ----------------------------------------------------------------------------
# 5. gated fusion

def gated_fusion(a: np.ndarray, gate: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Gate * A + (1 - Gate) * X ("Sparse Attention for Long-Context LLMs", section 4.3,
    step 6), in float64.  ``a`` and ``x`` have the output's shape [..., D]; ``gate`` has
    that shape (one gate per dimension) or that shape without the last axis (one gate per
    row, broadcast over D)."""
    a = np.asarray(a, np.float64)
    x = np.asarray(x, np.float64)
    g = np.asarray(gate, np.float64)
    if g.shape == a.shape[:-1]:
        g = g[..., None]
    elif g.shape != a.shape:
        raise ValueError("gate must have the output's shape or the output's shape without D")
    return g * a + (1.0 - g) * x


# ----------------------------------------------------------------------------
# 6. fp8 (OCP E4M3) KV cache and block cache
# ----------------------------------------------------------------------------
def e4m3_value(codes) -> np.ndarray:
    """float64 value of OCP E4M3 codes: sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN; no infinities."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


_E4M3_MAG = e4m3_value(np.arange(127, dtype=np.uint8))     # codes 0x00..0x7E: 0 .. 448, ascending


def e4m3_code(x) -> np.ndarray:
    """Nearest E4M3 code of finite |x| <= 448, ties to the even code (the code's last bit is
    the mantissa's last bit).  The sign bit follows the sign of x, -0.0 included."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    if not np.all(np.isfinite(a)) or np.any(a > 448.0):
        raise ValueError("e4m3_code takes finite values of magnitude <= 448")
    hi = np.minimum(np.searchsorted(_E4M3_MAG, a, side="left"), 126)   # first magnitude >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _E4M3_MAG[lo], _E4M3_MAG[hi] - a
    pick = np.where(d_hi == 0, hi, np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi))))
    return (pick | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def fp8_scale_exp(amax):
    """Smallest integer e with amax <= 448 * 2^e (0 for amax = 0), clamped to [-126, 127];
    elementwise for arrays.  With amax = f * 2^E, 0.5 <= f < 1, and 448 = 0.875 * 2^9:
    e = E - 9 if f <= 0.875, else E - 8."""
    a = np.asarray(amax, np.float64)
    f, E = np.frexp(a)
    e = np.where(f <= 0.875, E - 9, E - 8)
    e = np.clip(np.where(a == 0.0, 0, e), -126, 127).astype(np.int64)
    return int(e) if e.ndim == 0 else e


def _quantize_tiles(x: np.ndarray, axes) -> Tuple[np.ndarray, np.ndarray]:
    """Codes and exponents of tiles: one scale per index of the axes not in ``axes``."""
    e = fp8_scale_exp(np.abs(x).max(axis=axes))
    codes = e4m3_code(x / np.exp2(np.expand_dims(e, axes).astype(np.float64)))
    return codes, e


def quantize_pages_fp8(pages: np.ndarray, page_table: np.ndarray, kv_lens: Sequence[int],
                       page_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """(codes uint8 [P, Hkv, bs, D], scales float32 [P, Hkv]) of a paged cache [P, Hkv, bs, D].

    Every (page, head) tile of every sequence's blocks j < ceil(kv_len / bs) is quantised
    over its valid tokens n = min(bs, kv_len - j bs): scale 2^e with e = fp8_scale_exp of
    the tile's max |x|, codes e4m3_code(x / 2^e), code 0 past n.  Tiles no sequence
    reaches keep code 0 and scale 1."""
    P, Hkv, bs, D = pages.shape
    codes = np.zeros((P, Hkv, bs, D), np.uint8)
    scales = np.ones((P, Hkv), np.float32)
    for b, L in enumerate(kv_lens):
        L = int(L)
        nblk = min((L + bs - 1) // bs, page_table.shape[1])
        nfull = min(L // bs, nblk)
        for j0 in range(0, nfull, 1024):                          # complete pages, in chunks
            phys = np.asarray(page_table[b, j0:min(nfull, j0 + 1024)], np.int64)
            c, e = _quantize_tiles(np.asarray(pages[phys], np.float64), (2, 3))
            codes[phys] = c
            scales[phys] = np.exp2(e.astype(np.float64))
        if nblk > nfull:                                          # the partial last page
            p, n = int(page_table[b, nfull]), L - nfull * bs
            c, e = _quantize_tiles(np.asarray(pages[p, :, :n], np.float64), (1, 2))
            codes[p] = 0
            codes[p, :, :n] = c
            scales[p] = np.exp2(e.astype(np.float64))
    return codes, scales


def fp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decoded values e4m3_value(code) * scale of the code's (page, head), as float32 (exact:
    an E4M3 value times a power of two).  ``codes`` [P, Hkv, ..., D], ``scales`` [P, Hkv]."""
    v = e4m3_value(codes)
    return (v * np.asarray(scales, np.float64).reshape(scales.shape + (1,) * (v.ndim - 2))).astype(np.float32)


def block_pool_fp8(k_codes: np.ndarray, k_scales: np.ndarray, page_table: np.ndarray,
                   kv_lens: Sequence[int], blk_begin: Optional[Sequence[int]] = None,
                   rep_codes: Optional[np.ndarray] = None, rep_scales: Optional[np.ndarray] = None
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """fp8 block cache (codes uint8 [P, Hkv, D], scales float32 [P, Hkv]) of the complete
    blocks j in [blk_begin[b], kv_len // bs): the float32 sum of the block's decoded key
    codes in token order, times (scale / bs) in float32, quantised per (page, head) like the
    KV cache.  Other pages keep the given (or zero / unit) entries."""
    P, Hkv, bs, D = k_codes.shape
    rc = np.zeros((P, Hkv, D), np.uint8) if rep_codes is None else np.array(rep_codes, np.uint8)
    rs = np.ones((P, Hkv), np.float32) if rep_scales is None else np.array(rep_scales, np.float32)
    for b, L in enumerate(kv_lens):
        begin = 0 if blk_begin is None else int(blk_begin[b])
        end = min(int(L) // bs, page_table.shape[1])
        for j0 in range(begin, end, 1024):
            phys = np.asarray(page_table[b, j0:min(end, j0 + 1024)], np.int64)
            vals = e4m3_value(k_codes[phys]).astype(np.float32)           # [n, Hkv, bs, D], exact
            acc = np.zeros((len(phys), Hkv, D), np.float32)
            for i in range(bs):                                           # token order
                acc = acc + vals[:, :, i, :]
            mean = acc * (np.asarray(k_scales[phys], np.float32) * np.float32(1.0 / bs))[:, :, None]
            c, e = _quantize_tiles(mean.astype(np.float64), (2,))
            rc[phys] = c
            rs[phys] = np.exp2(e.astype(np.float64))
    return rc, rs


# ----------------------------------------------------------------------------
# 7. token-level selection, 8. two-level selection
# ----------------------------------------------------------------------------
def token_scores(q: np.ndarray, k_pages: np.ndarray, page_table: np.ndarray, kv_lens: Sequence[int],
                 t_idx: Optional[Sequence[int]] = None, block_idx: Optional[np.ndarray] = None) -> np.ndarray:
    """Scores [B, Hkv, T, L_max] in float64 (L_max = longest sequence): for query t of group g
    at position p, scores[.., s] = sum over the group's heads h of q[h, t] . k[s] for the
    candidate tokens s, -inf elsewhere.  Candidates: s <= p; with ``block_idx``
    [B, Hkv, T, k] (two-level selection) only the tokens of the listed blocks."""
    B, Hq, q_len, D = q.shape
    _, Hkv, bs, _ = k_pages.shape
    G = Hq // Hkv
    tsel = np.arange(q_len) if t_idx is None else np.asarray(t_idx, dtype=np.int64)
    T = len(tsel)
    Lmax = int(max(kv_lens))
    out = np.full((B, Hkv, T, Lmax), -np.inf, np.float64)
    for b in range(B):
        L = int(kv_lens[b])
        keys = gather_tokens(k_pages, page_table[b], L).astype(np.float64)      # [Hkv, L, D]
        pos = query_positions(L, q_len, tsel)
        for g in range(Hkv):
            qs = np.asarray(q[b, g * G:(g + 1) * G][:, tsel], np.float64).sum(axis=0)   # [T, D]
            sc = qs @ keys[g].T                                                    # [T, L]
            cand = np.arange(L)[None, :] <= pos[:, None]
            if block_idx is not None:
                inblk = np.zeros((T, L), bool)
                for ti in range(T):
                    for j in block_idx[b, g, ti]:
                        if j >= 0:
                            inblk[ti, int(j) * bs:min(L, (int(j) + 1) * bs)] = True
                cand &= inblk
            out[b, g, :, :L] = np.where(cand, sc, -np.inf)
    return out


def select_tokens(scores: np.ndarray, top_k: int) -> np.ndarray:
    """Kept tokens [B, Hkv, T, top_k] (int32, ascending, -1 padded): the top_k candidates
    (finite scores) by score, higher first, equal scores lower index first, decided on the
    float32 rounding of the scores."""
    B, Hkv, T, L = scores.shape
    s32 = scores.astype(np.float32)
    out = np.full((B, Hkv, T, top_k), -1, np.int32)
    for b in range(B):
        for g in range(Hkv):
            for t in range(T):
                row = s32[b, g, t]
                cand = np.nonzero(np.isfinite(row))[0]
                order = cand[np.lexsort((cand, -row[cand]))]                        # score desc, index asc
                keep = np.sort(order[:top_k])
                out[b, g, t, :len(keep)] = keep
    return out


def token_attention(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray, page_table: np.ndarray,
                    kv_lens: Sequence[int], token_idx: np.ndarray, scale: float,
                    t_idx: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(out [B, Hq, T, D], lse [B, Hq, T]) in float64: softmax((q . k_s) * scale) over the
    kept tokens s of ``token_idx`` [B, Hkv, T, K] (the query's group), times v_s."""
    B, Hq, q_len, D = q.shape
    _, Hkv, bs, _ = k_pages.shape
    G = Hq // Hkv
    tsel = np.arange(q_len) if t_idx is None else np.asarray(t_idx, dtype=np.int64)
    T = len(tsel)
    out = np.zeros((B, Hq, T, D), np.float64)
    lse = np.full((B, Hq, T), -np.inf, np.float64)
    for b in range(B):
        L = int(kv_lens[b])
        keys = gather_tokens(k_pages, page_table[b], L).astype(np.float64)
        vals = gather_tokens(v_pages, page_table[b], L).astype(np.float64)
        for g in range(Hkv):
            for ti in range(T):
                sel = np.asarray([int(x) for x in token_idx[b, g, ti] if x >= 0], np.int64)
                if sel.size == 0:
                    continue
                qh = np.asarray(q[b, g * G:(g + 1) * G, tsel[ti]], np.float64)      # [G, D]
                z = (qh @ keys[g, sel].T) * scale
                m = z.max(axis=1, keepdims=True)
                w = np.exp(z - m)
                l = w.sum(axis=1, keepdims=True)
                out[b, g * G:(g + 1) * G, ti] = (w @ vals[g, sel]) / l
                lse[b, g * G:(g + 1) * G, ti] = (m + np.log(l))[:, 0]
    return out, lse


def decode_tokens_reference(q, k_pages, v_pages, page_table, kv_lens, top_k_tokens: int,
                            scale: Optional[float] = None):
    """Token-level decode step (q_len = 1): token scores -> token top-K -> attention.
    Returns dict(scores, token_idx, out, lse)."""
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    sc = token_scores(q, k_pages, page_table, kv_lens)
    idx = select_tokens(sc, top_k_tokens)
    out, lse = token_attention(q, k_pages, v_pages, page_table, kv_lens, idx, scale)
    return dict(scores=sc, token_idx=idx, out=out, lse=lse)


def two_level_decode_reference(q, k_pages, v_pages, page_table, kv_lens, page_size, top_k_blocks: int,
                               top_k_tokens: int, cache_dtype, scale: Optional[float] = None, block_cache=None):
    """Two-level decode step (q_len = 1): block scores -> block top-k (steps 1-3) -> token
    scores over the kept blocks' tokens -> token top-K -> attention.  Returns dict(block_cache,
    block_scores, block_idx, scores, token_idx, out, lse)."""
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    Hkv = k_pages.shape[1]
    if block_cache is None:
        block_cache = block_pool(k_pages, page_table, kv_lens, cache_dtype)
    bsc = group_scores(q, block_cache, page_table, kv_lens, Hkv, page_size)
    bidx = select_blocks(bsc, kv_lens, 1, page_size, top_k_blocks)
    sc = token_scores(q, k_pages, page_table, kv_lens, block_idx=bidx)
    idx = select_tokens(sc, top_k_tokens)
    out, lse = token_attention(q, k_pages, v_pages, page_table, kv_lens, idx, scale)
    return dict(block_cache=block_cache, block_scores=bsc, block_idx=bidx, scores=sc, token_idx=idx, out=out,
                lse=lse)
