"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test ties one oracle step to an independent fact: a hand-derived worked
example, a library routine (torch's bf16 cast, torch's scaled-dot-product
attention), brute-force enumeration, a closed form, or an invariant the
method fixes.  None of these tests touches the GPU.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from workloads import SPECS, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(w):
    """Workload tensors as numpy (bf16 values widened exactly to float32)."""
    return (w.q.float().numpy(), w.k_cache.float().numpy(), w.v_cache.float().numpy(),
            w.page_table.numpy(), list(w.kv_lens_host))


def _eval(expr):
    ns = {"exp": math.exp, "sqrt": math.sqrt, "log": math.log}
    return float(eval(expr, {"__builtins__": {}}, ns))  # noqa: S307 (own fixture, math only)


# --------------------------------------------------------------------------
# worked example (hand-derived; tests/golden/tiny_worked_example.json)
# --------------------------------------------------------------------------
def _golden_inputs():
    with open(os.path.join(GOLDEN, "tiny_worked_example.json")) as f:
        g = json.load(f)
    sh = g["shape"]
    bs, D = sh["page_size"], sh["head_dim"]
    K = np.array(g["keys"], np.float32)
    V = np.array(g["values"], np.float32)
    S = K.shape[0]
    nb = S // bs
    # shuffled physical placement: logical block j -> page perm[j]
    perm = np.array([2, 0, 1], np.int32)
    kp = np.zeros((nb, 1, bs, D), np.float32)
    vp = np.zeros((nb, 1, bs, D), np.float32)
    for j in range(nb):
        kp[perm[j], 0] = K[j * bs:(j + 1) * bs]
        vp[perm[j], 0] = V[j * bs:(j + 1) * bs]
    q = np.stack([np.array(g["queries"]["head0"], np.float32),
                  np.array(g["queries"]["head1"], np.float32)])[None]        # [1, 2, S, D]
    return g, q, kp, vp, perm[None, :], [S]


def test_golden_worked_example_all_steps():
    g, q, kp, vp, pt, kv = _golden_inputs()
    sh = g["shape"]
    bs = sh["page_size"]
    cache = O.block_pool(kp, pt, kv, "f32")
    reps = cache[pt[0], 0]                                  # logical order
    np.testing.assert_array_equal(reps, np.array(g["block_reps"], np.float32))

    sc = O.group_scores(q, cache, pt, kv, 1, bs)
    for t, d in g["scores"].items():
        if t == "note":
            continue
        t = int(t)
        for j, v in d.items():
            assert sc[0, 0, t, int(j)] == v
        own = t // bs
        assert np.all(np.isneginf(sc[0, 0, t, own:]))

    idx = O.select_blocks(sc, kv, sh["seq_len"], bs, sh["top_k"])
    np.testing.assert_array_equal(idx[0, 0], np.array(g["selected"], np.int32))

    out, lse = O.sparse_attention(q, kp, vp, pt, kv, idx, 1.0 / math.sqrt(sh["head_dim"]))
    for h, key in enumerate(["head0", "head1"]):
        for t in range(sh["seq_len"]):
            ex = _eval(g["out_x"][key][t])
            assert out[0, h, t, 0] == pytest.approx(ex, rel=1e-13, abs=1e-13)
            assert out[0, h, t, 1] == pytest.approx(-ex, rel=1e-13, abs=1e-13)
            assert lse[0, h, t] == pytest.approx(_eval(g["lse"][key][t]), rel=1e-13, abs=1e-13)


def test_golden_token0_output_is_first_value_exactly():
    g, q, kp, vp, pt, kv = _golden_inputs()
    idx = np.array(g["selected"], np.int32)[None, None]
    out, _ = O.sparse_attention(q, kp, vp, pt, kv, idx, 0.7)
    assert np.all(out[0, :, 0] == vp[pt[0, 0], 0, 0])


# --------------------------------------------------------------------------
# bf16 rounding against hand-worked codes and torch's own cast
# --------------------------------------------------------------------------
def test_bf16_rounding_hand_codes():
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2.0 ** -8, 0x3F80),                 # exact tie -> even (down)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),             # exact tie -> even (up)
        (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),    # just above the tie
        (-2.5, 0xC020),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (3.0e38, 0x7F62),
    ]
    x = np.array([c[0] for c in cases], np.float32)
    got = O.bf16_bits(x)
    assert [int(v) for v in got] == [c[1] for c in cases]


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32),
                        (rng.standard_normal(20000) * 1e-30).astype(np.float32),
                        (rng.standard_normal(20000) * 1e30).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.bf16_bits(x), ref)


# --------------------------------------------------------------------------
# block representatives
# --------------------------------------------------------------------------
def test_block_pool_identical_rows_give_that_row():
    rng = np.random.default_rng(1)
    bs, D, Hkv, P = 64, 128, 2, 3
    row = O.round_to_cache(rng.standard_normal((P, Hkv, 1, D)).astype(np.float32), "bf16")
    kp = np.repeat(row, bs, axis=2)
    pt = np.array([[0, 1, 2]], np.int32)
    for dt in ("f32", "bf16"):
        c = O.block_pool(kp, pt, [3 * bs], dt)
        np.testing.assert_array_equal(c, row[:, :, 0])


def test_block_pool_close_to_exact_mean_and_rounded_once():
    w = make_workload(SPECS[1].replace(seq_len=2048 + 37), 3)   # bf16, ragged tail
    q, kp, vp, pt, kv = _np(w)
    bs = w.spec.page_size
    f32c = O.block_pool(kp, pt, kv, "f32")
    b16c = O.block_pool(kp, pt, kv, "bf16")
    nfull = kv[0] // bs
    phys = pt[0, :nfull].astype(np.int64)
    exact = kp[phys].astype(np.float64).mean(axis=2)                          # [n, Hkv, D]
    bound = bs * 2.0 ** -24 * np.abs(kp[phys]).astype(np.float64).mean(axis=2) * 2
    assert np.all(np.abs(f32c[phys] - exact) <= bound)
    # bf16 cache = nearest-even rounding of the float32 mean
    np.testing.assert_array_equal(b16c[phys], O.bf16_value(O.bf16_bits(f32c[phys])))
    # and therefore within half a bf16 ulp (+ the float32 error) of the exact mean
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
    assert np.all(np.abs(b16c[phys] - exact) <= 0.5 * ulp + bound + 1e-30)
    # the incomplete tail block is not written
    assert kv[0] % bs != 0
    assert np.all(b16c[pt[0, nfull]] == 0)


def test_block_pool_begin_and_page_table_invariance():
    spec = SPECS[2].replace(batch=3, ctx_len=64 * 9 + 5, num_q_heads=8, num_kv_heads=2, head_dim=64)
    w = make_workload(spec, 11)
    q, kp, vp, pt, kv = _np(w)
    full = O.block_pool(kp, pt, kv, "bf16")
    # incremental: first the blocks before 4, then the rest
    part = O.block_pool(kp, pt, [4 * 64] * 3, "bf16")
    part = O.block_pool(kp, pt, kv, "bf16", blk_begin=[4, 4, 4], block_cache=part)
    np.testing.assert_array_equal(part, full)
    # logical representatives do not depend on where the pages sit
    wi = make_workload(spec.replace(shuffle_pages=False), 11)
    qi, kpi, vpi, pti, kvi = _np(wi)
    fi = O.block_pool(kpi, pti, kvi, "bf16")
    for b in range(3):
        n = kv[b] // 64
        np.testing.assert_array_equal(full[pt[b, :n]], fi[pti[b, :n]])


# --------------------------------------------------------------------------
# group scores
# --------------------------------------------------------------------------
def test_scores_equal_block_mean_of_dense_group_logits():
    """Linearity: sum_h q_h . mean(K_block) = mean over the block of the dense
    group logits sum_h q_h . k_i (computed with torch's matmul over all keys)."""
    w = make_workload(SPECS[0].replace(seq_len=640 + 17), 5)
    q, kp, vp, pt, kv = _np(w)
    bs, Hkv, G = 64, 2, 4
    L = kv[0]
    nfull = L // bs
    exact_cache = np.zeros((kp.shape[0], Hkv, kp.shape[3]), np.float64)
    exact_cache[pt[0, :nfull]] = kp[pt[0, :nfull]].astype(np.float64).mean(axis=2)
    sc = O.group_scores(q, exact_cache, pt, kv, Hkv, bs)
    K = torch.from_numpy(O.gather_tokens(kp, pt[0], L).astype(np.float64))       # [Hkv, L, D]
    Q = torch.from_numpy(q[0].astype(np.float64))                                # [Hq, L, D]
    for g in range(Hkv):
        logits = torch.matmul(Q[g * G:(g + 1) * G], K[g].T).sum(0)                # [L, L]
        blk = logits[:, :nfull * bs].reshape(L, nfull, bs).mean(-1).numpy()
        for t in range(L):
            own = t // bs
            np.testing.assert_allclose(sc[0, g, t, :own], blk[t, :own], rtol=1e-10, atol=1e-9)
            assert np.all(np.isneginf(sc[0, g, t, own:]))


def test_scores_group_of_one_is_per_head_dot():
    w = make_workload(SPECS[0].replace(num_q_heads=2, num_kv_heads=2, seq_len=300), 6)
    q, kp, vp, pt, kv = _np(w)
    cache = O.block_pool(kp, pt, kv, "f32")
    sc = O.group_scores(q, cache, pt, kv, 2, 64, t_idx=[299])
    for h in range(2):
        for j in range(299 // 64):
            ref = float(np.dot(q[0, h, 299].astype(np.float64), cache[pt[0, j], h].astype(np.float64)))
            assert sc[0, h, 0, j] == pytest.approx(ref, rel=1e-12)


def test_scores_and_selection_invariant_to_head_order_within_group():
    w = make_workload(SPECS[0], 7)
    q, kp, vp, pt, kv = _np(w)
    cache = O.block_pool(kp, pt, kv, "f32")
    perm = np.array([3, 1, 0, 2, 6, 4, 7, 5])          # permutes heads inside each group of 4
    s1 = O.group_scores(q, cache, pt, kv, 2, 64)
    s2 = O.group_scores(q[:, perm], cache, pt, kv, 2, 64)
    np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-12)
    i1 = O.select_blocks(s1, kv, 1024, 64, 4)
    i2 = O.select_blocks(s2, kv, 1024, 64, 4)
    np.testing.assert_array_equal(i1, i2)


# --------------------------------------------------------------------------
# selection: brute force, ties, invariants
# --------------------------------------------------------------------------
def _brute_select(scores_row, own, k):
    """All (k-1)-subsets of the candidates; best = largest score sum, then the
    lexicographically smallest index tuple."""
    cands = list(range(own))
    m = min(k - 1, own)
    best = None
    for sub in itertools.combinations(cands, m):
        key = (-sum(scores_row[j] for j in sub), sub)
        if best is None or key < best:
            best = key
    sel = sorted(list(best[1]) + [own])
    return sel + [-1] * (k - len(sel))


@pytest.mark.parametrize("seed", range(6))
def test_selection_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    bs, k, nb = 4, 1 + (seed % 4) + 1, 9
    L = nb * bs
    s = rng.integers(-50, 50, size=(1, 1, L, nb)).astype(np.float64)   # exact in fp32, few ties
    own = np.arange(L) // bs
    s = np.where(np.arange(nb)[None, None, None, :] < own[None, None, :, None], s, -np.inf)
    idx = O.select_blocks(s, [L], L, bs, k)
    for t in range(L):
        row = s[0, 0, t]
        # with ties, the lexicographically smallest best-sum subset is the
        # one that keeps the lower indices among equal scores
        ref = _brute_select(row, int(own[t]), k)
        assert idx[0, 0, t].tolist() == ref, (t, row[:own[t]], k)


def test_selection_ties_prefer_lower_index():
    # duplicated representatives give exactly equal scores
    bs, D = 8, 16
    rng = np.random.default_rng(3)
    nb = 10
    reps = rng.standard_normal((nb, 1, D)).astype(np.float32)
    reps[7] = reps[2]
    reps[5] = reps[2]
    q = rng.standard_normal((1, 2, 1, D)).astype(np.float32)
    pt = np.arange(nb + 1, dtype=np.int32)[None]
    L = nb * bs + 1                      # own block = nb, candidates 0..nb-1
    cache = np.concatenate([reps, np.zeros((1, 1, D), np.float32)])
    sc = O.group_scores(q, cache, pt, [L], 1, bs)
    assert sc[0, 0, 0, 2] == sc[0, 0, 0, 5] == sc[0, 0, 0, 7]
    order = sorted(range(nb), key=lambda j: (-np.float32(sc[0, 0, 0, j]), j))
    pos2 = order.index(2)
    k = pos2 + 2                          # exactly one of the three tied blocks fits
    idx = O.select_blocks(sc, [L], 1, bs, k)[0, 0, 0].tolist()
    assert 2 in idx and 5 not in idx and 7 not in idx
    assert idx[-1] == nb and idx == sorted(idx)


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_selection_invariants_on_workloads(cfg):
    spec = SPECS[cfg]
    if cfg == 1:
        spec = spec.replace(seq_len=4096 + 40)
    if cfg == 3:
        spec = spec.replace(seq_len=8192, region=1024, num_q_heads=16, num_kv_heads=2)
    w = make_workload(spec, cfg)
    q, kp, vp, pt, kv = _np(w)
    bs, k = spec.page_size, spec.top_k
    cache = O.block_pool(kp, pt, kv, spec.dtype)
    T = q.shape[2]
    tsel = np.unique(np.concatenate([np.arange(0, T, max(1, T // 200)), [T - 1]]))
    sc = O.group_scores(q, cache, pt, kv, spec.num_kv_heads, bs, tsel)
    idx = O.select_blocks(sc, kv, T, bs, k, tsel)
    hit = tot = 0
    for g in range(spec.num_kv_heads):
        for ti, t in enumerate(tsel):
            own = t // bs
            row = idx[0, g, ti].tolist()
            val = [x for x in row if x >= 0]
            assert row == val + [-1] * (k - len(val))
            assert val == sorted(val) and len(set(val)) == len(val)
            assert own in val and max(val) == own
            assert len(val) == min(k, own + 1)
            # the unselected candidates never outrank a selected one (fp32 decision)
            s32 = sc[0, g, ti].astype(np.float32)
            chosen = [j for j in val if j != own]
            rest = [j for j in range(own) if j not in chosen]
            if chosen and rest:
                worst = min((s32[j], -j) for j in chosen)
                best_rest = max((s32[j], -j) for j in rest)
                assert worst > best_rest
            pl = w.planted_for(0, g, int(t))
            hit += sum(p in val for p in pl)
            tot += len(pl)
    assert tot == 0 or hit / tot > 0.97          # planted recall (soft)


def test_selection_is_exp_free_rank_invariant():
    """Ranking raw logits equals ranking their softmax weights (monotone map)."""
    rng = np.random.default_rng(9)
    s = rng.standard_normal((1, 1, 64, 16)) * 3
    own = np.arange(64) // 4
    s = np.where(np.arange(16)[None, None, None, :] < own[None, None, :, None], s, -np.inf)
    e = np.exp(s - 10.0)
    e = np.where(np.isfinite(s), e, -np.inf)
    np.testing.assert_array_equal(O.select_blocks(s, [64], 64, 4, 5), O.select_blocks(e, [64], 64, 4, 5))


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def _sdpa_dense(q, K, V, mask=None, causal=False, scale=None):
    """torch's scaled_dot_product_attention in float64 on CPU."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(K), torch.from_numpy(V),
        attn_mask=None if mask is None else torch.from_numpy(mask), is_causal=causal, scale=scale).numpy()


def test_topk_all_blocks_is_dense_causal_gqa():
    spec = SPECS[0].replace(seq_len=256 + 29, top_k=8)        # 5 blocks <= k
    w = make_workload(spec, 21)
    q, kp, vp, pt, kv = _np(w)
    r = O.prefill_reference(q, kp, vp, pt, kv, 64, spec.top_k, "f32")
    L = kv[0]
    K = O.gather_tokens(kp, pt[0], L).astype(np.float64)
    V = O.gather_tokens(vp, pt[0], L).astype(np.float64)
    G = 4
    Ke = np.repeat(K, G, axis=0)[None]
    Ve = np.repeat(V, G, axis=0)[None]
    ref = _sdpa_dense(q.astype(np.float64), Ke, Ve, causal=True)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-10, atol=1e-12)


def test_sparse_equals_dense_masked_softmax():
    """Gather-based attention = dense softmax with -inf outside the selection."""
    spec = SPECS[0].replace(seq_len=512 + 5)
    w = make_workload(spec, 22)
    q, kp, vp, pt, kv = _np(w)
    r = O.prefill_reference(q, kp, vp, pt, kv, 64, spec.top_k, "f32")
    L = kv[0]
    bs, G, Hkv = 64, 4, 2
    K = O.gather_tokens(kp, pt[0], L).astype(np.float64)
    V = O.gather_tokens(vp, pt[0], L).astype(np.float64)
    mask = np.zeros((Hkv * G, L, L), bool)
    pos = np.arange(L)
    for g in range(Hkv):
        for t in range(L):
            blk_ok = np.zeros(L // bs + 1, bool)
            sel = r["block_idx"][0, g, t]
            blk_ok[sel[sel >= 0]] = True
            mask[g * G:(g + 1) * G, t] = blk_ok[pos // bs] & (pos <= t)
    ref = _sdpa_dense(q.astype(np.float64), np.repeat(K, G, 0)[None], np.repeat(V, G, 0)[None], mask=mask[None])
    np.testing.assert_allclose(r["out"], ref, rtol=1e-10, atol=1e-12)
    # lse against the dense definition
    z = np.einsum("htd,hsd->hts", q[0].astype(np.float64), np.repeat(K, G, 0)) / 8.0
    z = np.where(mask, z, -np.inf)
    m = z.max(-1)
    lse = m + np.log(np.exp(z - m[..., None]).sum(-1))
    np.testing.assert_allclose(r["lse"][0], lse, rtol=1e-12, atol=1e-12)


def test_k1_is_block_local_causal_attention():
    spec = SPECS[0].replace(seq_len=200, top_k=1)
    w = make_workload(spec, 23)
    q, kp, vp, pt, kv = _np(w)
    r = O.prefill_reference(q, kp, vp, pt, kv, 64, 1, "f32")
    L, bs, G = 200, 64, 4
    pos = np.arange(L)
    mask = (pos[:, None] // bs == pos[None, :] // bs) & (pos[None, :] <= pos[:, None])
    K = O.gather_tokens(kp, pt[0], L).astype(np.float64)
    V = O.gather_tokens(vp, pt[0], L).astype(np.float64)
    ref = _sdpa_dense(q.astype(np.float64), np.repeat(K, G, 0)[None], np.repeat(V, G, 0)[None],
                      mask=np.broadcast_to(mask, (1, 8, L, L)).copy())
    np.testing.assert_allclose(r["out"], ref, rtol=1e-10, atol=1e-12)


def test_decode_equals_prefill_row_and_page_shuffle_invariance():
    spec = SPECS[0].replace(seq_len=64 * 9 + 13, top_k=3)
    w = make_workload(spec, 24)
    q, kp, vp, pt, kv = _np(w)
    r = O.prefill_reference(q, kp, vp, pt, kv, 64, 3, "f32")
    for t in (0, 63, 64, 300, 64 * 9 + 12):
        d = O.decode_reference(q[:, :, t:t + 1], kp, vp, pt, [t + 1], 64, 3, "f32",
                               block_cache=r["block_cache"])
        np.testing.assert_array_equal(d["block_idx"][:, :, 0], r["block_idx"][:, :, t])
        np.testing.assert_allclose(d["out"][:, :, 0], r["out"][:, :, t], rtol=1e-12, atol=1e-13)
    # shuffled physical pages give identical results
    perm = np.random.default_rng(0).permutation(kp.shape[0])
    inv = np.argsort(perm)
    kp2, vp2 = kp[perm], vp[perm]
    pt2 = inv[pt].astype(np.int32)
    r2 = O.prefill_reference(q, kp2, vp2, pt2, kv, 64, 3, "f32")
    np.testing.assert_array_equal(r2["block_idx"], r["block_idx"])
    np.testing.assert_array_equal(r2["out"], r["out"])


def test_chunked_prefill_rows_equal_full_prefill_rows():
    """Queries over an existing prefix (q_len < kv_len) give the same rows."""
    spec = SPECS[0].replace(seq_len=64 * 6 + 9)
    w = make_workload(spec, 25)
    q, kp, vp, pt, kv = _np(w)
    r = O.prefill_reference(q, kp, vp, pt, kv, 64, 4, "f32")
    ql = 100
    rc = O.prefill_reference(q[:, :, -ql:], kp, vp, pt, kv, 64, 4, "f32")
    np.testing.assert_array_equal(rc["block_idx"], r["block_idx"][:, :, -ql:])
    np.testing.assert_allclose(rc["out"], r["out"][:, :, -ql:], rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# gated fusion (Long-Context page, section 4.3, step 6)
# --------------------------------------------------------------------------
def test_gated_fusion_hand_values():
    a = np.array([[1.0, 2.0], [3.0, 4.0]])
    x = np.array([[5.0, 6.0], [7.0, 8.0]])
    # one gate per row: row 0 a quarter attention, row 1 all attention
    np.testing.assert_array_equal(O.gated_fusion(a, np.array([0.25, 1.0]), x), [[4.0, 5.0], [3.0, 4.0]])
    # one gate per element
    np.testing.assert_array_equal(O.gated_fusion(a, np.array([[0.0, 1.0], [0.5, 0.5]]), x), [[5.0, 2.0], [5.0, 6.0]])


def test_gated_fusion_limits_and_broadcast():
    rng = np.random.default_rng(3)
    a, x = rng.standard_normal((2, 3, 4, 8)), rng.standard_normal((2, 3, 4, 8))
    np.testing.assert_array_equal(O.gated_fusion(a, np.ones((2, 3, 4)), x), a)
    np.testing.assert_array_equal(O.gated_fusion(a, np.zeros((2, 3, 4, 8)), x), x)
    g = rng.uniform(-0.5, 1.5, (2, 3, 4))
    np.testing.assert_array_equal(O.gated_fusion(a, g, x), O.gated_fusion(a, np.repeat(g[..., None], 8, -1), x))
    with pytest.raises(ValueError):
        O.gated_fusion(a, np.ones((2, 3)), x)


# --------------------------------------------------------------------------
# generator
# --------------------------------------------------------------------------
def test_generator_is_deterministic_and_seed_sensitive():
    spec = SPECS[2].replace(batch=2, ctx_len=64 * 5 + 3, num_q_heads=4, num_kv_heads=2, head_dim=64)
    a = make_workload(spec, 5)
    b = make_workload(spec, 5)
    c = make_workload(spec, 6)
    for x, y in ((a.q, b.q), (a.k_cache, b.k_cache), (a.v_cache, b.v_cache), (a.page_table, b.page_table)):
        assert torch.equal(x, y)
    assert not torch.equal(a.q, c.q)
    assert a.kv_lens_host == [64 * 5 + 4] * 2
    # every physical page is used exactly once
    used = sorted(a.page_table[:, :6].flatten().tolist())
    assert used == list(range(12))


def test_generator_ragged_decode_lengths():
    spec = SPECS[4].replace(ctx_range=(1000, 3000), num_q_heads=4, num_kv_heads=2, head_dim=64)
    w = make_workload(spec, 4)
    for L in w.kv_lens_host:
        assert 1001 <= L <= 3001
    assert len(set(w.kv_lens_host)) > 1


# ----------------------------------------------------------------------------
# fp8 (OCP E4M3) KV cache: codes pinned to torch's float8_e4m3fn and to the format's
# published constants; scales and block representatives to brute force and closed forms
# ----------------------------------------------------------------------------
def _torch_e4m3_value(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_value_matches_format_and_torch():
    codes = np.arange(256, dtype=np.uint8)
    v = O.e4m3_value(codes)
    t = _torch_e4m3_value(codes)
    assert np.array_equal(np.isnan(v), np.isnan(t)) and np.array_equal(v[~np.isnan(v)], t[~np.isnan(t)])
    # constants of the OCP E4M3 format: largest finite, smallest normal and subnormal, one
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x38] == 1.0 and v[0xC0] == -2.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.sum(np.isnan(v)) == 2


def test_e4m3_code_ties_round_trip_and_torch():
    # ties go to the even code (mantissa last bit 0)
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (1.5 * 2.0 ** -9, 0x02), (7.5 * 2.0 ** -9, 0x08),
             (0.5 * 2.0 ** -9, 0x00), (2.5 * 2.0 ** -9, 0x02), (440.0, 0x7E), (-0.0, 0x80), (0.0, 0x00)]
    for x, c in cases:
        assert int(O.e4m3_code(x)) == c, (x, hex(int(O.e4m3_code(x))))
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(O.e4m3_code(O.e4m3_value(finite)), finite)
    rng = np.random.default_rng(5)
    x = np.clip(rng.standard_normal(20000) * np.exp2(rng.integers(-12, 8, 20000)), -448, 448)
    ct = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_code(x), ct)
    # brute force: the nearest finite value, ties to the even code
    vals = O.e4m3_value(finite)
    for xv in x[:400]:
        d = np.abs(vals - xv)
        best = finite[d == d.min()]
        best = best[(best & 1) == 0] if len(best) > 1 else best
        if len(best) > 1:                                   # +0 / -0: the sign follows x
            best = best[(best >> 7) == int(np.signbit(xv))]
        assert int(O.e4m3_code(xv)) == int(best[0])


def test_fp8_scale_exp_brute_force():
    rng = np.random.default_rng(6)
    vals = list(rng.random(300) * np.exp2(rng.integers(-60, 60, 300)))
    vals += [448.0 * 2.0 ** k for k in range(-20, 20)] + [np.nextafter(448.0 * 2.0 ** k, np.inf) for k in range(-5, 5)]
    vals += [0.875 * 2.0 ** k for k in range(-5, 5)] + [1.0, 3.0, 7.0]
    for a in vals:
        e_bf = next(e for e in range(-200, 200) if a <= 448.0 * 2.0 ** e)
        assert O.fp8_scale_exp(a) == max(-126, min(127, e_bf)), a
    assert O.fp8_scale_exp(0.0) == 0


def _small_fp8_case(seed=8, P=12, Hkv=2, bs=64, D=64):
    rng = np.random.default_rng(seed)
    pages = (rng.standard_normal((P, Hkv, bs, D)) * np.exp2(rng.integers(-3, 4, (P, Hkv, 1, 1)))).astype(np.float32)
    pt = np.array([[3, 7, 1, 10], [0, 5, 11, 2]], np.int32)
    kv = [64 * 3 + 17, 64 * 2]
    return pages, pt, kv


def test_quantize_pages_fp8_bounds_and_layout():
    pages, pt, kv = _small_fp8_case()
    bs = pages.shape[2]
    codes, scales = O.quantize_pages_fp8(pages, pt, kv, bs)
    used = set()
    for b, L in enumerate(kv):
        for j in range((L + bs - 1) // bs):
            p, n = int(pt[b, j]), min(bs, L - j * bs)
            used.add(p)
            for g in range(pages.shape[1]):
                s = float(scales[p, g])
                assert s == 2.0 ** round(math.log2(s))                   # a power of two
                x = pages[p, g, :n].astype(np.float64)
                y = O.e4m3_value(codes[p, g, :n]) * s
                assert np.abs(x).max() <= 448 * s and np.abs(x).max() > 224 * s   # the smallest such scale
                err = np.abs(y - x)
                assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s))   # half an ulp
                assert np.all(codes[p, g, n:] == 0)
    for p in range(pages.shape[0]):
        if p not in used:
            assert np.all(codes[p] == 0) and np.all(scales[p] == 1.0)
    # a tile whose maximum is 448 * 2^k is scaled by 2^k and its maximum gets code 0x7E
    pages2 = pages.copy()
    pages2[3, 0, 5, 7] = 448.0 * 2.0 ** -3
    pages2[3, 0] = np.clip(pages2[3, 0], -448.0 * 2.0 ** -3, 448.0 * 2.0 ** -3)
    c2, s2 = O.quantize_pages_fp8(pages2, pt, kv, bs)
    assert s2[3, 0] == 2.0 ** -3 and c2[3, 0, 5, 7] == 0x7E


def test_block_pool_fp8_closed_forms():
    pages, pt, kv = _small_fp8_case(seed=9)
    P, Hkv, bs, D = pages.shape
    codes, scales = O.quantize_pages_fp8(pages, pt, kv, bs)
    # constant keys: the representative decodes to the key itself
    const = codes.copy()
    const[:] = codes[:, :, :1, :]
    rc, rs = O.block_pool_fp8(const, scales, pt, kv)
    for b, L in enumerate(kv):
        for j in range(L // bs):
            p = int(pt[b, j])
            assert np.array_equal(O.fp8_dequant(rc[p][None], rs[p][None])[0], O.fp8_dequant(const[p][None, :, 0], scales[p][None])[0])
    # negated keys: sign bits flip, scales stay
    neg = codes ^ np.uint8(0x80)
    rc1, rs1 = O.block_pool_fp8(codes, scales, pt, kv)
    rc2, rs2 = O.block_pool_fp8(neg, scales, pt, kv)
    full = [int(pt[b, j]) for b, L in enumerate(kv) for j in range(L // bs)]
    nz = O.e4m3_value(rc1[full]) != 0
    assert np.array_equal((rc1[full] ^ np.uint8(0x80))[nz], rc2[full][nz]) and np.array_equal(rs1[full], rs2[full])
    # against the exact mean of the decoded keys: within half an ulp of E4M3 (+ float32 sums)
    for p in full:
        mean = O.fp8_dequant(codes[p][None], scales[p][None])[0].mean(axis=1)        # [Hkv, D]
        rep = O.fp8_dequant(rc1[p][None], rs1[p][None])[0]
        s = rs1[p].astype(np.float64)[:, None]
        assert np.all(np.abs(rep - mean) <= np.abs(mean) * (2.0 ** -4 + 1e-6) + 2.0 ** -10 * s + 1e-12)
    # untouched pages keep their entries; blk_begin skips earlier blocks
    rc3, rs3 = O.block_pool_fp8(codes, scales, pt, kv, blk_begin=[2, 1])
    assert np.all(rc3[int(pt[0, 0])] == 0) and np.array_equal(rc3[int(pt[0, 2])], rc1[int(pt[0, 2])])


# ----------------------------------------------------------------------------
# token-level and two-level selection: scores against torch einsum, the selection's
# threshold property by brute force, reductions to dense and to block-level attention
# ----------------------------------------------------------------------------
def _decode_case(seed, B=2, L=(64 * 5 + 9, 64 * 3 + 40), Hq=8, Hkv=2, D=64, shuffle=True):
    spec = SPECS[2].replace(batch=B, ctx_len=0, ctx_range=(min(L), max(L)), num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim=D, dtype="f32", shuffle_pages=shuffle)
    w = make_workload(spec, seed)
    q, kp, vp, pt, kv = _np(w)
    return spec, q, kp, vp, pt, kv


def test_token_scores_match_einsum_and_causality():
    spec, q, kp, vp, pt, kv = _decode_case(31)
    sc = O.token_scores(q, kp, pt, kv)
    G = spec.num_q_heads // spec.num_kv_heads
    for b, L in enumerate(kv):
        K = torch.from_numpy(O.gather_tokens(kp, pt[b], L).astype(np.float64))        # [Hkv, L, D]
        qt = torch.from_numpy(q[b, :, 0].astype(np.float64)).view(spec.num_kv_heads, G, -1)
        ref = torch.einsum("ghd,gsd->gs", qt, K).numpy()
        np.testing.assert_allclose(sc[b, :, 0, :L], ref, rtol=1e-12, atol=1e-12)
        assert np.all(np.isneginf(sc[b, :, 0, L:]))
    # prefill-shaped queries: tokens after the query's position are not candidates
    spec2 = SPECS[0].replace(seq_len=200)
    w = make_workload(spec2, 32)
    q2, kp2, vp2, pt2, kv2 = _np(w)
    s2 = O.token_scores(q2, kp2, pt2, kv2, t_idx=[0, 63, 64, 199])
    for ti, t in enumerate([0, 63, 64, 199]):
        assert np.all(np.isfinite(s2[0, :, ti, :t + 1])) and np.all(np.isneginf(s2[0, :, ti, t + 1:]))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_select_tokens_threshold_property(seed):
    rng = np.random.default_rng(seed)
    sc = np.round(rng.standard_normal((2, 3, 2, 300)) * 4) / 4              # many exact ties
    sc[..., 250:] = -np.inf                                                 # not candidates
    sc[1, 0, 1, 7:] = -np.inf                                               # fewer candidates than K
    K = 40
    idx = O.select_tokens(sc, K)
    for b, g, t in itertools.product(range(2), range(3), range(2)):
        row = sc[b, g, t].astype(np.float32)
        cand = np.nonzero(np.isfinite(row))[0]
        kept = [int(x) for x in idx[b, g, t] if x >= 0]
        assert kept == sorted(set(kept)) and len(kept) == min(K, len(cand))
        assert np.all(idx[b, g, t, len(kept):] == -1)
        dropped = sorted(set(cand.tolist()) - set(kept))
        for i in kept:                                   # every kept token beats every dropped one
            for j in dropped:
                assert row[i] > row[j] or (row[i] == row[j] and i < j)


def test_token_topk_of_all_tokens_is_dense_gqa():
    spec, q, kp, vp, pt, kv = _decode_case(33)
    r = O.decode_tokens_reference(q, kp, vp, pt, kv, top_k_tokens=max(kv))
    G = spec.num_q_heads // spec.num_kv_heads
    for b, L in enumerate(kv):
        K = O.gather_tokens(kp, pt[b], L).astype(np.float64)
        V = O.gather_tokens(vp, pt[b], L).astype(np.float64)
        ref = _sdpa_dense(q[b:b + 1].astype(np.float64), np.repeat(K, G, axis=0)[None],
                          np.repeat(V, G, axis=0)[None], scale=1.0 / math.sqrt(q.shape[-1]))
        np.testing.assert_allclose(r["out"][b], ref[0], rtol=1e-10, atol=1e-12)


def test_two_level_reduces_to_block_and_to_token_selection():
    spec, q, kp, vp, pt, kv = _decode_case(34)
    bs, kb = spec.page_size, 3
    # every token of the kept blocks kept -> the block-level decode step
    r2 = O.two_level_decode_reference(q, kp, vp, pt, kv, bs, kb, kb * bs, "f32")
    rb = O.decode_reference(q, kp, vp, pt, kv, bs, kb, "f32")
    assert np.array_equal(r2["block_idx"], rb["block_idx"])
    np.testing.assert_allclose(r2["out"], rb["out"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r2["lse"], rb["lse"], rtol=1e-12, atol=1e-12)
    # every block kept -> the token-level step
    nb = max((L + bs - 1) // bs for L in kv)
    Kt = 50
    r3 = O.two_level_decode_reference(q, kp, vp, pt, kv, bs, nb + 1, Kt, "f32")
    rt = O.decode_tokens_reference(q, kp, vp, pt, kv, Kt)
    assert np.array_equal(r3["token_idx"], rt["token_idx"])
    np.testing.assert_allclose(r3["out"], rt["out"], rtol=1e-12, atol=1e-12)
    # the kept tokens lie in the kept blocks and are the best of those blocks' tokens
    r4 = O.two_level_decode_reference(q, kp, vp, pt, kv, bs, kb, 70, "f32")
    for b in range(len(kv)):
        for g in range(spec.num_kv_heads):
            blocks = set(int(j) for j in r4["block_idx"][b, g, 0] if j >= 0)
            toks = [int(s) for s in r4["token_idx"][b, g, 0] if s >= 0]
            assert len(toks) == 70 and all(s // bs in blocks for s in toks)


# prefill rows of the token forms: every position of a prompt is a row at its own position
def test_token_topk_of_every_prefill_position_is_dense_causal_gqa():
    """K at least the prompt length: every row keeps every earlier token, so the token-level
    prefill is dense causal GQA attention (torch's scaled_dot_product_attention, is_causal)."""
    spec = SPECS[0].replace(seq_len=150)
    w = make_workload(spec, 35)
    q, kp, vp, pt, kv = _np(w)
    L = kv[0]
    sc = O.token_scores(q, kp, pt, kv)
    idx = O.select_tokens(sc, L)
    for t in (0, 1, 77, L - 1):                     # row t keeps tokens 0..t, ascending
        assert list(idx[0, 0, t, :t + 1]) == list(range(t + 1)) and np.all(idx[0, 0, t, t + 1:] == -1)
    out, lse = O.token_attention(q, kp, vp, pt, kv, idx, 1.0 / math.sqrt(spec.head_dim))
    K = O.gather_tokens(kp, pt[0], L).astype(np.float64)
    V = O.gather_tokens(vp, pt[0], L).astype(np.float64)
    G = spec.num_q_heads // spec.num_kv_heads
    ref = _sdpa_dense(q.astype(np.float64), np.repeat(K, G, axis=0)[None], np.repeat(V, G, axis=0)[None],
                      causal=True, scale=1.0 / math.sqrt(spec.head_dim))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_token_prefill_rows_equal_decode_steps():
    """Prefill row t (queries at the end of a longer context included) is the decode step at
    kv_len = position + 1 with that query: the same scores (up to the summation order of the
    two matrix products), kept tokens and output."""
    spec = SPECS[0].replace(seq_len=64 * 3 + 20, q_len=90)
    w = make_workload(spec, 36)
    q, kp, vp, pt, kv = _np(w)
    L, ql, K = kv[0], q.shape[2], 37
    sc = O.token_scores(q, kp, pt, kv)
    idx = O.select_tokens(sc, K)
    out, lse = O.token_attention(q, kp, vp, pt, kv, idx, 0.125)
    for t in (0, 5, ql - 1):
        p = L - ql + t
        r = O.decode_tokens_reference(q[:, :, t:t + 1], kp, vp, pt, [p + 1], K, 0.125)
        np.testing.assert_allclose(r["scores"][:, :, 0, :p + 1], sc[:, :, t, :p + 1], rtol=1e-13, atol=1e-12)
        assert np.array_equal(r["token_idx"][:, :, 0], idx[:, :, t])
        np.testing.assert_allclose(r["out"][:, :, 0], out[:, :, t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(r["lse"][:, :, 0], lse[:, :, t], rtol=1e-12, atol=1e-12)


def test_two_level_prefill_with_whole_blocks_is_block_prefill():
    """Two level at prefill, K = k * bs: every token of each row's kept blocks is kept, which
    is the block-level prefill of the same rows."""
    spec = SPECS[0].replace(seq_len=64 * 5 + 13, top_k=3)
    w = make_workload(spec, 37)
    q, kp, vp, pt, kv = _np(w)
    bs, k = spec.page_size, spec.top_k
    r = O.prefill_reference(q, kp, vp, pt, kv, bs, k, "f32")
    sc = O.token_scores(q, kp, pt, kv, block_idx=r["block_idx"])
    idx = O.select_tokens(sc, k * bs)
    for t in (0, 64, q.shape[2] - 1):                # the kept blocks' valid tokens, ascending
        want = sorted(s for j in r["block_idx"][0, 0, t] if j >= 0
                      for s in range(j * bs, min((j + 1) * bs, t + 1)))
        assert [int(s) for s in idx[0, 0, t] if s >= 0] == want
    out, lse = O.token_attention(q, kp, vp, pt, kv, idx, 1.0 / math.sqrt(spec.head_dim))
    np.testing.assert_allclose(out, r["out"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, r["lse"], rtol=1e-10, atol=1e-12)
