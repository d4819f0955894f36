"""GPU parity: each library call against the CPU oracle on the same seeded inputs.

Sizes are reduced versions of the five workloads (same heads, head_dim, block size, top-k,
planting), large enough to span several tiles and a ragged tail.  Stage tests feed the
oracle's own intermediate results into one library call; end-to-end tests run the whole
path on the device and compare selections (bit-exact up to the tie window) and outputs.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_gqa_pool_amd as bsg
import oracle as O
from workloads import SPECS, make_workload

from gpu_util import (check_out, compare_selection, gpu_prefill, note, np_inputs, sample_tokens, to_np)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# reduced shapes of the five workloads (name -> spec)
SMALL = {
    "c0_tiny_f32": SPECS[0],
    "c1_bf16_g8_bs64": SPECS[1].replace(seq_len=4096 + 40),
    "c3_bf16_g8_bs128": SPECS[3].replace(seq_len=8192 + 77, region=1024, num_q_heads=16, num_kv_heads=2),
    "c2_decode": SPECS[2].replace(batch=5, ctx_len=64 * 300 + 7),
    "c4_decode_ragged": SPECS[4].replace(batch=3, ctx_range=(64 * 200, 64 * 700), num_q_heads=16, num_kv_heads=2),
}
PREFILL = ["c0_tiny_f32", "c1_bf16_g8_bs64", "c3_bf16_g8_bs128"]
DECODE = ["c2_decode", "c4_decode_ragged"]


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    bsg.lib()


def _work(name, seed=7, **kw):
    note(f"[case] {name} seed={seed} {kw}")
    spec = SMALL[name].replace(**kw) if kw else SMALL[name]
    return make_workload(spec, seed).to(DEV)


# ---------------------------------------------------------------- block pool
@pytest.mark.parametrize("name", list(SMALL))
def test_block_pool_bit_exact(name):
    spec = SMALL[name]
    w = make_workload(spec, 3, tail_fill=float("nan")).to(DEV)
    note(f"[case] block_pool {name}")
    q, kp, vp, pt, kv = np_inputs(w)
    ref = O.block_pool(kp, pt, kv, spec.dtype)   # complete blocks never contain the NaN tail slots
    cache = torch.zeros(kp.shape[0], spec.num_kv_heads, spec.head_dim, dtype=w.k_cache.dtype, device=DEV)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
    torch.cuda.synchronize()
    got = to_np(cache)
    if spec.dtype == "bf16":
        gb = cache.view(torch.int16).cpu().numpy().view(np.uint16)
        rb = O.bf16_bits(ref)
        assert np.array_equal(gb, rb)
    else:
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_block_pool_incremental_refresh():
    """Refreshing one completed page per sequence (blk_begin) writes exactly that page."""
    w = _work("c2_decode")
    s = w.spec
    q, kp, vp, pt, kv = np_inputs(w)
    cache = torch.zeros(kp.shape[0], s.num_kv_heads, s.head_dim, dtype=w.k_cache.dtype, device=DEV)
    short = torch.tensor([x - 3 * 64 for x in kv], dtype=torch.int32, device=DEV)
    bsg.block_pool(w.k_cache, w.page_table, short, cache)
    begin = torch.tensor([(x - 3 * 64) // 64 for x in kv], dtype=torch.int32, device=DEV)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache, blk_begin=begin)
    torch.cuda.synchronize()
    ref = O.block_pool(kp, pt, kv, "bf16")
    assert np.array_equal(cache.view(torch.int16).cpu().numpy().view(np.uint16), O.bf16_bits(ref))


# ---------------------------------------------------------------- scores
@pytest.mark.parametrize("name", list(SMALL))
def test_group_score_matches_oracle(name):
    w = _work(name)
    s = w.spec
    q, kp, vp, pt, kv = np_inputs(w)
    ref_cache = O.block_pool(kp, pt, kv, s.dtype)
    # the oracle's block cache bytes are the input of this stage
    cache = torch.from_numpy(ref_cache).to(w.k_cache.dtype).to(DEV)
    B, Hq, ql, D = w.q.shape
    sc = torch.empty(B, s.num_kv_heads, ql, w.pt_stride, dtype=torch.float32, device=DEV)
    bsg.group_score(w.q, w.kv_lens, cache, w.page_table, sc, page_size=s.page_size)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    ref = O.group_scores(q, ref_cache, pt, kv, s.num_kv_heads, s.page_size)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.all(np.isneginf(got[~fin]))
    err = np.abs(got[fin] - ref[fin])
    note(f"  score max abs err {err.max() if err.size else 0:.3e}")
    assert np.all(err <= 1e-5 * np.maximum(np.abs(ref[fin]), 10.0))


# ---------------------------------------------------------------- top-k
def _oracle_scores_f32(name, seed=7):
    w = _work(name, seed)
    s = w.spec
    q, kp, vp, pt, kv = np_inputs(w)
    cache = O.block_pool(kp, pt, kv, s.dtype)
    sc = O.group_scores(q, cache, pt, kv, s.num_kv_heads, s.page_size)
    return w, sc


@pytest.mark.parametrize("name", list(SMALL))
def test_topk_blocks_bit_exact_on_oracle_scores(name):
    w, sc = _oracle_scores_f32(name)
    s = w.spec
    B, Hkv, ql, nb = sc.shape
    dsc = torch.from_numpy(sc.astype(np.float32)).to(DEV)
    idx = torch.empty(B, Hkv, ql, s.top_k, dtype=torch.int32, device=DEV)
    bsg.topk_blocks(dsc, w.kv_lens, idx, page_size=s.page_size)
    torch.cuda.synchronize()
    ref = O.select_blocks(sc, w.kv_lens_host, ql, s.page_size, s.top_k)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("rows_B,ncand,k", [(2, 3000, 32), (64, 700, 17), (1, 16385, 64), (3, 40, 1), (5, 9, 32)])
def test_topk_blocks_constructed_ties(rows_B, ncand, k):
    """Scores drawn from a handful of values (massive exact ties, +-0.0 mixed) -> lower index wins."""
    rng = np.random.default_rng(ncand)
    bs = 64
    kv = [ncand * bs + 1 + b for b in range(rows_B)]              # decode rows; own = ncand
    sc = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 2.0, 2.0000002], np.float32), size=(rows_B, 2, 1, ncand + 1))
    sc[..., ncand:] = -np.inf
    note(f"[case] ties B={rows_B} ncand={ncand} k={k}")
    dsc = torch.from_numpy(sc).to(DEV)
    kvl = torch.tensor(kv, dtype=torch.int32, device=DEV)
    idx = torch.empty(rows_B, 2, 1, k, dtype=torch.int32, device=DEV)
    bsg.topk_blocks(dsc, kvl, idx, page_size=bs)
    torch.cuda.synchronize()
    ref = O.select_blocks(sc.astype(np.float64), kv, 1, bs, k)
    assert np.array_equal(idx.cpu().numpy(), ref)


# ---------------------------------------------------------------- attention stages
def _prefill_stage(w, top_k, scale=None):
    s = w.spec
    q, kp, vp, pt, kv = np_inputs(w)
    D = s.head_dim
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    cache = O.block_pool(kp, pt, kv, s.dtype)
    ql = w.q.shape[2]
    tsel = None if ql <= 2048 else sample_tokens(ql, s.page_size, 300)
    sc = O.group_scores(q, cache, pt, kv, s.num_kv_heads, s.page_size, tsel)
    idx = O.select_blocks(sc, kv, ql, s.page_size, top_k, tsel)
    # the device needs a full block_idx: the oracle's rows where sampled, full oracle otherwise
    if tsel is not None:
        sc_all = O.group_scores(q, cache, pt, kv, s.num_kv_heads, s.page_size)
        idx_all = O.select_blocks(sc_all, kv, ql, s.page_size, top_k)
    else:
        idx_all = idx
    ref_out, ref_lse = O.sparse_attention(q, kp, vp, pt, kv, idx, scale, tsel)
    didx = torch.from_numpy(idx_all).to(DEV)
    out = torch.empty_like(w.q)
    lse = torch.empty(w.q.shape[:3], dtype=torch.float32, device=DEV)
    bsg.sparse_attn_prefill(w.q, w.kv_lens, w.k_cache, w.v_cache, w.page_table, didx, scale, out, lse)
    torch.cuda.synchronize()
    got = to_np(out)
    gl = lse.cpu().numpy()
    if tsel is not None:
        got, gl = got[:, :, tsel], gl[:, :, tsel]
    return got, gl, ref_out, ref_lse


@pytest.mark.parametrize("name", PREFILL)
def test_prefill_attention_on_oracle_selection(name):
    w = make_workload(SMALL[name], 11, tail_fill=float("nan")).to(DEV)
    note(f"[case] prefill attention {name}")
    got, gl, ref, rl = _prefill_stage(w, w.spec.top_k)
    check_out(got, ref, w.spec.dtype, "out")
    tol = 2e-3 if w.spec.dtype == "bf16" else 1e-4
    assert np.abs(gl - rl).max() <= tol


@pytest.mark.parametrize("case", [
    dict(top_k=1),                                   # block-local causal attention
    dict(top_k=64),                                  # every block: dense causal
    dict(num_q_heads=4, num_kv_heads=4),             # G = 1
    dict(num_q_heads=8, num_kv_heads=4),             # G = 2
    dict(num_q_heads=16, num_kv_heads=4),            # G = 4
    dict(num_q_heads=64, num_kv_heads=4),            # G = 16
    dict(num_q_heads=24, num_kv_heads=4),            # G = 6 (not a power of two)
    dict(head_dim=64),
    dict(page_size=128, top_k=5),
    dict(q_len=333),                                 # queries over an existing prefix
    dict(batch=3),
])
def test_prefill_attention_edge_shapes(case):
    spec = SPECS[1].replace(seq_len=64 * 24 + 13, **case)
    note(f"[case] prefill edge {case}")
    w = make_workload(spec, 5, tail_fill=float("nan")).to(DEV)
    got, gl, ref, rl = _prefill_stage(w, spec.top_k)
    check_out(got, ref, "bf16", f"out {case}")
    assert np.abs(gl - rl).max() <= 2e-3


@pytest.mark.parametrize("name", DECODE)
def test_decode_attention_on_oracle_selection(name):
    w = make_workload(SMALL[name], 13, tail_fill=float("nan")).to(DEV)
    note(f"[case] decode attention {name}")
    s = w.spec
    q, kp, vp, pt, kv = np_inputs(w)
    scale = 1.0 / math.sqrt(s.head_dim)
    r = O.decode_reference(q, kp, vp, pt, kv, s.page_size, s.top_k, s.dtype, scale)
    didx = torch.from_numpy(r["block_idx"][:, :, 0]).contiguous().to(DEV)
    B, Hq = w.q.shape[:2]
    out = torch.empty(B, Hq, s.head_dim, dtype=w.q.dtype, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.sparse_attn_decode(w.q[:, :, 0].contiguous(), w.kv_lens, w.k_cache, w.v_cache, w.page_table, didx, scale,
                           out, lse)
    torch.cuda.synchronize()
    check_out(to_np(out), r["out"][:, :, 0], s.dtype, "decode out")
    assert np.abs(lse.cpu().numpy() - r["lse"][:, :, 0]).max() <= 2e-3


# ---------------------------------------------------------------- end to end
@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name", PREFILL)
def test_prefill_end_to_end(name, fused):
    w = _work(name, seed=21)
    s = w.spec
    g = gpu_prefill(w, s.top_k, fused=fused)
    q, kp, vp, pt, kv = np_inputs(w)
    r = O.prefill_reference(q, kp, vp, pt, kv, s.page_size, s.top_k, s.dtype)
    assert np.array_equal(to_np(g["block_cache"]), r["block_cache"])
    gi = g["block_idx"].cpu().numpy()
    bad, exempt = compare_selection(gi, r["block_idx"], r["scores"], s.top_k)
    note(f"  selection rows: {gi.shape[0] * gi.shape[1] * gi.shape[2]}, exempt ties {len(exempt)}, bad {len(bad)}")
    assert not bad, bad[:10]
    same = ~(gi != r["block_idx"]).any(-1)                       # [B, Hkv, T]
    G = s.group_size
    rows = np.repeat(same, G, axis=1)                            # per query head
    check_out(to_np(g["out"])[rows], r["out"][rows], s.dtype, "out")


def run_decode_gpu(w, api="step", lse=True):
    """Whole decode step on the device: separate calls ("split") or bsg_decode_step ("step")."""
    s = w.spec
    B, Hq, _, D = w.q.shape
    scale = 1.0 / math.sqrt(D)
    cache = torch.zeros(w.k_cache.shape[0], s.num_kv_heads, D, dtype=w.k_cache.dtype, device=DEV)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
    out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
    l = torch.empty(B, Hq, dtype=torch.float32, device=DEV) if lse else None
    q1 = w.q[:, :, 0].contiguous()
    if api == "split":
        idx = torch.empty(B, s.num_kv_heads, 1, s.top_k, dtype=torch.int32, device=DEV)
        bsg.group_score_topk(w.q, w.kv_lens, cache, w.page_table, idx, page_size=s.page_size)
        idx = idx[:, :, 0].contiguous()
        bsg.sparse_attn_decode(q1, w.kv_lens, w.k_cache, w.v_cache, w.page_table, idx, scale, out, l)
    else:
        idx = torch.full((B, s.num_kv_heads, s.top_k), -7, dtype=torch.int32, device=DEV)
        bsg.decode_step(q1, w.kv_lens, cache, w.k_cache, w.v_cache, w.page_table, scale, idx, out, l)
    torch.cuda.synchronize()
    return cache, idx, out, l


def check_decode(w, idx, out, lse):
    s = w.spec
    q, kp, vp, pt, kv = np_inputs(w)
    r = O.decode_reference(q, kp, vp, pt, kv, s.page_size, s.top_k, s.dtype, 1.0 / math.sqrt(s.head_dim))
    gi = idx.cpu().numpy()[:, :, None]
    bad, exempt = compare_selection(gi, r["block_idx"], r["scores"], s.top_k)
    note(f"  exempt ties {len(exempt)}, bad {len(bad)}")
    assert not bad, bad
    same = np.repeat(~(gi != r["block_idx"]).any(-1)[:, :, 0], s.group_size, axis=1)
    check_out(to_np(out)[same], r["out"][:, :, 0][same], s.dtype, "decode out")
    if lse is not None:
        assert np.abs(lse.cpu().numpy()[same] - r["lse"][:, :, 0][same]).max() <= 2e-3


@pytest.mark.parametrize("api", ["split", "step"])
@pytest.mark.parametrize("name", DECODE)
def test_decode_end_to_end(name, api):
    w = _work(name, seed=23)
    cache, idx, out, lse = run_decode_gpu(w, api)
    check_decode(w, idx, out, lse)


@pytest.mark.parametrize("case", [
    dict(top_k=1), dict(top_k=2), dict(top_k=64), dict(top_k=33), dict(top_k=8), dict(top_k=16, head_dim=64),
    dict(num_q_heads=4, num_kv_heads=4), dict(num_q_heads=16, num_kv_heads=4), dict(num_q_heads=24, num_kv_heads=4),
    dict(head_dim=64), dict(page_size=128, top_k=5), dict(q_len=333), dict(batch=3), dict(seq_len=64 * 3 + 1),
])
def test_fused_selection_edge_shapes(case):
    """Fused score + top-k against the oracle's selection (tie window) on edge shapes."""
    kw = dict(seq_len=64 * 40 + 13)
    kw.update(case)
    spec = SPECS[1].replace(**kw)
    note(f"[case] fused selection {case}")
    w = make_workload(spec, 8).to(DEV)
    q, kp, vp, pt, kv = np_inputs(w)
    cache = O.block_pool(kp, pt, kv, "bf16")
    sc = O.group_scores(q, cache, pt, kv, spec.num_kv_heads, spec.page_size)
    ref = O.select_blocks(sc, kv, w.q.shape[2], spec.page_size, spec.top_k)
    dcache = torch.from_numpy(cache).to(torch.bfloat16).to(DEV)
    B, Hq, ql, D = w.q.shape
    idx = torch.empty(B, spec.num_kv_heads, ql, spec.top_k, dtype=torch.int32, device=DEV)
    bsg.group_score_topk(w.q, w.kv_lens, dcache, w.page_table, idx, page_size=spec.page_size)
    torch.cuda.synchronize()
    bad, exempt = compare_selection(idx.cpu().numpy(), ref, sc, spec.top_k)
    note(f"  exempt {len(exempt)} bad {len(bad)}")
    assert not bad, bad[:5]


@pytest.mark.parametrize("case", [
    dict(top_k=1), dict(top_k=3), dict(top_k=64), dict(num_q_heads=4, num_kv_heads=4),
    dict(num_q_heads=64, num_kv_heads=4), dict(head_dim=64), dict(page_size=128, top_k=9),
    dict(ctx_len=64 * 120 - 1),            # the new token completes its page
    dict(ctx_len=70),                      # fewer candidates than top_k - 1
    dict(num_q_heads=80, num_kv_heads=4, head_dim=64),  # G = 20: VALU split path
])
@pytest.mark.parametrize("api", ["split", "step"])
def test_decode_edge_shapes_end_to_end(case, api):
    spec = SPECS[2].replace(batch=3, ctx_len=64 * 150 + 11, **case) if "ctx_len" not in case else \
        SPECS[2].replace(batch=3, **case)
    note(f"[case] decode edge {case} {api}")
    w = make_workload(spec, 17, tail_fill=float("nan")).to(DEV)
    cache, idx, out, lse = run_decode_gpu(w, api)
    check_decode(w, idx, out, lse)


@pytest.mark.parametrize("batch", [40, 31, 32, 3], ids=["one_member", "two_members_idle_slots", "two_members",
                                                     "four_members"])
def test_decode_step_member_counts(batch):
    """The one-kernel decode step serves a (sequence, group) unit with S = 1, 2 or 4 workgroups
    (by the number of units against the CUs; 4 KV heads here): 160 units take one each and
    write the rows themselves, 124 and 128 units two (124 leaves four slots of the last group of
    eight idle), 12 units four; the partials of S > 1 go through the merge kernel."""
    spec = SPECS[2].replace(batch=batch, ctx_len=64 * 24 + 5)
    note(f"[case] decode_step with {batch * spec.num_kv_heads} units")
    w = make_workload(spec, 19, tail_fill=float("nan")).to(DEV)
    cache, idx, out, lse = run_decode_gpu(w, "step")
    check_decode(w, idx, out, lse)


def test_decode_step_ragged_batch_and_reuse():
    """Ragged lengths (some shorter than the others by many chunks); workspace reused."""
    spec = SPECS[4].replace(batch=4, ctx_range=(64 * 30, 64 * 900), num_q_heads=16, num_kv_heads=2)
    ws = None
    for seed in (41, 42):
        note(f"[case] ragged decode_step seed={seed}")
        w = make_workload(spec, seed, tail_fill=float("nan")).to(DEV)
        B, Hq, _, D = w.q.shape
        cache = torch.zeros(w.k_cache.shape[0], spec.num_kv_heads, D, dtype=w.k_cache.dtype, device=DEV)
        bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
        if ws is None:
            ws = torch.empty(bsg.decode_step_workspace_bytes(w.k_cache, w.page_table, Hq, spec.top_k) + 4096,
                             dtype=torch.uint8, device=DEV)
        idx = torch.empty(B, spec.num_kv_heads, spec.top_k, dtype=torch.int32, device=DEV)
        out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
        lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
        bsg.decode_step(w.q[:, :, 0].contiguous(), w.kv_lens, cache, w.k_cache, w.v_cache, w.page_table,
                        1.0 / math.sqrt(D), idx, out, lse, workspace=ws)
        torch.cuda.synchronize()
        check_decode(w, idx, out, lse)


def test_decode_workspace_reuse_across_calls():
    """The decode workspace is reused by consecutive calls (its counters reset themselves)."""
    spec = SPECS[2].replace(batch=4, ctx_len=64 * 90 + 3)
    ws = None
    for seed in (31, 32, 33):
        note(f"[case] workspace reuse seed={seed}")
        w = make_workload(spec, seed).to(DEV)
        B, Hq, _, D = w.q.shape
        scale = 1.0 / math.sqrt(D)
        if ws is None:
            ws = torch.zeros(bsg.decode_workspace_bytes(w.k_cache, w.page_table, Hq, spec.top_k),
                             dtype=torch.uint8, device=DEV)
        q, kp, vp, pt, kv = np_inputs(w)
        r = O.decode_reference(q, kp, vp, pt, kv, spec.page_size, spec.top_k, spec.dtype, scale)
        didx = torch.from_numpy(r["block_idx"][:, :, 0]).contiguous().to(DEV)
        out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
        for _ in range(2):
            bsg.sparse_attn_decode(w.q[:, :, 0].contiguous(), w.kv_lens, w.k_cache, w.v_cache, w.page_table, didx,
                                   scale, out, workspace=ws)
            torch.cuda.synchronize()
            check_out(to_np(out), r["out"][:, :, 0], "bf16", "decode out (reused workspace)")


def test_decode_step_graph_replay_matches_eager():
    """bsg_decode_step captured in a HIP graph: every replay equals the eager call bit for bit,
    with eager work and synchronisation between the replays."""
    spec = SPECS[2].replace(batch=6, ctx_len=64 * 200 + 9)
    w = make_workload(spec, 51).to(DEV)
    B, Hq, _, D = w.q.shape
    Hkv, k = spec.num_kv_heads, spec.top_k
    scale = 1.0 / math.sqrt(D)
    cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=DEV)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
    q1 = w.q[:, :, 0].contiguous()
    ws = torch.empty(bsg.decode_step_workspace_bytes(w.k_cache, w.page_table, Hq, k), dtype=torch.uint8, device=DEV)
    idx_e = torch.empty(B, Hkv, k, dtype=torch.int32, device=DEV)
    out_e = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
    lse_e = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.decode_step(q1, w.kv_lens, cache, w.k_cache, w.v_cache, w.page_table, scale, idx_e, out_e, lse_e, workspace=ws)
    torch.cuda.synchronize()
    idx_g = torch.empty_like(idx_e)
    out_g = torch.empty_like(out_e)
    lse_g = torch.empty_like(lse_e)
    ws_g = torch.empty_like(ws)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bsg.decode_step(q1, w.kv_lens, cache, w.k_cache, w.v_cache, w.page_table, scale, idx_g, out_g, lse_g,
                        workspace=ws_g)
    torch.cuda.synchronize()
    for rep in range(3):
        idx_g.fill_(-5)
        out_g.zero_()
        lse_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        note(f"  replay {rep}")
        assert torch.equal(idx_g, idx_e)
        assert torch.equal(out_g, out_e)
        assert torch.equal(lse_g, lse_e)
        # eager work between replays (same workspace as the eager call)
        bsg.decode_step(q1, w.kv_lens, cache, w.k_cache, w.v_cache, w.page_table, scale, idx_e, out_e, lse_e,
                        workspace=ws)
        torch.cuda.synchronize()
    check_decode(w, idx_e, out_e, lse_e)


@pytest.mark.parametrize("top_k", [2, 8, 16, 33, 64])
def test_fused_selection_exact_ties(top_k):
    """Fused score + top-k with a block cache whose representatives repeat three patterns, so
    most candidates tie exactly with many others: the kept blocks must be the lowest-indexed
    ones of the best pattern(s), as in the oracle, bit for bit.  (Identical representatives
    give identical scores on both sides; rows whose boundary falls between two different
    patterns closer than 1e-4 relative are left out.)"""
    spec = SPECS[1].replace(seq_len=64 * 200 + 13, top_k=top_k)
    note(f"[case] fused selection with exact ties, top_k={top_k}")
    w = make_workload(spec, 9).to(DEV)
    q, kp, vp, pt, kv = np_inputs(w)
    P, Hkv, D = kp.shape[0], spec.num_kv_heads, spec.head_dim
    rng = np.random.default_rng(5)
    pats = torch.from_numpy(rng.standard_normal((3, Hkv, D)).astype(np.float32)).to(torch.bfloat16).float().numpy()
    which = (np.arange(P)[:, None] * 5 + np.arange(Hkv)[None, :]) % 3          # [P, Hkv]
    cache = pats[which, np.arange(Hkv)[None, :]]                                # [P, Hkv, D]
    sc = O.group_scores(q, cache, pt, kv, Hkv, spec.page_size)
    ref = O.select_blocks(sc, kv, w.q.shape[2], spec.page_size, top_k)
    dcache = torch.from_numpy(cache).to(torch.bfloat16).to(DEV)
    B, Hq, ql, _ = w.q.shape
    idx = torch.empty(B, Hkv, ql, top_k, dtype=torch.int32, device=DEV)
    bsg.group_score_topk(w.q, w.kv_lens, dcache, w.page_table, idx, page_size=spec.page_size)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    s32 = np.sort(sc.astype(np.float32), axis=-1)[..., ::-1]                   # descending
    m = top_k - 1
    nb = s32.shape[-1]
    if m == 0 or m >= nb:
        ok = np.ones(got.shape[:-1], bool)
        ties = 0
    else:
        x, y = s32[..., m - 1], s32[..., m]
        with np.errstate(invalid="ignore"):
            tie = (x == y) & np.isfinite(y)
            far = ~np.isfinite(y) | (np.abs(x - y) > 1e-4 * np.maximum(np.maximum(np.abs(x), np.abs(y)), 1e-30))
        ok = tie | far
        ties = int(tie.sum())
    same = (got == ref).all(-1)
    bad = np.argwhere(ok & ~same)
    checked = int(ok.sum())
    note(f"  rows checked {checked} of {ok.size}, exact ties at the boundary {ties}, mismatches {len(bad)}")
    assert len(bad) == 0, [(tuple(i), got[tuple(i)], ref[tuple(i)]) for i in bad[:3]]
    assert ties > 0 and checked > 0.9 * ok.size


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("case", [dict(), dict(page_size=128, top_k=9), dict(head_dim=64, top_k=8)])
def test_decode_step_wide_page_table(case, fp8):
    """Page-table rows longer than the one-workgroup step takes (4096 blocks) run the chunked
    scan, selection-in-attention and merge kernels; the same sequences behind a wide table must
    give the oracle's result (and, in fp8, the bf16 result on decoded caches bit for bit)."""
    spec = SPECS[2].replace(**{"batch": 3, "ctx_len": 64 * 150 + 11, **case})
    note(f"[case] decode step, wide page table {case} fp8={fp8}")
    w = make_workload(spec, 27, tail_fill=float("nan")).to(DEV)
    wide = torch.zeros(w.page_table.shape[0], 4200, dtype=torch.int32, device=DEV)
    wide[:, :w.page_table.shape[1]] = w.page_table
    B, Hq, _, D = w.q.shape
    Hkv, k = spec.num_kv_heads, spec.top_k
    scale = 1.0 / math.sqrt(D)
    q1 = w.q[:, :, 0].contiguous()
    cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=DEV)
    bsg.block_pool(w.k_cache, wide, w.kv_lens, cache)
    idx = torch.full((B, Hkv, k), -7, dtype=torch.int32, device=DEV)
    out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    if not fp8:
        bsg.decode_step(q1, w.kv_lens, cache, w.k_cache, w.v_cache, wide, scale, idx, out, lse)
        torch.cuda.synchronize()
        check_decode(w, idx, out, lse)
        return
    P = w.k_cache.shape[0]
    bs = spec.page_size
    kc = torch.zeros(P, Hkv, bs, D, dtype=torch.uint8, device=DEV)
    vc = torch.zeros_like(kc)
    ks = torch.ones(P, Hkv, dtype=torch.float32, device=DEV)
    vs = torch.ones_like(ks)
    bsg.quantize_pages_fp8(w.k_cache, wide, w.kv_lens, kc, ks)
    bsg.quantize_pages_fp8(w.v_cache, wide, w.kv_lens, vc, vs)
    rc = torch.zeros(P, Hkv, D, dtype=torch.uint8, device=DEV)
    rs = torch.ones(P, Hkv, dtype=torch.float32, device=DEV)
    bsg.block_pool_fp8(kc, ks, wide, w.kv_lens, rc, rs)
    bsg.decode_step_fp8(q1, w.kv_lens, rc, rs, kc, ks, vc, vs, wide, scale, idx, out, lse)

    def dec(c, s):                     # code values times their (page, head) scale, exact in bf16
        return (c.view(torch.float8_e4m3fn).float() * s.reshape(s.shape + (1,) * (c.dim() - 2))).to(torch.bfloat16)
    kd, vd, rd = dec(kc, ks), dec(vc, vs), dec(rc, rs)
    idx2 = torch.full_like(idx, -7)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    bsg.decode_step(q1, w.kv_lens, rd, kd, vd, wide, scale, idx2, out2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse, lse2)


@pytest.mark.parametrize("nblk,wide", [(2000, False), (4000, False), (2000, True), (4000, True)],
                         ids=["2000", "4000", "2000_wide_table", "4000_wide_table"])
def test_decode_step_selection_with_piled_keys(nblk, wide):
    """Representatives whose scores grow with the block index put every kept block in the last
    groups of candidates, so many keys pass the one-workgroup step's lower bound: about 960
    (ranked directly) at 2000 blocks, about 1900 (the radix select over all keys) at 4000.
    Many scores tie exactly (bf16 representatives), and the lower index must win as in the
    oracle.  Behind a page table wider than 4096 columns the same rows take the chunked scan
    and the selection prologue, where the kept keys fill the last chunks' sorted lists past
    their first 8 keys, so the prologue reads those lists on."""
    spec = SPECS[2].replace(batch=1, ctx_len=64 * nblk + 5, num_q_heads=16, num_kv_heads=2)
    note(f"[case] decode step, piled keys, {nblk} blocks, wide table {wide}")
    w = make_workload(spec, 29).to(DEV)
    B, Hq, _, D = w.q.shape
    Hkv, k, G = spec.num_kv_heads, spec.top_k, spec.group_size
    q, kp, vp, pt, kv = np_inputs(w)
    own = (kv[0] - 1) // 64
    rep = np.zeros((kp.shape[0], Hkv, D), np.float32)
    for g in range(Hkv):
        u = np.sign(q[0, g * G:(g + 1) * G, 0].astype(np.float64).sum(0)).astype(np.float32)
        for j in range(own):
            rep[pt[0, j], g] = (j + 1) / own * u
    rep = O.bf16_value(O.bf16_bits(rep)).astype(np.float32)
    r = O.decode_reference(q, kp, vp, pt, kv, spec.page_size, k, "bf16", 1.0 / math.sqrt(D), block_cache=rep)
    cache = torch.from_numpy(rep).to(torch.bfloat16).to(DEV)
    idx = torch.full((B, Hkv, k), -7, dtype=torch.int32, device=DEV)
    out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    table = w.page_table
    if wide:
        table = torch.zeros(w.page_table.shape[0], 4200, dtype=torch.int32, device=DEV)
        table[:, :w.page_table.shape[1]] = w.page_table
    bsg.decode_step(w.q[:, :, 0].contiguous(), w.kv_lens, cache, w.k_cache, w.v_cache, table,
                    1.0 / math.sqrt(D), idx, out, lse)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), r["block_idx"][:, :, 0])
    check_out(to_np(out), r["out"][:, :, 0], "bf16", "decode out")
    assert np.abs(lse.cpu().numpy() - r["lse"][:, :, 0]).max() <= 2e-3
