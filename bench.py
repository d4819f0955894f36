"""Benchmark: block-sparse GQA attention at 128K context on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--only PARTS]

One step = one pass of the whole hot path over one batch of synthetic input:
  prefill: block_pool -> group_score_topk -> sparse_attn_prefill
  decode:  decode_step = group scores + top-k + sparse attention (the block cache is built beforehand,
           as at the end of a prefill); the step is three short kernels, so 8 steps are captured per
           HIP graph and the graph is replayed
Inputs are generated on the GPU and resident in HBM before timing starts.

The headline workload is the 128K prefill (B=1, S=131072, Hq=64, Hkv=8, D=128, 128-token blocks, top-16);
`value` is its tokens/s.  The same run also reports, as sub-objects:
  prefill_s32768      32K prefill (Hq=32, Hkv=4, 64-token blocks, top-32): per-token random plantings
  decode              128K decode step (B=32, Hq=32, Hkv=4, 64-token shuffled pages, top-32), warm (the same
                      step replayed) and cold (four disjoint workloads in rotation, so that a step's bytes
                      were last touched 3 steps = ~590 MB earlier, beyond the 256 MB Infinity Cache)
  decode_ragged_1m    ragged decode toward 1M (B=4, L ~ U[512K, 1M], Hq=64, Hkv=8, top-32), warm and cold
  decode_fp8, decode_tokens, decode_two_level   the fp8-cache, token-level and two-level decode steps
Kernel times are HIP events on the stream the library launches on, one pair per launch; the JSON gives the
mean (what `ms_per_step` and the roofline use) and the median.

`roofline` covers the dominant kernel (prefill attention): algorithmic FLOPs per launch (4*D per selected,
causally valid key per query head, counted from the actual selection) over the mean launch time.  Its
`traffic` and `mfma_util` come from committed rocprofv3 counter summaries under profiles/ and are null
when the kernel source has changed since they were taken.

`cpu_baseline` is the CPU oracle on the host's cores (a process pool, one worker per core of the affinity
mask, at most 16), timed on bounded samples of the same workloads and extrapolated linearly.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-sparse GQA attn: prefill tok/s + decode µs/step at 128K, % roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PROFILE_DIR = os.path.join(ROOT, "profiles")
PER_GRAPH = 8               # decode steps captured per HIP graph


def _kernel_hash(*files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "block_sparse_gqa_pool_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _profile_record(name: str, src_files):
    """A committed counter summary (profiles/<name>.json) if it matches the current kernel source."""
    path = os.path.join(PROFILE_DIR, f"{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != _kernel_hash(*src_files):
        return None
    return rec


def _traffic(kernel_key: str):
    """HBM bytes per launch from the committed counters of TRAFFIC_KERNELS[kernel_key], if the kernel's
    sources still hash as they did when the counters were taken."""
    rec = _profile_record(f"{kernel_key}_traffic", TRAFFIC_KERNELS[kernel_key][1])
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def _stats(xs):
    return dict(mean=sum(xs) / len(xs), median=statistics.median(xs), min=min(xs), n=len(xs))


# ------------------------------------------------------------------------------------ work counts
def prefill_flops(block_idx, kv_lens, q_len, page_size, G, D):
    """4*D FLOPs per (query head, selected key at a position <= the query)."""
    import torch
    B, Hkv, T, k = block_idx.shape
    pos = (kv_lens.view(B, 1, 1, 1).long() - q_len + torch.arange(T, device=block_idx.device).view(1, 1, T, 1))
    j = block_idx.long()
    n = torch.clamp(pos - j * page_size + 1, min=0, max=page_size)
    n = torch.where(j >= 0, n, torch.zeros_like(n))
    return float(n.sum().item()) * G * 4 * D


def prefill_tile_stats(block_idx, kv_lens, q_len, page_size, G, D):
    """What the matrix-core prefill kernel processes for this selection.

    A workgroup takes 256 query rows = TT tokens x HG heads of one group (HG = largest power of two
    dividing G, at most 32) and streams the union of its tokens' blocks once; each wave takes 32 rows
    (WT = 32 / HG tokens) and runs every 64-key sub-block that one of its rows attends to.  Returns the
    mean union size per workgroup, the K/V bytes the unions stream, and the FLOPs the waves issue
    (32 rows x 64 keys x 4 D per processed sub-block) against the algorithmic count."""
    import torch
    B, Hkv, T, k = block_idx.shape
    HG = 1
    while HG < 32 and G % (HG * 2) == 0:
        HG *= 2
    TT, WT = 256 // HG, 32 // HG
    dev = block_idx.device
    nb = int(block_idx.max().item()) + 1
    pos = kv_lens.view(B, 1, 1).long() - q_len + torch.arange(T, device=dev).view(1, 1, T)     # [B,1,T]
    unions, issued_sub = 0, 0
    for b in range(B):
        for g in range(Hkv):
            idx = block_idx[b, g].long()                                                    # [T, k]
            p = pos[b, 0].view(T, 1).expand(T, k)
            Tp = (T + TT - 1) // TT * TT
            idxp = torch.full((Tp, k), -1, dtype=torch.long, device=dev)
            idxp[:T] = idx
            pp = torch.full((Tp, k), -1, dtype=torch.long, device=dev)
            pp[:T] = p
            # union per workgroup tile
            tiles = idxp.view(Tp // TT, TT * k)
            mask = torch.zeros(Tp // TT, nb + 1, dtype=torch.bool, device=dev)
            mask.scatter_(1, tiles.clamp(min=-1) + 1, True)
            unions += int(mask[:, 1:].sum().item())
            # per wave: for each selected block the furthest query position among the wave's rows
            w_idx = idxp.view(Tp // WT, WT * k)
            w_pos = pp.view(Tp // WT, WT * k)
            mx = torch.full((Tp // WT, nb + 1), -1, dtype=torch.long, device=dev)
            mx.scatter_reduce_(1, w_idx + 1, w_pos, reduce="amax")
            mx = mx[:, 1:]
            jb = torch.arange(nb, device=dev).view(1, nb) * page_size
            nsub = torch.clamp((mx - jb) // 64 + 1, min=0, max=page_size // 64)
            nsub = torch.where(mx >= 0, nsub, torch.zeros_like(nsub))
            issued_sub += int(nsub.sum().item())
    n_tiles = B * Hkv * ((T + TT - 1) // TT) * (G // HG)
    issued = float(issued_sub) * (G // HG) * HG * (32 // HG) * 64 * 4 * D
    return dict(rows_per_workgroup=256, tokens_per_workgroup=TT, tokens_per_wave=WT,
                mean_union_blocks=unions * (G // HG) / n_tiles,
                union_kv_bytes=float(unions) * (G // HG) * page_size * D * 2 * 2,
                issued_flops=issued)


def decode_bytes(block_idx, kv_lens, page_size, Hkv, D, elem=2):
    """Selected K+V bytes + block-cache bytes of every candidate + page-table bytes (elem = 1:
    fp8 caches, plus one 4-byte scale per selected K and V page and per candidate)."""
    import torch
    B = block_idx.shape[0]
    pos = kv_lens.view(B, 1, 1).long() - 1
    j = block_idx.view(B, Hkv, -1).long()
    n = torch.clamp(pos - j * page_size + 1, min=0, max=page_size)
    n = torch.where(j >= 0, n, torch.zeros_like(n))
    kv = float(n.sum().item()) * D * elem * 2
    own = (kv_lens.long() - 1) // page_size
    reps = float(own.sum().item()) * Hkv * D * elem
    pt = float((own + 1).sum().item()) * 4
    if elem != 1:
        return kv + reps + pt, dict(selected_kv=kv, block_cache=reps, page_table=pt)
    sc = float((j >= 0).sum().item()) * 8 + float(own.sum().item()) * Hkv * 4
    return kv + reps + pt + sc, dict(selected_kv=kv, block_cache=reps, page_table=pt, scales=sc)


# ------------------------------------------------------------------------------------ prefill
def planted_recall(idx, w):
    """Share of the generator's planted blocks that the device selection kept.  The planted blocks
    are the group's true top blocks by construction, so this is the recall check of the index (a
    soft quality figure, not parity).  idx: device [B, Hkv, q_len, k] logical block ids."""
    import torch
    B, Hkv, q_len, k = idx.shape
    dev = idx.device
    if w.planted is not None:
        pl = w.planted.to(dev)                                        # [B, Hkv, q_len, n]
    else:
        pr = w.planted_region.to(dev)                                 # [B, Hkv, regions, n]
        pl = torch.empty(B, Hkv, q_len, pr.shape[-1], dtype=pr.dtype, device=dev)
        for b in range(B):
            pos = torch.arange(w.kv_lens_host[b] - q_len, w.kv_lens_host[b], device=dev)
            pl[b] = pr[b][:, pos // w.spec.region]
    hit = torch.zeros((), dtype=torch.int64, device=dev)
    tot = torch.zeros((), dtype=torch.int64, device=dev)
    step = max(1, (1 << 27) // max(1, B * Hkv * k * pl.shape[-1]))   # bound the comparison's memory
    for t0 in range(0, q_len, step):
        p = pl[:, :, t0:t0 + step]
        got = (idx[:, :, t0:t0 + step, None, :] == p[..., None]).any(-1) & (p >= 0)
        hit += got.sum()
        tot += (p >= 0).sum()
    n = int(tot)
    return {"planted": n, "kept": int(hit), "recall": (int(hit) / n) if n else None}


def run_prefill(spec, seed, steps, warmup, tile_stats=False, keep_ranges=None):
    """keep_ranges: (starts, length) of query ranges whose device selections and outputs are copied
    to the host (for the oracle comparison of the cpu_baseline leg)."""
    import torch
    import block_sparse_gqa_pool_amd as bsg
    from workloads import make_workload

    dev = torch.device("cuda:0")
    w = make_workload(spec, seed, device=dev)
    B, Hq, S, D = w.q.shape
    Hkv, bs, k = spec.num_kv_heads, spec.page_size, spec.top_k
    scale = 1.0 / math.sqrt(D)
    cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=dev)
    idx = torch.empty(B, Hkv, S, k, dtype=torch.int32, device=dev)
    out = torch.empty_like(w.q)
    need = bsg.group_score_topk_workspace_bytes(w.q, cache, w.page_table, bs, k)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
        if ev:
            ev[1].record(stream)
        bsg.group_score_topk(w.q, w.kv_lens, cache, w.page_table, idx, page_size=bs, workspace=ws)
        if ev:
            ev[2].record(stream)
        bsg.sparse_attn_prefill(w.q, w.kv_lens, w.k_cache, w.v_cache, w.page_table, idx, scale, out)
        if ev:
            ev[3].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    names = ("block_pool", "group_score_topk", "sparse_attn_prefill")
    stage = {n: _stats([e[i].elapsed_time(e[i + 1]) for e in evs]) for i, n in enumerate(names)}
    step_ms = [e[0].elapsed_time(e[3]) for e in evs]
    flops = prefill_flops(idx, w.kv_lens, S, bs, spec.group_size, D)
    res = dict(tokens=B * S, wall_s=wall, ms_per_step=sum(step_ms) / steps, wall_ms_per_step=1e3 * wall / steps,
               stage=stage, attn_flops=flops)
    if tile_stats:
        res["tiles"] = prefill_tile_stats(idx, w.kv_lens, S, bs, spec.group_size, D)
    res["planted_recall"] = planted_recall(idx, w)
    if keep_ranges is not None:
        starts, n = keep_ranges
        res["kept_rows"] = [(int(t0), idx[:, :, t0:t0 + n].cpu().numpy(), out[:, :, t0:t0 + n].float().cpu().numpy())
                            for t0 in starts]
    del w, cache, idx, out, ws
    torch.cuda.empty_cache()
    return res


def prefill_line(spec, r):
    attn = r["stage"]["sparse_attn_prefill"]
    achieved = r["attn_flops"] / (attn["mean"] / 1e3) / 1e12
    d = {"workload": spec.name, "tok_per_s": r["tokens"] / (r["ms_per_step"] / 1e3), "ms_per_step": r["ms_per_step"],
         "stages_ms": {n: {"mean": s["mean"], "median": s["median"]} for n, s in r["stage"].items()},
         "roofline": {"kernel": "sparse_attn_prefill", "bound": "mfma", "achieved": achieved,
                      "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                      "flops_per_launch": r["attn_flops"], "avg_launch_ms": attn["mean"],
                      "median_launch_ms": attn["median"], "launches": attn["n"]},
         "pipeline_mfma_frac": (r["attn_flops"] / (r["ms_per_step"] / 1e3) / 1e12) / PEAK_BF16_TFLOPS}
    if "tiles" in r:
        t = r["tiles"]
        d["tiles"] = dict(t, selected_over_issued=r["attn_flops"] / t["issued_flops"])
    if "planted_recall" in r:
        d["planted_recall"] = r["planted_recall"]
    return d


def run_prefill_tokens(spec, seed, steps, warmup, K, two):
    """Token-level (two False) or two-level prefill of the workload: [block_pool + block
    selection,] token scores + top-K, attention over the kept tokens; HIP events per stage.
    Work counts from the device selections: candidates scored (per row and group), tokens
    attended."""
    import torch
    import block_sparse_gqa_pool_amd as bsg
    from workloads import make_workload

    dev = torch.device("cuda:0")
    w = make_workload(spec, seed, device=dev)
    B, Hq, S, D = w.q.shape
    Hkv, bs, k = spec.num_kv_heads, spec.page_size, spec.top_k
    scale = 1.0 / math.sqrt(D)
    cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=dev)
    bidx = torch.empty(B, Hkv, S, k, dtype=torch.int32, device=dev) if two else None
    tok = torch.empty(B, Hkv, S, K, dtype=torch.int32, device=dev)
    out = torch.empty_like(w.q)
    d = bsg.dims(w.k_cache, w.page_table, Hq, k if two else 1)
    ws = torch.empty(int(bsg.lib().bsg_token_topk_prefill_workspace_bytes(__import__("ctypes").byref(d), S, int(two))),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        if two:
            bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
            bsg.group_score_topk(w.q, w.kv_lens, cache, w.page_table, bidx, page_size=bs)
        if ev:
            ev[1].record(stream)
        bsg.token_topk_prefill(w.q, w.kv_lens, w.k_cache, w.page_table, tok, block_idx=bidx, workspace=ws)
        if ev:
            ev[2].record(stream)
        bsg.sparse_attn_prefill_tokens(w.q, w.kv_lens, w.k_cache, w.v_cache, w.page_table, tok, scale, out)
        if ev:
            ev[3].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    names = ("block_selection", "token_topk_prefill", "sparse_attn_prefill_tokens")
    stage = {n: _stats([e[i].elapsed_time(e[i + 1]) for e in evs]) for i, n in enumerate(names)}
    if not two:
        del stage["block_selection"]
    step_ms = [e[0].elapsed_time(e[3]) for e in evs]
    L = int(w.kv_lens_host[0])
    pos = torch.arange(S, dtype=torch.float64) + (L - S)
    if two:                                          # candidates: the valid tokens of the kept blocks
        j = bidx.long()
        nk = torch.clamp(pos.to(dev).view(1, 1, S, 1) - j * bs + 1, min=0, max=bs)
        cand = float(torch.where(j >= 0, nk, torch.zeros_like(nk)).sum().item())
    else:
        cand = float((pos + 1).sum().item()) * B * Hkv
    kept = float((tok >= 0).sum().item())
    res = dict(tokens=B * S, ms_per_step=sum(step_ms) / steps, stage=stage, K=K,
               score_flops=2.0 * D * cand, score_bytes=8.0 * cand, candidates=cand,
               attn_flops=4.0 * D * spec.group_size * kept, attn_kv_bytes=4.0 * D * kept, kept_tokens=kept)
    del w, cache, bidx, tok, out, ws
    torch.cuda.empty_cache()
    return res


def prefill_tokens_line(spec, r, two):
    sel = r["stage"]["token_topk_prefill"]
    att = r["stage"]["sparse_attn_prefill_tokens"]
    a_tf = r["attn_flops"] / (att["mean"] / 1e3) / 1e12
    s_gbs = r["score_bytes"] / (sel["mean"] / 1e3) / 1e9
    d = {"workload": spec.name + (f" (block top-{spec.top_k}, then token top-{r['K']})" if two
                                  else f" (token top-{r['K']}, identity indexer)"),
         "api": ("bsg_group_score_topk + " if two else "") + "bsg_token_topk_prefill + bsg_sparse_attn_prefill_tokens",
         "tok_per_s": r["tokens"] / (r["ms_per_step"] / 1e3), "ms_per_step": r["ms_per_step"],
         "stages_ms": {n: {"mean": x["mean"], "median": x["median"]} for n, x in r["stage"].items()},
         "selection": {"bound": "hbm", "achieved": s_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": s_gbs / PEAK_HBM_GBS, "bytes_per_launch": r["score_bytes"],
                       "bytes_basis": "each candidate's fp32 score written once and read once",
                       "score_tflops": r["score_flops"] / (sel["mean"] / 1e3) / 1e12,
                       "candidates": r["candidates"]},
         "attention": {"bound": "mfma", "achieved": a_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                       "frac": a_tf / PEAK_BF16_TFLOPS, "flops_per_launch": r["attn_flops"],
                       "kv_gather_gbs": r["attn_kv_bytes"] / (att["mean"] / 1e3) / 1e9,
                       "kept_tokens": r["kept_tokens"]}}
    return d


# ------------------------------------------------------------------------------------ decode
def _decode_setup(spec, seed, dev, fp8=False):
    """One decode workload on the device with its block cache built (as at the end of a prefill)."""
    import torch
    import block_sparse_gqa_pool_amd as bsg
    from workloads import make_workload

    w = make_workload(spec, seed, device=dev)
    B, Hq, _, D = w.q.shape
    Hkv, bs, k = spec.num_kv_heads, spec.page_size, spec.top_k
    s = dict(w=w, q1=w.q[:, :, 0].contiguous(), idx=torch.empty(B, Hkv, k, dtype=torch.int32, device=dev),
             out=torch.empty(B, Hq, D, dtype=w.q.dtype, device=dev),
             ws=torch.empty(bsg.decode_step_workspace_bytes(w.k_cache, w.page_table, Hq, k), dtype=torch.uint8,
                            device=dev))
    if not fp8:
        cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=dev)
        bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
        s["cache"] = cache
        return s
    # fp8 caches, quantised from the bf16 ones at prefill; the bf16 caches are freed
    P = w.k_cache.shape[0]
    kc = torch.zeros(P, Hkv, bs, D, dtype=torch.uint8, device=dev)
    vc = torch.zeros_like(kc)
    ks = torch.ones(P, Hkv, dtype=torch.float32, device=dev)
    vs = torch.ones_like(ks)
    bsg.quantize_pages_fp8(w.k_cache, w.page_table, w.kv_lens, kc, ks)
    bsg.quantize_pages_fp8(w.v_cache, w.page_table, w.kv_lens, vc, vs)
    rc = torch.zeros(P, Hkv, D, dtype=torch.uint8, device=dev)
    rs = torch.ones(P, Hkv, dtype=torch.float32, device=dev)
    bsg.block_pool_fp8(kc, ks, w.page_table, w.kv_lens, rc, rs)
    w.k_cache = w.v_cache = None
    s.update(kc=kc, ks=ks, vc=vc, vs=vs, rc=rc, rs=rs)
    return s


def _decode_call(s, scale, fp8):
    import block_sparse_gqa_pool_amd as bsg
    w = s["w"]
    if fp8:
        bsg.decode_step_fp8(s["q1"], w.kv_lens, s["rc"], s["rs"], s["kc"], s["ks"], s["vc"], s["vs"], w.page_table,
                            scale, s["idx"], s["out"], workspace=s["ws"])
    else:
        bsg.decode_step(s["q1"], w.kv_lens, s["cache"], w.k_cache, w.v_cache, w.page_table, scale, s["idx"],
                        s["out"], workspace=s["ws"])


def run_decode(spec, seed, steps, warmup, fp8=False, rotate=1, graph_replay=True):
    """Decode steps captured PER_GRAPH to a HIP graph and replayed; with rotate = R > 1 the steps cycle
    through R workloads of different seeds (disjoint caches and queries), so every step finds its bytes
    evicted from the last-level cache by the R - 1 steps before it."""
    import torch

    dev = torch.device("cuda:0")
    sets = [_decode_setup(spec, seed + 1000 * r, dev, fp8) for r in range(rotate)]
    D = spec.head_dim
    scale = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream()
    for _ in range(max(warmup, 1)):
        for s in sets:
            _decode_call(s, scale, fp8)
    torch.cuda.synchronize()
    if not graph_replay:                      # eager steps (counter collection)
        for i in range(steps):
            _decode_call(sets[i % rotate], scale, fp8)
        torch.cuda.synchronize()
        del sets
        torch.cuda.empty_cache()
        return None
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(PER_GRAPH):
            _decode_call(sets[i % rotate], scale, fp8)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    n_rep = max(1, (steps + PER_GRAPH - 1) // PER_GRAPH)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_rep)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = [1e3 * a.elapsed_time(b) / PER_GRAPH for a, b in evs]      # us
    parts = [decode_bytes(s["idx"], s["w"].kv_lens, spec.page_size, spec.num_kv_heads, D, elem=1 if fp8 else 2)
             for s in sets]
    nbytes = sum(p[0] for p in parts) / rotate
    res = dict(us=_stats(per_step), wall_us_per_step=1e6 * wall / (n_rep * PER_GRAPH), bytes=nbytes,
               bytes_parts=parts[0][1], steps=n_rep * PER_GRAPH,
               planted_recall=planted_recall(sets[0]["idx"][:, :, None, :], sets[0]["w"]))
    del graph, sets
    torch.cuda.empty_cache()
    return res


def decode_line(spec, d, api, traffic=None, cold=None):
    def roof(r):
        us = r["us"]["mean"]
        gbs = r["bytes"] / (us / 1e6) / 1e9
        return {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                "bytes_per_step": r["bytes"]}
    line = {"workload": spec.name, "api": api, "us_per_step": d["us"]["mean"], "us_per_step_median": d["us"]["median"],
            "steps": d["steps"], "timing": f"{PER_GRAPH} steps per HIP graph replay, HIP events per replay",
            "roofline": dict(roof(d), bytes_parts=d["bytes_parts"], traffic=traffic)}
    if "planted_recall" in d:
        line["planted_recall"] = d["planted_recall"]
    if cold is not None:
        line["cold"] = {"us_per_step": cold["us"]["mean"], "us_per_step_median": cold["us"]["median"],
                        "steps": cold["steps"], "rotation": "4 workloads of different seeds, cycled step by step",
                        "roofline": roof(cold)}
    return line


def run_decode_tokens(spec, seed, steps, warmup, top_k_tokens, two_level):
    """Token-level (two_level False) or two-level decode steps, graph-replayed like run_decode.
    Algorithmic bytes: token level reads every key once (the identity indexer scores all
    tokens) plus the kept tokens' values and the page table; two level reads the block cache
    of every candidate, the keys of the kept blocks, and the kept tokens' values."""
    import ctypes
    import torch
    import block_sparse_gqa_pool_amd as bsg
    from workloads import make_workload

    dev = torch.device("cuda:0")
    w = make_workload(spec, seed, device=dev)
    B, Hq, _, D = w.q.shape
    Hkv, bs, k = spec.num_kv_heads, spec.page_size, spec.top_k
    scale = 1.0 / math.sqrt(D)
    q1 = w.q[:, :, 0].contiguous()
    out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=dev)
    tok = torch.empty(B, Hkv, top_k_tokens, dtype=torch.int32, device=dev)
    cache = bidx = None
    if two_level:
        cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=dev)
        bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)
        bidx = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
    d = bsg.dims(w.k_cache, w.page_table, Hq, k if two_level else 1)
    need = int(bsg.lib().bsg_decode_step_tokens_workspace_bytes(ctypes.byref(d), top_k_tokens, int(two_level)))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        bsg.decode_step_tokens(q1, w.kv_lens, w.k_cache, w.v_cache, w.page_table, scale, tok, out,
                               block_cache=cache, block_idx=bidx, workspace=ws)

    per = 4
    for _ in range(max(warmup, 1)):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per):
            step()
    graph.replay()
    torch.cuda.synchronize()
    n_rep = max(1, (steps + per - 1) // per)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_rep)]
    for a, b in evs:
        a.record(stream)
        graph.replay()
        b.record(stream)
    torch.cuda.synchronize()
    us = _stats([1e3 * a.elapsed_time(b) / per for a, b in evs])
    L = w.kv_lens.long()
    kept = float((tok >= 0).sum().item())
    v_bytes = kept * D * 2
    pt = float(((L + bs - 1) // bs).sum().item()) * 4
    if two_level:
        own = (L - 1) // bs
        reps = float(own.sum().item()) * Hkv * D * 2
        nb = float((bidx >= 0).sum().item())
        parts = dict(block_cache=reps, kept_block_keys=nb * bs * D * 2, kept_token_values=v_bytes, page_table=pt)
    else:
        parts = dict(all_keys=float(L.sum().item()) * Hkv * D * 2, kept_token_values=v_bytes, page_table=pt)
    nbytes = sum(parts.values())
    del graph, w, cache, bidx, tok, out, ws
    torch.cuda.empty_cache()
    gbt = nbytes / (us["mean"] / 1e6) / 1e9
    return {"us_per_step": us["mean"], "us_per_step_median": us["median"], "api": "bsg_decode_step_tokens",
            "steps": n_rep * per, "timing": f"{per} steps per HIP graph replay, HIP events per replay",
            "roofline": {"bound": "hbm", "achieved": gbt, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbt / PEAK_HBM_GBS, "bytes_per_step": nbytes, "bytes_parts": parts,
                         "traffic": None}}


# ------------------------------------------------------------------------------------ CPU oracle
# The oracle runs in spawned worker processes (one per core, no GPU); the paged pools reach them as
# memory-mapped float32 files, queries and tables as task arguments.
_ORACLE = {}


def _oracle_worker_init(paths):
    import numpy as np
    try:                                   # one BLAS thread per worker: the pool supplies the parallelism
        from threadpoolctl import threadpool_limits
        _ORACLE["blas"] = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass
    for name, (path, shape) in paths.items():
        _ORACLE[name] = np.memmap(path, dtype=np.float32, mode="r", shape=tuple(shape))


def _oracle_noop(_):
    return os.getpid()


def _oracle_prefill_range(args):
    """Oracle scores, top-k and attention for the queries [t0, t0 + n) of a prefill: the chunk of a
    prefill whose queries end at position t0 + n - 1, i.e. kv_len = t0 + n, q_len = n."""
    import oracle as O
    q_rows, pt, t0, Hkv, bs, k, scale = args[:7]
    n = q_rows.shape[2]
    kv = [t0 + n]
    sc = O.group_scores(q_rows, _ORACLE["cache"], pt, kv, Hkv, bs)
    idx = O.select_blocks(sc, kv, n, bs, k)
    out, _ = O.sparse_attention(q_rows, _ORACLE["k"], _ORACLE["v"], pt, kv, idx, scale)
    if len(args) == 7:
        return n, None
    return n, _compare_rows(args[7], args[8], idx, out, sc, k)


def _compare_rows(gpu_idx, gpu_out, ora_idx, ora_out, scores, k, tie_rel=1e-4):
    """Device selections and outputs of sampled rows against the oracle's: rows whose selection
    differs (and how many of those lie inside the tie window: the oracle's last kept and first
    dropped candidates within tie_rel of each other, every differing block inside that window),
    and the absolute output errors."""
    import numpy as np
    diff = np.nonzero((gpu_idx != ora_idx).any(-1))
    exempt = 0
    for b, g, t in zip(*diff):
        row = scores[b, g, t]
        own = int(ora_idx[b, g, t][ora_idx[b, g, t] >= 0][-1])
        cands = sorted(range(own), key=lambda j: (-np.float32(row[j]), j))
        m = k - 1
        if len(cands) > m >= 1:
            sa, sb = row[cands[m - 1]], row[cands[m]]
            win = tie_rel * max(abs(sa), abs(sb))
            sym = set(int(x) for x in gpu_idx[b, g, t] if x >= 0) ^ set(int(x) for x in ora_idx[b, g, t] if x >= 0)
            if abs(sa - sb) < win and all(abs(row[j] - sa) <= win or abs(row[j] - sb) <= win for j in sym if j < own):
                exempt += 1
    err = np.abs(gpu_out.astype(np.float64) - ora_out)
    return dict(rows=int(np.prod(gpu_idx.shape[:3])), idx_rows_differing=int(len(diff[0])), idx_rows_in_tie_window=exempt,
                out_max_abs_err=float(err.max()), out_abs_err_sum=float(err.sum()), out_elems=int(err.size))


def _oracle_decode_seq(args):
    """Oracle decode step (scores, top-k, attention) of one sequence; the block cache is given."""
    import oracle as O
    q1, pt, kv, Hkv, bs, k, scale = args
    sc = O.group_scores(q1, _ORACLE["cache"], pt, kv, Hkv, bs)
    idx = O.select_blocks(sc, kv, 1, bs, k)
    O.sparse_attention(q1, _ORACLE["k"], _ORACLE["v"], pt, kv, idx, scale)
    return 1


def _host_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _memmaps(tmp, arrays):
    import numpy as np
    paths = {}
    for name, a in arrays.items():
        path = os.path.join(tmp, name + ".f32")
        mm = np.memmap(path, dtype=np.float32, mode="w+", shape=a.shape)
        mm[:] = a
        mm.flush()
        del mm
        paths[name] = (path, list(a.shape))
    return paths


def _pool(paths, n):
    import concurrent.futures as cf
    import multiprocessing as mp
    ex = cf.ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"), initializer=_oracle_worker_init,
                                initargs=(paths,))
    list(ex.map(_oracle_noop, range(4 * n)))      # start every worker before timing
    return ex


BASELINE_RANGES = (32, 192)       # query ranges x tokens the prefill cpu_baseline samples


def baseline_ranges(S, n_ranges=BASELINE_RANGES[0], range_len=BASELINE_RANGES[1]):
    import numpy as np
    return np.linspace(0, S - range_len, n_ranges).astype(np.int64), range_len


def cpu_baseline_prefill(spec, seed, n_ranges=BASELINE_RANGES[0], range_len=BASELINE_RANGES[1], kept_rows=None):
    """The oracle on the host's cores: the block pool over all blocks (one process, vectorised), then
    scores + top-k + attention for n_ranges query ranges of range_len tokens spread over the sequence,
    extrapolated linearly to all tokens."""
    import numpy as np
    import torch
    import oracle as O
    from workloads import make_workload

    w = make_workload(spec, seed, device="cuda:0" if torch.cuda.is_available() else "cpu")
    kp = w.k_cache.float().cpu().numpy()
    vp = w.v_cache.float().cpu().numpy()
    pt = w.page_table.cpu().numpy()
    kv = list(w.kv_lens_host)
    S = w.q.shape[2]
    starts, _ = baseline_ranges(S, n_ranges, range_len)
    q_rows = [w.q[:, :, t0:t0 + range_len].float().cpu().numpy() for t0 in starts]
    gpu = {t0: (gi, go) for t0, gi, go in kept_rows} if kept_rows else {}
    del w
    torch.cuda.empty_cache()
    t0 = time.perf_counter()
    cache = O.block_pool(kp, pt, kv, spec.dtype)
    t_pool = time.perf_counter() - t0
    nw = _host_workers()
    scale = 1.0 / math.sqrt(spec.head_dim)
    with tempfile.TemporaryDirectory() as tmp:
        paths = _memmaps(tmp, dict(k=kp, v=vp, cache=cache))
        del kp, vp
        ex = _pool(paths, nw)
        try:
            t1 = time.perf_counter()
            res = list(ex.map(_oracle_prefill_range, [(q, pt, int(s), spec.num_kv_heads, spec.page_size, spec.top_k,
                                                        scale) + tuple(gpu.get(int(s), ())) for q, s in zip(q_rows, starts)]))
            t_att = time.perf_counter() - t1
        finally:
            ex.shutdown()
    done = sum(r[0] for r in res)
    cmp = [r[1] for r in res if r[1] is not None]
    parity = None
    if cmp:
        parity = {key: sum(c[key] for c in cmp) for key in ("rows", "idx_rows_differing", "idx_rows_in_tie_window",
                                                            "out_elems")}
        parity["out_max_abs_err"] = max(c["out_max_abs_err"] for c in cmp)
        parity["out_mean_abs_err"] = sum(c["out_abs_err_sum"] for c in cmp) / parity.pop("out_elems")
        parity["sample"] = (f"the device's selections and outputs of the same {done} query tokens (all heads) from the "
                            "timed prefill steps, against the oracle")
    est = t_pool + t_att / done * S
    return dict(value=S / est, unit="tok/s", cores=nw, kind="oracle", parity=parity,
                sample=(f"block_pool over all {pt.shape[1]} blocks ({t_pool:.1f} s, one process) + scores, top-k and "
                        f"attention for {n_ranges} query ranges of {range_len} tokens spread over the sequence "
                        f"({done} tokens, {t_att:.1f} s wall on {nw} worker processes), extrapolated linearly to all "
                        f"{S} tokens: {est:.0f} s per prefill"),
                seconds=t_pool + t_att)


def cpu_baseline_decode(spec, seed, n_sample=8, n_steps=5):
    """The oracle decode step on the host's cores: the pages of n_sample sequences are taken from the
    workload, their block cache built beforehand (as on the GPU); one step = all B sequences, each a
    task (sequence b runs sample b mod n_sample); median of n_steps steps."""
    import numpy as np
    import torch
    import oracle as O
    from workloads import make_workload

    w = make_workload(spec, seed, device="cuda:0" if torch.cuda.is_available() else "cpu")
    B = w.q.shape[0]
    bs = spec.page_size
    seqs = list(range(min(n_sample, B)))
    pt_full = w.page_table.cpu().numpy()
    rows, pages = [], []
    for b in seqs:
        n = (w.kv_lens_host[b] + bs - 1) // bs
        rows.append((len(pages), n))
        pages.extend(pt_full[b, :n].tolist())
    sel = torch.tensor(pages, dtype=torch.int64, device=w.k_cache.device)
    kp = w.k_cache.index_select(0, sel).float().cpu().numpy()
    vp = w.v_cache.index_select(0, sel).float().cpu().numpy()
    q = [w.q[b:b + 1].float().cpu().numpy() for b in seqs]
    kvs = [w.kv_lens_host[b] for b in seqs]
    del w, sel
    torch.cuda.empty_cache()
    pts = []
    for o, n in rows:
        pts.append(np.arange(o, o + n, dtype=np.int32)[None, :])
    cache = np.zeros((kp.shape[0], spec.num_kv_heads, spec.head_dim), np.float32)
    for i in range(len(seqs)):
        cache = O.block_pool(kp, pts[i], [kvs[i]], spec.dtype, block_cache=cache)
    nw = _host_workers()
    scale = 1.0 / math.sqrt(spec.head_dim)
    tasks = [(q[b % len(seqs)], pts[b % len(seqs)], [kvs[b % len(seqs)]], spec.num_kv_heads, bs, spec.top_k, scale)
             for b in range(B)]
    with tempfile.TemporaryDirectory() as tmp:
        paths = _memmaps(tmp, dict(k=kp, v=vp, cache=cache))
        del kp, vp
        ex = _pool(paths, nw)
        try:
            times = []
            for _ in range(n_steps):
                t1 = time.perf_counter()
                list(ex.map(_oracle_decode_seq, tasks))
                times.append(time.perf_counter() - t1)
        finally:
            ex.shutdown()
    med = statistics.median(times)
    return dict(value=1e6 * med, unit="us/step", cores=nw, kind="oracle",
                sample=(f"one step = all {B} sequences (sequence b replays sampled sequence b mod {len(seqs)}: "
                        f"their pages and block cache, built beforehand), {B} tasks on {nw} worker processes; "
                        f"median of {n_steps} steps"),
                seconds=sum(times))


# ------------------------------------------------------------------------------------ counters
# HBM traffic (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE) and matrix-core utilisation of the kernels
TRAFFIC_KERNELS = {
    # key: (kernel-name substring, source files, workload); the fp8 instantiations carry F8 = true
    "sparse_attn_prefill_s131072": ("attn_prefill_mfma", ["attn_prefill.hip", "bsg_device.h"], "prefill_bf16_s131072"),
    "decode_unit_b32_ctx131072": ("decode_unit_kernel<128, 64, false>", ["attn_decode.hip", "decode_prologue.h", "bsg_device.h"],
                                  "decode_bf16_b32_ctx131072"),
    "decode_merge_b32_ctx131072": ("attn_decode_merge_kernel<unsigned short, 128>", ["attn_decode.hip", "bsg_device.h"],
                                   "decode_bf16_b32_ctx131072 (bf16 and fp8 steps)"),
    "decode_fp8_unit_b32_ctx131072": ("decode_unit_kernel<128, 64, true>", ["attn_decode.hip", "decode_prologue.h", "bsg_device.h"],
                                      "decode_bf16_b32_ctx131072 in fp8"),
}
CALIB_BYTES = 1 << 30
# matrix-core counters of the prefill attention kernel: one rocprofv3 pass
MFMA_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
                 "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_WAVES", "GRBM_GUI_ACTIVE"]
NUM_SIMDS = 1024            # 256 CUs x 4 SIMDs
NUM_XCDS = 8


def traffic_run():
    """One prefill step, bf16 and fp8 decode steps, then a calibration copy of CALIB_BYTES (run under rocprofv3 --pmc)."""
    import torch
    from workloads import spec_by_name, SPECS
    sp = spec_by_name("prefill_bf16_s131072")
    run_prefill(sp, SPECS.index(sp), 1, 0)
    sd = spec_by_name("decode_bf16_b32_ctx131072")
    run_decode(sd, SPECS.index(sd), 4, 0, graph_replay=False)
    run_decode(sd, SPECS.index(sd), 4, 0, graph_replay=False, fp8=True)
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)          # the last dispatch: reads and writes CALIB_BYTES
    torch.cuda.synchronize()
    print("traffic run done", flush=True)


def counter_run():
    """Prefill steps of the 128K and 32K workloads (run under rocprofv3 --pmc MFMA_COUNTERS)."""
    from workloads import spec_by_name, SPECS
    for name in ("prefill_bf16_s131072", "prefill_bf16_s32768"):
        sp = spec_by_name(name)
        run_prefill(sp, SPECS.index(sp), 2, 1)
        print(f"counter run: {name} done", flush=True)


def _pmc_rows(directory):
    import csv
    import glob
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {directory}")
    rows = list(csv.DictReader(open(files[0])))
    per = {}
    for r in rows:
        did = int(r["Dispatch_Id"])
        e = per.setdefault(did, {"name": r["Kernel_Name"], "val": 0.0, "counters": {}})
        v = float(r["Counter_Value"])
        e["val"] += v
        e["counters"][r["Counter_Name"]] = e["counters"].get(r["Counter_Name"], 0.0) + v
    return [per[k] for k in sorted(per)]


def summarize_traffic(fetch_dir, write_dir):
    fetch, write = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    f_cal, w_cal = fetch[-1]["val"], write[-1]["val"]          # KiB read / written by the copy
    kf = CALIB_BYTES / (f_cal * 1024.0)
    kw = CALIB_BYTES / (w_cal * 1024.0)
    os.makedirs(PROFILE_DIR, exist_ok=True)
    lines = []
    for key, (sub, files, wl) in TRAFFIC_KERNELS.items():
        fv = [r["val"] for r in fetch if sub in r["name"]]
        wv = [r["val"] for r in write if sub in r["name"]]
        if not fv or not wv:
            continue
        f_b = sum(fv) / len(fv) * 1024.0 * kf
        w_b = sum(wv) / len(wv) * 1024.0 * kw
        rec = {"kernel": sub, "workload": wl, "source_hash": _kernel_hash(*files), "hbm_bytes_per_launch": f_b + w_b,
               "fetch_bytes_per_launch": f_b, "write_bytes_per_launch": w_b, "launches": len(fv),
               "calibration": {"copy_bytes": CALIB_BYTES, "fetch_kib": f_cal, "write_kib": w_cal,
                               "fetch_factor": kf, "write_factor": kw}}
        with open(os.path.join(PROFILE_DIR, f"{key}_traffic.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        lines.append(f"| {sub} | {wl} | {len(fv)} | {f_b / 1e6:.1f} | {w_b / 1e6:.1f} | {(f_b + w_b) / 1e6:.1f} |")
    print(f"fetch factor {kf:.4f}, write factor {kw:.4f} (copy of {CALIB_BYTES} B read {f_cal:.0f} KiB, "
          f"wrote {w_cal:.0f} KiB)")
    print("| kernel | workload | launches | read MB/launch | written MB/launch | total MB/launch |")
    print("|---|---|---|---|---|---|")
    print("\n".join(lines))


def summarize_counters(pmc_dir, trace_dir):
    """MFMA utilisation of the prefill attention kernel from one --pmc pass (MFMA_COUNTERS) and its
    kernel trace (durations).  Writes profiles/sparse_attn_prefill_<workload>_mfma.json per workload."""
    import csv
    import glob
    rows = [r for r in _pmc_rows(pmc_dir) if "attn_prefill_mfma" in r["name"]]
    tfiles = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    durs = []
    if tfiles:
        for r in csv.DictReader(open(tfiles[0])):
            if "attn_prefill_mfma" in r["Kernel_Name"]:
                durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    # the counter run launches 3 prefill steps of the 128K workload, then 3 of the 32K one
    groups = {"s131072": rows[:3], "s32768": rows[3:6]}
    dgroups = {"s131072": durs[:3], "s32768": durs[3:6]}
    out = []
    for wl, rs in groups.items():
        if not rs:
            continue
        c = {k: sum(r["counters"].get(k, 0.0) for r in rs) / len(rs) for k in MFMA_COUNTERS}
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"]
        # GRBM_GUI_ACTIVE is summed over the XCDs; per XCD it counts the kernel's active GPU cycles
        active = c["GRBM_GUI_ACTIVE"] / NUM_XCDS
        rec = {"kernel": "attn_prefill_mfma_kernel", "workload": f"prefill_bf16_{wl}",
               "source_hash": _kernel_hash("attn_prefill.hip", "bsg_device.h"), "launches": len(rs), "counters_per_launch": c,
               "mfma_busy_frac": busy / (active * NUM_SIMDS) if active else None,
               "mfma_valu_coexec_frac": c["SQ_VALU_MFMA_COEXEC_CYCLES"] / (active * NUM_SIMDS) if active else None,
               "valu_insts_per_mfma": c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"] if c["SQ_INSTS_MFMA"] else None,
               "active_cycles_per_xcd": active}
        dd = dgroups.get(wl) or []
        if dd:
            rec["trace_duration_ms"] = 1e3 * sum(dd) / len(dd)
            rec["observed_clock_ghz"] = active / (sum(dd) / len(dd)) / 1e9
        with open(os.path.join(PROFILE_DIR, f"sparse_attn_prefill_{wl}_mfma.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        out.append(rec)
        print(json.dumps(rec))
    return out


# ------------------------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="all",
                    help="comma list of parts: prefill,prefill32k,decode,decode1m,fp8,tokens (default all)")
    ap.add_argument("--traffic-run", action="store_true", help="one prefill + decode step and a calibration copy")
    ap.add_argument("--counter-run", action="store_true", help="prefill steps for rocprofv3 --pmc of MFMA counters")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE output directories -> profiles/*_traffic.json")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("PMC_DIR", "TRACE_DIR"),
                    help="rocprofv3 --pmc (MFMA counters) and --kernel-trace output directories of --counter-run "
                         "-> profiles/sparse_attn_prefill_*_mfma.json")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this library has no multi-GPU path; "
              "sharding would split KV heads or sequences across GPUs with no exchange.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_gqa_pool_amd as bsg
    from workloads import SPECS, spec_by_name

    bsg.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.traffic_run:
        traffic_run()
        return
    if args.counter_run:
        counter_run()
        return
    parts = set(("prefill,prefill32k,decode,decode1m,fp8,tokens,prefill_tokens" if args.only == "all"
                 else args.only).split(","))
    steps = max(args.steps, 1)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    spec = spec_by_name("prefill_bf16_s131072")
    line = {"metric": METRIC}
    if "prefill" in parts:
        r = r_pf = run_prefill(spec, SPECS.index(spec), steps, args.warmup, tile_stats=True,
                               keep_ranges=None if args.no_cpu_baseline else baseline_ranges(spec.seq_len))
        p = prefill_line(spec, r)
        log(f"prefill 128K: {p['tok_per_s'] / 1e6:.2f} M tok/s, attention {p['roofline']['avg_launch_ms']:.2f} ms")
        roof = dict(p["roofline"], traffic=_traffic("sparse_attn_prefill_s131072"))
        mf = _profile_record("sparse_attn_prefill_s131072_mfma", ["attn_prefill.hip", "bsg_device.h"])
        roof["mfma_util"] = None if mf is None else {k: mf.get(k) for k in (
            "mfma_busy_frac", "mfma_valu_coexec_frac", "valu_insts_per_mfma", "observed_clock_ghz")}
        line.update(value=p["tok_per_s"], unit="tok/s", n_gpus=1, steps=steps, warmup=args.warmup,
                    ms_per_step=r["ms_per_step"], higher_is_better=True, scaling="weak", vs_baseline=None,
                    dtype="bf16", data="synthetic (seeded planted-block generator)",
                    config={"workload": spec.name, "batch": spec.batch, "seq_len": spec.seq_len,
                            "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
                            "head_dim": spec.head_dim, "block_size": spec.page_size, "top_k": spec.top_k},
                    roofline=roof, stages_ms=p["stages_ms"], wall_ms_per_step=r["wall_ms_per_step"],
                    pipeline_mfma_frac=p["pipeline_mfma_frac"], tiles=p["tiles"],
                    planted_recall=p.get("planted_recall"))
    if "prefill32k" in parts:
        s1 = spec_by_name("prefill_bf16_s32768")
        r1 = run_prefill(s1, SPECS.index(s1), steps, args.warmup, tile_stats=True)
        p1 = prefill_line(s1, r1)
        mf1 = _profile_record("sparse_attn_prefill_s32768_mfma", ["attn_prefill.hip", "bsg_device.h"])
        p1["roofline"]["mfma_util"] = None if mf1 is None else {k: mf1.get(k) for k in (
            "mfma_busy_frac", "mfma_valu_coexec_frac", "valu_insts_per_mfma", "observed_clock_ghz")}
        line["prefill_s32768"] = p1
        log(f"prefill 32K: {p1['tok_per_s'] / 1e6:.2f} M tok/s, attention {p1['roofline']['avg_launch_ms']:.3f} ms")
    dsteps = max(steps, 400)
    if "decode" in parts:
        ds = spec_by_name("decode_bf16_b32_ctx131072")
        seed = SPECS.index(ds)
        warm = run_decode(ds, seed, dsteps, args.warmup)
        cold = run_decode(ds, seed, dsteps, args.warmup, rotate=4)
        tr_u = _traffic("decode_unit_b32_ctx131072")
        tr_m = _traffic("decode_merge_b32_ctx131072")
        line["decode"] = decode_line(ds, warm, "bsg_decode_step", (tr_u + tr_m) if (tr_u and tr_m) else None, cold)
        log(f"decode 128K x 32: warm {warm['us']['mean']:.1f} us, cold {cold['us']['mean']:.1f} us")
        if not args.no_cpu_baseline:
            line["decode"]["cpu_baseline"] = cpu_baseline_decode(ds, seed)
    if "fp8" in parts:
        ds = spec_by_name("decode_bf16_b32_ctx131072")
        d8 = run_decode(ds, SPECS.index(ds), dsteps, args.warmup, fp8=True)
        tr_u8 = _traffic("decode_fp8_unit_b32_ctx131072")
        tr_m = _traffic("decode_merge_b32_ctx131072")
        l8 = decode_line(ds, d8, "bsg_decode_step_fp8", (tr_u8 + tr_m) if (tr_u8 and tr_m) else None)
        l8["workload"] = ds.name + " (K, V and block cache in fp8 E4M3)"
        line["decode_fp8"] = l8
    if "decode1m" in parts:
        s4 = spec_by_name("decode_bf16_b4_ctx512k_1m")
        seed = SPECS.index(s4)
        warm = run_decode(s4, seed, dsteps, args.warmup)
        cold = run_decode(s4, seed, dsteps, args.warmup, rotate=4)
        line["decode_ragged_1m"] = decode_line(s4, warm, "bsg_decode_step", None, cold)
        log(f"decode ~1M x 4: warm {warm['us']['mean']:.1f} us, cold {cold['us']['mean']:.1f} us")
    if "tokens" in parts:
        ds = spec_by_name("decode_bf16_b32_ctx131072")
        for key, K, two in (("decode_tokens", 2048, False), ("decode_two_level", 512, True)):
            dt = run_decode_tokens(ds, SPECS.index(ds), max(steps, 64), args.warmup, K, two)
            dt["workload"] = ds.name + (f" (block top-{ds.top_k}, then token top-{K})" if two else f" (token top-{K})")
            line[key] = dt
        s4 = spec_by_name("decode_bf16_b4_ctx512k_1m")
        dt = run_decode_tokens(s4, SPECS.index(s4), max(steps, 16), args.warmup, 2048, False)
        dt["workload"] = s4.name + " (token top-2048)"
        line["decode_tokens_1m"] = dt
        log(f"token-level decode ~1M x 4: {dt['us_per_step']:.0f} us per step")
    if "prefill_tokens" in parts:
        s1 = spec_by_name("prefill_bf16_s32768")
        for key, K, two in (("prefill_tokens", 2048, False), ("prefill_two_level", 512, True)):
            r = run_prefill_tokens(s1, SPECS.index(s1), max(3, min(steps, 10)), 1, K, two)
            line[key] = prefill_tokens_line(s1, r, two)
            log(f"{key} 32K: {r['ms_per_step']:.2f} ms per prefill")
    if "prefill" in parts:
        line["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_prefill(
            spec, SPECS.index(spec), kept_rows=r_pf.pop("kept_rows", None))
        if line["cpu_baseline"] is not None:
            line["parity_sample"] = line["cpu_baseline"].pop("parity")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
