"""Benchmark: block-sparse GQA attention at 128K context on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one pass of the whole hot path over one batch of synthetic input:
  prefill workload: block_pool -> group_score_topk -> sparse_attn_prefill
  decode workload:  decode_step = group scores + top-k + sparse attention (block cache built beforehand),
                    captured (8 steps per HIP graph) and replayed: the step is three short kernels
Inputs are generated on the GPU and resident in HBM before timing starts.  The default
workload is the 128K prefill (B=1, S=131072, Hq=64, Hkv=8, D=128, 128-token blocks,
top-16); the 128K decode step (B=32, context 131072, Hq=32, Hkv=4, 64-token pages,
top-32) is measured in the same run and reported under "decode".

Prints ONE JSON line.  `value` is prefill tokens/s (or decode steps/s-free us/step for
--workload decode).  `roofline` covers the dominant kernel of the step, timed with HIP
events on the stream the library launches on; its algorithmic work is counted from the
actual selection (4*D FLOPs per selected, causally valid key per query head for prefill;
selected K+V bytes + block-cache bytes + page-table bytes for decode).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-sparse GQA attn: prefill tok/s + decode µs/step at 128K, % roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PROFILE_DIR = os.path.join(ROOT, "profiles")


def _kernel_hash(*files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "block_sparse_gqa_pool_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key: str, src_files) -> float | None:
    """HBM bytes per launch from a committed counter summary, if it matches the current source."""
    path = os.path.join(PROFILE_DIR, f"{kernel_key}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != _kernel_hash(*src_files):
        return None
    return rec.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------------------------
def prefill_flops(block_idx, kv_lens, q_len, page_size, G, D):
    """4*D FLOPs per (query head, selected key at a position <= the query)."""
    import torch
    B, Hkv, T, k = block_idx.shape
    pos = (kv_lens.view(B, 1, 1, 1).long() - q_len + torch.arange(T, device=block_idx.device).view(1, 1, T, 1))
    j = block_idx.long()
    n = torch.clamp(pos - j * page_size + 1, min=0, max=page_size)
    n = torch.where(j >= 0, n, torch.zeros_like(n))
    return float(n.sum().item()) * G * 4 * D


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


def run_decode_tokens(spec, seed, steps, warmup, top_k_tokens, two_level):
    """Token-level (two_level False) or two-level decode steps, graph-replayed like run_decode.
    Algorithmic bytes: token level reads every key once (the identity indexer scores all
    tokens) plus the kept tokens' values and the page table; two level reads the block cache
    of every candidate, the keys of the kept blocks, and the kept tokens' values."""
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
    import ctypes
    need = int(bsg.lib().bsg_decode_step_tokens_workspace_bytes(ctypes.byref(d), top_k_tokens, int(two_level)))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        bsg.decode_step_tokens(q1, w.kv_lens, w.k_cache, w.v_cache, w.page_table, scale, tok, out,
                               block_cache=cache, block_idx=bidx, workspace=ws)

    PER_GRAPH = 4
    for _ in range(max(warmup, 1)):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(PER_GRAPH):
            step()
    graph.replay()
    torch.cuda.synchronize()
    n_rep = max(1, (steps + PER_GRAPH - 1) // PER_GRAPH)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_rep):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    steps = n_rep * PER_GRAPH
    us = 1e3 * e0.elapsed_time(e1) / steps
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
    return dict(us_per_step=us, bytes=nbytes, bytes_parts=parts, steps=steps)


# ------------------------------------------------------------------------------------
def run_prefill(spec, seed, steps, warmup):
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
    stage = [[e[i].elapsed_time(e[i + 1]) for e in evs] for i in range(3)]
    step_ms = [e[0].elapsed_time(e[3]) for e in evs]
    flops = prefill_flops(idx, w.kv_lens, S, bs, spec.group_size, D)
    res = dict(
        tokens=B * S, wall_s=wall, ms_per_step=sum(step_ms) / steps, wall_ms_per_step=1e3 * wall / steps,
        stage_ms={n: sum(v) / steps for n, v in zip(("block_pool", "group_score_topk", "sparse_attn_prefill"), stage)},
        attn_flops=flops,
    )
    del w, cache, idx, out, ws
    torch.cuda.empty_cache()
    return res


def run_decode(spec, seed, steps, warmup, graph_replay=True, fp8=False):
    import torch
    import block_sparse_gqa_pool_amd as bsg
    from workloads import make_workload

    dev = torch.device("cuda:0")
    w = make_workload(spec, seed, device=dev)
    B, Hq, _, D = w.q.shape
    Hkv, bs, k = spec.num_kv_heads, spec.page_size, spec.top_k
    scale = 1.0 / math.sqrt(D)
    cache = torch.zeros(w.k_cache.shape[0], Hkv, D, dtype=w.k_cache.dtype, device=dev)
    bsg.block_pool(w.k_cache, w.page_table, w.kv_lens, cache)        # built at prefill (untimed)
    idx = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
    q1 = w.q[:, :, 0].contiguous()
    out = torch.empty(B, Hq, D, dtype=w.q.dtype, device=dev)
    ws = torch.empty(bsg.decode_step_workspace_bytes(w.k_cache, w.page_table, Hq, k), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        bsg.decode_step(q1, w.kv_lens, cache, w.k_cache, w.v_cache, w.page_table, scale, idx, out, workspace=ws)

    if fp8:
        # fp8 caches, quantised from the bf16 ones at prefill (untimed); the bf16 caches are freed
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
        cache = None
        torch.cuda.empty_cache()

        def step():
            bsg.decode_step_fp8(q1, w.kv_lens, rc, rs, kc, ks, vc, vs, w.page_table, scale, idx, out, workspace=ws)

    # the step is three short kernels, faster than Python can launch them: capture
    # PER_GRAPH whole steps in one HIP graph and replay it, so the timed region measures
    # back-to-back GPU work rather than host launch cost
    PER_GRAPH = 8
    for _ in range(max(warmup, 1)):
        step()
    torch.cuda.synchronize()
    if not graph_replay:                     # eager steps (counter collection)
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        del w, cache, idx, out, ws
        torch.cuda.empty_cache()
        return None
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(PER_GRAPH):
            step()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    n_rep = max(1, (steps + PER_GRAPH - 1) // PER_GRAPH)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(n_rep):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    steps = n_rep * PER_GRAPH
    step_ms = e0.elapsed_time(e1) / steps
    nbytes, parts = decode_bytes(idx, w.kv_lens, bs, Hkv, D, elem=1 if fp8 else 2)
    res = dict(us_per_step=1e3 * step_ms, wall_us_per_step=1e6 * wall / steps, bytes=nbytes, bytes_parts=parts,
               steps=steps)
    del graph, w, cache, idx, out, ws
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------------------
def cpu_baseline_prefill(spec, seed, n_tokens):
    """The CPU oracle on a bounded sample of the same workload (one BLAS thread)."""
    import numpy as np
    import torch
    import oracle as O
    from workloads import make_workload

    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    w = make_workload(spec, seed, device="cuda:0" if torch.cuda.is_available() else "cpu")
    q = w.q.float().cpu().numpy()
    kp = w.k_cache.float().cpu().numpy()
    vp = w.v_cache.float().cpu().numpy()
    pt = w.page_table.cpu().numpy()
    kv = list(w.kv_lens_host)
    del w
    torch.cuda.empty_cache()
    S = q.shape[2]
    rng = np.random.default_rng(0)
    tsel = np.sort(rng.choice(S, size=n_tokens, replace=False))
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        t0 = time.perf_counter()
        cache = O.block_pool(kp, pt, kv, spec.dtype)
        t1 = time.perf_counter()
        sc = O.group_scores(q, cache, pt, kv, spec.num_kv_heads, spec.page_size, tsel)
        idx = O.select_blocks(sc, kv, S, spec.page_size, spec.top_k, tsel)
        O.sparse_attention(q, kp, vp, pt, kv, idx, 1.0 / math.sqrt(spec.head_dim), tsel)
        t2 = time.perf_counter()
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    per_tok = (t2 - t1) / n_tokens
    est = (t1 - t0) + per_tok * S
    return dict(value=S / est, unit="tok/s", cores=1, kind="oracle",
                sample=(f"block_pool over all {pt.shape[1]} blocks ({t1 - t0:.1f} s) + scores, top-k and "
                        f"attention for {n_tokens} random query tokens ({t2 - t1:.1f} s), extrapolated "
                        f"linearly to all {S} tokens: {est:.0f} s per prefill"),
                seconds=t2 - t0)


# ------------------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters
TRAFFIC_KERNELS = {
    # key: (kernel-name substring, source files, workload); the fp8 instantiations carry F8 = true
    "sparse_attn_prefill_s131072": ("attn_prefill_mfma", ["attn_prefill.hip"], "prefill_bf16_s131072"),
    "decode_attn_b32_ctx131072": ("attn_decode_mfma_kernel<128, 64, true, false>", ["attn_decode.hip"],
                                  "decode_bf16_b32_ctx131072"),
    "decode_scan_b32_ctx131072": ("decode_score_chunk_kernel<128, false>", ["decode_select.hip"],
                                  "decode_bf16_b32_ctx131072"),
    "decode_fp8_attn_b32_ctx131072": ("attn_decode_mfma_kernel<128, 64, true, true>", ["attn_decode.hip"],
                                      "decode_bf16_b32_ctx131072 in fp8"),
    "decode_fp8_scan_b32_ctx131072": ("decode_score_chunk_kernel<128, true>", ["decode_select.hip"],
                                      "decode_bf16_b32_ctx131072 in fp8"),
}
CALIB_BYTES = 1 << 30


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
        per.setdefault(did, {"name": r["Kernel_Name"], "val": 0.0})
        per[did]["val"] += float(r["Counter_Value"])
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_bf16_s131072")
    ap.add_argument("--decode-workload", default="decode_bf16_b32_ctx131072")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1024)
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--traffic-run", action="store_true", help="one prefill + decode step and a calibration copy")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE output directories -> profiles/*_traffic.json")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
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
    spec = spec_by_name(args.workload)
    seed = args.seed if args.seed is not None else SPECS.index(spec)

    line = {"metric": METRIC}
    if spec.mode == "prefill":
        r = run_prefill(spec, seed, args.steps, args.warmup)
        tok_s = r["tokens"] / (r["ms_per_step"] / 1e3)
        attn_ms = r["stage_ms"]["sparse_attn_prefill"]
        achieved = r["attn_flops"] / (attn_ms / 1e3) / 1e12
        line.update(value=tok_s, unit="tok/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                    ms_per_step=r["ms_per_step"], higher_is_better=True, scaling="weak", vs_baseline=None,
                    dtype="bf16", data="synthetic (seeded planted-block generator)",
                    config={"workload": spec.name, "batch": spec.batch, "seq_len": spec.seq_len,
                            "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
                            "head_dim": spec.head_dim, "block_size": spec.page_size, "top_k": spec.top_k},
                    roofline={"kernel": "sparse_attn_prefill", "bound": "mfma", "achieved": achieved,
                              "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                              "traffic": _traffic("sparse_attn_prefill_s131072", ["attn_prefill.hip"]),
                              "flops_per_launch": r["attn_flops"], "avg_launch_ms": attn_ms},
                    stages_ms=r["stage_ms"], wall_ms_per_step=r["wall_ms_per_step"],
                    pipeline_mfma_frac=(r["attn_flops"] / (r["ms_per_step"] / 1e3) / 1e12) / PEAK_BF16_TFLOPS)
        dspec = spec_by_name(args.decode_workload)
        d = run_decode(dspec, SPECS.index(dspec), max(args.steps, 40), args.warmup)
        gbs = d["bytes"] / (d["us_per_step"] / 1e6) / 1e9
        tr_a = _traffic("decode_attn_b32_ctx131072", ["attn_decode.hip"])
        tr_s = _traffic("decode_scan_b32_ctx131072", ["decode_select.hip"])
        line["decode"] = {"workload": dspec.name, "us_per_step": d["us_per_step"], "api": "bsg_decode_step",
                          "steps": d["steps"], "timing": "8 steps per HIP graph replay, HIP events",
                          "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                       "frac": gbs / PEAK_HBM_GBS, "bytes_per_step": d["bytes"],
                                       "bytes_parts": d["bytes_parts"],
                                       "traffic": (tr_a + tr_s) if (tr_a and tr_s) else None},
                          "wall_us_per_step": d["wall_us_per_step"]}
        d8 = run_decode(dspec, SPECS.index(dspec), max(args.steps, 40), args.warmup, fp8=True)
        tr_a8 = _traffic("decode_fp8_attn_b32_ctx131072", ["attn_decode.hip"])
        tr_s8 = _traffic("decode_fp8_scan_b32_ctx131072", ["decode_select.hip"])
        gbs8 = d8["bytes"] / (d8["us_per_step"] / 1e6) / 1e9
        line["decode_fp8"] = {"workload": dspec.name + " (K, V and block cache in fp8 E4M3)",
                              "us_per_step": d8["us_per_step"], "api": "bsg_decode_step_fp8", "steps": d8["steps"],
                              "timing": "8 steps per HIP graph replay, HIP events",
                              "roofline": {"bound": "hbm", "achieved": gbs8, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                           "frac": gbs8 / PEAK_HBM_GBS, "bytes_per_step": d8["bytes"],
                                           "bytes_parts": d8["bytes_parts"],
                                           "traffic": (tr_a8 + tr_s8) if (tr_a8 and tr_s8) else None},
                              "wall_us_per_step": d8["wall_us_per_step"]}
        for key, K, two in (("decode_tokens", 2048, False), ("decode_two_level", 512, True)):
            dt = run_decode_tokens(dspec, SPECS.index(dspec), max(args.steps, 16), args.warmup, K, two)
            gbt = dt["bytes"] / (dt["us_per_step"] / 1e6) / 1e9
            line[key] = {"workload": dspec.name + (f" (block top-{dspec.top_k}, then token top-{K})" if two
                                                   else f" (token top-{K})"),
                         "us_per_step": dt["us_per_step"], "api": "bsg_decode_step_tokens", "steps": dt["steps"],
                         "timing": "4 steps per HIP graph replay, HIP events",
                         "roofline": {"bound": "hbm", "achieved": gbt, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": gbt / PEAK_HBM_GBS, "bytes_per_step": dt["bytes"],
                                      "bytes_parts": dt["bytes_parts"], "traffic": None}}
    else:
        d = run_decode(spec, seed, args.steps, args.warmup)
        gbs = d["bytes"] / (d["us_per_step"] / 1e6) / 1e9
        line.update(value=d["us_per_step"], unit="us/step", n_gpus=1, steps=args.steps, warmup=args.warmup,
                    ms_per_step=d["us_per_step"] / 1e3, higher_is_better=False, scaling="weak", vs_baseline=None,
                    dtype="bf16", data="synthetic (seeded planted-block generator)",
                    config={"workload": spec.name, "batch": spec.batch, "num_q_heads": spec.num_q_heads,
                            "num_kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim,
                            "block_size": spec.page_size, "top_k": spec.top_k},
                    roofline={"kernel": "decode step", "bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                              "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": None,
                              "bytes_per_step": d["bytes"]})
    if not args.no_cpu_baseline and spec.mode == "prefill":
        line["cpu_baseline"] = cpu_baseline_prefill(spec, seed, args.cpu_tokens)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
