"""GPU parity of the fp8 (OCP E4M3) KV cache and block cache path.

* bsg_quantize_pages_fp8 and bsg_block_pool_fp8 must reproduce the oracle's codes and
  scales bit for bit (every step is an exact scaling, an in-order fp32 sum or a
  nearest-even rounding, decided the same way on both sides);
* bsg_decode_step_fp8 must equal bsg_decode_step run on bf16 caches that hold the decoded
  values, bit for bit (selection, output and lse), since every scale is a power of two
  applied exactly;
* and it must match the oracle's decode step on the oracle's own quantisation of the
  same bf16 data (selection up to the tie window, outputs within the bf16 bounds).
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_gqa_pool_amd as bsg
import oracle as O
from workloads import SPECS, make_workload

from gpu_util import check_out, compare_selection, note, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _quantize(w):
    """Device fp8 caches of a bf16 workload: (kc, ks, vc, vs, rc, rs)."""
    P, Hkv, bs, D = w.k_cache.shape
    kc = torch.zeros(P, Hkv, bs, D, dtype=torch.uint8, device=DEV)
    vc = torch.zeros_like(kc)
    ks = torch.ones(P, Hkv, dtype=torch.float32, device=DEV)
    vs = torch.ones_like(ks)
    bsg.quantize_pages_fp8(w.k_cache, w.page_table, w.kv_lens, kc, ks)
    bsg.quantize_pages_fp8(w.v_cache, w.page_table, w.kv_lens, vc, vs)
    rc = torch.zeros(P, Hkv, D, dtype=torch.uint8, device=DEV)
    rs = torch.ones(P, Hkv, dtype=torch.float32, device=DEV)
    bsg.block_pool_fp8(kc, ks, w.page_table, w.kv_lens, rc, rs)
    return kc, ks, vc, vs, rc, rs


def _decoded_bf16(codes, scales):
    """bf16 tensor of code values times their (page, head) scale (exact in bf16)."""
    v = codes.view(torch.float8_e4m3fn).float()
    s = scales.reshape(scales.shape + (1,) * (codes.dim() - 2))
    return (v * s).to(torch.bfloat16)


def _seq_pages(w, seqs):
    pt = w.page_table.cpu().numpy()
    bs = w.spec.page_size
    out = []
    for b in seqs:
        n = (w.kv_lens_host[b] + bs - 1) // bs
        out.append(pt[b, :n].astype(np.int64))
    return out


def _oracle_fp8_pool(w, seqs):
    """Oracle quantisation of the given sequences' pages (remapped into a small pool):
    returns the remapped table, lengths, codes/scales of K, V and the block cache."""
    pages = _seq_pages(w, seqs)
    flat = np.concatenate(pages)
    sel = torch.from_numpy(flat).to(DEV)
    kp = to_np(w.k_cache.index_select(0, sel))
    vp = to_np(w.v_cache.index_select(0, sel))
    ptm = np.zeros((len(seqs), max(len(p) for p in pages)), np.int32)
    o = 0
    for i, p in enumerate(pages):
        ptm[i, :len(p)] = np.arange(o, o + len(p), dtype=np.int32)
        o += len(p)
    kv = [w.kv_lens_host[b] for b in seqs]
    bs = w.spec.page_size
    kc, ks = O.quantize_pages_fp8(kp, ptm, kv, bs)
    vc, vs = O.quantize_pages_fp8(vp, ptm, kv, bs)
    rc, rs = O.block_pool_fp8(kc, ks, ptm, kv)
    return flat, ptm, kv, (kc, ks, vc, vs, rc, rs)


SMALL = [
    SPECS[2].replace(batch=3, ctx_len=64 * 60 + 9),                                                  # G 8, bs 64
    SPECS[4].replace(batch=3, ctx_range=(64 * 40 + 1, 64 * 70 - 1)),                                 # ragged, G 8
    SPECS[2].replace(batch=2, ctx_len=128 * 21 + 100, page_size=128, head_dim=64, num_q_heads=32,
                     num_kv_heads=2, top_k=5),                                                       # bs 128, D 64, G 16
    SPECS[2].replace(batch=2, ctx_len=64 * 9 + 63, top_k=1),                                         # own block only
    SPECS[2].replace(batch=2, ctx_len=64 * 30 + 64, top_k=2),
]


@pytest.mark.parametrize("spec", SMALL, ids=["g8_bs64", "ragged", "bs128_d64_g16", "k1", "k2"])
def test_fp8_caches_bit_exact_against_oracle(spec):
    w = make_workload(spec, 51, device=DEV, tail_fill=float("nan"))
    note(f"[case] fp8 quantize + block pool {spec.name} B={spec.batch} bs={spec.page_size} D={spec.head_dim}")
    kc, ks, vc, vs, rc, rs = _quantize(w)
    torch.cuda.synchronize()
    seqs = list(range(spec.batch))
    flat, ptm, kv, (okc, oks, ovc, ovs, orc, ors) = _oracle_fp8_pool(w, seqs)
    sel = torch.from_numpy(flat).to(DEV)
    assert np.array_equal(kc.index_select(0, sel).cpu().numpy(), okc), "K codes"
    assert np.array_equal(ks.index_select(0, sel).cpu().numpy(), oks), "K scales"
    assert np.array_equal(vc.index_select(0, sel).cpu().numpy(), ovc), "V codes"
    assert np.array_equal(vs.index_select(0, sel).cpu().numpy(), ovs), "V scales"
    # block cache: complete blocks only
    bs = spec.page_size
    full = np.concatenate([ptm[i, :kv[i] // bs] for i in range(len(seqs))]).astype(np.int64)
    full_dev = torch.from_numpy(flat[full]).to(DEV)
    assert np.array_equal(rc.index_select(0, full_dev).cpu().numpy(), orc[full]), "block cache codes"
    assert np.array_equal(rs.index_select(0, full_dev).cpu().numpy(), ors[full]), "block cache scales"


@pytest.mark.parametrize("spec", SMALL, ids=["g8_bs64", "ragged", "bs128_d64_g16", "k1", "k2"])
def test_fp8_decode_step_equals_bf16_on_decoded_caches(spec):
    w = make_workload(spec, 52, device=DEV, tail_fill=float("nan"))
    note(f"[case] fp8 decode step vs bf16 on decoded caches {spec.name}")
    B, Hq, _, D = w.q.shape
    Hkv, k = spec.num_kv_heads, spec.top_k
    scale = 1.0 / math.sqrt(D)
    kc, ks, vc, vs, rc, rs = _quantize(w)
    q = w.q[:, :, 0].contiguous()
    idx8 = torch.full((B, Hkv, k), -7, dtype=torch.int32, device=DEV)
    out8 = torch.empty_like(q)
    lse8 = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.decode_step_fp8(q, w.kv_lens, rc, rs, kc, ks, vc, vs, w.page_table, scale, idx8, out8, lse8)
    kd, vd, rd = _decoded_bf16(kc, ks), _decoded_bf16(vc, vs), _decoded_bf16(rc, rs)
    idx = torch.full_like(idx8, -7)
    out = torch.empty_like(q)
    lse = torch.empty_like(lse8)
    bsg.decode_step(q, w.kv_lens, rd, kd, vd, w.page_table, scale, idx, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(idx8, idx), "selection"
    assert torch.equal(out8.view(torch.int16), out.view(torch.int16)), "output"
    assert torch.equal(lse8, lse), "lse"


def _check_against_oracle(w, seqs, idx8, out8, lse8, scale):
    spec = w.spec
    bs, k = spec.page_size, spec.top_k
    flat, ptm, kv, (okc, oks, ovc, ovs, orc, ors) = _oracle_fp8_pool(w, seqs)
    q = to_np(w.q[list(seqs)])
    kd, vd = O.fp8_dequant(okc, oks), O.fp8_dequant(ovc, ovs)
    rd = O.fp8_dequant(orc, ors)
    r = O.decode_reference(q, kd, vd, ptm, kv, bs, k, "f32", scale, block_cache=rd)
    gi = idx8.cpu().numpy()[list(seqs)][:, :, None, :]
    bad, exempt = compare_selection(gi, r["block_idx"], r["scores"], k)
    note(f"  exempt {len(exempt)}, bad {len(bad)}")
    assert not bad, bad
    same = np.repeat(~(gi != r["block_idx"]).any(-1)[:, :, 0], spec.group_size, axis=1)
    check_out(to_np(out8)[list(seqs)][same], r["out"][:, :, 0][same], "bf16", "fp8 decode out")
    assert np.abs(lse8.cpu().numpy()[list(seqs)][same] - r["lse"][:, :, 0][same]).max() <= 2e-3


@pytest.mark.parametrize("spec", SMALL, ids=["g8_bs64", "ragged", "bs128_d64_g16", "k1", "k2"])
def test_fp8_decode_step_matches_oracle(spec):
    w = make_workload(spec, 53, device=DEV, tail_fill=float("nan"))
    note(f"[case] fp8 decode step vs oracle {spec.name}")
    B, Hq, _, D = w.q.shape
    scale = 1.0 / math.sqrt(D)
    kc, ks, vc, vs, rc, rs = _quantize(w)
    q = w.q[:, :, 0].contiguous()
    idx8 = torch.empty(B, spec.num_kv_heads, spec.top_k, dtype=torch.int32, device=DEV)
    out8 = torch.empty_like(q)
    lse8 = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.decode_step_fp8(q, w.kv_lens, rc, rs, kc, ks, vc, vs, w.page_table, scale, idx8, out8, lse8)
    torch.cuda.synchronize()
    _check_against_oracle(w, list(range(B)), idx8, out8, lse8, scale)


@pytest.mark.parametrize("cfg,seqs", [(2, (0, 17)), (4, None)])
def test_fp8_decode_step_full_size_sampled(cfg, seqs):
    """The 128K x 32 and ragged ~1M decode workloads in fp8, in the launch configuration the
    benchmark times; sampled sequences against the oracle."""
    spec = SPECS[cfg]
    note(f"[case] fp8 full decode {spec.name}")
    w = make_workload(spec, cfg, device=DEV)
    B, Hq, _, D = w.q.shape
    scale = 1.0 / math.sqrt(D)
    kc, ks, vc, vs, rc, rs = _quantize(w)
    q = w.q[:, :, 0].contiguous()
    idx8 = torch.empty(B, spec.num_kv_heads, spec.top_k, dtype=torch.int32, device=DEV)
    out8 = torch.empty_like(q)
    lse8 = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    bsg.decode_step_fp8(q, w.kv_lens, rc, rs, kc, ks, vc, vs, w.page_table, scale, idx8, out8, lse8)
    torch.cuda.synchronize()
    if seqs is None:
        seqs = (int(np.argmin(w.kv_lens_host)),)
    note(f"  sampled sequences {seqs} of lengths {[w.kv_lens_host[b] for b in seqs]}")
    _check_against_oracle(w, list(seqs), idx8, out8, lse8, scale)
