"""Seeded planted-block workloads (paged K/V cache, page table, queries).

The generator follows the five workload descriptions that accompany this
library (tiny fp32 prefill, 32K and 128K bf16 prefill, 128K and ragged ~1M
bf16 decode).  Values:

* keys and values are i.i.d. N(0, 1); every key block of every KV head gets an
  extra offset vector o ~ N(0, offset_std^2)^D added to all of its keys,
* queries are N(0, 1); for each query token and GQA group a few strictly
  earlier blocks are "planted": ``plant_weight * sum(o_planted)`` is added to
  all query heads of the group, so the planted blocks are the group's true top
  blocks (this is what recall is measured against),
* "region" planting draws the planted blocks once per (region of tokens, group)
  from the blocks before the region, and adds ``recency_weight * o`` of the
  ``recency`` blocks just before the token's own block,
* bf16 workloads are drawn in fp32 and rounded to bf16 once.

Layouts produced (the library's boundary layouts):

* ``k_cache``, ``v_cache``: ``[num_pages, Hkv, page_size, D]``
* ``page_table``: int32 ``[B, pt_stride]``, logical block j of sequence b lives
  in physical page ``page_table[b, j]``; unused entries hold 0
* ``kv_lens``: int32 ``[B]`` tokens in the cache per sequence (the newest
  query sits at position ``kv_len - 1``)
* ``q``: ``[B, Hq, q_len, D]``; query t sits at position ``kv_len - q_len + t``

Slots of a sequence's last page beyond ``kv_len`` hold ``tail_fill``.

Everything is drawn with ``torch`` generators on the requested device, so large
workloads can be drawn directly in GPU memory.  The same (spec, seed, device)
always yields the same bytes.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

__all__ = ["WorkloadSpec", "Workload", "SPECS", "make_workload", "spec_by_name"]


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    mode: str                      # "prefill" | "decode"
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    top_k: int
    dtype: str                     # "f32" | "bf16"
    seq_len: int = 0               # prefill: tokens per sequence (all are queries)
    ctx_len: int = 0               # decode: prompt tokens before the new token
    ctx_range: Optional[tuple] = None  # decode: inclusive uniform range of prompt tokens
    q_len: int = 0                 # prefill over an existing prefix: queries = last q_len tokens
    plant: str = "token"           # "token" | "region"
    n_plant: int = 2
    plant_weight: float = 1.5
    region: int = 0                # tokens per region (plant == "region")
    recency: int = 0               # recent earlier blocks that get a bias
    recency_weight: float = 0.0
    offset_std: float = 0.5
    shuffle_pages: bool = False
    spare_pages: int = 0           # extra never-referenced pages in the pool

    def replace(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


SPECS: Sequence[WorkloadSpec] = (
    # 0: tiny causal prefill, fp32
    WorkloadSpec("prefill_tiny_f32_s1024", "prefill", 1, 8, 2, 64, 64, 4, "f32", seq_len=1024,
                 plant="token", n_plant=2),
    # 1: 32K prefill, bf16
    WorkloadSpec("prefill_bf16_s32768", "prefill", 1, 32, 4, 128, 64, 32, "bf16", seq_len=32768,
                 plant="token", n_plant=2),
    # 2: 128K decode, 32 sequences, shuffled 64-token pages
    WorkloadSpec("decode_bf16_b32_ctx131072", "decode", 32, 32, 4, 128, 64, 32, "bf16",
                 ctx_len=131072, plant="token", n_plant=2, shuffle_pages=True),
    # 3: 128K prefill, bf16, region planting + recency bias
    WorkloadSpec("prefill_bf16_s131072", "prefill", 1, 64, 8, 128, 128, 16, "bf16", seq_len=131072,
                 plant="region", n_plant=8, region=4096, recency=4, recency_weight=2.0),
    # 4: ragged decode toward 1M context
    WorkloadSpec("decode_bf16_b4_ctx512k_1m", "decode", 4, 64, 8, 128, 64, 32, "bf16",
                 ctx_range=(524288, 1048576), plant="token", n_plant=2, shuffle_pages=True),
)


def spec_by_name(name: str) -> WorkloadSpec:
    for s in SPECS:
        if s.name == name:
            return s
    raise KeyError(name)


@dataclass
class Workload:
    spec: WorkloadSpec
    seed: int
    q: torch.Tensor                # [B, Hq, q_len, D]
    k_cache: torch.Tensor          # [P, Hkv, bs, D]
    v_cache: torch.Tensor          # [P, Hkv, bs, D]
    page_table: torch.Tensor       # int32 [B, pt_stride]
    kv_lens: torch.Tensor          # int32 [B]
    q_len: int
    # planted blocks per query token, -1 where fewer exist: [B, Hkv, q_len, n]
    # (None for region planting; see planted_region)
    planted: Optional[torch.Tensor]
    # region planting: [B, Hkv, n_regions, n] (-1 padded)
    planted_region: Optional[torch.Tensor] = None
    kv_lens_host: list = field(default_factory=list)

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def pt_stride(self) -> int:
        return int(self.page_table.shape[1])

    def planted_for(self, b: int, g: int, t: int) -> list:
        """Planted blocks of query token t (group g, sequence b)."""
        if self.planted is not None:
            return [int(x) for x in self.planted[b, g, t].tolist() if x >= 0]
        s = self.spec
        pos = self.kv_lens_host[b] - self.q_len + t
        r = pos // s.region
        return [int(x) for x in self.planted_region[b, g, r].tolist() if x >= 0]

    def to(self, device) -> "Workload":
        def mv(x):
            return None if x is None else x.to(device)
        return dataclasses.replace(self, q=mv(self.q), k_cache=mv(self.k_cache), v_cache=mv(self.v_cache),
                                   page_table=mv(self.page_table), kv_lens=mv(self.kv_lens),
                                   planted=mv(self.planted), planted_region=mv(self.planted_region))


def _mix(*ids: int) -> int:
    """splitmix64 over a tuple of ints -> 63-bit torch seed."""
    x = 0x9E3779B97F4A7C15
    for v in ids:
        x = (x ^ (int(v) & 0xFFFFFFFFFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        x = (x + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        x = z ^ (z >> 31)
    return x & 0x7FFFFFFFFFFFFFFF


_STREAM = {"ctx": 1, "pages": 2, "k": 3, "v": 4, "off": 5, "q": 6, "plant": 7}


def _gen(device, seed: int, stream: str, *ids: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_mix(seed, _STREAM[stream], *ids))
    return g


def _pick_distinct(gen, shape_rows, avail, n, nb, device):
    """Draw min(n, avail[r]) distinct values from [0, avail[r]) per row.

    ``avail``: int64 [R]; returns int64 [R, n] with -1 where avail < n.
    """
    R = avail.numel()
    out = torch.full((R, n), -1, dtype=torch.int64, device=device)
    if nb == 0 or n == 0 or R == 0:
        return out
    chunk = max(1, (1 << 24) // max(nb, 1))
    ar = torch.arange(nb, device=device)
    for s in range(0, R, chunk):
        e = min(R, s + chunk)
        keys = torch.rand((e - s, nb), generator=gen, device=device)
        a = avail[s:e]
        keys = torch.where(ar[None, :] < a[:, None], keys, torch.full_like(keys, 2.0))
        kk = min(n, nb)
        idx = torch.topk(keys, kk, dim=1, largest=False).indices
        idx = torch.where(idx < a[:, None], idx, torch.full_like(idx, -1))
        # order picks ascending for readability (-1 last)
        idx = torch.where(idx < 0, torch.full_like(idx, 1 << 40), idx).sort(dim=1).values
        idx = torch.where(idx >= (1 << 40), torch.full_like(idx, -1), idx)
        out[s:e, :kk] = idx
    return out


def make_workload(spec: WorkloadSpec, seed: int, device="cpu", tail_fill: float = 0.0) -> Workload:
    dev = torch.device(device)
    B, Hq, Hkv, D, bs = spec.batch, spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.page_size
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    f32 = torch.float32

    # ---- context lengths
    if spec.mode == "prefill":
        kv = [spec.seq_len] * B
        q_len = spec.q_len if spec.q_len else spec.seq_len
    elif spec.mode == "decode":
        if spec.ctx_range is not None:
            lo, hi = spec.ctx_range
            g = _gen("cpu", seed, "ctx")
            L = torch.randint(lo, hi + 1, (B,), generator=g).tolist()
        else:
            L = [spec.ctx_len] * B
        kv = [x + 1 for x in L]
        q_len = 1
    else:
        raise ValueError(spec.mode)
    if q_len > min(kv):
        raise ValueError("q_len exceeds a context length")
    npg = [(x + bs - 1) // bs for x in kv]
    pt_stride = max(npg)
    P = sum(npg) + spec.spare_pages

    # ---- page table
    if spec.shuffle_pages:
        perm = torch.randperm(P, generator=_gen("cpu", seed, "pages"))
    else:
        perm = torch.arange(P)
    pt = torch.zeros((B, pt_stride), dtype=torch.int32)
    off = 0
    for b in range(B):
        pt[b, :npg[b]] = perm[off:off + npg[b]].to(torch.int32)
        off += npg[b]

    dt = spec.torch_dtype
    k_cache = torch.empty((P, Hkv, bs, D), dtype=dt, device=dev)
    v_cache = torch.empty((P, Hkv, bs, D), dtype=dt, device=dev)
    k_cache.fill_(tail_fill)
    v_cache.fill_(tail_fill)
    q = torch.empty((B, Hq, q_len, D), dtype=dt, device=dev)
    nb_max = pt_stride
    planted_all = None
    planted_region = None
    if spec.plant == "token":
        planted_all = torch.full((B, Hkv, q_len, spec.n_plant), -1, dtype=torch.int32)
    elif spec.plant == "region":
        n_regions = (max(kv) + spec.region - 1) // spec.region
        planted_region = torch.full((B, Hkv, n_regions, spec.n_plant), -1, dtype=torch.int32)
    else:
        raise ValueError(spec.plant)

    for b in range(B):
        L = kv[b]
        nbk = npg[b]
        offs = torch.randn((Hkv, nbk, D), generator=_gen(dev, seed, "off", b), device=dev, dtype=f32) * spec.offset_std
        kl = torch.randn((Hkv, L, D), generator=_gen(dev, seed, "k", b), device=dev, dtype=f32)
        tok_blk = torch.arange(L, device=dev) // bs
        kl += offs[:, tok_blk, :]
        vl = torch.randn((Hkv, L, D), generator=_gen(dev, seed, "v", b), device=dev, dtype=f32)
        pad = nbk * bs - L
        phys = pt[b, :nbk].to(torch.int64).to(dev)
        for src, dst in ((kl, k_cache), (vl, v_cache)):
            full = torch.full((Hkv, nbk * bs, D), tail_fill, device=dev, dtype=f32)
            full[:, :L] = src
            pages = full.view(Hkv, nbk, bs, D).permute(1, 0, 2, 3).to(dt)
            dst[phys] = pages
            del full, pages
        del kl, vl

        qb = torch.randn((Hq, q_len, D), generator=_gen(dev, seed, "q", b), device=dev, dtype=f32)
        pos = torch.arange(L - q_len, L, device=dev)
        own = pos // bs
        gplant = _gen(dev, seed, "plant", b)
        bias = torch.zeros((Hkv, q_len, D), device=dev, dtype=f32)
        if spec.plant == "token":
            avail = own.repeat(Hkv)                       # rows ordered (g, t)
            picks = _pick_distinct(gplant, None, avail, spec.n_plant, nb_max, dev).view(Hkv, q_len, spec.n_plant)
            valid = picks >= 0
            gidx = torch.arange(Hkv, device=dev)[:, None, None]
            o = offs[gidx, picks.clamp(min=0), :]         # [Hkv, q_len, n, D]
            bias += spec.plant_weight * (o * valid[..., None]).sum(dim=2)
            planted_all[b] = picks.to(torch.int32).cpu()
        else:
            rb = spec.region // bs                        # blocks per region
            n_regions = planted_region.shape[2]
            avail = (torch.arange(n_regions, device=dev) * rb).repeat(Hkv)   # rows (g, r)
            picks = _pick_distinct(gplant, None, avail, spec.n_plant, nb_max, dev).view(Hkv, n_regions, spec.n_plant)
            valid = picks >= 0
            gidx = torch.arange(Hkv, device=dev)[:, None, None]
            o = offs[gidx, picks.clamp(min=0), :]         # [Hkv, R, n, D]
            rbias = spec.plant_weight * (o * valid[..., None]).sum(dim=2)    # [Hkv, R, D]
            reg = pos // spec.region
            bias += rbias[:, reg, :]
            for i in range(1, spec.recency + 1):
                j = own - i
                ok = (j >= 0)
                bias += spec.recency_weight * offs[:, j.clamp(min=0), :] * ok[None, :, None].to(f32)
            planted_region[b] = picks.to(torch.int32).cpu()
        qb = qb.view(Hkv, G, q_len, D) + bias[:, None]
        q[b] = qb.view(Hq, q_len, D).to(dt)
        del qb, bias, offs

    kv_t = torch.tensor(kv, dtype=torch.int32, device=dev)
    return Workload(spec=spec, seed=seed, q=q, k_cache=k_cache, v_cache=v_cache,
                    page_table=pt.to(dev), kv_lens=kv_t, q_len=q_len,
                    planted=planted_all, planted_region=planted_region, kv_lens_host=list(kv))
