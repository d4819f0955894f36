"""ctypes binding of ``libbsg.so`` (argument marshalling only).

Each function checks the torch tensors it is given (device, dtype, contiguity, shape),
fills a ``bsg_dims`` and calls the C entry point of the same name on torch's current HIP
stream (or the stream passed in).  No step of the method is computed here.  Importing the
package works without the built library, but every call then raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# BSG_LIBRARY selects another build of the library (the debug or the host-ASan variant)
LIB_PATH = os.environ.get("BSG_LIBRARY") or os.path.join(_PKG, "libbsg.so")

BSG_F32, BSG_BF16 = 0, 1
STATUS = {0: "BSG_OK", -1: "BSG_ERR_NULL", -2: "BSG_ERR_SHAPE", -3: "BSG_ERR_UNSUPPORTED",
          -4: "BSG_ERR_WORKSPACE", -5: "BSG_ERR_HIP", -6: "BSG_ERR_SCRATCH"}

# every symbol include/bsg.h declares
EXPORTS = ("bsg_version", "bsg_status_str", "bsg_debug_errors", "bsg_block_pool", "bsg_group_score", "bsg_topk_blocks",
           "bsg_group_score_topk_workspace_bytes", "bsg_group_score_topk", "bsg_sparse_attn_prefill",
           "bsg_sparse_attn_prefill_gated", "bsg_decode_workspace_bytes", "bsg_sparse_attn_decode",
           "bsg_decode_step_workspace_bytes", "bsg_decode_step", "bsg_decode_step_gated",
           "bsg_noalloc_scratch_bytes", "bsg_decode_step_noalloc",
           "bsg_quantize_pages_fp8", "bsg_block_pool_fp8", "bsg_decode_step_fp8",
           "bsg_token_topk_workspace_bytes", "bsg_token_topk", "bsg_decode_tokens_workspace_bytes",
           "bsg_sparse_attn_decode_tokens", "bsg_decode_step_tokens_workspace_bytes", "bsg_decode_step_tokens",
           "bsg_token_topk_prefill_workspace_bytes", "bsg_token_topk_prefill", "bsg_sparse_attn_prefill_tokens")


class BsgDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("pt_stride", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class BsgError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_gqa_pool_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
        dp = ctypes.POINTER(BsgDims)
        sig = {
            "bsg_version": ([], ctypes.c_int),
            "bsg_status_str": ([ctypes.c_int], ctypes.c_char_p),
            "bsg_debug_errors": ([ctypes.POINTER(ctypes.c_uint32), ctypes.c_int], ctypes.c_int),
            "bsg_block_pool": ([dp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "bsg_group_score": ([dp, vp, i32, vp, vp, vp, vp, i32, vp], ctypes.c_int),
            "bsg_topk_blocks": ([dp, vp, i32, i32, vp, vp, vp], ctypes.c_int),
            "bsg_group_score_topk_workspace_bytes": ([dp, i32], sz),
            "bsg_group_score_topk": ([dp, vp, i32, vp, vp, vp, vp, vp, sz, vp], ctypes.c_int),
            "bsg_sparse_attn_prefill": ([dp, vp, i32, vp, vp, vp, vp, vp, f32, vp, vp, vp], ctypes.c_int),
            "bsg_sparse_attn_prefill_gated": ([dp, vp, i32, vp, vp, vp, vp, vp, f32, vp, i32, vp, vp, vp, vp],
                                              ctypes.c_int),
            "bsg_decode_workspace_bytes": ([dp], sz),
            "bsg_sparse_attn_decode": ([dp, vp, vp, vp, vp, vp, vp, f32, vp, sz, vp, vp, vp], ctypes.c_int),
            "bsg_decode_step_workspace_bytes": ([dp], sz),
            "bsg_decode_step": ([dp, vp, vp, vp, vp, vp, vp, f32, vp, vp, sz, vp, vp, vp], ctypes.c_int),
            "bsg_decode_step_gated": ([dp, vp, vp, vp, vp, vp, vp, f32, vp, vp, sz, vp, i32, vp, vp, vp, vp],
                                      ctypes.c_int),
            "bsg_noalloc_scratch_bytes": ([], sz),
            "bsg_decode_step_noalloc": ([dp, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, vp], ctypes.c_int),
            "bsg_quantize_pages_fp8": ([dp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "bsg_block_pool_fp8": ([dp, vp, vp, vp, vp, vp, vp, vp, vp], ctypes.c_int),
            "bsg_decode_step_fp8": ([dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, vp, sz, vp, vp, vp],
                                    ctypes.c_int),
            "bsg_token_topk_workspace_bytes": ([dp, i32], sz),
            "bsg_token_topk": ([dp, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp], ctypes.c_int),
            "bsg_decode_tokens_workspace_bytes": ([dp, i32], sz),
            "bsg_sparse_attn_decode_tokens": ([dp, vp, vp, vp, vp, vp, vp, i32, f32, vp, sz, vp, vp, vp], ctypes.c_int),
            "bsg_decode_step_tokens_workspace_bytes": ([dp, i32, i32], sz),
            "bsg_decode_step_tokens": ([dp, vp, vp, vp, vp, vp, vp, i32, i32, f32, vp, vp, vp, sz, vp, vp, vp],
                                       ctypes.c_int),
            "bsg_token_topk_prefill_workspace_bytes": ([dp, i32, i32], sz),
            "bsg_token_topk_prefill": ([dp, vp, i32, vp, vp, vp, vp, i32, vp, vp, sz, vp], ctypes.c_int),
            "bsg_sparse_attn_prefill_tokens": ([dp, vp, i32, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp],
                                               ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(fn: str, st: int):
    if st != 0:
        raise BsgError(fn, st, lib().bsg_status_str(st).decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _req(t, name: str, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return BSG_F32
    if dt == torch.bfloat16:
        return BSG_BF16
    raise ValueError(f"unsupported dtype {dt} (float32 or bfloat16)")


def _tables(page_table, kv_lens, dev):
    _req(page_table, "page_table", torch.int32, 2, dev)
    _req(kv_lens, "kv_lens", torch.int32, 1, dev)
    if kv_lens.shape[0] != page_table.shape[0]:
        raise ValueError("kv_lens and page_table disagree on the batch size")


def dims(k_cache: torch.Tensor, page_table: torch.Tensor, num_q_heads: int, top_k: int) -> BsgDims:
    """bsg_dims from the K cache [P, Hkv, bs, D] and the page table [B, pt_stride]."""
    P, Hkv, bs, D = k_cache.shape
    B, pts = page_table.shape
    return BsgDims(B, num_q_heads, Hkv, D, bs, top_k, P, pts, _dtype_code(k_cache.dtype))


# ---------------------------------------------------------------------------- calls
def block_pool(k_cache, page_table, kv_lens, block_cache, blk_begin=None, stream=None):
    """bsg_block_pool: block_cache[page, g, :] = mean of the page's keys, complete blocks."""
    _req(k_cache, "k_cache", None, 4)
    dev = k_cache.device
    _tables(page_table, kv_lens, dev)
    P, Hkv, bs, D = k_cache.shape
    _req(block_cache, "block_cache", k_cache.dtype, 3, dev)
    if tuple(block_cache.shape) != (P, Hkv, D):
        raise ValueError("block_cache must be [num_pages, Hkv, D]")
    if blk_begin is not None:
        _req(blk_begin, "blk_begin", torch.int32, 1, dev)
        if blk_begin.shape[0] != page_table.shape[0]:
            raise ValueError("blk_begin must be [B]")
    d = dims(k_cache, page_table, Hkv, 1)
    _check("bsg_block_pool", lib().bsg_block_pool(ctypes.byref(d), _ptr(k_cache), _ptr(page_table), _ptr(kv_lens),
                                                  _ptr(blk_begin), _ptr(block_cache), _stream(stream)))
    return block_cache


def _score_dims(q, block_cache, page_table, page_size, top_k):
    B, Hq, ql, D = q.shape
    P, Hkv, D2 = block_cache.shape
    if D2 != D:
        raise ValueError("q and block_cache disagree on head_dim")
    if page_table.shape[0] != B:
        raise ValueError("q and page_table disagree on the batch size")
    return BsgDims(B, Hq, Hkv, D, page_size, top_k, P, page_table.shape[1], _dtype_code(q.dtype))


def group_score(q, kv_lens, block_cache, page_table, scores, page_size: int, stream=None):
    """bsg_group_score: fp32 scores [B, Hkv, q_len, score_stride] (-inf off the candidates)."""
    _req(block_cache, "block_cache", None, 3)
    dev = block_cache.device
    _req(q, "q", block_cache.dtype, 4, dev)
    _tables(page_table, kv_lens, dev)
    _req(scores, "scores", torch.float32, 4, dev)
    d = _score_dims(q, block_cache, page_table, page_size, 1)
    if tuple(scores.shape[:3]) != (q.shape[0], block_cache.shape[1], q.shape[2]):
        raise ValueError("scores must be [B, Hkv, q_len, score_stride]")
    _check("bsg_group_score", lib().bsg_group_score(ctypes.byref(d), _ptr(q), q.shape[2], _ptr(kv_lens),
                                                    _ptr(block_cache), _ptr(page_table), _ptr(scores),
                                                    scores.shape[3], _stream(stream)))
    return scores


def topk_blocks(scores, kv_lens, block_idx, page_size: int, num_q_heads: int = None, stream=None):
    """bsg_topk_blocks: block_idx [B, Hkv, q_len, top_k] from scores [B, Hkv, q_len, stride]."""
    _req(scores, "scores", torch.float32, 4)
    dev = scores.device
    _req(kv_lens, "kv_lens", torch.int32, 1, dev)
    _req(block_idx, "block_idx", torch.int32, 4, dev)
    B, Hkv, ql, stride = scores.shape
    if tuple(block_idx.shape[:3]) != (B, Hkv, ql) or kv_lens.shape[0] != B:
        raise ValueError("block_idx must be [B, Hkv, q_len, top_k] with B = len(kv_lens)")
    top_k = block_idx.shape[3]
    d = BsgDims(B, num_q_heads or Hkv, Hkv, 64, page_size, top_k, 1, stride, BSG_F32)
    _check("bsg_topk_blocks", lib().bsg_topk_blocks(ctypes.byref(d), _ptr(scores), ql, stride, _ptr(kv_lens),
                                                    _ptr(block_idx), _stream(stream)))
    return block_idx


def group_score_topk_workspace_bytes(q, block_cache, page_table, page_size: int, top_k: int) -> int:
    d = _score_dims(q, block_cache, page_table, page_size, top_k)
    return int(lib().bsg_group_score_topk_workspace_bytes(ctypes.byref(d), q.shape[2]))


def group_score_topk(q, kv_lens, block_cache, page_table, block_idx, page_size: int, workspace=None,
                     stream=None):
    """bsg_group_score_topk: fused scoring + selection into block_idx [B, Hkv, q_len, top_k]."""
    _req(block_cache, "block_cache", None, 3)
    dev = block_cache.device
    _req(q, "q", block_cache.dtype, 4, dev)
    _tables(page_table, kv_lens, dev)
    _req(block_idx, "block_idx", torch.int32, 4, dev)
    if tuple(block_idx.shape[:3]) != (q.shape[0], block_cache.shape[1], q.shape[2]):
        raise ValueError("block_idx must be [B, Hkv, q_len, top_k]")
    d = _score_dims(q, block_cache, page_table, page_size, block_idx.shape[3])
    need = int(lib().bsg_group_score_topk_workspace_bytes(ctypes.byref(d), q.shape[2]))
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _req(workspace, "workspace", None, None, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("bsg_group_score_topk", lib().bsg_group_score_topk(
        ctypes.byref(d), _ptr(q), q.shape[2], _ptr(kv_lens), _ptr(block_cache), _ptr(page_table), _ptr(block_idx),
        _ptr(workspace), ws_bytes, _stream(stream)))
    return block_idx


def sparse_attn_prefill(q, kv_lens, k_cache, v_cache, page_table, block_idx, scale: float, out, lse=None,
                        stream=None):
    """bsg_sparse_attn_prefill: out [B, Hq, q_len, D] (and lse [B, Hq, q_len] fp32)."""
    _req(k_cache, "k_cache", None, 4)
    dev = k_cache.device
    _req(v_cache, "v_cache", k_cache.dtype, 4, dev)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    _req(q, "q", k_cache.dtype, 4, dev)
    _tables(page_table, kv_lens, dev)
    _req(block_idx, "block_idx", torch.int32, 4, dev)
    _req(out, "out", k_cache.dtype, 4, dev)
    B, Hq, ql, D = q.shape
    if out.shape != q.shape or D != k_cache.shape[3] or page_table.shape[0] != B:
        raise ValueError("shape mismatch between q, out, k_cache and page_table")
    if tuple(block_idx.shape[:3]) != (B, k_cache.shape[1], ql):
        raise ValueError("block_idx must be [B, Hkv, q_len, top_k]")
    if lse is not None:
        _req(lse, "lse", torch.float32, 3, dev)
        if tuple(lse.shape) != (B, Hq, ql):
            raise ValueError("lse must be [B, Hq, q_len]")
    d = dims(k_cache, page_table, Hq, block_idx.shape[3])
    _check("bsg_sparse_attn_prefill", lib().bsg_sparse_attn_prefill(
        ctypes.byref(d), _ptr(q), ql, _ptr(kv_lens), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        _ptr(block_idx), float(scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out


def _gate(gate, x, out):
    """Check a gated-fusion pair against out: x like out; gate fp32 with out's shape (one gate
    per element) or out's shape without its last dimension (one gate per row)."""
    _req(x, "x", out.dtype, out.dim(), out.device)
    if x.shape != out.shape:
        raise ValueError("x must have the shape of out")
    _req(gate, "gate", torch.float32, None, out.device)
    if gate.shape == out.shape:
        return 1
    if gate.shape == out.shape[:-1]:
        return 0
    raise ValueError("gate must have the shape of out, or of out without its last dimension")


def sparse_attn_prefill_gated(q, kv_lens, k_cache, v_cache, page_table, block_idx, scale: float, gate, x, out,
                              lse=None, stream=None):
    """bsg_sparse_attn_prefill_gated: out = gate * attention + (1 - gate) * x."""
    _req(k_cache, "k_cache", None, 4)
    dev = k_cache.device
    _req(v_cache, "v_cache", k_cache.dtype, 4, dev)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    _req(q, "q", k_cache.dtype, 4, dev)
    _tables(page_table, kv_lens, dev)
    _req(block_idx, "block_idx", torch.int32, 4, dev)
    _req(out, "out", k_cache.dtype, 4, dev)
    B, Hq, ql, D = q.shape
    if out.shape != q.shape or D != k_cache.shape[3] or page_table.shape[0] != B:
        raise ValueError("shape mismatch between q, out, k_cache and page_table")
    if tuple(block_idx.shape[:3]) != (B, k_cache.shape[1], ql):
        raise ValueError("block_idx must be [B, Hkv, q_len, top_k]")
    if lse is not None:
        _req(lse, "lse", torch.float32, 3, dev)
        if tuple(lse.shape) != (B, Hq, ql):
            raise ValueError("lse must be [B, Hq, q_len]")
    per_dim = _gate(gate, x, out)
    d = dims(k_cache, page_table, Hq, block_idx.shape[3])
    _check("bsg_sparse_attn_prefill_gated", lib().bsg_sparse_attn_prefill_gated(
        ctypes.byref(d), _ptr(q), ql, _ptr(kv_lens), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        _ptr(block_idx), float(scale), _ptr(gate), per_dim, _ptr(x), _ptr(out), _ptr(lse), _stream(stream)))
    return out


def decode_workspace_bytes(k_cache, page_table, num_q_heads: int, top_k: int) -> int:
    """Bytes of the decode workspace (no initialisation needed)."""
    d = dims(k_cache, page_table, num_q_heads, top_k)
    return int(lib().bsg_decode_workspace_bytes(ctypes.byref(d)))


def sparse_attn_decode(q, kv_lens, k_cache, v_cache, page_table, block_idx, scale: float, out, lse=None,
                       workspace=None, stream=None):
    """bsg_sparse_attn_decode: q [B, Hq, D], block_idx [B, Hkv, top_k] -> out [B, Hq, D]."""
    _req(k_cache, "k_cache", None, 4)
    dev = k_cache.device
    _req(v_cache, "v_cache", k_cache.dtype, 4, dev)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    _req(q, "q", k_cache.dtype, 3, dev)
    _tables(page_table, kv_lens, dev)
    _req(block_idx, "block_idx", torch.int32, 3, dev)
    _req(out, "out", k_cache.dtype, 3, dev)
    B, Hq, D = q.shape
    if out.shape != q.shape or D != k_cache.shape[3] or page_table.shape[0] != B:
        raise ValueError("shape mismatch between q, out, k_cache and page_table")
    if tuple(block_idx.shape[:2]) != (B, k_cache.shape[1]):
        raise ValueError("block_idx must be [B, Hkv, top_k]")
    if lse is not None:
        _req(lse, "lse", torch.float32, 2, dev)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse must be [B, Hq]")
    d = dims(k_cache, page_table, Hq, block_idx.shape[2])
    need = int(lib().bsg_decode_workspace_bytes(ctypes.byref(d)))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _req(workspace, "workspace", None, None, dev)
    _check("bsg_sparse_attn_decode", lib().bsg_sparse_attn_decode(
        ctypes.byref(d), _ptr(q), _ptr(kv_lens), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(block_idx),
        float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
        _stream(stream)))
    return out


def decode_step_workspace_bytes(k_cache, page_table, num_q_heads: int, top_k: int) -> int:
    d = dims(k_cache, page_table, num_q_heads, top_k)
    return int(lib().bsg_decode_step_workspace_bytes(ctypes.byref(d)))


def decode_step(q, kv_lens, block_cache, k_cache, v_cache, page_table, scale: float, block_idx, out, lse=None,
                workspace=None, stream=None):
    """bsg_decode_step: q [B, Hq, D] -> out [B, Hq, D]; the selection goes to block_idx [B, Hkv, top_k]."""
    _req(k_cache, "k_cache", None, 4)
    dev = k_cache.device
    _req(v_cache, "v_cache", k_cache.dtype, 4, dev)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    _req(block_cache, "block_cache", k_cache.dtype, 3, dev)
    P, Hkv, bs, D = k_cache.shape
    if tuple(block_cache.shape) != (P, Hkv, D):
        raise ValueError("block_cache must be [num_pages, Hkv, D]")
    _req(q, "q", k_cache.dtype, 3, dev)
    _tables(page_table, kv_lens, dev)
    _req(block_idx, "block_idx", torch.int32, 3, dev)
    _req(out, "out", k_cache.dtype, 3, dev)
    B, Hq, D2 = q.shape
    if out.shape != q.shape or D2 != D or page_table.shape[0] != B or tuple(block_idx.shape[:2]) != (B, Hkv):
        raise ValueError("shape mismatch between q, out, caches, page_table and block_idx")
    if lse is not None:
        _req(lse, "lse", torch.float32, 2, dev)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse must be [B, Hq]")
    d = dims(k_cache, page_table, Hq, block_idx.shape[2])
    need = int(lib().bsg_decode_step_workspace_bytes(ctypes.byref(d)))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _req(workspace, "workspace", None, None, dev)
    _check("bsg_decode_step", lib().bsg_decode_step(
        ctypes.byref(d), _ptr(q), _ptr(kv_lens), _ptr(block_cache), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        float(scale), _ptr(block_idx), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
        _ptr(lse), _stream(stream)))
    return out


def decode_step_gated(q, kv_lens, block_cache, k_cache, v_cache, page_table, scale: float, block_idx, gate, x, out,
                      lse=None, workspace=None, stream=None):
    """bsg_decode_step_gated: one decode step with out = gate * attention + (1 - gate) * x."""
    _req(k_cache, "k_cache", None, 4)
    dev = k_cache.device
    _req(v_cache, "v_cache", k_cache.dtype, 4, dev)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    _req(block_cache, "block_cache", k_cache.dtype, 3, dev)
    P, Hkv, bs, D = k_cache.shape
    if tuple(block_cache.shape) != (P, Hkv, D):
        raise ValueError("block_cache must be [num_pages, Hkv, D]")
    _req(q, "q", k_cache.dtype, 3, dev)
    _tables(page_table, kv_lens, dev)
    _req(block_idx, "block_idx", torch.int32, 3, dev)
    _req(out, "out", k_cache.dtype, 3, dev)
    B, Hq, D2 = q.shape
    if out.shape != q.shape or D2 != D or page_table.shape[0] != B or tuple(block_idx.shape[:2]) != (B, Hkv):
        raise ValueError("shape mismatch between q, out, caches, page_table and block_idx")
    if lse is not None:
        _req(lse, "lse", torch.float32, 2, dev)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse must be [B, Hq]")
    per_dim = _gate(gate, x, out)
    d = dims(k_cache, page_table, Hq, block_idx.shape[2])
    need = int(lib().bsg_decode_step_workspace_bytes(ctypes.byref(d)))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _req(workspace, "workspace", None, None, dev)
    _check("bsg_decode_step_gated", lib().bsg_decode_step_gated(
        ctypes.byref(d), _ptr(q), _ptr(kv_lens), _ptr(block_cache), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        float(scale), _ptr(block_idx), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(gate),
        per_dim, _ptr(x), _ptr(out), _ptr(lse), _stream(stream)))
    return out


def debug_errors(reset: bool = True) -> int:
    """Bits of the ids the kernels clamped since the last reset (a library built with
    -DBSG_DEBUG only: 1 page id, 2 block id, 4 token id); raises on a release build."""
    bits = ctypes.c_uint32(0)
    _check("bsg_debug_errors", lib().bsg_debug_errors(ctypes.byref(bits), 1 if reset else 0))
    return int(bits.value)


def noalloc_scratch_bytes() -> int:
    """Bytes of the static device scratch that bsg_decode_step_noalloc uses (per GPU)."""
    return int(lib().bsg_noalloc_scratch_bytes())


def decode_step_noalloc(q, kv_lens, block_cache, k_cache, v_cache, page_table, scale: float, block_idx, out,
                        lse=None, stream=None):
    """bsg_decode_step_noalloc: bsg_decode_step with the library's static scratch as workspace
    (nothing is allocated; calls that overlap in time on one GPU race)."""
    _req(k_cache, "k_cache", None, 4)
    dev = k_cache.device
    _req(v_cache, "v_cache", k_cache.dtype, 4, dev)
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    _req(block_cache, "block_cache", k_cache.dtype, 3, dev)
    P, Hkv, bs, D = k_cache.shape
    if tuple(block_cache.shape) != (P, Hkv, D):
        raise ValueError("block_cache must be [num_pages, Hkv, D]")
    _req(q, "q", k_cache.dtype, 3, dev)
    _tables(page_table, kv_lens, dev)
    _req(block_idx, "block_idx", torch.int32, 3, dev)
    _req(out, "out", k_cache.dtype, 3, dev)
    B, Hq, D2 = q.shape
    if out.shape != q.shape or D2 != D or page_table.shape[0] != B or tuple(block_idx.shape[:2]) != (B, Hkv):
        raise ValueError("shape mismatch between q, out, caches, page_table and block_idx")
    if lse is not None:
        _req(lse, "lse", torch.float32, 2, dev)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse must be [B, Hq]")
    d = dims(k_cache, page_table, Hq, block_idx.shape[2])
    _check("bsg_decode_step_noalloc", lib().bsg_decode_step_noalloc(
        ctypes.byref(d), _ptr(q), _ptr(kv_lens), _ptr(block_cache), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        float(scale), _ptr(block_idx), _ptr(out), _ptr(lse), _stream(stream)))
    return out


# ---------------------------------------------------------------------------- fp8 caches
def _fp8_pair(codes, scales, name, dev, shape):
    _req(codes, name + "_codes", torch.uint8, len(shape), dev)
    _req(scales, name + "_scales", torch.float32, 2, dev)
    if tuple(codes.shape) != tuple(shape) or tuple(scales.shape) != tuple(shape[:2]):
        raise ValueError(f"{name}: codes must be {tuple(shape)} uint8 and scales {tuple(shape[:2])} float32")


def quantize_pages_fp8(cache, page_table, kv_lens, codes, scales, stream=None):
    """bsg_quantize_pages_fp8: E4M3 codes + per-(page, head) power-of-two scales of a bf16 paged cache."""
    _req(cache, "cache", torch.bfloat16, 4)
    dev = cache.device
    _tables(page_table, kv_lens, dev)
    _fp8_pair(codes, scales, "cache", dev, cache.shape)
    d = dims(cache, page_table, cache.shape[1], 1)
    _check("bsg_quantize_pages_fp8", lib().bsg_quantize_pages_fp8(
        ctypes.byref(d), _ptr(cache), _ptr(page_table), _ptr(kv_lens), _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def _fp8_dims(k_codes, page_table, num_q_heads, top_k):
    P, Hkv, bs, D = k_codes.shape
    B, pts = page_table.shape
    return BsgDims(B, num_q_heads, Hkv, D, bs, top_k, P, pts, BSG_BF16)


def block_pool_fp8(k_codes, k_scales, page_table, kv_lens, rep_codes, rep_scales, blk_begin=None, stream=None):
    """bsg_block_pool_fp8: the fp8 block cache of the complete blocks from the fp8 key cache."""
    _req(k_codes, "k_codes", torch.uint8, 4)
    dev = k_codes.device
    P, Hkv, bs, D = k_codes.shape
    _fp8_pair(k_codes, k_scales, "k", dev, k_codes.shape)
    _tables(page_table, kv_lens, dev)
    _fp8_pair(rep_codes, rep_scales, "rep", dev, (P, Hkv, D))
    if blk_begin is not None:
        _req(blk_begin, "blk_begin", torch.int32, 1, dev)
        if blk_begin.shape[0] != page_table.shape[0]:
            raise ValueError("blk_begin must be [B]")
    d = _fp8_dims(k_codes, page_table, Hkv, 1)
    _check("bsg_block_pool_fp8", lib().bsg_block_pool_fp8(
        ctypes.byref(d), _ptr(k_codes), _ptr(k_scales), _ptr(page_table), _ptr(kv_lens), _ptr(blk_begin),
        _ptr(rep_codes), _ptr(rep_scales), _stream(stream)))
    return rep_codes, rep_scales


def decode_step_fp8(q, kv_lens, rep_codes, rep_scales, k_codes, k_scales, v_codes, v_scales, page_table,
                    scale: float, block_idx, out, lse=None, workspace=None, stream=None):
    """bsg_decode_step_fp8: bsg_decode_step over fp8 block, key and value caches (q, out bf16)."""
    _req(k_codes, "k_codes", torch.uint8, 4)
    dev = k_codes.device
    P, Hkv, bs, D = k_codes.shape
    _fp8_pair(k_codes, k_scales, "k", dev, k_codes.shape)
    _fp8_pair(v_codes, v_scales, "v", dev, k_codes.shape)
    _fp8_pair(rep_codes, rep_scales, "rep", dev, (P, Hkv, D))
    _req(q, "q", torch.bfloat16, 3, dev)
    _tables(page_table, kv_lens, dev)
    _req(block_idx, "block_idx", torch.int32, 3, dev)
    _req(out, "out", torch.bfloat16, 3, dev)
    B, Hq, D2 = q.shape
    if out.shape != q.shape or D2 != D or page_table.shape[0] != B or tuple(block_idx.shape[:2]) != (B, Hkv):
        raise ValueError("shape mismatch between q, out, caches, page_table and block_idx")
    if lse is not None:
        _req(lse, "lse", torch.float32, 2, dev)
        if tuple(lse.shape) != (B, Hq):
            raise ValueError("lse must be [B, Hq]")
    d = _fp8_dims(k_codes, page_table, Hq, block_idx.shape[2])
    need = int(lib().bsg_decode_step_workspace_bytes(ctypes.byref(d)))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _req(workspace, "workspace", None, None, dev)
    _check("bsg_decode_step_fp8", lib().bsg_decode_step_fp8(
        ctypes.byref(d), _ptr(q), _ptr(kv_lens), _ptr(rep_codes), _ptr(rep_scales), _ptr(k_codes), _ptr(k_scales),
        _ptr(v_codes), _ptr(v_scales), _ptr(page_table), float(scale), _ptr(block_idx), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))
    return out


# ---------------------------------------------------------------------------- token-level selection
def _ws(workspace, need, dev):
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _req(workspace, "workspace", None, None, dev)
    return workspace


def token_topk(q, kv_lens, k_cache, page_table, token_idx, block_idx=None, workspace=None, stream=None):
    """bsg_token_topk: q [B, Hq, D] -> token_idx [B, Hkv, K] (K = token_idx.shape[2]);
    block_idx [B, Hkv, k] makes it two-level."""
    _req(k_cache, "k_cache", torch.bfloat16, 4)
    dev = k_cache.device
    _req(q, "q", torch.bfloat16, 3, dev)
    _tables(page_table, kv_lens, dev)
    _req(token_idx, "token_idx", torch.int32, 3, dev)
    P, Hkv, bs, D = k_cache.shape
    B, Hq, _ = q.shape
    if tuple(token_idx.shape[:2]) != (B, Hkv) or q.shape[2] != D:
        raise ValueError("shape mismatch between q, k_cache and token_idx")
    kb = 1
    if block_idx is not None:
        _req(block_idx, "block_idx", torch.int32, 3, dev)
        if tuple(block_idx.shape[:2]) != (B, Hkv):
            raise ValueError("block_idx must be [B, Hkv, k]")
        kb = block_idx.shape[2]
    d = dims(k_cache, page_table, Hq, kb)
    workspace = _ws(workspace, int(lib().bsg_token_topk_workspace_bytes(ctypes.byref(d), int(block_idx is not None))),
                    dev)
    _check("bsg_token_topk", lib().bsg_token_topk(
        ctypes.byref(d), _ptr(q), _ptr(kv_lens), _ptr(k_cache), _ptr(page_table), _ptr(block_idx),
        token_idx.shape[2], _ptr(token_idx), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return token_idx


def sparse_attn_decode_tokens(q, kv_lens, k_cache, v_cache, page_table, token_idx, scale: float, out, lse=None,
                              workspace=None, stream=None):
    """bsg_sparse_attn_decode_tokens: attention of q [B, Hq, D] over token_idx [B, Hkv, K]."""
    _req(k_cache, "k_cache", torch.bfloat16, 4)
    dev = k_cache.device
    _req(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _req(q, "q", torch.bfloat16, 3, dev)
    _tables(page_table, kv_lens, dev)
    _req(token_idx, "token_idx", torch.int32, 3, dev)
    _req(out, "out", torch.bfloat16, 3, dev)
    B, Hq, D = q.shape
    if out.shape != q.shape or v_cache.shape != k_cache.shape or tuple(token_idx.shape[:2]) != (B, k_cache.shape[1]):
        raise ValueError("shape mismatch between q, out, caches and token_idx")
    if lse is not None:
        _req(lse, "lse", torch.float32, 2, dev)
    K = token_idx.shape[2]
    d = dims(k_cache, page_table, Hq, 1)
    workspace = _ws(workspace, int(lib().bsg_decode_tokens_workspace_bytes(ctypes.byref(d), K)), dev)
    _check("bsg_sparse_attn_decode_tokens", lib().bsg_sparse_attn_decode_tokens(
        ctypes.byref(d), _ptr(q), _ptr(kv_lens), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(token_idx), K,
        float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
        _stream(stream)))
    return out


def decode_step_tokens(q, kv_lens, k_cache, v_cache, page_table, scale: float, token_idx, out, lse=None,
                       block_cache=None, block_idx=None, workspace=None, stream=None):
    """bsg_decode_step_tokens: token-level step, or two-level when block_cache and block_idx
    [B, Hkv, k] are given (the block selection is written to block_idx)."""
    _req(k_cache, "k_cache", torch.bfloat16, 4)
    dev = k_cache.device
    _req(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _req(q, "q", torch.bfloat16, 3, dev)
    _tables(page_table, kv_lens, dev)
    _req(token_idx, "token_idx", torch.int32, 3, dev)
    _req(out, "out", torch.bfloat16, 3, dev)
    B, Hq, D = q.shape
    P, Hkv, bs, _ = k_cache.shape
    if out.shape != q.shape or v_cache.shape != k_cache.shape or tuple(token_idx.shape[:2]) != (B, Hkv):
        raise ValueError("shape mismatch between q, out, caches and token_idx")
    two = block_idx is not None
    kb = 1
    if two:
        if block_cache is None:
            raise ValueError("two-level steps need block_cache")
        _req(block_cache, "block_cache", torch.bfloat16, 3, dev)
        _req(block_idx, "block_idx", torch.int32, 3, dev)
        if tuple(block_idx.shape[:2]) != (B, Hkv) or tuple(block_cache.shape) != (P, Hkv, D):
            raise ValueError("block_idx must be [B, Hkv, k] and block_cache [P, Hkv, D]")
        kb = block_idx.shape[2]
    if lse is not None:
        _req(lse, "lse", torch.float32, 2, dev)
    K = token_idx.shape[2]
    d = dims(k_cache, page_table, Hq, kb)
    workspace = _ws(workspace, int(lib().bsg_decode_step_tokens_workspace_bytes(ctypes.byref(d), K, int(two))), dev)
    _check("bsg_decode_step_tokens", lib().bsg_decode_step_tokens(
        ctypes.byref(d), _ptr(q), _ptr(kv_lens), _ptr(block_cache), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        K, int(two), float(scale), _ptr(block_idx), _ptr(token_idx), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))
    return out


def token_topk_prefill(q, kv_lens, k_cache, page_table, token_idx, block_idx=None, workspace=None, stream=None):
    """bsg_token_topk_prefill: q [B, Hq, q_len, D] -> token_idx [B, Hkv, q_len, K]; two level
    when block_idx [B, Hkv, q_len, k] is given."""
    _req(k_cache, "k_cache", torch.bfloat16, 4)
    dev = k_cache.device
    _req(q, "q", torch.bfloat16, 4, dev)
    _tables(page_table, kv_lens, dev)
    _req(token_idx, "token_idx", torch.int32, 4, dev)
    B, Hq, ql, D = q.shape
    Hkv = k_cache.shape[1]
    if tuple(token_idx.shape[:3]) != (B, Hkv, ql) or D != k_cache.shape[3] or page_table.shape[0] != B:
        raise ValueError("token_idx must be [B, Hkv, q_len, K] and q match k_cache / page_table")
    kb = 1
    if block_idx is not None:
        _req(block_idx, "block_idx", torch.int32, 4, dev)
        if tuple(block_idx.shape[:3]) != (B, Hkv, ql):
            raise ValueError("block_idx must be [B, Hkv, q_len, k]")
        kb = block_idx.shape[3]
    d = dims(k_cache, page_table, Hq, kb)
    two = int(block_idx is not None)
    workspace = _ws(workspace, int(lib().bsg_token_topk_prefill_workspace_bytes(ctypes.byref(d), ql, two)), dev)
    _check("bsg_token_topk_prefill", lib().bsg_token_topk_prefill(
        ctypes.byref(d), _ptr(q), ql, _ptr(kv_lens), _ptr(k_cache), _ptr(page_table), _ptr(block_idx),
        token_idx.shape[3], _ptr(token_idx), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return token_idx


def sparse_attn_prefill_tokens(q, kv_lens, k_cache, v_cache, page_table, token_idx, scale: float, out, lse=None,
                               stream=None):
    """bsg_sparse_attn_prefill_tokens: out [B, Hq, q_len, D] (and lse [B, Hq, q_len])."""
    _req(k_cache, "k_cache", torch.bfloat16, 4)
    dev = k_cache.device
    _req(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _req(q, "q", torch.bfloat16, 4, dev)
    _tables(page_table, kv_lens, dev)
    _req(token_idx, "token_idx", torch.int32, 4, dev)
    _req(out, "out", torch.bfloat16, 4, dev)
    B, Hq, ql, D = q.shape
    Hkv = k_cache.shape[1]
    if out.shape != q.shape or v_cache.shape != k_cache.shape or tuple(token_idx.shape[:3]) != (B, Hkv, ql):
        raise ValueError("shape mismatch between q, out, caches and token_idx")
    if lse is not None:
        _req(lse, "lse", torch.float32, 3, dev)
        if tuple(lse.shape) != (B, Hq, ql):
            raise ValueError("lse must be [B, Hq, q_len]")
    d = dims(k_cache, page_table, Hq, 1)
    _check("bsg_sparse_attn_prefill_tokens", lib().bsg_sparse_attn_prefill_tokens(
        ctypes.byref(d), _ptr(q), ql, _ptr(kv_lens), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        _ptr(token_idx), token_idx.shape[3], float(scale), _ptr(out), _ptr(lse), _stream(stream)))
    return out
