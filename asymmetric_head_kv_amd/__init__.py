"""DiffQKV attention on AMD MI355X: Python binding of libdiffqkv.so.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory and the current stream.  The C ABI and its
contracts are documented in ``include/diffqkv.h``.

Tensor layouts (contiguous, on one GPU):
  q (decode)   [B, n_q, d_k]            q (prefill)  [B, t_new, n_q, d_k]
  k_cache      [B, n_k, l_cap, d_k]     v_cache      [B, n_v, l_cap, d_v]
  k_new        [B, t_new, n_k, d_k]     v_new        [B, t_new, n_v, d_v]
  ctx_len, pos int32 [B]
dtype float32 or bfloat16 (prefill: bfloat16).  ``scale=None`` passes 0, which
the library reads as its default 1/sqrt(d_k).
"""

from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["DQKVError", "lib_path", "load", "decode", "decode_chunk",
           "decode_workspace_bytes", "decode_selective", "selective_workspace_bytes",
           "decode_paged", "decode_selective_paged", "kv_append_paged", "kv_group_sharing", "augq", "augq_pack",
           "prefill", "prefill_paged", "prefill_workspace_bytes", "kv_append", "STATUS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree library; DQKV_LIBRARY names another build of the same sources
# (the test-suite's sanitizer build of the host code).
lib_path = os.environ.get("DQKV_LIBRARY") or os.path.join(_HERE, "libdiffqkv.so")

STATUS = {0: "DQKV_OK", -1: "DQKV_ERR_NULL", -2: "DQKV_ERR_SHAPE",
          -3: "DQKV_ERR_UNSUPPORTED", -4: "DQKV_ERR_WORKSPACE",
          -5: "DQKV_ERR_HIP", -6: "DQKV_ERR_ALIGN"}
F32, BF16 = 0, 1

_i32, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t

# Exported symbols and their C signatures (include/diffqkv.h).
SIGNATURES = {
    "dqkv_status_str": (ctypes.c_char_p, [_i32]),
    "diffqkv_decode_chunk": (_i32, [_i32] * 7 + [ctypes.POINTER(_i32)]),
    "diffqkv_decode_workspace": (_i32, [_i32] * 8 + [ctypes.POINTER(_sz)]),
    "kv_append": (_i32, [_i32] * 9 + [_vp] * 6),
    "diffqkv_decode": (_i32, [_i32] * 9 + [_f32] + [_vp] * 6 + [_i32, _vp, _sz, _vp]),
    "diffqkv_prefill": (_i32, [_i32] * 9 + [_f32] + [_vp] * 7 + [_sz, _vp]),
    "diffqkv_prefill_workspace": (_i32, [_i32] * 7 + [ctypes.POINTER(_sz)]),
    "diffqkv_prefill_paged": (_i32, [_i32] * 11 + [_f32] + [_vp] * 8 + [_sz, _vp]),
    "diffqkv_decode_split": (_i32, [_i32] * 9 + [_f32] + [_vp] * 6 + [_i32, _vp, _sz, _vp]),
    "diffqkv_decode_append": (_i32, [_i32] * 9 + [_f32] + [_vp] * 8 + [_i32, _vp, _sz, _vp]),
    "diffqkv_decode_append_noalloc": (_i32, [_i32] * 9 + [_f32] + [_vp] * 8 + [_i32, _vp]),
    "diffqkv_decode_combine": (_i32, [_i32] * 9 + [_vp] * 3 + [_i32, _vp, _sz, _vp]),
    "diffqkv_decode_selective_workspace": (_i32, [_i32] * 8 + [ctypes.POINTER(_sz)]),
    "diffqkv_decode_selective": (_i32, [_i32] * 9 + [_f32, _i32] + [_vp] * 10 + [_sz, _vp]),
    "diffqkv_decode_selective_paged": (_i32, [_i32] * 11 + [_f32, _i32] + [_vp] * 11 + [_sz, _vp]),
    "kv_append_paged": (_i32, [_i32] * 11 + [_vp] * 7),
    "diffqkv_decode_paged": (_i32, [_i32] * 11 + [_f32] + [_vp] * 9 + [_i32, _vp, _sz, _vp]),
    "kv_group_sharing": (_i32, [_i32] * 8 + [_vp] * 5),
    "augq_workspace": (_i32, [_i32] * 4 + [ctypes.POINTER(_sz)]),
    "augq_forward": (_i32, [_i32] * 4 + [_vp] * 6 + [_sz, _vp]),
    "augq_pack": (_i32, [_i32] * 2 + [_vp] * 3),
}

_lib = None


class DQKVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_str(status)}")


def load() -> ctypes.CDLL:
    """Load libdiffqkv.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise ImportError(
                f"{lib_path} is missing: build it with "
                "`python -m asymmetric_head_kv_amd.build` (or __graft_entry__.build())")
        lib = ctypes.CDLL(lib_path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load().dqkv_status_str(status).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise DQKVError(fn, status)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, dev) -> int:
    """The HIP stream to launch on: the tensors' device's current stream, or
    the given one (which must belong to that device)."""
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    if stream.device != dev:
        raise ValueError("stream is on another device than the tensors")
    return stream.cuda_stream


def _call(dev, fn: str, *args) -> None:
    """Call a library entry point with the tensors' device current, so its
    kernels launch on the GPU that holds the data."""
    with torch.cuda.device(dev):
        _check(fn, getattr(load(), fn)(*args))


def _device_tensors(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def decode_chunk(n_q, n_k, n_v, d_k, d_v, batch, max_ctx) -> int:
    """Rows per context chunk that diffqkv_decode picks automatically."""
    out = _i32()
    _check("diffqkv_decode_chunk",
           load().diffqkv_decode_chunk(n_q, n_k, n_v, d_k, d_v, batch, max_ctx,
                                       ctypes.byref(out)))
    return out.value


def decode_workspace_bytes(n_q, n_k, n_v, d_k, d_v, batch, max_ctx,
                           chunk_tokens: int = 0) -> int:
    out = _sz()
    _check("diffqkv_decode_workspace",
           load().diffqkv_decode_workspace(n_q, n_k, n_v, d_k, d_v, batch, max_ctx,
                                           chunk_tokens, ctypes.byref(out)))
    return out.value


def kv_append(k_new, v_new, pos, k_cache, v_cache, *, n_q=None, stream=None):
    """Write token-major rows k_new/v_new into the caches at rows pos[b] + t."""
    dev = _device_tensors(k_new, v_new, pos, k_cache, v_cache)
    B, T, n_k, d_k = k_new.shape
    n_v, d_v = v_new.shape[2], v_new.shape[3]
    if k_cache.shape[:2] != (B, n_k) or v_cache.shape[:2] != (B, n_v) or \
            k_cache.shape[3] != d_k or v_cache.shape[3] != d_v or \
            v_cache.shape[2] != k_cache.shape[2] or v_new.shape[:2] != (B, T):
        raise ValueError("inconsistent cache / new-row shapes")
    if pos.dtype != torch.int32 or pos.numel() != B:
        raise ValueError("pos must be int32 [B]")
    for t in (v_new, k_cache, v_cache):
        if t.dtype != k_new.dtype:
            raise TypeError("k_new, v_new and the caches must share one dtype")
    n_q = max(n_k, n_v) if n_q is None else n_q
    _call(dev, "kv_append",
          n_q, n_k, n_v, d_k, d_v, _dtype_code(k_new), B, T, k_cache.shape[2],
          _ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(k_cache), _ptr(v_cache), _stream(stream, dev))


def decode(q, k_cache, v_cache, ctx_len, *, max_ctx=None, scale=None, out=None,
           lse=None, chunk_tokens=0, workspace=None, k_new=None, v_new=None,
           stream=None):
    """One decode step; returns (out [B, n_q, d_v], lse [B, n_q] or None).

    With k_new [B, n_k, d_k] / v_new [B, n_v, d_v] the step first appends
    them at cache row ctx_len[b] - 1 (diffqkv_decode_append)."""
    dev = _device_tensors(q, k_cache, v_cache, ctx_len, out, lse, workspace, k_new, v_new)
    B, n_q, d_k = q.shape
    n_k, l_cap = k_cache.shape[1], k_cache.shape[2]
    n_v, d_v = v_cache.shape[1], v_cache.shape[3]
    if k_cache.shape != (B, n_k, l_cap, d_k) or v_cache.shape[:3] != (B, n_v, l_cap):
        raise ValueError("inconsistent q / cache shapes")
    if ctx_len.dtype != torch.int32 or ctx_len.numel() != B:
        raise ValueError("ctx_len must be int32 [B]")
    for t in (k_cache, v_cache, k_new, v_new):
        if t is not None and t.dtype != q.dtype:
            raise TypeError("q, the caches and the new rows must share one dtype")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None and (k_new.numel() != B * n_k * d_k or v_new.numel() != B * n_v * d_v):
        raise ValueError("k_new must hold [B, n_k, d_k] and v_new [B, n_v, d_v]")
    max_ctx = l_cap if max_ctx is None else int(max_ctx)
    scale = 0.0 if scale is None else float(scale)  # 0: the library's 1/sqrt(d_k)
    if out is None:
        out = torch.empty((B, n_q, d_v), dtype=q.dtype, device=q.device)
    elif out.shape != (B, n_q, d_v) or out.dtype != q.dtype:
        raise ValueError("out must be [B, n_q, d_v] in q's dtype")
    if lse is not None and (lse.shape != (B, n_q) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, n_q]")
    need = decode_workspace_bytes(n_q, n_k, n_v, d_k, d_v, B, max_ctx, chunk_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    if k_new is None:
        _call(dev, "diffqkv_decode",
              n_q, n_k, n_v, d_k, d_v, _dtype_code(q), B, l_cap, max_ctx, scale,
              _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len), _ptr(out), _ptr(lse),
              int(chunk_tokens), _ptr(workspace), ws_bytes, _stream(stream, dev))
    else:
        _call(dev, "diffqkv_decode_append",
              n_q, n_k, n_v, d_k, d_v, _dtype_code(q), B, l_cap, max_ctx, scale,
              _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len),
              _ptr(out), _ptr(lse), int(chunk_tokens), _ptr(workspace), ws_bytes,
              _stream(stream, dev))
    return out, lse


def selective_workspace_bytes(n_q, n_k, n_v, d_k, d_v, batch, max_ctx, top_k) -> int:
    out = _sz()
    _check("diffqkv_decode_selective_workspace",
           load().diffqkv_decode_selective_workspace(n_q, n_k, n_v, d_k, d_v, batch, max_ctx,
                                                     top_k, ctypes.byref(out)))
    return out.value


def decode_selective(q, k_cache, v_cache, ctx_len, *, top_k=100, max_ctx=None, scale=None,
                     out=None, lse=None, sel_idx=None, workspace=None, k_new=None,
                     v_new=None, stream=None):
    """Decode with selective V fetching: only the V rows of each query
    head's top_k attention weights are read and summed with their (full
    softmax) weights.  Returns (out [B, n_q, d_v], lse or None, sel_idx or
    None); pass sel_idx (int32 [B, n_q, top_k]) to receive the chosen rows.
    k_new / v_new fuse the append of the step's token as in decode()."""
    dev = _device_tensors(q, k_cache, v_cache, ctx_len, out, lse, sel_idx, workspace, k_new,
                          v_new)
    B, n_q, d_k = q.shape
    n_k, l_cap = k_cache.shape[1], k_cache.shape[2]
    n_v, d_v = v_cache.shape[1], v_cache.shape[3]
    if k_cache.shape != (B, n_k, l_cap, d_k) or v_cache.shape[:3] != (B, n_v, l_cap):
        raise ValueError("inconsistent q / cache shapes")
    if ctx_len.dtype != torch.int32 or ctx_len.numel() != B:
        raise ValueError("ctx_len must be int32 [B]")
    for t in (k_cache, v_cache, k_new, v_new):
        if t is not None and t.dtype != q.dtype:
            raise TypeError("q, the caches and the new rows must share one dtype")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None and (k_new.numel() != B * n_k * d_k or v_new.numel() != B * n_v * d_v):
        raise ValueError("k_new must hold [B, n_k, d_k] and v_new [B, n_v, d_v]")
    max_ctx = l_cap if max_ctx is None else int(max_ctx)
    scale = 0.0 if scale is None else float(scale)  # 0: the library's 1/sqrt(d_k)
    top_k = int(top_k)
    if out is None:
        out = torch.empty((B, n_q, d_v), dtype=q.dtype, device=q.device)
    elif out.shape != (B, n_q, d_v) or out.dtype != q.dtype:
        raise ValueError("out must be [B, n_q, d_v] in q's dtype")
    if lse is not None and (lse.shape != (B, n_q) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, n_q]")
    if sel_idx is not None and (sel_idx.shape != (B, n_q, top_k) or sel_idx.dtype != torch.int32):
        raise ValueError("sel_idx must be int32 [B, n_q, top_k]")
    if workspace is None:
        need = selective_workspace_bytes(n_q, n_k, n_v, d_k, d_v, B, max_ctx, top_k)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _call(dev, "diffqkv_decode_selective",
          n_q, n_k, n_v, d_k, d_v, _dtype_code(q), B, l_cap, max_ctx, scale, top_k,
          _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len),
          _ptr(out), _ptr(lse), _ptr(sel_idx), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(stream, dev))
    return out, lse, sel_idx


def _pages_shape(k_pages, v_pages, block_table, B=None):
    num_pages, n_k, P, d_k = k_pages.shape
    if v_pages.shape[0] != num_pages or v_pages.shape[2] != P:
        raise ValueError("k_pages [N, n_k, P, d_k] and v_pages [N, n_v, P, d_v] must agree")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or \
            (B is not None and block_table.shape[0] != B):
        raise ValueError("block_table must be int32 [B, max_blocks]")
    return num_pages, n_k, P, d_k, v_pages.shape[1], v_pages.shape[3], block_table.shape[1]


def kv_append_paged(k_new, v_new, pos, block_table, k_pages, v_pages, *, n_q=None,
                    stream=None):
    """kv_append into a paged cache: token t of sequence b goes to row
    pos[b] + t, i.e. slot (row % P) of page block_table[b, row // P]."""
    dev = _device_tensors(k_new, v_new, pos, block_table, k_pages, v_pages)
    B, T, n_k, d_k = k_new.shape
    num_pages, n_k2, P, d_k2, n_v, d_v, max_blocks = _pages_shape(k_pages, v_pages,
                                                                  block_table, B)
    if (n_k2, d_k2) != (n_k, d_k) or v_new.shape != (B, T, n_v, d_v):
        raise ValueError("inconsistent page / new-row shapes")
    if pos.dtype != torch.int32 or pos.numel() != B:
        raise ValueError("pos must be int32 [B]")
    for t in (v_new, k_pages, v_pages):
        if t.dtype != k_new.dtype:
            raise TypeError("k_new, v_new and the page pools must share one dtype")
    n_q = max(n_k, n_v) if n_q is None else n_q
    _call(dev, "kv_append_paged",
          n_q, n_k, n_v, d_k, d_v, _dtype_code(k_new), B, T, P, num_pages, max_blocks,
          _ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(block_table), _ptr(k_pages), _ptr(v_pages),
          _stream(stream, dev))


def decode_paged(q, k_pages, v_pages, block_table, ctx_len, *, max_ctx=None, scale=None,
                 out=None, lse=None, chunk_tokens=0, workspace=None, k_new=None, v_new=None,
                 stream=None):
    """decode() over a paged cache (k_pages [N, n_k, P, d_k], v_pages
    [N, n_v, P, d_v], block_table int32 [B, max_blocks])."""
    dev = _device_tensors(q, k_pages, v_pages, block_table, ctx_len, out, lse, workspace, k_new,
                          v_new)
    B, n_q, d_k = q.shape
    num_pages, n_k, P, d_k2, n_v, d_v, max_blocks = _pages_shape(k_pages, v_pages,
                                                                 block_table, B)
    if d_k2 != d_k:
        raise ValueError("q and k_pages disagree on d_k")
    if ctx_len.dtype != torch.int32 or ctx_len.numel() != B:
        raise ValueError("ctx_len must be int32 [B]")
    for t in (k_pages, v_pages, k_new, v_new):
        if t is not None and t.dtype != q.dtype:
            raise TypeError("q, the page pools and the new rows must share one dtype")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None and (k_new.numel() != B * n_k * d_k or v_new.numel() != B * n_v * d_v):
        raise ValueError("k_new must hold [B, n_k, d_k] and v_new [B, n_v, d_v]")
    max_ctx = max_blocks * P if max_ctx is None else int(max_ctx)
    scale = 0.0 if scale is None else float(scale)  # 0: the library's 1/sqrt(d_k)
    if out is None:
        out = torch.empty((B, n_q, d_v), dtype=q.dtype, device=q.device)
    elif out.shape != (B, n_q, d_v) or out.dtype != q.dtype:
        raise ValueError("out must be [B, n_q, d_v] in q's dtype")
    if lse is not None and (lse.shape != (B, n_q) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, n_q]")
    need = decode_workspace_bytes(n_q, n_k, n_v, d_k, d_v, B, max_ctx, chunk_tokens)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _call(dev, "diffqkv_decode_paged",
          n_q, n_k, n_v, d_k, d_v, _dtype_code(q), B, P, num_pages, max_blocks, max_ctx, scale,
          _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
          _ptr(ctx_len), _ptr(out), _ptr(lse), int(chunk_tokens), _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(stream, dev))
    return out, lse


def kv_group_sharing(k_cache, v_cache, *, n_q=None, stream=None):
    """Expand the side with fewer heads to max(n_k, n_v) heads (each head
    repeated in place); returns new (k, v) tensors."""
    dev = _device_tensors(k_cache, v_cache)
    B, n_k, l_cap, d_k = k_cache.shape
    n_v, d_v = v_cache.shape[1], v_cache.shape[3]
    if v_cache.shape[0] != B or v_cache.shape[2] != l_cap or v_cache.dtype != k_cache.dtype:
        raise ValueError("inconsistent K / V cache shapes")
    n_h = max(n_k, n_v)
    n_q = n_h if n_q is None else n_q
    k_out = torch.empty((B, n_h, l_cap, d_k), dtype=k_cache.dtype, device=k_cache.device)
    v_out = torch.empty((B, n_h, l_cap, d_v), dtype=v_cache.dtype, device=v_cache.device)
    _call(dev, "kv_group_sharing",
          n_q, n_k, n_v, d_k, d_v, _dtype_code(k_cache), B, l_cap, _ptr(k_cache), _ptr(v_cache),
          _ptr(k_out), _ptr(v_out), _stream(stream, dev))
    return k_out, v_out


def augq_pack(w, *, stream=None):
    """Pack a bf16 weight [n_out, n_in] (out, in layout) for augq: returns
    [n_out // 16, n_in // 32, 64, 8] in matrix-core fragment order."""
    dev = _device_tensors(w)
    if w.dtype != torch.bfloat16 or w.dim() != 2:
        raise TypeError("augq_pack takes a 2-D bfloat16 weight")
    n_out, n_in = w.shape
    wp = torch.empty((n_out // 16, n_in // 32, 64, 8), dtype=torch.bfloat16, device=w.device)
    _call(dev, "augq_pack",
          n_out, n_in, _ptr(w), _ptr(wp), _stream(stream, dev))
    return wp


def augq(h, w_gate_p, w_up_p, w_down_p, *, out=None, workspace=None, stream=None):
    """Augmented-Q projection, bf16: q = (silu(h W_gate^T) * h W_up^T) W_down^T.
    h [M, d_m]; weights packed by augq_pack (w_gate, w_up from [d_i, d_m],
    w_down from [d_out, d_i]).  Returns q [M, d_out]."""
    dev = _device_tensors(h, w_gate_p, w_up_p, w_down_p, out, workspace)
    M, d_m = h.shape
    d_i = w_gate_p.shape[0] * 16
    d_out = w_down_p.shape[0] * 16
    for w, n_out, n_in in ((w_gate_p, d_i, d_m), (w_up_p, d_i, d_m), (w_down_p, d_out, d_i)):
        if tuple(w.shape) != (n_out // 16, n_in // 32, 64, 8):
            raise ValueError("weights must come from augq_pack with matching sizes")
    for t in (h, w_gate_p, w_up_p, w_down_p):
        if t.dtype != torch.bfloat16:
            raise TypeError("augq takes bfloat16 tensors")
    if out is None:
        out = torch.empty((M, d_out), dtype=torch.bfloat16, device=h.device)
    elif out.shape != (M, d_out) or out.dtype != torch.bfloat16:
        raise ValueError("out must be bfloat16 [M, d_out]")
    need = _sz()
    _check("augq_workspace", load().augq_workspace(M, d_m, d_i, d_out, ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(max(need.value, 16), dtype=torch.uint8, device=h.device)
    _call(dev, "augq_forward",
          M, d_m, d_i, d_out, _ptr(h), _ptr(w_gate_p), _ptr(w_up_p), _ptr(w_down_p), _ptr(out),
          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, dev))
    return out


def prefill_workspace_bytes(n_q, n_k, n_v, d_k, d_v, batch, t_new) -> int:
    out = _sz()
    _check("diffqkv_prefill_workspace",
           load().diffqkv_prefill_workspace(n_q, n_k, n_v, d_k, d_v, batch, t_new,
                                            ctypes.byref(out)))
    return out.value


def prefill(q, k_cache, v_cache, ctx_len, *, scale=None, out=None, lse=None,
            workspace=None, stream=None):
    """Causal prefill of t_new rows (already appended); returns (out, lse).

    A workspace of prefill_workspace_bytes is allocated when none is given
    (pass one to avoid the allocation; an empty tensor runs unsplit)."""
    dev = _device_tensors(q, k_cache, v_cache, ctx_len, out, lse, workspace)
    B, T, n_q, d_k = q.shape
    n_k, l_cap = k_cache.shape[1], k_cache.shape[2]
    n_v, d_v = v_cache.shape[1], v_cache.shape[3]
    if k_cache.shape != (B, n_k, l_cap, d_k) or v_cache.shape[:3] != (B, n_v, l_cap):
        raise ValueError("inconsistent q / cache shapes")
    if ctx_len.dtype != torch.int32 or ctx_len.numel() != B:
        raise ValueError("ctx_len must be int32 [B]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the caches must share one dtype")
    scale = 0.0 if scale is None else float(scale)  # 0: the library's 1/sqrt(d_k)
    if out is None:
        out = torch.empty((B, T, n_q, d_v), dtype=q.dtype, device=q.device)
    elif out.shape != (B, T, n_q, d_v) or out.dtype != q.dtype:
        raise ValueError("out must be [B, t_new, n_q, d_v] in q's dtype")
    if lse is not None and (lse.shape != (B, T, n_q) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, t_new, n_q]")
    if workspace is None:
        need = prefill_workspace_bytes(n_q, n_k, n_v, d_k, d_v, B, T)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _call(dev, "diffqkv_prefill",
          n_q, n_k, n_v, d_k, d_v, _dtype_code(q), B, T, l_cap, scale,
          _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(ctx_len), _ptr(out), _ptr(lse),
          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, dev))
    return out, lse



def prefill_paged(q, k_pages, v_pages, block_table, ctx_len, *, scale=None, out=None,
                  lse=None, workspace=None, stream=None):
    """prefill() over a paged cache (k_pages [N, n_k, P, d_k], v_pages
    [N, n_v, P, d_v], block_table int32 [B, max_blocks]); bit-identical to
    prefill() on the equivalent contiguous cache."""
    dev = _device_tensors(q, k_pages, v_pages, block_table, ctx_len, out, lse, workspace)
    B, T, n_q, d_k = q.shape
    num_pages, n_k, P, d_k2, n_v, d_v, max_blocks = _pages_shape(k_pages, v_pages,
                                                                 block_table, B)
    if d_k2 != d_k:
        raise ValueError("q and k_pages disagree on d_k")
    if ctx_len.dtype != torch.int32 or ctx_len.numel() != B:
        raise ValueError("ctx_len must be int32 [B]")
    if k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("q and the page pools must share one dtype")
    scale = 0.0 if scale is None else float(scale)  # 0: the library's 1/sqrt(d_k)
    if out is None:
        out = torch.empty((B, T, n_q, d_v), dtype=q.dtype, device=q.device)
    elif out.shape != (B, T, n_q, d_v) or out.dtype != q.dtype:
        raise ValueError("out must be [B, t_new, n_q, d_v] in q's dtype")
    if lse is not None and (lse.shape != (B, T, n_q) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, t_new, n_q]")
    if workspace is None:
        need = prefill_workspace_bytes(n_q, n_k, n_v, d_k, d_v, B, T)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _call(dev, "diffqkv_prefill_paged",
          n_q, n_k, n_v, d_k, d_v, _dtype_code(q), B, T, P, num_pages, max_blocks, scale,
          _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(ctx_len), _ptr(out),
          _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
          _stream(stream, dev))
    return out, lse



def decode_selective_paged(q, k_pages, v_pages, block_table, ctx_len, *, top_k=100,
                           max_ctx=None, scale=None, out=None, lse=None, sel_idx=None,
                           workspace=None, k_new=None, v_new=None, stream=None):
    """decode_selective() over a paged cache (k_pages [N, n_k, P, d_k],
    v_pages [N, n_v, P, d_v], block_table int32 [B, max_blocks])."""
    dev = _device_tensors(q, k_pages, v_pages, block_table, ctx_len, out, lse, sel_idx,
                          workspace, k_new, v_new)
    B, n_q, d_k = q.shape
    num_pages, n_k, P, d_k2, n_v, d_v, max_blocks = _pages_shape(k_pages, v_pages,
                                                                 block_table, B)
    if d_k2 != d_k:
        raise ValueError("q and k_pages disagree on d_k")
    if ctx_len.dtype != torch.int32 or ctx_len.numel() != B:
        raise ValueError("ctx_len must be int32 [B]")
    for t in (k_pages, v_pages, k_new, v_new):
        if t is not None and t.dtype != q.dtype:
            raise TypeError("q, the page pools and the new rows must share one dtype")
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None and (k_new.numel() != B * n_k * d_k or v_new.numel() != B * n_v * d_v):
        raise ValueError("k_new must hold [B, n_k, d_k] and v_new [B, n_v, d_v]")
    max_ctx = max_blocks * P if max_ctx is None else int(max_ctx)
    scale = 0.0 if scale is None else float(scale)  # 0: the library's 1/sqrt(d_k)
    top_k = int(top_k)
    if out is None:
        out = torch.empty((B, n_q, d_v), dtype=q.dtype, device=q.device)
    elif out.shape != (B, n_q, d_v) or out.dtype != q.dtype:
        raise ValueError("out must be [B, n_q, d_v] in q's dtype")
    if lse is not None and (lse.shape != (B, n_q) or lse.dtype != torch.float32):
        raise ValueError("lse must be float32 [B, n_q]")
    if sel_idx is not None and (sel_idx.shape != (B, n_q, top_k) or sel_idx.dtype != torch.int32):
        raise ValueError("sel_idx must be int32 [B, n_q, top_k]")
    if workspace is None:
        need = selective_workspace_bytes(n_q, n_k, n_v, d_k, d_v, B, max_ctx, top_k)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _call(dev, "diffqkv_decode_selective_paged",
          n_q, n_k, n_v, d_k, d_v, _dtype_code(q), B, P, num_pages, max_blocks, max_ctx, scale,
          top_k, _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages),
          _ptr(block_table), _ptr(ctx_len), _ptr(out), _ptr(lse), _ptr(sel_idx),
          _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, dev))
    return out, lse, sel_idx
