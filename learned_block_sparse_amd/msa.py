"""Thin Python binding of the C ABI in ``include/msa.h`` (``libmsa.so``).

Argument marshalling only: every step of the MSA hot path runs in the HIP
kernels of the library.  PyTorch provides device memory (tensors, and the
workspace when the caller passes none) and the current stream.  There is no
fallback: if the library is missing or a call fails, an exception is raised.

The functions carry the C names.  Tensor layouts are those of the header:

* ``q_idx [Tq, G, d_idx]``, ``k_idx [Tk, d_idx]`` (fp32, bf16 or float8_e4m3fn)
* ``q [Tq, Hq, D]``, ``k, v [Tk, Hkv, D]``
* ``block_idx [Tq, G, topk]`` int32, ``cu_seqlens_q/k [B + 1]`` int32
* decode: ``q [B, Hq, D]``, ``cache_offsets [B]`` int64, ``ctx_lens [B]`` int32
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP = range(5)
MSA_F32, MSA_BF16, MSA_FP8_E4M3 = 0, 1, 2

_lib = None


class MSAError(RuntimeError):
    def __init__(self, status: int, where: str):
        name = lib().msa_status_string(status).decode()
        extra = ""
        if status == MSA_ERR_HIP:
            extra = f" (hipError {lib().msa_last_hip_error()})"
        super().__init__(f"{where}: {name}{extra}")
        self.status = status


def lib():
    """The loaded ``libmsa.so`` (ctypes); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m learned_block_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.msa_status_string.restype = ctypes.c_char_p
        L.msa_status_string.argtypes = [i32]
        L.msa_last_hip_error.restype = i32
        L.msa_last_hip_error.argtypes = []
        L.msa_index_topk_workspace_size.restype = sz
        L.msa_index_topk_workspace_size.argtypes = [i32] * 6
        L.msa_index_topk.restype = i32
        L.msa_index_topk.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, sz, vp]
        L.msa_index_topk_noalloc.restype = i32
        L.msa_index_topk_noalloc.argtypes = [vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp]
        L.msa_sparse_attn_workspace_size.restype = sz
        L.msa_sparse_attn_workspace_size.argtypes = [i32] * 8
        L.msa_sparse_attn_prefill.restype = i32
        L.msa_sparse_attn_prefill.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                              i32, ctypes.c_float, i32, vp, vp, vp, sz, vp]
        L.msa_sparse_attn_decode.restype = i32
        L.msa_sparse_attn_decode.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                             ctypes.c_float, i32, vp, vp, vp, sz, vp]
        L.msa_sparse_attn_prefill_ex.restype = i32
        L.msa_sparse_attn_prefill_ex.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                 i32, i32, ctypes.c_float, i32, vp, vp, vp, vp, sz, vp]
        L.msa_sparse_attn_decode_ex.restype = i32
        L.msa_sparse_attn_decode_ex.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                i32, ctypes.c_float, i32, vp, vp, vp, vp, sz, vp]
        L.msa_sparse_attn_backward_workspace_size.restype = sz
        L.msa_sparse_attn_backward_workspace_size.argtypes = [i32] * 7
        L.msa_sparse_attn_backward.restype = i32
        L.msa_sparse_attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32,
                                               i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, sz, vp]
        L.msa_index_kl_workspace_size.restype = sz
        L.msa_index_kl_workspace_size.argtypes = [i32] * 5
        L.msa_index_kl_backward.restype = i32
        L.msa_index_kl_backward.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                            vp, vp, vp, vp, sz, vp]
        L.msa_index_frontend.restype = i32
        L.msa_index_frontend.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, ctypes.c_int64, i32, i32, i32, i32,
                                         ctypes.c_float, ctypes.c_float, vp, vp, i32, vp]
        L.msa_index_frontend_backward_workspace_size.restype = sz
        L.msa_index_frontend_backward_workspace_size.argtypes = [ctypes.c_int64, i32, i32, i32]
        L.msa_index_frontend_backward.restype = i32
        L.msa_index_frontend_backward.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, ctypes.c_int64, i32, i32, i32,
                                                  i32, ctypes.c_float, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp,
                                                  sz, vp]
        _lib = L
    return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MSA_F32
    if t.dtype == torch.bfloat16:
        return MSA_BF16
    if t.dtype == torch.float8_e4m3fn:
        return MSA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16, or float8_e4m3fn for index and K/V tensors)")


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _on_launch_stream(fn):
    """Run ``fn`` with its launch stream as torch's current stream.

    Outputs and workspaces the binding allocates are then owned by the stream
    the library's kernels run on: the caching allocator hands their memory to
    a later allocation only on that same stream, ordered after the kernels,
    even when the caller launches on a side stream and drops the workspace.
    A raw ``hipStream_t`` handle is wrapped as an external stream."""
    @functools.wraps(fn)
    def wrapped(*args, stream=None, **kwargs):
        if stream is None:
            return fn(*args, stream=None, **kwargs)
        s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
        with torch.cuda.stream(s):
            return fn(*args, stream=s, **kwargs)
    return wrapped


def _check(status: int, where: str):
    if status != MSA_OK:
        raise MSAError(status, where)


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace smaller than the {nbytes} bytes required")
    return workspace, workspace.numel() * workspace.element_size()


def msa_index_topk_workspace_size(batch, max_q_len, max_kv_len, num_groups, block_size, topk) -> int:
    return lib().msa_index_topk_workspace_size(batch, max_q_len, max_kv_len, num_groups, block_size, topk)


def msa_sparse_attn_workspace_size(batch, max_q_len, max_kv_len, num_heads, num_kv_heads, head_dim,
                                   topk, num_splits=0) -> int:
    return lib().msa_sparse_attn_workspace_size(batch, max_q_len, max_kv_len, num_heads, num_kv_heads,
                                                head_dim, topk, num_splits)


@_on_launch_stream
def msa_index_topk(q_idx, k_idx, cu_seqlens_q, cu_seqlens_k, max_q_len: int, max_kv_len: int,
                   block_size: int = 128, topk: int = 16, block_idx=None, workspace=None, stream=None):
    """Selected block ids ``[Tq, G, topk]`` (int32, ascending, -1 padded)."""
    if q_idx.dim() != 3 or k_idx.dim() != 2 or q_idx.shape[2] != k_idx.shape[1]:
        raise ValueError("q_idx must be [Tq, G, d_idx] and k_idx [Tk, d_idx]")
    if q_idx.dtype != k_idx.dtype:
        raise TypeError("q_idx and k_idx must share a dtype")
    tq, G, di = q_idx.shape
    batch = cu_seqlens_q.numel() - 1
    if block_idx is None:
        block_idx = torch.empty((tq, G, topk), dtype=torch.int32, device=q_idx.device)
    need = msa_index_topk_workspace_size(batch, max_q_len, max_kv_len, G, block_size, topk)
    ws, ws_bytes = _workspace(need, q_idx.device, workspace)
    st = lib().msa_index_topk(_dev(q_idx, "q_idx"), _dev(k_idx, "k_idx"), _dtype_code(q_idx),
                              _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
                              _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32), batch, max_q_len, max_kv_len,
                              G, di, block_size, topk, _dev(block_idx, "block_idx", torch.int32),
                              ws.data_ptr() if ws is not None else None, ws_bytes, _stream(stream))
    _check(st, "msa_index_topk")
    return block_idx


def _prefill(ex, q, k, v, block_idx, cu_seqlens_q, cu_seqlens_k, max_q_len, max_kv_len, block_size, topk,
             softmax_scale, num_splits, out, lse, return_lse, workspace, stream, block_lse=None):
    tq, hq, d = q.shape
    hkv = k.shape[1]
    batch = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    need = msa_sparse_attn_workspace_size(batch, max_q_len, max_kv_len, hq, hkv, d, topk, num_splits)
    ws, ws_bytes = _workspace(need, q.device, workspace)
    kv_dtype = k.dtype if ex else q.dtype
    ptrs = [_dev(q, "q"), _dev(k, "k", kv_dtype), _dev(v, "v", kv_dtype), _dtype_code(q)]
    if ex:
        ptrs.append(_dtype_code(k))
    fn = lib().msa_sparse_attn_prefill_ex if ex else lib().msa_sparse_attn_prefill
    st = fn(*ptrs, _dev(block_idx, "block_idx", torch.int32), _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
            _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32), batch, max_q_len, max_kv_len, hq, hkv, d,
            block_size, topk, float(softmax_scale), num_splits, _dev(out, "out", q.dtype),
            _dev(lse, "lse", torch.float32) if lse is not None else None,
            *([_dev(block_lse, "block_lse", torch.float32) if block_lse is not None else None] if ex else []),
            ws.data_ptr() if ws is not None else None, ws_bytes, _stream(stream))
    _check(st, "msa_sparse_attn_prefill_ex" if ex else "msa_sparse_attn_prefill")
    return out, lse


def _decode(ex, q, k_cache, v_cache, block_idx, cache_offsets, ctx_lens, max_ctx, block_size, topk,
            softmax_scale, num_splits, out, lse, return_lse, workspace, stream, block_lse=None):
    batch, hq, d = q.shape
    hkv = k_cache.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    need = msa_sparse_attn_workspace_size(batch, 1, max_ctx, hq, hkv, d, topk, num_splits)
    ws, ws_bytes = _workspace(need, q.device, workspace)
    kv_dtype = k_cache.dtype if ex else q.dtype
    ptrs = [_dev(q, "q"), _dev(k_cache, "k_cache", kv_dtype), _dev(v_cache, "v_cache", kv_dtype), _dtype_code(q)]
    if ex:
        ptrs.append(_dtype_code(k_cache))
    fn = lib().msa_sparse_attn_decode_ex if ex else lib().msa_sparse_attn_decode
    st = fn(*ptrs, _dev(block_idx, "block_idx", torch.int32), _dev(cache_offsets, "cache_offsets", torch.int64),
            _dev(ctx_lens, "ctx_lens", torch.int32), batch, max_ctx, hq, hkv, d, block_size, topk,
            float(softmax_scale), num_splits, _dev(out, "out", q.dtype),
            _dev(lse, "lse", torch.float32) if lse is not None else None,
            *([_dev(block_lse, "block_lse", torch.float32) if block_lse is not None else None] if ex else []),
            ws.data_ptr() if ws is not None else None, ws_bytes, _stream(stream))
    _check(st, "msa_sparse_attn_decode_ex" if ex else "msa_sparse_attn_decode")
    return out, lse


# Size of the static scratch msa_index_topk_noalloc uses (MSA_NOALLOC_SCRATCH_BYTES in include/msa.h).
NOALLOC_SCRATCH_BYTES = 32 << 20


@_on_launch_stream
def msa_index_topk_noalloc(q_idx, k_idx, cu_seqlens_q, cu_seqlens_k, max_q_len: int, max_kv_len: int,
                           block_size: int = 128, topk: int = 16, block_idx=None, stream=None):
    """msa_index_topk with the library's static scratch instead of a workspace.

    Pass ``block_idx`` (``[Tq, G, topk]`` int32) to make the call allocate
    nothing at all; calls on one GPU must not overlap in time."""
    if q_idx.dim() != 3 or k_idx.dim() != 2 or q_idx.shape[2] != k_idx.shape[1]:
        raise ValueError("q_idx must be [Tq, G, d_idx] and k_idx [Tk, d_idx]")
    if q_idx.dtype != k_idx.dtype:
        raise TypeError("q_idx and k_idx must share a dtype")
    tq, G, di = q_idx.shape
    batch = cu_seqlens_q.numel() - 1
    if block_idx is None:
        block_idx = torch.empty((tq, G, topk), dtype=torch.int32, device=q_idx.device)
    st = lib().msa_index_topk_noalloc(_dev(q_idx, "q_idx"), _dev(k_idx, "k_idx"), _dtype_code(q_idx),
                                      _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
                                      _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32), batch, max_q_len,
                                      max_kv_len, G, di, block_size, topk,
                                      _dev(block_idx, "block_idx", torch.int32), _stream(stream))
    _check(st, "msa_index_topk_noalloc")
    return block_idx


@_on_launch_stream
def msa_sparse_attn_prefill(q, k, v, block_idx, cu_seqlens_q, cu_seqlens_k, max_q_len: int,
                            max_kv_len: int, block_size: int = 128, topk: int = 16,
                            softmax_scale: float = 0.0, num_splits: int = 0, out=None, lse=None,
                            return_lse: bool = True, workspace=None, stream=None):
    """``(out [Tq, Hq, D], lse [Tq, Hq] fp32 or None)``; q, k, v share a dtype."""
    return _prefill(False, q, k, v, block_idx, cu_seqlens_q, cu_seqlens_k, max_q_len, max_kv_len, block_size,
                    topk, softmax_scale, num_splits, out, lse, return_lse, workspace, stream)


@_on_launch_stream
def msa_sparse_attn_prefill_ex(q, k, v, block_idx, cu_seqlens_q, cu_seqlens_k, max_q_len: int,
                               max_kv_len: int, block_size: int = 128, topk: int = 16,
                               softmax_scale: float = 0.0, num_splits: int = 0, out=None, lse=None,
                               return_lse: bool = True, workspace=None, stream=None, block_lse=None):
    """As msa_sparse_attn_prefill with the K/V element type taken from ``k``
    (e.g. bfloat16 q with float8_e4m3fn k and v); ``block_lse`` ([Tq, Hq,
    topk] fp32, optional) receives the per-slot block LSEs."""
    return _prefill(True, q, k, v, block_idx, cu_seqlens_q, cu_seqlens_k, max_q_len, max_kv_len, block_size,
                    topk, softmax_scale, num_splits, out, lse, return_lse, workspace, stream, block_lse)


@_on_launch_stream
def msa_sparse_attn_decode(q, k_cache, v_cache, block_idx, cache_offsets, ctx_lens, max_ctx: int,
                           block_size: int = 128, topk: int = 16, softmax_scale: float = 0.0,
                           num_splits: int = 0, out=None, lse=None, return_lse: bool = True,
                           workspace=None, stream=None):
    """``(out [B, Hq, D], lse [B, Hq] fp32 or None)`` for one decode step."""
    return _decode(False, q, k_cache, v_cache, block_idx, cache_offsets, ctx_lens, max_ctx, block_size, topk,
                   softmax_scale, num_splits, out, lse, return_lse, workspace, stream)


@_on_launch_stream
def msa_sparse_attn_decode_ex(q, k_cache, v_cache, block_idx, cache_offsets, ctx_lens, max_ctx: int,
                              block_size: int = 128, topk: int = 16, softmax_scale: float = 0.0,
                              num_splits: int = 0, out=None, lse=None, return_lse: bool = True,
                              workspace=None, stream=None, block_lse=None):
    """As msa_sparse_attn_decode with the KV-cache element type taken from
    ``k_cache``; ``block_lse`` ([B, Hq, topk] fp32, optional) receives the
    per-slot block LSEs."""
    return _decode(True, q, k_cache, v_cache, block_idx, cache_offsets, ctx_lens, max_ctx, block_size, topk,
                   softmax_scale, num_splits, out, lse, return_lse, workspace, stream, block_lse)


def msa_sparse_attn_backward_workspace_size(batch, max_q_len, max_kv_len, num_heads, num_kv_heads, head_dim,
                                            topk) -> int:
    return lib().msa_sparse_attn_backward_workspace_size(batch, max_q_len, max_kv_len, num_heads, num_kv_heads,
                                                         head_dim, topk)


@_on_launch_stream
def msa_sparse_attn_backward(q, k, v, out, dout, lse, block_idx, cu_seqlens_q, cu_seqlens_k, max_q_len: int,
                             max_kv_len: int, block_size: int = 128, topk: int = 16, softmax_scale: float = 0.0,
                             dq=None, dk=None, dv=None, workspace=None, stream=None):
    """``(dq [Tq, Hq, D], dk [Tk, Hkv, D], dv [Tk, Hkv, D])`` fp32 gradients of
    msa_sparse_attn_prefill, given its inputs, its ``out`` and ``lse`` and the
    gradient ``dout`` of out (bf16)."""
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    batch = cu_seqlens_q.numel() - 1
    if dq is None:
        dq = torch.empty((tq, hq, d), dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty((tk, hkv, d), dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty((tk, hkv, d), dtype=torch.float32, device=q.device)
    need = msa_sparse_attn_backward_workspace_size(batch, max_q_len, max_kv_len, hq, hkv, d, topk)
    ws, ws_bytes = _workspace(need, q.device, workspace)
    st = lib().msa_sparse_attn_backward(
        _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(out, "out", q.dtype),
        _dev(dout, "dout", q.dtype), _dev(lse, "lse", torch.float32), _dtype_code(q),
        _dev(block_idx, "block_idx", torch.int32), _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32), batch, max_q_len, max_kv_len, hq, hkv, d, block_size,
        topk, float(softmax_scale), _dev(dq, "dq", torch.float32), _dev(dk, "dk", torch.float32),
        _dev(dv, "dv", torch.float32), ws.data_ptr() if ws is not None else None, ws_bytes, _stream(stream))
    _check(st, "msa_sparse_attn_backward")
    return dq, dk, dv


def msa_index_kl_workspace_size(batch, max_q_len, max_kv_len, num_groups, topk) -> int:
    return lib().msa_index_kl_workspace_size(batch, max_q_len, max_kv_len, num_groups, topk)


@_on_launch_stream
def msa_index_kl_backward(q_idx, k_idx, block_idx, lse, block_lse, cu_seqlens_q, cu_seqlens_k, max_q_len: int,
                          max_kv_len: int, block_size: int = 128, topk: int = 16, loss=None, dq_idx=None,
                          dk_idx=None, workspace=None, stream=None):
    """``(loss [Tq, G], dq_idx [Tq, G, d_idx], dk_idx [Tk, d_idx])`` fp32: the
    index branch's KL alignment loss against the main branch's block shares
    (``lse`` / ``block_lse`` from msa_sparse_attn_prefill_ex) and its
    gradients."""
    tq, G, di = q_idx.shape
    tk = k_idx.shape[0]
    hq = lse.shape[1]
    batch = cu_seqlens_q.numel() - 1
    if loss is None:
        loss = torch.empty((tq, G), dtype=torch.float32, device=q_idx.device)
    if dq_idx is None:
        dq_idx = torch.empty((tq, G, di), dtype=torch.float32, device=q_idx.device)
    if dk_idx is None:
        dk_idx = torch.empty((tk, di), dtype=torch.float32, device=q_idx.device)
    need = msa_index_kl_workspace_size(batch, max_q_len, max_kv_len, G, topk)
    ws, ws_bytes = _workspace(need, q_idx.device, workspace)
    st = lib().msa_index_kl_backward(
        _dev(q_idx, "q_idx"), _dev(k_idx, "k_idx", q_idx.dtype), _dtype_code(q_idx),
        _dev(block_idx, "block_idx", torch.int32), _dev(lse, "lse", torch.float32),
        _dev(block_lse, "block_lse", torch.float32), _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32), batch, max_q_len, max_kv_len, hq, G, di, block_size, topk,
        _dev(loss, "loss", torch.float32), _dev(dq_idx, "dq_idx", torch.float32), _dev(dk_idx, "dk_idx", torch.float32),
        ws.data_ptr() if ws is not None else None, ws_bytes, _stream(stream))
    _check(st, "msa_index_kl_backward")
    return loss, dq_idx, dk_idx


@_on_launch_stream
def msa_index_frontend(x, w_q, w_k, q_norm_weight, k_norm_weight, cu_seqlens_q, cu_seqlens_k, num_groups: int,
                       rope_dim: int = 64, rope_theta: float = 10000.0, norm_eps: float = 1e-6, out_dtype=None,
                       q_idx=None, k_idx=None, num_keys=None, stream=None):
    """Index front-end: ``x [T, d_model]`` through the projections ``w_q
    [G*d_idx, d_model]`` / ``w_k [d_idx, d_model]``, the RMS norm (fp32 gains
    ``[d_idx]``) and RoPE on the first ``rope_dim`` dims.  Returns ``(q_idx
    [T, G, d_idx], k_idx)``; the new tokens' key rows are written into
    ``k_idx`` at ``cu_seqlens_k[b] + position`` (pass the index-key cache to
    append to it; otherwise a zero tensor of ``num_keys`` rows is made, by
    default ``cu_seqlens_k[-1]``, read from the device)."""
    t, d_model = x.shape
    di = w_k.shape[0]
    G = int(num_groups)
    batch = cu_seqlens_q.numel() - 1
    odt = x.dtype if out_dtype is None else out_dtype
    if q_idx is None:
        q_idx = torch.empty((t, G, di), dtype=odt, device=x.device)
    if k_idx is None:
        rows = int(cu_seqlens_k[-1].item()) if num_keys is None else int(num_keys)
        k_idx = torch.zeros((rows, di), dtype=odt, device=x.device)
    if q_idx.dtype != k_idx.dtype:
        raise TypeError("q_idx and k_idx must share a dtype")
    st = lib().msa_index_frontend(
        _dev(x, "x"), _dev(w_q, "w_q", x.dtype), _dev(w_k, "w_k", x.dtype), _dtype_code(x),
        _dev(q_norm_weight, "q_norm_weight", torch.float32), _dev(k_norm_weight, "k_norm_weight", torch.float32),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32), batch, t,
        d_model, G, di, int(rope_dim), float(rope_theta), float(norm_eps), _dev(q_idx, "q_idx"), _dev(k_idx, "k_idx"),
        _dtype_code(q_idx), _stream(stream))
    _check(st, "msa_index_frontend")
    return q_idx, k_idx


def msa_index_frontend_backward_workspace_size(total_q, d_model, num_groups, index_dim) -> int:
    return int(lib().msa_index_frontend_backward_workspace_size(int(total_q), d_model, num_groups, index_dim))


@_on_launch_stream
def msa_index_frontend_backward(x, w_q, w_k, q_norm_weight, k_norm_weight, cu_seqlens_q, cu_seqlens_k,
                                num_groups: int, dq_idx, dk_idx, rope_dim: int = 64, rope_theta: float = 10000.0,
                                norm_eps: float = 1e-6, dw_q=None, dw_k=None, dq_norm_weight=None,
                                dk_norm_weight=None, workspace=None, stream=None):
    """Gradients of the index front-end's parameters for upstream gradients
    ``dq_idx [T, G, d_idx]`` and ``dk_idx`` (index-key rows, read at
    ``cu_seqlens_k[b] + position``), x held constant: ``(dw_q, dw_k,
    dq_norm_weight, dk_norm_weight)``, fp32."""
    t, d_model = x.shape
    di = w_k.shape[0]
    G = int(num_groups)
    batch = cu_seqlens_q.numel() - 1
    dev = x.device
    if dw_q is None:
        dw_q = torch.empty((G * di, d_model), dtype=torch.float32, device=dev)
    if dw_k is None:
        dw_k = torch.empty((di, d_model), dtype=torch.float32, device=dev)
    if dq_norm_weight is None:
        dq_norm_weight = torch.empty((di,), dtype=torch.float32, device=dev)
    if dk_norm_weight is None:
        dk_norm_weight = torch.empty((di,), dtype=torch.float32, device=dev)
    need = msa_index_frontend_backward_workspace_size(t, d_model, G, di)
    ws, ws_bytes = _workspace(need, dev, workspace)
    st = lib().msa_index_frontend_backward(
        _dev(x, "x"), _dev(w_q, "w_q", x.dtype), _dev(w_k, "w_k", x.dtype), _dtype_code(x),
        _dev(q_norm_weight, "q_norm_weight", torch.float32), _dev(k_norm_weight, "k_norm_weight", torch.float32),
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32), batch, t,
        d_model, G, di, int(rope_dim), float(rope_theta), float(norm_eps),
        _dev(dq_idx, "dq_idx", torch.float32), _dev(dk_idx, "dk_idx", torch.float32),
        _dev(dw_q, "dw_q", torch.float32), _dev(dw_k, "dw_k", torch.float32),
        _dev(dq_norm_weight, "dq_norm_weight", torch.float32), _dev(dk_norm_weight, "dk_norm_weight", torch.float32),
        ws.data_ptr() if ws is not None else None, ws_bytes, _stream(stream))
    _check(st, "msa_index_frontend_backward")
    return dw_q, dw_k, dq_norm_weight, dk_norm_weight
