"""Plain CPU oracle for MiniMax Sparse Attention (MSA).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the GPU
library (``learned_block_sparse_amd``) and never imports it; the C source
``msa_oracle.c`` holds the arithmetic, this module only marshals arguments.

What it computes follows "MiniMax Sparse Attention: let each query pick its own
blocks" (ai.thesatyajit.com), section "The mechanism, precisely", and the atlas
record of MiniMax M3 (atlas.lewiswon.me), summary paragraph:

* ``index_topk``: per query row and GQA group, raw index scores against every
  key of each earlier block, max-pooled per block, the best ``topk - 1`` earlier
  blocks (score descending, block id ascending) plus the query's local block,
  returned ascending and padded with -1.  Index scores are accumulated in fp32
  (the GPU path's precision, so both sides take the selection decision in the
  same precision).
* ``sparse_attn``: exact softmax attention in fp64 over the keys of the
  selected blocks, causal inside the local block, natural-log LSE.
* ``sparse_attn_bwd``: its gradients with respect to q, k and v (fp64),
  recomputed from the inputs.
* ``block_lse``: the main branch's LSE over each selected block's attended
  keys, per (row, head, selection slot).
* ``index_frontend``: the index branch's front end, hidden states through a
  linear projection, a norm and RoPE to the index-query heads and the shared
  index-key head (Figure 1 of the first page; the norm's kind and the rotary
  base are readings, written out in ``msa_oracle.c``); ``index_frontend_bwd``:
  its gradients with respect to the projections and the norm gains.
* ``index_kl``: the KL alignment loss of the index branch (the index scores of
  the selected blocks against the group-averaged share of main attention in
  each block) and its gradients with respect to q_idx and k_idx.

Query row t of a sequence with ``q_len = M`` and ``kv_len = N`` sits at
absolute position ``p = N - M + t``; blocks are aligned to position 0.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_SO = os.path.join(_HERE, "libmsa_oracle.so")

# Portable flags: the library may run on another host than the one it was
# built on.  No contraction of a*b+c into fma and no fast-math, so each line of
# the C source is the arithmetic that runs.
CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile ``msa_oracle.c`` into ``libmsa_oracle.so`` with gcc."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        cmd = ["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=True)
        lib = ctypes.CDLL(_SO)
        vp, i64p, i32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        lib.oracle_index_topk.restype = ctypes.c_int
        lib.oracle_index_topk.argtypes = [vp, vp, ctypes.c_int, i64p, i64p, ctypes.c_int64,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          i32p, vp, ctypes.c_int64]
        lib.oracle_decode_e4m3.restype = None
        lib.oracle_decode_e4m3.argtypes = [vp, vp, ctypes.c_int64]
        lib.oracle_sparse_attn.restype = ctypes.c_int
        lib.oracle_sparse_attn.argtypes = [vp, vp, vp, ctypes.c_int, i64p, i64p, i32p,
                                           ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_double, vp, vp]
        lib.oracle_sparse_attn_kv.restype = ctypes.c_int
        lib.oracle_sparse_attn_kv.argtypes = [vp, vp, vp, ctypes.c_int, ctypes.c_int, i64p, i64p, i32p,
                                              ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_double, vp, vp]
        lib.oracle_sparse_attn_bwd.restype = ctypes.c_int
        lib.oracle_sparse_attn_bwd.argtypes = [vp, vp, vp, vp, ctypes.c_int, i64p, i64p, i32p,
                                               ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_double, vp, vp, vp]
        lib.oracle_block_lse.restype = ctypes.c_int
        lib.oracle_block_lse.argtypes = [vp, vp, ctypes.c_int, i64p, i64p, i32p, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                         vp]
        lib.oracle_index_kl.restype = ctypes.c_int
        lib.oracle_index_kl.argtypes = [vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, i64p, i64p, i32p,
                                        ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_double, vp, vp, vp]
        lib.oracle_index_frontend.restype = ctypes.c_int
        lib.oracle_index_frontend.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, i64p, ctypes.c_int64, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                              ctypes.c_double, vp, vp]
        lib.oracle_index_frontend_bwd.restype = ctypes.c_int
        lib.oracle_index_frontend_bwd.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, i64p, ctypes.c_int64,
                                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                  ctypes.c_double, ctypes.c_double, vp, vp, vp, vp, vp, vp]
        _lib = lib
    return _lib


def _host_array(x):
    """Return (contiguous numpy array, dtype code): 0 = fp32, 1 = bf16 bits,
    2 = E4M3 bits."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                x = x.cpu()
            if x.dtype == torch.bfloat16:
                return np.ascontiguousarray(x.contiguous().view(torch.int16).numpy().view(np.uint16)), 1
            if x.dtype == torch.float32:
                return np.ascontiguousarray(x.contiguous().numpy()), 0
            if x.dtype == torch.float8_e4m3fn:
                return np.ascontiguousarray(x.contiguous().view(torch.uint8).numpy()), 2
            raise TypeError(f"oracle input dtype {x.dtype} not supported")
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    x = np.asarray(x)
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), 0
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 1
    if x.dtype == np.uint8:
        return np.ascontiguousarray(x), 2
    raise TypeError(f"oracle input dtype {x.dtype} not supported")


def decode_e4m3(bits) -> np.ndarray:
    """fp32 values of E4M3 bit patterns (uint8), as the oracle reads them."""
    lib = _load()
    a = np.ascontiguousarray(np.asarray(bits, dtype=np.uint8))
    out = np.empty(a.shape, dtype=np.float32)
    lib.oracle_decode_e4m3(_ptr(a), _ptr(out), a.size)
    return out


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def rows_prefill(cu_seqlens_q, cu_seqlens_k, rows=None):
    """Per requested packed query row: (rows, key start row, absolute position)."""
    cu_q = np.asarray(cu_seqlens_q, dtype=np.int64)
    cu_k = np.asarray(cu_seqlens_k, dtype=np.int64)
    if rows is None:
        rows = np.arange(cu_q[-1], dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    b = np.searchsorted(cu_q, rows, side="right") - 1
    m = cu_q[b + 1] - cu_q[b]
    n = cu_k[b + 1] - cu_k[b]
    pos = n - m + (rows - cu_q[b])
    return rows, np.ascontiguousarray(cu_k[b]), np.ascontiguousarray(pos)


def rows_decode(k_offsets, ctx_lens):
    """Decode: one query per sequence, the newest token at position ctx - 1."""
    off = np.asarray(k_offsets, dtype=np.int64)
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    return np.arange(len(off), dtype=np.int64), np.ascontiguousarray(off), np.ascontiguousarray(ctx - 1)


def _gather_rows(x, rows):
    """Rows of a [T, ...] tensor/array, as a compact host array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            idx = torch.as_tensor(rows, dtype=torch.long, device=x.device)
            return _host_array(x.index_select(0, idx))
    except ImportError:  # pragma: no cover
        pass
    return _host_array(np.asarray(x)[np.asarray(rows)])


def index_topk(q_idx, k_idx, kstart, pos, rows, block_size: int, topk: int,
               return_scores: bool = False):
    """Selected blocks [n, G, topk] (int32) for the given query rows.

    ``q_idx`` is the full [T, G, d_idx] array; ``rows`` index into it.  With
    ``return_scores`` also returns the pooled block scores [n, G, nbmax] (fp32,
    -inf beyond each row's earlier blocks).
    """
    lib = _load()
    qa, qt = _gather_rows(q_idx, rows)
    ka, kt = _host_array(k_idx)
    if qt != kt:
        raise TypeError("q_idx and k_idx must share a dtype")
    n, G, DI = qa.shape
    kstart = np.ascontiguousarray(kstart, dtype=np.int64)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    sel = np.empty((n, G, topk), dtype=np.int32)
    scores = None
    nbmax = 0
    if return_scores:
        nbmax = max(1, int(pos.max()) // block_size if n else 1)
        scores = np.empty((n, G, nbmax), dtype=np.float32)
    rc = lib.oracle_index_topk(_ptr(qa), _ptr(ka), qt, _ptr(kstart), _ptr(pos), n, G, DI,
                               block_size, topk, _ptr(sel),
                               _ptr(scores) if scores is not None else None, nbmax)
    if rc != 0:
        raise ValueError(f"oracle_index_topk failed ({rc})")
    return (sel, scores) if return_scores else sel


def sparse_attn(q, k, v, sel, kstart, pos, rows, block_size: int, topk: int, scale=None):
    """(out [n, Hq, D] fp64, lse [n, Hq] fp64) for the given query rows."""
    lib = _load()
    qa, qt = _gather_rows(q, rows)
    ka, kt = _host_array(k)
    va, vt = _host_array(v)
    if kt != vt:
        raise TypeError("k and v must share a dtype")
    n, Hq, D = qa.shape
    Hkv = ka.shape[1]
    sel = np.ascontiguousarray(np.asarray(sel), dtype=np.int32)
    if sel.shape != (n, Hkv, topk):
        raise ValueError(f"sel shape {sel.shape} != {(n, Hkv, topk)}")
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    kstart = np.ascontiguousarray(kstart, dtype=np.int64)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    out = np.empty((n, Hq, D), dtype=np.float64)
    lse = np.empty((n, Hq), dtype=np.float64)
    rc = lib.oracle_sparse_attn_kv(_ptr(qa), _ptr(ka), _ptr(va), qt, kt, _ptr(kstart), _ptr(pos),
                                   _ptr(sel), n, Hq, Hkv, D, block_size, topk, float(scale),
                                   _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"oracle_sparse_attn failed ({rc})")
    return out, lse


def sparse_attn_bwd(q, k, v, dout, sel, kstart, pos, rows, block_size: int, topk: int, scale=None):
    """Gradients of ``sparse_attn`` for the given query rows:
    (dq [n, Hq, D], dk [Tk, Hkv, D], dv [Tk, Hkv, D]), all fp64.  dk and dv
    hold the contributions of these rows only."""
    lib = _load()
    qa, qt = _gather_rows(q, rows)
    da, dt = _gather_rows(dout, rows)
    ka, kt = _host_array(k)
    va, vt = _host_array(v)
    if not (qt == kt == vt == dt) or qt not in (0, 1):
        raise TypeError("q, k, v and dout must share a dtype (fp32 or bf16)")
    n, Hq, D = qa.shape
    Hkv = ka.shape[1]
    sel = np.ascontiguousarray(np.asarray(sel), dtype=np.int32)
    if sel.shape != (n, Hkv, topk):
        raise ValueError(f"sel shape {sel.shape} != {(n, Hkv, topk)}")
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    kstart = np.ascontiguousarray(kstart, dtype=np.int64)
    pos = np.ascontiguousarray(pos, dtype=np.int64)
    dq = np.empty((n, Hq, D), dtype=np.float64)
    dk = np.zeros(ka.shape, dtype=np.float64)
    dv = np.zeros(va.shape, dtype=np.float64)
    rc = lib.oracle_sparse_attn_bwd(_ptr(qa), _ptr(ka), _ptr(va), _ptr(da), qt, _ptr(kstart), _ptr(pos),
                                    _ptr(sel), n, Hq, Hkv, D, block_size, topk, float(scale),
                                    _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError(f"oracle_sparse_attn_bwd failed ({rc})")
    return dq, dk, dv


def block_lse(q, k, sel, kstart, pos, rows, block_size: int, topk: int, scale=None):
    """Per-slot block LSEs [n, Hq, topk] (fp64) of the main branch."""
    lib = _load()
    qa, qt = _gather_rows(q, rows)
    ka, kt = _host_array(k)
    if qt != kt:
        raise TypeError("q and k must share a dtype")
    n, Hq, D = qa.shape
    Hkv = ka.shape[1]
    sel = np.ascontiguousarray(np.asarray(sel), dtype=np.int32)
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    out = np.empty((n, Hq, topk), dtype=np.float64)
    rc = lib.oracle_block_lse(_ptr(qa), _ptr(ka), qt, _ptr(np.ascontiguousarray(kstart, dtype=np.int64)),
                              _ptr(np.ascontiguousarray(pos, dtype=np.int64)), _ptr(sel), n, Hq, Hkv, D,
                              block_size, topk, float(scale), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_block_lse failed ({rc})")
    return out


def index_kl(q_idx, k_idx, q, k, sel, kstart, pos, rows, block_size: int, topk: int, scale=None):
    """KL alignment loss of the index branch: (loss [n, G], dq_idx [n, G, d_idx],
    dk_idx [Tk, d_idx]), fp64; dk_idx holds these rows' contributions."""
    lib = _load()
    qia, qit = _gather_rows(q_idx, rows)
    kia, kit = _host_array(k_idx)
    qa, qt = _gather_rows(q, rows)
    ka, kt = _host_array(k)
    if qit != kit or qt != kt:
        raise TypeError("q_idx / k_idx and q / k must share a dtype pairwise")
    n, G, DI = qia.shape
    Hq, D = qa.shape[1], qa.shape[2]
    sel = np.ascontiguousarray(np.asarray(sel), dtype=np.int32)
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(D)
    loss = np.empty((n, G), dtype=np.float64)
    dq = np.empty((n, G, DI), dtype=np.float64)
    dk = np.zeros(kia.shape, dtype=np.float64)
    rc = lib.oracle_index_kl(_ptr(qia), _ptr(kia), qit, _ptr(qa), _ptr(ka), qt,
                             _ptr(np.ascontiguousarray(kstart, dtype=np.int64)),
                             _ptr(np.ascontiguousarray(pos, dtype=np.int64)), _ptr(sel), n, G, DI, Hq, D,
                             block_size, topk, float(scale), _ptr(loss), _ptr(dq), _ptr(dk))
    if rc != 0:
        raise ValueError(f"oracle_index_kl failed ({rc})")
    return loss, dq, dk


def index_frontend(x, w_q, w_k, gain_q, gain_k, pos, num_groups: int, d_idx: int, rope_dim: int,
                   theta: float, eps: float):
    """Index front-end of n tokens at absolute positions ``pos``:
    (q_idx [n, G, d_idx], k_idx [n, d_idx]), fp64."""
    lib = _load()
    xa, xt = _host_array(x)
    wqa, wqt = _host_array(w_q)
    wka, wkt = _host_array(w_k)
    if not (xt == wqt == wkt) or xt == 2:
        raise TypeError("x, w_q and w_k must share a dtype (fp32 or bf16)")
    n, d_model = xa.shape
    G, DI = int(num_groups), int(d_idx)
    if wqa.shape != (G * DI, d_model) or wka.shape != (DI, d_model):
        raise ValueError("projection shapes do not match")
    gq = np.ascontiguousarray(np.asarray(gain_q, dtype=np.float64).reshape(DI))
    gk = np.ascontiguousarray(np.asarray(gain_k, dtype=np.float64).reshape(DI))
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64).reshape(n))
    q = np.empty((n, G, DI), dtype=np.float64)
    k = np.empty((n, DI), dtype=np.float64)
    rc = lib.oracle_index_frontend(_ptr(xa), _ptr(wqa), _ptr(wka), xt, _ptr(gq), _ptr(gk), _ptr(pos), n, d_model,
                                   G, DI, int(rope_dim), float(theta), float(eps), _ptr(q), _ptr(k))
    if rc != 0:
        raise ValueError(f"oracle_index_frontend failed ({rc})")
    return q, k


def index_frontend_bwd(x, w_q, w_k, gain_q, gain_k, pos, num_groups: int, d_idx: int, rope_dim: int,
                       theta: float, eps: float, dq, dk):
    """Parameter gradients of the index front-end for upstream gradients
    ``dq [n, G, d_idx]`` and ``dk [n, d_idx]`` (one key row per token): (dw_q,
    dw_k, dgain_q, dgain_k), fp64; x is held constant."""
    lib = _load()
    xa, xt = _host_array(x)
    wqa, wqt = _host_array(w_q)
    wka, wkt = _host_array(w_k)
    if not (xt == wqt == wkt) or xt == 2:
        raise TypeError("x, w_q and w_k must share a dtype (fp32 or bf16)")
    n, d_model = xa.shape
    G, DI = int(num_groups), int(d_idx)
    if wqa.shape != (G * DI, d_model) or wka.shape != (DI, d_model):
        raise ValueError("projection shapes do not match")
    gq = np.ascontiguousarray(np.asarray(gain_q, dtype=np.float64).reshape(DI))
    gk = np.ascontiguousarray(np.asarray(gain_k, dtype=np.float64).reshape(DI))
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int64).reshape(n))
    dqa = np.ascontiguousarray(np.asarray(dq, dtype=np.float64).reshape(n, G, DI))
    dka = np.ascontiguousarray(np.asarray(dk, dtype=np.float64).reshape(n, DI))
    dwq = np.empty((G * DI, d_model), dtype=np.float64)
    dwk = np.empty((DI, d_model), dtype=np.float64)
    dgq = np.empty(DI, dtype=np.float64)
    dgk = np.empty(DI, dtype=np.float64)
    rc = lib.oracle_index_frontend_bwd(_ptr(xa), _ptr(wqa), _ptr(wka), xt, _ptr(gq), _ptr(gk), _ptr(pos), n,
                                       d_model, G, DI, int(rope_dim), float(theta), float(eps), _ptr(dqa), _ptr(dka),
                                       _ptr(dwq), _ptr(dwk), _ptr(dgq), _ptr(dgk))
    if rc != 0:
        raise ValueError(f"oracle_index_frontend_bwd failed ({rc})")
    return dwq, dwk, dgq, dgk


def prefill(q_idx, k_idx, q, k, v, cu_seqlens_q, cu_seqlens_k, block_size: int, topk: int,
            scale=None, rows=None):
    """Index selection then attention for packed prefill rows: (sel, out, lse)."""
    rows, kstart, pos = rows_prefill(cu_seqlens_q, cu_seqlens_k, rows)
    sel = index_topk(q_idx, k_idx, kstart, pos, rows, block_size, topk)
    out, lse = sparse_attn(q, k, v, sel, kstart, pos, rows, block_size, topk, scale)
    return sel, out, lse


def decode(q_idx, k_idx_cache, q, k_cache, v_cache, k_offsets, ctx_lens, block_size: int,
           topk: int, scale=None, rows=None):
    """One decode step per sequence: (sel, out, lse) for the given sequences."""
    all_rows, kstart, pos = rows_decode(k_offsets, ctx_lens)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        kstart, pos = kstart[rows], pos[rows]
    else:
        rows = all_rows
    sel = index_topk(q_idx, k_idx_cache, kstart, pos, rows, block_size, topk)
    out, lse = sparse_attn(q, k_cache, v_cache, sel, kstart, pos, rows, block_size, topk, scale)
    return sel, out, lse
