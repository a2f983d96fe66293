"""Algorithmic work of the MSA hot path: the units the roofline is priced in.

FLOPs count 2 per multiply-add and exclude softmax/exp, masked lanes and MFMA
padding.  Bytes count each input element once per reader that needs it, with
no re-reads.

* index score + block max-pool: every key of every earlier block is scored
  against one index query per group: 2 * d_idx * G * Bk * l(p) FLOPs per query
  (the forced local block is never scored, so it costs nothing).
* sparse attention: QK^T and PV over the attended keys J:
  4 * D * Hq * |J| FLOPs per query, with
  |J| = min(k - 1, l) * Bk + (p - l * Bk + 1)   (earlier blocks are full,
  the local block is causal).
* decode bytes: the whole index-key cache is read once for all groups
  (ctx * d_idx * elem), each selected K and V block once per (sequence, group),
  plus q, q_idx and the output.

The per-token FLOP ratio against dense GQA at average causal context L/2
reproduces the pages' 28.4x at 1M tokens ("MiniMax Sparse Attention: let each
query pick its own blocks", paper Figure 4 caption), pinned by a golden test.
"""
from __future__ import annotations

import numpy as np


def attended_keys(pos, block_size: int, topk: int):
    """|J| per query position (any selection that keeps min(k-1, l) earlier blocks)."""
    pos = np.asarray(pos, dtype=np.int64)
    local = pos // block_size
    earlier = np.minimum(topk - 1, local)
    return earlier * block_size + (pos - local * block_size + 1)


def prefill_positions(q_len: int, kv_len: int):
    return np.arange(kv_len - q_len, kv_len, dtype=np.int64)


def index_flops(pos, num_groups: int, index_dim: int, block_size: int) -> float:
    pos = np.asarray(pos, dtype=np.int64)
    scored = (pos // block_size) * block_size
    return float(2.0 * index_dim * num_groups * scored.sum(dtype=np.float64))


def attn_flops(pos, num_heads: int, head_dim: int, block_size: int, topk: int) -> float:
    return float(4.0 * head_dim * num_heads
                 * attended_keys(pos, block_size, topk).sum(dtype=np.float64))


def prefill_flops(q_len, kv_len, num_heads, num_kv_heads, head_dim, index_dim, block_size, topk):
    """(index FLOPs, attention FLOPs) for one sequence's query rows."""
    pos = prefill_positions(q_len, kv_len)
    return (index_flops(pos, num_kv_heads, index_dim, block_size),
            attn_flops(pos, num_heads, head_dim, block_size, topk))


def decode_bytes(ctx_lens, num_heads, num_kv_heads, head_dim, index_dim, block_size, topk,
                 elem_bytes: int = 2, kv_elem_bytes: int | None = None, qo_elem_bytes: int | None = None):
    """(index-scan bytes, attention bytes) for one decode step.  ``elem_bytes``
    is the size of an index-tensor element; K/V and q/out elements default to
    the same size."""
    kv_eb = elem_bytes if kv_elem_bytes is None else kv_elem_bytes
    qo_eb = elem_bytes if qo_elem_bytes is None else qo_elem_bytes
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    pos = ctx - 1
    idx_bytes = float((ctx * index_dim * elem_bytes).sum()
                      + len(ctx) * num_kv_heads * index_dim * elem_bytes)
    J = attended_keys(pos, block_size, topk)
    kv_bytes = float((J * num_kv_heads * head_dim * kv_eb * 2).sum())
    qo_bytes = float(len(ctx) * num_heads * head_dim * qo_eb * 2)
    return idx_bytes, kv_bytes + qo_bytes


def per_token_flop_ratio(context: int, num_heads: int, num_kv_heads: int, head_dim: int,
                         index_dim: int, block_size: int, topk: int) -> float:
    """Dense GQA / MSA attention FLOPs per token at average causal context L/2."""
    avg = context / 2.0
    dense = num_heads * 4.0 * head_dim * avg
    msa = num_heads * 4.0 * head_dim * topk * block_size + num_kv_heads * 2.0 * index_dim * avg
    return dense / msa
