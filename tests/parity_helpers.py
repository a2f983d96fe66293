"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding and the CPU oracle on the same seeded inputs, and compare.

Tolerances (stated for the workloads: max-abs 1e-4 for fp32; max-abs 2e-2 and
relative RMS 1e-2 for bf16).  LSE is computed in fp32 from exact inputs by
both the kernel and (in fp64) the oracle; its error is a few fp32 ulps of the
logits, so 1e-4 (fp32) and 1e-3 (bf16) absolute leave ample margin.
Block ids must match exactly: the index inputs are on the 1/8 grid, so every
score is exact on both sides.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

TOL = {"f32": dict(max_abs=1e-4, rel_rms=None, lse=1e-4),
       "bf16": dict(max_abs=2e-2, rel_rms=1e-2, lse=1e-3)}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def compare_outputs(gpu_out, gpu_lse, ref_out, ref_lse, dtype: str, what: str):
    tol = TOL[dtype]
    g = gpu_out.detach().float().cpu().double().numpy()
    err = np.abs(g - ref_out)
    max_abs = float(err.max()) if err.size else 0.0
    assert max_abs <= tol["max_abs"], f"{what}: max-abs {max_abs:.3g} > {tol['max_abs']}"
    if tol["rel_rms"] is not None and err.size:
        rel = float(np.sqrt((err ** 2).sum() / max((ref_out ** 2).sum(), 1e-300)))
        assert rel <= tol["rel_rms"], f"{what}: rel-RMS {rel:.3g} > {tol['rel_rms']}"
    if gpu_lse is not None:
        gl = gpu_lse.detach().cpu().double().numpy()
        both_inf = np.isneginf(gl) & np.isneginf(ref_lse)
        assert np.array_equal(np.isneginf(gl), np.isneginf(ref_lse)), f"{what}: -inf lse pattern differs"
        d = np.abs(np.where(both_inf, 0.0, gl - np.where(both_inf, 0.0, ref_lse)))
        assert float(d.max()) <= tol["lse"], f"{what}: lse err {float(d.max()):.3g}"
    return max_abs


def compare_ids(gpu_ids, ref_ids, what: str):
    g = gpu_ids.detach().cpu().numpy()
    if not np.array_equal(g, ref_ids):
        bad = np.argwhere((g != ref_ids).any(axis=-1))
        r = tuple(bad[0])
        raise AssertionError(f"{what}: block ids differ in {len(bad)} (row, group) pairs; "
                             f"first {r}: gpu {g[r].tolist()} oracle {ref_ids[r].tolist()}")


def gpu_prefill(msa, inp, wl, q_lo=0, q_hi=None, num_splits=0):
    """Run one prefill call for query rows [q_lo, q_hi) of a batch-1 input
    against the causal key prefix ending at q_hi (a chunk of a long prefill).
    Returns (block_idx, out, lse) for those rows."""
    L = inp["cu_k_host"][-1]
    if q_hi is None:
        q_hi = L
    dev = inp["q"].device
    cu_q = torch.tensor([0, q_hi - q_lo], dtype=torch.int32, device=dev)
    cu_k = torch.tensor([0, q_hi], dtype=torch.int32, device=dev)
    ids = msa.msa_index_topk(inp["q_idx"][q_lo:q_hi], inp["k_idx"], cu_q, cu_k, q_hi - q_lo, q_hi,
                             wl.block_size, wl.topk)
    out, lse = msa.msa_sparse_attn_prefill(inp["q"][q_lo:q_hi], inp["k"], inp["v"], ids, cu_q, cu_k,
                                           q_hi - q_lo, q_hi, wl.block_size, wl.topk,
                                           num_splits=num_splits)
    return ids, out, lse


def oracle_prefill_rows(oracle, inp, wl, rows, q_lo=0, q_hi=None):
    """Oracle for absolute positions ``rows`` of a batch-1 input, seen as query
    rows of the call [q_lo, q_hi)."""
    L = inp["cu_k_host"][-1]
    if q_hi is None:
        q_hi = L
    rows = np.asarray(rows, dtype=np.int64)
    kstart = np.zeros(len(rows), dtype=np.int64)
    pos = rows.copy()
    ids = oracle.index_topk(inp["q_idx"], inp["k_idx"], kstart, pos, rows, wl.block_size, wl.topk)
    out, lse = oracle.sparse_attn(inp["q"], inp["k"], inp["v"], ids, kstart, pos, rows, wl.block_size,
                                  wl.topk)
    return ids, out, lse


def host(t):
    return t.detach().cpu() if isinstance(t, torch.Tensor) else t


def sample_rows(lo, hi, block, rng, n_blocks=3, extra=24):
    """Rows of [lo, hi): the first and last block, a few random blocks in full,
    and random single rows."""
    rows = set(range(lo, min(lo + block, hi)))
    rows |= set(range(max(lo, hi - block), hi))
    nb = max(1, (hi - lo) // block)
    for b in rng.choice(nb, size=min(n_blocks, nb), replace=False):
        s = lo + int(b) * block
        rows |= set(range(s, min(s + block, hi)))
    rows |= set(int(x) for x in rng.integers(lo, hi, size=extra))
    return np.array(sorted(rows), dtype=np.int64)


def rel_rms(a, b):
    return math.sqrt(float(((a - b) ** 2).sum()) / max(float((b ** 2).sum()), 1e-300))
