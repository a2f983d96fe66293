"""Seeded synthetic inputs for MiniMax Sparse Attention workloads.

This module only draws random tensors; it holds none of the method's
arithmetic.  The GPU path and the CPU oracle both consume what it returns, and
the oracle gets host copies of exactly the same bits.

Recipe (shapes and distributions of the workloads measured on "MiniMax Sparse
Attention: let each query pick its own blocks", paper Figure 4 caption: 64
query / 4 KV heads, head dim 128, block 128, k = 16, contexts from 32K to 1M):

* Q, K, V ~ N(0, 1), drawn in fp32 and rounded to bf16 (round-to-nearest-even)
  for bf16 workloads.
* Index queries / keys are multiples of 1/8, uniform over the integers u in
  [-16, 16] (values u / 8 in [-2, 2]).  Every such value is exact in bf16, and
  every index score is a multiple of 1/64 below 2**16 / 64 in magnitude, so the
  scores are exact in fp32 in any summation order.
* Planted blocks: P distinct key blocks (uniform over all blocks) get +1.0 on
  every index-key element of each of their tokens; values stay multiples of
  1/8, so exactness is kept.  This makes a few blocks "hot", as the pages note
  real selections have (a first-token sink emerges).
* Index front-end (hidden states -> index heads): d_model = 3072 (the
  testbed's stated width, atlas record of MiniMax M3); hidden states
  ~ N(0, 1); projection weights ~ N(0, 1/d_model) (so projected values are
  about N(0, 1)); norm gains uniform on [0.5, 1.5] in fp32.  Synthetic
  weights: the pages publish none.
* Decode: one new token per sequence, context lengths uniform on
  [65536, 1048576]; the caches are packed one sequence after another.

Each tensor draws from its own generator seeded with (seed, tensor id), so any
tensor can be regenerated alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

BLOCK = 128


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.  Sizes follow the measured MSA configuration."""
    name: str
    dtype: str                 # "f32" or "bf16"
    num_heads: int             # Hq
    num_kv_heads: int          # Hkv = number of GQA groups G
    head_dim: int              # D
    index_dim: int             # d_idx
    block_size: int
    topk: int                  # counts the forced local block
    seq_len: int = 0           # prefill: L (q_len = kv_len = L)
    q_tile: int = 0            # prefill: queries per call, 0 = whole sequence
    planted: int = 0           # number of planted high-score blocks
    batch: int = 1
    ctx_min: int = 0           # decode: context length range
    ctx_max: int = 0
    decode: bool = False
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny_prefill_2k_f32": Workload(
        "tiny_prefill_2k_f32", "f32", 8, 2, 128, 64, 128, 4, seq_len=2048,
        notes="batch 1, L=2048, 8 Q / 2 KV heads, d_idx 64, top-k 4 incl. local, fp32"),
    "prefill_32k": Workload(
        "prefill_32k", "bf16", 64, 4, 128, 128, 128, 16, seq_len=32768, planted=32,
        notes="batch 1, L=32768, 64 Q / 4 KV heads, d_idx 128, k 16, 32 planted blocks"),
    "prefill_128k": Workload(
        "prefill_128k", "bf16", 64, 4, 128, 128, 128, 16, seq_len=131072, q_tile=8192,
        planted=32,
        notes="batch 1, L=131072 in 8192-query tiles against the causal prefix"),
    "decode_1m": Workload(
        "decode_1m", "bf16", 64, 4, 128, 128, 128, 16, batch=32, ctx_min=65536,
        ctx_max=1048576, decode=True,
        notes="32 sequences, 1 new token each, contexts uniform in [64K, 1M]"),
    "prefill_1m": Workload(
        "prefill_1m", "bf16", 64, 4, 128, 128, 128, 16, seq_len=1048576, q_tile=8192,
        planted=256,
        notes="batch 1, L=1048576 in 8192-query tiles, 256 planted blocks"),
}

_TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "q_idx": 4, "k_idx": 5, "planted": 6, "ctx": 7, "dout": 8,
               "hidden": 9, "w_q_idx": 10, "w_k_idx": 11, "gain_q_idx": 12, "gain_k_idx": 13}
_CHUNK_ELEMS = 1 << 28  # draw big tensors in pieces to bound fp32 temporaries


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _gen(device, seed: int, tensor: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + _TENSOR_IDS[tensor])
    return g


def normal(shape, dtype, device, seed: int, tensor: str) -> torch.Tensor:
    """N(0, 1) in fp32, rounded to ``dtype``; drawn in row chunks."""
    g = _gen(device, seed, tensor)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    row = max(1, flat.shape[1])
    step = max(1, _CHUNK_ELEMS // row)
    for s in range(0, shape[0], step):
        e = min(shape[0], s + step)
        flat[s:e] = torch.randn((e - s, flat.shape[1]), generator=g, device=device,
                                dtype=torch.float32).to(dtype)
    return out


def index_grid(shape, dtype, device, seed: int, tensor: str) -> torch.Tensor:
    """Uniform multiples of 1/8 in [-2, 2]."""
    g = _gen(device, seed, tensor)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    row = max(1, flat.shape[1])
    step = max(1, _CHUNK_ELEMS // row)
    for s in range(0, shape[0], step):
        e = min(shape[0], s + step)
        u = torch.randint(-16, 17, (e - s, flat.shape[1]), generator=g, device=device,
                          dtype=torch.int32)
        flat[s:e] = (u.to(torch.float32) * 0.125).to(dtype)
    return out


def plant_blocks(k_idx: torch.Tensor, seq_starts, seq_lens, count: int, seed: int,
                 block_size: int = BLOCK):
    """Add +1.0 to every index-key element of ``count`` random blocks per sequence.

    Returns the planted block ids per sequence (host lists)."""
    g = _gen("cpu", seed, "planted")
    planted = []
    for start, n in zip(seq_starts, seq_lens):
        nblocks = (int(n) + block_size - 1) // block_size
        c = min(count, nblocks)
        ids = torch.randperm(nblocks, generator=g)[:c].sort().values.tolist()
        for b in ids:
            lo = int(start) + b * block_size
            hi = min(int(start) + int(n), lo + block_size)
            k_idx[lo:hi] += 1.0
        planted.append(ids)
    return planted


def prefill_inputs(wl: Workload, device="cpu", seed: int = 0, seq_lens=None, q_lens=None,
                   with_main: bool = True):
    """Packed varlen prefill inputs.

    ``seq_lens`` are kv lengths per sequence (default ``[wl.seq_len] * batch``);
    ``q_lens`` the query lengths (default equal: full causal prefill).  The
    query rows of a sequence are its last ``q_len`` positions.
    """
    if seq_lens is None:
        seq_lens = [wl.seq_len] * wl.batch
    if q_lens is None:
        q_lens = list(seq_lens)
    dt = torch_dtype(wl.dtype)
    cu_k = [0]
    for n in seq_lens:
        cu_k.append(cu_k[-1] + int(n))
    cu_q = [0]
    for m in q_lens:
        cu_q.append(cu_q[-1] + int(m))
    tk, tq = cu_k[-1], cu_q[-1]
    G = wl.num_kv_heads
    out = {
        "cu_seqlens_q": torch.tensor(cu_q, dtype=torch.int32, device=device),
        "cu_seqlens_k": torch.tensor(cu_k, dtype=torch.int32, device=device),
        "cu_q_host": cu_q, "cu_k_host": cu_k,
        "q_idx": index_grid((tq, G, wl.index_dim), dt, device, seed, "q_idx"),
        "k_idx": index_grid((tk, wl.index_dim), dt, device, seed, "k_idx"),
    }
    out["planted"] = plant_blocks(out["k_idx"], cu_k[:-1], seq_lens, wl.planted, seed,
                                  wl.block_size) if wl.planted else []
    if with_main:
        out["q"] = normal((tq, wl.num_heads, wl.head_dim), dt, device, seed, "q")
        out["k"] = normal((tk, wl.num_kv_heads, wl.head_dim), dt, device, seed, "k")
        out["v"] = normal((tk, wl.num_kv_heads, wl.head_dim), dt, device, seed, "v")
    return out


def decode_ctx_lens(wl: Workload, seed: int = 0):
    g = _gen("cpu", seed, "ctx")
    return torch.randint(wl.ctx_min, wl.ctx_max + 1, (wl.batch,), generator=g).tolist()


def decode_inputs(wl: Workload, device="cpu", seed: int = 0, ctx_lens=None):
    """One decode step: packed caches (index-K, K, V) and one query per sequence."""
    if ctx_lens is None:
        ctx_lens = decode_ctx_lens(wl, seed)
    dt = torch_dtype(wl.dtype)
    offs = [0]
    for n in ctx_lens:
        offs.append(offs[-1] + int(n))
    tk = offs[-1]
    B = len(ctx_lens)
    G = wl.num_kv_heads
    out = {
        "ctx_lens_host": [int(x) for x in ctx_lens],
        "k_offsets_host": offs[:-1],
        "ctx_lens": torch.tensor(ctx_lens, dtype=torch.int32, device=device),
        "k_offsets": torch.tensor(offs[:-1], dtype=torch.int64, device=device),
        "cu_seqlens_q": torch.arange(B + 1, dtype=torch.int32, device=device),
        "cu_seqlens_k": torch.tensor(offs, dtype=torch.int32, device=device),
        "q_idx": index_grid((B, G, wl.index_dim), dt, device, seed, "q_idx"),
        "k_idx": index_grid((tk, wl.index_dim), dt, device, seed, "k_idx"),
        "q": normal((B, wl.num_heads, wl.head_dim), dt, device, seed, "q"),
        "k": normal((tk, wl.num_kv_heads, wl.head_dim), dt, device, seed, "k"),
        "v": normal((tk, wl.num_kv_heads, wl.head_dim), dt, device, seed, "v"),
    }
    out["planted"] = plant_blocks(out["k_idx"], offs[:-1], ctx_lens, wl.planted, seed,
                                  wl.block_size) if wl.planted else []
    return out


D_MODEL = 3072


def frontend_inputs(num_tokens: int, num_groups: int = 4, index_dim: int = 128, d_model: int = D_MODEL,
                    dtype=torch.bfloat16, device="cpu", seed: int = 0):
    """Hidden states and synthetic index front-end weights: ``x [T, d_model]``,
    ``w_q [G*d_idx, d_model]``, ``w_k [d_idx, d_model]``, fp32 gains
    ``[d_idx]`` each."""
    x = normal((num_tokens, d_model), dtype, device, seed, "hidden")
    sc = d_model ** -0.5
    w_q = (normal((num_groups * index_dim, d_model), torch.float32, device, seed, "w_q_idx") * sc).to(dtype)
    w_k = (normal((index_dim, d_model), torch.float32, device, seed, "w_k_idx") * sc).to(dtype)
    gains = []
    for name in ("gain_q_idx", "gain_k_idx"):
        g = _gen(device, seed, name)
        gains.append(torch.rand((index_dim,), generator=g, device=device, dtype=torch.float32) + 0.5)
    return {"x": x, "w_q": w_q, "w_k": w_k, "gain_q": gains[0], "gain_k": gains[1]}
