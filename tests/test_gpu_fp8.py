"""GPU parity of the fp8 (E4M3) index path against the CPU oracle.

The index tensors are the seeded 1/8-grid values of the bf16 workloads (with
the +1.0 planted bias) rounded to E4M3 by round-to-nearest-even.  Every such
value is still a multiple of 1/8, so fp32 scores stay exact on both sides and
the block ids must match the oracle bit for bit.  Without the planted bias the
rounding is the identity, so the fp8 ids must also equal the bf16 path's.
"""
import dataclasses

import numpy as np
import pytest
import torch

from parity_helpers import compare_ids, host, say

pytestmark = pytest.mark.gpu

FP8 = torch.float8_e4m3fn


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from learned_block_sparse_amd import msa as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def synth():
    from learned_block_sparse_amd import synth as s
    return s


def _prefill_ids(msa, inp, wl, q_idx, k_idx, kv, ql):
    ids = msa.msa_index_topk(q_idx, k_idx, inp["cu_seqlens_q"], inp["cu_seqlens_k"], max(ql), max(kv),
                             wl.block_size, wl.topk)
    torch.cuda.synchronize()
    return ids


@pytest.mark.parametrize("index_dim", [128, 64])
def test_fp8_prefill_ids(msa, synth, oracle_lib, index_dim):
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], index_dim=index_dim, planted=8)
    kv, ql = [3000, 700], [3000, 129]
    say(f"[fp8] prefill d_idx={index_dim} kv={kv} q={ql}")
    inp = synth.prefill_inputs(wl, device="cuda", seed=31, seq_lens=kv, q_lens=ql, with_main=False)
    q8, k8 = inp["q_idx"].to(FP8), inp["k_idx"].to(FP8)
    ids = _prefill_ids(msa, inp, wl, q8, k8, kv, ql)
    rows, kstart, pos = oracle_lib.rows_prefill(inp["cu_q_host"], inp["cu_k_host"])
    ref = oracle_lib.index_topk(host(q8), host(k8), kstart, pos, rows, wl.block_size, wl.topk)
    compare_ids(ids, ref, f"fp8 prefill d_idx {index_dim}")


def test_fp8_prefill_equals_bf16_on_exact_values(msa, synth):
    """No planting: every index value is exact in E4M3, so both element types
    must select the same blocks (tie-dense data included)."""
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], planted=0)
    kv = [4100]
    inp = synth.prefill_inputs(wl, device="cuda", seed=32, seq_lens=kv, with_main=False)
    g = torch.Generator(device="cuda").manual_seed(33)
    # half the rows tie-dense ({-1/8, 0, 1/8}), half on the full grid
    qd = (torch.randint(-1, 2, inp["q_idx"].shape, generator=g, device="cuda").float() / 8).bfloat16()
    q = torch.where(torch.arange(kv[0], device="cuda")[:, None, None] % 2 == 0, qd, inp["q_idx"])
    k = inp["k_idx"]
    assert torch.equal(q.to(FP8).float(), q.float()) and torch.equal(k.to(FP8).float(), k.float())
    say("[fp8] prefill fp8 == bf16 on exact values")
    a = _prefill_ids(msa, inp, wl, q, k, kv, kv)
    b = _prefill_ids(msa, inp, wl, q.to(FP8), k.to(FP8), kv, kv)
    assert torch.equal(a, b)


@pytest.mark.parametrize("index_dim", [128, 64])
def test_fp8_decode_ids(msa, synth, oracle_lib, index_dim):
    wl = dataclasses.replace(synth.WORKLOADS["decode_1m"], index_dim=index_dim, planted=16)
    ctx = [1, 129, 4000, 70001]
    say(f"[fp8] decode d_idx={index_dim} ctx={ctx}")
    d = synth.decode_inputs(wl, device="cuda", seed=34, ctx_lens=ctx)
    q8, k8 = d["q_idx"].to(FP8), d["k_idx"].to(FP8)
    ids = msa.msa_index_topk(q8, k8, d["cu_seqlens_q"], d["cu_seqlens_k"], 1, max(ctx), wl.block_size, wl.topk)
    torch.cuda.synchronize()
    _, kstart, pos = oracle_lib.rows_decode(d["k_offsets_host"], ctx)
    ref = oracle_lib.index_topk(host(q8), host(k8), kstart, pos, np.arange(len(ctx)), wl.block_size, wl.topk)
    compare_ids(ids, ref, f"fp8 decode d_idx {index_dim}")


def test_fp8_decode_and_prefill_paths_agree(msa, synth):
    wl = synth.WORKLOADS["decode_1m"]
    ctx = [3000, 129, 9000]
    d = synth.decode_inputs(wl, device="cuda", seed=35, ctx_lens=ctx)
    q8, k8 = d["q_idx"].to(FP8), d["k_idx"].to(FP8)
    dec = msa.msa_index_topk(q8, k8, d["cu_seqlens_q"], d["cu_seqlens_k"], 1, max(ctx), wl.block_size, wl.topk)
    qi = torch.stack([q8.view(torch.uint8), q8.view(torch.uint8)], dim=1).reshape(-1, *q8.shape[1:])
    qi = qi.contiguous().view(FP8)
    cu_q = torch.arange(0, 2 * len(ctx) + 1, 2, dtype=torch.int32, device="cuda")
    pre = msa.msa_index_topk(qi, k8, cu_q, d["cu_seqlens_k"], 2, max(ctx), wl.block_size, wl.topk)
    torch.cuda.synchronize()
    assert torch.equal(dec, pre[1::2])


def test_fp8_attention_is_unsupported(msa, synth):
    wl = synth.WORKLOADS["decode_1m"]
    d = synth.decode_inputs(wl, device="cuda", seed=36, ctx_lens=[300])
    ids = msa.msa_index_topk(d["q_idx"], d["k_idx"], d["cu_seqlens_q"], d["cu_seqlens_k"], 1, 300,
                             wl.block_size, wl.topk)
    with pytest.raises(msa.MSAError) as e:
        msa.msa_sparse_attn_decode(d["q"].to(FP8), d["k"].to(FP8), d["v"].to(FP8), ids, d["k_offsets"],
                                   d["ctx_lens"], 300, wl.block_size, wl.topk)
    assert e.value.status == msa.MSA_ERR_UNSUPPORTED
