"""GPU parity of the fp8 (E4M3) paths against the CPU oracle.

Index tensors: the seeded 1/8-grid values of the bf16 workloads (with the
+1.0 planted bias) rounded to E4M3 by round-to-nearest-even.  Every such value
is still a multiple of 1/8, so fp32 scores stay exact on both sides and the
block ids must match the oracle bit for bit.  Without the planted bias the
rounding is the identity, so the fp8 ids must also equal the bf16 path's.

K/V (the *_ex attention calls, bf16 q and out): the seeded N(0, 1) K and V
rounded to E4M3.  The kernels widen E4M3 to bf16 exactly, so out and lse must
be bit-identical to the bf16 call on k.to(bf16) and v.to(bf16), on both
schedules and on decode; against the oracle (fp64 on the exact E4M3 values)
the bf16 tolerances apply.
"""
import dataclasses

import numpy as np
import pytest
import torch

from parity_helpers import compare_ids, compare_outputs, host, say

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


def test_fp8_attention_type_pairs(msa, synth):
    """fp8 q/out is not implemented (plain and _ex calls), nor fp32 q with E4M3
    K/V; bf16 q with E4M3 K/V is."""
    wl = synth.WORKLOADS["decode_1m"]
    d = synth.decode_inputs(wl, device="cuda", seed=36, ctx_lens=[300])
    ids = msa.msa_index_topk(d["q_idx"], d["k_idx"], d["cu_seqlens_q"], d["cu_seqlens_k"], 1, 300,
                             wl.block_size, wl.topk)
    k8, v8 = d["k"].to(FP8), d["v"].to(FP8)
    for fn, q in ((msa.msa_sparse_attn_decode, d["q"].to(FP8)), (msa.msa_sparse_attn_decode_ex, d["q"].to(FP8)),
                  (msa.msa_sparse_attn_decode_ex, d["q"].float())):
        with pytest.raises(msa.MSAError) as e:
            fn(q, k8, v8, ids, d["k_offsets"], d["ctx_lens"], 300, wl.block_size, wl.topk)
        assert e.value.status == msa.MSA_ERR_UNSUPPORTED
    out, lse = msa.msa_sparse_attn_decode_ex(d["q"], k8, v8, ids, d["k_offsets"], d["ctx_lens"], 300,
                                             wl.block_size, wl.topk)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def _fp8_kv(inp):
    return inp["k"].to(FP8), inp["v"].to(FP8)


@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_fp8_kv_prefill_vs_oracle(msa, synth, oracle_lib, num_splits):
    """bf16 q, E4M3 K/V; num_splits 0 takes the KV-outer schedule (6,516
    (query, group) items), 1 and 3 the query-outer one.  Planted blocks and a
    short second sequence make hot buckets and a ragged tail."""
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], planted=8)
    kv, ql = [3000, 700], [1500, 129]
    say(f"[fp8 kv] prefill kv={kv} q={ql} splits={num_splits}")
    inp = synth.prefill_inputs(wl, device="cuda", seed=37, seq_lens=kv, q_lens=ql)
    k8, v8 = _fp8_kv(inp)
    ids = _prefill_ids(msa, inp, wl, inp["q_idx"], inp["k_idx"], kv, ql)
    out, lse = msa.msa_sparse_attn_prefill_ex(inp["q"], k8, v8, ids, inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                              max(ql), max(kv), wl.block_size, wl.topk, num_splits=num_splits)
    torch.cuda.synchronize()
    ref_ids, ref_out, ref_lse = oracle_lib.prefill(host(inp["q_idx"]), host(inp["k_idx"]), host(inp["q"]),
                                                   host(k8), host(v8), inp["cu_q_host"], inp["cu_k_host"],
                                                   wl.block_size, wl.topk)
    compare_ids(ids, ref_ids, "fp8 kv prefill ids")
    compare_outputs(out, lse, ref_out, ref_lse, "bf16", f"fp8 kv prefill splits {num_splits}")


@pytest.mark.parametrize("num_splits", [0, 1, 2])
def test_fp8_kv_prefill_bitwise_equals_bf16(msa, synth, num_splits):
    """E4M3 K/V are widened to bf16 exactly, so the _ex call on E4M3 K/V and
    the plain bf16 call on the same values agree bit for bit."""
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], planted=8)
    kv, ql = [4100, 300], [4100, 300]
    say(f"[fp8 kv] prefill bitwise kv={kv} splits={num_splits}")
    inp = synth.prefill_inputs(wl, device="cuda", seed=38, seq_lens=kv, q_lens=ql)
    k8, v8 = _fp8_kv(inp)
    ids = _prefill_ids(msa, inp, wl, inp["q_idx"], inp["k_idx"], kv, ql)
    a = msa.msa_sparse_attn_prefill_ex(inp["q"], k8, v8, ids, inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                       max(ql), max(kv), wl.block_size, wl.topk, num_splits=num_splits)
    b = msa.msa_sparse_attn_prefill(inp["q"], k8.bfloat16(), v8.bfloat16(), ids, inp["cu_seqlens_q"],
                                    inp["cu_seqlens_k"], max(ql), max(kv), wl.block_size, wl.topk,
                                    num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.parametrize("num_splits", [0, 1])
def test_fp8_kv_decode_vs_oracle(msa, synth, oracle_lib, num_splits):
    """Decode with an E4M3 KV cache (bf16 index tensors), ragged contexts."""
    wl = synth.WORKLOADS["decode_1m"]
    ctx = [1, 129, 4000, 70001]
    say(f"[fp8 kv] decode ctx={ctx} splits={num_splits}")
    d = synth.decode_inputs(wl, device="cuda", seed=39, ctx_lens=ctx)
    k8, v8 = _fp8_kv(d)
    ids = msa.msa_index_topk(d["q_idx"], d["k_idx"], d["cu_seqlens_q"], d["cu_seqlens_k"], 1, max(ctx),
                             wl.block_size, wl.topk)
    out, lse = msa.msa_sparse_attn_decode_ex(d["q"], k8, v8, ids, d["k_offsets"], d["ctx_lens"], max(ctx),
                                             wl.block_size, wl.topk, num_splits=num_splits)
    b = msa.msa_sparse_attn_decode(d["q"], k8.bfloat16(), v8.bfloat16(), ids, d["k_offsets"], d["ctx_lens"],
                                   max(ctx), wl.block_size, wl.topk, num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(lse.view(torch.int32), b[1].view(torch.int32))
    ref_ids, ref_out, ref_lse = oracle_lib.decode(host(d["q_idx"]), host(d["k_idx"]), host(d["q"]), host(k8),
                                                  host(v8), d["k_offsets_host"], ctx, wl.block_size, wl.topk)
    compare_ids(ids, ref_ids, "fp8 kv decode ids")
    compare_outputs(out, lse, ref_out, ref_lse, "bf16", f"fp8 kv decode splits {num_splits}")


def test_fp8_decode_step_all_fp8(msa, synth, oracle_lib):
    """A whole decode step with every cache in E4M3: index keys and queries
    (planted, so scores stay exact), K and V; bf16 q and out."""
    wl = dataclasses.replace(synth.WORKLOADS["decode_1m"], planted=16)
    ctx = [300, 9000, 33000]
    say(f"[fp8 kv] all-fp8 decode ctx={ctx}")
    d = synth.decode_inputs(wl, device="cuda", seed=40, ctx_lens=ctx)
    qi8, ki8 = d["q_idx"].to(FP8), d["k_idx"].to(FP8)
    k8, v8 = _fp8_kv(d)
    ids = msa.msa_index_topk(qi8, ki8, d["cu_seqlens_q"], d["cu_seqlens_k"], 1, max(ctx), wl.block_size, wl.topk)
    out, lse = msa.msa_sparse_attn_decode_ex(d["q"], k8, v8, ids, d["k_offsets"], d["ctx_lens"], max(ctx),
                                             wl.block_size, wl.topk)
    torch.cuda.synchronize()
    ref_ids, ref_out, ref_lse = oracle_lib.decode(host(qi8), host(ki8), host(d["q"]), host(k8), host(v8),
                                                  d["k_offsets_host"], ctx, wl.block_size, wl.topk)
    compare_ids(ids, ref_ids, "all-fp8 decode ids")
    compare_outputs(out, lse, ref_out, ref_lse, "bf16", "all-fp8 decode")
