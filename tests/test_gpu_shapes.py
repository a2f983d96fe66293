"""GPU parity at shapes other than the measured head configuration.

The measured workloads are 64 query / 4 KV heads, index dim 128, bf16.  The
library also takes 8 groups (8 heads per group, so the 16 MFMA columns of a
group's heads are half used), index dim 64 in bf16, fp32 on the decode path,
and packed batches where a sequence has no query rows or more query rows than
keys (rows with p < 0 attend to nothing).  Every case is checked against the
CPU oracle on the same seeded inputs, ids exactly, outputs within the
tolerances of parity_helpers.
"""
import dataclasses

import numpy as np
import pytest
import torch

from parity_helpers import compare_ids, compare_outputs, host, say

pytestmark = pytest.mark.gpu


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


def _prefill_check(msa, oracle, synth, wl, kv, ql, seed, what, num_splits=0):
    say(f"[shapes] {what}: kv={kv} q={ql} splits={num_splits}")
    inp = synth.prefill_inputs(wl, device="cuda", seed=seed, seq_lens=kv, q_lens=ql)
    ids = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], inp["cu_seqlens_q"], inp["cu_seqlens_k"], max(ql),
                             max(kv), wl.block_size, wl.topk)
    out, lse = msa.msa_sparse_attn_prefill(inp["q"], inp["k"], inp["v"], ids, inp["cu_seqlens_q"],
                                           inp["cu_seqlens_k"], max(ql), max(kv), wl.block_size, wl.topk,
                                           num_splits=num_splits)
    torch.cuda.synchronize()
    cu_q, cu_k = inp["cu_q_host"], inp["cu_k_host"]
    ref_ids, ref_out, ref_lse = oracle.prefill(host(inp["q_idx"]), host(inp["k_idx"]), host(inp["q"]),
                                               host(inp["k"]), host(inp["v"]), cu_q, cu_k, wl.block_size,
                                               wl.topk)
    compare_ids(ids, ref_ids, what)
    compare_outputs(out, lse, ref_out, ref_lse, wl.dtype, what)


def _decode_check(msa, oracle, synth, wl, ctx, seed, what, num_splits=0):
    say(f"[shapes] {what}: ctx={ctx} splits={num_splits}")
    inp = synth.decode_inputs(wl, device="cuda", seed=seed, ctx_lens=ctx)
    ids = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], inp["cu_seqlens_q"], inp["cu_seqlens_k"], 1, max(ctx),
                             wl.block_size, wl.topk)
    out, lse = msa.msa_sparse_attn_decode(inp["q"], inp["k"], inp["v"], ids, inp["k_offsets"], inp["ctx_lens"],
                                          max(ctx), wl.block_size, wl.topk, num_splits=num_splits)
    torch.cuda.synchronize()
    ref_ids, ref_out, ref_lse = oracle.decode(host(inp["q_idx"]), host(inp["k_idx"]), host(inp["q"]),
                                              host(inp["k"]), host(inp["v"]), inp["k_offsets_host"], ctx,
                                              wl.block_size, wl.topk)
    compare_ids(ids, ref_ids, what)
    compare_outputs(out, lse, ref_out, ref_lse, wl.dtype, what)


@pytest.mark.parametrize("num_splits", [0, 1])
def test_eight_groups(msa, synth, oracle_lib, num_splits):
    """64 query / 8 KV heads: the scan's 512 columns hold 64 queries x 8 groups
    (two slices per query block) and each group has 8 heads."""
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], num_kv_heads=8, planted=8)
    _prefill_check(msa, oracle_lib, synth, wl, [3000], [3000], 21, "8 groups", num_splits)


def test_eight_groups_decode(msa, synth, oracle_lib):
    wl = dataclasses.replace(synth.WORKLOADS["decode_1m"], num_kv_heads=8)
    _decode_check(msa, oracle_lib, synth, wl, [129, 4000, 20000], 22, "8 groups decode")


def test_bf16_index_dim_64(msa, synth, oracle_lib):
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], index_dim=64, planted=8)
    _prefill_check(msa, oracle_lib, synth, wl, [2500], [2500], 23, "bf16 d_idx 64")
    wld = dataclasses.replace(synth.WORKLOADS["decode_1m"], index_dim=64)
    _decode_check(msa, oracle_lib, synth, wld, [3000, 700, 129], 24, "bf16 d_idx 64 decode")


@pytest.mark.parametrize("num_splits", [0, 1])
def test_fp32_decode(msa, synth, oracle_lib, num_splits):
    """fp32 inputs on the decode path (8 Q / 2 KV heads, d_idx 64, k 4)."""
    wl = synth.WORKLOADS["tiny_prefill_2k_f32"]
    _decode_check(msa, oracle_lib, synth, wl, [1, 300, 2048, 5000], 25, "fp32 decode", num_splits)


@pytest.mark.parametrize("num_splits", [0, 1])
def test_empty_and_overlong_query_ranges(msa, synth, oracle_lib, num_splits):
    """A sequence with no query rows, one with more query rows than keys (its
    first rows have p < 0: ids -1, output 0, lse -inf) and an ordinary one,
    packed in one call, large enough for the KV-outer schedule."""
    wl = synth.WORKLOADS["prefill_32k"]
    _prefill_check(msa, oracle_lib, synth, wl, [500, 300, 1500], [0, 400, 1500], 26, "empty/overlong",
                   num_splits)
