"""GPU parity over a seeded random sweep of shapes.

Each case draws a head configuration (groups, heads per group up to 16, not
only powers of two), the index dim, k, the element type, a packed batch of
1-3 sequences with ragged key lengths and query lengths (whole prefills,
chunked prefills, and sequences with more query rows than keys), the number of
planted blocks and the split count, then runs the index call and the prefill
call and one decode step on the same caches, and compares with the CPU oracle:
block ids exactly, outputs and LSEs within the tolerances of parity_helpers.
The draws come from a fixed numpy seed, so the cases are the same on every run.
A second set of cases packs long ragged sequences and compares block ids only.
"""
import dataclasses

import numpy as np
import pytest
import torch

from parity_helpers import compare_ids, compare_outputs, host, say

pytestmark = pytest.mark.gpu

HEADS = [(8, 2), (12, 4), (16, 4), (32, 8), (48, 4), (64, 4)]


def _cases(n=12, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hq, g = HEADS[i % len(HEADS)]  # every head configuration appears twice
        f32 = i % 4 == 3
        batch = int(rng.integers(1, 4))
        kv, ql = [], []
        for _ in range(batch):
            n_kv = int(rng.integers(1, 2600))
            r = rng.random()
            n_q = n_kv if r < 0.5 else (int(rng.integers(1, n_kv + 1)) if r < 0.85 else n_kv + int(rng.integers(1, 50)))
            kv.append(n_kv)
            ql.append(n_q)
        cases.append(dict(id=i, hq=hq, g=g, f32=f32, d_idx=int(rng.choice([64, 128])),
                          topk=int(rng.choice([1, 3, 8, 16])), planted=int(rng.integers(0, 5)),
                          kv=kv, ql=ql, splits=int(rng.choice([0, 0, 1, 3]))))
    return cases


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


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c['id']}")
def test_random_shapes(msa, synth, oracle_lib, case):
    base = synth.WORKLOADS["tiny_prefill_2k_f32" if case["f32"] else "prefill_32k"]
    wl = dataclasses.replace(base, num_heads=case["hq"], num_kv_heads=case["g"], index_dim=case["d_idx"],
                             topk=case["topk"], planted=case["planted"])
    kv, ql = case["kv"], case["ql"]
    what = (f"case{case['id']} {wl.dtype} heads {wl.num_heads}/{wl.num_kv_heads} d_idx {wl.index_dim} "
            f"k {wl.topk} kv={kv} q={ql} splits={case['splits']}")
    say(f"[sweep] {what}")
    seed = 1000 + case["id"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=seed, seq_lens=kv, q_lens=ql)
    ids = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], inp["cu_seqlens_q"], inp["cu_seqlens_k"], max(ql),
                             max(kv), wl.block_size, wl.topk)
    out, lse = msa.msa_sparse_attn_prefill(inp["q"], inp["k"], inp["v"], ids, inp["cu_seqlens_q"],
                                           inp["cu_seqlens_k"], max(ql), max(kv), wl.block_size, wl.topk,
                                           num_splits=case["splits"])
    torch.cuda.synchronize()
    ref_ids, ref_out, ref_lse = oracle_lib.prefill(host(inp["q_idx"]), host(inp["k_idx"]), host(inp["q"]),
                                                   host(inp["k"]), host(inp["v"]), inp["cu_q_host"],
                                                   inp["cu_k_host"], wl.block_size, wl.topk)
    compare_ids(ids, ref_ids, what + " prefill ids")
    compare_outputs(out, lse, ref_out, ref_lse, wl.dtype, what + " prefill")

    # one decode step per sequence on caches of the same lengths
    d = synth.decode_inputs(wl, device="cuda", seed=seed, ctx_lens=kv)
    dids = msa.msa_index_topk(d["q_idx"], d["k_idx"], d["cu_seqlens_q"], d["cu_seqlens_k"], 1, max(kv),
                              wl.block_size, wl.topk)
    dout, dlse = msa.msa_sparse_attn_decode(d["q"], d["k"], d["v"], dids, d["k_offsets"], d["ctx_lens"], max(kv),
                                            wl.block_size, wl.topk, num_splits=case["splits"])
    torch.cuda.synchronize()
    r_ids, r_out, r_lse = oracle_lib.decode(host(d["q_idx"]), host(d["k_idx"]), host(d["q"]), host(d["k"]),
                                            host(d["v"]), d["k_offsets_host"], kv, wl.block_size, wl.topk)
    compare_ids(dids, r_ids, what + " decode ids")
    compare_outputs(dout, dlse, r_out, r_lse, wl.dtype, what + " decode")


def _long_cases(n=4, seed=4242):
    """Packed batches of 2-5 long ragged sequences (2,000-24,000 keys): scans
    with several key chunks and, for the larger batches, two rounds of items
    (each workgroup then scores an item and its mirror); selections over up to
    187 earlier blocks."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        hq, g = HEADS[(2 * i + 1) % len(HEADS)]
        d_idx = int(rng.choice([64, 128]))
        topk = int(rng.choice([3, 8, 16]))
        planted = int(rng.integers(0, 9))
        batch = int(rng.integers(2, 6))
        kv = [int(rng.integers(2000, 24000)) for _ in range(batch)]
        ql = [n if rng.random() < 0.7 else int(rng.integers(1, n + 1)) for n in kv]
        cases.append(dict(id=i, hq=hq, g=g, d_idx=d_idx, topk=topk, planted=planted, kv=kv, ql=ql))
    return cases


@pytest.mark.parametrize("case", _long_cases(), ids=lambda c: f"long{c['id']}")
def test_long_ragged_batch_ids(msa, synth, oracle_lib, case):
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], num_heads=case["hq"], num_kv_heads=case["g"],
                             index_dim=case["d_idx"], topk=case["topk"], planted=case["planted"])
    kv, ql = case["kv"], case["ql"]
    what = (f"long{case['id']} heads {wl.num_heads}/{wl.num_kv_heads} d_idx {wl.index_dim} k {wl.topk} "
            f"kv={kv} q={ql}")
    say(f"[sweep] {what}")
    inp = synth.prefill_inputs(wl, device="cuda", seed=5000 + case["id"], seq_lens=kv, q_lens=ql, with_main=False)
    ids = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], inp["cu_seqlens_q"], inp["cu_seqlens_k"], max(ql),
                             max(kv), wl.block_size, wl.topk)
    torch.cuda.synchronize()
    rows, kstart, pos = oracle_lib.rows_prefill(inp["cu_q_host"], inp["cu_k_host"])
    ref = oracle_lib.index_topk(host(inp["q_idx"]), host(inp["k_idx"]), kstart, pos, rows, wl.block_size, wl.topk)
    compare_ids(ids, ref, what + " ids")
