"""GPU parity of the main-branch backward against the CPU oracle.

The forward call (ids from the GPU index call, exact on grid inputs, then the
GPU attention) produces out and lse; dO ~ N(0, 1) rounded to bf16.  The
backward call returns fp32 dq, dk, dv; the oracle recomputes everything in
fp64 from q, k, v, dO and the same ids.

Tolerance.  The GPU rounds P and dS to bf16 before the dV, dK and dQ products
(relative 2^-9 each), keeps each block's dq contribution in bf16 until the
fp32 sum over the row's blocks, and takes delta = dO . out from the bf16
forward output;
everything else accumulates in fp32 from exact bf16 inputs.  These are
independent relative perturbations of about 2^-9 per term, so the error of a
gradient relative to its own scale is a few parts in 10^3: the tests require
relative RMS (||err|| / ||ref||) <= 1e-2 and max |err| <= 2e-2 * max |ref| for
each of dq, dk, dv (measured values are printed).
"""
import dataclasses

import numpy as np
import pytest
import torch

from parity_helpers import host, say

pytestmark = pytest.mark.gpu

REL_RMS = 1e-2
MAX_REL = 2e-2


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


def _forward_backward(msa, synth, wl, kv, ql, seed):
    inp = synth.prefill_inputs(wl, device="cuda", seed=seed, seq_lens=kv, q_lens=ql)
    mq, mk = max(ql), max(kv)
    ids = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], inp["cu_seqlens_q"], inp["cu_seqlens_k"], mq, mk,
                             wl.block_size, wl.topk)
    out, lse = msa.msa_sparse_attn_prefill(inp["q"], inp["k"], inp["v"], ids, inp["cu_seqlens_q"],
                                           inp["cu_seqlens_k"], mq, mk, wl.block_size, wl.topk)
    dout = synth.normal(inp["q"].shape, torch.bfloat16, "cuda", seed, "dout")
    grads = msa.msa_sparse_attn_backward(inp["q"], inp["k"], inp["v"], out, dout, lse, ids, inp["cu_seqlens_q"],
                                         inp["cu_seqlens_k"], mq, mk, wl.block_size, wl.topk)
    torch.cuda.synchronize()
    return inp, ids, dout, grads


def _compare(name, gpu, ref, what):
    g = gpu.detach().cpu().double().numpy()
    err = np.abs(g - ref)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    rel = float(np.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300))) if ref.size else 0.0
    mx = float(err.max()) if err.size else 0.0
    say(f"    {what} {name}: rel-RMS {rel:.2e}, max-abs {mx:.2e} (max |ref| {scale:.3g})")
    assert rel <= REL_RMS, f"{what} {name}: rel-RMS {rel:.3g} > {REL_RMS}"
    assert mx <= MAX_REL * max(scale, 1e-30), f"{what} {name}: max-abs {mx:.3g} > {MAX_REL} * {scale:.3g}"


def _check_vs_oracle(oracle_lib, inp, ids, dout, grads, wl, what):
    rows, kstart, pos = oracle_lib.rows_prefill(inp["cu_q_host"], inp["cu_k_host"])
    dq, dk, dv = oracle_lib.sparse_attn_bwd(host(inp["q"]), host(inp["k"]), host(inp["v"]), host(dout),
                                            host(ids).numpy(), kstart, pos, rows, wl.block_size, wl.topk)
    for name, gpu, ref in zip(("dq", "dk", "dv"), grads, (dq, dk, dv)):
        _compare(name, gpu, ref, what)
    return dq, dk, dv


def test_backward_vs_oracle(msa, synth, oracle_lib):
    """Measured head configuration (64 Q / 4 KV heads), two packed sequences,
    the second a chunk (q_len < kv_len), planted hot blocks."""
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], planted=8)
    kv, ql = [1000, 300], [1000, 129]
    say(f"[bwd] kv={kv} q={ql}")
    inp, ids, dout, grads = _forward_backward(msa, synth, wl, kv, ql, 41)
    _check_vs_oracle(oracle_lib, inp, ids, dout, grads, wl, "bwd")


@pytest.mark.parametrize("max_kv_len", [1 << 18, 1 << 20])
def test_backward_loose_kv_bound(msa, synth, oracle_lib, max_kv_len):
    """max_kv_len passed as a loose upper bound, so the edge lists hold 2 x 4 x
    2048 or 2 x 4 x 8192 (sequence, group, block) buckets: the second is past
    the LDS table and places edges by one global atomic each."""
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], planted=8)
    kv, ql = [1000, 300], [1000, 129]
    say(f"[bwd] kv={kv} q={ql} max_kv_len={max_kv_len}")
    inp = synth.prefill_inputs(wl, device="cuda", seed=43, seq_lens=kv, q_lens=ql)
    mq = max(ql)
    ids = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], inp["cu_seqlens_q"], inp["cu_seqlens_k"], mq, max(kv),
                             wl.block_size, wl.topk)
    out, lse = msa.msa_sparse_attn_prefill(inp["q"], inp["k"], inp["v"], ids, inp["cu_seqlens_q"],
                                           inp["cu_seqlens_k"], mq, max_kv_len, wl.block_size, wl.topk)
    dout = synth.normal(inp["q"].shape, torch.bfloat16, "cuda", 43, "dout")
    grads = msa.msa_sparse_attn_backward(inp["q"], inp["k"], inp["v"], out, dout, lse, ids, inp["cu_seqlens_q"],
                                         inp["cu_seqlens_k"], mq, max_kv_len, wl.block_size, wl.topk)
    torch.cuda.synchronize()
    _check_vs_oracle(oracle_lib, inp, ids, dout, grads, wl, f"bwd max_kv_len={max_kv_len}")


def test_backward_is_deterministic(msa, synth):
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], planted=8)
    kv, ql = [2100, 700], [2100, 700]
    say(f"[bwd] determinism kv={kv}")
    _, _, _, g1 = _forward_backward(msa, synth, wl, kv, ql, 42)
    _, _, _, g2 = _forward_backward(msa, synth, wl, kv, ql, 42)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_backward_several_windows(msa, synth, oracle_lib):
    """9,000 query rows: the edge lists are built in two windows of at most
    8,192 rows and dK / dV accumulate across them.  8 Q / 2 KV heads keep the
    oracle fast."""
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], num_heads=8, num_kv_heads=2, planted=8)
    kv = [9000]
    say(f"[bwd] two windows kv={kv} heads 8/2")
    inp, ids, dout, grads = _forward_backward(msa, synth, wl, kv, kv, 43)
    _check_vs_oracle(oracle_lib, inp, ids, dout, grads, wl, "bwd 2 windows")


def test_backward_chunk_of_long_prefill(msa, synth, oracle_lib):
    """The last 1,024 query rows of a 32K sequence against the whole prefix
    (a chunked-prefill call): dk / dv over all 32K keys."""
    wl = synth.WORKLOADS["prefill_32k"]
    kv, ql = [32768], [1024]
    say(f"[bwd] chunk kv={kv} q={ql}")
    inp, ids, dout, grads = _forward_backward(msa, synth, wl, kv, ql, 44)
    _check_vs_oracle(oracle_lib, inp, ids, dout, grads, wl, "bwd chunk")


def test_backward_empty_and_overlong(msa, synth, oracle_lib):
    """A sequence with no query rows and one with more query rows than keys
    (rows with p < 0 attend to nothing: dq = 0) packed with an ordinary one."""
    wl = synth.WORKLOADS["prefill_32k"]
    kv, ql = [500, 300, 1500], [0, 400, 1500]
    say(f"[bwd] empty/overlong kv={kv} q={ql}")
    inp, ids, dout, grads = _forward_backward(msa, synth, wl, kv, ql, 45)
    _check_vs_oracle(oracle_lib, inp, ids, dout, grads, wl, "bwd empty/overlong")
    assert torch.all(grads[0][:100] == 0)  # the first 100 rows of the second sequence have p < 0
    # no query row of the first sequence: its 500 key rows get exactly 0
    assert torch.all(grads[1][:500] == 0) and torch.all(grads[2][:500] == 0)


def test_backward_unsupported_type(msa, synth):
    wl = synth.WORKLOADS["tiny_prefill_2k_f32"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=46, seq_lens=[300])
    ids = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], inp["cu_seqlens_q"], inp["cu_seqlens_k"], 300, 300,
                             wl.block_size, wl.topk)
    out, lse = msa.msa_sparse_attn_prefill(inp["q"], inp["k"], inp["v"], ids, inp["cu_seqlens_q"],
                                           inp["cu_seqlens_k"], 300, 300, wl.block_size, wl.topk)
    with pytest.raises(msa.MSAError) as e:
        msa.msa_sparse_attn_backward(inp["q"], inp["k"], inp["v"], out, out, lse, ids, inp["cu_seqlens_q"],
                                     inp["cu_seqlens_k"], 300, 300, wl.block_size, wl.topk)
    assert e.value.status == msa.MSA_ERR_UNSUPPORTED


def test_backward_beyond_sort_capacity(msa, synth, oracle_lib):
    """65 packed sequences, one of 16,384 tokens and 64 of 3: 65 x 4 groups x 128
    blocks = 33,280 buckets, more than the dK/dV dispatch sort holds, so the
    fixed last-block-first order is used instead; results as for any order."""
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], planted=8)
    kv = [16384] + [3] * 64
    ql = [256] + [3] * 64
    say(f"[bwd] 65 sequences, {65 * 4 * 128} buckets")
    inp, ids, dout, grads = _forward_backward(msa, synth, wl, kv, ql, 47)
    _check_vs_oracle(oracle_lib, inp, ids, dout, grads, wl, "bwd many buckets")


def test_backward_hot_buckets(msa, synth, oracle_lib):
    """8,192 rows against 8,192 keys: the early blocks are picked by nearly
    every row (every block of rows below 2,048, a growing share after), so
    buckets hold up to several thousand edges and dK / dV are summed from
    many 256-edge chunks; checked against the oracle and for bitwise
    reproducibility.  8 Q / 2 KV heads keep the oracle fast."""
    wl = dataclasses.replace(synth.WORKLOADS["prefill_32k"], num_heads=8, num_kv_heads=2, planted=8)
    kv = [8192]
    say(f"[bwd] hot buckets kv={kv} heads 8/2")
    inp, ids, dout, grads = _forward_backward(msa, synth, wl, kv, kv, 49)
    largest = max(int(torch.bincount(ids[:, g][ids[:, g] >= 0]).max()) for g in range(ids.shape[1]))
    say(f"    largest bucket {largest} edges")
    assert largest > 4 * 256
    _check_vs_oracle(oracle_lib, inp, ids, dout, grads, wl, "bwd hot buckets")
    _, _, _, again = _forward_backward(msa, synth, wl, kv, kv, 49)
    for a, b in zip(grads, again):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("tile", [0, 15])
def test_backward_128k_tile_sampled(msa, synth, oracle_lib, tile):
    """The bench's launches: 8192 query rows against the 128K causal prefix,
    the first call (hot early blocks) and the last.  dO is zero except on 48
    sampled rows, so dk / dv are exactly those rows' contributions (which the
    oracle computes row by row) and dq is exactly 0 on every other row."""
    wl = synth.WORKLOADS["prefill_128k"]
    lo, hi = tile * wl.q_tile, (tile + 1) * wl.q_tile
    m = hi - lo
    say(f"[bwd] 128K tile rows [{lo}, {hi}), sampled dO")
    inp = synth.prefill_inputs(wl, device="cuda", seed=0)
    cu_q = torch.tensor([0, m], dtype=torch.int32, device="cuda")
    cu_k = torch.tensor([0, hi], dtype=torch.int32, device="cuda")
    q = inp["q"][lo:hi]
    ids = msa.msa_index_topk(inp["q_idx"][lo:hi], inp["k_idx"], cu_q, cu_k, m, hi, wl.block_size, wl.topk)
    out, lse = msa.msa_sparse_attn_prefill(q, inp["k"], inp["v"], ids, cu_q, cu_k, m, hi, wl.block_size, wl.topk)
    rng = np.random.default_rng(48)
    sample = np.unique(np.concatenate([[0, m - 1], rng.integers(0, m, 46)]))
    sidx = torch.as_tensor(sample, device="cuda")
    dout = torch.zeros_like(q)
    dout[sidx] = synth.normal((len(sample), wl.num_heads, wl.head_dim), torch.bfloat16, "cuda", 48, "dout")
    # K / V of the call's causal prefix: dk / dv have one row per key of the call
    kp, vp = inp["k"][:hi], inp["v"][:hi]
    dq, dk, dv = msa.msa_sparse_attn_backward(q, kp, vp, out, dout, lse, ids, cu_q, cu_k, m, hi,
                                              wl.block_size, wl.topk)
    torch.cuda.synchronize()
    others = torch.ones(m, dtype=torch.bool, device="cuda")
    others[sidx] = False
    assert bool((dq[others] == 0).all()), "dq must be exactly 0 where dO is 0"
    rows, kstart, pos = oracle_lib.rows_prefill([0, m], [0, hi], sample)
    rdq, rdk, rdv = oracle_lib.sparse_attn_bwd(host(q), host(kp), host(vp), host(dout),
                                               host(ids).numpy()[sample], kstart, pos, rows, wl.block_size, wl.topk)
    _compare("dq", dq[sidx], rdq, "128K tile")
    _compare("dk", dk, rdk, "128K tile")
    _compare("dv", dv, rdv, "128K tile")
