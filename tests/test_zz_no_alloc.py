"""msa_index_topk_noalloc (static scratch, no workspace) against msa_index_topk.

Both go through the C ABI on the same inputs; block ids must be identical
(integer output).  Two calls in a row per path, the second smaller, so the
second call runs on scratch that still holds the first call's scores; decode
and prefill; an oversized call is refused before any launch.
"""
import pytest
import torch

from parity_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def msa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from learned_block_sparse_amd import msa as m
    m.lib()
    return m


def _both(msa, q_idx, k_idx, cu_q, cu_k, mq, mk, topk=16):
    ref = msa.msa_index_topk(q_idx, k_idx, cu_q, cu_k, mq, mk, 128, topk)
    out = torch.full_like(ref, -7)
    got = msa.msa_index_topk_noalloc(q_idx, k_idx, cu_q, cu_k, mq, mk, 128, topk, block_idx=out)
    torch.cuda.synchronize()
    return ref, got


def test_prefill_two_calls_second_smaller(msa):
    from learned_block_sparse_amd import synth
    wl = synth.WORKLOADS["prefill_32k"]
    for L, seed in ((9000, 31), (3001, 32)):
        need = msa.msa_index_topk_workspace_size(1, L, L, 4, 128, 16)
        assert 0 < need <= msa.NOALLOC_SCRATCH_BYTES
        say(f"[noalloc] prefill L={L} scratch {need} bytes")
        inp = synth.prefill_inputs(wl, device="cuda", seed=seed, seq_lens=[L], with_main=False)
        ref, got = _both(msa, inp["q_idx"], inp["k_idx"], inp["cu_seqlens_q"], inp["cu_seqlens_k"], L, L)
        assert torch.equal(ref, got), f"L={L}: ids differ from msa_index_topk"


def test_decode_two_calls_second_smaller(msa):
    from learned_block_sparse_amd import synth
    wl = synth.WORKLOADS["decode_1m"]
    for ctx, seed in (([70001, 129, 1, 300000, 2049, 128], 33), ([5000, 127, 40000], 34)):
        say(f"[noalloc] decode ctx={ctx}")
        d = synth.decode_inputs(wl, device="cuda", seed=seed, ctx_lens=ctx)
        ref, got = _both(msa, d["q_idx"], d["k_idx"], d["cu_seqlens_q"], d["cu_seqlens_k"], 1, max(ctx))
        assert torch.equal(ref, got), f"ctx={ctx}: ids differ from msa_index_topk"


def test_varlen_chunks_fp32_and_small_k(msa):
    """Packed chunked prefill in fp32 with k = 5, then bf16 with k = 16."""
    from learned_block_sparse_amd import synth
    wl = synth.WORKLOADS["prefill_32k"]
    kv, ql = [3000, 1000, 300, 700], [1517, 1000, 1, 129]
    say(f"[noalloc] varlen kv={kv} q={ql}")
    inp = synth.prefill_inputs(wl, device="cuda", seed=35, seq_lens=kv, q_lens=ql, with_main=False)
    for qi, ki, k in ((inp["q_idx"].float(), inp["k_idx"].float(), 5), (inp["q_idx"], inp["k_idx"], 16)):
        ref, got = _both(msa, qi, ki, inp["cu_seqlens_q"], inp["cu_seqlens_k"], max(ql), max(kv), topk=k)
        assert torch.equal(ref, got), f"topk={k}: ids differ"


def test_oversized_call_is_refused(msa):
    """32K-row prefill against 32K keys needs 128 MiB of scores: refused."""
    L = 32768
    assert msa.msa_index_topk_workspace_size(1, L, L, 4, 128, 16) > msa.NOALLOC_SCRATCH_BYTES
    q_idx = torch.zeros((L, 4, 128), dtype=torch.bfloat16, device="cuda")
    k_idx = torch.zeros((L, 128), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
    out = torch.full((L, 4, 16), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(msa.MSAError) as e:
        msa.msa_index_topk_noalloc(q_idx, k_idx, cu, cu, L, L, 128, 16, block_idx=out)
    assert e.value.status == msa.MSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == -7).all()), "a refused call must not launch anything"
