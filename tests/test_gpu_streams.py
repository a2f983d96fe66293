"""Calls on a side stream with no caller workspace.

The binding allocates the workspace and the outputs itself when the caller
passes none.  Those allocations must belong to the stream the kernels run on:
if they belonged to torch's current stream, the caching allocator could hand
the freed workspace to the next allocation on that stream while the side
stream's kernels still use it.  Here every call runs on a side stream, the
default stream then immediately allocates and overwrites buffers of the same
sizes, and the results must equal (bitwise: same schedule, same inputs) those
of the same calls on the default stream.
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


def _calls(msa, inp, wl, L, stream):
    cu_q, cu_k = inp["cu_seqlens_q"], inp["cu_seqlens_k"]
    ids = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], cu_q, cu_k, L, L, wl.block_size, wl.topk, stream=stream)
    out, lse = msa.msa_sparse_attn_prefill(inp["q"], inp["k"], inp["v"], ids, cu_q, cu_k, L, L, wl.block_size,
                                           wl.topk, stream=stream)
    return ids, out, lse


def _scribble(msa, wl, L, G, Hq):
    """Allocate and overwrite buffers the size of the freed workspaces."""
    sizes = [msa.msa_index_topk_workspace_size(1, L, L, G, wl.block_size, wl.topk),
             msa.msa_sparse_attn_workspace_size(1, L, L, Hq, G, 128, wl.topk, 0)]
    junk = []
    for _ in range(3):
        for n in sizes:
            junk.append(torch.full((n,), 0x7f, dtype=torch.uint8, device="cuda"))
    return junk


@pytest.mark.parametrize("handle", [False, True])
def test_side_stream_without_workspace(msa, handle):
    from learned_block_sparse_amd import synth
    wl = synth.WORKLOADS["prefill_32k"]
    L = 9000
    say(f"[streams] side stream, L={L}, raw handle={handle}")
    inp = synth.prefill_inputs(wl, device="cuda", seed=21, seq_lens=[L])
    G, Hq = inp["k"].shape[1], inp["q"].shape[1]
    ref = _calls(msa, inp, wl, L, None)
    torch.cuda.synchronize()
    ref = [t.clone() for t in ref]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = _calls(msa, inp, wl, L, side.cuda_stream if handle else side)
    junk = _scribble(msa, wl, L, G, Hq)     # default stream, while the side stream may still run
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    for a, b, name in zip(got, ref, ["block_idx", "out", "lse"]):
        assert torch.equal(a, b), f"{name} differs from the default-stream run"
