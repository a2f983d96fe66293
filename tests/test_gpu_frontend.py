"""GPU parity of the index front-end (projection, RMS norm, RoPE) against the
CPU oracle.

Inputs: hidden states ~ N(0, 1) and projections ~ N(0, 1/d_model) rounded to
the input type, fp32 gains (seeded, from the synthetic input module).  The
GPU accumulates the bf16 (or fp32) products in fp32 and takes the angle's
quarter-turn reduction in fp64; the oracle does everything in fp64.  The
projected values are about N(0, 1), so the fp32 accumulation error over 3072
terms is ~1e-6: fp32 outputs must match to max |err| <= 1e-4; bf16 outputs
(rounded once, relative 2^-9) to max |err| <= 2e-2 and relative RMS <= 1e-2.
Key rows land at cu_seqlens_k[b] + p, and every other row of the index-key
tensor must be left bit-for-bit as it was.
"""
import numpy as np
import pytest
import torch

from parity_helpers import host, say

pytestmark = pytest.mark.gpu

THETA = 10000.0
EPS = 1e-6


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


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def _check(gpu, ref, out_dtype, what):
    g = gpu.detach().float().cpu().double().numpy()
    err = np.abs(g - ref)
    mx = float(err.max()) if err.size else 0.0
    rel = float(np.sqrt((err ** 2).sum() / max((ref ** 2).sum(), 1e-300))) if err.size else 0.0
    say(f"    {what}: max-abs {mx:.2e}, rel-RMS {rel:.2e} (max |ref| {np.abs(ref).max() if ref.size else 0:.3g})")
    if out_dtype == torch.float32:
        assert mx <= 1e-4, f"{what}: max-abs {mx:.3g}"
    else:
        assert mx <= 2e-2 and rel <= 1e-2, f"{what}: max-abs {mx:.3g}, rel-RMS {rel:.3g}"


def _run(msa, synth, oracle_lib, q_lens, kv_lens, *, G=4, DI=128, d_model=3072, rope=64, dtype=torch.bfloat16,
         out_dtype=torch.float32, seed=0, what=""):
    T = int(sum(q_lens))
    cu_q, cu_k = _cu(q_lens), _cu(kv_lens)
    inp = synth.frontend_inputs(T, G, DI, d_model, dtype, "cuda", seed)
    cuq_d = torch.tensor(cu_q, dtype=torch.int32, device="cuda")
    cuk_d = torch.tensor(cu_k, dtype=torch.int32, device="cuda")
    # the index-key tensor starts with a sentinel so untouched rows can be checked
    k_idx = torch.full((int(cu_k[-1]), DI), 7.0, dtype=out_dtype, device="cuda")
    before = k_idx.clone()
    q_idx, k_out = msa.msa_index_frontend(inp["x"], inp["w_q"], inp["w_k"], inp["gain_q"], inp["gain_k"], cuq_d,
                                          cuk_d, G, rope_dim=rope, rope_theta=THETA, norm_eps=EPS,
                                          out_dtype=out_dtype, k_idx=k_idx)
    torch.cuda.synchronize()
    assert k_out.data_ptr() == k_idx.data_ptr()
    rows, kstart, pos = oracle_lib.rows_prefill(cu_q, cu_k)
    rq, rk = oracle_lib.index_frontend(host(inp["x"]), host(inp["w_q"]), host(inp["w_k"]),
                                       inp["gain_q"].cpu().numpy(), inp["gain_k"].cpu().numpy(), pos, G, DI,
                                       rope, THETA, EPS)
    _check(q_idx, rq, out_dtype, f"{what} q_idx")
    has_key = pos >= 0
    key_rows = (kstart + pos)[has_key]
    _check(k_idx[torch.as_tensor(key_rows, device="cuda")], rk[has_key], out_dtype, f"{what} k_idx rows")
    mask = torch.ones(k_idx.shape[0], dtype=torch.bool, device="cuda")
    mask[torch.as_tensor(key_rows, device="cuda")] = False
    assert torch.equal(k_idx[mask], before[mask]), f"{what}: rows other than the new tokens' keys changed"
    return q_idx, k_idx


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_frontend_measured_config(msa, synth, oracle_lib, out_dtype):
    """d_model 3072, 4 index-query heads + 1 key head of 128 dims, rotary
    width 64; two packed sequences (the second a chunk of a longer one) and a
    ragged tail (1,300 tokens: five workgroups of 256, the last partial)."""
    say(f"[frontend] measured config out={out_dtype}")
    _run(msa, synth, oracle_lib, [1000, 300], [1000, 2500], out_dtype=out_dtype, seed=1, what="measured")


@pytest.mark.parametrize("rope", [0, 128])
def test_frontend_rotary_widths(msa, synth, oracle_lib, rope):
    say(f"[frontend] rope_dim {rope}")
    _run(msa, synth, oracle_lib, [513], [513], rope=rope, seed=2, what=f"rope {rope}")


def test_frontend_fp32_small_index_dim(msa, synth, oracle_lib):
    """fp32 hidden states and weights (fp32 MFMAs), d_idx 64, 2 groups."""
    say("[frontend] fp32, d_idx 64")
    _run(msa, synth, oracle_lib, [700], [700], G=2, DI=64, d_model=256, dtype=torch.float32, seed=3,
         what="fp32 di64")


def test_frontend_decode_append_at_long_positions(msa, synth, oracle_lib):
    """One new token per sequence (q_len 1) at positions up to 2^20 + 5: the
    key row is appended at cu_seqlens_k[b] + ctx - 1, the rotation angles
    reach 10^6 radians (quarter-turn reduction in fp64)."""
    ctx = [1, 129, 4000, 65536, (1 << 20) + 6]
    say(f"[frontend] decode append ctx={ctx}")
    _run(msa, synth, oracle_lib, [1] * len(ctx), ctx, seed=4, what="decode")


def test_frontend_tokens_before_sequence_start(msa, synth, oracle_lib):
    """q_len > kv_len: the first tokens sit at p < 0, get their query heads
    (angle p * freq) and write no key row; an empty sequence in between."""
    say("[frontend] p < 0 and empty sequence")
    _run(msa, synth, oracle_lib, [40, 0, 200], [30, 50, 200], seed=5, what="p<0")


def test_frontend_is_deterministic(msa, synth):
    inp = synth.frontend_inputs(600, device="cuda", seed=6)
    cu = torch.tensor([0, 600], dtype=torch.int32, device="cuda")
    a = msa.msa_index_frontend(inp["x"], inp["w_q"], inp["w_k"], inp["gain_q"], inp["gain_k"], cu, cu, 4)
    b = msa.msa_index_frontend(inp["x"], inp["w_q"], inp["w_k"], inp["gain_q"], inp["gain_k"], cu, cu, 4)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_frontend_feeds_index_topk(msa, synth):
    """End to end on the GPU: the front-end's bf16 heads go straight into the
    selection call (shapes and types line up; ids valid and ascending with the
    local block present)."""
    T = 1024
    inp = synth.frontend_inputs(T, device="cuda", seed=7)
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    q_idx, k_idx = msa.msa_index_frontend(inp["x"], inp["w_q"], inp["w_k"], inp["gain_q"], inp["gain_k"], cu, cu, 4)
    ids = msa.msa_index_topk(q_idx, k_idx, cu, cu, T, T, 128, 16)
    torch.cuda.synchronize()
    ids = ids.cpu()
    local = torch.arange(T) // 128
    for g in range(4):
        sel = ids[:, g]
        assert bool((sel == local[:, None]).any(dim=1).all())
        valid = sel >= 0
        assert bool(((sel <= local[:, None]) | ~valid).all())
        assert valid.sum(dim=1).equal(torch.clamp(local + 1, max=16))


# ---------------------------------------------------------------- backward
# The GPU recomputes y in fp32 from bf16 x and W, forms dy in fp32, rounds it
# to bf16 (relative 2^-9) and accumulates dW = dy^T x in fp32 on MFMAs; the
# gain gradients stay fp32 throughout.  dW: relative RMS <= 1e-2 and max |err|
# <= 2e-2 * max |ref| (the bf16 bounds of the other backward); gains: relative
# RMS <= 1e-3.

def _bwd_run(msa, synth, oracle_lib, q_lens, kv_lens, *, G=4, DI=128, d_model=3072, rope=64, seed=0, what=""):
    T = int(sum(q_lens))
    cu_q, cu_k = _cu(q_lens), _cu(kv_lens)
    inp = synth.frontend_inputs(T, G, DI, d_model, torch.bfloat16, "cuda", seed)
    cuq_d = torch.tensor(cu_q, dtype=torch.int32, device="cuda")
    cuk_d = torch.tensor(cu_k, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + seed)
    dq = torch.randn((T, G, DI), generator=g, device="cuda", dtype=torch.float32)
    dk = torch.randn((int(cu_k[-1]), DI), generator=g, device="cuda", dtype=torch.float32)
    got = msa.msa_index_frontend_backward(inp["x"], inp["w_q"], inp["w_k"], inp["gain_q"], inp["gain_k"], cuq_d,
                                          cuk_d, G, dq, dk, rope_dim=rope, rope_theta=THETA, norm_eps=EPS)
    torch.cuda.synchronize()
    rows, kstart, pos = oracle_lib.rows_prefill(cu_q, cu_k)
    n_k = (cu_k[1:] - cu_k[:-1])[np.searchsorted(cu_q, rows, side="right") - 1]
    has_key = (pos >= 0) & (pos < n_k)
    dk_tok = np.zeros((T, DI))
    dk_host = dk.cpu().double().numpy()
    dk_tok[has_key] = dk_host[(kstart + pos)[has_key]]
    ref = oracle_lib.index_frontend_bwd(host(inp["x"]), host(inp["w_q"]), host(inp["w_k"]),
                                        inp["gain_q"].cpu().numpy(), inp["gain_k"].cpu().numpy(), pos, G, DI, rope,
                                        THETA, EPS, dq.cpu().double().numpy(), dk_tok)
    for name, gg, r in zip(("dw_q", "dw_k", "dgain_q", "dgain_k"), got, ref):
        gv = gg.cpu().double().numpy()
        err = np.abs(gv - r)
        rel = float(np.sqrt((err ** 2).sum() / max((r ** 2).sum(), 1e-300)))
        mx = float(err.max())
        say(f"    {what} {name}: rel-RMS {rel:.2e}, max-abs {mx:.2e} (max |ref| {np.abs(r).max():.3g})")
        if name.startswith("dw"):
            assert rel <= 1e-2 and mx <= 2e-2 * float(np.abs(r).max()), f"{what} {name}"
        else:
            assert rel <= 1e-3, f"{what} {name}"
    return got


def test_frontend_backward_measured_config(msa, synth, oracle_lib):
    """d_model 3072, 4 + 1 heads of 128 dims, rotary width 64; two packed
    sequences (the second a chunk), a ragged tail."""
    say("[frontend bwd] measured config")
    _bwd_run(msa, synth, oracle_lib, [1000, 300], [1000, 2500], seed=11, what="bwd")


def test_frontend_backward_rope128_and_missing_keys(msa, synth, oracle_lib):
    """Rotary width 128; tokens at p < 0 (no key row) and an empty sequence."""
    say("[frontend bwd] rope 128, p < 0")
    _bwd_run(msa, synth, oracle_lib, [40, 0, 300], [30, 50, 300], rope=128, seed=12, what="bwd rope128")


def test_frontend_backward_small_index_dim(msa, synth, oracle_lib):
    """d_idx 64 with 2 groups: 192 projection rows (a partial 128-row tile of
    the weight-gradient GEMM), d_model 256."""
    say("[frontend bwd] d_idx 64")
    _bwd_run(msa, synth, oracle_lib, [700], [700], G=2, DI=64, d_model=256, seed=13, what="bwd di64")


def test_frontend_backward_deterministic_and_empty(msa, synth):
    inp = synth.frontend_inputs(900, device="cuda", seed=14)
    cu = torch.tensor([0, 900], dtype=torch.int32, device="cuda")
    dq = torch.randn((900, 4, 128), device="cuda")
    dk = torch.randn((900, 128), device="cuda")
    a = msa.msa_index_frontend_backward(inp["x"], inp["w_q"], inp["w_k"], inp["gain_q"], inp["gain_k"], cu, cu, 4,
                                        dq, dk)
    b = msa.msa_index_frontend_backward(inp["x"], inp["w_q"], inp["w_k"], inp["gain_q"], inp["gain_k"], cu, cu, 4,
                                        dq, dk)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    # no tokens: every gradient is exactly zero
    cu0 = torch.tensor([0, 0], dtype=torch.int32, device="cuda")
    z = msa.msa_index_frontend_backward(inp["x"][:0], inp["w_q"], inp["w_k"], inp["gain_q"], inp["gain_k"], cu0, cu0,
                                        4, dq[:0], dk)
    torch.cuda.synchronize()
    assert all(bool((t == 0).all()) for t in z)


# ------------------------------------------------------- full size (128K)
def test_frontend_full_128k_sampled(msa, synth, oracle_lib):
    """The bench's call: 131,072 tokens, d_model 3072, bf16 out.  Sampled rows
    (the first and last 256-token tiles and 512 random tokens) against the
    oracle on exactly those rows and positions."""
    L = 131072
    say("[frontend] 128K tokens, sampled rows")
    inp = synth.frontend_inputs(L, device="cuda", seed=21)
    cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
    q_idx, k_idx = msa.msa_index_frontend(inp["x"], inp["w_q"], inp["w_k"], inp["gain_q"], inp["gain_k"], cu, cu, 4,
                                          rope_theta=THETA, norm_eps=EPS)
    torch.cuda.synchronize()
    rng = np.random.default_rng(21)
    rows = np.unique(np.concatenate([np.arange(256), np.arange(L - 256, L), rng.integers(0, L, 512)]))
    ridx = torch.as_tensor(rows, device="cuda")
    rq, rk = oracle_lib.index_frontend(host(inp["x"][ridx]), host(inp["w_q"]), host(inp["w_k"]),
                                       inp["gain_q"].cpu().numpy(), inp["gain_k"].cpu().numpy(), rows, 4, 128, 64,
                                       THETA, EPS)
    _check(q_idx[ridx], rq, torch.bfloat16, "128K q_idx")
    _check(k_idx[ridx], rk, torch.bfloat16, "128K k_idx")


def test_frontend_backward_full_128k_sampled(msa, synth, oracle_lib):
    """The bench's backward call over 131,072 tokens with the upstream
    gradients zero except on 384 sampled tokens: the parameter gradients are
    then exactly those of the sampled tokens, which the oracle computes."""
    L = 131072
    say("[frontend bwd] 128K tokens, sampled upstream gradients")
    inp = synth.frontend_inputs(L, device="cuda", seed=22)
    cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(22)
    rows = np.unique(np.concatenate([np.arange(128), np.arange(L - 128, L), rng.integers(0, L, 128)]))
    ridx = torch.as_tensor(rows, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(22)
    dq = torch.zeros((L, 4, 128), device="cuda")
    dk = torch.zeros((L, 128), device="cuda")
    dq[ridx] = torch.randn((len(rows), 4, 128), generator=g, device="cuda")
    dk[ridx] = torch.randn((len(rows), 128), generator=g, device="cuda")
    got = msa.msa_index_frontend_backward(inp["x"], inp["w_q"], inp["w_k"], inp["gain_q"], inp["gain_k"], cu, cu, 4,
                                          dq, dk, rope_theta=THETA, norm_eps=EPS)
    torch.cuda.synchronize()
    ref = oracle_lib.index_frontend_bwd(host(inp["x"][ridx]), host(inp["w_q"]), host(inp["w_k"]),
                                        inp["gain_q"].cpu().numpy(), inp["gain_k"].cpu().numpy(), rows, 4, 128, 64,
                                        THETA, EPS, dq[ridx].cpu().double().numpy(), dk[ridx].cpu().double().numpy())
    for name, gg, r in zip(("dw_q", "dw_k", "dgain_q", "dgain_k"), got, ref):
        gv = gg.cpu().double().numpy()
        err = np.abs(gv - r)
        rel = float(np.sqrt((err ** 2).sum() / max((r ** 2).sum(), 1e-300)))
        say(f"    128K {name}: rel-RMS {rel:.2e}, max-abs {float(err.max()):.2e} (max |ref| {np.abs(r).max():.3g})")
        if name.startswith("dw"):
            assert rel <= 1e-2 and float(err.max()) <= 2e-2 * float(np.abs(r).max()), name
        else:
            assert rel <= 1e-3, name
