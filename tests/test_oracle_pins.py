"""Pins for the CPU oracle, independent of the oracle's own code.

Each test checks the oracle against something the pages or the mathematics
fix, chosen so that a plausible slip in the oracle (a wrong causal bound, a
dropped local block, a reversed tie-break, a wrong head-to-group map, a
transposed operand, a missing scale) fails at least one of them:

* block selection vs brute force on integer-exact scores (tiny inputs, several
  block sizes, k values, varlen and bottom-right-aligned chunks, tie-dense data);
* a selection certificate on a medium input with the measured head config;
* attention vs dense causal GQA attention (torch SDPA, fp64) when every causal
  block fits in the budget: the pages' dense "escape hatch" equals MSA then;
* attention vs a dense boolean-mask formulation for arbitrary selections;
* closed forms: K == 0 gives the mean of V over the attended keys with
  lse = ln |J|; a single dominant key gives that key's value row; per-group
  constant values expose the head-to-group map.
"""
import math

import numpy as np
import pytest
import torch


def _grid(rng, shape, lo=-16, hi=16):
    """Integer grid values u (the data is u / 8)."""
    return rng.integers(lo, hi + 1, size=shape).astype(np.int64)


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def _brute_selection(uq, uk, cu_q, cu_k, bk, topk):
    """Block selection from integer scores (64 x the real scores), by sorting."""
    nrows, G, _ = uq.shape
    out = np.full((nrows, G, topk), -1, dtype=np.int64)
    pooled = {}
    for b in range(len(cu_q) - 1):
        m = cu_q[b + 1] - cu_q[b]
        n = cu_k[b + 1] - cu_k[b]
        keys = uk[cu_k[b]:cu_k[b + 1]]
        for t in range(m):
            row = cu_q[b] + t
            p = n - m + t
            local = p // bk
            for g in range(G):
                tok = keys[: local * bk] @ uq[row, g]          # all token scores
                S = [int(tok[c * bk:(c + 1) * bk].max()) for c in range(local)]
                order = sorted(range(local), key=lambda c: (-S[c], c))
                chosen = sorted(order[: topk - 1] + [local])
                out[row, g, :len(chosen)] = chosen
                pooled[(row, g)] = S
    return out, pooled


CASES = [
    # (seq kv lens, q lens, G, DI, Bk, topk, lo, hi)
    ([37], [37], 1, 4, 4, 1, -16, 16),
    ([64], [64], 2, 8, 8, 2, -16, 16),
    ([130, 77], [130, 77], 2, 4, 8, 4, -16, 16),
    ([300], [45], 2, 8, 8, 4, -16, 16),        # bottom-right aligned chunk
    ([257, 100, 129], [1, 100, 2], 1, 4, 4, 4, -16, 16),
    ([200], [200], 2, 4, 4, 4, -1, 1),        # tie-dense: values in {-1/8, 0, 1/8}
    ([160], [160], 1, 2, 8, 3, 0, 0),         # all scores equal: pure tie-break
    ([512], [512], 2, 8, 128, 4, -16, 16),    # production block size
    ([383], [129], 2, 8, 128, 2, -1, 1),
]


@pytest.mark.parametrize("case", CASES)
def test_selection_matches_bruteforce(oracle_lib, case):
    kv, ql, G, DI, bk, topk, lo, hi = case
    rng = np.random.default_rng(len(kv) * 1000 + sum(kv) + topk)
    cu_k, cu_q = _cu(kv), _cu(ql)
    uq = _grid(rng, (cu_q[-1], G, DI), lo, hi)
    uk = _grid(rng, (cu_k[-1], DI), lo, hi)
    want, pooled = _brute_selection(uq, uk, cu_q, cu_k, bk, topk)

    rows, kstart, pos = oracle_lib.rows_prefill(cu_q, cu_k)
    sel, scores = oracle_lib.index_topk((uq / 8).astype(np.float32), (uk / 8).astype(np.float32),
                                        kstart, pos, rows, bk, topk, return_scores=True)
    np.testing.assert_array_equal(sel, want)
    # the oracle's fp32 pooled scores are exact: 64 x score == integer score
    for (row, g), S in pooled.items():
        got = scores[row, g, :len(S)].astype(np.float64) * 64.0
        np.testing.assert_array_equal(got, np.asarray(S, dtype=np.float64))
        assert np.all(np.isneginf(scores[row, g, len(S):]))


def test_selection_bf16_inputs_equal_fp32(oracle_lib):
    """bf16 bit patterns widen exactly: same selection as the fp32 copy."""
    rng = np.random.default_rng(7)
    cu = _cu([700])
    uq = _grid(rng, (700, 2, 16))
    uk = _grid(rng, (700, 16))
    qf = torch.from_numpy((uq / 8).astype(np.float32))
    kf = torch.from_numpy((uk / 8).astype(np.float32))
    rows, kstart, pos = oracle_lib.rows_prefill(cu, cu)
    a = oracle_lib.index_topk(qf, kf, kstart, pos, rows, 8, 5)
    b = oracle_lib.index_topk(qf.bfloat16(), kf.bfloat16(), kstart, pos, rows, 8, 5)
    np.testing.assert_array_equal(a, b)


def test_selection_certificate_measured_config(oracle_lib):
    """Certificate per (row, group) on 64/4 heads, d_idx 128, block 128, k 16.

    Integer-valued fp64 matmul gives exact block scores independently of the
    oracle; the certificate is: local block present, count = min(k, l + 1),
    ids distinct, ascending and <= l, and the worst selected earlier block
    precedes the best unselected one in the order (score desc, id asc)."""
    from learned_block_sparse_amd import synth
    wl = synth.WORKLOADS["prefill_32k"]
    L, topk, bk = 4096 + 37, wl.topk, wl.block_size
    inp = synth.prefill_inputs(wl, seq_lens=[L], with_main=False, seed=3)
    cu = inp["cu_q_host"]
    rows, kstart, pos = oracle_lib.rows_prefill(cu, cu)
    sel = oracle_lib.index_topk(inp["q_idx"], inp["k_idx"], kstart, pos, rows, bk, topk)

    qd = inp["q_idx"].double().numpy() * 8.0    # integer-valued
    kd = inp["k_idx"].double().numpy() * 8.0
    nb = (L + bk - 1) // bk
    G = qd.shape[1]
    ties = 0
    for g in range(G):
        tok = qd[:, g, :] @ kd.T                       # exact: integers < 2**53
        full = tok[:, : (nb - 1) * bk].reshape(L, nb - 1, bk).max(axis=2)
        for t in range(L):
            local = t // bk
            s = sel[t, g]
            ids = s[s >= 0]
            assert local in ids
            assert len(ids) == min(topk, local + 1)
            assert np.all(np.diff(ids) > 0) and ids.max() == local
            assert np.all(s[len(ids):] == -1)
            earlier = [c for c in ids if c != local]
            rest = sorted(set(range(local)) - set(earlier))
            if earlier and rest:
                worst = min(earlier, key=lambda c: (full[t, c], -c))
                best = max(rest, key=lambda c: (full[t, c], -c))
                assert (full[t, worst], -worst) > (full[t, best], -best)
                ties += full[t, worst] == full[t, best]
    assert ties > 0, "expected ties at the selection boundary on grid data"


def _dense_reference(q, k, v, cu_q, cu_k, scale):
    """Dense causal GQA attention in fp64 with torch SDPA (bottom-right causal)."""
    outs, lses = [], []
    Hq, Hkv = q.shape[1], k.shape[1]
    rep = Hq // Hkv
    for b in range(len(cu_q) - 1):
        m, n = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        qb = q[cu_q[b]:cu_q[b + 1]].double().permute(1, 0, 2)[None]
        kb = k[cu_k[b]:cu_k[b + 1]].double().repeat_interleave(rep, dim=1).permute(1, 0, 2)[None]
        vb = v[cu_k[b]:cu_k[b + 1]].double().repeat_interleave(rep, dim=1).permute(1, 0, 2)[None]
        t = torch.arange(m)[:, None]
        j = torch.arange(n)[None, :]
        allow = j <= (n - m + t)
        o = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=allow,
                                                             scale=scale)
        z = (qb @ kb.transpose(-1, -2)) * scale
        z = z.masked_fill(~allow, float("-inf"))
        outs.append(o[0].permute(1, 0, 2))
        lses.append(torch.logsumexp(z, dim=-1)[0].permute(1, 0))
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


@pytest.mark.parametrize("kv,ql,Hq,Hkv,D,bk,topk", [
    ([512], [512], 8, 2, 32, 128, 4),
    ([300, 41], [300, 41], 4, 1, 16, 64, 5),
    ([511], [77], 16, 4, 64, 128, 4),
    ([96], [96], 6, 3, 8, 8, 12),
])
def test_attention_equals_dense_when_all_blocks_fit(oracle_lib, kv, ql, Hq, Hkv, D, bk, topk):
    g = torch.Generator().manual_seed(11)
    cu_k, cu_q = _cu(kv), _cu(ql)
    assert max(kv) <= topk * bk
    q = torch.randn(cu_q[-1], Hq, D, generator=g)
    k = torch.randn(cu_k[-1], Hkv, D, generator=g)
    v = torch.randn(cu_k[-1], Hkv, D, generator=g)
    qi = torch.randint(-16, 17, (cu_q[-1], Hkv, 8), generator=g).float() / 8
    ki = torch.randint(-16, 17, (cu_k[-1], 8), generator=g).float() / 8
    scale = 1.0 / math.sqrt(D)
    sel, out, lse = oracle_lib.prefill(qi, ki, q, k, v, cu_q, cu_k, bk, topk)
    ref_o, ref_l = _dense_reference(q, k, v, cu_q, cu_k, scale)
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)


def test_attention_matches_mask_formulation(oracle_lib):
    """Arbitrary selections (duplicates, future and missing local blocks
    included) against a dense boolean-mask softmax written independently."""
    rng = np.random.default_rng(5)
    kv, ql, Hq, Hkv, D, bk, topk = [333, 200], [120, 200], 6, 2, 16, 16, 4
    cu_k, cu_q = _cu(kv), _cu(ql)
    q = rng.standard_normal((cu_q[-1], Hq, D)).astype(np.float32)
    k = rng.standard_normal((cu_k[-1], Hkv, D)).astype(np.float32)
    v = rng.standard_normal((cu_k[-1], Hkv, D)).astype(np.float32)
    rows, kstart, pos = oracle_lib.rows_prefill(cu_q, cu_k)
    sel = rng.integers(-1, 25, size=(len(rows), Hkv, topk)).astype(np.int32)
    for r in range(len(rows)):     # keep at least the local block in most rows
        if r % 3:
            sel[r, :, 0] = pos[r] // bk
    out, lse = oracle_lib.sparse_attn(q, k, v, sel, kstart, pos, rows, bk, topk)
    scale = 1.0 / math.sqrt(D)
    for r in range(len(rows)):
        b = int(np.searchsorted(cu_q, rows[r], side="right") - 1)
        n = cu_k[b + 1] - cu_k[b]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            j = np.arange(n)
            mask = np.isin(j // bk, sel[r, g]) & (j <= pos[r])
            kk = k[cu_k[b]:cu_k[b + 1], g].astype(np.float64)
            vv = v[cu_k[b]:cu_k[b + 1], g].astype(np.float64)
            z = kk @ q[rows[r], h].astype(np.float64) * scale
            if not mask.any():
                assert np.isneginf(lse[r, h]) and np.all(out[r, h] == 0)
                continue
            z = np.where(mask, z, -np.inf)
            w = np.exp(z - z.max())
            np.testing.assert_allclose(out[r, h], (w / w.sum()) @ vv, atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[r, h], z.max() + np.log(w.sum()), atol=1e-12, rtol=0)


def test_zero_keys_give_mean_of_values(oracle_lib):
    """K == 0: every logit is 0, so o = mean of v over J and lse = ln |J|.
    |J| is counted here from the selection and the causal bound alone."""
    rng = np.random.default_rng(9)
    kv, ql, Hq, Hkv, D, bk, topk = [1000], [390], 4, 2, 8, 32, 5
    cu_k, cu_q = _cu(kv), _cu(ql)
    q = rng.standard_normal((cu_q[-1], Hq, D)).astype(np.float32)
    k = np.zeros((cu_k[-1], Hkv, D), dtype=np.float32)
    v = rng.standard_normal((cu_k[-1], Hkv, D)).astype(np.float32)
    qi = (_grid(rng, (cu_q[-1], Hkv, 4)) / 8).astype(np.float32)
    ki = (_grid(rng, (cu_k[-1], 4)) / 8).astype(np.float32)
    sel, out, lse = oracle_lib.prefill(qi, ki, q, k, v, cu_q, cu_k, bk, topk)
    rows, kstart, pos = oracle_lib.rows_prefill(cu_q, cu_k)
    for r in range(len(rows)):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            blocks = sel[r, g][sel[r, g] >= 0]
            keys = [j for c in blocks for j in range(c * bk, (c + 1) * bk) if j <= pos[r]]
            expect_n = sum(min(bk, pos[r] - c * bk + 1) for c in blocks)
            assert len(keys) == expect_n
            np.testing.assert_allclose(lse[r, h], math.log(expect_n), atol=1e-12, rtol=0)
            np.testing.assert_allclose(out[r, h], v[keys, g].astype(np.float64).mean(0),
                                       atol=1e-12, rtol=0)


def test_dominant_key_selects_its_value_row(oracle_lib):
    """One key aligned with the query dominates the softmax: o == v of that
    key's row and KV head (pins the value gather and the head-to-group map)."""
    rng = np.random.default_rng(13)
    N, Hq, Hkv, D, bk, topk = 256, 4, 2, 16, 16, 3
    cu = _cu([N])
    q = (0.01 * rng.standard_normal((N, Hq, D))).astype(np.float32)
    k = (0.01 * rng.standard_normal((N, Hkv, D))).astype(np.float32)
    v = rng.standard_normal((N, Hkv, D)).astype(np.float32)
    t = N - 1
    q[t, :, 0] = 30.0
    star = 250                                   # inside the local block of t
    k[star, :, 0] = 30.0
    qi = np.zeros((N, Hkv, 2), dtype=np.float32)
    ki = np.zeros((N, 2), dtype=np.float32)
    sel, out, lse = oracle_lib.prefill(qi, ki, q, k, v, cu, cu, bk, topk, rows=[t])
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], v[star, h // (Hq // Hkv)], atol=1e-9, rtol=0)


def test_head_to_group_map(oracle_lib):
    """Per-KV-head constant values: head h reads group h // (Hq / Hkv)."""
    rng = np.random.default_rng(17)
    N, Hq, Hkv, D, bk, topk = 64, 8, 4, 8, 8, 2
    cu = _cu([N])
    q = rng.standard_normal((N, Hq, D)).astype(np.float32)
    k = rng.standard_normal((N, Hkv, D)).astype(np.float32)
    v = np.zeros((N, Hkv, D), dtype=np.float32)
    for g in range(Hkv):
        v[:, g, :] = g + 1.0
    qi = (_grid(rng, (N, Hkv, 4)) / 8).astype(np.float32)
    ki = (_grid(rng, (N, 4)) / 8).astype(np.float32)
    _, out, _ = oracle_lib.prefill(qi, ki, q, k, v, cu, cu, bk, topk)
    for h in range(Hq):
        np.testing.assert_allclose(out[:, h], h // 2 + 1.0, atol=1e-12, rtol=0)


def test_empty_rows_and_negative_positions(oracle_lib):
    """q_len > kv_len leaves leading rows with p < 0: no keys, -1 ids, lse -inf."""
    rng = np.random.default_rng(19)
    cu_k, cu_q = _cu([3]), _cu([5])
    q = rng.standard_normal((5, 2, 4)).astype(np.float32)
    k = rng.standard_normal((3, 1, 4)).astype(np.float32)
    v = rng.standard_normal((3, 1, 4)).astype(np.float32)
    qi = np.ones((5, 1, 2), dtype=np.float32)
    ki = np.ones((3, 2), dtype=np.float32)
    sel, out, lse = oracle_lib.prefill(qi, ki, q, k, v, cu_q, cu_k, 2, 2)
    assert np.all(sel[:2] == -1) and np.all(np.isneginf(lse[:2])) and np.all(out[:2] == 0)
    assert np.all(np.isfinite(lse[2:]))


def test_e4m3_decoder(oracle_lib):
    """The oracle's E4M3 decoder against torch's float8_e4m3fn conversion on
    all 256 codes, and closed forms of the format (bias 7, 3 mantissa bits,
    subnormals, no infinity, S.1111.111 = NaN)."""
    codes = np.arange(256, dtype=np.uint8)
    got = oracle_lib.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(got)
    np.testing.assert_array_equal(got[ok], ref[ok])
    closed = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
              0x3C: 1.5, 0x7E: 448.0, 0x40: 2.0, 0x41: 2.25}
    for c, v in closed.items():
        assert got[c] == v, (hex(c), got[c], v)
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_fp8_grid_is_exact_and_selection_matches_bruteforce(oracle_lib):
    """Index inputs on the 1/8 grid (with the +1.0 planted bias) rounded to
    E4M3 stay multiples of 1/8, so fp32 scores remain exact: the oracle's
    selection on E4M3 inputs equals brute force on the integers 8 x value."""
    from learned_block_sparse_amd import synth
    wl = synth.WORKLOADS["prefill_32k"]
    inp = synth.prefill_inputs(wl, seq_lens=[1500], with_main=False, seed=5)
    q8 = inp["q_idx"].to(torch.float8_e4m3fn)
    k8 = inp["k_idx"].float().clone()
    k8[:256] += 1.0            # a planted pair of blocks, including values like 17/8
    k8 = k8.to(torch.float8_e4m3fn)
    uq = (q8.float().double().numpy() * 8.0)
    uk = (k8.float().double().numpy() * 8.0)
    assert np.all(uq == np.round(uq)) and np.all(uk == np.round(uk))
    cu = _cu([1500])
    want, _ = _brute_selection(uq.astype(np.int64), uk.astype(np.int64), cu, cu, wl.block_size, wl.topk)
    rows, kstart, pos = oracle_lib.rows_prefill(cu, cu)
    sel = oracle_lib.index_topk(q8, k8, kstart, pos, rows, wl.block_size, wl.topk)
    np.testing.assert_array_equal(sel, want)


@pytest.mark.parametrize("kv,ql", [([512], [512]), ([300, 41], [100, 41])])
def test_fp8_kv_attention_equals_dense(oracle_lib, kv, ql):
    """bf16 queries with an E4M3 KV cache: when every causal block fits the
    budget, the oracle equals dense causal GQA attention (torch SDPA, fp64) on
    the values torch's own float8_e4m3fn conversion gives for K and V."""
    g = torch.Generator().manual_seed(12)
    Hq, Hkv, D, bk, topk = 8, 2, 32, 128, 4
    cu_k, cu_q = _cu(kv), _cu(ql)
    q = torch.randn(cu_q[-1], Hq, D, generator=g).bfloat16()
    k8 = torch.randn(cu_k[-1], Hkv, D, generator=g).to(torch.float8_e4m3fn)
    v8 = (3 * torch.randn(cu_k[-1], Hkv, D, generator=g)).to(torch.float8_e4m3fn)
    qi = torch.randint(-16, 17, (cu_q[-1], Hkv, 8), generator=g).float() / 8
    ki = torch.randint(-16, 17, (cu_k[-1], 8), generator=g).float() / 8
    sel, out, lse = oracle_lib.prefill(qi, ki, q, k8, v8, cu_q, cu_k, bk, topk)
    ref_o, ref_l = _dense_reference(q.float(), k8.float(), v8.float(), cu_q, cu_k, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(out, ref_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-12)


def _masked_attention_torch(q, k, v, mask_rows, scale, Hkv):
    """Dense softmax attention with an explicit boolean mask per (row, group),
    written with torch ops so autograd gives its gradients."""
    n, Hq, D = q.shape
    rep = Hq // Hkv
    outs = []
    for r, (kk_idx, mask) in enumerate(mask_rows):
        heads = []
        for h in range(Hq):
            g = h // rep
            if not mask[g].any():
                heads.append(torch.zeros(D, dtype=q.dtype) + 0.0 * q[r, h].sum())
                continue
            kk = k[kk_idx, g]
            vv = v[kk_idx, g]
            z = (kk @ q[r, h]) * scale
            z = z.masked_fill(~mask[g], float("-inf"))
            heads.append(torch.softmax(z, dim=0) @ vv)
        outs.append(torch.stack(heads))
    return torch.stack(outs)


def test_backward_matches_autograd_of_mask_formulation(oracle_lib):
    """dq, dk, dv of the oracle against torch autograd (fp64) through a dense
    boolean-mask softmax, for arbitrary selections (duplicates, -1, future
    blocks, missing local blocks) over two packed sequences."""
    rng = np.random.default_rng(21)
    kv, ql, Hq, Hkv, D, bk, topk = [150, 90], [60, 90], 4, 2, 8, 16, 4
    cu_k, cu_q = _cu(kv), _cu(ql)
    q = rng.standard_normal((cu_q[-1], Hq, D)).astype(np.float32)
    k = rng.standard_normal((cu_k[-1], Hkv, D)).astype(np.float32)
    v = rng.standard_normal((cu_k[-1], Hkv, D)).astype(np.float32)
    do = rng.standard_normal((cu_q[-1], Hq, D)).astype(np.float32)
    rows, kstart, pos = oracle_lib.rows_prefill(cu_q, cu_k)
    sel = rng.integers(-1, 11, size=(len(rows), Hkv, topk)).astype(np.int32)
    for r in range(len(rows)):
        if r % 4:
            sel[r, :, 0] = pos[r] // bk
    dq, dk, dv = oracle_lib.sparse_attn_bwd(q, k, v, do, sel, kstart, pos, rows, bk, topk)

    qt = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    kt = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    vt = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    mask_rows = []
    for r in range(len(rows)):
        b = int(np.searchsorted(cu_q, rows[r], side="right") - 1)
        n = cu_k[b + 1] - cu_k[b]
        j = np.arange(n)
        idx = torch.tensor(cu_k[b] + j)
        mask = torch.tensor(np.stack([np.isin(j // bk, sel[r, g]) & (j <= pos[r]) for g in range(Hkv)]))
        mask_rows.append((idx, mask))
    out = _masked_attention_torch(qt, kt, vt, mask_rows, 1.0 / math.sqrt(D), Hkv)
    (out * torch.tensor(do, dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, vt.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_matches_finite_differences(oracle_lib):
    """Central differences of L = sum(dO * out) through the oracle's own
    forward pass (fp64 inside), at a few coordinates of q, k and v, including
    keys in the causal partial local block."""
    rng = np.random.default_rng(22)
    kv, ql, Hq, Hkv, D, bk, topk = [70], [70], 4, 2, 8, 16, 3
    cu_k, cu_q = _cu(kv), _cu(ql)
    q = rng.standard_normal((70, Hq, D)).astype(np.float32)
    k = rng.standard_normal((70, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((70, Hkv, D)).astype(np.float32)
    do = rng.standard_normal((70, Hq, D)).astype(np.float32)
    rows, kstart, pos = oracle_lib.rows_prefill(cu_q, cu_k)
    sel = np.full((70, Hkv, topk), -1, dtype=np.int32)
    for r in range(70):
        loc = pos[r] // bk
        sel[r, 0, :2] = [loc, (loc + 2) // 2 - 1 if loc else -1]
        sel[r, 1, :3] = [0, loc, max(loc - 1, 0)]
    dq, dk, dv = oracle_lib.sparse_attn_bwd(q, k, v, do, sel, kstart, pos, rows, bk, topk)

    def loss(qq, kk, vv):
        out, _ = oracle_lib.sparse_attn(qq, kk, vv, sel, kstart, pos, rows, bk, topk)
        return float((out * do.astype(np.float64)).sum())

    eps = 2.0 ** -10
    for name, arr, grad, coords in (("q", q, dq, [(5, 1, 3), (69, 3, 0), (40, 2, 7)]),
                                    ("k", k, dk, [(0, 1, 2), (33, 0, 5), (66, 1, 1)]),
                                    ("v", v, dv, [(17, 0, 4), (64, 1, 6), (2, 1, 0)])):
        for c in coords:
            plus, minus = arr.copy(), arr.copy()
            plus[c] += eps
            minus[c] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = plus, minus
            fd = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
            assert abs(fd - grad[c]) <= 1e-5 * max(1.0, abs(grad[c])), (name, c, fd, grad[c])


def _kl_case(rng, kv, ql, Hq, Hkv, D, DI, bk, topk, zero_k=False, zero_qidx=False):
    cu_k, cu_q = _cu(kv), _cu(ql)
    q = rng.standard_normal((cu_q[-1], Hq, D)).astype(np.float32)
    k = np.zeros((cu_k[-1], Hkv, D), np.float32) if zero_k else rng.standard_normal((cu_k[-1], Hkv, D)).astype(np.float32)
    qi = np.zeros((cu_q[-1], Hkv, DI), np.float32) if zero_qidx else rng.standard_normal((cu_q[-1], Hkv, DI)).astype(np.float32)
    ki = rng.standard_normal((cu_k[-1], DI)).astype(np.float32)
    return cu_k, cu_q, q, k, qi, ki


def _attended(sel_row, p, bk):
    """Distinct attended blocks of a selection row, in slot order (Sel as a set)."""
    seen, out = set(), []
    for i, c in enumerate(sel_row):
        if c >= 0 and c <= p // bk and c not in seen:
            seen.add(c)
            out.append((i, int(c)))
    return out


def test_block_lse_closed_form_and_consistency(oracle_lib):
    """K == 0: every logit is 0, so a block's LSE is ln(number of its attended
    keys) (128 for a full block, p - 128 l + 1 for the local one).  With random
    K the logsumexp over a row's slots is the attention's own LSE."""
    rng = np.random.default_rng(31)
    kv, ql, Hq, Hkv, D, bk, topk = [700, 260], [300, 260], 4, 2, 16, 128, 4
    cu_k, cu_q, q, k, _, _ = _kl_case(rng, kv, ql, Hq, Hkv, D, 8, bk, topk, zero_k=True)
    rows, kstart, pos = oracle_lib.rows_prefill(cu_q, cu_k)
    sel = rng.integers(-1, 6, size=(len(rows), Hkv, topk)).astype(np.int32)
    sel[:, :, 0] = (pos // bk)[:, None]
    bl = oracle_lib.block_lse(q, k, sel, kstart, pos, rows, bk, topk)
    for r in range(len(rows)):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            att = dict(_attended(sel[r, g], pos[r], bk))
            for i in range(topk):
                if i in att:
                    c = att[i]
                    nk = min(bk, pos[r] - c * bk + 1)
                    assert bl[r, h, i] == pytest.approx(math.log(nk), abs=1e-12)
                else:
                    assert np.isneginf(bl[r, h, i])
    k = rng.standard_normal(k.shape).astype(np.float32)
    bl = oracle_lib.block_lse(q, k, sel, kstart, pos, rows, bk, topk)
    _, lse = oracle_lib.sparse_attn(q, k, k, sel, kstart, pos, rows, bk, topk)
    m = bl.max(axis=-1, keepdims=True)
    np.testing.assert_allclose(m[..., 0] + np.log(np.exp(bl - m).sum(-1)), lse, rtol=0, atol=1e-12)


def test_index_kl_closed_form(oracle_lib):
    """K == 0 makes the main attention uniform over the attended keys, so the
    target share of block c is n_c / |J|; q_idx == 0 makes every index score 0,
    so the index distribution is uniform over the m attended blocks and every
    argmax is the block's first key.  Then loss = sum_c (n_c/|J|) ln(m n_c/|J|),
    dS_c = 1/m - n_c/|J|, dq_idx = sum_c dS_c k_idx[first key of c] and
    dk_idx[first key of c] = sum over rows of dS_c q_idx = 0."""
    rng = np.random.default_rng(32)
    kv, ql, Hq, Hkv, D, DI, bk, topk = [600], [600], 4, 2, 16, 8, 128, 4
    cu_k, cu_q, q, k, qi, ki = _kl_case(rng, kv, ql, Hq, Hkv, D, DI, bk, topk, zero_k=True, zero_qidx=True)
    rows, kstart, pos = oracle_lib.rows_prefill(cu_q, cu_k)
    sel = rng.integers(-1, 5, size=(len(rows), Hkv, topk)).astype(np.int32)
    sel[:, :, 1] = (pos // bk)[:, None]
    loss, dq, dk = oracle_lib.index_kl(qi, ki, q, k, sel, kstart, pos, rows, bk, topk)
    for r in range(len(rows)):
        for g in range(Hkv):
            att = _attended(sel[r, g], pos[r], bk)
            ns = np.array([min(bk, pos[r] - c * bk + 1) for _, c in att], dtype=np.float64)
            A, m = ns / ns.sum(), len(att)
            assert loss[r, g] == pytest.approx(float((A * np.log(m * A)).sum()), abs=1e-12)
            want = sum((1.0 / m - A[j]) * ki[c * bk].astype(np.float64) for j, (_, c) in enumerate(att))
            np.testing.assert_allclose(dq[r, g], want, rtol=0, atol=1e-12)
    assert np.all(dk == 0)
    assert np.all(loss >= -1e-12)


def test_index_kl_matches_finite_differences(oracle_lib):
    """Central differences of the summed loss through the oracle's own loss,
    at coordinates of q_idx and at the argmax keys of k_idx (random fp32 data:
    the maxima are unique, so the max is differentiable there)."""
    rng = np.random.default_rng(33)
    kv, ql, Hq, Hkv, D, DI, bk, topk = [300], [120], 4, 2, 8, 8, 32, 4
    cu_k, cu_q, q, k, qi, ki = _kl_case(rng, kv, ql, Hq, Hkv, D, DI, bk, topk)
    rows, kstart, pos = oracle_lib.rows_prefill(cu_q, cu_k)
    sel = rng.integers(0, 9, size=(len(rows), Hkv, topk)).astype(np.int32)
    sel[:, :, 0] = (pos // bk)[:, None]
    loss, dq, dk = oracle_lib.index_kl(qi, ki, q, k, sel, kstart, pos, rows, bk, topk)
    assert np.all(loss >= -1e-12)

    def total(qq, kk):
        return float(oracle_lib.index_kl(qq, kk, q, k, sel, kstart, pos, rows, bk, topk)[0].sum())

    # the index scores are fp32 (as the index branch computes them), so the
    # differences carry fp32 rounding of S: 1e-3 relative still fails any
    # wrong sign, factor or term
    eps = 2.0 ** -10
    for c in [(0, 0, 3), (57, 1, 0), (119, 0, 7)]:
        plus, minus = qi.copy(), qi.copy()
        plus[c] += eps
        minus[c] -= eps
        fd = (total(plus, ki) - total(minus, ki)) / (2 * eps)
        assert abs(fd - dq[c]) <= 1e-3 * max(1.0, abs(dq[c])), (c, fd, dq[c])
    rows_k = np.argsort(-np.abs(dk).sum(axis=1))[:3]
    for j in rows_k:
        for d in (0, DI - 1):
            plus, minus = ki.copy(), ki.copy()
            plus[j, d] += eps
            minus[j, d] -= eps
            fd = (total(qi, plus) - total(qi, minus)) / (2 * eps)
            assert abs(fd - dk[j, d]) <= 1e-3 * max(1.0, abs(dk[j, d])), (j, d, fd, dk[j, d])
