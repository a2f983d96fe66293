"""Pins for the oracle's decode step (``oracle.decode`` / ``oracle.rows_decode``).

A decode step appends one token per sequence; its K, V and index key are
already in the caches, so the query is the newest token of the context, at
position ctx - 1 ("llama.cpp Merges MiniMax M3's Sparse Attention", key facts:
the block the model is currently writing in is always kept; "MiniMax Sparse
Attention: let each query pick its own blocks", "The mechanism, precisely").

Checked against things fixed independently of the oracle's decode addressing:

* brute force from the integer index grid and a dense masked softmax over the
  sequence's own cache slice, at contexts 1, 127, 128, 129, 2049 and 3000;
* dense softmax over all ``ctx`` keys when every block fits the budget
  (``ctx <= k * 128``): MSA is dense attention there;
* the closed form for K = 0 and q_idx = 0: lse = ln |J| with
  |J| = ctx (all blocks fit) or 128 (k - 1) + (ctx - 1) % 128 + 1;
* the same rows through ``oracle.prefill`` with one query per sequence;
* a planted slip (position ctx instead of ctx - 1) fails the brute-force check.
"""
import math

import numpy as np
import pytest
import torch

BK = 128


def _caches(rng, ctx, G, DI, Hkv, D, gap=37):
    """Per-sequence caches packed with gaps of junk rows between sequences."""
    offs, total = [], 0
    for c in ctx:
        total += gap
        offs.append(total)
        total += c
    total += gap
    uk = rng.integers(-16, 17, size=(total, DI)).astype(np.int64)
    k = rng.standard_normal((total, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((total, Hkv, D)).astype(np.float32)
    uq = rng.integers(-16, 17, size=(len(ctx), G, DI)).astype(np.int64)
    return np.asarray(offs, dtype=np.int64), uk, k, v, uq


def _brute_decode(uq, uk, q, k, v, offs, ctx, topk, scale, Hq, Hkv):
    """Selection from integer scores and masked dense softmax, newest token."""
    B, G, _ = uq.shape
    sel = np.full((B, G, topk), -1, dtype=np.int64)
    out = np.zeros((B, Hq, q.shape[2]))
    lse = np.zeros((B, Hq))
    r = Hq // Hkv
    for b in range(B):
        n = int(ctx[b])
        keys = uk[offs[b]:offs[b] + n]
        p = n - 1                       # the new token is the context's last one
        local = p // BK
        for g in range(G):
            tok = keys[: local * BK] @ uq[b, g]
            S = [int(tok[c * BK:(c + 1) * BK].max()) for c in range(local)]
            order = sorted(range(local), key=lambda c: (-S[c], c))
            chosen = sorted(order[: topk - 1] + [local])
            sel[b, g, :len(chosen)] = chosen
        for h in range(Hq):
            g = h // r
            j = np.arange(n)
            mask = np.isin(j // BK, sel[b, g]) & (j <= p)
            z = k[offs[b]:offs[b] + n, g].astype(np.float64) @ q[b, h].astype(np.float64) * scale
            z = np.where(mask, z, -np.inf)
            w = np.exp(z - z.max())
            out[b, h] = (w / w.sum()) @ v[offs[b]:offs[b] + n, g].astype(np.float64)
            lse[b, h] = z.max() + np.log(w.sum())
    return sel, out, lse


def _check(got, want):
    sel, out, lse = got
    wsel, wout, wlse = want
    np.testing.assert_array_equal(np.asarray(sel, dtype=np.int64), wsel)
    np.testing.assert_allclose(out, wout, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, wlse, atol=1e-12, rtol=0)


CTX = [1, 127, 128, 129, 2049, 3000]


@pytest.mark.parametrize("topk", [4, 16])
def test_decode_matches_bruteforce(oracle_lib, topk):
    rng = np.random.default_rng(100 + topk)
    Hq, Hkv, D, DI = 4, 2, 16, 8
    offs, uk, k, v, uq = _caches(rng, CTX, Hkv, DI, Hkv, D)
    q = rng.standard_normal((len(CTX), Hq, D)).astype(np.float32)
    scale = 1.0 / math.sqrt(D)
    ctx = np.asarray(CTX, dtype=np.int64)
    want = _brute_decode(uq, uk, q, k, v, offs, ctx, topk, scale, Hq, Hkv)
    got = oracle_lib.decode((uq / 8).astype(np.float32), (uk / 8).astype(np.float32), q, k, v,
                            offs, ctx, BK, topk)
    _check(got, want)
    # the selections past the budget are real top-k choices, not all blocks
    assert (np.asarray(got[0])[-1] >= 0).sum() == Hkv * topk


def test_planted_position_slip_fails(oracle_lib):
    """The check above catches a decode position of ctx instead of ctx - 1."""
    rng = np.random.default_rng(7)
    Hq, Hkv, D, DI, topk = 4, 2, 16, 8, 4
    offs, uk, k, v, uq = _caches(rng, CTX, Hkv, DI, Hkv, D)
    q = rng.standard_normal((len(CTX), Hq, D)).astype(np.float32)
    ctx = np.asarray(CTX, dtype=np.int64)
    want = _brute_decode(uq, uk, q, k, v, offs, ctx, topk, 1.0 / math.sqrt(D), Hq, Hkv)
    rows = np.arange(len(CTX), dtype=np.int64)
    slip_pos = ctx.copy()                            # the planted mistake
    qi, ki = (uq / 8).astype(np.float32), (uk / 8).astype(np.float32)
    sel = oracle_lib.index_topk(qi, ki, offs, slip_pos, rows, BK, topk)
    out, lse = oracle_lib.sparse_attn(q, k, v, sel, offs, slip_pos, rows, BK, topk)
    with pytest.raises(AssertionError):
        _check((sel, out, lse), want)


def test_decode_equals_dense_when_all_blocks_fit(oracle_lib):
    """ctx <= k * 128: the step is plain softmax attention over all ctx keys."""
    rng = np.random.default_rng(3)
    Hq, Hkv, D, DI, topk = 6, 3, 8, 4, 8
    ctx = np.asarray([1, 127, 128, 129, 1024], dtype=np.int64)
    offs, uk, k, v, uq = _caches(rng, ctx, Hkv, DI, Hkv, D, gap=5)
    q = torch.from_numpy(rng.standard_normal((len(ctx), Hq, D)).astype(np.float32))
    sel, out, lse = oracle_lib.decode((uq / 8).astype(np.float32), (uk / 8).astype(np.float32), q,
                                      torch.from_numpy(k), torch.from_numpy(v), offs, ctx, BK, topk)
    q = q.double()
    for b, n in enumerate(ctx):
        kk = torch.from_numpy(k[offs[b]:offs[b] + n]).double().repeat_interleave(Hq // Hkv, dim=1)
        vv = torch.from_numpy(v[offs[b]:offs[b] + n]).double().repeat_interleave(Hq // Hkv, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[b][:, None, :], kk.permute(1, 0, 2), vv.permute(1, 0, 2))[:, 0, :]
        z = (kk.permute(1, 0, 2) @ q[b][:, :, None])[:, :, 0] / math.sqrt(D)
        np.testing.assert_allclose(out[b], ref.numpy(), atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse[b], torch.logsumexp(z, dim=-1).numpy(), atol=1e-12, rtol=0)
        nblk = (int(n) - 1) // BK + 1
        np.testing.assert_array_equal(sel[b, :, :nblk], np.tile(np.arange(nblk), (Hkv, 1)))


@pytest.mark.parametrize("topk", [1, 3, 16])
def test_decode_zero_keys_closed_form(oracle_lib, topk):
    """K = 0 and q_idx = 0: every score and logit ties, the lowest earlier
    blocks are taken, and lse = ln |J| counts the keys up to ctx - 1."""
    Hq, Hkv, D, DI = 2, 1, 4, 4
    ctx = np.asarray([1, 127, 128, 129, 2049, 2200], dtype=np.int64)
    offs = np.concatenate([[3], 3 + np.cumsum(ctx[:-1] + 3)]).astype(np.int64)
    total = int(offs[-1] + ctx[-1] + 3)
    k = np.zeros((total, Hkv, D), np.float32)
    v = np.random.default_rng(1).standard_normal((total, Hkv, D)).astype(np.float32)
    q = np.ones((len(ctx), Hq, D), np.float32)
    sel, out, lse = oracle_lib.decode(np.zeros((len(ctx), Hkv, DI), np.float32),
                                      np.zeros((total, DI), np.float32), q, k, v, offs, ctx, BK, topk)
    for b, n in enumerate(ctx):
        n = int(n)
        local = (n - 1) // BK
        earlier = list(range(min(topk - 1, local)))
        want_sel = earlier + [local] + [-1] * (topk - 1 - len(earlier))
        np.testing.assert_array_equal(sel[b, 0], want_sel)
        J = [j for j in range(n) if j // BK in set(earlier + [local])]
        assert len(J) == (n if local < topk else BK * (topk - 1) + (n - 1) % BK + 1)
        np.testing.assert_allclose(lse[b], math.log(len(J)), atol=1e-13, rtol=0)
        np.testing.assert_allclose(out[b, 0], v[offs[b] + np.asarray(J), 0].astype(np.float64).mean(axis=0), atol=1e-12)


def test_decode_equals_prefill_with_one_query_per_sequence(oracle_lib):
    """Contiguous caches: the decode step equals prefill with q_len 1 each."""
    rng = np.random.default_rng(11)
    Hq, Hkv, D, DI, topk = 4, 2, 8, 8, 4
    ctx = np.asarray([129, 1, 700, 2049], dtype=np.int64)
    offs, uk, k, v, uq = _caches(rng, ctx, Hkv, DI, Hkv, D, gap=0)
    q = rng.standard_normal((len(ctx), Hq, D)).astype(np.float32)
    qi, ki = (uq / 8).astype(np.float32), (uk / 8).astype(np.float32)
    dec = oracle_lib.decode(qi, ki, q, k, v, offs, ctx, BK, topk)
    cu_k = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int64)
    cu_q = np.arange(len(ctx) + 1, dtype=np.int64)
    pre = oracle_lib.prefill(qi, ki, q, k, v, cu_q, cu_k, BK, topk)
    for a, b in zip(dec, pre):
        np.testing.assert_array_equal(a, b)
