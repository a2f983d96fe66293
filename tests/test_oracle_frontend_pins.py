"""Pins for the oracle's index front-end (hidden states -> projection -> norm ->
RoPE -> index-query heads and the shared index-key head), independent of the
oracle's own code.

Figure 1 of "MiniMax Sparse Attention: let each query pick its own blocks"
gives the three steps and their order; the atlas record of MiniMax M3 gives
the model width (3072) and a rotary width of half the head dimension.  The
norm's kind (RMS norm with a gain per dimension) and the rotary base are
readings.  Each test below fails for a plausible slip in the oracle:

* projection: a transposed weight or a wrong head slice (brute-force loops on
  tiny inputs, compared up to the positive scale the norm removes);
* norm: a sum in place of the mean, eps outside the root, the norm taken over
  all heads at once, the gain applied before the norm (closed-form example,
  per-head isolation, gain linearity);
* RoPE: adjacent pairs (2i, 2i+1) in place of (i, i + r/2), a reversed
  rotation sense, a wrong frequency exponent, dims past the rotary width
  rotated, positions relative to the chunk instead of absolute (unit vectors
  with textbook angles, a frequency of exactly one half, pass-through dims,
  and the front-end of a chunk against the rows of the whole sequence);
* backward (gradients of the projections and gains, x held constant): torch
  autograd through a front-end written independently in torch ops, and
  central differences of the oracle's own forward.
"""
import math

import numpy as np
import pytest


def _eye_weights(G, DI):
    """W with d_model = DI: every head is the identity, so y = x."""
    wq = np.concatenate([np.eye(DI, dtype=np.float32)] * G, axis=0)
    return wq, np.eye(DI, dtype=np.float32)


def test_projection_matches_brute_force(oracle_lib):
    rng = np.random.default_rng(1)
    n, d_model, G, DI = 3, 16, 2, 8
    x = rng.standard_normal((n, d_model)).astype(np.float32)
    wq = rng.standard_normal((G * DI, d_model)).astype(np.float32)
    wk = rng.standard_normal((DI, d_model)).astype(np.float32)
    q, k = oracle_lib.index_frontend(x, wq, wk, np.ones(DI), np.ones(DI), [0, 0, 0], G, DI, 0, 1e4, 0.0)
    for t in range(n):
        for h in range(G + 1):
            y = []
            for i in range(DI):
                s = 0.0
                for c in range(d_model):
                    w = wq[h * DI + i, c] if h < G else wk[i, c]
                    s += float(w) * float(x[t, c])
                y.append(s)
            y = np.array(y)
            got = q[t, h] if h < G else k[t]
            # same direction (positive factor) and unit RMS: together they fix y / rms(y)
            cos = float(got @ y) / (np.linalg.norm(got) * np.linalg.norm(y))
            assert cos == pytest.approx(1.0, abs=1e-12)
            assert math.sqrt(float(np.mean(got ** 2))) == pytest.approx(1.0, abs=1e-12)


def test_norm_closed_form_with_eps(oracle_lib):
    """y = (3, 4, 0, ..., 0) over 8 dims: mean square 25/8; with eps = 7/8 the
    root is exactly 2, so the output is (1.5, 2, 0, ...)."""
    G, DI = 1, 8
    wq, wk = _eye_weights(G, DI)
    x = np.zeros((1, DI), dtype=np.float32)
    x[0, 0], x[0, 1] = 3.0, 4.0
    q, k = oracle_lib.index_frontend(x, wq, wk, np.ones(DI), np.ones(DI), [0], G, DI, 0, 1e4, 7.0 / 8.0)
    want = np.zeros(DI)
    want[0], want[1] = 1.5, 2.0
    assert np.allclose(q[0, 0], want, atol=1e-15) and np.allclose(k[0], want, atol=1e-15)


def test_norm_is_per_head_and_gain_is_applied_after(oracle_lib):
    rng = np.random.default_rng(2)
    n, d_model, G, DI = 4, 24, 3, 8
    x = rng.standard_normal((n, d_model)).astype(np.float32)
    wq = rng.standard_normal((G * DI, d_model)).astype(np.float32)
    wk = rng.standard_normal((DI, d_model)).astype(np.float32)
    gq = rng.uniform(0.5, 2.0, DI)
    gk = rng.uniform(0.5, 2.0, DI)
    pos = [5, 6, 7, 8]
    q1, k1 = oracle_lib.index_frontend(x, wq, wk, np.ones(DI), np.ones(DI), pos, G, DI, 0, 1e4, 1e-6)
    # a head whose projection is 1024 times larger leaves the other heads unchanged (norm per head)
    wq2 = wq.copy()
    wq2[DI:2 * DI] *= 1024.0
    q2, _ = oracle_lib.index_frontend(x, wq2, wk, np.ones(DI), np.ones(DI), pos, G, DI, 0, 1e4, 1e-6)
    assert np.allclose(q2[:, 0], q1[:, 0], atol=1e-13) and np.allclose(q2[:, 2], q1[:, 2], atol=1e-13)
    # with no rotation the gain multiplies each output dim (it does not enter the mean square)
    q3, k3 = oracle_lib.index_frontend(x, wq, wk, gq, gk, pos, G, DI, 0, 1e4, 1e-6)
    assert np.allclose(q3, q1 * gq, atol=1e-13) and np.allclose(k3, k1 * gk, atol=1e-13)


@pytest.mark.parametrize("i, p, theta", [(0, 1, 10000.0), (1, 2, 16.0), (3, 7, 16.0)])
def test_rope_unit_vectors(oracle_lib, i, p, theta):
    """x = e_i (DI = 8, rotary width 8, so the pair of dim i is dim i + 4): the
    norm maps it to sqrt(8) e_i, and RoPE turns the pair by p * theta^(-2i/8).
    Pair 0 has frequency 1 (angle p); with theta = 16 pair 1 has frequency
    1/2, so p = 2 gives exactly one radian; pair 3 has 16^(-3/4) = 1/8."""
    G, DI = 1, 8
    wq, wk = _eye_weights(G, DI)
    x = np.zeros((1, DI), dtype=np.float32)
    x[0, i] = 1.0
    q, k = oracle_lib.index_frontend(x, wq, wk, np.ones(DI), np.ones(DI), [p], G, DI, DI, theta, 0.0)
    freq = {0: 1.0, 1: 0.5, 3: 0.125}[i] if theta == 16.0 or i == 0 else None
    ang = p * freq
    want = np.zeros(DI)
    want[i] = math.sqrt(8.0) * math.cos(ang)
    want[i + 4] = math.sqrt(8.0) * math.sin(ang)
    assert np.allclose(q[0, 0], want, atol=1e-13), (q[0, 0], want)
    assert np.allclose(k[0], want, atol=1e-13)
    # the partner dim turns the other way: e_{i+4} -> (-sin, cos)
    x[0, i], x[0, i + 4] = 0.0, 1.0
    q, _ = oracle_lib.index_frontend(x, wq, wk, np.ones(DI), np.ones(DI), [p], G, DI, DI, theta, 0.0)
    want = np.zeros(DI)
    want[i] = -math.sqrt(8.0) * math.sin(ang)
    want[i + 4] = math.sqrt(8.0) * math.cos(ang)
    assert np.allclose(q[0, 0], want, atol=1e-13)


def test_rope_partial_width_passes_the_rest_through(oracle_lib):
    """Rotary width 4 of 8 dims: pairs (0, 2) and (1, 3) turn, dims 4..7 do not."""
    G, DI = 1, 8
    wq, wk = _eye_weights(G, DI)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, DI)).astype(np.float32)
    q0, _ = oracle_lib.index_frontend(x, wq, wk, np.ones(DI), np.ones(DI), [0], G, DI, 4, 100.0, 0.0)
    q9, _ = oracle_lib.index_frontend(x, wq, wk, np.ones(DI), np.ones(DI), [9], G, DI, 4, 100.0, 0.0)
    assert np.array_equal(q0[0, 0, 4:], q9[0, 0, 4:])
    # position 0 is the identity; each turned pair keeps its length
    xs = x[0].astype(np.float64) / math.sqrt(float(np.mean(x[0].astype(np.float64) ** 2)))
    assert np.allclose(q0[0, 0], xs, atol=1e-13)
    for a, b in ((0, 2), (1, 3)):
        assert math.hypot(q9[0, 0, a], q9[0, 0, b]) == pytest.approx(math.hypot(xs[a], xs[b]), abs=1e-13)
    # pair 1 turns by 9 * 100^(-1/2) = 0.9 radians
    c, s = math.cos(0.9), math.sin(0.9)
    assert q9[0, 0, 1] == pytest.approx(xs[1] * c - xs[3] * s, abs=1e-13)
    assert q9[0, 0, 3] == pytest.approx(xs[3] * c + xs[1] * s, abs=1e-13)


def test_rope_scores_depend_on_relative_position(oracle_lib):
    """q_idx(p) . k_idx(s) is unchanged when both positions move by the same
    amount (full rotary width), but not when only one moves."""
    rng = np.random.default_rng(4)
    d_model, G, DI = 32, 2, 16
    x = rng.standard_normal((2, d_model)).astype(np.float32)
    wq = rng.standard_normal((G * DI, d_model)).astype(np.float32)
    wk = rng.standard_normal((DI, d_model)).astype(np.float32)
    one = np.ones(DI)

    def score(p, s):
        q, _ = oracle_lib.index_frontend(x[:1], wq, wk, one, one, [p], G, DI, DI, 500.0, 1e-6)
        _, k = oracle_lib.index_frontend(x[1:], wq, wk, one, one, [s], G, DI, DI, 500.0, 1e-6)
        return q[0] @ k[0]

    base = score(40, 13)
    assert np.allclose(score(40 + 1000, 13 + 1000), base, atol=1e-9)
    assert not np.allclose(score(41, 13), base, atol=1e-3)


def test_chunk_positions_are_absolute(oracle_lib):
    """The last 5 tokens of an 11-token sequence processed as a chunk
    (q_len 5, kv_len 11) equal rows 6..10 of the whole-sequence front-end."""
    rng = np.random.default_rng(5)
    d_model, G, DI = 32, 2, 16
    x = rng.standard_normal((11, d_model)).astype(np.float32)
    wq = rng.standard_normal((G * DI, d_model)).astype(np.float32)
    wk = rng.standard_normal((DI, d_model)).astype(np.float32)
    one = np.ones(DI)
    _, _, pos_full = oracle_lib.rows_prefill([0, 11], [0, 11])
    _, _, pos_chunk = oracle_lib.rows_prefill([0, 5], [0, 11])
    qf, kf = oracle_lib.index_frontend(x, wq, wk, one, one, pos_full, G, DI, 8, 1e4, 1e-6)
    qc, kc = oracle_lib.index_frontend(x[6:], wq, wk, one, one, pos_chunk, G, DI, 8, 1e4, 1e-6)
    assert np.array_equal(qc, qf[6:]) and np.array_equal(kc, kf[6:])


def test_bad_arguments_are_rejected(oracle_lib):
    G, DI = 1, 8
    wq, wk = _eye_weights(G, DI)
    x = np.ones((1, DI), dtype=np.float32)
    for rope_dim, theta, eps in ((3, 1e4, 0.0), (10, 1e4, 0.0), (8, 0.0, 0.0), (8, 1e4, -1.0)):
        with pytest.raises(ValueError):
            oracle_lib.index_frontend(x, wq, wk, np.ones(DI), np.ones(DI), [0], G, DI, rope_dim, theta, eps)


def _torch_frontend(x, wq, wk, gq, gk, pos, G, DI, rope_dim, theta, eps):
    """The front-end written independently in torch ops (fp64), for autograd."""
    import torch
    y = torch.cat([(x @ wq.T).reshape(x.shape[0], G, DI), (x @ wk.T)[:, None, :]], dim=1)  # [n, G+1, DI]
    n = y / torch.sqrt((y * y).mean(dim=-1, keepdim=True) + eps)
    gain = torch.cat([gq.expand(G, DI), gk[None, :]], dim=0)
    z = n * gain
    if rope_dim:
        half = rope_dim // 2
        i = torch.arange(half, dtype=torch.float64)
        ang = pos[:, None].double() * theta ** (-2.0 * i / rope_dim)  # [n, half]
        c, s = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
        a, b = z[..., :half], z[..., half:rope_dim]
        z = torch.cat([a * c - b * s, b * c + a * s, z[..., rope_dim:]], dim=-1)
    return z[:, :G], z[:, G]


@pytest.mark.parametrize("rope_dim", [0, 8, 16])
def test_frontend_backward_matches_autograd(oracle_lib, rope_dim):
    import torch
    rng = np.random.default_rng(6)
    n, d_model, G, DI, theta, eps = 7, 24, 3, 16, 50.0, 1e-3
    x = rng.standard_normal((n, d_model)).astype(np.float32)
    wq = rng.standard_normal((G * DI, d_model)).astype(np.float32)
    wk = rng.standard_normal((DI, d_model)).astype(np.float32)
    gq = rng.uniform(0.5, 1.5, DI)
    gk = rng.uniform(0.5, 1.5, DI)
    pos = np.array([0, 3, 17, 100, 5, 2, 999])
    dq = rng.standard_normal((n, G, DI))
    dk = rng.standard_normal((n, DI))
    tw = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (wq, wk, gq, gk)]
    q, k = _torch_frontend(torch.tensor(x, dtype=torch.float64), *tw, torch.tensor(pos), G, DI, rope_dim, theta, eps)
    ((q * torch.tensor(dq)).sum() + (k * torch.tensor(dk)).sum()).backward()
    got = oracle_lib.index_frontend_bwd(x, wq, wk, gq, gk, pos, G, DI, rope_dim, theta, eps, dq, dk)
    for name, g, t in zip(("dw_q", "dw_k", "dgain_q", "dgain_k"), got, tw):
        assert np.allclose(g, t.grad.numpy(), rtol=1e-10, atol=1e-10), name
    # the forward of the torch formulation agrees with the oracle's forward too
    rq, rk = oracle_lib.index_frontend(x, wq, wk, gq, gk, pos, G, DI, rope_dim, theta, eps)
    assert np.allclose(q.detach().numpy(), rq, atol=1e-12) and np.allclose(k.detach().numpy(), rk, atol=1e-12)


def test_frontend_backward_matches_finite_differences(oracle_lib):
    """Central differences of L = sum(dq * q_idx) + sum(dk * k_idx), with the
    oracle's own forward, at coordinates of every parameter."""
    rng = np.random.default_rng(7)
    n, d_model, G, DI, rope, theta, eps = 5, 16, 2, 8, 8, 30.0, 1e-2
    x = rng.standard_normal((n, d_model))
    wq = rng.standard_normal((G * DI, d_model))
    wk = rng.standard_normal((DI, d_model))
    gq = rng.uniform(0.5, 1.5, DI)
    gk = rng.uniform(0.5, 1.5, DI)
    pos = np.array([1, 4, 9, 33, 70])
    dq = rng.standard_normal((n, G, DI))
    dk = rng.standard_normal((n, DI))
    # fp32 inputs for the oracle's loader; the perturbed copies stay fp64 until here
    f32 = lambda a: np.asarray(a, dtype=np.float32)
    x, wq, wk = f32(x), f32(wq), f32(wk)
    dwq, dwk, dgq, dgk = oracle_lib.index_frontend_bwd(x, wq, wk, gq, gk, pos, G, DI, rope, theta, eps, dq, dk)

    def loss(wq_, wk_, gq_, gk_):
        q, k = oracle_lib.index_frontend(x, wq_, wk_, gq_, gk_, pos, G, DI, rope, theta, eps)
        return float((q * dq).sum() + (k * dk).sum())

    # weights: steps that are exact in fp32 (the loader reads fp32), gains: fp64
    h = 2.0 ** -8
    for (r, c) in ((0, 0), (5, 7), (G * DI - 1, d_model - 1)):
        a, b = wq.copy(), wq.copy()
        a[r, c] += h
        b[r, c] -= h
        fd = (loss(a, wk, gq, gk) - loss(b, wk, gq, gk)) / (2 * h)
        assert fd == pytest.approx(dwq[r, c], rel=1e-3, abs=1e-4)
    for (r, c) in ((0, 3), (DI - 1, 11)):
        a, b = wk.copy(), wk.copy()
        a[r, c] += h
        b[r, c] -= h
        fd = (loss(wq, a, gq, gk) - loss(wq, b, gq, gk)) / (2 * h)
        assert fd == pytest.approx(dwk[r, c], rel=1e-3, abs=1e-4)
    e = 1e-6
    for i in (0, 3, DI - 1):
        a, b = gq.copy(), gq.copy()
        a[i] += e
        b[i] -= e
        assert (loss(wq, wk, a, gk) - loss(wq, wk, b, gk)) / (2 * e) == pytest.approx(dgq[i], rel=1e-6, abs=1e-8)
        a, b = gk.copy(), gk.copy()
        a[i] += e
        b[i] -= e
        assert (loss(wq, wk, gq, a) - loss(wq, wk, gq, b)) / (2 * e) == pytest.approx(dgk[i], rel=1e-6, abs=1e-8)
