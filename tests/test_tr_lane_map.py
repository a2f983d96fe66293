"""Lane mapping of the transposed LDS read used by the backward's dV / dK
products (CPU).

gfx950's ds_read_b64_tr_b16: every lane names 8 bytes (four 16-bit values);
lane 16 g + i receives, as element e, value i % 4 of the four named by lane
16 g + 4 e + i / 4.  (That model was checked on the GPU against random
addresses and inside MFMA chains before the kernel used the instruction.)

bwd_dkdv reads the row-major Q / dO tile (the quad's 64 MFMA rows, pitch
136 bf16, MFMA row 16 s + 4 k + e stored at tile row 16 s + 4 e + k so
that both read kinds avoid LDS bank conflicts) this way for the B operand of
dV += P^T dO and dK += dS^T Q: lane L needs dim 32 dt + L % 32 and, for
k-step s4, the MFMA rows that the P / dS registers hold in the same slots --
16 s4 + 4 (L / 32) + j for j < 4 and 16 s4 + 8 + 4 (L / 32) + j - 4 for
j >= 4.  The lane addresses below restate the kernel's formula; the test
checks that the modelled instruction then delivers exactly those elements,
for every lane, dt and s4.  A missing row permutation, a swapped lane half,
a wrong pitch or a transposed tile each fail.
"""
import numpy as np

PITCH = 136          # bf16 per LDS row of the quad tiles
ROWS, DIMS = 64, 128


def tr_read(tile_flat, addr):
    """The instruction model: addr[L] = element offset named by lane L."""
    out = np.empty((64, 4), dtype=tile_flat.dtype)
    for L in range(64):
        g, i = divmod(L, 16)
        for e in range(4):
            src = 16 * g + 4 * e + i // 4
            out[L, e] = tile_flat[addr[src] + i % 4]
    return out


def tile_row(m):
    """Tile row of MFMA row m = 16 s + 4 k + e."""
    s, r = divmod(m, 16)
    k, e = divmod(r, 4)
    return 16 * s + 4 * e + k


def kernel_addresses(s4, dt, pitch=PITCH):
    """Lane addresses of the low read (the high read is 2 tile rows further)."""
    addr = np.empty(64, dtype=np.int64)
    for lam in range(64):
        a32 = lam >> 5
        tr_off = (4 * ((lam & 15) >> 2) + a32) * pitch + 16 * ((lam >> 4) & 1) + 4 * (lam & 3)
        addr[lam] = tr_off + 16 * s4 * pitch + 32 * dt
    return addr


def expected_fragment(tile2d, s4, dt):
    frag = np.empty((64, 8), dtype=tile2d.dtype)
    for L in range(64):
        a32, n = L >> 5, 32 * dt + (L & 31)
        for j in range(8):
            row = 16 * s4 + 4 * a32 + j if j < 4 else 16 * s4 + 8 + 4 * a32 + (j - 4)
            frag[L, j] = tile2d[row, n]
    return frag


def fragments(tile_flat, s4, dt, pitch=PITCH):
    lo_addr = kernel_addresses(s4, dt, pitch)
    lo = tr_read(tile_flat, lo_addr)
    hi = tr_read(tile_flat, lo_addr + 2 * pitch)
    return np.concatenate([lo, hi], axis=1)


def _tile(permute=True):
    """MFMA-row values (row * 1000 + col) laid out as bwd_dkdv stages them;
    pad columns hold a marker that must never appear."""
    t = np.full((ROWS, PITCH), -1, dtype=np.int64)
    vals = np.arange(ROWS)[:, None] * 1000 + np.arange(DIMS)[None, :]
    for m in range(ROWS):
        t[tile_row(m) if permute else m, :DIMS] = vals[m]
    return t, vals


def test_tile_row_is_a_permutation():
    assert sorted(tile_row(m) for m in range(ROWS)) == list(range(ROWS))


def test_backward_operand_fragments():
    t, vals = _tile()
    flat = t.reshape(-1)
    for s4 in range(4):
        for dt in range(4):
            got = fragments(flat, s4, dt)
            want = expected_fragment(vals, s4, dt)
            assert np.array_equal(got, want), (s4, dt)
            assert (got >= 0).all()   # no pad slot is ever read


def test_planted_mistakes_fail():
    t, vals = _tile()
    flat = t.reshape(-1)
    want = expected_fragment(vals, 1, 2)
    # the tile staged without the row permutation
    t_id, _ = _tile(permute=False)
    assert not np.array_equal(fragments(t_id.reshape(-1), 1, 2), want)
    # addresses for padded rows over a tile staged without the pad slot
    flat128 = np.concatenate([t[:, :128].reshape(-1), np.full(8 * PITCH, -1)])
    assert not np.array_equal(fragments(flat128, 1, 2), want)
    # lane halves swapped
    bad = kernel_addresses(1, 2)
    bad = np.concatenate([bad[32:], bad[:32]])
    got = np.concatenate([tr_read(flat, bad), tr_read(flat, bad + 2 * PITCH)], axis=1)
    assert not np.array_equal(got, want)
    # rows and columns exchanged (a transposed tile)
    tt = np.full((ROWS, PITCH), -1, dtype=np.int64)
    tt[:, :ROWS] = t[:, :ROWS].T
    assert not np.array_equal(fragments(tt.reshape(-1), 1, 2), want)
