"""Lane mapping of the transposed LDS read used by the backward's dV / dK
products (CPU).

gfx950's ds_read_b64_tr_b16: every lane names 8 bytes (four 16-bit values);
lane 16 g + i receives, as element e, value i % 4 of the four named by lane
16 g + 4 e + i / 4.  (That model was checked on the GPU against random
addresses and inside MFMA chains before the kernel used the instruction.)

bwd_dkdv reads the row-major Q / dO tile (rows = the quad's 64 MFMA rows,
pitch 136 bf16) this way for the B operand of dV += P^T dO and
dK += dS^T Q: lane L needs dim 32 dt + L % 32 and, for k-step s4, the rows
that the P / dS registers hold in the same slots -- 16 s4 + 4 (L / 32) + j
for j < 4 and 16 s4 + 8 + 4 (L / 32) + j - 4 for j >= 4.  The lane addresses
below restate the kernel's formula; the test checks that the modelled
instruction then delivers exactly those elements, for every lane, dt and
s4.  A transposed dim/row, a swapped lane half or a wrong pitch each fail.
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


def kernel_addresses(s4, dt, pitch=PITCH):
    """Lane addresses of the low read (the high read is 8 rows further)."""
    addr = np.empty(64, dtype=np.int64)
    for lam in range(64):
        a32 = lam >> 5
        tr_off = (4 * a32 + ((lam & 15) >> 2)) * pitch + 16 * ((lam >> 4) & 1) + 4 * (lam & 3)
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
    hi = tr_read(tile_flat, lo_addr + 8 * pitch)
    return np.concatenate([lo, hi], axis=1)


def _tile():
    # distinct value per (row, col); pad columns hold a marker that must never appear
    t = np.full((ROWS, PITCH), -1, dtype=np.int64)
    t[:, :DIMS] = np.arange(ROWS)[:, None] * 1000 + np.arange(DIMS)[None, :]
    return t


def test_backward_operand_fragments():
    t = _tile()
    flat = t.reshape(-1)
    for s4 in range(4):
        for dt in range(4):
            got = fragments(flat, s4, dt)
            want = expected_fragment(t, s4, dt)
            assert np.array_equal(got, want), (s4, dt)
            assert (got >= 0).all()   # no pad slot is ever read


def test_planted_mistakes_fail():
    t = _tile()
    flat = t.reshape(-1)
    want = expected_fragment(t, 1, 2)
    # addresses for padded rows over a tile staged without the pad slot
    flat128 = np.concatenate([t[:, :128].reshape(-1), np.full(8 * PITCH, -1)])
    assert not np.array_equal(fragments(flat128, 1, 2), want)
    # lane halves swapped: rows of the other half
    bad = kernel_addresses(1, 2)
    bad = np.concatenate([bad[32:], bad[:32]])
    got = np.concatenate([tr_read(flat, bad), tr_read(flat, bad + 8 * PITCH)], axis=1)
    assert not np.array_equal(got, want)
    # rows and columns exchanged in the address (a transposed tile)
    tt = np.ascontiguousarray(t[:, :ROWS].T)
    tpad = np.full((ROWS, PITCH), -1, dtype=np.int64)
    tpad[:, :ROWS] = tt
    assert not np.array_equal(fragments(tpad.reshape(-1), 1, 2)[:, :], want)
