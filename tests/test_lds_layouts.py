"""CPU checks of two data layouts of the GPU kernels, restated here from their
definitions (no GPU): the key-major dS tile of the main-branch backward and
the run-major partial outputs of the KV-outer attention.

The dS tile holds, for each of a block's 128 keys, the bf16 dS of a quad's 64
MFMA rows; the 8-byte unit of rows 4u .. 4u + 3 of key `key` sits at element
key * 96 + 4 * (u ^ ((key // 4) % 8)).  The checks: every (key, unit) has its
own 8 bytes inside the tile, and under a model of gfx950's LDS (64 banks of 4
bytes, an 8-byte access served 32 lanes at a time, or 16 lanes at a time) the
writes of the V waves and the transposed reads of the dQ product take the
fewest cycles their 512 bytes allow, as they did with the earlier 160-element
rows; an unswizzled tile of the same pitch would not.  (On the GPU the
transposed reads measure as modelled; the 8-byte writes of this pattern count
twice the minimum cycles, so the model is a necessary check for the writes,
not a sufficient one.)

A selection slot's partial output holds 16 heads x 128 dims in bf16, stored
run-major: the 16-byte run of dims 8r .. 8r + 7 of head h at element
(r * 16 + h) * 8.  The checks: the map is a bijection onto the slot's 4 KB, and
the accesses of the attention kernel's stores and the combine's loads each
cover whole 128-byte lines.
"""
import itertools

import pytest

DS_ROW = 96          # elements per key row of the dS tile
KEYS, ROWS = 128, 64


def ds_off(key, row4, pitch=DS_ROW, swizzle=True):
    """Element offset of MFMA rows row4 .. row4 + 3 (row4 % 4 == 0) of `key`."""
    u = row4 // 4
    return key * pitch + 4 * (u ^ ((key // 4) % 8) if swizzle else u)


def cycles(addr_bytes, lanes_per_pass, width=8, banks=64):
    """LDS cycles of one 64-lane access under the bank model: each pass of
    `lanes_per_pass` lanes takes as many cycles as its most-used bank."""
    tot = 0
    for p in range(0, 64, lanes_per_pass):
        use = {}
        for lane in range(p, p + lanes_per_pass):
            for w in range(width // 4):
                b = (addr_bytes[lane] // 4 + w) % banks
                use[b] = use.get(b, 0) + 1
        tot += max(use.values())
    return tot


def ds_writes(**kw):
    """The V waves' dS writes: lane (col = lane % 32, a32 = lane // 32) of key
    tile kt writes key 32 kt + col, rows 32 rh + 8 q4 + 4 a32 .. + 3."""
    for kt, rh, q4 in itertools.product(range(4), range(2), range(4)):
        yield [2 * ds_off(32 * kt + (L & 31), 32 * rh + 8 * q4 + 4 * (L >> 5), **kw) for L in range(64)]


def ds_tr_reads(**kw):
    """The dQ product's transposed reads: lane 16 g + 4 e + q reads key
    16 ks + 8 (g // 2) + e (+ 4 for the second read), rows rb + 16 (g % 2) + 4 q."""
    for ks, rb, hi in itertools.product(range(8), (0, 32), (0, 4)):
        addrs = []
        for L in range(64):
            g, e, q = L >> 4, (L & 15) >> 2, L & 3
            addrs.append(2 * ds_off(16 * ks + 8 * (g >> 1) + e + hi, rb + 16 * (g & 1) + 4 * q, **kw))
        yield addrs


def test_ds_tile_units_are_distinct_and_inside():
    seen = set()
    for key in range(KEYS):
        for u in range(ROWS // 4):
            o = ds_off(key, 4 * u)
            assert 0 <= o and o + 4 <= KEYS * DS_ROW
            # an 8-byte unit never crosses into the next key's row
            assert o // DS_ROW == key
            for e in range(4):
                assert o + e not in seen
                seen.add(o + e)
    assert len(seen) == KEYS * ROWS


@pytest.mark.parametrize("lanes", [32, 16])
def test_ds_tile_accesses_take_the_minimum_cycles(lanes):
    minimum = 64 * 8 // 256  # 512 bytes, 256 bytes per cycle
    if lanes == 16:
        minimum = 4  # 16 lanes x 8 bytes = 128 bytes per pass
    for kw in ({"pitch": 96}, {"pitch": 160}):
        assert all(cycles(a, lanes) == minimum for a in ds_writes(**kw))
        assert all(cycles(a, lanes) == minimum for a in ds_tr_reads(**kw))


def test_ds_tile_without_swizzle_conflicts():
    # the swizzle is what spreads the writes: without it 32 keys at one unit
    # fall on a few bank groups
    worst = max(cycles(a, 32) for a in ds_writes(swizzle=False))
    assert worst > 2


RMAX, DIM = 16, 128


def run_off(r, h):
    return (r * RMAX + h) * 8


def test_run_major_partial_is_a_bijection():
    units = sorted(run_off(r, h) // 8 for r in range(DIM // 8) for h in range(RMAX))
    assert units == list(range(RMAX * DIM // 8))


def lines_of(byte_offsets, size=16):
    return {o // 128 for o in byte_offsets} | {(o + size - 1) // 128 for o in byte_offsets}


def test_attention_store_covers_whole_lines():
    # one store of the attention kernel: lane (col = lane % 32 -> query jq =
    # col // 16, head h = col % 16; a32 = lane // 32) writes run 4 dt + 2 m + a32
    # of head h in the slot of query jq (slots far apart: offset jq * 1 MB)
    for dt, m in itertools.product(range(4), range(2)):
        offs = []
        for L in range(64):
            col, a32 = L & 31, L >> 5
            jq, h = col >> 4, col & 15
            offs.append(jq * (1 << 20) + 2 * run_off(4 * dt + 2 * m + a32, h))
        lines = lines_of(offs)
        assert len(lines) * 128 == 64 * 16  # 1 KB in exactly 8 whole lines
        assert len(set(offs)) == 64


def test_combine_load_covers_whole_lines():
    # one load of the combine: lane (h = lane % 16, quarter q = lane // 16)
    # reads run 4 q + j of head h
    for j in range(4):
        offs = [2 * run_off(4 * (L >> 4) + j, L & 15) for L in range(64)]
        assert len(lines_of(offs)) * 128 == 64 * 16
