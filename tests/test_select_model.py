"""CPU model of the prefill index selection's rounds, restated from the kernel
(idx_select_prefill) and checked against a brute-force top-k (no GPU).

What is restated: 64-bit selection keys (order-preserving score bits above the
inverted block id, 0 = no block); rounds of 1024 earlier blocks, block
r0 + lane + 64 u in key u of a lane, with the round's slice count rounded up
to a power of two; the threshold T = the 16th largest lane maximum (a
bitwise search on the high words that stops once exactly 16 lanes reach it,
the low bits an id can have only when high words tie), raised to best[15], or best[15] at once when fewer than 16 lanes
reach it; candidates compacted lane by lane at offsets from a prefix sum built
from one ballot per bit of the lanes' counts; exact ranks.  The checks: the
best 16 after every row equal the brute-force best 16 (score descending, id
ascending), the candidates never exceed the 16 * 16 + 16 slots the kernel
holds, the bit-sliced offsets are the exclusive prefix sum, and the skipped
search never changes T.
"""
import struct

import numpy as np
import pytest

W = 64
ROUND = 16 * W
CAND_CAP = 16 * 16 + 16


def sel_key(score, c):
    b = struct.unpack("<I", struct.pack("<f", float(score)))[0]
    hi = (~b & 0xFFFFFFFF) if b & 0x80000000 else (b | 0x80000000)
    return (hi << 32) | (0xFFFFFFFF - c)


def key_id(k):
    return 0xFFFFFFFF - (k & 0xFFFFFFFF)


def kth_hi(xh, kth):
    """A th with at least kth of xh >= th; the search stops once exactly kth
    reach it (those are the kth largest and th is below all of them)."""
    th = 0
    for b in range(31, -1, -1):
        t = th | (1 << b)
        c = sum(1 for x in xh if x >= t)
        if c >= kth:
            th = t
        if c == kth:
            break
    return th


def kth_lo(x, th, kth, lo_bits):
    tl = 0 if lo_bits >= 32 else (0xFFFFFFFF << lo_bits) & 0xFFFFFFFF
    for b in range(lo_bits - 1, -1, -1):
        t = (th << 32) | (tl | (1 << b))
        if sum(1 for v in x if v >= t) >= kth:
            tl |= 1 << b
    return (th << 32) | tl


def bit_sliced_offsets(cnt, bits):
    """Lane offsets as the kernel forms them: for each bit j of the counts, the
    number of lower lanes with that bit set (a ballot and a masked bit count),
    shifted by j."""
    off = [0] * W
    for j in range(bits):
        m = [(c >> j) & 1 for c in cnt]
        for lane in range(W):
            off[lane] += sum(m[:lane]) << j
    return off


def sel_round(sc, r0, local, lo_bits, best, stats):
    nu = (local - r0 + W - 1) // W
    NU = 16 if nu > 8 else 8 if nu > 4 else 4 if nu > 2 else 2 if nu > 1 else 1
    k = [[0] * W for _ in range(NU)]
    for u in range(NU):
        for lane in range(W):
            c = r0 + lane + W * u
            k[u][lane] = sel_key(sc[min(c, local - 1)], c) if c < local else 0
    mxh = [max(k[u][lane] >> 32 for u in range(NU)) for lane in range(W)]
    b15 = best[15]

    def full_threshold():
        th = kth_hi(mxh, 16)
        t_round = th << 32
        if sum(1 for x in mxh if x >= th) > 16:
            mx = [max(k[u][lane] for u in range(NU)) for lane in range(W)]
            t_round = kth_lo(mx, th, 16, lo_bits)
        return max(t_round, b15)

    search = True
    if b15 != 0:
        reach = [any(k[u][lane] >= b15 for u in range(NU)) for lane in range(W)]
        search = sum(reach) >= 16
    if search:
        T = full_threshold()
    else:
        T = b15
        stats["skipped"] += 1
        assert full_threshold() == b15  # the skip never changes T
    T = max(T, 1)
    x = [best[lane] if lane < 16 else 0 for lane in range(W)]
    cnt = [(1 if x[lane] >= T else 0) + sum(1 for u in range(NU) if k[u][lane] >= T) for lane in range(W)]
    bits = 5 if NU >= 16 else 4 if NU >= 8 else 3 if NU >= 4 else 2
    assert max(cnt) < (1 << bits)
    off = bit_sliced_offsets(cnt, bits)
    assert off == list(np.concatenate([[0], np.cumsum(cnt)[:-1]]))
    n = off[-1] + cnt[-1]
    assert n <= CAND_CAP
    stats["max_cand"] = max(stats["max_cand"], n)
    cand = [0] * n
    for lane in range(W):
        o = off[lane]
        for u in range(NU):
            if k[u][lane] >= T:
                cand[o] = k[u][lane]
                o += 1
        if x[lane] >= T:
            cand[o] = x[lane]
            o += 1
    assert len(set(cand)) == n  # distinct keys, so ranks are distinct
    new = [0] * 16
    for c in cand:
        r = sum(1 for d in cand if d > c)
        if r < 16:
            new[r] = c
    return new


def model_select(scores, local, stats):
    lo_bits = (local - 1).bit_length() if local > 1 else 0
    best = [0] * 16
    for r0 in range(0, local, ROUND):
        best = sel_round(scores, r0, local, lo_bits, best, stats)
    return best


def brute_best16(scores, local):
    order = sorted(range(local), key=lambda c: (-float(scores[c]), c))
    return order[:16]


def _check(scores, local, stats):
    best = model_select(scores, local, stats)
    got = [key_id(k) for k in best if k != 0]
    assert got == brute_best16(scores, local)


@pytest.mark.parametrize("local", [1, 2, 15, 16, 17, 63, 64, 65, 129, 300, 1023, 1024, 1025, 2500])
def test_rounds_match_brute_force_random(local):
    rng = np.random.default_rng(local)
    stats = {"skipped": 0, "max_cand": 0}
    for _ in range(2):
        scores = rng.standard_normal(local).astype(np.float32) * 3.0
        _check(scores, local, stats)


@pytest.mark.parametrize("local", [40, 700, 1500])
def test_ties_take_the_low_bit_search(local):
    # few distinct values: many lanes tie on the high word of the threshold
    rng = np.random.default_rng(7 + local)
    stats = {"skipped": 0, "max_cand": 0}
    for levels in (1, 2, 5):
        scores = rng.integers(0, levels, local).astype(np.float32) - 0.5
        _check(scores, local, stats)


def test_later_rounds_skip_the_search_without_changing_it():
    rng = np.random.default_rng(3)
    stats = {"skipped": 0, "max_cand": 0}
    local = 5000  # five rounds
    for _ in range(2):
        _check(rng.standard_normal(local).astype(np.float32), local, stats)
    assert stats["skipped"] > 0
    # rising scores: every round beats the previous best, so the search runs
    stats2 = {"skipped": 0, "max_cand": 0}
    _check(np.linspace(-4.0, 4.0, 3000).astype(np.float32), 3000, stats2)
    assert stats2["skipped"] == 0


def test_candidate_bound_on_adversarial_rounds():
    # every lane's 16 keys just above the others' maxima would break a
    # threshold that is not a lane-maximum order statistic; the bound holds
    local = 1024
    scores = np.zeros(local, dtype=np.float32)
    for lane in range(W):
        for u in range(16):
            scores[lane + W * u] = lane + u / 32.0
    stats = {"skipped": 0, "max_cand": 0}
    _check(scores, local, stats)
    assert stats["max_cand"] <= CAND_CAP


def test_a_planted_mistake_fails():
    # dropping the previous best from the candidates loses blocks of earlier rounds
    rng = np.random.default_rng(11)
    scores = rng.standard_normal(2048).astype(np.float32)
    scores[:5] += 10.0  # the best blocks sit in the first round
    best = model_select(scores, 2048, {"skipped": 0, "max_cand": 0})
    assert sorted(key_id(k) for k in best[:5]) == [0, 1, 2, 3, 4]
    global sel_round
    real = sel_round

    def broken(sc, r0, local, lo_bits, best, stats):
        return real(sc, r0, local, lo_bits, [0] * 16, stats)

    sel_round = broken
    try:
        best = model_select(scores, 2048, {"skipped": 0, "max_cand": 0})
    finally:
        sel_round = real
    assert [key_id(k) for k in best if k != 0] != brute_best16(scores, 2048)
