"""CPU model of the prefill index scan's work split, restated from the
library's plan and the scan kernel's workgroup decode (no GPU).

The plan cuts each query block's earlier key blocks into chunks of a multiple
of 16 blocks, sized for about 256 workgroups; items (query block, query slice,
key chunk, sequence) are numbered query block fastest, heaviest block first.
When there are at least two rounds of items, a workgroup scores item k and
its mirror n - 1 - k.  The checks: every item is scored exactly once (odd
counts included), every chunk of every query block is some item, and for one
causal sequence (the 32K and 64K single-call prefills) the mirror pairs carry
nearly equal work, so one round of workgroups is balanced.
"""
import pytest

BLOCK = 128
TARGET_WGS = 256


def cdiv(a, b):
    return -(-a // b)


def plan(batch, max_q_len, max_kv_len, G):
    nb_max = cdiv(max_kv_len, BLOCK)
    qw = min(512 // G, BLOCK)
    nsub = cdiv(BLOCK, qw)
    qb = min(cdiv(max_q_len, BLOCK) + 1, nb_max)
    c_max = nb_max - 1
    c_first = max(c_max - qb + 1, 0)
    work = batch * nsub * (c_first + c_max) * (c_max - c_first + 1) // 2
    chunk = cdiv(cdiv(work, TARGET_WGS), 16) * 16
    max_chunks = cdiv(c_max, chunk)
    items = batch * qb * nsub * max_chunks
    return dict(qw=qw, nsub=nsub, max_qblocks=qb, chunk=chunk, max_chunks=max_chunks, items=items,
                pair=items >= 2 * TARGET_WGS)


def item_work(p, bid, lens):
    """Blocks scanned by item `bid` of causal sequences with q_len = kv_len."""
    qb = p["max_qblocks"]
    slot = qb - 1 - (bid % qb)
    bid //= qb
    sub = bid % p["nsub"]
    bid //= p["nsub"]
    ch = bid % p["max_chunks"]
    b = bid // p["max_chunks"]
    n = lens[b]
    c = slot  # q_len == kv_len: the first position with keys is 0
    if c * BLOCK >= n:
        return 0
    plo = c * BLOCK + sub * p["qw"]
    if plo >= min((c + 1) * BLOCK, n):
        return 0
    s_lo = ch * p["chunk"]
    s_hi = min(s_lo + p["chunk"], c)
    return max(s_hi - s_lo, 0)


def workgroups(p):
    n = p["items"]
    if not p["pair"]:
        return [[k] for k in range(n)]
    groups = []
    for w in range(cdiv(n, 2)):
        m = n - 1 - w
        groups.append([w] if m == w else [w, m])
    return groups


@pytest.mark.parametrize("lens", [[32768], [65536], [9000, 3000, 20000, 12000], [21888, 5000, 15000], [8192],
                                  [131072]])
def test_every_item_once(lens):
    p = plan(len(lens), max(lens), max(lens), 4)
    seen = [k for g in workgroups(p) for k in g]
    assert sorted(seen) == list(range(p["items"]))
    # every (query block, chunk) of every sequence with work is an item
    total = sum(item_work(p, k, lens) for k in range(p["items"]))
    assert total == sum(c for n in lens for c in range(cdiv(n, BLOCK)))


@pytest.mark.parametrize("L", [32768, 65536])
def test_mirror_pairs_balance_one_causal_sequence(L):
    p = plan(1, L, L, 4)
    assert p["pair"]
    loads = [sum(item_work(p, k, [L]) for k in g) for g in workgroups(p)]
    assert len(loads) <= TARGET_WGS
    mean = sum(loads) / len(loads)
    assert max(loads) <= 1.02 * mean
    # unpaired, the largest item would be the whole call's critical path
    single = [item_work(p, k, [L]) for k in range(p["items"])]
    assert max(single) > 0.95 * max(loads) and len([x for x in single if x]) > TARGET_WGS


def test_long_calls_stay_unpaired():
    # an 8192-query tile against a long prefix has one round of items
    for kv in (32768, 131072, 1048576):
        p = plan(1, 8192, kv, 4)
        assert not p["pair"] and p["items"] < 2 * TARGET_WGS
