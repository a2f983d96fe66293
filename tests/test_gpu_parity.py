"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every input is seeded and synthetic (see learned_block_sparse_amd.synth).  The
oracle sees host copies of exactly the same bits.  Block ids must match
exactly; outputs within the tolerances in parity_helpers.
"""
import math

import numpy as np
import pytest
import torch

from parity_helpers import (compare_ids, compare_outputs, gpu_prefill, host, oracle_prefill_rows,
                            sample_rows, say)

pytestmark = pytest.mark.gpu


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


def _full_prefill_check(msa, oracle, inp, wl, what, num_splits=0):
    say(f"[parity] {what}: L={inp['cu_k_host'][-1]} splits={num_splits}")
    ids, out, lse = gpu_prefill(msa, inp, wl, num_splits=num_splits)
    torch.cuda.synchronize()
    cu = inp["cu_q_host"]
    ref_ids, ref_out, ref_lse = oracle.prefill(host(inp["q_idx"]), host(inp["k_idx"]), host(inp["q"]),
                                               host(inp["k"]), host(inp["v"]), cu, cu, wl.block_size, wl.topk)
    compare_ids(ids, ref_ids, what)
    compare_outputs(out, lse, ref_out, ref_lse, wl.dtype, what)
    return ids, out, lse


def test_tiny_prefill_2k_f32(msa, synth, oracle_lib):
    """batch 1, L=2048, 8 Q / 2 KV heads, d_idx 64, top-k 4, fp32: every row."""
    wl = synth.WORKLOADS["tiny_prefill_2k_f32"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=0)
    _full_prefill_check(msa, oracle_lib, inp, wl, "tiny fp32 2K")


@pytest.mark.parametrize("L", [128, 129, 1000, 2048 + 37])
def test_bf16_prefill_small_ragged(msa, synth, oracle_lib, L):
    """Measured head config (64/4, d_idx 128, k 16) at lengths with ragged tails."""
    wl = synth.WORKLOADS["prefill_32k"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=1, seq_lens=[L])
    _full_prefill_check(msa, oracle_lib, inp, wl, f"bf16 L={L}")


@pytest.mark.parametrize("num_splits", [0, 1])
def test_bf16_prefill_varlen_chunks(msa, synth, oracle_lib, num_splits):
    """Several sequences in one call, with q_len < kv_len (chunks of longer
    prefills, bottom-right aligned) including a single-query sequence; both
    the automatic (KV-outer) and the query-outer schedule."""
    wl = synth.WORKLOADS["prefill_32k"]
    kv, ql = [3000, 1000, 300, 700], [1517, 1000, 1, 129]
    say(f"[parity] varlen kv={kv} q={ql} splits={num_splits}")
    inp = synth.prefill_inputs(wl, device="cuda", seed=2, seq_lens=kv, q_lens=ql)
    cu_q, cu_k = inp["cu_q_host"], inp["cu_k_host"]
    ids = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], inp["cu_seqlens_q"], inp["cu_seqlens_k"], max(ql),
                             max(kv), wl.block_size, wl.topk)
    out, lse = msa.msa_sparse_attn_prefill(inp["q"], inp["k"], inp["v"], ids, inp["cu_seqlens_q"],
                                           inp["cu_seqlens_k"], max(ql), max(kv), wl.block_size, wl.topk,
                                           num_splits=num_splits)
    torch.cuda.synchronize()
    ref_ids, ref_out, ref_lse = oracle_lib.prefill(host(inp["q_idx"]), host(inp["k_idx"]), host(inp["q"]),
                                                   host(inp["k"]), host(inp["v"]), cu_q, cu_k, wl.block_size,
                                                   wl.topk)
    compare_ids(ids, ref_ids, "varlen")
    compare_outputs(out, lse, ref_out, ref_lse, "bf16", "varlen")


def test_kvouter_matches_query_outer(msa, synth):
    """The KV-outer schedule (automatic for large prefills) and the query-outer
    schedule agree to bf16 rounding on the same selection."""
    wl = synth.WORKLOADS["prefill_32k"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=9, seq_lens=[5000])
    say("[parity] kv-outer vs query-outer")
    ids, out_kv, lse_kv = gpu_prefill(msa, inp, wl, num_splits=0)
    _, out_q, lse_q = gpu_prefill(msa, inp, wl, num_splits=1)
    torch.cuda.synchronize()
    assert (out_kv.float() - out_q.float()).abs().max().item() <= 2 * 2.0 ** -8
    assert (lse_kv - lse_q).abs().max().item() <= 1e-4


@pytest.mark.parametrize("topk", [1, 2, 5, 16])
def test_topk_values_f32(msa, synth, oracle_lib, topk):
    """k = 1 (local block only), small k, and the deployed 16, in fp32."""
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["tiny_prefill_2k_f32"], topk=topk)
    inp = synth.prefill_inputs(wl, device="cuda", seed=3, seq_lens=[1500])
    _full_prefill_check(msa, oracle_lib, inp, wl, f"f32 topk={topk}")


def test_tie_dense_index_inputs(msa, synth, oracle_lib):
    """Index values in {-1/8, 0, 1/8}: many equal block scores, so the lowest-id
    tie-break decides most selections."""
    wl = synth.WORKLOADS["prefill_32k"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=4, seq_lens=[3000])
    g = torch.Generator(device="cuda").manual_seed(44)
    inp["q_idx"] = (torch.randint(-1, 2, inp["q_idx"].shape, generator=g, device="cuda").float() / 8).bfloat16()
    inp["k_idx"] = (torch.randint(-1, 2, inp["k_idx"].shape, generator=g, device="cuda").float() / 8).bfloat16()
    _full_prefill_check(msa, oracle_lib, inp, wl, "tie-dense")


@pytest.mark.parametrize("splits", [2, 3, 16])
def test_prefill_splits_and_combine(msa, synth, oracle_lib, splits):
    """Selections split into chunks and merged by the LSE combine: same ids,
    outputs within tolerance of the oracle and of the unsplit run."""
    wl = synth.WORKLOADS["prefill_32k"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=5, seq_lens=[2500])
    ids1, out1, lse1 = gpu_prefill(msa, inp, wl, num_splits=1)
    ids, out, lse = _full_prefill_check(msa, oracle_lib, inp, wl, f"splits={splits}", num_splits=splits)
    assert torch.equal(ids, ids1)
    assert (out.float() - out1.float()).abs().max().item() <= 2 * 2.0 ** -8
    assert (lse - lse1).abs().max().item() <= 1e-5


def test_determinism(msa, synth):
    wl = synth.WORKLOADS["prefill_32k"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=6, seq_lens=[4096 + 5])
    say("[parity] determinism")
    a = gpu_prefill(msa, inp, wl)
    b = gpu_prefill(msa, inp, wl)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _decode_check(msa, oracle, synth, wl, ctx, what, seed=7, seqs=None, num_splits=0):
    say(f"[parity] {what}: ctx={ctx if len(ctx) < 12 else str(len(ctx)) + ' seqs'} splits={num_splits}")
    inp = synth.decode_inputs(wl, device="cuda", seed=seed, ctx_lens=ctx)
    B = len(ctx)
    ids = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], inp["cu_seqlens_q"], inp["cu_seqlens_k"], 1, max(ctx),
                             wl.block_size, wl.topk)
    out, lse = msa.msa_sparse_attn_decode(inp["q"], inp["k"], inp["v"], ids, inp["k_offsets"], inp["ctx_lens"],
                                          max(ctx), wl.block_size, wl.topk, num_splits=num_splits)
    torch.cuda.synchronize()
    rows = np.arange(B) if seqs is None else np.asarray(seqs)
    # compact host copies of the sampled sequences' caches only
    offs, lens = inp["k_offsets_host"], inp["ctx_lens_host"]
    sl = [slice(offs[b], offs[b] + lens[b]) for b in rows]
    kc = torch.cat([inp["k"][s] for s in sl]).cpu()
    vc = torch.cat([inp["v"][s] for s in sl]).cpu()
    kic = torch.cat([inp["k_idx"][s] for s in sl]).cpu()
    new_offs = np.concatenate([[0], np.cumsum([lens[b] for b in rows])[:-1]])
    sel_rows = torch.as_tensor(rows, device=inp["q"].device)
    ref_ids, ref_out, ref_lse = oracle.decode(host(inp["q_idx"][sel_rows]), kic, host(inp["q"][sel_rows]), kc, vc,
                                              new_offs, [lens[b] for b in rows], wl.block_size, wl.topk)
    compare_ids(ids[torch.as_tensor(rows, device=ids.device)], ref_ids, what)
    compare_outputs(out[torch.as_tensor(rows, device=out.device)], lse[torch.as_tensor(rows, device=lse.device)],
                    ref_out, ref_lse, wl.dtype, what)
    return inp, ids, out, lse


@pytest.mark.parametrize("splits", [0, 1, 4])
def test_decode_ragged_small(msa, synth, oracle_lib, splits):
    """Ragged decode batch including ctx = 1, block-boundary +-1, and contexts
    shorter than the budget."""
    wl = synth.WORKLOADS["decode_1m"]
    ctx = [1, 127, 128, 129, 2047, 2048, 2049, 5000, 20000, 70001]
    _decode_check(msa, oracle_lib, synth, wl, ctx, "decode small", num_splits=splits)


def _handmade_selection(rng, pos, G, topk, block):
    """Unsorted selections with a repeated id, -1 holes and ids past the local
    block: the attention must use exactly the set of valid blocks in each."""
    sel = np.full((len(pos), G, topk), -1, dtype=np.int32)
    for r, p in enumerate(pos):
        local = int(p) // block
        for g in range(G):
            ids = rng.integers(0, local + 3, size=topk)
            ids[rng.random(topk) < 0.2] = -1
            if topk > 2:
                ids[1] = ids[0]
            sel[r, g] = ids
    return sel


@pytest.mark.parametrize("splits", [0, 1, 4])
def test_decode_attention_handmade_selection(msa, synth, oracle_lib, splits):
    """Decode attention on hand-made selections, with the selection split into
    one chunk per block (splits 0 here), one chunk, or four."""
    wl = synth.WORKLOADS["decode_1m"]
    ctx = [1, 200, 1000, 4097, 9000]
    say(f"[parity] decode hand-made selections ctx={ctx} splits={splits}")
    inp = synth.decode_inputs(wl, device="cuda", seed=11, ctx_lens=ctx)
    pos = np.asarray(ctx, dtype=np.int64) - 1
    sel = _handmade_selection(np.random.default_rng(11), pos, wl.num_kv_heads, wl.topk, wl.block_size)
    sel[0, 0, :] = -1  # a (row, group) with nothing to attend
    ids = torch.as_tensor(sel, device="cuda")
    out, lse = msa.msa_sparse_attn_decode(inp["q"], inp["k"], inp["v"], ids, inp["k_offsets"], inp["ctx_lens"],
                                          max(ctx), wl.block_size, wl.topk, num_splits=splits)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_lib.sparse_attn(host(inp["q"]), host(inp["k"]), host(inp["v"]), sel,
                                              np.asarray(inp["k_offsets_host"], dtype=np.int64), pos,
                                              np.arange(len(ctx)), wl.block_size, wl.topk)
    compare_outputs(out, lse, ref_out, ref_lse, wl.dtype, "decode hand-made")


@pytest.mark.parametrize("splits", [0, 1, 16])
def test_prefill_attention_handmade_selection(msa, synth, oracle_lib, splits):
    """Prefill attention (KV-outer for splits 0, query-outer otherwise) on
    hand-made selections."""
    wl = synth.WORKLOADS["prefill_32k"]
    L = 1500
    say(f"[parity] prefill hand-made selections L={L} splits={splits}")
    inp = synth.prefill_inputs(wl, device="cuda", seed=12, seq_lens=[L])
    pos = np.arange(L, dtype=np.int64)
    sel = _handmade_selection(np.random.default_rng(12), pos, wl.num_kv_heads, wl.topk, wl.block_size)
    ids = torch.as_tensor(sel, device="cuda")
    out, lse = msa.msa_sparse_attn_prefill(inp["q"], inp["k"], inp["v"], ids, inp["cu_seqlens_q"],
                                           inp["cu_seqlens_k"], L, L, wl.block_size, wl.topk, num_splits=splits)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_lib.sparse_attn(host(inp["q"]), host(inp["k"]), host(inp["v"]), sel,
                                              np.zeros(L, dtype=np.int64), pos, pos, wl.block_size, wl.topk)
    compare_outputs(out, lse, ref_out, ref_lse, wl.dtype, "prefill hand-made")


@pytest.mark.parametrize("max_kv_len", [2100, 1 << 18, 1 << 20])
def test_prefill_attention_bucket_table_sizes(msa, synth, oracle_lib, max_kv_len):
    """KV-outer edge lists with (sequence, group, block) bucket counts below,
    well above the 8,192 an older table held, and above the 32,768 the LDS table
    holds (one global atomic per entry there): a ragged batch of three with
    hand-made selections, max_kv_len passed as a loose upper bound."""
    wl = synth.WORKLOADS["prefill_32k"]
    lens = [1500, 700, 2100]
    nbk = len(lens) * wl.num_kv_heads * -(-max_kv_len // wl.block_size)
    say(f"[parity] prefill buckets: lens={lens} max_kv_len={max_kv_len} buckets={nbk}")
    inp = synth.prefill_inputs(wl, device="cuda", seed=13, seq_lens=lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    pos = np.concatenate([np.arange(n) for n in lens]).astype(np.int64)
    kstart = np.concatenate([np.full(n, s) for n, s in zip(lens, starts)]).astype(np.int64)
    sel = _handmade_selection(np.random.default_rng(13), pos, wl.num_kv_heads, wl.topk, wl.block_size)
    ids = torch.as_tensor(sel, device="cuda")
    out, lse = msa.msa_sparse_attn_prefill(inp["q"], inp["k"], inp["v"], ids, inp["cu_seqlens_q"],
                                           inp["cu_seqlens_k"], max(lens), max_kv_len, wl.block_size, wl.topk)
    torch.cuda.synchronize()
    rows = np.arange(sum(lens), dtype=np.int64)
    ref_out, ref_lse = oracle_lib.sparse_attn(host(inp["q"]), host(inp["k"]), host(inp["v"]), sel, kstart, pos,
                                              rows, wl.block_size, wl.topk)
    compare_outputs(out, lse, ref_out, ref_lse, wl.dtype, f"prefill buckets max_kv_len={max_kv_len}")


def test_decode_tie_dense_index_inputs(msa, synth, oracle_lib):
    """Decode rows whose index values lie in {-1/8, 0, 1/8}: block scores tie
    often, so the decode selection's search over the high words of the thread
    maxima ends on ties, its exact fallback runs, and the lowest-id tie-break
    decides most selections."""
    wl = synth.WORKLOADS["decode_1m"]
    ctx = [129, 2049, 20000, 70001]
    say(f"[parity] tie-dense decode ctx={ctx}")
    d = synth.decode_inputs(wl, device="cuda", seed=46, ctx_lens=ctx)
    g = torch.Generator(device="cuda").manual_seed(47)
    q = (torch.randint(-1, 2, d["q_idx"].shape, generator=g, device="cuda").float() / 8).bfloat16()
    k = (torch.randint(-1, 2, d["k_idx"].shape, generator=g, device="cuda").float() / 8).bfloat16()
    ids = msa.msa_index_topk(q, k, d["cu_seqlens_q"], d["cu_seqlens_k"], 1, max(ctx), wl.block_size, wl.topk)
    torch.cuda.synchronize()
    _, kstart, pos = oracle_lib.rows_decode(d["k_offsets_host"], ctx)
    ref = oracle_lib.index_topk(host(q), host(k), kstart, pos, np.arange(len(ctx)), wl.block_size, wl.topk)
    compare_ids(ids, ref, "tie-dense decode")


def test_decode_and_prefill_paths_agree(msa, synth):
    """The decode index path (block scores + select) and the prefill path
    (chunked scan + merge) give the same ids for the same newest tokens."""
    wl = synth.WORKLOADS["decode_1m"]
    ctx = [3000, 129, 9000]
    inp = synth.decode_inputs(wl, device="cuda", seed=8, ctx_lens=ctx)
    dec = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], inp["cu_seqlens_q"], inp["cu_seqlens_k"], 1, max(ctx),
                             wl.block_size, wl.topk)
    # the same query rows as a prefill call with q_len 2 (pad row before each)
    qi = torch.stack([inp["q_idx"], inp["q_idx"]], dim=1).reshape(-1, *inp["q_idx"].shape[1:]).contiguous()
    cu_q = torch.arange(0, 2 * len(ctx) + 1, 2, dtype=torch.int32, device="cuda")
    pre = msa.msa_index_topk(qi, inp["k_idx"], cu_q, inp["cu_seqlens_k"], 2, max(ctx), wl.block_size, wl.topk)
    torch.cuda.synchronize()
    assert torch.equal(dec, pre[1::2])


# ---------------------------------------------------------------- full sizes
def test_fullsize_prefill_32k_sampled(msa, synth, oracle_lib):
    """batch 1, L=32768, 64/4, k=16, 32 planted blocks: one call; sampled rows."""
    wl = synth.WORKLOADS["prefill_32k"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=0)
    say("[parity] full 32K prefill")
    ids, out, lse = gpu_prefill(msa, inp, wl)
    torch.cuda.synchronize()
    rows = sample_rows(0, wl.seq_len, wl.block_size, np.random.default_rng(0))
    ref_ids, ref_out, ref_lse = oracle_prefill_rows(oracle_lib, inp, wl, rows)
    r = torch.as_tensor(rows, device="cuda")
    compare_ids(ids[r], ref_ids, "32K")
    compare_outputs(out[r], lse[r], ref_out, ref_lse, "bf16", "32K")
    # properties at every row: local block present, ids ascending, count
    pos = torch.arange(wl.seq_len, device="cuda")
    local = (pos // wl.block_size)[:, None]
    assert bool((ids == local[:, :, None]).any(-1).all())
    valid = ids >= 0
    assert bool((valid.sum(-1) == torch.clamp(local + 1, max=wl.topk)).all())


def test_fullsize_ids_32k_every_row(msa, synth, oracle_lib):
    """L=32768, 64/4, k=16, 32 planted blocks, the bench's one-call launch:
    block ids of every one of the 32,768 rows x 4 groups against the oracle
    (index branch only; the oracle scores every row on the host cores)."""
    wl = synth.WORKLOADS["prefill_32k"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=0, with_main=False)
    L = wl.seq_len
    say("[parity] 32K ids, every row")
    cu = inp["cu_seqlens_q"]
    ids = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], cu, cu, L, L, wl.block_size, wl.topk)
    torch.cuda.synchronize()
    rows = np.arange(L, dtype=np.int64)
    ref = oracle_lib.index_topk(host(inp["q_idx"]), host(inp["k_idx"]), np.zeros(L, dtype=np.int64), rows.copy(),
                                rows, wl.block_size, wl.topk)
    compare_ids(ids, ref, "32K every row")


@pytest.mark.parametrize("lens", [[9000, 3000, 20000, 12000], [21888, 5000, 15000]])
def test_mirror_paired_scan_ragged_batch(msa, synth, oracle_lib, lens):
    """Ragged causal batches whose index scan has two rounds of items (4
    sequences x 157 query blocks x 1 key chunk = 628; 3 x 171 = 513, an odd
    count whose middle item has no partner), so each workgroup scores an item
    and its mirror, here from another sequence: ids of every row against the
    oracle."""
    wl = synth.WORKLOADS["prefill_32k"]
    say(f"[parity] mirror-paired scan, ragged batch {lens}")
    inp = synth.prefill_inputs(wl, device="cuda", seed=51, seq_lens=lens, with_main=False)
    ids = msa.msa_index_topk(inp["q_idx"], inp["k_idx"], inp["cu_seqlens_q"], inp["cu_seqlens_k"], max(lens),
                             max(lens), wl.block_size, wl.topk)
    torch.cuda.synchronize()
    rows, kstart, pos = oracle_lib.rows_prefill(inp["cu_q_host"], inp["cu_k_host"])
    ref = oracle_lib.index_topk(host(inp["q_idx"]), host(inp["k_idx"]), kstart, pos, rows, wl.block_size, wl.topk)
    compare_ids(ids, ref, "mirror-paired ragged batch")


def test_fullsize_ids_128k_every_tile_edge(msa, synth, oracle_lib):
    """L=131072 in 8192-query calls against the causal prefix (the bench's
    launches): ids of the first and last query block (128 rows each) of every
    one of the 16 calls, all 4 groups, against the oracle."""
    wl = synth.WORKLOADS["prefill_128k"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=0, with_main=False)
    T, B = wl.q_tile, wl.block_size
    got, rows = [], []
    for lo in range(0, wl.seq_len, T):
        hi = lo + T
        say(f"[parity] 128K ids, call [{lo}, {hi})")
        cu_q = torch.tensor([0, T], dtype=torch.int32, device="cuda")
        cu_k = torch.tensor([0, hi], dtype=torch.int32, device="cuda")
        ids = msa.msa_index_topk(inp["q_idx"][lo:hi], inp["k_idx"], cu_q, cu_k, T, hi, wl.block_size, wl.topk)
        edge = torch.cat([ids[:B], ids[T - B:]])
        got.append(edge.cpu())
        rows.append(np.r_[lo:lo + B, hi - B:hi])
    rows = np.concatenate(rows).astype(np.int64)
    ref = oracle_lib.index_topk(host(inp["q_idx"]), host(inp["k_idx"]), np.zeros(len(rows), dtype=np.int64),
                                rows.copy(), rows, wl.block_size, wl.topk)
    compare_ids(torch.cat(got), ref, "128K tile edges")


@pytest.mark.parametrize("tile", [0, 7, 15])
def test_fullsize_prefill_128k_tiles(msa, synth, oracle_lib, tile):
    """L=131072 in 8192-query tiles against the full causal prefix: the first,
    a middle and the last (heaviest) tile; sampled rows."""
    wl = synth.WORKLOADS["prefill_128k"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=0)
    lo, hi = tile * wl.q_tile, (tile + 1) * wl.q_tile
    say(f"[parity] 128K tile {tile}: rows [{lo}, {hi})")
    ids, out, lse = gpu_prefill(msa, inp, wl, lo, hi)
    torch.cuda.synchronize()
    rows = sample_rows(lo, hi, wl.block_size, np.random.default_rng(tile), n_blocks=1, extra=16)
    ref_ids, ref_out, ref_lse = oracle_prefill_rows(oracle_lib, inp, wl, rows, lo, hi)
    r = torch.as_tensor(rows - lo, device="cuda")
    compare_ids(ids[r], ref_ids, f"128K tile {tile}")
    compare_outputs(out[r], lse[r], ref_out, ref_lse, "bf16", f"128K tile {tile}")


def test_fullsize_decode_1m(msa, synth, oracle_lib):
    """32 sequences, contexts uniform in [64K, 1M]: outputs of sampled
    sequences, block ids of every sequence."""
    wl = synth.WORKLOADS["decode_1m"]
    ctx = synth.decode_ctx_lens(wl, 0)
    seqs = [int(np.argmin(ctx)), int(np.argmax(ctx)), 3, 11, 20, 31]
    inp, ids, _, _ = _decode_check(msa, oracle_lib, synth, wl, ctx, "decode 1M", seed=0, seqs=sorted(set(seqs)))
    _, kstart, pos = oracle_lib.rows_decode(inp["k_offsets_host"], ctx)
    ref = oracle_lib.index_topk(host(inp["q_idx"]), host(inp["k_idx"]), kstart, pos, np.arange(len(ctx)),
                                wl.block_size, wl.topk)
    compare_ids(ids, ref, "decode 1M, every sequence")


def test_decode_beyond_one_round_of_blocks(msa, synth, oracle_lib):
    """Contexts past 8192 earlier blocks (over 1M tokens): the decode selection
    runs several rounds and carries its best keys across them; with planted
    blocks so that winners sit in different rounds."""
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["decode_1m"], planted=64)
    ctx = [1_300_000, 8193 * 128 + 1, 5000]
    _decode_check(msa, oracle_lib, synth, wl, ctx, "decode >1M", seed=13)


def test_fullsize_ids_1m_three_tiles(msa, synth, oracle_lib):
    """L=1048576, 256 planted blocks, the bench's 8192-query calls: block ids
    of the first and last 8 rows and 8 random rows of the first, the 64th and
    the last call, all 4 groups, against the oracle (index branch only)."""
    wl = synth.WORKLOADS["prefill_1m"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=0, with_main=False)
    T = wl.q_tile
    rng = np.random.default_rng(2)
    got, rows = [], []
    for lo in (0, 63 * T, wl.seq_len - T):
        hi = lo + T
        say(f"[parity] 1M ids, call [{lo}, {hi})")
        cu_q = torch.tensor([0, T], dtype=torch.int32, device="cuda")
        cu_k = torch.tensor([0, hi], dtype=torch.int32, device="cuda")
        ids = msa.msa_index_topk(inp["q_idx"][lo:hi], inp["k_idx"], cu_q, cu_k, T, hi, wl.block_size, wl.topk)
        r = np.array(sorted(set(range(8)) | set(range(T - 8, T)) | set(int(x) for x in rng.integers(0, T, 8))))
        got.append(ids[torch.as_tensor(r, device="cuda")].cpu())
        rows.append(lo + r)
    rows = np.concatenate(rows).astype(np.int64)
    ref = oracle_lib.index_topk(host(inp["q_idx"]), host(inp["k_idx"]), np.zeros(len(rows), dtype=np.int64),
                                rows.copy(), rows, wl.block_size, wl.topk)
    compare_ids(torch.cat(got), ref, "1M three calls")


def test_fullsize_prefill_1m_last_tile(msa, synth, oracle_lib):
    """L=1048576, 256 planted blocks: the last 8192-query tile against the whole
    1M prefix (8191 earlier blocks per query); sampled rows."""
    wl = synth.WORKLOADS["prefill_1m"]
    inp = synth.prefill_inputs(wl, device="cuda", seed=0)
    lo, hi = wl.seq_len - wl.q_tile, wl.seq_len
    say(f"[parity] 1M last tile rows [{lo}, {hi})")
    ids, out, lse = gpu_prefill(msa, inp, wl, lo, hi)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.array(sorted(set(range(lo, lo + 8)) | set(range(hi - 8, hi))
                           | set(int(x) for x in rng.integers(lo, hi, 16))), dtype=np.int64)
    ref_ids, ref_out, ref_lse = oracle_prefill_rows(oracle_lib, inp, wl, rows, lo, hi)
    r = torch.as_tensor(rows - lo, device="cuda")
    compare_ids(ids[r], ref_ids, "1M last tile")
    compare_outputs(out[r], lse[r], ref_out, ref_lse, "bf16", "1M last tile")
