#!/usr/bin/env python3
"""Benchmark of the MSA hot path on one MI355X.

A step is one pass of the whole prefill hot path over a synthetic 128K-token
sequence (batch 1, 64 Q / 4 KV heads, head dim 128, index dim 128, block 128,
k 16, 32 planted blocks), run as 16 calls of 8192 queries against the growing
causal prefix: per call, index scoring + block max-pool + top-k
(msa_index_topk) and block-sparse attention (msa_sparse_attn_prefill).  The
headline value is prefill tokens/s.  The same JSON line also carries one
decode step (32 sequences, contexts uniform in [64K, 1M]: msa_index_topk on
the decode path + msa_sparse_attn_decode) in microseconds per step.

Inputs are resident in HBM before the timed region starts.  The timed steps
issue nothing but the library calls (prefill: host clock between two device
synchronisations; decode: two HIP events around the run of steps).  Per-call
durations come from a second run of the same steps with HIP events recorded
between the calls, on the stream the calls are launched on (torch's current
stream, passed to the library).  With --two-stream the prefill step is also
timed with its 16 index calls on a second stream and each attention call
waiting for its tile's block ids, so index scoring of later tiles overlaps the
attention of earlier ones (prefill.two_stream_ms_per_step).

Roofline: algorithmic FLOPs (index: 2 * d_idx * G * Bk * l(p) per query;
attention: 4 * D * Hq * |J| per query) per call divided by the call's mean
duration, against MI355X's dense bf16 MFMA peak (2.5 PFLOP/s); decode against
HBM (8 TB/s) with the index-key scan plus selected K/V bytes.

The default run also times the other prefill lengths of the sweep the pages
measure (32K in one call; 1M in 128 calls of 8192 queries, 256 planted
blocks) and reports them under "prefill_32k" / "prefill_1m".

cpu_baseline: the CPU oracle (unchanged, as the tests use it) on this host's
cores: a stratified sample of query rows of the same 128K workload, and
(under "decode") every fourth sequence of the decode step, scaled to the
whole step by context tokens.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "MSA prefill tokens/s @128K + decode µs/step @1M ctx, % of roofline (1 GPU)"


def note(msg: str) -> None:
    """A progress line on stderr after each measured leg (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra-prefill", action="store_true",
                    help="skip the 32K and 1M prefill legs of the default 128K run")
    ap.add_argument("--workload", default="prefill_128k", choices=["prefill_128k", "prefill_32k", "prefill_1m"],
                    help="prefill workload of the headline measurement; other than the default, only the "
                         "prefill leg runs (32K: one call for the whole sequence; 1M: 128 calls of 8192 queries)")
    ap.add_argument("--two-stream", action="store_true",
                    help="also time the prefill step with its index calls on a second stream ahead of the "
                         "attention calls (reported as prefill.two_stream_ms_per_step)")
    ap.add_argument("--profile", choices=["prefill_tile", "train_tile", "frontend", "decode", "copy"],
                    help="run one workload a few times for hardware-counter collection and exit "
                         "(prefill_tile: the last 8192-query call of the 128K prefill; train_tile: that "
                         "tile's index front-end (forward and backward), index call, forward, backward and KL loss; frontend: "
                         "the index front-end over all "
                         "128K tokens; decode: one "
                         "decode step of the 1M-context batch; copy: a 1 GiB device-to-device copy "
                         "that calibrates the byte counters)")
    ap.add_argument("--profile-reps", type=int, default=3)
    return ap.parse_args()


def prefill_workload(args, msa, synth, workmodel, torch, np, wl, stream, steps, warmup, two_stream=False):
    """Set up one prefill workload on the GPU and time its step.

    A step runs the workload's query tiles in order (one call for the whole
    sequence when the workload has no tile size), each tile an index call
    (msa_index_topk) then an attention call (msa_sparse_attn_prefill) against
    the causal prefix ending at the tile.  Returns the inputs, the calls, the
    step function and the measurements."""
    dev = "cuda"
    L = wl.seq_len
    T = wl.q_tile or L
    inp = synth.prefill_inputs(wl, device=dev, seed=0)
    G, DI, Hq, D = wl.num_kv_heads, wl.index_dim, wl.num_heads, wl.head_dim
    tiles = [(lo, min(lo + T, L)) for lo in range(0, L, T)]
    # one workspace per kind, sized for the largest call (calls run in order on one stream)
    ws_i_bytes = max(msa.msa_index_topk_workspace_size(1, hi - lo, hi, G, wl.block_size, wl.topk)
                     for lo, hi in tiles)
    ws_a_bytes = max(msa.msa_sparse_attn_workspace_size(1, hi - lo, hi, Hq, G, D, wl.topk, 0) for lo, hi in tiles)
    ws_i = torch.empty(max(1, ws_i_bytes), dtype=torch.uint8, device=dev)
    ws_a = torch.empty(max(1, ws_a_bytes), dtype=torch.uint8, device=dev)
    calls = []
    for lo, hi in tiles:
        m = hi - lo
        cu_q = torch.tensor([0, m], dtype=torch.int32, device=dev)
        cu_k = torch.tensor([0, hi], dtype=torch.int32, device=dev)
        ids = torch.empty((m, G, wl.topk), dtype=torch.int32, device=dev)
        out = torch.empty((m, Hq, D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((m, Hq), dtype=torch.float32, device=dev)
        calls.append(dict(lo=lo, hi=hi, m=m, cu_q=cu_q, cu_k=cu_k, ws_i=ws_i, ws_a=ws_a, ids=ids, out=out,
                          lse=lse, q_idx=inp["q_idx"][lo:hi], q=inp["q"][lo:hi]))

    def run_step(events=None):
        for j, c in enumerate(calls):
            if events is not None:
                events[j][0].record(stream)
            msa.msa_index_topk(c["q_idx"], inp["k_idx"], c["cu_q"], c["cu_k"], c["m"], c["hi"], wl.block_size,
                               wl.topk, block_idx=c["ids"], workspace=c["ws_i"], stream=stream)
            if events is not None:
                events[j][1].record(stream)
            msa.msa_sparse_attn_prefill(c["q"], inp["k"], inp["v"], c["ids"], c["cu_q"], c["cu_k"], c["m"], c["hi"],
                                        wl.block_size, wl.topk, out=c["out"], lse=c["lse"], workspace=c["ws_a"],
                                        stream=stream)
            if events is not None:
                events[j][2].record(stream)

    # The index branch of a tile needs only q_idx / k_idx, so a step issues all
    # its index calls on a second stream (default priority) and each attention
    # call waits for its own tile's block ids: the scan of tile j + 1 runs while
    # the attention of tile j is still draining.  Steps do not overlap (the
    # second stream waits for the previous step's last attention call).
    side = torch.cuda.Stream()
    ids_ready = [torch.cuda.Event() for _ in calls]

    def run_step_pipelined():
        side.wait_stream(stream)
        for c, e in zip(calls, ids_ready):
            msa.msa_index_topk(c["q_idx"], inp["k_idx"], c["cu_q"], c["cu_k"], c["m"], c["hi"], wl.block_size,
                               wl.topk, block_idx=c["ids"], workspace=c["ws_i"], stream=side)
            e.record(side)
        for c, e in zip(calls, ids_ready):
            stream.wait_event(e)
            msa.msa_sparse_attn_prefill(c["q"], inp["k"], inp["v"], c["ids"], c["cu_q"], c["cu_k"], c["m"], c["hi"],
                                        wl.block_size, wl.topk, out=c["out"], lse=c["lse"], workspace=c["ws_a"],
                                        stream=stream)
        stream.wait_stream(side)

    def timed(step):
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        # the timed steps: nothing but the library calls between the two synchronisations
        t0 = time.perf_counter()
        for s in range(steps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    ms_step = timed(run_step)
    # opt-in: the same step with the index calls running ahead on the second
    # stream (its kernels overlap, so it is kept out of default runs, whose
    # per-kernel profiles must match the one-stream per-call timings)
    ms_step_two_stream = timed(run_step_pipelined) if two_stream else None
    # the per-call breakdown: the same steps again, with events around every call
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in calls] for _ in range(steps)]
    for s in range(steps):
        run_step(ev[s])
    torch.cuda.synchronize()
    idx_ms = np.mean([sum(ev[s][j][0].elapsed_time(ev[s][j][1]) for j in range(len(calls))) for s in range(steps)])
    att_ms = np.mean([sum(ev[s][j][1].elapsed_time(ev[s][j][2]) for j in range(len(calls))) for s in range(steps)])
    per_call_idx = [np.mean([ev[s][j][0].elapsed_time(ev[s][j][1]) for s in range(steps)]) for j in range(len(calls))]
    per_call_att = [np.mean([ev[s][j][1].elapsed_time(ev[s][j][2]) for s in range(steps)]) for j in range(len(calls))]

    idx_flops = att_flops = 0.0
    for c in calls:
        pos = np.arange(c["lo"], c["hi"])
        idx_flops += workmodel.index_flops(pos, G, DI, wl.block_size)
        att_flops += workmodel.attn_flops(pos, Hq, D, wl.block_size, wl.topk)

    # planted-block share of the selections (workload skew), last tile
    last = calls[-1]
    planted = set(inp["planted"][0]) if inp["planted"] else set()
    sel = last["ids"].cpu().numpy()
    local = (np.arange(last["lo"], last["hi"]) // wl.block_size)[:, None, None]
    nonlocal_sel = sel[(sel >= 0) & (sel != local)]
    planted_share = float(np.isin(nonlocal_sel, list(planted)).mean()) if planted else 0.0
    return dict(inp=inp, calls=calls, run_step=run_step, T=T, ms_step=ms_step, ms_step_two_stream=ms_step_two_stream,
                idx_ms=float(idx_ms), att_ms=float(att_ms), per_call_idx=per_call_idx, per_call_att=per_call_att,
                idx_flops=idx_flops, att_flops=att_flops, planted_share=planted_share)


def prefill_summary(wl, P):
    """The JSON record of a prefill workload measured by prefill_workload."""
    ms = P["ms_step"]
    flops = P["idx_flops"] + P["att_flops"]
    idx_t = P["idx_flops"] / (P["idx_ms"] / 1e3) / 1e12
    att_t = P["att_flops"] / (P["att_ms"] / 1e3) / 1e12
    return {"seq_len": wl.seq_len, "q_tile": P["T"], "calls": len(P["calls"]), "planted_blocks": wl.planted,
            "ms_per_step": round(ms, 3), "tokens_s": round(wl.seq_len / (ms / 1e3), 1),
            "total_tflops": round(flops / (ms / 1e3) / 1e12, 1),
            "frac_mfma": round(flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "index_ms": round(P["idx_ms"], 3), "attention_ms": round(P["att_ms"], 3),
            "index_frac_mfma": round(idx_t / PEAK_BF16_TFLOPS, 4),
            "attention_frac_mfma": round(att_t / PEAK_BF16_TFLOPS, 4), "algorithmic_flops": flops,
            "planted_share_last_tile": round(P["planted_share"], 3)}


def traffic_record(kernel_key):
    """HBM bytes per launch measured with rocprofv3 counters, if the kernel
    source is unchanged since they were taken (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    from learned_block_sparse_amd import build
    if rec.get("source_sha") != build.source_digest():
        return None
    return rec.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the MSA path here is a "
              "single-GPU library and no multi-GPU figure is produced", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from learned_block_sparse_amd import msa, synth, workmodel

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    msa.lib()
    dev = "cuda"
    stream = torch.cuda.current_stream()
    if args.profile:
        profile_run(args, msa, synth, torch)
        return

    # ------------------------------------------------------------------ prefill
    wl = synth.WORKLOADS[args.workload]
    L = wl.seq_len
    G, DI, Hq, D = wl.num_kv_heads, wl.index_dim, wl.num_heads, wl.head_dim
    P = prefill_workload(args, msa, synth, workmodel, torch, np, wl, stream, args.steps, args.warmup,
                         two_stream=args.two_stream)
    inp, calls, run_step, T = P["inp"], P["calls"], P["run_step"], P["T"]
    ms_step, ms_step_two_stream = P["ms_step"], P["ms_step_two_stream"]
    idx_ms, att_ms, per_call_idx, per_call_att = P["idx_ms"], P["att_ms"], P["per_call_idx"], P["per_call_att"]
    idx_flops, att_flops = P["idx_flops"], P["att_flops"]
    tokens_s = L / (ms_step / 1e3)
    idx_tflops = idx_flops / (idx_ms / 1e3) / 1e12
    att_tflops = att_flops / (att_ms / 1e3) / 1e12
    tot_tflops = (idx_flops + att_flops) / (ms_step / 1e3) / 1e12
    planted_share = P["planted_share"]

    dominant = "index" if idx_ms >= att_ms else "attention"
    if dominant == "index":
        dom_ms = float(np.mean(per_call_idx))
        dom_flops = idx_flops / len(calls)
        kernel = "idx_scan_prefill<bf16,128> + idx_select_prefill (one msa_index_topk call)"
        traffic = traffic_record(f"index_{args.workload}")
    else:
        dom_ms = float(np.mean(per_call_att))
        dom_flops = att_flops / len(calls)
        kernel = "kvo_attn + kvo_combine + edge-list kernels (one msa_sparse_attn_prefill call)"
        traffic = traffic_record(f"attention_{args.workload}")
    achieved = dom_flops / (dom_ms / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": kernel, "launch_ms": round(dom_ms, 4),
                "per_launch_flops": dom_flops}
    if traffic is not None:
        # the same call seen from the memory side: counted HBM bytes per second
        roofline["traffic_GBs"] = round(traffic / (dom_ms / 1e3) / 1e9, 1)
        roofline["traffic_frac_hbm"] = round(traffic / (dom_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4)

    result = {
        "metric": METRIC, "value": round(tokens_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": 1, "seq_len": L, "q_tile": T, "num_heads": Hq,
                   "num_kv_heads": G, "head_dim": D, "index_dim": DI, "block_size": wl.block_size,
                   "topk": wl.topk, "planted_blocks": wl.planted},
        "roofline": roofline,
        # the pages' own figures (H800, 1M context, against dense GQA with the same heads): context only,
        # not a target; the FLOP ratio is also recomputed from the work model used for the roofline
        "context": {"pages_prefill_speedup_vs_gqa_1m_h800": 14.2, "pages_decode_speedup_vs_gqa_1m_h800": 7.6,
                    "pages_attention_flop_cut_1m": 28.4,
                    "work_model_attention_flop_cut_1m": round(workmodel.per_token_flop_ratio(
                        1 << 20, Hq, G, D, DI, wl.block_size, wl.topk), 2)},
        "prefill": {"index_ms": round(float(idx_ms), 3), "attention_ms": round(float(att_ms), 3),
                    "index_tflops": round(idx_tflops, 1), "attention_tflops": round(att_tflops, 1),
                    "total_tflops": round(tot_tflops, 1),
                    "index_frac_mfma": round(idx_tflops / PEAK_BF16_TFLOPS, 4),
                    "attention_frac_mfma": round(att_tflops / PEAK_BF16_TFLOPS, 4),
                    "algorithmic_flops": idx_flops + att_flops,
                    "planted_share_last_tile": round(planted_share, 3)},
    }
    if ms_step_two_stream is not None:
        result["prefill"]["two_stream_ms_per_step"] = round(ms_step_two_stream, 3)
    note(f"prefill: {ms_step:.3f} ms/step")
    if args.workload != "prefill_128k":
        # the other prefill lengths: the prefill measurement alone (the decode and extra legs are sized for
        # the 128K workload)
        print(json.dumps(result), flush=True)
        return
    # ------------------------------------------------------------------ decode
    # (run right after the headline prefill measurement: the extra prefill
    # legs below allocate and free several GB, after which the 5 GB decode
    # caches measured about 3% slower)
    def decode_leg():
        if not args.no_decode:
            wd = synth.WORKLOADS["decode_1m"]
            ctx = synth.decode_ctx_lens(wd, 0)
            d = synth.decode_inputs(wd, device=dev, seed=0, ctx_lens=ctx)
            B = len(ctx)
            ws_i = torch.empty(max(1, msa.msa_index_topk_workspace_size(B, 1, max(ctx), G, wd.block_size, wd.topk)),
                               dtype=torch.uint8, device=dev)
            ws_a = torch.empty(max(1, msa.msa_sparse_attn_workspace_size(B, 1, max(ctx), Hq, G, D, wd.topk, 0)),
                               dtype=torch.uint8, device=dev)
            ids = torch.empty((B, G, wd.topk), dtype=torch.int32, device=dev)
            out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
            lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)

            def dstep(e=None):
                if e is not None:
                    e[0].record(stream)
                msa.msa_index_topk(d["q_idx"], d["k_idx"], d["cu_seqlens_q"], d["cu_seqlens_k"], 1, max(ctx),
                                   wd.block_size, wd.topk, block_idx=ids, workspace=ws_i, stream=stream)
                if e is not None:
                    e[1].record(stream)
                msa.msa_sparse_attn_decode(d["q"], d["k"], d["v"], ids, d["k_offsets"], d["ctx_lens"], max(ctx),
                                           wd.block_size, wd.topk, out=out, lse=lse, workspace=ws_a, stream=stream)
                if e is not None:
                    e[2].record(stream)

            for _ in range(5):
                dstep()
            torch.cuda.synchronize()
            # steady-state step time: events only around the whole run of steps
            e_lo, e_hi = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e_lo.record(stream)
            for s in range(args.decode_steps):
                dstep()
            e_hi.record(stream)
            torch.cuda.synchronize()
            dwall = (time.perf_counter() - t0) / args.decode_steps
            d_step_us = e_lo.elapsed_time(e_hi) * 1e3 / args.decode_steps
            # per-call breakdown from a second run with events between the calls
            dev_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.decode_steps)]
            for s in range(args.decode_steps):
                dstep(dev_ev[s])
            torch.cuda.synchronize()
            d_idx_us = float(np.mean([e[0].elapsed_time(e[1]) for e in dev_ev])) * 1e3
            d_att_us = float(np.mean([e[1].elapsed_time(e[2]) for e in dev_ev])) * 1e3
            idx_b, att_b = workmodel.decode_bytes(ctx, Hq, G, D, DI, wd.block_size, wd.topk)
            gbs = (idx_b + att_b) / (d_step_us * 1e-6) / 1e9
            idx_gbs = idx_b / (d_idx_us * 1e-6) / 1e9
            result["decode"] = {
                "workload": "decode_1m", "batch": B, "ctx_sum": int(sum(ctx)), "us_per_step": round(d_step_us, 1),
                "wall_us_per_step": round(dwall * 1e6, 1), "index_us": round(d_idx_us, 1),
                "attention_us": round(d_att_us, 1), "bytes_per_step": idx_b + att_b,
                "achieved_GBs": round(gbs, 1), "peak_GBs": PEAK_HBM_GBS, "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                "index_scan_GBs": round(idx_gbs, 1), "index_scan_frac_hbm": round(idx_gbs / PEAK_HBM_GBS, 4),
                "index_scan_traffic": traffic_record("index_decode_1m"),
            }
            # the same decode step with the index tensors in fp8 E4M3 (half the scan bytes)
            q8, k8 = d["q_idx"].to(torch.float8_e4m3fn), d["k_idx"].to(torch.float8_e4m3fn)

            def dstep8():
                msa.msa_index_topk(q8, k8, d["cu_seqlens_q"], d["cu_seqlens_k"], 1, max(ctx), wd.block_size,
                                   wd.topk, block_idx=ids, workspace=ws_i, stream=stream)
                msa.msa_sparse_attn_decode(d["q"], d["k"], d["v"], ids, d["k_offsets"], d["ctx_lens"], max(ctx),
                                           wd.block_size, wd.topk, out=out, lse=lse, workspace=ws_a, stream=stream)

            for _ in range(5):
                dstep8()
            torch.cuda.synchronize()
            e_lo.record(stream)
            for s in range(args.decode_steps):
                dstep8()
            e_hi.record(stream)
            torch.cuda.synchronize()
            d8_us = e_lo.elapsed_time(e_hi) * 1e3 / args.decode_steps
            idx8_b, _ = workmodel.decode_bytes(ctx, Hq, G, D, DI, wd.block_size, wd.topk, elem_bytes=1)
            gbs8 = (idx8_b + att_b) / (d8_us * 1e-6) / 1e9
            result["decode"]["fp8_index"] = {
                "us_per_step": round(d8_us, 1), "bytes_per_step": idx8_b + att_b, "achieved_GBs": round(gbs8, 1),
                "frac_hbm": round(gbs8 / PEAK_HBM_GBS, 4)}
            # every cache in fp8 E4M3: index keys (and index queries), K and V; bf16 q and out
            kc8, vc8 = d["k"].to(torch.float8_e4m3fn), d["v"].to(torch.float8_e4m3fn)

            def dstep_all8():
                msa.msa_index_topk(q8, k8, d["cu_seqlens_q"], d["cu_seqlens_k"], 1, max(ctx), wd.block_size,
                                   wd.topk, block_idx=ids, workspace=ws_i, stream=stream)
                msa.msa_sparse_attn_decode_ex(d["q"], kc8, vc8, ids, d["k_offsets"], d["ctx_lens"], max(ctx),
                                              wd.block_size, wd.topk, out=out, lse=lse, workspace=ws_a, stream=stream)

            for _ in range(5):
                dstep_all8()
            torch.cuda.synchronize()
            e_lo.record(stream)
            for s in range(args.decode_steps):
                dstep_all8()
            e_hi.record(stream)
            torch.cuda.synchronize()
            da8_us = e_lo.elapsed_time(e_hi) * 1e3 / args.decode_steps
            ia8_b, aa8_b = workmodel.decode_bytes(ctx, Hq, G, D, DI, wd.block_size, wd.topk, elem_bytes=1,
                                                  kv_elem_bytes=1, qo_elem_bytes=2)
            gbsa8 = (ia8_b + aa8_b) / (da8_us * 1e-6) / 1e9
            result["decode"]["fp8_index_and_kv"] = {
                "us_per_step": round(da8_us, 1), "bytes_per_step": ia8_b + aa8_b, "achieved_GBs": round(gbsa8, 1),
                "frac_hbm": round(gbsa8 / PEAK_HBM_GBS, 4)}
            if not args.no_cpu_baseline:
                cpu_decode.update(cpu_baseline_decode(d, ctx, wd, args.cpu_seconds / 2))
                note("CPU decode baseline done")
            del d, q8, k8, kc8, vc8
            torch.cuda.empty_cache()

    cpu_decode = {}
    decode_leg()
    note("decode leg done")

    # The same index calls with the index tensors rounded to fp8 E4M3 (an extra
    # measurement beside the bf16 headline; the block ids are exact for these
    # inputs on both paths, see the fp8 tests).
    q8, k8 = inp["q_idx"].to(torch.float8_e4m3fn), inp["k_idx"].to(torch.float8_e4m3fn)

    def index_fp8_step():
        for c in calls:
            msa.msa_index_topk(q8[c["lo"]:c["hi"]], k8, c["cu_q"], c["cu_k"], c["m"], c["hi"], wl.block_size,
                               wl.topk, block_idx=c["ids"], workspace=c["ws_i"], stream=stream)

    index_fp8_step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        index_fp8_step()
    e1.record(stream)
    torch.cuda.synchronize()
    idx8_ms = e0.elapsed_time(e1) / args.steps
    note("fp8 index leg done")
    result["prefill"]["index_fp8"] = {
        "ms": round(idx8_ms, 3), "tflops": round(idx_flops / (idx8_ms / 1e3) / 1e12, 1),
        "frac_fp8_mfma": round(idx_flops / (idx8_ms / 1e3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
    # The attention calls with K and V in fp8 E4M3 (bf16 q and out; the ids of
    # the calls above, which equal the bf16 ones on these inputs).
    kv8, vv8 = inp["k"].to(torch.float8_e4m3fn), inp["v"].to(torch.float8_e4m3fn)

    def attn_fp8kv_step():
        for c in calls:
            msa.msa_sparse_attn_prefill_ex(c["q"], kv8, vv8, c["ids"], c["cu_q"], c["cu_k"], c["m"], c["hi"],
                                           wl.block_size, wl.topk, out=c["out"], lse=c["lse"],
                                           workspace=c["ws_a"], stream=stream)

    attn_fp8kv_step()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        attn_fp8kv_step()
    e1.record(stream)
    torch.cuda.synchronize()
    att8_ms = e0.elapsed_time(e1) / args.steps
    note("fp8 K/V leg done")
    result["prefill"]["attention_fp8_kv"] = {
        "ms": round(att8_ms, 3), "tflops": round(att_flops / (att8_ms / 1e3) / 1e12, 1),
        "frac_mfma": round(att_flops / (att8_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    # The backward of the attention calls (an extra measurement): dq, dk, dv
    # for every tile from its forward out / lse and a seeded dO.
    dout = synth.normal(inp["q"].shape, torch.bfloat16, dev, 0, "dout")
    ws_b = torch.empty(max(1, max(msa.msa_sparse_attn_backward_workspace_size(1, c["m"], c["hi"], Hq, G, D, wl.topk)
                                  for c in calls)), dtype=torch.uint8, device=dev)
    dq_b = torch.empty((T, Hq, D), dtype=torch.float32, device=dev)
    dk_b = torch.empty((L, G, D), dtype=torch.float32, device=dev)
    dv_b = torch.empty_like(dk_b)
    run_step()  # bf16 K/V forward outputs for the backward

    def bwd_step():
        for c in calls:
            msa.msa_sparse_attn_backward(c["q"], inp["k"][:c["hi"]], inp["v"][:c["hi"]], c["out"],
                                         dout[c["lo"]:c["hi"]], c["lse"], c["ids"], c["cu_q"], c["cu_k"], c["m"],
                                         c["hi"], wl.block_size, wl.topk, dq=dq_b[:c["m"]], dk=dk_b[:c["hi"]],
                                         dv=dv_b[:c["hi"]], workspace=ws_b, stream=stream)

    bwd_step()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        bwd_step()
    e1.record(stream)
    torch.cuda.synchronize()
    bwd_ms = e0.elapsed_time(e1) / args.steps
    bwd_flops = 2.5 * att_flops  # S recomputed, dP, dV, dK, dQ: five products of the forward's size
    note("backward leg done")
    result["prefill"]["backward"] = {
        "ms": round(bwd_ms, 3), "tflops": round(bwd_flops / (bwd_ms / 1e3) / 1e12, 1),
        "frac_mfma": round(bwd_flops / (bwd_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "algorithmic_flops": bwd_flops}
    del dout, dq_b, dk_b, dv_b, ws_b
    # The index branch's KL alignment loss (an extra measurement): block LSEs
    # from the attention calls, then one msa_index_kl_backward call per tile.
    for c in calls:
        c["blse"] = torch.empty((c["m"], Hq, wl.topk), dtype=torch.float32, device=dev)
        msa.msa_sparse_attn_prefill_ex(c["q"], inp["k"], inp["v"], c["ids"], c["cu_q"], c["cu_k"], c["m"], c["hi"],
                                       wl.block_size, wl.topk, out=c["out"], lse=c["lse"], workspace=c["ws_a"],
                                       stream=stream, block_lse=c["blse"])
    ws_kl = torch.empty(max(1, max(msa.msa_index_kl_workspace_size(1, c["m"], c["hi"], G, wl.topk) for c in calls)),
                        dtype=torch.uint8, device=dev)
    kl_loss = torch.empty((T, G), dtype=torch.float32, device=dev)
    kl_dq = torch.empty((T, G, DI), dtype=torch.float32, device=dev)
    kl_dk = torch.empty((L, DI), dtype=torch.float32, device=dev)

    def kl_step():
        for c in calls:
            msa.msa_index_kl_backward(c["q_idx"], inp["k_idx"][:c["hi"]], c["ids"], c["lse"], c["blse"], c["cu_q"],
                                      c["cu_k"], c["m"], c["hi"], wl.block_size, wl.topk, loss=kl_loss[:c["m"]],
                                      dq_idx=kl_dq[:c["m"]], dk_idx=kl_dk[:c["hi"]], workspace=ws_kl,
                                      stream=stream)

    kl_step()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        kl_step()
    e1.record(stream)
    torch.cuda.synchronize()
    kl_ms = e0.elapsed_time(e1) / args.steps
    # scoring the selected blocks' attended keys: 2 d_idx per key and group
    kl_flops = att_flops / (4 * D * Hq) * 2 * DI * G
    note("KL leg done")
    result["prefill"]["index_kl"] = {"ms": round(kl_ms, 3), "tflops": round(kl_flops / (kl_ms / 1e3) / 1e12, 1),
                                     "algorithmic_flops": kl_flops}
    del inp, calls, q8, k8, kv8, vv8, kl_loss, kl_dq, kl_dk, ws_kl
    P = run_step = None
    torch.cuda.empty_cache()
    # The other prefill lengths of the pages' 32K -> 1M sweep, timed like the
    # headline: 32K in one call for the whole sequence, 1M in 128 calls of 8192
    # queries against the causal prefix (two timed steps of about 0.6 s).
    if not args.no_extra_prefill:
        for name, st, wu in (("prefill_32k", args.steps, args.warmup), ("prefill_1m", 2, 1)):
            wx = synth.WORKLOADS[name]
            Px = prefill_workload(args, msa, synth, workmodel, torch, np, wx, stream, st, wu)
            result[name] = dict(prefill_summary(wx, Px), steps=st, warmup=wu)
            del Px
            torch.cuda.empty_cache()
            note(f"{name} leg done")
    # The index front-end (an extra measurement): the whole 128K sequence's
    # hidden states through the index projections, RMS norm and RoPE in one
    # call (q_idx for every token, the index-key rows of every position).
    fe = synth.frontend_inputs(L, G, DI, synth.D_MODEL, torch.bfloat16, dev, 0)
    cu_fe = torch.tensor([0, L], dtype=torch.int32, device=dev)
    fe_q = torch.empty((L, G, DI), dtype=torch.bfloat16, device=dev)
    fe_k = torch.empty((L, DI), dtype=torch.bfloat16, device=dev)

    def fe_step():
        msa.msa_index_frontend(fe["x"], fe["w_q"], fe["w_k"], fe["gain_q"], fe["gain_k"], cu_fe, cu_fe, G,
                               rope_dim=64, q_idx=fe_q, k_idx=fe_k, stream=stream)

    fe_step()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        fe_step()
    e1.record(stream)
    torch.cuda.synchronize()
    fe_ms = e0.elapsed_time(e1) / args.steps
    fe_flops = 2.0 * L * synth.D_MODEL * (G + 1) * DI
    fe_bytes = 2.0 * (L * synth.D_MODEL + (G + 1) * DI * synth.D_MODEL + L * (G + 1) * DI)
    note("front-end leg done")
    result["prefill"]["index_frontend"] = {
        "ms": round(fe_ms, 3), "tflops": round(fe_flops / (fe_ms / 1e3) / 1e12, 1),
        "frac_mfma": round(fe_flops / (fe_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "algorithmic_flops": fe_flops, "bytes": fe_bytes, "GBs": round(fe_bytes / (fe_ms / 1e3) / 1e9, 1),
        "d_model": synth.D_MODEL, "tokens": L}
    # Its backward (an extra measurement): the projections' and gains'
    # gradients for seeded upstream gradients of q_idx / k_idx, x held constant.
    g_up = torch.Generator(device=dev)
    g_up.manual_seed(17)
    fe_dq = torch.randn((L, G, DI), generator=g_up, device=dev, dtype=torch.float32)
    fe_dk = torch.randn((L, DI), generator=g_up, device=dev, dtype=torch.float32)
    ws_feb = torch.empty(max(1, msa.msa_index_frontend_backward_workspace_size(L, synth.D_MODEL, G, DI)),
                         dtype=torch.uint8, device=dev)

    def feb_step():
        msa.msa_index_frontend_backward(fe["x"], fe["w_q"], fe["w_k"], fe["gain_q"], fe["gain_k"], cu_fe, cu_fe, G,
                                        fe_dq, fe_dk, rope_dim=64, workspace=ws_feb, stream=stream)

    feb_step()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        feb_step()
    e1.record(stream)
    torch.cuda.synchronize()
    feb_ms = e0.elapsed_time(e1) / args.steps
    # the weight-gradient contraction dW = dy^T x; y is recomputed (another fe_flops) rather than stored
    note("front-end backward leg done")
    result["prefill"]["index_frontend_backward"] = {
        "ms": round(feb_ms, 3), "tflops": round(fe_flops / (feb_ms / 1e3) / 1e12, 1),
        "tflops_with_recompute": round(2 * fe_flops / (feb_ms / 1e3) / 1e12, 1),
        "algorithmic_flops": fe_flops}
    del fe, fe_q, fe_k, fe_dq, fe_dk, ws_feb
    torch.cuda.empty_cache()

    # what this GPU reaches on a plain 1 GiB device-to-device copy (bytes read + written per second), for
    # comparison with the attention call's counted traffic rate (measured last: its 2 GiB of buffers
    # would otherwise precede the decode leg)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    result["roofline"]["copy_GBs"] = round(2 * (1 << 30) * 10 / (c0.elapsed_time(c1) / 1e3) / 1e9, 1)
    del src, dst
    # and what the vendor GEMM library reaches on a large dense bf16 product on this GPU (a calibration of the
    # MFMA rate under its sustained clock, for comparison with the index scan's fraction of peak)
    ga = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    gb = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    gc = torch.matmul(ga, gb)
    c0.record(stream)
    for _ in range(20):
        torch.matmul(ga, gb, out=gc)
    c1.record(stream)
    torch.cuda.synchronize()
    gemm_tf = 2 * 8192 ** 3 * 20 / (c0.elapsed_time(c1) / 1e3) / 1e12
    result["roofline"]["library_gemm_bf16"] = {"shape": "8192x8192x8192", "tflops": round(gemm_tf, 1),
                                               "frac": round(gemm_tf / PEAK_BF16_TFLOPS, 4)}
    del ga, gb, gc

    # ------------------------------------------------------------ CPU baseline
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        if cpu_decode:
            result["cpu_baseline"]["decode"] = cpu_decode
        note("CPU baseline done")

    print(json.dumps(result), flush=True)


def profile_run(args, msa, synth, torch):
    """One workload, repeated, for rocprofv3 counter passes (no JSON line)."""
    if args.profile == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.profile_reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"profile copy: {args.profile_reps} x {n} bytes read + written", flush=True)
        return
    if args.profile == "prefill_tile":
        wl = synth.WORKLOADS["prefill_128k"]
        inp = synth.prefill_inputs(wl, device="cuda", seed=0)
        lo, hi = wl.seq_len - wl.q_tile, wl.seq_len
        cu_q = torch.tensor([0, hi - lo], dtype=torch.int32, device="cuda")
        cu_k = torch.tensor([0, hi], dtype=torch.int32, device="cuda")
        for _ in range(args.profile_reps):
            ids = msa.msa_index_topk(inp["q_idx"][lo:hi], inp["k_idx"], cu_q, cu_k, hi - lo, hi, wl.block_size,
                                     wl.topk)
            msa.msa_sparse_attn_prefill(inp["q"][lo:hi], inp["k"], inp["v"], ids, cu_q, cu_k, hi - lo, hi,
                                        wl.block_size, wl.topk)
        torch.cuda.synchronize()
        print(f"profile prefill_tile: rows [{lo}, {hi}) x {args.profile_reps}", flush=True)
        return
    if args.profile == "train_tile":
        # the last 8192-row tile of the 128K prefill: forward with block LSEs,
        # backward of the main branch and the index KL loss
        wl = synth.WORKLOADS["prefill_128k"]
        inp = synth.prefill_inputs(wl, device="cuda", seed=0)
        lo, hi = wl.seq_len - wl.q_tile, wl.seq_len
        m = hi - lo
        cu_q = torch.tensor([0, m], dtype=torch.int32, device="cuda")
        cu_k = torch.tensor([0, hi], dtype=torch.int32, device="cuda")
        dout = synth.normal((m, wl.num_heads, wl.head_dim), torch.bfloat16, "cuda", 0, "dout")
        blse = torch.empty((m, wl.num_heads, wl.topk), dtype=torch.float32, device="cuda")
        # the tile's index front-end (its 8192 tokens at positions lo..hi-1) and its backward
        fe = synth.frontend_inputs(m, wl.num_kv_heads, wl.index_dim, synth.D_MODEL, torch.bfloat16, "cuda", 0)
        fe_k = torch.empty((hi, wl.index_dim), dtype=torch.bfloat16, device="cuda")
        fe_dq = torch.randn((m, wl.num_kv_heads, wl.index_dim), device="cuda")
        fe_dk = torch.randn((hi, wl.index_dim), device="cuda")
        for _ in range(args.profile_reps):
            msa.msa_index_frontend(fe["x"], fe["w_q"], fe["w_k"], fe["gain_q"], fe["gain_k"], cu_q, cu_k,
                                   wl.num_kv_heads, k_idx=fe_k)
            msa.msa_index_frontend_backward(fe["x"], fe["w_q"], fe["w_k"], fe["gain_q"], fe["gain_k"], cu_q, cu_k,
                                            wl.num_kv_heads, fe_dq, fe_dk)
            ids = msa.msa_index_topk(inp["q_idx"][lo:hi], inp["k_idx"], cu_q, cu_k, m, hi, wl.block_size, wl.topk)
            out, lse = msa.msa_sparse_attn_prefill_ex(inp["q"][lo:hi], inp["k"], inp["v"], ids, cu_q, cu_k, m, hi,
                                                      wl.block_size, wl.topk, block_lse=blse)
            msa.msa_sparse_attn_backward(inp["q"][lo:hi], inp["k"], inp["v"], out, dout, lse, ids, cu_q, cu_k, m, hi,
                                         wl.block_size, wl.topk)
            msa.msa_index_kl_backward(inp["q_idx"][lo:hi], inp["k_idx"], ids, lse, blse, cu_q, cu_k, m, hi,
                                      wl.block_size, wl.topk)
        torch.cuda.synchronize()
        print(f"profile train_tile: rows [{lo}, {hi}) x {args.profile_reps}", flush=True)
        return
    if args.profile == "frontend":
        wl = synth.WORKLOADS["prefill_128k"]
        L, G, DI = wl.seq_len, wl.num_kv_heads, wl.index_dim
        fe = synth.frontend_inputs(L, G, DI, synth.D_MODEL, torch.bfloat16, "cuda", 0)
        cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        q_idx = torch.empty((L, G, DI), dtype=torch.bfloat16, device="cuda")
        k_idx = torch.empty((L, DI), dtype=torch.bfloat16, device="cuda")
        for _ in range(args.profile_reps):
            msa.msa_index_frontend(fe["x"], fe["w_q"], fe["w_k"], fe["gain_q"], fe["gain_k"], cu, cu, G,
                                   rope_dim=64, q_idx=q_idx, k_idx=k_idx)
        torch.cuda.synchronize()
        print(f"profile frontend: {L} tokens x {args.profile_reps}", flush=True)
        return
    wd = synth.WORKLOADS["decode_1m"]
    ctx = synth.decode_ctx_lens(wd, 0)
    d = synth.decode_inputs(wd, device="cuda", seed=0, ctx_lens=ctx)
    for _ in range(args.profile_reps):
        ids = msa.msa_index_topk(d["q_idx"], d["k_idx"], d["cu_seqlens_q"], d["cu_seqlens_k"], 1, max(ctx),
                                 wd.block_size, wd.topk)
        msa.msa_sparse_attn_decode(d["q"], d["k"], d["v"], ids, d["k_offsets"], d["ctx_lens"], max(ctx),
                                   wd.block_size, wd.topk)
    torch.cuda.synchronize()
    print(f"profile decode: {len(ctx)} sequences, sum ctx {sum(ctx)} x {args.profile_reps}", flush=True)


def cpu_baseline(target_s: float):
    """The oracle on a stratified sample of query rows of the 128K workload."""
    import numpy as np
    import torch

    import oracle
    from learned_block_sparse_amd import synth

    wl = synth.WORKLOADS["prefill_128k"]
    inp = synth.prefill_inputs(wl, device="cpu", seed=0)
    cores = os.cpu_count() or 1
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = int(omp) if omp and omp.isdigit() else cores

    def run(n):
        rows = np.linspace(0, wl.seq_len - 1, n).astype(np.int64)
        t0 = time.perf_counter()
        oracle.prefill(inp["q_idx"], inp["k_idx"], inp["q"], inp["k"], inp["v"], inp["cu_q_host"],
                       inp["cu_k_host"], wl.block_size, wl.topk, rows=rows)
        return time.perf_counter() - t0

    n0 = max(64, 8 * threads)  # enough rows that per-call overheads do not skew the calibration
    t_cal = run(n0)
    n = int(max(n0, min(8192, n0 * target_s / max(t_cal, 1e-3))))
    t = run(n)
    # one core: the oracle's OpenMP regions limited to one thread, on a smaller sample (about half the time)
    single = None
    try:
        import ctypes
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        n1 = max(8, n // (2 * threads))
        t1 = run(n1)
        gomp.omp_set_num_threads(threads)
        single = {"value": round(n1 / t1, 2), "rows": n1, "seconds": round(t1, 1)}
    except OSError:
        pass
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    del inp
    torch.set_num_threads(torch.get_num_threads())
    return {"value": round(n / t, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} query rows evenly spaced over positions 0..131071 of the 128K prefill "
                      f"(index scan + top-k + attention per row), {t:.1f} s",
            "cpu_model": model, "single_core": single}


def cpu_baseline_decode(d, ctx, wd, target_s: float):
    """The oracle's decode step on a sample of the decode workload's sequences:
    every fourth of the 32 (their index-key, K and V caches copied from the
    GPU inputs, so the values are those the GPU step reads), repeated for
    about ``target_s`` seconds; scaled to the 32-sequence step by context
    tokens (the index-key scan, linear in the context, is nearly all the
    work)."""
    import numpy as np
    import torch

    import oracle

    B = len(ctx)
    sample = list(range(0, B, 4))
    offs, lens = d["k_offsets_host"], d["ctx_lens_host"]
    sl = [slice(offs[b], offs[b] + lens[b]) for b in sample]
    kc = torch.cat([d["k"][s] for s in sl]).cpu()
    vc = torch.cat([d["v"][s] for s in sl]).cpu()
    kic = torch.cat([d["k_idx"][s] for s in sl]).cpu()
    r = torch.as_tensor(sample, device=d["q"].device)
    qi, q = d["q_idx"][r].cpu(), d["q"][r].cpu()
    slens = [lens[b] for b in sample]
    soffs = np.concatenate([[0], np.cumsum(slens)[:-1]]).astype(np.int64)

    def run():
        t0 = time.perf_counter()
        oracle.decode(qi, kic, q, kc, vc, soffs, slens, wd.block_size, wd.topk)
        return time.perf_counter() - t0

    t_cal = run()
    reps = int(max(1, min(50, target_s / max(t_cal, 1e-3))))
    t = sum(run() for _ in range(reps)) / reps
    scale = float(sum(ctx)) / float(sum(slens))
    del kc, vc, kic
    return {"value": round(t * scale * 1e6, 1), "unit": "us/step", "higher_is_better": False,
            "sample": f"sequences {sample} of the 32 (contexts {slens}, {sum(slens)} tokens of {sum(ctx)}): "
                      f"oracle decode step (index scan + top-k + attention) {t:.3f} s, mean of {reps} runs; "
                      f"value = that time x {scale:.3f} (all contexts / sampled contexts)",
            "sample_seconds": round(t, 4)}


if __name__ == "__main__":
    main()
