"""Turn rocprofv3 counter passes into per-call HBM traffic for bench.py.

Usage (on the GPU host, from the repository root, after the counter passes):

    python -m learned_block_sparse_amd.profiling \
        --prefill-fetch DIR --prefill-write DIR --decode-fetch DIR --decode-write DIR \
        --copy-fetch DIR --copy-write DIR --copy-bytes 1073741824 --out profiles

Each DIR is a ``rocprofv3 --pmc FETCH_SIZE`` (or ``WRITE_SIZE``) output
directory holding ``*_counter_collection.csv``.  The copy passes calibrate the
counters: a device-to-device copy of a known size reads and writes exactly
that many bytes, so the scale factor of each counter is measured value /
known bytes.  Per-call traffic is the sum over the kernels of one library
call, averaged over the calls recorded; it is written to
``profiles/traffic.json`` with the digest of the kernel sources it was taken
on, and as a text summary.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os

# kernels of one library call, by kernel-name prefix
CALLS = {
    "attention_prefill_128k": ("kvo_zero", "kvo_bucket", "kvo_scan", "kvo_attn", "kvo_combine"),
    "attention_prefill_128k_fp8kv": ("kvo_zero", "kvo_bucket", "kvo_scan", "kvo_attn", "kvo_combine"),
    "index_prefill_128k": ("_ZN3msa16idx_scan_prefill", "idx_scan_prefill", "idx_select_prefill"),
    "index_prefill_128k_fp8": ("_ZN3msa16idx_scan_prefill", "idx_scan_prefill", "idx_select_prefill"),
    "index_decode_1m": ("_ZN3msa17idx_decode_scores", "idx_decode_scores", "idx_decode_select"),
    "attention_decode_1m": ("_ZN3msa15sparse_attn_fwd", "sparse_attn_fwd", "_ZN3msa12attn_combine",
                            "attn_combine"),
    "index_frontend_128k": ("_ZN3msa14index_frontend", "index_frontend"),
}
# the call's first kernel marks a new call
CALL_START = {"attention_prefill_128k": "kvo_zero", "attention_prefill_128k_fp8kv": "kvo_zero",
              "index_prefill_128k": "idx_scan_prefill", "index_prefill_128k_fp8": "idx_scan_prefill",
              "index_decode_1m": "idx_decode_scores", "attention_decode_1m": "sparse_attn_fwd",
              "index_frontend_128k": "index_frontend"}


def _is_bf16(name):
    """A bf16 instantiation: rocprofv3 cannot demangle the __bf16 template
    argument (DF16b) and leaves those names mangled; the others it demangles
    (and with -T cuts down to the bare function name)."""
    return "DF16b" in name or "bf16" in name


# calls of the same kernels told apart by the element type of one kernel:
# (kernel whose type decides, keep the call if that kernel is bf16)
CALL_TYPE = {"index_prefill_128k": ("idx_scan_prefill", True),
             "index_prefill_128k_fp8": ("idx_scan_prefill", False),
             "attention_prefill_128k": ("kvo_attn", True),
             "attention_prefill_128k_fp8kv": ("kvo_attn", False)}


def _rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def _matches(name, prefixes):
    return any(name.startswith(p) or p in name for p in prefixes)


def per_call_kb(rows, call):
    """Sum of the counter (KB) over each call's kernels, one entry per call."""
    calls, cur = [], None
    for r in rows:
        name = r["Kernel_Name"]
        if not _matches(name, CALLS[call]):
            continue
        if CALL_START[call] in name:
            if cur is not None:
                calls.append(cur)
            cur = []
        if cur is not None:
            cur.append((name, float(r["Counter_Value"])))
    if cur is not None:
        calls.append(cur)
    if call in CALL_TYPE:
        kernel, want_bf16 = CALL_TYPE[call]
        calls = [c for c in calls
                 if any(kernel in n and _is_bf16(n) == want_bf16 for n, _ in c)]
    return [sum(v for _, v in c) for c in calls]


def per_kernel_kb(rows):
    agg = collections.defaultdict(list)
    for r in rows:
        agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def copy_factor(rows, nbytes):
    vals = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
    big = max(vals)  # the calibration copy is the largest copy dispatch
    return big * 1024.0 / nbytes


# readable names for the kernels rocprofv3 leaves mangled (the bf16
# instantiations: it cannot demangle the __bf16 template argument)
KERNEL_NAMES = {
    "_ZN3msa8kvo_attnIDF16bEEvNS_7KvoArgsE": "kvo_attn<bf16>", "kvo_attn": "kvo_attn<fp8e4m3>",
    "_ZN3msa16idx_scan_prefillIDF16bLi128EEEvPKT_S3_PKiS5_iiiiiiiPf": "idx_scan_prefill<bf16,128>",
    "idx_scan_prefill": "idx_scan_prefill<fp8e4m3,128>",
    "_ZN3msa17idx_decode_scoresIDF16bLi128ELb1EEEvPKT_S3_PKiS5_S5_iiiPf": "idx_decode_scores<bf16,128,lds>",
    "idx_decode_scores": "idx_decode_scores<fp8e4m3,128,lds>",
    "_ZN3msa5kl_dkIDF16bLi128EEEvNS_6KlArgsEi": "kl_dk<bf16,128>",
    "_ZN3msa7kl_lossIDF16bEEvNS_6KlArgsE": "kl_loss<bf16>",
    "_ZN3msa9kl_scoresIDF16bLi128EEEvNS_6KlArgsE": "kl_scores<bf16,128>",
    "_ZN3msa14index_frontendIDF16bDF16bLi128EEEvNS_6FeArgsE": "index_frontend<bf16,bf16,128>",
    "_ZN3msa15sparse_attn_fwdIDF16bDF16bEEvNS_14AttnKernelArgsE": "sparse_attn_fwd<bf16,bf16>",
    "_ZN3msa15sparse_attn_fwdIDF16bNS_7fp8e4m3EEEvNS_14AttnKernelArgsE": "sparse_attn_fwd<bf16,fp8e4m3>",
    "_ZN3msa12attn_combineIDF16bEEvPKfS2_PKiiliiPT_Pf": "attn_combine<bf16>",
}
OURS = ("kvo_", "idx_", "bwd_", "kl_", "fe_bwd", "index_frontend", "sparse_attn", "attn_combine")


def kernel_table(stats_csv):
    """Rows (name, calls, avg_us, min_us, max_us, total_ms, pct of all kernel
    time) of a rocprofv3 --stats kernel csv, the library's kernels only,
    largest total first."""
    rows = list(csv.DictReader(open(stats_csv)))
    total_all = sum(float(r["TotalDurationNs"]) for r in rows)
    tab = []
    for r in rows:
        n = KERNEL_NAMES.get(r["Name"], r["Name"])
        if not n.startswith(OURS):
            continue
        tab.append((n, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                    float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6,
                    100 * float(r["TotalDurationNs"]) / total_all))
    tab.sort(key=lambda x: -x[5])
    return tab


def kernels_main(argv):
    """``kernels --stats CSV --title T --command C --out FILE``: the kernel
    table of one rocprofv3 --kernel-trace --stats run as a text summary."""
    ap = argparse.ArgumentParser(prog="profiling kernels")
    ap.add_argument("--stats", required=True)
    ap.add_argument("--title", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--note", action="append", default=[])
    ap.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    from learned_block_sparse_amd import build
    lines = [f"# {a.title}", "", "Command (repository root, GPU host):", "  " + a.command, ""]
    lines += a.note + ([""] if a.note else [])
    lines.append(f"{'kernel':44s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_ms':>9s} {'pct':>6s}")
    for n, c, av, mn, mx, t, pc in kernel_table(a.stats):
        lines.append(f"{n[:44]:44s} {c:6d} {av:9.1f} {mn:9.1f} {mx:9.1f} {t:9.2f} {pc:6.1f}")
    lines.append("")
    lines.append("pct is of all GPU kernel time in the run, input generation included.")
    lines.append(f"kernel source digest: {build.source_digest()}")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counters_main(argv):
    """``counters --dir DIR --title T --command C --out FILE``: MFMA busy,
    wait and LDS bank conflicts per kernel from one rocprofv3 --pmc pass with
    SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_ANY
    SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE (kernel cycles = SQ_BUSY_CYCLES /
    32: the counter sums over the 32 shader engines; mfma_busy =
    SQ_VALU_MFMA_BUSY_CYCLES / (kernel cycles x 1024 SIMDs))."""
    ap = argparse.ArgumentParser(prog="profiling counters")
    ap.add_argument("--dir", required=True)
    ap.add_argument("--title", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--note", action="append", default=[])
    ap.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    from learned_block_sparse_amd import build
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    dur = collections.defaultdict(dict)  # kernel -> dispatch -> ns
    for r in _rows(a.dir):
        n = KERNEL_NAMES.get(r["Kernel_Name"], r["Kernel_Name"])
        if not n.startswith(OURS):
            continue
        per[n][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[n].add(r["Dispatch_Id"])
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            dur[n][r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    tab = []
    for n, c in per.items():
        nd = len(disp[n])
        kc = c["SQ_BUSY_CYCLES"] / 32 / nd
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / nd / (kc * 1024) if kc else 0.0
        wait = c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"] if c["SQ_WAVE_CYCLES"] else 0.0
        conf = c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"] if c["SQ_LDS_IDX_ACTIVE"] else 0.0
        ns = sum(dur[n].values()) / len(dur[n]) if dur[n] else 0.0
        ghz = kc / ns if ns > 0 else 0.0
        tab.append((n, nd, kc, busy, wait, conf, ghz))
    tab.sort(key=lambda x: -x[2])
    lines = [f"# {a.title}", "", "Command (repository root, GPU host):", "  " + a.command, ""]
    lines += a.note + ([""] if a.note else [])
    lines.append("Columns: kernel cycles = SQ_BUSY_CYCLES / 32 (the counter sums over the 32 shader engines);")
    lines.append("mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (kernel cycles x 1024 SIMDs); wait = SQ_WAIT_ANY /")
    lines.append("SQ_WAVE_CYCLES (share of wave time spent waiting); lds_conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE;")
    lines.append("GHz = kernel cycles / the dispatch's duration (its timestamps): the shader clock while the kernel ran, less any")
    lines.append("time whole shader engines sat idle (MFMA busy x kernel cycles x 1024 SIMDs x 1024 FLOP accounts for a bf16 MFMA")
    lines.append("kernel's FLOPs, so these are shader clock cycles).")
    lines.append("")
    lines.append(f"{'kernel':32s} {'disp':>5s} {'kcycles':>10s} {'mfma_busy':>10s} {'wait':>7s} {'lds_conflict':>13s} {'GHz':>6s}")
    for n, nd, kc, b, w, cf, ghz in tab:
        lines.append(f"{n[:32]:32s} {nd:5d} {kc:10.3g} {100 * b:9.1f}% {100 * w:6.1f}% {100 * cf:12.1f}% {ghz:6.2f}")
    lines.append("")
    lines.append(f"kernel source digest: {build.source_digest()}")
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    import sys
    if len(sys.argv) > 1 and sys.argv[1] == "kernels":
        kernels_main(sys.argv[2:])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        counters_main(sys.argv[2:])
        return
    ap = argparse.ArgumentParser()
    for k in ("prefill-fetch", "prefill-write", "decode-fetch", "decode-write", "copy-fetch", "copy-write"):
        ap.add_argument("--" + k, required=True)
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--out", default="profiles")
    ap.add_argument("--command", default="", help="the counter commands, recorded in the summary")
    args = ap.parse_args()

    from learned_block_sparse_amd import build
    f_fetch = copy_factor(_rows(args.copy_fetch), args.copy_bytes)
    f_write = copy_factor(_rows(args.copy_write), args.copy_bytes)
    result, lines = {}, []
    lines.append("# HBM traffic per library call (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated)")
    lines.append("")
    lines.append(f"calibration: a {args.copy_bytes} B device copy reads {f_fetch:.4f} x and writes "
                 f"{f_write:.4f} x its size in counter units; counters are divided by these factors")
    if args.command:
        lines.append("commands:")
        lines += ["  " + c for c in args.command.split(";")]
    lines.append("")
    sources = {"attention_prefill_128k": ("prefill-fetch", "prefill-write"),
               "index_prefill_128k": ("prefill-fetch", "prefill-write"),
               "index_prefill_128k_fp8": ("prefill-fetch", "prefill-write"),
               "attention_prefill_128k_fp8kv": ("prefill-fetch", "prefill-write"),
               "index_decode_1m": ("decode-fetch", "decode-write"),
               "attention_decode_1m": ("decode-fetch", "decode-write"),
               "index_frontend_128k": ("prefill-fetch", "prefill-write")}
    digest = build.source_digest()
    for call, (fd, wd) in sources.items():
        fr = _rows(getattr(args, fd.replace("-", "_")))
        wr = _rows(getattr(args, wd.replace("-", "_")))
        fk, wk = per_call_kb(fr, call), per_call_kb(wr, call)
        if not fk or not wk:
            continue
        fb = sum(fk) / len(fk) * 1024.0 / f_fetch
        wb = sum(wk) / len(wk) * 1024.0 / f_write
        result[call] = {"bytes_per_launch": fb + wb, "fetch_bytes": fb, "write_bytes": wb,
                        "calls": len(fk), "source_sha": digest}
        lines.append(f"{call:28s} calls={len(fk):3d} fetch={fb / 1e9:8.3f} GB write={wb / 1e9:8.3f} GB "
                     f"total={(fb + wb) / 1e9:8.3f} GB per call")
    lines.append("")
    lines.append("per kernel (mean per dispatch, GB):")
    for label, fd, wd in (("prefill", args.prefill_fetch, args.prefill_write),
                          ("decode", args.decode_fetch, args.decode_write)):
        fk, wk = per_kernel_kb(_rows(fd)), per_kernel_kb(_rows(wd))
        for name in sorted(fk):
            if "msa" not in name and not name.startswith(("kvo", "idx", "attn", "sparse")):
                continue
            lines.append(f"  {label:8s} {name[:60]:60s} fetch={fk[name] * 1024 / f_fetch / 1e9:8.4f} "
                         f"write={wk.get(name, 0.0) * 1024 / f_write / 1e9:8.4f}")
    lines.append(f"\nkernel source digest: {digest}")
    os.makedirs(args.out, exist_ok=True)
    with open(os.path.join(args.out, "traffic.json"), "w") as f:
        json.dump(result, f, indent=1, sort_keys=True)
    with open(os.path.join(args.out, "hbm_traffic_prefill128k_decode1m.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
