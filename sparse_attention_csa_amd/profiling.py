"""Summaries of rocprofv3 output for the hot path's kernels.

Two inputs, both written by rocprofv3 with ``--output-format csv``:

* a kernel trace (``--kernel-trace --stats``): per-kernel launch count and
  average / min / max duration;
* PMC passes of ``FETCH_SIZE`` and ``WRITE_SIZE`` (KiB per dispatch, one
  counter per run) over the benchmark, and the same two counters over a plain
  device copy of known size (``bench.py --copy-calibration MIB``).  The copy
  gives one factor per counter, bytes moved / bytes counted, which scales the
  kernels' counter values into HBM bytes per launch.

``summarize`` writes a text summary per workload and a JSON record of the
traffic per kernel, with the hash of the kernel's source so that ``bench.py``
reports the traffic only while the kernel is unchanged.

    python -m sparse_attention_csa_amd.profiling --workload decode_1m \\
        --trace DIR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \\
        --copy-mib 512 --command "..." --out OUTDIR

``--mfma-util DIR --mops DIR`` (a ``MfmaUtil`` pass and a pass of the
``SQ_INSTS_VALU_MFMA_MOPS_*`` counters) writes the MFMA utilisation summary
instead.
"""

import argparse
import collections
import csv
import glob
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# kernel name prefix -> the sources that define it (hashed together)
KERNEL_SOURCES = {
    "index_score_mfma": ["indexer_mfma.hip", "common.h", "topk.h", "kernels.h", "fold.h"],
    "index_score": ["indexer.hip", "common.h", "kernels.h"],
    "topk_": ["topk.hip", "common.h", "topk.h", "kernels.h"],
    "attend_mfma": ["attend_mfma.hip", "mfma_tile.h", "common.h", "kernels.h"],
    "attend_rows": ["attend_rows.hip", "mfma_tile.h", "common.h", "kernels.h"],
    "attend_merge": ["attend_mfma.hip", "mfma_tile.h", "common.h", "kernels.h"],
    "attend_generic": ["attend.hip", "common.h", "kernels.h"],
    "fold_append": ["compress.hip", "common.h", "kernels.h", "fold.h"],
    "compress_chunk": ["compress.hip", "common.h", "kernels.h", "fold.h"],
    "compress_slices": ["compress.hip", "common.h", "kernels.h", "fold.h"],
    "prefill_state": ["compress.hip", "common.h", "kernels.h", "fold.h"],
    "prep_rows": ["compress.hip", "common.h", "kernels.h", "fold.h"],
}


def short_name(full):
    """'void csa::attend_mfma_kernel<true>(csa::AttendArgs, int, int)' ->
    'attend_mfma_kernel<true>'"""
    n = full.split("(")[0]
    if n.startswith("void "):
        n = n[5:]
    return n.replace("csa::", "").strip()


def source_hash(kernel):
    for prefix, files in KERNEL_SOURCES.items():
        if kernel.startswith(prefix):
            h = hashlib.sha256()
            for f in files:
                with open(os.path.join(CSRC, f), "rb") as fh:
                    h.update(fh.read())
            return h.hexdigest()
    return None


def _csv_rows(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def kernel_stats(trace_dir):
    """{kernel: (calls, avg_us, min_us, max_us)} from *_kernel_stats.csv, or
    from the kernel trace when no stats file exists."""
    rows = _csv_rows(trace_dir, "kernel_stats.csv")
    out = {}
    if rows:
        for r in rows:
            out[short_name(r["Name"])] = (int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                                          float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3)
        return out
    d = collections.defaultdict(list)
    for r in _csv_rows(trace_dir, "kernel_trace.csv"):
        d[short_name(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for k, v in d.items():
        out[k] = (len(v), sum(v) / len(v), min(v), max(v))
    return out


def counter_means(pmc_dir, counter):
    """{kernel: mean counter value per dispatch}"""
    d = collections.defaultdict(list)
    for r in _csv_rows(pmc_dir, "counter_collection.csv"):
        if r["Counter_Name"] == counter:
            d[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in d.items()}


def copy_factor(pmc_dir, counter, copy_bytes):
    """bytes / (counter KiB * 1024) for the largest-traffic copy dispatch."""
    m = counter_means(pmc_dir, counter)
    copies = {k: v for k, v in m.items() if "copy" in k.lower() or "elementwise" in k.lower()}
    if not copies:
        raise SystemExit(f"no copy kernel found in {pmc_dir}")
    k, v = max(copies.items(), key=lambda kv: kv[1])
    return copy_bytes / (v * 1024.0), k, v


def summarize(args):
    stats = kernel_stats(args.trace)
    fetch = counter_means(args.fetch, "FETCH_SIZE")
    write = counter_means(args.write, "WRITE_SIZE")
    cb = args.copy_mib * 1024 * 1024
    fr, fk, fv = copy_factor(args.copy_fetch, "FETCH_SIZE", cb)
    wr, wk, wv = copy_factor(args.copy_write, "WRITE_SIZE", cb)
    os.makedirs(args.out, exist_ok=True)
    lines = [f"# rocprofv3 summary: workload {args.workload}", "",
             "command (kernel trace):", f"  {args.command_trace}", "",
             "commands (counters):", f"  {args.command_pmc}", "",
             f"calibration: {args.copy_mib} MiB device copy ({fk}):",
             f"  FETCH_SIZE {fv:.1f} KiB/dispatch -> factor {fr:.4f} bytes per counted byte",
             f"  WRITE_SIZE {wv:.1f} KiB/dispatch -> factor {wr:.4f} bytes per counted byte", "",
             f"{'kernel':40s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} "
             f"{'fetch_MB':>9s} {'write_MB':>9s}"]
    traffic = {}
    for k, (n, avg, mn, mx) in sorted(stats.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        f = fetch.get(k)
        w = write.get(k)
        fb = f * 1024 * fr if f is not None else None
        wb = w * 1024 * wr if w is not None else None
        lines.append(f"{k[:40]:40s} {n:6d} {avg:9.2f} {mn:9.2f} {mx:9.2f} "
                     f"{(fb or 0) / 1e6:9.2f} {(wb or 0) / 1e6:9.2f}")
        h = source_hash(k)
        if h and fb is not None and wb is not None:
            traffic[k] = {"avg_us": avg, "fetch_bytes": fb, "write_bytes": wb,
                          "traffic_bytes": fb + wb, "source_sha256": h}
    txt = os.path.join(args.out, f"{args.workload}_kernels.txt")
    with open(txt, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    js = os.path.join(args.out, f"{args.workload}_traffic.json")
    with open(js, "w") as fh:
        json.dump({"workload": args.workload, "command_trace": args.command_trace,
                   "command_pmc": args.command_pmc,
                   "calibration": {"copy_mib": args.copy_mib, "fetch_factor": fr, "write_factor": wr,
                                   "copy_kernel": fk},
                   "kernels": traffic}, fh, indent=1)
    print("\n".join(lines))
    print(f"wrote {txt} and {js}")


MOPS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F6F4")


def summarize_mfma(args):
    """MFMA utilisation per kernel: the derived MfmaUtil (percent of the
    time the matrix cores are busy, summed over the SIMDs over GPU-active
    cycles times the SIMD count) and the MFMA operation counts (512 FLOP
    per counted op, as the derived MfmaFlops* counters define them), with
    the trace's average duration for the achieved rate."""
    stats = kernel_stats(args.trace)
    util = counter_means(args.mfma_util, "MfmaUtil")
    mops = {c: counter_means(args.mops, c) for c in MOPS}
    lines = [f"# rocprofv3 MFMA summary: workload {args.workload}", "",
             "commands:", f"  {args.command_pmc}", "",
             "MfmaUtil = sum over SIMDs of SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE max * SIMDs) * 100;",
             "flop = 512 * SQ_INSTS_VALU_MFMA_MOPS_<type> per dispatch; rate over the trace's average duration", "",
             f"{'kernel':40s} {'avg_us':>9s} {'MfmaUtil%':>10s} {'bf16_GF':>9s} {'f8_GF':>9s} {'f6f4_GF':>9s} "
             f"{'TFLOP/s':>9s}"]
    for k in sorted(util, key=lambda k: -util[k]):
        if "at::" in k or "rocclr" in k or k not in stats:
            continue
        avg = stats[k][1]
        gf = [mops[c].get(k, 0.0) * 512 / 1e9 for c in MOPS]
        rate = sum(gf) / 1e3 / (avg / 1e6) if avg > 0 else 0.0
        lines.append(f"{k[:40]:40s} {avg:9.2f} {util[k]:10.2f} {gf[0]:9.2f} {gf[1]:9.2f} {gf[2]:9.2f} {rate:9.1f}")
    os.makedirs(args.out, exist_ok=True)
    path = os.path.join(args.out, f"{args.workload}_mfma.txt")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    print("wrote", path)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-mib", type=int)
    ap.add_argument("--mfma-util", help="MfmaUtil counter run (MFMA summary instead of traffic)")
    ap.add_argument("--mops", help="SQ_INSTS_VALU_MFMA_MOPS_* counter run")
    ap.add_argument("--command-trace", default="")
    ap.add_argument("--command-pmc", default="")
    ap.add_argument("--out", required=True)
    args = ap.parse_args()
    if args.mfma_util:
        summarize_mfma(args)
    else:
        summarize(args)


if __name__ == "__main__":
    main()
