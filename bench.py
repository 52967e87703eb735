"""Benchmark of the CSA/HCA hybrid-attention hot path on one MI355X.

Default workload (the metric's "@1M ctx (Flash/Pro)" decode): one step is a
Pro-shaped CSA decode layer (B=4, 1,048,576-token context = 262,144 entries,
128 heads x 512, fp8-e4m3 indexer 64 x 128, top-k 1024) followed by a
Flash-shaped HCA decode layer (B=8, 1,048,576 tokens = 8,192 entries, 64 heads
x 512).  Each layer step runs the whole hot path: fold of the block completed
by the previous token, indexer scan + top-k (CSA), attention over the
selected / all visible entries + 128-token window + sink, merge.

value = decode tokens per second per layer = (4 + 8) tokens / step time, each
token passing through one layer.  Inputs are resident in HBM before timing.
Every timed step starts from the same state (entry counts are restored between
steps, outside the timed events) and cycles through --rotate independent copies
of the state so that the working set exceeds the 256 MiB MALL.

Prints one JSON line.  Other workloads: --workload flash_csa_128k |
flash_hca_1m | pro_csa_1m | prefill.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "hybrid-attn decode tokens/s per layer @1M ctx (Flash/Pro); % HBM & MFMA roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_cases(name):
    import workloads
    if name == "decode_1m":
        return [("pro_csa_1m", workloads.pro_csa_decode()), ("flash_hca_1m", workloads.flash_hca_decode())]
    if name == "flash_csa_128k":
        return [("flash_csa_128k", workloads.flash_csa_decode())]
    if name == "flash_hca_1m":
        return [("flash_hca_1m", workloads.flash_hca_decode())]
    if name == "pro_csa_1m":
        return [("pro_csa_1m", workloads.pro_csa_decode())]
    if name == "prefill":
        a, h = workloads.flash_prefill()
        return [("prefill_csa", a), ("prefill_hca", h)]
    raise SystemExit(f"unknown workload {name}")


def attend_splits(BT, H, rows_max, heads_per_wg=64):
    """Row splits the MFMA attention uses (mirrors attend_mfma_plan, 64 heads
    per workgroup, and attend_rows_plan, 16)."""
    cols = BT * max(1, H // heads_per_wg)
    want = max(1, min(64, 256 // cols))
    rps = -(-rows_max // want)
    rps = -(-rps // 16) * 16
    if heads_per_wg == 16:
        rps = min(rps, 2304)
    return -(-rows_max // rps)


# benchmark timing-hook names -> the kernel symbols rocprofv3 reports
ROCPROF_NAMES = {
    "attend_dense_mfma": "attend_mfma_kernel",
    "attend_sparse_rows": "attend_rows_kernel",
    "topk_resolve": "topk_fused_resolve_kernel",
}


def profiled_traffic(workload, hook_name):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary, if it exists and the kernel's source is unchanged since."""
    from sparse_attention_csa_amd import profiling as P
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    want = ROCPROF_NAMES.get(hook_name)
    names = [k for k in rec["kernels"] if (k == want if want else k.startswith(hook_name + "_kernel"))]
    if len(names) != 1:
        return None
    k = names[0]
    if rec["kernels"][k]["source_sha256"] != P.source_hash(k):
        return None
    return int(rec["kernels"][k]["traffic_bytes"])


def kernel_work(kname, g):
    """(algorithmic bytes, algorithmic flops, bound, peak, unit) of one launch
    of kernel ``kname`` for workload ``g`` (see accounting.py)."""
    from sparse_attention_csa_amd import accounting as A
    B = g["B"]
    prefill = "T" in g
    Tq = g["T"] if prefill else 1
    if kname.startswith("index_score"):
        E = g["E_cap"]
        if prefill:  # causal: query i sees (pos0 + i) // m entries
            pairs = sum((g["pos0"] + i) // g["m"] for i in range(Tq))
            E_eff = pairs / Tq
        else:
            E_eff = E
        byt = A.index_scan_bytes(B, 1, E, g["H_I"], g["d_I"], g["idx_dtype"]) if not prefill else \
            A.index_scan_bytes(B, Tq, E, g["H_I"], g["d_I"], g["idx_dtype"])
        fl = A.index_scan_flops(B, Tq, E_eff, g["H_I"], g["d_I"])
        fp8 = g["idx_dtype"] == "e4m3"
        if prefill:
            return byt, fl, "mfma", A.PEAK_BF16_TFLOPS, "TFLOP/s"
        return byt, fl, "hbm", A.PEAK_HBM_GBS, "GB/s"
    if kname == "attend_merge":
        # combination of the row splits: partials in, output out (implementation
        # traffic; the algorithmic bytes are counted in the attention kernel)
        rows = (g["k"] if g["kind"] == "csa" else g["E_cap"]) + g["n_win"]
        ns = attend_splits(B * Tq, g["H"], rows, heads_per_wg=16 if g["kind"] == "csa" else 64)
        byt = B * Tq * g["H"] * (ns * (g["c"] * 2 + 8) + g["c"] * 2 + 4)
        return byt, 0.0, "hbm", A.PEAK_HBM_GBS, "GB/s"
    if kname.startswith("attend"):
        if g["kind"] == "csa":
            rows = g["k"] + g["n_win"]
        else:
            if prefill:
                rows = sum((g["pos0"] + i) // g["m"] for i in range(Tq)) / Tq + g["n_win"]
            else:
                rows = g["E_cap"] + g["n_win"]
        if prefill:
            byt = A.attend_bytes(B, Tq, g["E_cap"] if g["kind"] == "hca" else rows, g["H"], g["c"])
            return byt, A.attend_flops(B, Tq, rows, g["H"], g["c"]), "mfma", A.PEAK_BF16_TFLOPS, "TFLOP/s"
        byt = A.attend_bytes(B, 1, rows, g["H"], g["c"])
        return byt, A.attend_flops(B, 1, rows, g["H"], g["c"]), "hbm", A.PEAK_HBM_GBS, "GB/s"
    if kname.startswith("fold"):
        S = 4 if g["overlap"] else 2
        byt = A.fold_bytes(B, g["m"], g["c"], S)
        if g["kind"] == "csa":
            byt += A.fold_bytes(B, g["m"], g["d_I"], 4)
        return byt, 0.0, "hbm", A.PEAK_HBM_GBS, "GB/s"
    if kname.startswith("topk"):
        return B * Tq * g["E_cap"] * 4, 0.0, "hbm", A.PEAK_HBM_GBS, "GB/s"
    if kname.startswith("compress"):
        S = 4 if g["overlap"] else 2
        byt = B * Tq * S * g["c"] * 2
        return byt, 0.0, "hbm", A.PEAK_HBM_GBS, "GB/s"
    return 0, 0.0, "hbm", A.PEAK_HBM_GBS, "GB/s"


def cpu_baseline(cases, prefill):
    """Time the oracle (as it stands) on a bounded sample of the same work."""
    import numpy as np
    from oracle import layer as OL
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    tokens, secs, parts = 0, 0.0, []
    per_step_tokens, per_step_secs = 0, 0.0
    for name, g in cases:
        if prefill:
            t0 = time.perf_counter()
            kv_new, idx_new = OL.prefill_entries(g, 0)
            n_q = 4
            for i in np.linspace(0, g["T"] - 1, n_q).astype(int):
                OL.prefill_query(g, 0, int(i), kv_new, idx_new)
            dt = time.perf_counter() - t0
            # the chunk's compression is shared; queries scale linearly
            tokens += n_q
            parts.append(f"{name}: compress chunk + {n_q} queries")
        else:
            # whole decode steps of every sequence, repeated until about 7 s
            # of CPU work per layer (at most 64 passes)
            t0 = time.perf_counter()
            passes = 0
            while passes < 64 and (passes == 0 or time.perf_counter() - t0 < 7.0):
                for b in range(g["B"]):
                    OL.decode_step(g, b)
                passes += 1
            dt = time.perf_counter() - t0
            # one step of every layer, as the timed GPU step: the time of one
            # pass per layer, the tokens of one pass
            per_step_secs += dt / passes
            per_step_tokens += g["B"]
            tokens += g["B"] * passes
            parts.append(f"{name}: {passes} x full decode step of all {g['B']} sequences")
        secs += dt
    unit = "prefill tokens/s per layer" if prefill else "decode tokens/s per layer"
    value = tokens / secs if prefill else per_step_tokens / per_step_secs
    return {"value": value, "unit": unit, "cores": int(cores), "kind": "oracle",
            "sample": "; ".join(parts) + f" ({secs:.1f} s of CPU work)" +
                      ("" if prefill else "; value = tokens of one step of each layer / time of one step of each layer")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_1m")
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB 10 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 10}), flush=True)
        return

    from sparse_attention_csa_amd import _lib as L
    from sparse_attention_csa_amd.harness import DecodeSession, PrefillSession

    L.lib()
    prefill = args.workload == "prefill"
    t0 = time.time()
    cases = build_cases(args.workload)
    log(f"generated inputs in {time.time() - t0:.1f} s")
    rot = 1 if prefill else max(1, args.rotate)
    sessions = []
    for name, g in cases:
        S = PrefillSession if prefill else DecodeSession
        sessions.append((name, g, [S(g) for _ in range(rot)]))
    saved = [[s.state.n_entries.clone() for s in ss] for _, _, ss in sessions]
    torch.cuda.synchronize()
    log(f"uploaded {rot} state copies in {time.time() - t0:.1f} s")

    def reset(i):
        for li, (_, _, ss) in enumerate(sessions):
            ss[i % rot].state.n_entries.copy_(saved[li][i % rot])

    def step(i):
        for _, _, ss in sessions:
            ss[i % rot].run()

    for i in range(args.warmup):
        reset(i)
        step(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(args.steps):
        reset(i)
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms = sum(step_ms) / len(step_ms)
    tokens = sum(g["B"] * (g["T"] if prefill else 1) for _, g, _ in sessions)
    value = tokens / (ms / 1e3)
    log(f"steps: mean {ms:.4f} ms, min {min(step_ms):.4f} ms, wall/step {wall / args.steps * 1e3:.3f} ms")

    # per-layer times and per-kernel durations (timing hook, a separate pass)
    layers = {}
    for name, g, ss in sessions:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
        for i in range(args.steps):
            reset(i)
            ev[2 * i].record()
            ss[i % rot].run()
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        lm = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)) / args.steps
        toks = g["B"] * (g["T"] if prefill else 1)
        layers[name] = {"ms": round(lm, 5), "tokens_per_s": round(toks / (lm / 1e3), 1)}
    L.profile_enable(True)
    kern = {}
    for name, g, ss in sessions:
        L.profile_collect()
        for i in range(args.steps):
            reset(i)
            ss[i % rot].run()
        torch.cuda.synchronize()
        for kname, (n, tot) in L.profile_collect().items():
            kern[f"{name}:{kname}"] = (n, tot, g, kname)
    L.profile_enable(False)
    kernels = {}
    best = None
    for key, (n, tot, g, kname) in kern.items():
        avg = tot / n
        byt, fl, bound, peak, unit = kernel_work(kname, g)
        ach = (byt / (avg / 1e3) / 1e9) if unit == "GB/s" else (fl / (avg / 1e3) / 1e12)
        kernels[key] = {"avg_ms": round(avg, 5), "launches": n,
                        "alg_bytes": int(byt), "alg_flops": float(fl),
                        "achieved": round(ach, 2), "unit": unit, "frac": round(ach / peak, 4)}
        if best is None or tot > best[1]:
            best = (key, tot, ach, peak, unit, bound, byt)
    key, _, ach, peak, unit, bound, byt = best
    traffic = profiled_traffic(args.workload, key.split(":", 1)[1])
    roofline = {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": traffic, "kernel": key,
                "alg_bytes_per_launch": int(byt)}

    cpu = None
    if not args.no_cpu:
        log("timing the oracle on a bounded sample ...")
        cpu = cpu_baseline([(n, g) for n, g, _ in sessions], prefill)

    names = "+".join(n for n, _, _ in sessions)
    cfg = {"workload": names, "layers": list(layers.keys()),
           "batch": {n: g["B"] for n, g, _ in sessions},
           "context_tokens": {n: int(g.get("n", g.get("pos0", 0))) for n, g, _ in sessions},
           "rotate_state_copies": rot}
    out = {"metric": METRIC, "value": round(value, 2),
           "unit": "prefill tokens/s per layer" if prefill else "decode tokens/s per layer",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded; shapes of the pages' Flash/Pro configurations)",
           "config": cfg, "roofline": roofline, "cpu_baseline": cpu,
           "layer_times": layers, "kernels": kernels}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
