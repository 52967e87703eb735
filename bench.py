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
flash_hca_1m | pro_csa_1m | pro_csa_1m_mxfp4 | decode_1m_norm_rope | decode_1m_paged | prefill.
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
    if name == "pro_csa_1m_mxfp4":
        # the pages' FP4 indexer path: MXFP4 queries and keys, bf16 scores
        return [("pro_csa_1m_mxfp4", workloads.pro_csa_decode(idx_dtype="mxfp4", score_dtype="bf16"))]
    if name == "decode_1m_norm_rope":
        # the default step with the steps on either side of the core
        # attention: RMSNorm and rotary positions of queries and produced KV,
        # the output rotated back
        return [("pro_csa_1m_norm_rope", workloads.with_norm_rope(workloads.pro_csa_decode())),
                ("flash_hca_1m_norm_rope", workloads.with_norm_rope(workloads.flash_hca_decode()))]
    if name == "decode_1m_paged":
        # the default step with the compressed caches in 128-token pages
        # (32 CSA entries, one HCA entry per page), pages in random order
        return [("pro_csa_1m_paged", workloads.with_pages(workloads.pro_csa_decode(), 32, seed=31)),
                ("flash_hca_1m_paged", workloads.with_pages(workloads.flash_hca_decode(), 1, seed=32))]
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
# (prefixes: a workload's profile holds one instantiation of each)
ROCPROF_NAMES = {
    "attend_dense_mfma": "attend_mfma_kernel<",
    "attend_sparse_rows": "attend_rows_kernel<",
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
    names = [k for k in rec["kernels"] if k.startswith(want if want else hook_name + "_kernel")]
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


def layer_work(g):
    """(algorithmic bytes, algorithmic flops) of one step of layer g."""
    from sparse_attention_csa_amd import accounting as A
    if "T" in g:
        fl = A.prefill_layer_flops(g["kind"], g["T"], g["pos0"], g["m"], g["H"], g["c"], g["n_win"], g.get("k"),
                                   g.get("H_I"), g.get("d_I")) * g["B"]
        return 0, fl
    E = int(g["n_entries"][0]) + 1 if int(g["pos"][0]) % g["m"] == 0 else int(g["n_entries"][0])
    byt = A.decode_layer_bytes(g["kind"], g["B"], E, g["H"], g["c"], g["n_win"], g.get("k"), g.get("H_I"),
                               g.get("d_I"), g.get("idx_dtype"), g["m"], g["overlap"], g["kv_dtype"])
    return byt, 0.0


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            blas = "{} {} ({})".format(infos[0].get("internal_api"), infos[0].get("version"),
                                       infos[0].get("threading_layer", ""))
    except Exception:  # noqa: BLE001
        pass
    return model, blas


def cpu_baseline(cases, prefill):
    """Time the oracle (as it stands) on a bounded sample of the same work:
    three timed repetitions, the median reported."""
    import numpy as np
    from oracle import layer as OL
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    model, blas = cpu_info()
    reps = []
    parts = []
    for rep in range(3):
        tokens, secs = 0, 0.0
        for name, g in cases:
            t0 = time.perf_counter()
            if prefill:
                kv_new, idx_new = OL.prefill_entries(g, 0)
                n_q = 4
                for i in np.linspace(0, g["T"] - 1, n_q).astype(int):
                    OL.prefill_query(g, 0, int(i), kv_new, idx_new)
                tokens += n_q
                if rep == 0:
                    parts.append(f"{name}: compress chunk + {n_q} queries")
            else:
                # one whole decode step of every sequence of the layer
                for b in range(g["B"]):
                    OL.decode_step(g, b)
                tokens += g["B"]
                if rep == 0:
                    parts.append(f"{name}: one decode step of all {g['B']} sequences")
            secs += time.perf_counter() - t0
        reps.append((secs, tokens))
    secs = sorted(r[0] for r in reps)[1]
    tokens = reps[0][1]
    unit = "prefill tokens/s per layer" if prefill else "decode tokens/s per layer"
    return {"value": tokens / secs, "unit": unit, "cores": int(cores), "kind": "oracle",
            "cpu_model": model, "blas": blas, "repetitions": 3, "statistic": "median",
            "sample": "; ".join(parts) + f" (median of 3 repetitions: {secs:.2f} s); value = tokens of one "
                      "step of each layer / time of one step of each layer"}


def measure(cases, steps, warmup, rotate, prefill, profile=True, use_graph=False):
    """Time `steps` steps (every layer of `cases` once per step) after
    `warmup` untimed ones, cycling through `rotate` state copies; then each
    layer alone, and each kernel through the timing hook.  With use_graph each
    (layer, state copy) step is captured once into a HIP graph and the timed
    steps replay the graphs (the launch path of a serving loop); the kernel
    timing hook always runs eagerly."""
    import torch
    from sparse_attention_csa_amd import _lib as L
    from sparse_attention_csa_amd.harness import DecodeSession, PrefillSession

    rot = 1 if prefill else max(1, rotate)
    t0 = time.time()
    sessions = []
    for name, g in cases:
        S = PrefillSession if prefill else DecodeSession
        sessions.append((name, g, [S(g) for _ in range(rot)]))
    for _, _, ss in sessions:
        for sess in ss:
            sess.state.auto_gather = False  # (paged caches: no host-side views needed)
    saved = [[s.state.n_entries.clone() for s in ss] for _, _, ss in sessions]
    torch.cuda.synchronize()
    log(f"uploaded {rot} state copies of {'+'.join(n for n, _ in cases)} in {time.time() - t0:.1f} s")

    def reset(i):
        for li, (_, _, ss) in enumerate(sessions):
            ss[i % rot].state.n_entries.copy_(saved[li][i % rot])

    def step(i):
        for _, _, ss in sessions:
            ss[i % rot].run()

    for i in range(max(warmup, rot)):
        reset(i)
        step(i)
    torch.cuda.synchronize()
    if use_graph:
        graphs = []
        for li, (_, _, ss) in enumerate(sessions):
            gl = []
            for r, sess in enumerate(ss):
                ss[r].state.n_entries.copy_(saved[li][r])
                torch.cuda.synchronize()
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr):
                    sess.run()
                gl.append(gr)
            graphs.append(gl)
        torch.cuda.synchronize()

        def run_layer(li, i):
            graphs[li][i % rot].replay()
    else:
        def run_layer(li, i):
            sessions[li][2][i % rot].run()

    def step(i):  # noqa: F811
        for li in range(len(sessions)):
            run_layer(li, i)

    for i in range(warmup):
        reset(i)
        step(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(steps):
        reset(i)
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    ms = sum(step_ms) / len(step_ms)
    log(f"steps: mean {ms:.4f} ms, min {min(step_ms):.4f} ms, wall/step {wall / steps * 1e3:.3f} ms")

    layers = {}
    for li, (name, g, ss) in enumerate(sessions):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
        for i in range(steps):
            reset(i)
            ev[2 * i].record()
            run_layer(li, i)
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        lm = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)) / steps
        toks = g["B"] * (g["T"] if prefill else 1)
        byt, fl = layer_work(g)
        rec = {"ms": round(lm, 5), "tokens_per_s": round(toks / (lm / 1e3), 1)}
        from sparse_attention_csa_amd import accounting as A
        if prefill:
            tf = fl / (lm / 1e3) / 1e12
            rec.update(alg_tflop=round(fl / 1e12, 4), achieved_tflops=round(tf, 2), bound="mfma",
                       peak_tflops=A.PEAK_BF16_TFLOPS, frac=round(tf / A.PEAK_BF16_TFLOPS, 4))
        else:
            gbs = byt / (lm / 1e3) / 1e9
            rec.update(alg_bytes=int(byt), achieved_gbs=round(gbs, 1), bound="hbm", peak_gbs=A.PEAK_HBM_GBS,
                       frac=round(gbs / A.PEAK_HBM_GBS, 4))
        layers[name] = rec

    kernels = {}
    best = None
    if profile:
        L.profile_enable(True)
        kern = {}
        for name, g, ss in sessions:
            L.profile_collect()
            for i in range(steps):
                reset(i)
                ss[i % rot].run()
            torch.cuda.synchronize()
            for kname, (n, tot) in L.profile_collect().items():
                kern[f"{name}:{kname}"] = (n, tot, g, kname)
        L.profile_enable(False)
        for key, (n, tot, g, kname) in kern.items():
            avg = tot / n
            byt, fl, bound, peak, unit = kernel_work(kname, g)
            ach = (byt / (avg / 1e3) / 1e9) if unit == "GB/s" else (fl / (avg / 1e3) / 1e12)
            kernels[key] = {"avg_ms": round(avg, 5), "launches": n,
                            "alg_bytes": int(byt), "alg_flops": float(fl),
                            "achieved": round(ach, 2), "unit": unit, "frac": round(ach / peak, 4)}
            if best is None or tot > best[1]:
                best = (key, tot, ach, peak, unit, bound, byt, fl)
    tokens = sum(g["B"] * (g["T"] if prefill else 1) for _, g, _ in sessions)
    out = {"ms_per_step": ms, "tokens": tokens, "layers": layers, "kernels": kernels, "best": best,
           "sessions": sessions, "rot": rot, "graph": bool(use_graph)}
    if use_graph:
        del graphs
    return out


def hbm_reference(nbytes=1 << 30, reps=5):
    """What plain streaming kernels reach on this GPU, timed in the same run
    (events around torch's own kernels; median of `reps`): a device-to-device
    copy (read + write bytes) and a sum reduction (read bytes).  Context for
    the roofline fractions, which stay against the published 8 TB/s."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    out = {}
    for name, fn, moved in (("device_copy_gbs", lambda: y.copy_(x), 2 * nbytes),
                            ("sum_read_gbs", lambda: x.sum(), nbytes)):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts.sort()
        out[name] = round(moved / (ts[len(ts) // 2] / 1e3) / 1e9, 1)
    out["bytes"] = nbytes
    del x, y
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_1m")
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay each layer step from a captured HIP graph instead of launching eagerly")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra workloads measured after the headline one")
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

    L.lib()
    prefill = args.workload == "prefill"
    t0 = time.time()
    cases = build_cases(args.workload)
    log(f"generated inputs in {time.time() - t0:.1f} s")
    res = measure(cases, args.steps, args.warmup, args.rotate, prefill, use_graph=args.graph)
    ms, tokens, layers, kernels = res["ms_per_step"], res["tokens"], res["layers"], res["kernels"]
    value = tokens / (ms / 1e3)
    key, _, ach, peak, unit, bound, byt, fl = res["best"]
    traffic = profiled_traffic(args.workload, key.split(":", 1)[1])
    roofline = {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
                "frac": round(ach / peak, 4), "traffic": traffic, "kernel": key,
                "alg_bytes_per_launch": int(byt) if unit == "GB/s" else None,
                "alg_flops_per_launch": float(fl) if unit != "GB/s" else None}
    rot = res["rot"]
    sessions = res["sessions"]
    names = "+".join(n for n, _, _ in sessions)
    cfg = {"workload": names, "layers": list(layers.keys()),
           "batch": {n: g["B"] for n, g, _ in sessions},
           "context_tokens": {n: int(g.get("n", g.get("pos0", 0))) for n, g, _ in sessions},
           "rotate_state_copies": rot, "launch": "hip graph replay" if res["graph"] else "eager"}
    # the whole step against the roofline: every layer's algorithmic bytes
    # (flops for prefill) over the step time
    tot_b = sum(layer_work(g)[0] for _, g, _ in sessions)
    tot_f = sum(layer_work(g)[1] for _, g, _ in sessions)
    from sparse_attention_csa_amd import accounting as A
    if prefill:
        step_roof = {"bound": "mfma", "alg_tflop": round(tot_f / 1e12, 4),
                     "achieved_tflops": round(tot_f / (ms / 1e3) / 1e12, 2), "peak_tflops": A.PEAK_BF16_TFLOPS,
                     "frac": round(tot_f / (ms / 1e3) / 1e12 / A.PEAK_BF16_TFLOPS, 4)}
    else:
        step_roof = {"bound": "hbm", "alg_bytes": int(tot_b),
                     "achieved_gbs": round(tot_b / (ms / 1e3) / 1e9, 1), "peak_gbs": A.PEAK_HBM_GBS,
                     "frac": round(tot_b / (ms / 1e3) / 1e9 / A.PEAK_HBM_GBS, 4)}
    del res, sessions
    torch.cuda.empty_cache()

    # the other configurations, timed in the same run: the Flash-shaped CSA
    # decode at 128K context, the Pro CSA layer with the FP4 indexer and
    # bf16 scores, and the hybrid prefill chunk
    extra = {}
    if args.workload == "decode_1m" and not args.no_extra:
        for wl, steps, warm in (("flash_csa_128k", args.steps, args.warmup),
                                ("pro_csa_1m_mxfp4", args.steps, args.warmup),
                                ("decode_1m_paged", args.steps, args.warmup),
                                ("decode_1m_norm_rope", args.steps, args.warmup),
                                ("prefill", max(3, min(args.steps, 5)), 1)):
            t1 = time.time()
            c2 = build_cases(wl)
            log(f"generated {wl} inputs in {time.time() - t1:.1f} s")
            r2 = measure(c2, steps, warm, args.rotate, wl == "prefill", profile=False, use_graph=args.graph)
            ms2 = r2["ms_per_step"]
            byt2 = sum(layer_work(g)[0] for _, g in c2)
            fl2 = sum(layer_work(g)[1] for _, g in c2)
            rec = {"ms_per_step": round(ms2, 5), "tokens_per_s_per_layer": round(r2["tokens"] / (ms2 / 1e3), 1),
                   "steps": steps, "layers": r2["layers"]}
            if wl == "prefill":
                rec["unit"] = "prefill tokens/s per layer"
                rec["frac_bf16_peak"] = round(fl2 / (ms2 / 1e3) / 1e12 / A.PEAK_BF16_TFLOPS, 4)
            else:
                rec["unit"] = "decode tokens/s per layer"
                rec["frac_hbm"] = round(byt2 / (ms2 / 1e3) / 1e9 / A.PEAK_HBM_GBS, 4)
            extra[wl] = rec
            del r2, c2
            torch.cuda.empty_cache()

    ref = hbm_reference()
    log(f"plain streaming kernels here: copy {ref['device_copy_gbs']} GB/s, sum {ref['sum_read_gbs']} GB/s")
    if not prefill:
        # the step's and the layers' algorithmic bytes against what a plain
        # copy reaches on this GPU (the roofline fractions above stay
        # against the published peak)
        ref["step_frac_of_copy"] = round(step_roof["achieved_gbs"] / ref["device_copy_gbs"], 4)

    cpu = None
    if not args.no_cpu:
        log("timing the oracle on a bounded sample ...")
        cpu = cpu_baseline(cases, prefill)

    out = {"metric": METRIC, "value": round(value, 2),
           "unit": "prefill tokens/s per layer" if prefill else "decode tokens/s per layer",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded; shapes of the pages' Flash/Pro configurations)",
           "config": cfg, "roofline": roofline, "step_roofline": step_roof, "cpu_baseline": cpu,
           "layer_times": layers, "kernels": kernels, "other_workloads": extra, "hbm_reference": ref}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
