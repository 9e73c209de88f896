"""Benchmark of the sparse MoE FFN layer on one MI355X.

One step = one pass of the whole prefill path (router + top-k, align, grouped
gate/up GEMM with SwiGLU, grouped down GEMM, combine with the gated shared
expert) over the 8192-token workload (hidden 2048, 256 experts, top-8, FFN
512, shared expert 512, router bias ~ N(0,1)); weights and tokens are already
in HBM when the timed region starts.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Also reported in the same line: the single-token decode path (GB/s against
HBM), a per-stage time breakdown, the roofline of the dominant kernel
(grouped gate/up GEMM, timed with HIP events on its launch stream) and the CPU
oracle's throughput on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at T=8192 (MFMA % of peak); T=1 decode GB/s (% of HBM peak)"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense BF16 MFMA (AMD specification)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gate_up_prefill8k_hbm_traffic.md")


def measured_traffic(kernel):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 --pmc record
    (FETCH_SIZE and WRITE_SIZE passes, scaled by a device copy of known size), or None when
    the record is missing, was taken on another kernel, or any source it was taken on has
    changed since."""
    import hashlib
    try:
        line = [ln for ln in open(TRAFFIC_RECORD) if ln.startswith("traffic-record:")][0]
        rec = json.loads(line.split(":", 1)[1])
        if rec["kernel"] != kernel:
            return None
        for path, digest in rec["sources"].items():
            if hashlib.sha256(open(os.path.join(ROOT, path), "rb").read()).hexdigest()[:16] != digest:
                return None
        return rec["traffic_bytes"]
    except (OSError, IndexError, KeyError, ValueError):
        return None


def gate_up_kernel_name(tile_rows):
    """The kernel that runs the gate/up launch for a tile height (as rocprofv3 names it)."""
    if tile_rows == 256:
        # the two-stage ring: at a mean of 192 rows per expert or more (the 8192-token workload)
        return "grouped_gemm_dma_kernel<0, false, false, false>"
    return f"grouped_gemm_kernel<{tile_rows}, 32, 2, 0, false>"


def algorithmic(T, H, E, k, I, I_s):
    """Flops of the layer per call (what the method must compute, no padding)."""
    routed = 6 * T * k * H * I          # gate, up (2 * 2HI) and down (2HI) per assignment
    shared = 6 * T * H * I_s
    router = 2 * T * H * E + 2 * T * H  # logits + shared gate
    gate_up = 4 * T * H * (k * I + I_s)  # the gate/up launch: routed tiles + the shared expert's token tiles
    return routed + shared + router, gate_up


def prefill_bytes(T, H, E, k, I, I_s, n_touched):
    """Bytes a prefill call must move at least: the touched experts' weights, the router, the shared
    gate and the shared expert, x in and y out."""
    return 2 * (n_touched * 3 * H * I + E * H + H + 3 * H * I_s + 2 * T * H)


def decode_bytes(H, E, k, I, I_s):
    """Bytes one T=1 call must move: router, shared gate, k experts, shared expert, x, y."""
    return 2 * (E * H + H + k * 3 * H * I + 3 * H * I_s + H + H)


def kernel_only(args):
    """The dominant kernel alone (for rocprofv3 --pmc passes): route and align once, then
    --warmup + --steps launches of the gate/up GEMM (routed and shared tiles, as moe_forward
    launches it), then a 256 MiB device copy."""
    import torch
    from sparse_moe_layer_03_amd import moe, synth
    from sparse_moe_layer_03_amd.layer import DeviceLayer, to_device_bf16
    dev = torch.device("cuda:0")
    wl = synth.workload("prefill8k")
    T, H, E, k, I, I_s = wl.T, wl.H, wl.E, wl.k, wl.I, wl.I_s
    inp = synth.make_inputs(wl, seed=0)
    lay = DeviceLayer.from_inputs(inp, dev)
    x = to_device_bf16(inp["x"], dev)
    b = lay.alloc_stage_buffers(T)
    lay.run_route(x, b)
    lay.run_align(T, b)
    W = lay.w
    def launch():
        moe.moe_grouped_gate_up(x, W["w_gate"], W["w_up"], W["ws_gate"], W["ws_up"], b["sorted"], b["tiles"],
                                b["n_tiles"], T, H, E, k, I, I_s, b["h"], b["h_s"])
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        launch()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    c = torch.empty_like(a)
    c.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"kernel": "gate/up GEMM (routed + shared tiles)", "workload": "8192 tokens", "launches": args.warmup + args.steps,
                      "us_per_launch": us, "copy_bytes": a.numel() * 4}), flush=True)
    return 0


def cpu_model():
    """The host CPU's model name (lscpu's "Model name", read from /proc/cpuinfo)."""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.lower().startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, T, sample=0):
    """The CPU oracle on the first tokens of the workload: median of 3 timed runs with every host thread
    (OMP_NUM_THREADS, else all), and median of 3 with one thread; each sample sized to ~3-5 s of work."""
    import statistics
    import subprocess
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    code = ("import sys, time, numpy as np; sys.path.insert(0, %r); import oracle; "
            "from sparse_moe_layer_03_amd import synth; "
            "inp = synth.make_inputs(synth.workload('prefill8k'), seed=0); n = int(sys.argv[1]); "
            "sub = dict(inp); sub['x'] = inp['x'][:n]; oracle.forward(synth.make_inputs(synth.workload('tiny'), seed=0)); "
            "r = []\nfor _ in range(3):\n    t = time.perf_counter(); oracle.forward(sub); r.append(time.perf_counter() - t)\n"
            "print('SECS', *r)") % ROOT

    def run(n, nthreads):
        env = dict(os.environ, OMP_NUM_THREADS=str(nthreads))
        p = subprocess.run([sys.executable, "-c", code, str(n)], env=env, capture_output=True, text=True, timeout=600)
        line = [ln for ln in p.stdout.splitlines() if ln.startswith("SECS")]
        if p.returncode or not line:
            raise RuntimeError(f"oracle run failed: {p.stderr[-2000:]}")
        return [float(v) for v in line[0].split()[1:]]

    res = {}
    for label, nth, n0 in (("all_threads", threads, sample or max(64, 40 * threads)), ("one_thread", 1, 48)):
        secs = run(n0, nth)
        n = n0
        med = statistics.median(secs)
        if med < 2.0:  # size the sample to ~3-5 s per run
            n = int(min(T, max(n0, n0 * 4.0 / max(med, 1e-3))))
            secs = run(n, nth)
            med = statistics.median(secs)
        res[label] = {"tokens": n, "secs": secs, "tokens_per_s": n / med, "threads": nth}
        log(f"[bench] cpu oracle, {nth} thread(s): {n / med:.1f} tokens/s (median of {[round(v, 2) for v in secs]} s "
            f"on {n} tokens)")
    a = res["all_threads"]
    return {"value": a["tokens_per_s"], "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {a['tokens']} of the {T} tokens of the same workload, whole layer (route, align, "
                      f"expert FFNs, shared expert, combine); median of 3 runs of {[round(v, 2) for v in a['secs']]} s",
            "one_thread": res["one_thread"], "cpu_model": cpu_model(), "runs": 3}


def decode_only(args):
    """Single-token and 8-token calls alone (for rocprofv3 --pmc passes): --steps calls of each, rotating
    16 weight copies (no copy's weights stay in the 256 MB Infinity Cache between its calls), then a
    256 MiB device copy that calibrates the byte counters."""
    import torch
    from sparse_moe_layer_03_amd import moe, synth
    from sparse_moe_layer_03_amd.layer import DeviceLayer, to_device_bf16
    dev = torch.device("cuda:0")
    dwl = synth.workload("decode")
    H, E, k, I, I_s = dwl.H, dwl.E, dwl.k, dwl.I, dwl.I_s
    dinp = synth.make_inputs(dwl, seed=0)
    dbase = DeviceLayer.from_inputs(dinp, dev)
    copies = [dbase.w] + [{key: (None if v is None else v.clone()) for key, v in dbase.w.items()} for _ in range(15)]
    for Tb in (1, 8):
        xs = to_device_bf16(synth._draw_bf16(1 if Tb == 1 else 2, "x", (args.steps * Tb, H), 1.0), dev)
        ys = torch.empty((args.steps * Tb, H), dtype=torch.bfloat16, device=dev)
        ws, nb = dbase.workspace(Tb)
        for i in range(args.steps):
            W = copies[i % len(copies)]
            moe.moe_forward(xs[i * Tb:(i + 1) * Tb], W["w_router"], None, W["w_gate"], W["w_up"], W["w_down"],
                            W["ws_gate"], W["ws_up"], W["ws_down"], W["w_sg"], Tb, H, E, k, I, I_s,
                            ys[i * Tb:(i + 1) * Tb], ws, nb)
        torch.cuda.synchronize()
        if Tb == 8:
            off = moe.moe_forward_ids_offset(Tb, H, E, k, I, I_s)
            touched = len(np.unique(ws[off:off + Tb * k * 4].view(torch.int32).cpu().numpy()))
            print(json.dumps({"T": Tb, "touched_experts_last_call": touched}), flush=True)
    a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
    c = torch.empty_like(a)
    c.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"kernel": "decode and 8-token calls", "calls": args.steps, "copy_bytes": a.numel() * 4}),
          flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # the clock settles after a few dozen steps of sustained MFMA work: untimed warm-up steps
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--copies", type=int, default=4, help="weight copies rotated across prefill steps")
    ap.add_argument("--decode-steps", type=int, default=64, help="decode calls per captured graph")
    ap.add_argument("--decode-copies", type=int, default=16, help="weight copies rotated across decode calls")
    ap.add_argument("--cpu-sample", type=int, default=0, help="oracle sample tokens (0: sized to ~15 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-weight calls")
    ap.add_argument("--no-chunks", action="store_true", help="skip the bucketed-prefill runner")
    ap.add_argument("--no-q4", action="store_true", help="skip the 4-bit-weight calls")
    ap.add_argument("--no-reports", action="store_true", help="skip the 1024- and 32768-token report lines")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--kernel", choices=["gate_up", "decode"], default=None,
                    help="gate_up: only the dominant kernel (routed gate/up GEMM of the 8192-token workload) "
                         "--steps times; decode: only single-token and 8-token calls, --steps of each; then a "
                         "256 MiB device copy: the runs that hardware counters are taken on")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_moe_layer_03_amd import moe, synth
    from sparse_moe_layer_03_amd.layer import DeviceLayer, to_device_bf16

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    moe.lib()
    if args.kernel == "decode":
        return decode_only(args)
    if args.kernel:
        return kernel_only(args)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(0)

    # ------------------------------------------------------------ prefill
    wl = synth.workload("prefill8k")
    T, H, E, k, I, I_s = wl.T, wl.H, wl.E, wl.k, wl.I, wl.I_s
    t0 = time.time()
    inp = synth.make_inputs(wl, seed=0)
    log(f"[bench] inputs drawn in {time.time() - t0:.1f}s; uploading")
    base = DeviceLayer.from_inputs(inp, dev)
    layers = [base]
    for _ in range(max(0, args.copies - 1)):
        c = DeviceLayer.__new__(DeviceLayer)
        c.__dict__.update(base.__dict__)
        c.w = {key: (None if v is None else v.clone()) for key, v in base.w.items()}
        c._ws, c._ws_bytes = base.workspace(T)
        layers.append(c)
    x = to_device_bf16(inp["x"], dev)
    y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    ws, ws_bytes = base.workspace(T)
    for c in layers:
        c._ws, c._ws_bytes = ws, ws_bytes
    stream = torch.cuda.current_stream()

    flops, gate_up_flops = algorithmic(T, H, E, k, I, I_s)
    for i in range(args.warmup):
        layers[i % len(layers)].forward(x, y)
    torch.cuda.synchronize()

    # timed region 1: the product entry point, K steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.steps):
        layers[i % len(layers)].forward(x, y)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps

    # timed region 2: the same kernels stage by stage, HIP events around each launch
    bufs = base.alloc_stage_buffers(T)
    names = ("route", "align", "gate_up", "down", "combine")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    for i in range(args.warmup):
        base.run_stages(x, bufs)
    torch.cuda.synchronize()
    for i in range(args.steps):
        lay = layers[i % len(layers)]
        e = evs[i]
        e[0].record(stream)
        lay.run_route(x, bufs)
        e[1].record(stream)
        lay.run_align(T, bufs)
        e[2].record(stream)
        lay.run_gate_up(x, bufs)
        e[3].record(stream)
        lay.run_down(T, bufs)
        e[4].record(stream)
        lay.run_combine(T, bufs)
        e[5].record(stream)
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]))
                for j, n in enumerate(names)}
    # The dominant kernel's duration for the roofline: the gate/up launch (routed tiles and the shared
    # expert's token tiles, as moe_forward launches it) inside the stage-by-stage steps above, HIP
    # events around each launch on its stream.  Timed region 3 runs the same launch back to back with
    # nothing between (reported as isolated_launch_us): there the previous launch's weight stream has
    # evicted x from the Infinity Cache and the matrix cores run hot for the whole loop, neither of
    # which holds inside a step.
    gu_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    def gate_up_launch(lay):
        moe.moe_grouped_gate_up(x, lay.w["w_gate"], lay.w["w_up"], lay.w["ws_gate"], lay.w["ws_up"], bufs["sorted"],
                                bufs["tiles"], bufs["n_tiles"], T, H, E, k, I, I_s, bufs["h"], bufs["h_s"], stream)
    for i in range(args.warmup):
        gate_up_launch(layers[i % len(layers)])
    torch.cuda.synchronize()
    gu_ev[0].record(stream)
    for i in range(args.steps):
        gate_up_launch(layers[i % len(layers)])
    gu_ev[1].record(stream)
    torch.cuda.synchronize()
    gu_iso_ms = gu_ev[0].elapsed_time(gu_ev[1]) / args.steps
    gu_ms = stage_ms["gate_up"]
    achieved = gate_up_flops / (gu_ms * 1e-3) / 1e12
    counts = np.bincount(bufs["ids"].cpu().numpy().ravel(), minlength=E)
    BIG = moe.moe_align_tile_rows(T, E, k)
    SMALL = moe.moe_align_small_tile_rows(T, E, k)
    nbig = counts // BIG
    padded_rows = int(np.sum(nbig * BIG + np.ceil((counts - nbig * BIG) / SMALL) * SMALL))
    log(f"[bench] prefill T={T}: {ms:.3f} ms/step ({T / ms * 1e3 / 1e6:.2f} M tok/s); stages "
        + ", ".join(f"{n} {v * 1e3:.1f}us" for n, v in stage_ms.items()))

    out = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "long prefill: T=8192 tokens, hidden 2048, 256 experts, top-8, expert FFN 512, "
                               "shared expert 512 gated by sigmoid(x.w_sg), router bias ~ N(0,1)",
                   "T": T, "H": H, "E": E, "k": k, "I": I, "I_s": I_s, "tile_rows": [BIG, SMALL],
                   "weight_copies": len(layers)},
        "layer_tflops": flops / (ms * 1e-3) / 1e12,
        "layer_mfma_frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "stage_us": {n: v * 1e3 for n, v in stage_ms.items()},
        "padding_overhead": padded_rows / (T * k) - 1.0,
        "roofline": {"kernel": gate_up_kernel_name(BIG) + ": gate/up GEMM with SwiGLU epilogue, one launch over all "
                               "expert tiles and the shared expert's token tiles",
                     "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(gate_up_kernel_name(BIG)),
                     "flops_per_launch": gate_up_flops, "avg_launch_us": gu_ms * 1e3,
                     "avg_launch_from": "the gate/up launches of the stage-by-stage timed steps",
                     "isolated_launch_us": gu_iso_ms * 1e3,
                     "padded_rows": padded_rows},
        "device": {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count},
    }
    # ------------------------ the other prefill workloads (report lines, their own rooflines)
    if not args.no_reports:
        reports = {}
        for name, bound in (("prefill1k", "hbm"), ("skew32k", "mfma")):
            rwl = synth.workload(name)
            Tr = rwl.T
            rinp = synth.make_inputs(rwl, seed=0, reuse=inp)
            rlay = DeviceLayer.__new__(DeviceLayer)  # the same weights in HBM, this workload's router bias
            rlay.__dict__.update(base.__dict__)
            rlay.bias = None if rinp["bias"] is None else torch.from_numpy(rinp["bias"]).to(dev)
            rlay._ws, rlay._ws_bytes = None, 0
            xr = to_device_bf16(rinp["x"], dev)
            yr = torch.empty((Tr, H), dtype=torch.bfloat16, device=dev)
            rcop = [rlay]
            for lay_c in layers[1:]:
                c = DeviceLayer.__new__(DeviceLayer)
                c.__dict__.update(rlay.__dict__)
                c.w = lay_c.w
                rcop.append(c)
            ws_r, wsb_r = rlay.workspace(Tr)
            for c in rcop:
                c._ws, c._ws_bytes = ws_r, wsb_r
            nrep = max(5, min(args.steps, int(40e-3 / max(Tr / 8192 * 0.8e-3, 1e-5))))
            for i in range(5):
                rcop[i % len(rcop)].forward(xr, yr)
            torch.cuda.synchronize()
            ev0.record(stream)
            for i in range(nrep):
                rcop[i % len(rcop)].forward(xr, yr)
            ev1.record(stream)
            torch.cuda.synchronize()
            rms = ev0.elapsed_time(ev1) / nrep
            ids_r = rlay.forward_ids(Tr).cpu().numpy()
            touched = int(len(np.unique(ids_r)))
            rflops, _ = algorithmic(Tr, H, E, k, I, I_s)
            rbytes = prefill_bytes(Tr, H, E, k, I, I_s, touched)
            ent = {"workload": f"T={Tr} tokens, same layer; " + ("no router bias (near-uniform load)" if name ==
                   "prefill1k" else "Zipf(1.1) router bias, 1% exact-tie tokens"),
                   "ms_per_step": rms, "tokens_per_s": Tr / (rms * 1e-3), "steps": nrep,
                   "touched_experts": touched, "tflops": rflops / (rms * 1e-3) / 1e12,
                   "GB_per_s": rbytes / (rms * 1e-3) / 1e9, "algorithmic_bytes": rbytes, "flops": rflops}
            if bound == "hbm":
                ent["roofline"] = {"bound": "hbm", "achieved": ent["GB_per_s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": ent["GB_per_s"] / PEAK_HBM_GBS}
            else:
                ent["roofline"] = {"bound": "mfma", "achieved": ent["tflops"], "peak": PEAK_BF16_TFLOPS,
                                   "unit": "TFLOP/s", "frac": ent["tflops"] / PEAK_BF16_TFLOPS}
            reports[str(Tr)] = ent
            log(f"[bench] T={Tr}: {rms:.3f} ms/step ({Tr / rms / 1e3:.2f} M tok/s), {ent['tflops']:.0f} TF/s, "
                f"{ent['GB_per_s']:.0f} GB/s ({touched} experts touched); {bound} frac "
                f"{ent['roofline']['frac']:.3f}")
            del rcop, rlay, xr, yr, ws_r
            torch.cuda.empty_cache()
        out["reports"] = reports

    del layers, bufs
    torch.cuda.empty_cache()

    # ------------------------------------- prefill through buckets (runner)
    if not args.no_chunks:
        from sparse_moe_layer_03_amd.layer import PrefillRunner
        Tc = 16380  # just under two 8192-token buckets: the last segment is padded
        xc = to_device_bf16(synth._draw_bf16(3, "x", (Tc, H), 1.0), dev)
        yc = torch.empty((Tc, H), dtype=torch.bfloat16, device=dev)
        run = PrefillRunner(base)
        segs, lens = run.plan(Tc)
        ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def timed(fn, reps=10):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ce0.record(stream)
            for _ in range(reps):
                fn()
            ce1.record(stream)
            torch.cuda.synchronize()
            return ce0.elapsed_time(ce1) / reps

        run_ms = timed(lambda: run.run(xc, yc))
        one_ms = timed(lambda: base.forward(xc, yc))  # one moe_forward call over all Tc tokens
        run.close()
        out["chunks"] = {"workload": f"T={Tc} tokens (prefill8k layer), buckets {list(run.buckets)}",
                         "segments": segs, "segment_tokens": lens,
                         "runner_ms": run_ms, "runner_tokens_per_s": Tc / (run_ms * 1e-3),
                         "single_call_ms": one_ms, "single_call_tokens_per_s": Tc / (one_ms * 1e-3)}
        log(f"[bench] T={Tc} through buckets {segs}: {run_ms:.3f} ms ({Tc / run_ms / 1e3:.2f} M tok/s); "
            f"one moe_forward call {one_ms:.3f} ms")
        del xc, yc
        base._ws = None
        torch.cuda.empty_cache()

    if args.calib_copy:
        a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        bcopy = torch.empty_like(a)
        for _ in range(3):
            bcopy.copy_(a)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = a.numel() * 4
        del a, bcopy

    # ------------------------------------------------------------- decode
    if not args.no_decode:
        dwl = synth.workload("decode")
        dinp = synth.make_inputs(dwl, seed=0, reuse=inp)
        dbase = DeviceLayer.from_inputs(dinp, dev)
        dcopies = [dbase.w]
        for _ in range(max(0, args.decode_copies - 1)):
            dcopies.append({key: (None if v is None else v.clone()) for key, v in dbase.w.items()})
        nx = args.decode_steps
        xs = to_device_bf16(synth._draw_bf16(1, "x", (nx, H), 1.0), dev)
        ys = torch.empty((nx, H), dtype=torch.bfloat16, device=dev)
        dws, dws_bytes = dbase.workspace(1)

        def dstep(i):
            W = dcopies[i % len(dcopies)]
            moe.moe_forward(xs[i:i + 1], W["w_router"], None, W["w_gate"], W["w_up"], W["w_down"], W["ws_gate"],
                            W["ws_up"], W["ws_down"], W["w_sg"], 1, H, E, k, I, I_s, ys[i:i + 1], dws, dws_bytes)

        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(nx):
                dstep(i)
        torch.cuda.current_stream().wait_stream(s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(nx):
                dstep(i)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        reps = 5
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record()
        for _ in range(reps):
            g.replay()
        d1.record()
        torch.cuda.synchronize()
        dus = d0.elapsed_time(d1) * 1e3 / (reps * nx)
        nbytes = decode_bytes(H, E, k, I, I_s)
        gbs = nbytes / (dus * 1e-6) / 1e9
        # eager launches (host launch overhead included) for context
        torch.cuda.synchronize()
        d0.record()
        for i in range(nx):
            dstep(i)
        d1.record()
        torch.cuda.synchronize()
        eager_us = d0.elapsed_time(d1) * 1e3 / nx
        out["decode"] = {"workload": "decode step: T=1, hidden 2048, 256 experts, top-8, FFN 512, shared expert 512",
                         "us_per_call": dus, "GB_per_s": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
                         "bytes_per_call": nbytes, "weight_copies": len(dcopies), "timing": "HIP graph of "
                         f"{nx} calls, {reps} replays", "eager_us_per_call": eager_us}
        log(f"[bench] decode: {dus:.2f} us/call, {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS * 100:.1f}% of HBM); "
            f"eager {eager_us:.2f} us/call")

        def graph_us(step, ncall):
            """Average µs per call of step(0..ncall-1) captured in one HIP graph, over `reps` replays."""
            s2 = torch.cuda.Stream()
            s2.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s2):
                for i in range(ncall):
                    step(i)
            torch.cuda.current_stream().wait_stream(s2)
            gb = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gb):
                for i in range(ncall):
                    step(i)
            gb.replay()
            torch.cuda.synchronize()
            d0.record()
            for _ in range(reps):
                gb.replay()
            d1.record()
            torch.cuda.synchronize()
            del gb
            return d0.elapsed_time(d1) * 1e3 / (reps * ncall)

        def touched_experts(step, Tb, ws, ncall):
            ids_off = moe.moe_forward_ids_offset(Tb, H, E, k, I, I_s)
            out_n = []
            for i in range(ncall):
                step(i)
                torch.cuda.synchronize()
                out_n.append(len(np.unique(ws[ids_off:ids_off + Tb * k * 4].view(torch.int32).cpu().numpy())))
            return out_n

        # small batches (the small-batch kernels): bytes = router + the touched experts of each call
        # (counted from the call's own selection) + the shared expert + x + y
        sb = {}
        ncall = 16
        for Tb in (2, 8, 32):
            xb = to_device_bf16(synth._draw_bf16(2, "x", (ncall * Tb, H), 1.0), dev)
            yb = torch.empty((ncall * Tb, H), dtype=torch.bfloat16, device=dev)
            bws, bws_bytes = dbase.workspace(Tb)

            def bstep(i, Tb=Tb, xb=xb, yb=yb, bws=bws, bws_bytes=bws_bytes):
                W = dcopies[i % len(dcopies)]
                moe.moe_forward(xb[i * Tb:(i + 1) * Tb], W["w_router"], None, W["w_gate"], W["w_up"], W["w_down"],
                                W["ws_gate"], W["ws_up"], W["ws_down"], W["w_sg"], Tb, H, E, k, I, I_s,
                                yb[i * Tb:(i + 1) * Tb], bws, bws_bytes)
            touched = touched_experts(bstep, Tb, bws, ncall)
            sbytes = float(np.mean([2 * (E * H + H + n * 3 * H * I + 3 * H * I_s + 2 * Tb * H) for n in touched]))
            bus = graph_us(bstep, ncall)
            sb[str(Tb)] = {"us_per_call": bus, "tokens_per_s": Tb / (bus * 1e-6), "touched_experts": float(np.mean(touched)),
                           "bytes_per_call": sbytes, "GB_per_s": sbytes / (bus * 1e-6) / 1e9,
                           "hbm_frac": sbytes / (bus * 1e-6) / 1e9 / PEAK_HBM_GBS}
            log(f"[bench] small batch T={Tb}: {bus:.1f} us/call, {sb[str(Tb)]['GB_per_s']:.0f} GB/s")
        out["small_batch"] = {"workload": "2, 8 and 32 tokens per call, decode-config shapes, no router bias",
                              "timing": f"HIP graph of 16 calls over {len(dcopies)} weight copies, {reps} replays",
                              "per_T": sb}
        del dcopies, g
        torch.cuda.empty_cache()

        # FP8 expert weights (E4M3 codes, one fp32 scale per output row): T = 1, 2, 8, 32.
        # bytes = router (bf16) + per touched expert 3*H*I code bytes and (2*I + H) scales
        # + the shared expert likewise + x + y
        if not args.no_fp8:
            t0 = time.time()
            q = synth.add_fp8_weights(dinp)
            log(f"[bench] FP8 weights made in {time.time() - t0:.1f}s")
            qbase = DeviceLayer.from_inputs(q, dev, fp8=True)
            qcopies = [qbase.q]
            for _ in range(max(0, args.decode_copies - 1)):
                qcopies.append({key: (None if v is None else v.clone()) for key, v in qbase.q.items()})
            Wr, Wsg = qbase.w["w_router"], qbase.w["w_sg"]

            def fp8_bytes(n_touched, Tb):
                per_e = 3 * H * I + 4 * (2 * I + H)
                shared = 3 * H * I_s + 4 * (2 * I_s + H)
                return 2 * (E * H + H) + n_touched * per_e + shared + 2 * 2 * Tb * H

            f8 = {}
            for Tb in (1, 2, 8, 32):
                nc = nx if Tb == 1 else ncall
                xb = to_device_bf16(synth._draw_bf16(1 if Tb == 1 else 2, "x", (nc * Tb, H), 1.0), dev)
                yb = torch.empty((nc * Tb, H), dtype=torch.bfloat16, device=dev)
                qws, qws_bytes = qbase.workspace(Tb)

                def qstep(i, Tb=Tb, xb=xb, yb=yb, qws=qws, qws_bytes=qws_bytes):
                    Q = qcopies[i % len(qcopies)]
                    moe.moe_forward_fp8(xb[i * Tb:(i + 1) * Tb], Wr, None, Q["w_gate"], Q["w_gate_scale"],
                                        Q["w_up"], Q["w_up_scale"], Q["w_down"], Q["w_down_scale"], Q["ws_gate"],
                                        Q["ws_gate_scale"], Q["ws_up"], Q["ws_up_scale"], Q["ws_down"],
                                        Q["ws_down_scale"], Wsg, Tb, H, E, k, I, I_s, yb[i * Tb:(i + 1) * Tb],
                                        qws, qws_bytes)
                touched = [k] * nc if Tb == 1 else touched_experts(qstep, Tb, qws, nc)
                qb = float(np.mean([fp8_bytes(n, Tb) for n in touched]))
                qus = graph_us(qstep, nc)
                f8[str(Tb)] = {"us_per_call": qus, "tokens_per_s": Tb / (qus * 1e-6),
                               "touched_experts": float(np.mean(touched)), "bytes_per_call": qb,
                               "GB_per_s": qb / (qus * 1e-6) / 1e9, "hbm_frac": qb / (qus * 1e-6) / 1e9 / PEAK_HBM_GBS}
                log(f"[bench] FP8 weights T={Tb}: {qus:.1f} us/call, {f8[str(Tb)]['GB_per_s']:.0f} GB/s")
            # the 8192-token prefill with FP8 expert weights (tiled GEMMs on widened codes)
            Q0 = qcopies[0]
            yq = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            pws, pws_bytes = qbase.workspace(T)

            def qprefill():
                moe.moe_forward_fp8(x, Wr, base.bias, Q0["w_gate"], Q0["w_gate_scale"], Q0["w_up"], Q0["w_up_scale"],
                                    Q0["w_down"], Q0["w_down_scale"], Q0["ws_gate"], Q0["ws_gate_scale"], Q0["ws_up"],
                                    Q0["ws_up_scale"], Q0["ws_down"], Q0["ws_down_scale"], Wsg, T, H, E, k, I, I_s,
                                    yq, pws, pws_bytes)
            for _ in range(5):
                qprefill()
            torch.cuda.synchronize()
            d0.record()
            for _ in range(10):
                qprefill()
            d1.record()
            torch.cuda.synchronize()
            qms = d0.elapsed_time(d1) / 10
            log(f"[bench] FP8 weights prefill T={T}: {qms:.3f} ms/step ({T / qms / 1e3:.2f} M tok/s)")
            fp8_runner = None
            if not args.no_chunks:
                # 16380 tokens through the 8192-token bucket with FP8 expert weights (no router bias)
                from sparse_moe_layer_03_amd.layer import PrefillRunner
                Tc = 16380
                xc = to_device_bf16(synth._draw_bf16(3, "x", (Tc, H), 1.0), dev)
                yc = torch.empty((Tc, H), dtype=torch.bfloat16, device=dev)
                qrun = PrefillRunner(qbase)
                for _ in range(3):
                    qrun.run(xc, yc)
                torch.cuda.synchronize()
                d0.record()
                for _ in range(10):
                    qrun.run(xc, yc)
                d1.record()
                torch.cuda.synchronize()
                rms = d0.elapsed_time(d1) / 10
                qrun.close()
                fp8_runner = {"T": Tc, "segments": qrun.plan(Tc)[0], "ms_per_call": rms,
                              "tokens_per_s": Tc / (rms * 1e-3)}
                log(f"[bench] FP8 weights, T={Tc} through buckets: {rms:.3f} ms ({Tc / rms / 1e3:.2f} M tok/s)")
                del xc, yc
            out["fp8"] = {"workload": "1, 2, 8 and 32 tokens per call, decode-config shapes, expert weights as OCP "
                                      "FP8 E4M3 with one fp32 scale per output row, no router bias; and the "
                                      f"{T}-token prefill workload (router bias) with the same FP8 weights",
                          "timing": f"HIP graph of {nx} (T=1) or 16 calls over {len(qcopies)} weight copies, "
                                    f"{reps} replays; prefill: 10 eager steps after 5", "per_T": f8,
                          "prefill": {"T": T, "ms_per_step": qms, "tokens_per_s": T / (qms * 1e-3)},
                          "runner": fp8_runner}
            del qcopies, qbase
            torch.cuda.empty_cache()

        # 4-bit expert weights (signed nibbles, fp16 scale per 32 weights): T = 1, 2, 8, 32.
        # bytes = router (bf16) + per touched expert 3*H*I/2 code bytes and 3*H*I/32 fp16 scales
        # + the shared expert likewise + x + y
        if not args.no_q4:
            t0 = time.time()
            q4 = synth.add_q4_weights(dinp)
            log(f"[bench] 4-bit weights made in {time.time() - t0:.1f}s")
            q4base = DeviceLayer.from_inputs(q4, dev, q4=True)
            q4copies = [q4base.q]
            for _ in range(max(0, args.decode_copies - 1)):
                q4copies.append({key: (None if v is None else v.clone()) for key, v in q4base.q.items()})
            Wr4, Wsg4 = q4base.w["w_router"], q4base.w["w_sg"]

            def q4_bytes(n_touched, Tb):
                per_e = 3 * H * I // 2 + 3 * H * I // 32 * 2
                shared = 3 * H * I_s // 2 + 3 * H * I_s // 32 * 2
                return 2 * (E * H + H) + n_touched * per_e + shared + 2 * 2 * Tb * H

            f4 = {}
            for Tb in (1, 2, 8, 32):
                nc = nx if Tb == 1 else ncall
                xb = to_device_bf16(synth._draw_bf16(1 if Tb == 1 else 2, "x", (nc * Tb, H), 1.0), dev)
                yb = torch.empty((nc * Tb, H), dtype=torch.bfloat16, device=dev)
                q4ws, q4ws_bytes = q4base.workspace(Tb)

                def q4step(i, Tb=Tb, xb=xb, yb=yb, q4ws=q4ws, q4ws_bytes=q4ws_bytes):
                    Q = q4copies[i % len(q4copies)]
                    moe.moe_forward_q4(xb[i * Tb:(i + 1) * Tb], Wr4, None, Q["w_gate_q4"], Q["w_gate_q4scale"],
                                       Q["w_up_q4"], Q["w_up_q4scale"], Q["w_down_q4"], Q["w_down_q4scale"],
                                       Q["ws_gate_q4"], Q["ws_gate_q4scale"], Q["ws_up_q4"], Q["ws_up_q4scale"],
                                       Q["ws_down_q4"], Q["ws_down_q4scale"], Wsg4, Tb, H, E, k, I, I_s,
                                       yb[i * Tb:(i + 1) * Tb], q4ws, q4ws_bytes)
                touched = [k] * nc if Tb == 1 else touched_experts(q4step, Tb, q4ws, nc)
                qb = float(np.mean([q4_bytes(n, Tb) for n in touched]))
                qus = graph_us(q4step, nc)
                f4[str(Tb)] = {"us_per_call": qus, "tokens_per_s": Tb / (qus * 1e-6),
                               "touched_experts": float(np.mean(touched)), "bytes_per_call": qb,
                               "GB_per_s": qb / (qus * 1e-6) / 1e9, "hbm_frac": qb / (qus * 1e-6) / 1e9 / PEAK_HBM_GBS}
                log(f"[bench] 4-bit weights T={Tb}: {qus:.1f} us/call, {f4[str(Tb)]['GB_per_s']:.0f} GB/s")
            out["q4"] = {"workload": "1, 2, 8 and 32 tokens per call, decode-config shapes, expert weights as "
                                     "signed 4-bit integers with an fp16 scale per 32 weights, no router bias",
                         "timing": f"HIP graph of {nx} (T=1) or 16 calls over {len(q4copies)} weight copies, "
                                   f"{reps} replays", "per_T": f4}
            del q4copies, q4base
            torch.cuda.empty_cache()

    # -------------------------------------------------------- cpu baseline
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, T, args.cpu_sample)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    sys.exit(main())
