#!/usr/bin/env python3
"""Benchmark of the Fourier-approximated KV-cache hot path on one MI355X.

One step = the whole path on one batch of synthetic input:
``fa_project`` (coefficients of K and V plus the retained edge rows) followed by
``fa_decode`` (one decode step for every query head).  The default workload is
the LLaMA-2-7B-shaped layer (32/32 heads, head_dim 128, L = 4096, 64 of 128 dims
compressible, k = 401).  Inputs are resident in HBM before timing starts and
are rotated over enough copies that one step's inputs are not in the 256 MB
last-level cache.

Prints ONE JSON line: metric/value (KV-positions per second of the whole
step), per-call figures (decode HBM GB/s, projection TFLOP/s), the roofline of
the dominant kernel (algorithmic bytes or flops over its event-timed duration)
and the CPU oracle's rate on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
LLC_BYTES = 256 << 20          # MI355X Infinity Cache
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def algorithmic(w):
    """(decode must-read+write bytes, projection flops, KV positions) per step."""
    c = w.cfg
    esz = 2 if c.dtype == "bf16" else 4
    E = c.sink + c.recent
    dec = 0
    flops = 0.0
    for b in range(c.batch):
        L, M = int(w.lens[b]), w.mid_len(b)
        dec += c.n_kv_heads * L * c.n_exact * 2 * esz                 # kx, vx
        dec += c.n_kv_heads * min(L, E) * c.n_comp * 2 * esz          # ke, ve
        if M > 0:
            dec += c.n_kv_heads * c.n_coef * c.n_comp * 2 * 4          # ck, cv
            flops += 2.0 * M * c.n_coef * c.n_kv_heads * c.n_comp * 2  # K and V
    dec += c.batch * c.n_query * c.n_q_heads * c.head_dim * (esz + 4)  # q in, out
    pos = int(w.lens.sum()) * c.n_kv_heads
    return dec, flops, pos


def kernel_sources_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_decode_fourier_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from committed rocprofv3 counters, if still valid."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload, {}).get(kernel)
    if not e or e.get("sources") != kernel_sources_hash():
        return None
    return e.get("bytes_per_launch")


def box_peaks(torch):
    """Achieved streaming-copy bandwidth and fp16 GEMM rate on this GPU."""
    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps
    n = (2 << 30) // 4  # 2 GiB read + 2 GiB written
    src = torch.empty(n, device="cuda").uniform_()
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), 20)
    del src, dst
    m = 8192
    a = torch.randn(m, m, device="cuda", dtype=torch.float16)
    b = torch.randn(m, m, device="cuda", dtype=torch.float16)
    t_mm = timed(lambda: torch.matmul(a, b), 20)
    return {"copy_GBps": 2 * n * 4 / t_copy / 1e9, "copy_frac_of_8TBps": 2 * n * 4 / t_copy / 8e12,
            "fp16_gemm_TFLOPs": 2.0 * m ** 3 / t_mm / 1e12, "fp16_gemm_frac_of_2.5PF": 2.0 * m ** 3 / t_mm / 2.5e15,
            "gemm": "torch.matmul fp16 %dx%dx%d" % (m, m, m), "copy": "torch copy_ of 2 GiB fp32"}


def approximation_context(w, out, ck, cv, scale):
    """How far the compressed cache's result is from the uncompressed one, as
    context (not a gate).  Decode: the GPU's outputs against plain softmax
    attention over the full K and V (float64 numpy, written here), on sampled
    (sequence, KV head) blocks.  Projection only: the share of each sampled
    middle column's energy that the k coefficients miss, which for an
    orthonormal basis is sqrt(|x|^2 - |c|^2) / |x| (no reconstruction needed)."""
    c = w.cfg
    G = c.n_q_heads // c.n_kv_heads
    longest = int(np.argmax(w.lens))
    if c.batch * c.n_kv_heads <= 32:
        blocks = [(b, h) for b in range(c.batch) for h in range(c.n_kv_heads)]
    else:
        blocks = [(longest, 0), (longest, c.n_kv_heads - 1)]
    if out is None:
        M = w.mid_len(longest)
        worst, miss, energy = 0.0, 0.0, 0.0
        for h in (0, c.n_kv_heads - 1):
            for X, C in ((w.kc, ck), (w.vc, cv)):
                x = w.f64(w.block(X, longest, h))[c.sink:c.sink + M]
                coef = C[longest * c.n_kv_heads + h].astype(np.float64)
                nx, ncf = (x * x).sum(0), (coef * coef).sum(0)
                worst = max(worst, float(np.sqrt(np.maximum(nx - ncf, 0.0) / nx).max()))
                miss += float(np.maximum(nx - ncf, 0.0).sum())
                energy += float(nx.sum())
        return {"kind": "middle-row energy the coefficients miss (K and V, sampled KV heads)",
                "rel_l2": float(np.sqrt(miss / energy)), "worst_column_rel_l2": worst,
                "blocks": "(sequence, KV head) blocks %s" % [[longest, 0], [longest, c.n_kv_heads - 1]]}
    q4 = w.q if w.q.ndim == 4 else w.q[:, None]
    o4 = out if out.ndim == 4 else out[:, None]
    num = den = 0.0
    mab = 0.0
    for b, h in blocks:
        K, V = w.natural_kv(b, h)
        q = w.f64(q4[b, :, h * G:(h + 1) * G]).reshape(-1, c.head_dim)
        sc = scale * (q @ K.T)
        p = np.exp(sc - sc.max(1, keepdims=True))
        exact = (p / p.sum(1, keepdims=True)) @ V
        got = o4[b, :, h * G:(h + 1) * G].reshape(-1, c.head_dim).astype(np.float64)
        mab = max(mab, float(np.abs(got - exact).max()))
        num += float(((got - exact) ** 2).sum())
        den += float((exact ** 2).sum())
    where = ("all %d (sequence, KV head) blocks" % len(blocks) if len(blocks) > 2
             else "(sequence, KV head) blocks %s" % [list(x) for x in blocks])
    return {"kind": "GPU output vs uncompressed attention", "max_abs": mab,
            "rel_l2": float(np.sqrt(num / den)), "blocks": where}


def cpu_baseline(w, scale, seconds):
    """The oracle (fp64 numpy) on the same workload, repeated ~`seconds`."""
    from oracle import batch as ob
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    steps = w.cfg.steps
    n = 0
    t0 = time.perf_counter()
    while True:
        ck, cv = ob.project_all(w)
        if "decode" in steps:
            if w.cfg.n_query > 1:
                ob.attend_all(w, ck, cv, scale)
            else:
                ob.decode_all(w, ck, cv, scale)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / n
    return dt, threads, n


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama2_7b_layer")
    ap.add_argument("--copies", type=int, default=0, help="input copies (0: enough to beat the LLC)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay one HIP graph per call and input copy (default: launch every call from the host, "
                         "which measures faster on this ROCm)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure what the box reaches: a streaming copy (HBM GB/s) and a large fp16 "
                         "GEMM (hipBLASLt through torch, MFMA TFLOP/s), as context for the roofline fractions")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain copy kernel over MIB MiB (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_decode_fourier_amd import binding as fb
    from long_context_decode_fourier_amd import workloads as wl

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.peaks:
        print(json.dumps(box_peaks(torch)))
        return
    if args.calibrate_copy:
        # torch elementwise negation: reads and writes exactly n * 4 bytes
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4}))
        return
    fb.lib()
    cfg = wl.CONFIGS[args.workload]
    w = wl.make(cfg)
    c = cfg
    steps = c.steps
    dec_bytes, proj_flops, positions = algorithmic(w)
    scale = 1.0 / np.sqrt(c.head_dim)

    dev = "cuda"
    dims = torch.from_numpy(w.dims).to(dev)
    desc = fb.Desc.from_workload(w, dims)
    nblk = c.batch * c.n_kv_heads
    E = c.sink + c.recent
    base = dict(kc=fb.to_device(w.kc), vc=fb.to_device(w.vc))
    if "decode" in steps:
        base.update(q=fb.to_device(w.q), kx=fb.to_device(w.kx), vx=fb.to_device(w.vx))
    per_copy = sum(t.numel() * t.element_size() for t in base.values())
    copies = args.copies or max(2, int(np.ceil(2 * LLC_BYTES / per_copy)) + 1)
    sets = []
    for i in range(copies):
        s = {k: (v if i == 0 else v.clone()) for k, v in base.items()}
        s["ck"] = torch.empty((nblk, c.n_coef, c.n_comp), device=dev)
        s["cv"] = torch.empty_like(s["ck"])
        s["ke"] = torch.empty((nblk, E, c.n_comp), dtype=base["kc"].dtype, device=dev)
        s["ve"] = torch.empty_like(s["ke"])
        if "decode" in steps:
            oshape = (c.batch, c.n_q_heads, c.head_dim) if c.n_query == 1 else \
                (c.batch, c.n_query, c.n_q_heads, c.head_dim)
            s["out"] = torch.empty(oshape, device=dev)
        sets.append(s)
    ws_p = fb.workspace(fb.project_workspace_size(desc))
    ws_d = fb.workspace(fb.attend_workspace_size(desc, c.n_query)) if "decode" in steps else None
    if "decode" in steps and "project" not in steps:
        for s in sets:  # decode-only workloads: coefficients and edges made once
            fb.project(desc, s["kc"], s["vc"], s["ck"], s["cv"], s["ke"], s["ve"], ws_p)
    stream = torch.cuda.current_stream()

    def call_project(s, st):
        fb.project(desc, s["kc"], s["vc"], s["ck"], s["cv"], s["ke"], s["ve"], ws_p, st)

    def call_decode(s, st):
        if c.n_query > 1:  # several queries per sequence: fa_attend
            fb.attend(desc, c.n_query, s["q"], s.get("kx"), s.get("vx"), s["ke"], s["ve"], s["ck"],
                      s["cv"], scale, s["out"], None, ws_d, st)
        else:
            fb.decode(desc, s["q"], s.get("kx"), s.get("vx"), s["ke"], s["ve"], s["ck"], s["cv"],
                      scale, s["out"], ws_d, st)

    graphs = None  # per input copy: (project graph, decode graph)

    def step(i, ev=None):
        s = sets[i % copies]
        if ev is not None:
            ev[0].record(stream)
        if "project" in steps:
            if graphs: graphs[i % copies][0].replay()
            else: call_project(s, stream)
        if ev is not None:
            ev[1].record(stream)
        if "decode" in steps:
            if graphs: graphs[i % copies][1].replay()
            else: call_decode(s, stream)
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.graph:
        # the step as HIP graphs: the calls are captured once per input copy
        # (the library makes no allocation, memset or host sync)
        side = torch.cuda.Stream()
        graphs = []
        for s in sets:
            pair = []
            for fn, name in ((call_project, "project"), (call_decode, "decode")):
                g = None
                if name in steps:
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=side):
                        fn(s, torch.cuda.current_stream())
                pair.append(g)
            graphs.append(tuple(pair))
        torch.cuda.synchronize()
        for i in range(max(args.warmup, copies)):
            step(i)
        torch.cuda.synchronize()

    # timed region: whole-step throughput
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps

    # per-call durations with events on the launch stream (same calls again)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    d_proj = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    d_dec = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    t_proj = float(d_proj.mean())
    t_dec = float(d_dec.mean())

    def spread(d):  # per-call durations, microseconds
        p10, p50, p90 = np.percentile(d, [10, 50, 90]) * 1e6
        return {"p10": float(p10), "median": float(p50), "p90": float(p90)}

    extra = {}
    full_b, comp_b = fb.cache_bytes(desc)
    extra["cache_bytes_full"] = full_b
    extra["cache_bytes_compressed"] = comp_b
    extra["cache_compression"] = 1.0 - comp_b / full_b
    extra["pages_budget_k"] = fb.coef_budget(w.mid_len(int(np.argmax(w.lens))), 0.3)
    if "decode" in steps:
        extra["decode_us"] = t_dec * 1e6
        extra["decode_us_spread"] = spread(d_dec)
        extra["decode_kv_positions_per_s"] = positions / t_dec
        extra["decode_hbm_GBps"] = dec_bytes / t_dec / 1e9
        extra["decode_algorithmic_bytes"] = dec_bytes
    if "project" in steps:
        extra["project_us"] = t_proj * 1e6
        extra["project_us_spread"] = spread(d_proj)
        extra["project_tflops"] = proj_flops / t_proj / 1e12
        extra["project_algorithmic_flops"] = proj_flops
    # dominant call: the larger share of the step
    if "decode" in steps and (t_dec >= t_proj or "project" not in steps):
        ach = dec_bytes / t_dec / 1e9
        roof = {"kernel": "fa_decode" if c.n_query == 1 else "fa_attend", "bound": "hbm",
                "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                "traffic": measured_traffic(args.workload, "fa_decode")}
    else:
        ach = proj_flops / t_proj / 1e12
        roof = {"kernel": "fa_project", "bound": "mfma", "achieved": ach,
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / MFMA_F16_PEAK_TFLOPS,
                "traffic": measured_traffic(args.workload, "fa_project")}

    # context: the same achieved rate against what the box reaches outside the
    # library (streaming copy / hipBLASLt GEMM, measured by bench.py --peaks)
    try:
        with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "box_peaks.json")) as f:
            bp = json.load(f)
        box = bp["copy_GBps"] if roof["unit"] == "GB/s" else bp["fp16_gemm_TFLOPs"]
        roof["box_peak"] = box
        roof["frac_of_box_peak"] = roof["achieved"] / box
    except (OSError, ValueError, KeyError):
        pass

    # context: the result against attention over the uncompressed cache
    s0 = sets[0]
    if "project" in steps:
        call_project(s0, stream)
    if "decode" in steps:
        call_decode(s0, stream)
    torch.cuda.synchronize()
    approx = approximation_context(
        w, s0["out"].cpu().numpy() if "decode" in steps else None,
        s0["ck"].cpu().numpy(), s0["cv"].cpu().numpy(), scale)

    cpu = None
    if not args.no_cpu_baseline:
        dt, threads, n = cpu_baseline(w, scale, args.cpu_seconds)
        cpu = {"value": positions / dt, "unit": "KV-positions/s", "cores": threads, "kind": "oracle",
               "sample": "%d full step(s) of %s (oracle project of K and V%s), %.2f s each"
                         % (n, args.workload, " + decode" if "decode" in steps else "", dt)}

    line = {
        "metric": "KV-positions/s (fa_project K,V + fa_decode per step)" if len(steps) == 2
                  else ("KV-positions/s (%s)" % "+".join(steps) if c.n_query == 1
                        else "KV-positions/s (fa_attend, %d queries per sequence)" % c.n_query),
        "value": positions / (ms_step * 1e-3),
        "unit": "KV-positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 in, fp16 MFMA operands, fp32 accumulate" if c.dtype == "bf16" else "f32",
        "data": "synthetic (seeded generator; no dataset or weights)",
        "config": {"workload": args.workload, "note": c.note, "batch": c.batch,
                   "seq_len": [int(x) for x in w.lens] if c.len_range else int(w.lens[0]),
                   "n_q_heads": c.n_q_heads, "n_kv_heads": c.n_kv_heads, "head_dim": c.head_dim,
                   "n_comp_dims": c.n_comp, "n_coef": c.n_coef, "sink": c.sink,
                   "recent": c.recent, "n_query": c.n_query, "input_copies": copies},
        "launch": "hip graph replay (one graph per call and input copy)" if args.graph else "eager",
        "roofline": roof,
        "cpu_baseline": cpu,
        "approx_error_vs_exact": approx,
        "calls": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
