#!/usr/bin/env python3
"""Benchmark of the Fourier-approximated KV-cache hot path on one MI355X.

Default run: one decode step of the ragged long-context batch (16 sequences,
32 query / 8 KV heads, head_dim 128, L_b ~ U[32768, 65536] by seed, 64
compressible dims per KV head, k = 2049) is the step; the JSON line's value is
its KV positions per second.  The line also carries, under ``calls``, the
prefill projection measured on its own workload (8 KV heads, 64 compressible
dims of K and V, M = 131040, k = 4097): projection TFLOP/s and its fraction of
the MFMA peak.  ``--workload`` picks another step (e.g. ``llama2_7b_layer``,
whose step is fa_project of K and V followed by fa_decode).

Inputs are resident in HBM before timing starts and rotated over enough copies
that one step's inputs are not in the 256 MB last-level cache.

Prints ONE JSON line: metric/value, per-call figures (decode HBM GB/s,
projection TFLOP/s), the roofline of the dominant kernel (its algorithmic bytes
or flops over its own event-timed duration: the library records two HIP
events around that kernel on the launch stream) and the CPU oracle's rate on a
bounded sample of the same workload.
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
DEFAULT_WORKLOAD = "ragged_batch"
DEFAULT_PROJECTION = "prefill_projection"


def algorithmic(c, lens):
    """Per step of workload config ``c`` with sequence lengths ``lens``:
    decode must-read+write bytes, the main decode kernel's share of them
    (exact dims of the middle rows), projection flops, KV positions."""
    esz = 2 if c.dtype == "bf16" else 4
    E = c.sink + c.recent
    dec = main = 0
    flops = 0.0
    if "sensitivity" in c.steps:
        # dimension analysis: keys and noise of every token, all dims (the
        # main kernel's stream), queries in and the [Hq, D] result out
        main = c.n_kv_heads * int(np.sum(lens)) * c.head_dim * 2 * esz
        dec = main + c.batch * c.n_query * c.n_q_heads * c.head_dim * esz + c.n_q_heads * c.head_dim * 4
        return dec, main, flops, int(np.sum(lens)) * c.n_kv_heads
    for b in range(c.batch):
        L = int(lens[b])
        M = max(0, L - E)
        dec += c.n_kv_heads * L * c.n_exact * 2 * esz                 # kx, vx
        main += c.n_kv_heads * M * c.n_exact * 2 * esz                # kx, vx middle rows
        dec += c.n_kv_heads * min(L, E) * c.n_comp * 2 * esz          # ke, ve
        if M > 0:
            dec += c.n_kv_heads * c.n_coef * c.n_comp * 2 * 4          # ck, cv
            flops += 2.0 * M * c.n_coef * c.n_kv_heads * c.n_comp * 2  # K and V
    dec += c.batch * c.n_query * c.n_q_heads * c.head_dim * (esz + 4)  # q in, out
    pos = int(np.sum(lens)) * c.n_kv_heads
    return dec, main, flops, pos


# the source files behind each main kernel (its own file and the headers it
# includes): a change to any of them voids that kernel's committed counters
MAIN_KERNEL_FILES = {
    "decode_score_kernel": ["decode_two_pass.hip", "mfma_util.hpp", "kernels.hpp", "common.hpp"],
    "decode_mfma_kernel": ["decode_mfma.hip", "mfma_util.hpp", "kernels.hpp", "common.hpp"],
    "decode_split_kernel": ["decode.hip", "kernels.hpp", "common.hpp"],
    "project_f16_kernel": ["project.hip", "kernels.hpp", "common.hpp"],
    "project_tall_kernel": ["project.hip", "kernels.hpp", "common.hpp"],
    "project_f32_kernel": ["project.hip", "kernels.hpp", "common.hpp"],
}


def sources_hash(files):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_decode_fourier_amd", "csrc")
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of a main kernel ("decode_main" / "project_main")
    from committed rocprofv3 counters, if its sources have not changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(workload, {}).get(kernel)
    if not e or e.get("sources") != sources_hash(e.get("files", [])):
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
    t_sum = timed(lambda: src.sum(), 20)  # read-only stream
    del src, dst
    m = 8192
    a = torch.randn(m, m, device="cuda", dtype=torch.float16)
    b = torch.randn(m, m, device="cuda", dtype=torch.float16)
    t_mm = timed(lambda: torch.matmul(a, b), 20)
    return {"copy_GBps": 2 * n * 4 / t_copy / 1e9, "copy_frac_of_8TBps": 2 * n * 4 / t_copy / 8e12,
            "read_GBps": n * 4 / t_sum / 1e9, "read_frac_of_8TBps": n * 4 / t_sum / 8e12,
            "fp16_gemm_TFLOPs": 2.0 * m ** 3 / t_mm / 1e12, "fp16_gemm_frac_of_2.5PF": 2.0 * m ** 3 / t_mm / 2.5e15,
            "gemm": "torch.matmul fp16 %dx%dx%d" % (m, m, m), "copy": "torch copy_ of 2 GiB fp32",
            "read": "torch sum of 2 GiB fp32"}


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
    """The oracle (fp64 numpy), as it stands, on a bounded sample of the same
    workload: whole (sequence, KV head) blocks of the shortest sequence (its K
    and V projected, then its G query heads decoded, or its n_query * G rows
    attended), one after another until ``seconds`` have passed.  The rate is
    the sample's KV positions (one per token and KV head) per second, the
    unit of the GPU's figure."""
    from oracle import batch as ob
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    c = w.cfg
    b = int(np.argmin(w.lens))
    n = positions = 0
    if "sensitivity" in c.steps:
        # the dimension analysis of whole (sequence, KV head) blocks: every
        # query head of the block perturbed dim by dim (fa.dim_sensitivity)
        from oracle import fourier_attention as fa
        G = c.n_q_heads // c.n_kv_heads
        noise = w.value_noise()
        q4 = w.q if w.q.ndim == 4 else w.q[:, None]
        t0 = time.perf_counter()
        while True:
            h = n % c.n_kv_heads
            K, V = w.natural_kv(b, h)
            eps = w.natural_rows(noise, b, h)
            for i in range(h * G, (h + 1) * G):
                fa.dim_sensitivity(w.f64(q4[b, :, i]), K, V, eps, scale)
            n += 1
            positions += int(w.lens[b])
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
        return {"value": positions / dt, "unit": "KV-positions/s", "cores": threads, "kind": "oracle",
                "sample": "%d (sequence, KV head) block(s) of sequence %d (L = %d): the oracle's "
                          "perturb-and-rerun analysis of its %d query heads x %d queries, %.1f s in all"
                          % (n, b, int(w.lens[b]), G, c.n_query, dt)}
    t0 = time.perf_counter()
    while True:
        h = n % c.n_kv_heads
        ck, cv = ob.project_block(w, b, h)
        if "decode" in c.steps:
            if c.n_query > 1:
                # attend_all over one block: the same per-head oracle call
                from oracle import fourier_attention as fa
                G = c.n_q_heads // c.n_kv_heads
                K, V = w.natural_kv(b, h)
                q = w.f64(w.q[b, :, h * G:(h + 1) * G]).reshape(-1, c.head_dim)
                fa.attend(q, K, V, w.comp_dims(h), ck, cv, c.sink, c.recent, scale)
            else:
                ob.decode_block(w, ck, cv, scale, b, h)
        n += 1
        positions += int(w.lens[b])
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    sample = ("%d (sequence, KV head) block(s) of sequence %d (L = %d, M = %d): oracle projection of "
              "K and V%s, %.1f s in all" % (n, b, int(w.lens[b]), w.mid_len(b),
                                            " + decode of its query rows" if "decode" in c.steps else "",
                                            dt))
    return {"value": positions / dt, "unit": "KV-positions/s", "cores": threads, "kind": "oracle",
            "sample": sample}


class Bench:
    """One workload uploaded in rotating copies, with its calls."""

    def __init__(self, torch, fb, w, copies=0):
        self.torch, self.fb, self.w = torch, fb, w
        c = self.c = w.cfg
        self.steps = c.steps
        dev = "cuda"
        self.scale = 1.0 / np.sqrt(c.head_dim)
        self.dims = torch.from_numpy(w.dims).to(dev)
        self.desc = fb.Desc.from_workload(w, self.dims)
        self.stream = torch.cuda.current_stream()
        self.sens = "sensitivity" in self.steps
        if self.sens:  # dimension analysis: keys and noise in natural dim order
            base = dict(q=fb.to_device(w.q), k=fb.to_device(w.natural_k_rows()),
                        noise=fb.to_device(w.value_noise()))
            per_copy = sum(t.numel() * t.element_size() for t in base.values())
            self.copies = copies or max(2, int(np.ceil(2 * LLC_BYTES / per_copy)) + 1)
            self.sets = []
            for i in range(self.copies):
                s = {k: (v if i == 0 else v.clone()) for k, v in base.items()}
                s["sq"] = torch.empty((c.n_q_heads, c.head_dim), device=dev)
                self.sets.append(s)
            self.ws_p = None
            self.ws_d = fb.workspace(fb.dim_sensitivity_workspace_size(self.desc, c.n_query))
            return
        nblk = c.batch * c.n_kv_heads
        E = c.sink + c.recent
        base = dict(kc=fb.to_device(w.kc), vc=fb.to_device(w.vc))
        if "decode" in self.steps:
            base.update(q=fb.to_device(w.q), kx=fb.to_device(w.kx), vx=fb.to_device(w.vx))
        per_copy = sum(t.numel() * t.element_size() for t in base.values())
        if "project" not in self.steps:  # decode reads kx, vx, q and the compressed parts
            per_copy -= sum(base[k].numel() * base[k].element_size() for k in ("kc", "vc"))
            per_copy += 2 * nblk * (c.n_coef * c.n_comp * 4 + E * c.n_comp * base["kc"].element_size())
        self.copies = copies or max(2, int(np.ceil(2 * LLC_BYTES / per_copy)) + 1)
        self.sets = []
        for i in range(self.copies):
            s = {}
            for k, v in base.items():
                # decode-only steps read kc / vc only through fa_project, run once per copy below
                s[k] = v if (i == 0 or (k in ("kc", "vc") and "project" not in self.steps)) else v.clone()
            s["ck"] = torch.empty((nblk, c.n_coef, c.n_comp), device=dev)
            s["cv"] = torch.empty_like(s["ck"])
            s["ke"] = torch.empty((nblk, E, c.n_comp), dtype=base["kc"].dtype, device=dev)
            s["ve"] = torch.empty_like(s["ke"])
            if "decode" in self.steps:
                oshape = (c.batch, c.n_q_heads, c.head_dim) if c.n_query == 1 else \
                    (c.batch, c.n_query, c.n_q_heads, c.head_dim)
                s["out"] = torch.empty(oshape, device=dev)
            self.sets.append(s)
        self.ws_p = fb.workspace(fb.project_workspace_size(self.desc))
        self.ws_d = fb.workspace(fb.attend_workspace_size(self.desc, c.n_query)) \
            if "decode" in self.steps else None
        if "decode" in self.steps and "project" not in self.steps:
            for s in self.sets:  # decode-only steps: coefficients and edges made once
                fb.project(self.desc, s["kc"], s["vc"], s["ck"], s["cv"], s["ke"], s["ve"], self.ws_p)

    def call_project(self, s):
        self.fb.project(self.desc, s["kc"], s["vc"], s["ck"], s["cv"], s["ke"], s["ve"], self.ws_p,
                        self.stream)

    def call_decode(self, s):
        c, fb = self.c, self.fb
        if self.sens:
            fb.dim_sensitivity(self.desc, c.n_query, s["q"], s["k"], s["noise"], self.scale, s["sq"],
                               self.ws_d, self.stream)
        elif c.n_query > 1:  # several queries per sequence: fa_attend
            fb.attend(self.desc, c.n_query, s["q"], s.get("kx"), s.get("vx"), s["ke"], s["ve"],
                      s["ck"], s["cv"], self.scale, s["out"], None, self.ws_d, self.stream)
        else:
            fb.decode(self.desc, s["q"], s.get("kx"), s.get("vx"), s["ke"], s["ve"], s["ck"],
                      s["cv"], self.scale, s["out"], self.ws_d, self.stream)

    def step(self, i, ev=None):
        s = self.sets[i % self.copies]
        if ev is not None:
            ev[0].record(self.stream)
        if "project" in self.steps:
            self.call_project(s)
        if ev is not None:
            ev[1].record(self.stream)
        if "decode" in self.steps or self.sens:
            self.call_decode(s)
        if ev is not None:
            ev[2].record(self.stream)

    def run(self, steps, warmup):
        """(ms per step over the timed region, per-call durations [s] of
        project and decode, per-launch durations [s] of the dominant kernel of
        each call)."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / steps
        # per-call durations: events on the launch stream around each call
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(steps):
            self.step(i, evs[i])
        torch.cuda.synchronize()
        d_proj = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
        d_dec = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
        # dominant kernel of each call: the library records a pair of events
        # around it on the same stream (fa_time_main_kernel)
        kern = {}
        for name, fn in (("project", self.call_project), ("decode", self.call_decode)):
            if name not in self.steps and not (name == "decode" and self.sens):
                continue
            pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(steps)]
            for i in range(steps):
                s = self.sets[i % self.copies]
                if name == "decode" and "project" in self.steps:
                    self.call_project(s)  # the step's own order, not timed here
                self.fb.time_main_kernel(*pairs[i])
                fn(s)
                self.fb.time_main_kernel(None, None)
            torch.cuda.synchronize()
            kern[name] = np.array([a.elapsed_time(b) for a, b in pairs]) * 1e-3
        return ms_step, d_proj, d_dec, kern


def spread(d):  # durations [s] -> microseconds
    p10, p50, p90 = np.percentile(d, [10, 50, 90]) * 1e6
    return {"p10": float(p10), "median": float(p50), "p90": float(p90)}


def projection_figures(torch, fb, wl, name, steps, warmup):
    """fa_project on its own workload: TFLOP/s of the call and of its main kernel."""
    w = wl.make(wl.CONFIGS[name])
    bn = Bench(torch, fb, w)
    _, _, flops, _ = algorithmic(w.cfg, w.lens)
    ms, d_proj, _, kern = bn.run(steps, warmup)
    t_call, t_kern = float(d_proj.mean()), float(kern["project"].mean())
    out = {"workload": name, "note": w.cfg.note, "n_coef": w.cfg.n_coef,
           "middle_tokens": w.mid_len(0), "columns": 2 * w.cfg.n_kv_heads * w.cfg.n_comp,
           "algorithmic_flops": flops, "steps": steps, "ms_per_step": ms,
           "project_us": t_call * 1e6, "project_us_spread": spread(d_proj),
           "project_tflops": flops / t_call / 1e12,
           "project_mfma_frac": flops / t_call / 1e12 / MFMA_F16_PEAK_TFLOPS,
           "main_kernel_us": t_kern * 1e6, "main_kernel_tflops": flops / t_kern / 1e12,
           "main_kernel_mfma_frac": flops / t_kern / 1e12 / MFMA_F16_PEAK_TFLOPS,
           "input_copies": bn.copies,
           "traffic_bytes_per_launch": measured_traffic(name, "project_main")}
    del bn
    torch.cuda.synchronize()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--projection", default=DEFAULT_PROJECTION,
                    help="workload whose fa_project is measured beside the step ('none' to skip)")
    ap.add_argument("--copies", type=int, default=0, help="input copies (0: enough to beat the LLC)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true", help="skip the approximation-error context")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure what the box reaches: a streaming copy and a read-only sum (HBM "
                         "GB/s) and a large fp16 GEMM (hipBLASLt through torch, MFMA TFLOP/s)")
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
    print("bench: %s, %d steps after %d warm-up" % (args.workload, args.steps, args.warmup),
          file=sys.stderr, flush=True)
    w = wl.make(wl.CONFIGS[args.workload])
    c = w.cfg
    steps = c.steps
    sens = "sensitivity" in steps
    if sens:  # the analysis is the step's one call, in the decode slot
        steps = ("decode",)
        args.no_context = True
    dec_bytes, main_bytes, proj_flops, positions = algorithmic(w.cfg, w.lens)
    bn = Bench(torch, fb, w, args.copies)
    ms_step, d_proj, d_dec, kern = bn.run(args.steps, args.warmup)
    t_proj = float(d_proj.mean())
    t_dec = float(d_dec.mean())

    extra = {}
    full_b, comp_b = fb.cache_bytes(bn.desc)
    extra["cache_bytes_full"] = full_b
    extra["cache_bytes_compressed"] = comp_b
    extra["cache_compression"] = 1.0 - comp_b / full_b
    extra["pages_budget_k"] = fb.coef_budget(w.mid_len(int(np.argmax(w.lens))), 0.3)
    if "decode" in steps:
        extra["decode_us"] = t_dec * 1e6
        extra["decode_us_spread"] = spread(d_dec)
        extra["decode_kv_positions_per_s"] = positions / t_dec
        extra["decode_hbm_GBps"] = dec_bytes / t_dec / 1e9
        extra["decode_hbm_frac"] = dec_bytes / t_dec / 1e9 / HBM_PEAK_GBS
        extra["decode_algorithmic_bytes"] = dec_bytes
        extra["decode_main_kernel_us"] = float(kern["decode"].mean()) * 1e6
        extra["decode_main_kernel_bytes"] = main_bytes
    if "project" in steps:
        extra["project_us"] = t_proj * 1e6
        extra["project_us_spread"] = spread(d_proj)
        extra["project_tflops"] = proj_flops / t_proj / 1e12
        extra["project_algorithmic_flops"] = proj_flops
        extra["project_main_kernel_us"] = float(kern["project"].mean()) * 1e6
    # dominant kernel: the main kernel of the call that takes the larger share
    # of the step, at its algorithmic bytes (flops) over its own duration
    if "decode" in steps and (t_dec >= t_proj or "project" not in steps):
        tk = float(kern["decode"].mean())
        ach = main_bytes / tk / 1e9
        roof = {"kernel": "main split kernel of %s" % (
                    "fa_dim_sensitivity (fa_attend with the noise as the values)" if sens
                    else "fa_decode" if c.n_query == 1 else "fa_attend"),
                "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "launch_us": tk * 1e6,
                "algorithmic_bytes_per_launch": main_bytes,
                "algorithmic": ("keys and noise of every token, all dims: Hkv * sum_b L_b * D * 2 * 2 B" if sens
                                else "exact dims of the middle rows, K and V: sum_b Hkv * M_b * Du * 2 * 2 B"),
                "traffic": measured_traffic(args.workload, "decode_main"),
                "call_achieved": dec_bytes / t_dec / 1e9,
                "call_frac": dec_bytes / t_dec / 1e9 / HBM_PEAK_GBS}
    else:
        tk = float(kern["project"].mean())
        ach = proj_flops / tk / 1e12
        roof = {"kernel": "projection kernel of fa_project", "bound": "mfma", "achieved": ach,
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / MFMA_F16_PEAK_TFLOPS,
                "launch_us": tk * 1e6, "algorithmic_flops_per_launch": proj_flops,
                "traffic": measured_traffic(args.workload, "project_main"),
                "call_achieved": proj_flops / t_proj / 1e12,
                "call_frac": proj_flops / t_proj / 1e12 / MFMA_F16_PEAK_TFLOPS}
    # context: the same achieved rate against what the box reaches outside the
    # library (streaming copy / hipBLASLt GEMM, measured by bench.py --peaks)
    try:
        with open(os.path.join(ROOT, "profiles", "box_peaks.json")) as f:
            bp = json.load(f)
        box = bp["copy_GBps"] if roof["unit"] == "GB/s" else bp["fp16_gemm_TFLOPs"]
        roof["box_peak"] = box
        roof["frac_of_box_peak"] = roof["achieved"] / box
    except (OSError, ValueError, KeyError):
        pass

    approx = None
    if not args.no_context:
        s0 = bn.sets[0]
        if "project" in steps:
            bn.call_project(s0)
        if "decode" in steps:
            bn.call_decode(s0)
        torch.cuda.synchronize()
        approx = approximation_context(
            w, s0["out"].cpu().numpy() if "decode" in steps else None,
            s0["ck"].cpu().numpy(), s0["cv"].cpu().numpy(), bn.scale)
    copies = bn.copies
    del bn
    torch.cuda.synchronize()

    if args.projection != "none" and args.projection != args.workload:
        print("bench: projection on %s" % args.projection, file=sys.stderr, flush=True)
        extra["projection"] = projection_figures(torch, fb, wl, args.projection,
                                                 max(5, args.steps // 3), min(args.warmup, 3))

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: CPU baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, 1.0 / np.sqrt(c.head_dim), args.cpu_seconds)

    if sens:
        metric = "KV-positions/s (dimension analysis, %d queries per sequence)" % c.n_query
    elif len(steps) == 2:
        metric = "KV-positions/s (fa_project K,V + fa_decode per step)"
    elif c.n_query == 1:
        metric = "decode KV-positions/s (%s)" % "+".join(steps)
    else:
        metric = "KV-positions/s (fa_attend, %d queries per sequence)" % c.n_query
    line = {
        "metric": metric,
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
        "launch": "eager",
        "roofline": roof,
        "cpu_baseline": cpu,
        "approx_error_vs_exact": approx,
        "calls": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
