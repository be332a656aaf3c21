"""Throughput of the fused GQA attention path on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 3] [--no-cpu-baseline]
                    [--modes decode_window,decode_varlen,append_rows,prefill_long,
                             prefill_qwen,prefill_tiny,gpu_clock,read_ceiling,copy_calibration]

One step = one decode step of the batched-decode workload (32 sequences,
12 Q / 2 KV heads, head_dim 128, 4096 cached tokens): append the new token's
K/V rows at position 4095 and attend over all 4096 positions, as one
attn_decode_append call (one launch: the split pass, whose last workgroup
per unit merges the splits and appends). The timed region
holds exactly --steps such steps back to back, bracketed by
torch.cuda.synchronize(); inputs rotate over three independent cache sets
(3 x 256 MiB, larger than the 256 MB Infinity Cache) so every step reads its
K/V from HBM. value = algorithmic K+V bytes per step / step time.

roofline: the attn_decode_append call, timed with HIP events on the stream it
is launched on around the timed region; achieved = algorithmic K+V bytes
(each attended K and V row read once) / mean time per call. The call is one
kernel, whose rocprofv3 duration matches the event time.

cpu_baseline: the fp64 oracle, built on this host with -O3 -march=native (no
-ffast-math, no FMA contraction), on the host's cores over the same decode
workload and inputs (repeated to >= 10 s; best pass reported).

modes: the other workloads, each timed the same way (mean per call over calls
launched back to back between one event pair; the median of per-call event
pairs, which add the events' own gaps, is reported beside it), each with the
oracle timed beside it on the same inputs (best of 3 for
the small and the decode workloads, once for the Qwen-shaped prefill, a stated
subset of the long prefill) and the parity of the GPU result against it:
sliding-window decode, varlen and rotary decode steps, bulk append (GB/s
against 8 TB/s HBM), causal prefill (TFLOP/s of 2*d*m*(m+1)*Hq against the
157.3 TFLOP/s fp32 matrix peak). gpu_clock samples the graphics clock while
the prefills run; read_ceiling times plain read kernels of the decode's byte
count (built with hipcc at run time) for the practical HBM read ceiling.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import subprocess
import sys
import tempfile
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix (256 CUs x 2.4 GHz x 256 FLOP/clk)
PEAK_CLOCK_MHZ = 2400.0
METRIC = ("decode K/V HBM GB/s (% of 8 TB/s); "
          "causal prefill fp32 TFLOP/s (% MFMA peak)")
HEADLINE = "decode_b32_hq12_hkv2_d128_t4096"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
TOL = 2e-5  # max|GPU - oracle| <= TOL * max|V| (fp32 against fp64)
DEFAULT_MODES = ("decode_window,decode_varlen,append_rows,prefill_long,prefill_qwen,"
                 "prefill_tiny,gpu_clock")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    """Hash of the kernel sources; traffic counters are only reported while
    the kernels are the ones they were measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_gqa_online_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key: str):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    rec = t.get(kernel_key)
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


def time_calls(fn, n, warmup, stream):
    """Per-call HIP event times (ms) of fn() on `stream`, plus wall ms/call."""
    import torch
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    t0 = time.perf_counter()
    for i in range(n):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / n
    return [a.elapsed_time(b) for a, b in evs], wall


def time_back_to_back(fn, n, warmup, stream, reps=3):
    """GPU time (ms) per call of fn(i): the mean over n calls launched back to
    back between one pair of HIP events on `stream` (no host work between
    calls, so dispatch gaps stay as short as in a serving loop); the median
    of `reps` such runs, so one slow stretch of clock does not decide it."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    means = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        means.append(e0.elapsed_time(e1) / n)
    return statistics.median(means)


# ------------------------------------------------------------------ host side

def host_info() -> dict:
    """This host's CPU: core counts and model name (lscpu)."""
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            if ln.strip().lower().startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            with open("/proc/cpuinfo") as f:
                for ln in f:
                    if ln.lower().startswith("model name"):
                        model = ln.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
    return {"nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": model, "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


class CpuOracle:
    """The oracle built for this host (-O3 -march=native, no -ffast-math, no
    FMA contraction) in a scratch directory, and timing helpers around it."""

    def __init__(self, host: dict):
        import oracle
        self._dir = tempfile.mkdtemp(prefix="oracle_native_")
        so = oracle.build(so_path=os.path.join(self._dir, "liboracle_native.so"), native=True)
        self.o = oracle.Oracle(so)
        self.threads = self.o.num_threads()
        self.host = host

    def time(self, fn, reps=3, min_seconds=0.0):
        """Run fn() at least `reps` times and until min_seconds have passed;
        returns (result of the last run, list of seconds per run)."""
        ts, out = [], None
        while len(ts) < reps or sum(ts) < min_seconds:
            t0 = time.perf_counter()
            out = fn()
            ts.append(time.perf_counter() - t0)
            if len(ts) >= 2000:
                break
        return out, ts

    def record(self, amount, unit_scale, unit, ts, sample, best=True):
        """cpu_baseline entry: `amount` of work (bytes or FLOP) per run,
        scaled by unit_scale (1e9 for GB/s or GFLOP/s, 1e12 for TFLOP/s)."""
        t = min(ts) if best else ts[-1]
        return {"value": round(amount / t / unit_scale, 6), "unit": unit,
                "cores": self.threads, "kind": "oracle",
                "seconds_per_run": round(t, 6), "runs": len(ts),
                "timing": "best of %d runs" % len(ts) if best else "one run",
                "sample": sample, "build": "gcc -O3 -march=native -fopenmp -ffp-contract=off",
                "nproc": self.host["nproc"], "cpu_model": self.host["cpu_model"]}


def parity(got, ref, vmax) -> dict:
    import numpy as np
    err = float(np.abs(got.astype(np.float64) - ref).max()) if got.size else 0.0
    return {"max_abs_err": err, "max_abs_v": vmax, "bound": TOL * vmax,
            "err_over_max_v": err / vmax if vmax else None, "ok": bool(err <= TOL * vmax)}


class ClockSampler:
    """Samples the graphics clock of every XCD (amd-smi metric -c) in a
    thread while the GPU runs a workload."""

    def __init__(self, gpu_index=0):
        self.gpu = gpu_index
        self.samples = []
        self._stop = threading.Event()
        self._t = None
        self.error = None

    def _one(self):
        out = subprocess.run(["amd-smi", "metric", "-g", str(self.gpu), "-c", "--json"],
                             capture_output=True, text=True, timeout=20).stdout
        data = json.loads(out)
        if isinstance(data, dict):
            data = data.get("gpu_data", [data])
        clk = data[0]["clock"]
        vals = [v["clk"]["value"] for k, v in sorted(clk.items())
                if k.startswith("gfx") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
                and isinstance(v["clk"].get("value"), (int, float))]
        if vals:
            self.samples.append(vals)

    def _run(self):
        while not self._stop.is_set():
            try:
                self._one()
            except Exception as e:  # tool missing or output changed: no clock figure
                self.error = f"{type(e).__name__}: {e}"
                return

    def __enter__(self):
        self._t = threading.Thread(target=self._run, daemon=True)
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join(timeout=30)

    def summary(self):
        if not self.samples:
            return {"mhz": None, "error": self.error}
        flat = [x for s in self.samples for x in s]
        return {"mhz": round(statistics.mean(flat), 1), "min_mhz": min(flat),
                "max_mhz": max(flat), "samples": len(self.samples),
                "xcds": len(self.samples[0]), "source": "amd-smi metric -c (gfx clocks)"}


# ------------------------------------------------------------------ workloads

def bench_headline(args, dev, orc):
    import numpy as np
    import torch
    import attention_gqa_online_amd as A
    import synth

    w = synth.WORKLOADS[HEADLINE]
    stream = torch.cuda.current_stream()
    sets, host0 = [], None
    for r in range(3):
        q, k, v = synth.decode_inputs(w, seed=w.seed + r)
        ks, vs = synth.append_inputs(w.batch, w.kv_heads, w.head_dim, seed=w.seed + 10 + r)
        sets.append(tuple(torch.from_numpy(x).to(dev) for x in (q, k, v, ks, vs)))
        if r == 0:
            host0 = (q, k, v, ks, vs)
    out = torch.empty(w.batch, w.num_heads, w.head_dim, device=dev)
    ws = A.decode_workspace(w.batch, w.num_heads, w.kv_heads, w.head_dim, w.total_seq,
                            w.window, device=dev)
    pos = w.total_seq - 1

    # device addresses and the stream as plain ints: the binding passes them
    # straight through, so the host side of a step is one ctypes call
    sint = stream.cuda_stream
    ptrs = [tuple(x.data_ptr() for x in st) for st in sets]
    outp, wsp, wsb = out.data_ptr(), ws.data_ptr(), ws.numel()

    def step(i):
        qp, kp, vp, ksp, vsp = ptrs[i % 3]
        A.attn_decode_append(qp, ksp, vsp, kp, vp, outp, w.batch, w.num_heads, w.kv_heads,
                             w.head_dim, w.max_seq, pos, w.window, w.scale, wsp, wsb, stream=sint)

    def two_call_step(i):
        q, k, v, ks, vs = sets[i % 3]
        A.kv_append(ks, vs, k, v, w.batch, w.kv_heads, w.head_dim, w.max_seq, pos)
        A.attn_decode(q, k, v, out, w.batch, w.num_heads, w.kv_heads, w.head_dim,
                      w.max_seq, w.total_seq, w.window, w.scale, ws)

    for i in range(args.warmup):
        step(i)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    mean_kern = ev0.elapsed_time(ev1) / args.steps  # GPU time per call over the timed region
    # per-call event times, for the spread (a separate pass)
    kern_ms, _ = time_calls(step, args.steps, 0, stream)
    bytes_ = w.kv_bytes()
    value = bytes_ / (ms_per_step * 1e-3) / 1e9
    achieved = bytes_ / (mean_kern * 1e-3) / 1e9
    log(f"[bench] headline decode step: {ms_per_step * 1e3:.1f} us/step wall, "
        f"{mean_kern * 1e3:.1f} us/step by events (per-call median "
        f"{statistics.median(kern_ms) * 1e3:.1f}, min {min(kern_ms) * 1e3:.1f}), "
        f"{achieved:.0f} GB/s")
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("attn_decode_append"),
            "kernel": "attn_decode_append: decode_kernel<128, 6, ...> split pass with "
                      "the merge and append in its last workgroup per unit",
            "kernel_mean_us": round(mean_kern * 1e3, 2),
            "per_call_median_us": round(statistics.median(kern_ms) * 1e3, 2),
            "algorithmic_bytes_per_launch": bytes_}

    # parity of the timed step on input set 0 against the oracle (the cache
    # with the appended row, attended over all 4096 rows)
    step(0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    q0, k0, v0, ks0, vs0 = host0
    k0, v0 = k0.copy(), v0.copy()
    cpu = None
    if orc is not None:
        orc.o.kv_append(ks0, vs0, k0, v0, w.batch, w.kv_heads, w.head_dim, w.max_seq, pos)
        ref, ts = orc.time(lambda: orc.o.decode(q0, k0, v0, w.batch, w.num_heads, w.kv_heads,
                                                w.head_dim, w.max_seq, w.total_seq, w.window,
                                                w.scale), reps=3, min_seconds=10.0)
        roof["parity"] = parity(got, ref, float(np.abs(v0).max()))
        cpu = orc.record(bytes_, 1e9, "GB/s", ts,
                         f"the whole decode workload ({w.batch} sequences x {w.num_heads} heads "
                         f"over {w.total_seq} positions, input set 0 with the appended row), "
                         f"fp64 two-pass softmax; {len(ts)} passes in {sum(ts):.1f} s")
        log(f"[bench] cpu oracle (headline): {len(ts)} passes in {sum(ts):.1f} s, best "
            f"{min(ts) * 1e3:.1f} ms = {cpu['value']:.2f} GB/s; parity {roof['parity']}")

    # the same step as two calls (kv_append, then attn_decode), for comparison
    ms2, _ = time_calls(two_call_step, args.steps, args.warmup, stream)
    two = {"step": "kv_append + attn_decode", "median_us": round(statistics.median(ms2) * 1e3, 2),
           "GB/s": round(bytes_ / (statistics.median(ms2) * 1e-3) / 1e9, 1)}
    log(f"[bench] two-call step: median {two['median_us']:.1f} us")
    # the same step replayed from a captured HIP graph (one graph per input set)
    graphs = []
    for i in range(3):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            qp, kp, vp, ksp, vsp = ptrs[i]
            A.attn_decode_append(qp, ksp, vsp, kp, vp, outp, w.batch, w.num_heads,
                                 w.kv_heads, w.head_dim, w.max_seq, pos, w.window, w.scale,
                                 wsp, wsb)
        graphs.append(g)
    for i in range(3):
        graphs[i].replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record(stream)
    for i in range(args.steps):
        graphs[i % 3].replay()
    g1.record(stream)
    torch.cuda.synchronize()
    gwall = (time.perf_counter() - t0) * 1e3 / args.steps
    gev = g0.elapsed_time(g1) / args.steps
    graph = {"step": "attn_decode_append replayed from a captured HIP graph",
             "us_per_step_wall": round(gwall * 1e3, 2),
             "us_per_step_events": round(gev * 1e3, 2)}
    log(f"[bench] graph replay: {gwall * 1e3:.1f} us/step wall, {gev * 1e3:.1f} us by events")
    # the same step with rotary embedding (attn_decode_rope_append)
    cos_h, sin_h = synth.rope_tables(w.head_dim, pos)
    cs = [torch.from_numpy(x).to(dev) for x in (cos_h, sin_h)]
    cp, sp = cs[0].data_ptr(), cs[1].data_ptr()

    def rope_step(i):
        qp, kp, vp, ksp, vsp = ptrs[i % 3]
        A.attn_decode_rope_append(qp, ksp, vsp, cp, sp, kp, vp, outp, w.batch, w.num_heads,
                                  w.kv_heads, w.head_dim, w.max_seq, pos, w.window, w.scale,
                                  wsp, wsb, stream=sint)

    # timed as the headline step is: back to back between one event pair
    # (per-call event pairs add host work per call, which can leave the GPU
    # idle between calls and expose each dispatch)
    for i in range(args.warmup):
        rope_step(i)
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(args.steps):
        rope_step(i)
    r1.record(stream)
    torch.cuda.synchronize()
    rwall = (time.perf_counter() - t0) * 1e3 / args.steps
    rev = r0.elapsed_time(r1) / args.steps
    ms3, _ = time_calls(rope_step, args.steps, 0, stream)
    rope = {"step": "attn_decode_rope_append", "us_per_step_events": round(rev * 1e3, 2),
            "us_per_step_wall": round(rwall * 1e3, 2),
            "median_us": round(statistics.median(ms3) * 1e3, 2),
            "GB/s": round(bytes_ / (rev * 1e-3) / 1e9, 1)}
    log(f"[bench] rotary decode step: {rev * 1e3:.1f} us/step by events, "
        f"{rwall * 1e3:.1f} us/step wall (per-call median {rope['median_us']:.1f})")
    if orc is not None:
        # the rotary step on input set 0: the step wrote the rotated row at
        # `pos` into the device cache; the oracle starts from the host cache
        # and writes its own rotated row
        rope_step(0)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        q0, k0r, v0r = host0[0], host0[1].copy(), host0[2].copy()
        ref, ts = orc.time(lambda: orc.o.decode_rope_append(
            q0, ks0, vs0, cos_h, sin_h, k0r, v0r, w.batch, w.num_heads, w.kv_heads,
            w.head_dim, w.max_seq, pos, w.window, w.scale))
        v0r[:, :, pos, :] = vs0
        rope["parity"] = parity(got, ref, float(np.abs(v0r).max()))
        rope["cpu_baseline"] = orc.record(bytes_, 1e9, "GB/s", ts,
                                          "the whole rotary decode step on input set 0")
        log(f"[bench] cpu oracle (rotary step): best {min(ts) * 1e3:.1f} ms; "
            f"parity {rope['parity']}")
    return w, value, ms_per_step, roof, cpu, two, rope, graph


def bench_decode_window(args, dev, orc):
    import numpy as np
    import torch
    import attention_gqa_online_amd as A
    import synth
    w = synth.WORKLOADS["decode_b16_hq32_hkv8_d128_t32768_w4096"]
    # input set 0 from the numpy recipe (what the oracle sees), set 1 drawn
    # on the device with the same distributions
    qh, kh, vh = synth.decode_inputs(w)
    sets = [tuple(torch.from_numpy(x).to(dev) for x in (qh, kh, vh)),
            synth.decode_inputs_device(w, w.seed + 1, dev)]
    out = torch.empty(w.batch, w.num_heads, w.head_dim, device=dev)
    ws = A.decode_workspace(w.batch, w.num_heads, w.kv_heads, w.head_dim, w.total_seq,
                            w.window, device=dev)
    stream = torch.cuda.current_stream()

    def call(i):
        q, k, v = sets[i % 2]
        A.attn_decode(q, k, v, out, w.batch, w.num_heads, w.kv_heads, w.head_dim,
                      w.max_seq, w.total_seq, w.window, w.scale, ws)
    n = max(args.steps, 10)
    mean = time_back_to_back(call, n, args.warmup, stream)
    ms, wall = time_calls(call, n, 0, stream)
    med = statistics.median(ms)
    gbs = w.kv_bytes() / (mean * 1e-3) / 1e9
    call(0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del sets
    torch.cuda.empty_cache()
    log(f"[bench] window decode: {mean * 1e3:.1f} us per call back to back, {gbs:.0f} GB/s "
        f"(per-call event median {med * 1e3:.1f} us)")
    res = {"workload": w.name, "us_per_call": round(mean * 1e3, 2),
           "median_us": round(med * 1e3, 2), "min_us": round(min(ms) * 1e3, 2),
           "GB/s": round(gbs, 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic("attn_decode_window")},
           "algorithmic_bytes": w.kv_bytes()}
    if orc is not None:
        ref, ts = orc.time(lambda: orc.o.decode(qh, kh, vh, w.batch, w.num_heads, w.kv_heads,
                                                w.head_dim, w.max_seq, w.total_seq, w.window,
                                                w.scale))
        res["parity"] = parity(got, ref, float(np.abs(vh[:, :, w.window_start:]).max()))
        res["cpu_baseline"] = orc.record(
            w.kv_bytes(), 1e9, "GB/s", ts,
            "the whole windowed decode workload (input set 0: 16 sequences x 32 heads over "
            "the 4096-row window of 32768)")
        log(f"[bench] cpu oracle (window): best {min(ts) * 1e3:.1f} ms; parity {res['parity']}")
    return res


def bench_prefill(args, dev, name, orc, clock=False):
    import numpy as np
    import torch
    import attention_gqa_online_amd as A
    import synth
    w = synth.WORKLOADS[name]
    qh, kh, vh = synth.prefill_inputs(w)
    q, k, v = (torch.from_numpy(x).to(dev) for x in (qh, kh, vh))
    o = torch.empty(w.m, w.q_stride, device=dev)
    stream = torch.cuda.current_stream()

    def call(i):
        A.attn_prefill_causal(q, k, v, o, w.m, w.q_stride, w.kv_stride, w.num_q_heads,
                              w.heads_per_kv, w.head_dim)
    n = max(args.steps, 10) if w.m <= 4096 else max(5, min(args.steps, 10))
    mean = time_back_to_back(call, n, args.warmup, stream)
    ms, wall = time_calls(call, n, 0, stream)
    med = statistics.median(ms)
    # a launch-latency-bound call (a few microseconds: back to back, the host's
    # launches set the pace) is timed by its own latency, the per-call median
    latency_bound = w.m <= 64
    t_used = med if latency_bound else mean
    tfl = w.flops() / (t_used * 1e-3) / 1e12
    res = {"workload": name, "us_per_call": round(mean * 1e3, 2),
           "median_us": round(med * 1e3, 2), "min_us": round(min(ms) * 1e3, 2),
           "TFLOP/s": round(tfl, 3),
           "timing": "per-call event median (launch-latency bound)" if latency_bound
                     else "back-to-back mean per call, median of 3 runs",
           "roofline": {"bound": "mfma", "achieved": round(tfl, 3),
                        "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tfl / FP32_MFMA_PEAK_TFLOPS, 4),
                        "traffic": measured_traffic("attn_prefill_causal:" + name)},
           "algorithmic_flops": w.flops(), "launches_per_call": 1}
    log(f"[bench] {name}: {mean * 1e3:.1f} us per call back to back, per-call event median "
        f"{med * 1e3:.1f} us; {tfl:.2f} TFLOP/s")
    if clock:
        # the graphics clock while this prefill runs back to back for ~3 s
        sampler = ClockSampler()
        reps = max(1, int(3.0 / (t_used * 1e-3)))
        with sampler:
            for _ in range(reps):
                call(0)
            torch.cuda.synchronize()
        c = sampler.summary()
        if c.get("mhz"):
            peak_at = FP32_MFMA_PEAK_TFLOPS * c["mhz"] / PEAK_CLOCK_MHZ
            c["peak_TFLOP/s_at_clock"] = round(peak_at, 2)
            c["frac_at_clock"] = round(tfl / peak_at, 4)
        res["gpu_clock"] = c
        log(f"[bench] {name}: graphics clock while running {c}")
    call(0)
    torch.cuda.synchronize()
    heads = o[:, : w.num_q_heads * w.head_dim].view(w.m, w.num_q_heads, w.head_dim)
    vmax = float(np.abs(vh[:, : w.kv_heads * w.head_dim]).max())
    if orc is not None:
        if w.m <= 4096:
            ref, ts = orc.time(lambda: orc.o.prefill_causal(
                qh, kh, vh, w.m, w.q_stride, w.kv_stride, w.num_q_heads, w.heads_per_kv,
                w.head_dim), reps=3 if w.m <= 64 else 1)
            res["parity"] = parity(heads.cpu().numpy(), ref, vmax)
            res["cpu_baseline"] = orc.record(
                w.flops(), 1e9, "GFLOP/s", ts, f"the whole prefill workload ({name})",
                best=len(ts) > 1)
        else:
            # every row of heads 0, 7 and 63 and 4096 seeded random (row,
            # head) pairs, timed once; the rate extrapolates to the workload
            rng = np.random.default_rng(2005)
            rows = np.concatenate([np.tile(np.arange(w.m), 3), rng.integers(0, w.m, 4096)])
            hsel = np.concatenate([np.repeat([0, 7, 63], w.m),
                                   rng.integers(0, w.num_q_heads, 4096)])
            ref, ts = orc.time(lambda: orc.o.prefill_causal(
                qh, kh, vh, w.m, w.q_stride, w.kv_stride, w.num_q_heads, w.heads_per_kv,
                w.head_dim, rows=rows, heads=hsel), reps=1)
            got = heads[torch.from_numpy(rows).to(dev), torch.from_numpy(hsel).to(dev)]
            res["parity"] = parity(got.cpu().numpy(), ref, vmax)
            sub_flops = int(4 * w.head_dim * (rows.astype(np.int64) + 1).sum())
            rec = orc.record(sub_flops, 1e9, "GFLOP/s", ts,
                             "every row of heads 0, 7 and 63 plus 4096 seeded random "
                             f"(row, head) pairs: {sub_flops / 1e9:.1f} GFLOP of the "
                             f"{w.flops() / 1e9:.0f}, timed once", best=False)
            rec["extrapolated_seconds_for_workload"] = round(ts[-1] * w.flops() / sub_flops, 1)
            res["cpu_baseline"] = rec
        log(f"[bench] cpu oracle ({name}): {ts[-1]:.2f} s; parity {res['parity']}")
    del q, k, v, o, heads
    torch.cuda.empty_cache()
    return res


def bench_decode_varlen(args, dev, orc):
    """Serving-shaped decode step: the decode workload's shape (32 sequences,
    12 query / 2 KV heads of 128, caches of 4096 rows) with each sequence at
    its own position, lengths uniform in [1, 4096] (seeded); one
    attn_decode_append_varlen call per step."""
    import numpy as np
    import torch
    import attention_gqa_online_amd as A
    import synth
    w = synth.WORKLOADS[HEADLINE]
    lens = synth.seq_lengths(w.batch, w.total_seq, seed=w.seed + 100)
    qh, kh, vh = synth.decode_inputs(w, seed=w.seed + 20)
    sets = [tuple(torch.from_numpy(x).to(dev) for x in (qh, kh, vh))]
    sets += [synth.decode_inputs_device(w, w.seed + 20 + r, dev) for r in (1, 2)]
    knh, vnh = synth.append_inputs(w.batch, w.kv_heads, w.head_dim, seed=w.seed + 30)
    kn, vn = torch.from_numpy(knh).to(dev), torch.from_numpy(vnh).to(dev)
    pos = torch.from_numpy((lens - 1).astype(np.int32)).to(dev)
    out = torch.empty(w.batch, w.num_heads, w.head_dim, device=dev)
    ws = A.decode_workspace(w.batch, w.num_heads, w.kv_heads, w.head_dim, w.total_seq,
                            w.window, device=dev)
    stream = torch.cuda.current_stream()

    def call(i):
        q, k, v = sets[i % 3]
        A.attn_decode_append_varlen(q, kn, vn, k, v, out, pos, w.batch, w.num_heads,
                                    w.kv_heads, w.head_dim, w.max_seq, w.total_seq, w.window,
                                    w.scale, ws)
    n = max(args.steps, 10)
    mean = time_back_to_back(call, n, args.warmup, stream)
    ms, wall = time_calls(call, n, 0, stream)
    med = statistics.median(ms)
    bytes_ = int(2 * w.kv_heads * w.head_dim * 4 * int(lens.astype(np.int64).sum()))
    gbs = bytes_ / (mean * 1e-3) / 1e9
    call(0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()

    # the same step with rotary embedding, one cos/sin table per sequence
    tabs = [synth.rope_tables(w.head_dim, int(p)) for p in lens - 1]
    cos_t = torch.from_numpy(np.ascontiguousarray(np.stack([t[0] for t in tabs]))).to(dev)
    sin_t = torch.from_numpy(np.ascontiguousarray(np.stack([t[1] for t in tabs]))).to(dev)

    def rope_call(i):
        q, k, v = sets[i % 3]
        A.attn_decode_rope_append_varlen(q, kn, vn, cos_t, sin_t, k, v, out, pos, w.batch,
                                         w.num_heads, w.kv_heads, w.head_dim, w.max_seq,
                                         w.total_seq, w.window, w.scale, ws)
    mean_r = time_back_to_back(rope_call, n, args.warmup, stream)
    del sets
    torch.cuda.empty_cache()
    log(f"[bench] varlen decode step: {mean * 1e3:.1f} us per call back to back, {gbs:.0f} GB/s "
        f"(per-call event median {med * 1e3:.1f} us; mean length {lens.mean():.0f}); "
        f"rotary varlen step: {mean_r * 1e3:.1f} us per call back to back")
    res = {"workload": "decode_varlen_b32_hq12_hkv2_d128_t4096_uniform",
           "step": "attn_decode_append_varlen", "mean_len": round(float(lens.mean()), 1),
           "us_per_call": round(mean * 1e3, 2),
           "median_us": round(med * 1e3, 2), "min_us": round(min(ms) * 1e3, 2),
           "GB/s": round(gbs, 1),
           "rope_step": {"step": "attn_decode_rope_append_varlen",
                         "us_per_call": round(mean_r * 1e3, 2),
                         "GB/s": round(bytes_ / (mean_r * 1e-3) / 1e9, 1)},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic("attn_decode_append_varlen")},
           "algorithmic_bytes": bytes_}
    if orc is not None:
        # the oracle's cache: input set 0 with each sequence's new row at its
        # own position (the append is a copy, per sequence)
        kh, vh = kh.copy(), vh.copy()
        for b in range(w.batch):
            orc.o.kv_append(knh[b:b + 1], vnh[b:b + 1], kh[b:b + 1], vh[b:b + 1], 1,
                            w.kv_heads, w.head_dim, w.max_seq, int(lens[b]) - 1)
        ref, ts = orc.time(lambda: orc.o.decode_varlen(qh, kh, vh, lens, w.batch, w.num_heads,
                                                       w.kv_heads, w.head_dim, w.max_seq,
                                                       w.window, w.scale))
        vmax = max(float(np.abs(vh[b, :, :int(t)]).max()) for b, t in enumerate(lens))
        res["parity"] = parity(got, ref, vmax)
        res["cpu_baseline"] = orc.record(bytes_, 1e9, "GB/s", ts,
                                         "the whole varlen step on input set 0")
        log(f"[bench] cpu oracle (varlen): best {min(ts) * 1e3:.1f} ms; parity {res['parity']}")
    return res


def bench_append_rows(args, dev, orc):
    """Prefill -> cache hand-over at the long prefill's shape: 16384 rows of
    8 KV heads x 128 into [8, 16384, 128] caches (K and V read once, written
    once)."""
    import numpy as np
    import torch
    import attention_gqa_online_amd as A
    import synth
    m, hkv, d = 16384, 8, 128
    rng = np.random.default_rng(7)
    kh = synth.normal(rng, (m, hkv * d), 1.0)
    vh = synth.normal(rng, (m, hkv * d), 1.0)
    k, v = torch.from_numpy(kh).to(dev), torch.from_numpy(vh).to(dev)
    caches = [(torch.empty((hkv, m, d), device=dev), torch.empty((hkv, m, d), device=dev))
              for _ in range(2)]
    stream = torch.cuda.current_stream()

    def call(i):
        kc, vc = caches[i % 2]
        A.kv_append_rows(k, v, kc, vc, m, hkv * d, hkv, d, m, 0)
    n = max(args.steps, 10)
    mean = time_back_to_back(call, n, args.warmup, stream)
    ms, wall = time_calls(call, n, 0, stream)
    med = statistics.median(ms)
    bytes_ = 4 * m * hkv * d * 4
    gbs = bytes_ / (mean * 1e-3) / 1e9
    log(f"[bench] kv_append_rows: {mean * 1e3:.1f} us per call back to back, {gbs:.0f} GB/s "
        f"(per-call event median {med * 1e3:.1f} us)")
    res = {"workload": "append_rows_m16384_hkv8_d128", "us_per_call": round(mean * 1e3, 2),
           "median_us": round(med * 1e3, 2), "min_us": round(min(ms) * 1e3, 2),
           "GB/s": round(gbs, 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic("kv_append_rows")},
           "algorithmic_bytes": bytes_}
    if orc is not None:
        kc_h = np.zeros((hkv, m, d), np.float32)
        vc_h = np.zeros((hkv, m, d), np.float32)
        _, ts = orc.time(lambda: orc.o.kv_append_rows(kh, vh, kc_h, vc_h, m, hkv * d, hkv, d,
                                                      m, 0))
        same = bool(np.array_equal(caches[0][0].cpu().numpy(), kc_h) and
                    np.array_equal(caches[0][1].cpu().numpy(), vc_h))
        res["parity"] = {"bit_exact": same, "ok": same}
        res["cpu_baseline"] = orc.record(bytes_, 1e9, "GB/s", ts, "the whole bulk append")
        log(f"[bench] cpu oracle (bulk append): best {min(ts) * 1e3:.1f} ms; bit-exact {same}")
    del k, v, caches
    torch.cuda.empty_cache()
    return res


READ_CEILING_SRC = r"""
// Plain read kernels: each workgroup reads one contiguous chunk of two
// buffers (like K and V), U 16-byte nontemporal loads of each in flight per
// thread, and keeps a sum so the loads are not dropped.
#include <hip/hip_runtime.h>
typedef float v4 __attribute__((ext_vector_type(4)));
template <int U, int NT>
__global__ __launch_bounds__(NT) void rd2(const v4 *__restrict__ a, const v4 *__restrict__ b,
                                          size_t n4, size_t chunk4, float *out) {
    const size_t lo = blockIdx.x * chunk4;
    const size_t hi = lo + chunk4 < n4 ? lo + chunk4 : n4;
    v4 acc = {0, 0, 0, 0};
    size_t i = lo + threadIdx.x;
    for (; i + (U - 1) * NT < hi; i += U * NT) {
        v4 x[U], y[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load(a + i + u * NT);
#pragma unroll
        for (int u = 0; u < U; ++u) y[u] = __builtin_nontemporal_load(b + i + u * NT);
#pragma unroll
        for (int u = 0; u < U; ++u) acc += x[u] * y[u];
    }
    for (; i < hi; i += NT) acc += __builtin_nontemporal_load(a + i) * __builtin_nontemporal_load(b + i);
    if (acc.x + acc.y + acc.z + acc.w == 1234.5f) out[0] = acc.x;
}
// n4: float4 per buffer; a and b must each hold n4 float4.
extern "C" int read_two(int kind, const void *a, const void *b, size_t n4, unsigned grid,
                        float *out, hipStream_t s) {
    const size_t chunk4 = (n4 + grid - 1) / grid;
    if (kind == 0)
        hipLaunchKernelGGL((rd2<4, 256>), dim3(grid), dim3(256), 0, s, (const v4 *)a,
                           (const v4 *)b, n4, chunk4, out);
    else
        hipLaunchKernelGGL((rd2<2, 512>), dim3(grid), dim3(512), 0, s, (const v4 *)a,
                           (const v4 *)b, n4, chunk4, out);
    return (int)hipGetLastError();
}
"""


def build_read_ceiling(so: str) -> str:
    """Compile the plain read kernels (READ_CEILING_SRC) with hipcc into `so`."""
    os.makedirs(os.path.dirname(os.path.abspath(so)), exist_ok=True)
    src = os.path.splitext(os.path.abspath(so))[0] + ".hip"
    with open(src, "w") as f:
        f.write(READ_CEILING_SRC)
    subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "-o", so, src], stderr=subprocess.DEVNULL)
    return so


def bench_read_ceiling(args, dev):
    """Practical HBM read ceiling at the decode step's byte count: plain read
    kernels (two buffers of 128 MiB per call, like the caches' K and V; three
    such pairs in rotation), built with hipcc here unless --read-ceiling-so
    names one built beforehand (--build-read-ceiling)."""
    import ctypes
    import torch
    so = args.read_ceiling_so
    if not so or not os.path.exists(so):
        so = build_read_ceiling(so or os.path.join(tempfile.mkdtemp(prefix="read_ceiling_"),
                                                   "libread_ceiling.so"))
    lib = ctypes.CDLL(so)
    lib.read_two.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                             ctypes.c_uint, ctypes.c_void_p, ctypes.c_void_p]
    half = 128 * 2**20
    bufs = [(torch.zeros(half // 4, device=dev), torch.zeros(half // 4, device=dev))
            for _ in range(3)]
    out = torch.zeros(1, device=dev)
    stream = torch.cuda.current_stream()
    n4 = half // 16
    res = {"bytes_per_call": 2 * half, "kernels": {}}
    for kind, label in ((0, "4 waves/workgroup, 8 loads of 16 B in flight per lane"),
                        (1, "8 waves/workgroup, 4 loads of 16 B in flight per lane")):
        for grid in (256, 512, 1024, 4096):
            def call(i):
                a, b = bufs[i % 3]
                rc = lib.read_two(kind, a.data_ptr(), b.data_ptr(), n4, grid, out.data_ptr(),
                                  stream.cuda_stream)
                assert rc == 0, rc
            for i in range(6):
                call(i)
            torch.cuda.synchronize()
            per = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(20):
                    call(i)
                e1.record(stream)
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) / 20 * 1e3)
            med = statistics.median(per)
            res["kernels"][f"{label}, grid {grid}"] = {
                "us_per_call": round(med, 2), "GB/s": round(2 * half / (med * 1e-6) / 1e9, 1)}
    best = min(v["us_per_call"] for v in res["kernels"].values())
    res["best_us"] = best
    res["best_GB/s"] = round(2 * half / (best * 1e-6) / 1e9, 1)
    log(f"[bench] read ceiling at {2 * half} B: best {best:.2f} us = {res['best_GB/s']} GB/s")
    del bufs
    torch.cuda.empty_cache()
    return res


def copy_calibration(dev, mib=256, reps=3):
    """A plain device copy of known size, for scaling HBM byte counters: each
    copy reads and writes exactly `mib` MiB."""
    import torch
    src = torch.ones(mib * 2**20 // 4, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes_read_per_copy": mib * 2**20, "bytes_written_per_copy": mib * 2**20,
            "copies": reps, "kernel": "torch copy_ (elementwise copy kernel)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--modes", default=DEFAULT_MODES,
                    help="comma list; the headline decode step always runs "
                         "(also: read_ceiling, copy_calibration)")
    ap.add_argument("--read-ceiling-so", default=None,
                    help="read_ceiling: the plain read kernels' library (built there if missing)")
    ap.add_argument("--build-read-ceiling", default=None, metavar="SO",
                    help="only build the read_ceiling library at SO (no GPU use), then exit")
    args = ap.parse_args()
    if args.build_read_ceiling:
        print(build_read_ceiling(args.build_read_ceiling))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU code; each GPU would run its own share)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_gqa_online_amd as A
    if not os.path.exists(A.SO_PATH):
        import __graft_entry__
        __graft_entry__.build()
    A.library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    modes = set(args.modes.split(","))
    host = host_info()
    orc = None if args.no_cpu_baseline else CpuOracle(host)

    w, value, ms_per_step, roof, cpu, two, rope, graph = bench_headline(args, dev, orc)
    extra = {"decode_step_two_calls": two, "decode_step_graph": graph, "decode_step_rope": rope}
    if "decode_window" in modes:
        extra["decode_window"] = bench_decode_window(args, dev, orc)
    if "decode_varlen" in modes:
        extra["decode_varlen"] = bench_decode_varlen(args, dev, orc)
    if "append_rows" in modes:
        extra["append_rows"] = bench_append_rows(args, dev, orc)
    clock = "gpu_clock" in modes
    if "prefill_long" in modes:
        extra["prefill_long"] = bench_prefill(args, dev, "prefill_hq64_hkv8_d128_m16384", orc,
                                              clock)
    if "prefill_qwen" in modes:
        extra["prefill_qwen"] = bench_prefill(args, dev, "prefill_hq28_hkv4_d128_m2048", orc,
                                              clock)
    if "prefill_tiny" in modes:
        extra["prefill_tiny"] = bench_prefill(args, dev, "prefill_hq4_hkv2_d32_m16", orc)
    if "read_ceiling" in modes:
        extra["read_ceiling"] = bench_read_ceiling(args, dev)
        extra["read_ceiling"]["decode_step_frac_of_ceiling"] = round(
            roof["achieved"] / extra["read_ceiling"]["best_GB/s"], 4)
    if "copy_calibration" in modes:
        extra["copy_calibration"] = copy_calibration(dev)

    # the pages' one figure for this path, beside this library's counterpart
    context = {
        "pages": "fusing the prefill attention of each of 28 Qwen 2.5 layers from five "
                 "launches into one (140 -> 28 launches) saves about 7.5 ms of time to first "
                 "token, fp32, on an RTX 4060 Laptop GPU (aprender-gpu 0.32.0 "
                 "prefill_fused.rs page, module doc); another machine, context only",
        "this_library": {"prefill_launches_per_layer": 1,
                         "prefill_launches_28_layers": 28}}
    if "prefill_qwen" in extra:
        per = extra["prefill_qwen"]["us_per_call"]
        context["this_library"]["attention_ms_28_layers_m2048_qwen_shaped"] = round(
            28 * per / 1e3, 3)
        context["this_library"]["note"] = (
            "28 x one attn_prefill_causal call of the Qwen-2.5-7B-shaped layer (28 Q / 4 KV "
            "heads, d 128, 2048 tokens); the pages give neither prompt length nor model size")

    props = torch.cuda.get_device_properties(dev)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "num_heads": w.num_heads,
                   "kv_heads": w.kv_heads, "head_dim": w.head_dim,
                   "total_seq": w.total_seq, "window": w.window,
                   "step": "attn_decode_append (append at 4095 + attend 4096)",
                   "input_sets": 3},
        "roofline": roof,
        "cpu_baseline": cpu,
        "modes": extra,
        "context": context,
        "host": host,
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "kernel_sources": source_digest(),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
