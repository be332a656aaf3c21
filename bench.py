"""Throughput of the fused GQA attention path on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-cpu-baseline]
                    [--modes headline,decode_window,prefill_long,prefill_qwen,prefill_tiny]

One step = one decode step of the batched-decode workload (32 sequences,
12 Q / 2 KV heads, head_dim 128, 4096 cached tokens): append the new token's
K/V rows at position 4095 and attend over all 4096 positions, as one
attn_decode_append call (one launch: the split pass, whose last workgroup
per unit merges the splits and appends). The timed region
holds exactly --steps such steps back to back, bracketed by
torch.cuda.synchronize(); inputs rotate over three independent cache sets
(3 x 256 MiB, larger than the 256 MB Infinity Cache) so every step reads its
K/V from HBM. value = algorithmic K+V bytes per step / step time.

roofline: the attn_decode_append call, timed with HIP events recorded around
each call on the stream it is launched on; achieved = algorithmic K+V bytes
(each attended K and V row read once) / mean event time. The call is one
kernel, whose rocprofv3 duration matches the event time.

cpu_baseline: the fp64 oracle on this host's cores over the same decode
workload (all 32 x 12 heads, repeated to >= 10 s).

modes: the other workloads, each timed the same way (median of per-call event
times): sliding-window decode (GB/s against 8 TB/s HBM), causal prefill
(TFLOP/s of 2*d*m*(m+1)*Hq against the 157.3 TFLOP/s fp32 matrix peak).

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix
METRIC = ("decode K/V HBM GB/s (% of 8 TB/s); "
          "causal prefill fp32 TFLOP/s (% MFMA peak)")
HEADLINE = "decode_b32_hq12_hkv2_d128_t4096"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    """Hash of the kernel sources; traffic counters are only reported while
    the kernels are the ones they were measured on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_gqa_online_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
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


def bench_headline(args, dev):
    import numpy as np
    import torch
    import attention_gqa_online_amd as A
    import synth

    w = synth.WORKLOADS[HEADLINE]
    stream = torch.cuda.current_stream()
    sets = []
    for r in range(3):
        q, k, v = synth.decode_inputs(w, seed=w.seed + r)
        ks, vs = synth.append_inputs(w.batch, w.kv_heads, w.head_dim, seed=w.seed + 10 + r)
        sets.append(tuple(torch.from_numpy(x).to(dev) for x in (q, k, v, ks, vs)))
        if r == 0:
            host_set0 = (q, k, v)
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
    cs = [torch.from_numpy(x).to(dev) for x in synth.rope_tables(w.head_dim, pos)]
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
    return w, value, ms_per_step, roof, host_set0, two, rope, graph


def cpu_baseline(w, host_set):
    import oracle
    q, k, v = host_set
    reps, t_total = 0, 0.0
    while t_total < 10.0 and reps < 1000:
        t0 = time.perf_counter()
        oracle.decode(q, k, v, w.batch, w.num_heads, w.kv_heads, w.head_dim, w.max_seq,
                      w.total_seq, w.window, w.scale)
        t_total += time.perf_counter() - t0
        reps += 1
    gbs = w.kv_bytes() * reps / t_total / 1e9
    log(f"[bench] cpu oracle: {reps} passes in {t_total:.1f} s, {gbs:.2f} GB/s")
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the whole decode workload ({w.batch} sequences x {w.num_heads} heads, "
                      f"4096 positions), fp64 two-pass softmax, {reps} passes, "
                      f"{t_total:.1f} s"}


def bench_decode_window(args, dev):
    import torch
    import attention_gqa_online_amd as A
    import synth
    w = synth.WORKLOADS["decode_b16_hq32_hkv8_d128_t32768_w4096"]
    sets = [synth.decode_inputs_device(w, w.seed + r, dev) for r in range(2)]
    out = torch.empty(w.batch, w.num_heads, w.head_dim, device=dev)
    ws = A.decode_workspace(w.batch, w.num_heads, w.kv_heads, w.head_dim, w.total_seq,
                            w.window, device=dev)
    stream = torch.cuda.current_stream()

    def call(i):
        q, k, v = sets[i % 2]
        A.attn_decode(q, k, v, out, w.batch, w.num_heads, w.kv_heads, w.head_dim,
                      w.max_seq, w.total_seq, w.window, w.scale, ws)
    ms, wall = time_calls(call, max(args.steps, 10), args.warmup, stream)
    med = statistics.median(ms)
    gbs = w.kv_bytes() / (med * 1e-3) / 1e9
    del sets
    torch.cuda.empty_cache()
    log(f"[bench] window decode: median {med * 1e3:.1f} us, {gbs:.0f} GB/s")
    return {"workload": w.name, "median_us": round(med * 1e3, 2),
            "min_us": round(min(ms) * 1e3, 2), "GB/s": round(gbs, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("attn_decode_window")},
            "algorithmic_bytes": w.kv_bytes()}


def bench_prefill(args, dev, name, device_inputs=True):
    import torch
    import attention_gqa_online_amd as A
    import synth
    w = synth.WORKLOADS[name]
    if device_inputs:
        q, k, v = synth.prefill_inputs_device(w, w.seed, dev)
    else:
        q, k, v = (torch.from_numpy(x).to(dev) for x in synth.prefill_inputs(w))
    o = torch.empty(w.m, w.q_stride, device=dev)
    stream = torch.cuda.current_stream()

    def call(i):
        A.attn_prefill_causal(q, k, v, o, w.m, w.q_stride, w.kv_stride, w.num_q_heads,
                              w.heads_per_kv, w.head_dim)
    n = max(args.steps, 10) if w.m <= 4096 else max(5, min(args.steps, 10))
    ms, wall = time_calls(call, n, args.warmup, stream)
    med = statistics.median(ms)
    tfl = w.flops() / (med * 1e-3) / 1e12
    del q, k, v, o
    torch.cuda.empty_cache()
    log(f"[bench] {name}: median {med * 1e3:.1f} us, {tfl:.2f} TFLOP/s")
    return {"workload": name, "median_us": round(med * 1e3, 2),
            "min_us": round(min(ms) * 1e3, 2), "TFLOP/s": round(tfl, 3),
            "roofline": {"bound": "mfma", "achieved": round(tfl, 3),
                         "peak": FP32_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tfl / FP32_MFMA_PEAK_TFLOPS, 4)},
            "algorithmic_flops": w.flops()}


def bench_decode_varlen(args, dev):
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
    sets = [synth.decode_inputs_device(w, w.seed + 20 + r, dev) for r in range(3)]
    kn, vn = (torch.from_numpy(x).to(dev)
              for x in synth.append_inputs(w.batch, w.kv_heads, w.head_dim, seed=w.seed + 30))
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
    ms, wall = time_calls(call, max(args.steps, 10), args.warmup, stream)
    med = statistics.median(ms)
    bytes_ = int(2 * w.kv_heads * w.head_dim * 4 * int(lens.astype(np.int64).sum()))
    gbs = bytes_ / (med * 1e-3) / 1e9

    # the same step with rotary embedding, one cos/sin table per sequence
    tabs = [synth.rope_tables(w.head_dim, int(p)) for p in lens - 1]
    cos_t = torch.from_numpy(np.ascontiguousarray(np.stack([t[0] for t in tabs]))).to(dev)
    sin_t = torch.from_numpy(np.ascontiguousarray(np.stack([t[1] for t in tabs]))).to(dev)

    def rope_call(i):
        q, k, v = sets[i % 3]
        A.attn_decode_rope_append_varlen(q, kn, vn, cos_t, sin_t, k, v, out, pos, w.batch,
                                         w.num_heads, w.kv_heads, w.head_dim, w.max_seq,
                                         w.total_seq, w.window, w.scale, ws)
    ms_r, _ = time_calls(rope_call, max(args.steps, 10), args.warmup, stream)
    med_r = statistics.median(ms_r)
    del sets
    torch.cuda.empty_cache()
    log(f"[bench] varlen decode step: median {med * 1e3:.1f} us, {gbs:.0f} GB/s "
        f"(mean length {lens.mean():.0f}); rotary varlen step: median {med_r * 1e3:.1f} us")
    return {"workload": "decode_varlen_b32_hq12_hkv2_d128_t4096_uniform",
            "step": "attn_decode_append_varlen", "mean_len": round(float(lens.mean()), 1),
            "median_us": round(med * 1e3, 2), "min_us": round(min(ms) * 1e3, 2),
            "GB/s": round(gbs, 1),
            "rope_step": {"step": "attn_decode_rope_append_varlen",
                          "median_us": round(med_r * 1e3, 2),
                          "GB/s": round(bytes_ / (med_r * 1e-3) / 1e9, 1)},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("attn_decode_append_varlen")},
            "algorithmic_bytes": bytes_}


def bench_append_rows(args, dev):
    """Prefill -> cache hand-over at the long prefill's shape: 16384 rows of
    8 KV heads x 128 into [8, 16384, 128] caches (K and V read once, written
    once)."""
    import torch
    import attention_gqa_online_amd as A
    m, hkv, d = 16384, 8, 128
    g = torch.Generator(device=dev).manual_seed(7)
    k = torch.randn((m, hkv * d), generator=g, device=dev)
    v = torch.randn((m, hkv * d), generator=g, device=dev)
    caches = [(torch.empty((hkv, m, d), device=dev), torch.empty((hkv, m, d), device=dev))
              for _ in range(2)]
    stream = torch.cuda.current_stream()

    def call(i):
        kc, vc = caches[i % 2]
        A.kv_append_rows(k, v, kc, vc, m, hkv * d, hkv, d, m, 0)
    ms, wall = time_calls(call, max(args.steps, 10), args.warmup, stream)
    med = statistics.median(ms)
    bytes_ = 4 * m * hkv * d * 4
    gbs = bytes_ / (med * 1e-3) / 1e9
    del k, v, caches
    torch.cuda.empty_cache()
    log(f"[bench] kv_append_rows: median {med * 1e3:.1f} us, {gbs:.0f} GB/s")
    return {"workload": "append_rows_m16384_hkv8_d128", "median_us": round(med * 1e3, 2),
            "min_us": round(min(ms) * 1e3, 2), "GB/s": round(gbs, 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("kv_append_rows")},
            "algorithmic_bytes": bytes_}


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
    ap.add_argument("--modes", default="headline,decode_window,decode_varlen,append_rows,"
                                       "prefill_long,prefill_qwen,prefill_tiny",
                    help="comma list; the headline decode step always runs "
                         "(also: copy_calibration)")
    args = ap.parse_args()
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

    w, value, ms_per_step, roof, host_set, two, rope, graph = bench_headline(args, dev)
    extra = {"decode_step_two_calls": two, "decode_step_graph": graph, "decode_step_rope": rope}
    if "decode_window" in modes:
        extra["decode_window"] = bench_decode_window(args, dev)
    if "decode_varlen" in modes:
        extra["decode_varlen"] = bench_decode_varlen(args, dev)
    if "append_rows" in modes:
        extra["append_rows"] = bench_append_rows(args, dev)
    if "prefill_long" in modes:
        extra["prefill_long"] = bench_prefill(args, dev, "prefill_hq64_hkv8_d128_m16384")
    if "prefill_qwen" in modes:
        extra["prefill_qwen"] = bench_prefill(args, dev, "prefill_hq28_hkv4_d128_m2048")
    if "prefill_tiny" in modes:
        extra["prefill_tiny"] = bench_prefill(args, dev, "prefill_hq4_hkv2_d32_m16",
                                              device_inputs=False)
    if "copy_calibration" in modes:
        extra["copy_calibration"] = copy_calibration(dev)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, host_set)

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
        "device": {"name": props.name, "cus": props.multi_processor_count},
        "kernel_sources": source_digest(),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
