"""Child process of tests/test_gpu_cus_limit.py: with ATTN_GQA_CUS set in its
environment the library plans every call for that many compute units (fewer
decode splits, other varlen tables, other prefill grids). Each call below is
checked against the fp64 oracle at max|err| <= 2e-5 max|V|; prints one line
per case and "all ok" at the end, exits non-zero on a mismatch."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import attention_gqa_online_amd as A  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402

TOL = 2e-5
dev = torch.device("cuda:0")
bad = 0


def check(name, got, ref, vmax):
    global bad
    err = float(np.abs(got.astype(np.float64) - ref).max())
    ok = err <= TOL * vmax
    bad += not ok
    print(f"{name}: max|err| {err:.3e} bound {TOL * vmax:.3e} {'ok' if ok else 'FAIL'}", flush=True)


def T(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev)


print("ATTN_GQA_CUS =", os.environ.get("ATTN_GQA_CUS"), flush=True)

# decode step of the batched workload (32 sequences, 12 Q / 2 KV heads)
w = synth.WORKLOADS["decode_b32_hq12_hkv2_d128_t4096"]
q, k, v = synth.decode_inputs(w, seed=501)
kn, vn = synth.append_inputs(w.batch, w.kv_heads, w.head_dim, seed=502)
pos = w.total_seq - 1
kd, vd = T(k), T(v)
out = torch.empty(w.batch, w.num_heads, w.head_dim, device=dev)
ws = A.decode_workspace(w.batch, w.num_heads, w.kv_heads, w.head_dim, w.total_seq, 0, device=dev)
A.attn_decode_append(T(q), T(kn), T(vn), kd, vd, out, w.batch, w.num_heads, w.kv_heads,
                     w.head_dim, w.max_seq, pos, 0, w.scale, ws)
oracle.kv_append(kn, vn, k, v, w.batch, w.kv_heads, w.head_dim, w.max_seq, pos)
ref = oracle.decode(q, k, v, w.batch, w.num_heads, w.kv_heads, w.head_dim, w.max_seq,
                    w.total_seq, 0, w.scale)
torch.cuda.synchronize()
check("attn_decode_append b32 hq12 hkv2 T4096", out.cpu().numpy(), ref, float(np.abs(v).max()))
A.attn_decode(T(q), kd, vd, out, w.batch, w.num_heads, w.kv_heads, w.head_dim, w.max_seq,
              w.total_seq, 0, w.scale, ws)
torch.cuda.synchronize()
check("attn_decode b32 hq12 hkv2 T4096", out.cpu().numpy(), ref, float(np.abs(v).max()))

# windowed decode, fewer sequences than the workload
ww = synth.DecodeWorkload("win", batch=4, num_heads=32, kv_heads=8, head_dim=128, max_seq=9000,
                          total_seq=9000, window=4096, sigma=0.5, seed=503)
q, k, v = synth.decode_inputs(ww)
out = torch.empty(4, 32, 128, device=dev)
ws = A.decode_workspace(4, 32, 8, 128, 9000, 4096, device=dev)
A.attn_decode(T(q), T(k), T(v), out, 4, 32, 8, 128, 9000, 9000, 4096, ww.scale, ws)
ref = oracle.decode(q, k, v, 4, 32, 8, 128, 9000, 9000, 4096, ww.scale)
torch.cuda.synchronize()
check("attn_decode b4 hq32 hkv8 T9000 window 4096", out.cpu().numpy(), ref,
      float(np.abs(v[:, :, 9000 - 4096:]).max()))

# varlen decode step (per-sequence positions)
lens = synth.seq_lengths(w.batch, w.total_seq, seed=504)
q, k, v = synth.decode_inputs(w, seed=505)
kn, vn = synth.append_inputs(w.batch, w.kv_heads, w.head_dim, seed=506)
posv = lens.astype(np.int64) - 1
out = torch.empty(w.batch, w.num_heads, w.head_dim, device=dev)
ws = A.decode_workspace(w.batch, w.num_heads, w.kv_heads, w.head_dim, w.total_seq, 0, device=dev)
A.attn_decode_append_varlen(T(q), T(kn), T(vn), T(k), T(v), out, T(posv.astype(np.int32)),
                            w.batch, w.num_heads, w.kv_heads, w.head_dim, w.max_seq,
                            w.total_seq, 0, w.scale, ws)
for b in range(w.batch):
    oracle.kv_append(kn[b:b + 1], vn[b:b + 1], k[b:b + 1], v[b:b + 1], 1, w.kv_heads,
                     w.head_dim, w.max_seq, int(posv[b]))
ref = oracle.decode_varlen(q, k, v, posv + 1, w.batch, w.num_heads, w.kv_heads, w.head_dim,
                           w.max_seq, 0, w.scale)
torch.cuda.synchronize()
vmax = max(float(np.abs(v[b, :, :int(posv[b]) + 1]).max()) for b in range(w.batch))
check("attn_decode_append_varlen b32 hq12 hkv2 (mixed positions)", out.cpu().numpy(), ref, vmax)


# prefills: the Qwen-shaped layer and a head_dim 256 grid under two per CU
def prefill(name, pw):
    qh, kh, vh = synth.prefill_inputs(pw)
    o = torch.zeros(pw.m, pw.q_stride, device=dev)
    A.attn_prefill_causal(T(qh), T(kh), T(vh), o, pw.m, pw.q_stride, pw.kv_stride,
                          pw.num_q_heads, pw.heads_per_kv, pw.head_dim)
    ref = oracle.prefill_causal(qh, kh, vh, pw.m, pw.q_stride, pw.kv_stride, pw.num_q_heads,
                                pw.heads_per_kv, pw.head_dim)
    torch.cuda.synchronize()
    got = o.cpu().numpy()[:, : pw.num_q_heads * pw.head_dim].reshape(ref.shape)
    check(name, got, ref, float(np.abs(vh[:, : pw.kv_heads * pw.head_dim]).max()))


prefill("attn_prefill_causal m2048 hq28 hkv4 d128", synth.WORKLOADS["prefill_hq28_hkv4_d128_m2048"])
prefill("attn_prefill_causal m1024 hq16 hkv8 d256",
        synth.PrefillWorkload("p256", m=1024, num_q_heads=16, heads_per_kv=2, head_dim=256,
                              q_stride=16 * 256, kv_stride=8 * 256, seed=507))
print("all ok" if bad == 0 else f"{bad} FAILED", flush=True)
sys.exit(1 if bad else 0)
