"""Build libattn.so (the HIP kernels and the C ABI of include/attn.h) for gfx950.

    python -m attention_gqa_online_amd.build

One hipcc invocation, ahead of time; no JIT. Packed fp32 instructions are
switched off for all device code (-packed-fp32-ops); the host pass warns that
it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SO_PATH = os.path.join(PKG, "libattn.so")
SOURCES = ["api.hip", "decode.hip", "prefill.hip", "kv_append.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def command(out: str = SO_PATH, extra=()) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *extra, "-o", out, *[os.path.join(CSRC, s) for s in SOURCES],
    ]


def build(out: str = SO_PATH, extra=()) -> str:
    tmp = out + ".tmp"
    proc = subprocess.run(command(tmp, extra), capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; drop that line only
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(ln for ln in proc.stderr.splitlines() if noise not in ln)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
