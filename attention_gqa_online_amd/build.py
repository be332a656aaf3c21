"""Build libattn.so (the HIP kernels and the C ABI of include/attn.h) for gfx950.

    python -m attention_gqa_online_amd.build

Ahead of time, no JIT: each source compiles to an object in parallel, then one
link. Packed fp32 instructions are switched off for all device code
(-packed-fp32-ops); the host pass warns that it does not know the feature,
which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SO_PATH = os.path.join(PKG, "libattn.so")
SOURCES = ["api.hip", "plan.cpp", "decode.hip", "prefill.hip", "kv_append.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops"]
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _includes() -> list[str]:
    return ["-I", os.path.join(ROOT, "include"), "-I", CSRC]


def command(out: str = SO_PATH, extra=()) -> list[str]:
    """One hipcc line that compiles and links everything (single-process)."""
    return [hipcc(), f"--offload-arch={ARCH}", *FLAGS, "-shared", *_includes(), *extra,
            "-o", out, *[os.path.join(CSRC, s) for s in SOURCES]]


def _run(cmd: list[str]) -> str:
    proc = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in proc.stderr.splitlines() if NOISE not in ln)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(out: str = SO_PATH, extra=()) -> str:
    with tempfile.TemporaryDirectory() as tmpdir:
        objs = [os.path.join(tmpdir, s + ".o") for s in SOURCES]
        cmds = [[hipcc(), f"--offload-arch={ARCH}", *FLAGS, *_includes(), *extra, "-c",
                 "-o", o, os.path.join(CSRC, s)] for s, o in zip(SOURCES, objs)]
        workers = max(1, min(len(cmds), os.cpu_count() or 1))
        with ThreadPoolExecutor(workers) as pool:
            errs = list(pool.map(_run, cmds))
        tmp = out + ".tmp"
        errs.append(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs]))
    err = "\n".join(e for e in errs if e.strip())
    if err.strip():
        sys.stderr.write(err + "\n")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
