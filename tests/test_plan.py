"""Launch plans on the CPU: the decode split and the prefill grid follow the
device's compute-unit count (a whole MI355X has 256; a partitioned one, or
another gfx950 part, fewer), and the decode workspace sized for 256 covers
every smaller count.

The plans are plain host arithmetic (csrc/plan.cpp); tests/plan_probe.cpp
wraps them in C and is built here with the host compiler.
"""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_gqa_online_amd", "csrc")
U64P = ctypes.POINTER(ctypes.c_uint64)
DEC = ("head_chunk", "n_chunks", "units", "n_split", "rows_per_split", "w0", "g_target",
       "part_floats", "part_offset", "workspace_bytes")
PRE = ("waves", "n_rb", "n_pairs", "zigzag", "nsub", "wg_per_group", "grid", "rows16", "n_rb16",
       "n_tasks16", "small")


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    so = str(tmp_path_factory.mktemp("plan") / "libplanprobe.so")
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-Wall", "-Werror",
                           "-I", CSRC, "-o", so, os.path.join(ROOT, "tests", "plan_probe.cpp"),
                           os.path.join(CSRC, "plan.cpp")])
    lib = ctypes.CDLL(so)
    lib.probe_plan_decode.argtypes = [ctypes.c_uint32] * 6 + [ctypes.c_int] * 2 + [
        ctypes.c_uint32, U64P]
    lib.probe_plan_prefill.argtypes = [ctypes.c_uint32] * 5 + [U64P]
    lib.probe_max_cus.restype = ctypes.c_uint32
    return lib


def decode_plan(lib, b, hq, hkv, d, t, w, append=False, varlen=False, cus=256):
    out = (ctypes.c_uint64 * 10)()
    lib.probe_plan_decode(b, hq, hkv, d, t, w, int(append), int(varlen), cus, out)
    return dict(zip(DEC, out))


def prefill_plan(lib, m, hq, hpk, d, cus=256):
    out = (ctypes.c_uint64 * 11)()
    lib.probe_plan_prefill(m, hq, hpk, d, cus, out)
    return dict(zip(PRE, out))


def test_max_cus_is_a_whole_mi355x(probe):
    assert probe.probe_max_cus() == 256


@pytest.mark.parametrize("cus,n_split,rows", [(256, 4, 1024), (128, 2, 2048), (64, 1, 4096),
                                              (32, 1, 4096)])
def test_decode_split_follows_compute_units(probe, cus, n_split, rows):
    """The decode step of 32 sequences x 2 KV heads (64 units of 6 Q heads)
    over 4095 cached rows: one workgroup per compute unit while the units
    fall short of them, one per unit once they do not."""
    p = decode_plan(probe, 32, 12, 2, 128, 4096, 0, append=True, cus=cus)
    assert (p["units"], p["head_chunk"]) == (64, 6)
    assert (p["n_split"], p["rows_per_split"]) == (n_split, rows)
    assert p["units"] * p["n_split"] == max(cus, 64)


def test_windowed_decode_split(probe):
    """16 sequences x 8 KV heads (128 units), window of 4096 rows of 32768."""
    p256 = decode_plan(probe, 16, 32, 8, 128, 32768, 4096, cus=256)
    assert (p256["units"], p256["n_split"], p256["w0"]) == (128, 2, 28672)
    p128 = decode_plan(probe, 16, 32, 8, 128, 32768, 4096, cus=128)
    assert (p128["n_split"], p128["rows_per_split"]) == (1, 4096)


@pytest.mark.parametrize("cus,target", [(256, 224), (128, 96), (96, 64), (32, 64)])
def test_varlen_target_follows_compute_units(probe, cus, target):
    """Per-sequence lengths: the proportional table aims at one workgroup
    per compute unit less half a split per unit (the rounding up), never
    below 64."""
    p = decode_plan(probe, 32, 12, 2, 128, 4096, 0, append=True, varlen=True, cus=cus)
    assert p["g_target"] == target
    # the workspace holds every proportional split and one more per unit
    assert p["part_floats"] == (target + 64) * 6 * (128 + 4)


def test_counts_outside_the_range_are_clamped(probe):
    for lo in (0, 1):
        assert decode_plan(probe, 32, 12, 2, 128, 4096, 0, cus=lo)["n_split"] == 1
    assert decode_plan(probe, 32, 12, 2, 128, 4096, 0, cus=4096) == \
        decode_plan(probe, 32, 12, 2, 128, 4096, 0, cus=256)


SHAPES = [(1, 1, 1, 32, 1, 0), (1, 8, 1, 64, 100, 0), (32, 12, 2, 128, 4096, 0),
          (16, 32, 8, 128, 32768, 4096), (3, 6, 2, 96, 1000, 129), (2, 56, 8, 160, 5000, 0),
          (5, 12, 2, 224, 777, 0), (1, 64, 8, 256, 65536, 0), (128, 8, 8, 128, 300, 0),
          (4096, 4, 4, 64, 64, 0)]


@pytest.mark.parametrize("shape", SHAPES)
def test_workspace_for_256_covers_every_smaller_count(probe, shape):
    """The C ABI checks a call against the plan for 256 compute units and
    launches the plan for the device's count: that plan must never need more
    workspace or more split slots."""
    for append in (False, True):
        for varlen in (False, True):
            full = decode_plan(probe, *shape, append=append, varlen=varlen, cus=256)
            for cus in (1, 2, 7, 32, 33, 64, 100, 128, 160, 200, 255):
                p = decode_plan(probe, *shape, append=append, varlen=varlen, cus=cus)
                assert p["workspace_bytes"] <= full["workspace_bytes"], (shape, cus)
                assert p["units"] * p["n_split"] <= full["units"] * full["n_split"]
                assert p["g_target"] <= full["g_target"]
                # every attended row of the split pass is covered
                t, w = shape[4], shape[5]
                w0 = t - w if (w and t > w) else 0
                rows = t - w0 - (1 if append else 0)
                assert p["n_split"] * p["rows_per_split"] >= rows
                if p["n_split"]:
                    assert (p["n_split"] - 1) * p["rows_per_split"] < rows


def test_prefill_grid_follows_compute_units(probe):
    # Qwen-2.5-7B-shaped layer (28 Q / 4 KV heads, m 2048): under two
    # workgroups per compute unit, so short and long row blocks pair up
    p = prefill_plan(probe, 2048, 28, 7, 128, cus=256)
    assert (p["zigzag"], p["rows16"], p["nsub"], p["grid"], p["waves"]) == (1, 0, 2, 256, 8)
    # head_dim 256 on such a grid: 16-row blocks, a pair per wave (64 pairs x
    # 2 heads = 128 equal tasks per KV head, 8 per workgroup)
    p = prefill_plan(probe, 2048, 16, 2, 256, cus=256)
    assert (p["zigzag"], p["rows16"], p["waves"]) == (1, 1, 8)
    assert (p["n_rb16"], p["n_tasks16"], p["grid"]) == (128, 128, 128)
    # head_dim 224 (not a multiple of 64) keeps the 32-row zigzag kernel
    assert prefill_plan(probe, 2048, 16, 2, 224, cus=256)["rows16"] == 0
    # an odd number of 16-row blocks: the middle one pairs with itself
    p = prefill_plan(probe, 40, 4, 2, 192, cus=256)
    assert (p["rows16"], p["n_rb16"], p["n_tasks16"], p["grid"]) == (1, 3, 4, 2)
    # a quarter of the compute units: 224 row-block-major workgroups fill
    # them more than twice over
    p = prefill_plan(probe, 2048, 28, 7, 128, cus=64)
    assert (p["zigzag"], p["grid"]) == (0, 224)
    # m 16384, 64 Q / 8 KV heads: always row-block major
    p = prefill_plan(probe, 16384, 64, 8, 128, cus=256)
    assert (p["zigzag"], p["grid"], p["waves"]) == (0, 4096, 8)
    # head_dim 256 takes 4-wave workgroups only on grids that fill the chip twice
    assert prefill_plan(probe, 8192, 32, 4, 256, cus=256)["waves"] == 4
    assert prefill_plan(probe, 1024, 32, 8, 256, cus=256)["waves"] == 8
    assert prefill_plan(probe, 1024, 32, 8, 256, cus=32)["waves"] == 4


@pytest.mark.parametrize("m,hq,small,grid", [(1, 4, 1, 1), (16, 4, 1, 1), (16, 28, 1, 7), (5, 9, 1, 3),
                                             (17, 4, 0, None)])
def test_small_prompts_take_one_wave_per_head(probe, m, hq, small, grid):
    """Up to 16 rows: the small kernel, one wave per Q head in 4-wave
    workgroups, whatever the compute-unit count; 17 rows and up: the tiled
    kernel."""
    for cus in (256, 32):
        p = prefill_plan(probe, m, hq, 1, 128, cus=cus)
        assert p["small"] == small
        if small:
            assert (p["grid"], p["waves"]) == (grid, 4)
