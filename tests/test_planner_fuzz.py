"""The host planner on seeded random batches, from C++ (no GPU).

`tests/c_abi/plan_fuzz.cpp` plans random batches with `pg_pack_host` and checks
every descriptor against what the batch alone fixes (packed offsets, baseline
position ids, the visibility rule and pair counts by brute force, tile and
work-list coverage, the scored entries), and that invalid batches are refused
with a message.  It runs once against the built library and once with the
planner's source rebuilt under AddressSanitizer (host code only; the kernels'
objects are linked unchanged), so an out-of-bounds access or a leak in the
planner fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "shared_prefix_grouped_amd")
LIB = os.path.join(PKG, "libpg_attn.so")
SRC = os.path.join(ROOT, "tests", "c_abi", "plan_fuzz.cpp")
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
KERNEL_OBJS = ["pg_fwd_bf16.o", "pg_bwd_bf16.o", "pg_f32.o", "pg_rows.o", "pg_head.o",
               "pg_head_mfma.o"]


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res.stdout


def test_planner_random_batches(tmp_path):
    if not os.path.exists(LIB):
        pytest.skip("libpg_attn.so is not built")
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "plan_fuzz")
    _run([gxx, "-O1", "-std=c++17", "-Wall", "-I", INCLUDE, SRC, "-o", exe, "-L", PKG, "-lpg_attn",
          f"-Wl,-rpath,{PKG}"])
    out = _run([exe, "3000"]).split()
    assert out[0] == "ok" and int(out[1]) > 2500 and int(out[2]) > 50, out


def test_planner_random_batches_asan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clangxx = "/opt/rocm/llvm/bin/clang++"
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)):
        pytest.skip("ROCm toolchain not found")
    objs = [os.path.join(BUILD, o) for o in KERNEL_OBJS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects are not built")
    api = str(tmp_path / "pg_api_asan.o")
    drv = str(tmp_path / "plan_fuzz.o")
    exe = str(tmp_path / "plan_fuzz_asan")
    # the sanitizer applies to host code only (-Xarch_host)
    _run([hipcc, "-x", "hip", "-c", os.path.join(CSRC, "pg_api.cpp"), "-o", api, "-O1", "-g",
          "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"])
    _run([clangxx, "-c", SRC, "-o", drv, "-O1", "-g", "-std=c++17", "-I", INCLUDE,
          "-fsanitize=address", "-fno-omit-frame-pointer"])
    _run([hipcc, "-Xarch_host", "-fsanitize=address", "-o", exe, drv, api] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    out = _run([exe, "1500"], env=env).split()
    assert out[0] == "ok" and int(out[1]) > 1200, out
