"""The C ABI driven from plain C on the GPU: a C99 program
(tests/c_abi/attn_device_run.c) that allocates device memory with the HIP
runtime API, plans with pg_pack and runs pg_attn_fwd / pg_attn_bwd gives
bitwise the outputs of the Python binding on the same inputs (same kernels;
both are checked against the oracle elsewhere)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from tests.parity import run_gpu
from workloads import bf16_bits, draw_attention_inputs, scaled_down

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "shared_prefix_grouped_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_client_matches_binding_bitwise(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import shared_prefix_grouped_amd as pg
    pg.lib()  # fails loudly if the library is not built
    exe = str(tmp_path / "attn_device_run")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi", "attn_device_run.c"),
                    "-L", LIBDIR, "-lpg_attn", "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath," + LIBDIR, "-o", exe], check=True)
    P, rs, hq, hkv, d = 200, [37, 130, 1, 64], 4, 2, 128
    w = scaled_down("c_client", [(P, rs)], "bf16", hq, hkv, d, seed=31)
    arrs = draw_attention_inputs(w)
    inp, out = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    np.concatenate([bf16_bits(arrs[n]).ravel() for n in ("q", "k", "v", "do")]).tofile(inp)
    print(f"[c-client] one group P={P} responses={rs} heads={hq}/{hkv} d={d}", flush=True)
    res = subprocess.run([exe, inp, out, str(hq), str(hkv), str(d), str(P)] + [str(r) for r in rs],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    T = P + sum(rs)
    nq, nk = T * hq * d, T * hkv * d
    raw = np.fromfile(out, dtype=np.uint8)
    bits = raw[:2 * (2 * nq + 2 * nk)].view(np.uint16)
    lse = raw[2 * (2 * nq + 2 * nk):].view(np.float32)
    c = {"o": bits[:nq], "dq": bits[nq:2 * nq], "dk": bits[2 * nq:2 * nq + nk],
         "dv": bits[2 * nq + nk:], "lse": lse}
    ref = run_gpu([(P, rs)], hq, hkv, d, arrs, torch.bfloat16)
    for key in ("o", "dq", "dk", "dv"):
        got = ref[key].contiguous().view(torch.int16).cpu().numpy().view(np.uint16).ravel()
        assert np.array_equal(got, c[key]), key
    assert np.array_equal(ref["lse"].cpu().numpy().ravel(), c["lse"])
