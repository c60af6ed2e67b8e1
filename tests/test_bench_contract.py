"""bench.py's output contract: one JSON line with the metric, the roofline of the
dominant kernel and each kernel's rate; one GPU only."""
import contextlib
import io
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    err = io.StringIO()
    with contextlib.redirect_stderr(err):
        assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in err.getvalue()


def test_kernel_flop_accounting():
    """Executed MFMA work per visible (query, key) pair, query head and unit of
    d: forward 4 (S, O), dK/dV 8 (S, dP, dV, dK), dQ 6 (S, dP, dQ) -- 18 in
    all, of which the step is credited 14 (forward 4, backward 10: the S and dP
    recomputed by the second backward kernel are not credited)."""
    assert bench.KERNEL_FLOPS_PER_PAIR_D == {"fwd": 4, "bwd_dkdv": 8, "bwd_dq": 6}
    assert sum(bench.KERNEL_FLOPS_PER_PAIR_D.values()) == 18


@pytest.mark.gpu
def test_bench_line_has_the_contract_fields():
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        assert bench.main(["--steps", "2", "--warmup", "1", "--no-baseline", "--no-cpu"]) == 0
    lines = [ln for ln in out.getvalue().splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    res = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "kernel_rooflines", "cpu_baseline"):
        assert key in res, key
    assert res["n_gpus"] == 1 and res["steps"] == 2 and res["warmup"] == 1
    assert res["unit"] == "TFLOP/s" and res["higher_is_better"] is True
    assert res["config"]["workload"] == "bf16_gqa_g16_p8192"
    assert res["value"] > 0 and res["ms_per_step"] > 0
    roof = res["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    assert roof["peak"] == bench.PEAK_BF16_TFLOPS
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    assert set(res["kernel_rooflines"]) >= {"fwd", "bwd_dkdv", "bwd_dq"}  # bf16: no separate preprocess
    # the kernels run one after another on one stream, inside the step
    total = sum(k["avg_launch_ms"] for k in res["kernel_rooflines"].values())
    assert total <= res["ms_per_step"] * 1.02
