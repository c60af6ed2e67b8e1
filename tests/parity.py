"""Helpers for GPU-vs-oracle parity tests.

Tolerances (fixed per element type):
  float32: max |gpu - oracle| <= 1e-4 on O, LSE, dQ, dK, dV.
  bfloat16 (fp32 accumulation): O max-abs <= 2e-2; LSE max-abs <= 1e-3;
  every gradient tensor ||g - g*||_F / ||g*||_F <= 1e-2, also per segment
  (prefix rows, response rows) so large prefix norms cannot hide response errors.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F32_ATOL = 1e-4
BF16_O_ATOL = 2e-2
BF16_LSE_ATOL = 1e-3
BF16_GRAD_RTOL = 1e-2


def to_dev(a, dtype, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device).to(dtype)


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run_gpu(groups, hq, hkv, d, arrs, dtype, scale=None, with_bwd=True):
    import torch
    import shared_prefix_grouped_amd as pg
    batch = pg.pg_pack(groups, hq, hkv, d, "cuda")
    q, k, v = (to_dev(arrs[n], dtype) for n in ("q", "k", "v"))
    o, lse = pg.pg_attn_fwd(batch, q, k, v, scale)
    out = {"o": o, "lse": lse, "batch": batch}
    if with_bwd:
        do = to_dev(arrs["do"], dtype)
        dq, dk, dv = pg.pg_attn_bwd(batch, q, k, v, o, lse, do, scale)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return out


def segment_rows(groups):
    """Boolean mask of prefix rows in the packed layout."""
    T = sum(p + sum(rs) for p, rs in groups)
    pre = np.zeros(T, dtype=bool)
    t = 0
    for p, rs in groups:
        pre[t:t + p] = True
        t += p + sum(rs)
    return pre


def rel_fro(a, b):
    den = np.linalg.norm(b)
    num = np.linalg.norm(a - b)
    if den == 0:
        return num
    return num / den


def compare(gpu, ref, dtype_name, prefix_mask=None, grads=True, report=None):
    """Assert gpu (numpy float64) matches ref (oracle) at the stated tolerances."""
    msgs = []
    if dtype_name == "f32":
        for key in ("o", "lse") + (("dq", "dk", "dv") if grads else ()):
            err = float(np.max(np.abs(gpu[key] - ref[key]))) if ref[key].size else 0.0
            msgs.append(f"{key} max-abs {err:.3e}")
            assert err <= F32_ATOL, f"{key}: max-abs {err} > {F32_ATOL}"
    else:
        err = float(np.max(np.abs(gpu["o"] - ref["o"]))) if ref["o"].size else 0.0
        msgs.append(f"o max-abs {err:.3e}")
        assert err <= BF16_O_ATOL, f"o: max-abs {err} > {BF16_O_ATOL}"
        err = float(np.max(np.abs(gpu["lse"] - ref["lse"]))) if ref["lse"].size else 0.0
        msgs.append(f"lse max-abs {err:.3e}")
        assert err <= BF16_LSE_ATOL, f"lse: max-abs {err} > {BF16_LSE_ATOL}"
        if grads:
            for key in ("dq", "dk", "dv"):
                e = rel_fro(gpu[key], ref[key])
                msgs.append(f"{key} rel-fro {e:.3e}")
                assert e <= BF16_GRAD_RTOL, f"{key}: rel-fro {e} > {BF16_GRAD_RTOL}"
                if prefix_mask is not None:
                    for name, m in (("prefix", prefix_mask), ("response", ~prefix_mask)):
                        if m.any() and np.linalg.norm(ref[key][m]) > 0:
                            e = rel_fro(gpu[key][m], ref[key][m])
                            msgs.append(f"{key}[{name}] rel-fro {e:.3e}")
                            assert e <= BF16_GRAD_RTOL, f"{key}[{name}]: rel-fro {e}"
    if report is not None:
        report.extend(msgs)
    return msgs


def host_threads() -> int:
    """CPU threads this process may use (its affinity mask), at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def pool_sum(fn, tasks, blas_threads=1):
    """Sum of the dicts fn(task) returns (numpy arrays added, other values
    taken from the first), computed in a thread pool: numpy releases the GIL
    inside its ufuncs and BLAS calls, so independent oracle evaluations (one
    member sequence, one kv head) run side by side."""
    from threadpoolctl import threadpool_limits
    tasks = list(tasks)
    with threadpool_limits(blas_threads):
        with ThreadPoolExecutor(max_workers=min(host_threads(), len(tasks))) as ex:
            parts = list(ex.map(fn, tasks))
    out = dict(parts[0])
    for part in parts[1:]:
        for key, val in part.items():
            if isinstance(val, np.ndarray) and val.dtype.kind == "f":
                out[key] = out[key] + val
    return out
