"""GPU parity of the packed grouped decoder against the fp64 repeated-prefix decoder oracle.

Element by element (outputs, input gradient and every parameter gradient) on a
scaled-down decoder of the same structure, and at the full 4-layer, d_model
2048 size: the oracle runs all 16 member sequences [P; R_i] with the
upstream gradient, in four parts of four members (each part checks its
members' outputs and response-row input gradients, which belong to one
member each, and keeps its partial parameter gradients); the last test adds
the parts and compares every parameter gradient and the whole input gradient
(prefix rows: the sum over the 16 copies, Pith review "Core claim",
Lemma 2.1).  The same harness on the repeated-prefix layout must also give the
grouped results.
"""
import time

import numpy as np
import pytest

from oracle.attention import member_sequences
from oracle.decoder import PARAM_NAMES, repeated_prefix_decoder
from workloads import Group, DecoderWorkload, decoder_workload, draw_decoder_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _groups(w):
    return [(g.prefix_len, list(g.resp_lens)) for g in w.groups]


def _oracle_params(arrs, w):
    p = {n: [arrs[f"{n}{l}"].astype(np.float64) for l in range(w.num_layers)]
         for n in ("wq", "wk", "wv", "wo", "w1", "w3", "w2")}
    p["g_attn"] = [np.ones(w.d_model) for _ in range(w.num_layers)]
    p["g_mlp"] = [np.ones(w.d_model) for _ in range(w.num_layers)]
    p["g_final"] = np.ones(w.d_model)
    return p


def _run_gpu(w, arrs, backward=True, groups=None):
    import shared_prefix_grouped_amd as pg
    from shared_prefix_grouped_amd.decoder import (DecoderConfig, decoder_forward,
                                                   make_parameters)
    cfg = DecoderConfig(w.num_layers, w.d_model, w.num_heads, w.ffn_dim, w.rope_theta, w.rms_eps)
    batch = pg.pg_pack(groups or _groups(w), w.num_heads, w.num_heads, w.head_dim)
    p = make_parameters(arrs, cfg)
    x = torch.from_numpy(arrs["x"]).cuda().requires_grad_(backward)
    y = decoder_forward(x, p, batch, cfg)
    if backward:
        y.backward(torch.from_numpy(arrs["dy"]).cuda())
    torch.cuda.synchronize()
    return y, x, p


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_small_decoder_elementwise():
    w = DecoderWorkload("decoder_small", (Group(200, (40, 0, 63, 17)), Group(0, (30, 5))),
                        num_layers=2, d_model=256, num_heads=2, head_dim=128, ffn_dim=512, seed=7)
    arrs = draw_decoder_inputs(w)
    y, x, p = _run_gpu(w, arrs)
    ref = repeated_prefix_decoder(_groups(w), arrs["x"], _oracle_params(arrs, w), arrs["dy"],
                                  num_heads=w.num_heads, theta=w.rope_theta, eps=w.rms_eps)
    e_y = float(np.max(np.abs(y.detach().cpu().numpy() - ref["y"])))
    e_x = _rel(x.grad.cpu().numpy(), ref["x"])
    msgs = [f"y max-abs {e_y:.2e}", f"dX rel-fro {e_x:.2e}"]
    assert e_y <= 2e-2 and e_x <= 1e-2
    for n in PARAM_NAMES:
        for l in range(w.num_layers):
            e = _rel(p[n][l].grad.cpu().numpy(), ref["grads"][n][l])
            msgs.append(f"{n}{l} {e:.1e}")
            assert e <= 1e-2, (n, l, e)
    e = _rel(p["g_final"].grad.cpu().numpy(), ref["grads"]["g_final"])
    assert e <= 1e-2
    print("[decoder small] " + "; ".join(msgs), flush=True)


@pytest.fixture(scope="module")
def full_run():
    """The full-size decoder workload, forward and backward on the GPU."""
    w = decoder_workload()
    t0 = time.time()
    arrs = draw_decoder_inputs(w)
    print(f"[decoder full] inputs drawn in {time.time() - t0:.1f}s, T={w.total_rows}", flush=True)
    y, x, p = _run_gpu(w, arrs, backward=True)
    grads = {n: [p[n][l].grad.cpu().numpy().astype(np.float64) for l in range(w.num_layers)]
             for n in PARAM_NAMES}
    grads["g_final"] = p["g_final"].grad.cpu().numpy().astype(np.float64)
    return {"w": w, "arrs": arrs, "y": y.detach().cpu().numpy().astype(np.float64),
            "dx": x.grad.cpu().numpy().astype(np.float64), "grads": grads, "parts": {}}


N_PARTS = 4


@pytest.mark.parametrize("part", range(N_PARTS))
def test_full_decoder_members(full_run, part):
    """Members 4 part .. 4 part + 3: their output rows and their response
    rows' input gradients against the oracle; partial parameter gradients kept."""
    w, arrs = full_run["w"], full_run["arrs"]
    groups = _groups(w)
    members, _ = member_sequences(groups)
    per = len(members) // N_PARTS
    mine = list(range(part * per, (part + 1) * per))
    t0 = time.time()
    ref = repeated_prefix_decoder(groups, arrs["x"], _oracle_params(arrs, w), arrs["dy"],
                                  num_heads=w.num_heads, theta=w.rope_theta, eps=w.rms_eps,
                                  members_only=mine)
    full_run["parts"][part] = ref
    rows = ~np.isnan(ref["y"][:, 0])
    e_y = float(np.max(np.abs(full_run["y"][rows] - ref["y"][rows])))
    resp = np.concatenate([np.arange(*members[i].resp) for i in mine])
    e_x = _rel(full_run["dx"][resp], ref["x"][resp])
    print(f"[decoder full] members {mine}: oracle {time.time() - t0:.1f}s, {int(rows.sum())} rows "
          f"y max-abs {e_y:.2e}, response-row dX rel-fro {e_x:.2e}", flush=True)
    assert e_y <= 2e-2 and e_x <= 1e-2


def test_full_decoder_param_and_input_grads(full_run):
    """Every parameter gradient and the whole input gradient (prefix rows and
    response rows separately too) against the sum of the oracle's parts."""
    parts = full_run["parts"]
    if len(parts) != N_PARTS:
        pytest.fail("the member parts did not all run")
    w = full_run["w"]
    dx = sum(parts[i]["x"] for i in range(N_PARTS))
    pre = np.zeros(w.total_rows, dtype=bool)
    t = 0
    for P, rs in _groups(w):
        pre[t:t + P] = True
        t += P + sum(rs)
    msgs = []
    for name, m in (("all", slice(None)), ("prefix", pre), ("response", ~pre)):
        e = _rel(full_run["dx"][m], dx[m])
        msgs.append(f"dX[{name}] {e:.1e}")
        assert e <= 1e-2, (name, e)
    for n in PARAM_NAMES:
        for l in range(w.num_layers):
            ref = sum(parts[i]["grads"][n][l] for i in range(N_PARTS))
            e = _rel(full_run["grads"][n][l], ref)
            msgs.append(f"{n}{l} {e:.1e}")
            assert e <= 1e-2, (n, l, e)
    ref = sum(parts[i]["grads"]["g_final"] for i in range(N_PARTS))
    e = _rel(full_run["grads"]["g_final"], ref)
    msgs.append(f"g_final {e:.1e}")
    assert e <= 1e-2
    print("[decoder full] gradients vs oracle: " + "; ".join(msgs), flush=True)


def test_full_decoder_repeated_prefix_layout(full_run):
    """The same harness on the repeated-prefix layout (every [P; R_i] its own
    group, prefix rows copied) gives the grouped response-row outputs and
    parameter gradients (Lemma 2.1 through the whole model)."""
    w, arrs = full_run["w"], full_run["arrs"]
    groups = _groups(w)
    idx, bgroups, t = [], [], 0
    for P, rs in groups:
        s0 = t + P
        for r in rs:
            idx.append(np.concatenate([np.arange(t, t + P), np.arange(s0, s0 + r)]))
            bgroups.append((P, [r]))
            s0 += r
        t = s0
    idx = np.concatenate(idx)
    barrs = dict(arrs)
    barrs["x"] = arrs["x"][idx]
    barrs["dy"] = arrs["dy"][idx]  # zero on every prefix copy, as on the packed prefix
    yb, xb, pb = _run_gpu(w, barrs, backward=True, groups=bgroups)
    resp = np.concatenate([np.arange(P, P + r) + off for (P, (r,)), off in
                           zip(bgroups, np.cumsum([0] + [P + r[0] for P, r in bgroups[:-1]]))])
    resp_packed = np.concatenate([np.arange(s, s + r) for (P, rs), g0 in zip(groups, [0])
                                  for s, r in zip(np.cumsum([P] + rs[:-1]) + g0, rs)])
    e_resp = float(np.max(np.abs(yb.detach().cpu().numpy()[resp] - full_run["y"][resp_packed])))
    msgs = [f"response-row y max-abs {e_resp:.2e}"]
    assert e_resp <= 2e-2
    for n in PARAM_NAMES:
        for l in range(w.num_layers):
            e = _rel(full_run["grads"][n][l], pb[n][l].grad.cpu().numpy())
            msgs.append(f"{n}{l} {e:.1e}")
            assert e <= 1e-2, (n, l, e)
    print("[decoder full] grouped vs repeated-prefix layout: " + "; ".join(msgs), flush=True)
