"""GPU parity of the packed grouped decoder against the fp64 repeated-prefix decoder oracle.

Element by element (outputs, input gradient and every parameter gradient) on a
scaled-down decoder of the same structure; at the full 4-layer, d_model 2048
size, the outputs of two sampled members (the oracle runs those [P; R_i]
sequences only), and the full-size parameter gradients against the same
harness run on the repeated-prefix layout (the method's equivalence claim,
Lemma 2.1), where the fp64 oracle would need ~40 TFLOP.
"""
import time

import numpy as np
import pytest

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


def test_full_decoder_sampled_members():
    w = decoder_workload()
    t0 = time.time()
    arrs = draw_decoder_inputs(w)
    print(f"[decoder full] inputs drawn in {time.time() - t0:.1f}s, T={w.total_rows}", flush=True)
    y, x, p = _run_gpu(w, arrs, backward=True)
    yg = y.detach().cpu().numpy()
    groups = _groups(w)
    members = [0, 15]
    t0 = time.time()
    ref = repeated_prefix_decoder(groups, arrs["x"], _oracle_params(arrs, w), None,
                                  num_heads=w.num_heads, theta=w.rope_theta, eps=w.rms_eps,
                                  members_only=members)
    rows = ~np.isnan(ref["y"][:, 0])
    e_y = float(np.max(np.abs(yg[rows] - ref["y"][rows])))
    print(f"[decoder full] members {members}: {int(rows.sum())} rows, oracle {time.time() - t0:.1f}s, "
          f"y max-abs {e_y:.2e}", flush=True)
    assert e_y <= 2e-2
    # Gradients at full size: the same harness on the repeated-prefix layout
    # (every [P; R_i] as its own group, prefix rows copied) must give the same
    # parameter gradients and response-row outputs (Lemma 2.1).
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
    e_resp = float(np.max(np.abs(yb.detach().cpu().numpy()[resp] - yg[resp_packed])))
    msgs = [f"response-row y max-abs {e_resp:.2e}"]
    assert e_resp <= 2e-2
    for n in PARAM_NAMES:
        for l in range(w.num_layers):
            e = _rel(p[n][l].grad.cpu().numpy(), pb[n][l].grad.cpu().numpy())
            msgs.append(f"{n}{l} {e:.1e}")
            assert e <= 1e-2, (n, l, e)
    print("[decoder full] grouped vs repeated-prefix layout: " + "; ".join(msgs), flush=True)
