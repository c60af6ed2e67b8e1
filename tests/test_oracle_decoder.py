"""Pins of the decoder oracle (repeated-prefix baseline, hand-written backward).  No GPU.

  * central finite differences of the oracle's own loss, for every parameter
    kind and the input;
  * an independent torch fp64 implementation of the same decoder, run per
    baseline sequence with torch's SDPA and autograd;
  * the grouped-vs-baseline invariant (Pith review of Prefix Grouper, "Core
    claim", Lemma 2.1): one torch fp64 pass over the *packed* rows with the
    closed-form grouped mask and the packed position ids gives the oracle's
    outputs and gradients (shared-prefix gradients summed over members).
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import member_sequences, position_ids
from oracle.decoder import PARAM_NAMES, make_params, repeated_prefix_decoder

GROUPS = [(3, [2, 0, 3]), (2, [2])]
D, H, F, NL = 16, 2, 24, 2
THETA, EPS = 10000.0, 1e-6


def _setup(seed=0):
    rng = np.random.default_rng(seed)
    _, T = member_sequences(GROUPS)
    p = make_params(rng, NL, D, F, std=0.3)
    for l in range(NL):  # non-trivial gains so their gradients are tested
        p["g_attn"][l] = 1.0 + 0.2 * rng.standard_normal(D)
        p["g_mlp"][l] = 1.0 + 0.2 * rng.standard_normal(D)
    p["g_final"] = 1.0 + 0.2 * rng.standard_normal(D)
    x = rng.standard_normal((T, D))
    dy = rng.standard_normal((T, D))
    return p, x, dy


def _loss(p, x, dy):
    y = repeated_prefix_decoder(GROUPS, x, p, None, num_heads=H, theta=THETA, eps=EPS)["y"]
    return float((y * dy).sum())


def test_finite_differences():
    p, x, dy = _setup(1)
    res = repeated_prefix_decoder(GROUPS, x, p, dy, num_heads=H, theta=THETA, eps=EPS)
    g = res["grads"]
    rng = np.random.default_rng(2)
    h = 1e-6
    checks = [(n, l) for n in PARAM_NAMES for l in range(NL)] + [("g_final", None), ("x", None)]
    for n, l in checks:
        for _ in range(3):
            if n == "x":
                arr, grad = x, res["x"]
            elif l is None:
                arr, grad = p[n], g[n]
            else:
                arr, grad = p[n][l], g[n][l]
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(p, x, dy)
            arr[idx] = old - h
            lm = _loss(p, x, dy)
            arr[idx] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-6 * max(1.0, abs(fd)), (n, l, idx, fd, grad[idx])


def _torch_params(p):
    tp = {n: [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in p[n]]
          for n in PARAM_NAMES}
    tp["g_final"] = torch.tensor(p["g_final"], dtype=torch.float64, requires_grad=True)
    return tp


def _t_rope(x, pos):
    half = x.shape[-1] // 2
    inv = THETA ** (-torch.arange(half, dtype=torch.float64) * 2.0 / x.shape[-1])
    ang = pos.to(torch.float64)[:, None] * inv[None, :]
    c, s = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return torch.cat([a * c - b * s, b * c + a * s], dim=-1)


def _t_rms(x, g):
    return x * torch.rsqrt((x * x).mean(dim=-1, keepdim=True) + EPS) * g


def _t_decoder(x, tp, pos, attn):
    L = x.shape[0]
    hd = D // H
    for l in range(NL):
        h = _t_rms(x, tp["g_attn"][l])
        q = _t_rope((h @ tp["wq"][l].T).reshape(L, H, hd), pos)
        k = _t_rope((h @ tp["wk"][l].T).reshape(L, H, hd), pos)
        v = (h @ tp["wv"][l].T).reshape(L, H, hd)
        a = attn(q, k, v).reshape(L, D)
        x = x + a @ tp["wo"][l].T
        h2 = _t_rms(x, tp["g_mlp"][l])
        u = h2 @ tp["w1"][l].T
        x = x + (torch.nn.functional.silu(u) * (h2 @ tp["w3"][l].T)) @ tp["w2"][l].T
    return _t_rms(x, tp["g_final"])


def _sdpa_causal(q, k, v):
    return torch.nn.functional.scaled_dot_product_attention(
        q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), is_causal=True).transpose(0, 1)


def _compare(res, y, tp, tx):
    assert np.allclose(res["y"], y.detach().numpy(), atol=1e-10, rtol=0)
    assert np.allclose(res["x"], tx.grad.numpy(), atol=1e-10, rtol=0)
    for n in PARAM_NAMES:
        for l in range(NL):
            assert np.allclose(res["grads"][n][l], tp[n][l].grad.numpy(), atol=1e-10, rtol=0), (n, l)
    assert np.allclose(res["grads"]["g_final"], tp["g_final"].grad.numpy(), atol=1e-10, rtol=0)


def test_matches_torch_per_member():
    p, x, dy = _setup(3)
    res = repeated_prefix_decoder(GROUPS, x, p, dy, num_heads=H, theta=THETA, eps=EPS)
    tp = _torch_params(p)
    tx = torch.tensor(x, requires_grad=True)
    members, T = member_sequences(GROUPS)
    y = torch.zeros((T, D), dtype=torch.float64)
    ys = []
    for m in members:
        idx = torch.from_numpy(m.rows)
        if idx.numel() == 0:
            continue
        out = _t_decoder(tx[idx], tp, torch.arange(idx.numel()), _sdpa_causal)
        w = torch.ones(idx.numel(), 1, dtype=torch.float64)
        w[:m.prefix_len] = 1.0 / m.group_size
        ys.append((out * torch.tensor(dy)[idx] * w).sum())
        y = y.index_copy(0, idx[m.prefix_len:], out[m.prefix_len:])
        if m.member == 0:
            y = y.index_copy(0, idx[:m.prefix_len], out[:m.prefix_len])
    torch.stack(ys).sum().backward()
    _compare(res, y, tp, tx)


def test_grouped_packed_rows_equal_baseline():
    """Lemma 2.1 at model level: one packed pass with the grouped mask and baseline ids."""
    p, x, dy = _setup(4)
    res = repeated_prefix_decoder(GROUPS, x, p, dy, num_heads=H, theta=THETA, eps=EPS)
    members, T = member_sequences(GROUPS)
    seg = np.full(T, -1)
    grp = np.full(T, -1)
    for mi, m in enumerate(members):
        grp[m.prefix[0]:m.prefix[1]] = m.group
        grp[m.resp[0]:m.resp[1]] = m.group
        seg[m.resp[0]:m.resp[1]] = mi
    qi, kj = np.arange(T)[:, None], np.arange(T)[None, :]
    mask = torch.from_numpy((grp[:, None] == grp[None, :]) & (kj <= qi) &
                            ((seg[None, :] == -1) | (seg[None, :] == seg[:, None])))

    def grouped_attn(q, k, v):
        s = torch.einsum("qhd,khd->hqk", q, k) / math.sqrt(q.shape[-1])
        s = s.masked_fill(~mask, float("-inf"))
        return torch.einsum("hqk,khd->qhd", torch.softmax(s, dim=-1), v)

    tp = _torch_params(p)
    tx = torch.tensor(x, requires_grad=True)
    y = _t_decoder(tx, tp, torch.from_numpy(position_ids(GROUPS)), grouped_attn)
    (y * torch.tensor(dy)).sum().backward()
    _compare(res, y, tp, tx)


def test_member_subsets_sum_to_full():
    """members_only with dy: the outputs of the listed members' rows equal the
    full run's, and the gradients over a partition of the members add up to
    the full gradients (prefix gradients are sums over the copies)."""
    p, x, dy = _setup(5)
    kw = dict(num_heads=H, theta=THETA, eps=EPS)
    full = repeated_prefix_decoder(GROUPS, x, p, dy, **kw)
    members, T = member_sequences(GROUPS)
    acc_x = np.zeros_like(full["x"])
    acc = None
    for part in ([0, 3], [1, 2]):
        sub = repeated_prefix_decoder(GROUPS, x, p, dy, members_only=part, **kw)
        rows = np.concatenate([members[i].rows for i in part])
        assert np.allclose(sub["y"][rows], full["y"][rows], atol=1e-12, rtol=0)
        acc_x += sub["x"]
        if acc is None:
            acc = {n: ([a.copy() for a in v] if isinstance(v, list) else v.copy())
                   for n, v in sub["grads"].items()}
        else:
            for n, v in sub["grads"].items():
                if isinstance(v, list):
                    for l in range(len(v)):
                        acc[n][l] += v[l]
                else:
                    acc[n] += v
    assert np.allclose(acc_x, full["x"], atol=1e-12, rtol=0)
    for n, v in full["grads"].items():
        for a, b in zip(acc[n] if isinstance(v, list) else [acc[n]], v if isinstance(v, list) else [v]):
            assert np.allclose(a, b, atol=1e-12, rtol=0), n
