"""Repeated-prefix baseline of a small pre-norm decoder, fp64, with a hand-written backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say Prefix Grouper changes only input construction and attention
(abstract page of "Prefix Grouper: Efficient GRPO Training through
Shared-Prefix Forward", English abstract; Pith review, "Core claim": training
equivalence, Lemma 2.1).  So the whole-model oracle runs an ordinary decoder on
every baseline sequence [P; R_i] separately, at positions 0..L-1, and maps the
results back to packed rows: outputs of prefix rows are member 0's (all members
agree), gradients of shared inputs and of every parameter are summed over the
members.  The decoder itself is not described by the pages; this reading is
used:

  x_0 = X
  per layer l:
    h   = rmsnorm(x) * g_attn
    q,k,v = h Wq^T, h Wk^T, h Wv^T           (heads of size hd, rotate-half RoPE on q, k)
    x  += attention(q, k, v) Wo^T            (causal, scale 1/sqrt(hd))
    h2  = rmsnorm(x) * g_mlp
    x  += (silu(h2 W1^T) * (h2 W3^T)) W2^T
  Y = rmsnorm(x) * g_final;  rmsnorm(x) = x / sqrt(mean(x^2) + eps)

The loss is sum(Y * dY); the upstream gradient of a prefix row is split evenly
over the G copies (any split summing to it gives the same result).
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

from oracle.attention import causal_attention_backward, causal_attention_forward, member_sequences

PARAM_NAMES = ("wq", "wk", "wv", "wo", "w1", "w3", "w2", "g_attn", "g_mlp")


def rope(x, pos, theta, inverse=False):
    """Rotate-half rotary embedding of x [L, H, d] at positions pos [L] (fp64)."""
    L, H, d = x.shape
    half = d // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    if inverse:
        s = -s
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def _rms(x, eps):
    return 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)


def _rmsnorm_bwd(x, r, g, dy):
    """Gradient of y = x * r * g (r = rms factor) w.r.t. x and g."""
    gy = dy * g
    n = x.shape[-1]
    dx = r * gy - (r ** 3) * x * (gy * x).sum(axis=-1, keepdims=True) / n
    dg = (dy * x * r).sum(axis=0)
    return dx, dg


def _silu(u):
    return u / (1.0 + np.exp(-u))


def decoder_member(x, params, dy, num_heads, theta, eps):
    """Forward and backward of the decoder on one sequence (fp64).

    x: [L, D]; params: dict with per-layer lists and "g_final"; dy: [L, D] or None.
    Returns (y, grads) where grads has the same structure as params plus "x".
    """
    L, D = x.shape
    nl = len(params["wq"])
    hd = D // num_heads
    scale = 1.0 / math.sqrt(hd)
    pos = np.arange(L)
    caches = []
    h_ = x
    for l in range(nl):
        c = {"x_in": h_}
        r1 = _rms(h_, eps)
        hn = h_ * r1 * params["g_attn"][l]
        q = (hn @ params["wq"][l].T).reshape(L, num_heads, hd)
        k = (hn @ params["wk"][l].T).reshape(L, num_heads, hd)
        v = (hn @ params["wv"][l].T).reshape(L, num_heads, hd)
        qr, kr = rope(q, pos, theta), rope(k, pos, theta)
        a = np.zeros((L, num_heads, hd))
        for hh in range(num_heads):
            a[:, hh], _ = causal_attention_forward(qr[:, hh], kr[:, hh], v[:, hh], scale)
        af = a.reshape(L, D)
        x1 = h_ + af @ params["wo"][l].T
        r2 = _rms(x1, eps)
        hn2 = x1 * r2 * params["g_mlp"][l]
        u = hn2 @ params["w1"][l].T
        gt = hn2 @ params["w3"][l].T
        act = _silu(u) * gt
        x2 = x1 + act @ params["w2"][l].T
        c.update(r1=r1, hn=hn, qr=qr, kr=kr, v=v, af=af, x1=x1, r2=r2, hn2=hn2, u=u, gt=gt, act=act)
        caches.append(c)
        h_ = x2
    rf = _rms(h_, eps)
    y = h_ * rf * params["g_final"]
    if dy is None:
        return y, None
    grads = {n: [None] * nl for n in PARAM_NAMES}
    dxl, grads["g_final"] = _rmsnorm_bwd(h_, rf, params["g_final"], dy)
    for l in reversed(range(nl)):
        c = caches[l]
        # MLP: x2 = x1 + act W2^T
        grads["w2"][l] = dxl.T @ c["act"]
        dact = dxl @ params["w2"][l]
        sig = 1.0 / (1.0 + np.exp(-c["u"]))
        du = dact * c["gt"] * sig * (1.0 + c["u"] * (1.0 - sig))
        dgt = dact * _silu(c["u"])
        grads["w1"][l] = du.T @ c["hn2"]
        grads["w3"][l] = dgt.T @ c["hn2"]
        dhn2 = du @ params["w1"][l] + dgt @ params["w3"][l]
        dx1, grads["g_mlp"][l] = _rmsnorm_bwd(c["x1"], c["r2"], params["g_mlp"][l], dhn2)
        dx1 = dx1 + dxl
        # attention: x1 = x_in + af Wo^T
        grads["wo"][l] = dx1.T @ c["af"]
        da = (dx1 @ params["wo"][l]).reshape(L, num_heads, hd)
        dqr = np.zeros_like(c["qr"]); dkr = np.zeros_like(c["kr"]); dv = np.zeros_like(c["v"])
        for hh in range(num_heads):
            dqr[:, hh], dkr[:, hh], dv[:, hh] = causal_attention_backward(
                c["qr"][:, hh], c["kr"][:, hh], c["v"][:, hh], da[:, hh], scale)
        dq = rope(dqr, pos, theta, inverse=True).reshape(L, D)
        dk = rope(dkr, pos, theta, inverse=True).reshape(L, D)
        dv = dv.reshape(L, D)
        grads["wq"][l] = dq.T @ c["hn"]
        grads["wk"][l] = dk.T @ c["hn"]
        grads["wv"][l] = dv.T @ c["hn"]
        dhn = dq @ params["wq"][l] + dk @ params["wk"][l] + dv @ params["wv"][l]
        dxin, grads["g_attn"][l] = _rmsnorm_bwd(c["x_in"], c["r1"], params["g_attn"][l], dhn)
        dxl = dxin + dx1
    grads["x"] = dxl
    return y, grads


def repeated_prefix_decoder(groups, x, params, dy=None, num_heads=1, theta=10000.0, eps=1e-6,
                            members_only=None):
    """The decoder on every [P; R_i] separately, mapped back to packed rows.

    groups: (prefix_len, resp_lens) per group; x: [T, D] packed; params as in
    decoder_member; dy: [T, D] or None.  members_only: optional list of member
    indices (group-major) to evaluate (for checks at full size, where the
    members can be spread over several calls).  Returns {"y": [T, D] (rows of
    evaluated members, NaN elsewhere), and with dy "grads": parameter
    gradients and "x" [T, D], summed over the evaluated members}.  Over a
    partition of the members these partial sums add up to the full result;
    the upstream gradient of a prefix row is divided by the group's full G
    either way.
    """
    members, T = member_sequences(groups)
    x = np.asarray(x, np.float64)
    y = np.full((T, x.shape[1]), np.nan)
    want = dy is not None
    total = None
    dx = np.zeros_like(x) if want else None
    for mi, m in enumerate(members):
        if members_only is not None and mi not in members_only:
            continue
        idx = m.rows
        if idx.size == 0:
            continue
        dys = None
        if want:
            dys = np.asarray(dy[idx], np.float64).copy()
            dys[:m.prefix_len] /= m.group_size
        ys, g = decoder_member(x[idx], params, dys, num_heads, theta, eps)
        y[idx[m.prefix_len:]] = ys[m.prefix_len:]
        if m.member == 0 or members_only is not None:
            y[idx[:m.prefix_len]] = ys[:m.prefix_len]
        if want:
            dx[idx] += g["x"]
            if total is None:
                total = {n: ([a.copy() for a in g[n]] if isinstance(g[n], list) else g[n].copy())
                         for n in g if n != "x"}
            else:
                for n in total:
                    if isinstance(total[n], list):
                        for l in range(len(total[n])):
                            total[n][l] += g[n][l]
                    else:
                        total[n] += g[n]
    out = {"y": y}
    if want:
        out["grads"] = total
        out["x"] = dx
    return out


def make_params(rng, num_layers, d_model, ffn, std=0.02, dtype_round=None):
    """Random decoder parameters (for pins); norm gains start at one."""
    p = {n: [] for n in PARAM_NAMES}
    for _ in range(num_layers):
        for n, shape in (("wq", (d_model, d_model)), ("wk", (d_model, d_model)),
                         ("wv", (d_model, d_model)), ("wo", (d_model, d_model)),
                         ("w1", (ffn, d_model)), ("w3", (ffn, d_model)), ("w2", (d_model, ffn))):
            w = rng.standard_normal(shape) * std
            p[n].append(dtype_round(w) if dtype_round else w)
        p["g_attn"].append(np.ones(d_model))
        p["g_mlp"].append(np.ones(d_model))
    p["g_final"] = np.ones(d_model)
    return p
