"""Pre-norm decoder over packed grouped batches (the 4-layer decoder workload).

Prefix Grouper changes only input construction and attention (abstract page
of "Prefix Grouper: Efficient GRPO Training through Shared-Prefix Forward";
Pith review, "Core claim"), so every other layer runs unchanged, once per
packed row: RMSNorm, the Q/K/V/O projections and the SwiGLU MLP are plain
PyTorch (hipBLASLt GEMMs), while attention and the rotary embedding at
baseline position ids go through libpg_attn (GroupedAttention, pg_rope).

Precision: the attention sublayer computes in bf16 -- the Q/K/V projections
take the bf16-rounded normed input and bf16 weights and produce bf16 Q/K/V,
RoPE and the grouped-attention kernels run in bf16, and the O projection
multiplies the bf16 attention output by bf16 weights with fp32 accumulation
and an fp32 result.  The residual stream, the norms and the SwiGLU MLP (a layer
the method leaves unchanged) stay in fp32: with a bf16 MLP the rounding noise
of a d_model 2048, 4-layer stack alone reaches ~1.7e-2 max-abs on the
normalised output.  Parameters are fp32 leaves holding bf16-representable
values.

Layer (per l):  x += Attn(RoPE(q, k), v) Wo^T with q, k, v = RMSNorm(x) W^T;
                x += (silu(h W1^T) * (h W3^T)) W2^T with h = RMSNorm(x);
output RMSNorm(x).  RMSNorm(x) = x / sqrt(mean(x^2) + eps) * g.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List

import torch
import torch.nn.functional as F

from . import PackedBatch, grouped_attention, pg_rope

PARAM_NAMES = ("wq", "wk", "wv", "wo", "w1", "w3", "w2", "g_attn", "g_mlp")


class _Rope(torch.autograd.Function):
    """RoPE at the batch's baseline position ids; backward applies the inverse rotation."""

    @staticmethod
    def forward(ctx, x, batch, theta):
        y = x.contiguous().clone()
        pg_rope(batch, y, theta)
        ctx.batch, ctx.theta = batch, theta
        return y

    @staticmethod
    def backward(ctx, dy):
        g = dy.contiguous().clone()
        pg_rope(ctx.batch, g, ctx.theta, inverse=True)
        return g, None, None


def rope(x, batch: PackedBatch, theta: float = 10000.0):
    return _Rope.apply(x, batch, theta)


def rmsnorm(x, g, eps):
    return x * torch.rsqrt(x.pow(2).mean(dim=-1, keepdim=True) + eps) * g


@dataclass
class DecoderConfig:
    num_layers: int
    d_model: int
    num_heads: int
    ffn_dim: int
    rope_theta: float = 10000.0
    eps: float = 1e-6


def make_parameters(weights: Dict[str, object], cfg: DecoderConfig, device="cuda") -> Dict:
    """fp32 leaf parameters from per-layer arrays named wq0, wk0, ... (norm gains start at one)."""
    p = {n: [] for n in PARAM_NAMES}
    for l in range(cfg.num_layers):
        for n in ("wq", "wk", "wv", "wo", "w1", "w3", "w2"):
            t = torch.as_tensor(weights[f"{n}{l}"], dtype=torch.float32).to(device)
            p[n].append(t.requires_grad_(True))
        p["g_attn"].append(torch.ones(cfg.d_model, device=device, requires_grad=True))
        p["g_mlp"].append(torch.ones(cfg.d_model, device=device, requires_grad=True))
    p["g_final"] = torch.ones(cfg.d_model, device=device, requires_grad=True)
    return p


def parameter_list(p: Dict) -> List[torch.Tensor]:
    out = [t for n in PARAM_NAMES for t in p[n]]
    out.append(p["g_final"])
    return out


def decoder_forward(x, p: Dict, batch: PackedBatch, cfg: DecoderConfig,
                    compute_dtype=torch.bfloat16):
    """Output [T, d_model] (fp32) of the decoder on the packed rows of `batch`."""
    T, D = x.shape
    H = cfg.num_heads
    hd = D // H
    cd = compute_dtype
    for l in range(cfg.num_layers):
        h = rmsnorm(x, p["g_attn"][l], cfg.eps).to(cd)
        q = F.linear(h, p["wq"][l].to(cd)).view(T, H, hd)
        k = F.linear(h, p["wk"][l].to(cd)).view(T, H, hd)
        v = F.linear(h, p["wv"][l].to(cd)).view(T, H, hd)
        q = rope(q, batch, cfg.rope_theta)
        k = rope(k, batch, cfg.rope_theta)
        a = grouped_attention(q, k, v.contiguous(), batch)
        # bf16 operands, fp32 accumulation and result
        x = x + F.linear(a.view(T, D).float(), p["wo"][l].to(cd).float())
        h2 = rmsnorm(x, p["g_mlp"][l], cfg.eps)
        u = F.linear(h2, p["w1"][l])
        gt = F.linear(h2, p["w3"][l])
        x = x + F.linear(F.silu(u) * gt, p["w2"][l])
    return rmsnorm(x, p["g_final"], cfg.eps)
