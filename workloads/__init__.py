"""Seeded synthetic workloads for grouped shared-prefix attention.

This module only describes workloads (group lengths, head counts, head size,
dtype) and draws their seeded random inputs.  It holds none of the attention
arithmetic, so both the fp64 CPU oracle and the HIP path may import it.

A workload is a list of groups.  Group g has one shared prefix of P_g tokens
and G_g responses of lengths R_g1..R_gG.  The packed row order is the
sequential concatenation [P; R1; ...; RG] per group, groups one after another
(the input format of the "prefix-grouper-grpo" page on skillsmp.com, section
"Step 3: Restructure Input Format"), without padding.  This module only needs
the total row count T = sum_g (P_g + sum_i R_gi); row offsets are computed by
each side on its own.

Input recipe (one numpy PCG64 generator per workload, seeded with its index):
  1. ragged response lengths, when the workload has them, are drawn first as
     integers uniform on the closed interval [lo, hi];
  2. then, in this order, standard normal float32 arrays Q [T,Hq,d],
     K [T,Hkv,d], V [T,Hkv,d] and dO [T,Hq,d];
  3. for bf16 workloads each array is rounded to bfloat16 with
     round-to-nearest-even; the returned float32 arrays hold exactly the
     bf16 values, so every consumer sees identical inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Group", "AttnWorkload", "DecoderWorkload", "HeadWorkload", "attention_workloads",
    "decoder_workload", "head_workloads", "round_to_bf16", "bf16_bits", "draw_attention_inputs",
    "draw_decoder_inputs", "draw_head_inputs", "scaled_down",
]


@dataclass(frozen=True)
class Group:
    prefix_len: int
    resp_lens: Tuple[int, ...]

    @property
    def rows(self) -> int:
        return self.prefix_len + sum(self.resp_lens)


@dataclass(frozen=True)
class AttnWorkload:
    name: str
    dtype: str              # "f32" or "bf16"
    groups: Tuple[Group, ...]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seed: int
    description: str = ""

    @property
    def total_rows(self) -> int:
        return sum(g.rows for g in self.groups)

    def lengths(self) -> Tuple[List[int], List[int], List[int]]:
        """(prefix_len per group, responses per group, response lengths group-major)."""
        return ([g.prefix_len for g in self.groups],
                [len(g.resp_lens) for g in self.groups],
                [r for g in self.groups for r in g.resp_lens])


@dataclass(frozen=True)
class DecoderWorkload:
    name: str
    groups: Tuple[Group, ...]
    num_layers: int
    d_model: int
    num_heads: int
    head_dim: int
    ffn_dim: int
    seed: int
    rope_theta: float = 10000.0
    rms_eps: float = 1e-6
    weight_std: float = 0.02

    @property
    def total_rows(self) -> int:
        return sum(g.rows for g in self.groups)


@dataclass(frozen=True)
class HeadWorkload:
    """The response log-probability head of a GRPO step: packed hidden states
    [T, d_model] of the last layer, an LM head [vocab, d_model], token ids and
    one reward per response."""
    name: str
    groups: Tuple[Group, ...]
    d_model: int
    vocab: int
    seed: int
    weight_std: float = 0.02
    description: str = ""

    @property
    def total_rows(self) -> int:
        return sum(g.rows for g in self.groups)


def _ragged(rng: np.random.Generator, lo: int, hi: int, n: int) -> Tuple[int, ...]:
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=n))


def attention_workloads() -> Dict[str, AttnWorkload]:
    """The attention workloads, keyed by a short name (the last one is scored
    forward-only: many short responses against one long shared context).

    The ragged lengths are drawn from the same generator that then draws the
    tensors (see ``draw_attention_inputs``), so they are recomputed here with
    a fresh generator of the same seed.
    """
    out = {}
    out["fp32_g4_p64"] = AttnWorkload(
        "fp32_g4_p64", "f32", (Group(64, (16,) * 4),), 2, 2, 64, seed=1,
        description="fp32, 1 group, G=4, P=64, responses of 16, 2/2 heads, d=64")
    out["bf16_g8_p4096"] = AttnWorkload(
        "bf16_g8_p4096", "bf16", (Group(4096, (256,) * 8),), 32, 32, 128, seed=2,
        description="bf16, 1 group, G=8, P=4096, responses of 256, 32/32 heads, d=128")
    rng = np.random.default_rng(3)
    out["bf16_gqa_g16_p8192"] = AttnWorkload(
        "bf16_gqa_g16_p8192", "bf16", (Group(8192, _ragged(rng, 64, 1024, 16)),), 32, 8, 128,
        seed=3,
        description="bf16, GQA 32/8, 1 group, G=16, P=8192, responses uniform in [64,1024], d=128")
    rng = np.random.default_rng(4)
    out["bf16_varlen_2groups"] = AttnWorkload(
        "bf16_varlen_2groups", "bf16",
        (Group(32768, (512,) * 8), Group(2048, _ragged(rng, 128, 2048, 8))), 64, 8, 128, seed=4,
        description="bf16, GQA 64/8, groups (P=32768, 8x512) + (P=2048, 8 responses in [128,2048]), d=128")
    out["bf16_scoring_p32768"] = AttnWorkload(
        "bf16_scoring_p32768", "bf16", (Group(32768, (32,) * 64),), 32, 8, 128, seed=6,
        description="bf16 forward-only scoring: GQA 32/8, 1 group, P=32768, 64 responses of 32, d=128")
    return out


def decoder_workload() -> DecoderWorkload:
    """4-layer decoder on one group: G=16, P=2048, responses of 128."""
    return DecoderWorkload("decoder_4l_g16_p2048", (Group(2048, (128,) * 16),),
                           num_layers=4, d_model=2048, num_heads=16, head_dim=128,
                           ffn_dim=5632, seed=5)


def head_workloads() -> Dict[str, HeadWorkload]:
    """Log-probability head workloads.  The full one reuses the layout of the
    GQA attention workload (P = 8192, 16 responses drawn from seed 3) with a
    2048-wide model and a 32000-token vocabulary (the pages name neither; a
    common 7B-class head size)."""
    rng = np.random.default_rng(3)
    layout = (Group(8192, _ragged(rng, 64, 1024, 16)),)
    return {
        "grpo_head_g16_p8192": HeadWorkload(
            "grpo_head_g16_p8192", layout, 2048, 32000, seed=7,
            description="GRPO log-prob head: bf16, 1 group, G=16, P=8192, responses in [64,1024], "
                        "d_model=2048, vocab=32000"),
    }


def draw_head_inputs(w: HeadWorkload) -> Dict[str, np.ndarray]:
    """Hidden states [T, d_model] ~ N(0,1), LM head [vocab, d_model] ~
    N(0, std^2) (both bf16-rounded), token ids [T] uniform in [0, vocab), one
    reward ~ N(0,1) per response (float32), in that order."""
    rng = np.random.default_rng(w.seed)
    T = w.total_rows
    hidden = round_to_bf16(rng.standard_normal((T, w.d_model), dtype=np.float32))
    weight = round_to_bf16(rng.standard_normal((w.vocab, w.d_model), dtype=np.float32)
                           * np.float32(w.weight_std))
    tokens = rng.integers(0, w.vocab, size=T).astype(np.int32)
    n_resp = sum(len(g.resp_lens) for g in w.groups)
    rewards = rng.standard_normal(n_resp, dtype=np.float32)
    return {"hidden": hidden, "weight": weight, "tokens": tokens, "rewards": rewards}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); return float32 holding it.

    Works in place on a float32 copy, in chunks, with uint32 arithmetic (finite
    inputs only: standard normal draws never produce NaN or Inf).
    """
    out = np.array(x, dtype=np.float32, copy=True, order="C")
    u = out.reshape(-1).view(np.uint32)
    step = 1 << 24
    for s in range(0, u.size, step):
        c = u[s:s + step]
        c += ((c >> 16) & 1) + np.uint32(0x7FFF)
        c &= np.uint32(0xFFFF0000)
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-representable."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bf16-representable; call round_to_bf16 first")
    return (u >> 16).astype(np.uint16)


def draw_attention_inputs(w: AttnWorkload) -> Dict[str, np.ndarray]:
    """Q, K, V, dO as float32 arrays in packed layout (bf16-exact for bf16 workloads)."""
    rng = np.random.default_rng(w.seed)
    # replay the length draws so the tensor draws follow them in one stream
    _replay_length_draws(rng, w)
    T = w.total_rows
    arrs = {}
    for name, h in (("q", w.num_q_heads), ("k", w.num_kv_heads), ("v", w.num_kv_heads),
                    ("do", w.num_q_heads)):
        a = rng.standard_normal((T, h, w.head_dim), dtype=np.float32)
        if w.dtype == "bf16":
            a = round_to_bf16(a)
        arrs[name] = a
    return arrs


def _replay_length_draws(rng: np.random.Generator, w: AttnWorkload) -> None:
    if w.name == "bf16_gqa_g16_p8192":
        _ragged(rng, 64, 1024, 16)
    elif w.name == "bf16_varlen_2groups":
        _ragged(rng, 128, 2048, 8)


def scaled_down(name: str, groups: Sequence[Tuple[int, Sequence[int]]], dtype: str,
                hq: int, hkv: int, d: int, seed: int) -> AttnWorkload:
    """A small workload of the same structure, for element-wise parity tests."""
    return AttnWorkload(name, dtype, tuple(Group(int(p), tuple(int(r) for r in rs))
                                           for p, rs in groups), hq, hkv, d, seed)


def draw_decoder_inputs(w: DecoderWorkload) -> Dict[str, np.ndarray]:
    """Hidden states X [T, d_model], per-layer weights and upstream gradient dY.

    Draw order: X ~ N(0,1); then per layer Wq, Wk, Wv, Wo [d_model, d_model],
    W1, W3 [ffn, d_model], W2 [d_model, ffn], each N(0, std^2); then dY ~ N(0,1)
    on response rows and 0 on prefix rows.  Weights are stored as
    [out_features, in_features].  All values are bf16-rounded.
    """
    rng = np.random.default_rng(w.seed)
    T, D, F = w.total_rows, w.d_model, w.ffn_dim
    out = {"x": round_to_bf16(rng.standard_normal((T, D), dtype=np.float32))}
    for l in range(w.num_layers):
        for nm, shape in (("wq", (D, D)), ("wk", (D, D)), ("wv", (D, D)), ("wo", (D, D)),
                          ("w1", (F, D)), ("w3", (F, D)), ("w2", (D, F))):
            out[f"{nm}{l}"] = round_to_bf16(
                (rng.standard_normal(shape, dtype=np.float32) * np.float32(w.weight_std)))
    dy = rng.standard_normal((T, D), dtype=np.float32)
    t = 0
    for g in w.groups:
        dy[t:t + g.prefix_len] = 0.0
        t += g.rows
    out["dy"] = round_to_bf16(dy)
    return out
