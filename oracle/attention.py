"""Repeated-prefix baseline of grouped attention, in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definitions used here, restated from the pages on Prefix Grouper:
  * Baseline (skillsmp.com "prefix-grouper-grpo", "Step 1: Set Up Standard
    GRPO Baseline"): member i of a group is the sequence [P; R_i], encoded on
    its own, so the prefix is encoded once per member.
  * Packed layout ("Step 3: Restructure Input Format" on the same page, and
    the Pith review's "Core claim"): rows [P; R_1; ...; R_G] per group,
    groups one after another.  Here there is no padding: response i starts
    right after response i-1.
  * Equivalence (Pith review, "What carries the argument" and "Core claim",
    Lemma 2.1): the method's packed outputs equal the baseline's; a prefix
    row's output is the (identical) output of any member's copy, and the
    gradient of a shared prefix input is the sum of the gradients of its G
    copies.
  * Position ids (Pith review, "What carries the argument"): each packed row
    keeps the index it has in its baseline sequence.

Readings where the pages leave a point open:
  * softmax scale 1/sqrt(d) unless given (the printed sketch lost its
    exponent);
  * causal masking is inclusive (a token sees itself);
  * the upstream gradient of a prefix row is split evenly over the G copies
    (any split that sums to it gives the same result, since the backward is
    linear in the upstream gradient and the copies are the same function);
  * grouped-query attention: query head h reads key/value head
    h // (Hq / Hkv).

Array layout: q, do [T, Hq, d]; k, v [T, Hkv, d]; lse [Hq, T] natural log.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

ROW_BLOCK = 512  # query rows per block, so no L x L fp64 matrix is ever held


@dataclass(frozen=True)
class MemberSeq:
    """One baseline sequence [P; R_i] and where its rows sit in the packed layout."""
    group: int
    member: int
    group_size: int          # G of its group
    prefix: Tuple[int, int]  # packed rows of the shared prefix [start, end)
    resp: Tuple[int, int]    # packed rows of this member's response [start, end)

    @property
    def prefix_len(self) -> int:
        return self.prefix[1] - self.prefix[0]

    @property
    def rows(self) -> np.ndarray:
        """Packed row index of each position of the baseline sequence."""
        return np.concatenate([np.arange(*self.prefix), np.arange(*self.resp)]).astype(np.int64)


def member_sequences(groups: Sequence[Tuple[int, Sequence[int]]]) -> Tuple[List[MemberSeq], int]:
    """Baseline sequences of a packed batch, from (prefix_len, resp_lens) per group.

    Packed order is [P; R_1; ...; R_G] per group, groups concatenated.
    Returns the member list (group-major) and the total packed row count.
    """
    out: List[MemberSeq] = []
    t = 0
    for gi, (P, rs) in enumerate(groups):
        P = int(P)
        rs = [int(r) for r in rs]
        if P < 0 or any(r < 0 for r in rs) or len(rs) < 1:
            raise ValueError("prefix and response lengths must be >= 0, with >= 1 response")
        pre = (t, t + P)
        t += P
        for i, r in enumerate(rs):
            out.append(MemberSeq(gi, i, len(rs), pre, (t, t + r)))
            t += r
    return out, t


def position_ids(groups) -> np.ndarray:
    """Baseline position of every packed row: prefix token t -> t, response token j -> P + j."""
    members, T = member_sequences(groups)
    pos = np.full(T, -1, dtype=np.int64)
    for m in members:
        pos[m.rows] = np.arange(m.rows.size)
    return pos


def pair_counts(groups) -> Tuple[int, int]:
    """Unmasked (query, key) pairs per head: (grouped packed layout, repeated-prefix baseline).

    Grouped: the prefix once, P(P+1)/2, plus per response R*P + R(R+1)/2.
    Baseline: each [P; R_i] on its own, (P+R_i)(P+R_i+1)/2.
    Both count causal pairs including the diagonal (Pith review, "Core claim",
    Lemma 2.2's comparison of the two computations).
    """
    pg = pb = 0
    for P, rs in groups:
        pg += P * (P + 1) // 2
        for r in rs:
            pg += r * P + r * (r + 1) // 2
            L = P + r
            pb += L * (L + 1) // 2
    return pg, pb


def _softmax_rows(s: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row softmax of a score block with -inf for masked entries; returns (p, logsumexp)."""
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return e / z, (m + np.log(z))[:, 0]


def _causal_scores(q: np.ndarray, k: np.ndarray, r0: int, r1: int, scale: float) -> np.ndarray:
    """scale * q[r0:r1] k[:r1]^T with -inf where the key comes after the query."""
    s = scale * (q[r0:r1] @ k[:r1].T)
    qi = np.arange(r0, r1)[:, None]
    kj = np.arange(r1)[None, :]
    s[kj > qi] = -np.inf
    return s


def causal_attention_forward(q, k, v, scale):
    """Standard causal softmax attention of one sequence and one head, fp64.

    q, k, v: [L, d].  Returns o [L, d] and the natural-log logsumexp [L] of
    the scaled scores of each row.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    L = q.shape[0]
    o = np.zeros_like(q)
    lse = np.zeros(L)
    for r0 in range(0, L, ROW_BLOCK):
        r1 = min(L, r0 + ROW_BLOCK)
        p, lse[r0:r1] = _softmax_rows(_causal_scores(q, k, r0, r1, scale))
        o[r0:r1] = p @ v[:r1]
    return o, lse


def causal_attention_backward(q, k, v, do, scale):
    """Gradients of sum(o * do) for causal attention of one sequence and one head, fp64.

    Textbook chain rule through softmax: with P = softmax(S) and dP = dO V^T,
    dS = P * (dP - rowsum(P * dP)); then dQ = scale dS K, dK = scale dS^T Q,
    dV = P^T dO.  The probabilities are recomputed from the scores.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); do = np.asarray(do, np.float64)
    L = q.shape[0]
    dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
    for r0 in range(0, L, ROW_BLOCK):
        r1 = min(L, r0 + ROW_BLOCK)
        p, _ = _softmax_rows(_causal_scores(q, k, r0, r1, scale))
        dob = do[r0:r1]
        dv[:r1] += p.T @ dob
        dp = dob @ v[:r1].T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dq[r0:r1] = scale * (ds @ k[:r1])
        dk[:r1] += scale * (ds.T @ q[r0:r1])
    return dq, dk, dv


def _kv_groups(hq: int, hkv: int, kv_heads: Optional[Iterable[int]]):
    if hq % hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    rep = hq // hkv
    kvs = list(range(hkv)) if kv_heads is None else [int(h) for h in kv_heads]
    return rep, kvs


def repeated_prefix_attention(groups, q, k, v, do=None, scale=None, kv_heads=None,
                              check_prefix_copies=True, members=None) -> Dict[str, np.ndarray]:
    """Baseline grouped attention: every [P; R_i] on its own, mapped back to packed rows.

    groups: (prefix_len, resp_lens) per group.  q, do: [T, Hq, d]; k, v: [T, Hkv, d].
    kv_heads: optional subset of key/value heads; the result then holds only
    those kv heads and their query heads, in order (heads are independent).
    Returns o [T, hq', d], lse [hq', T] and, with do, dq [T, hq', d],
    dk/dv [T, hkv', d]; q heads listed in "q_heads", kv heads in "kv_heads".

    Per member sequence and query head: forward and backward of standard
    causal attention.  Prefix rows take member 0's output and logsumexp (all
    members must agree, which is checked), and sum the gradient over the G
    copies; response rows take their own member's values.

    members: optional subset of member sequences (indices in group-major
    order, as member_sequences lists them).  Only those are evaluated: O and
    LSE are filled on their rows (a group's prefix rows from its first listed
    member; other rows stay zero) and the gradients are the sums over the
    listed members only, so the sums over a partition of the members add up
    to the full result (the prefix gradient is a sum over copies).  The
    upstream gradient of a prefix row is still divided by the group's full G.
    """
    T, hq, d = q.shape
    hkv = k.shape[1]
    rep, kvs = _kv_groups(hq, hkv, kv_heads)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qh = [kv * rep + j for kv in kvs for j in range(rep)]
    members_all, T2 = member_sequences(groups)
    if T2 != T:
        raise ValueError(f"packed rows {T} != sum of lengths {T2}")
    o = np.zeros((T, len(qh), d)); lse = np.zeros((len(qh), T))
    want_grad = do is not None
    if want_grad:
        dq = np.zeros((T, len(qh), d)); dk = np.zeros((T, len(kvs), d)); dv = np.zeros((T, len(kvs), d))
    chosen = None if members is None else {int(i) for i in members}
    first_seen = set()  # groups whose prefix output is already filled
    for mi, m in enumerate(members_all):
        if chosen is not None and mi not in chosen:
            continue
        idx = m.rows
        if idx.size == 0:
            continue
        P = m.prefix_len
        first = m.group not in first_seen
        first_seen.add(m.group)
        for a, h in enumerate(qh):
            b = a // rep
            hk = kvs[b]
            qs = q[idx, h].astype(np.float64)
            ks = k[idx, hk].astype(np.float64)
            vs = v[idx, hk].astype(np.float64)
            os_, ls_ = causal_attention_forward(qs, ks, vs, scale)
            if first:
                o[idx[:P], a] = os_[:P]
                lse[a, idx[:P]] = ls_[:P]
            elif check_prefix_copies and P:
                err = np.max(np.abs(o[idx[:P], a] - os_[:P]))
                if err > 1e-12 * max(1.0, np.max(np.abs(os_[:P]))):
                    raise AssertionError(f"prefix copies disagree by {err}")
            o[idx[P:], a] = os_[P:]
            lse[a, idx[P:]] = ls_[P:]
            if want_grad:
                dos = do[idx, h].astype(np.float64)
                dos[:P] /= m.group_size
                g_q, g_k, g_v = causal_attention_backward(qs, ks, vs, dos, scale)
                # rows of one member sequence are distinct, so += accumulates exactly
                dq[idx, a] += g_q
                dk[idx, b] += g_k
                dv[idx, b] += g_v
    res = {"o": o, "lse": lse, "q_heads": np.array(qh), "kv_heads": np.array(kvs)}
    if want_grad:
        res.update(dq=dq, dk=dk, dv=dv)
    return res


def _row_member_map(groups):
    members, T = member_sequences(groups)
    owner = {}
    for mi, m in enumerate(members):
        for r in range(*m.resp):
            owner[r] = mi
    return members, T, owner


def repeated_prefix_rows(groups, q, k, v, do, q_rows, q_heads, scale=None) -> Dict[str, np.ndarray]:
    """O, logsumexp and dQ of the baseline at sampled packed query rows.

    A response row is a row of its own member sequence.  A prefix row is
    present in all G member sequences; its output is member 0's and its dQ
    is the sum over the G copies (each with dO / G), as in the full oracle.
    Cost per row is one softmax row of its sequence, so this works at any size.
    Returns o [n_rows, n_heads, d], lse [n_heads, n_rows], dq like o (zeros
    when do is None: forward only, one sequence per row).
    """
    T, hq, d = q.shape
    rep = hq // k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    members, T2, owner = _row_member_map(groups)
    q_rows = [int(r) for r in q_rows]
    q_heads = [int(h) for h in q_heads]
    o = np.zeros((len(q_rows), len(q_heads), d)); lse = np.zeros((len(q_heads), len(q_rows)))
    dq = np.zeros_like(o)
    for ri, r in enumerate(q_rows):
        if r in owner:
            seqs = [members[owner[r]]]
        else:
            seqs = [m for m in members if m.prefix[0] <= r < m.prefix[1]]
            if do is None:
                seqs = seqs[:1]
        for hi, h in enumerate(q_heads):
            hk = h // rep
            for si, m in enumerate(seqs):
                idx = m.rows
                pos = int(np.nonzero(idx == r)[0][0])
                kk = k[idx[:pos + 1], hk].astype(np.float64)
                vv = v[idx[:pos + 1], hk].astype(np.float64)
                qq = q[r, h].astype(np.float64)
                s = scale * (kk @ qq)
                p, l = _softmax_rows(s[None, :])
                p = p[0]
                if si == 0:
                    o[ri, hi] = p @ vv
                    lse[hi, ri] = l[0]
                if do is None:
                    continue
                g = do[r, h].astype(np.float64) / len(seqs)
                dp = vv @ g
                ds = p * (dp - (p * dp).sum())
                dq[ri, hi] += scale * (ds @ kk)
    return {"o": o, "lse": lse, "dq": dq}


def repeated_prefix_key_rows(groups, q, k, v, do, k_rows, kv_heads, scale=None,
                             members=None) -> Dict[str, np.ndarray]:
    """dK and dV of the baseline at sampled packed key rows.

    For key row r: sum over every member sequence containing r (all G for a
    prefix row, one for a response row), over every query position at or
    after r in that sequence and over the query heads of the kv head, of the
    textbook softmax gradient.  Each contributing query needs its full
    softmax row, so the cost is a forward pass over the queries that follow r.
    The softmax rows of a member sequence are computed once for all the
    requested key rows it contains, from the earliest of them on: a query
    before key r gives probability exactly 0 at r, so it adds exact zeros.
    members: optional subset of member sequences (group-major indices); the
    sums then run over those members only (partial sums, as in
    repeated_prefix_attention).
    Returns dk, dv [n_rows, n_kv_heads, d].
    """
    T, hq, d = q.shape
    rep = hq // k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    members_sel = None if members is None else {int(i) for i in members}
    members, T2, owner = _row_member_map(groups)
    k_rows = [int(r) for r in k_rows]
    dk = np.zeros((len(k_rows), len(kv_heads), d)); dv = np.zeros_like(dk)
    # member index -> [(output slot, position of the key row in the sequence)]
    wanted: Dict[int, List[Tuple[int, int]]] = {}
    for ri, r in enumerate(k_rows):
        if r in owner:
            mis = [owner[r]]
        else:
            mis = [mi for mi, m in enumerate(members) if m.prefix[0] <= r < m.prefix[1]]
        for mi in mis:
            if members_sel is not None and mi not in members_sel:
                continue
            pos = int(np.nonzero(members[mi].rows == r)[0][0])
            wanted.setdefault(mi, []).append((ri, pos))
    for mi, slots in wanted.items():
        m = members[mi]
        idx = m.rows
        L = idx.size
        start = min(pos for _, pos in slots)
        for bi, hk in enumerate(kv_heads):
            ks = k[idx, hk].astype(np.float64)
            vs = v[idx, hk].astype(np.float64)
            for j in range(rep):
                h = hk * rep + j
                qs = q[idx, h].astype(np.float64)
                dos = do[idx, h].astype(np.float64)
                dos[:m.prefix_len] /= m.group_size
                for r0 in range(start, L, ROW_BLOCK):
                    r1 = min(L, r0 + ROW_BLOCK)
                    p, _ = _softmax_rows(_causal_scores(qs, ks, r0, r1, scale))
                    dp = dos[r0:r1] @ vs[:r1].T
                    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                    for ri, pos in slots:
                        if pos < r1:
                            dk[ri, bi] += scale * (ds[:, pos] @ qs[r0:r1])
                            dv[ri, bi] += p[:, pos] @ dos[r0:r1]
    return {"dk": dk, "dv": dv}


def repeated_prefix_rope(groups, x, theta=10000.0, positions_from_baseline=True):
    """Rotary embedding of packed rows at their baseline positions, fp64.

    x: [T, H, d] (d even).  Rotate-half pairing: coordinate i (i < d/2) is
    paired with i + d/2, rotated by angle pos * theta^(-2i/d).  Each member
    sequence [P; R_i] is rotated with positions 0..L-1 and mapped back
    (prefix copies agree by construction).
    """
    T, H, d = x.shape
    members, T2 = member_sequences(groups)
    out = np.zeros((T, H, d))
    half = d // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / d)
    for m in members:
        idx = m.rows
        if idx.size == 0:
            continue
        ang = np.arange(idx.size, dtype=np.float64)[:, None] * inv[None, :]
        c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
        xs = x[idx].astype(np.float64)
        a, b = xs[..., :half], xs[..., half:]
        out[idx, :, :half] = a * c - b * s
        out[idx, :, half:] = b * c + a * s
    return out
