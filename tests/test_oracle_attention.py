"""Pins of the fp64 attention oracle against things other than itself.

No GPU.  Each test names what it pins:
  * a hand-written fixture of the visibility pattern and position ids,
    derived from the pages' description (tests/golden/);
  * brute-force pure-Python softmax attention (math.exp, loops);
  * central finite differences of the oracle's own forward;
  * torch autograd (fp64, CPU) on a dense masked formulation on packed rows;
  * library special cases (G = 1 is ordinary causal attention; P = 0 is
    independent causal attention per response) via torch's SDPA;
  * closed forms (zero queries give uniform attention over the visible keys);
  * invariants (convex hull, logsumexp >= row max, key shift invariance,
    permutation of responses, linearity in the upstream gradient);
  * pair counts by brute force, and the 1/G limit of the pair ratio.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import (causal_attention_backward, causal_attention_forward,
                              member_sequences, pair_counts, position_ids,
                              repeated_prefix_attention, repeated_prefix_key_rows,
                              repeated_prefix_rows)
from tests.golden_io import read_visibility_fixture

RNG = np.random.default_rng(1234)


def _rand(T, hq, hkv, d, rng=RNG):
    return (rng.standard_normal((T, hq, d)), rng.standard_normal((T, hkv, d)),
            rng.standard_normal((T, hkv, d)), rng.standard_normal((T, hq, d)))


# ---------------------------------------------------------------- fixture pins

def test_golden_positions_and_pairs():
    groups, positions, pairs, vis = read_visibility_fixture()
    assert np.array_equal(position_ids(groups), positions)
    assert pair_counts(groups) == pairs
    assert int(vis.sum()) == pairs[0]


def test_golden_visibility_from_jacobian():
    """Key k influences query row q's output iff the fixture says k is visible to q."""
    groups, _, _, vis = read_visibility_fixture()
    T = vis.shape[0]
    rng = np.random.default_rng(7)
    q, k, v, _ = _rand(T, 1, 1, 5, rng)
    seen = np.zeros((T, T), dtype=bool)
    for r in range(T):
        do = np.zeros((T, 1, 5))
        do[r, 0] = rng.standard_normal(5)
        res = repeated_prefix_attention(groups, q, k, v, do)
        seen[r] = np.abs(res["dv"][:, 0]).sum(axis=1) > 0
    assert np.array_equal(seen, vis)


def test_zero_queries_closed_form():
    """With Q = 0 every visible score is 0: lse = log(#visible), O = mean of visible V."""
    groups, _, _, vis = read_visibility_fixture()
    T = vis.shape[0]
    rng = np.random.default_rng(8)
    q = np.zeros((T, 2, 4))
    k = rng.standard_normal((T, 1, 4))
    v = rng.standard_normal((T, 1, 4))
    res = repeated_prefix_attention(groups, q, k, v)
    cnt = vis.sum(axis=1)
    for h in range(2):
        assert np.allclose(res["lse"][h], np.log(cnt), atol=1e-14, rtol=0)
        mean_v = (vis.astype(float) @ v[:, 0]) / cnt[:, None]
        assert np.allclose(res["o"][:, h], mean_v, atol=1e-14, rtol=0)


# ---------------------------------------------------------------- brute force

def _brute_force_forward(groups, q, k, v, scale):
    """Pure-Python loops: per baseline sequence [P; R_i], per head, per row."""
    T, hq, d = q.shape
    rep = hq // k.shape[1]
    o = [[None] * hq for _ in range(T)]
    lse = [[None] * T for _ in range(hq)]
    t = 0
    for P, rs in groups:
        pre = list(range(t, t + P))
        t += P
        for r in rs:
            seq = pre + list(range(t, t + r))
            t += r
            for h in range(hq):
                for a, row in enumerate(seq):
                    scores = []
                    for key in seq[:a + 1]:
                        s = 0.0
                        for c in range(d):
                            s += float(q[row, h, c]) * float(k[key, h // rep, c])
                        scores.append(s * scale)
                    m = max(scores)
                    w = [math.exp(s - m) for s in scores]
                    z = sum(w)
                    out = [0.0] * d
                    for wi, key in zip(w, seq[:a + 1]):
                        for c in range(d):
                            out[c] += wi / z * float(v[key, h // rep, c])
                    o[row][h] = out
                    lse[h][row] = m + math.log(z)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("groups,hq,hkv", [
    ([(4, [3, 2, 5])], 2, 2),
    ([(3, [2, 0, 1]), (0, [2, 1]), (1, [1, 1])], 4, 2),
    ([(0, [4]), (6, [1])], 3, 1),
])
def test_brute_force_forward(groups, hq, hkv):
    _, T = member_sequences(groups)
    assert T <= 40
    q, k, v, _ = _rand(T, hq, hkv, 3)
    res = repeated_prefix_attention(groups, q, k, v, scale=0.7)
    o, lse = _brute_force_forward(groups, q, k, v, 0.7)
    assert np.allclose(res["o"], o, atol=1e-12, rtol=0)
    assert np.allclose(res["lse"], lse, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- finite differences

def test_finite_differences():
    groups = [(3, [2, 0, 3]), (2, [1, 2])]
    _, T = member_sequences(groups)
    rng = np.random.default_rng(11)
    q, k, v, do = _rand(T, 4, 2, 3, rng)
    scale = 0.6
    res = repeated_prefix_attention(groups, q, k, v, do, scale=scale)

    def loss(q_, k_, v_):
        return float((repeated_prefix_attention(groups, q_, k_, v_, scale=scale)["o"] * do).sum())

    h = 1e-6
    for name, arr, grad in (("q", q, res["dq"]), ("k", k, res["dk"]), ("v", v, res["dv"])):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
            ap = arr.copy(); ap[idx] += h
            am = arr.copy(); am[idx] -= h
            args_p = {"q": q, "k": k, "v": v}; args_p[name] = ap
            args_m = {"q": q, "k": k, "v": v}; args_m[name] = am
            fd = (loss(**{kk + "_": vv for kk, vv in args_p.items()})
                  - loss(**{kk + "_": vv for kk, vv in args_m.items()})) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-7 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


# ---------------------------------------------------------------- torch, dense packed mask

def _closed_form_mask(groups):
    """M(q,k) = same group and k <= q and (k in the prefix or same response as q)."""
    members, T = member_sequences(groups)
    seg = np.full(T, -1)      # response id of a row, -1 for prefix rows
    grp = np.full(T, -1)
    for mi, m in enumerate(members):
        grp[m.prefix[0]:m.prefix[1]] = m.group
        grp[m.resp[0]:m.resp[1]] = m.group
        seg[m.resp[0]:m.resp[1]] = mi
    qi = np.arange(T)[:, None]
    kj = np.arange(T)[None, :]
    same_group = grp[:, None] == grp[None, :]
    return same_group & (kj <= qi) & ((seg[None, :] == -1) | (seg[None, :] == seg[:, None]))


def _torch_dense(groups, q, k, v, do, scale):
    mask = torch.from_numpy(_closed_form_mask(groups))
    rep = q.shape[1] // k.shape[1]
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    kk = tk.repeat_interleave(rep, dim=1)
    vv = tv.repeat_interleave(rep, dim=1)
    s = torch.einsum("qhd,khd->hqk", tq, kk) * scale
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    o = torch.einsum("hqk,khd->qhd", torch.softmax(s, dim=-1), vv)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return (o.detach().numpy(), lse.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(),
            tv.grad.numpy())


@pytest.mark.parametrize("groups,hq,hkv,d", [
    ([(6, [3, 4, 1, 2])], 2, 2, 4),
    ([(5, [2, 0, 3]), (0, [3, 1]), (4, [1]), (2, [2, 2, 2])], 4, 2, 3),
    ([(9, [1, 5])], 6, 2, 5),
])
def test_matches_dense_masked_torch(groups, hq, hkv, d):
    _, T = member_sequences(groups)
    rng = np.random.default_rng(T)
    q, k, v, do = _rand(T, hq, hkv, d, rng)
    scale = 1.0 / math.sqrt(d)
    res = repeated_prefix_attention(groups, q, k, v, do)
    o, lse, dq, dk, dv = _torch_dense(groups, q, k, v, do, scale)
    for a, b in ((res["o"], o), (res["lse"], lse), (res["dq"], dq), (res["dk"], dk),
                 (res["dv"], dv)):
        assert np.allclose(a, b, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- library special cases

def _sdpa_causal(q, k, v, do):
    """torch SDPA (causal) in fp64 on one sequence [L, H, d], with autograd."""
    rep = q.shape[1] // k.shape[1]
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.transpose(0, 1), tk.repeat_interleave(rep, 1).transpose(0, 1),
        tv.repeat_interleave(rep, 1).transpose(0, 1), is_causal=True).transpose(0, 1)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def test_single_member_is_causal_attention():
    groups = [(7, [5])]
    q, k, v, do = _rand(12, 4, 2, 8)
    res = repeated_prefix_attention(groups, q, k, v, do)
    o, dq, dk, dv = _sdpa_causal(q, k, v, do)
    for a, b in ((res["o"], o), (res["dq"], dq), (res["dk"], dk), (res["dv"], dv)):
        assert np.allclose(a, b, atol=1e-12, rtol=0)


def test_empty_prefix_is_independent_causal():
    groups = [(0, [4, 6, 1])]
    q, k, v, do = _rand(11, 2, 1, 8)
    res = repeated_prefix_attention(groups, q, k, v, do)
    for a, b in ((0, 4), (4, 10), (10, 11)):
        o, dq, dk, dv = _sdpa_causal(q[a:b], k[a:b], v[a:b], do[a:b])
        assert np.allclose(res["o"][a:b], o, atol=1e-12, rtol=0)
        assert np.allclose(res["dq"][a:b], dq, atol=1e-12, rtol=0)
        assert np.allclose(res["dk"][a:b], dk, atol=1e-12, rtol=0)
        assert np.allclose(res["dv"][a:b], dv, atol=1e-12, rtol=0)


def test_single_sequence_helpers_match_sdpa_across_row_blocks(monkeypatch):
    """The row blocking of the one-sequence helpers (several blocks plus a tail)."""
    import oracle.attention as oa
    monkeypatch.setattr(oa, "ROW_BLOCK", 7)
    L = 30
    q, k, v, do = _rand(L, 1, 1, 6)
    o, lse = causal_attention_forward(q[:, 0], k[:, 0], v[:, 0], 1 / math.sqrt(6))
    dq, dk, dv = causal_attention_backward(q[:, 0], k[:, 0], v[:, 0], do[:, 0], 1 / math.sqrt(6))
    o2, dq2, dk2, dv2 = _sdpa_causal(q, k, v, do)
    for a, b in ((o, o2[:, 0]), (dq, dq2[:, 0]), (dk, dk2[:, 0]), (dv, dv2[:, 0])):
        assert np.allclose(a, b, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- invariants

def test_invariants():
    groups = [(6, [3, 5, 2]), (3, [4, 1])]
    members, T = member_sequences(groups)
    vis = _closed_form_mask(groups)
    rng = np.random.default_rng(5)
    q, k, v, do = _rand(T, 2, 1, 4, rng)
    res = repeated_prefix_attention(groups, q, k, v, do)
    # convex hull of visible V rows, coordinate-wise
    for r in range(T):
        vv = v[vis[r], 0]
        assert np.all(res["o"][r] >= vv.min(axis=0) - 1e-12)
        assert np.all(res["o"][r] <= vv.max(axis=0) + 1e-12)
    # lse >= max visible score
    scale = 0.5
    for h in range(2):
        s = scale * q[:, h] @ k[:, 0].T
        s[~vis] = -np.inf
        assert np.all(res["lse"][h] >= s.max(axis=1) - 1e-12)
    # adding one vector to every key leaves outputs and gradients unchanged
    shift = rng.standard_normal(4)
    res2 = repeated_prefix_attention(groups, q, k + shift, v, do)
    for key in ("o", "dq", "dk", "dv"):
        assert np.allclose(res[key], res2[key], atol=1e-11, rtol=0)
    # linearity in the upstream gradient
    do2 = rng.standard_normal(do.shape)
    r_a = repeated_prefix_attention(groups, q, k, v, do2)
    r_b = repeated_prefix_attention(groups, q, k, v, 2.0 * do - 3.0 * do2)
    for key in ("dq", "dk", "dv"):
        assert np.allclose(r_b[key], 2.0 * res[key] - 3.0 * r_a[key], atol=1e-11, rtol=0)
    # exact sum rules: sum over a group's keys of dK is 0; of dV is the sum of dO
    t = 0
    for P, rs in groups:
        n = P + sum(rs)
        assert np.allclose(res["dk"][t:t + n].sum(axis=0), 0.0, atol=1e-12)
        assert np.allclose(res["dv"][t:t + n, 0].sum(axis=0), do[t:t + n].sum(axis=(0, 1)),
                           atol=1e-12)
        t += n
    assert np.isclose((res["dq"] * q).sum(), (res["dk"] * k).sum(), atol=1e-12)


def test_permuting_responses_permutes_outputs():
    P, rs = 4, [3, 1, 5]
    groups = [(P, rs)]
    T = P + sum(rs)
    q, k, v, do = _rand(T, 2, 2, 3)
    res = repeated_prefix_attention(groups, q, k, v, do)
    starts = np.cumsum([P] + rs[:-1])
    perm = [2, 0, 1]
    rows = list(range(P)) + [r for i in perm for r in range(starts[i], starts[i] + rs[i])]
    rows = np.array(rows)
    res_p = repeated_prefix_attention([(P, [rs[i] for i in perm])], q[rows], k[rows], v[rows],
                                      do[rows])
    for key in ("o", "dq", "dk", "dv"):
        assert np.allclose(res_p[key], res[key][rows], atol=1e-12, rtol=0)
    assert np.allclose(res_p["lse"], res["lse"][:, rows], atol=1e-12, rtol=0)


# ---------------------------------------------------------------- pair counts

def test_pair_counts_match_brute_force_masks():
    rng = np.random.default_rng(3)
    for _ in range(20):
        groups = [(int(rng.integers(0, 6)), [int(x) for x in rng.integers(0, 5, size=rng.integers(1, 4))])
                  for _ in range(int(rng.integers(1, 4)))]
        pg, pb = pair_counts(groups)
        assert pg == int(_closed_form_mask(groups).sum())
        members, _ = member_sequences(groups)
        brute_b = sum(sum(1 for a in range(m.rows.size) for b in range(a + 1)) for m in members)
        assert pb == brute_b


def test_pair_ratio_tends_to_one_over_g():
    """Lemma 2.2 (Pith review, "Core claim"): cost -> 1/G of the baseline as P/R grows."""
    for G in (4, 8, 16):
        ratios = [pair_counts([(P, [64] * G)]) for P in (10 ** 3, 10 ** 5, 10 ** 7)]
        r = [a / b for a, b in ratios]
        assert r[0] > r[1] > r[2] > 1.0 / G
        assert abs(r[2] - 1.0 / G) < 1e-4


# ---------------------------------------------------------------- sampled-row variants

def test_sampled_rows_match_full_oracle():
    groups = [(9, [4, 0, 7]), (5, [3, 6])]
    members, T = member_sequences(groups)
    rng = np.random.default_rng(21)
    q, k, v, do = _rand(T, 4, 2, 5, rng)
    full = repeated_prefix_attention(groups, q, k, v, do)
    rows = list(range(T))
    s = repeated_prefix_rows(groups, q, k, v, do, rows, range(4))
    assert np.allclose(s["o"], full["o"], atol=1e-13, rtol=0)
    assert np.allclose(s["lse"], full["lse"], atol=1e-13, rtol=0)
    assert np.allclose(s["dq"], full["dq"], atol=1e-13, rtol=0)
    kr = repeated_prefix_key_rows(groups, q, k, v, do, rows, [0, 1])
    assert np.allclose(kr["dk"], full["dk"], atol=1e-13, rtol=0)
    assert np.allclose(kr["dv"], full["dv"], atol=1e-13, rtol=0)


def test_kv_head_subset_matches_full():
    groups = [(6, [2, 3])]
    q, k, v, do = _rand(11, 6, 3, 4)
    full = repeated_prefix_attention(groups, q, k, v, do)
    sub = repeated_prefix_attention(groups, q, k, v, do, kv_heads=[1])
    assert list(sub["q_heads"]) == [2, 3]
    assert np.allclose(sub["o"], full["o"][:, 2:4], atol=0, rtol=0)
    assert np.allclose(sub["dk"][:, 0], full["dk"][:, 1], atol=0, rtol=0)


def test_sampled_rows_forward_only_matches_full_oracle():
    """do=None (forward only) gives the same O and LSE as the full oracle."""
    from oracle.attention import repeated_prefix_rows
    groups = [(5, [3, 0, 4]), (2, [2])]
    rng = np.random.default_rng(21)
    members, T = member_sequences(groups)
    q = rng.standard_normal((T, 2, 8)); k = rng.standard_normal((T, 1, 8))
    v = rng.standard_normal((T, 1, 8)); do = rng.standard_normal((T, 2, 8))
    full = repeated_prefix_attention(groups, q, k, v, do)
    rows = list(range(T))
    fwd = repeated_prefix_rows(groups, q, k, v, None, rows, [0, 1])
    assert np.allclose(fwd["o"], full["o"][rows][:, [0, 1]], atol=1e-12, rtol=0)
    assert np.allclose(fwd["lse"], full["lse"][[0, 1]][:, rows], atol=1e-12, rtol=0)
    assert not fwd["dq"].any()


def test_key_rows_across_row_blocks_match_full_oracle(monkeypatch):
    """Several key rows of one member sequence share its softmax rows, which
    then start at the earliest of them and span several row blocks."""
    import oracle.attention as oa
    monkeypatch.setattr(oa, "ROW_BLOCK", 3)
    groups = [(11, [6, 0, 9]), (4, [7])]
    members, T = member_sequences(groups)
    rng = np.random.default_rng(33)
    q, k, v, do = _rand(T, 4, 2, 5, rng)
    full = repeated_prefix_attention(groups, q, k, v, do)
    rows = [0, 5, 10, 12, 16, 17, 25, 26, 30, 33]
    kr = repeated_prefix_key_rows(groups, q, k, v, do, rows, [1, 0])
    assert np.allclose(kr["dk"], full["dk"][rows][:, [1, 0]], atol=1e-13, rtol=0)
    assert np.allclose(kr["dv"], full["dv"][rows][:, [1, 0]], atol=1e-13, rtol=0)
    # partial sums over a partition of the members add up to the same rows
    parts = [repeated_prefix_key_rows(groups, q, k, v, do, rows, [1, 0], members=m)
             for m in ([0, 3], [1], [2])]
    assert np.allclose(sum(x["dk"] for x in parts), kr["dk"], atol=1e-13, rtol=0)
    assert np.allclose(sum(x["dv"] for x in parts), kr["dv"], atol=1e-13, rtol=0)


def test_member_subsets_sum_to_full():
    """members=: outputs on the listed members' rows equal the full oracle's,
    and the gradients over a partition of the members add up to the full
    gradients (the prefix gradient is a sum over copies, Lemma 2.1)."""
    groups = [(8, [3, 5, 0, 4]), (0, [6]), (5, [2, 2])]
    members, T = member_sequences(groups)
    rng = np.random.default_rng(44)
    q, k, v, do = _rand(T, 4, 2, 6, rng)
    full = repeated_prefix_attention(groups, q, k, v, do)
    parts = [[0, 2, 5], [1, 4], [3, 6]]
    acc = {n: np.zeros_like(full[n]) for n in ("dq", "dk", "dv")}
    for part in parts:
        sub = repeated_prefix_attention(groups, q, k, v, do, members=part)
        rows = np.concatenate([members[i].rows for i in part])
        assert np.allclose(sub["o"][rows], full["o"][rows], atol=1e-13, rtol=0)
        assert np.allclose(sub["lse"][:, rows], full["lse"][:, rows], atol=1e-13, rtol=0)
        for n in acc:
            acc[n] += sub[n]
    for n in acc:
        assert np.allclose(acc[n], full[n], atol=1e-13, rtol=0), n
