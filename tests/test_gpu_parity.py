"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Element by element on seeded inputs at sizes the oracle finishes in seconds
(several tiles, ragged tails, varlen batches, GQA), on whole kv-head subsets of
the full-size 32-head workload, and on sampled rows plus exact identities at
the full sizes of the two largest workloads, launched exactly as the
benchmark launches them.
"""
import math
import zlib
import os
import sys
import time

import numpy as np
import pytest

from oracle.attention import (repeated_prefix_attention, repeated_prefix_key_rows,
                              repeated_prefix_rows)
from tests.parity import compare, rel_fro, run_gpu, segment_rows, to_np
from workloads import attention_workloads, draw_attention_inputs, scaled_down

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import shared_prefix_grouped_amd as pg
    pg.lib()  # fails loudly if the library is not built


def _groups_of(w):
    return [(g.prefix_len, list(g.resp_lens)) for g in w.groups]


def _full_check(w, kv_heads=None):
    groups = _groups_of(w)
    arrs = draw_attention_inputs(w)
    dtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
    _say(f"[parity] {w.name}: groups={[(p, len(r)) for p, r in groups]} T={w.total_rows} "
         f"heads={w.num_q_heads}/{w.num_kv_heads} d={w.head_dim} dtype={w.dtype}")
    out = run_gpu(groups, w.num_q_heads, w.num_kv_heads, w.head_dim, arrs, dtype)
    t0 = time.time()
    ref = repeated_prefix_attention(groups, arrs["q"], arrs["k"], arrs["v"], arrs["do"],
                                    kv_heads=kv_heads)
    qh, kh = ref["q_heads"], ref["kv_heads"]
    gpu = {"o": to_np(out["o"])[:, qh], "lse": to_np(out["lse"])[qh],
           "dq": to_np(out["dq"])[:, qh], "dk": to_np(out["dk"])[:, kh],
           "dv": to_np(out["dv"])[:, kh]}
    msgs = compare(gpu, ref, w.dtype, prefix_mask=segment_rows(groups))
    _say(f"[parity] {w.name}: oracle {time.time() - t0:.1f}s; " + "; ".join(msgs))


def test_fp32_config_full():
    _full_check(attention_workloads()["fp32_g4_p64"])


SMALL = [
    ("ragged_gqa", [(200, [37, 0, 130, 64, 1])], 4, 2, 128),
    ("varlen_p0_d64", [(0, [70, 1, 33]), (129, [128, 5]), (1, [1])], 2, 2, 64),
    ("tile_multiples", [(256, [128, 128])], 2, 1, 128),
    ("single_member", [(300, [77])], 2, 2, 128),
    ("gqa8_long_ragged", [(700, [300, 17, 450, 2, 64, 129])], 8, 1, 128),
    ("many_short", [(65, [3] * 40)], 2, 2, 64),
    ("empty_prefix_only_resp", [(0, [257])], 2, 2, 128),
    ("prefix_only", [(333, [0, 0])], 4, 4, 64),
    # short prefix shared by many responses: the prefix key tiles are cut into
    # pieces whose float partial sums are added by a second kernel
    ("short_prefix_g24", [(40, [97] * 24)], 8, 2, 128),
    ("short_prefix_2groups_d64", [(150, [61] * 20 + [3, 200]), (7, [33] * 12)], 4, 2, 64),
    ("short_prefix_mha", [(130, [50] * 40)], 2, 2, 128),
]


@pytest.mark.parametrize("name,groups,hq,hkv,d", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_layouts(name, groups, hq, hkv, d, dtype):
    w = scaled_down(name, groups, dtype, hq, hkv, d, seed=zlib.crc32(name.encode()) % 1000)
    _full_check(w)


def test_bf16_g8_p4096_full_size_kv_subset():
    """Full-size 32-head workload on the GPU; oracle on kv heads 0 and 31, every row."""
    _full_check(attention_workloads()["bf16_g8_p4096"], kv_heads=[0, 31])


def _sample_rows(groups, rng, extra=12):
    rows = set()
    t = 0
    for p, rs in groups:
        if p:
            rows.update([t, t + p - 1, t + min(p - 1, 127), t + min(p - 1, 128)])
        s = t + p
        for r in rs:
            if r:
                rows.update([s, s + r - 1])
            s += r
        t = s
    T = t
    rows.update(int(x) for x in rng.integers(0, T, size=extra))
    return sorted(rows)


def _identities(groups, hq, hkv, arrs, out):
    """Exact identities of softmax-attention gradients, per group and kv head.

    sum_k dV[k] = sum over the group's rows and the kv head's query heads of dO;
    sum_k dK[k] = 0;  <dQ, Q> = <dK, K>.  Returned as relative deviations.  The
    inner-product sums cancel heavily (|sum| is ~1e-3 of sum |terms|), so their
    deviation is scaled by sum |dQ * Q| + sum |dK * K|: an element-wise
    relative error e in the gradients moves the difference by at most e times
    that."""
    rep = hq // hkv
    dq, dk, dv = to_np(out["dq"]), to_np(out["dk"]), to_np(out["dv"])
    res = []
    t = 0
    for p, rs in groups:
        n = p + sum(rs)
        sl = slice(t, t + n)
        for hk in range(hkv):
            hs = slice(hk * rep, (hk + 1) * rep)
            lhs = dv[sl, hk].sum(axis=0)
            rhs = arrs["do"][sl, hs].astype(np.float64).sum(axis=(0, 1))
            e_v = np.linalg.norm(lhs - rhs) / np.linalg.norm(rhs)
            e_k = np.linalg.norm(dk[sl, hk].sum(axis=0)) / np.linalg.norm(dk[sl, hk])
            tq = dq[sl, hs] * arrs["q"][sl, hs]
            tk = dk[sl, hk] * arrs["k"][sl, hk]
            e_qk = abs(float(tq.sum()) - float(tk.sum())) / float(np.abs(tq).sum() + np.abs(tk).sum())
            res.append((e_v, e_k, e_qk))
        t += n
    return np.array(res)


def _sampled_check(w, q_heads, kv_heads, key_rows_fn):
    groups = _groups_of(w)
    t0 = time.time()
    arrs = draw_attention_inputs(w)
    _say(f"[parity] {w.name}: inputs drawn in {time.time() - t0:.1f}s, T={w.total_rows}")
    out = run_gpu(groups, w.num_q_heads, w.num_kv_heads, w.head_dim, arrs, torch.bfloat16)
    rng = np.random.default_rng(w.seed + 100)
    rows = _sample_rows(groups, rng)
    t0 = time.time()
    ref = repeated_prefix_rows(groups, arrs["q"], arrs["k"], arrs["v"], arrs["do"], rows, q_heads)
    o = to_np(out["o"][rows][:, q_heads])
    lse = to_np(out["lse"][q_heads][:, rows])
    dq = to_np(out["dq"][rows][:, q_heads])
    e_o = float(np.max(np.abs(o - ref["o"])))
    e_l = float(np.max(np.abs(lse - ref["lse"])))
    e_q = rel_fro(dq, ref["dq"])
    _say(f"[parity] {w.name}: {len(rows)} rows x {len(q_heads)} heads, oracle "
         f"{time.time() - t0:.1f}s: o max-abs {e_o:.3e}, lse max-abs {e_l:.3e}, dq rel-fro {e_q:.3e}")
    assert e_o <= 2e-2 and e_l <= 1e-3 and e_q <= 1e-2
    krows = key_rows_fn(groups)
    t0 = time.time()
    kref = repeated_prefix_key_rows(groups, arrs["q"], arrs["k"], arrs["v"], arrs["do"], krows,
                                    kv_heads)
    dk = to_np(out["dk"][krows][:, kv_heads])
    dv = to_np(out["dv"][krows][:, kv_heads])
    e_k, e_v = rel_fro(dk, kref["dk"]), rel_fro(dv, kref["dv"])
    _say(f"[parity] {w.name}: {len(krows)} key rows, oracle {time.time() - t0:.1f}s: "
         f"dk rel-fro {e_k:.3e}, dv rel-fro {e_v:.3e}")
    assert e_k <= 1e-2 and e_v <= 1e-2
    ids = _identities(groups, w.num_q_heads, w.num_kv_heads, arrs, out)
    _say(f"[parity] {w.name}: identity max deviations dV-sum {ids[:, 0].max():.2e}, "
         f"dK-sum {ids[:, 1].max():.2e}, <dQ,Q>-<dK,K> {ids[:, 2].max():.2e}")
    assert ids[:, 0].max() <= 1e-2 and ids[:, 1].max() <= 2e-2 and ids[:, 2].max() <= 1e-2
    return out


def _resp_key_rows(groups, per_group=4):
    rows = []
    t = 0
    for p, rs in groups:
        s = t + p
        for i, r in enumerate(rs):
            if r and i < per_group:
                rows += [s, s + r - 1]
            s += r
        t = s
    return rows


def test_bf16_gqa_g16_p8192_full_size_sampled():
    w = attention_workloads()["bf16_gqa_g16_p8192"]

    def keys(groups):
        p = groups[0][0]
        return [p - 1] + _resp_key_rows(groups, 3)

    _sampled_check(w, q_heads=[0, 13, 31], kv_heads=[0, 7], key_rows_fn=keys)


def test_bf16_varlen_2groups_full_size_sampled():
    w = attention_workloads()["bf16_varlen_2groups"]

    def keys(groups):
        (p0, r0), (p1, r1) = groups
        g1 = p0 + sum(r0)
        return [g1 + p1 - 1] + _resp_key_rows(groups, 2)

    _sampled_check(w, q_heads=[0, 63], kv_heads=[3], key_rows_fn=keys)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_deterministic_bitwise(dtype, d):
    # both groups' prefix key tiles are cut for bf16 (partial sums + second kernel)
    w = scaled_down("det", [(1000, [333, 12, 700]), (64, [500])], dtype, 8, 2, d, seed=5)
    groups = _groups_of(w)
    arrs = draw_attention_inputs(w)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    a = run_gpu(groups, 8, 2, d, arrs, tdt)
    junk = torch.randn(1 << 22, device="cuda")  # perturb allocator and stream state
    b = run_gpu(groups, 8, 2, d, arrs, tdt)
    del junk
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[key], b[key]), key


def test_repeated_prefix_layout_through_same_kernels():
    """Each [P; R_i] packed as its own group gives the grouped results (Lemma 2.1)."""
    P, rs = 300, [45, 200, 1, 130]
    w = scaled_down("rep", [(P, rs)], "bf16", 4, 2, 128, seed=9)
    arrs = draw_attention_inputs(w)
    grouped = run_gpu([(P, rs)], 4, 2, 128, arrs, torch.bfloat16)
    # build the repeated-prefix layout: prefix copied before every response
    starts = np.cumsum([P] + rs[:-1])
    idx = np.concatenate([np.concatenate([np.arange(P), np.arange(s, s + r)])
                          for s, r in zip(starts, rs)])
    rep = {k: v[idx] for k, v in arrs.items()}
    rep["do"] = rep["do"].copy()
    off = 0
    for r in rs:  # split the prefix upstream gradient over the copies (exact: G = 4)
        rep["do"][off:off + P] /= len(rs)
        off += P + r
    base = run_gpu([(P, [r]) for r in rs], 4, 2, 128, rep, torch.bfloat16)
    g = {k: to_np(grouped[k]) for k in ("o", "dq", "dk", "dv")}
    b = {k: to_np(base[k]) for k in ("o", "dq", "dk", "dv")}
    off = 0
    acc = {k: np.zeros_like(g[k][:P]) for k in ("dq", "dk", "dv")}
    for s, r in zip(starts, rs):
        assert np.max(np.abs(b["o"][off:off + P] - g["o"][:P])) <= 2e-2
        assert np.max(np.abs(b["o"][off + P:off + P + r] - g["o"][s:s + r])) <= 2e-2
        for k in acc:
            acc[k] += b[k][off:off + P]
            assert rel_fro(b[k][off + P:off + P + r], g[k][s:s + r]) <= 1e-2 or r == 0
        off += P + r
    for k in acc:
        assert rel_fro(acc[k], g[k][:P]) <= 1e-2, k


def test_autograd_function_matches_direct_calls():
    import shared_prefix_grouped_amd as pg
    w = scaled_down("ag", [(150, [20, 90])], "bf16", 4, 1, 64, seed=3)
    groups = _groups_of(w)
    arrs = draw_attention_inputs(w)
    batch = pg.pg_pack(groups, 4, 1, 64)
    q, k, v, do = (torch.from_numpy(arrs[n]).cuda().to(torch.bfloat16) for n in ("q", "k", "v", "do"))
    q.requires_grad_(True); k.requires_grad_(True); v.requires_grad_(True)
    o = pg.grouped_attention(q, k, v, batch)
    o.backward(do)
    o2, lse = pg.pg_attn_fwd(batch, q.detach(), k.detach(), v.detach())
    dq, dk, dv = pg.pg_attn_bwd(batch, q.detach(), k.detach(), v.detach(), o2, lse, do)
    assert torch.equal(o, o2)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)


def test_empty_batch():
    import shared_prefix_grouped_amd as pg
    batch = pg.pg_pack([(0, [0, 0])], 2, 2, 64)
    q = torch.empty((0, 2, 64), device="cuda", dtype=torch.bfloat16)
    o, lse = pg.pg_attn_fwd(batch, q, q.clone(), q.clone())
    dq, dk, dv = pg.pg_attn_bwd(batch, q, q.clone(), q.clone(), o, lse, q.clone())
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 64) and dq.shape == (0, 2, 64)


def test_bf16_tensors_over_2gib():
    """Q and dO of 2.3 GB each (17 copies of a 16384-row prefix + 256-row
    response, GQA 32/8): the dK/dV kernel's 32-bit buffer offsets pass 2^31.
    The last group, whose rows all lie past 2 GiB, is checked against the
    oracle on sampled query rows and on key rows near the prefix end and in
    the response (each seen by at most 257 query rows)."""
    import shared_prefix_grouped_amd as pg
    P, R, G, hq, hkv, d = 16384, 256, 17, 32, 8, 128
    groups = [(P, [R])] * G
    T = G * (P + R)
    assert (T - (P + R)) * hq * d * 2 > 2 ** 31  # the last group starts past 2 GiB
    _say(f"[parity] over-2GiB: T={T}, q bytes {T * hq * d * 2 / 2**30:.2f} GiB")
    gen = torch.Generator(device="cuda").manual_seed(21)
    q, k, v, do = (torch.randn((T, h, d), generator=gen, device="cuda").to(torch.bfloat16)
                   for h in (hq, hkv, hkv, hq))
    batch = pg.pg_pack(groups, hq, hkv, d)
    o, lse = pg.pg_attn_fwd(batch, q, k, v)
    dq, dk, dv = pg.pg_attn_bwd(batch, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    g0 = T - (P + R)
    sub = {n: x[g0:].float().cpu().numpy() for n, x in (("q", q), ("k", k), ("v", v), ("do", do))}
    one = [(P, [R])]
    rows = [0, 1, P - 1, P, P + 1, P + R - 1, 5000, 12345]
    heads = [0, 31]
    ref = repeated_prefix_rows(one, sub["q"], sub["k"], sub["v"], sub["do"], rows, heads)
    gr = [g0 + r for r in rows]
    e_o = float(np.max(np.abs(to_np(o[gr][:, heads]) - ref["o"])))
    e_l = float(np.max(np.abs(to_np(lse[heads][:, gr]) - ref["lse"])))
    e_q = rel_fro(to_np(dq[gr][:, heads]), ref["dq"])
    _say(f"[parity] over-2GiB: o {e_o:.3e}, lse {e_l:.3e}, dq rel-fro {e_q:.3e}")
    assert e_o <= 2e-2 and e_l <= 1e-3 and e_q <= 1e-2
    krows = [P - 2, P - 1, P, P + 100, P + R - 1]
    kref = repeated_prefix_key_rows(one, sub["q"], sub["k"], sub["v"], sub["do"], krows, [0, 7])
    gk = [g0 + r for r in krows]
    e_k = rel_fro(to_np(dk[gk][:, [0, 7]]), kref["dk"])
    e_v = rel_fro(to_np(dv[gk][:, [0, 7]]), kref["dv"])
    _say(f"[parity] over-2GiB: dk rel-fro {e_k:.3e}, dv rel-fro {e_v:.3e}")
    assert e_k <= 1e-2 and e_v <= 1e-2
