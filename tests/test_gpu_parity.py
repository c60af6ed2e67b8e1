"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Element by element on seeded inputs at sizes the oracle finishes in seconds
(several tiles, ragged tails, varlen batches, GQA), on whole kv heads of the
full-size workloads (every row, every query head of the kv head), and on the
longest prefix-key walks of the two-group workload, launched exactly as the
benchmark launches them.  The oracle's member sequences run side by side in
a thread pool at the full sizes.
"""
import math
import zlib
import os
import sys
import time

import numpy as np
import pytest

from oracle.attention import (member_sequences, repeated_prefix_attention,
                              repeated_prefix_key_rows, repeated_prefix_rows)
from tests.parity import compare, host_threads, pool_sum, rel_fro, run_gpu, segment_rows, to_np
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
    # several plan tiles per group, long walks over many staged chunks (float32
    # path: 32-row chunks, 8-row sub-tiles), a second group after a long one
    ("multi_tile_two_groups", [(1000, [333, 12, 700]), (64, [500])], 8, 2, 128),
    # 16 query heads on one kv head: every dK/dV walk sums 16 heads
    ("gqa16_d64", [(190, [70, 5, 130])], 16, 1, 64),
]


@pytest.mark.parametrize("name,groups,hq,hkv,d", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_layouts(name, groups, hq, hkv, d, dtype):
    w = scaled_down(name, groups, dtype, hq, hkv, d, seed=zlib.crc32(name.encode()) % 1000)
    _full_check(w)


def test_fp32_at_headline_shape_kv_head0():
    """The float32 path at the GQA 32/8, G=16, P=8192 shape (T=15139): walks of
    hundreds of staged chunks and thousands of workgroups; every row of kv head
    0 (its 4 query heads) against the oracle, to the float32 tolerance."""
    hw = attention_workloads()["bf16_gqa_g16_p8192"]
    w = scaled_down("fp32_gqa_g16_p8192", _groups_of(hw), "f32", hw.num_q_heads,
                    hw.num_kv_heads, hw.head_dim, seed=11)
    _full_check(w, kv_heads=[0])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sharp_softmax_custom_scale(dtype):
    """softmax_scale = 8/sqrt(d) instead of 1/sqrt(d): scores of standard
    deviation about 8, so a row's running maximum keeps jumping by more than
    the forward's lazy-rescale threshold and probabilities span many orders of
    magnitude; the scale reaches every kernel through the C ABI."""
    groups = [(300, [130, 7, 64])]
    w = scaled_down("sharp_softmax", groups, dtype, 4, 2, 128, seed=21)
    arrs = draw_attention_inputs(w)
    scale = 8.0 / math.sqrt(128)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = run_gpu(groups, 4, 2, 128, arrs, tdt, scale=scale)
    ref = repeated_prefix_attention(groups, arrs["q"], arrs["k"], arrs["v"], arrs["do"], scale=scale)
    gpu = {"o": to_np(out["o"]), "lse": to_np(out["lse"]), "dq": to_np(out["dq"]),
           "dk": to_np(out["dk"]), "dv": to_np(out["dv"])}
    msgs = compare(gpu, ref, dtype, prefix_mask=segment_rows(groups))
    _say(f"[parity] sharp softmax ({dtype}, scale {scale:.3f}): " + "; ".join(msgs))


# Head configurations beyond the ones above: kv head counts that are multiples
# of 8 take the XCD-aware block-to-work maps (one or two kv heads per XCD, 1-3
# query heads per kv head); the others the plain maps, with odd GQA ratios.
HEADS = [
    ("xcd_rep3", [(150, [90, 7, 61])], 24, 8, 128),
    ("xcd_two_kv_per_xcd", [(97, [64, 130]), (33, [5])], 32, 16, 64),
    ("xcd_mha16", [(70, [40, 41])], 16, 16, 128),
    ("rep3_plain", [(200, [33, 120, 1])], 12, 4, 128),
    ("rep5_plain", [(66, [100, 20])], 10, 2, 64),
    ("odd_kv3", [(129, [31, 64])], 6, 3, 128),
]


@pytest.mark.parametrize("name,groups,hq,hkv,d", HEADS, ids=[s[0] for s in HEADS])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_configurations(name, groups, hq, hkv, d, dtype):
    _full_check(scaled_down(name, groups, dtype, hq, hkv, d, seed=zlib.crc32(name.encode()) % 1000))


def _many_tiny_groups():
    rng = np.random.default_rng(77)
    return [(int(rng.integers(0, 6)), [int(r) for r in rng.integers(0, 6, size=int(rng.integers(1, 4)))])
            for _ in range(300)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_long_response_short_prefix(dtype):
    """One 6000-row response behind a 64-row prefix: the own-segment part of
    every walk dominates (forward and dQ rows stream up to 94 response key
    chunks; dK/dV response key tiles walk thousands of rows)."""
    w = scaled_down("long_response", [(64, [6000, 3])], dtype, 8, 2, 128, seed=41)
    _full_check(w, kv_heads=[1])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_many_tiny_groups(dtype):
    """300 groups of 0-5 prefix rows and 1-3 responses of 0-5 rows: tiles
    and key tiles far smaller than a workgroup's rows, many group borders."""
    w = scaled_down("many_tiny_groups", _many_tiny_groups(), dtype, 4, 2, 64, seed=42)
    _full_check(w)


def _random_layout(seed):
    """A seeded random varlen batch: 1-3 groups, prefixes 0-400 rows, 1-12
    responses of 0-200 rows each, a random head configuration and d."""
    rng = np.random.default_rng(1000 + seed)
    groups = []
    for _ in range(int(rng.integers(1, 4))):
        P = int(rng.integers(0, 401))
        rs = [int(r) for r in rng.integers(0, 201, size=int(rng.integers(1, 13)))]
        if P + sum(rs) == 0:
            rs[0] = 1
        groups.append((P, rs))
    hq, hkv = [(2, 1), (4, 2), (8, 2), (4, 4), (16, 2)][int(rng.integers(0, 5))]
    d = (64, 128)[int(rng.integers(0, 2))]
    return groups, hq, hkv, d


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_random_layouts(seed, dtype):
    groups, hq, hkv, d = _random_layout(seed)
    _full_check(scaled_down(f"random_{seed}", groups, dtype, hq, hkv, d, seed=seed))


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
    """Exact identities of softmax-attention gradients, per group and kv head,
    as relative deviations: sum_k dV[k] = the sum of dO over the group's rows
    and the kv head's query heads, and sum_k dK[k] = 0.  (Neither sum cancels
    much, so bf16 rounding of the stored gradients stays far below 1e-2.)"""
    rep = hq // hkv
    dk, dv = to_np(out["dk"]), to_np(out["dv"])
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
            res.append((e_v, e_k))
        t += n
    return np.array(res)


def _oracle_whole_kv_head(groups, arrs, hk):
    """The full oracle restricted to kv head hk, its member sequences computed
    side by side (each a partial sum; prefix O and LSE from member 0)."""
    members, _ = member_sequences(groups)

    def one(i):
        r = repeated_prefix_attention(groups, arrs["q"], arrs["k"], arrs["v"], arrs["do"],
                                      kv_heads=[hk], members=[i])
        m = members[i]
        if m.member != 0:  # the prefix outputs come from each group's member 0
            r["o"][m.prefix[0]:m.prefix[1]] = 0.0
            r["lse"][:, m.prefix[0]:m.prefix[1]] = 0.0
        return r

    return pool_sum(one, range(len(members)))


def _gpu_kv_head(out, rows, hk, rep):
    """GPU results on packed rows `rows` (a slice) for kv head hk and its query heads."""
    qh = slice(hk * rep, (hk + 1) * rep)
    return {"o": to_np(out["o"][rows, qh]), "lse": to_np(out["lse"][qh, rows]),
            "dq": to_np(out["dq"][rows, qh]), "dk": to_np(out["dk"][rows, hk:hk + 1]),
            "dv": to_np(out["dv"][rows, hk:hk + 1])}


@pytest.fixture(scope="module")
def headline_run():
    """GQA 32/8, G = 16, P = 8192 workload on the GPU, as the benchmark runs it."""
    w = attention_workloads()["bf16_gqa_g16_p8192"]
    groups = _groups_of(w)
    arrs = draw_attention_inputs(w)
    _say(f"[parity] {w.name}: T={w.total_rows}, host threads {host_threads()}")
    out = run_gpu(groups, w.num_q_heads, w.num_kv_heads, w.head_dim, arrs, torch.bfloat16)
    return w, groups, arrs, out


@pytest.mark.parametrize("hk", [0, 7])
def test_bf16_gqa_g16_p8192_full_size_whole_kv_head(headline_run, hk):
    """Every row (prefix and all 16 responses) of O, LSE, dQ, dK, dV for kv
    head hk and its 4 query heads against the full oracle: every prefix key
    row's whole walk (Lemma 2.1's sum over the 16 copies) is compared."""
    w, groups, arrs, out = headline_run
    rep = w.num_q_heads // w.num_kv_heads
    t0 = time.time()
    ref = _oracle_whole_kv_head(groups, arrs, hk)
    gpu = _gpu_kv_head(out, slice(0, w.total_rows), hk, rep)
    msgs = compare(gpu, ref, "bf16", prefix_mask=segment_rows(groups))
    _say(f"[parity] {w.name} kv head {hk}: oracle {time.time() - t0:.1f}s; " + "; ".join(msgs))


def test_bf16_gqa_g16_p8192_full_size_identities(headline_run):
    w, groups, arrs, out = headline_run
    ids = _identities(groups, w.num_q_heads, w.num_kv_heads, arrs, out)
    _say(f"[parity] {w.name}: identity max deviations dV-sum {ids[:, 0].max():.2e}, "
         f"dK-sum {ids[:, 1].max():.2e}")
    assert ids[:, 0].max() <= 1e-2 and ids[:, 1].max() <= 2e-2


@pytest.fixture(scope="module")
def varlen_run():
    """Two-group GQA 64/8 workload (P = 32768 x 8 responses of 512, then
    P = 2048 x 8 ragged responses) on the GPU, as the benchmark runs it."""
    w = attention_workloads()["bf16_varlen_2groups"]
    groups = _groups_of(w)
    t0 = time.time()
    arrs = draw_attention_inputs(w)
    _say(f"[parity] {w.name}: inputs drawn in {time.time() - t0:.1f}s, T={w.total_rows}")
    out = run_gpu(groups, w.num_q_heads, w.num_kv_heads, w.head_dim, arrs, torch.bfloat16)
    return w, groups, arrs, out


def _group_slice(groups, gi):
    t = 0
    for j, (p, rs) in enumerate(groups):
        n = p + sum(rs)
        if j == gi:
            return slice(t, t + n)
        t += n
    raise IndexError(gi)


def test_bf16_varlen_2groups_group1_whole_kv_head(varlen_run):
    """Group 1 (P = 2048, responses 128..2048) in full for kv head 5 and its 8
    query heads.  Groups are independent, so the oracle runs on group 1's rows
    alone."""
    w, groups, arrs, out = varlen_run
    rep = w.num_q_heads // w.num_kv_heads
    sl = _group_slice(groups, 1)
    sub = {n: a[sl] for n, a in arrs.items()}
    t0 = time.time()
    ref = _oracle_whole_kv_head([groups[1]], sub, 5)
    gpu = _gpu_kv_head(out, sl, 5, rep)
    msgs = compare(gpu, ref, "bf16", prefix_mask=segment_rows([groups[1]]))
    _say(f"[parity] {w.name} group 1 kv head 5: oracle {time.time() - t0:.1f}s; " + "; ".join(msgs))


def test_bf16_varlen_2groups_group0_prefix_key_rows(varlen_run):
    """dK/dV of group 0's prefix key rows at key-tile boundaries near the
    prefix end and in the middle of the prefix, for kv heads 0 and 7 (8 query
    heads each): each is the sum over the 8 copies of the 32768-row prefix,
    walked over every later prefix row and all 8 responses.  Plus the first
    and last rows of each response as keys."""
    w, groups, arrs, out = varlen_run
    sl = _group_slice(groups, 0)
    p0, r0 = groups[0]
    sub = {n: a[sl] for n, a in arrs.items()}
    krows = [30719, 30720, 32511, 32512, 32639, 32640, 32767]
    s = p0
    for r in r0:
        krows += [s, s + r - 1]
        s += r
    kv = [0, 7]
    n_mem = len(r0)
    t0 = time.time()
    parts = {}

    def one(t):
        return t, repeated_prefix_key_rows([groups[0]], sub["q"], sub["k"], sub["v"], sub["do"],
                                           krows, [t[0]], members=[t[1]])

    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    tasks = [(hk, i) for hk in kv for i in range(n_mem)]
    with threadpool_limits(1), ThreadPoolExecutor(max_workers=host_threads()) as ex:
        for (hk, i), r in ex.map(one, tasks):
            acc = parts.setdefault(hk, {"dk": 0.0, "dv": 0.0})
            acc["dk"] = acc["dk"] + r["dk"][:, 0]
            acc["dv"] = acc["dv"] + r["dv"][:, 0]
    g0 = sl.start
    for hk in kv:
        dk = to_np(out["dk"][[g0 + r for r in krows], hk])
        dv = to_np(out["dv"][[g0 + r for r in krows], hk])
        npre = sum(r < p0 for r in krows)
        e = {"dk prefix": rel_fro(dk[:npre], parts[hk]["dk"][:npre]),
             "dv prefix": rel_fro(dv[:npre], parts[hk]["dv"][:npre]),
             "dk response": rel_fro(dk[npre:], parts[hk]["dk"][npre:]),
             "dv response": rel_fro(dv[npre:], parts[hk]["dv"][npre:])}
        _say(f"[parity] {w.name} group 0 kv head {hk}, {len(krows)} key rows: oracle "
             f"{time.time() - t0:.1f}s; " + "; ".join(f"{k} rel-fro {v:.3e}" for k, v in e.items()))
        assert all(v <= 1e-2 for v in e.values()), e


def test_bf16_varlen_2groups_group0_sampled_query_rows(varlen_run):
    """O, LSE and dQ of sampled group-0 query rows (prefix start and end, tile
    boundaries, every response's first and last row, random rows) for query
    heads 0 and 63."""
    w, groups, arrs, out = varlen_run
    sl = _group_slice(groups, 0)
    sub = {n: a[sl] for n, a in arrs.items()}
    rng = np.random.default_rng(w.seed + 100)
    rows = _sample_rows([groups[0]], rng)
    heads = [0, 63]
    t0 = time.time()
    ref = repeated_prefix_rows([groups[0]], sub["q"], sub["k"], sub["v"], sub["do"], rows, heads)
    o = to_np(out["o"][rows][:, heads])
    lse = to_np(out["lse"][heads][:, rows])
    dq = to_np(out["dq"][rows][:, heads])
    e_o = float(np.max(np.abs(o - ref["o"])))
    e_l = float(np.max(np.abs(lse - ref["lse"])))
    e_q = rel_fro(dq, ref["dq"])
    _say(f"[parity] {w.name} group 0: {len(rows)} rows x {len(heads)} heads, oracle "
         f"{time.time() - t0:.1f}s: o max-abs {e_o:.3e}, lse max-abs {e_l:.3e}, dq rel-fro {e_q:.3e}")
    assert e_o <= 2e-2 and e_l <= 1e-3 and e_q <= 1e-2


def test_bf16_varlen_2groups_full_size_identities(varlen_run):
    w, groups, arrs, out = varlen_run
    ids = _identities(groups, w.num_q_heads, w.num_kv_heads, arrs, out)
    _say(f"[parity] {w.name}: identity max deviations dV-sum {ids[:, 0].max():.2e}, "
         f"dK-sum {ids[:, 1].max():.2e}")
    assert ids[:, 0].max() <= 1e-2 and ids[:, 1].max() <= 2e-2


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


def test_bf16_tensors_over_4gib():
    """Q and dO of 4.5 GB each (33 copies of a 16384-row prefix + 256-row
    response, GQA 32/8): the dK/dV kernel bases its buffer descriptors at
    each work item's first query row, so walks past 2^31 and 2^32 bytes of Q
    use the same 32-bit offsets.  The last group, whose rows all lie past
    4 GiB, is checked against the oracle on sampled query rows and on key
    rows near the prefix end and in the response (each seen by at most 257
    query rows)."""
    import shared_prefix_grouped_amd as pg
    P, R, G, hq, hkv, d = 16384, 256, 33, 32, 8, 128
    groups = [(P, [R])] * G
    T = G * (P + R)
    assert (T - (P + R)) * hq * d * 2 > 2 ** 32  # the last group starts past 4 GiB
    _say(f"[parity] over-4GiB: T={T}, q bytes {T * hq * d * 2 / 2**30:.2f} GiB")
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
    _say(f"[parity] over-4GiB: o {e_o:.3e}, lse {e_l:.3e}, dq rel-fro {e_q:.3e}")
    assert e_o <= 2e-2 and e_l <= 1e-3 and e_q <= 1e-2
    krows = [P - 2, P - 1, P, P + 100, P + R - 1]
    kref = repeated_prefix_key_rows(one, sub["q"], sub["k"], sub["v"], sub["do"], krows, [0, 7])
    gk = [g0 + r for r in krows]
    e_k = rel_fro(to_np(dk[gk][:, [0, 7]]), kref["dk"])
    e_v = rel_fro(to_np(dv[gk][:, [0, 7]]), kref["dv"])
    _say(f"[parity] over-4GiB: dk rel-fro {e_k:.3e}, dv rel-fro {e_v:.3e}")
    assert e_k <= 1e-2 and e_v <= 1e-2
