"""Host-side tests of libpg_attn: exports, planner, validation.  No GPU.

The library is loaded and called only through entry points that touch no
device: pg_pack_host (the planner into host memory), the size functions, and
argument validation, which rejects the call before anything is enqueued.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import shared_prefix_grouped_amd as pg
from oracle.attention import member_sequences, pair_counts, position_ids
from tests.golden_io import read_visibility_fixture

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "pg_attn.h")


def _lib():
    try:
        return pg.lib()
    except pg.LibraryNotBuilt as e:  # the build step must have run first
        pytest.fail(str(e))


def test_exports_every_declared_function():
    L = _lib()
    text = open(HEADER).read()
    names = set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(pg_\w+)\s*\(", text, flags=re.M))
    assert {"pg_pack", "pg_attn_fwd", "pg_attn_bwd", "pg_pack_host", "pg_rope"} <= names
    for n in sorted(names):
        assert hasattr(L, n), f"{n} declared in pg_attn.h but not exported"
    assert set(pg.EXPORTED) == names


def _visibility_from_plan(plan):
    """Key k is visible to query q iff k <= q < row_hi[k]; check row_lo gives the same."""
    T = plan["total_rows"]
    hi = plan["row_hi"]
    q = np.arange(T)[:, None]
    k = np.arange(T)[None, :]
    vis_hi = (k <= q) & (q < hi[None, :])
    # row_lo form: k in [group start, prefix end) or [row_lo[q], q], within the group
    gs, pe = plan["group_start"], plan["prefix_end"]
    grp = np.searchsorted(gs, np.arange(T), side="right") - 1
    g0 = gs[grp][:, None]
    p_end = pe[grp][:, None]
    vis_lo = (k >= g0) & (k <= q) & ((k < p_end) | (k >= plan["row_lo"][:, None]))
    assert np.array_equal(vis_hi, vis_lo)
    return vis_hi


def test_planner_matches_golden_fixture():
    groups, positions, pairs, vis = read_visibility_fixture()
    plan = pg.pg_pack_host(groups, 4, 2, 64)
    assert np.array_equal(plan["pos_ids"], positions)
    assert (plan["pairs"], plan["baseline_pairs"]) == pairs
    assert np.array_equal(_visibility_from_plan(plan), vis)


def _random_groups(rng, max_groups=4, max_p=300, max_r=200, max_g=6):
    return [(int(rng.integers(0, max_p)),
             [int(x) for x in rng.integers(0, max_r, size=int(rng.integers(1, max_g + 1)))])
            for _ in range(int(rng.integers(1, max_groups + 1)))]


def _tile_chunks(plan, q0, q1, g0, pe, chunk=64):
    """64-key chunks a forward / dQ work item over rows [q0, q1) streams: the
    prefix keys [g0, min(pe, q1)), then [max(pe, row_lo[q0]), q1)."""
    a = min(pe, q1) - g0
    b = q1 - max(pe, int(plan["row_lo"][q0]))
    return (-(-a // chunk) if a > 0 else 0) + (-(-b // chunk) if b > 0 else 0)


def test_query_tiles_ordered_by_streamed_chunks():
    """At the headline shape the short last tile of the group (few rows, but
    every prefix chunk) is among the first work items, not the last."""
    from workloads import attention_workloads
    w = attention_workloads()["bf16_gqa_g16_p8192"]
    groups = [(g.prefix_len, list(g.resp_lens)) for g in w.groups]
    plan = pg.pg_pack_host(groups, 32, 8, 128)
    T = plan["total_rows"]
    tiles = [tuple(int(x) for x in t) for t in plan["q_tiles"]]
    last = [i for i, t in enumerate(tiles) if t[1] == T]
    assert len(last) == 1 and tiles[last[0]][1] - tiles[last[0]][0] < pg.PG_TILE_Q
    chunks = [_tile_chunks(plan, *t) for t in tiles]
    assert chunks == sorted(chunks, reverse=True)
    assert last[0] < len(tiles) // 2


def test_planner_random_layouts():
    rng = np.random.default_rng(99)
    for _ in range(30):
        groups = _random_groups(rng)
        plan = pg.pg_pack_host(groups, 8, 2, 128)
        _, T = member_sequences(groups)
        assert plan["total_rows"] == T
        assert np.array_equal(plan["pos_ids"], position_ids(groups))
        assert (plan["pairs"], plan["baseline_pairs"]) == pair_counts(groups)
        vis = _visibility_from_plan(plan)
        assert int(vis.sum()) == plan["pairs"]
        # query tiles partition the rows, stay in one group, and are ordered
        # by the key chunks their work item streams, then by visible pairs
        covered = np.zeros(T, dtype=int)
        costs = []
        for q0, q1, g0, pe in plan["q_tiles"]:
            assert 0 < q1 - q0 <= pg.PG_TILE_Q
            covered[q0:q1] += 1
            gi = np.searchsorted(plan["group_start"], q0, side="right") - 1
            assert plan["group_start"][gi] == g0 and plan["prefix_end"][gi] == pe
            assert q1 <= plan["group_start"][gi + 1]
            costs.append((_tile_chunks(plan, q0, q1, g0, pe), int(vis[q0:q1].sum())))
        assert np.all(covered == 1)
        assert costs == sorted(costs, reverse=True)
        # key tiles partition the rows; q_end bounds every query that sees them
        covered[:] = 0
        costs = []
        for k0, k1, qend, pe in plan["kv_tiles"]:
            assert 0 < k1 - k0 <= pg.PG_TILE_KV
            covered[k0:k1] += 1
            seen_by = np.nonzero(vis[:, k0:k1].any(axis=1))[0]
            assert seen_by.min() >= k0 and seen_by.max() < qend
            assert seen_by.max() == qend - 1
            costs.append(int(vis[:, k0:k1].sum()))
        assert np.all(covered == 1)
        assert costs == sorted(costs, reverse=True)
        _check_kv_items(plan, vis, rep=4)


def _check_kv_items(plan, vis, rep):
    """The dK/dV work list covers every visible (query, key) pair exactly once.

    Uncut key tiles appear whole; a cut tile's pieces split [k0, q_end) at
    32-row query blocks, number their float partial slots consecutively in
    query order, each hold at least 32 (query head, block) steps, and are
    listed in kv_sums; the list is ordered by decreasing walk length (32-row
    blocks), then visible pairs."""
    items, sums = plan["kv_items"], plan["kv_sums"]
    tiles = {(int(k0), int(k1)): int(qend) for k0, k1, qend, _ in plan["kv_tiles"]}
    assert np.all(items[:, 5:] == 0)
    by_tile = {}
    costs = []
    for k0, k1, qa, qb, part, *_ in items.tolist():
        assert (k0, k1) in tiles and k0 <= qa < qb <= tiles[(k0, k1)]
        by_tile.setdefault((k0, k1), []).append((qa, qb, part))
        costs.append((-(-(qb - qa) // 32), int(vis[qa:qb, k0:k1].sum())))
    assert costs == sorted(costs, reverse=True)
    assert sum(c[1] for c in costs) == plan["pairs"]
    assert set(by_tile) == set(tiles)
    cut = {(int(k0), int(k1)): (int(first), int(n)) for k0, k1, first, n in sums}
    used = []
    for key, pieces in by_tile.items():
        k0, qend = key[0], tiles[key]
        pieces.sort()
        if key not in cut:
            assert pieces == [(k0, qend, -1)]
            continue
        first, n = cut[key]
        assert n >= 2 and len(pieces) == n
        assert [pc[2] for pc in pieces] == list(range(first, first + n))
        assert pieces[0][0] == k0 and pieces[-1][1] == qend
        for (qa, qb, _), nxt in zip(pieces, pieces[1:] + [None]):
            assert (qa - k0) % 32 == 0
            assert -(-(qb - qa) // 32) * rep >= 32
            if nxt is not None:
                assert nxt[0] == qb
        used += [pc[2] for pc in pieces]
    assert sorted(used) == list(range(plan["num_kv_parts"]))


def test_short_prefix_tiles_are_cut_and_long_ones_are_not():
    """A 40-row prefix shared by 24 responses holds most of the dK/dV work in
    one key tile: it is cut.  At the headline shape (8192-row prefix, 16
    responses) every tile is under the per-unit mean and stays whole."""
    groups = [(40, [97] * 24)]
    plan = pg.pg_pack_host(groups, 8, 2, 128)
    _, T = member_sequences(groups)
    vis = _visibility_from_plan(plan)
    assert len(plan["kv_sums"]) == 1 and plan["kv_sums"][0, :2].tolist() == [0, 128]
    _check_kv_items(plan, vis, rep=4)
    from workloads import attention_workloads
    w = attention_workloads()["bf16_gqa_g16_p8192"]
    plan = pg.pg_pack_host([(g.prefix_len, list(g.resp_lens)) for g in w.groups],
                           w.num_q_heads, w.num_kv_heads, w.head_dim)
    assert plan["num_kv_parts"] == 0 and len(plan["kv_items"]) == plan["num_kv_tiles"]


def test_full_size_layouts_plan():
    from workloads import attention_workloads
    for w in attention_workloads().values():
        groups = [(g.prefix_len, list(g.resp_lens)) for g in w.groups]
        plan = pg.pg_pack_host(groups, w.num_q_heads, w.num_kv_heads, w.head_dim)
        assert plan["total_rows"] == w.total_rows
        assert (plan["pairs"], plan["baseline_pairs"]) == pair_counts(groups)


def test_empty_and_degenerate_layouts():
    plan = pg.pg_pack_host([], 2, 2, 64)
    assert plan["total_rows"] == 0 and plan["num_q_tiles"] == 0
    plan = pg.pg_pack_host([(0, [0, 0])], 2, 2, 64)
    assert plan["total_rows"] == 0 and plan["num_q_tiles"] == 0 and plan["num_kv_tiles"] == 0
    plan = pg.pg_pack_host([(0, [1])], 2, 1, 128)
    assert plan["total_rows"] == 1 and plan["pairs"] == 1


# ---------------------------------------------------------------- validation

def _groups(groups, hq=4, hkv=2, d=64):
    return pg._groups_struct(groups, hq, hkv, d)


@pytest.mark.parametrize("groups,hq,hkv,d,status", [
    ([(-1, [3])], 2, 2, 64, pg.PG_ERR_INVALID_ARG),
    ([(4, [])], 2, 2, 64, pg.PG_ERR_INVALID_ARG),
    ([(4, [2, -3])], 2, 2, 64, pg.PG_ERR_INVALID_ARG),
    ([(4, [2])], 3, 2, 64, pg.PG_ERR_INVALID_ARG),
    ([(4, [2])], 2, 0, 64, pg.PG_ERR_INVALID_ARG),
    ([(4, [2])], 2, 2, 96, pg.PG_ERR_UNSUPPORTED),
    ([(4, [2])], 2, 2, 256, pg.PG_ERR_UNSUPPORTED),
])
def test_pack_rejects_bad_descriptions(groups, hq, hkv, d, status):
    L = _lib()
    g, keep = _groups(groups, hq, hkv, d)
    assert L.pg_pack_buffer_size(ctypes.byref(g)) == 0
    buf = np.zeros(1024, dtype=np.int32)
    desc = pg.PgDesc()
    st = L.pg_pack_host(ctypes.byref(g), buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes, None,
                        ctypes.byref(desc))
    assert st == status
    assert L.pg_last_error()


def test_pack_rejects_small_buffer_and_overflow():
    L = _lib()
    g, keep = _groups([(100, [50, 50])])
    need = L.pg_pack_buffer_size(ctypes.byref(g))
    buf = np.zeros(need // 4, dtype=np.int32)
    desc = pg.PgDesc()
    st = L.pg_pack_host(ctypes.byref(g), buf.ctypes.data_as(ctypes.c_void_p), need - 16, None,
                        ctypes.byref(desc))
    assert st == pg.PG_ERR_WORKSPACE
    g, keep = _groups([(2 ** 30, [2 ** 30])])
    st = L.pg_pack_host(ctypes.byref(g), buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes, None,
                        ctypes.byref(desc))
    assert st == pg.PG_ERR_INVALID_ARG
    # device pack validates before touching the device
    st = L.pg_pack(ctypes.byref(g), None, 0, None, ctypes.byref(desc), None)
    assert st == pg.PG_ERR_INVALID_ARG


def _host_desc(groups=((5, [3, 2]),), hq=4, hkv=2, d=64):
    L = _lib()
    g, keep = _groups(list(groups), hq, hkv, d)
    need = L.pg_pack_buffer_size(ctypes.byref(g))
    buf = np.zeros(need // 4 + 4, dtype=np.int32)
    desc = pg.PgDesc()
    assert L.pg_pack_host(ctypes.byref(g), buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes, None,
                          ctypes.byref(desc)) == pg.PG_OK
    return desc, buf


def test_fwd_bwd_validate_before_launch():
    """Bad arguments are rejected on the host; nothing is launched (no GPU here)."""
    L = _lib()
    desc, buf = _host_desc()
    p = ctypes.c_void_p(4096)       # aligned, never dereferenced: validation fails first
    bad = ctypes.c_void_p(4096 + 4)  # misaligned
    f = ctypes.c_float(0.0)
    assert L.pg_attn_fwd(None, pg.PG_BF16, f, p, p, p, p, p, None) == pg.PG_ERR_INVALID_ARG
    assert L.pg_attn_fwd(ctypes.byref(desc), 7, f, p, p, p, p, p, None) == pg.PG_ERR_UNSUPPORTED
    assert L.pg_attn_fwd(ctypes.byref(desc), pg.PG_BF16, f, None, p, p, p, p, None) == pg.PG_ERR_INVALID_ARG
    assert "q" in L.pg_last_error().decode()
    assert L.pg_attn_fwd(ctypes.byref(desc), pg.PG_BF16, f, p, bad, p, p, p, None) == pg.PG_ERR_INVALID_ARG
    assert "aligned" in L.pg_last_error().decode()
    ws = L.pg_attn_bwd_workspace_size(ctypes.byref(desc), pg.PG_BF16)
    rows = -(-desc.num_q_heads * desc.total_rows * 4 // 16) * 16
    assert ws == max(16, 2 * rows + desc.num_kv_parts * desc.num_kv_heads * 2 * pg.PG_TILE_KV
                     * desc.head_dim * 4)
    assert L.pg_attn_bwd_workspace_size(ctypes.byref(desc), pg.PG_F32) == 16
    cut, _cbuf = _host_desc(((40, [97] * 24),), 8, 2, 128)  # one cut prefix tile
    assert cut.num_kv_parts >= 2
    rows_c = -(-8 * cut.total_rows * 4 // 16) * 16
    assert (L.pg_attn_bwd_workspace_size(ctypes.byref(cut), pg.PG_BF16)
            == 2 * rows_c + cut.num_kv_parts * 2 * 2 * pg.PG_TILE_KV * 128 * 4)
    args = [p] * 10
    st = L.pg_attn_bwd(ctypes.byref(desc), pg.PG_BF16, f, *args, ws - 1, None)
    assert st == pg.PG_ERR_WORKSPACE
    args[9] = None
    st = L.pg_attn_bwd(ctypes.byref(desc), pg.PG_BF16, f, *args, ws, None)
    assert st == pg.PG_ERR_INVALID_ARG
    # a descriptor with an unsupported head size is refused
    d2 = pg.PgDesc.from_buffer_copy(desc)
    d2.head_dim = 80
    assert L.pg_attn_fwd(ctypes.byref(d2), pg.PG_BF16, f, p, p, p, p, p, None) == pg.PG_ERR_UNSUPPORTED
    d2.head_dim = 64
    d2.num_kv_heads = 3
    assert L.pg_attn_fwd(ctypes.byref(d2), pg.PG_BF16, f, p, p, p, p, p, None) == pg.PG_ERR_INVALID_ARG
    # rope argument checks
    assert L.pg_rope(ctypes.byref(desc), pg.PG_BF16, p, 2, 63, p, ctypes.c_float(1e4), 0, None) == pg.PG_ERR_INVALID_ARG
    assert L.pg_rope(ctypes.byref(desc), pg.PG_BF16, p, 2, 64, p, ctypes.c_float(0.5), 0, None) == pg.PG_ERR_INVALID_ARG
    assert L.pg_rope(ctypes.byref(desc), pg.PG_BF16, p, 2, 64, None, ctypes.c_float(1e4), 0, None) == pg.PG_ERR_INVALID_ARG


def test_empty_batch_calls_are_no_ops():
    L = _lib()
    desc, buf = _host_desc(groups=((0, [0]),))
    assert desc.total_rows == 0
    f = ctypes.c_float(0.0)
    assert L.pg_attn_fwd(ctypes.byref(desc), pg.PG_BF16, f, None, None, None, None, None, None) == pg.PG_OK
    assert L.pg_attn_bwd(ctypes.byref(desc), pg.PG_BF16, f, *([None] * 10), 0, None) == pg.PG_OK


def test_row_gather_plan_and_validation():
    """prefix_before is the running count of prefix rows; pg_pack_rows /
    pg_unpack_rows reject bad row sizes, NULL or misaligned buffers on the
    host, allow NULL for a part with no rows, and do nothing on an empty batch."""
    groups = [(5, [3, 2]), (0, [4]), (7, [0, 1])]
    plan = pg.pg_pack_host(groups, 4, 2, 64)
    assert plan["prefix_before"].tolist() == [0, 5, 5, 12]
    assert plan["total_prefix_rows"] == 12
    L = _lib()
    desc, buf = _host_desc(tuple(groups))
    p = ctypes.c_void_p(4096)
    odd = ctypes.c_void_p(4096 + 4)
    for fn in (L.pg_pack_rows, L.pg_unpack_rows):
        assert fn(ctypes.byref(desc), p, p, p, 0, None) == pg.PG_ERR_INVALID_ARG
        assert fn(ctypes.byref(desc), p, p, p, 6, None) == pg.PG_ERR_INVALID_ARG
        assert "multiple of 4" in L.pg_last_error().decode()
        assert fn(None, p, p, p, 16, None) == pg.PG_ERR_INVALID_ARG
    assert L.pg_pack_rows(ctypes.byref(desc), p, p, odd, 16, None) == pg.PG_ERR_INVALID_ARG
    assert "aligned" in L.pg_last_error().decode()
    assert L.pg_pack_rows(ctypes.byref(desc), None, p, p, 16, None) == pg.PG_ERR_INVALID_ARG
    assert "prefix_rows" in L.pg_last_error().decode()
    assert L.pg_unpack_rows(ctypes.byref(desc), p, p, None, 16, None) == pg.PG_ERR_INVALID_ARG
    assert "resp_rows" in L.pg_last_error().decode()
    assert L.pg_unpack_rows(ctypes.byref(desc), None, p, p, 16, None) == pg.PG_ERR_INVALID_ARG
    # 4-byte rows need only 4-byte alignment
    no_pre, _b2 = _host_desc(((0, [3]),))
    empty, _b3 = _host_desc(((0, [0]),))
    assert L.pg_pack_rows(ctypes.byref(empty), None, None, None, 8, None) == pg.PG_OK
    assert L.pg_unpack_rows(ctypes.byref(empty), None, None, None, 4, None) == pg.PG_OK
    assert no_pre.total_prefix_rows == 0 and no_pre.total_rows == 3


def test_head_sizes_and_validation():
    """Log-probability head: workspace size from the descriptor, and bad
    arguments rejected on the host before anything is enqueued."""
    L = _lib()
    desc, buf = _host_desc(((5, [3, 0, 4]), (0, [2, 1]), (1, [1])))
    assert desc.num_scored == 9
    n, V, dm = 9, 1000, 64
    a256 = lambda x: -(-x // 256) * 256
    nvt = -(-V // 256)  # vocab tiles of the logits kernels
    n64, V64 = -(-n // 64) * 64, -(-V // 64) * 64  # row strides: whole 128-byte lines
    g = n * V64 * 2  # gradient of the logits, bf16; the logits are never stored
    gt = a256(g) + V * n64 * 2  # and its transpose
    hp = a256(gt) + n * dm * 2
    hpt = a256(hp) + dm * n64 * 2
    wt = a256(hpt) + dm * V64 * 2
    dhp = a256(wt) + n * dm * 4
    pm = a256(dhp) + nvt * n * 4
    ps = a256(pm) + nvt * n * 4
    want = a256(ps)
    assert L.pg_logprob_workspace_size(ctypes.byref(desc), V, dm) == want
    assert L.pg_logprob_workspace_size(ctypes.byref(desc), 0, dm) == 0
    assert L.pg_logprob_workspace_size(ctypes.byref(desc), V, 12) == 0
    # the tile kernels address each operand with 32-bit byte offsets: a 4 GiB
    # transposed weight (vocab rounded up to a multiple of 64) is refused
    assert L.pg_logprob_workspace_size(ctypes.byref(desc), (1 << 20) - 63, 2048) == 0
    assert L.pg_logprob_workspace_size(ctypes.byref(desc), (1 << 20) - 64, 2048) > 0
    p = ctypes.c_void_p(4096)
    assert L.pg_logprob_fwd(ctypes.byref(desc), p, p, V, dm, p, p, p, p, want - 1,
                            None) == pg.PG_ERR_WORKSPACE
    assert L.pg_logprob_fwd(ctypes.byref(desc), None, p, V, dm, p, p, p, p, want,
                            None) == pg.PG_ERR_INVALID_ARG
    assert "hidden" in L.pg_last_error().decode()
    assert L.pg_logprob_bwd(ctypes.byref(desc), p, p, V, dm, p, p, p, p, None, p, want,
                            None) == pg.PG_ERR_INVALID_ARG
    assert "dweight" in L.pg_last_error().decode()
    assert L.pg_grpo_loss(ctypes.byref(desc), p, None, p, p, None) == pg.PG_ERR_INVALID_ARG


def test_python_binding_has_no_fallback():
    """The binding imports neither the oracle nor any CPU path."""
    src = open(pg.__file__).read()
    assert "oracle" not in src.replace("no fallback", "")
    assert "import numpy" in src  # numpy only marshals host arrays for the planner


def test_bf16_backward_bound_is_per_walk_not_per_tensor():
    """The bf16 dK/dV kernel bases its Q/dO descriptors at each work item's
    first query row, so the 32-bit limit applies to one walk (at most one
    group), not to the whole tensor: the repeated-prefix layout of the
    two-group workload (295,228 rows, 64 query heads: q is 4.8 GB) plans walks
    of at most 33,280 rows, while one 300,000-row group is refused before
    anything is launched."""
    L = _lib()
    rep_groups = tuple((32768, [512]) for _ in range(8)) + tuple(
        (2048, [r]) for r in (1523, 1939, 1821, 1110, 1934, 2003, 1991, 283))
    desc, _buf = _host_desc(rep_groups, 64, 8, 128)
    assert desc.total_rows == 295228
    assert desc.total_rows * 64 * 128 * 2 > 2 ** 32
    items = np.frombuffer(ctypes.string_at(desc.kv_items, desc.num_kv_items * 32), dtype=np.int32)
    items = items.reshape(-1, 8)
    assert desc.max_walk_rows == int((items[:, 3] - items[:, 2]).max()) == 33280
    assert (desc.max_walk_rows + 32) * 64 * 128 * 2 < 2 ** 32
    big, _bbuf = _host_desc(((299000, [1000]),), 64, 8, 128)
    p = ctypes.c_void_p(4096)
    args = [p] * 10
    ws = L.pg_attn_bwd_workspace_size(ctypes.byref(big), pg.PG_BF16)
    st = L.pg_attn_bwd(ctypes.byref(big), pg.PG_BF16, ctypes.c_float(0.0), *args, ws, None)
    assert st == pg.PG_ERR_UNSUPPORTED
    assert "4 GiB" in L.pg_last_error().decode()


def test_binding_checks_backward_outputs_before_launch():
    """Caller-supplied dq / dk / dv / workspace of the wrong shape, type,
    layout or size are refused by the binding before the library is called
    (CPU tensors: a wrong one never reaches a kernel)."""
    import torch
    desc, _buf = _host_desc(((5, [3]),), 2, 1, 64)
    batch = pg.PackedBatch(desc, None, None, ((5, (3,)),))
    T, hq, hkv, d = 8, 2, 1, 64
    q = torch.zeros((T, hq, d), dtype=torch.bfloat16)
    kv = torch.zeros((T, hkv, d), dtype=torch.bfloat16)
    lse = torch.zeros((hq, T), dtype=torch.float32)
    bad = {"dq": torch.zeros((T, hq + 1, d), dtype=torch.bfloat16),
           "dk": torch.zeros((T, hkv, d), dtype=torch.float32),
           "dv": torch.zeros((T, hkv, 2 * d), dtype=torch.bfloat16)[:, :, ::2]}
    for name, t in bad.items():
        with pytest.raises(pg.PgError) as e:
            pg.pg_attn_bwd(batch, q, kv, kv, q, lse, q, **{name: t})
        assert name in str(e.value)
    with pytest.raises(pg.PgError) as e:
        pg.pg_attn_bwd(batch, q, kv, kv, q, lse, q, workspace=torch.zeros(4, dtype=torch.uint8))
    assert e.value.status == pg.PG_ERR_WORKSPACE


def test_binding_checks_head_vectors_before_launch():
    """lse / dlogp of the head backward and logp / advantages of the loss that
    are short, of the wrong type or strided are refused by the binding before
    the library is called (CPU tensors: a wrong one never reaches a kernel)."""
    import torch
    desc, _buf = _host_desc(((5, [3, 2]),), 2, 1, 64)
    batch = pg.PackedBatch(desc, None, None, ((5, (3, 2)),))
    n, T, dm, V = desc.num_scored, desc.total_rows, 16, 11
    assert n > 0
    h = torch.zeros((T, dm), dtype=torch.bfloat16)
    W = torch.zeros((V, dm), dtype=torch.bfloat16)
    tok = torch.zeros(T, dtype=torch.int32)
    good = torch.zeros(n, dtype=torch.float32)
    for bad in (torch.zeros(n - 1), torch.zeros(n, dtype=torch.float64), torch.zeros(2 * n)[::2]):
        for which in ("lse", "dlogp"):
            args = {"lse": good, "dlogp": good}
            args[which] = bad
            with pytest.raises(pg.PgError) as e:
                pg.pg_logprob_bwd(batch, h, W, tok, args["lse"], args["dlogp"])
            assert which in str(e.value)
    with pytest.raises(pg.PgError) as e:
        pg.pg_grpo_loss(batch, good, torch.zeros(desc.num_resp - 1))
    assert "advantages" in str(e.value)
    with pytest.raises(pg.PgError) as e:
        pg.pg_grpo_loss(batch, torch.zeros(n - 1), torch.zeros(desc.num_resp))
    assert "logp" in str(e.value)
