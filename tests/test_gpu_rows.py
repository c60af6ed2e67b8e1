"""Row gather / scatter on the GPU (pg_pack_rows, pg_unpack_rows): the packed
order [P; R_1; ...; R_G] per group (skillsmp.com "prefix-grouper-grpo",
"Step 3: Restructure Input Format", without padding), bit for bit against the
order built here with plain slicing, for 4-, 8-, 12-byte and multi-KiB rows,
empty prefixes and responses, and more groups than the kernel stages in LDS.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _packed_order(groups, pre, resp):
    """Concatenate slices: each group's prefix rows, then its responses' rows."""
    parts, po, ro = [], 0, 0
    for p, rs in groups:
        parts.append(pre[po:po + p])
        po += p
        n = sum(rs)
        parts.append(resp[ro:ro + n])
        ro += n
    return torch.cat(parts) if parts else pre[:0]


LAYOUTS = [
    ("mixed", [(5, [3, 0, 2]), (0, [4]), (7, [0, 1]), (300, [129, 64])]),
    ("prefix_only", [(33, [0, 0])]),
    ("responses_only", [(0, [17, 5]), (0, [1])]),
    ("many_groups", None),  # 1500 groups: offsets read from global memory
]
SHAPES = [("i32", torch.int32, ()), ("i64", torch.int64, ()), ("bf16x6", torch.bfloat16, (6,)),
          ("bf16_heads", torch.bfloat16, (32, 128)), ("f32_model", torch.float32, (2048,))]


@pytest.mark.parametrize("name,groups", LAYOUTS, ids=[x[0] for x in LAYOUTS])
@pytest.mark.parametrize("sname,dtype,tail", SHAPES, ids=[x[0] for x in SHAPES])
def test_pack_unpack_rows(name, groups, sname, dtype, tail):
    import shared_prefix_grouped_amd as pg
    if groups is None:
        rng = np.random.default_rng(11)
        groups = [(int(rng.integers(0, 4)), [int(x) for x in rng.integers(0, 3, size=int(rng.integers(1, 3)))])
                  for _ in range(1500)]
    if sname in ("bf16_heads", "f32_model") and name == "many_groups":
        groups = groups[:300]
    print(f"[rows] {name} {sname} groups={len(groups)}", flush=True)
    batch = pg.pg_pack(groups, 4, 2, 64)
    n_pre = sum(p for p, _ in groups)
    n_resp = sum(sum(rs) for _, rs in groups)
    g = torch.Generator(device="cpu").manual_seed(3)
    if dtype.is_floating_point:
        pre = torch.randn((n_pre,) + tail, generator=g).to(dtype)
        resp = torch.randn((n_resp,) + tail, generator=g).to(dtype)
    else:
        pre = torch.randint(-2**31, 2**31 - 1, (n_pre,) + tail, generator=g).to(dtype)
        resp = torch.randint(-2**31, 2**31 - 1, (n_resp,) + tail, generator=g).to(dtype)
    want = _packed_order(groups, pre, resp)
    out = pg.pg_pack_rows(batch, pre.cuda(), resp.cuda())
    torch.cuda.synchronize()
    assert out.shape == want.shape
    assert torch.equal(out.cpu(), want)
    p2, r2 = pg.pg_unpack_rows(batch, out)
    torch.cuda.synchronize()
    assert torch.equal(p2.cpu(), pre) and torch.equal(r2.cpu(), resp)


def test_packed_token_ids_give_baseline_positions():
    """Packing token ids and reading pos_ids: response row j of a group sits at
    position P + j, as in the repeated-prefix sequence [P; R_i]."""
    import shared_prefix_grouped_amd as pg
    groups = [(6, [2, 3]), (4, [1])]
    batch = pg.pg_pack(groups, 2, 1, 64)
    pre = torch.arange(100, 110, dtype=torch.int32)          # prefix tokens
    resp = torch.arange(200, 206, dtype=torch.int32)         # response tokens
    ids = pg.pg_pack_rows(batch, pre.cuda(), resp.cuda()).cpu().tolist()
    pos = batch.pos_ids.cpu().tolist()
    assert ids == [100, 101, 102, 103, 104, 105, 200, 201, 202, 203, 204, 106, 107, 108, 109, 205]
    assert pos == [0, 1, 2, 3, 4, 5, 6, 7, 6, 7, 8, 0, 1, 2, 3, 4]
