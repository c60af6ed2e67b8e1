"""pg_attn_bwd_noalloc (library-held scratch, no allocation inside the call)
against pg_attn_bwd (caller workspace), through the C ABI on the GPU.

Two bf16 calls in a row, the second on a smaller batch, then a float32 call:
the gradients must be bitwise those of pg_attn_bwd (same kernels, fixed
reduction order).  The first batch has cut prefix key tiles, so the partial
dK/dV sums live in the scratch too.  A batch whose scratch need exceeds the
fixed size is refused before anything is enqueued.
"""
import numpy as np
import pytest

from tests.parity import to_dev
from workloads import draw_attention_inputs, scaled_down

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import shared_prefix_grouped_amd as pg
    pg.lib()


def _both(name, groups, hq, hkv, d, dtype, seed):
    import shared_prefix_grouped_amd as pg
    w = scaled_down(name, groups, dtype, hq, hkv, d, seed=seed)
    arrs = draw_attention_inputs(w)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    batch = pg.pg_pack(groups, hq, hkv, d)
    q, k, v, do = (to_dev(arrs[n], tdt) for n in ("q", "k", "v", "do"))
    o, lse = pg.pg_attn_fwd(batch, q, k, v)
    ref = pg.pg_attn_bwd(batch, q, k, v, o, lse, do)
    # outputs prefilled with NaN: every element must be written
    out = tuple(torch.full_like(x, float("nan")) for x in ref)
    pg.pg_attn_bwd_noalloc(batch, q, k, v, o, lse, do, *out)
    torch.cuda.synchronize()
    print(f"[no-alloc] {name}: T={batch.total_rows} heads={hq}/{hkv} d={d} {dtype} "
          f"cut parts={batch.desc.num_kv_parts}", flush=True)
    for n, a, b in zip(("dq", "dk", "dv"), ref, out):
        assert torch.equal(a, b), n
    return batch


def test_noalloc_matches_workspace_entry_point_twice():
    b1 = _both("noalloc_big", [(40, [97] * 24), (300, [128, 5, 70])], 8, 2, 128, "bf16", 3)
    assert b1.desc.num_kv_parts > 0  # the partial sums go through the scratch
    b2 = _both("noalloc_small", [(100, [30, 7])], 4, 2, 64, "bf16", 4)
    assert b2.total_rows < b1.total_rows
    _both("noalloc_f32", [(70, [33, 0, 12])], 2, 1, 64, "f32", 5)


def test_noalloc_refuses_oversized_scratch():
    import shared_prefix_grouped_amd as pg
    T, hq, hkv, d = 70000, 128, 8, 64
    batch = pg.pg_pack([(T - 1000, [1000])], hq, hkv, d)
    need = pg.lib().pg_attn_bwd_workspace_size(__import__("ctypes").byref(batch.desc), pg.PG_BF16)
    assert need > pg.NOALLOC_SCRATCH_BYTES
    q = torch.empty((T, hq, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((T, hkv, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((hq, T), dtype=torch.float32, device="cuda")
    with pytest.raises(pg.PgError) as e:
        pg.pg_attn_bwd_noalloc(batch, q, kv, kv, q, lse, q, q, kv, kv)
    assert e.value.status == pg.PG_ERR_WORKSPACE
    torch.cuda.synchronize()
