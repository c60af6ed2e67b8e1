"""pg_pack enqueues its upload without waiting for the GPU: packs issued back
to back behind a running kernel, enough of them that the library's pinned
staging buffers are reused, must each leave their own plan on the device."""
import numpy as np
import pytest

from oracle.attention import position_ids
from workloads import draw_attention_inputs, scaled_down

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import shared_prefix_grouped_amd as pg
    pg.lib()


def _layout(i):
    rng = np.random.default_rng(1000 + i)
    return [(int(rng.integers(0, 200)), [int(x) for x in rng.integers(0, 90, size=int(rng.integers(1, 5)))])
            for _ in range(int(rng.integers(1, 3)))]


def test_back_to_back_packs_keep_their_plans():
    import shared_prefix_grouped_amd as pg
    hq, hkv, d = 4, 2, 64
    dev = torch.device("cuda:0")
    # a long forward on the stream first, so the uploads below queue behind it
    big = [(4096, [512] * 8)]
    wb = scaled_down("pack_async_big", big, "bf16", 8, 2, 128, seed=5)
    ab = draw_attention_inputs(wb)
    qb, kb, vb = (torch.from_numpy(ab[n]).to(dev).to(torch.bfloat16) for n in ("q", "k", "v"))
    bb = pg.pg_pack(big, 8, 2, 128, dev)
    torch.cuda.synchronize()
    pg.pg_attn_fwd(bb, qb, kb, vb)
    n = 80  # more packs than staging buffers the library keeps in flight
    layouts = [_layout(i) for i in range(n)]
    batches = [pg.pg_pack(g, hq, hkv, d, dev) for g in layouts]
    torch.cuda.synchronize()
    for g, b in zip(layouts, batches):
        T = sum(P + sum(rs) for P, rs in g)
        assert b.total_rows == T
        assert np.array_equal(b.pos_ids.cpu().numpy(), position_ids(g))
    # the same forward through each asynchronously packed plan and through a
    # plan packed after a synchronisation gives bitwise the same output
    for i in range(0, n, 7):
        g = layouts[i]
        w = scaled_down(f"pack_async_{i}", g, "bf16", hq, hkv, d, seed=i)
        a = draw_attention_inputs(w)
        q, k, v = (torch.from_numpy(a[x]).to(dev).to(torch.bfloat16) for x in ("q", "k", "v"))
        o1, l1 = pg.pg_attn_fwd(batches[i], q, k, v)
        torch.cuda.synchronize()
        fresh = pg.pg_pack(g, hq, hkv, d, dev)
        torch.cuda.synchronize()
        o2, l2 = pg.pg_attn_fwd(fresh, q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"layout {i}: {g}"
