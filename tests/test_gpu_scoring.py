"""Forward-only grouped scoring on the GPU: many short responses scored
against one long shared context, with no logsumexp stored (the shared-context
scoring use of the same two-part attention, Pith review of Prefix Grouper,
"Editorial extensions").

  * pg_attn_fwd without LSE gives bitwise the same O as with it (bf16 and fp32);
  * the full-size scoring layout (P = 32768, 64 responses of 32 rows), launched
    as bench.py --forward-only launches it, against the fp64 repeated-prefix
    oracle on sampled rows of every kind (prefix start / end, first and last
    row of responses, random rows) and three query heads.
"""
import time

import numpy as np
import pytest

from oracle.attention import repeated_prefix_rows
from tests.parity import to_np
from workloads import attention_workloads, draw_attention_inputs

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_no_lse_same_output(dtype):
    import shared_prefix_grouped_amd as pg
    groups = [(200, [40, 0, 63, 17]), (0, [30, 5]), (129, [1])]
    hq, hkv, d = 4, 2, 128
    batch = pg.pg_pack(groups, hq, hkv, d)
    T = batch.total_rows
    g = torch.Generator().manual_seed(11)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn(T, hq, d, generator=g).to(dt).cuda()
    k = torch.randn(T, hkv, d, generator=g).to(dt).cuda()
    v = torch.randn(T, hkv, d, generator=g).to(dt).cuda()
    o1, lse = pg.pg_attn_fwd(batch, q, k, v)
    o2, none = pg.pg_attn_fwd(batch, q, k, v, store_lse=False)
    torch.cuda.synchronize()
    assert none is None and lse is not None
    assert torch.equal(o1, o2)


def test_scoring_full_size_sampled():
    import shared_prefix_grouped_amd as pg
    w = attention_workloads()["bf16_scoring_p32768"]
    groups = [(gr.prefix_len, list(gr.resp_lens)) for gr in w.groups]
    t0 = time.time()
    arrs = draw_attention_inputs(w)
    _say(f"[scoring] inputs drawn in {time.time() - t0:.1f}s, T={w.total_rows}")
    q, k, v = (torch.from_numpy(arrs[n]).to(torch.bfloat16).cuda() for n in ("q", "k", "v"))
    batch = pg.pg_pack(groups, w.num_q_heads, w.num_kv_heads, w.head_dim)
    o, lse = pg.pg_attn_fwd(batch, q, k, v, store_lse=False)
    torch.cuda.synchronize()
    assert lse is None
    P, rs = groups[0]
    rng = np.random.default_rng(w.seed + 100)
    rows = {0, P - 1, 127, 128}
    s = P
    for i, r in enumerate(rs):
        if i % 9 == 0 or i == len(rs) - 1:
            rows.update([s, s + r - 1])
        s += r
    rows.update(int(x) for x in rng.integers(P, w.total_rows, size=8))
    rows = sorted(rows)
    heads = [0, 17, 31]
    t0 = time.time()
    ref = repeated_prefix_rows(groups, arrs["q"], arrs["k"], arrs["v"], None, rows, heads)
    got = to_np(o[rows][:, heads])
    err = float(np.max(np.abs(got - ref["o"])))
    _say(f"[scoring] {len(rows)} rows x {len(heads)} heads, oracle {time.time() - t0:.1f}s: "
         f"o max-abs {err:.3e}")
    assert err <= 2e-2
