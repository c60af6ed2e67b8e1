"""GPU parity of pg_rope (rotary embedding at baseline position ids) against the oracle."""
import numpy as np
import pytest

from oracle.attention import repeated_prefix_rope
from workloads import round_to_bf16

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CASES = [
    ([(200, [37, 0, 130]), (0, [5, 9]), (64, [1])], 4, 128),
    ([(2048, [128] * 4)], 2, 64),
    ([(32768, [40])], 1, 128),  # large positions
]


@pytest.mark.parametrize("groups,H,d", CASES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_matches_oracle(groups, H, d, dtype):
    import shared_prefix_grouped_amd as pg
    T = sum(p + sum(r) for p, r in groups)
    rng = np.random.default_rng(T + d)
    x = rng.standard_normal((T, H, d)).astype(np.float32)
    if dtype == "bf16":
        x = round_to_bf16(x)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    batch = pg.pg_pack(groups, 2, 1, 128)
    t = torch.from_numpy(x).cuda().to(tdt)
    pg.pg_rope(batch, t)
    torch.cuda.synchronize()
    got = t.float().cpu().numpy().astype(np.float64)
    ref = repeated_prefix_rope(groups, x.astype(np.float64))
    if dtype == "f32":
        assert np.max(np.abs(got - ref)) <= 1e-5
    else:  # one rounding of the float32 result to bf16: relative error <= 2^-8
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    # the inverse rotation undoes it
    pg.pg_rope(batch, t, inverse=True)
    torch.cuda.synchronize()
    back = t.float().cpu().numpy()
    if dtype == "f32":
        assert np.max(np.abs(back - x)) <= 1e-5
    else:
        # two bf16 roundings (after each rotation), each at most 2^-9 of the
        # rotated pair's norm; the inverse rotation preserves that norm
        half = d // 2
        pair = np.hypot(x[..., :half], x[..., half:])
        bound = 2.0 ** -8 * (np.concatenate([pair, pair], axis=-1) + np.abs(x)) + 1e-6
        assert np.all(np.abs(back - x) <= bound)
