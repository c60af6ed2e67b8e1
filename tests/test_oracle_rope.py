"""Pins of the oracle's rotary embedding at baseline positions.  No GPU.

The oracle rotates each baseline sequence [P; R_i] at positions 0..L-1 and
maps the rows back (Pith review of Prefix Grouper, "What carries the
argument": position ids as in the repeated-prefix baseline).  Pinned against:
  * the complex-number form of rotate-half RoPE, applied with the position
    ids of the hand-written fixture (tests/golden/);
  * the defining property: <rope(q, m), rope(k, n)> depends on m - n only;
  * identity at position 0 and preserved pair norms.
"""
import numpy as np

from oracle.attention import member_sequences, repeated_prefix_rope
from tests.golden_io import read_visibility_fixture


def _complex_rope(x, pos, theta=10000.0):
    T, H, d = x.shape
    half = d // 2
    z = x[..., :half] + 1j * x[..., half:]
    freq = theta ** (-2.0 * np.arange(half) / d)
    rot = np.exp(1j * pos[:, None, None] * freq[None, None, :])
    w = z * rot
    return np.concatenate([w.real, w.imag], axis=-1)


def test_matches_complex_form_at_fixture_positions():
    groups, positions, _, _ = read_visibility_fixture()
    T = len(positions)
    x = np.random.default_rng(0).standard_normal((T, 3, 8))
    assert np.allclose(repeated_prefix_rope(groups, x), _complex_rope(x, positions.astype(float)),
                       atol=1e-12, rtol=0)


def test_relative_position_property():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 1, 16))
    k = rng.standard_normal((1, 1, 16))
    for m, n, s in ((5, 2, 7), (100, 40, 3000), (0, 0, 11)):
        a = (_complex_rope(q, np.array([m + s], float)) * _complex_rope(k, np.array([n + s], float))).sum()
        b = (_complex_rope(q, np.array([m], float)) * _complex_rope(k, np.array([n], float))).sum()
        assert abs(a - b) < 1e-9
    # and the oracle on a packed batch: a response row j of group g scores
    # against prefix row t as at positions (P + j, t)
    groups = [(5, [3, 4])]
    members, T = member_sequences(groups)
    x = rng.standard_normal((T, 1, 16))
    r = repeated_prefix_rope(groups, x)
    for row, pos in ((6, 6), (9, 6)):  # row 6 = response 0 token 1; row 9 = response 1 token 1
        ref = _complex_rope(x[row:row + 1], np.array([pos], float))
        assert np.allclose(r[row], ref[0], atol=1e-12)


def test_identity_at_zero_and_norms():
    rng = np.random.default_rng(2)
    groups = [(0, [1, 1, 1])]   # every row is position 0
    x = rng.standard_normal((3, 2, 10))
    assert np.allclose(repeated_prefix_rope(groups, x), x, atol=0)
    groups = [(7, [5])]
    x = rng.standard_normal((12, 2, 10))
    y = repeated_prefix_rope(groups, x)
    n0 = x[..., :5] ** 2 + x[..., 5:] ** 2
    n1 = y[..., :5] ** 2 + y[..., 5:] ** 2
    assert np.allclose(n0, n1, atol=1e-12)
