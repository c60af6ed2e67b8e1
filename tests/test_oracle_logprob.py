"""Pins of the fp64 response log-probability oracle (oracle/logprob.py) to
things other than itself: a library log-softmax, brute force, finite
differences, autograd, invariants, a constructed next-token case, and a hand
computation of the policy loss.  CPU only."""
import math

import numpy as np
import pytest

from oracle.attention import member_sequences
from oracle.logprob import (advantages_from_rewards, baseline_logprob_grads, baseline_logprobs,
                            grpo_loss, sampled_head, scored_rows)

torch = pytest.importorskip("torch")

GROUPS = [(5, [3, 0, 4]), (0, [2, 1]), (1, [1])]


def _inputs(groups, V=11, dm=6, seed=0):
    _, T = member_sequences(groups)
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, dm)), rng.standard_normal((V, dm)) * 0.7,
            rng.integers(0, V, size=T))


def test_scored_rows_by_hand():
    # group 0: prefix rows 0..4, responses [5,6,7], [], [8..11]; group 1 (P = 0):
    # [12,13], [14]; group 2: prefix row 15, response [16]
    tgt, pred = scored_rows(GROUPS)
    assert tgt.tolist() == [5, 6, 7, 8, 9, 10, 11, 13, 16]
    assert pred.tolist() == [4, 5, 6, 4, 8, 9, 10, 12, 15]


def test_matches_torch_log_softmax_gather():
    """Per member: torch.log_softmax over the vocabulary, gather at the next
    token (the page's two calls), in fp64 on the CPU."""
    hidden, W, tokens = _inputs(GROUPS)
    ref = baseline_logprobs(GROUPS, hidden, W, tokens)
    members, _ = member_sequences(GROUPS)
    got = {}
    for m in members:
        rows = m.rows
        if m.resp[1] == m.resp[0]:
            continue
        logits = torch.from_numpy(hidden[rows]) @ torch.from_numpy(W).T
        lp = torch.log_softmax(logits, dim=-1)
        start = max(m.prefix_len, 1)
        nxt = torch.from_numpy(tokens[rows[start:]]).long()
        g = lp[start - 1:len(rows) - 1].gather(1, nxt[:, None])[:, 0]
        lse = torch.logsumexp(logits, dim=-1)[start - 1:len(rows) - 1]
        for k, r in enumerate(rows[start:]):
            got[int(r)] = (float(g[k]), float(lse[k]))
    assert sorted(got) == ref["rows"].tolist()
    np.testing.assert_allclose([got[r][0] for r in ref["rows"]], ref["logp"], rtol=0, atol=1e-12)
    np.testing.assert_allclose([got[r][1] for r in ref["rows"]], ref["lse"], rtol=0, atol=1e-12)


def test_brute_force_tiny():
    groups = [(2, [2, 1])]
    hidden, W, tokens = _inputs(groups, V=4, dm=3, seed=3)
    ref = baseline_logprobs(groups, hidden, W, tokens)
    tgt, pred = scored_rows(groups)
    for k, (t, p) in enumerate(zip(tgt, pred)):
        z = [sum(hidden[p][i] * W[v][i] for i in range(3)) for v in range(4)]
        lse = math.log(sum(math.exp(x) for x in z))
        assert abs(ref["logp"][k] - (z[tokens[t]] - lse)) < 1e-12
        assert abs(ref["lse"][k] - lse) < 1e-12


def test_invariants():
    hidden, W, tokens = _inputs(GROUPS, seed=4)
    ref = baseline_logprobs(GROUPS, hidden, W, tokens)
    assert np.all(ref["logp"] <= 0)
    # adding one vector to every vocabulary row shifts every logit of a row
    # by the same amount: the log-softmax over the vocabulary is unchanged
    c = np.random.default_rng(5).standard_normal(W.shape[1])
    ref2 = baseline_logprobs(GROUPS, hidden, W + c[None, :], tokens)
    np.testing.assert_allclose(ref2["logp"], ref["logp"], atol=1e-12)


def test_next_token_alignment_constructed():
    """Each predicting row encodes the next token (identity head, large scale):
    the correct alignment scores every token near 0.  All first response
    tokens are the same token, predicted by the last prefix row; the row
    before each response in packed order (another response's last row)
    encodes a different token, so taking the packed neighbour as predictor,
    or skipping the shift, would score near -40."""
    groups = [(3, [2, 3, 2])]
    members, T = member_sequences(groups)
    V = dm = 8
    tokens = np.zeros(T, dtype=np.int64)
    hidden = np.zeros((T, dm))
    first = 5
    for m in members:
        rows = m.rows
        for p in range(1, len(rows)):
            tokens[rows[p]] = first if p == m.prefix_len else (p * 3 + m.member) % 5
    for m in members:
        rows = m.rows
        for p in range(len(rows) - 1):
            hidden[rows[p]] = 0.0
            hidden[rows[p], tokens[rows[p + 1]]] = 40.0
        hidden[rows[-1]] = 0.0
        hidden[rows[-1], 7] = 40.0  # a last row predicts nothing; it points elsewhere
    ref = baseline_logprobs(groups, hidden, np.eye(V), tokens)
    assert ref["logp"].size == 7 and np.all(ref["logp"] > -1e-12)


def test_grpo_loss_by_hand():
    groups = [(2, [2, 1])]
    tgt, _ = scored_rows(groups)          # rows 2, 3 (response 0) and 4 (response 1)
    logp = np.array([-1.0, -2.0, -0.5])
    adv = advantages_from_rewards(groups, [1.0, 3.0])  # [-1, 1]
    loss, dlogp = grpo_loss(groups, tgt, logp, adv)
    # -mean(A_i * sum_i) = -((-1)(-3) + (1)(-0.5)) / 2 = -1.25
    assert abs(loss - (-1.25)) < 1e-15
    np.testing.assert_allclose(dlogp, [0.5, 0.5, -0.5])


def test_gradients_finite_differences():
    hidden, W, tokens = _inputs(GROUPS, V=7, dm=4, seed=6)
    tgt, _ = scored_rows(GROUPS)
    dl = np.random.default_rng(7).standard_normal(tgt.size)
    g = baseline_logprob_grads(GROUPS, hidden, W, tokens, dl)

    def f(h, w):
        return float(np.dot(dl, baseline_logprobs(GROUPS, h, w, tokens)["logp"]))

    eps = 1e-6
    for (r, c) in [(4, 0), (4, 3), (6, 1), (12, 2), (15, 0), (0, 1)]:  # 4, 15: last prefix rows
        hp, hm = hidden.copy(), hidden.copy()
        hp[r, c] += eps
        hm[r, c] -= eps
        assert abs((f(hp, W) - f(hm, W)) / (2 * eps) - g["dhidden"][r, c]) < 1e-7
    for (v, c) in [(0, 0), (3, 2), (6, 3)]:
        wp, wm = W.copy(), W.copy()
        wp[v, c] += eps
        wm[v, c] -= eps
        assert abs((f(hidden, wp) - f(hidden, wm)) / (2 * eps) - g["dW"][v, c]) < 1e-7
    # rows that predict nothing and are not a last prefix row get no gradient
    assert np.all(g["dhidden"][[0, 1, 2, 3, 7, 11, 13, 14, 16]] == 0)


def test_grpo_gradients_match_autograd():
    """The whole GRPO loss through torch autograd in fp64, per member
    sequence, summed into the packed rows."""
    hidden, W, tokens = _inputs(GROUPS, seed=8)
    members, _ = member_sequences(GROUPS)
    rewards = np.random.default_rng(9).standard_normal(len(members))
    adv = advantages_from_rewards(GROUPS, rewards)
    ref = baseline_logprobs(GROUPS, hidden, W, tokens)
    loss, dlogp = grpo_loss(GROUPS, ref["rows"], ref["logp"], adv)
    g = baseline_logprob_grads(GROUPS, hidden, W, tokens, dlogp)

    h = torch.from_numpy(hidden).requires_grad_()
    w = torch.from_numpy(W).requires_grad_()
    sums = []
    for m in members:
        rows = torch.from_numpy(m.rows)
        n = m.resp[1] - m.resp[0]
        lp = torch.log_softmax(h[rows] @ w.T, dim=-1)
        start = max(m.prefix_len, 1)
        if n == 0 or start >= len(m.rows):
            sums.append(torch.zeros((), dtype=torch.float64))
            continue
        nxt = torch.from_numpy(tokens[m.rows[start:]]).long()
        sums.append(lp[start - 1:len(m.rows) - 1].gather(1, nxt[:, None]).sum())
    tloss = -(torch.stack(sums) * torch.from_numpy(adv)).mean()
    tloss.backward()
    assert abs(float(tloss.detach()) - loss) < 1e-12
    np.testing.assert_allclose(g["dhidden"], h.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dW"], w.grad.numpy(), atol=1e-12)


def test_sampled_head_matches_full_oracle():
    hidden, W, tokens = _inputs(GROUPS, V=9, dm=5, seed=10)
    tgt, _ = scored_rows(GROUPS)
    dl = np.random.default_rng(11).standard_normal(tgt.size)
    full = baseline_logprobs(GROUPS, hidden, W, tokens)
    g = baseline_logprob_grads(GROUPS, hidden, W, tokens, dl)
    ks, hs, vs = [0, 3, 7, 8], [4, 5, 12, 15, 0, 16], [0, 4, 8]
    s = sampled_head(GROUPS, hidden, W, tokens, dl, ks, hs, vs, row_block=2)
    np.testing.assert_allclose(s["logp"], full["logp"][ks], atol=1e-12)
    np.testing.assert_allclose(s["lse"], full["lse"][ks], atol=1e-12)
    np.testing.assert_allclose(s["dhidden"], g["dhidden"][hs], atol=1e-12)
    np.testing.assert_allclose(s["dW"], g["dW"][vs], atol=1e-12)
