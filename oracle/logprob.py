"""Response-token log-probabilities of the GRPO step, on the repeated-prefix
baseline, in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages compute ("prefix-grouper-grpo" page on skillsmp.com, "Step 4:
Training Integration with GRPO"): the model's logits are turned into log-
probabilities with a log-softmax over the vocabulary, the log-probability of
every response token is gathered, summed per response, and the policy loss is
minus the mean over responses of (summed log-probability) x (advantage), with
the advantage treated as a constant; the page's helper takes the advantage as
the reward minus the mean reward (or the reward itself).

Readings where the page leaves a point open (each listed in the design notes):
  * logits = hidden @ W^T with an LM head W [V, d_model] and no bias (the page
    only says "model logits"; the head is the last layer of that model);
  * next-token alignment: the log-probability of the token at position p of a
    sequence is read from the logits at position p - 1, the usual causal-LM
    convention (the page's sketch slices logits and tokens at the same
    positions, which for a causal model would score each token with the
    distribution that already saw it).  So response token j of member
    [P; R_i] is predicted by position P + j - 1: the last prefix position for
    j = 0, which in the packed layout is the same row for all G responses of
    a group.  With P = 0 the first response token has no predictor and is not
    scored;
  * mean over responses: over every response of the batch (the page's (B, G)
    array with B groups of G responses).

Array layout: hidden [T, d_model] in packed order; W [V, d_model]; tokens [T]
integer token ids in packed order (the token of each packed row).
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np

from .attention import member_sequences


def _log_softmax(z: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row-wise log-softmax and logsumexp of logits z [n, V] (fp64)."""
    m = z.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))
    return z - lse, lse[:, 0]


def scored_rows(groups) -> Tuple[np.ndarray, np.ndarray]:
    """(target rows, predictor rows) in packed order: every response row whose
    token is scored, and the packed row whose logits score it (the previous
    position of its baseline sequence [P; R_i])."""
    members, _ = member_sequences(groups)
    tgt, pred = [], []
    for m in members:
        rows = m.rows
        for j in range(m.resp[1] - m.resp[0]):
            p = m.prefix_len + j          # position of response token j in [P; R_i]
            if p == 0:
                continue                  # no predictor: first token of an empty-prefix sequence
            tgt.append(int(rows[p]))
            pred.append(int(rows[p - 1]))
    order = np.argsort(np.asarray(tgt, dtype=np.int64), kind="stable")
    return (np.asarray(tgt, dtype=np.int64)[order], np.asarray(pred, dtype=np.int64)[order])


def baseline_logprobs(groups, hidden, W, tokens) -> Dict[str, np.ndarray]:
    """Per scored response row (packed order, as scored_rows): log-probability
    of its token, and the logsumexp of the logits that score it.  Computed per
    member sequence [P; R_i] exactly as the baseline runs it: logits of every
    position, log-softmax, gather at the next token."""
    members, _ = member_sequences(groups)
    Wd = np.asarray(W, dtype=np.float64)
    out_lp, out_lse, out_row = [], [], []
    for m in members:
        rows = m.rows
        if m.resp[1] == m.resp[0]:
            continue
        X = np.asarray(hidden, dtype=np.float64)[rows]
        lsm, lse = _log_softmax(X @ Wd.T)
        for j in range(m.resp[1] - m.resp[0]):
            p = m.prefix_len + j
            if p == 0:
                continue
            out_row.append(int(rows[p]))
            out_lp.append(lsm[p - 1, int(tokens[rows[p]])])
            out_lse.append(lse[p - 1])
    order = np.argsort(np.asarray(out_row, dtype=np.int64), kind="stable")
    return {"rows": np.asarray(out_row, dtype=np.int64)[order],
            "logp": np.asarray(out_lp)[order], "lse": np.asarray(out_lse)[order]}


def grpo_loss(groups, logp_rows: np.ndarray, logp: np.ndarray, advantages: Sequence[float]):
    """Policy loss -mean_i(A_i * sum_j logp_ij) over all responses of the batch
    and its gradient with respect to each scored token's log-probability
    (-A_i / n_responses, the same for every token of response i)."""
    members, _ = member_sequences(groups)
    adv = np.asarray(advantages, dtype=np.float64)
    if adv.size != len(members):
        raise ValueError("one advantage per response")
    owner = {}
    for i, m in enumerate(members):
        for r in range(*m.resp):
            owner[r] = i
    sums = np.zeros(len(members))
    dlogp = np.zeros(len(logp_rows))
    for k, r in enumerate(logp_rows):
        i = owner[int(r)]
        sums[i] += logp[k]
        dlogp[k] = -adv[i] / len(members)
    return float(-(sums * adv).mean()), dlogp


def advantages_from_rewards(groups, rewards: Sequence[float], use_baseline: bool = True) -> np.ndarray:
    """The page's helper: reward minus the mean reward of the batch, or the reward."""
    r = np.asarray(rewards, dtype=np.float64)
    return r - r.mean() if use_baseline else r.copy()


def baseline_logprob_grads(groups, hidden, W, tokens, dlogp: np.ndarray) -> Dict[str, np.ndarray]:
    """Gradients of sum_k dlogp[k] * logp[k] (k over scored rows, in the order
    of scored_rows) with respect to the packed hidden states and W, by the
    chain rule per member sequence: d logp / d z = onehot(token) - softmax(z)
    at the predicting position; dX = dz W, dW = dz^T X.  A shared prefix row's
    gradient is the sum over the G member copies (Pith review of Prefix
    Grouper, "Core claim", Lemma 2.1); here only the last prefix row gets any,
    from the first token of each response."""
    members, T = member_sequences(groups)
    Wd = np.asarray(W, dtype=np.float64)
    tgt, _ = scored_rows(groups)
    index = {int(r): k for k, r in enumerate(tgt)}
    dh = np.zeros((T, Wd.shape[1]))
    dW = np.zeros_like(Wd)
    for m in members:
        rows = m.rows
        n_resp = m.resp[1] - m.resp[0]
        if n_resp == 0:
            continue
        X = np.asarray(hidden, dtype=np.float64)[rows]
        lsm, _ = _log_softmax(X @ Wd.T)
        dz = np.zeros_like(lsm)
        for j in range(n_resp):
            p = m.prefix_len + j
            if p == 0:
                continue
            g = dlogp[index[int(rows[p])]]
            dz[p - 1] -= g * np.exp(lsm[p - 1])
            dz[p - 1, int(tokens[rows[p]])] += g
        dh[rows] += dz @ Wd
        dW += dz.T @ X
    return {"dhidden": dh, "dW": dW}


def sampled_head(groups, hidden, W, tokens, dlogp, k_sample, hid_sample, vocab_sample,
                 row_block: int = 256) -> Dict[str, np.ndarray]:
    """The same quantities at sampled indices, for sizes where the full
    per-member computation is too slow: logp and lse at scored entries
    k_sample (order of scored_rows), the hidden-state gradient at packed rows
    hid_sample, and the LM-head gradient at vocabulary rows vocab_sample.
    Each scored token only depends on its predicting row (the next-token
    reading above), so this computes, in fp64, the logits of predicting rows
    in blocks (keeping only their logsumexp) and then the sampled sums of the
    chain rule of baseline_logprob_grads."""
    tgt, pred = scored_rows(groups)
    Wd = np.asarray(W, dtype=np.float64)
    H = np.asarray(hidden, dtype=np.float64)
    n = tgt.size
    lse = np.empty(n)
    for b0 in range(0, n, row_block):
        z = H[pred[b0:b0 + row_block]] @ Wd.T
        m = z.max(axis=1, keepdims=True)
        lse[b0:b0 + row_block] = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    ks = np.asarray(k_sample, dtype=np.int64)
    zt = np.einsum("kd,kd->k", H[pred[ks]], Wd[np.asarray(tokens)[tgt[ks]]])
    out = {"logp": zt - lse[ks], "lse": lse[ks]}
    # dhidden[t] = sum over entries k predicted by t of dlogp_k (W[tok_k] - softmax_k W)
    dh = np.zeros((len(hid_sample), Wd.shape[1]))
    for i, t in enumerate(hid_sample):
        for k in np.nonzero(pred == int(t))[0]:
            p = np.exp(H[t] @ Wd.T - lse[k])
            dh[i] += dlogp[k] * (Wd[int(tokens[tgt[k]])] - p @ Wd)
    out["dhidden"] = dh
    # dW[v] = sum_k dlogp_k ([v == tok_k] - p_kv) h_pred_k
    vs = np.asarray(vocab_sample, dtype=np.int64)
    pv = np.exp(H[pred] @ Wd[vs].T - lse[:, None])            # [n, len(vs)]
    onehot = (np.asarray(tokens)[tgt][:, None] == vs[None, :]).astype(np.float64)
    out["dW"] = ((onehot - pv) * np.asarray(dlogp)[:, None]).T @ H[pred]
    return out
