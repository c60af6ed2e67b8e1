"""Response log-probability head of the GRPO step on the GPU, against the
fp64 oracle (oracle/logprob.py: per member sequence [P; R_i], next-token
alignment).

Tolerances (bf16 operands, fp32 accumulation; the gradient of the logits is
rounded to bf16 before the two backward products):
  logp, lse: max-abs <= 2e-3; loss: abs <= 1e-4 * (1 + |loss|);
  dhidden, dweight: ||g - g*||_F / ||g*||_F <= 1e-2 (dhidden also on the
  predicting prefix rows alone).
"""
import numpy as np
import pytest

from oracle.logprob import (advantages_from_rewards, baseline_logprob_grads, baseline_logprobs,
                            grpo_loss, sampled_head, scored_rows)
from tests.parity import rel_fro
from workloads import Group, HeadWorkload, draw_head_inputs, head_workloads

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


def _groups(w):
    return [(g.prefix_len, list(g.resp_lens)) for g in w.groups]


def _run(w, arrs, adv):
    import shared_prefix_grouped_amd as pg
    groups = _groups(w)
    batch = pg.pg_pack(groups, 1, 1, 64)
    h = torch.from_numpy(arrs["hidden"]).cuda().to(torch.bfloat16)
    W = torch.from_numpy(arrs["weight"]).cuda().to(torch.bfloat16)
    tok = torch.from_numpy(arrs["tokens"]).cuda()
    a = torch.from_numpy(np.asarray(adv, dtype=np.float32)).cuda()
    logp, lse = pg.pg_logprob_fwd(batch, h, W, tok)
    loss, dlogp = pg.pg_grpo_loss(batch, logp, a)
    dh, dW = pg.pg_logprob_bwd(batch, h, W, tok, lse, dlogp)
    torch.cuda.synchronize()
    return batch, {"logp": logp, "lse": lse, "loss": loss, "dlogp": dlogp, "dhidden": dh,
                   "dW": dW}


SMALL = [
    ("mixed", [(5, [3, 0, 4]), (0, [2, 1]), (1, [1])], 64, 1000),
    ("odd_vocab", [(40, [17, 1, 33]), (3, [9])], 136, 5003),
    ("wide", [(130, [64, 64, 2, 70])], 256, 4096),
]


@pytest.mark.parametrize("name,groups,dm,V", SMALL, ids=[s[0] for s in SMALL])
def test_small_against_full_oracle(name, groups, dm, V):
    w = HeadWorkload(name, tuple(Group(p, tuple(rs)) for p, rs in groups), dm, V, seed=17)
    arrs = draw_head_inputs(w)
    adv = advantages_from_rewards(groups, arrs["rewards"])
    batch, out = _run(w, arrs, adv)
    ref = baseline_logprobs(groups, arrs["hidden"], arrs["weight"], arrs["tokens"])
    tgt, pred = scored_rows(groups)
    assert batch.desc.num_scored == tgt.size
    loss, dlogp = grpo_loss(groups, ref["rows"], ref["logp"], adv)
    g = baseline_logprob_grads(groups, arrs["hidden"], arrs["weight"], arrs["tokens"], dlogp)
    e_lp = float(np.max(np.abs(out["logp"].cpu().numpy() - ref["logp"])))
    e_l = float(np.max(np.abs(out["lse"].cpu().numpy() - ref["lse"])))
    e_loss = abs(float(out["loss"].cpu()[0]) - loss)
    e_d = float(np.max(np.abs(out["dlogp"].cpu().numpy() - dlogp)))
    dh = out["dhidden"].cpu().numpy()
    e_h = rel_fro(dh, g["dhidden"])
    last_prefix = sorted({int(p) for p, t in zip(pred, tgt) if p < t - 1})
    e_hp = rel_fro(dh[last_prefix], g["dhidden"][last_prefix]) if last_prefix else 0.0
    e_w = rel_fro(out["dW"].cpu().numpy(), g["dW"])
    _say(f"[head] {name}: logp {e_lp:.2e} lse {e_l:.2e} loss {e_loss:.2e} dlogp {e_d:.2e} "
         f"dhidden {e_h:.2e} (prefix rows {e_hp:.2e}) dW {e_w:.2e}")
    assert e_lp <= 2e-3 and e_l <= 2e-3 and e_d <= 1e-6
    assert e_loss <= 1e-4 * (1 + abs(loss))
    assert e_h <= 1e-2 and e_hp <= 1e-2 and e_w <= 1e-2
    # rows that score nothing get exactly zero
    scoring = set(int(p) for p in pred)
    others = [t for t in range(dh.shape[0]) if t not in scoring]
    assert np.all(dh[others] == 0)


def test_deterministic_bitwise():
    groups = [(40, [17, 1, 33]), (3, [9])]
    w = HeadWorkload("det", tuple(Group(p, tuple(rs)) for p, rs in groups), 128, 3000, seed=18)
    arrs = draw_head_inputs(w)
    adv = advantages_from_rewards(groups, arrs["rewards"])
    _, a = _run(w, arrs, adv)
    junk = torch.randn(1 << 20, device="cuda")
    _, b = _run(w, arrs, adv)
    del junk
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_full_size_sampled():
    """The full head workload (P = 8192, 16 responses, d_model 2048, vocab
    32000) launched as bench.py launches it; the oracle on sampled entries:
    logp/lse at 64 scored rows (incl. every response's first and last token),
    dhidden at the last prefix row and sampled response rows, dW at 24
    vocabulary rows (incl. sampled target tokens)."""
    w = head_workloads()["grpo_head_g16_p8192"]
    groups = _groups(w)
    arrs = draw_head_inputs(w)
    adv = advantages_from_rewards(groups, arrs["rewards"])
    _, out = _run(w, arrs, adv)
    tgt, pred = scored_rows(groups)
    rng = np.random.default_rng(19)
    first = [k for k in range(tgt.size) if pred[k] != tgt[k] - 1]
    last = [k for k in range(tgt.size - 1) if pred[k + 1] != tgt[k]] + [tgt.size - 1]
    ks = sorted(set(first + last + rng.choice(tgt.size, 32, replace=False).tolist()))
    P = groups[0][0]
    hs = [P - 1] + sorted(rng.choice(np.unique(pred[pred >= P]), 8, replace=False).tolist())
    vs = sorted(set(rng.choice(w.vocab, 12, replace=False).tolist()
                    + arrs["tokens"][tgt[ks[:12]]].tolist()))
    dlogp = out["dlogp"].cpu().numpy().astype(np.float64)
    _, dlogp_ref = grpo_loss(groups, tgt, np.zeros(tgt.size), adv)
    assert np.max(np.abs(dlogp - dlogp_ref)) <= 1e-6
    ref = sampled_head(groups, arrs["hidden"], arrs["weight"], arrs["tokens"], dlogp_ref, ks, hs, vs)
    e_lp = float(np.max(np.abs(out["logp"].cpu().numpy()[ks] - ref["logp"])))
    e_l = float(np.max(np.abs(out["lse"].cpu().numpy()[ks] - ref["lse"])))
    e_h = rel_fro(out["dhidden"].cpu().numpy()[hs], ref["dhidden"])
    e_w = rel_fro(out["dW"].cpu().numpy()[vs], ref["dW"])
    _say(f"[head] full: {len(ks)} rows logp {e_lp:.2e} lse {e_l:.2e}; dhidden {len(hs)} rows "
         f"{e_h:.2e}; dW {len(vs)} rows {e_w:.2e}")
    assert e_lp <= 2e-3 and e_l <= 2e-3 and e_h <= 1e-2 and e_w <= 1e-2


def test_nothing_scored_gives_zero_gradients():
    """No scored token (empty responses, and single-token responses of an
    empty prefix): logp is empty, the loss is 0 and both gradients are
    exactly zero (dweight from a product over zero rows)."""
    groups = [(5, [0, 0]), (0, [1, 1, 0])]
    w = HeadWorkload("none", tuple(Group(p, tuple(rs)) for p, rs in groups), 64, 300, seed=20)
    arrs = draw_head_inputs(w)
    adv = advantages_from_rewards(groups, arrs["rewards"])
    # leave NaN in the allocator's cached blocks of the output sizes, so an
    # output the library did not write would show
    junk = [torch.full((300, 64), float("nan"), device="cuda"),
            torch.full((w.total_rows, 64), float("nan"), device="cuda")]
    del junk
    batch, out = _run(w, arrs, adv)
    assert batch.desc.num_scored == 0 and out["logp"].numel() == 0
    assert float(out["loss"].cpu()[0]) == 0.0
    assert torch.count_nonzero(out["dhidden"]).item() == 0
    assert torch.count_nonzero(out["dW"]).item() == 0
