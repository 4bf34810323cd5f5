"""Parity of the loss-only replay (rl_loss_elementwise) with the oracle at full size."""

import numpy as np
import pytest
import torch

from lm_head_logprobs_amd import ops
from oracle import replay as orp
from synth import make_replay

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

BAND = 1e-6  # both sides read the same fp32 inputs; fp32 vs fp64 rounding only


def _run(r):
    rp = ops.Replay(r.lp, r.lq, r.adv, r.params)
    rp()
    torch.cuda.synchronize()
    return rp, {k: v.cpu().numpy() for k, v in rp.o.items()}


# 2.16M: 2-3 chunks per wave, partial chunk on slot 245; 2**21: whole chunks only, two
# rounds; 2**20 + 1: one-token partial chunk on slot 0 of the second round
@pytest.mark.parametrize("N", [2_160_000, 1, 1023, 4097, 2_097_152, 1_048_577])
def test_replay_parity(N):
    r = make_replay(N=N, device="cuda:0")
    print(f"[case] replay N={N}", flush=True)
    _, got = _run(r)
    check_replay(r, got)


def check_replay(r, got):
    """Every output of one replay call against the oracle: mask words bit for
    bit outside the near-threshold band, the primary weight to rounding, the
    counts exactly up to the near-threshold decisions, the sums to 1e-4
    relative plus what the near-threshold tokens can move."""
    ref = orp.replay_reference(r.lp.cpu().numpy(), r.lq.cpu().numpy(), r.adv.cpu().numpy(),
                               r.params)
    near = orp.near_threshold_bits(ref, BAND)
    word = got["mask_word"].view(np.uint16)
    diff = (word ^ ref["mask_word"]) & ~near
    n_near = int(np.count_nonzero(near))
    print(f"near-threshold decisions: {n_near}")
    assert not np.any(diff), np.nonzero(diff)[0][:10]
    near_tok = near != 0
    # primary IPO weight: rounding-level agreement away from thresholds
    wp = got["w_primary"].astype(np.float64)
    assert np.allclose(wp[~near_tok], ref["w_primary"][~near_tok], rtol=2e-6, atol=1e-7)
    s = got["sums"]
    A = r.adv.cpu().numpy().astype(np.float64)
    lp = r.lp.cpu().numpy().astype(np.float64)
    # tokens near a threshold can move a loss sum by their own contribution
    slack = np.sum(np.abs(A[near_tok]) * 5.0 * (np.abs(lp[near_tok]) + 1.0))
    n_eps = len(r.params["eps"])
    for i in range(n_eps):
        assert abs(s[3 * i] - ref[f"ipo{i}_kept"]) <= n_near
        assert abs(s[3 * i + 1] - ref[f"ipo{i}_loss_sum"]) <= 1e-4 * abs(ref[f"ipo{i}_loss_sum"]) + slack + 1e-6
        assert abs(s[3 * i + 2] - ref[f"ipo{i}_weight_sum"]) <= 1e-5 * abs(ref[f"ipo{i}_weight_sum"]) + 5 * n_near + 1e-6
    checks = [(24, "icepop_kept"), (25, "icepop_low"), (26, "icepop_high"), (31, "ppo_clip"),
              (32, "ppo_clip_lower"), (35, "tis_truncated")]
    for idx, k in checks:
        assert abs(s[idx] - ref[k]) <= n_near, (k, s[idx], ref[k])
    for idx, k in [(27, "icepop_loss_sum"), (29, "reinforce_loss_sum"), (30, "ppo_loss_sum"),
                   (33, "ppo_kl_sum"), (34, "tis_loss_sum"), (28, "icepop_weight_sum"),
                   (36, "tis_weight_sum")]:
        assert abs(s[idx] - ref[k]) <= 1e-4 * abs(ref[k]) + slack + 1e-6, (k, s[idx], ref[k])
    # the recipe's own statistics: masked fractions grow as eps shrinks
    kept = [s[3 * i] for i in range(n_eps)]
    assert all(a <= b for a, b in zip(kept, kept[1:]))


def test_replay_deterministic():
    r = make_replay(N=300_001, device="cuda:0")
    rp, a = _run(r)
    rp()
    torch.cuda.synchronize()
    assert np.array_equal(a["sums"], rp.o["sums"].cpu().numpy())
