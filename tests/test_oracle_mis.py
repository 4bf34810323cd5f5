"""Pins of the sequence-aware rollout-correction oracle (oracle/mis.py).

The worked example: with a = ln 2 and three sequences,
  d = lp - lq = (a, a | -2a | 0, a, 0),  rho = (2, 2 | 1/4 | 1, 2, 1),
every weight, flag and metric has a closed form (Rollout Correction Methods
page, "Importance Sampling", "Rejection Sampling", "Veto Mechanism" and the two
metric tables; readings as stated in oracle/mis.py).  The invariants below hold
at any size.
"""

import math

import numpy as np
import pytest

from oracle import mis
from oracle import replay as orp


a = math.log(2.0)
LP = np.array([-a, -a, -3 * a, -a, -a, -a])
LQ = np.array([-2 * a, -2 * a, -a, -a, -2 * a, -a])
A = np.array([1.0, -1.0, 2.0, 0.5, -2.0, 1.5])
OFF = np.array([0, 2, 3, 6])
BASE = dict(tis_level="token", tis_mode="truncate", tis_lower=0.5, tis_upper=3.0, use_rs=False,
            rs_level="token", rs_lower=None, rs_upper=None, veto=0.0, batch_normalize=False)


def run(**kw):
    cfg = dict(BASE)
    cfg.update(kw)
    return mis.mis_reference(LP, LQ, A, OFF, cfg)


def close(x, y):
    return abs(x - y) <= 1e-12 * max(1.0, abs(y))


def test_monitoring_metrics_closed_form():
    m = run()["metrics"]
    c43 = 2.0 ** (4.0 / 3.0)
    want = {
        "kl": -a / 6, "k3_kl": (2.25 - a) / 6,
        "chi2_token": (4 + 4 + 1 / 16 + 1 + 4 + 1) / 6 - 1,
        "chi2_seq": (16 + 1 / 16 + 4) / 3 - 1,
        "logprob_abs_diff": 5 * a / 6,
        "training_log_ppl": 5 * a / 3, "training_ppl": 4.0,
        "rollout_log_ppl": 13 * a / 9, "rollout_ppl": (4 + 2 + c43) / 3,
        "log_ppl_diff": 2 * a / 9, "log_ppl_abs_diff": 10 * a / 9,
        "ppl_ratio": (0.5 + 4 + 2.0 ** (-1.0 / 3.0)) / 3,
    }
    for k, v in want.items():
        assert close(m[k], v), (k, m[k], v)


def test_token_truncate():
    r = run()
    assert np.allclose(r["weight"], [2, 2, 0.25, 1, 2, 1], rtol=0, atol=1e-15)
    assert not r["flags"].any()
    m = r["metrics"]
    assert close(m["loss_sum"], 1.5) and close(m["loss"], 0.25)
    assert close(m["tis_weight_before_bound"], 8.25 / 6)
    assert close(m["tis_weight_after_bound"], 8.25 / 6)
    assert m["kept_tokens"] == 6 and m["batch_norm_factor"] == 1.0


def test_sequence_truncate():
    r = run(tis_level="sequence")
    assert np.allclose(r["weight"], [3, 3, 0.25, 2, 2, 2], rtol=0, atol=1e-14)
    assert list(r["flags"]) == [mis.F_TIS_HIGH, mis.F_TIS_HIGH, 0, 0, 0, 0]
    m = r["metrics"]
    assert close(m["loss_sum"], -0.5)
    assert close(m["tis_weight_before_bound"], 14.25 / 6)
    assert close(m["tis_weight_after_bound"], 12.25 / 6)
    assert close(m["tis_fraction_high"], 2 / 6) and m["tis_fraction_low"] == 0


def test_geometric_clip():
    r = run(tis_level="geometric", tis_mode="clip")
    c = 2.0 ** (1.0 / 3.0)
    assert np.allclose(r["weight"], [2, 2, 0.5, c, c, c], rtol=0, atol=1e-14)
    assert list(r["flags"]) == [0, 0, mis.F_TIS_LOW, 0, 0, 0]
    assert close(r["metrics"]["loss_sum"], -1.0)
    assert close(r["metrics"]["tis_fraction_low"], 1 / 6)


def test_mask_rs_veto_batch_norm():
    r = run(tis_mode="mask", use_rs=True, rs_level="sequence", rs_lower=0.5, rs_upper=1.5,
            veto=0.3, batch_normalize=True)
    assert np.allclose(r["weight"], [0, 0, 0, 1, 2, 1], rtol=0, atol=1e-15)
    rej = mis.F_REJECTED
    assert list(r["flags"]) == [
        mis.F_RS_HIGH | rej, mis.F_RS_HIGH | rej,
        mis.F_TIS_LOW | mis.F_RS_LOW | mis.F_VETO | mis.F_CATASTROPHIC | rej, 0, 0, 0]
    m = r["metrics"]
    want = {"batch_norm_factor": 0.75, "is_ratio_mean_final": 1.0, "is_ratio_min_final": 0.75,
            "is_ratio_max_final": 1.5, "loss_sum": 1.5, "loss": 0.5, "kept_tokens": 3.0,
            "rejected_tokens": 3.0, "rs_fraction_low": 1 / 6, "rs_fraction_high": 2 / 6,
            "catastrophic_token_fraction": 1 / 6, "catastrophic_seq_fraction": 1 / 3,
            "is_ratio_mean_after_tis_rs": 4 / 6, "tis_weight_before_bound": 8.25 / 6,
            "tis_weight_after_bound": 8 / 6, "tis_fraction_low": 1 / 6, "tis_fraction_high": 0.0}
    for k, v in want.items():
        assert close(m[k], v), (k, m[k], v)


def test_geometric_rs_rejects_everything():
    r = run(use_rs=True, rs_level="geometric", rs_lower=0.9, rs_upper=1.1)
    m = r["metrics"]
    assert m["kept_tokens"] == 0 and m["loss"] == 0 and m["loss_sum"] == 0
    assert close(m["rs_fraction_low"], 1 / 6) and close(m["rs_fraction_high"], 5 / 6)
    assert not r["weight"].any()


def test_rs_bounds_default_to_tis_bounds():
    r1 = run(use_rs=True, rs_level="token")
    r2 = run(use_rs=True, rs_level="token", rs_lower=0.5, rs_upper=3.0)
    assert np.array_equal(r1["flags"], r2["flags"])
    # rho = 1/4 < 0.5 is rejected low; nothing exceeds 3
    assert list(r1["flags"] & (mis.F_RS_LOW | mis.F_RS_HIGH)) == [0, 0, mis.F_RS_LOW, 0, 0, 0]


# ---- invariants on random replays -------------------------------------------

def _rand(seed, N, S):
    g = np.random.default_rng(seed)
    lq = -g.exponential(1.0, N)
    lp = np.minimum(lq + g.normal(0, 0.4, N), 0)
    A = g.normal(size=N)
    cuts = np.sort(g.choice(np.arange(1, N), S - 1, replace=False))
    return lp, lq, A, np.concatenate([[0], cuts, [N]])


@pytest.mark.parametrize("mode", mis.MODES)
def test_single_token_sequences_make_levels_agree(mode):
    g = np.random.default_rng(3)
    N = 200
    lq = -g.exponential(1.0, N)
    lp = np.minimum(lq + g.normal(0, 0.5, N), 0)
    A = g.normal(size=N)
    off = np.arange(N + 1)
    outs = []
    for lev in mis.LEVELS:
        cfg = dict(BASE, tis_level=lev, tis_mode=mode, use_rs=True, rs_level=lev, rs_lower=0.6,
                   rs_upper=1.8, veto=0.2, batch_normalize=True)
        outs.append(mis.mis_reference(lp, lq, A, off, cfg))
    for o in outs[1:]:
        assert np.allclose(o["weight"], outs[0]["weight"], rtol=1e-12, atol=0)
        assert np.array_equal(o["flags"], outs[0]["flags"])
    m = outs[0]["metrics"]
    assert abs(m["chi2_seq"] - m["chi2_token"]) < 1e-9


def test_identical_policies():
    lp, _, A, off = _rand(5, 500, 20)
    r = mis.mis_reference(lp, lp, A, off, dict(BASE, tis_level="sequence", tis_mode="mask"))
    m = r["metrics"]
    for k in ("kl", "k3_kl", "chi2_token", "chi2_seq", "logprob_abs_diff", "log_ppl_diff",
              "log_ppl_abs_diff"):
        assert abs(m[k]) < 1e-12, k
    assert abs(m["ppl_ratio"] - 1) < 1e-12
    assert np.all(r["weight"] == 1.0) and not r["flags"].any()
    assert abs(m["loss_sum"] + A.sum()) < 1e-9


@pytest.mark.parametrize("level", mis.LEVELS)
def test_batch_norm_mean_one_and_divergences_nonnegative(level):
    lp, lq, A, off = _rand(7, 3000, 40)
    cfg = dict(BASE, tis_level=level, tis_mode="clip", use_rs=True, rs_level="geometric",
               rs_lower=0.8, rs_upper=1.25, veto=1e-3, batch_normalize=True)
    r = mis.mis_reference(lp, lq, A, off, cfg)
    m = r["metrics"]
    assert m["kept_tokens"] > 0
    assert abs(m["is_ratio_mean_final"] - 1.0) < 1e-12
    assert m["k3_kl"] >= 0 and m["chi2_token"] >= -1e-12
    # AM >= GM: the sequence-level rejection statistic is never below the geometric one
    d = lp - lq
    am = np.add.reduceat(np.exp(d), off[:-1]) / np.diff(off)
    gm = np.exp(np.add.reduceat(d, off[:-1]) / np.diff(off))
    assert np.all(am >= gm * (1 - 1e-12))


def test_open_rs_bounds_reject_nothing():
    lp, lq, A, off = _rand(9, 1000, 10)
    c0 = dict(BASE, tis_level="geometric", tis_mode="clip")
    r0 = mis.mis_reference(lp, lq, A, off, c0)
    r1 = mis.mis_reference(lp, lq, A, off, dict(c0, use_rs=True, rs_level="sequence",
                                                rs_lower=1e-30, rs_upper=1e30))
    assert np.array_equal(r0["weight"], r1["weight"])
    assert r1["metrics"]["rejected_tokens"] == 0


def test_token_truncate_matches_replay_tis():
    lp, lq, A, off = _rand(11, 4000, 30)
    r = mis.mis_reference(lp, lq, A, off, dict(BASE, tis_upper=2.0))
    params = dict(eps=(0.3,), primary_eps_index=0, max_ratio=5.0, icepop_lo=0.5, icepop_hi=2.0,
                  clip_low=0.2, clip_high=0.2, clip_c=3.0, tis_upper=2.0)
    ref = orp.replay_reference(lp, lq, A, params)
    assert abs(r["metrics"]["loss_sum"] - ref["tis_loss_sum"]) < 1e-9 * abs(ref["tis_loss_sum"])
    assert r["metrics"]["tis_fraction_high"] * len(lp) == ref["tis_truncated"]


def test_mask_bounds_inclusive_and_masked_tokens_stay_in_average():
    # rho = 1 exactly for tokens 3 and 5 (d = 0): a weight equal to the bound is kept
    r = run(tis_mode="mask", tis_lower=1.0, tis_upper=2.0)
    assert np.allclose(r["weight"], [2, 2, 0, 1, 2, 1], rtol=0, atol=1e-15)
    assert list(r["flags"]) == [0, 0, mis.F_TIS_LOW, 0, 0, 0]
    m = r["metrics"]
    # the masked token has weight 0 but is still counted in the loss average
    assert m["kept_tokens"] == 6 and close(m["loss"], m["loss_sum"] / 6)
    assert close(m["loss_sum"], -(2 - 2 + 0 + 0.5 - 4 + 1.5))


def test_veto_without_rejection_sampling():
    r = run(veto=0.3)
    rej = mis.F_REJECTED
    assert list(r["flags"]) == [0, 0, mis.F_VETO | mis.F_CATASTROPHIC | rej, 0, 0, 0]
    m = r["metrics"]
    assert m["kept_tokens"] == 5 and close(m["catastrophic_seq_fraction"], 1 / 3)
    assert close(m["loss_sum"], -(2 - 2 + 0.5 - 4 + 1.5))


def test_catastrophic_is_per_token_veto_per_sequence():
    # veto 1.5: tokens 2 (1/4), 3 (1), 5 (1) are catastrophic; sequences 1 and 2 are vetoed,
    # so token 4 (rho = 2) is vetoed without being catastrophic itself
    r = run(veto=1.5)
    V, C, R = mis.F_VETO, mis.F_CATASTROPHIC, mis.F_REJECTED
    assert list(r["flags"]) == [0, 0, V | C | R, V | C | R, V | R, V | C | R]
    m = r["metrics"]
    assert close(m["catastrophic_token_fraction"], 3 / 6)
    assert close(m["catastrophic_seq_fraction"], 2 / 3)
    assert m["kept_tokens"] == 2
