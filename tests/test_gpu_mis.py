"""Parity of the sequence-aware rollout correction (rl_mis_replay) with the oracle."""

import numpy as np
import pytest
import torch

from lm_head_logprobs_amd import ops
from oracle import mis as om
from synth import MIS_PARAMS, make_replay, replay_sequences

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# Decisions within BAND (log space) of a threshold are not compared bit for bit:
# token-level log ratios are exact fp64 on both sides, but sequence sums add in
# different orders and the sequence-mean ratio sums fp32 exponentials.
BAND = 1e-5
COUNT_METRICS = ("kept_tokens", "rejected_tokens")
FRACTION_METRICS = ("tis_fraction_low", "tis_fraction_high", "rs_fraction_low",
                    "rs_fraction_high", "catastrophic_token_fraction")


def _near(a, b, tol):
    """|a - b| <= tol, with equal non-finite values (an overflowing e^(2 sum d)) as equal."""
    if not np.isfinite(b):
        return a == b
    return abs(a - b) <= tol


def _run(lp, lq, A, off, params):
    mr = ops.MisReplay(lp, lq, A, torch.as_tensor(off, dtype=torch.int64), params)
    mr()
    torch.cuda.synchronize()
    return mr, mr.o["weight"].cpu().numpy(), mr.o["flags"].cpu().numpy(), mr.metrics()


def _check(lp, lq, A, off, params, max_near_frac=1e-3):
    mr, w, fl, m = _run(lp, lq, A, off, params)
    ref = om.mis_reference(lp.cpu().numpy(), lq.cpu().numpy(), A.cpu().numpy(), off, params)
    near = om.near_threshold_tokens(ref, params, BAND)
    n_near = int(near.sum())
    N = len(w)
    print(f"N={N} S={len(off) - 1} near={n_near}", flush=True)
    assert n_near <= max(16, max_near_frac * N)
    far = ~near
    assert np.array_equal(fl[far], ref["flags"][far]), np.nonzero(fl[far] != ref["flags"][far])[0][:8]
    rw = ref["weight"]
    assert np.allclose(w[far], rw[far], rtol=2e-6, atol=1e-30)
    rm = ref["metrics"]
    U = max(params["tis_upper"], 1.0)
    slack_w = n_near * U  # a flipped decision moves a weight sum by at most one weight
    Aabs = np.abs(A.cpu().numpy())
    slack_wa = U * float(np.sort(Aabs)[::-1][:n_near].sum()) if n_near else 0.0
    for k in COUNT_METRICS:
        assert abs(m[k] - rm[k]) <= n_near, (k, m[k], rm[k])
    for k in FRACTION_METRICS:
        assert abs(m[k] - rm[k]) * N <= n_near + 1e-6, (k, m[k], rm[k])
    S = len(off) - 1
    assert abs(m["catastrophic_seq_fraction"] - rm["catastrophic_seq_fraction"]) * S <= (
        n_near + 1e-6)
    for k in ("training_log_ppl", "training_ppl", "rollout_log_ppl", "rollout_ppl",
              "log_ppl_abs_diff", "ppl_ratio", "chi2_token", "chi2_seq", "logprob_abs_diff",
              "tis_weight_before_bound", "k3_kl"):
        assert _near(m[k], rm[k], 2e-5 * abs(rm[k]) + 1e-12), (k, m[k], rm[k])
    # signed means: relative to the mean absolute term
    dabs = float(np.mean(np.abs(ref["d"])))
    for k in ("kl", "log_ppl_diff"):
        assert abs(m[k] - rm[k]) <= 2e-5 * dabs + 1e-12, (k, m[k], rm[k])
    for k in ("tis_weight_after_bound", "is_ratio_mean_after_tis_rs"):
        assert abs(m[k] - rm[k]) * N <= 2e-5 * abs(rm[k]) * N + slack_w + 1e-9, (k, m[k], rm[k])
    kept = rm["kept_tokens"]
    if kept > 0 and n_near == 0:
        for k in ("batch_norm_factor", "is_ratio_mean_final", "is_ratio_min_final",
                  "is_ratio_max_final"):
            assert abs(m[k] - rm[k]) <= 2e-5 * abs(rm[k]) + 1e-12, (k, m[k], rm[k])
    wa_scale = float(np.sum(rw * Aabs)) * max(rm["batch_norm_factor"], 1.0)
    assert abs(m["loss_sum"] - rm["loss_sum"]) <= 2e-5 * wa_scale + 2 * slack_wa + 1e-9
    return mr, ref


def _replay(N, seed=1002):
    r = make_replay(N=N, device="cuda:0", seed=seed)
    return r.lp, r.lq, r.adv


def test_full_size_bench_configuration():
    N = 2_160_000
    print(f"[case] mis full N={N}", flush=True)
    lp, lq, A = _replay(N)
    _check(lp, lq, A, replay_sequences(N).numpy(), dict(MIS_PARAMS))


@pytest.mark.parametrize("level", om.LEVELS)
@pytest.mark.parametrize("mode", om.MODES)
def test_levels_and_modes(level, mode):
    N = 200_003
    print(f"[case] mis level={level} mode={mode} N={N}", flush=True)
    lp, lq, A = _replay(N, seed=7)
    off = replay_sequences(N, seed=7, median=300.0).numpy()
    # bounds inside each statistic's spread on this input, so that every case
    # mixes kept, bounded and rejected tokens (per-sequence sums of d are near
    # -25 here, geometric means of rho near 0.92, sequence means near 0.96)
    tis = {"token": (0.5, 2.0), "sequence": (1e-13, 1e-9), "geometric": (0.9, 0.93)}[level]
    rs_level = {"token": "sequence", "sequence": "geometric", "geometric": "token"}[level]
    rs = {"token": (0.6, 1.4), "sequence": (0.95, 0.99), "geometric": (0.91, 0.94)}[rs_level]
    params = dict(tis_level=level, tis_mode=mode, tis_lower=tis[0], tis_upper=tis[1], use_rs=True,
                  rs_level=rs_level, rs_lower=rs[0], rs_upper=rs[1], veto=0.3,
                  batch_normalize=(mode != "truncate"))
    mr, ref = _check(lp, lq, A, off, params)
    m = ref["metrics"]
    assert 0 < m["kept_tokens"] < N  # the veto and RS reject something
    assert m["catastrophic_seq_fraction"] > 0
    assert 0 < m["tis_fraction_low"] + m["tis_fraction_high"] < 1


@pytest.mark.parametrize("case", ["one_token", "all_single", "one_long", "chunk_edges",
                                  "tail_sizes"])
def test_edge_cases(case):
    print(f"[case] mis edge {case}", flush=True)
    if case == "one_token":
        N, off = 1, np.array([0, 1])
    elif case == "all_single":
        N = 1029
        off = np.arange(N + 1)
    elif case == "one_long":
        N = 100_001
        off = np.array([0, N])
    elif case == "chunk_edges":
        N = 256 * 9
        off = np.array([0, 256, 512, 513, 1024, 1280, 1281, 2048, N])
    else:
        N = 4099
        off = np.array([0, 1, 2, 255, 257, 1000, 4095, 4098, N])
    lp, lq, A = _replay(N, seed=11)
    for params in (dict(MIS_PARAMS),
                   dict(MIS_PARAMS, tis_level="sequence", tis_mode="mask", rs_level="geometric",
                        veto=0.2),
                   dict(MIS_PARAMS, tis_level="token", tis_mode="truncate", use_rs=False,
                        veto=0.0, batch_normalize=False)):
        _check(lp, lq, A, off, params, max_near_frac=1.0)


def test_deterministic():
    N = 300_001
    lp, lq, A = _replay(N, seed=13)
    off = replay_sequences(N, seed=13).numpy()
    mr, w1, f1, _ = _run(lp, lq, A, off, dict(MIS_PARAMS))
    m1 = mr.o["metrics"].clone()
    mr()
    torch.cuda.synchronize()
    assert torch.equal(m1, mr.o["metrics"])
    assert np.array_equal(w1, mr.o["weight"].cpu().numpy())
    assert np.array_equal(f1, mr.o["flags"].cpu().numpy())
