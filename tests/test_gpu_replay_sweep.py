"""Seeded sweep of loss-only replay configurations against the oracle.

The fixed replay tests use the recipe's five IPO thresholds; the kernel is
compiled once per threshold count (1 to 8).  Each seed here draws a count (the
eight seeds take every count once), sorted thresholds, the max ratio, the
IcePop band, the PPO clip range and dual-clip constant, the TIS bound and a
ragged token count, and checks every output with the same bounds as the fixed
tests.
"""

import numpy as np
import pytest
import torch

import test_gpu_replay as tr
from synth import make_replay

DEV = "cuda:0"
SEEDS = list(range(8))


def draw_params(seed):
    """Replay settings and token count, drawn on the host from `seed` alone."""
    rs = np.random.RandomState(100 + seed)
    n_eps = seed % 8 + 1
    eps = tuple(float(x) for x in np.sort(rs.uniform(0.01, 0.6, n_eps)))
    params = dict(eps=eps, primary_eps_index=int(rs.randint(n_eps)),
                  max_ratio=float(rs.choice([1.5, 2.0, 5.0])),
                  icepop_lo=float(rs.uniform(0.3, 0.9)), icepop_hi=float(rs.uniform(1.1, 3.0)),
                  clip_low=float(rs.uniform(0.1, 0.3)), clip_high=float(rs.uniform(0.1, 0.4)),
                  clip_c=float(rs.uniform(2.0, 5.0)), tis_upper=float(rs.uniform(1.2, 4.0)))
    N = int(rs.randint(1, 400_000))
    return N, params


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
@pytest.mark.parametrize("seed", SEEDS)
def test_seeded_replay(seed):
    N, params = draw_params(seed)
    print(f"[case] replay sweep seed {seed}: N={N} {params}", flush=True)
    r = make_replay(N=N, device=DEV, seed=3000 + seed)
    r.params = params
    _, got = tr._run(r)
    tr.check_replay(r, got)


def test_replay_sweep_covers_every_threshold_count():
    counts = sorted(len(draw_params(s)[1]["eps"]) for s in SEEDS)
    assert counts == list(range(1, 9))
    for s in SEEDS:
        N, p = draw_params(s)
        assert 1 <= N < 400_000 and 0 <= p["primary_eps_index"] < len(p["eps"])
        assert list(p["eps"]) == sorted(p["eps"]) and p["icepop_lo"] < 1 < p["icepop_hi"]
