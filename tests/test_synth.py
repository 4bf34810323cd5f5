"""The seeded input generators: determinism and the recipe's distributions."""

import math

import numpy as np
import torch

from synth import make_head, make_replay


def test_head_generator_is_deterministic():
    a = make_head("c4_head16k_ipo_topp_replay", N=40, H=32, V=700)
    b = make_head("c4_head16k_ipo_topp_replay", N=40, H=32, V=700)
    for k in ("h", "W", "labels", "infer_logprobs", "adv", "offsets", "ids", "u", "logq"):
        assert torch.equal(getattr(a, k), getattr(b, k)), k
    c = make_head("c4_head16k_ipo_topp_replay", N=40, H=32, V=700, seed=7)
    assert not torch.equal(a.h, c.h)


def test_topp_support_recipe():
    wl = make_head("c4_head16k_ipo_topp_replay", N=200, H=64, V=3000)
    off = wl.offsets.numpy()
    sizes = np.diff(off)
    assert sizes.min() >= 1 and off[-1] == wl.ids.numel()
    u = wl.u.double().numpy()
    for t in range(wl.N):
        e0, e1 = off[t], off[t + 1]
        assert abs(u[e0:e1].sum() - 1.0) < 1e-4
        assert wl.labels[t].item() in set(wl.ids[e0:e1].tolist())
        j = wl.ids[e0:e1].tolist().index(wl.labels[t].item())
        assert wl.infer_logprobs[t].item() == wl.logq[e0 + j].item()
    # long-tailed sizes around the target median 30
    assert 10 <= np.median(sizes) <= 90
    assert wl.h.dtype == torch.bfloat16 and wl.W.dtype == torch.bfloat16


def test_draws_support_recipe():
    wl = make_head("c5a_head64k_draws_ipo_k1", N=64, H=32, V=500)
    assert wl.offsets.tolist() == list(range(0, 65 * 16, 16))
    assert torch.all(wl.u == 1.0 / 16)
    assert torch.all(wl.logq <= 0)
    assert wl.ids.min() >= 0 and wl.ids.max() < 500


def test_tiny_config_distributions():
    wl = make_head("c1_tiny_fp32_ipo")
    assert (wl.N, wl.H, wl.V) == (64, 64, 1000) and wl.h.dtype == torch.float32
    assert abs(wl.W.std().item() - 1 / math.sqrt(64)) < 0.01
    assert wl.offsets is None
    assert torch.all(wl.infer_logprobs <= 0)


def test_replay_generator_recipe():
    r = make_replay(N=200_000)
    lq = r.lq.double().numpy()
    lp = r.lp.double().numpy()
    assert np.all(lq <= 0) and np.all(lp <= 0)
    near = -lq < 0.5
    # 60% of the mixture has mean 0.05, 40% mean 3
    assert abs(-lq.mean() - (0.6 * 0.05 + 0.4 * 3.0)) < 0.03
    assert 0.55 < near.mean() < 0.72
    assert r.info["clamped_to_zero"] > 0
    assert torch.equal(make_replay(N=1000).lp, make_replay(N=1000).lp)


def test_replay_sequences_recipe():
    from synth import replay_sequences
    off = replay_sequences(2_160_000)
    n = torch.diff(off)
    assert int(off[0]) == 0 and int(off[-1]) == 2_160_000
    assert int(n.min()) >= 1 and int(n.max()) <= 32768
    # lognormal with median 1024 and sigma_log 1: the sample median is near 1024
    assert 900 < float(n[:-1].double().median()) < 1160
    assert torch.equal(off, replay_sequences(2_160_000))
    small = replay_sequences(10)
    assert int(small[-1]) == 10 and torch.all(torch.diff(small) >= 1)
