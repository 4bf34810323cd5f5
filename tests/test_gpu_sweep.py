"""Seeded sweep of fused-head configurations against the oracle.

Each seed draws a recipe (no support, a replayed top-p set, or K draws), a
small ragged shape, the loss type, the KL settings, temperature, advantage
scale, normaliser, token chunk and gradient dtype, and compares every output of
rl_loss_fwd_bwd (through the C ABI) with the fp64 oracle to the same bounds as
the fixed cases.  The combinations the fixed tests do not pin down (icepop on
draws with k1 KL and a chunk that splits the tokens unevenly, reinforce with a
temperature on a replayed support, ...) come from here.
"""

import numpy as np
import pytest
import torch

from gpu_util import compare_all, run_head
from oracle import head as ohead
from synth import make_head, policy_ages

needs_gpu = [pytest.mark.gpu,
             pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
RECIPES = ["c3_head16k_ipo", "c4_head16k_ipo_topp_replay", "c5a_head64k_draws_ipo_k1",
           "c5b_head64k_draws_reinforce"]


def draw_config(seed):
    """One configuration, drawn on the host from `seed` alone."""
    rs = np.random.RandomState(seed)
    name = RECIPES[rs.randint(len(RECIPES))]
    shape = dict(N=int(rs.randint(1, 700)), H=int(8 * rs.randint(1, 42)),
                 V=int(rs.randint(1, 4500)), seed=20000 + seed)
    params, kw = {}, {}
    sparse = name == "c5b_head64k_draws_reinforce" and rs.rand() < 0.5
    if sparse:
        params.update(backward="sparse")  # reinforce without KL: the sparse backward
    else:
        params.update(backward="dense",
                      loss_type=["ipo", "icepop", "reinforce"][rs.randint(3)])
        if name in ("c4_head16k_ipo_topp_replay", "c5a_head64k_draws_ipo_k1"):
            # exact KL on the replayed support, k1 on the draws
            params.update(kl_coeff=float(rs.choice([0.0, 0.05, 0.2, 0.2])))
            if params["kl_coeff"] > 0 and rs.rand() < 0.5:
                params.update(kl_staleness="inv_sqrt")
        if rs.rand() < 0.3:
            params.update(entropy_coeff=float(rs.choice([-0.05, 0.03])))
    if params.get("loss_type") == "icepop":
        params.update(icepop_lo=float(rs.choice([0.5, 0.8])), icepop_hi=float(rs.choice([1.5, 2.0])))
    if params.get("loss_type") == "ipo":
        params.update(ipo_eps=float(rs.choice([0.1, 0.3])), max_ratio=float(rs.choice([2.0, 5.0])))
    params.update(inv_temperature=float(rs.choice([1.0, 1.0, 0.8, 1.25])),
                  adv_tau=float(rs.choice([1.0, 0.5])))
    if rs.rand() < 0.3:
        params.update(loss_norm=float(rs.randint(1, 1000)))
    kw["token_chunk"] = int(rs.choice([0, 0, 64, 100, 256]))
    if rs.rand() < 0.25:
        kw["grad_dtype"] = torch.float32
    return name, shape, params, kw


SEEDS = list(range(16))


@pytest.mark.parametrize("seed", SEEDS)
@needs_gpu[0]
@needs_gpu[1]
def test_seeded_configuration(seed):
    name, shape, params, kw = draw_config(seed)
    print(f"[case] sweep seed {seed}: {name} {shape} {params} "
          f"{ {k: str(v) for k, v in kw.items()} }", flush=True)
    wl = make_head(name, device=DEV, **shape)
    wl.params.update(params)
    age = None
    if params.get("kl_staleness") == "inv_sqrt":
        age = policy_ages(wl.N, device=DEV)
    wl.age = age
    _, got = run_head(wl, **kw)
    ref = ohead.from_workload(wl, age=None if age is None else age.cpu().numpy())
    r = compare_all(wl, got, ref, case=f"sweep seed {seed} ({name})")
    print(r)


def test_sweep_covers_the_options():
    """The drawn set spans every recipe, loss type, both backwards, KL on and
    off, staleness, the entropy term, token chunks and an fp32 gradient."""
    cfgs = [draw_config(s) for s in SEEDS]
    assert {c[0] for c in cfgs} == set(RECIPES)
    assert {c[2].get("loss_type") for c in cfgs} >= {"ipo", "icepop", "reinforce"}
    assert {c[2]["backward"] for c in cfgs} == {"dense", "sparse"}
    for r in ("c4_head16k_ipo_topp_replay", "c5a_head64k_draws_ipo_k1"):
        assert any(c[0] == r and c[2].get("kl_coeff", 0) > 0 for c in cfgs)  # exact, k1
    assert any(c[2].get("kl_staleness") == "inv_sqrt" for c in cfgs)
    assert any(c[2].get("entropy_coeff", 0) != 0 for c in cfgs)
    assert any(c[3]["token_chunk"] not in (0,) for c in cfgs)
    assert any(c[3].get("grad_dtype") is torch.float32 for c in cfgs)
