"""Device validation flags against the oracle, bit for bit."""

import numpy as np
import pytest
import torch

from lm_head_logprobs_amd import ops
from lm_head_logprobs_amd import _lib as L
from oracle import validate as ov
from synth import make_head

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _both(V, labels, lq, adv, offsets=None, ids=None, u=None, logq=None, replayed=False):
    st, flags = ops.validate(labels.to(DEV), lq.to(DEV), adv.to(DEV), V, offsets,
                             None if ids is None else ids.to(DEV),
                             None if u is None else u.to(DEV),
                             None if logq is None else logq.to(DEV), replayed)
    ref = ov.validate_reference(V, labels.numpy(), lq.numpy(), adv.numpy(),
                                None if offsets is None else offsets.numpy(),
                                None if ids is None else ids.numpy(),
                                None if u is None else u.numpy(),
                                None if logq is None else logq.numpy(), replayed)
    return st, flags, ref


def test_generated_supports_are_clean():
    for name, kw in (("c4_head16k_ipo_topp_replay", dict(N=200, H=64, V=3000)),
                     ("c5a_head64k_draws_ipo_k1", dict(N=200, H=64, V=3000)),
                     ("c3_head16k_ipo", dict(N=200, H=64, V=3000))):
        wl = make_head(name, device=DEV, **kw)
        st, flags = ops.validate(wl.labels, wl.infer_logprobs, wl.adv, wl.V, wl.offsets, wl.ids,
                                 wl.u, wl.logq, wl.params["replayed"])
        assert (st, flags) == (L.RL_OK, 0), (name, flags)


def _base():
    labels = torch.tensor([3, 7, 9], dtype=torch.int32)
    lq = torch.log(torch.tensor([0.5, 0.25, 1.0]))
    adv = torch.tensor([1.0, -1.0, 0.5])
    offsets = torch.tensor([0, 2, 4, 5], dtype=torch.int64)
    ids = torch.tensor([3, 4, 7, 8, 9], dtype=torch.int32)
    u = torch.tensor([0.5, 0.5, 0.25, 0.75, 1.0])
    return dict(V=50, labels=labels, lq=lq, adv=adv, offsets=offsets, ids=ids, u=u,
                logq=torch.log(u), replayed=True)


MUTATIONS = [
    ("labels", 1, 50), ("labels", 0, -1), ("ids", 2, 99), ("u", 3, -0.1), ("u", 3, float("nan")),
    ("logq", 0, float("inf")), ("logq", 0, 0.1), ("lq", 2, float("nan")), ("lq", 2, 0.5),
    ("u", 0, 0.4), ("labels", 2, 8), ("adv", 0, float("inf")),
]


@pytest.mark.parametrize("field,i,val", MUTATIONS)
def test_flags_match_oracle(field, i, val):
    d = _base()
    d[field] = d[field].clone()
    d[field][i] = val
    st, flags, ref = _both(**d)
    assert flags == ref and ref != 0
    assert st == L.RL_E_INVALID_INPUT


def test_device_offsets_checked_on_device():
    # the host copy is valid, the device copy is corrupted
    d = _base()
    labels, lq, adv = d["labels"].to(DEV), d["lq"].to(DEV), d["adv"].to(DEV)
    bad_dev = torch.tensor([0, 5, 4, 5], dtype=torch.int64, device=DEV)
    flags = torch.zeros(1, dtype=torch.int32, device=DEV)
    st, f = L.rl_validate_support_sync(3, 50, 5, labels, lq, adv, d["offsets"], bad_dev,
                                       d["ids"].to(DEV), d["u"].to(DEV), None, 1, flags)
    ref = ov.validate_reference(50, d["labels"].numpy(), d["lq"].numpy(), d["adv"].numpy(),
                                bad_dev.cpu().numpy(), d["ids"].numpy(), d["u"].numpy(), None, True)
    assert f == ref
    assert f & 0x100  # RL_BAD_OFFSETS
    assert st == L.RL_E_INVALID_INPUT
