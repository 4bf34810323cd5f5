"""Pins of the sampler-evidence validation oracle: one crafted violation per bit."""

import numpy as np
import pytest

from oracle import validate as ov


def _good(replayed=True):
    V = 50
    labels = np.array([3, 7, 9], np.int32)
    lq = np.log(np.array([0.5, 0.25, 1.0], np.float32))
    adv = np.array([1.0, -1.0, 0.5], np.float32)
    offsets = np.array([0, 2, 4, 5], np.int64)
    ids = np.array([3, 4, 7, 8, 9], np.int32)
    u = np.array([0.5, 0.5, 0.25, 0.75, 1.0], np.float32)
    logq = np.log(u)
    return dict(V=V, labels=labels, infer_logprobs=lq, adv=adv, offsets=offsets, ids=ids,
                u=u, logq=logq, replayed=replayed)


def test_clean_support_has_no_flags():
    assert ov.validate_reference(**_good()) == 0
    assert ov.validate_reference(**_good(replayed=False)) == 0


@pytest.mark.parametrize("mutate,bit", [
    (lambda d: d["labels"].__setitem__(1, 50), ov.BAD_LABEL | ov.BAD_REPLAY_LABEL),
    (lambda d: d["labels"].__setitem__(0, -1), ov.BAD_LABEL | ov.BAD_REPLAY_LABEL),
    (lambda d: d["ids"].__setitem__(2, 99), ov.BAD_ID | ov.BAD_REPLAY_LABEL),
    (lambda d: d["u"].__setitem__(3, -0.1), ov.BAD_U | ov.BAD_REPLAY_MASS),
    (lambda d: d["u"].__setitem__(3, np.nan), ov.BAD_U | ov.BAD_REPLAY_MASS),
    (lambda d: d["logq"].__setitem__(0, np.inf), ov.BAD_LOGQ),
    (lambda d: d["logq"].__setitem__(0, 0.1), ov.BAD_LOGQ),
    (lambda d: d["infer_logprobs"].__setitem__(2, np.nan), ov.BAD_INFER_LOGPROB),
    (lambda d: d["infer_logprobs"].__setitem__(2, 0.5), ov.BAD_INFER_LOGPROB),
    (lambda d: d["u"].__setitem__(0, 0.4), ov.BAD_REPLAY_MASS),
    (lambda d: d["labels"].__setitem__(2, 8), ov.BAD_REPLAY_LABEL),
    (lambda d: d["adv"].__setitem__(0, np.inf), ov.BAD_ADV),
    (lambda d: d["offsets"].__setitem__(1, 5), ov.BAD_OFFSETS | ov.BAD_REPLAY_MASS),
    (lambda d: d["offsets"].__setitem__(3, 4), ov.BAD_OFFSETS),
])
def test_each_violation_sets_its_bit(mutate, bit):
    d = _good()
    mutate(d)
    assert ov.validate_reference(**d) == bit


def test_mass_tolerance_edges():
    d = _good()
    d["u"] = d["u"].copy()
    d["u"][0] = np.float32(0.5 + 5e-4)  # within 1e-3
    assert ov.validate_reference(**d) == 0
    d["u"][0] = np.float32(0.5 + 2e-3)
    assert ov.validate_reference(**d) == ov.BAD_REPLAY_MASS
