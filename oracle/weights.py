"""Per-token importance weights w(p, q) of the three RL loss types (fp64).

Source: prime-rl pull request 4233 (one RLLoss for ipo, icepop, reinforce),
section "What changes", first bullet: the types differ only in w --
  ipo:       1(|p - q| <= eps) * min(p/q, max_importance_ratio)
  icepop:    1(low <= p/q <= high) * p/q
  reinforce: 1
and the IPO documentation page, section "Masking by Probability, Not Ratio":
IPO masks a token when |pi_train(y) - pi_infer(y)| > eps, IcePop when the
ratio pi_train/pi_infer leaves a fixed band.

Inputs are log-probabilities; p = exp(lp), q = exp(lq), and the ratio is
formed as exp(lp - lq).  Ties keep the token (|p - q| = eps is kept, the band
is closed on both ends).
"""

import numpy as np

LOSS_TYPES = ("ipo", "icepop", "reinforce")


def ratio(lp, lq):
    return np.exp(np.asarray(lp, np.float64) - np.asarray(lq, np.float64))


def ipo_keep(lp, lq, eps):
    P = np.exp(np.asarray(lp, np.float64))
    Q = np.exp(np.asarray(lq, np.float64))
    return np.abs(P - Q) <= eps


def icepop_keep(lp, lq, lo, hi):
    r = ratio(lp, lq)
    return (lo <= r) & (r <= hi)


def weight(lp, lq, params):
    """Return (w, keep) for the loss type in ``params``.

    params keys: loss_type, ipo_eps, max_ratio, icepop_lo, icepop_hi.
    """
    t = params["loss_type"]
    lp = np.asarray(lp, np.float64)
    lq = np.asarray(lq, np.float64)
    if t == "ipo":
        keep = ipo_keep(lp, lq, params["ipo_eps"])
        w = np.where(keep, np.minimum(ratio(lp, lq), params["max_ratio"]), 0.0)
    elif t == "icepop":
        keep = icepop_keep(lp, lq, params.get("icepop_lo", 0.5), params.get("icepop_hi", 2.0))
        w = np.where(keep, ratio(lp, lq), 0.0)
    elif t == "reinforce":
        keep = np.ones(np.broadcast(lp, lq).shape, dtype=bool)
        w = np.ones(keep.shape, np.float64)
    else:
        raise ValueError(f"unknown loss type {t!r}")
    return w, keep
