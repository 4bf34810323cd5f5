"""Helpers of the GPU parity tests: run the HIP path, compare with the oracle.

Tolerances (stated by the workload description): per-token log-probs within
2e-3 absolute, loss within 1e-4 relative, dh and dW within 1e-2 relative
Frobenius error, masks bit-exact except decisions that lie within a band of
their threshold (counted and reported).  Entropy uses the log-prob tolerance.

Near-threshold accounting.  A decision's margin is the oracle's distance of
the compared quantity from its threshold (|P - Q| against eps for IPO, the
ratio against the band edges for IcePop).  The kernel forms log p from fp32
logits, whose rounding grows with the logits' magnitude, and from an fp32
log-sum-exp.  Measured (u = 2^-24): at full size the log-prob error stays
below 12.5 u max_v |z_v| (16384 tokens each of the 16k and 16k top-p
workloads; logits up to 1.8e3 in magnitude on the top-p workload's sharpest
tokens), and with logits near zero below 24 u (the log-sum-exp's own
rounding).  A decision on P or on the ratio r = p/q moves by P or r times
that error, so a token's band is max(1e-6, C_BAND u (max|z| + 2) max(P, r))
with C_BAND = 32 (at least 2.5 times either measurement): about 1e-5 on
tokens whose logits stay below 4 in magnitude, wider on sharp ones.
Decisions with a margin of at most 1e-6 (the stated band) and those in
(1e-6, band] are counted separately, with how many of each actually differ;
every decision beyond its band must agree.  Every comparison appends its
figures to a JSON-lines report: the file RL_PARITY_REPORT names, by default
rl_parity_report.jsonl in the temp directory; tests/parity_summary.py turns
it into a table.
"""

from __future__ import annotations

import json
import os
import tempfile

import numpy as np
import torch

from lm_head_logprobs_amd import ops
from oracle import head as ohead

TOL_LP = 2e-3
TOL_LOSS = 1e-4
TOL_GRAD = 1e-2
NS_BAND = 1e-6   # the stated near-threshold band
C_BAND = 32.0    # decision band: max(NS_BAND, C_BAND u (max|z| + 2) max(P, r))
U32 = 2.0**-24

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# Where the parity tests append their per-case figures (JSON lines): set
# RL_PARITY_REPORT to keep them; by default they go to the temp directory.
REPORT = os.environ.get("RL_PARITY_REPORT",
                        os.path.join(tempfile.gettempdir(), "rl_parity_report.jsonl"))


def record(case, rep):
    """Append one case's figures to the parity report."""
    os.makedirs(os.path.dirname(REPORT), exist_ok=True)
    row = {"case": case}
    for k, v in rep.items():
        row[k] = v.item() if isinstance(v, np.generic) else v
    with open(REPORT, "a") as f:
        f.write(json.dumps(row) + "\n")


def to_np(t):
    if t is None:
        return None
    return t.detach().double().cpu().numpy() if t.dtype != torch.uint8 else t.cpu().numpy()


def run_head(wl, **kw):
    fh = ops.FusedHead(wl.h, wl.W, wl.labels, wl.infer_logprobs, wl.adv, wl.params,
                       wl.offsets, wl.ids, wl.u, wl.logq, age=getattr(wl, "age", None), **kw)
    fh()
    torch.cuda.synchronize()
    return fh, {k: to_np(v) for k, v in fh.o.items()}


def _margins(lp, lq, params):
    """Distance of each weight decision from its threshold (oracle values),
    and the factor by which a log-prob error moves the decided quantity."""
    lp = np.asarray(lp, np.float64)
    lq = np.asarray(lq, np.float64)
    t = params["loss_type"]
    if t == "ipo":
        P = np.exp(lp)
        return np.abs(np.abs(P - np.exp(lq)) - params["ipo_eps"]), P
    if t == "icepop":
        r = np.exp(lp - lq)
        return np.minimum(np.abs(r - params.get("icepop_lo", 0.5)),
                          np.abs(r - params.get("icepop_hi", 2.0))), r
    return np.full(lp.shape, np.inf), np.zeros(lp.shape)


def _band(zmax_abs, scale):
    return np.maximum(NS_BAND, C_BAND * U32 * (np.asarray(zmax_abs) + 2.0) * np.asarray(scale))


def near_threshold(wl, ref, tokens=None):
    """Token mask of label decisions near a threshold, and the loss bound they
    can move (sum of |s w lp| / D over near labels and near entries)."""
    d = wl.to_host_numpy()
    tok = np.arange(wl.N) if tokens is None else np.asarray(tokens)
    lq = d["infer_logprobs"][tok].astype(np.float64)
    margin, scale = _margins(ref["logprobs"], lq, wl.params)
    band = _band(ref["zmax_abs"], scale)
    near_lab = margin <= band
    s = d["adv"][tok].astype(np.float64) * wl.params.get("adv_tau", 1.0)
    D = wl.params["loss_norm"]
    M = wl.params.get("max_ratio", 5.0)
    bound = np.sum(np.abs(s[near_lab]) * max(M, 1.0) * np.abs(ref["logprobs"][near_lab])) / D
    near_tok = near_lab.copy()
    n_entries = 0
    if wl.offsets is not None and "support_entries" in ref:
        ent = ref["support_entries"]
        lq_e = (np.log(d["u"][ent].astype(np.float64)) if d["logq"] is None
                else d["logq"][ent].astype(np.float64))
        off = d["offsets"]
        rows = np.searchsorted(off, ent, side="right") - 1
        pos = {t: i for i, t in enumerate(tok)}
        m_e, sc_e = _margins(ref["support_logprobs"], lq_e, wl.params)
        zrow = ref["zmax_abs"][np.array([pos[t] for t in rows], np.int64)] if len(ent) else []
        near_e = m_e <= _band(zrow, sc_e)
        n_entries = int(near_e.sum())
        if n_entries:
            for e_i in np.nonzero(near_e)[0]:
                i = pos[rows[e_i]]
                near_tok[i] = True
                bound += (abs(s[i]) * d["u"][ent[e_i]] * max(M, 1.0)
                          * abs(ref["support_logprobs"][e_i]) / D)
    return near_tok, bound, int(near_lab.sum()), n_entries, margin, band


def rel_fro(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def compare_forward(wl, got, ref, tokens=None, report=None):
    tok = np.arange(wl.N) if tokens is None else np.asarray(tokens)
    near, bound, n_lab, n_ent, margin, band = near_threshold(wl, ref, tokens)
    ok = ~near
    r = {} if report is None else report
    r["tokens_compared"] = int(len(tok))
    r["band_rule"] = f"max({NS_BAND:g}, {C_BAND:g} u (max|z| + 2) max(P, r))"
    r["band_max"], r["band_median"] = float(band.max()), float(np.median(band))
    r["near_labels"], r["near_entries"] = n_lab, n_ent
    lp_err = np.max(np.abs(got["logprobs"][tok] - ref["logprobs"]))
    ent_err = np.max(np.abs(got["entropy"][tok] - ref["entropy"]))
    r["max_lp_err"], r["max_entropy_err"] = float(lp_err), float(ent_err)
    r["max_lp_err_over_u_zmax"] = float(np.max(np.abs(got["logprobs"][tok] - ref["logprobs"]) /
                                              (U32 * np.maximum(ref["zmax_abs"], 1e-30))))
    r["max_lp_err_over_u_zmax2"] = float(np.max(np.abs(got["logprobs"][tok] - ref["logprobs"]) /
                                               (U32 * (ref["zmax_abs"] + 2.0))))
    assert lp_err <= TOL_LP, r
    assert ent_err <= TOL_LP, r
    # the bands below assume the log-prob error stays within the rounding model
    assert r["max_lp_err_over_u_zmax2"] <= C_BAND, r
    keep_got = got["keep"][tok].astype(bool)
    differ = keep_got != ref["keep"]
    in_ns = margin <= NS_BAND
    in_band = (margin > NS_BAND) & (margin <= band)
    r["labels_within_1e-6"], r["labels_within_1e-6_differing"] = int(in_ns.sum()), int(
        (differ & in_ns).sum())
    r["labels_in_(1e-6,band]"], r["labels_in_(1e-6,band]_differing"] = int(in_band.sum()), int(
        (differ & in_band).sum())
    r["labels_beyond_band_differing"] = int((differ & ~near).sum())
    r["min_label_margin"] = float(margin.min()) if margin.size else None
    assert np.array_equal(keep_got[ok], ref["keep"][ok]), r
    w_err = np.abs(got["weight"][tok] - ref["weight"])[ok]
    assert np.all(w_err <= 5e-3 * np.maximum(np.abs(ref["weight"][ok]), 1.0)), r
    tl_err = np.abs(got["token_loss"][tok] - ref["token_loss"])[ok]
    r["max_token_loss_err"] = float(tl_err.max()) if tl_err.size else 0.0
    assert np.all(tl_err <= 1e-3 * np.abs(ref["token_loss"][ok]) + 2e-3), r
    if "support_logprobs" in got and "support_entries" in ref:
        sl = np.abs(got["support_logprobs"][ref["support_entries"]] - ref["support_logprobs"])
        r["max_support_lp_err"] = float(sl.max()) if sl.size else 0.0
        assert r["max_support_lp_err"] <= TOL_LP, r
    return near, bound


def grad_floors(wl, ref):
    """Absolute error floors of dh and dW from rounding the dense operand
    G = dL/dz to the compute dtype.  G holds the softmax part kappa_t p_t and
    the label and support coefficients (-s_t w_t at the label, s_t c_e -
    beta_t u_e at each entry), all divided by D, so a token's row of G sums in
    absolute value to at most (|kappa_t| + |s_t w_t| + sum_e |s_t c_e -
    beta_t u_e|) / D.  It is rounded up to three times (the softmax part, plus
    the label, plus a run of support entries), 2^-9 relative each in bf16
    (2^-24 in fp32); doubled for margin: |dG_t W| <= eps k_t max_v |W_v| and
    |dG^T h|_F <= sum_t eps k_t |h_t|.  They matter only when the exact
    gradient is (near) zero, e.g. a one-word vocabulary."""
    eps = 2.0**-7 if wl.dtype == "bf16" else 2.0**-22
    d = wl.to_host_numpy()
    prm = wl.params
    D = prm["loss_norm"]
    s = np.abs(d["adv"].astype(np.float64)) * abs(prm.get("adv_tau", 1.0))
    su = np.zeros(wl.N)
    if d["offsets"] is not None:
        u = d["u"].astype(np.float64)
        su = np.add.reduceat(np.concatenate([u, [0.0]]), d["offsets"][:-1]) * (
            np.diff(d["offsets"]) > 0)
    wmax = max(prm.get("max_ratio", 5.0), prm.get("icepop_hi", 2.0), 1.0)
    beta = ohead.beta_per_token(prm, np.zeros(wl.N) if getattr(wl, "age", None) is None
                                else to_np(wl.age))
    k = (np.abs(ref["kappa"]) + s * np.abs(ref["weight"]) + s * wmax * su + beta * su)
    k = k / D * prm.get("inv_temperature", 1.0)
    Wn = np.max(np.linalg.norm(d["W"].astype(np.float64), axis=1))
    hn = np.linalg.norm(d["h"].astype(np.float64), axis=1)
    # dW: the worst case adds the tokens' rounding errors (a sum over tokens);
    # independent roundings add in quadrature (a root-sum-square), which is
    # what decides whether the exact gradient is below the rounding level
    return (eps * np.sqrt(np.sum(k**2)) * Wn,
            (eps * np.sum(k * hn), eps * np.sqrt(np.sum((k * hn)**2))))


def check_grad(name, got, ref, floor, r):
    """Relative Frobenius error within TOL_GRAD.  Only when the exact gradient
    is itself no larger than the rounding level of the dense operand (a
    gradient that vanishes, e.g. a one-word vocabulary) is the absolute floor
    added.  floor: one bound, or (worst-case bound, rounding level)."""
    bound, level = floor if isinstance(floor, tuple) else (floor, floor)
    nref = float(np.linalg.norm(ref))
    err = float(np.linalg.norm(got - ref))
    r[name + "_rel"] = err / max(nref, 1e-300)
    r[name + "_floor_used"] = nref <= level
    assert err <= TOL_GRAD * nref + (bound if nref <= level else 0.0), r


def compare_all(wl, got, ref, report=None, case=None):
    r = {} if report is None else report
    near, bound = compare_forward(wl, got, ref, report=r)
    loss_err = abs(got["loss"][0] - ref["loss"])
    r["loss"], r["loss_ref"], r["loss_err"] = float(got["loss"][0]), float(ref["loss"]), loss_err
    r["loss_rel_err"] = loss_err / max(abs(float(ref["loss"])), 1e-300)
    assert loss_err <= TOL_LOSS * abs(ref["loss"]) + bound + 1e-7, r
    f_dh, f_dW = grad_floors(wl, ref)
    if "dh" in got:
        check_grad("dh", got["dh"], ref["dh"], f_dh, r)
    if "dW" in got:
        check_grad("dW", got["dW"], ref["dW"], f_dW, r)
    m = dict(zip(ohead.METRIC_NAMES, got["metrics"]))
    for k in ("kl", "support_mass", "entropy_mean", "kl_age0"):
        assert abs(m[k] - ref["metrics"][k]) <= 1e-3 * abs(ref["metrics"][k]) + 1e-5, (k, m, r)
    if wl.params.get("kl_staleness", "none") == "none":
        assert m["kl_beta"] == np.float32(ref["metrics"]["kl_beta"])
    else:  # a mean of fp32 reciprocal square roots
        assert abs(m["kl_beta"] - ref["metrics"]["kl_beta"]) <= 1e-5 * ref["metrics"]["kl_beta"]
    n_near = int(near.sum())
    for k in ("masked_fraction", "mask_tv"):
        assert abs(m[k] - ref["metrics"][k]) <= (n_near + 0.5) / wl.N, (k, m, r)
    if case is not None:
        record(case, r)
    return r
