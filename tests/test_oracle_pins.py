"""Pins of the CPU oracle against facts the pages and the mathematics fix.

Each test names the pin it applies.  None of them call the HIP library.
"""

import math
import os

import numpy as np
import pytest
import scipy.special as sps
import scipy.stats as sst
from scipy.spatial import distance

from oracle import head as ohead
from oracle import replay as oreplay
from oracle import weights as ow

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _params(**kw):
    p = dict(loss_type="ipo", ipo_eps=0.3, max_ratio=5.0, icepop_lo=0.5, icepop_hi=2.0,
             adv_tau=1.0, kl_coeff=0.0, kl_estimator="none", inv_temperature=1.0, loss_norm=1.0)
    p.update(kw)
    return p


# ---------------------------------------------------------------- weights ----

def _worked_examples():
    rows = []
    with open(os.path.join(GOLDEN, "worked_examples.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([float(x) for x in line.split()])
    return rows


def test_worked_examples_from_ipo_page():
    rows = _worked_examples()
    assert len(rows) == 2
    for (pt, qi, ratio, moved, lo, hi, band_kept, eps, ipo_kept, M, w_ipo, w_band) in rows:
        lp, lq = math.log(pt), math.log(qi)
        assert ow.ratio(lp, lq) == pytest.approx(ratio, rel=1e-12)
        assert abs(pt - qi) == pytest.approx(moved, abs=1e-12)
        assert bool(ow.icepop_keep(lp, lq, lo, hi)) == bool(band_kept)
        assert bool(ow.ipo_keep(lp, lq, eps)) == bool(ipo_kept)
        w, keep = ow.weight(lp, lq, _params(loss_type="ipo", ipo_eps=eps, max_ratio=M))
        assert bool(keep) == bool(ipo_kept)
        assert float(w) == pytest.approx(w_ipo, rel=1e-12)
        w, keep = ow.weight(lp, lq, _params(loss_type="icepop", icepop_lo=lo, icepop_hi=hi))
        assert float(w) == pytest.approx(w_band, rel=1e-12)
        w, keep = ow.weight(lp, lq, _params(loss_type="reinforce"))
        assert float(w) == 1.0 and bool(keep)


def test_ipo_mask_is_two_outcome_total_variation():
    # IPO page: |p - q| is the total-variation distance of the split
    # {this token, everything else}.  TV computed by scipy's L1 distance.
    rng = np.random.default_rng(0)
    P = rng.uniform(1e-4, 1 - 1e-4, 4000)
    Q = rng.uniform(1e-4, 1 - 1e-4, 4000)
    for eps in (0.05, 0.1, 0.3, 0.5):
        keep = ow.ipo_keep(np.log(P), np.log(Q), eps)
        tv = np.array([0.5 * distance.cityblock([p, 1 - p], [q, 1 - q]) for p, q in zip(P, Q)])
        margin = np.abs(tv - eps) > 1e-12
        assert np.array_equal(keep[margin], (tv <= eps)[margin])


def test_threshold_ties_keep():
    # Reading: ties keep (closed band, |p - q| = eps kept).
    lp, lq = np.log(0.5), np.log(0.25)
    assert bool(ow.icepop_keep(lp, lq, 0.5, 2.0))  # ratio exactly 2
    assert bool(ow.icepop_keep(lq, lp, 0.5, 2.0))  # ratio exactly 0.5
    assert bool(ow.ipo_keep(np.log(0.75), np.log(0.5), 0.25))


# ----------------------------------------------------- head: forward pins ----

def _tiny_problem(seed, N=6, H=5, V=11, support="draws", K=4, scale=1.0):
    rng = np.random.default_rng(seed)
    h = rng.normal(size=(N, H))
    W = rng.normal(size=(V, H)) * scale
    labels = rng.integers(0, V, N)
    lq = -rng.exponential(1.5, N)
    adv = rng.normal(size=N)
    if support is None:
        return h, W, labels, lq, adv, None, None, None, None
    sizes = rng.integers(0, K + 1, N) if support == "ragged" else np.full(N, K)
    offsets = np.concatenate([[0], np.cumsum(sizes)])
    nnz = int(offsets[-1])
    ids = rng.integers(0, V, nnz)
    u = rng.uniform(0.05, 1.0, nnz)
    logq = -rng.exponential(1.0, nnz)
    return h, W, labels, lq, adv, offsets, ids, u, logq


def test_uniform_logits_closed_form():
    # W = 0: every logit is 0, so log p(v) = -log V and the entropy is log V.
    # With constant log p the loss is a closed form of the inputs:
    #  loss_t = -s (w - sum_e c_e)(-log V) + beta sum_e u_e (lq_e + log V).
    N, H, V = 5, 3, 17
    h, _, labels, lq, adv, offsets, ids, u, logq = _tiny_problem(1, N, H, V, support="ragged")
    W = np.zeros((V, H))
    for lt, est in (("ipo", "k1"), ("icepop", "exact"), ("reinforce", "k1")):
        prm = _params(loss_type=lt, kl_coeff=0.2, kl_estimator=est, adv_tau=0.7, loss_norm=3.0,
                      icepop_lo=0.01, icepop_hi=50.0)
        out = ohead.head_reference(h, W, labels, lq, adv, prm, offsets, ids, u, logq)
        lV = math.log(V)
        assert np.allclose(out["logprobs"], -lV, rtol=0, atol=1e-14)
        assert np.allclose(out["entropy"], lV, rtol=0, atol=1e-13)
        expect = []
        for t in range(N):
            P = 1.0 / V
            Q = math.exp(lq[t])
            r = P / Q
            if lt == "ipo":
                w = min(r, 5.0) if abs(P - Q) <= 0.3 else 0.0
            elif lt == "icepop":
                w = r if 0.01 <= r <= 50.0 else 0.0
            else:
                w = 1.0
            sc, kl = 0.0, 0.0
            for e in range(offsets[t], offsets[t + 1]):
                Qe = math.exp(logq[e])
                re = P / Qe
                if lt == "ipo":
                    we = min(re, 5.0) if abs(P - Qe) <= 0.3 else 0.0
                elif lt == "icepop":
                    we = re if 0.01 <= re <= 50.0 else 0.0
                else:
                    we = 1.0
                sc += u[e] * we
                kl += u[e] * (logq[e] + lV)
            s = 0.7 * adv[t]
            expect.append(-s * (w - sc) * (-lV) + 0.2 * kl)
        assert np.allclose(out["token_loss"], expect, rtol=1e-13, atol=1e-13)
        assert out["loss"] == pytest.approx(sum(expect) / 3.0, rel=1e-13)


def test_logsumexp_and_entropy_match_scipy():
    # Textbook log-sum-exp and Shannon entropy, computed by scipy.
    h, W, labels, lq, adv, *_ = _tiny_problem(2, N=7, H=9, V=300, support=None, scale=3.0)
    prm = _params(inv_temperature=0.8)
    out = ohead.head_reference(h, W, labels, lq, adv, prm)
    z = 0.8 * (h @ W.T)
    assert np.allclose(out["lse"], sps.logsumexp(z, axis=1), rtol=1e-14, atol=1e-12)
    assert np.allclose(out["entropy"], sst.entropy(sps.softmax(z, axis=1), axis=1),
                       rtol=1e-12, atol=1e-12)
    lp_lib = sps.log_softmax(z, axis=1)[np.arange(len(labels)), labels]
    assert np.allclose(out["logprobs"], lp_lib, rtol=1e-14, atol=1e-12)


def test_lse_direct_summation_on_tiny_config_shape():
    # Direct fp64 summation of exp(z) (no max shift) at the tiny workload's
    # shape (64 x 64 x 1000, W ~ N(0, 1/H)) agrees with the shifted form.
    rng = np.random.default_rng(3)
    N, H, V = 64, 64, 1000
    h = rng.normal(size=(N, H))
    W = rng.normal(size=(V, H)) / math.sqrt(H)
    labels = rng.integers(0, V, N)
    out = ohead.head_reference(h, W, labels, -np.ones(N), rng.normal(size=N), _params())
    z = h @ W.T
    direct = np.log(np.exp(z).sum(axis=1))
    assert np.allclose(out["lse"], direct, rtol=1e-14, atol=1e-13)


def test_exact_kl_equals_dense_kl_on_full_support():
    # PR 4233 validation bullet: the KL over a replayed support against a
    # dense KL.  Full-vocabulary replay (u = q over all V): sum_e u_e (log q - log p)
    # equals KL(q || p) computed densely by scipy's relative entropy.
    rng = np.random.default_rng(4)
    N, H, V = 4, 6, 40
    h = rng.normal(size=(N, H))
    W = rng.normal(size=(V, H))
    y = h @ W.T + rng.normal(size=(N, V)) * 0.5
    q = sps.softmax(y, axis=1)
    offsets = np.arange(N + 1) * V
    ids = np.tile(np.arange(V), N)
    u = q.reshape(-1)
    logq = sps.log_softmax(y, axis=1).reshape(-1)
    labels = rng.integers(0, V, N)
    prm = _params(kl_coeff=1.0, kl_estimator="exact")
    out = ohead.head_reference(h, W, labels, logq.reshape(N, V)[np.arange(N), labels],
                               np.zeros(N), prm, offsets, ids, u, logq)
    p = sps.softmax(h @ W.T, axis=1)
    dense = sps.rel_entr(q, p).sum(axis=1)
    assert np.allclose(out["kl"], dense, rtol=1e-12, atol=1e-13)
    assert np.allclose(out["token_loss"], dense, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------- head: gradient pins ----

def _frozen_loss(h, W, labels, adv, prm, offsets, ids, u, logq, w_lab, c_e, lq_e, age=None):
    """The loss with every importance weight frozen, written with scipy's log_softmax
    and entropy (scipy.special.entr); beta_t = kl_coeff / sqrt(1 + age_t) when
    kl_staleness is inv_sqrt."""
    inv_t = prm["inv_temperature"]
    zz = inv_t * (h @ W.T)
    lps = sps.log_softmax(zz, axis=1)
    ent = sps.entr(sps.softmax(zz, axis=1)).sum(axis=1)
    gamma = prm.get("entropy_coeff", 0.0)
    total = 0.0
    for t in range(len(labels)):
        beta = ohead.kl_beta(prm)
        if prm.get("kl_staleness", "none") == "inv_sqrt":
            beta /= math.sqrt(1.0 + age[t])
        s = prm["adv_tau"] * adv[t]
        term = w_lab[t] * lps[t, labels[t]]
        kl = 0.0
        if offsets is not None:
            for e in range(offsets[t], offsets[t + 1]):
                term -= c_e[e] * lps[t, ids[e]]
                kl += u[e] * (lq_e[e] - lps[t, ids[e]])
        total += -s * term + beta * kl - gamma * ent[t]
    return total / prm["loss_norm"]


@pytest.mark.parametrize("lt,est,support,extra", [
    ("ipo", "k1", "ragged", {}), ("icepop", "exact", "draws", {}),
    ("reinforce", "none", "draws", {}), ("ipo", "none", None, {}),
    ("ipo", "k1", "ragged", {"kl_staleness": "inv_sqrt", "entropy_coeff": 0.4}),
    ("reinforce", "none", None, {"entropy_coeff": -0.7}),
])
def test_gradients_match_frozen_weight_finite_differences(lt, est, support, extra):
    # Central differences of the loss with w_t and c_e frozen at the base point
    # (the sg[.] reading) against the oracle's dh and dW.
    h, W, labels, lq, adv, offsets, ids, u, logq = _tiny_problem(5, N=5, H=4, V=13,
                                                                  support=support, K=5)
    prm = _params(loss_type=lt, kl_coeff=0.3, kl_estimator=est, adv_tau=1.3, loss_norm=2.5,
                  inv_temperature=0.9, icepop_lo=0.2, icepop_hi=5.0, ipo_eps=0.6, **extra)
    age = np.array([0, 3, 1, 8, 0])
    out = ohead.head_reference(h, W, labels, lq, adv, prm, offsets, ids, u, logq, age=age)
    w_lab = out["weight"]
    c_e = lq_e = None
    if offsets is not None:
        lpe = out["support_logprobs"]
        we, _ = ow.weight(lpe, logq, prm)
        c_e = u * we
        lq_e = logq
    f = lambda hh, WW: _frozen_loss(hh, WW, labels, adv, prm, offsets, ids, u, logq,
                                    w_lab, c_e, lq_e, age)
    assert f(h, W) == pytest.approx(out["loss"], rel=1e-12, abs=1e-14)
    step = 1e-5
    g_h = np.zeros_like(h)
    for idx in np.ndindex(h.shape):
        hp, hm = h.copy(), h.copy()
        hp[idx] += step
        hm[idx] -= step
        g_h[idx] = (f(hp, W) - f(hm, W)) / (2 * step)
    g_W = np.zeros_like(W)
    for idx in np.ndindex(W.shape):
        Wp, Wm = W.copy(), W.copy()
        Wp[idx] += step
        Wm[idx] -= step
        g_W[idx] = (f(h, Wp) - f(h, Wm)) / (2 * step)
    assert np.linalg.norm(out["dh"] - g_h) <= 1e-7 * np.linalg.norm(g_h) + 1e-12
    assert np.linalg.norm(out["dW"] - g_W) <= 1e-7 * np.linalg.norm(g_W) + 1e-12


def test_inv_sqrt_staleness_closed_form_and_metrics():
    # beta_t = kl_coeff / sqrt(1 + age): ages 0, 3, 8 give kl_coeff, kl_coeff / 2,
    # kl_coeff / 3; kl/beta is their mean and kl/age0 the mean KL of age-0 tokens.
    h, W, labels, lq, adv, offsets, ids, u, logq = _tiny_problem(8, N=4, H=4, V=9,
                                                                  support="draws", K=3)
    base = _params(kl_coeff=0.6, kl_estimator="k1")
    age = np.array([0, 3, 0, 8])
    r0 = ohead.head_reference(h, W, labels, lq, adv, base, offsets, ids, u, logq, age=age)
    r1 = ohead.head_reference(h, W, labels, lq, adv, dict(base, kl_staleness="inv_sqrt"),
                              offsets, ids, u, logq, age=age)
    kl = r0["kl"]
    assert np.allclose(r1["token_loss"] - r0["token_loss"],
                       kl * 0.6 * (np.array([1, 1 / 2, 1, 1 / 3]) - 1), rtol=0, atol=1e-14)
    assert r1["metrics"]["kl_beta"] == pytest.approx(0.6 * (1 + 1 / 2 + 1 + 1 / 3) / 4, rel=1e-14)
    assert r1["metrics"]["kl_age0"] == pytest.approx((kl[0] + kl[2]) / 2, rel=1e-14)
    assert r0["metrics"]["kl_beta"] == pytest.approx(0.6, rel=1e-15)
    # no age input: every token is fresh
    r2 = ohead.head_reference(h, W, labels, lq, adv, dict(base, kl_staleness="inv_sqrt"),
                              offsets, ids, u, logq)
    assert np.array_equal(r2["token_loss"], r0["token_loss"])


def test_entropy_bonus_at_uniform_logits():
    # W = 0: p is uniform, H = log V and log p + H = 0, so the bonus adds
    # -gamma log V to every token loss and nothing to the gradient.
    N, H, V = 4, 3, 13
    h, _, labels, lq, adv, offsets, ids, u, logq = _tiny_problem(2, N, H, V, support="ragged")
    W = np.zeros((V, H))
    prm = _params(loss_type="reinforce", loss_norm=2.0)
    r0 = ohead.head_reference(h, W, labels, lq, adv, prm, offsets, ids, u, logq)
    r1 = ohead.head_reference(h, W, labels, lq, adv, dict(prm, entropy_coeff=0.35), offsets, ids,
                              u, logq)
    assert np.allclose(r1["token_loss"] - r0["token_loss"], -0.35 * math.log(V), atol=1e-14)
    assert r1["loss"] - r0["loss"] == pytest.approx(-0.35 * math.log(V) * N / 2.0, rel=1e-12)
    assert np.allclose(r1["dh"], r0["dh"], atol=1e-15) and np.allclose(r1["dW"], r0["dW"],
                                                                       atol=1e-15)


def test_full_support_with_u_equal_p_cancels_centering():
    # REINFORCE with the support = whole vocabulary and u = p (training softmax):
    # the centering removes the softmax term and dL/dz = -s (e_a - p) / D.
    rng = np.random.default_rng(6)
    N, H, V = 5, 4, 23
    h = rng.normal(size=(N, H))
    W = rng.normal(size=(V, H))
    labels = rng.integers(0, V, N)
    adv = rng.normal(size=N)
    p = sps.softmax(h @ W.T, axis=1)
    offsets = np.arange(N + 1) * V
    ids = np.tile(np.arange(V), N)
    prm = _params(loss_type="reinforce", loss_norm=4.0)
    out = ohead.head_reference(h, W, labels, -np.ones(N), adv, prm, offsets, ids,
                               p.reshape(-1), np.log(p.reshape(-1)))
    G = p.copy()
    G[np.arange(N), labels] -= 1.0
    G *= adv[:, None] / 4.0
    assert np.allclose(out["dh"], G @ W, rtol=1e-12, atol=1e-13)
    assert np.allclose(out["dW"], G.T @ h, rtol=1e-12, atol=1e-13)
    assert np.allclose(out["kappa"], 0.0, atol=1e-13)


def test_on_policy_replay_exact_kl_closed_form():
    # On-policy replay: q is the training softmax truncated to a top-p set S and
    # renormalised.  Then KL(q || p) = -log p(S) and dKL/dz = p - q_S.
    rng = np.random.default_rng(7)
    N, H, V = 4, 5, 30
    h = rng.normal(size=(N, H))
    W = rng.normal(size=(V, H)) * 1.5
    p = sps.softmax(h @ W.T, axis=1)
    offsets = [0]
    ids, u = [], []
    qS = np.zeros_like(p)
    for t in range(N):
        order = np.argsort(-p[t])
        k = int(np.searchsorted(np.cumsum(p[t, order]), 0.9) + 1)
        S = order[:k]
        ids.extend(S.tolist())
        q = p[t, S] / p[t, S].sum()
        u.extend(q.tolist())
        qS[t, S] = q
        offsets.append(offsets[-1] + k)
    offsets = np.array(offsets)
    ids = np.array(ids)
    u = np.array(u)
    labels = np.array([ids[offsets[t]] for t in range(N)])
    prm = _params(kl_coeff=1.0, kl_estimator="exact", loss_norm=1.0)
    out = ohead.head_reference(h, W, labels, np.log(u[offsets[:-1]]), np.zeros(N), prm,
                               offsets, ids, u, None)
    PS = np.array([p[t, ids[offsets[t]:offsets[t + 1]]].sum() for t in range(N)])
    assert np.allclose(out["token_loss"], -np.log(PS), rtol=1e-12)
    assert np.allclose(out["dh"], (p - qS) @ W, rtol=1e-11, atol=1e-12)


def test_linear_in_adv_tau_and_loss_norm():
    h, W, labels, lq, adv, offsets, ids, u, logq = _tiny_problem(8, support="ragged")
    base = _params(loss_type="icepop", icepop_lo=0.1, icepop_hi=10.0, loss_norm=2.0)
    a = ohead.head_reference(h, W, labels, lq, adv, base, offsets, ids, u, logq)
    b = ohead.head_reference(h, W, labels, lq, adv, dict(base, adv_tau=3.0), offsets, ids, u, logq)
    c = ohead.head_reference(h, W, labels, lq, adv, dict(base, loss_norm=8.0), offsets, ids, u, logq)
    assert b["loss"] == pytest.approx(3.0 * a["loss"], rel=1e-12)
    assert np.allclose(b["dW"], 3.0 * a["dW"], rtol=1e-12, atol=1e-14)
    assert c["loss"] == pytest.approx(a["loss"] / 4.0, rel=1e-12)
    assert np.allclose(c["dh"], a["dh"] / 4.0, rtol=1e-12, atol=1e-14)


def test_duplicate_ids_add_up():
    # Repeated draw ids are separate entries: a support [v, v] with u = 1/2 each
    # gives the same loss and gradient as [v] with u = 1.
    h, W, labels, lq, adv, *_ = _tiny_problem(9, N=1, H=3, V=9, support=None)
    prm = _params(loss_type="reinforce", kl_coeff=0.4, kl_estimator="k1")
    one = ohead.head_reference(h, W, labels, lq, adv, prm, np.array([0, 1]), np.array([4]),
                               np.array([1.0]), np.array([-0.7]))
    two = ohead.head_reference(h, W, labels, lq, adv, prm, np.array([0, 2]), np.array([4, 4]),
                               np.array([0.5, 0.5]), np.array([-0.7, -0.7]))
    assert two["loss"] == pytest.approx(one["loss"], rel=1e-13)
    assert np.allclose(two["dW"], one["dW"], rtol=1e-12, atol=1e-15)


def test_k_draw_estimator_is_unbiased():
    # PR 4233: K i.i.d. sampler draws with u = 1/K estimate E_q[f]; checked
    # against the exact centre sum_v q_v w_v log p_v over 10^4 draw sets.
    rng = np.random.default_rng(10)
    H, V, K, S = 6, 25, 16, 10000
    h1 = rng.normal(size=H)
    W = rng.normal(size=(V, H)) * 0.7
    y = W @ h1 + rng.normal(size=V) * 0.4
    q = sps.softmax(y)
    logq_v = sps.log_softmax(y)
    lp_v = sps.log_softmax(W @ h1)
    prm = _params(loss_type="ipo", ipo_eps=0.05)
    w_v, _ = ow.weight(lp_v, logq_v, prm)
    exact = float((q * w_v * lp_v).sum())
    draws = rng.choice(V, size=(S, K), p=q)
    h = np.tile(h1, (S, 1))
    offsets = np.arange(S + 1) * K
    ids = draws.reshape(-1)
    label = np.zeros(S, np.int64)
    out = ohead.head_reference(h, W, label, np.full(S, logq_v[0]), np.ones(S), prm, offsets,
                               ids, np.full(S * K, 1.0 / K), logq_v[ids], want_grads=False)
    # loss_t = -(w lp - centre)  =>  centre = loss_t + w lp
    centre = out["token_loss"] + out["weight"] * out["logprobs"]
    se = centre.std(ddof=1) / math.sqrt(S)
    assert abs(centre.mean() - exact) <= 4 * se


# ------------------------------------------------------------ replay pins ----

RP = dict(eps=(0.05, 0.1, 0.2, 0.3, 0.5), primary_eps_index=3, max_ratio=5.0,
          icepop_lo=0.5, icepop_hi=2.0, clip_low=0.2, clip_high=0.2, clip_c=3.0, tis_upper=2.0)


def test_replay_worked_examples():
    rows = _worked_examples()
    lp = np.log([r[0] for r in rows])
    lq = np.log([r[1] for r in rows])
    res = oreplay.replay_reference(lp, lq, np.ones(2), RP)
    word = res["mask_word"]
    assert (word[0] >> oreplay.BIT_ICEPOP_HIGH) & 1 == 1  # ratio 6 above the [0.5, 2] band
    assert (word[0] >> (oreplay.BIT_IPO0 + 3)) & 1 == 0  # kept by eps 0.3
    assert (word[1] >> (oreplay.BIT_IPO0 + 3)) & 1 == 1  # moved 0.70 > 0.3
    assert res["w_primary"][0] == pytest.approx(5.0)
    assert res["w_primary"][1] == 0.0


def test_replay_on_policy_has_no_clipping():
    rng = np.random.default_rng(11)
    lq = -rng.exponential(1.0, 1000)
    A = rng.normal(size=1000)
    res = oreplay.replay_reference(lq, lq, A, RP)
    assert res["ppo_clip"] == 0 and res["ppo_clip_lower"] == 0 and res["tis_truncated"] == 0
    assert res["ppo_loss_sum"] == pytest.approx(-A.sum(), rel=1e-12)
    assert res["ppo_kl_sum"] == 0.0
    assert all(res[f"ipo{i}_kept"] == 1000 for i in range(5))
    assert res["icepop_kept"] == 1000


def test_replay_dual_clip_cases():
    # Dual clip from its definition: J = min(rA, clip(r, 0.8, 1.2) A), then
    # for A < 0, J = max(J, 3A).
    cases = [  # r, A, expected loss -J, clip?, dual?
        (5.0, -1.0, 3.0, False, True),
        (2.0, -1.0, 2.0, False, False),
        (0.5, -1.0, 0.8, True, False),
        (2.0, 1.0, -1.2, True, False),
        (0.5, 1.0, -0.5, False, False),
    ]
    lq = np.full(len(cases), math.log(0.1))
    lp = lq + np.log([c[0] for c in cases])
    A = np.array([c[1] for c in cases])
    res = oreplay.replay_reference(lp, lq, A, RP)
    word = res["mask_word"]
    for i, (_, _, loss, clip, dual) in enumerate(cases):
        one = oreplay.replay_reference(lp[i:i + 1], lq[i:i + 1], A[i:i + 1], RP)
        assert one["ppo_loss_sum"] == pytest.approx(loss, rel=1e-12)
        assert bool((word[i] >> oreplay.BIT_PPO_CLIP) & 1) == clip
        assert bool((word[i] >> oreplay.BIT_DUAL_CLIP) & 1) == dual


def test_replay_tis_truncation():
    lq = np.full(3, math.log(0.1))
    lp = lq + np.log([3.0, 1.5, 2.0])
    A = np.array([1.0, -2.0, 1.0])
    res = oreplay.replay_reference(lp, lq, A, RP)
    assert res["tis_truncated"] == 1
    assert res["tis_weight_sum"] == pytest.approx(2.0 + 1.5 + 2.0, rel=1e-12)
    assert res["tis_loss_sum"] == pytest.approx(-(2.0 - 3.0 + 2.0), rel=1e-12)


def test_replay_ipo_masked_fraction_monotone_in_eps():
    rng = np.random.default_rng(12)
    lq = -rng.exponential(1.0, 5000)
    lp = np.minimum(lq + rng.normal(size=5000) * 0.6, 0.0)
    eps = (0.01, 0.05, 0.1, 0.2, 0.3, 0.5, 0.8, 1.0)
    res = oreplay.replay_reference(lp, lq, rng.normal(size=5000), dict(RP, eps=eps))
    kept = [res[f"ipo{i}_kept"] for i in range(len(eps))]
    assert all(a <= b for a, b in zip(kept, kept[1:]))
    assert kept[-1] == 5000


# ------------------------------------------- head metrics: closed forms ----
#
# Three tokens over V = 3 whose training softmax is set by hand: with W = I
# (H = V) the logits are h_t, and h_t = log p_t makes softmax(h_t) = p_t
# (the row sums to 1, so its log-sum-exp is 0).  Each metric then has a value
# computed by hand from the table below (prime-rl PR 4233, "What changes",
# metrics bullet: support mass is E_q[p/q] from the support; mask_tv is the
# fraction of label tokens failing the IPO total-variation test).
#
#  t  p_t               label  q(label)  |P-Q|  band ratio   support (v, u, q_v)
#  0  (0.5, 0.3, 0.2)   0      0.4       0.10   1.25         (1, .5, .5), (2, .5, .25)
#  1  (0.1, 0.6, 0.3)   0      0.9       0.80   0.111        (1, 1., .3)
#  2  (0.2, 0.2, 0.6)   1      0.05      0.15   4.0          none

def _metric_problem():
    p = np.array([[0.5, 0.3, 0.2], [0.1, 0.6, 0.3], [0.2, 0.2, 0.6]])
    h = np.log(p)
    W = np.eye(3)
    labels = np.array([0, 0, 1])
    lq = np.log([0.4, 0.9, 0.05])
    adv = np.array([1.0, -0.5, 2.0])
    offsets = np.array([0, 2, 3, 3])
    ids = np.array([1, 2, 1])
    u = np.array([0.5, 0.5, 1.0])
    logq = np.log([0.5, 0.25, 0.3])
    return p, h, W, labels, lq, adv, offsets, ids, u, logq


def test_head_metrics_closed_form():
    p, h, W, labels, lq, adv, offsets, ids, u, logq = _metric_problem()
    beta = 0.05
    for lt, masked_fraction in (("ipo", 1 / 3), ("icepop", 2 / 3), ("reinforce", 0.0)):
        prm = _params(loss_type=lt, ipo_eps=0.3, icepop_lo=0.5, icepop_hi=2.0, kl_coeff=beta,
                      kl_estimator="k1", loss_norm=3.0)
        out = ohead.head_reference(h, W, labels, lq, adv, prm, offsets, ids, u, logq)
        m = out["metrics"]
        # per-token softmax reproduced
        assert np.allclose(out["logprobs"], np.log([0.5, 0.1, 0.2]), rtol=0, atol=1e-14)
        # masked fraction: IPO masks token 1; the band masks tokens 1 and 2
        assert m["masked_fraction"] == pytest.approx(masked_fraction, abs=1e-15)
        # mask_tv: the IPO test at ipo_eps on the label, whatever the loss type
        assert m["mask_tv"] == pytest.approx(1 / 3, abs=1e-15)
        # support mass: sum_e u_e p(v_e)/q(v_e) per row with a support
        # (token 0: .5*.3/.5 + .5*.2/.25 = 0.7; token 1: .6/.3 = 2), mean over
        # those two rows (token 2 has none)
        assert m["support_mass"] == pytest.approx((0.7 + 2.0) / 2, rel=1e-13)
        # kl: sum_e u_e (log q - log p) per token, mean over all three tokens
        kl0 = 0.5 * math.log(0.5 / 0.3) + 0.5 * math.log(0.25 / 0.2)
        kl1 = math.log(0.3 / 0.6)
        assert np.allclose(out["kl"], [kl0, kl1, 0.0], rtol=1e-13, atol=1e-15)
        assert m["kl"] == pytest.approx((kl0 + kl1) / 3, rel=1e-12)
        assert m["kl_beta"] == pytest.approx(beta, rel=1e-15)
        # entropy mean from the table
        ent = [-(r * np.log(r)).sum() for r in p]
        assert m["entropy_mean"] == pytest.approx(np.mean(ent), rel=1e-13)


def test_head_metric_kappa_closed_form():
    # kappa_t = s_t (w_t - sum_e u_e w_e) + beta sum_e u_e with reinforce
    # (every w = 1): token 0: s (1 - 1) + beta = beta; token 1: same; token 2
    # (no support): s_2 = 2.  max |kappa| = 2.
    p, h, W, labels, lq, adv, offsets, ids, u, logq = _metric_problem()
    prm = _params(loss_type="reinforce", kl_coeff=0.05, kl_estimator="k1", loss_norm=3.0)
    out = ohead.head_reference(h, W, labels, lq, adv, prm, offsets, ids, u, logq)
    assert np.allclose(out["kappa"], [0.05, 0.05, 2.0], rtol=1e-15, atol=1e-15)
    assert out["metrics"]["max_abs_kappa"] == pytest.approx(2.0, rel=1e-15)


# ------------------------------------- replay: per-variant sums by hand ----

def test_replay_variant_sums_on_worked_examples():
    # The IPO page's two tokens (0.01 -> 0.06 and 0.90 -> 0.20) with
    # advantages 1.5 and -2: every per-variant sum is a closed form.
    rows = _worked_examples()
    P = np.array([r[0] for r in rows])
    Q = np.array([r[1] for r in rows])
    lp, lq = np.log(P), np.log(Q)
    A = np.array([1.5, -2.0])
    prm = dict(RP, eps=(0.01, 0.3, 0.8), primary_eps_index=1, icepop_lo=0.2, icepop_hi=2.0)
    res = oreplay.replay_reference(lp, lq, A, prm)
    r1 = 0.2 / 0.9
    # eps 0.01 masks both (moved 0.05 and 0.70)
    assert res["ipo0_kept"] == 0
    assert res["ipo0_loss_sum"] == 0.0 and res["ipo0_weight_sum"] == 0.0
    # eps 0.3 keeps token 0 (w = min(6, 5) = 5), masks token 1
    assert res["ipo1_kept"] == 1
    assert res["ipo1_weight_sum"] == pytest.approx(5.0, rel=1e-14)
    assert res["ipo1_loss_sum"] == pytest.approx(-1.5 * 5.0 * math.log(0.06), rel=1e-14)
    # eps 0.8 keeps both; token 1's weight is its ratio 0.2/0.9
    assert res["ipo2_kept"] == 2
    assert res["ipo2_weight_sum"] == pytest.approx(5.0 + r1, rel=1e-14)
    assert res["ipo2_loss_sum"] == pytest.approx(
        -1.5 * 5.0 * math.log(0.06) + 2.0 * r1 * math.log(0.2), rel=1e-14)
    # band [0.2, 2]: token 0 (ratio 6) above it, token 1 (0.222) inside
    assert (res["icepop_kept"], res["icepop_low"], res["icepop_high"]) == (1, 0, 1)
    assert res["icepop_weight_sum"] == pytest.approx(r1, rel=1e-14)
    assert res["icepop_loss_sum"] == pytest.approx(2.0 * r1 * math.log(0.2), rel=1e-14)
    # REINFORCE: -sum A lp
    assert res["reinforce_loss_sum"] == pytest.approx(
        -(1.5 * math.log(0.06) - 2.0 * math.log(0.2)), rel=1e-14)
    # ppo_kl sums lq - lp: log(0.01/0.06) + log(0.9/0.2) = log 0.75
    assert res["ppo_kl_sum"] == pytest.approx(math.log(0.75), rel=1e-13)
    # the primary weight is eps 0.3's
    assert np.allclose(res["w_primary"], [5.0, 0.0], rtol=1e-14, atol=0)


def test_replay_ppo_kl_estimates_kl_of_rollout_to_trainer():
    # Tokens drawn from the rollout policy q: the mean of lq - lp is the k1
    # estimate of KL(q || p) = sum_v q_v log(q_v / p_v) >= 0, so ppo_kl_sum / N
    # must land on that (positive) divergence within 4 standard errors; the
    # opposite sign, or lp - lq, lands near -KL(q || p).
    rng = np.random.default_rng(21)
    V = 50
    q = rng.dirichlet(np.ones(V))
    p = rng.dirichlet(np.ones(V))
    kl_qp = float(np.sum(q * np.log(q / p)))
    y = rng.choice(V, size=200_000, p=q)
    lq, lp = np.log(q[y]), np.log(p[y])
    res = oreplay.replay_reference(lp, lq, np.zeros(len(y)), RP)
    est = res["ppo_kl_sum"] / len(y)
    se = np.std(lq - lp, ddof=1) / math.sqrt(len(y))
    assert kl_qp > 10 * se
    assert abs(est - kl_qp) <= 4 * se
