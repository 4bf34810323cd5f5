"""Fused LM head + RLLoss, forward and backward, in fp64 (test infrastructure).

Source: prime-rl pull request 4233, PR description.  Per token t with label a,
sampler log-prob lq(a), advantage A_t and support entries e = (v_e, u_e):

  loss_t = -adv_tau * A_t * (w(a) * log p(a) - sum_e sg[u_e * w_e] * log p(v_e))
           + beta_t * KL(q || p)

where p = softmax(z_t), z_t = W h_t / tau (the LM head), w(.) is the weight of
the loss type (oracle.weights), sum_e u_e f(v_e) estimates E_q[f] (replayed
top-p support with u = q, or K sampler draws with u = 1/K, "sum_v u_v f(v)"
bullets of the PR description), and the KL over the same support is
sum_e u_e (log q(v_e) - log p(v_e)) ("What changes", KL bullet; one formula for
the exact and the k1 estimator, exact meaning u = q on a replayed support).
beta_t = kl_coeff with kl_staleness "none"; with "inv_sqrt" the same bullet
scales the KL by the token's policy age (engine weight-version lag), read here
as beta_t = kl_coeff / sqrt(1 + age_t).  An entropy bonus with coefficient
gamma subtracts gamma * H_t from loss_t (the Tencent article on KL/clip/entropy,
section 3: the policy loss minus entropy_coeff times the aggregated entropy).
The loss is L = sum_t loss_t / D.

Readings taken where the pages are silent (each listed in the design notes):
* w(a) and every w_e are held constant in the gradient (score-function form;
  the PR marks the centering term with sg[.] and the label weight is treated
  the same way).  The loss value does not depend on this choice.
* log p is the full-vocabulary log-softmax at temperature tau; entropy is
  that softmax's Shannon entropy, a forward output with no gradient.
* Support entries are taken in stored order; repeated ids are separate
  entries and add up.
* A missing per-entry sampler log-prob defaults to log u_e (valid on a
  replayed support, where u = q).
* Without an age input every token has age 0.  Metrics "kl/beta" and
  "kl/age0" of the PR's metrics bullet are the mean beta_t and the mean KL
  over tokens of age 0.

Gradient (w, c held constant), with kappa_t = s_t (w_t - sum_e c_e) + beta_t sum_e u_e:
  dL/dz_t = ( kappa_t p_t + gamma p_t (log p_t + H_t) - s_t w_t e_a
              + sum_e (s_t c_e - beta_t u_e) e_{v_e} ) / D
because d log p(v) / dz = e_v - p and dH/dz = -p (log p + H).  Then dh = (dL/dz) W / tau and
dW = (dL/dz)^T h / tau.  The oracle always forms the dense gradient.
"""

import numpy as np
import torch

from . import weights as _w

METRIC_NAMES = (
    "masked_fraction",
    "support_mass",
    "mask_tv",
    "kl",
    "kl_beta",
    "max_abs_kappa",
    "entropy_mean",
    "kl_age0",
)


def _row_index(offsets):
    sizes = np.diff(offsets)
    return np.repeat(np.arange(len(sizes)), sizes)


def kl_beta(params):
    if params.get("kl_estimator", "none") == "none":
        return 0.0
    return float(params.get("kl_coeff", 0.0))


def beta_per_token(params, age):
    """beta_t: kl_coeff, divided by sqrt(1 + age_t) under kl_staleness inv_sqrt.

    The PR's KL bullet names the inv_sqrt option and the per-token age but
    gives no formula; 1/sqrt(1 + age) is the plainest reading of the name.
    Parity unpinned: nothing on the pages fixes this formula, so its test only
    restates the reading (ages 0, 3, 8 give factors 1, 1/2, 1/3).
    """
    beta = kl_beta(params)
    age = np.asarray(age, np.float64)
    if params.get("kl_staleness", "none") == "inv_sqrt":
        return beta / np.sqrt(1.0 + age)
    return np.full(age.shape, beta)


def head_reference(h, W, labels, infer_logprobs, adv, params, offsets=None, ids=None,
                   u=None, logq=None, tokens=None, want_grads=True, chunk=None, age=None,
                   progress=None):
    """Dense fp64 forward + backward.

    h [N,H], W [V,H] (any float dtype; read exactly), labels [N] ints,
    infer_logprobs [N], adv [N], CSR offsets [N+1] / ids / u / logq (or None).
    params: loss_type, ipo_eps, max_ratio, icepop_lo, icepop_hi, adv_tau,
    kl_coeff, kl_estimator, kl_staleness, entropy_coeff, inv_temperature,
    loss_norm (D).  age: per-token policy age [N] (None: all 0).

    ``tokens`` restricts the evaluation to a subset of token indices (the
    per-token outputs and dh rows of those tokens, and dW from those tokens
    only); D stays params["loss_norm"].  ``chunk`` bounds memory by handling
    that many tokens per dense [tokens, V] block; it does not change any
    per-token arithmetic.  ``progress``, if given, is called with (tokens
    done, tokens) after each block.
    Returns a dict of numpy arrays (fp64) and scalars.
    """
    # The [tokens, V] steps run on torch CPU tensors in fp64, which spread the
    # elementwise work over the host cores; the arithmetic is the same.
    W = torch.as_tensor(np.asarray(W, np.float64))
    V, H = W.shape
    N = len(labels)
    tok = np.arange(N) if tokens is None else np.asarray(tokens, np.int64)
    inv_t = float(params.get("inv_temperature", 1.0))
    D = float(params["loss_norm"])
    s_all = float(params.get("adv_tau", 1.0)) * np.asarray(adv, np.float64)
    beta_all = beta_per_token(params, np.zeros(N) if age is None else age)
    gamma = float(params.get("entropy_coeff", 0.0))
    age_all = np.zeros(N, np.int64) if age is None else np.asarray(age, np.int64)
    has_support = offsets is not None and ids is not None
    if has_support:
        offsets = np.asarray(offsets, np.int64)
        ids = np.asarray(ids, np.int64)
        u = np.asarray(u, np.float64)
        lq_e_all = np.log(u) if logq is None else np.asarray(logq, np.float64)
    n_tok = len(tok)
    out = dict(
        logprobs=np.zeros(n_tok), entropy=np.zeros(n_tok), lse=np.zeros(n_tok),
        weight=np.zeros(n_tok), keep=np.zeros(n_tok, bool), token_loss=np.zeros(n_tok),
        kappa=np.zeros(n_tok), kl=np.zeros(n_tok), support_mass=np.zeros(n_tok),
        beta=np.zeros(n_tok), zmax_abs=np.zeros(n_tok),
        support_count=np.zeros(n_tok, np.int64),
    )
    sup_lp = {}  # entry index -> log p(v_e)
    dh = np.zeros((n_tok, H)) if want_grads else None
    dW = torch.zeros((V, H), dtype=torch.float64) if want_grads else None
    step = n_tok if chunk is None else int(chunk)
    for c0 in range(0, n_tok, max(step, 1)):
        sel = np.arange(c0, min(n_tok, c0 + step))
        rows = tok[sel]
        hc = torch.as_tensor(np.asarray(h[rows], np.float64))
        # LM head logits at temperature tau.
        z = inv_t * (hc @ W.T)
        # Log-sum-exp with the max subtracted, then log-softmax and softmax.
        zmax = z.max(dim=1, keepdim=True).values
        lse_t = zmax[:, 0] + torch.log(torch.exp(z - zmax).sum(dim=1))
        logp_t = z - lse_t[:, None]
        p = torch.exp(logp_t)
        # Shannon entropy of the training softmax.
        ent = (-(p * logp_t).sum(dim=1)).numpy()
        lse = lse_t.numpy()
        a = np.asarray(labels, np.int64)[rows]
        lp = logp_t[torch.arange(len(rows)), torch.as_tensor(a)].numpy()
        lq = np.asarray(infer_logprobs, np.float64)[rows]
        w, keep = _w.weight(lp, lq, params)
        s = s_all[rows]
        beta = beta_all[rows]
        sum_c = np.zeros(len(rows))
        cent = np.zeros(len(rows))
        sum_u = np.zeros(len(rows))
        kl = np.zeros(len(rows))
        smass = np.zeros(len(rows))
        cnt = np.zeros(len(rows), np.int64)
        G = None
        if want_grads:
            G = torch.zeros_like(z)
        if has_support:
            for i, t in enumerate(rows):
                e0, e1 = offsets[t], offsets[t + 1]
                if e1 == e0:
                    continue
                v = ids[e0:e1]
                ue = u[e0:e1]
                lpe = logp_t[i, torch.as_tensor(v)].numpy()
                lqe = lq_e_all[e0:e1]
                we, _ = _w.weight(lpe, lqe, params)
                ce = ue * we
                sum_c[i] = ce.sum()
                cent[i] = (ce * lpe).sum()
                sum_u[i] = ue.sum()
                kl[i] = (ue * (lqe - lpe)).sum()
                smass[i] = (ue * np.exp(lpe - lqe)).sum()
                cnt[i] = e1 - e0
                for k in range(e0, e1):
                    sup_lp[k] = lpe[k - e0]
                if want_grads:
                    # repeated ids add up
                    G[i].index_add_(0, torch.as_tensor(v), torch.as_tensor(s[i] * ce - beta[i] * ue))
        klterm = kl if kl_beta(params) != 0.0 else np.zeros_like(kl)
        loss = -s * (w * lp - cent) + beta * klterm - gamma * ent
        kappa = s * (w - sum_c) + beta * sum_u
        if want_grads:
            G += torch.as_tensor(kappa)[:, None] * p
            if gamma != 0.0:
                G += gamma * p * (logp_t + torch.as_tensor(ent)[:, None])
            G[torch.arange(len(rows)), torch.as_tensor(a)] -= torch.as_tensor(s * w)
            G /= D
            dh[sel] = (inv_t * (G @ W)).numpy()
            dW += inv_t * (G.T @ hc)
        out["logprobs"][sel] = lp
        out["entropy"][sel] = ent
        out["lse"][sel] = lse
        out["weight"][sel] = w
        out["keep"][sel] = keep
        out["token_loss"][sel] = loss
        out["kappa"][sel] = kappa
        out["kl"][sel] = klterm
        out["support_mass"][sel] = smass
        out["support_count"][sel] = cnt
        out["beta"][sel] = beta
        # largest logit magnitude of the token (the scale of fp32 rounding in
        # an implementation's logits, used by the tests' decision bands)
        out["zmax_abs"][sel] = z.abs().max(dim=1).values.numpy()
        if progress is not None:
            progress(int(sel[-1]) + 1, n_tok)
    out["loss"] = out["token_loss"].sum() / D
    if want_grads:
        out["dh"] = dh
        out["dW"] = dW.numpy()
    if has_support:
        e_list = sorted(sup_lp)
        out["support_entries"] = np.array(e_list, np.int64)
        out["support_logprobs"] = np.array([sup_lp[k] for k in e_list], np.float64)
    # Metrics of the PR's "Metrics" bullet plus the masked fraction.
    P = np.exp(out["logprobs"])
    Q = np.exp(np.asarray(infer_logprobs, np.float64)[tok])
    has = out["support_count"] > 0
    out["metrics"] = dict(
        masked_fraction=float(np.mean(~out["keep"])) if n_tok else 0.0,
        support_mass=float(out["support_mass"][has].mean()) if has.any() else 0.0,
        mask_tv=float(np.mean(np.abs(P - Q) > params.get("ipo_eps", 0.3))) if n_tok else 0.0,
        kl=float(out["kl"].mean()) if n_tok else 0.0,
        kl_beta=float(out["beta"].mean()) if n_tok else 0.0,
        max_abs_kappa=float(np.abs(out["kappa"]).max()) if n_tok else 0.0,
        entropy_mean=float(out["entropy"].mean()) if n_tok else 0.0,
        kl_age0=(float(out["kl"][age_all[tok] == 0].mean())
                 if np.any(age_all[tok] == 0) else 0.0),
    )
    return out


def from_workload(wl, **kw):
    """Run head_reference on a synth.HeadWorkload (host copies, exact)."""
    d = wl.to_host_numpy()
    return head_reference(d["h"], d["W"], d["labels"], d["infer_logprobs"], d["adv"],
                          wl.params, offsets=d["offsets"], ids=d["ids"], u=d["u"],
                          logq=d["logq"], **kw)
