"""Sequence-aware rollout correction over a replay, fp64.  Test infrastructure.

The plain definition of what the correction pass computes, for the tests and
the benchmark's CPU baseline only.

Source: the "Rollout Correction Methods" page (miles documentation, train /
inference mismatch helper):
* "Config keys": tis_mode in {truncate, clip, mask}, lower / upper bounds,
  tis_level in {token, sequence, geometric}, batch normalisation to mean 1;
  use_rs with its own level and bounds (unset bounds fall back to the TIS
  bounds) and a veto threshold;
* "Importance Sampling": the token weight is exp(log pi_train - log
  pi_rollout); the sequence weight is the exponential of the sum of the token
  log ratios; the geometric weight is the exponential of their mean;
* "Rejection Sampling": tokens or sequences whose IS statistic lies outside
  the bounds are masked and leave the loss average; "Veto Mechanism": a
  sequence holding any token with ratio below C_veto is rejected whole;
* "Mismatch Monitoring Metrics" and "IS/RS Correction Metrics": the metric
  names and the formulas the tables give.

The replay has no separate proximal policy (pi_old := pi_train), so the token
ratio is rho_t = exp(lp_t - lq_t) and the decoupled PPO inner ratio is 1: the
clipped surrogate equals A_t and the token loss is -w_t A_t ("Decoupled,
3-policy PPO Importance Sampling").

Readings where the page is silent or loose (each also listed with the design
notes):
* sequences are given by offsets [S + 1], every sequence non-empty;
* truncate uses the upper bound only; clip clamps to [L, U]; mask sets the
  weight to 0 outside [L, U]; bounds are inclusive (a weight equal to a bound
  is kept and not counted); decisions compare log weights with log bounds;
* rejection statistic: token level the token ratio, sequence level the mean of
  the sequence's token ratios ("mean IS weight"), geometric level the
  exponential of the mean log ratio;
* TIS-masked tokens keep their place in the loss average with weight 0;
  rejected tokens (RS or veto) leave it;
* the veto applies whenever its threshold is > 0, with or without RS;
* batch normalisation divides by the mean weight of the kept tokens
  (factor = kept / sum of kept weights; 1 when that sum is 0 or off);
* token means for kl, k3_kl, chi2_token and the absolute log-prob difference;
  the perplexity family is per sequence (mean log-prob over the sequence)
  averaged over sequences; chi2_seq = mean_s exp(2 sum_t d_t) - 1 and
  chi2_token = mean_t rho_t^2 - 1 (chi-square of the training policy against
  the rollout policy, estimated on rollout samples);
* fractions are over tokens, except the catastrophic-sequence fraction, over
  sequences; weight means are over all tokens (rejected ones count 0 after
  RS); the final weight statistics are over the kept tokens.
"""

import numpy as np

LEVELS = ("token", "sequence", "geometric")
MODES = ("truncate", "clip", "mask")

# Per-token flag bits.
F_TIS_LOW = 1
F_TIS_HIGH = 2
F_RS_LOW = 4
F_RS_HIGH = 8
F_VETO = 16          # the token's sequence is vetoed
F_CATASTROPHIC = 32  # the token's own ratio is below the veto threshold
F_REJECTED = 64      # left out of the loss (RS or veto)

METRICS = (
    "training_log_ppl", "training_ppl", "rollout_log_ppl", "rollout_ppl", "kl", "k3_kl",
    "log_ppl_diff", "log_ppl_abs_diff", "ppl_ratio", "chi2_token", "chi2_seq",
    "logprob_abs_diff", "tis_weight_before_bound", "tis_weight_after_bound",
    "tis_fraction_low", "tis_fraction_high", "rs_fraction_low", "rs_fraction_high",
    "catastrophic_token_fraction", "catastrophic_seq_fraction", "is_ratio_mean_after_tis_rs",
    "batch_norm_factor", "is_ratio_mean_final", "is_ratio_min_final", "is_ratio_max_final",
    "loss", "loss_sum", "kept_tokens", "rejected_tokens",
)


def resolve(cfg):
    """Fill the RS bounds from the TIS bounds where unset (None)."""
    c = dict(cfg)
    if c.get("rs_lower") is None:
        c["rs_lower"] = c["tis_lower"]
    if c.get("rs_upper") is None:
        c["rs_upper"] = c["tis_upper"]
    return c


def mis_reference(lp, lq, A, offsets, cfg):
    """Per-token weight (before batch normalisation) and flags, and the metrics.

    lp, lq, A: [N]; offsets: int [S + 1], 0 = offsets[0] < ... < offsets[S] = N.
    cfg: tis_level, tis_mode, tis_lower, tis_upper, use_rs, rs_level,
    rs_lower, rs_upper (None: the TIS bound), veto (<= 0: off),
    batch_normalize.
    """
    c = resolve(cfg)
    lp = np.asarray(lp, np.float64)
    lq = np.asarray(lq, np.float64)
    A = np.asarray(A, np.float64)
    off = np.asarray(offsets, np.int64)
    N, S = len(lp), len(off) - 1
    n = np.diff(off).astype(np.float64)
    seq = np.repeat(np.arange(S), np.diff(off))  # sequence of each token
    d = lp - lq                                  # token log ratio
    sum_d = np.add.reduceat(d, off[:-1])
    sum_rho = np.add.reduceat(np.exp(d), off[:-1])
    min_d = np.minimum.reduceat(d, off[:-1])

    def log_stat(level, rs):
        if level == "token":
            return d
        if level == "sequence":
            s = np.log(sum_rho / n) if rs else sum_d
            return s[seq]
        return (sum_d / n)[seq]

    # Importance weight by level, then the mode's bound.
    logw = log_stat(c["tis_level"], rs=False)
    lL, lU = np.log(np.float64(c["tis_lower"])), np.log(np.float64(c["tis_upper"]))
    mode = c["tis_mode"]
    flags = np.zeros(N, np.uint32)
    if mode == "truncate":
        high = logw > lU
        low = np.zeros(N, bool)
        logw_b = np.minimum(logw, lU)
        w_b = np.exp(logw_b)
    elif mode == "clip":
        low, high = logw < lL, logw > lU
        w_b = np.exp(np.clip(logw, lL, lU))
    else:
        low, high = logw < lL, logw > lU
        w_b = np.where(low | high, 0.0, np.exp(logw))
    flags |= np.where(low, F_TIS_LOW, 0).astype(np.uint32)
    flags |= np.where(high, F_TIS_HIGH, 0).astype(np.uint32)
    w_raw = np.exp(logw)

    # Rejection sampling and veto.
    rejected = np.zeros(N, bool)
    rs_low = np.zeros(N, bool)
    rs_high = np.zeros(N, bool)
    if c["use_rs"]:
        ls = log_stat(c["rs_level"], rs=True)
        rs_low = ls < np.log(np.float64(c["rs_lower"]))
        rs_high = ls > np.log(np.float64(c["rs_upper"]))
        rejected |= rs_low | rs_high
    flags |= np.where(rs_low, F_RS_LOW, 0).astype(np.uint32)
    flags |= np.where(rs_high, F_RS_HIGH, 0).astype(np.uint32)
    C = c["veto"]
    if C > 0:
        lC = np.log(np.float64(C))
        catastrophic = d < lC
        vetoed_seq = min_d < lC
        vetoed = vetoed_seq[seq]
        rejected |= vetoed
        flags |= np.where(vetoed, F_VETO, 0).astype(np.uint32)
        flags |= np.where(catastrophic, F_CATASTROPHIC, 0).astype(np.uint32)
        n_cat_tok = int(catastrophic.sum())
        n_cat_seq = int(vetoed_seq.sum())
    else:
        n_cat_tok = n_cat_seq = 0
    flags |= np.where(rejected, F_REJECTED, 0).astype(np.uint32)
    kept = ~rejected
    weight = np.where(kept, w_b, 0.0)  # before batch normalisation

    n_kept = int(kept.sum())
    sw = weight[kept].sum()
    factor = n_kept / sw if (c["batch_normalize"] and sw > 0) else 1.0
    final = factor * weight[kept]
    loss_sum = (-factor * weight * A)[kept].sum()

    # Monitoring metrics.
    lppl_t = -np.add.reduceat(lp, off[:-1]) / n
    lppl_r = -np.add.reduceat(lq, off[:-1]) / n
    m = {
        "training_log_ppl": lppl_t.mean(),
        "training_ppl": np.exp(lppl_t).mean(),
        "rollout_log_ppl": lppl_r.mean(),
        "rollout_ppl": np.exp(lppl_r).mean(),
        "kl": (lq - lp).mean(),
        "k3_kl": (np.exp(d) - d - 1.0).mean(),
        "log_ppl_diff": (lppl_t - lppl_r).mean(),
        "log_ppl_abs_diff": np.abs(lppl_t - lppl_r).mean(),
        "ppl_ratio": np.exp(lppl_t - lppl_r).mean(),
        "chi2_token": np.exp(2.0 * d).mean() - 1.0,
        "chi2_seq": np.exp(2.0 * sum_d).mean() - 1.0,
        "logprob_abs_diff": np.abs(d).mean(),
        "tis_weight_before_bound": w_raw.mean(),
        "tis_weight_after_bound": w_b.mean(),
        "tis_fraction_low": low.sum() / N,
        "tis_fraction_high": high.sum() / N,
        "rs_fraction_low": rs_low.sum() / N,
        "rs_fraction_high": rs_high.sum() / N,
        "catastrophic_token_fraction": n_cat_tok / N,
        "catastrophic_seq_fraction": n_cat_seq / S,
        "is_ratio_mean_after_tis_rs": weight.mean(),
        "batch_norm_factor": factor,
        "is_ratio_mean_final": final.mean() if n_kept else 0.0,
        "is_ratio_min_final": final.min() if n_kept else 0.0,
        "is_ratio_max_final": final.max() if n_kept else 0.0,
        "loss": loss_sum / n_kept if n_kept else 0.0,
        "loss_sum": loss_sum,
        "kept_tokens": float(n_kept),
        "rejected_tokens": float(N - n_kept),
    }
    return {"weight": weight, "flags": flags.astype(np.uint8), "metrics": m,
            "logw": logw, "log_rs_stat": log_stat(c["rs_level"], rs=True) if c["use_rs"] else None,
            "d": d, "min_d": min_d, "seq": seq}


def near_threshold_tokens(res, cfg, band):
    """Tokens whose TIS, RS or veto decision lies within ``band`` (in log space)
    of its threshold; for sequence-level decisions every token of the sequence."""
    c = resolve(cfg)
    near = np.zeros(len(res["d"]), bool)
    lw = res["logw"]
    for b in (c["tis_lower"], c["tis_upper"]):
        near |= np.abs(lw - np.log(np.float64(b))) <= band
    if c["use_rs"]:
        ls = res["log_rs_stat"]
        for b in (c["rs_lower"], c["rs_upper"]):
            near |= np.abs(ls - np.log(np.float64(b))) <= band
    if c["veto"] > 0:
        lC = np.log(np.float64(c["veto"]))
        near |= np.abs(res["d"] - lC) <= band
        near |= (np.abs(res["min_d"] - lC) <= band)[res["seq"]]
    return near
