"""Loss-only mismatch replay over (log p_train, log q_infer, A) pairs, fp64.

Test infrastructure.  Per token, from lp = log pi_train(y), lq = log
pi_infer(y) and advantage A:  P = e^lp, Q = e^lq, r = e^(lp - lq).

Variants, each with its source:
* IPO for every eps of a sweep -- IPO documentation page, "Masking by
  Probability, Not Ratio": masked iff |P - Q| > eps; weight (prime-rl PR 4233,
  "What changes") w = 1(kept) * min(r, max_importance_ratio).
* IcePop band [lo, hi] -- same two sources: kept iff lo <= r <= hi, w = kept * r.
  "low" counts r < lo, "high" counts r > hi.
* REINFORCE -- PR 4233: w = 1.
  For these three the per-token loss is the RLLoss value with no support and
  no KL: l = -A * w * lp.
* PPO with the rollout log-prob as the old policy -- Rollout Correction
  Methods page, "Bypassing PPO importance sampling": ratio r = pi_theta /
  pi_rollout; J1 = r A, J2 = clip(r, 1 - eps_low, 1 + eps_high) A,
  J = min(J1, J2); with dual clip (Tencent article on KL/clip/entropy, section
  2, defaults 0.2 / 0.2 / 3.0): for A < 0, J = max(J, c A).  l = -J.
  clipfrac counts J2 < J1; clipfrac_lower counts A < 0 with c A > min(J1, J2);
  ppo_kl sums lq - lp.
* Decoupled 3-policy PPO with token-level TIS, truncate mode -- Rollout
  Correction Methods page, "Decoupled, 3-policy PPO Importance Sampling" and
  "Importance Sampling / Token Level": rho = exp(log pi_old - log pi_rollout),
  truncated at U: w_tis = min(rho, U).  The replay has no separate proximal
  policy, so pi_old := pi_train and the inner PPO ratio pi_theta / pi_old is 1;
  the clipped surrogate then equals A and l = -w_tis * A.  "truncated"
  counts rho > U.

Outputs: per-token mask word bits and the primary IPO weight, and per-variant
sums (loss sum, kept count, weight sum, band counts).  Loss reductions:
primary token-mean  sum(l) / N, secondary rejection-style mean over kept
tokens  sum(kept * l) / sum(kept).
"""

import numpy as np

# Mask-word bit positions (one uint16 per token).
BIT_IPO0 = 0  # bits 0..7: IPO eps[i] masked
BIT_ICEPOP_LOW = 8
BIT_ICEPOP_HIGH = 9
BIT_PPO_CLIP = 10
BIT_DUAL_CLIP = 11
BIT_TIS_TRUNC = 12


def replay_reference(lp, lq, A, params):
    lp = np.asarray(lp, np.float64)
    lq = np.asarray(lq, np.float64)
    A = np.asarray(A, np.float64)
    N = len(lp)
    P = np.exp(lp)
    Q = np.exp(lq)
    r = np.exp(lp - lq)
    M = params["max_ratio"]
    word = np.zeros(N, np.uint32)
    res = {"N": N}
    near = {}
    for i, eps in enumerate(params["eps"]):
        masked = np.abs(P - Q) > eps
        w = np.where(masked, 0.0, np.minimum(r, M))
        loss = -A * w * lp
        word |= masked.astype(np.uint32) << (BIT_IPO0 + i)
        res[f"ipo{i}_kept"] = int((~masked).sum())
        res[f"ipo{i}_loss_sum"] = loss.sum()
        res[f"ipo{i}_weight_sum"] = w.sum()
        near[f"ipo{i}"] = np.abs(np.abs(P - Q) - eps)
        if i == params["primary_eps_index"]:
            res["w_primary"] = w
    lo, hi = params["icepop_lo"], params["icepop_hi"]
    low = r < lo
    high = r > hi
    kept = ~(low | high)
    w = np.where(kept, r, 0.0)
    loss = -A * w * lp
    word |= low.astype(np.uint32) << BIT_ICEPOP_LOW
    word |= high.astype(np.uint32) << BIT_ICEPOP_HIGH
    res.update(icepop_kept=int(kept.sum()), icepop_low=int(low.sum()),
               icepop_high=int(high.sum()), icepop_loss_sum=loss.sum(),
               icepop_weight_sum=w.sum())
    near["icepop_low"] = np.abs(r - lo)
    near["icepop_high"] = np.abs(r - hi)
    res["reinforce_loss_sum"] = (-A * lp).sum()
    # PPO-bypass with dual clip.
    el, eh, c = params["clip_low"], params["clip_high"], params["clip_c"]
    J1 = r * A
    J2 = np.clip(r, 1.0 - el, 1.0 + eh) * A
    Jmin = np.minimum(J1, J2)
    dual = (A < 0) & (c * A > Jmin)
    J = np.where(A < 0, np.maximum(Jmin, c * A), Jmin)
    clip = J2 < J1
    word |= clip.astype(np.uint32) << BIT_PPO_CLIP
    word |= dual.astype(np.uint32) << BIT_DUAL_CLIP
    res.update(ppo_loss_sum=(-J).sum(), ppo_clip=int(clip.sum()),
               ppo_clip_lower=int(dual.sum()), ppo_kl_sum=(lq - lp).sum())
    near["ppo_clip"] = np.minimum(np.abs(r - (1.0 - el)), np.abs(r - (1.0 + eh)))
    near["dual_clip"] = np.abs(Jmin - c * A)
    # Decoupled PPO, token-level TIS in truncate mode, pi_old := pi_train.
    U = params["tis_upper"]
    rho = np.exp(lp - lq)
    trunc = rho > U
    w_tis = np.minimum(rho, U)
    word |= trunc.astype(np.uint32) << BIT_TIS_TRUNC
    res.update(tis_loss_sum=(-w_tis * A).sum(), tis_truncated=int(trunc.sum()),
               tis_weight_sum=w_tis.sum())
    near["tis"] = np.abs(rho - U)
    res["mask_word"] = word.astype(np.uint16)
    res["near"] = near
    res["P"] = P
    return res


def near_threshold_bits(res, band):
    """Per-token mask of word bits whose decision lies within ``band`` of its threshold."""
    N = res["N"]
    bits = np.zeros(N, np.uint32)
    near = res["near"]
    i = 0
    while f"ipo{i}" in near:
        bits |= (near[f"ipo{i}"] <= band).astype(np.uint32) << (BIT_IPO0 + i)
        i += 1
    bits |= (near["icepop_low"] <= band).astype(np.uint32) << BIT_ICEPOP_LOW
    bits |= (near["icepop_high"] <= band).astype(np.uint32) << BIT_ICEPOP_HIGH
    bits |= (near["ppo_clip"] <= band).astype(np.uint32) << BIT_PPO_CLIP
    bits |= (near["dual_clip"] <= band).astype(np.uint32) << BIT_DUAL_CLIP
    bits |= (near["tis"] <= band).astype(np.uint32) << BIT_TIS_TRUNC
    return bits.astype(np.uint16)
