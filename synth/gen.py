"""Seeded generators for the five workloads of the fused head and the replay.

Notation: N tokens, H hidden size, V vocabulary.  ``N(0, x)`` in the workload
descriptions means variance x (so ``N(0, 0.3)`` is standard deviation
sqrt(0.3)); ``Exp(m)`` has mean m.

What is drawn here is what an inference engine and a batch packer hand to the
trainer:

* hidden states ``h`` [N,H] and head weights ``W`` [V,H] (bf16 by round to
  nearest even from fp32 draws, or fp32);
* the sampled label of each token;
* the sampler's log-probability of that label (``infer_logprobs``), taken
  from "inference logits" = training logits + Gaussian noise, which models the
  trainer/inference mismatch;
* per-token advantages;
* optionally a ragged per-token support in CSR form: either the replayed
  top-p set of the inference softmax (weights u = renormalised q), or K
  i.i.d. draws from the untruncated inference softmax (u = 1/K).

The sampler needs the logits to draw from them, so this module multiplies
h by W and normalises the inference logits; that is the inference engine's
arithmetic.  The trainer-side quantities the method computes (training
log-softmax, entropy, weights, masks, loss, gradients) are never formed
here.

Every random stream has its own ``torch.Generator`` derived from (seed,
stream, chunk), so results do not depend on which device-side kernels ran
before.  Work over [tokens, V] is done in token chunks of fixed size, so a
given (config, seed, device) always yields the same tensors.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

_STREAMS = {
    "h": 1,
    "W": 2,
    "label": 3,
    "noise": 4,
    "adv": 5,
    "support": 6,
    "scale": 7,
    "extra": 8,
}

# Token chunk used for every [chunk, V] pass of the generator.  Part of the
# recipe: changing it changes the drawn numbers.
GEN_CHUNK = 1024


def _gen(device, seed: int, stream: str, chunk: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    mixed = (seed * 0x9E3779B1 + _STREAMS[stream] * 0x85EBCA6B + chunk * 0xC2B2AE35) % (2**62)
    g.manual_seed(int(mixed))
    return g


@dataclasses.dataclass
class HeadWorkload:
    """Inputs of one fused-head call plus the loss settings of the workload."""

    name: str
    N: int
    H: int
    V: int
    dtype: str  # "bf16" or "fp32": storage type of h and W
    h: torch.Tensor  # [N,H]
    W: torch.Tensor  # [V,H]
    labels: torch.Tensor  # int32 [N]
    infer_logprobs: torch.Tensor  # fp32 [N], sampler log q(label)
    adv: torch.Tensor  # fp32 [N]
    offsets: Optional[torch.Tensor]  # int64 [N+1], host memory
    ids: Optional[torch.Tensor]  # int32 [nnz]
    u: Optional[torch.Tensor]  # fp32 [nnz]
    logq: Optional[torch.Tensor]  # fp32 [nnz], sampler log q(id)
    params: dict  # loss settings (type, eps, max_ratio, KL, ...)
    info: dict  # generation report (support sizes, seeds)

    @property
    def nnz(self) -> int:
        return 0 if self.ids is None else int(self.ids.numel())

    def to_host_numpy(self) -> dict:
        """Exact host copies (bf16 widened to fp32 exactly) for the oracle."""
        def cpu(t):
            if t is None:
                return None
            t = t.detach().to("cpu")
            if t.dtype == torch.bfloat16:
                t = t.float()
            return t.numpy()

        return dict(
            h=cpu(self.h), W=cpu(self.W), labels=cpu(self.labels),
            infer_logprobs=cpu(self.infer_logprobs), adv=cpu(self.adv),
            offsets=cpu(self.offsets), ids=cpu(self.ids), u=cpu(self.u),
            logq=cpu(self.logq),
        )


# Workload recipes.  ``w_std`` is the standard deviation of W, ``noise_std``
# that of the inference-logit noise.  Loss settings follow the workloads:
# IPO eps 0.3 with max ratio 5 everywhere IPO is used.
HEAD_CONFIGS = {
    "c1_tiny_fp32_ipo": dict(
        N=64, H=64, V=1000, dtype="fp32", w_std=None, noise_std=math.sqrt(0.3),
        support=None, seed=1001,
        params=dict(loss_type="ipo", ipo_eps=0.3, max_ratio=5.0, kl_coeff=0.0,
                    kl_estimator="none", replayed=False, backward="dense"),
    ),
    "c3_head16k_ipo": dict(
        N=16384, H=2048, V=152064, dtype="bf16", w_std=0.02, noise_std=math.sqrt(0.1),
        support=None, seed=1003,
        params=dict(loss_type="ipo", ipo_eps=0.3, max_ratio=5.0, kl_coeff=0.0,
                    kl_estimator="none", replayed=False, backward="dense"),
    ),
    "c4_head16k_ipo_topp_replay": dict(
        N=16384, H=2048, V=152064, dtype="bf16", w_std=0.02, noise_std=math.sqrt(0.1),
        support="topp", top_p=0.97, k_median=30.0, k_sigma=1.0, k_max=2048, seed=1004,
        params=dict(loss_type="ipo", ipo_eps=0.3, max_ratio=5.0, kl_coeff=0.05,
                    kl_estimator="exact", replayed=True, backward="dense"),
    ),
    "c5a_head64k_draws_ipo_k1": dict(
        N=65536, H=2048, V=152064, dtype="bf16", w_std=0.02, noise_std=math.sqrt(0.1),
        support="draws", K=16, seed=1005,
        params=dict(loss_type="ipo", ipo_eps=0.3, max_ratio=5.0, kl_coeff=0.05,
                    kl_estimator="k1", replayed=False, backward="dense"),
    ),
    "c5b_head64k_draws_reinforce": dict(
        N=65536, H=2048, V=152064, dtype="bf16", w_std=0.02, noise_std=math.sqrt(0.1),
        support="draws", K=16, seed=1005,
        params=dict(loss_type="reinforce", ipo_eps=0.3, max_ratio=5.0, kl_coeff=0.0,
                    kl_estimator="none", replayed=False, backward="sparse"),
    ),
}


def _round_store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return x.to(torch.bfloat16)  # round to nearest even
    return x.to(torch.float32)


def _logits(h_chunk: torch.Tensor, W32: torch.Tensor) -> torch.Tensor:
    # The sampler's logits from the stored (rounded) values, in fp32.
    return h_chunk.float() @ W32.t()


def _top_p_sizes(y: torch.Tensor, p: float) -> torch.Tensor:
    """Size of the smallest most-likely prefix of softmax(y) with mass >= p."""
    pr = torch.softmax(y.float(), dim=1)
    srt, _ = torch.sort(pr, dim=1, descending=True)
    cs = torch.cumsum(srt.double(), dim=1)
    k = (cs < p).sum(dim=1) + 1
    return k.clamp_(max=y.shape[1])


def make_head(name: str, device="cpu", *, N: Optional[int] = None, H: Optional[int] = None,
              V: Optional[int] = None, seed: Optional[int] = None,
              adv_zero_except: Optional[torch.Tensor] = None) -> HeadWorkload:
    """Draw one fused-head workload.

    ``N``, ``H``, ``V`` override the recipe's sizes (same distributions) for
    small parity cases.  ``adv_zero_except`` (a bool [N] mask) zeroes the
    advantage of every other token; with no KL term such tokens carry no
    gradient, which lets the full-size weight gradient be checked against
    the oracle on a token sample.
    """
    rc = HEAD_CONFIGS[name]
    N = rc["N"] if N is None else N
    H = rc["H"] if H is None else H
    V = rc["V"] if V is None else V
    seed = rc["seed"] if seed is None else seed
    dtype = rc["dtype"]
    dev = torch.device(device)
    w_std = rc["w_std"] if rc["w_std"] is not None else 1.0 / math.sqrt(H)
    noise_std = rc["noise_std"]

    h = torch.randn(N, H, generator=_gen(dev, seed, "h"), device=dev, dtype=torch.float32)
    W = torch.randn(V, H, generator=_gen(dev, seed, "W"), device=dev, dtype=torch.float32) * w_std
    adv = torch.randn(N, generator=_gen(dev, seed, "adv"), device=dev, dtype=torch.float32)
    if adv_zero_except is not None:
        adv = torch.where(adv_zero_except.to(dev), adv, torch.zeros_like(adv))
    W_st = _round_store(W, dtype)
    del W
    W32 = W_st.float()

    support = rc.get("support")
    info: dict = dict(seed=seed, recipe=name, N=N, H=H, V=V)
    if support == "topp":
        kmax = min(rc["k_max"], V)
        kt = torch.exp(math.log(rc["k_median"]) + rc["k_sigma"]
                       * torch.randn(N, generator=_gen(dev, seed, "scale"), device=dev,
                                     dtype=torch.float64))
        k_target = torch.round(kt).clamp_(1, kmax).to(torch.int64)
        alpha = torch.ones(N, device=dev, dtype=torch.float32)
        h_rounded = _round_store(h, dtype).float()
        for c0 in range(0, N, GEN_CHUNK):
            c1 = min(N, c0 + GEN_CHUNK)
            ci = c0 // GEN_CHUNK
            z = _logits(h_rounded[c0:c1], W32)
            n = torch.randn(c1 - c0, V, generator=_gen(dev, seed, "noise", ci), device=dev) * noise_std
            lo = torch.full((c1 - c0,), -5.0, device=dev, dtype=torch.float64)
            hi = torch.full((c1 - c0,), 7.0, device=dev, dtype=torch.float64)
            tgt = k_target[c0:c1]
            for _ in range(24):
                mid = 0.5 * (lo + hi)
                k = _top_p_sizes(torch.exp(mid).float()[:, None] * z + n, rc["top_p"])
                too_big = k > tgt
                lo = torch.where(too_big, mid, lo)
                hi = torch.where(too_big, hi, mid)
            alpha[c0:c1] = torch.exp(0.5 * (lo + hi)).float()
            del z, n
        h = h * alpha[:, None]
        info["k_target_median"] = float(k_target.double().median())
    h_st = _round_store(h, dtype)
    del h

    labels = torch.empty(N, dtype=torch.int32, device=dev)
    infer_lp = torch.empty(N, dtype=torch.float32, device=dev)
    offs_list, ids_list, u_list, lq_list = [0], [], [], []
    nnz_acc = 0
    for c0 in range(0, N, GEN_CHUNK):
        c1 = min(N, c0 + GEN_CHUNK)
        ci = c0 // GEN_CHUNK
        z = _logits(h_st[c0:c1], W32)
        n = torch.randn(c1 - c0, V, generator=_gen(dev, seed, "noise", ci), device=dev) * noise_std
        y = z + n  # inference logits
        if support == "topp":
            ys, idx = torch.sort(y, dim=1, descending=True)
            lse_full = torch.logsumexp(y.double(), dim=1)
            csum = torch.cumsum(torch.exp(ys.double() - lse_full[:, None]), dim=1)
            k = ((csum < rc["top_p"]).sum(dim=1) + 1).clamp_(max=V)
            kmax_c = int(k.max())
            ys_k = ys[:, :kmax_c].double()
            keep = torch.arange(kmax_c, device=dev)[None, :] < k[:, None]
            lse_s = torch.logsumexp(torch.where(keep, ys_k, torch.full_like(ys_k, -math.inf)), dim=1)
            logq_pad = ys_k - lse_s[:, None]
            q_pad = torch.where(keep, torch.exp(logq_pad), torch.zeros_like(logq_pad))
            logq32 = logq_pad.float()
            j = torch.multinomial(q_pad, 1, generator=_gen(dev, seed, "label", ci)).squeeze(1)
            labels[c0:c1] = idx[:, :kmax_c].gather(1, j[:, None]).squeeze(1).to(torch.int32)
            infer_lp[c0:c1] = logq32.gather(1, j[:, None]).squeeze(1)
            ids_list.append(idx[:, :kmax_c][keep].to(torch.int32))
            u_list.append(q_pad[keep].float())
            lq_list.append(logq32[keep])
            for kk in k.tolist():
                nnz_acc += kk
                offs_list.append(nnz_acc)
            del ys, idx, csum
        else:
            pz = torch.softmax(z, dim=1)
            a = torch.multinomial(pz, 1, generator=_gen(dev, seed, "label", ci)).squeeze(1)
            labels[c0:c1] = a.to(torch.int32)
            lq_full = torch.log_softmax(y.double(), dim=1)
            infer_lp[c0:c1] = lq_full.gather(1, a[:, None]).squeeze(1).float()
            if support == "draws":
                K = rc["K"]
                py = torch.softmax(y.double(), dim=1)
                d = torch.multinomial(py, K, replacement=True, generator=_gen(dev, seed, "support", ci))
                ids_list.append(d.reshape(-1).to(torch.int32))
                lq_list.append(lq_full.gather(1, d).reshape(-1).float())
                u_list.append(torch.full((d.numel(),), 1.0 / K, device=dev, dtype=torch.float32))
                del py, d
            del pz, lq_full
        del z, n, y

    if support == "draws":
        K = rc["K"]
        offsets = torch.arange(N + 1, dtype=torch.int64) * K
    elif support == "topp":
        offsets = torch.tensor(offs_list, dtype=torch.int64)
    else:
        offsets = None
    ids = torch.cat(ids_list) if ids_list else None
    u = torch.cat(u_list) if u_list else None
    logq = torch.cat(lq_list) if lq_list else None
    if offsets is not None:
        sizes = (offsets[1:] - offsets[:-1]).double()
        info.update(nnz=int(offsets[-1]), k_median=float(sizes.median()),
                    k_mean=float(sizes.mean()), k_max=int(sizes.max()), k_min=int(sizes.min()))
    params = dict(rc["params"])
    params.update(adv_tau=1.0, inv_temperature=1.0, loss_norm=float(N))
    return HeadWorkload(name=name, N=N, H=H, V=V, dtype=dtype, h=h_st, W=W_st,
                        labels=labels, infer_logprobs=infer_lp, adv=adv,
                        offsets=offsets, ids=ids, u=u, logq=logq,
                        params=params, info=info)


@dataclasses.dataclass
class ReplayWorkload:
    """Token pairs of the loss-only mismatch replay."""

    N: int
    lp: torch.Tensor  # fp32 [N], trainer log p(label)
    lq: torch.Tensor  # fp32 [N], sampler log q(label)
    adv: torch.Tensor  # fp32 [N]
    params: dict
    info: dict


REPLAY_PARAMS = dict(
    eps=(0.05, 0.1, 0.2, 0.3, 0.5),
    primary_eps_index=3,
    max_ratio=5.0,
    icepop_lo=0.5,
    icepop_hi=2.0,
    clip_low=0.2,
    clip_high=0.2,
    clip_c=3.0,
    tis_upper=2.0,
)


def make_replay(N: int = 2_160_000, device="cpu", seed: int = 1002) -> ReplayWorkload:
    """log q: 60% -Exp(mean 0.05), 40% -Exp(mean 3); log p = min(log q + N(0, 0.15), 0)."""
    dev = torch.device(device)
    g = _gen(dev, seed, "extra")
    comp = torch.rand(N, generator=g, device=dev, dtype=torch.float64) < 0.6
    e_near = torch.empty(N, device=dev, dtype=torch.float64).exponential_(1.0 / 0.05, generator=g)
    e_far = torch.empty(N, device=dev, dtype=torch.float64).exponential_(1.0 / 3.0, generator=g)
    lq = -torch.where(comp, e_near, e_far)
    n = torch.randn(N, generator=_gen(dev, seed, "noise"), device=dev, dtype=torch.float64) * math.sqrt(0.15)
    lp_raw = lq + n
    clamped = int((lp_raw > 0).sum())
    lp = torch.clamp(lp_raw, max=0.0)
    adv = torch.randn(N, generator=_gen(dev, seed, "adv"), device=dev, dtype=torch.float32)
    return ReplayWorkload(N=N, lp=lp.float(), lq=lq.float(), adv=adv,
                          params=dict(REPLAY_PARAMS),
                          info=dict(seed=seed, clamped_to_zero=clamped))


# Sequence-aware rollout correction on the replay (Rollout Correction Methods
# page, "Config keys"): geometric-level TIS in clip mode, sequence-level
# rejection with the TIS bounds, the veto at the low end of the page's typical
# range, batch normalisation on.
MIS_PARAMS = dict(
    tis_level="geometric",
    tis_mode="clip",
    tis_lower=0.5,
    tis_upper=2.0,
    use_rs=True,
    rs_level="sequence",
    rs_lower=None,
    rs_upper=None,
    veto=1e-4,
    batch_normalize=True,
)


def replay_sequences(N: int, seed: int = 1002, median: float = 1024.0, sigma_log: float = 1.0,
                     max_len: int = 32768) -> torch.Tensor:
    """Offsets [S + 1] (int64, CPU) cutting N replay tokens into responses.

    The pages give no response lengths for the replayed agentic run; lengths
    are lognormal (median 1024 tokens, sigma of the log 1.0), rounded, clipped
    to [1, max_len], and the last response is cut to end at N.
    """
    g = _gen("cpu", seed, "scale")
    lens = []
    total = 0
    while total < N:
        z = torch.randn(4096, generator=g, dtype=torch.float64)
        L = torch.clamp(torch.round(median * torch.exp(sigma_log * z)), 1, max_len).long()
        for x in L.tolist():
            if total >= N:
                break
            x = min(x, N - total)
            lens.append(x)
            total += x
    off = torch.zeros(len(lens) + 1, dtype=torch.int64)
    off[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0)
    return off


def policy_ages(N: int, device="cpu", seed: int = 1003, max_age: int = 8) -> torch.Tensor:
    """Per-token policy age (inference weight-version lag) as int32 [N].

    The pages name the per-token age stream without its distribution: ages
    follow a geometric lag (P(age = k) = 2^-(k+1)), capped at max_age, so about
    half the tokens are fresh.
    """
    g = _gen("cpu", seed, "extra", chunk=1)
    u = torch.rand(N, generator=g, dtype=torch.float64)
    age = torch.clamp(torch.floor(-torch.log2(1.0 - u)), 0, max_age).to(torch.int32)
    return age.to(device)
