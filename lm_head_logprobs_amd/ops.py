"""Torch-facing wrappers over the C ABI: allocate outputs and workspace, marshal.

These functions do no arithmetic of the method; they size and allocate device
buffers with torch (memory plumbing), fill the C structs and call the library
on the current HIP stream.
"""

from __future__ import annotations

import torch

from . import _lib as L

_LOSS = {"ipo": L.RL_LOSS_IPO, "icepop": L.RL_LOSS_ICEPOP, "reinforce": L.RL_LOSS_REINFORCE}
_KL = {"none": L.RL_KL_NONE, "exact": L.RL_KL_EXACT, "k1": L.RL_KL_K1}
_BWD = {"auto": L.RL_BWD_AUTO, "dense": L.RL_BWD_DENSE, "sparse": L.RL_BWD_SPARSE,
        "none": L.RL_BWD_NONE}


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return L.RL_DTYPE_BF16
    if t == torch.float32:
        return L.RL_DTYPE_FP32
    raise TypeError(f"unsupported dtype {t}")


_STALE = {"none": L.RL_STALENESS_NONE, "inv_sqrt": L.RL_STALENESS_INV_SQRT}


def make_cfg(N, H, V, nnz, dtype: torch.dtype, params: dict, backward=None, token_chunk=0,
             grad_dtype: torch.dtype | None = None, accumulate_dW=False) -> L.RlLossCfg:
    c = L.RlLossCfg()
    c.N, c.H, c.V, c.nnz = int(N), int(H), int(V), int(nnz)
    c.token_chunk = int(token_chunk)
    c.dtype = _dtype_code(dtype)
    c.grad_dtype = _dtype_code(grad_dtype if grad_dtype is not None else dtype)
    c.loss_type = _LOSS[params["loss_type"]]
    c.kl_estimator = _KL[params.get("kl_estimator", "none")]
    c.backward = _BWD[backward if backward is not None else params.get("backward", "auto")]
    c.replayed = int(bool(params.get("replayed", False)))
    c.accumulate_dW = int(bool(accumulate_dW))
    c.kl_staleness = _STALE[params.get("kl_staleness", "none")]
    c.entropy_coeff = float(params.get("entropy_coeff", 0.0))
    c.reserved1 = 0
    c.ipo_eps = float(params.get("ipo_eps", 0.3))
    c.max_ratio = float(params.get("max_ratio", 5.0))
    c.icepop_lo = float(params.get("icepop_lo", 0.5))
    c.icepop_hi = float(params.get("icepop_hi", 2.0))
    c.adv_tau = float(params.get("adv_tau", 1.0))
    c.kl_coeff = float(params.get("kl_coeff", 0.0))
    c.inv_temperature = float(params.get("inv_temperature", 1.0))
    c.loss_norm = float(params.get("loss_norm", N))
    return c


class FusedHead:
    """Preallocated outputs + workspace for repeated rl_loss_fwd_bwd calls."""

    def __init__(self, h, W, labels, infer_logprobs, adv, params, offsets_host=None, ids=None,
                 u=None, logq=None, want_dh=True, want_dW=True, backward=None, token_chunk=0,
                 grad_dtype=None, accumulate_dW=False, want_token_outputs=True, age=None):
        dev = h.device
        N, H = h.shape
        V = W.shape[0]
        self.args = (h, W, labels, infer_logprobs, adv)
        self.has_support = offsets_host is not None
        nnz = int(ids.numel()) if self.has_support else 0
        self.offsets_host = offsets_host.contiguous() if self.has_support else None
        self.offsets_dev = offsets_host.to(dev) if self.has_support else None
        self.ids, self.u, self.logq = ids, u, logq
        self.age = age  # int32 [N] device policy age, or None
        self.cfg = make_cfg(N, H, V, nnz, h.dtype, params, backward, token_chunk, grad_dtype,
                            accumulate_dW)
        gd = grad_dtype if grad_dtype is not None else h.dtype
        f32 = dict(device=dev, dtype=torch.float32)
        self.o = dict(loss=torch.empty(1, **f32),
                      metrics=torch.empty(L.RL_METRIC_COUNT, **f32))
        if want_token_outputs:
            self.o.update(token_loss=torch.empty(N, **f32), logprobs=torch.empty(N, **f32),
                          entropy=torch.empty(N, **f32), weight=torch.empty(N, **f32),
                          keep=torch.empty(N, device=dev, dtype=torch.uint8))
            if self.has_support:
                self.o["support_logprobs"] = torch.empty(nnz, **f32)
        if want_dh:
            self.o["dh"] = torch.empty(N, H, device=dev, dtype=gd)
        if want_dW:
            self.o["dW"] = torch.zeros(V, H, **f32) if accumulate_dW else torch.empty(V, H, **f32)
        self.out = L.RlLossOut()
        for k, v in self.o.items():
            setattr(self.out, k, v.data_ptr())
        self.ws_bytes = L.rl_loss_workspace_size(self.cfg, self.has_support, want_dh, want_dW)
        self.workspace = torch.empty(max(self.ws_bytes, 256), device=dev, dtype=torch.uint8)

    def __call__(self, stream=None, check=True):
        h, W, labels, lq, adv = self.args
        return L.rl_loss_fwd_bwd(h, W, labels, lq, adv, self.age, self.offsets_host,
                                 self.offsets_dev,
                                 self.ids, self.u, self.logq, self.cfg, self.out, self.workspace,
                                 self.ws_bytes, stream=stream, check=check)


def fused_head(h, W, labels, infer_logprobs, adv, params, offsets_host=None, ids=None, u=None,
               logq=None, **kw) -> dict:
    """One call; returns the output tensors (device)."""
    fh = FusedHead(h, W, labels, infer_logprobs, adv, params, offsets_host, ids, u, logq, **kw)
    fh()
    return fh.o


def elem_cfg(params: dict) -> L.RlElemCfg:
    c = L.RlElemCfg()
    eps = list(params["eps"])
    c.n_eps = len(eps)
    c.primary_eps_index = int(params["primary_eps_index"])
    for i in range(L.RL_ELEM_MAX_EPS):
        c.eps[i] = float(eps[i]) if i < len(eps) else 0.0
    c.max_ratio = float(params["max_ratio"])
    c.icepop_lo = float(params["icepop_lo"])
    c.icepop_hi = float(params["icepop_hi"])
    c.clip_low = float(params["clip_low"])
    c.clip_high = float(params["clip_high"])
    c.clip_c = float(params["clip_c"])
    c.tis_upper = float(params["tis_upper"])
    return c


class Replay:
    """Preallocated outputs + workspace for rl_loss_elementwise."""

    def __init__(self, lp, lq, adv, params):
        dev = lp.device
        self.N = lp.numel()
        self.args = (lp, lq, adv)
        self.cfg = elem_cfg(params)
        self.o = dict(mask_word=torch.empty(self.N, device=dev, dtype=torch.int16),
                      w_primary=torch.empty(self.N, device=dev, dtype=torch.float32),
                      sums=torch.empty(L.RL_ELEM_SUM_COUNT, device=dev, dtype=torch.float64))
        self.out = L.RlElemOut()
        for k, v in self.o.items():
            setattr(self.out, k, v.data_ptr())
        self.ws_bytes = L.rl_elementwise_workspace_size(self.N)
        self.workspace = torch.empty(self.ws_bytes, device=dev, dtype=torch.uint8)

    def __call__(self, stream=None, check=True):
        lp, lq, adv = self.args
        return L.rl_loss_elementwise(lp, lq, adv, self.N, self.cfg, self.out, self.workspace,
                                     self.ws_bytes, stream=stream, check=check)


_LEVELS = {"token": L.RL_LEVEL_TOKEN, "sequence": L.RL_LEVEL_SEQUENCE,
           "geometric": L.RL_LEVEL_GEOMETRIC}
_MODES = {"truncate": L.RL_TIS_TRUNCATE, "clip": L.RL_TIS_CLIP, "mask": L.RL_TIS_MASK}


def mis_cfg(params: dict) -> L.RlMisCfg:
    c = L.RlMisCfg()
    c.tis_level = _LEVELS[params["tis_level"]]
    c.tis_mode = _MODES[params["tis_mode"]]
    c.tis_lower = float(params["tis_lower"])
    c.tis_upper = float(params["tis_upper"])
    c.use_rs = int(bool(params["use_rs"]))
    c.rs_level = _LEVELS[params["rs_level"]]
    nan = float("nan")
    c.rs_lower = nan if params.get("rs_lower") is None else float(params["rs_lower"])
    c.rs_upper = nan if params.get("rs_upper") is None else float(params["rs_upper"])
    c.veto = float(params["veto"])
    c.batch_normalize = int(bool(params["batch_normalize"]))
    return c


class MisReplay:
    """Preallocated outputs, device offsets and workspace for rl_mis_replay.

    offsets: int64 [S + 1] on the host (CPU tensor); a device copy is made once.
    """

    def __init__(self, lp, lq, adv, offsets, params):
        dev = lp.device
        self.N = lp.numel()
        self.args = (lp, lq, adv)
        self.offsets_host = offsets.to(torch.int64).contiguous().cpu()
        self.S = self.offsets_host.numel() - 1
        self.offsets_dev = self.offsets_host.to(dev)
        self.cfg = mis_cfg(params)
        self.o = dict(weight=torch.empty(self.N, device=dev, dtype=torch.float32),
                      flags=torch.empty(self.N, device=dev, dtype=torch.uint8),
                      metrics=torch.empty(L.RL_MIS_METRIC_COUNT, device=dev, dtype=torch.float64))
        self.out = L.RlMisOut()
        for k, v in self.o.items():
            setattr(self.out, k, v.data_ptr())
        self.ws_bytes = L.rl_mis_workspace_size(self.N, self.S)
        self.workspace = torch.empty(self.ws_bytes, device=dev, dtype=torch.uint8)

    def __call__(self, stream=None, check=True):
        lp, lq, adv = self.args
        return L.rl_mis_replay(lp, lq, adv, self.N, self.offsets_host, self.offsets_dev, self.S,
                               self.cfg, self.out, self.workspace, self.ws_bytes, stream=stream,
                               check=check)

    def metrics(self) -> dict:
        m = self.o["metrics"].cpu().numpy()
        return {k: float(m[i]) for i, k in enumerate(L.MIS_METRIC_NAMES)}


def validate(labels, infer_logprobs, adv, V, offsets_host=None, ids=None, u=None, logq=None,
             replayed=False, sync=True):
    dev = labels.device
    N = labels.numel()
    nnz = 0 if offsets_host is None else int(ids.numel())
    offsets_dev = None if offsets_host is None else offsets_host.to(dev)
    flags = torch.zeros(1, device=dev, dtype=torch.int32)
    if sync:
        return L.rl_validate_support_sync(N, V, nnz, labels, infer_logprobs, adv, offsets_host,
                                          offsets_dev, ids, u, logq, replayed, flags)
    L.rl_validate_support(N, V, nnz, labels, infer_logprobs, adv, offsets_host, offsets_dev, ids,
                          u, logq, replayed, flags)
    return flags
