"""ctypes binding of librlloss (include/rlloss.h).

Argument marshalling only: the functions below carry the C names, take torch
tensors (device memory) or plain integers, and pass their data pointers and the
caller's HIP stream to the library.  Every step of the computation runs in the
library's HIP kernels.  If the shared library is missing this module raises on
first use: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# RL_LIB_PATH selects another build of the same library (the host-sanitizer
# build the ABI tests run under); by default the in-tree librlloss.so.
LIB_PATH = os.environ.get("RL_LIB_PATH") or os.path.join(_HERE, "librlloss.so")

RL_OK, RL_E_ARG, RL_E_CFG, RL_E_CSR, RL_E_WORKSPACE, RL_E_HIP, RL_E_INVALID_INPUT = range(7)
RL_DTYPE_FP32, RL_DTYPE_BF16 = 0, 1
RL_LOSS_IPO, RL_LOSS_ICEPOP, RL_LOSS_REINFORCE = 0, 1, 2
RL_KL_NONE, RL_KL_EXACT, RL_KL_K1 = 0, 1, 2
RL_STALENESS_NONE, RL_STALENESS_INV_SQRT = 0, 1
RL_BWD_AUTO, RL_BWD_DENSE, RL_BWD_SPARSE, RL_BWD_NONE = 0, 1, 2, 3
METRIC_NAMES = ("masked_fraction", "support_mass", "mask_tv", "kl", "kl_beta", "max_abs_kappa",
                "entropy_mean", "kl_age0")
RL_METRIC_COUNT = len(METRIC_NAMES)
RL_ELEM_MAX_EPS = 8
RL_ELEM_SUM_COUNT = 37
RL_LEVEL_TOKEN, RL_LEVEL_SEQUENCE, RL_LEVEL_GEOMETRIC = range(3)
RL_TIS_TRUNCATE, RL_TIS_CLIP, RL_TIS_MASK = range(3)
MIS_METRIC_NAMES = (
    "training_log_ppl", "training_ppl", "rollout_log_ppl", "rollout_ppl", "kl", "k3_kl",
    "log_ppl_diff", "log_ppl_abs_diff", "ppl_ratio", "chi2_token", "chi2_seq",
    "logprob_abs_diff", "tis_weight_before_bound", "tis_weight_after_bound",
    "tis_fraction_low", "tis_fraction_high", "rs_fraction_low", "rs_fraction_high",
    "catastrophic_token_fraction", "catastrophic_seq_fraction", "is_ratio_mean_after_tis_rs",
    "batch_norm_factor", "is_ratio_mean_final", "is_ratio_min_final", "is_ratio_max_final",
    "loss", "loss_sum", "kept_tokens", "rejected_tokens")
RL_MIS_METRIC_COUNT = len(MIS_METRIC_NAMES)
RL_MIS_MAX_N = (1 << 31) - 256

EXPORTED = (
    "rl_loss_workspace_size",
    "rl_loss_fwd_bwd",
    "rl_elementwise_workspace_size",
    "rl_loss_elementwise",
    "rl_loss_elementwise_noalloc",
    "rl_mis_workspace_size",
    "rl_mis_replay",
    "rl_validate_support",
    "rl_validate_support_sync",
    "rl_profile_begin",
    "rl_profile_end",
    "rl_calib_mfma_bf16",
    "rl_calib_copy",
    "rl_status_string",
    "rl_version",
)


class RlLossCfg(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int64), ("H", ctypes.c_int64), ("V", ctypes.c_int64),
        ("nnz", ctypes.c_int64), ("token_chunk", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32),
        ("loss_type", ctypes.c_int32), ("kl_estimator", ctypes.c_int32),
        ("backward", ctypes.c_int32), ("replayed", ctypes.c_int32),
        ("accumulate_dW", ctypes.c_int32), ("kl_staleness", ctypes.c_int32),
        ("ipo_eps", ctypes.c_float), ("max_ratio", ctypes.c_float),
        ("icepop_lo", ctypes.c_float), ("icepop_hi", ctypes.c_float),
        ("adv_tau", ctypes.c_float), ("kl_coeff", ctypes.c_float),
        ("inv_temperature", ctypes.c_float), ("loss_norm", ctypes.c_float),
        ("entropy_coeff", ctypes.c_float), ("reserved1", ctypes.c_int32),
    ]


class RlLossOut(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "loss", "token_loss", "logprobs", "entropy", "weight", "keep", "support_logprobs",
        "dh", "dW", "metrics")]


class RlElemCfg(ctypes.Structure):
    _fields_ = [
        ("n_eps", ctypes.c_int32), ("primary_eps_index", ctypes.c_int32),
        ("eps", ctypes.c_float * RL_ELEM_MAX_EPS),
        ("max_ratio", ctypes.c_float), ("icepop_lo", ctypes.c_float),
        ("icepop_hi", ctypes.c_float), ("clip_low", ctypes.c_float),
        ("clip_high", ctypes.c_float), ("clip_c", ctypes.c_float), ("tis_upper", ctypes.c_float),
    ]


class RlElemOut(ctypes.Structure):
    _fields_ = [("mask_word", ctypes.c_void_p), ("w_primary", ctypes.c_void_p),
                ("sums", ctypes.c_void_p)]


class RlMisCfg(ctypes.Structure):
    _fields_ = [
        ("tis_level", ctypes.c_int32), ("tis_mode", ctypes.c_int32),
        ("tis_lower", ctypes.c_float), ("tis_upper", ctypes.c_float),
        ("use_rs", ctypes.c_int32), ("rs_level", ctypes.c_int32),
        ("rs_lower", ctypes.c_float), ("rs_upper", ctypes.c_float),
        ("veto", ctypes.c_float), ("batch_normalize", ctypes.c_int32),
    ]


class RlMisOut(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("flags", ctypes.c_void_p),
                ("metrics", ctypes.c_void_p)]


class RlProfileEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


class RlError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load librlloss.so (built in-tree); raise if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; "
                "g.build()'); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.rl_loss_workspace_size.argtypes = [ctypes.POINTER(RlLossCfg), i32, i32, i32,
                                             ctypes.POINTER(sz)]
        L.rl_loss_workspace_size.restype = ctypes.c_int
        L.rl_loss_fwd_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      ctypes.POINTER(RlLossCfg), ctypes.POINTER(RlLossOut), vp,
                                      sz, vp]
        L.rl_loss_fwd_bwd.restype = ctypes.c_int
        L.rl_elementwise_workspace_size.argtypes = [i64, ctypes.POINTER(sz)]
        L.rl_elementwise_workspace_size.restype = ctypes.c_int
        L.rl_loss_elementwise.argtypes = [vp, vp, vp, i64, ctypes.POINTER(RlElemCfg),
                                          ctypes.POINTER(RlElemOut), vp, sz, vp]
        L.rl_loss_elementwise.restype = ctypes.c_int
        L.rl_loss_elementwise_noalloc.argtypes = [vp, vp, vp, i64, ctypes.POINTER(RlElemCfg),
                                                  ctypes.POINTER(RlElemOut), vp]
        L.rl_loss_elementwise_noalloc.restype = ctypes.c_int
        L.rl_mis_workspace_size.argtypes = [i64, i64, ctypes.POINTER(sz)]
        L.rl_mis_workspace_size.restype = ctypes.c_int
        L.rl_mis_replay.argtypes = [vp, vp, vp, i64, vp, vp, i64, ctypes.POINTER(RlMisCfg),
                                    ctypes.POINTER(RlMisOut), vp, sz, vp]
        L.rl_mis_replay.restype = ctypes.c_int
        L.rl_validate_support.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp,
                                          vp]
        L.rl_validate_support.restype = ctypes.c_int
        L.rl_validate_support_sync.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                               vp, ctypes.POINTER(ctypes.c_int32), vp]
        L.rl_validate_support_sync.restype = ctypes.c_int
        L.rl_status_string.argtypes = [ctypes.c_int]
        L.rl_status_string.restype = ctypes.c_char_p
        L.rl_version.argtypes = []
        L.rl_version.restype = ctypes.c_char_p
        L.rl_profile_begin.argtypes = []
        L.rl_profile_begin.restype = ctypes.c_int
        L.rl_profile_end.argtypes = [ctypes.POINTER(RlProfileEntry), i32,
                                     ctypes.POINTER(ctypes.c_int32)]
        L.rl_profile_end.restype = ctypes.c_int
        L.rl_calib_mfma_bf16.argtypes = [i32, i32, i64, vp, vp, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(i32), vp]
        L.rl_calib_mfma_bf16.restype = ctypes.c_int
        L.rl_calib_copy.argtypes = [vp, vp, i64, i32, vp]
        L.rl_calib_copy.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(x):
    """Data pointer of a tensor (or None -> NULL, int passes through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def status_string(status: int) -> str:
    return lib().rl_status_string(status).decode()


def rl_version() -> str:
    return lib().rl_version().decode()


def rl_loss_workspace_size(cfg: RlLossCfg, has_support: bool, want_dh: bool, want_dW: bool) -> int:
    n = ctypes.c_size_t(0)
    st = lib().rl_loss_workspace_size(ctypes.byref(cfg), int(has_support), int(want_dh),
                                      int(want_dW), ctypes.byref(n))
    if st != RL_OK:
        raise RlError(st, "rl_loss_workspace_size")
    return n.value


def rl_loss_fwd_bwd(h, W, labels, infer_logprobs, adv, policy_age, csr_offsets_host,
                    csr_offsets_dev, csr_ids, csr_u, csr_logq, cfg: RlLossCfg, out: RlLossOut,
                    workspace, workspace_bytes, stream=None, check=True) -> int:
    st = lib().rl_loss_fwd_bwd(_ptr(h), _ptr(W), _ptr(labels), _ptr(infer_logprobs), _ptr(adv),
                               _ptr(policy_age), _ptr(csr_offsets_host), _ptr(csr_offsets_dev), _ptr(csr_ids),
                               _ptr(csr_u), _ptr(csr_logq), ctypes.byref(cfg), ctypes.byref(out),
                               _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check and st != RL_OK:
        raise RlError(st, "rl_loss_fwd_bwd")
    return st


def rl_elementwise_workspace_size(N: int) -> int:
    n = ctypes.c_size_t(0)
    st = lib().rl_elementwise_workspace_size(int(N), ctypes.byref(n))
    if st != RL_OK:
        raise RlError(st, "rl_elementwise_workspace_size")
    return n.value


def rl_loss_elementwise(lp, lq, adv, N, cfg: RlElemCfg, out: RlElemOut, workspace,
                        workspace_bytes, stream=None, check=True) -> int:
    st = lib().rl_loss_elementwise(_ptr(lp), _ptr(lq), _ptr(adv), int(N), ctypes.byref(cfg),
                                   ctypes.byref(out), _ptr(workspace), int(workspace_bytes),
                                   _stream(stream))
    if check and st != RL_OK:
        raise RlError(st, "rl_loss_elementwise")
    return st


def rl_loss_elementwise_noalloc(lp, lq, adv, N, cfg: RlElemCfg, out: RlElemOut, stream=None,
                                check=True) -> int:
    st = lib().rl_loss_elementwise_noalloc(_ptr(lp), _ptr(lq), _ptr(adv), int(N),
                                           ctypes.byref(cfg), ctypes.byref(out), _stream(stream))
    if check and st != RL_OK:
        raise RlError(st, "rl_loss_elementwise_noalloc")
    return st


def rl_mis_workspace_size(N: int, S: int) -> int:
    n = ctypes.c_size_t(0)
    st = lib().rl_mis_workspace_size(int(N), int(S), ctypes.byref(n))
    if st != RL_OK:
        raise RlError(st, "rl_mis_workspace_size")
    return n.value


def rl_mis_replay(lp, lq, adv, N, seq_offsets_host, seq_offsets_dev, S, cfg: RlMisCfg,
                  out: RlMisOut, workspace, workspace_bytes, stream=None, check=True) -> int:
    st = lib().rl_mis_replay(_ptr(lp), _ptr(lq), _ptr(adv), int(N), _ptr(seq_offsets_host),
                             _ptr(seq_offsets_dev), int(S), ctypes.byref(cfg), ctypes.byref(out),
                             _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check and st != RL_OK:
        raise RlError(st, "rl_mis_replay")
    return st


def rl_validate_support(N, V, nnz, labels, infer_logprobs, adv, csr_offsets_host, csr_offsets_dev,
                        csr_ids, csr_u, csr_logq, replayed, flags_dev, stream=None,
                        check=True) -> int:
    st = lib().rl_validate_support(int(N), int(V), int(nnz), _ptr(labels), _ptr(infer_logprobs),
                                   _ptr(adv), _ptr(csr_offsets_host), _ptr(csr_offsets_dev),
                                   _ptr(csr_ids), _ptr(csr_u), _ptr(csr_logq), int(replayed),
                                   _ptr(flags_dev), _stream(stream))
    if check and st != RL_OK:
        raise RlError(st, "rl_validate_support")
    return st


def rl_validate_support_sync(N, V, nnz, labels, infer_logprobs, adv, csr_offsets_host,
                             csr_offsets_dev, csr_ids, csr_u, csr_logq, replayed, flags_dev,
                             stream=None):
    """Returns (status, flags)."""
    f = ctypes.c_int32(0)
    st = lib().rl_validate_support_sync(int(N), int(V), int(nnz), _ptr(labels),
                                        _ptr(infer_logprobs), _ptr(adv), _ptr(csr_offsets_host),
                                        _ptr(csr_offsets_dev), _ptr(csr_ids), _ptr(csr_u),
                                        _ptr(csr_logq), int(replayed), _ptr(flags_dev),
                                        ctypes.byref(f), _stream(stream))
    if st not in (RL_OK, RL_E_INVALID_INPUT):
        raise RlError(st, "rl_validate_support_sync")
    return st, f.value


def rl_profile_begin() -> None:
    st = lib().rl_profile_begin()
    if st != RL_OK:
        raise RlError(st, "rl_profile_begin")


def rl_profile_end() -> dict:
    """{kernel name: (launches, total_ms)} since rl_profile_begin."""
    arr = (RlProfileEntry * 64)()
    n = ctypes.c_int32(0)
    st = lib().rl_profile_end(arr, 64, ctypes.byref(n))
    if st != RL_OK:
        raise RlError(st, "rl_profile_end")
    return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms))
            for i in range(min(n.value, 64))}


def rl_calib_mfma_bf16(random_operands: bool, n_blocks: int, iters: int, sink, stamps,
                       stream=None):
    """Enqueue the register-only MFMA loop; returns (FLOP of the launch, wall-clock kHz)."""
    flop = ctypes.c_double(0.0)
    khz = ctypes.c_int32(0)
    st = lib().rl_calib_mfma_bf16(int(bool(random_operands)), int(n_blocks), int(iters),
                                  _ptr(sink), _ptr(stamps), ctypes.byref(flop), ctypes.byref(khz),
                                  _stream(stream))
    if st != RL_OK:
        raise RlError(st, "rl_calib_mfma_bf16")
    return flop.value, khz.value


def rl_calib_copy(src, dst, nbytes: int, n_blocks: int, stream=None) -> None:
    st = lib().rl_calib_copy(_ptr(src), _ptr(dst), int(nbytes), int(n_blocks), _stream(stream))
    if st != RL_OK:
        raise RlError(st, "rl_calib_copy")
