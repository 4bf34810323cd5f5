"""The C ABI on the host: the library loads, exports every declared symbol, and
rejects bad arguments, configurations, CSR offsets and workspaces before it
touches the device.  No compute call is made (no GPU here)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from lm_head_logprobs_amd import _lib as L
from lm_head_logprobs_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rlloss.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH),
                                reason="librlloss.so not built (run __graft_entry__.build())")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:rl_status|const char\*)\s+(rl_\w+)\(", src, re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) == 15
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for n in names:
        assert n in exported, n
        assert hasattr(L.lib(), n)
    assert set(L.EXPORTED) == set(names)


def test_status_strings_and_version():
    for s in range(7):
        assert len(L.status_string(s)) >= 2
    assert "unknown" in L.status_string(99)
    assert "gfx950" in L.rl_version()


def test_profile_calls_without_launches():
    L.rl_profile_begin()
    assert L.rl_profile_end() == {}
    n = ctypes.c_int32(0)
    assert L.lib().rl_profile_end(None, 4, ctypes.byref(n)) == L.RL_E_ARG


def test_struct_layout_matches_header():
    # The header's structs are plain C: sizes follow from field order.
    assert ctypes.sizeof(L.RlLossCfg) == 5 * 8 + 8 * 4 + 8 * 4 + 2 * 4
    assert ctypes.sizeof(L.RlLossOut) == 10 * 8
    assert ctypes.sizeof(L.RlElemCfg) == 2 * 4 + 8 * 4 + 7 * 4
    assert ctypes.sizeof(L.RlElemOut) == 3 * 8
    assert ctypes.sizeof(L.RlMisCfg) == 10 * 4
    assert ctypes.sizeof(L.RlMisOut) == 3 * 8


def test_mis_metric_order_matches_header():
    src = open(HEADER).read()
    block = src[src.index("RL_MIS_TRAINING_LOG_PPL = 0"):src.index("RL_MIS_METRIC_COUNT = ")]
    names = re.findall(r"RL_MIS_([A-Z0-9_]+)", block)
    assert [n.lower() for n in names] == list(L.MIS_METRIC_NAMES)
    assert f"RL_MIS_METRIC_COUNT = {len(names)}" in src


class HostBufs:
    """Aligned host buffers standing in for device pointers; never dereferenced
    by the tested calls because every one of them fails its host-side checks."""

    def __init__(self):
        self.keep = []

    def buf(self, nbytes, align=256):
        a = np.zeros(nbytes + align, np.uint8)
        self.keep.append(a)
        p = a.ctypes.data
        return p + (-p) % align


def _params(**kw):
    p = dict(loss_type="ipo", ipo_eps=0.3, max_ratio=5.0, icepop_lo=0.5, icepop_hi=2.0,
             kl_coeff=0.0, kl_estimator="none", replayed=False, backward="dense", loss_norm=8.0)
    p.update(kw)
    return p


def _ws(cfg, sup=False):
    return L.rl_loss_workspace_size(cfg, sup, True, True)


@pytest.mark.parametrize("mut,code", [
    (dict(N=0), L.RL_E_ARG), (dict(H=4), L.RL_E_ARG), (dict(H=20), L.RL_E_ARG),
    (dict(V=0), L.RL_E_ARG), (dict(V=2**31), L.RL_E_ARG), (dict(token_chunk=-1), L.RL_E_ARG),
    (dict(dtype=7), L.RL_E_ARG), (dict(grad_dtype=-1), L.RL_E_ARG), (dict(reserved1=1), L.RL_E_ARG),
    (dict(loss_type=3), L.RL_E_CFG), (dict(ipo_eps=-0.1), L.RL_E_CFG),
    (dict(max_ratio=0.0), L.RL_E_CFG), (dict(icepop_lo=3.0), L.RL_E_CFG),
    (dict(loss_norm=0.0), L.RL_E_CFG), (dict(loss_norm=float("nan")), L.RL_E_CFG),
    (dict(inv_temperature=0.0), L.RL_E_CFG), (dict(adv_tau=float("inf")), L.RL_E_CFG),
    (dict(kl_estimator=1, kl_coeff=0.1), L.RL_E_CFG),  # KL needs a support
    (dict(kl_coeff=-1.0), L.RL_E_CFG), (dict(backward=9), L.RL_E_CFG),
    (dict(backward=L.RL_BWD_SPARSE), L.RL_E_CFG),  # sparse needs reinforce + support
    (dict(replayed=1), L.RL_E_CFG),  # replay needs a support
    (dict(kl_staleness=2), L.RL_E_CFG), (dict(entropy_coeff=float("nan")), L.RL_E_CFG),
])
def test_workspace_size_rejects(mut, code):
    cfg = ops.make_cfg(8, 16, 50, 0, __import__("torch").bfloat16, _params())
    for k, v in mut.items():
        setattr(cfg, k, v)
    n = ctypes.c_size_t(0)
    assert L.lib().rl_loss_workspace_size(ctypes.byref(cfg), 0, 1, 1, ctypes.byref(n)) == code


def test_support_configuration_rules():
    import torch
    base = dict(N=8, H=16, V=50, nnz=20)
    # exact KL needs a replayed support; k1 on draws is fine
    cfg = ops.make_cfg(**base, dtype=torch.bfloat16,
                       params=_params(kl_estimator="exact", kl_coeff=0.1))
    n = ctypes.c_size_t(0)
    assert L.lib().rl_loss_workspace_size(ctypes.byref(cfg), 1, 1, 1, ctypes.byref(n)) == L.RL_E_CFG
    cfg.replayed = 1
    assert L.lib().rl_loss_workspace_size(ctypes.byref(cfg), 1, 1, 1, ctypes.byref(n)) == L.RL_OK
    # sparse backward: allowed for reinforce without KL on a support only
    cfg = ops.make_cfg(**base, dtype=torch.bfloat16,
                       params=_params(loss_type="reinforce", backward="sparse"))
    assert L.lib().rl_loss_workspace_size(ctypes.byref(cfg), 1, 1, 1, ctypes.byref(n)) == L.RL_OK
    sparse_bytes = n.value
    cfg.kl_estimator, cfg.kl_coeff = L.RL_KL_K1, 0.05
    assert L.lib().rl_loss_workspace_size(ctypes.byref(cfg), 1, 1, 1, ctypes.byref(n)) == L.RL_E_CFG
    cfg = ops.make_cfg(**base, dtype=torch.bfloat16,
                       params=_params(loss_type="reinforce", backward="dense"))
    assert L.lib().rl_loss_workspace_size(ctypes.byref(cfg), 1, 1, 1, ctypes.byref(n)) == L.RL_OK
    assert n.value > sparse_bytes  # the dense backward needs the [V, Tc] operand
    # the entropy bonus makes the gradient dense: a forced sparse backward is refused and
    # AUTO plans the dense one
    cfg = ops.make_cfg(**base, dtype=torch.bfloat16,
                       params=_params(loss_type="reinforce", backward="sparse", entropy_coeff=0.1))
    assert L.lib().rl_loss_workspace_size(ctypes.byref(cfg), 1, 1, 1, ctypes.byref(n)) == L.RL_E_CFG
    cfg.backward = L.RL_BWD_AUTO
    assert L.lib().rl_loss_workspace_size(ctypes.byref(cfg), 1, 1, 1, ctypes.byref(n)) == L.RL_OK
    assert n.value > sparse_bytes


def test_workspace_size_scales_and_does_not_overflow():
    import torch
    cfg = ops.make_cfg(16384, 2048, 152064, 0, torch.bfloat16, _params(loss_norm=16384.0))
    dense = _ws(cfg)
    # the one [Tc, V] bf16 operand G of a chunk dominates (dh reads it as is, dW
    # transposed): no second [V, Tc] copy, and by default a chunk of 8192 tokens,
    # not the batch
    Tc = 8192
    assert 2 * 152064 * Tc < dense < 2 * 2 * 152064 * Tc
    cfg.token_chunk = 16384  # the whole batch in one chunk
    assert 2 * 152064 * 16384 < _ws(cfg) < 2 * 2 * 152064 * 16384
    cfg.token_chunk = 0
    cfg.backward = L.RL_BWD_NONE
    fwd = _ws(cfg)
    # the forward alone holds the tiled copies of W and of a chunk of h (at
    # most the batch) and per-token partials; nothing of size [Tc, V]
    tiled = 2 * (152064 + 256) * 2048 + 2 * 16384 * 2048
    assert tiled < fwd < tiled + dense // 40
    cfg.backward = L.RL_BWD_DENSE
    cfg.token_chunk = 4096
    assert _ws(cfg) < dense
    # sizes whose byte counts overflow 64-bit arithmetic are rejected
    big = ops.make_cfg(2**31 - 1, 2**40, 2**31 - 3, 0, torch.float32, _params(loss_norm=1.0))
    n = ctypes.c_size_t(0)
    assert L.lib().rl_loss_workspace_size(ctypes.byref(big), 0, 1, 1, ctypes.byref(n)) == L.RL_E_ARG


def _call(hb, cfg, offsets=None, ids=True, ws_bytes=None, h=None, W=None, out=None, loss=True,
          ws=None):
    N, H, V = cfg.N, cfg.H, cfg.V
    h = hb.buf(N * H * 2) if h is None else h
    W = hb.buf(V * H * 2) if W is None else W
    lab, lq, adv = hb.buf(4 * N), hb.buf(4 * N), hb.buf(4 * N)
    if out is None:
        out = L.RlLossOut()
        out.loss = hb.buf(4) if loss else None
        out.dh = hb.buf(N * H * 2)
        out.dW = hb.buf(V * H * 4)
    off_dev = idp = up = None
    offp = None
    if offsets is not None:
        offp = offsets.ctypes.data
        off_dev = hb.buf(8 * (N + 1))
        if ids:
            idp, up = hb.buf(4 * max(cfg.nnz, 1)), hb.buf(4 * max(cfg.nnz, 1))
    if ws_bytes is None:
        ws_bytes = L.rl_loss_workspace_size(cfg, offsets is not None, True, True)
    wsp = hb.buf(ws_bytes) if ws is None else ws
    return L.lib().rl_loss_fwd_bwd(h, W, lab, lq, adv, None, offp, off_dev, idp, up, None,
                                   ctypes.byref(cfg), ctypes.byref(out), wsp, ws_bytes, None)


def test_fwd_bwd_host_errors_return_before_launch():
    import torch
    hb = HostBufs()
    cfg = ops.make_cfg(8, 16, 50, 0, torch.bfloat16, _params())
    assert _call(hb, cfg, loss=False) == L.RL_E_ARG  # out->loss is required
    assert _call(hb, cfg, h=hb.buf(256, 256) + 2) == L.RL_E_ARG  # misaligned h
    need = L.rl_loss_workspace_size(cfg, False, True, True)
    assert _call(hb, cfg, ws_bytes=need - 1) == L.RL_E_WORKSPACE
    assert _call(hb, cfg, ws=hb.buf(need) + 8, ws_bytes=need) == L.RL_E_WORKSPACE  # misaligned
    assert L.lib().rl_loss_fwd_bwd(None, None, None, None, None, None, None, None, None, None, None,
                                   ctypes.byref(cfg), None, None, 0, None) == L.RL_E_ARG
    # CSR checks on the host offsets
    cfg = ops.make_cfg(4, 16, 50, 6, torch.bfloat16, _params())
    good = np.array([0, 2, 2, 5, 6], np.int64)
    for bad in ([1, 2, 2, 5, 6], [0, 3, 2, 5, 6], [0, 2, 2, 5, 7]):
        assert _call(hb, cfg, offsets=np.array(bad, np.int64)) == L.RL_E_CSR
    assert _call(hb, cfg, offsets=good, ids=False) == L.RL_E_ARG  # ids / u missing


def test_elementwise_and_validate_host_errors():
    hb = HostBufs()
    n = ctypes.c_size_t(0)
    assert L.lib().rl_elementwise_workspace_size(0, ctypes.byref(n)) == L.RL_E_ARG
    assert L.lib().rl_elementwise_workspace_size(2_160_000, ctypes.byref(n)) == L.RL_OK
    assert n.value == 1024 * 37 * 8  # min(ceil(ceil(N / 256) / 4), 1024) blocks of 37 fp64 sums
    assert L.lib().rl_elementwise_workspace_size(1000, ctypes.byref(n)) == L.RL_OK
    assert n.value == 1 * 37 * 8
    assert L.lib().rl_elementwise_workspace_size((1 << 38) + 1, ctypes.byref(n)) == L.RL_E_ARG
    from synth.gen import REPLAY_PARAMS
    good = ops.elem_cfg(REPLAY_PARAMS)
    N = 1000
    lp, lq, adv = hb.buf(4 * N), hb.buf(4 * N), hb.buf(4 * N)
    out = L.RlElemOut()
    out.sums = hb.buf(8 * 37)
    ws = hb.buf(n.value)

    def call(cfg, ws_bytes=1 << 16, o=out, lpp=lp):
        return L.lib().rl_loss_elementwise(lpp, lq, adv, N, ctypes.byref(cfg), ctypes.byref(o), ws,
                                           ws_bytes, None)

    for field, val in (("n_eps", 0), ("n_eps", 9), ("primary_eps_index", 5), ("max_ratio", 0.0),
                       ("clip_c", 1.0), ("clip_low", 1.0), ("tis_upper", 0.0),
                       ("icepop_lo", 3.0)):
        c = ops.elem_cfg(REPLAY_PARAMS)
        setattr(c, field, val)
        assert call(c) == L.RL_E_CFG, field
    c = ops.elem_cfg(REPLAY_PARAMS)
    c.eps[2] = -0.1
    assert call(c) == L.RL_E_CFG
    assert call(good, ws_bytes=8) == L.RL_E_WORKSPACE
    assert call(good, lpp=lp + 4) == L.RL_E_ARG  # misaligned input
    o2 = L.RlElemOut()
    assert call(good, o=o2) == L.RL_E_ARG  # sums required
    # the allocation-free variant checks the same arguments before it touches a device
    na = L.lib().rl_loss_elementwise_noalloc
    assert na(lp, lq, adv, N, ctypes.byref(good), ctypes.byref(o2), None) == L.RL_E_ARG
    assert na(lp + 4, lq, adv, N, ctypes.byref(good), ctypes.byref(out), None) == L.RL_E_ARG
    assert na(lp, lq, adv, 0, ctypes.byref(good), ctypes.byref(out), None) == L.RL_E_ARG
    assert na(lp, lq, adv, (1 << 38) + 1, ctypes.byref(good), ctypes.byref(out),
              None) == L.RL_E_ARG
    c = ops.elem_cfg(REPLAY_PARAMS)
    c.clip_c = 0.5
    assert na(lp, lq, adv, N, ctypes.byref(c), ctypes.byref(out), None) == L.RL_E_CFG
    # validation: host offsets are checked before any launch
    lab, ilq, A, flags = hb.buf(4 * 4), hb.buf(16), hb.buf(16), hb.buf(4)
    bad = np.array([0, 3, 2, 5, 6], np.int64)
    st = L.lib().rl_validate_support(4, 50, 6, lab, ilq, A, bad.ctypes.data, hb.buf(40),
                                     hb.buf(24), hb.buf(24), None, 1, flags, None)
    assert st == L.RL_E_CSR
    st = L.lib().rl_validate_support(4, 50, 6, lab, ilq, A, None, None, None, None, None, 0, flags,
                                     None)
    assert st == L.RL_E_ARG  # nnz without a support
    st = L.lib().rl_validate_support(0, 50, 0, lab, ilq, A, None, None, None, None, None, 0, flags,
                                     None)
    assert st == L.RL_E_ARG


def test_mis_host_errors_return_before_launch():
    hb = HostBufs()
    n = ctypes.c_size_t(0)
    ws_size = L.lib().rl_mis_workspace_size
    assert ws_size(0, 1, ctypes.byref(n)) == L.RL_E_ARG
    assert ws_size(10, 0, ctypes.byref(n)) == L.RL_E_ARG
    assert ws_size(10, 11, ctypes.byref(n)) == L.RL_E_ARG
    assert ws_size(L.RL_MIS_MAX_N + 1, 1, ctypes.byref(n)) == L.RL_E_ARG
    assert ws_size(2_160_000, 1282, ctypes.byref(n)) == L.RL_OK
    # chunk records, first sequences, bitmap, per-sequence data and partials: a few 0.1 B/token
    assert 2_160_000 * 0.2 < n.value < 2_160_000 * 0.5
    from synth.gen import MIS_PARAMS
    N, S = 1000, 3
    off = np.array([0, 10, 600, 1000], np.int64)
    lp, lq, adv = hb.buf(4 * N), hb.buf(4 * N), hb.buf(4 * N)
    offd = hb.buf(8 * (S + 1))
    assert ws_size(N, S, ctypes.byref(n)) == L.RL_OK
    ws = hb.buf(n.value)
    out = L.RlMisOut()
    out.metrics = hb.buf(8 * L.RL_MIS_METRIC_COUNT)

    def call(cfg=None, offh=off, ws_bytes=None, o=out, s_=S, flags=None):
        cfg = cfg if cfg is not None else ops.mis_cfg(MIS_PARAMS)
        if flags is not None:
            o = L.RlMisOut()
            o.metrics, o.flags = out.metrics, flags
        return L.lib().rl_mis_replay(lp, lq, adv, N, offh.ctypes.data, offd, s_, ctypes.byref(cfg),
                                     ctypes.byref(o), ws, n.value if ws_bytes is None else ws_bytes,
                                     None)

    for field, val in (("tis_level", 3), ("rs_level", -1), ("tis_mode", 3), ("use_rs", 2),
                       ("batch_normalize", 5), ("tis_lower", 0.0), ("tis_upper", 0.1),
                       ("tis_upper", float("inf")), ("veto", -1.0), ("veto", float("inf")),
                       ("rs_lower", 0.0), ("rs_upper", 0.01)):
        c = ops.mis_cfg(MIS_PARAMS)
        setattr(c, field, val)
        assert call(c) == L.RL_E_CFG, (field, val)
    for bad in ([1, 10, 600, 1000], [0, 10, 10, 1000], [0, 600, 10, 1000], [0, 10, 600, 999]):
        assert call(offh=np.array(bad, np.int64)) == L.RL_E_CSR, bad
    assert call(ws_bytes=n.value - 1) == L.RL_E_WORKSPACE
    assert call(flags=hb.buf(N) + 2) == L.RL_E_ARG  # flags must be 4-byte aligned
    assert call(o=L.RlMisOut()) == L.RL_E_ARG       # metrics required
    assert call(s_=0) == L.RL_E_ARG


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        L.lib()


def test_calibration_calls_reject_bad_arguments_before_any_launch():
    """The measurement helpers check their arguments on the host first."""
    import ctypes

    lib = L.lib()
    flop, khz = ctypes.c_double(0.0), ctypes.c_int32(0)
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails its checks
    assert lib.rl_calib_mfma_bf16(1, 512, 10, None, fake, ctypes.byref(flop), ctypes.byref(khz),
                                  None) == L.RL_E_ARG
    assert lib.rl_calib_mfma_bf16(1, 0, 10, fake, fake, ctypes.byref(flop), ctypes.byref(khz),
                                  None) == L.RL_E_ARG
    assert lib.rl_calib_mfma_bf16(1, 512, 0, fake, fake, ctypes.byref(flop), ctypes.byref(khz),
                                  None) == L.RL_E_ARG
    assert lib.rl_calib_mfma_bf16(1, 1 << 11, 1 << 24, fake, fake, ctypes.byref(flop),
                                  ctypes.byref(khz), None) == L.RL_E_ARG  # n_blocks * iters > 2^34
    assert lib.rl_calib_copy(fake, fake, 24, 64, None) == L.RL_E_ARG       # not a multiple of 16
    assert lib.rl_calib_copy(fake, ctypes.c_void_p((1 << 20) + 16), 64, 64, None) == L.RL_E_ARG
    assert lib.rl_calib_copy(fake, ctypes.c_void_p((1 << 20) + 8), 64, 64, None) == L.RL_E_ARG
    assert lib.rl_calib_copy(None, fake, 64, 64, None) == L.RL_E_ARG
    assert lib.rl_calib_copy(fake, ctypes.c_void_p(1 << 21), 64, 0, None) == L.RL_E_ARG

