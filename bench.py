#!/usr/bin/env python3
"""Benchmark of the fused LM head + RLLoss forward and backward on one MI355X.

One step = one pass of the hot path over one batch of synthetic input that is
already resident in HBM: the sampler-evidence validation of the batch, then
rl_loss_fwd_bwd (LM-head GEMM with online log-sum-exp, per-token log-probs,
entropy, weights, loss, dense backward dh and dW).  Default workload: 16384
tokens, H=2048, V=152064, bf16, IPO eps 0.3, no support.

Prints ONE JSON line (rank 0).  `roofline` is for the kernel with the largest
summed time, timed with HIP events around each of its launches on the launch
stream inside the timed region (rl_profile_begin / rl_profile_end).
`cpu_baseline` times the fp64 oracle on a bounded token sample of the same
workload on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tokens/s fused LM-head+RLLoss fwd+bwd (H=2048,V=152k) + % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3
DEFAULT_TOKEN_CHUNK = 8192  # the library's default tokens per pass (rl_loss_cfg.token_chunk = 0)
PEAK_HBM_GBS = 8000.0
GEMMS = ("gemm_fwd", "gemm_dh", "gemm_dw")
# Sources a kernel's counter summary was taken on (a summary is ignored once
# any of them changes).
KERNEL_SOURCES = {
    "gemm": ("gemm.hip", "common.h", "kernels.h"),
    "elementwise": ("elementwise.hip", "common.h", "kernels.h"),
    "mis_token": ("mis.hip", "common.h", "kernels.h"),
}


_CODE_TOKENS = re.compile(r'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)


def strip_comments(src: str) -> str:
    """C++ source with its comments removed (string and character literals
    kept) and every run of whitespace made one space."""
    code = _CODE_TOKENS.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), src)
    return " ".join(code.split())


def kernel_src_sha(kernel: str = "gemm_fwd") -> str:
    """Hash of the code (comments and layout stripped) of the sources a kernel
    is built from: a counter summary stays valid across comment-only edits."""
    files = KERNEL_SOURCES["gemm" if kernel.startswith("gemm") else kernel]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "lm_head_logprobs_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_src_sha") != kernel_src_sha(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, target_s: float, seed: int = 0):
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import head as ohead

    cores = len(os.sched_getaffinity(0))
    d = wl.to_host_numpy()
    h64 = d["h"].astype(np.float64)
    W64 = d["W"].astype(np.float64)
    rng = np.random.default_rng(seed)
    args = (d["labels"], d["infer_logprobs"], d["adv"], wl.params)
    age = getattr(wl, "age", None)
    kw = dict(offsets=d["offsets"], ids=d["ids"], u=d["u"], logq=d["logq"], want_grads=True,
              chunk=64, age=None if age is None else age.cpu().numpy())
    with threadpool_limits(limits=cores):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        n0 = 16
        tok = np.sort(rng.choice(wl.N, n0, replace=False))
        t0 = time.perf_counter()
        ohead.head_reference(h64, W64, *args, tokens=tok, **kw)
        dt0 = time.perf_counter() - t0
        n = int(min(max(16, round(n0 * target_s / max(dt0, 1e-3))), wl.N, 4096))
        for _ in range(2):  # the pilot includes one-off costs; rescale once
            tok = np.sort(rng.choice(wl.N, n, replace=False))
            t0 = time.perf_counter()
            ohead.head_reference(h64, W64, *args, tokens=tok, **kw)
            dt = time.perf_counter() - t0
            if dt >= 0.6 * target_s or n >= min(wl.N, 4096):
                break
            n = int(min(round(n * target_s / max(dt, 1e-3)), wl.N, 4096))
    return {
        "value": n / dt,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{n} of {wl.N} tokens of the same workload (full H={wl.H}, V={wl.V}), "
                   f"fp64 forward + dense backward (dh rows, dW from those tokens), "
                   f"{dt:.1f} s on {cores} host cores"),
    }


def cpu_baseline_replay(kind, host, target_s):
    """The replay oracles (numpy fp64, vectorised) over the whole 2,160,000-token
    input, repeated until about target_s seconds have passed."""
    from threadpoolctl import threadpool_limits

    from oracle import mis as om
    from oracle import replay as orp

    # numpy's elementwise kernels run on one thread (no BLAS call here)
    with threadpool_limits(limits=1):
        n_pass, t0 = 0, time.perf_counter()
        while True:
            if kind == "replay":
                orp.replay_reference(host["lp"], host["lq"], host["adv"], host["params"])
            else:
                om.mis_reference(host["lp"], host["lq"], host["adv"], host["offsets"],
                                 host["params"])
            n_pass += 1
            dt = time.perf_counter() - t0
            if dt >= target_s or n_pass >= 200:
                break
    N = len(host["lp"])
    return {"value": n_pass * N / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": (f"the whole input ({N} tokens) {n_pass} times, fp64 numpy on one "
                       f"thread, {dt:.1f} s")}


def bench_head(args, torch):
    from lm_head_logprobs_amd import _lib as L
    from lm_head_logprobs_amd import ops
    from synth import make_head, policy_ages

    dev = torch.device("cuda:0")
    wl = make_head(args.workload, device=dev)
    age = None
    if args.kl_staleness != "none":
        wl.params["kl_staleness"] = args.kl_staleness
        age = policy_ages(wl.N, device=dev)
    if args.entropy_coeff != 0.0:
        wl.params["entropy_coeff"] = args.entropy_coeff
        if wl.params.get("backward") == "sparse":
            wl.params["backward"] = "dense"  # the entropy term is dense
    wl.age = age
    fh = ops.FusedHead(wl.h, wl.W, wl.labels, wl.infer_logprobs, wl.adv, wl.params, wl.offsets,
                       wl.ids, wl.u, wl.logq, token_chunk=args.token_chunk, age=age)
    flags = torch.zeros(1, device=dev, dtype=torch.int32)

    def step():
        L.rl_validate_support(wl.N, wl.V, wl.nnz, wl.labels, wl.infer_logprobs, wl.adv,
                              fh.offsets_host, fh.offsets_dev, wl.ids, wl.u, wl.logq,
                              wl.params["replayed"], flags)
        fh()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    if int(flags.item()) != 0:
        raise RuntimeError(f"validation flags {int(flags.item()):#x} on the synthetic batch")
    L.rl_profile_begin()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    prof = L.rl_profile_end()
    ms = e0.elapsed_time(e1) / args.steps
    N, H, V = wl.N, wl.H, wl.V
    # Device memory of the path: the caller's inputs, outputs and workspace
    # (the library allocates nothing); torch's allocator peak over the timed
    # steps is the same set of buffers plus the flag word.
    def nbytes(*ts):
        return int(sum(t.numel() * t.element_size() for t in ts if t is not None))
    mem_in = nbytes(wl.h, wl.W, wl.labels, wl.infer_logprobs, wl.adv, fh.offsets_dev, wl.ids,
                    wl.u, wl.logq, age)
    mem_out = nbytes(*fh.o.values())
    memory = {"peak_device_bytes": mem_in + mem_out + fh.ws_bytes, "inputs_bytes": mem_in,
              "outputs_bytes": mem_out, "workspace_bytes": int(fh.ws_bytes),
              "torch_allocator_peak_bytes": int(torch.cuda.max_memory_allocated())}
    memory["peak_gib"] = memory["peak_device_bytes"] / 2**30
    value = N / (ms * 1e-3)
    # MFMA work per step: the forward, dh and dW GEMMs (6NHV) on the dense
    # backward; the forward alone (2NHV) on the sparse one, whose gradients
    # are gathers and a scatter
    dense_bwd = wl.params["backward"] != "sparse"
    gemm_flops = (6.0 if dense_bwd else 2.0) * N * H * V
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
    kernels = {k: {"launches": n, "avg_ms": t / n, "ms_per_step": t / args.steps}
               for k, (n, t) in sorted(prof.items(), key=lambda kv: -kv[1][1])}
    dom = max(prof, key=lambda k: prof[k][1])
    n_launch, tot_ms = prof[dom]
    avg_ms = tot_ms / n_launch
    roof = None
    if dom in GEMMS:
        work = 2.0 * N * H * V * args.steps  # each GEMM contracts N x H x V once per step
        achieved = work / (tot_ms * 1e-3) / 1e12
        traffic = read_traffic(dom, args.workload)
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak, "traffic": traffic, "kernel": dom,
                "avg_launch_ms": avg_ms, "algorithmic_tflop_per_launch": 2.0 * N * H * V /
                n_launch * args.steps / 1e12}
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": N, "H": H, "V": V,
                   "loss": wl.params["loss_type"], "support_nnz": wl.nnz,
                   "kl": wl.params["kl_estimator"], "backward": wl.params["backward"],
                   "kl_staleness": wl.params.get("kl_staleness", "none"),
                   "entropy_coeff": wl.params.get("entropy_coeff", 0.0),
                   "token_chunk": fh.cfg.token_chunk or min(N, DEFAULT_TOKEN_CHUNK)},
        ("mfma_frac_6nhv" if dense_bwd else "mfma_frac_2nhv"):
            gemm_flops / (ms * 1e-3) / 1e12 / peak,
        "peak_device_bytes": memory["peak_device_bytes"],
        "memory": memory,
        "roofline": roof,
        "kernels": kernels,
        "wall_s_timed": wall,
    }
    return out, wl


def copy_floor(torch, copies, N, steps):
    """A plain torch elementwise op with nearly the same traffic (addcmul: reads
    three fp32 streams, writes one, 16 B/token) on the same rotated buffers:
    what a kernel with no per-token arithmetic reaches at this size."""
    outs = [torch.empty_like(c.args[0]) for c in copies]
    for i in range(8):
        torch.addcmul(copies[i % 16].args[0], copies[i % 16].args[1], copies[i % 16].args[2],
                      out=outs[i % 16])
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        c = copies[i % 16]
        torch.addcmul(c.args[0], c.args[1], c.args[2], out=outs[i % 16])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"op": "torch.addcmul fp32", "bytes": 16.0 * N, "avg_ms": ms,
            "GB/s": 16.0 * N / (ms * 1e-3) / 1e9}


def wl_replay_host():
    """The replay input on the host, for the oracle CPU baseline."""
    from synth import make_replay

    r = make_replay()
    return {"lp": r.lp.numpy(), "lq": r.lq.numpy(), "adv": r.adv.numpy(), "params": r.params}


def event_overhead(torch, steps):
    """An event pair around nothing, timed like the per-launch events: the
    fixed part of a short kernel's event-measured duration."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    tot = 0.0
    for _ in range(steps):
        e0.record()
        e1.record()
        e1.synchronize()
        tot += e0.elapsed_time(e1)
    return tot / steps


def graph_per_call_ms(torch, calls, steps):
    """Launch-overhead-free time per call: the calls (one step each, on their
    own input copies) are captured once into a HIP graph, which is replayed
    until about `steps` calls ran.  Before timing, every replay's outputs are
    checked bit for bit against an eager run of the same calls, with eager
    work and synchronisations between the replays.  Returns (ms per call, or
    None if a replay disagreed)."""
    outs = [list(c.o.values()) for c in calls]

    def snapshot():
        return [[t.clone() for t in o] for o in outs]

    for c in calls:
        c()
    torch.cuda.synchronize()
    eager = snapshot()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    ok = True
    for _ in range(3):
        for o in outs:
            for t in o:
                t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        ok = ok and all(torch.equal(a, b) for ea, ga in zip(eager, got) for a, b in zip(ea, ga))
        calls[0]()  # eager work between the replays
        torch.cuda.synchronize()
    if not ok:
        return None
    reps = max(1, -(-steps // len(calls)))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / (reps * len(calls))


def replay_16x(torch, L, ops, r, steps):
    """The same pass over 16 N tokens (the replay input repeated 16 times), two
    rotated copies of 1.24 GB: launch and tail costs amortise at this size."""
    big = [ops.Replay(r.lp.repeat(16), r.lq.repeat(16), r.adv.repeat(16), r.params)
           for _ in range(2)]
    for i in range(4):
        big[i % 2]()
    torch.cuda.synchronize()
    L.rl_profile_begin()
    n = max(steps // 2, 4)
    for i in range(n):
        big[i % 2]()
    torch.cuda.synchronize()
    prof = L.rl_profile_end()
    cnt, tot = prof["elementwise"]
    avg = tot / cnt
    byt = 18.0 * big[0].N
    gbs = byt / (avg * 1e-3) / 1e9
    out = {"tokens": big[0].N, "launches": cnt, "avg_ms": avg,
           "algorithmic_bytes_per_launch": byt, "GB/s": gbs, "frac": gbs / PEAK_HBM_GBS}
    del big
    torch.cuda.empty_cache()
    return out


def bench_replay(args, torch):
    from lm_head_logprobs_amd import _lib as L
    from lm_head_logprobs_amd import ops
    from synth import make_replay

    r = make_replay(device="cuda:0")
    # Rotate over independent copies (> 620 MB) so every pass reads HBM, not the
    # 256 MB Infinity Cache.
    copies = [ops.Replay(r.lp.clone(), r.lq.clone(), r.adv.clone(), r.params) for _ in range(16)]
    for i in range(args.warmup):
        copies[i % 16]()
    torch.cuda.synchronize()
    # step time: the 16 rotated passes captured in a graph (a pass is two
    # kernels of a few microseconds; eager launches from Python cost more)
    ms_graph = graph_per_call_ms(torch, copies, args.steps)
    # per-kernel times: eager launches with the library's event timing
    L.rl_profile_begin()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        copies[i % 16]()
    e1.record()
    torch.cuda.synchronize()
    prof = L.rl_profile_end()
    ms_eager = e0.elapsed_time(e1) / args.steps
    ms = ms_graph if ms_graph is not None else ms_eager
    n, tot = prof["elementwise"]
    avg = tot / n
    nf, totf = prof.get("elementwise_final", (1, 0.0))
    byt = 18.0 * r.N  # reads lp, lq, A (12 B), writes the mask word and w_primary (6 B)
    achieved = byt / (avg * 1e-3) / 1e9
    return {
        "metric": "tokens/s loss-only mismatch replay (fp32 elementwise)",
        "value": r.N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": "c2_replay", "tokens": r.N},
        "step_timing": ("hip graph of the 16 rotated passes, replays checked bit for bit against "
                        "eager runs" if ms_graph is not None else "eager launches"),
        "eager_ms_per_step_with_kernel_events": ms_eager,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": read_traffic("elementwise", "c2_replay"),
                     "kernel": "elem_main (the per-token pass)", "avg_launch_ms": avg,
                     "algorithmic_bytes_per_launch": byt},
        "kernels": {"elementwise": {"launches": n, "avg_ms": avg},
                    "elementwise_final": {"launches": nf, "avg_ms": totf / max(nf, 1)}},
        "torch_elementwise_floor": copy_floor(torch, copies, r.N, args.steps),
        "replay_16x": replay_16x(torch, L, ops, r, args.steps),
        "event_pair_overhead_ms": event_overhead(torch, args.steps),
        "cpu_baseline": None,
    }, None


def bench_mis(args, torch):
    """Sequence-aware rollout correction over the replay: one call of
    rl_mis_replay (five launches) per step."""
    from lm_head_logprobs_amd import _lib as L
    from lm_head_logprobs_amd import ops
    from synth import MIS_PARAMS, make_replay, replay_sequences

    r = make_replay(device="cuda:0")
    off = replay_sequences(r.N)
    params = dict(MIS_PARAMS)
    # 16 independent copies (> 620 MB) so that every pass reads HBM
    copies = [ops.MisReplay(r.lp.clone(), r.lq.clone(), r.adv.clone(), off, params)
              for _ in range(16)]
    for i in range(args.warmup):
        copies[i % 16]()
    torch.cuda.synchronize()
    ms_graph = graph_per_call_ms(torch, copies, args.steps)
    L.rl_profile_begin()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        copies[i % 16]()
    e1.record()
    torch.cuda.synchronize()
    prof = L.rl_profile_end()
    ms_eager = e0.elapsed_time(e1) / args.steps
    ms = ms_graph if ms_graph is not None else ms_eager
    kern = {k: {"launches": n, "avg_ms": t / n} for k, (n, t) in prof.items()}
    tok = kern["mis_token"]["avg_ms"]
    byt = 17.0 * r.N  # reads lp, lq, A; writes the fp32 weight and the uint8 flags
    achieved = byt / (tok * 1e-3) / 1e9
    pass_ms = sum(v["avg_ms"] for v in kern.values())
    pass_bytes = 25.0 * r.N  # + the first pass over lp, lq (8 B/token)
    out = {
        "metric": "tokens/s sequence-aware rollout correction (IS/RS/veto + metrics, fp32)",
        "value": r.N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": "c2_mis", "tokens": r.N, "sequences": int(off.numel() - 1),
                   "tis": f'{params["tis_level"]}/{params["tis_mode"]}',
                   "rs": params["rs_level"] if params["use_rs"] else "off",
                   "veto": params["veto"], "batch_normalize": params["batch_normalize"]},
        "step_timing": ("hip graph of the 16 rotated passes, replays checked bit for bit against "
                        "eager runs" if ms_graph is not None else "eager launches"),
        "eager_ms_per_step_with_kernel_events": ms_eager,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": read_traffic("mis_token", "c2_mis"),
                     "kernel": "mis_token (the per-token pass)", "avg_launch_ms": tok,
                     "algorithmic_bytes_per_launch": byt},
        "whole_pass": {"kernels_ms": pass_ms, "algorithmic_bytes": pass_bytes,
                       "GB/s": pass_bytes / (pass_ms * 1e-3) / 1e9},
        "kernels": kern,
        "event_pair_overhead_ms": event_overhead(torch, args.steps),
        "cpu_baseline": None,
    }
    host = {"lp": r.lp.cpu().numpy(), "lq": r.lq.cpu().numpy(), "adv": r.adv.cpu().numpy(),
            "offsets": off.numpy(), "params": params}
    return out, host


def measured_peaks(torch):
    """What the bf16 matrix pipe and HBM deliver on this device with kernels that
    do nothing else (the library's calibration calls): a register-only MFMA loop
    at two waves per SIMD, with all-zero and with random operands (operand
    toggling costs power, so the sustained clock differs), and a grid-stride
    copy of 1 GiB, out of place and in place.  Reported beside the published
    peaks, which the roofline fractions use."""
    from lm_head_logprobs_amd import _lib as L

    dev = torch.device("cuda:0")
    nb = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(nb * 256, device=dev, dtype=torch.float32)
    stamps = torch.zeros(nb * 4, device=dev, dtype=torch.int64)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    res = {"mfma_blocks": nb, "published_bf16_tflops": PEAK_BF16_TFLOPS,
           "published_hbm_gbs": PEAK_HBM_GBS}
    for name, rnd in (("mfma_bf16_zero_operands", False), ("mfma_bf16_random_operands", True)):
        L.rl_calib_mfma_bf16(rnd, nb, 2000, sink, stamps)
        e0.record()
        flop, khz = L.rl_calib_mfma_bf16(rnd, nb, 100000, sink, stamps)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        st = stamps.view(nb, 4).cpu().double()
        ghz = float(((st[:, 1] - st[:, 0]) / (st[:, 3] - st[:, 2])).median()) * khz * 1e3 / 1e9
        tf = flop / (ms * 1e-3) / 1e12
        res[name] = {"tflops": tf, "frac_of_published": tf / PEAK_BF16_TFLOPS,
                     "clock_ghz": ghz, "ms": ms}
    nbytes = 1 << 30
    src = torch.empty(nbytes // 4, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    src.fill_(1.0)
    for name, d in (("copy", dst), ("copy_in_place", src)):
        best = None
        for blocks in (1024, 2048, 4096, 8192):
            L.rl_calib_copy(src, d, nbytes, blocks)
            e0.record()
            for _ in range(5):
                L.rl_calib_copy(src, d, nbytes, blocks)
            e1.record()
            torch.cuda.synchronize()
            gbs = 2 * nbytes * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if best is None or gbs > best["gbs"]:
                best = {"gbs": gbs, "frac_of_published": gbs / PEAK_HBM_GBS, "blocks": blocks}
        res[name] = best
    del src, dst
    return res


def secondary(args, torch):
    """Compact figures of the other workloads in the same run: the 16k top-p
    replay with exact KL, the two 64k-token draw workloads (IPO with k1 KL on
    the dense backward, reinforce on the sparse one), the 2.16M-token
    loss-only replay and the sequence-aware correction over it, each with its
    step time, roofline fraction and memory; the 16k top-p replay and the
    loss-only replay also with their oracle CPU baselines (the 64k workloads'
    per-token oracle work is that of the 16k ones)."""
    from types import SimpleNamespace

    res = {}
    for name, steps, warmup, cpu_s in (("c4_head16k_ipo_topp_replay", 10, 3, 10.0),
                                       ("c5a_head64k_draws_ipo_k1", 5, 2, None),
                                       ("c5b_head64k_draws_reinforce", 5, 2, None)):
        a = SimpleNamespace(**vars(args))
        a.workload, a.steps, a.warmup = name, steps, warmup
        a.kl_staleness, a.entropy_coeff, a.token_chunk = "none", 0.0, 0
        out, wl = bench_head(a, torch)
        res[name] = {
            "ms_per_step": out["ms_per_step"], "tokens_per_s": out["value"],
            "steps": steps,
            **{k: out[k] for k in ("mfma_frac_6nhv", "mfma_frac_2nhv") if k in out},
            "support_nnz": out["config"]["support_nnz"],
            "backward": out["config"]["backward"], "token_chunk": out["config"]["token_chunk"],
            "peak_device_bytes": out["peak_device_bytes"],
            "roofline": {k: out["roofline"][k] for k in ("kernel", "frac", "avg_launch_ms")},
            "kernels_ms_per_step": {k: v["ms_per_step"] for k, v in out["kernels"].items()
                                    if v["ms_per_step"] >= 0.05},
            "cpu_baseline": (None if args.no_cpu_baseline or cpu_s is None
                             else cpu_baseline(wl, cpu_s)),
        }
        del out, wl
        torch.cuda.empty_cache()
    a2 = SimpleNamespace(**vars(args))
    a2.workload, a2.steps, a2.warmup = "c2_replay", 200, 20
    out, _ = bench_replay(a2, torch)
    res["c2_replay"] = {
        "us_per_step": out["ms_per_step"] * 1e3, "tokens_per_s": out["value"],
        "step_timing": out["step_timing"],
        "roofline": {"kernel": out["roofline"]["kernel"], "frac": out["roofline"]["frac"],
                     "avg_launch_us": out["roofline"]["avg_launch_ms"] * 1e3,
                     "GB/s": out["roofline"]["achieved"]},
        "kernels_avg_us": {k: v["avg_ms"] * 1e3 for k, v in out["kernels"].items()},
        "replay_16x_frac": out["replay_16x"]["frac"],
        "cpu_baseline": (None if args.no_cpu_baseline
                         else cpu_baseline_replay("replay", wl_replay_host(), 5.0)),
    }
    torch.cuda.empty_cache()
    am = SimpleNamespace(**vars(args))
    am.workload, am.steps, am.warmup = "c2_mis", 200, 20
    out, _ = bench_mis(am, torch)
    res["c2_mis"] = {
        "us_per_step": out["ms_per_step"] * 1e3, "tokens_per_s": out["value"],
        "sequences": out["config"]["sequences"], "step_timing": out["step_timing"],
        "roofline": {"kernel": out["roofline"]["kernel"], "frac": out["roofline"]["frac"],
                     "avg_launch_us": out["roofline"]["avg_launch_ms"] * 1e3,
                     "GB/s": out["roofline"]["achieved"]},
        "kernels_avg_us": {k: v["avg_ms"] * 1e3 for k, v in out["kernels"].items()},
    }
    del out
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3_head16k_ipo",
                    help="c3_head16k_ipo (default), c4_head16k_ipo_topp_replay, "
                         "c5a_head64k_draws_ipo_k1, c5b_head64k_draws_reinforce, c2_replay, "
                         "c2_mis")
    ap.add_argument("--token-chunk", type=int, default=0)
    ap.add_argument("--kl-staleness", default="none", choices=("none", "inv_sqrt"),
                    help="head workloads: scale the KL by 1/sqrt(1 + policy age), with "
                         "synthetic per-token ages")
    ap.add_argument("--entropy-coeff", type=float, default=0.0,
                    help="head workloads: entropy bonus coefficient")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target length of the oracle CPU baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peak-check", action="store_true",
                    help="skip the measured MFMA and copy peaks")
    ap.add_argument("--no-secondary", action="store_true",
                    help="default workload only: skip the figures of the other workloads "
                         "(16k top-p replay, 64k draws, loss-only replay, sequence-aware "
                         "correction)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only; --gpus N > 1 is not supported (the path "
              "would shard by tokens, with dW as the one exchange)", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    host = None
    if args.workload == "c2_replay":
        out, wl = bench_replay(args, torch)
        r = wl_replay_host()
        host = ("replay", r)
    elif args.workload == "c2_mis":
        out, h = bench_mis(args, torch)
        wl, host = None, ("mis", h)
    else:
        out, wl = bench_head(args, torch)
    if not args.no_peak_check:
        out["measured_peaks"] = measured_peaks(torch)
    if args.copy_calibration:
        a = torch.empty(1 << 28, device="cuda:0", dtype=torch.float32)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
    if wl is not None:
        out["cpu_baseline"] = (None if args.no_cpu_baseline
                               else cpu_baseline(wl, args.cpu_seconds))
    elif host is not None and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_replay(host[0], host[1], args.cpu_seconds)
    if args.workload == "c3_head16k_ipo" and not args.no_secondary:
        del wl
        torch.cuda.empty_cache()
        out["secondary"] = secondary(args, torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
