"""Every token of the 16k workloads against the oracle, at full size.

Two 16384-token batches (H=2048, V=152064, bf16) in the launch configuration
bench.py times: the IPO workload without a support that bench.py reports as
its headline, and the replay workload with its ragged replayed top-p support
(u = q) and the exact KL.  Checked: every token's log-prob, entropy, mask,
weight and token loss, every support entry's log-prob, the loss against the
oracle's loss, the metrics, and dh and dW in full against the fp64 oracle
(prime-rl PR 4233, "Validation": gradients against a dense reference on a
replayed support; the KL, exact on that support, against the dense oracle).
The oracle takes one to two minutes of host time per workload; it writes its
progress to a file next to the parity report.
"""
import os
import time

import pytest
import torch

from gpu_util import REPORT, compare_all, run_head
from lm_head_logprobs_amd import ops
from oracle import head as ohead
from synth import make_head

pytestmark = [pytest.mark.gpu, pytest.mark.slow,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("name", ["c3_head16k_ipo", "c4_head16k_ipo_topp_replay"])
def test_full_size_every_token_against_oracle(name):
    wl = make_head(name, device="cuda:0")
    print(f"[case] {name} full size, every token, N={wl.N} nnz={wl.nnz}", flush=True)
    st, flags = ops.validate(wl.labels, wl.infer_logprobs, wl.adv, wl.V, wl.offsets, wl.ids,
                             wl.u, wl.logq, wl.params["replayed"])
    assert flags == 0, hex(flags)
    _, got = run_head(wl)
    os.makedirs(os.path.dirname(REPORT), exist_ok=True)
    log = open(os.path.join(os.path.dirname(REPORT), f"full_{name}_oracle_progress.log"), "a")
    t0 = time.perf_counter()

    def progress(done, total):
        log.write(f"{time.perf_counter() - t0:7.1f} s  {done}/{total} tokens\n")
        log.flush()

    ref = ohead.from_workload(wl, want_grads=True, chunk=512, progress=progress)
    log.close()
    r = compare_all(wl, got, ref, case=f"{name} full size, every token")
    print(r)
