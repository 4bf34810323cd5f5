"""The allocation-free replay entry point against the workspace entry point.

rl_loss_elementwise_noalloc runs the same kernel as rl_loss_elementwise on the
library's own scratch; its outputs must equal the workspace entry point's bit
for bit.  Two calls in a row, the second on a smaller input, check that the
scratch left by one call does not leak into the next.
"""

import numpy as np
import pytest
import torch

from lm_head_logprobs_amd import _lib as L
from lm_head_logprobs_amd import ops
from synth import make_replay

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _outs(N, dev):
    o = dict(mask_word=torch.full((N,), -1, device=dev, dtype=torch.int16),
             w_primary=torch.full((N,), float("nan"), device=dev, dtype=torch.float32),
             sums=torch.full((L.RL_ELEM_SUM_COUNT,), float("nan"), device=dev,
                             dtype=torch.float64))
    s = L.RlElemOut()
    for k, v in o.items():
        setattr(s, k, v.data_ptr())
    return o, s


def test_noalloc_matches_workspace_entry_on_two_calls():
    dev = torch.device("cuda:0")
    for N, seed in ((2_160_000, 31), (100_003, 32)):  # the second call is smaller
        print(f"[case] noalloc replay N={N}", flush=True)
        r = make_replay(N=N, seed=seed, device=dev)
        ref = ops.Replay(r.lp, r.lq, r.adv, r.params)
        ref()
        o, out = _outs(N, dev)
        L.rl_loss_elementwise_noalloc(r.lp, r.lq, r.adv, N, ops.elem_cfg(r.params), out)
        torch.cuda.synchronize()
        for k in ("mask_word", "w_primary", "sums"):
            a, b = ref.o[k].cpu().numpy(), o[k].cpu().numpy()
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (N, k)
        assert np.all(np.isfinite(o["sums"].cpu().numpy()))
