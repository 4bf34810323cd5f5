"""The machine-calibration calls: the copy is exact, the MFMA loop leaves the
accumulators where the arithmetic puts them, and the clock stamps are sane."""

import numpy as np
import pytest
import torch

from lm_head_logprobs_amd import _lib as L

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096 + 48, 3), (1 << 20, 64),
                                           ((1 << 22) + 16 * 5, 1000)])
def test_copy_out_of_place_and_in_place(nbytes, blocks):
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8).to(DEV)
    ref = src.clone()
    dst = torch.zeros_like(src)
    guard = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
    L.rl_calib_copy(src, dst, nbytes, blocks)
    L.rl_calib_copy(src, src, nbytes, blocks)
    # a shorter copy into a larger buffer leaves the rest untouched
    L.rl_calib_copy(src, guard, nbytes, blocks)
    torch.cuda.synchronize()
    assert torch.equal(dst, ref)
    assert torch.equal(src, ref)
    assert torch.equal(guard[:nbytes], ref)
    assert int(guard[nbytes:].abs().sum()) == 0


def test_mfma_zero_operands_keep_the_start_values_and_stamps_are_ordered():
    nb = 8
    sink = torch.full((nb * 256,), float("nan"), device=DEV)
    stamps = torch.zeros(nb * 4, dtype=torch.int64, device=DEV)
    flop, khz = L.rl_calib_mfma_bf16(False, nb, 500, sink, stamps)
    torch.cuda.synchronize()
    assert flop == nb * 4 * 500 * 16 * 2 * 16 * 16 * 32
    assert khz > 0
    # zero operands add nothing: each chain keeps z = (c * 256 + thread) / 2^20 in
    # all four lanes, summed in the kernel's order (exact in fp32 here)
    tid = np.arange(nb * 256) % 256
    exp = np.zeros(nb * 256, np.float32)
    for c in range(16):
        z = ((c * 256 + tid) * 2.0 ** -20).astype(np.float32)
        exp = exp + ((z + z) + (z + z))
    np.testing.assert_array_equal(sink.cpu().numpy(), exp)
    st = stamps.view(nb, 4).cpu().numpy()
    assert (st[:, 1] > st[:, 0]).all() and (st[:, 3] > st[:, 2]).all()
    ghz = np.median((st[:, 1] - st[:, 0]) / (st[:, 3] - st[:, 2])) * khz * 1e3 / 1e9
    assert 0.3 < ghz < 3.5, ghz


def test_mfma_random_operands_are_finite_and_deterministic():
    nb = 4
    outs = []
    for _ in range(2):
        sink = torch.empty(nb * 256, device=DEV)
        stamps = torch.zeros(nb * 4, dtype=torch.int64, device=DEV)
        L.rl_calib_mfma_bf16(True, nb, 300, sink, stamps)
        torch.cuda.synchronize()
        outs.append(sink.cpu())
    assert torch.isfinite(outs[0]).all()
    assert torch.equal(outs[0], outs[1])
    assert float(outs[0].abs().max()) > 0.0
