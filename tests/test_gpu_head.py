"""Parity of the fused head (rl_loss_fwd_bwd through the C ABI) with the oracle."""

import numpy as np
import pytest
import torch

from gpu_util import compare_all, compare_forward, record, rel_fro, run_head, to_np
from oracle import head as ohead
from synth import make_head, policy_ages

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"

# Small shapes that still span several 128-wide tiles in every dimension and
# end in a ragged tail (none of N, V is a multiple of 128; H = 320 is not a
# multiple of the 64-wide K tile of the dh / dW contractions).
SMALL = dict(N=300, H=320, V=5000)


def _case(name, **kw):
    shape = dict(SMALL)
    shape.update(kw)
    wl = make_head(name, device=DEV, **shape)
    print(f"[case] {name} {shape} nnz={wl.nnz} info={wl.info}", flush=True)
    return wl


@pytest.mark.parametrize("name", ["c1_tiny_fp32_ipo"])
def test_tiny_fp32_full_size(name):
    wl = make_head(name, device=DEV)
    print(f"[case] {name} full size", flush=True)
    _, got = run_head(wl)
    ref = ohead.from_workload(wl)
    r = compare_all(wl, got, ref, case=f"{name} full size")
    print(r)


@pytest.mark.parametrize("name", [
    "c3_head16k_ipo", "c4_head16k_ipo_topp_replay", "c5a_head64k_draws_ipo_k1",
    "c5b_head64k_draws_reinforce",
])
def test_small_parity(name):
    wl = _case(name)
    _, got = run_head(wl)
    ref = ohead.from_workload(wl)
    r = compare_all(wl, got, ref, case=f"{name} small")
    print(r)


def test_icepop_and_fp32_grad():
    wl = _case("c4_head16k_ipo_topp_replay", N=257, V=3001 + 7)
    wl.params.update(loss_type="icepop", icepop_lo=0.5, icepop_hi=2.0)
    _, got = run_head(wl, grad_dtype=torch.float32)
    ref = ohead.from_workload(wl)
    r = compare_all(wl, got, ref, case="icepop, fp32 dh")
    print(r)


def test_temperature_adv_tau_and_accumulate():
    wl = _case("c5a_head64k_draws_ipo_k1", N=200, V=2048)
    wl.params.update(inv_temperature=1.25, adv_tau=0.5, loss_norm=77.0)
    fh, got = run_head(wl, accumulate_dW=True)
    ref = ohead.from_workload(wl)
    compare_all(wl, got, ref, case="temperature, adv_tau, D, accumulate")
    fh()  # dW accumulates a second copy of the gradient
    torch.cuda.synchronize()
    assert rel_fro(to_np(fh.o["dW"]), 2.0 * ref["dW"]) <= 1e-2


def test_dense_and_sparse_backward_agree_when_kappa_vanishes():
    # reinforce, no KL, u = 1/16 over 16 draws: kappa = s (1 - sum u) = 0 exactly.
    wl = _case("c5b_head64k_draws_reinforce")
    _, sp = run_head(wl, backward="sparse")
    _, de = run_head(wl, backward="dense")
    assert sp["metrics"][5] == 0.0  # max |kappa|
    assert np.array_equal(sp["logprobs"], de["logprobs"])
    assert np.array_equal(sp["loss"], de["loss"])
    # the dense softmax part is zero; the dense path carries the label and
    # support coefficients inside the bf16 operand G (relative rounding 2^-9
    # per element) while the sparse path keeps them in fp32
    ref = ohead.from_workload(wl)
    rep = {"dense_vs_sparse_dh": rel_fro(de["dh"], sp["dh"]),
           "dense_vs_sparse_dW": rel_fro(de["dW"], sp["dW"]),
           "dense_dh_vs_oracle": rel_fro(de["dh"], ref["dh"]),
           "dense_dW_vs_oracle": rel_fro(de["dW"], ref["dW"]),
           "sparse_dh_vs_oracle": rel_fro(sp["dh"], ref["dh"]),
           "sparse_dW_vs_oracle": rel_fro(sp["dW"], ref["dW"])}
    record("c5b small: dense vs sparse backward", rep)
    print(rep)
    assert rep["dense_vs_sparse_dh"] <= 2.0**-8
    assert rep["dense_vs_sparse_dW"] <= 2.0**-8


def _ref(wl, **kw):
    age = getattr(wl, "age", None)
    return ohead.from_workload(wl, age=None if age is None else to_np(age), **kw)


@pytest.mark.parametrize("name", ["c5a_head64k_draws_ipo_k1", "c4_head16k_ipo_topp_replay"])
def test_kl_staleness_and_entropy_bonus(name):
    # inv_sqrt KL staleness from per-token ages and an entropy bonus, bf16 tiled path
    wl = _case(name)
    wl.age = policy_ages(wl.N, device=DEV)
    wl.params.update(kl_staleness="inv_sqrt", entropy_coeff=0.05)
    _, got = run_head(wl)
    ref = _ref(wl)
    assert 0 < np.count_nonzero(to_np(wl.age)) < wl.N
    r = compare_all(wl, got, ref, case=f"{name} small, inv_sqrt staleness, entropy bonus")
    print(r)


def test_entropy_bonus_fp32_and_negative():
    wl = make_head("c1_tiny_fp32_ipo", device=DEV)
    print("[case] c1 fp32 with an entropy penalty", flush=True)
    wl.params.update(entropy_coeff=-0.2)
    _, got = run_head(wl)
    r = compare_all(wl, got, _ref(wl), case="c1 fp32, entropy penalty")
    print(r)


def test_entropy_bonus_makes_reinforce_dense():
    # reinforce without KL on a support would take the sparse backward; the
    # entropy term puts mass on every logit, so AUTO plans the dense one
    wl = _case("c5b_head64k_draws_reinforce")
    wl.params.update(entropy_coeff=0.03, backward="auto")
    _, got = run_head(wl)
    assert np.abs(got["dW"]).sum() > 0
    r = compare_all(wl, got, _ref(wl), case="c5b small, entropy bonus (dense)")
    print(r)


def test_token_chunking_invariance():
    wl = _case("c4_head16k_ipo_topp_replay", N=333)
    _, a = run_head(wl)
    _, b = run_head(wl, token_chunk=64)
    for k in ("logprobs", "entropy", "token_loss", "weight", "keep", "support_logprobs"):
        assert np.array_equal(a[k], b[k]), k
    assert rel_fro(b["dh"], a["dh"]) <= 1e-5
    assert rel_fro(b["dW"], a["dW"]) <= 1e-5


def test_full_size_one_chunk_matches_two():
    """The 16k workload as one 16384-token chunk against the default two of
    8192.  With one chunk G spans 4.98 GB, so the persistent dW reaches its
    panels through a descriptor rebuilt at each stage; with two (2.49 GB each)
    one descriptor per tile and 32-bit offsets serve every panel.  Per-token
    outputs must agree bit for bit, dh and dW to fp32 rounding."""
    wl = make_head("c3_head16k_ipo", device="cuda:0")
    print("[case] c3 full size, token chunk 16384 against 8192", flush=True)
    _, a = run_head(wl)
    _, b = run_head(wl, token_chunk=16384)
    for k in ("logprobs", "entropy", "token_loss", "weight", "keep"):
        assert np.array_equal(a[k], b[k]), k
    assert rel_fro(b["dh"], a["dh"]) <= 1e-5
    e = rel_fro(b["dW"], a["dW"])
    print(f"dW rel fro {e:.3g}")
    assert e <= 1e-5


@pytest.mark.parametrize("chunk", [160, 129])
def test_short_token_chunks_through_the_persistent_dW(chunk):
    # dW's persistent kernel needs at least five 32-token K-steps: chunks of
    # 129..160 tokens give exactly five (and the tail chunk fewer, which takes
    # the one-tile kernel); V = 70000, H = 512 give more tiles than workgroups,
    # so the epilogue stores of one tile overlap the next tile's first stages.
    wl = _case("c5a_head64k_draws_ipo_k1", N=300, H=512, V=70000)
    _, got = run_head(wl, token_chunk=chunk)
    ref = ohead.from_workload(wl)
    compare_all(wl, got, ref, case=f"token chunk {chunk}, V=70000, H=512")


@pytest.mark.parametrize("H,chunk", [(224, 0), (224, 160), (224, 128), (160, 96)])
def test_odd_stage_counts(H, chunk):
    # The persistent forward (K = H) and dW (K = the chunk's tokens) pick the
    # fragment set that holds stage 0 by the parity of their stage count:
    # H = 224 and 160 give 7 and 5 stages of 32 (odd; the workloads' H are
    # even multiples), chunks of 160 tokens 5 dW stages, the default chunk 10;
    # 128- and 96-token chunks give 4 and 3, too few for the persistent dW's
    # five-stage ring (the one-tile dW kernel takes them).
    wl = _case("c4_head16k_ipo_topp_replay", N=300, H=H, V=5000)
    _, got = run_head(wl, token_chunk=chunk)
    ref = ohead.from_workload(wl)
    compare_all(wl, got, ref, case=f"H={H}, token chunk {chunk or 'default'}")


def test_bitwise_deterministic():
    wl = _case("c5a_head64k_draws_ipo_k1", N=260)
    fh, a = run_head(wl)
    fh()
    torch.cuda.synchronize()
    b = {k: to_np(v) for k, v in fh.o.items()}
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_forward_only_and_single_gradient():
    wl = _case("c3_head16k_ipo", N=130, V=1000)
    _, f = run_head(wl, backward="none", want_dh=False, want_dW=False)
    _, full = run_head(wl)
    for k in ("logprobs", "entropy", "token_loss", "loss"):
        assert np.array_equal(f[k], full[k]), k
    _, only_dh = run_head(wl, want_dW=False)
    assert np.array_equal(only_dh["dh"], full["dh"])
    _, only_dw = run_head(wl, want_dh=False)
    assert np.array_equal(only_dw["dW"], full["dW"])


@pytest.mark.parametrize("shape", [dict(N=1, H=8, V=1), dict(N=5, H=8, V=3),
                                   dict(N=129, H=136, V=129)])
def test_degenerate_shapes(shape):
    wl = _case("c5a_head64k_draws_ipo_k1", **shape)
    _, got = run_head(wl)
    ref = ohead.from_workload(wl)
    compare_all(wl, got, ref, case=f"degenerate {shape}")


@pytest.mark.parametrize("shape", [dict(N=1, H=8, V=1), dict(N=5, H=8, V=3),
                                   dict(N=129, H=136, V=129)])
def test_degenerate_shapes_fp32(shape):
    # the fp32 path (its own GEMM tiles and partial tile height) at the same
    # edge shapes
    wl = _case("c1_tiny_fp32_ipo", **shape)
    _, got = run_head(wl)
    ref = ohead.from_workload(wl)
    compare_all(wl, got, ref, case=f"fp32 degenerate {shape}")


def test_empty_support_rows_and_duplicates():
    wl = _case("c5a_head64k_draws_ipo_k1", N=64, V=900)
    off = wl.offsets.clone()
    # empty the support of every 5th row by moving its entries to the next row
    sizes = (off[1:] - off[:-1]).clone()
    for t in range(0, 63, 5):
        sizes[t + 1] += sizes[t]
        sizes[t] = 0
    wl.offsets = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(sizes, 0)])
    wl.ids[1] = wl.ids[0]  # a repeated id inside one row
    _, got = run_head(wl)
    ref = ohead.from_workload(wl)
    compare_all(wl, got, ref, case="empty support rows, repeated id")


def test_invalid_ids_give_nan_only_where_used():
    """Ids outside [0, V) are reported by the validation call; the head itself
    must not read through them.  The tokens that use one get NaN; every other
    token's per-token outputs and dh row are bit-identical to the clean run
    (the label / support logits are formed per entry and G row by row)."""
    wl = _case("c4_head16k_ipo_topp_replay", N=64, V=900)
    V = wl.W.shape[0]
    _, clean = run_head(wl)
    off = wl.offsets.cpu().numpy()
    sizes = off[1:] - off[:-1]
    t_lab = 3
    t_low, t_high = [int(t) for t in np.nonzero(sizes >= 2)[0] if t != t_lab][:2]
    e_low, e_high = int(off[t_low]), int(off[t_high]) + 1
    wl.labels[t_lab] = V + 7
    wl.ids[e_low] = -2
    wl.ids[e_high] = V
    _, got = run_head(wl)
    bad = [t_lab, t_low, t_high]
    good = np.setdiff1d(np.arange(wl.N), bad)
    assert np.isnan(got["logprobs"][t_lab])
    assert np.all(np.isnan(got["token_loss"][bad]))
    assert np.isnan(got["support_logprobs"][e_low]) and np.isnan(got["support_logprobs"][e_high])
    for k in ("logprobs", "entropy", "token_loss", "weight"):
        assert np.array_equal(got[k][good], clean[k][good]), k
    assert np.array_equal(got["entropy"], clean["entropy"])
    assert np.array_equal(got["dh"][good], clean["dh"][good])


# ---------------------------------------------------------------- full size --

def _sample(n, k, seed):
    return np.sort(np.random.default_rng(seed).choice(n, size=k, replace=False))


FULL = ["c3_head16k_ipo", "c4_head16k_ipo_topp_replay", "c5a_head64k_draws_ipo_k1",
        "c5b_head64k_draws_reinforce", "c4_head16k_ipo_topp_replay+stale_entropy"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_tokens(name):
    """The benchmarked launch configuration at full size (H=2048, V=152064;
    16384 or 65536 tokens): per-token outputs, support log-probs and dh rows
    on a token sample against the oracle token by token; the loss against the
    fp64 sum of the per-token losses; the batch passes validation; dW column
    sums vanish (each token's logit gradient sums to zero over the
    vocabulary)."""
    from lm_head_logprobs_amd import ops as _ops
    base, _, variant = name.partition("+")
    wl = make_head(base, device=DEV)
    if variant == "stale_entropy":  # inv_sqrt KL staleness and an entropy bonus
        wl.age = policy_ages(wl.N, device=DEV)
        wl.params.update(kl_staleness="inv_sqrt", entropy_coeff=0.02)
    print(f"[case] {name} full size N={wl.N} nnz={wl.nnz} info={wl.info}", flush=True)
    st, flags = _ops.validate(wl.labels, wl.infer_logprobs, wl.adv, wl.V, wl.offsets, wl.ids,
                              wl.u, wl.logq, wl.params["replayed"])
    assert flags == 0, hex(flags)
    _, got = run_head(wl)
    tok = _sample(wl.N, 24, 1)
    ref = _ref(wl, tokens=tok, want_grads=True)
    rep = {}
    near, _ = compare_forward(wl, got, ref, tokens=tok, report=rep)
    ok = ~near
    dh_err = rel_fro(got["dh"][tok][ok], ref["dh"][ok])
    rep["dh_rel_sampled_rows"] = dh_err
    record(f"{name} full size, 24 sampled tokens", rep)
    assert dh_err <= 1e-2, dh_err
    total = got["token_loss"].sum() / wl.params["loss_norm"]
    assert abs(got["loss"][0] - total) <= 1e-5 * abs(total) + 1e-7
    # Column sums of dW: the label, support and softmax parts of each token's
    # logit gradient cancel; scale = sum_t (|s_t| (w_t + sum_e c_e) + beta sum_e u_e) |h_t| / D.
    col = got["dW"].sum(axis=0)
    hn = np.linalg.norm(to_np(wl.h), axis=1)
    a = np.abs(to_np(wl.adv))
    beta = ohead.kl_beta(wl.params)
    gamma = abs(wl.params.get("entropy_coeff", 0.0))
    scale = np.sum((a * (np.abs(got["weight"]) + 5.0) + 2 * beta + 2 * gamma * np.log(wl.V)) *
                   hn) / wl.params["loss_norm"]
    assert np.linalg.norm(col) <= 1e-3 * scale


@pytest.mark.parametrize("name", ["c3_head16k_ipo", "c5b_head64k_draws_reinforce"])
def test_full_size_dW_on_token_sample(name):
    """Full-size launch with the advantage zeroed outside a token sample (no
    KL): only sampled tokens carry gradient, so dW over all 152064 rows is the
    oracle's dW from those tokens."""
    from synth.gen import HEAD_CONFIGS
    n = HEAD_CONFIGS[name]["N"]
    mask = torch.zeros(n, dtype=torch.bool)
    tok = _sample(n, 16, 2)
    mask[torch.as_tensor(tok)] = True
    wl = make_head(name, device=DEV, adv_zero_except=mask)
    print(f"[case] {name} full size, advantage on {len(tok)} tokens", flush=True)
    _, got = run_head(wl)
    ref = ohead.from_workload(wl, tokens=tok, want_grads=True)
    rep = {}
    compare_forward(wl, got, ref, tokens=tok, report=rep)
    rep["dW_rel"] = rel_fro(got["dW"], ref["dW"])
    record(f"{name} full size, advantage on 16 tokens", rep)
    assert rep["dW_rel"] <= 1e-2
    other = np.setdiff1d(np.arange(n), tok)
    assert np.all(got["dh"][other] == 0.0)
