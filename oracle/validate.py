"""Sampler-evidence checks on a CSR per-token support, as a flag word.

Test infrastructure.  Source: prime-rl pull request 4233, "What changes"
(sampler-evidence validation runs on the GPU on the CSR entries, once per step
before the optimizer) and the TokenSupport bullet (int32 ids, host int64
offsets, replayed flag, sampler log-probs).  The pages do not list the checks;
the ones below follow from what the loss needs of its inputs:

  bit 0  a label outside [0, V)
  bit 1  a support id outside [0, V)
  bit 2  a support weight u < 0 or not finite
  bit 3  a per-entry sampler log-prob not finite or > 0
  bit 4  a label sampler log-prob not finite or > 0
  bit 5  replayed: a row whose weights do not sum to 1 within 1e-3
         (sums formed in fp64 from the stored fp32 values)
  bit 6  replayed: a row that does not hold its own label
  bit 7  an advantage not finite
  bit 8  device offsets not a valid CSR (off[0] != 0, decreasing,
         off[N] != nnz, or a row outside [0, nnz])

Entry checks (bits 1-3) do not depend on the offsets and always run; the
replayed-row checks (bits 5-6) run on every row whose own offsets are sane.
"""

import numpy as np

BAD_LABEL = 1 << 0
BAD_ID = 1 << 1
BAD_U = 1 << 2
BAD_LOGQ = 1 << 3
BAD_INFER_LOGPROB = 1 << 4
BAD_REPLAY_MASS = 1 << 5
BAD_REPLAY_LABEL = 1 << 6
BAD_ADV = 1 << 7
BAD_OFFSETS = 1 << 8

REPLAY_MASS_TOL = 1e-3


def validate_reference(V, labels, infer_logprobs, adv, offsets=None, ids=None, u=None,
                       logq=None, replayed=False):
    labels = np.asarray(labels, np.int64)
    lq = np.asarray(infer_logprobs, np.float32).astype(np.float64)
    A = np.asarray(adv, np.float32).astype(np.float64)
    N = len(labels)
    flags = 0
    if np.any((labels < 0) | (labels >= V)):
        flags |= BAD_LABEL
    if np.any(~np.isfinite(lq) | (lq > 0)):
        flags |= BAD_INFER_LOGPROB
    if np.any(~np.isfinite(A)):
        flags |= BAD_ADV
    if offsets is None:
        return flags
    off = np.asarray(offsets, np.int64)
    ids = np.asarray(ids, np.int64)
    nnz = len(ids)

    def row_sane(t):
        e0, e1 = off[t], off[t + 1]
        ok = 0 <= e0 <= e1 <= nnz
        if t == 0 and e0 != 0:
            ok = False
        if t == N - 1 and e1 != nnz:
            ok = False
        return ok

    sane = [row_sane(t) for t in range(N)]
    if not all(sane):
        flags |= BAD_OFFSETS
    if np.any((ids < 0) | (ids >= V)):
        flags |= BAD_ID
    uu = np.asarray(u, np.float32).astype(np.float64)
    if np.any(~np.isfinite(uu) | (uu < 0)):
        flags |= BAD_U
    if logq is not None:
        lg = np.asarray(logq, np.float32).astype(np.float64)
        if np.any(~np.isfinite(lg) | (lg > 0)):
            flags |= BAD_LOGQ
    if replayed:
        for t in range(N):
            if not sane[t]:
                continue
            e0, e1 = off[t], off[t + 1]
            s = uu[e0:e1].sum()
            if not abs(s - 1.0) <= REPLAY_MASS_TOL:
                flags |= BAD_REPLAY_MASS
            if not np.any(ids[e0:e1] == labels[t]):
                flags |= BAD_REPLAY_LABEL
    return flags
