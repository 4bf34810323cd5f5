"""Seeded synthetic inputs for the fused LM-head + RL-loss path.

This package only draws input data (hidden states, head weights, sampled
labels, sampler log-probabilities, advantages, per-token supports).  It plays
the role of the inference engine and the data loader.  It computes nothing of
the trainer-side method: no training log-softmax, entropy, importance weight,
mask, loss or gradient lives here.  Both the CPU oracle and the HIP path read
the tensors it returns.
"""

from .gen import (  # noqa: F401
    HEAD_CONFIGS,
    MIS_PARAMS,
    HeadWorkload,
    ReplayWorkload,
    make_head,
    make_replay,
    policy_ages,
    replay_sequences,
)
