"""CPU oracle for the fused LM-head + RL-loss path (test infrastructure).

Plain, slow fp64 numpy written from the source pages.  Only the tests, the
smoke check and the bench's CPU baseline may import it; the library never
does.  It shares no code with the HIP path.

Modules:
  weights  - per-token importance weights and masks (IPO, IcePop, REINFORCE)
  head     - the fused head forward + backward, always with a dense gradient
  replay   - the loss-only mismatch replay (IPO eps sweep, IcePop band,
             PPO-bypass with dual clip, decoupled token-level TIS)
  validate - sampler-evidence checks of a CSR support, as a flag word

Parity status: every function here is pinned by tests under tests/ (worked
examples from the pages, closed forms, brute force, finite differences,
library special cases).  The masked fractions measured on real runs cannot be
reproduced without that run's data: parity unpinned for those two figures
only (they are not computed here).
"""
