"""Fused LM head + RL policy loss on MI355X (gfx950): binding of librlloss.

The computation lives in hand-written HIP kernels behind the C ABI declared in
include/rlloss.h; this package only loads the shared library and marshals
arguments (ctypes), with torch providing device memory and streams.
"""

from . import _lib  # noqa: F401
from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    RlError,
    rl_elementwise_workspace_size,
    rl_loss_elementwise,
    rl_loss_fwd_bwd,
    rl_loss_workspace_size,
    rl_validate_support,
    rl_validate_support_sync,
    rl_version,
    status_string,
)
