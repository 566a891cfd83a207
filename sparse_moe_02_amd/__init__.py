"""MI355X (gfx950) sparse mixture-of-experts feed-forward layer.

The layer runs in hand-written HIP kernels behind the C ABI of ``include/moe.h``;
``binding`` marshals arguments to it and ``layer.MoeLayer`` keeps one layer's device
tensors, plan and workspace.  Importing this package does not load the library;
the first call does, and fails loudly if it has not been built.
"""

from .binding import (  # noqa: F401
    EXPORTED,
    HipEvents,
    MoeError,
    moe_config,
    moe_debug_out,
    moe_forward_decode,
    moe_forward_prefill,
    moe_plan_create,
    moe_plan_destroy,
    moe_qmat,
    moe_status_string,
    moe_version,
    moe_weights,
    moe_workspace_init,
)


def MoeLayer(*args, **kwargs):
    """See :class:`sparse_moe_02_amd.layer.MoeLayer` (imports torch on first use)."""
    from .layer import MoeLayer as _L

    return _L(*args, **kwargs)
