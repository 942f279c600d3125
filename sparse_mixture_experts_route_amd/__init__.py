"""MI355X (gfx950) sparse MoE FFN layer: HIP kernels behind the C-ABI of
libmoe_mi355x.so (include/moe.h), with a ctypes binding of the same names."""
from ._lib import (  # noqa: F401
    EXPORTED, LIB_PATH, MoeError, MoeShape, load, make_shape, moe_aux_loss, moe_balance_counts,
    moe_combine, moe_dispatch, moe_ffn_backward, moe_ffn_forward, moe_ffn_forward_partial,
    moe_parallel_block_forward, moe_route, workspace_bytes,
)
