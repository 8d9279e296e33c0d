"""MI355X (gfx950) MoE layer hot path: route, align, expert FFN, combine.

The kernels are hand-written HIP in ``csrc/`` behind the C ABI of
``include/moe.h`` (``libmoe.so``, built in-tree by ``build.build()``); this
package is a thin ctypes binding with the same names.
"""
from .binding import (  # noqa: F401
    MOE_BF16, MOE_F32, MOE_I4, MOE_I4A8, MOE_I8, Layer, MoeError, align, capacity, combine, combine_shared, expert_ffn,
    ffn_block_m, ffn_down, ffn_up, ffn_workspace, last_dispatch, layer, lib, pack_int4, route, route_align, version, LIB_PATH, SIGNATURES,
)
