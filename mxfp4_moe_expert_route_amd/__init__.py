"""MXFP4 Mixture-of-Experts expert layer for AMD Instinct MI355X (gfx950).

The compute lives in libmxfp4moe.so (hand-written HIP kernels behind a C ABI,
include/mxfp4moe.h).  This package only marshals torch tensors (device memory
and the current stream) into those calls; see `ops`."""

from . import _lib  # noqa: F401
from .ops import (  # noqa: F401
    LayerBuffers, dflash_verify_accept, moe_combine, moe_mxfp4_down, moe_mxfp4_gate_up_swiglu, moe_mxfp4_layer,
    moe_mxfp4_layer_noalloc, moe_mxfp4_decode_layer, moe_mxfp4_decode_layer_workspace_bytes,
    decode_layer_workspace,
    moe_permute, moe_permute_workspace_bytes, moe_route_permute, moe_route_topk, moe_router_topk, mxfp4_pack,
    mxfp4_unpack, mxm_stream_xor,
)

MXM_F32, MXM_BF16 = 0, 1
