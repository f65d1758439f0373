"""GLM-5.2 mixture-of-experts feed-forward layer for AMD Instinct MI355X (gfx950).

The layer runs in hand-written HIP kernels behind the C ABI of
``include/glm_moe.h`` (``libglm_moe.so``); this package is its thin Python
binding.  Build the library with ``python -m sparse_moe_transformer_glm_amd.build``.
"""
from ._lib import (BF16, EHIP, EINVAL, EUNSUPPORTED, EWORKSPACE, F32, LIB_PATH, MXFP8, OK,
                   STAGES, GlmMoeError, HiddenLayout, MxWeights, Options, Trace, dense_ffn, dense_workspace_size,
                   forward, forward_mx, forward_noalloc, hidden_layout, lib, new_workspace, options, pack_mx_scales, route,
                   workspace_bytes, workspace_size)

__all__ = ["BF16", "EHIP", "EINVAL", "EUNSUPPORTED", "EWORKSPACE", "F32", "LIB_PATH", "MXFP8",
           "OK", "STAGES", "GlmMoeError", "HiddenLayout", "MxWeights", "Options", "Trace", "dense_ffn",
           "dense_workspace_size", "forward", "forward_mx", "forward_noalloc", "hidden_layout", "lib", "new_workspace", "options",
           "pack_mx_scales",
           "route", "workspace_bytes", "workspace_size"]
