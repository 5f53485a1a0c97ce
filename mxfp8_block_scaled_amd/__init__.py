"""MXFP8 dense linear layer (and its top-k routed MoE variant) for AMD
Instinct MI355X (gfx950).

The arithmetic lives in hand-written HIP kernels behind a C-ABI shared library
(``libmxfp8.so``); this package is the thin Python binding over it.  Importing
the package does not load the library; the first call does, and fails with an
error if it has not been built.
"""

_API = (
    "PreparedWeight", "linear", "prepare_weight", "quantize_act", "moe_grouped",
    "mxfp8_quantize_act", "mxfp8_prepared_weight_bytes", "mxfp8_prepare_weight",
    "mxfp8_unpack_weight", "mxfp8_linear_workspace_bytes", "mxfp8_linear",
    "mxfp8_packed_act_bytes", "mxfp8_quantize_act_packed", "mxfp8_gemm_packed",
    "quantize_act_packed", "gemm_packed", "PackedActivation",
    "mxfp8_moe_grouped", "mxfp8_moe_workspace_bytes", "mxfp8_moe_prepared_bytes",
    "mxfp8_moe_prepare_weights", "mxfp8_moe_debug_capture", "MoEWeights", "moe_prepare_weights",
    "moe_debug_capture",
    "PreparedWeightFP4", "prepare_weight_fp4", "quantize_fp4", "mxfp8_quantize_fp4", "mxfp8_prepared_weight_fp4_bytes", "mxfp8_prepare_weight_fp4",
    "mxfp8_linear_w4a8_workspace_bytes", "mxfp8_linear_w4a8",
    "mxfp8_status_string", "MXFP8Error",
)


def __getattr__(name):
    if name in _API:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
