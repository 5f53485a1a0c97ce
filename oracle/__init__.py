"""Slow, obviously-correct CPU oracle for the MXFP8 dense linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``mxfp8_block_scaled_amd``) never imports it and shares no code,
tables or constants with it.
"""

from .mx import (  # noqa: F401
    E4M3_MAX,
    bf16_round,
    dequantize_mx,
    e4m3_decode,
    e4m3_encode,
    e8m0_decode,
    gemm_dequant,
    linear_ref,
    quantize_mx,
    scale_exponent,
)
from .moe import moe_ref, route_topk_softmax  # noqa: F401
from .mxfp4 import (  # noqa: F401
    dequantize_mxfp4,
    e2m1_decode,
    e2m1_encode,
    linear_w4a8_ref,
    pack_fp4,
    quantize_mxfp4,
    unpack_fp4,
)
