"""Grouped 4-bit mixture-of-experts GEMM for AMD MI355X (gfx950).

The compute path is the HIP library libgnf4.so (csrc/, C ABI in
include/gnf4.h); ``gnf4`` is its Python binding. Build with
``python -m bit_mixture_experts_topk_amd.build``.
"""

from . import gnf4  # noqa: F401
from .gnf4 import (MXFP4, NF4, NF4_DQ, PackedWeights, build_id, combine, dequant,  # noqa: F401
                   grouped_gemm, quantize, route)
