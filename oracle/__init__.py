"""CPU oracle for the grouped 4-bit mixture-of-experts GEMM.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. The GPU library never imports,
links or executes anything here, and nothing here imports the GPU library.

Everything is plain numpy, computed in float64 unless a format fixes the
precision, written for a reader checking it against the pages by eye:

* ``nf4``      NormalFloat-4 codebook, block quantizer (block 64, fp32 absmax),
               double-quantized absmax, dequantizer, bitsandbytes nibble order.
* ``mxfp4``    OCP MX e2m1 codes with one e8m0 scale per 32 values.
* ``routing``  expert histogram, exclusive prefix sum, stable permutation.
* ``grouped_gemm``  per-expert fp64 matmul on the gathered rows.
* ``combine``  weighted sum of the top-k rows back per token.
* ``layer``    the router's top-k choice with softmax weights, SwiGLU between
               the projections, and exact float64 -> bfloat16 rounding.
* ``backward`` input gradient of the grouped GEMM through the frozen packed
               weights, and its sum over a token's routed copies.
* ``streaming`` which experts an HBM cache of S slots holds, step by step,
               when the layer's experts are streamed from host RAM.

Sources. The pages describe a kernel that computes mixture-of-experts matmuls
directly on 4-bit packed expert weights, one launch for all active experts,
with the 16-entry codebook decoded in registers and no bf16 copy of the
weights (Jordan Anderson, jordananderson-pages.pages.dev, section
"grouped-nf4-gemm & experts-4bit", first bullet; GitHub profile
pjordanandrsn, grouped-nf4-gemm bullets). They print no formulas, tables or
worked examples, so each module states which public definition it follows.

Parity status per function is listed in each module header. Every function
here is pinned by at least one test that does not re-run its own formula.
"""

from . import nf4, mxfp4, routing, grouped_gemm, combine, layer, backward, streaming  # noqa: F401
