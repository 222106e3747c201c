"""Grouped expert GEMM on dequantized weights, in float64 (oracle).

TEST INFRASTRUCTURE (see the package docstring): never imported by the GPU path.

The operation (Jordan Anderson, jordananderson-pages.pages.dev, section
"grouped-nf4-gemm & experts-4bit", first bullet; GitHub profile
pjordanandrsn, grouped-nf4-gemm bullets): one call computes the matmul of
every active expert on its own rows, reading that expert's packed weights.
For expert e and every routed row p in [offsets[e], offsets[e+1]):

    Y[p, :] = A[p, :] @ W'[e].T          W'[e] = dequant(packed W[e]) [N, K]

with A[p] = X[perm[p] // k] when the rows are gathered from the token
activations (the first projection) and A[p] = X[p] when X already holds the
routed rows in permuted order (the second projection). X is bfloat16, held
exactly in float64; the dequantized weights are float32, also exact in
float64; the product is the float64 matmul (a library primitive), and rows
p >= offsets[E] (dropped assignments) are left as NaN (not computed).

Parity: pinned (E = 1, k = 1 reduces to a plain matmul; one-hot rows
select single weights exactly; integer-valued cases are exact).
"""

import numpy as np

from . import mxfp4, nf4

FORMATS = ("nf4", "nf4_dq", "mxfp4")


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) to float64, exactly (bits << 16 is the fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def dequant_expert(fmt, codes, scales, scales2, e, N, K):
    """float32 [N, K] dequantized weights of expert e.

    codes uint8 [E, N, K/2]; scales: NF4 float32 [E, N, K/64], NF4_DQ int8
    [E, N, K/64] with scales2 float32 over the flat block index, MXFP4 uint8
    e8m0 [E, N, K/32].
    """
    if fmt == "nf4":
        return nf4.dequantize(codes[e], scales[e], K)
    if fmt == "nf4_dq":
        nb = K // nf4.BLOCK
        q8 = np.asarray(scales).reshape(-1)
        s2 = np.asarray(scales2, dtype=np.float32)
        first = e * N * nb                          # flat index of this expert's first block
        blk = np.arange(first, first + N * nb)
        a = (q8[blk].astype(np.float64) * s2[blk // nf4.DQ_GROUP].astype(np.float64)).astype(np.float32)
        return nf4.dequantize(codes[e], a.reshape(N, nb), K)
    if fmt == "mxfp4":
        return mxfp4.dequantize(codes[e], scales[e], K)
    raise ValueError("unknown format %r" % (fmt,))


def dequant_rows(fmt, codes, scales, scales2, e, rows, N, K):
    """float32 [len(rows), K]: rows `rows` of expert e, dequantized exactly as
    dequant_expert does for the whole expert (same block scales, same flat
    block index for NF4_DQ), without decoding the other rows."""
    rows = np.asarray(rows, dtype=np.int64)
    if fmt == "nf4":
        return nf4.dequantize(codes[e][rows], scales[e][rows], K)
    if fmt == "nf4_dq":
        nb = K // nf4.BLOCK
        q8 = np.asarray(scales).reshape(-1)
        s2 = np.asarray(scales2, dtype=np.float32)
        blk = ((e * N + rows)[:, None] * nb + np.arange(nb)[None, :]).reshape(-1)
        a = (q8[blk].astype(np.float64) * s2[blk // nf4.DQ_GROUP].astype(np.float64)).astype(np.float32)
        return nf4.dequantize(codes[e][rows], a.reshape(len(rows), nb), K)
    if fmt == "mxfp4":
        return mxfp4.dequantize(codes[e][rows], scales[e][rows], K)
    raise ValueError("unknown format %r" % (fmt,))


def grouped_gemm(fmt, codes, scales, scales2, X_bits, gather, offsets, perm, k, N, K):
    """Y float64 [rows, N] of the grouped GEMM (rows = T*k).

    X_bits: bfloat16 bits, [T, K] when gather else [T*k, K] in permuted order.
    """
    X = bf16_bits_to_f64(X_bits)
    offsets = np.asarray(offsets).reshape(-1)
    perm = np.asarray(perm).reshape(-1)
    E = offsets.size - 1
    rows = perm.size
    Y = np.full((rows, N), np.nan, dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        W = dequant_expert(fmt, codes, scales, scales2, e, N, K).astype(np.float64)
        if gather:
            A = X[perm[lo:hi] // k]
        else:
            A = X[lo:hi]
        Y[lo:hi] = A @ W.T
    return Y
