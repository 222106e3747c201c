"""Input gradient of the grouped expert GEMM through frozen packed weights (oracle).

TEST INFRASTRUCTURE (see the package docstring): never imported by the GPU path.

The pages say the fused kernel is differentiable, that fine-tuning keeps
computing on the packed 4-bit expert weights in the backward pass instead of
decoding them to a dense copy, and that this backward is a single launch
(Jordan Anderson, jordananderson-pages.pages.dev, section
"grouped-nf4-gemm & experts-4bit", fourth bullet). The expert weights are
frozen there (a QLoRA-style fine-tune), so the only gradient that flows
through the grouped GEMM is the one with respect to its input rows.

The forward call computes, for expert e and each routed row p in
[offsets[e], offsets[e+1]), Y[p, :] = A[p, :] @ W'[e].T with W'[e] the
dequantized [N, K] weights. Its derivative with respect to A is therefore

    dA[p, :] = dY[p, :] @ W'[e]          ([N] times [N, K] -> [K])

a contraction over the N output features of the forward call, reading every
weight row of the expert once per routed row. dY is bfloat16 (held exactly in
float64), W'[e] the float32 dequantized weights (exact in float64), and the
product is the float64 matmul. Rows p >= offsets[E] (dropped assignments) are
left as NaN, as in the forward oracle.

When the forward call gathered its rows from the token activations
(A[p] = X[perm[p] // k]), the gradient of a token's activation row is the sum
of the gradients of its k routed copies:

    dX[t, :] = sum_j dA[inv[t*k + j], :]     (copies with inv = -1 add nothing)

Parity: pinned (the adjoint identity <dA, A> = <dY, Y> against the forward
oracle; a one-hot gradient row returns one dequantized weight row; a
brute-force triple loop on tiny shapes; the token sum against the definition
of the forward gather).
"""

import numpy as np

from . import mxfp4, nf4
from .grouped_gemm import bf16_bits_to_f64, dequant_expert


def grouped_gemm_dx(fmt, codes, scales, scales2, dY_bits, offsets, N, K):
    """dA float64 [rows, K] (rows = dY_bits.shape[0]), in the routed order of dY.

    dY_bits: bfloat16 bits [rows, N]; offsets int [E + 1] from routing.
    """
    dY = bf16_bits_to_f64(dY_bits).reshape(-1, N)
    offsets = np.asarray(offsets).reshape(-1)
    E = offsets.size - 1
    dA = np.full((dY.shape[0], K), np.nan, dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        W = dequant_expert(fmt, codes, scales, scales2, e, N, K).astype(np.float64)
        dA[lo:hi] = dY[lo:hi] @ W
    return dA


def token_grad(dA, inv, T, k):
    """dX float64 [T, K]: the sum over each token's k routed copies of dA,
    taken in copy order j = 0 .. k-1; a copy with inv = -1 (dropped) adds 0."""
    dA = np.asarray(dA, dtype=np.float64)
    inv = np.asarray(inv).reshape(T, k)
    dX = np.zeros((T, dA.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            p = int(inv[t, j])
            if p >= 0:
                dX[t] += dA[p]
    return dX


def dequant_cols(fmt, codes, scales, scales2, e, c0, width, N, K):
    """float32 [N, width]: columns [c0, c0 + width) of expert e's dequantized
    weights, decoded from the matching slice of every row (c0 and width are
    multiples of the format's block, 64 for NF4 / NF4_DQ and 32 for MXFP4),
    with the same block scales as dequant_expert."""
    if fmt == "mxfp4":
        return mxfp4.dequantize(codes[e][:, c0 // 2:(c0 + width) // 2],
                                scales[e][:, c0 // 32:(c0 + width) // 32], width)
    b0, nb = c0 // nf4.BLOCK, width // nf4.BLOCK
    if fmt == "nf4":
        a = np.asarray(scales[e][:, b0:b0 + nb], dtype=np.float32)
    else:
        q8 = np.asarray(scales).reshape(-1)
        s2 = np.asarray(scales2, dtype=np.float32)
        blk = ((e * N + np.arange(N))[:, None] * (K // nf4.BLOCK) + b0 + np.arange(nb)[None, :]).reshape(-1)
        a = (q8[blk].astype(np.float64) * s2[blk // nf4.DQ_GROUP].astype(np.float64)).astype(np.float32)
        a = a.reshape(N, nb)
    return nf4.dequantize(codes[e][:, c0 // 2:(c0 + width) // 2], a, width)


def grouped_gemm_dx_entries(fmt, codes, scales, scales2, dY_bits, offsets, N, K, p, j):
    """float64 dA[p[i], j[i]] for sampled (routed row, column) pairs, as
    grouped_gemm_dx defines them, decoding only the 64-column (NF4) or
    32-column (MXFP4) block of each sampled column, for every weight row."""
    p = np.asarray(p, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    offsets = np.asarray(offsets).reshape(-1)
    blk = 32 if fmt == "mxfp4" else nf4.BLOCK
    expert = np.searchsorted(offsets, p, side="right") - 1
    out = np.empty(p.size, dtype=np.float64)
    for e, cb in sorted(set(zip(expert.tolist(), (j // blk).tolist()))):
        sel = np.nonzero((expert == e) & (j // blk == cb))[0]
        W = dequant_cols(fmt, codes, scales, scales2, e, cb * blk, blk, N, K).astype(np.float64)
        dY = bf16_bits_to_f64(np.asarray(dY_bits)[p[sel]]).reshape(sel.size, N)
        out[sel] = np.einsum("sn,sn->s", dY, W[:, j[sel] - cb * blk].T)
    return out
