"""The mixture-of-experts FFN layer around the grouped GEMM (oracle): the
router's top-k choice with its softmax weights, and the SwiGLU step between
the two projections.

TEST INFRASTRUCTURE (see the package docstring): never imported by the GPU path.

The pages run the fused kernel behind a real router and attention (Jordan
Anderson, jordananderson-pages.pages.dev, section "grouped-nf4-gemm &
experts-4bit", the demonstration paragraph of the first bullet) but describe
neither the router nor the activation between the projections. Readings
taken, those of the public models the workloads are shaped after:

* ``topk_softmax``: per token, the k largest logits, ties to the lower
  expert id (a stable sort of the negated logits); NaN ranks below every
  number, so it is chosen only when fewer than k numbers remain, in
  ascending id. Weights are the softmax over the k chosen logits alone,
  in float64 with the largest chosen logit subtracted and the exponentials
  summed in rank order, then rounded to float32.
* ``swiglu``: a gate_up output row holds the gate in columns [0, I) and the
  up projection in [I, 2I); H = silu(gate) * up with silu(x) = x / (1 +
  exp(-x)), in float64, rounded to bfloat16 (nearest, ties to even) because
  H is the bf16 input of the second projection.

Parity: topk_softmax pinned (brute force over ranks on tiny inputs, shift
invariance, weights summing to one, k = E keeping every expert); swiglu
pinned (closed forms at 0 and in the limits, up = 1 reducing to silu, exact
bf16 values rounding to themselves, halfway cases rounding to even).
"""

import math

import numpy as np


def topk_softmax(logits, k):
    """(ids int32 [T, k], weights float32 [T, k]) from float32 logits [T, E]."""
    x = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = x.shape
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float32)
    for t in range(T):
        # ascending sort of -x puts the largest logit first and NaN last;
        # the stable sort keeps equal logits in ascending id
        order = np.argsort(-x[t], kind="stable")[:k]
        ids[t] = order
        sel = x[t][order]
        m = sel[0]
        ex = [math.exp(v - m) if not (math.isnan(v) or math.isnan(m)) else math.nan
              for v in sel]
        s = 0.0
        for v in ex:                       # rank order
            s += v
        w[t] = np.array([v / s for v in ex], dtype=np.float64).astype(np.float32)
    return ids, w


def f64_to_bf16_bits(v):
    """Round float64 values to bfloat16 bits (nearest, ties to even).

    bfloat16 keeps 8 significant bits and float32's exponent range: a finite
    x is M * 2^(E-7) with the integer significand M in [128, 256) for
    normals (E >= -126) and M < 128 at E = -126 for subnormals. The scaled
    value x / 2^(E-7) is exact in float64, so its integer part and remainder
    decide the rounding exactly. NaN maps to 0x7FC0; values that round past
    the largest finite bf16 give infinity."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros(v.shape, dtype=np.uint16)
    res = out.reshape(-1)
    for i, a in enumerate(v.reshape(-1)):
        a = float(a)
        if math.isnan(a):
            res[i] = 0x7FC0
            continue
        sign = 0x8000 if math.copysign(1.0, a) < 0 else 0
        x = abs(a)
        if x == 0.0:
            res[i] = sign
            continue
        if math.isinf(x):
            res[i] = sign | 0x7F80
            continue
        m, e = math.frexp(x)                # x = m * 2^e, m in [0.5, 1)
        E = max(e - 1, -126)
        q = math.ldexp(x, 7 - E)            # exact: a power-of-two scaling
        n = math.floor(q)
        r = q - n
        if r > 0.5 or (r == 0.5 and n % 2 == 1):
            n += 1
        if n == 256:                        # carried into the next binade
            n, E = 128, E + 1
        if E > 127:
            res[i] = sign | 0x7F80
        elif n < 128:                       # subnormal (E = -126)
            res[i] = sign | n
        else:
            res[i] = sign | ((E + 127) << 7) | (n - 128)
    return out


def silu(x):
    """x / (1 + exp(-x)) in float64 (exp(-x) overflowing to inf gives -0)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu(Y, I):
    """H bf16 bits [rows, I] from the gate_up output Y [rows, 2I] (float32 or
    float64): H = bf16(silu(Y[:, :I]) * Y[:, I:])."""
    Y = np.asarray(Y)
    g = Y[:, :I].astype(np.float64)
    u = Y[:, I:2 * I].astype(np.float64)
    return f64_to_bf16_bits(silu(g) * u)
