"""MXFP4 (e2m1 codes, one e8m0 scale per 32 values), as the oracle computes it.

TEST INFRASTRUCTURE (see the package docstring): never imported by the GPU path.

What the pages fix. The kernel also serves MXFP4, computing on a
checkpoint's exact released bytes instead of re-quantizing them (Jordan
Anderson, jordananderson-pages.pages.dev, section "grouped-nf4-gemm &
experts-4bit", third bullet); the format is e2m1 codes with e8m0 scales
("MoE Training on Consumer GPUs -- Loggetta & Cerin Amroth", Task guides
table, native MXFP4 inference row).

What the pages leave open, and the reading taken (OCP Microscaling Formats
(MX) Specification v1.0, sections 5.3 (E2M1), 5.4 (E8M0) and 6.3
(conversion)):

* e2m1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0. Magnitudes
  by the low three bits: 0, 0.5, 1, 1.5, 2, 3, 4, 6. No inf, no NaN.
* e8m0: an unsigned biased exponent; the scale is 2^(s - 127); s = 255 is NaN.
  s = 0 is 2^-127, a float32 subnormal.
* Blocks of 32 consecutive values along K. Shared exponent
  e = floor(log2(max|w|)) - 2 (2 is the largest e2m1 exponent), taken exactly
  from the float32 bits (frexp), s = clamp(e + 127, 0, 254); an all-zero block
  gets s = 0 and all codes +0.
* Each value w / 2^(s-127) (exact in float64) is rounded to the nearest e2m1
  magnitude, ties to the even mantissa, magnitudes above 6 saturate to 6, and
  the sign bit is the sign bit of w (negative values that round to 0 give -0).
* Nibble order: element 2i in the LOW nibble of byte i (the order of the
  released gpt-oss bytes).
* Dequant: w' = e2m1(q) * 2^(s - 127), exact in float64; its float32 cast is
  exact except that s = 255 gives NaN and 6 * 2^127 overflows to +-inf.

Parity: pinned (e2m1 table by the bit formula; ties and saturation against a
brute-force nearest-value search; dequant over all 256 scales x 16 codes by
the closed form; round trips).
"""

import math

import numpy as np

BLOCK = 32

# e2m1 magnitudes indexed by the 3 low code bits (exponent:mantissa).
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_value(code):
    """Value of a 4-bit e2m1 code (float64)."""
    code = int(code) & 0xF
    mag = E2M1_MAG[code & 7]
    return -mag if code & 8 else mag


def e8m0_scale(s):
    """Scale 2^(s-127) of an e8m0 byte as float64 (NaN for 255)."""
    s = int(s)
    if s == 255:
        return float("nan")
    return math.ldexp(1.0, s - 127)


def shared_exponent(amax):
    """e8m0 byte for a block whose float32 max |w| is amax.

    floor(log2(amax)) comes from frexp (amax = m * 2^ex, 0.5 <= m < 1, so
    floor(log2 amax) = ex - 1), never from a floating-point log.
    """
    amax = float(np.float32(amax))
    if amax == 0.0:
        return 0
    _, ex = math.frexp(amax)
    e = (ex - 1) - 2
    return int(min(max(e + 127, 0), 254))


def round_e2m1(v):
    """e2m1 codes (uint8) nearest to the float64 values v (any shape).

    Nearest magnitude; on an exact tie between two neighbours, the one whose
    code has an even mantissa bit (bit 0); magnitudes above 6 saturate to 6.
    Sign bit from v's sign bit.
    """
    v = np.asarray(v, dtype=np.float64)
    m = np.minimum(np.abs(v).reshape(-1), 6.0)               # saturate first
    dist = np.abs(m[:, None] - E2M1_MAG[None, :])          # [n, 8]
    near = dist == dist.min(axis=1, keepdims=True)          # one or two neighbours
    even = near & ((np.arange(8) & 1) == 0)[None, :]
    idx = np.where(even.any(axis=1), even.argmax(axis=1), near.argmax(axis=1))
    sign = np.where(np.signbit(v.reshape(-1)), 8, 0)
    return (idx | sign).astype(np.uint8).reshape(v.shape)


def quantize(w):
    """MXFP4-quantize W[..., K] (K % 32 == 0).

    Returns (codes_packed uint8 [..., K/2], scales uint8 e8m0 [..., K/32]).
    """
    w = np.asarray(w, dtype=np.float32)
    if w.shape[-1] % BLOCK:
        raise ValueError("last dimension must be a multiple of 32")
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    blocks = w.reshape(-1, BLOCK)
    amax = np.abs(blocks).max(axis=1)
    scales = np.array([shared_exponent(a) for a in amax], dtype=np.uint8)
    # w / 2^(s-127): exact in float64 (power-of-two scaling, no under/overflow).
    inv = np.ldexp(np.ones(scales.size), 127 - scales.astype(np.int64))
    codes = round_e2m1(blocks.astype(np.float64) * inv[:, None])
    lead = w.shape[:-1]
    kk = w.shape[-1]
    return pack(codes.reshape(-1)).reshape(lead + (kk // 2,)), scales.reshape(lead + (kk // BLOCK,))


def pack(codes):
    """Two codes per byte, element 2i in the low nibble."""
    q = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if q.size % 2:
        raise ValueError("odd number of codes")
    return (q[0::2] | (q[1::2] << 4)).astype(np.uint8)


def unpack(packed):
    """Inverse of pack: byte i -> (low nibble, high nibble) = (code 2i, code 2i+1)."""
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & 0x0F
    out[1::2] = p >> 4
    return out


def dequantize(packed, scales, K):
    """Decode MXFP4 bytes to float32: e2m1(q) * 2^(s - 127) per 32-value block."""
    p = np.asarray(packed, dtype=np.uint8)
    lead = p.shape[:-1]
    q = unpack(p).reshape(-1, BLOCK)
    s = np.asarray(scales, dtype=np.uint8).reshape(-1)
    vals = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
    sc = np.array([e8m0_scale(x) for x in range(256)], dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        w = (vals[q] * sc[s][:, None]).astype(np.float32)
    return w.reshape(lead + (K,))
