"""NF4 (4-bit NormalFloat) block encoding, as the oracle computes it.

TEST INFRASTRUCTURE (see the package docstring): never imported by the GPU path.

What the pages fix. The kernel consumes NF4 weights "on the bitsandbytes
packed layout unchanged": a sixteen-entry codebook, two codes per byte, one
absmax per block (Jordan Anderson, jordananderson-pages.pages.dev, section
"grouped-nf4-gemm & experts-4bit", first and third bullets; GitHub profile
pjordanandrsn, grouped-nf4-gemm bullets). The experts of one layer are a
single fused 3-D parameter (Jordan Anderson, jordananderson.work,
experts4bit-qlora entry, first bullet), here ``W[E, N, K]`` with
``Y = X @ W[e].T``.

What the pages leave open, and the reading taken:

* Codebook values: not printed. Reading: the NormalFloat-4 construction of
  the QLoRA paper (Dettmers et al., 2023, section 3, "4-bit NormalFloat"):
  8 positive quantiles of N(0,1) and 7 negative ones taken from the same
  offset, plus an exact zero, normalised so the extremes are -1 and +1, then
  stored as float32.
* Block size 64 along K with a float32 absmax per block (the workload
  definitions); blocks are consecutive elements of the row-major flatten of
  ``[E, N, K]``, so with K % 64 == 0 a block never straddles a row.
* Rounding: x = w / absmax in float64, the code is the nearest codebook
  value, ties go to the lower index. An all-zero block stores absmax 0 and
  code 7 (the exact zero).
* Nibble order: element 2i sits in the high nibble of byte i (bitsandbytes).
* Double quantization (NF4_DQ): linear symmetric int8 absmax with one float32
  scale per 256 consecutive blocks: scale2 = fp32(max/127),
  q8 = clip(rint_half_even(absmax / scale2), 0, 127), decoded absmax
  fp32(q8 * scale2). Codes are taken against the original absmax.
* Dequant: w' = fp32(c[q] * absmax), a single rounding of an exact product.

Parity: pinned (codebook by its defining quantile property; quantizer by an
independent midpoint search, round trips and hand-built blocks; dequant by the
closed form over all 256 byte values).
"""

from statistics import NormalDist

import numpy as np

BLOCK = 64          # values per absmax block
DQ_GROUP = 256      # blocks per float32 second-level scale (NF4_DQ)
ZERO_CODE = 7       # index of the exact 0.0 in the codebook

# Offset of the outermost quantile: midway between 1 - 1/30 and 1 - 1/32
# (QLoRA section 3; this keeps the extreme quantile finite).
NF4_OFFSET = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))


def codebook_f64():
    """The 16 NormalFloat-4 values in float64, ascending, before fp32 rounding.

    Positive half: the N(0,1) quantiles at 8 evenly spaced probabilities from
    NF4_OFFSET down to (but excluding) 1/2. Negative half: the mirrored
    quantiles at 7 evenly spaced probabilities over the same range. Add the
    exact zero, sort, divide by the largest value.
    """
    ppf = NormalDist().inv_cdf
    pos = [ppf(p) for p in np.linspace(NF4_OFFSET, 0.5, 9)[:-1]]
    neg = [-ppf(p) for p in np.linspace(NF4_OFFSET, 0.5, 8)[:-1]]
    vals = sorted(pos + neg + [0.0])
    top = max(vals)
    return np.array([v / top for v in vals], dtype=np.float64)


def codebook():
    """The NF4 codebook as stored and used: float32, index = 4-bit code."""
    return codebook_f64().astype(np.float32)


def _blocks(w, block):
    w = np.asarray(w, dtype=np.float32)
    if w.shape[-1] % block:
        raise ValueError("last dimension %d is not a multiple of %d" % (w.shape[-1], block))
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")
    return w.reshape(-1, block)


def block_absmax(w):
    """Exact float32 max |w| over each 64-value block, flat block order."""
    b = _blocks(w, BLOCK)
    return np.abs(b).max(axis=1).astype(np.float32)


def encode_codes(w, absmax):
    """NF4 codes (uint8 0..15, one per value) of w against per-block absmax.

    The code of each value is the index of the codebook entry nearest to
    w / absmax (float64), the lower index on an exact tie. Blocks whose absmax
    is 0 get the zero code.
    """
    b = _blocks(w, BLOCK).astype(np.float64)
    a = np.asarray(absmax, dtype=np.float32).astype(np.float64).reshape(-1)
    if a.shape[0] != b.shape[0]:
        raise ValueError("one absmax per block required")
    cb = codebook().astype(np.float64)
    codes = np.full(b.shape, ZERO_CODE, dtype=np.uint8)
    step = 1 << 14                               # blocks per slice (bounds memory)
    for s in range(0, b.shape[0], step):
        bs, as_ = b[s:s + step], a[s:s + step]
        nz = as_ > 0
        x = bs[nz] / as_[nz, None]
        dist = np.abs(x[..., None] - cb)         # [blocks, 64, 16]
        sub = codes[s:s + step]
        sub[nz] = np.argmin(dist, axis=-1)       # first minimum = lower index
    return codes.reshape(-1)


def pack(codes):
    """Two codes per byte, element 2i in the high nibble (bitsandbytes order)."""
    q = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if q.size % 2:
        raise ValueError("odd number of codes")
    return ((q[0::2] << 4) | q[1::2]).astype(np.uint8)


def unpack(packed):
    """Inverse of pack: byte i -> (high nibble, low nibble) = (code 2i, code 2i+1)."""
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 0x0F
    return out


def quantize(w):
    """NF4-quantize W[..., K] (K % 64 == 0).

    Returns (codes_packed uint8 [..., K/2], absmax float32 [..., K/64]).
    """
    w = np.asarray(w, dtype=np.float32)
    a = block_absmax(w)
    q = encode_codes(w, a)
    lead = w.shape[:-1]
    kk = w.shape[-1]
    return pack(q).reshape(lead + (kk // 2,)), a.reshape(lead + (kk // BLOCK,))


def double_quantize_absmax(absmax):
    """Second-level quantization of a flat float32 absmax array.

    Groups of 256 consecutive blocks (the last group may be shorter) share one
    float32 scale2 = fp32(group max / 127) (float64 division, one rounding);
    each absmax becomes q8 = clip(rint_half_even(absmax / scale2), 0, 127) as
    int8, or 0 when scale2 is 0.
    Returns (q8 int8 [n], scale2 float32 [ceil(n / 256)]).
    """
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    n = a.size
    ng = -(-n // DQ_GROUP)
    q8 = np.zeros(n, dtype=np.int8)
    s2 = np.zeros(ng, dtype=np.float32)
    for g in range(ng):
        seg = a[g * DQ_GROUP:(g + 1) * DQ_GROUP].astype(np.float64)
        s = np.float32(seg.max() / 127.0)
        s2[g] = s
        if s > 0:
            r = np.rint(seg / np.float64(s))      # numpy rint: half to even
            q8[g * DQ_GROUP:(g + 1) * DQ_GROUP] = np.clip(r, 0, 127).astype(np.int8)
    return q8, s2


def dq_absmax(q8, scale2):
    """Decoded absmax of NF4_DQ: fp32(q8 * scale2[block // 256])."""
    q = np.asarray(q8, dtype=np.int8).reshape(-1).astype(np.float64)
    s = np.asarray(scale2, dtype=np.float32).astype(np.float64)
    g = np.arange(q.size) // DQ_GROUP
    return (q * s[g]).astype(np.float32)


def quantize_dq(w):
    """NF4 with double-quantized absmax.

    Returns (codes_packed uint8 [..., K/2], q8 int8 [..., K/64],
    scale2 float32 [ceil(blocks / 256)]). Codes use the original absmax.
    """
    w = np.asarray(w, dtype=np.float32)
    packed, a = quantize(w)
    q8, s2 = double_quantize_absmax(a.reshape(-1))
    return packed, q8.reshape(a.shape), s2


def dequantize(packed, absmax, K):
    """Decode NF4 bytes to float32: w' = fp32(c[q] * absmax[block]).

    packed uint8 [..., K/2], absmax float32 [..., K/64] (already decoded for
    NF4_DQ, see dq_absmax). The float64 product of two float32 values is
    exact, so the single cast to float32 is the one correctly rounded product.
    """
    p = np.asarray(packed, dtype=np.uint8)
    lead = p.shape[:-1]
    q = unpack(p).reshape(-1, BLOCK)
    a = np.asarray(absmax, dtype=np.float32).reshape(-1).astype(np.float64)
    cb = codebook().astype(np.float64)
    w = (cb[q] * a[:, None]).astype(np.float32)
    return w.reshape(lead + (K,))
