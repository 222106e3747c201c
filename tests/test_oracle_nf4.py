"""Pins of the oracle's NF4 encoding against facts that do not come from it.

* the codebook against the defining quantile property, evaluated with scipy's
  normal CDF (the oracle builds it with the stdlib inverse CDF);
* the nearest-code quantizer against an independent midpoint search;
* hand-built blocks whose codes follow from the construction alone;
* dequantization against float32 products over all 256 byte values;
* round trips, the double-quantized absmax, and the reconstruction-error
  ordering NF4 (block 64) < MXFP4 (block 32) on N(0, 0.02) weights (the
  pages keep such an ordering test-pinned: Jordan Anderson,
  jordananderson.work, experts4bit-qlora entry, second bullet).
"""

import numpy as np
import pytest
from scipy.special import ndtr, ndtri

from oracle import mxfp4, nf4
from synth import W_STD


def test_codebook_structure():
    c = nf4.codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert c[0] == -1.0 and c[15] == 1.0 and c[7] == 0.0
    assert np.all(np.diff(c) > 0)
    assert (c < 0).sum() == 7 and (c > 0).sum() == 8


def test_codebook_quantile_property():
    # Un-normalised, the positive values are N(0,1) quantiles at 8 evenly
    # spaced probabilities from 0.9677083 to 1/2 (exclusive), the negative
    # ones the mirrored quantiles at 7 such probabilities.
    offset = 0.96770833333333333
    top = ndtri(offset)
    c = nf4.codebook().astype(np.float64)
    pos = c[8:][::-1]                     # 1.0 first
    neg = -c[:7]                          # 1.0 first
    p_pos = np.array([offset - i * (offset - 0.5) / 8 for i in range(8)])
    p_neg = np.array([offset - i * (offset - 0.5) / 7 for i in range(7)])
    # fp32 storage perturbs each value by <= 2^-24 relative
    assert np.allclose(ndtr(pos * top), p_pos, rtol=0, atol=2e-7)
    assert np.allclose(ndtr(neg * top), p_neg, rtol=0, atol=2e-7)


def _midpoint_codes(w, a):
    """Independent formulation: count of codebook midpoints strictly below x."""
    c = nf4.codebook().astype(np.float64)
    mids = (c[:-1] + c[1:]) / 2.0          # exact in float64
    x = w.astype(np.float64) / a.astype(np.float64)
    return np.searchsorted(mids, x, side="left").astype(np.uint8)


def test_quantizer_matches_midpoint_search():
    g = np.random.default_rng(7)
    w = (g.standard_normal((64, 256)) * W_STD).astype(np.float32)
    w[3, :64] = 0.0                        # an all-zero block
    w[5, 64:128] = 1e-40                   # a subnormal block
    packed, a = nf4.quantize(w)
    codes = nf4.unpack(packed).reshape(-1, 64)
    ab = a.reshape(-1)
    for b in range(codes.shape[0]):
        blk = w.reshape(-1, 64)[b]
        if ab[b] == 0:
            assert np.all(codes[b] == 7)
        else:
            assert np.array_equal(codes[b], _midpoint_codes(blk, np.full(64, ab[b])))


def test_ties_go_to_the_lower_code():
    c = nf4.codebook().astype(np.float64)
    mids = (c[:-1] + c[1:]) / 2.0
    exact = [i for i in range(15) if float(np.float32(mids[i])) == mids[i]]
    assert exact, "expected some midpoints representable in float32"
    blk = np.zeros(64, dtype=np.float32)
    blk[0] = 1.0                           # absmax 1: x = w exactly
    for j, i in enumerate(exact):
        blk[1 + j] = np.float32(mids[i])
    packed, a = nf4.quantize(blk[None, :])
    q = nf4.unpack(packed)
    assert a[0, 0] == 1.0
    for j, i in enumerate(exact):
        assert q[1 + j] == i, (i, q[1 + j])


def test_hand_built_blocks_and_nibble_order():
    blk = np.zeros((1, 64), dtype=np.float32)
    blk[0, 0] = 0.5                        # the absmax, positive -> code 15
    blk[0, 2] = -0.5                       # -absmax -> code 0
    packed, a = nf4.quantize(blk)
    assert a[0, 0] == 0.5
    assert packed[0, 0] == 0xF7            # element 0 high nibble, element 1 (zero) low
    assert packed[0, 1] == 0x07
    assert np.all(packed[0, 2:] == 0x77)
    zero = np.zeros((2, 128), dtype=np.float32)
    pz, az = nf4.quantize(zero)
    assert np.all(az == 0) and np.all(pz == 0x77)
    assert np.all(nf4.dequantize(pz, az, 128) == 0)


ABSMAX_SET = np.array([0.0, 1.0, 2.0 ** -20, 0.0371, 3.5e-39, 1e-45,
                       np.finfo(np.float32).max, 0.06], dtype=np.float32)


@pytest.mark.parametrize("a", ABSMAX_SET)
def test_dequant_all_256_bytes(a):
    c = nf4.codebook()
    packed = np.arange(256, dtype=np.uint8).repeat(32).reshape(-1, 32)[:, :32]
    packed = packed.reshape(-1)[:32 * 256].reshape(256, 32)  # one block per byte value
    absmax = np.full((256, 1), a, dtype=np.float32)
    with np.errstate(over="ignore"):
        got = nf4.dequantize(packed, absmax, 64)
        hi = np.float32(c[np.arange(256) >> 4]) * np.float32(a)   # float32 products
        lo = np.float32(c[np.arange(256) & 15]) * np.float32(a)
    assert np.array_equal(got[:, 0].view(np.uint32), hi.astype(np.float32).view(np.uint32))
    assert np.array_equal(got[:, 1].view(np.uint32), lo.astype(np.float32).view(np.uint32))


def test_round_trip():
    g = np.random.default_rng(11)
    w = (g.standard_normal((16, 512)) * W_STD).astype(np.float32)
    packed, a = nf4.quantize(w)
    w2 = nf4.dequantize(packed, a, 512)
    packed2, a2 = nf4.quantize(w2)
    assert np.array_equal(packed, packed2)
    assert np.array_equal(a, a2)


def test_every_code_round_trips():
    c = nf4.codebook()
    for a in [1.0, 0.02, 3.0e-3, 1024.0]:
        blk = np.zeros(64, dtype=np.float32)
        blk[:16] = c * np.float32(a)
        blk[16:] = np.float32(a)
        packed, aa = nf4.quantize(blk[None, :])
        assert aa[0, 0] == np.float32(a)
        assert np.array_equal(nf4.unpack(packed)[:16], np.arange(16, dtype=np.uint8))


def test_double_quantized_absmax():
    g = np.random.default_rng(5)
    w = (g.standard_normal((40, 64 * 20)) * W_STD).astype(np.float32)   # 800 blocks: 3 full groups + 1 partial
    packed, q8, s2 = nf4.quantize_dq(w)
    packed_plain, a = nf4.quantize(w)
    assert np.array_equal(packed, packed_plain)          # codes use the original absmax
    af = a.reshape(-1)
    q = q8.reshape(-1)
    assert s2.shape == (4,)
    for gi in range(4):
        seg = af[gi * 256:(gi + 1) * 256]
        assert s2[gi] == np.float32(float(seg.max()) / 127.0)
        assert q[gi * 256:(gi + 1) * 256].max() == 127
    assert q.min() >= 0
    dec = nf4.dq_absmax(q8, s2)
    step = s2[np.arange(af.size) // 256].astype(np.float64)
    assert np.all(np.abs(dec.astype(np.float64) - af) <= 0.5 * step * (1 + 1e-6))
    # round trip: requantizing the decoded weights reproduces codes and q8
    w2 = nf4.dequantize(packed, dec.reshape(a.shape), w.shape[1])
    p2, q82, s22 = nf4.quantize_dq(w2)
    assert np.array_equal(p2, packed)
    assert np.array_equal(q82, q8)
    ulp = np.spacing(s2)
    assert np.all(np.abs(s22.astype(np.float64) - s2) <= ulp)


def test_reconstruction_error_ordering():
    g = np.random.default_rng(3)
    w = (g.standard_normal((64, 2048)) * W_STD).astype(np.float32)
    pn, an = nf4.quantize(w)
    pm, sm = mxfp4.quantize(w)
    rel = lambda r: float(np.sqrt(np.mean((r.astype(np.float64) - w) ** 2)) / np.sqrt(np.mean(w.astype(np.float64) ** 2)))
    e_nf4 = rel(nf4.dequantize(pn, an, 2048))
    e_mx = rel(mxfp4.dequantize(pm, sm, 2048))
    assert e_nf4 < e_mx
    assert 0.08 < e_nf4 < 0.10 and 0.10 < e_mx < 0.13
