"""Comparison bars for floating-point outputs of the grouped GEMM and combine.

Per call (one projection, one workload, one T), over every element of that
call's output compared against the float64 oracle:

* max |got - ref| <= 1e-2 * rms(ref)
* ||got - ref||_F / ||ref||_F <= 2e-3

Integer and byte outputs (routing, dequantized weights) are compared exactly.

A whole FFN layer chains two GEMM calls through a bf16 activation H (route
-> gate_up -> SwiGLU -> down -> combine), and the oracle chains its own
float64 results. Three errors then reach the layer output, each bounded by
the per-call bars: the gate_up call's error carried through SwiGLU, the
bf16 roundings of H that this error moves across a rounding boundary (one
bf16 step, 2^-8 relative, on a share of the elements), and the down call's
own error. The layer bar adds the three per-call bars:

* max |got - ref| <= 3e-2 * rms(ref)
* ||got - ref||_F / ||ref||_F <= 6e-3

The SwiGLU output H = bf16(silu(gate) * up) of the first projection is
itself compared with the oracle's H (bf16 of the float64 value formed from
the oracle's float64 gate_up output). H is heavy-tailed (a product of two
nearly Gaussian values), so a bar relative to rms(H) is set by its few
largest elements. Its error has two parts: the gate_up call's error carried
through silu(g) * u, at most about (|u| + |silu(g)|) * 1e-2 * rms(Y) <=
2^-8 max|H| at the largest elements (|g|, |u| near 5 rms(Y)), and the two
roundings to bf16, together at most one bf16 step, 2^-8 |H|. The bar is
twice their sum, against the largest element, with the layer's Frobenius
bar for the bulk:

* max |got - ref| <= 2^-6 * max|ref|
* ||got - ref||_F / ||ref||_F <= 6e-3

The input gradient through the frozen experts (gnf4_grouped_gemm_dx) feeds
each dequantized float32 weight to the MFMA as bf16 hi + lo; the part left
out is below 2^-16 of each weight (RNE twice: 2^-9 then 2^-9 of that), and
the float32 accumulation adds about 2^-24 sqrt(N) relative. Its own bar,
which a dropped lo term (a 2^-9 relative error per weight, about 1.6e-3
relative Frobenius) fails:

* max |got - ref| <= 1e-4 * rms(ref)
* ||got - ref||_F / ||ref||_F <= 2e-5
"""

import numpy as np

MAX_REL_RMS = 1e-2
FROB_REL = 2e-3
LAYER_MAX_REL_RMS = 3 * MAX_REL_RMS
LAYER_FROB_REL = 3 * FROB_REL
DX_MAX_REL_RMS = 1e-4
DX_FROB_REL = 2e-5


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert ref.size > 0, "comparing empty outputs proves nothing"
    assert np.all(np.isfinite(got)), "non-finite values in the result under test"
    d = got - ref
    rms = float(np.sqrt(np.mean(ref * ref)))
    fro = float(np.linalg.norm(ref))
    max_rel = float(np.max(np.abs(d))) / rms if rms > 0 else float(np.max(np.abs(d)))
    frob = float(np.linalg.norm(d)) / fro if fro > 0 else float(np.linalg.norm(d))
    return max_rel, frob


def within(got, ref):
    max_rel, frob = errors(got, ref)
    return max_rel <= MAX_REL_RMS and frob <= FROB_REL


def assert_within(got, ref, what=""):
    max_rel, frob = errors(got, ref)
    assert max_rel <= MAX_REL_RMS and frob <= FROB_REL, (
        "%s: max|err|/rms = %.3e (bar %.0e), rel Frobenius = %.3e (bar %.0e)"
        % (what, max_rel, MAX_REL_RMS, frob, FROB_REL))
    return max_rel, frob


def assert_within_layer(got, ref, what=""):
    max_rel, frob = errors(got, ref)
    assert max_rel <= LAYER_MAX_REL_RMS and frob <= LAYER_FROB_REL, (
        "%s: max|err|/rms = %.3e (bar %.0e), rel Frobenius = %.3e (bar %.0e)"
        % (what, max_rel, LAYER_MAX_REL_RMS, frob, LAYER_FROB_REL))
    return max_rel, frob


H_MAX_REL_MAX = 2.0 ** -6


def assert_within_h(got, ref, what=""):
    """SwiGLU output H (as float values) against the oracle's bf16 H."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape and ref.size > 0, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite values in the result under test"
    peak = float(np.max(np.abs(ref)))
    max_rel = float(np.max(np.abs(got - ref))) / peak if peak > 0 else float(np.max(np.abs(got)))
    fro = float(np.linalg.norm(ref))
    frob = float(np.linalg.norm(got - ref)) / fro if fro > 0 else float(np.linalg.norm(got))
    assert max_rel <= H_MAX_REL_MAX and frob <= LAYER_FROB_REL, (
        "%s: max|err|/max|ref| = %.3e (bar %.2e), rel Frobenius = %.3e (bar %.0e)"
        % (what, max_rel, H_MAX_REL_MAX, frob, LAYER_FROB_REL))
    return max_rel, frob


def assert_within_dx(got, ref, what=""):
    max_rel, frob = errors(got, ref)
    assert max_rel <= DX_MAX_REL_RMS and frob <= DX_FROB_REL, (
        "%s: max|err|/rms = %.3e (bar %.0e), rel Frobenius = %.3e (bar %.0e)"
        % (what, max_rel, DX_MAX_REL_RMS, frob, DX_FROB_REL))
    return max_rel, frob
