"""Comparison bars for floating-point outputs of the grouped GEMM and combine.

Per call (one projection, one workload, one T), over every element of that
call's output compared against the float64 oracle:

* max |got - ref| <= 1e-2 * rms(ref)
* ||got - ref||_F / ||ref||_F <= 2e-3

Integer and byte outputs (routing, dequantized weights) are compared exactly.
"""

import numpy as np

MAX_REL_RMS = 1e-2
FROB_REL = 2e-3


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
