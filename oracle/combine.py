"""Weighted top-k combine of expert rows back to tokens (oracle).

TEST INFRASTRUCTURE (see the package docstring): never imported by the GPU path.

The pages imply it only (a mixture-of-experts layer behind a real router,
Jordan Anderson, jordananderson-pages.pages.dev, section "grouped-nf4-gemm &
experts-4bit", first bullet). Reading: the standard top-k mixture

    out[t, :] = sum over j = 0..k-1 of w[t, j] * Y[inv[t*k + j], :]

in float64, j ascending; an assignment with inv = -1 (dropped id)
contributes nothing.

Parity: pinned (k = 1, w = 1 copies rows exactly; linear in w).
"""

import numpy as np


def combine(Y, inv, topk_w, T, k):
    """out float64 [T, N] from Y [T*k, N] (permuted rows), inv [T*k], topk_w [T, k]."""
    Y = np.asarray(Y, dtype=np.float64)
    inv = np.asarray(inv).reshape(-1)
    w = np.asarray(topk_w, dtype=np.float32).astype(np.float64).reshape(T, k)
    out = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            p = int(inv[t * k + j])
            if p >= 0:
                out[t] += w[t, j] * Y[p]
    return out
