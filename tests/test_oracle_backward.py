"""Pins of the oracle's input gradient through the grouped GEMM.

* the adjoint identity <dA[p], A[p]> = <dY[p], Y[p]> per routed row, with Y
  from the forward oracle (itself pinned): a wrong expert, a transposed
  weight or a dropped scale breaks it on a non-square N x K;
* the same identity per token for the sum over a token's routed copies;
* a one-hot gradient row returns one row of the dequantized weights;
* a brute-force triple loop that decodes each nibble by hand;
* a closed form: MXFP4 weights that are all 1.0 turn dA into row sums of dY;
* dropped rows stay NaN, empty experts are skipped;
* a negative control: one flipped weight byte must break the identity.
"""

import numpy as np
import pytest

import synth
from oracle import backward, grouped_gemm, mxfp4, nf4, routing


def pack(fmt, w):
    if fmt == "nf4":
        c, s = nf4.quantize(w)
        return c, s, None
    if fmt == "nf4_dq":
        return nf4.quantize_dq(w)
    c, s = mxfp4.quantize(w)
    return c, s, None


def case(fmt, E, N, K, T, k, seed, bad=False):
    g = np.random.default_rng([seed, E, N, K, T, k])
    w = (g.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    codes, scales, scales2 = pack(fmt, w)
    ids = g.integers(0, E, size=(T, k)).astype(np.int32)     # duplicates allowed
    if bad and T:
        ids[0, 0] = E                                        # dropped assignment
    r = routing.route(ids, E)
    rows = T * k
    A = synth.f32_to_bf16_bits(g.standard_normal((rows, K)).astype(np.float32))
    dY = synth.f32_to_bf16_bits(g.standard_normal((rows, N)).astype(np.float32))
    return codes, scales, scales2, r, A, dY


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
def test_adjoint_identity_per_row(fmt):
    E, N, K, T, k = 5, 24, 192, 9, 3
    codes, scales, scales2, r, A, dY = case(fmt, E, N, K, T, k, 1, bad=True)
    Y = grouped_gemm.grouped_gemm(fmt, codes, scales, scales2, A, 0, r["offsets"], r["perm"], k, N, K)
    dA = backward.grouped_gemm_dx(fmt, codes, scales, scales2, dY, r["offsets"], N, K)
    Af = grouped_gemm.bf16_bits_to_f64(A)
    dYf = grouped_gemm.bf16_bits_to_f64(dY)
    nv = int(r["offsets"][-1])
    assert nv == T * k - 1
    for p in range(nv):
        lhs = float(dA[p] @ Af[p])
        rhs = float(dYf[p] @ Y[p])
        assert abs(lhs - rhs) <= 1e-12 * (np.abs(dA[p]) @ np.abs(Af[p])), (p, lhs, rhs)
    assert np.all(np.isnan(dA[nv:]))


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_token_sum_adjoint(fmt):
    """Gathered forward: Y[p] = W'[e] X[perm[p] // k]; then for each token
    <dX[t], X[t]> equals the sum of <dY[p], Y[p]> over its routed copies."""
    E, N, K, T, k = 4, 40, 128, 7, 2
    codes, scales, scales2, r, _, dY = case(fmt, E, N, K, T, k, 2, bad=True)
    g = np.random.default_rng(5)
    X = synth.f32_to_bf16_bits(g.standard_normal((T, K)).astype(np.float32))
    Y = grouped_gemm.grouped_gemm(fmt, codes, scales, scales2, X, 1, r["offsets"], r["perm"], k, N, K)
    dA = backward.grouped_gemm_dx(fmt, codes, scales, scales2, dY, r["offsets"], N, K)
    dX = backward.token_grad(dA, r["inv"], T, k)
    Xf = grouped_gemm.bf16_bits_to_f64(X)
    dYf = grouped_gemm.bf16_bits_to_f64(dY)
    inv = r["inv"].reshape(T, k)
    assert inv[0, 0] == -1
    for t in range(T):
        rhs = sum(float(dYf[p] @ Y[p]) for p in inv[t] if p >= 0)
        lhs = float(dX[t] @ Xf[t])
        assert abs(lhs - rhs) <= 1e-12 * (np.abs(dX[t]) @ np.abs(Xf[t]) + 1e-300), (t, lhs, rhs)
    # token 0 lost its first copy: only the second one contributes
    assert np.array_equal(dX[0], dA[inv[0, 1]])


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
def test_one_hot_gradient_row_selects_weight_row(fmt):
    E, N, K = 3, 16, 128
    g = np.random.default_rng(7)
    w = (g.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    codes, scales, scales2 = pack(fmt, w)
    ids = np.array([[2], [0], [2]], dtype=np.int32)
    r = routing.route(ids, E)              # rows: p0 -> e0, p1, p2 -> e2
    dY = np.zeros((3, N), dtype=np.float32)
    n_of = {0: 5, 1: 11, 2: 0}
    for p, n in n_of.items():
        dY[p, n] = 1.0
    dA = backward.grouped_gemm_dx(fmt, codes, scales, scales2, synth.f32_to_bf16_bits(dY), r["offsets"], N, K)
    for p, e in [(0, 0), (1, 2), (2, 2)]:
        n = n_of[p]
        if fmt == "nf4":
            row = nf4.dequantize(codes[e, n], scales[e, n], K)
        elif fmt == "mxfp4":
            row = mxfp4.dequantize(codes[e, n], scales[e, n], K)
        else:
            nb = K // nf4.BLOCK
            blk = (e * N + n) * nb + np.arange(nb)          # flat block index of row n
            a = (np.asarray(scales).reshape(-1)[blk].astype(np.float64)
                 * scales2[blk // nf4.DQ_GROUP].astype(np.float64)).astype(np.float32)
            row = nf4.dequantize(codes[e, n], a, K)
        assert np.array_equal(dA[p], row.astype(np.float64)), (fmt, p)


def test_brute_force_triple_loop():
    E, N, K = 2, 5, 64
    g = np.random.default_rng(11)
    w = (g.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    codes, absmax = nf4.quantize(w)
    ids = np.array([[1, 0], [1, 1], [0, 1]], dtype=np.int32)
    r = routing.route(ids, E)
    dY = synth.f32_to_bf16_bits(g.standard_normal((6, N)).astype(np.float32))
    dA = backward.grouped_gemm_dx("nf4", codes, absmax, None, dY, r["offsets"], N, K)
    table = [float(v) for v in nf4.codebook()]
    dYf = (dY.astype(np.uint32) << 16).view(np.float32)
    for e in range(E):
        for p in range(int(r["offsets"][e]), int(r["offsets"][e + 1])):
            for kk in range(K):
                s = 0.0
                for n in range(N):
                    byte = int(codes[e, n, kk // 2])
                    q = (byte >> 4) if kk % 2 == 0 else (byte & 15)       # element 2i: high nibble
                    wv = float(np.float32(table[q] * float(absmax[e, n, kk // 64])))
                    s += float(dYf[p, n]) * wv
                assert abs(dA[p, kk] - s) <= 1e-13 * max(1.0, abs(s)), (e, p, kk)


def test_mxfp4_all_ones_gives_row_sums():
    """e2m1 code 2 is 1.0 and e8m0 127 is 2^0: every weight is exactly 1, so
    dA[p, :] is the (exact, small-integer) sum of dY[p, :] in every column."""
    E, N, K = 3, 20, 64
    codes = np.full((E, N, K // 2), 0x22, dtype=np.uint8)
    scales = np.full((E, N, K // 32), 127, dtype=np.uint8)
    ids = np.array([[0, 2], [2, 2]], dtype=np.int32)
    r = routing.route(ids, E)
    g = np.random.default_rng(3)
    dYi = g.integers(-4, 5, size=(4, N)).astype(np.float32)
    dA = backward.grouped_gemm_dx("mxfp4", codes, scales, None, synth.f32_to_bf16_bits(dYi),
                                  r["offsets"], N, K)
    for p in range(4):
        assert np.array_equal(dA[p], np.full(K, dYi[p].sum()))


def test_empty_experts_and_no_rows():
    E, N, K = 6, 8, 64
    g = np.random.default_rng(4)
    w = (g.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    codes, absmax = nf4.quantize(w)
    r = routing.route(np.array([[3], [3]], dtype=np.int32), E)       # only expert 3 active
    dY = synth.f32_to_bf16_bits(g.standard_normal((2, N)).astype(np.float32))
    dA = backward.grouped_gemm_dx("nf4", codes, absmax, None, dY, r["offsets"], N, K)
    W3 = nf4.dequantize(codes[3], absmax[3], K).astype(np.float64)
    assert np.array_equal(dA, grouped_gemm.bf16_bits_to_f64(dY) @ W3)
    r0 = routing.route(np.zeros((0, 1), dtype=np.int32), E)
    assert backward.grouped_gemm_dx("nf4", codes, absmax, None, np.zeros((0, N), np.uint16),
                                    r0["offsets"], N, K).shape == (0, K)


def test_flipped_weight_byte_breaks_identity():
    """Negative control: the identity above can fail. Flip one packed byte of
    an active expert in the copy the gradient reads; the forward keeps the
    original bytes, and the identity must break on the rows of that expert."""
    fmt, E, N, K, T, k = "nf4", 3, 24, 128, 6, 2
    codes, scales, scales2, r, A, dY = case(fmt, E, N, K, T, k, 9)
    Y = grouped_gemm.grouped_gemm(fmt, codes, scales, scales2, A, 0, r["offsets"], r["perm"], k, N, K)
    e = int(r["active"][0])
    bad = codes.copy()
    bad[e, 3, 10] ^= 0x5A
    dA = backward.grouped_gemm_dx(fmt, bad, scales, scales2, dY, r["offsets"], N, K)
    Af = grouped_gemm.bf16_bits_to_f64(A)
    dYf = grouped_gemm.bf16_bits_to_f64(dY)
    lo, hi = int(r["offsets"][e]), int(r["offsets"][e + 1])
    broken = [abs(float(dA[p] @ Af[p]) - float(dYf[p] @ Y[p])) > 1e-9 for p in range(lo, hi)]
    assert hi > lo and all(broken)


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
def test_sampled_entries_and_column_blocks(fmt):
    """The column-block decoder returns the same float32 weights as the whole
    expert's decode, and the sampled entries equal the full gradient's."""
    E, N, K, T, k = 4, 40, 256, 10, 3
    codes, scales, scales2, r, _, dY = case(fmt, E, N, K, T, k, 13)
    for e in range(E):
        W = grouped_gemm.dequant_expert(fmt, codes, scales, scales2, e, N, K)
        for c0 in (0, 64, 192):
            assert np.array_equal(backward.dequant_cols(fmt, codes, scales, scales2, e, c0, 64, N, K),
                                  W[:, c0:c0 + 64])
    dA = backward.grouped_gemm_dx(fmt, codes, scales, scales2, dY, r["offsets"], N, K)
    g = np.random.default_rng(2)
    nv = int(r["offsets"][-1])
    p = g.integers(0, nv, size=200)
    j = g.integers(0, K, size=200)
    got = backward.grouped_gemm_dx_entries(fmt, codes, scales, scales2, dY, r["offsets"], N, K, p, j)
    assert np.allclose(got, dA[p, j], rtol=1e-12, atol=1e-14)
