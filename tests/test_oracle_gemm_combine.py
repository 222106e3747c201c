"""Pins of the oracle's grouped GEMM and combine.

* per-assignment recomputation without any routing (catches a wrong segment,
  a wrong gather index or a transposed weight, on a non-square N x K);
* brute-force sums on tiny inputs;
* one-hot rows that select single weights exactly;
* integer-valued MXFP4 cases that are exact in floating point;
* combine against the direct per-token mixture and its k = 1 copy case;
* a byte-flip negative control: flipping one packed byte must break the
  comparison, so the bar can fail.
"""

import numpy as np
import pytest

import synth
from oracle import combine, grouped_gemm, mxfp4, nf4, routing

from .tolerance import errors, within


def tiny_layer(fmt="nf4", E=4, N=24, K=128, T=6, k=2, seed=0):
    g = np.random.default_rng(seed)
    w = (g.standard_normal((E, N, K)) * 0.02).astype(np.float32)
    if fmt == "nf4":
        codes, scales = nf4.quantize(w)
        scales2 = None
    elif fmt == "nf4_dq":
        codes, scales, scales2 = nf4.quantize_dq(w)
    else:
        codes, scales = mxfp4.quantize(w)
        scales2 = None
    X = synth.f32_to_bf16_bits(g.standard_normal((T, K)).astype(np.float32))
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    tw = g.random((T, k)).astype(np.float32)
    return codes, scales, scales2, X, ids, tw


def test_per_assignment_recomputation():
    for fmt in ("nf4", "nf4_dq", "mxfp4"):
        E, N, K, T, k = 4, 24, 128, 6, 2
        codes, scales, scales2, X, ids, tw = tiny_layer(fmt, E, N, K, T, k)
        r = routing.route(ids, E)
        Y = grouped_gemm.grouped_gemm(fmt, codes, scales, scales2, X, 1, r["offsets"], r["perm"], k, N, K)
        Xf = grouped_gemm.bf16_bits_to_f64(X)
        for t in range(T):
            for j in range(k):
                e = ids[t, j]
                W = grouped_gemm.dequant_expert(fmt, codes, scales, scales2, e, N, K).astype(np.float64)
                ref = W @ Xf[t]                      # [N]: W is [N, K]
                assert np.array_equal(Y[r["inv"][t * k + j]], ref) or np.allclose(
                    Y[r["inv"][t * k + j]], ref, rtol=1e-12, atol=1e-15)


def test_brute_force_sum():
    E, N, K, T, k = 3, 5, 64, 4, 2
    codes, scales, scales2, X, ids, tw = tiny_layer("nf4", E, N, K, T, k, seed=3)
    r = routing.route(ids, E)
    Y = grouped_gemm.grouped_gemm("nf4", codes, scales, None, X, 1, r["offsets"], r["perm"], k, N, K)
    Xf = grouped_gemm.bf16_bits_to_f64(X)
    c = nf4.codebook()
    for p in range(T * k):
        f = int(r["perm"][p])
        t, e = f // k, int(ids.reshape(-1)[f])
        for n in range(N):
            s = 0.0
            for kk in range(K):
                byte = int(codes[e, n, kk // 2])
                q = (byte >> 4) if kk % 2 == 0 else (byte & 15)
                w = float(np.float32(c[q]) * np.float32(scales[e, n, kk // 64]))
                s += Xf[t, kk] * w
            assert abs(Y[p, n] - s) <= 1e-12 * max(1.0, abs(s))


def test_one_hot_rows_select_weights():
    E, N, K, T, k = 4, 24, 128, 6, 2
    codes, scales, scales2, _, ids, _ = tiny_layer("nf4", E, N, K, T, k, seed=1)
    X = np.zeros((T, K), dtype=np.uint16)
    cols = [0, 5, 63, 64, 100, 127]
    for t in range(T):
        X[t, cols[t]] = 0x3F80                        # bf16 1.0
    r = routing.route(ids, E)
    Y = grouped_gemm.grouped_gemm("nf4", codes, scales, None, X, 1, r["offsets"], r["perm"], k, N, K)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            W = nf4.dequantize(codes[e], scales[e], K)
            assert np.array_equal(Y[r["inv"][t * k + j]], W[:, cols[t]].astype(np.float64))


def test_integer_valued_mxfp4_is_exact():
    E, N, K, T, k = 2, 8, 64, 3, 1
    g = np.random.default_rng(9)
    q = g.integers(0, 16, size=(E, N, K)).astype(np.uint8)
    codes = mxfp4.pack(q.reshape(-1)).reshape(E, N, K // 2)
    scales = np.full((E, N, K // 32), 128, dtype=np.uint8)      # scale 2: values are integers
    X = synth.f32_to_bf16_bits(g.integers(-8, 9, size=(T, K)).astype(np.float32))
    ids = np.array([[0], [1], [0]], dtype=np.int32)
    r = routing.route(ids, E)
    Y = grouped_gemm.grouped_gemm("mxfp4", codes, scales, None, X, 1, r["offsets"], r["perm"], k, N, K)
    vals = np.array([mxfp4.e2m1_value(c) * 2 for c in range(16)])
    for t in range(T):
        e = ids[t, 0]
        xi = grouped_gemm.bf16_bits_to_f64(X)[t].astype(np.int64)
        ref = [int(sum(int(vals[q[e, n, kk]]) * int(xi[kk]) for kk in range(K))) for n in range(N)]
        assert Y[r["inv"][t]].tolist() == [float(v) for v in ref]


def test_permuted_input_projection():
    E, N, K, T, k = 4, 16, 64, 5, 2
    codes, scales, scales2, _, ids, _ = tiny_layer("nf4", E, N, K, T, k, seed=4)
    g = np.random.default_rng(4)
    Xp = synth.f32_to_bf16_bits(g.standard_normal((T * k, K)).astype(np.float32))
    r = routing.route(ids, E)
    Y = grouped_gemm.grouped_gemm("nf4", codes, scales, None, Xp, 0, r["offsets"], r["perm"], k, N, K)
    Xf = grouped_gemm.bf16_bits_to_f64(Xp)
    for p in range(T * k):
        e = int(ids.reshape(-1)[r["perm"][p]])
        W = nf4.dequantize(codes[e], scales[e], K).astype(np.float64)
        assert np.allclose(Y[p], W @ Xf[p], rtol=1e-13, atol=1e-16)


def test_combine_direct_mixture():
    E, N, K, T, k = 4, 24, 128, 6, 2
    codes, scales, scales2, X, ids, tw = tiny_layer("nf4", E, N, K, T, k, seed=2)
    r = routing.route(ids, E)
    Y = grouped_gemm.grouped_gemm("nf4", codes, scales, None, X, 1, r["offsets"], r["perm"], k, N, K)
    out = combine.combine(Y, r["inv"], tw, T, k)
    Xf = grouped_gemm.bf16_bits_to_f64(X)
    for t in range(T):
        ref = np.zeros(N)
        for j in range(k):
            W = nf4.dequantize(codes[ids[t, j]], scales[ids[t, j]], K).astype(np.float64)
            ref += float(tw[t, j]) * (W @ Xf[t])
        assert np.allclose(out[t], ref, rtol=1e-12, atol=1e-15)


def test_combine_k1_copies_rows_and_drops_bad():
    Y = np.arange(12, dtype=np.float64).reshape(4, 3)
    inv = np.array([2, 0, -1, 1])
    out = combine.combine(Y, inv, np.ones((4, 1), dtype=np.float32), 4, 1)
    assert out.tolist() == [Y[2].tolist(), Y[0].tolist(), [0.0, 0.0, 0.0], Y[1].tolist()]


def test_byte_flip_negative_control():
    E, N, K, T, k = 4, 24, 128, 6, 2
    codes, scales, scales2, X, ids, tw = tiny_layer("nf4", E, N, K, T, k, seed=6)
    r = routing.route(ids, E)
    ref = grouped_gemm.grouped_gemm("nf4", codes, scales, None, X, 1, r["offsets"], r["perm"], k, N, K)
    same = grouped_gemm.grouped_gemm("nf4", codes, scales, None, X, 1, r["offsets"], r["perm"], k, N, K)
    assert within(same, ref)
    e_used = int(ids[0, 0])
    flipped = codes.copy()
    flipped[e_used, 3, 0] ^= 0xFF                    # one byte of a routed expert
    bad = grouped_gemm.grouped_gemm("nf4", flipped, scales, None, X, 1, r["offsets"], r["perm"], k, N, K)
    assert not within(bad, ref)
    max_rel, _ = errors(bad, ref)
    assert max_rel > 2e-2


@pytest.mark.parametrize("name,projname", [("olmoe", "down"), ("qwen30", "down"), ("gptoss", "down")])
def test_dequant_rows_matches_expert_rows(name, projname):
    """The row-subset dequant used by the full-size parity tests decodes
    exactly the rows the whole-expert dequant decodes (including the flat
    block index of the double-quantized absmax)."""
    cfg = synth.CONFIGS[name]
    proj = cfg.proj(projname)
    codes, scales, scales2 = synth.packed_weights(cfg, proj)
    E, N, K = cfg.E, proj.N, proj.K
    for e in (0, E - 1):
        rows = np.array([0, 1, N // 2, N - 1])
        full = grouped_gemm.dequant_expert(cfg.fmt, codes, scales, scales2, e, N, K)
        part = grouped_gemm.dequant_rows(cfg.fmt, codes, scales, scales2, e, rows, N, K)
        assert np.array_equal(full[rows], part)


def test_packed_weights_are_seeded_and_in_range():
    cfg = synth.CONFIGS["qwen30"]
    proj = cfg.proj("down")
    a = synth.packed_weights(cfg, proj)
    b = synth.packed_weights(cfg, proj)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    codes, q8, s2 = a
    assert codes.shape == (cfg.E, proj.N, proj.K // 2) and codes.dtype == np.uint8
    assert q8.dtype == np.int8 and q8.min() >= 1
    assert s2.shape == (-(-(cfg.E * proj.N * (proj.K // 64)) // 256),)
    codes, e8, _ = synth.packed_weights(synth.CONFIGS["gptoss"], synth.CONFIGS["gptoss"].proj("down"))
    assert e8.min() >= 118 and e8.max() <= 124
