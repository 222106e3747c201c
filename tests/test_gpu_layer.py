"""GPU parity of the layer steps either side of the grouped GEMM (router top-k
with softmax weights, SwiGLU) and of a whole FFN layer chained through the
C ABI: route_logits -> gate_up GEMM -> SwiGLU -> down GEMM -> combine."""

import numpy as np
import pytest
import torch

import synth
from oracle import combine as ocombine
from oracle import grouped_gemm as ogemm
from oracle import layer as olayer
from oracle import routing

from .gpu_util import bits_to_device, check_route, gnf4, oracle_pack, packed_to_device, say
from .tolerance import assert_within_h, assert_within_layer

pytestmark = pytest.mark.gpu


def run_route_logits(logits, k):
    g = gnf4()
    T, E = logits.shape
    r = g.route_logits(torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda(), k)
    torch.cuda.synchronize()
    ids_ref, w_ref = olayer.topk_softmax(logits, k)
    if T:
        assert np.array_equal(r["topk_ids"].cpu().numpy(), ids_ref), "topk ids"
        w = r["topk_w"].cpu().numpy()
        both_nan = np.isnan(w) & np.isnan(w_ref)
        assert np.array_equal(np.isnan(w), np.isnan(w_ref))
        assert np.array_equal(w[~both_nan], w_ref[~both_nan]), "topk weights"
    check_route(r, routing.route(ids_ref, E), T * k)
    return r


@pytest.mark.parametrize("name", ["tiny", "olmoe", "qwen30", "qwen235", "gptoss", "mixtral"])
def test_route_logits_workloads(name):
    cfg = synth.CONFIGS[name]
    for T in sorted(set(cfg.Ts) | {1}):
        say("route_logits", name, "T", T, "E", cfg.E, "k", cfg.k)
        run_route_logits(synth.router_logits(cfg, T).astype(np.float32), cfg.k)


@pytest.mark.parametrize("T,E,k", [(0, 8, 2), (1, 1, 1), (7, 64, 64), (33, 100, 7), (5, 1024, 64),
                                   (300, 129, 8), (70, 513, 3)])
def test_route_logits_shapes(T, E, k):
    g = np.random.default_rng([T, E, k])
    say("route_logits shape", T, E, k)
    run_route_logits(g.standard_normal((T, E)).astype(np.float32), k)


def test_route_logits_ties_nan_and_infinities():
    g = np.random.default_rng(21)
    logits = g.integers(-3, 4, size=(200, 40)).astype(np.float32)      # many ties
    logits[0, :] = np.nan
    logits[1, 5] = np.nan
    logits[2, :] = -np.inf
    logits[3, 7] = np.inf
    logits[4, :] = 0.0
    logits[5, ::3] = np.nan
    logits[6, :] = 0.0
    logits[6, ::2] = -0.0                   # -0 and +0 tie: lower id first
    logits[7, :] = -1.0
    logits[7, 1::4] = -0.0
    logits[7, 3::4] = 0.0
    say("route_logits ties/nan/inf")
    run_route_logits(logits, 5)


def swiglu_case(rows, I, seed):
    g = np.random.default_rng([rows, I, seed])
    Y = (g.standard_normal((rows, 2 * I)) * 3.0).astype(np.float32)
    flat = Y.reshape(-1)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 88.0, -88.0, 1e30, -1e30, 1e-40,
                        -1e-40, 3.4e38, -3.4e38], dtype=np.float32)
    pos = g.choice(flat.size, size=min(flat.size, 64), replace=False)
    flat[pos] = special[np.arange(pos.size) % special.size]
    return Y


@pytest.mark.parametrize("rows,I", [(1, 4), (8, 1024), (37, 768), (300, 2880), (5, 14336)])
def test_swiglu_matches_oracle(rows, I):
    g = gnf4()
    Y = swiglu_case(rows, I, 1)
    say("swiglu", rows, I)
    H = g.swiglu(torch.from_numpy(Y).cuda(), I).cpu().numpy().view(np.uint16)[:rows]
    H_ref = olayer.swiglu(Y, I)
    assert np.array_equal(H, H_ref), int((H != H_ref).sum())


def layer_case(E, d, I, T, k, seed):
    g = np.random.default_rng([E, d, I, T, k, seed])
    W1 = (g.standard_normal((E, 2 * I, d)) * 0.02).astype(np.float32)
    W2 = (g.standard_normal((E, d, I)) * 0.02).astype(np.float32)
    X = synth.f32_to_bf16_bits(g.standard_normal((T, d)).astype(np.float32))
    logits = g.standard_normal((T, E)).astype(np.float32)
    return W1, W2, X, logits


def ffn_oracle(fmt, packs, X, logits, k, d, I):
    (c1, s1, t1), (c2, s2, t2) = packs
    T, E = logits.shape
    ids, w = olayer.topk_softmax(logits, k)
    r = routing.route(ids, E)
    Y1 = ogemm.grouped_gemm(fmt, c1, s1, t1, X, 1, r["offsets"], r["perm"], k, 2 * I, d)
    H = olayer.swiglu(Y1, I)
    Y2 = ogemm.grouped_gemm(fmt, c2, s2, t2, H, 0, r["offsets"], r["perm"], k, d, I)
    return ocombine.combine(Y2, r["inv"], w, T, k), H


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
@pytest.mark.parametrize("T", [1, 5, 300])                 # GEMV (T*k <= 64) and MFMA paths
def test_ffn_layer_end_to_end(fmt, T, fused):
    gl = gnf4()
    E, d, I, k = 8, 256, 128, 2
    W1, W2, X, logits = layer_case(E, d, I, T, k, 2)
    packs = [oracle_pack(fmt, W1), oracle_pack(fmt, W2)]
    say("ffn layer", fmt, "T", T, "E", E, "d", d, "I", I, "k", k, "fused", fused)
    pw1 = packed_to_device(gl, fmt, *packs[0], E, 2 * I, d)
    pw2 = packed_to_device(gl, fmt, *packs[1], E, d, I)
    r = gl.route_logits(torch.from_numpy(logits).cuda(), k)
    if fused:
        H = gl.grouped_gemm_swiglu(pw1, bits_to_device(X), 1, r, T, k)
    else:
        Y1 = gl.grouped_gemm(pw1, bits_to_device(X), 1, r, T, k)
        H = gl.swiglu(Y1, I)
    Y2 = gl.grouped_gemm(pw2, H, 0, r, T, k)
    out = gl.combine(Y2, r["inv"], r["topk_w"], T, k)
    torch.cuda.synchronize()
    ref, H_ref = ffn_oracle(fmt, packs, X, logits, k, d, I)
    max_rel, frob = assert_within_layer(out.cpu().numpy()[:T], ref, "ffn layer %s T=%d fused=%d" % (fmt, T, fused))
    print("ffn layer %s T=%d: max|err|/rms %.2e, rel Frobenius %.2e" % (fmt, T, max_rel, frob))
    # H itself: the GPU rounds its own float32 gate_up output, so a value
    # near a bf16 rounding boundary may land one bf16 step away
    fg = (H.cpu().numpy().view(np.uint16)[:T * k].astype(np.uint32) << 16).view(np.float32)
    fr = (H_ref.astype(np.uint32) << 16).view(np.float32)
    assert_within_h(fg, fr, "H %s T=%d fused=%d" % (fmt, T, fused))


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
@pytest.mark.parametrize("E,I,K,T,k,gather,distinct", [
    (6, 100, 256, 1, 4, 1, True),       # one token, gathered: persistent GEMV; ragged I
    (6, 100, 256, 1, 4, 0, True),       # one token, routed order
    (6, 100, 256, 1, 6, 0, False),      # routed order with repeated experts
    (5, 72, 2880, 3, 4, 1, True),       # a few tokens: multi-token GEMV, K = 2880
    (8, 300, 512, 40, 2, 1, True),      # MFMA: ragged M and H-column tails
    (4, 64, 1024, 200, 2, 0, True),     # MFMA, routed-order input
])
def test_fused_swiglu_equals_gemm_then_swiglu(fmt, E, I, K, T, k, gather, distinct):
    """The epilogue computes the same float32 products as the plain GEMM and
    rounds them as gnf4_swiglu does: bit-identical H, on every path."""
    gl = gnf4()
    if fmt == "mxfp4" and K % 64:
        K = 2944                              # the MFMA path needs K % 64 == 0
    case = synth.small_layer(E, 2 * I, K, T, k, seed=4, distinct=distinct, gather=gather)
    codes, scales, scales2 = oracle_pack(fmt, case["W"])
    pw = packed_to_device(gl, fmt, codes, scales, scales2, E, 2 * I, K)
    say("fused swiglu", fmt, E, I, K, T, k, gather, distinct)
    r = gl.route(torch.from_numpy(case["ids"]).cuda(), E)
    Xd = bits_to_device(case["X"])
    Y = gl.grouped_gemm(pw, Xd, gather, r, T, k)
    H_ref = gl.swiglu(Y, I)
    H = gl.grouped_gemm_swiglu(pw, Xd, gather, r, T, k)
    torch.cuda.synchronize()
    nv = int(r["offsets"][-1].item())
    assert nv > 0
    a = H.cpu().numpy()[:nv]
    b = H_ref.cpu().numpy()[:nv]
    assert np.array_equal(a, b), int((a != b).sum())
