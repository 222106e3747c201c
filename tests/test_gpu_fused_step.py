"""The fused entry points of the decode step give what the separate calls
give: gnf4_route_grouped_gemm equals gnf4_route followed by the first
projection (routing arrays and Y or H bit for bit), on the one-launch path
(T = 1) and on the two-launch path (T > 1); and every output of each fused
call is also compared with the float64 oracle directly (routing, top-k ids
and weights bit for bit, Y and out at the per-call bars, H at the layer
bar)."""

import numpy as np
import pytest
import torch

import synth
from oracle import combine as ocombine
from oracle import grouped_gemm as ogemm
from oracle import layer as olayer
from oracle import routing

from .gpu_util import bits_to_device, check_route, gnf4, oracle_pack, packed_to_device, say
from .tolerance import assert_within, assert_within_h, assert_within_layer


def oracle_first_projection(fmt, packed, X, ids, E, N, K, k, swiglu, got):
    """got (Y float32, or H bf16 bits with the SwiGLU epilogue) against the
    oracle's grouped GEMM of the same routing."""
    codes, scales, scales2 = packed
    r_ref = routing.route(ids, E)
    nv = int(r_ref["offsets"][-1])
    Y_ref = ogemm.grouped_gemm(fmt, codes, scales, scales2, X, 1, r_ref["offsets"], r_ref["perm"],
                               k, N, K)[:nv]
    if not swiglu:
        assert_within(got[:nv], Y_ref, "Y vs oracle")
        return r_ref
    H_ref = olayer.swiglu(Y_ref, N // 2)
    Hg = (got[:nv].view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    Hr = (H_ref.astype(np.uint32) << 16).view(np.float32)
    assert_within_h(Hg, Hr, "H vs oracle")
    return r_ref


pytestmark = pytest.mark.gpu


def same_route(r_a, r_b, n):
    for key in ("counts", "offsets", "active", "n_active", "bad"):
        a, b = r_a[key].cpu().numpy(), r_b[key].cpu().numpy()
        assert np.array_equal(a, b), (key, a, b)
    if n:
        for key in ("perm", "inv"):
            a, b = r_a[key].cpu().numpy()[:n], r_b[key].cpu().numpy()[:n]
            assert np.array_equal(a, b), (key, a, b)


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("E,N,K,T,k,ids_kind", [
    (8, 256, 256, 1, 2, "distinct"),
    (64, 512, 2048, 1, 8, "distinct"),
    (16, 128, 512, 1, 6, "duplicates"),
    (16, 128, 512, 1, 6, "bad"),          # out-of-range ids: dropped, flag raised
    (128, 96, 2880, 1, 4, "distinct"),    # K = 2880
    (1024, 64, 256, 1, 64, "distinct"),   # E = 1024, k = 64
    (3, 64, 256, 1, 1, "distinct"),       # k = 1
    (8, 256, 256, 5, 2, "duplicates"),    # T > 1: two launches
])
def test_route_grouped_gemm_equals_separate_calls(fmt, swiglu, E, N, K, T, k, ids_kind):
    g = gnf4()
    if fmt == "mxfp4" and K % 32:
        pytest.skip("MXFP4 needs K % 32 == 0")
    case = synth.small_layer(E, N, K, T, k, seed=8, distinct=(ids_kind == "distinct"), gather=1)
    ids = case["ids"].copy()
    if ids_kind == "bad":
        ids[0, 1] = E + 5
        ids[0, 3] = -2
    codes, scales, scales2 = oracle_pack(fmt, case["W"])
    pw = packed_to_device(g, fmt, codes, scales, scales2, E, N, K)
    X = bits_to_device(case["X"])
    ids_d = torch.from_numpy(ids).cuda()
    say("route_grouped_gemm", fmt, "swiglu", swiglu, E, N, K, T, k, ids_kind)
    r_ref = g.route(ids_d, E)
    if swiglu:
        ref = g.grouped_gemm_swiglu(pw, X, 1, r_ref, T, k)
    else:
        ref = g.grouped_gemm(pw, X, 1, r_ref, T, k)
    r, got = g.route_grouped_gemm(ids_d, pw, X, swiglu=swiglu)
    torch.cuda.synchronize()
    same_route(r, r_ref, T * k)
    nv = int(r_ref["offsets"][-1].item())
    a = got.cpu().numpy()[:nv]
    b = ref.cpu().numpy()[:nv]
    assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                          b.view(np.uint32) if b.dtype == np.float32 else b), "outputs differ"
    if ids_kind == "bad":
        assert int(r["bad"].item()) == 1 and nv == T * k - 2
    r_ref = oracle_first_projection(fmt, (codes, scales, scales2), case["X"], ids, E, N, K, k, swiglu,
                                    got.cpu().numpy())
    check_route(r, r_ref, T * k)


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
@pytest.mark.parametrize("E,N,K,T,k,ids_kind", [
    (8, 256, 256, 1, 2, "distinct"),
    (64, 2048, 1024, 1, 8, "distinct"),   # the OLMoE-shaped down projection (two rows per slot)
    (8, 8192, 512, 1, 8, "distinct"),     # 8192 output rows: four rows per wave slot
    (6, 2880, 1024, 1, 4, "duplicates"),  # k = 4: two row blocks per workgroup, two rows per slot
    (16, 200, 512, 1, 6, "duplicates"),   # copies of one expert with different inputs
    (16, 128, 512, 1, 6, "bad"),          # dropped copies add nothing
    (128, 96, 2880, 1, 4, "distinct"),    # K = 2880 (three chunks per lane)
    (1024, 64, 256, 1, 64, "distinct"),   # k = 64
    (6, 64, 6144, 1, 5, "distinct"),      # K = 6144: four chunks per lane
    (3, 64, 256, 1, 1, "distinct"),       # k = 1
    (8, 200, 256, 1, 2, "distinct"),      # 25 row blocks, 4 per workgroup: the last holds 1
    (8, 3000, 2048, 1, 2, "distinct"),    # 750 row blocks, 4 per workgroup: the last holds 2
    (8, 64, 8192, 1, 4, "distinct"),      # K = 8192: the largest K of the one-launch path
    (8, 64, 8256, 1, 5, "distinct"),      # K past it: two launches (MFMA GEMM, then combine)
    (8, 256, 256, 7, 2, "duplicates"),    # T > 1: two launches
])
def test_grouped_gemm_combine_equals_separate_calls(fmt, E, N, K, T, k, ids_kind):
    g = gnf4()
    case = synth.small_layer(E, N, K, T, k, seed=9, distinct=(ids_kind == "distinct"), gather=0)
    ids = case["ids"].copy()
    if ids_kind == "bad":
        ids[0, 0] = E
        ids[0, 4] = -1
    codes, scales, scales2 = oracle_pack(fmt, case["W"])
    pw = packed_to_device(g, fmt, codes, scales, scales2, E, N, K)
    X = bits_to_device(case["X"])
    tw = torch.from_numpy(case["tw"]).cuda()
    say("grouped_gemm_combine", fmt, E, N, K, T, k, ids_kind)
    r = g.route(torch.from_numpy(ids).cuda(), E)
    Y = g.grouped_gemm(pw, X, 0, r, T, k)
    ref = g.combine(Y, r["inv"], tw, T, k)
    got = g.grouped_gemm_combine(pw, X, r, tw, T, k)
    torch.cuda.synchronize()
    a = got.cpu().numpy()[:T]
    b = ref.cpu().numpy()[:T]
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), int((a != b).sum())
    r_ref = routing.route(ids, E)
    check_route(r, r_ref, T * k)
    Y_ref = ogemm.grouped_gemm(fmt, codes, scales, scales2, case["X"], 0, r_ref["offsets"],
                               r_ref["perm"], k, N, K)
    assert_within(a, ocombine.combine(Y_ref, r_ref["inv"], case["tw"], T, k), "out vs oracle")


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("E,N,K,T,k,logits_kind", [
    (64, 512, 2048, 1, 8, "normal"),
    (128, 256, 512, 1, 4, "ties"),        # equal logits: lower id first
    (1024, 64, 256, 1, 64, "normal"),     # E = 1024, k = 64
    (8, 128, 256, 1, 8, "nan"),           # NaN logits rank last
    (16, 128, 256, 6, 3, "normal"),       # T > 1: separate launches
])
def test_route_logits_grouped_gemm_equals_separate_calls(fmt, swiglu, E, N, K, T, k, logits_kind):
    g = gnf4()
    case = synth.small_layer(E, N, K, T, k, seed=10, distinct=True, gather=1)
    gl = np.random.default_rng([E, N, K, T, k])
    logits = gl.standard_normal((T, E)).astype(np.float32)
    if logits_kind == "ties":
        logits = np.round(logits).astype(np.float32)
    if logits_kind == "nan":
        logits[0, ::3] = np.nan
    codes, scales, scales2 = oracle_pack(fmt, case["W"])
    pw = packed_to_device(g, fmt, codes, scales, scales2, E, N, K)
    X = bits_to_device(case["X"])
    lg = torch.from_numpy(logits).cuda()
    say("route_logits_grouped_gemm", fmt, "swiglu", swiglu, E, N, K, T, k, logits_kind)
    r_ref = g.route_logits(lg, k)
    if swiglu:
        ref = g.grouped_gemm_swiglu(pw, X, 1, r_ref, T, k)
    else:
        ref = g.grouped_gemm(pw, X, 1, r_ref, T, k)
    r, got = g.route_logits_grouped_gemm(lg, k, pw, X, swiglu=swiglu)
    torch.cuda.synchronize()
    same_route(r, r_ref, T * k)
    assert np.array_equal(r["topk_ids"].cpu().numpy(), r_ref["topk_ids"].cpu().numpy())
    assert np.array_equal(r["topk_w"].cpu().numpy().view(np.uint32),
                          r_ref["topk_w"].cpu().numpy().view(np.uint32))
    nv = int(r_ref["offsets"][-1].item())
    a = got.cpu().numpy()[:nv]
    b = ref.cpu().numpy()[:nv]
    assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                          b.view(np.uint32) if b.dtype == np.float32 else b), "outputs differ"
    ids_o, w_o = olayer.topk_softmax(logits, k)
    assert np.array_equal(r["topk_ids"].cpu().numpy(), ids_o), "top-k ids vs oracle"
    w = r["topk_w"].cpu().numpy()
    assert np.array_equal(np.isnan(w), np.isnan(w_o))
    assert np.array_equal(w[~np.isnan(w)], w_o[~np.isnan(w_o)]), "top-k weights vs oracle"
    ro = oracle_first_projection(fmt, (codes, scales, scales2), case["X"], ids_o, E, N, K, k, swiglu,
                                 got.cpu().numpy())
    check_route(r, ro, T * k)
