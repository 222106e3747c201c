"""GPU parity of the grouped GEMM and combine against the float64 oracle.

Small layers cover both paths (decode GEMV at T*k <= 64, MFMA prefill above),
every format, several tiles with ragged N and M tails, duplicate ids, bad ids
and gather = 0 / 1. Exactness pins: one-hot activation rows return single
decoded weights bit for bit. Also: determinism, chunk invariance, untouched
weights, and a byte-flip negative control.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import grouped_gemm as ogemm
from oracle import mxfp4, nf4, routing

from .gpu_util import (bits_to_device, compare_rows, gnf4, oracle_combine, oracle_pack,
                       packed_to_device, run_layer_call, say)
from .tolerance import assert_within, within

pytestmark = pytest.mark.gpu

# (E, N, K, T, k): decode shapes (T*k <= 64) and prefill shapes (T*k > 64)
SHAPES = [
    (8, 512, 256, 16, 2),      # the tiny workload: decode path, 32 rows
    (6, 200, 384, 3, 2),       # ragged N
    (5, 96, 2880, 1, 4),       # K = 2880 (45 NF4 / 90 MXFP4 blocks)
    (16, 336, 768, 8, 8),      # 64 rows, K = 768
    (8, 320, 512, 40, 2),      # prefill, ragged M and N tails, several tiles
    (4, 256, 1024, 200, 2),    # prefill, 400 rows over 4 experts: ~100 rows each, so
                               # one whole 64-row tile and a ragged tail per expert
    (3, 130, 2880, 37, 3),     # prefill, K = 2880, ragged N
    (4, 192, 384, 50, 2),      # prefill, K = 384: three 128-K stages, no tail
    (3, 64, 64, 40, 2),        # prefill, K = 64: one block, one stage
    (3, 96, 192, 40, 2),       # prefill, K = 192: a last stage with one block
]


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "E%d_N%d_K%d_T%d_k%d" % s)
def test_gemm_small(fmt, shape):
    g = gnf4()
    E, N, K, T, k = shape
    case = synth.small_layer(E, N, K, T, k, seed=1)
    Y, Y_ref, r_ref = run_layer_call(g, fmt, case["W"], case["X"], case["ids"], 1, k, "small")
    compare_rows(Y, Y_ref, r_ref, "%s %s" % (fmt, shape))


# Prefill shapes for the MFMA kernel's tile count and its share per XCD:
# each workgroup counts the real M tiles over all experts (in chunks of 64
# experts) and takes one eighth of them per XCD, so the cases cover a ragged
# last chunk of experts, fewer tiles than XCDs, and a few busy experts among
# many empty ones (HOT: every token picks k of the HOT experts 0, E/2, E-1).
@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
@pytest.mark.parametrize("E,N,K,T,k,hot", [
    (200, 96, 128, 100, 4, False),     # 4 chunks of experts, the last one ragged
    (2, 64, 128, 40, 2, False),        # 40 rows on each of 2 experts: 2 tiles, fewer than the XCDs
    (300, 320, 128, 70, 2, True),      # 140 rows on 3 of 300 experts, 2 N tiles
])
def test_mfma_tile_count_and_xcd_share(fmt, E, N, K, T, k, hot):
    g = gnf4()
    case = synth.small_layer(E, N, K, T, k, seed=9)
    ids = case["ids"]
    if hot:
        busy = np.array([0, E // 2, E - 1], dtype=np.int32)
        rng = np.random.Generator(np.random.PCG64(11))
        ids = np.stack([rng.permutation(busy)[:k] for _ in range(T)]).astype(np.int32)
    assert T * k > 64                              # the MFMA path
    Y, Y_ref, r_ref = run_layer_call(g, fmt, case["W"], case["X"], ids, 1, k, "tile share")
    compare_rows(Y, Y_ref, r_ref, "tile share %s E=%d" % (fmt, E))


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("T,k,distinct", [(1, 4, True), (1, 6, False), (4, 4, True), (30, 4, True)])
def test_gemm_permuted_input(fmt, T, k, distinct):
    """Input already in routed order (the down projection). One token with
    repeated experts puts the routed rows of later experts past their slot
    index."""
    g = gnf4()
    E, N, K = 8, 160, 512
    case = synth.small_layer(E, N, K, T, k, seed=2, gather=0, distinct=distinct)
    if not distinct:
        assert len(np.unique(case["ids"])) < k           # the case needs a repeat
    Y, Y_ref, r_ref = run_layer_call(g, fmt, case["W"], case["X"], case["ids"], 0, k, "gather0")
    compare_rows(Y, Y_ref, r_ref, "gather=0 %s T=%d" % (fmt, T))


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
@pytest.mark.parametrize("T,k", [(1, 8), (6, 4), (50, 4)])
def test_gemm_duplicates_and_bad_ids(fmt, T, k):
    """Repeated experts (several routed rows share one expert's products, or
    one expert's weights serve several token rows) and dropped ids; T = 1
    is the one-token gathered kernel."""
    g = gnf4()
    E, N, K = 5, 128, 256
    case = synth.small_layer(E, N, K, T, k, seed=3, distinct=False)
    ids = case["ids"].copy()
    ids[0, 0] = -1
    ids[-1, -1] = E + 3
    valid = ids[(ids >= 0) & (ids < E)]
    assert len(np.unique(valid)) < len(valid)            # the case needs a repeat
    Y, Y_ref, r_ref = run_layer_call(g, fmt, case["W"], case["X"], ids, 1, k, "dup/bad")
    assert r_ref["bad"][0] == 1
    compare_rows(Y, Y_ref, r_ref, "duplicates and bad ids %s T=%d" % (fmt, T))


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
@pytest.mark.parametrize("E,N,K,T,k", [
    (4, 192, 4096, 1, 8),      # one token, k > E: every expert gets several copies of token 0
    (2, 160, 512, 2, 4),       # two tokens, 4 rows per expert: more rows than a token group
])
def test_gemv_repeated_rows(fmt, E, N, K, T, k):
    """Decode path with ids drawn with replacement, so an expert holds more
    routed rows than the token slice registers cover (rows are streamed
    again) and, for one token, every row is the same activation."""
    g = gnf4()
    case = synth.small_layer(E, N, K, T, k, seed=5, distinct=False)
    Y, Y_ref, r_ref = run_layer_call(g, fmt, case["W"], case["X"], case["ids"], 1, k, "repeated")
    compare_rows(Y, Y_ref, r_ref, "repeated rows %s E%d T%d k%d" % (fmt, E, T, k))


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_gemv_more_items_than_workgroups(fmt):
    """64 routed rows over up to 64 experts with 4096 outputs: more (expert,
    row block) items than resident workgroups, so each workgroup walks several
    items with the next item's rows in flight; slots past the active count end
    the walk."""
    g = gnf4()
    E, N, K, T, k = 64, 4096, 64, 8, 8
    case = synth.small_layer(E, N, K, T, k, seed=6)
    Y, Y_ref, r_ref = run_layer_call(g, fmt, case["W"], case["X"], case["ids"], 1, k, "many items")
    assert int(r_ref["n_active"][0]) < E            # some slots are -1
    compare_rows(Y, Y_ref, r_ref, "many items %s" % fmt)


def one_hot_case(fmt, T, k, E=4, N=96, K=256):
    case = synth.small_layer(E, N, K, T, k, seed=4)
    X = np.zeros((T, K), dtype=np.uint16)
    cols = (np.arange(T) * 37) % K
    X[np.arange(T), cols] = 0x3F80                 # bf16 1.0
    return case, X, cols


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
@pytest.mark.parametrize("T,k", [(3, 2), (60, 2)])      # decode and prefill path
def test_one_hot_rows_are_exact(fmt, T, k):
    """A one-hot activation row selects one weight per output. NF4 enters the
    product as the bf16 operand value bf16(s * c) times fp32(absmax * (1/s)),
    so the output must be exactly fp32(fp32(absmax * fp32(1/s)) * bf16(s * c));
    MXFP4 decodes exactly, so the output is the dequantized weight itself."""
    g = gnf4()
    case, X, cols = one_hot_case(fmt, T, k)
    E, N, K = case["W"].shape
    codes, scales, scales2 = oracle_pack(fmt, case["W"])
    pw = packed_to_device(g, fmt, codes, scales, scales2, E, N, K)
    ids = case["ids"]
    say("one-hot", fmt, T, k)
    r = g.route(torch.from_numpy(ids).cuda(), E)
    Y = g.grouped_gemm(pw, bits_to_device(X), 1, r, T, k).cpu().numpy()
    ref = routing.route(ids, E)
    vals, s_op = g.nf4_codebook_bf16()          # pinned to the oracle codebook on the CPU
    cb = (np.float32(s_op) * nf4.codebook()).astype(np.float32)
    cb_bf16 = (np.ascontiguousarray(cb).view(np.uint32) + 0x7FFF + ((cb.view(np.uint32) >> 16) & 1)) >> 16
    cb_bf16 = (cb_bf16 << 16).astype(np.uint32).view(np.float32)
    inv_s = np.float32(1.0) / np.float32(s_op)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            p = int(ref["inv"][t * k + j])
            col = int(cols[t])
            if fmt == "mxfp4":
                expect = mxfp4.dequantize(codes[e], scales[e], K)[:, col]
            else:
                if fmt == "nf4":
                    a = scales[e][:, col // 64].astype(np.float32)
                else:
                    a = nf4.dq_absmax(scales, scales2).reshape(E, N, K // 64)[e][:, col // 64]
                q = nf4.unpack(codes[e].reshape(-1)).reshape(N, K)[:, col]
                expect = ((a * inv_s).astype(np.float32) * cb_bf16[q]).astype(np.float32)
            # exact values (a zero may come out as +0 where the weight is -0)
            assert np.array_equal(Y[p], expect), (t, j)


def test_deterministic_and_chunk_invariant():
    """Two identical calls give identical bits; a 64-row call and four 16-row
    calls both meet the bar against the oracle and agree with each other
    within it."""
    g = gnf4()
    E, N, K, k = 8, 256, 512, 2
    case = synth.small_layer(E, N, K, 64, k, seed=6)
    codes, scales, _ = oracle_pack("nf4", case["W"])
    pw = packed_to_device(g, "nf4", codes, scales, None, E, N, K)
    ids, X = case["ids"], case["X"]
    say("determinism / chunk invariance")
    r = g.route(torch.from_numpy(ids).cuda(), E)
    Y1 = g.grouped_gemm(pw, bits_to_device(X), 1, r, 64, k)
    Y2 = g.grouped_gemm(pw, bits_to_device(X), 1, r, 64, k)
    assert torch.equal(Y1, Y2)
    ref = routing.route(ids, E)
    Yr = ogemm.grouped_gemm("nf4", codes, scales, None, X, 1, ref["offsets"], ref["perm"], k, N, K)
    wide = Y1.cpu().numpy()[ref["inv"]].reshape(64, k, N)
    full_ref = Yr[ref["inv"]].reshape(64, k, N)
    chunks = []
    for c in range(4):
        ids_c, X_c = ids[16 * c:16 * c + 16], X[16 * c:16 * c + 16]
        rc = g.route(torch.from_numpy(np.ascontiguousarray(ids_c)).cuda(), E)
        Yc = g.grouped_gemm(pw, bits_to_device(X_c), 1, rc, 16, k).cpu().numpy()
        refc = routing.route(ids_c, E)
        chunks.append(Yc[refc["inv"]].reshape(16, k, N))
    narrow = np.concatenate(chunks)
    assert_within(wide, full_ref, "64-row call")
    assert_within(narrow, full_ref, "4 x 16-row calls")
    assert_within(narrow, wide, "chunked vs wide")


def test_byte_flip_negative_control():
    """Flipping one packed byte of a routed expert on the device must make the
    output fail the bar against the oracle of the unflipped weights."""
    g = gnf4()
    E, N, K, T, k = 4, 128, 256, 8, 2
    case = synth.small_layer(E, N, K, T, k, seed=7)
    codes, scales, _ = oracle_pack("nf4", case["W"])
    pw = packed_to_device(g, "nf4", codes, scales, None, E, N, K)
    ids = case["ids"]
    r = g.route(torch.from_numpy(ids).cuda(), E)
    ref = routing.route(ids, E)
    Yr = ogemm.grouped_gemm("nf4", codes, scales, None, case["X"], 1, ref["offsets"], ref["perm"], k, N, K)
    Y = g.grouped_gemm(pw, bits_to_device(case["X"]), 1, r, T, k).cpu().numpy()
    assert within(Y, Yr)
    pw.codes[int(ids[0, 0]), 5, 0] ^= 0xFF
    say("byte flip")
    Yb = g.grouped_gemm(pw, bits_to_device(case["X"]), 1, r, T, k).cpu().numpy()
    assert not within(Yb, Yr)


@pytest.mark.parametrize("T,k,N", [(16, 2, 512), (3, 8, 2048), (130, 4, 64), (5, 13, 1028),
                                   (2, 64, 96)])
def test_combine(T, k, N):
    g = gnf4()
    cfg = synth.CONFIGS["tiny"]
    E = max(16, k)
    rs = np.random.default_rng(T)
    ids = np.stack([rs.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[0, 0] = -1                                  # a dropped assignment
    tw = rs.random((T, k)).astype(np.float32)
    Yin = synth.random_rows(cfg, T * k, N, extra=T)
    ref_r = routing.route(ids, E)
    say("combine", T, k, N)
    r = g.route(torch.from_numpy(ids).cuda(), E)
    out = g.combine(torch.from_numpy(Yin).cuda(), r["inv"], torch.from_numpy(tw).cuda(), T, k)
    ref = oracle_combine(Yin.astype(np.float64), ref_r, tw, T, k)
    assert_within(out.cpu().numpy(), ref, "combine")


def test_combine_k1_copies_exactly():
    g = gnf4()
    T, N, E = 40, 96, 8
    ids = (np.arange(T) % E).astype(np.int32).reshape(T, 1)
    Yin = synth.random_rows(synth.CONFIGS["tiny"], T, N, extra=1)
    r = g.route(torch.from_numpy(ids).cuda(), E)
    out = g.combine(torch.from_numpy(Yin).cuda(), r["inv"], torch.ones((T, 1), device="cuda"), T, 1)
    ref_r = routing.route(ids, E)
    assert np.array_equal(out.cpu().numpy(), Yin[ref_r["inv"]])


@pytest.mark.parametrize("T", [16])
def test_tiny_layer_end_to_end(T):
    """The tiny workload end to end: route, grouped GEMM, combine."""
    g = gnf4()
    cfg = synth.CONFIGS["tiny"]
    proj = cfg.projs[0]
    W = synth.layer_weight(cfg, proj)
    ids, tw = synth.routing_inputs(cfg, T)
    X = synth.token_inputs(cfg, T)
    Y, Y_ref, r_ref = run_layer_call(g, cfg.fmt, W, X, ids, 1, cfg.k, "tiny e2e")
    compare_rows(Y, Y_ref, r_ref, "tiny gemm")
    r = g.route(torch.from_numpy(ids).cuda(), cfg.E)
    out = g.combine(torch.from_numpy(Y).cuda(), r["inv"], torch.from_numpy(tw).cuda(), T, cfg.k)
    assert_within(out.cpu().numpy(), oracle_combine(Y_ref, r_ref, tw, T, cfg.k), "tiny combine")


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
@pytest.mark.parametrize("gather", [1, 0])
@pytest.mark.parametrize("swiglu", [False, True])
def test_mfma_last_tile_row_classes(fmt, gather, swiglu):
    """The prefill kernel computes an expert's last 64-row tile with only the
    16-row tiles that hold rows: 65, 81, 97 and 113 routed rows leave last
    tiles of 1, 17, 33 and 49 rows (one, two, three and four 16-row tiles).
    Every element against the oracle (Y, or H with the SwiGLU epilogue)."""
    from oracle import layer as olayer
    from .tolerance import assert_within_h
    g = gnf4()
    E, N, K, k = 4, 320, 512, 1
    counts = [65, 81, 97, 113]
    ids = np.concatenate([np.full(c, e, dtype=np.int32) for e, c in enumerate(counts)])
    ids = np.random.default_rng(31).permutation(ids).reshape(-1, 1)
    T = ids.shape[0]
    case = synth.small_layer(E, N, K, T, k, seed=12, gather=gather)
    codes, scales, scales2 = oracle_pack(fmt, case["W"])
    pw = packed_to_device(g, fmt, codes, scales, scales2, E, N, K)
    say("mfma last tiles", fmt, "gather", gather, "swiglu", swiglu)
    r = g.route(torch.from_numpy(ids).cuda(), E)
    Xd = bits_to_device(case["X"])
    got = (g.grouped_gemm_swiglu(pw, Xd, gather, r, T, k) if swiglu
           else g.grouped_gemm(pw, Xd, gather, r, T, k)).cpu().numpy()
    ref_r = routing.route(ids, E)
    Y_ref = ogemm.grouped_gemm(fmt, codes, scales, scales2, case["X"], gather, ref_r["offsets"],
                               ref_r["perm"], k, N, K)
    if swiglu:
        H_ref = olayer.swiglu(Y_ref, N // 2)
        Hg = (got.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
        Hr = (H_ref.astype(np.uint32) << 16).view(np.float32)
        assert_within_h(Hg, Hr, "H last tiles %s" % fmt)
    else:
        assert_within(got, Y_ref, "last tiles %s gather %d" % (fmt, gather))
