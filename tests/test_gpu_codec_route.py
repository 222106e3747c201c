"""GPU parity, bit-exact: dequantization, quantization and routing."""

import numpy as np
import pytest
import torch

import synth
from oracle import mxfp4, nf4, routing

from .gpu_util import FMT_ID, check_route, gnf4, oracle_pack, packed_to_device, say

pytestmark = pytest.mark.gpu

ABSMAX = np.array([0.0, 1.0, 2.0 ** -20, 0.0371, 3.5e-39, 1e-45, np.finfo(np.float32).max, 0.06],
                  dtype=np.float32)


def test_dequant_nf4_every_byte_and_absmax():
    g = gnf4()
    # expert 0: row r uses absmax ABSMAX[r % 8]; bytes cycle through 0..255
    N, K = 16, 512
    codes = (np.arange(N * K // 2) % 256).astype(np.uint8).reshape(1, N, K // 2)
    scales = np.resize(ABSMAX, N * K // 64).reshape(1, N, K // 64).astype(np.float32)
    say("dequant nf4 all bytes")
    pw = packed_to_device(g, "nf4", codes, scales, None, 1, N, K)
    got = g.dequant(pw, 0).cpu().numpy()
    with np.errstate(over="ignore"):
        ref = nf4.dequantize(codes[0], scales[0], K)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_nf4_dq():
    g = gnf4()
    W = synth.small_layer(3, 40, 192, 1, 1, seed=5)["W"]
    codes, q8, s2 = nf4.quantize_dq(W)
    pw = packed_to_device(g, "nf4_dq", codes, q8, s2, 3, 40, 192)
    for e in range(3):
        say("dequant nf4_dq expert", e)
        got = g.dequant(pw, e).cpu().numpy()
        a = nf4.dq_absmax(q8, s2).reshape(3, 40, 3)[e]
        ref = nf4.dequantize(codes[e], a, 192)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_mxfp4_every_scale_and_code():
    g = gnf4()
    N, K = 256, 32
    row = mxfp4.pack(np.tile(np.arange(16, dtype=np.uint8), 2))
    codes = np.tile(row, (N, 1)).reshape(1, N, K // 2)
    scales = np.arange(256, dtype=np.uint8).reshape(1, N, 1)
    say("dequant mxfp4 all scales")
    pw = packed_to_device(g, "mxfp4", codes, scales, None, 1, N, K)
    got = g.dequant(pw, 0).cpu().numpy()
    ref = mxfp4.dequantize(codes[0], scales[0], K)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def adversarial_weights(fmt, E=2, N=24, K=256):
    W = synth.small_layer(E, N, K, 1, 1, seed=11)["W"].copy()
    flat = W.reshape(-1, 64 if fmt != "mxfp4" else 32)
    flat[0] = 0.0                                   # all-zero block
    flat[1] = 1e-40                                 # subnormal block
    flat[2, :] = -0.0
    flat[3] *= 1e30                                 # large magnitudes
    c = nf4.codebook().astype(np.float64)
    mids = (c[:-1] + c[1:]) / 2
    ties = [np.float32(m) for m in mids if float(np.float32(m)) == m]
    flat[4, 0] = 1.0
    for j, v in enumerate(ties):
        flat[4, 1 + j] = v                          # exact NF4 midpoints (absmax 1)
    if fmt == "mxfp4":
        flat[5] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.25, -5.0] * 3 + [6.0, 4.0],
                           dtype=np.float32)       # e2m1 ties with scale 2^0
    return W


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
def test_quantize_matches_oracle(fmt):
    g = gnf4()
    for W in (adversarial_weights(fmt), synth.small_layer(4, 96, 2880 if fmt == "mxfp4" else 1536,
                                                          1, 1, seed=3)["W"]):
        E, N, K = W.shape
        say("quantize", fmt, W.shape)
        pw = g.quantize(fmt, torch.from_numpy(W).cuda())
        codes, scales, scales2 = oracle_pack(fmt, W)
        assert np.array_equal(pw.codes.cpu().numpy().reshape(-1), codes.reshape(-1))
        assert np.array_equal(pw.scales.cpu().numpy().reshape(-1).view(np.uint8),
                              np.ascontiguousarray(scales).reshape(-1).view(np.uint8))
        if scales2 is not None:
            assert np.array_equal(pw.scales2.cpu().numpy().view(np.uint32), scales2.view(np.uint32))


ROUTE_CASES = [("tiny", 16), ("olmoe", 1), ("olmoe", 512), ("qwen30", 1), ("qwen30", 8),
               ("qwen30", 2048), ("qwen235", 1), ("qwen235", 4096), ("gptoss", 1), ("gptoss", 2048),
               ("mixtral", 2048)]


@pytest.mark.parametrize("name,T", ROUTE_CASES)
def test_route_workloads(name, T):
    g = gnf4()
    cfg = synth.CONFIGS[name]
    ids, _ = synth.routing_inputs(cfg, T)
    say("route", name, T)
    r = g.route(torch.from_numpy(ids).cuda(), cfg.E)
    check_route(r, routing.route(ids, cfg.E), T * cfg.k)
    r2 = g.route(torch.from_numpy(ids).cuda(), cfg.E)
    for key in r:
        if key != "workspace":                         # scratch: contents unspecified
            assert torch.equal(r[key], r2[key]), key   # deterministic


@pytest.mark.parametrize("E,T,k", [
    (1, 5, 1), (7, 33, 3), (1024, 100, 8), (300, 4000, 8), (5, 0, 4),
    (64, 128, 8),          # 1024 assignments: the largest one-workgroup route
    (64, 1025, 1),         # 1025: two chunks, the second holding one assignment
    (128, 257, 8),         # 2056: three chunks, a ragged last chunk
    (1, 3000, 1),          # one expert: every chunk adds to one segment
    (1024, 4096, 8),       # 32 chunks over 1024 experts
    (16, 40000, 8),        # 320,000: past 256 chunks, chunks of 2048
])
def test_route_edge_cases(E, T, k):
    g = gnf4()
    rs = np.random.default_rng(E * 1000 + T)
    ids = rs.integers(-2, E + 2, size=(T, k)).astype(np.int32)   # duplicates and bad ids
    say("route edge", E, T, k, "workspace", g.route_workspace_bytes(T, k, E))
    r = g.route(torch.from_numpy(ids).cuda().reshape(T, k), E)
    ref = routing.route(ids, E)
    check_route(r, ref, T * k)


@pytest.mark.parametrize("where", ["first", "last", "none"])
def test_route_bad_id_flag_from_any_chunk(where):
    """The flag is the OR over chunks: one bad id in the first or the last of
    five chunks raises it; none leaves it 0."""
    g = gnf4()
    E, T, k = 32, 4100, 1
    ids = np.random.default_rng(5).integers(0, E, size=(T, k)).astype(np.int32)
    if where == "first":
        ids[3, 0] = E
    elif where == "last":
        ids[T - 1, 0] = -7
    say("route bad id", where)
    r = g.route(torch.from_numpy(ids).cuda(), E)
    check_route(r, routing.route(ids, E), T * k)
    assert int(r["bad"].item()) == (0 if where == "none" else 1)


def test_route_workspace_contents_do_not_matter():
    """The same call with a workspace full of garbage gives the same result."""
    g = gnf4()
    E, T, k = 128, 4096, 8
    ids = np.random.default_rng(9).integers(0, E, size=(T, k)).astype(np.int32)
    ids_d = torch.from_numpy(ids).cuda()
    out = g.route_buffers(T, k, E)
    out["workspace"].fill_(0xA5)
    say("route garbage workspace")
    r1 = g.route(ids_d, E, out=out)
    a = {key: v.clone() for key, v in r1.items() if key != "workspace"}
    out["workspace"].fill_(0x3C)
    r2 = g.route(ids_d, E, out=out)
    for key in a:
        assert torch.equal(a[key], r2[key]), key
    check_route(r2, routing.route(ids, E), T * k)


def dequant_bf16_ref(fmt, codes, scales, scales2, e, N, K):
    """The oracle's float32 dequant of expert e rounded to bf16 bits."""
    from oracle import grouped_gemm as ogemm
    from oracle import layer as olayer
    W = ogemm.dequant_rows(fmt, codes, scales, scales2, e, np.arange(N), N, K)
    return olayer.f64_to_bf16_bits(W.astype(np.float64))


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
def test_dequant_experts_bf16_matches_oracle(fmt):
    g = gnf4()
    E, N, K = 6, 40, 256
    W = adversarial_weights(fmt, E=E, N=N, K=K)
    codes, scales, scales2 = oracle_pack(fmt, W)
    if fmt == "mxfp4":                               # the extreme e8m0 scales too
        scales = scales.copy()
        scales.reshape(-1)[:6] = np.array([0, 1, 127, 253, 254, 255], dtype=np.uint8)
    pw = packed_to_device(g, fmt, codes, scales, scales2, E, N, K)
    experts = torch.tensor([4, 1, 5, -1, 2, 0], dtype=torch.int32, device="cuda")
    count = torch.tensor([5], dtype=torch.int32, device="cuda")
    out = torch.full((6, N, K), 0x1234, dtype=torch.int16, device="cuda")
    say("dequant bf16", fmt)
    got = g.dequant_experts_bf16(pw, experts, count, 6, out).cpu().numpy().view(np.uint16)
    for slot, e in enumerate([4, 1, 5]):
        ref = dequant_bf16_ref(fmt, codes, scales, scales2, e, N, K)
        nan = (ref & 0x7FFF) > 0x7F80
        assert np.array_equal(nan, (got[slot] & 0x7FFF) > 0x7F80)
        assert np.array_equal(got[slot][~nan], ref[~nan]), (fmt, slot)
    assert np.all(got[3] == 0x1234)                  # id -1: left untouched
    assert np.array_equal(got[4], dequant_bf16_ref(fmt, codes, scales, scales2, 2, N, K))
    assert np.all(got[5] == 0x1234)                  # past the count
