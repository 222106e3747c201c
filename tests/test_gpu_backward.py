"""GPU parity of the input gradient through the frozen packed experts
(gnf4_grouped_gemm_dx) against the float64 oracle: every element at small
shapes that span several row tiles, K tiles and ragged tails, the sum over a
token's routed copies, dropped and duplicate assignments, and a seeded
sample of outputs at the workloads' full sizes. The bar is the backward's
own (tolerance.DX_*), tighter than the forward's: it fails if the bf16 lo
part of the weights were left out."""

import numpy as np
import pytest
import torch

import synth
from oracle import backward as obwd
from oracle import routing

from .gpu_util import bits_to_device, check_route, gnf4, oracle_pack, packed_to_device, say
from .tolerance import DX_FROB_REL, DX_MAX_REL_RMS, assert_within_dx

pytestmark = pytest.mark.gpu

SENTINEL = -12345.5


def run_dx(fmt, E, N, K, T, k, seed, distinct=True, bad=False):
    g = gnf4()
    case = synth.small_layer(E, N, K, T, k, seed=seed, distinct=distinct, gather=0)
    ids = case["ids"].copy()
    if bad and T:
        ids[0, 0] = E + 3                          # dropped assignment
    codes, scales, scales2 = oracle_pack(fmt, case["W"])
    pw = packed_to_device(g, fmt, codes, scales, scales2, E, N, K)
    gr = np.random.default_rng([seed, N, T])
    dY = synth.f32_to_bf16_bits(gr.standard_normal((T * k, N)).astype(np.float32))
    say("grouped_gemm_dx", fmt, "E", E, "N", N, "K", K, "T", T, "k", k, "distinct", distinct, "bad", bad)
    r = g.route(torch.from_numpy(ids).cuda(), E)
    dA0 = torch.full((max(T * k, 1), K), SENTINEL, dtype=torch.float32, device="cuda")
    dA = g.grouped_gemm_dx(pw, bits_to_device(dY), r, T, k, dA=dA0)
    torch.cuda.synchronize()
    r_ref = routing.route(ids, E)
    check_route(r, r_ref, T * k)
    ref = obwd.grouped_gemm_dx(fmt, codes, scales, scales2, dY, r_ref["offsets"], N, K)
    return g, r, r_ref, dA.cpu().numpy(), ref


CASES = [
    # E, N, K, T, k, distinct
    (4, 64, 256, 1, 2, True),          # one token: 16-row tiles, one K tile
    (8, 200, 320, 40, 2, True),        # N % 32 = 8 (short last step), K tail of 64 columns
    (8, 96, 256, 100, 2, False),       # ~25 rows per expert: 32-row tiles, duplicates
    (4, 128, 512, 100, 2, True),       # ~50 rows per expert: 64-row tiles
    (6, 512, 1024, 300, 3, False),     # ~150 rows per expert: 64-row tiles, three per expert
    (3, 96, 2880, 50, 2, True),        # K = 2880: eleven full K tiles and a 64-column tail
    (16, 72, 512, 20, 4, False),       # many experts, some empty
    (5, 1032, 128, 700, 1, True),      # K = 128 (half a tile), N = 32 * 32 + 8
    (4, 136, 640, 500, 1, True),       # ~125 rows per expert: 128-row tiles, 32 columns per wave
    # few routed rows (T*k <= 64): one wave per (expert, rows, 32 columns)
    (64, 136, 2880, 8, 8, True),       # one row per item, K = 2880, N = 2 * 64 + 8
    (32, 200, 320, 16, 4, False),      # two rows per item, duplicates span row blocks
    (16, 96, 512, 12, 4, False),       # four rows per item
    (3, 1032, 128, 2, 2, True),        # N = 1032: four full batches and a tail
]


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
@pytest.mark.parametrize("E,N,K,T,k,distinct", CASES)
def test_dx_matches_oracle(fmt, E, N, K, T, k, distinct):
    _, _, r_ref, got, ref = run_dx(fmt, E, N, K, T, k, 3, distinct)
    nv = int(r_ref["offsets"][-1])
    assert nv == T * k
    assert_within_dx(got[:nv], ref[:nv], "dx %s E=%d N=%d K=%d T=%d k=%d" % (fmt, E, N, K, T, k))


@pytest.mark.parametrize("T", [10, 400])
def test_dx_mxfp4_half_block_tail(T):
    """MXFP4 with K % 64 == 32: with 64-row tiles the last wave of the last K
    tile has only lanes 0..7 (columns 0..31) in range; with 128-row tiles
    (32 columns per wave) the last wave of the last tile is out of range."""
    _, _, r_ref, got, ref = run_dx("mxfp4", 3, 64, 2912, T, 1 if T > 64 else 2, 5)
    assert_within_dx(got, ref, "dx mxfp4 K=2912 T=%d" % T)


@pytest.mark.parametrize("fmt", ["nf4", "mxfp4"])
def test_dx_dropped_rows_untouched(fmt):
    _, _, r_ref, got, ref = run_dx(fmt, 6, 64, 256, 30, 2, 7, distinct=False, bad=True)
    nv = int(r_ref["offsets"][-1])
    assert nv == 30 * 2 - 1
    assert_within_dx(got[:nv], ref[:nv], "dx dropped")
    assert np.all(got[nv:] == SENTINEL)


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
def test_token_grad_matches_oracle(fmt):
    """Gradient of the gathered token rows: dA of each token's routed copies
    summed (gnf4_combine with unit weights)."""
    T, k = 37, 3
    g, r, r_ref, got, ref = run_dx(fmt, 8, 128, 256, T, k, 9, distinct=False, bad=True)
    dA = torch.from_numpy(got).cuda()
    dX = g.token_grad(dA, r, T, k)
    torch.cuda.synchronize()
    dX_ref = obwd.token_grad(ref, r_ref["inv"], T, k)
    assert_within_dx(dX.cpu().numpy()[:T], dX_ref, "token grad %s" % fmt)


def test_dx_zero_tokens():
    g = gnf4()
    case = synth.small_layer(4, 64, 128, 1, 1, seed=1)
    codes, scales, scales2 = oracle_pack("nf4", case["W"])
    pw = packed_to_device(g, "nf4", codes, scales, scales2, 4, 64, 128)
    r = g.route(torch.zeros((0, 1), dtype=torch.int32, device="cuda"), 4)
    dA = torch.full((1, 128), SENTINEL, dtype=torch.float32, device="cuda")
    g.grouped_gemm_dx(pw, torch.zeros((1, 64), dtype=torch.int16, device="cuda"), r, 0, 1, dA=dA)
    torch.cuda.synchronize()
    assert torch.all(dA == SENTINEL)


# ------------------------------------------------------------ full sizes

SAMPLES = 1024
FULL = [(name, proj.name, T)
        for name in ("olmoe", "qwen30", "qwen235", "gptoss", "mixtral")
        for proj in synth.CONFIGS[name].projs
        for T in synth.CONFIGS[name].Ts]

_cache = {}


def packed_layer(name, projname):
    key = (name, projname)
    if key not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        cfg = synth.CONFIGS[name]
        proj = cfg.proj(projname)
        codes, scales, scales2 = synth.packed_weights(cfg, proj)
        pw = packed_to_device(gnf4(), cfg.fmt, codes, scales, scales2, cfg.E, proj.N, proj.K)
        _cache[key] = (codes, scales, scales2, pw)
    return _cache[key]


@pytest.mark.parametrize("name,projname,T", FULL, ids=lambda v: str(v))
def test_dx_fullsize_sampled(name, projname, T):
    g = gnf4()
    cfg = synth.CONFIGS[name]
    proj = cfg.proj(projname)
    E, N, K, k = cfg.E, proj.N, proj.K, cfg.k
    say("dx fullsize", name, projname, "T", T, "N", N, "K", K, cfg.fmt)
    codes, scales, scales2, pw = packed_layer(name, projname)
    ids, _ = synth.routing_inputs(cfg, T)
    dY = synth.grad_rows(cfg, T * k, N, 0, T)
    r = g.route(torch.from_numpy(ids).cuda(), E)
    dA = g.grouped_gemm_dx(pw, bits_to_device(dY), r, T, k)
    torch.cuda.synchronize()
    r_ref = routing.route(ids, E)
    check_route(r, r_ref, T * k)
    nv = int(r_ref["offsets"][-1])
    s = np.random.default_rng([cfg.config_id, proj.tensor_id, T, 21])
    p = s.integers(0, nv, size=SAMPLES)
    j = s.integers(0, K, size=SAMPLES)
    got = dA[torch.from_numpy(p).cuda(), torch.from_numpy(j).cuda()].cpu().numpy().astype(np.float64)
    ref = obwd.grouped_gemm_dx_entries(cfg.fmt, codes, scales, scales2, dY, r_ref["offsets"], N, K, p, j)
    d = got - ref
    rms = float(np.sqrt(np.mean(ref * ref)))
    max_rel = float(np.max(np.abs(d))) / rms
    frob = float(np.linalg.norm(d) / np.linalg.norm(ref))
    print("dx fullsize %s %s T=%d: max|err|/rms %.2e, rel Frobenius %.2e" % (name, projname, T, max_rel, frob))
    assert np.all(np.isfinite(got))
    assert max_rel <= DX_MAX_REL_RMS and frob <= DX_FROB_REL, (max_rel, frob)
