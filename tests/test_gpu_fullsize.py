"""Parity at the workloads' full sizes, in the launch configuration bench.py
times (gnf4_route on the device, then gnf4_grouped_gemm on all experts of a
projection): every routing output is compared bit for bit with the oracle's
counting sort, and a seeded sample of the GEMM outputs against the oracle's
float64 dot products of the dequantized weight row with the activation row.

Packed weights are drawn directly as stored bytes by ``synth.packed_weights``
(quantizing a whole layer with the oracle would take minutes), so both sides
read the same bytes and no expected value passes through the HIP path."""

import numpy as np
import pytest
import torch

import synth
from oracle import grouped_gemm as ogemm
from oracle import routing

from .gpu_util import bits_to_device, check_route, gnf4, oracle_pack, packed_to_device, say
from .tolerance import MAX_REL_RMS, FROB_REL

pytestmark = pytest.mark.gpu

SAMPLES = 1536

CASES = [(name, proj.name, T)
         for name in ("olmoe", "qwen30", "qwen235", "gptoss", "mixtral")
         for proj in synth.CONFIGS[name].projs
         for T in synth.CONFIGS[name].Ts]

_cache = {}


def layer(name, projname):
    """Packed weights of one projection, host and device (the last one kept)."""
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


@pytest.mark.parametrize("name,projname,T", CASES, ids=lambda v: str(v))
def test_fullsize_sampled(name, projname, T):
    g = gnf4()
    cfg = synth.CONFIGS[name]
    proj = cfg.proj(projname)
    E, N, K, k = cfg.E, proj.N, proj.K, cfg.k
    say("fullsize", name, projname, "T", T, "N", N, "K", K, cfg.fmt)
    codes, scales, scales2, pw = layer(name, projname)
    ids, _ = synth.routing_inputs(cfg, T)
    rows = T if proj.gather else T * k
    X = synth.activations(cfg, rows, K, synth.T_X if proj.gather else synth.T_X_DOWN, 0, T)

    r = g.route(torch.from_numpy(ids).cuda(), E)
    Y = g.grouped_gemm(pw, bits_to_device(X), proj.gather, r, T, k)
    torch.cuda.synchronize()
    r_ref = routing.route(ids, E)
    check_route(r, r_ref, T * k)

    # seeded sample of (routed row, output column)
    nv = int(r_ref["offsets"][-1])
    s = np.random.default_rng([cfg.config_id, proj.tensor_id, T, 11])
    p = s.integers(0, nv, size=SAMPLES)
    n = s.integers(0, N, size=SAMPLES)
    got = Y[torch.from_numpy(p).cuda(), torch.from_numpy(n).cuda()].cpu().numpy().astype(np.float64)

    expert = np.searchsorted(r_ref["offsets"], p, side="right") - 1
    src = r_ref["perm"][p] // k if proj.gather else p
    Xf = ogemm.bf16_bits_to_f64(X)
    ref = np.empty(SAMPLES)
    for e in np.unique(expert):
        sel = np.nonzero(expert == e)[0]
        cols, inv = np.unique(n[sel], return_inverse=True)
        W = ogemm.dequant_rows(cfg.fmt, codes, scales, scales2, int(e), cols, N, K).astype(np.float64)
        ref[sel] = np.einsum("ij,ij->i", W[inv], Xf[src[sel]])
    err = got - ref
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(err)) <= MAX_REL_RMS * rms, (np.max(np.abs(err)) / rms)
    assert np.linalg.norm(err) <= FROB_REL * np.linalg.norm(ref), (np.linalg.norm(err) / np.linalg.norm(ref))


# Activations past 4 GiB: token rows beyond byte offset 2^32 are read through
# 64-bit addresses. K = 2048 bf16 values is 4 KiB per row, so tokens
# t >= 2^20 lie past 4 GiB; T = 2^20 + 77 puts 77 of them there. Rows repeat
# with period R = 4099, and 2^20 is not a multiple of R, so an address that
# wrapped at 2^32 would read a different row.
BIG = dict(E=4, N=80, K=2048, T=(1 << 20) + 77, k=1, R=4099)
_big = {}


def big_case():
    if not _big:
        c = synth.wide_layer(BIG["E"], BIG["N"], BIG["K"], BIG["T"], BIG["k"], BIG["R"], seed=3)
        _big.update(c)
        _big["route"] = routing.route(c["ids"], BIG["E"])
    return _big


@pytest.mark.parametrize("fmt,gather", [("nf4", 1), ("nf4_dq", 1), ("mxfp4", 1), ("nf4", 0)])
def test_activations_past_4gib(fmt, gather):
    g = gnf4()
    E, N, K, T, k, R = (BIG[x] for x in ("E", "N", "K", "T", "k", "R"))
    c = big_case()
    say("past 4 GiB", fmt, "gather", gather, "E", E, "N", N, "K", K, "T", T, "k", k)
    codes, scales, scales2 = oracle_pack(fmt, c["W"])
    pw = packed_to_device(g, fmt, codes, scales, scales2, E, N, K)
    rows = T if gather else T * k
    base = bits_to_device(c["X_base"])
    X = base[torch.arange(rows, device="cuda") % R]
    assert X.numel() * 2 >= 1 << 32
    del base
    r = g.route(torch.from_numpy(c["ids"]).cuda(), E)
    Y = g.grouped_gemm(pw, X, gather, r, T, k)
    torch.cuda.synchronize()
    del X
    r_ref = c["route"]
    check_route(r, r_ref, T * k)

    # every routed row whose activation row lies past 4 GiB, plus a seeded sample
    perm = r_ref["perm"]
    src_of = perm // k if gather else np.arange(T * k)
    far = np.nonzero(src_of >= (1 << 32) // (2 * K))[0]
    s = np.random.default_rng([BIG["T"], 17, gather])
    p = np.concatenate([np.repeat(far, N), s.integers(0, T * k, size=SAMPLES)])
    n = np.concatenate([np.tile(np.arange(N), far.size), s.integers(0, N, size=SAMPLES)])
    got = Y[torch.from_numpy(p).cuda(), torch.from_numpy(n).cuda()].cpu().numpy().astype(np.float64)
    expert = np.searchsorted(r_ref["offsets"], p, side="right") - 1
    Xf = ogemm.bf16_bits_to_f64(c["X_base"])[src_of[p] % R]
    ref = np.empty(p.size)
    for e in np.unique(expert):
        sel = np.nonzero(expert == e)[0]
        W = ogemm.dequant_rows(fmt, codes, scales, scales2, int(e), np.arange(N), N, K).astype(np.float64)
        ref[sel] = np.einsum("ij,ij->i", W[n[sel]], Xf[sel])
    err = got - ref
    rms = np.sqrt(np.mean(ref ** 2))
    assert far.size == 77 * k
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(err)) <= MAX_REL_RMS * rms, (np.max(np.abs(err)) / rms)
    assert np.linalg.norm(err) <= FROB_REL * np.linalg.norm(ref), (np.linalg.norm(err) / np.linalg.norm(ref))
