"""Parity at the workloads' full sizes, through the entry points bench.py
times, with EVERY output element compared against the float64 oracle.

Per workload, projection and token count:
  gate_up  gnf4_route_grouped_gemm (one launch at T = 1: the routing is fused
           into the one-token GEMV; route + grouped GEMM launches otherwise)
  down     gnf4_grouped_gemm_combine on the routed-order input (one launch
           at T = 1 that never writes Y; grouped GEMM + combine otherwise,
           where Y is checked as well)
and, at T = 1, the whole FFN decode step of bench.py's ffn_layer leg:
  gnf4_route_logits_grouped_gemm (router top-k and softmax weights, routing,
  gate_up with the SwiGLU epilogue, one launch) then gnf4_grouped_gemm_combine
  on the bf16 H.

Routing outputs, top-k ids and weights are compared bit for bit; every
element of Y, H and out against the oracle's float64 results at the bars of
tests/tolerance.py (per call; the H bar for the SwiGLU output and the layer
bar for the output of the chained layer). The oracle's grouped GEMM dequantizes each routed expert in
full and multiplies it with the gathered rows in float64, so a fault
confined to one tile (the last M tile of the hottest expert, the last N tile
at N = 2880 or 5760, one XCD's share of the grid) shows in its elements.

Packed weights are drawn directly as stored bytes by ``synth.packed_weights``
(quantizing a whole layer with the oracle would take minutes), so both sides
read the same bytes and no expected value passes through the HIP path."""

import numpy as np
import pytest
import torch

import synth
from oracle import combine as ocombine
from oracle import grouped_gemm as ogemm
from oracle import layer as olayer
from oracle import routing

from .gpu_util import bits_to_device, check_route, gnf4, packed_to_device, say
from .tolerance import assert_within, assert_within_h, assert_within_layer

pytestmark = pytest.mark.gpu

NAMES = ("olmoe", "qwen30", "qwen235", "gptoss", "mixtral")

# grouped by workload so that each layer's bytes are drawn once
CASES = []
for _name in NAMES:
    _cfg = synth.CONFIGS[_name]
    for _T in _cfg.Ts:
        for _proj in _cfg.projs:
            CASES.append((_name, _proj.name, _T))
    if min(_cfg.Ts) == 1:
        CASES.append((_name, "ffn_decode", 1))

_cache = {}


def layer(name):
    """Packed weights of both projections of a workload, host and device (the
    last workload is kept)."""
    if name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        cfg = synth.CONFIGS[name]
        out = {}
        for proj in cfg.projs:
            codes, scales, scales2 = synth.packed_weights(cfg, proj)
            pw = packed_to_device(gnf4(), cfg.fmt, codes, scales, scales2, cfg.E, proj.N, proj.K)
            out[proj.name] = (codes, scales, scales2, pw)
        _cache[name] = out
    return _cache[name]


def oracle_y(cfg, proj, packed, X, gather, r_ref):
    codes, scales, scales2 = packed[:3]
    return ogemm.grouped_gemm(cfg.fmt, codes, scales, scales2, X, gather, r_ref["offsets"],
                              r_ref["perm"], cfg.k, proj.N, proj.K)


def report(what, errs):
    print("%s: max|err|/rms %.3e, rel Frobenius %.3e" % ((what,) + tuple(errs)), flush=True)


@pytest.mark.parametrize("name,what,T", CASES, ids=lambda v: str(v))
def test_fullsize_every_element(name, what, T):
    g = gnf4()
    cfg = synth.CONFIGS[name]
    E, k = cfg.E, cfg.k
    packs = layer(name)
    say("fullsize", name, what, "T", T, cfg.fmt)
    if what == "ffn_decode":
        ffn_decode(g, cfg, packs)
        return
    proj = cfg.proj(what)
    N, K = proj.N, proj.K
    codes, scales, scales2, pw = packs[what]
    ids, tw = synth.routing_inputs(cfg, T)
    ids_d = torch.from_numpy(ids).cuda()
    r_ref = routing.route(ids, E)
    nv = int(r_ref["offsets"][-1])
    if proj.gather:
        X = synth.activations(cfg, T, K, synth.T_X, 0, T)
        r, Y = g.route_grouped_gemm(ids_d, pw, bits_to_device(X))
        torch.cuda.synchronize()
        check_route(r, r_ref, T * k)
        Y = Y.cpu().numpy()[:nv]
        Y_ref = oracle_y(cfg, proj, packs[what], X, 1, r_ref)[:nv]
        report("%s %s T=%d Y" % (name, what, T), assert_within(Y, Y_ref, "%s %s T=%d" % (name, what, T)))
        return
    X = synth.activations(cfg, T * k, K, synth.T_X_DOWN, 0, T)
    r = g.route(ids_d, E)
    Ybuf = torch.full((T * k, N), float("nan"), dtype=torch.float32, device="cuda")
    out = g.grouped_gemm_combine(pw, bits_to_device(X), r, torch.from_numpy(tw).cuda(), T, k, Y=Ybuf)
    torch.cuda.synchronize()
    check_route(r, r_ref, T * k)
    Y_ref = oracle_y(cfg, proj, packs[what], X, 0, r_ref)
    if T > 1:                                   # two launches: Y is written too
        report("%s %s T=%d Y" % (name, what, T),
               assert_within(Ybuf.cpu().numpy()[:nv], Y_ref[:nv], "%s %s T=%d Y" % (name, what, T)))
    else:                                       # one launch: Y is never written
        assert torch.isnan(Ybuf).all().item(), "the one-launch path wrote Y"
    out_ref = ocombine.combine(Y_ref, r_ref["inv"], tw, T, k)
    report("%s %s T=%d out" % (name, what, T),
           assert_within(out.cpu().numpy()[:T], out_ref, "%s %s T=%d out" % (name, what, T)))


def ffn_decode(g, cfg, packs):
    """One token through the two launches of bench.py's FFN decode step."""
    E, k, I = cfg.E, cfg.k, cfg.inter
    gu, dn = cfg.proj("gate_up"), cfg.proj("down")
    logits = synth.router_logits(cfg, 1).astype(np.float32)
    X = synth.activations(cfg, 1, gu.K, synth.T_X, 0, 1)
    lg = torch.from_numpy(logits).cuda()
    Xd = bits_to_device(X)

    # the router and the routing, and gate_up as float32 Y
    ids_ref, w_ref = olayer.topk_softmax(logits, k)
    r_ref = routing.route(ids_ref, E)
    nv = int(r_ref["offsets"][-1])
    r1, Y = g.route_logits_grouped_gemm(lg, k, packs["gate_up"][3], Xd)
    # with the SwiGLU epilogue: bf16 H, then down + combine on H
    r2, H = g.route_logits_grouped_gemm(lg, k, packs["gate_up"][3], Xd, swiglu=True)
    out = g.grouped_gemm_combine(packs["down"][3], H, r2, r2["topk_w"], 1, k)
    torch.cuda.synchronize()
    for r in (r1, r2):
        assert np.array_equal(r["topk_ids"].cpu().numpy(), ids_ref), "top-k ids"
        assert np.array_equal(r["topk_w"].cpu().numpy().view(np.uint32), w_ref.view(np.uint32)), \
            "top-k weights"
        check_route(r, r_ref, k)
    Y_ref = oracle_y(cfg, gu, packs["gate_up"], X, 1, r_ref)
    report("%s ffn gate_up Y" % cfg.name, assert_within(Y.cpu().numpy()[:nv], Y_ref[:nv], "gate_up Y"))
    H_ref = olayer.swiglu(Y_ref[:nv], I)
    Hg = (H.cpu().numpy().view(np.uint16)[:nv].astype(np.uint32) << 16).view(np.float32)
    Hr = (H_ref.astype(np.uint32) << 16).view(np.float32)
    report("%s ffn H" % cfg.name, assert_within_h(Hg, Hr, "SwiGLU H"))
    Y2_ref = oracle_y(cfg, dn, packs["down"], H_ref, 0, r_ref)
    out_ref = ocombine.combine(Y2_ref, r_ref["inv"], w_ref, 1, k)
    report("%s ffn out" % cfg.name, assert_within_layer(out.cpu().numpy()[:1], out_ref, "layer out"))


# Activations past 4 GiB: token rows beyond byte offset 2^32 are read through
# 64-bit addresses. K = 2048 bf16 values is 4 KiB per row, so tokens
# t >= 2^20 lie past 4 GiB; T = 2^20 + 77 puts 77 of them there. Rows repeat
# with period R = 4099, and 2^20 is not a multiple of R, so an address that
# wrapped at 2^32 would read a different row.
BIG = dict(E=4, N=80, K=2048, T=(1 << 20) + 77, k=1, R=4099)
SAMPLES = 1536
_big = {}


def big_case():
    if not _big:
        c = synth.wide_layer(BIG["E"], BIG["N"], BIG["K"], BIG["T"], BIG["k"], BIG["R"], seed=3)
        _big.update(c)
        _big["route"] = routing.route(c["ids"], BIG["E"])
    return _big


@pytest.mark.parametrize("fmt,gather", [("nf4", 1), ("nf4_dq", 1), ("mxfp4", 1), ("nf4", 0)])
def test_activations_past_4gib(fmt, gather):
    """Every routed row whose activation row lies past 4 GiB in full, plus a
    seeded sample of the other 2^20 rows (the rows repeat with period R, so
    the sample stands for rows the element-wise tests cover at other sizes)."""
    from .gpu_util import oracle_pack
    from .tolerance import FROB_REL, MAX_REL_RMS
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
