"""The dequantize-then-matmul comparison path that bench.py times against the
fused kernel: its step (route, bf16 decode of the routed experts, torch's
library GEMMs, combine) computes the same layer step as the oracle, on the
batched T = 1 path and on the per-expert path.

The comparison path multiplies bf16-rounded weights and writes bf16 GEMM
outputs, so each output carries up to two bf16 roundings (2^-8 relative);
its bar is a sanity bar, max|err| <= 5e-2 * rms and relative Frobenius
<= 1e-2, not the product's."""

import numpy as np
import pytest
import torch

import bench
import synth
from oracle import combine as ocombine
from oracle import grouped_gemm as ogemm
from oracle import routing

from .gpu_util import gnf4, oracle_pack, packed_to_device, say
from .tolerance import errors

pytestmark = pytest.mark.gpu


class PackedLayer:
    def __init__(self, cfg, projs):
        self.cfg = cfg
        self.projs = projs


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
@pytest.mark.parametrize("T", [1, 40])
def test_dequant_path_step_matches_oracle(fmt, T):
    g = gnf4()
    cfg = synth.Config("mini", 90, 8, 2, 256, 128, fmt, (1, 40), "normal",
                       (synth.Proj("gate_up", 256, 256, synth.T_W_GATE_UP, 1),
                        synth.Proj("down", 256, 128, synth.T_W_DOWN, 0)))
    packs = []
    pws = []
    for proj in cfg.projs:
        W = synth.layer_weight(cfg, proj)
        c, s, s2 = oracle_pack(fmt, W)
        packs.append((c, s, s2))
        pws.append(packed_to_device(g, fmt, c, s, s2, cfg.E, proj.N, proj.K))
    layer = PackedLayer(cfg, pws)
    ms = min(cfg.E, T * cfg.k)
    wbuf = [torch.empty((ms, p.N, p.K), dtype=torch.int16, device="cuda") for p in pws]
    say("dequant path", fmt, "T", T)
    slot = bench.DequantSlot(torch, g, cfg, layer, T, 7, wbuf)
    slot.run(g)
    torch.cuda.synchronize()
    out = slot.out.cpu().numpy()[:T]

    ids, tw = synth.routing_inputs(cfg, T, seed=7)          # the slot's own inputs
    r = routing.route(ids, cfg.E)
    down = cfg.projs[1]
    c, s, s2 = packs[1]
    Xd = synth.activations(cfg, T * cfg.k, down.K, synth.T_X_DOWN, 7, T)
    Y = ogemm.grouped_gemm(fmt, c, s, s2, Xd, 0, r["offsets"], r["perm"], cfg.k, down.N, down.K)
    ref = ocombine.combine(Y, r["inv"], tw, T, cfg.k)
    max_rel, frob = errors(out, ref)
    assert max_rel <= 5e-2 and frob <= 1e-2, (max_rel, frob)
