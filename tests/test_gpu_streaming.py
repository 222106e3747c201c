"""GPU checks of the expert streaming cache (gnf4_expert_cache_*):

* the residency decision of gnf4_expert_cache_stage equals the oracle model
  step by step: the whole state array, the slot ids and the copy list;
* gnf4_expert_cache_fill leaves in every occupied slot the exact packed bytes
  of its expert, read from pinned host memory;
* a layer step on the cache (route over the slot ids, grouped GEMM on the S
  cached experts, combine) gives the resident layer's output bit for bit, on
  the one-token, few-token and MFMA paths and the fused one-token calls;
* host weights in pageable memory are refused before any launch."""

import numpy as np
import pytest
import torch

import synth
from oracle.streaming import Cache

from .gpu_util import FMT_ID, bits_to_device, gnf4, oracle_pack, packed_to_device, say

pytestmark = pytest.mark.gpu


def host_packed(g, fmt, codes, scales, scales2, E, N, K):
    c = torch.from_numpy(np.ascontiguousarray(codes).reshape(E, N, K // 2)).pin_memory()
    s = torch.from_numpy(np.ascontiguousarray(scales)).reshape(E, N, -1).pin_memory()
    s2 = torch.from_numpy(np.ascontiguousarray(scales2)).pin_memory() if scales2 is not None else None
    for t in (c, s, s2):
        assert t is None or (t.is_pinned() and t.data_ptr() % 16 == 0)
    return g.PackedWeights(FMT_ID[fmt], E, N, K, c, s, s2)


def step_ids(rng, hot, E, T, k, bad):
    ids = np.where(rng.random((T, k)) < 0.5, rng.choice(hot, (T, k)),
                   rng.integers(0, E, (T, k))).astype(np.int32)
    if bad:
        ids[0, 0] = rng.choice([-1, E, E + 5])
    return ids


@pytest.mark.parametrize("E,S,T,k,steps,seed", [
    (64, 16, 1, 8, 40, 1),
    (128, 32, 1, 8, 30, 2),
    (64, 16, 2, 8, 20, 3),
    (1024, 1024, 1, 64, 10, 4),        # the largest E and S
    (1000, 700, 2, 64, 8, 5),          # S not a power of two
    (200, 50, 8, 6, 20, 6),
    (8, 2, 1, 2, 30, 7),
    (5, 5, 0, 3, 3, 8),                # T = 0: the step still advances
    (1024, 1024, 80, 64, 3, 9),        # 5120 ids: more than the 4096 a thread block holds
])
def test_stage_matches_oracle(E, S, T, k, steps, seed):
    g = gnf4()
    state = g.expert_cache_state(E, S)
    model = Cache(E, S)
    rng = np.random.default_rng([E, S, T, k, seed])
    hot = rng.choice(E, max(1, E // 4), replace=False)
    for step in range(steps):
        ids = step_ids(rng, hot, E, T, k, T > 0 and rng.random() < 0.15)
        say("cache stage E", E, "S", S, "T", T, "k", k, "step", step)
        slot_ids, copies = g.expert_cache_stage(torch.from_numpy(ids).cuda(), E, S, state)
        torch.cuda.synchronize()
        ref_ids, ref_cp = model.stage(ids.tolist())
        assert slot_ids.cpu().numpy().reshape(-1).tolist() == ref_ids
        cp = copies.cpu().numpy()
        m = int(cp[0])
        assert m == len(ref_cp)
        assert [(int(cp[1 + 2 * i]), int(cp[2 + 2 * i])) for i in range(m)] == ref_cp
        assert state.cpu().numpy().tolist() == model.words()


def cache_holds(cache, host, state, E, S):
    st = state.cpu().numpy()
    expert_of = st[1 + E:1 + E + S]
    for s, e in enumerate(expert_of):
        if e < 0:
            continue
        assert torch.equal(cache.codes[s].cpu(), host.codes[e]), ("codes", s, e)
        assert torch.equal(cache.scales[s].cpu(), host.scales[e]), ("scales", s, e)
        if host.scales2 is not None:
            per = host.scales2.numel() // E
            assert torch.equal(cache.scales2[s * per:(s + 1) * per].cpu(),
                               host.scales2[e * per:(e + 1) * per]), ("scales2", s, e)


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
@pytest.mark.parametrize("T,k,S", [(1, 4, 6), (3, 2, 6), (40, 2, 16)])
def test_streamed_layer_equals_resident(fmt, T, k, S):
    g = gnf4()
    E, N, K = 16, 256, 512
    case = synth.small_layer(E, N, K, T, k, seed=31, gather=1)
    codes, scales, scales2 = oracle_pack(fmt, case["W"])
    dev = packed_to_device(g, fmt, codes, scales, scales2, E, N, K)
    host = host_packed(g, fmt, codes, scales, scales2, E, N, K)
    cache = g.empty_packed(fmt, S, N, K)
    cache.codes.zero_()
    state = g.expert_cache_state(E, S)
    X = bits_to_device(case["X"])
    rng = np.random.default_rng([T, k, S, 5])
    hot = rng.choice(E, 4, replace=False)
    max_copies = min(T * k, E, S)
    for step in range(12):
        ids = torch.from_numpy(step_ids(rng, hot, E, T, k, step == 5)).cuda()
        tw = torch.from_numpy(rng.random((T, k)).astype(np.float32)).cuda()
        say("streamed layer", fmt, "T", T, "k", k, "S", S, "step", step)
        slot_ids, copies = g.expert_cache_stage(ids, E, S, state)
        g.expert_cache_fill(host, cache, copies, max_copies)
        r_c = g.route(slot_ids, S)
        out_c = g.combine(g.grouped_gemm(cache, X, 1, r_c, T, k), r_c["inv"], tw, T, k)
        r = g.route(ids, E)
        out = g.combine(g.grouped_gemm(dev, X, 1, r, T, k), r["inv"], tw, T, k)
        torch.cuda.synchronize()
        assert int(r_c["bad"].item()) == int(r["bad"].item()) == (1 if step == 5 else 0)
        a, b = out_c.cpu().numpy(), out.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), int((a != b).sum())
        if T == 1:
            # the fused one-token calls on the cache
            rc2, Hc = g.route_grouped_gemm(slot_ids, cache, X, swiglu=True)
            r2, H = g.route_grouped_gemm(ids, dev, X, swiglu=True)
            torch.cuda.synchronize()
            inv_c, inv = rc2["inv"].cpu().numpy(), r2["inv"].cpu().numpy()
            assert np.array_equal(inv_c < 0, inv < 0)
            keep = inv >= 0
            assert torch.equal(Hc.cpu()[torch.from_numpy(inv_c[keep]).long()],
                               H.cpu()[torch.from_numpy(inv[keep]).long()])
        cache_holds(cache, host, state, E, S)


def test_fill_refuses_pageable_host_memory():
    g = gnf4()
    E, N, K, S = 4, 16, 64, 2
    host = g.empty_packed("nf4", E, N, K, device="cpu")           # not pinned
    cache = g.empty_packed("nf4", S, N, K)
    copies = torch.zeros((5,), dtype=torch.int32, device="cuda")
    with pytest.raises(g.Gnf4Error) as ei:
        g.expert_cache_fill(host, cache, copies, 2)
    assert ei.value.status == 1 and "pinned" in str(ei.value)
