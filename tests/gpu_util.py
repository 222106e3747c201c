"""Helpers shared by the GPU parity tests: oracle packing, device upload,
comparison against the oracle. Inputs come from the seeded generators in
``synth``; expected values come only from ``oracle``."""

import hashlib
import sys

import numpy as np
import pytest
import torch

from oracle import combine as ocombine
from oracle import grouped_gemm as ogemm
from oracle import mxfp4, nf4, routing

from .tolerance import assert_within

FMT_ID = {"nf4": 0, "nf4_dq": 1, "mxfp4": 2}


def gnf4():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible to torch")
    from bit_mixture_experts_topk_amd import gnf4 as g
    g.lib()
    return g


def say(*args):
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def oracle_pack(fmt, W):
    """(codes, scales, scales2) as numpy, from the oracle's quantizers."""
    if fmt == "nf4":
        c, s = nf4.quantize(W)
        return c, s, None
    if fmt == "nf4_dq":
        return nf4.quantize_dq(W)
    c, s = mxfp4.quantize(W)
    return c, s, None


def packed_to_device(g, fmt, codes, scales, scales2, E, N, K):
    dev = "cuda"
    c = torch.from_numpy(np.ascontiguousarray(codes).reshape(E, N, K // 2)).to(dev)
    s = torch.from_numpy(np.ascontiguousarray(scales)).to(dev).reshape(E, N, -1)
    s2 = torch.from_numpy(np.ascontiguousarray(scales2)).to(dev) if scales2 is not None else None
    return g.PackedWeights(FMT_ID[fmt], E, N, K, c, s, s2)


def bits_to_device(X):
    return torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).to("cuda")


def sha(t):
    return hashlib.sha256(t.detach().cpu().numpy().tobytes()).hexdigest()


def check_route(r_gpu, r_ref, n):
    for key in ("counts", "offsets", "active", "n_active"):
        assert np.array_equal(r_gpu[key].cpu().numpy(), r_ref[key]), key
    assert int(r_gpu["bad"].item()) == int(r_ref["bad"][0])
    if n:
        assert np.array_equal(r_gpu["perm"].cpu().numpy(), r_ref["perm"]), "perm"
        assert np.array_equal(r_gpu["inv"].cpu().numpy(), r_ref["inv"]), "inv"


def run_layer_call(g, fmt, W, X, ids, gather, k, what=""):
    """Route + grouped GEMM on the GPU vs oracle; returns (Y_gpu, Y_ref, r_ref)."""
    E, N, K = W.shape
    T = ids.shape[0]
    codes, scales, scales2 = oracle_pack(fmt, W)
    pw = packed_to_device(g, fmt, codes, scales, scales2, E, N, K)
    r_ref = routing.route(ids, E)
    say(what, fmt, "E", E, "N", N, "K", K, "T", T, "k", k, "gather", gather)
    ids_d = torch.from_numpy(ids).to("cuda")
    r = g.route(ids_d, E)
    Xd = bits_to_device(X)
    before = sha(pw.codes)
    Y = g.grouped_gemm(pw, Xd, gather, r, T, k)
    torch.cuda.synchronize()
    assert sha(pw.codes) == before, "packed weights modified"
    check_route(r, r_ref, T * k)
    Y_ref = ogemm.grouped_gemm(fmt, codes, scales, scales2, X, gather, r_ref["offsets"],
                               r_ref["perm"], k, N, K)
    return Y.cpu().numpy(), Y_ref, r_ref


def compare_rows(Y, Y_ref, r_ref, what):
    nv = int(r_ref["offsets"][-1])
    assert nv > 0
    return assert_within(Y[:nv], Y_ref[:nv], what)


def oracle_combine(Y_ref, r_ref, tw, T, k):
    return ocombine.combine(Y_ref, r_ref["inv"], tw, T, k)
