"""Seeded synthetic inputs for the grouped 4-bit MoE GEMM.

This module is the only code shared by the oracle side and the GPU side. It
holds no step of the method: it draws activations, float32 expert weights and
router outputs, and describes the workload shapes. Quantization, routing,
the GEMM and the combine live in ``oracle`` (CPU) and in the HIP library.

Workload shapes follow public model layers (no checkpoints are used):

====  ============================  =====  ===  =====  =====  =========  =================
name  shaped after                  E      k    d      I      format     T values
====  ============================  =====  ===  =====  =====  =========  =================
tiny  small single-projection layer 8      2    256    512*   nf4        16
olmoe OLMoE FFN                     64     8    2048   1024   nf4        1, 512
qwen30 Qwen3-30B-A3B FFN            128    8    2048   768    nf4_dq     1, 8, 2048
qwen235 Qwen3-235B-A22B FFN         128    8    4096   1536   nf4        1, 4096
gptoss gpt-oss-120b FFN             128    4    2880   2880   mxfp4      1, 2048
mixtral Mixtral FFN                 8      2    4096   14336  nf4        2048
====  ============================  =====  ===  =====  =====  =========  =================

(* tiny has a single projection Y = X W^T with N = 512, K = 256.)

Each FFN layer has two projections: gate_up, W [E, 2I, d] (rows [0, I) gate,
[I, 2I) up), whose input is the token activations gathered through the
routing; and down, W [E, d, I], whose input is a separate bf16 N(0,1) matrix
[T*k, I] already in routed order.

Distributions. X ~ N(0, 1) drawn in float32 and rounded to bfloat16 (round to
nearest even). Output gradients dY for the backward pass through the frozen
experts are drawn the same way ([T*k, N], routed order; the pages give no
gradient statistics, and the comparison bars are relative to the result's
own scale). W ~ N(0, 0.02) (0.02 is the standard deviation) in float32.
Router logits: N(0, 1) (tiny, qwen235, gptoss, mixtral), U(0, 1) (olmoe),
N(0, 1) plus a Zipf(1.1) bias ln(p_e), p_e proportional to (e+1)^-1.1
(qwen30, expert 0 hottest). Top-k by logit, ties to the lower expert id; the
weights are the softmax over the k selected logits, float64 then float32.

Seeds. Every tensor has its own stream
``SeedSequence([seed, config_id, tensor_id, expert])`` so that one expert's
weights can be drawn without drawing the layer.
"""

from dataclasses import dataclass, field

import numpy as np

W_STD = 0.02

# tensor ids in the seed sequence
T_X = 1
T_W_GATE_UP = 2
T_W_DOWN = 3
T_LOGITS = 4
T_X_DOWN = 5
T_W_SINGLE = 6
T_Y = 7
T_PACKED = 8
T_DY = 9


@dataclass(frozen=True)
class Proj:
    name: str
    N: int
    K: int
    tensor_id: int
    gather: int        # 1: rows gathered from token activations; 0: routed order


@dataclass(frozen=True)
class Config:
    name: str
    config_id: int
    E: int
    k: int
    d: int
    inter: int
    fmt: str
    Ts: tuple
    logits: str
    projs: tuple = field(default=())

    def proj(self, name):
        for p in self.projs:
            if p.name == name:
                return p
        raise KeyError(name)


def _ffn(name, cid, E, k, d, inter, fmt, Ts, logits):
    return Config(name, cid, E, k, d, inter, fmt, tuple(Ts), logits,
                  (Proj("gate_up", 2 * inter, d, T_W_GATE_UP, 1),
                   Proj("down", d, inter, T_W_DOWN, 0)))


CONFIGS = {
    "tiny": Config("tiny", 0, 8, 2, 256, 512, "nf4", (16,), "normal",
                   (Proj("single", 512, 256, T_W_SINGLE, 1),)),
    "olmoe": _ffn("olmoe", 1, 64, 8, 2048, 1024, "nf4", (1, 512), "uniform"),
    "qwen30": _ffn("qwen30", 2, 128, 8, 2048, 768, "nf4_dq", (1, 8, 2048), "normal_zipf"),
    "qwen235": _ffn("qwen235", 3, 128, 8, 4096, 1536, "nf4", (1, 4096), "normal"),
    "gptoss": _ffn("gptoss", 4, 128, 4, 2880, 2880, "mxfp4", (1, 2048), "normal"),
    "mixtral": _ffn("mixtral", 5, 8, 2, 4096, 14336, "nf4", (2048,), "normal"),
}


def rng(seed, config_id, tensor_id, expert=0, extra=0):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([seed, config_id, tensor_id, expert, extra])))


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest even), returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def grad_rows(cfg, rows, N, seed=0, extra=0):
    """bf16 bits [rows, N] of N(0,1) output gradients in routed order."""
    return activations(cfg, rows, N, T_DY, seed, extra)


def activations(cfg, rows, K, tensor_id=T_X, seed=0, extra=0):
    """bf16 bits [rows, K] of N(0,1) activations."""
    g = rng(seed, cfg.config_id, tensor_id, 0, extra)
    return f32_to_bf16_bits(g.standard_normal((rows, K), dtype=np.float32))


def expert_weight(cfg, proj, e, seed=0, rows=None):
    """float32 [N, K] weights of expert e for projection proj, ~N(0, 0.02).

    rows: optional (lo, hi) to return only rows [lo, hi) (drawn identically).
    """
    g = rng(seed, cfg.config_id, proj.tensor_id, e)
    w = g.standard_normal((proj.N, proj.K), dtype=np.float32)
    w *= np.float32(W_STD)
    if rows is not None:
        w = w[rows[0]:rows[1]]
    return w


def layer_weight(cfg, proj, seed=0):
    """float32 [E, N, K] weights of every expert (small configs only)."""
    return np.stack([expert_weight(cfg, proj, e, seed) for e in range(cfg.E)])


def router_logits(cfg, T, seed=0):
    g = rng(seed, cfg.config_id, T_LOGITS, 0, T)
    if cfg.logits == "uniform":
        return g.uniform(0.0, 1.0, (T, cfg.E))
    z = g.standard_normal((T, cfg.E))
    if cfg.logits == "normal_zipf":
        p = (np.arange(cfg.E) + 1.0) ** -1.1
        p /= p.sum()
        z = z + np.log(p)[None, :]
    return z


def topk(logits, k):
    """(ids int32 [T, k], weights float32 [T, k]); ties go to the lower id."""
    logits = np.asarray(logits, dtype=np.float64)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits, order, axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    w = ex / ex.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def routing_inputs(cfg, T, seed=0):
    return topk(router_logits(cfg, T, seed), cfg.k)


def down_inputs(cfg, T, seed=0):
    """bf16 bits [T*k, I]: the second projection's input in routed order."""
    return activations(cfg, T * cfg.k, cfg.inter, T_X_DOWN, seed, extra=T)


def token_inputs(cfg, T, seed=0):
    """bf16 bits [T, d]: token activations for the first projection."""
    K = cfg.projs[0].K
    return activations(cfg, T, K, T_X, seed, extra=T)


def random_rows(cfg, rows, N, seed=0, extra=0):
    """float32 [rows, N] N(0,1) matrix (stand-in expert outputs for combine tests)."""
    g = rng(seed, cfg.config_id, T_Y, 0, extra)
    return g.standard_normal((rows, N), dtype=np.float32)


def small_layer(E, N, K, T, k, seed=0, distinct=True, gather=1):
    """A small seeded layer for parity tests at arbitrary shapes.

    Returns dict(W float32 [E, N, K] ~ N(0, 0.02), X bf16 bits ([T, K] when
    gather else [T*k, K]), ids int32 [T, k], tw float32 [T, k]).
    distinct: each token picks k different experts (else ids are drawn with
    replacement, so duplicates occur).
    """
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99, E, N, K, T, k])))
    W = g.standard_normal((E, N, K), dtype=np.float32) * np.float32(W_STD)
    rows = T if gather else T * k
    X = f32_to_bf16_bits(g.standard_normal((rows, K), dtype=np.float32))
    if distinct:
        ids = np.stack([g.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k))
    else:
        ids = g.integers(0, E, size=(T, k))
    tw = g.random((T, k)).astype(np.float32)
    return {"W": W, "X": X, "ids": np.asarray(ids, dtype=np.int32).reshape(T, k), "tw": tw}


def wide_layer(E, N, K, T, k, R, seed=0):
    """A layer whose activation tensor is too large to draw on the host: R
    distinct N(0,1) rows, token t taking row t % R (the tiling is done where
    the tensor is needed), with W float32 [E, N, K] ~ N(0, 0.02) and ids
    int32 [T, k] drawn uniformly with replacement.

    Returns dict(W, X_base bf16 bits [R, K], ids)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 98, E, N, K, T, k, R])))
    W = g.standard_normal((E, N, K), dtype=np.float32) * np.float32(W_STD)
    X_base = f32_to_bf16_bits(g.standard_normal((R, K), dtype=np.float32))
    ids = g.integers(0, E, size=(T, k), dtype=np.int32)
    return {"W": W, "X_base": X_base, "ids": ids}


def packed_weights(cfg, proj, seed=0):
    """Packed weights of one projection drawn directly as stored bytes, for
    full-size parity checks where quantizing a whole layer on the CPU would
    take minutes. No quantizer is involved: every code byte is uniform over
    0..255 (all 16 codes equally likely in both nibbles), and the scales are
    drawn in the range a quantized N(0, 0.02) layer produces.

    Returns (codes uint8 [E, N, K/2], scales, scales2):
      nf4:    scales float32 [E, N, K/64] ~ U(0.02, 0.08), scales2 None
      nf4_dq: scales int8 [E, N, K/64] ~ U{1..127}, scales2 float32
              [ceil(E*N*K/64 / 256)] ~ U(2e-4, 6e-4)
      mxfp4:  scales uint8 e8m0 [E, N, K/32] ~ U{118..124} (2^-9 .. 2^-3),
              scales2 None
    """
    E, N, K = cfg.E, proj.N, proj.K
    g = rng(seed, cfg.config_id, T_PACKED, 0, proj.tensor_id)
    codes = g.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    if cfg.fmt == "nf4":
        scales = g.uniform(0.02, 0.08, size=(E, N, K // 64)).astype(np.float32)
        return codes, scales, None
    if cfg.fmt == "nf4_dq":
        scales = g.integers(1, 128, size=(E, N, K // 64), dtype=np.int8)
        groups = -(-(E * N * (K // 64)) // 256)
        scales2 = g.uniform(2e-4, 6e-4, size=groups).astype(np.float32)
        return codes, scales, scales2
    if cfg.fmt == "mxfp4":
        scales = g.integers(118, 125, size=(E, N, K // 32), dtype=np.uint8)
        return codes, scales, None
    raise ValueError("unknown format %r" % (cfg.fmt,))
