"""Pins of the layer oracle (router top-k with softmax weights, SwiGLU, bf16
rounding) against brute force, closed forms and an independent rounding."""

import math

import numpy as np
import pytest

import synth
from oracle import layer


def brute_rank_order(row):
    """Experts in rank order, ranks counted directly: rank(e) = #{e' with a
    larger logit} + #{e' < e with an equal logit}, NaN below every number."""
    E = len(row)

    def greater(a, b):                     # a ranks above b (ignoring ids)
        if math.isnan(a):
            return False
        if math.isnan(b):
            return True
        return a > b

    def equal(a, b):
        return (math.isnan(a) and math.isnan(b)) or a == b

    rank = []
    for e in range(E):
        r = sum(1 for f in range(E) if greater(row[f], row[e]))
        r += sum(1 for f in range(e) if equal(row[f], row[e]))
        rank.append(r)
    assert sorted(rank) == list(range(E))
    return [rank.index(i) for i in range(E)]


@pytest.mark.parametrize("k", [1, 3, 6])
def test_topk_matches_brute_force_ranks_with_ties(k):
    g = np.random.default_rng(5)
    logits = g.integers(-2, 3, size=(60, 6)).astype(np.float32)   # many ties
    logits[3, 2] = np.nan
    logits[7, :] = np.nan
    ids, w = layer.topk_softmax(logits, k)
    for t in range(logits.shape[0]):
        assert list(ids[t]) == brute_rank_order([float(v) for v in logits[t]])[:k]


def test_topk_weights_closed_form_two_experts():
    a, b = 1.25, -0.5
    ids, w = layer.topk_softmax(np.array([[b, a, -7.0]], dtype=np.float32), 2)
    assert list(ids[0]) == [1, 0]
    p = 1.0 / (1.0 + math.exp(b - a))                     # logistic of the gap
    assert abs(float(w[0, 0]) - p) <= 2 ** -24 and abs(float(w[0, 1]) - (1.0 - p)) <= 2 ** -25


def test_topk_weights_sum_to_one_and_shift_invariant():
    g = np.random.default_rng(6)
    logits = g.integers(-40, 40, size=(50, 16)).astype(np.float32) / np.float32(8)
    ids, w = layer.topk_softmax(logits, 4)
    assert np.all(w > 0)
    assert np.allclose(w.astype(np.float64).sum(axis=1), 1.0, atol=4e-7)
    ids2, w2 = layer.topk_softmax(logits + np.float32(3.0), 4)   # exact shift
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2)


def test_topk_all_experts_is_the_full_softmax():
    g = np.random.default_rng(7)
    logits = g.standard_normal((20, 9)).astype(np.float32)
    ids, w = layer.topk_softmax(logits, 9)
    for t in range(20):
        x = logits[t].astype(np.float64)
        assert list(ids[t]) == list(np.argsort(-x, kind="stable"))
        full = np.exp(x - x.max()) / np.exp(x - x.max()).sum()
        assert np.allclose(w[t], full[ids[t]], rtol=2e-7, atol=0)


def test_topk_nan_ranks_last_in_ascending_id():
    logits = np.array([[np.nan, 1.0, np.nan, 0.0]], dtype=np.float32)
    ids, w = layer.topk_softmax(logits, 3)
    assert list(ids[0]) == [1, 3, 0]
    assert np.isnan(w[0]).all()            # a NaN in the chosen set poisons the softmax


def test_bf16_rounding_fixes_every_bf16_value():
    bits = np.arange(1 << 16, dtype=np.uint32)
    vals = (bits << 16).astype(np.uint32).view(np.float32)
    keep = ~np.isnan(vals)
    got = layer.f64_to_bf16_bits(vals[keep].astype(np.float64))
    assert np.array_equal(got, bits[keep].astype(np.uint16))


def test_bf16_rounding_halfway_cases_go_to_even():
    # consecutive positive bf16 values a < b (same binade), halfway point exact in float64
    g = np.random.default_rng(8)
    lo = g.integers(0x0080, 0x7F7F, size=2000).astype(np.uint32)
    a = (lo << 16).view(np.float32).astype(np.float64)
    b = ((lo + 1) << 16).view(np.float32).astype(np.float64)
    got = layer.f64_to_bf16_bits((a + b) / 2)
    expect = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(got, expect)
    # just off the halfway point the nearer neighbour wins
    assert np.array_equal(layer.f64_to_bf16_bits((a + b) / 2 + (b - a) * 1e-6), (lo + 1).astype(np.uint16))
    assert np.array_equal(layer.f64_to_bf16_bits(-((a + b) / 2 - (b - a) * 1e-6)),
                          (lo | 0x8000).astype(np.uint16))


def test_bf16_rounding_matches_float32_rounding_on_float32_inputs():
    # a float32 input has at most 24 significant bits, so rounding it to bf16
    # directly and through the generator's integer rounding trick must agree
    g = np.random.default_rng(9)
    x = (g.standard_normal(200000) * np.exp(g.uniform(-60, 60, 200000))).astype(np.float32)
    assert np.array_equal(layer.f64_to_bf16_bits(x.astype(np.float64)), synth.f32_to_bf16_bits(x))


def test_bf16_rounding_edges():
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127                   # largest finite bf16
    assert layer.f64_to_bf16_bits([big])[0] == 0x7F7F
    assert layer.f64_to_bf16_bits([(2.0 - 2.0 ** -8) * 2.0 ** 127])[0] == 0x7F80   # halfway -> even = inf
    assert layer.f64_to_bf16_bits([2.0 ** -133])[0] == 0x0001                        # smallest subnormal
    assert layer.f64_to_bf16_bits([2.0 ** -134])[0] == 0x0000                        # halfway -> even = 0
    assert layer.f64_to_bf16_bits([-0.0])[0] == 0x8000
    assert layer.f64_to_bf16_bits([np.nan])[0] == 0x7FC0


def test_swiglu_closed_forms():
    I = 5
    g = np.array([[0.0, 1.0, -1.0, 50.0, -50.0]])
    up_one = np.concatenate([g, np.ones_like(g)], axis=1)
    H = layer.swiglu(up_one, I)
    # silu(0) = 0, silu(1) = 1/(1 + 1/e), silu(-1) = -1/(1 + e), silu(50) = 50 to
    # far below a bf16 ulp, silu(-50) = -50 e^-50 (tiny, negative)
    s1 = 1.0 / (1.0 + math.exp(-1.0))
    sm1 = -1.0 / (1.0 + math.e)
    expect = [0x0000, int(layer.f64_to_bf16_bits([s1])[0]), int(layer.f64_to_bf16_bits([sm1])[0]),
              0x4248, int(layer.f64_to_bf16_bits([-50.0 * math.exp(-50.0)])[0])]
    assert list(H[0]) == expect
    assert H[0, 1] == 0x3F3B                               # 0.7310... -> 187 / 256
    assert H[0, 4] & 0x8000                                # negative
    # up = 0 gives +-0, and the gate and up halves are not swapped
    H0 = layer.swiglu(np.concatenate([g, np.zeros_like(g)], axis=1), I)
    assert np.all((H0 & 0x7FFF) == 0)
    Hs = layer.swiglu(np.concatenate([np.ones_like(g), g], axis=1), I)
    assert list(Hs[0]) == list(layer.f64_to_bf16_bits(s1 * g[0]))
