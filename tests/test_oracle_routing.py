"""Pins of the oracle's routing against numpy primitives and invariants."""

import numpy as np
import pytest

import synth
from oracle import routing


def check_against_numpy(ids, E):
    r = routing.route(ids, E)
    flat = np.asarray(ids).reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    assert np.array_equal(r["counts"], counts)
    assert np.array_equal(r["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    # stable argsort of the ids, with dropped ids sent past the end
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")
    nv = int(valid.sum())
    assert np.array_equal(r["perm"][:nv], order[:nv])
    assert np.all(r["perm"][nv:] == -1)
    inv = np.full(flat.size, -1)
    inv[order[:nv]] = np.arange(nv)
    assert np.array_equal(r["inv"], inv)
    act = np.nonzero(counts)[0]
    assert r["n_active"][0] == act.size
    assert np.array_equal(r["active"][:act.size], act)
    assert np.all(r["active"][act.size:] == -1)
    assert r["bad"][0] == int(not valid.all())
    # invariants
    for e in range(E):
        seg = r["perm"][r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)
    for p in range(nv):
        assert r["inv"][r["perm"][p]] == p
    return r


@pytest.mark.parametrize("name,T", [("tiny", 16), ("olmoe", 1), ("olmoe", 512), ("qwen30", 8),
                                    ("qwen30", 2048), ("gptoss", 1), ("mixtral", 2048)])
def test_route_workloads(name, T):
    cfg = synth.CONFIGS[name]
    ids, _ = synth.routing_inputs(cfg, T)
    check_against_numpy(ids, cfg.E)


def test_zipf_skew():
    cfg = synth.CONFIGS["qwen30"]
    ids, _ = synth.routing_inputs(cfg, 2048)
    r = routing.route(ids, cfg.E)
    assert int(np.argmax(r["counts"])) == 0         # expert 0 is the hottest
    assert r["counts"][0] > 1500                     # heavily skewed
    assert 100 <= r["n_active"][0] <= 128


def test_bad_ids_and_duplicates():
    ids = np.array([[0, 0], [3, -1], [7, 2], [2, 9]], dtype=np.int32)
    r = check_against_numpy(ids, 8)
    assert r["bad"][0] == 1
    assert r["inv"][3] == -1 and r["inv"][7] == -1
    assert r["counts"][0] == 2                       # duplicates routed twice


def test_empty_and_single_expert():
    r = routing.route(np.zeros((0, 4), dtype=np.int32), 16)
    assert r["offsets"].tolist() == [0] * 17 and r["n_active"][0] == 0
    ids = np.zeros((5, 1), dtype=np.int32)
    r = check_against_numpy(ids, 1)
    assert r["perm"].tolist() == [0, 1, 2, 3, 4]


def test_brute_force_tiny():
    g = np.random.default_rng(0)
    for _ in range(50):
        E = int(g.integers(1, 6))
        T = int(g.integers(0, 5))
        k = int(g.integers(1, 4))
        ids = g.integers(-1, E + 1, size=(T, k)).astype(np.int32)
        r = routing.route(ids, E)
        # brute force: for each expert, list the flat indices holding it
        pos = 0
        for e in range(E):
            fl = [f for f in range(T * k) if ids.reshape(-1)[f] == e]
            assert r["perm"][pos:pos + len(fl)].tolist() == fl
            pos += len(fl)
