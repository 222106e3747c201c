"""gnf4_route_noalloc (the route's workspace in the library's static device
array, for callers that cannot allocate) gives what gnf4_route with a caller
workspace gives, bit for bit, on two calls in a row, the second smaller
than the first (the array keeps the first call's contents); the one-
workgroup sizes need no workspace at all; and a need beyond the array is
refused before any launch."""

import numpy as np
import pytest
import torch

from oracle import routing

from .gpu_util import check_route, gnf4, say

pytestmark = pytest.mark.gpu

KEYS = ("counts", "offsets", "perm", "inv", "active", "n_active", "bad")


def same(a, b):
    for key in KEYS:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("E,T1,T2,k", [
    (128, 4096, 300, 8),      # 32 chunks, then 3 chunks over stale array contents
    (1024, 2000, 129, 8),     # 1024 experts: 16 chunks, then 2
    (64, 500, 100, 8),        # 4 chunks, then one workgroup (no workspace)
])
def test_noalloc_route_equals_route_with_workspace(E, T1, T2, k):
    g = gnf4()
    for call, T in enumerate((T1, T2)):
        ids = np.random.default_rng([E, T, k, call]).integers(-1, E + 1, size=(T, k)).astype(np.int32)
        ids_d = torch.from_numpy(ids).cuda()
        say("noalloc route", "call", call, "E", E, "T", T, "k", k,
            "workspace", g.route_workspace_bytes(T, k, E))
        r_ws = g.route(ids_d, E)
        r_na = g.route_noalloc(ids_d, E)
        torch.cuda.synchronize()
        same(r_na, r_ws)
        check_route(r_na, routing.route(ids, E), T * k)


def test_noalloc_route_refuses_more_than_its_array():
    g = gnf4()
    E, k = 1024, 64
    T = 261120 // 64 + 1                   # 261,184 assignments: 256 chunks of 1025 words
    assert g.route_workspace_bytes(T, k, E) > (1 << 20)
    assert g.route_workspace_bytes(261120 // 64, k, E) <= (1 << 20)
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    say("noalloc route refused", E, T, k)
    with pytest.raises(g.Gnf4Error) as exc:
        g.route_noalloc(ids, E)
    assert exc.value.status == 3 and "static" in str(exc.value)
