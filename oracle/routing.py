"""Routing of top-k assignments into per-expert row segments (oracle).

TEST INFRASTRUCTURE (see the package docstring): never imported by the GPU path.

The pages run one launch for all active experts (Jordan Anderson,
jordananderson-pages.pages.dev, section "grouped-nf4-gemm & experts-4bit",
first bullet) behind a real router (same bullet's demonstration paragraph),
but never describe how rows are grouped. Reading taken: a counting sort of the
flat assignment list f = t*k + j by expert id:

* counts[e]   number of valid assignments with id e;
* offsets     exclusive prefix sum, offsets[0] = 0, offsets[E] = valid total;
* perm[p]     for p in [offsets[e], offsets[e+1]) the flat indices f with
              id e, in ascending f (stable); perm[p] = -1 for p >= offsets[E];
* inv[f]      the p with perm[p] = f, or -1 for a dropped assignment;
* active      ascending e with counts[e] > 0, then -1 padding; n_active;
* bad         1 if any id lies outside [0, E) (those entries are dropped).

Written as the plain counting sort with Python loops (sizes here are at most
a few tens of thousands of assignments). Parity: pinned (numpy bincount,
cumsum and stable argsort; permutation invariants; brute force on tiny cases).
"""

import numpy as np


def route(topk_ids, E):
    """Counting-sort routing of topk_ids [T, k] (int) over E experts.

    Returns a dict of int32 numpy arrays: counts [E], offsets [E+1],
    perm [T*k], inv [T*k], active [E], n_active [1], bad [1].
    """
    ids = np.asarray(topk_ids).reshape(-1)
    n = ids.size
    counts = [0] * E
    bad = 0
    for f in range(n):
        e = int(ids[f])
        if 0 <= e < E:
            counts[e] += 1
        else:
            bad = 1
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E]
    cursor = list(cursor)
    perm = [-1] * n
    inv = [-1] * n
    for f in range(n):                      # ascending f keeps each segment stable
        e = int(ids[f])
        if 0 <= e < E:
            p = cursor[e]
            perm[p] = f
            inv[f] = p
            cursor[e] += 1
    active = [e for e in range(E) if counts[e] > 0]
    n_active = len(active)
    active = active + [-1] * (E - n_active)
    as32 = lambda v: np.asarray(v, dtype=np.int32)
    return {
        "counts": as32(counts),
        "offsets": as32(offsets),
        "perm": as32(perm),
        "inv": as32(inv),
        "active": as32(active),
        "n_active": as32([n_active]),
        "bad": as32([bad]),
    }
