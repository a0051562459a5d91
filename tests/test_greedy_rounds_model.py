"""CPU models of the round-based greedies the DAPD and CAP kernels run on one
wave, checked against the node-by-node scans they must reproduce (DAPD note,
key design 2: the independent set in degree x confidence order; DepCap
summary, Methodology: CAP's greedy over the candidate order).  The models
follow the kernels' steps: for DAPD, the keys sorted into rank order, an
exclusive OR scan of the ranks' node bits by an xor butterfly, each rank's set
sent back to its node, then rounds in which a node with a chosen earlier
neighbour is out at once and one whose earlier neighbours have all decided,
none chosen, is chosen; for CAP, the same rounds with forced candidates."""
import random

import pytest


def _scan_mis(n, adj, key):
    chosen = set()
    # ascending key, a NaN key after every other (it never counts anyway)
    for u in sorted(range(n), key=lambda u: (key[u][0] is None, key[u][0] or 0, u)):
        if key[u][0] is None:  # a NaN key is never chosen
            continue
        if not (adj[u] & chosen):
            chosen.add(u)
    return chosen


def _wave_mis(n, adj, key):
    lanes = range(64)
    big = (float("inf"), 1 << 40)
    k = [(float("inf") if key[u][0] is None else key[u][0], u) if u < n else big for u in lanes]
    order = sorted(lanes, key=lambda t: k[t])  # rank t holds node order[t]
    seg = [(1 << order[t]) if t < n else 0 for t in lanes]
    below = [0] * 64
    for d in (1, 2, 4, 8, 16, 32):  # exclusive OR scan, xor butterfly
        other = [seg[t ^ d] for t in lanes]
        for t in lanes:
            if t & d:
                below[t] |= other[t]
            seg[t] |= other[t]
    earlier = [0] * 64
    for t in lanes:  # rank t's set to its node's lane
        earlier[order[t] if t < n else t] = below[t]
    E = [sum(1 << w for w in adj[u]) & earlier[u] if u < n else 0 for u in lanes]
    open_ = sum(1 << u for u in range(n) if key[u][0] is not None)
    sel = 0
    while open_:
        pick = out = 0
        for u in range(n):
            if (open_ >> u) & 1:
                if E[u] & sel:
                    out |= 1 << u
                elif not (E[u] & open_):
                    pick |= 1 << u
        assert pick | out, "every round decides the lowest undecided node"
        sel |= pick
        open_ &= ~(pick | out)
    return {u for u in range(n) if (sel >> u) & 1}


def _scan_cap(k, conflicts, forced):
    s = set()
    for a in range(k):
        if forced[a] or not any(b in s for b in conflicts[a] if b < a):
            s.add(a)
    return s


def _rounds_cap(k, conflicts, forced):
    earlier = [sum(1 << b for b in conflicts[a] if b < a) for a in range(k)]
    open_, s = (1 << k) - 1, 0
    while open_:
        take = out = 0
        for a in range(k):
            if (open_ >> a) & 1:
                if not forced[a] and earlier[a] & s:
                    out |= 1 << a
                elif forced[a] or not (earlier[a] & open_):
                    take |= 1 << a
        assert take | out
        s |= take
        open_ &= ~(take | out)
    return {a for a in range(k) if (s >> a) & 1}


def _graph(rng, n, p):
    adj = [set() for _ in range(n)]
    for i in range(n):
        for j in range(i + 1, n):
            if rng.random() < p:
                adj[i].add(j)
                adj[j].add(i)
    return adj


@pytest.mark.parametrize("p", [0.0, 0.05, 0.3, 0.8, 1.0])
def test_single_wave_dapd_greedy_model_equals_the_scan(p):
    rng = random.Random(int(p * 1000) + 7)
    for _ in range(150):
        n = rng.randint(1, 64)
        adj = _graph(rng, n, p)
        vals = rng.sample(range(1 << 20), n)
        key = [(None if rng.random() < 0.05 else vals[u], u) for u in range(n)]
        assert _wave_mis(n, adj, key) == _scan_mis(n, adj, key)


@pytest.mark.parametrize("p", [0.0, 0.02, 0.2, 0.9])
def test_cap_rounds_model_equals_the_scan(p):
    rng = random.Random(int(p * 1000) + 11)
    for _ in range(120):
        k = rng.randint(1, 128)
        conflicts = _graph(rng, k, p)
        forced = [rng.random() < 0.3 for _ in range(k)]
        assert _rounds_cap(k, conflicts, forced) == _scan_cap(k, conflicts, forced)
