"""Pins for the oracle's selection rules: Fast-dLLM threshold, DepGA-Block
boundary, CAP-Decoding and DAPD's Welsh-Powell independent set.

Pins are hand-derived fixtures (tests/golden/, each citing its passage),
properties the pages state (progress guarantee, length clip, maximality),
brute force over all subsets on tiny inputs, and library routines
(torch fp64 log-softmax for D_ij, torch mean for the attention average,
networkx's largest-first greedy colouring for Welsh-Powell).
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- Fast-dLLM
# Fast-dLLM review, Method; Fast-dLLM notes, Key ideas / Technical details.

def test_fastdllm_hand_example(oracle):
    conf = [0.95, 0.5, 0.91, 0.3, 0.2, 0.4, 0.4, 0.1]
    so = [0, 4, 8]
    commit, n = oracle.fastdllm_select(conf, so, 0.9)
    # seq 0: 0.95 and 0.91 exceed 0.9; seq 1: none does -> top-1, ties -> lower position
    assert list(commit) == [1, 0, 1, 0, 0, 1, 0, 0]
    assert list(n) == [2, 1]


def test_fastdllm_properties(oracle):
    rng = np.random.default_rng(0)
    for trial in range(50):
        n = int(rng.integers(1, 40))
        conf = rng.random(n) ** rng.uniform(0.2, 3)
        el = (rng.random(n) < 0.7).astype(np.uint8)
        so = [0, n]
        prev = None
        for tau in (0.0, 0.3, 0.6, 0.9, 0.99, 1.5):
            commit, cnt = oracle.fastdllm_select(conf, so, tau, eligible=el)
            assert np.all(commit <= el)                       # C subset of E
            if el.any():
                assert cnt[0] >= 1                            # progress guarantee
            else:
                assert cnt[0] == 0
            if prev is not None and (conf[el == 1] > tau).any():
                assert np.all(commit <= prev)                 # shrinks as tau rises
            prev = commit
        # tau > 1: exactly one per step, the top-1 eligible (vanilla one-token decoding)
        commit, cnt = oracle.fastdllm_select(conf, so, 1.5, eligible=el)
        if el.any():
            masked = np.where(el == 1, conf, -1.0)
            assert cnt[0] == 1 and commit[int(np.argmax(masked))] == 1


def test_fastdllm_nan_never_commits(oracle):
    conf = [float("nan"), 0.2, float("nan")]
    commit, n = oracle.fastdllm_select(conf, [0, 3], 0.9)
    assert list(commit) == [0, 1, 0] and n[0] == 1
    commit, n = oracle.fastdllm_select([float("nan")], [0, 1], 0.9)
    assert list(commit) == [0] and n[0] == 0


# --------------------------------------------------------------- DepGA-Block
# DepCap page, Methodology bullets 1-3; Technical Contribution.

def _load_depcap_cases():
    cases = []
    for line in open(os.path.join(GOLDEN, "depcap_hand.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = [x.strip() for x in line.split("|")]
        cases.append(dict(
            name=f[0], I=[float(x) for x in f[1].split(",")], H=[float(x) for x in f[2].split(",")],
            r=int(f[3]), lam=float(f[4]), eps=float(f[5]), l_min=int(f[6]), l_max=int(f[7]),
            has_prev=int(f[8]), L=int(f[9]),
            S=None if f[10] == "-" else [float(x) for x in f[10].split(",")]))
    return cases


@pytest.mark.parametrize("case", _load_depcap_cases(), ids=lambda c: c["name"])
def test_depcap_hand_fixtures(oracle, case):
    n = len(case["I"])
    L, S = oracle.depcap_boundary(case["I"], case["H"], [0, n], case["l_max"], case["l_min"],
                                  case["lam"], radius=case["r"], eps=case["eps"],
                                  has_prev=[case["has_prev"]])
    assert L[0] == case["L"]
    if case["S"] is not None:
        assert np.allclose(S[:len(case["S"])], case["S"], rtol=0, atol=1e-15)


def test_depcap_properties(oracle):
    rng = np.random.default_rng(1)
    for trial in range(200):
        n = int(rng.integers(1, 200))
        I = rng.gamma(0.5, 0.2, n)
        H = rng.gamma(2.0, 2.0, n)
        l_max = int(rng.integers(1, 160))
        l_min = int(rng.integers(0, l_max + 1))
        lam = float(rng.uniform(0, 3))
        r = int(rng.integers(0, 3))
        W = min(l_max, n)
        L, S = oracle.depcap_boundary(I, H, [0, n], l_max, l_min, lam, radius=r)
        assert min(l_min, W) <= L[0] <= W
        # mean normalisation is scale-free: scaling I or H by c > 0 keeps the boundary
        for c in (0.37, 12.0):
            L2, _ = oracle.depcap_boundary(I * c, H, [0, n], l_max, l_min, lam, radius=r,
                                           eps=0.0)
            L3, _ = oracle.depcap_boundary(I, H * c, [0, n], l_max, l_min, lam, radius=r,
                                           eps=0.0)
            L1, S1 = oracle.depcap_boundary(I, H, [0, n], l_max, l_min, lam, radius=r, eps=0.0)
            near = np.any(np.abs(S1[:W]) < 1e-9)
            if not near:
                assert L2[0] == L1[0] and L3[0] == L1[0]
        # lambda = 0 with I > 0 gives the full window
        L0, _ = oracle.depcap_boundary(I + 1e-3, H, [0, n], l_max, l_min, 0.0, radius=r)
        assert L0[0] == W
        # outside the window the score is NaN
        assert np.all(np.isnan(S[W:]))


def test_depcap_multi_sequence_and_cold_start(oracle):
    I = np.concatenate([np.ones(8), np.zeros(5), np.ones(20)])
    H = np.concatenate([np.zeros(8), np.ones(5), np.ones(20)])
    so = [0, 8, 13, 33]
    L, S = oracle.depcap_boundary(I, H, so, 16, 4, 1.2, has_prev=[1, 1, 0])
    assert list(L) == [8, 4, 4]          # H=0 -> W ; I=0 -> L_min ; cold -> L_min
    assert np.all(np.isnan(S[13:]))


# -------------------------------------------------------------- CAP-Decoding
# DepCap page, Methodology bullets 4-6; Technical Contribution; AI Executive Summary.

def _read_kv(path):
    kv = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=")
            kv[k.strip()] = v.strip()
    return kv


def test_cap_hand_example(oracle):
    kv = _read_kv(os.path.join(GOLDEN, "cap_hand.txt"))
    conf = np.array([float(x) for x in kv["conf"].split(",")])
    pool, fb = oracle.cap_pool(conf, float(kv["tau_low"]), 32)
    assert list(pool) == [int(x) for x in kv["pool"].split(",")] and fb == -1
    n = len(pool)
    D = np.full((n, n), -100.0)
    pos = {r: a for a, r in enumerate(pool)}
    for pair in kv["conflicts"].split(","):
        i, j = (int(x) for x in pair.split("-"))
        D[pos[i], pos[j]] = D[pos[j], pos[i]] = -1.0
    take = oracle.cap_greedy(conf[pool], D, float(kv["tau_high"]), float(kv["gamma"]))
    chosen = sorted(int(pool[a]) for a in range(n) if take[a])
    assert chosen == [int(x) for x in kv["commit"].split(",")]


def test_cap_pool_cap_and_fallback(oracle):
    conf = np.array([0.81, 0.99, 0.85, 0.85, 0.2, 0.95, 0.9, 0.87])
    pool, fb = oracle.cap_pool(conf, 0.8, 4)
    assert list(pool) == [1, 5, 6, 7] and fb == -1            # top-4 by (conf desc, idx asc)
    pool, fb = oracle.cap_pool(conf, 0.8, 100)
    assert list(pool) == [1, 5, 6, 7, 2, 3, 0]
    pool, fb = oracle.cap_pool(conf, 0.999, 4)
    assert len(pool) == 0 and fb == 1                         # empty pool -> top-1
    el = np.array([1, 0, 1, 1, 1, 0, 0, 0], np.uint8)
    pool, fb = oracle.cap_pool(conf, 0.999, 4, eligible=el)
    assert len(pool) == 0 and fb == 2                         # ties -> lower index
    pool, fb = oracle.cap_pool(conf, 0.5, 4, eligible=np.zeros(8, np.uint8))
    assert len(pool) == 0 and fb == -1


def _brute_cap(conf, conflict, tau_high):
    """Lexicographically-first (priority order) subset that contains every
    tau_high member and has no conflicting pair other than forced-forced."""
    n = len(conf)
    forced = [a for a in range(n) if conf[a] > tau_high]
    best = None
    for bits in itertools.product((1, 0), repeat=n):      # lexicographically greatest first
        if any(bits[a] == 0 for a in forced):
            continue
        ok = True
        for a in range(n):
            for b in range(a + 1, n):
                if bits[a] and bits[b] and conflict[a][b] and not (a in forced and b in forced):
                    ok = False
                    break
            if not ok:
                break
        if ok:
            best = bits
            break
    return np.array(best, np.uint8)


def test_cap_greedy_brute_force(oracle):
    rng = np.random.default_rng(2)
    for trial in range(300):
        n = int(rng.integers(1, 12))
        conf = np.sort(rng.uniform(0.8, 1.0, n))[::-1].copy()
        conf[rng.random(n) < 0.1] = 0.97
        conf = np.sort(conf)[::-1].copy()
        D = rng.normal(-16, 4, (n, n))
        D = D + D.T
        D /= 2
        conflict = D > -16.0
        tau_high = float(rng.choice([0.9, 0.95, 1.1]))
        take = oracle.cap_greedy(conf, D, tau_high, -16.0)
        ref = _brute_cap(conf, conflict, tau_high)
        assert np.array_equal(take, ref)
        # every unselected candidate conflicts with a selected one
        for a in range(n):
            if not take[a]:
                assert any(take[b] and conflict[a][b] for b in range(n) if b != a)


def test_cap_gamma_limits(oracle):
    rng = np.random.default_rng(3)
    n = 10
    conf = np.sort(rng.uniform(0.8, 1.0, n))[::-1].copy()
    D = rng.normal(-10, 5, (n, n))
    D = (D + D.T) / 2
    assert np.all(oracle.cap_greedy(conf, D, 0.95, math.inf) == 1)          # gamma=+inf: S = P
    take = oracle.cap_greedy(conf, D, 0.95, -math.inf)                       # all conflict
    forced = conf > 0.95
    if forced.any():
        assert np.array_equal(take.astype(bool), forced)
    else:
        assert take.sum() == 1 and take[0] == 1
    conf2 = np.full(n, 0.9)
    take = oracle.cap_greedy(conf2, D, 0.95, -math.inf)
    assert take.sum() == 1 and take[0] == 1


def test_cap_dmatrix_against_torch_log_softmax(oracle):
    g = torch.Generator().manual_seed(4)
    V = 777
    x = (torch.randn(9, V, generator=g) * 2).to(torch.bfloat16)
    x[3, 5] = 30.0
    x[6, 5] = 28.0                          # rows 3 and 6 share their argmax
    st = oracle.step_stats(x)
    rows = np.arange(9, dtype=np.int64)
    cand = np.array([3, 6, 0, 8, 2], np.int32)
    D = oracle.cap_dmatrix(x, rows, st["argmax"], st["lse"], cand)
    lp = torch.log_softmax(x.double(), -1).numpy()
    for a, ra in enumerate(cand):
        for b, rb in enumerate(cand):
            if a == b:
                assert np.isnan(D[a, b])
                continue
            ref = lp[ra, st["argmax"][rb]] + lp[rb, st["argmax"][ra]]
            assert abs(D[a, b] - ref) < 1e-12
            assert D[a, b] == D[b, a]                   # symmetric bit for bit
    # shared argmax: D = log conf_i + log conf_j
    assert abs(D[0, 1] - (math.log(st["conf"][3]) + math.log(st["conf"][6]))) < 1e-12


def test_cap_select_end_to_end(oracle):
    g = torch.Generator().manual_seed(6)
    V = 512
    x = torch.randn(24, V, generator=g) * 2
    ids = torch.randint(0, 6, (24,), generator=g)        # few ids -> shared argmaxes
    x[torch.arange(24), ids] += torch.rand(24, generator=g) * 14
    x = x.to(torch.bfloat16)
    st = oracle.step_stats(x)
    so = [0, 10, 24]
    out = oracle.cap_select(x, np.arange(24), so, st["conf"], st["argmax"], st["lse"],
                            0.7, 0.95, -16.0, 8)
    for b in range(2):
        lo, hi = so[b], so[b + 1]
        pool, fb = oracle.cap_pool(st["conf"][lo:hi], 0.7, 8)
        chosen = np.where(out["commit"][lo:hi])[0]
        if len(pool) == 0:
            assert list(chosen) == ([fb] if fb >= 0 else [])
            continue
        assert list(out["cand"][b][: len(pool)]) == list(pool + lo)
        D = out["dmat"][b][: len(pool), : len(pool)]
        conflict = D > -16.0
        ref = _brute_cap(st["conf"][lo:hi][pool], conflict, 0.95) if len(pool) <= 11 else None
        if ref is not None:
            assert sorted(chosen) == sorted(pool[ref == 1])
        assert out["n_commit"][b] == len(chosen)


# ----------------------------------------------------------------------- DAPD
# DAPD page: overall framework; key design 1 (s_ij, edges); key design 2
# (proxy degree, Welsh-Powell order by d~ * conf); ablation table.

def _brute_mis(adj, order):
    """Lexicographically-first maximal independent set, brute force."""
    n = len(order)
    for bits in itertools.product((1, 0), repeat=n):
        chosen = [order[t] for t in range(n) if bits[t]]
        ok = all(not adj[u][v] for u, v in itertools.combinations(chosen, 2))
        if ok:
            return set(chosen)
    return set()


def test_dapd_average_against_torch(oracle):
    g = torch.Generator().manual_seed(7)
    maps = torch.softmax(torch.randn(6, 40, 40, generator=g) * 1.5, -1)
    pos = np.array([3, 10, 11, 12, 30, 39], np.int32)
    for dt in (torch.float32, torch.bfloat16):
        m = maps.to(dt)
        a = oracle.dapd_average(m, pos)
        p = torch.as_tensor(pos, dtype=torch.long)
        ref = m.double()[:, p][:, :, p].mean(0).numpy()
        assert np.allclose(a, ref, rtol=0, atol=1e-15)


def test_dapd_graph_constant_attention(oracle):
    M, S = 7, 20
    a = np.full((M, M), 1.0 / S)
    conf = np.linspace(0.5, 0.9, M)
    s, deg, key = oracle.dapd_graph(a, conf)
    assert np.allclose(s, 1.0 / S, rtol=0, atol=1e-18)
    assert np.allclose(deg, (M - 1) / S, rtol=0, atol=1e-15)
    assert np.allclose(key, deg * conf, rtol=0, atol=1e-18)


def test_dapd_thresholds(oracle):
    rng = np.random.default_rng(5)
    M = 12
    a = rng.random((M, M)) * 0.1
    conf = rng.uniform(0.3, 1.0, M)
    s, deg, key = oracle.dapd_graph(a, conf)
    assert np.array_equal(s, s.T)                               # symmetric bit for bit
    off = s[~np.eye(M, dtype=bool)]
    assert np.all(oracle.dapd_greedy(s, off.max(), key) == 1)   # no edges: all nodes
    take = oracle.dapd_greedy(s, off.min() * 0.5, key)          # complete graph
    assert take.sum() == 1 and take[int(np.argmax(key))] == 1


def test_dapd_greedy_brute_force(oracle):
    rng = np.random.default_rng(6)
    for trial in range(150):
        M = int(rng.integers(1, 14))
        a = rng.random((M, M)) * 0.02
        conf = rng.uniform(0.2, 1.0, M)
        conf[rng.random(M) < 0.2] = conf[0]
        s, deg, key = oracle.dapd_graph(a, conf)
        tau = 0.01
        take = oracle.dapd_greedy(s, tau, key)
        adj = (s > tau) & ~np.eye(M, dtype=bool)
        order = sorted(range(M), key=lambda i: (-key[i], i))
        assert set(np.where(take)[0]) == _brute_mis(adj, order)
        for i in range(M):                                      # independent and maximal
            if take[i]:
                assert not any(take[j] and adj[i][j] for j in range(M))
            else:
                assert any(take[j] and adj[i][j] for j in range(M))


def test_dapd_matches_networkx_welsh_powell(oracle):
    nx = pytest.importorskip("networkx")
    rng = np.random.default_rng(8)
    for trial in range(60):
        M = int(rng.integers(2, 40))
        adj = np.triu(rng.random((M, M)) < rng.uniform(0.05, 0.5), 1)
        adj = adj | adj.T
        w = 0.25
        s = np.where(adj, w, 0.0)                  # equal edge weights, zero elsewhere
        conf = np.full(M, 0.8)                      # equal confidence
        _, deg, key = oracle.dapd_graph(s, conf)    # a = s already symmetric
        take = oracle.dapd_greedy(s, 0.1, key)
        G = nx.Graph()
        G.add_nodes_from(range(M))
        G.add_edges_from(zip(*np.nonzero(np.triu(adj, 1))))
        col = nx.coloring.greedy_color(G, strategy="largest_first")
        class0 = {v for v, c in col.items() if c == 0}
        assert set(np.where(take)[0]) == class0


def test_dapd_mrf_nine_nodes(oracle):
    # DAPD page, key design 1: the synthetic MRF X1..X5, Y1..Y4 with
    # Y_i = (X_i + X_{i+1}) mod 3, i.e. edges Y_i-X_i and Y_i-X_{i+1}.
    # Nodes 0..4 = X1..X5, 5..8 = Y1..Y4.
    M = 9
    s = np.full((M, M), 0.001)
    for i in range(4):
        for x in (i, i + 1):
            s[5 + i, x] = s[x, 5 + i] = 0.05
    conf = np.full(M, 0.9)
    _, deg, key = oracle.dapd_graph(s, conf)
    take = oracle.dapd_greedy(s, 0.01, key)
    adj = (s > 0.01) & ~np.eye(M, dtype=bool)
    order = sorted(range(M), key=lambda i: (-key[i], i))
    assert set(np.where(take)[0]) == _brute_mis(adj, order)
    # X2..X4 and Y1..Y4 have degree 2, X1 and X5 degree 1: hubs first picks
    # X2 (node 1), X3 (node 2), X4 (node 3) ... the set is the X nodes
    assert set(np.where(take)[0]) == {0, 1, 2, 3, 4}


def test_dapd_select_end_to_end(oracle):
    g = torch.Generator().manual_seed(9)
    B, L, S = 2, 4, 24
    attn = torch.softmax(torch.randn(B, L, S, S, generator=g) * 3, -1)
    pos = np.concatenate([np.arange(10, 24), np.arange(12, 24)]).astype(np.int32)
    so = [0, 14, 26]
    conf = np.random.default_rng(1).uniform(0.2, 1.0, 26)
    conf[3] = np.nan
    out = oracle.dapd_select(attn, pos, so, conf, 0.05)
    for b in range(B):
        lo, hi = so[b], so[b + 1]
        a = oracle.dapd_average(attn[b], pos[lo:hi])
        s, deg, key = oracle.dapd_graph(a, conf[lo:hi])
        assert np.allclose(out["degree"][lo:hi], deg, rtol=0, atol=0)
        M = hi - lo
        adj = (s > 0.05) & ~np.eye(M, dtype=bool)
        valid = [i for i in range(M) if not np.isnan(key[i])]
        order = sorted(valid, key=lambda i: (-key[i], i))
        sub = _brute_mis(adj, order) if M <= 14 else None
        chosen = set(np.where(out["commit"][lo:hi])[0])
        if sub is not None:
            assert chosen == sub
        assert all(not np.isnan(conf[lo + i]) for i in chosen)      # NaN never selected
        assert out["n_commit"][b] == len(chosen)
