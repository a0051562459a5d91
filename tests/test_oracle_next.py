"""Pins for the oracle's schedule rules beyond the core step: fixed top-K,
factor decoding (+ Theorem-1 certificate), fixed-block eligibility and the full
DAPD step (late-stage switch, conf = 1 pre-unmask).

Each expected value is worked out by hand in the comments, comes from a library
routine (numpy's stable argsort), or is an invariant that holds for any input.
The cases are chosen so that the plausible mistakes fail: n against n + 1 in the
factor bound, strict against non-strict comparisons, the wrong order statistic,
a block index taken from the absolute position, pre-unmask dropped.
"""
import math

import numpy as np
import pytest
import torch

import oracle

NAN = float("nan")


def so_of(*lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


# ------------------------------------------------------------------ top-K

def test_topk_hand():
    conf = [0.3, 0.9, 0.9, NAN, 0.5, 0.1]
    so = so_of(6)
    c, n = oracle.topk_select(conf, so, 2)
    assert list(np.flatnonzero(c)) == [1, 2] and n[0] == 2          # tie at 0.9: both
    c, n = oracle.topk_select(conf, so, 3)
    assert list(np.flatnonzero(c)) == [1, 2, 4] and n[0] == 3
    c, n = oracle.topk_select(conf, so, 10)
    assert list(np.flatnonzero(c)) == [0, 1, 2, 4, 5] and n[0] == 5  # NaN never
    el = np.array([1, 0, 1, 1, 1, 1], np.uint8)
    c, n = oracle.topk_select(conf, so, 2, eligible=el)
    assert list(np.flatnonzero(c)) == [2, 4]
    c, n = oracle.topk_select([0.2, 0.2, 0.2], so_of(3), 2)         # all tied: lowest rows
    assert list(np.flatnonzero(c)) == [0, 1]


def test_topk_matches_stable_argsort():
    # library special case: the first K of numpy's stable argsort of -conf
    # (descending, ties by ascending index) over the eligible non-NaN rows
    rng = np.random.default_rng(3)
    lens = [1, 7, 32, 50, 0, 128]
    so = so_of(*lens)
    n = int(so[-1])
    conf = np.round(rng.random(n), 2)                 # coarse values: many ties
    conf[rng.random(n) < 0.05] = np.nan
    el = (rng.random(n) < 0.8).astype(np.uint8)
    for k in (1, 2, 4, 8, 200):
        c, cnt = oracle.topk_select(conf, so, k, eligible=el)
        for b in range(len(lens)):
            lo, hi = so[b], so[b + 1]
            rows = np.arange(lo, hi)
            ok = rows[(el[lo:hi] == 1) & ~np.isnan(conf[lo:hi])]
            order = ok[np.argsort(-conf[ok], kind="stable")]
            want = np.zeros(hi - lo, np.uint8)
            want[order[:k] - lo] = 1
            assert np.array_equal(c[lo:hi], want), (k, b)
            assert cnt[b] == min(k, ok.size)


# --------------------------------------------------------- factor decoding

@pytest.mark.parametrize("conf,f,n_star,cert", [
    # sorted .99 .95 .90 .60, f = 1: 2(.01)=.02, 3(.05)=.15, 4(.10)=.40 < 1, 5(.40)=2 -> n* = 3
    ([0.6, 0.99, 0.9, 0.95], 1.0, 3, 1),
    # sorted .8 .74 .7: 2(.2)=.4, 3(.26)=.78, 4(.3)=1.2 -> 2 (a factor n instead of n+1 gives 3)
    ([0.7, 0.8, 0.74], 1.0, 2, 1),
    # equality is not admitted: 4(.25) = 1 exactly -> 2
    ([0.75, 0.75, 0.75], 1.0, 2, 1),
    # 2(.1)=.2, 3(.4)=1.2 -> 1 (using c(n+1) at n = 1 would give 2(.4) = .8 and admit it)
    ([0.6, 0.9], 1.0, 1, 1),
    # nothing admissible: 2(.6) = 1.2 >= 1 -> top-1 fallback; certificate 2(.6) > 1 -> 0
    ([0.4, 0.3], 1.0, 1, 0),
    # large f admits everything: 3(.8) = 2.4 < 100; certificate 2.4 > 1 -> 0
    ([0.3, 0.2], 100.0, 2, 0),
    # tiny f: fallback to the single most confident row; 2(.01) <= 1 -> certified
    ([0.5, 0.99, 0.98], 1e-12, 1, 1),
    # certificate at equality: 2(1 - .5) = 1 <= 1 (fallback commit of one row)
    ([0.5], 1.0, 1, 1),
    # f = 1.5 admits 4(.25) = 1 < 1.5 -> 3; certificate 4(.25) = 1 <= 1
    ([0.75, 0.75, 0.75], 1.5, 3, 1),
])
def test_factor_hand(conf, f, n_star, cert):
    c, n, ce = oracle.factor_select(conf, so_of(len(conf)), f)
    assert n[0] == n_star and int(c.sum()) == n_star
    order = np.argsort(-np.asarray(conf), kind="stable")
    assert set(np.flatnonzero(c)) == set(order[:n_star])            # the n* most confident
    assert ce[0] == cert


def test_factor_nan_ineligible_and_empty():
    conf = [NAN, 0.97, 0.2, 0.96]
    el = np.array([1, 1, 1, 0], np.uint8)
    c, n, ce = oracle.factor_select(conf, so_of(4), 1.0, eligible=el)
    # eligible non-NaN sorted .97 .2: 2(.03) < 1, 3(.8) = 2.4 -> n* = 1
    assert list(np.flatnonzero(c)) == [1] and ce[0] == 1
    c, n, ce = oracle.factor_select([NAN, NAN], so_of(2), 1.0)
    assert n[0] == 0 and c.sum() == 0 and ce[0] == 0


def test_factor_invariants():
    rng = np.random.default_rng(11)
    for trial in range(200):
        m = int(rng.integers(1, 40))
        conf = 1.0 - rng.random(m) ** rng.uniform(1, 8)              # mass near 1
        f = float(rng.choice([0.25, 0.5, 1.0, 2.0, 8.0]))
        c, n, ce = oracle.factor_select(conf, so_of(m), f)
        k = int(n[0])
        srt = np.sort(conf)[::-1]
        lhs = np.arange(2, m + 2) * (1.0 - srt)
        assert np.all(np.diff(lhs) >= 0)                             # monotone: a prefix
        assert 1 <= k <= m
        if k > 1 or lhs[0] < f:
            assert lhs[k - 1] < f                                    # admissible ...
        if k < m:
            assert lhs[k] >= f                                       # ... and largest
        # with f <= 1 every admissible commit is certified (x < f <= 1 -> x <= 1)
        if f <= 1.0 and lhs[0] < f:
            assert ce[0] == 1
        # committed rows are the k largest
        assert np.min(conf[c == 1]) >= np.max(conf[c == 0], initial=-1.0)


# ------------------------------------------------------ fixed-block decoding

def test_fixed_block_hand():
    pos = [515, 530, 545, 600, 700,   545, 560, 580,   5, 40, 70,   500, 520]
    so = so_of(5, 3, 3, 2)
    gs = [512, 512, 0, 512]
    el = oracle.fixed_block_eligible(pos, so, 32, gen_start=gs)
    # seq 0: relative 3 18 33 88 188 -> blocks 0 0 1 2 5 -> block 0
    # seq 1: relative 33 48 68 -> blocks 1 1 2 -> block 1 (block 0 already decoded)
    # seq 2: gen_start 0: blocks 0 1 2 -> block 0
    # seq 3: 500 lies before the generation -> never eligible; 520 -> block 0
    assert list(el) == [1, 1, 0, 0, 0,   1, 1, 0,   1, 0, 0,   0, 1]
    el16 = oracle.fixed_block_eligible(pos, so, 16, gen_start=gs)
    # seq 0 with 16-blocks: 0 1 2 5 11 -> only 515; seq 1: 2 3 4 -> only 545
    assert list(el16[:8]) == [1, 0, 0, 0, 0,   1, 0, 0]
    # absolute positions without gen_start: seq 0 blocks 16 16 17 18 21 -> 515, 530
    el_abs = oracle.fixed_block_eligible(pos[:5], so_of(5), 32)
    assert list(el_abs) == [1, 1, 0, 0, 0]


# -------------------------------------------------------------- DAPD step

def const_attention(B, n_lh, S, value):
    return torch.full((B, n_lh, S, S), value, dtype=torch.float32)


def test_dapd_step_hand():
    # constant attention: a_ij = s_ij = 0.05 for every pair; tau = 0.01 < 0.05
    # makes every masked pair an edge (complete graph), so the graph stage
    # commits exactly one row: equal proxy degrees, so the most confident row
    S = 64
    attn = const_attention(3, 2, S, 0.05)
    pos = np.array([40, 41, 42, 43, 44, 45, 46, 47, 48, 49,
                    40, 41, 42, 43, 44, 45, 46,
                    50, 51, 52], np.int32)
    so = so_of(10, 7, 3)
    conf = np.array([0.5, 0.7, 1.0, 0.2, 0.6, 1.0, 0.3, 0.1, 0.4, 0.65,   # seq 0
                     0.95, 0.9, 0.91, 0.2, 1.0, 0.5, 0.3,                 # seq 1
                     0.5, 0.8, 0.7])                                      # seq 2
    gen_len = np.array([16, 16, 16], np.int32)
    # seq 0: 10 of 16 masked (62.5%) -> graph stage; the complete graph keeps
    #   the top key = top conf, row 2 (1.0, lowest index among the two 1.0s);
    #   pre-unmask adds row 5 (conf exactly 1.0)
    # seq 1: 7 of 16 (43.75% < 50%) -> late stage: conf > 0.9 -> .95, .91, 1.0
    #   (0.9 itself is not above 0.9); pre-unmask adds nothing new
    # seq 2: 3 of 16 -> late stage; nothing above 0.9 -> top-1 fallback (0.8)
    out = oracle.dapd_step(attn, pos, so, conf, 0.01, gen_len=gen_len)
    assert list(out["stage"]) == [0, 1, 1]
    assert list(np.flatnonzero(out["commit"][:10])) == [2, 5]
    assert list(np.flatnonzero(out["commit"][10:17])) == [0, 2, 4]
    assert list(np.flatnonzero(out["commit"][17:])) == [1]
    assert list(out["n_commit"]) == [2, 3, 1]
    # without pre-unmask the graph stage keeps only row 2
    out = oracle.dapd_step(attn, pos, so, conf, 0.01, gen_len=gen_len, pre_unmask=False)
    assert list(np.flatnonzero(out["commit"][:10])) == [2]
    # tau above every score: no edges, every masked row of seq 0 is committed
    out = oracle.dapd_step(attn, pos, so, conf, 0.06, gen_len=gen_len)
    assert out["commit"][:10].sum() == 10


def test_dapd_step_switch_boundary():
    # 8 of 16 masked is not below 50%: graph stage; 7 of 16 is
    attn = const_attention(2, 1, 32, 0.05)
    pos = np.arange(16, 24, dtype=np.int32)
    conf = np.linspace(0.5, 0.95, 8)
    out = oracle.dapd_step(attn, pos, so_of(8), conf, 0.01, gen_len=np.array([16], np.int32))
    assert out["stage"][0] == 0
    out = oracle.dapd_step(attn, pos[:7], so_of(7), conf[:7], 0.01,
                           gen_len=np.array([16], np.int32))
    assert out["stage"][0] == 1


def test_dapd_step_graph_stage_is_maximal_independent():
    # invariant on random attention: outside the pre-unmasked rows, the graph
    # stage commits an independent set of the tau-graph, and every other row
    # with a finite key has a committed neighbour
    rng = np.random.default_rng(5)
    B, n_lh, S, M = 2, 4, 48, 20
    attn = torch.softmax(torch.from_numpy(rng.normal(0, 1.5, (B, n_lh, S, S))).float(), dim=-1)
    pos = np.concatenate([np.sort(rng.choice(S, M, replace=False)) for _ in range(B)])
    pos = pos.astype(np.int32)
    so = so_of(M, M)
    conf = rng.random(B * M)
    conf[3] = 1.0
    tau = 0.02
    ref = oracle.dapd_select(attn, pos, so, conf, tau)
    out = oracle.dapd_step(attn, pos, so, conf, tau, gen_len=np.array([30, 30], np.int32))
    assert list(out["stage"]) == [0, 0]
    for b in range(B):
        s = ref["sym"][b]
        com = out["commit"][so[b]:so[b + 1]].astype(bool)
        core = com & (conf[so[b]:so[b + 1]] != 1.0)
        idx = np.flatnonzero(core)
        for i in idx:
            for j in idx:
                assert i == j or not s[i, j] > tau
        for i in np.flatnonzero(~com):
            assert np.any(s[i, com] > tau)
    assert out["commit"][3] == 1


def test_dapd_step_without_policy_is_the_plain_step():
    rng = np.random.default_rng(6)
    attn = torch.softmax(torch.from_numpy(rng.normal(0, 1.0, (1, 3, 40, 40))).float(), dim=-1)
    pos = np.arange(10, 40, dtype=np.int32)
    conf = rng.random(30)
    ref = oracle.dapd_select(attn, pos, so_of(30), conf, 0.03)
    out = oracle.dapd_step(attn, pos, so_of(30), conf, 0.03, gen_len=None, pre_unmask=False)
    assert np.array_equal(out["commit"], ref["commit"]) and out["stage"][0] == 0
    assert not math.isnan(float(ref["key"][0]))
