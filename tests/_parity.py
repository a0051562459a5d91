"""Shared helpers for the GPU parity tests.

Tolerances: statistics (conf, entropy, KL, lse, S_k, D_ij, s_ij, degree) within
1e-5 absolute of the fp64 oracle; argmax bit-exact.  Decisions are compared two
ways:
  decision-only  the oracle's rule applied to the GPU's exported scores (fp32;
                 S_k in fp64) must reproduce the GPU's masks and boundaries bit
                 for bit, always;
  end-to-end     GPU decisions from GPU statistics vs oracle decisions from oracle
                 statistics.  A sequence whose decision differs is accepted (and
                 counted as flagged) only if decision-only parity holds for it and
                 the difference is explained by an oracle quantity within 1e-5 of
                 its threshold, or by a near-tie (within 1e-5) between two items
                 that interact in the rule:
                   Fast-dLLM  each differing row has |conf - tau| < 1e-5, or is a
                              fallback pick with another eligible row within
                              1e-5 of the top confidence;
                   DepCap     some |S_k| < 1e-5 with k up to the larger boundary;
                   CAP        |conf - tau_low| or |conf - tau_high| < 1e-5, a
                              pool pair with |D_ij - gamma| < 1e-5, a near-tie
                              between two pool members that conflict, a near-tie
                              at the K_max cut, or a near-tie of the fallback's
                              top two;
                   DAPD       a pair with |s_ij - tau| < 1e-5, or a near-tie of
                              keys between two nodes joined by an edge.
                 An order swap between items that do not interact cannot change
                 a greedy's result, so it explains nothing.
The named workloads are seeded and expected to flag nothing: their tests
assert a flagged count of zero.
"""
from __future__ import annotations

import numpy as np
import torch

TOL = 1e-5
NEAR = 1e-5


def host(t):
    return None if t is None else t.detach().cpu()


def f64(t):
    return host(t).double().numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def assert_close(gpu, ref, name, tol=TOL):
    g = f64(gpu)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    nan_g, nan_r = np.isnan(g), np.isnan(r)
    bad_nan = np.nonzero(nan_g != nan_r)[0]
    assert bad_nan.size == 0, f"{name}: NaN mismatch at {bad_nan[:10]}"
    inf_ok = np.isinf(r) & (g == r)
    with np.errstate(invalid="ignore"):
        diff = np.where(nan_r | inf_ok, 0.0, np.abs(g - r))
    worst = float(np.max(diff)) if diff.size else 0.0
    assert worst <= tol, f"{name}: max |gpu - oracle| = {worst:.3e} > {tol} at {int(np.argmax(diff))}"
    return worst


def near_any(values, thresholds, eps=NEAR):
    v = np.asarray(values, np.float64)
    v = v[np.isfinite(v)]
    return any(np.any(np.abs(v - t) < eps) for t in thresholds)


# ------------------------------------------------------------ explanations
# Each returns True when an end-to-end difference in one sequence is
# explained by the oracle's own quantities (see the module docstring).

def fastdllm_explained(commit_g, commit_o, conf_o, eligible, tau, eps=NEAR):
    """One sequence: commit masks (GPU, oracle), oracle confidences, eligible
    mask (bool), the fp32 threshold as a float."""
    conf_o = np.asarray(conf_o, np.float64)
    el = np.asarray(eligible, bool) & np.isfinite(conf_o)
    if not el.any():
        return False
    top = conf_o[el].max()
    near_top = el & (conf_o >= top - eps)
    fallback_tie = top <= tau + eps and int(near_top.sum()) >= 2
    for i in np.nonzero(np.asarray(commit_g) != np.asarray(commit_o))[0]:
        if el[i] and abs(conf_o[i] - tau) < eps:
            continue
        if fallback_tie and near_top[i]:
            continue
        return False
    return True


def depcap_explained(L_g, L_o, S_o, eps=NEAR):
    """One sequence: GPU and oracle boundaries, oracle scores over the window."""
    kk = min(len(S_o), max(int(L_g), int(L_o)) + 1)
    return near_any(np.asarray(S_o, np.float64)[:kk], [0.0], eps)


def cap_explained(conf_o, eligible, pool_o, D_o, tau_low, tau_high, gamma, k_max, eps=NEAR):
    """One sequence: oracle confidences (rows of the sequence), eligible mask,
    the oracle's candidate list (row offsets in priority order, after the
    K_max cap), its D over those candidates, and the fp32 parameters."""
    conf_o = np.asarray(conf_o, np.float64)
    el = np.asarray(eligible, bool) & np.isfinite(conf_o)
    c = conf_o[el]
    if near_any(c, [tau_low], eps):                                   # pool membership
        return True
    pool_o = np.asarray(pool_o, np.int64)
    nc = len(pool_o)
    if nc == 0:                                                       # fallback top two
        s = np.sort(c)[::-1]
        return s.size >= 2 and s[0] - s[1] < eps
    pc = conf_o[pool_o]
    if near_any(pc, [tau_high], eps):                                 # forced set
        return True
    D = np.asarray(D_o, np.float64)[:nc, :nc]
    off = ~np.eye(nc, dtype=bool)
    if np.any(off & np.isfinite(D) & (np.abs(D - gamma) < eps)):      # conflict edge
        return True
    conflict = off & (D > gamma - eps)
    tie = np.abs(pc[:, None] - pc[None, :]) < eps
    if np.any(conflict & tie):                                        # conflicting near-tie
        return True
    full = np.sort(c[c >= tau_low])[::-1]
    if full.size > k_max and full[k_max - 1] - full[k_max] < eps:     # the K_max cut
        return True
    return False


def dapd_explained(s_o, key_o, tau, eps=NEAR):
    """One sequence: the oracle's s (M x M) and keys (M)."""
    s = np.asarray(s_o, np.float64)
    M = s.shape[0]
    off = ~np.eye(M, dtype=bool)
    if np.any(off & np.isfinite(s) & (np.abs(s - tau) < eps)):       # edge flips
        return True
    key = np.asarray(key_o, np.float64)
    edge = off & (s > tau - eps)
    tie = np.abs(key[:, None] - key[None, :]) < eps
    return bool(np.any(edge & tie))                                   # adjacent near-tie


class Flags:
    """Counts sequences whose end-to-end decision differed but was explained
    (see the module docstring); any unexplained difference fails."""

    def __init__(self, name):
        self.name, self.flagged, self.total = name, 0, 0

    def check(self, same: bool, decision_only_ok: bool, explained, where: str):
        """`explained` is a bool or a zero-argument callable (evaluated only
        when the decisions differ)."""
        self.total += 1
        if same:
            return
        assert decision_only_ok, f"{self.name} {where}: decision-only parity broken"
        ok = explained() if callable(explained) else explained
        assert ok, f"{self.name} {where}: decision differs with no explaining near-threshold " \
                   f"quantity or interacting near-tie"
        self.flagged += 1

    def report(self) -> int:
        print(f"[parity] {self.name}: {self.flagged} flagged of {self.total} sequences")
        return self.flagged

    def assert_none(self):
        n = self.report()
        assert n == 0, f"{self.name}: {n} flagged sequences on a seeded workload"
