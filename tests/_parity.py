"""Shared helpers for the GPU parity tests.

Tolerances: statistics (conf, entropy, KL, lse, S_k, D_ij, s_ij, degree) within
1e-5 absolute of the fp64 oracle; argmax bit-exact.  Decisions are compared two
ways:
  decision-only  the oracle's rule applied to the GPU's exported scores (fp32;
                 S_k in fp64) must reproduce the GPU's masks and boundaries bit
                 for bit, always;
  end-to-end     GPU decisions from GPU statistics vs oracle decisions from oracle
                 statistics.  A differing sequence is accepted (and counted as
                 flagged) only if decision-only parity holds for it and the oracle
                 has a decision quantity within 1e-5 of its threshold or a near-tie.
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
    diff = np.where(nan_r | inf_ok, 0.0, np.abs(g - r))
    worst = float(np.max(diff)) if diff.size else 0.0
    assert worst <= tol, f"{name}: max |gpu - oracle| = {worst:.3e} > {tol} at {int(np.argmax(diff))}"
    return worst


def near_any(values, thresholds, eps=NEAR):
    v = np.asarray(values, np.float64)
    v = v[np.isfinite(v)]
    return any(np.any(np.abs(v - t) < eps) for t in thresholds)


def near_tie(values, eps=NEAR):
    v = np.sort(np.asarray(values, np.float64)[np.isfinite(values)])
    return v.size > 1 and bool(np.any(np.diff(v) < eps))


class Flags:
    """Counts sequences whose end-to-end decision differed but was accepted."""

    def __init__(self, name):
        self.name, self.flagged, self.total = name, 0, 0

    def check(self, same: bool, decision_only_ok: bool, near: bool, where: str):
        self.total += 1
        if same:
            return
        assert decision_only_ok, f"{self.name} {where}: decision-only parity broken"
        assert near, f"{self.name} {where}: decision differs with no near-threshold quantity"
        self.flagged += 1

    def report(self):
        print(f"[parity] {self.name}: {self.flagged} flagged of {self.total} sequences")
