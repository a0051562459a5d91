"""Pins for the oracle's step statistics (conf, argmax, entropy, KL, lse).

Each test fixes the oracle against something other than itself: closed forms
(uniform, one-hot, two-point rows), invariants of the information measures,
shift invariance, and torch's own fp64 log-softmax / entropy / KL routines
(an independent library implementation of the same definitions).

Definitions followed (DepCap page, Methodology: H_k = H(p_curr^k),
I_k = KL(p_curr^k || p_prev^k), c_i = max_v p_i(v); Fast-dLLM review, Method:
max-softmax confidence).
"""
import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.filterwarnings("ignore")


def _bf16(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def test_uniform_row_closed_form(oracle):
    for V, dt in ((4096, torch.float32), (126464, torch.bfloat16)):
        row = torch.full((1, V), 1.5, dtype=dt)
        out = oracle.step_stats(row, prev=row.clone())
        assert out["argmax"][0] == 0
        assert abs(out["conf"][0] - 1.0 / V) < 1e-15
        assert abs(out["entropy"][0] - math.log(V)) < 1e-9  # natural log
        assert abs(out["lse"][0] - (1.5 + math.log(V))) < 1e-9
        assert out["kl"][0] == 0.0


def test_closed_forms_at_extreme_magnitudes(oracle):
    # The definitions do not depend on where the logits sit: a uniform row
    # has conf 1/V and entropy log V whether its value is 0 or 3e38, and
    # equal rows have KL 0.  At |x| near 3e38 the log-normaliser m + log z
    # equals m in double, so log p must be formed as (x - m) - log z.
    V = 4096
    for dt in (torch.float32, torch.bfloat16):
        for c in (3.0e38, -3.0e38, 1.0e20, -1.5e30):
            row = torch.full((1, V), c, dtype=dt)
            out = oracle.step_stats(row, prev=row.clone())
            assert abs(out["conf"][0] - 1.0 / V) < 1e-15, (dt, c, out["conf"][0])
            assert abs(out["entropy"][0] - math.log(V)) < 1e-9, (dt, c, out["entropy"][0])
            assert out["kl"][0] == 0.0
            x = float(row[0, 0])
            assert out["lse"][0] == x + math.log(V)
        # two entries 1 apart, far from zero: the two-point closed form
        row = torch.full((1, V), float("-inf"), dtype=dt)
        row[0, 7], row[0, 9] = 2.0e30, 2.0e30
        out = oracle.step_stats(row)
        assert abs(out["conf"][0] - 0.5) < 1e-15 and abs(out["entropy"][0] - math.log(2)) < 1e-15


def test_one_hot_rows(oracle):
    V = 4096
    x = torch.zeros((2, V), dtype=torch.float32)
    x[0, 17] = 1000.0  # exp(-1000) underflows: a point mass in fp64
    x[1, :] = float("-inf")
    x[1, 4000] = 3.0
    out = oracle.step_stats(x.to(torch.bfloat16))
    assert list(out["argmax"]) == [17, 4000]
    assert np.all(out["conf"] == 1.0)
    assert np.all(out["entropy"] == 0.0)
    assert abs(out["lse"][0] - 1000.0) < 1e-12 and abs(out["lse"][1] - 3.0) < 1e-15


@pytest.mark.parametrize("a,b", [(0.0, 0.0), (1.0, -2.5), (-3.0, 4.0), (7.25, 7.0)])
def test_two_point_row(oracle, a, b):
    V = 64
    x = torch.full((1, V), float("-inf"), dtype=torch.float32)
    x[0, 5], x[0, 40] = a, b
    # prev: a different two-point distribution on the same support
    q = torch.full((1, V), float("-inf"), dtype=torch.float32)
    q[0, 5], q[0, 40] = 0.0, 1.0
    out = oracle.step_stats(x, prev=q)
    p = 1.0 / (1.0 + math.exp(-(a - b)))  # P(index 5)
    conf = max(p, 1 - p)
    h = -(p * math.log(p) + (1 - p) * math.log(1 - p))
    pq = 1.0 / (1.0 + math.exp(1.0))
    kl = p * math.log(p / pq) + (1 - p) * math.log((1 - p) / (1 - pq))
    assert abs(out["conf"][0] - conf) < 1e-14
    assert abs(out["entropy"][0] - h) < 1e-14
    assert abs(out["kl"][0] - kl) < 1e-14
    assert out["argmax"][0] == (5 if a >= b else 40)


def test_against_torch_fp64_library(oracle):
    g = torch.Generator().manual_seed(11)
    V = 3000
    cur = (torch.randn(6, V, generator=g) * 2.0)
    prev = cur + 0.5 * torch.randn(6, V, generator=g)
    for dt in (torch.float32, torch.bfloat16):
        c, p = cur.to(dt), prev.to(dt)
        out = oracle.step_stats(c, prev=p)
        c64, p64 = c.double(), p.double()
        lp = torch.log_softmax(c64, dim=-1)
        lq = torch.log_softmax(p64, dim=-1)
        ref_conf = lp.exp().max(dim=-1).values
        ref_arg = torch.argmax(c64, dim=-1)  # first maximal index
        ref_h = torch.distributions.Categorical(logits=c64).entropy()
        # kl_div(input=log q, target=log p, log_target) = sum p (log p - log q) = KL(p || q)
        ref_kl = torch.nn.functional.kl_div(lq, lp, log_target=True, reduction="none").sum(-1)
        ref_lse = torch.logsumexp(c64, dim=-1)
        assert np.allclose(out["conf"], ref_conf.numpy(), rtol=0, atol=1e-12)
        assert np.array_equal(out["argmax"], ref_arg.numpy().astype(np.int32))
        assert np.allclose(out["entropy"], ref_h.numpy(), rtol=0, atol=1e-11)
        assert np.allclose(out["kl"], ref_kl.numpy(), rtol=0, atol=1e-12)
        assert np.allclose(out["lse"], ref_lse.numpy(), rtol=0, atol=1e-12)


def test_kl_direction_is_current_given_previous(oracle):
    # Asymmetric pair: KL(p||q) != KL(q||p).  The pages fix KL(p_curr || p_prev).
    x = torch.tensor([[0.0, 2.0, -1.0, 0.5]])
    y = torch.tensor([[1.0, -1.0, 0.0, 0.0]])
    out = oracle.step_stats(x, prev=y)
    p = torch.softmax(x.double(), -1)
    q = torch.softmax(y.double(), -1)
    kl_pq = float((p * (p.log() - q.log())).sum())
    kl_qp = float((q * (q.log() - p.log())).sum())
    assert abs(out["kl"][0] - kl_pq) < 1e-14
    assert abs(kl_pq - kl_qp) > 1e-3


def test_argmax_ties_lowest_index(oracle):
    x = torch.zeros((3, 1024))
    x[0, [9, 3, 700]] = 5.0
    x[1, [1023, 512]] = 2.0
    out = oracle.step_stats(x.to(torch.bfloat16))
    assert list(out["argmax"]) == [3, 512, 0]


def test_invariants_random_rows(oracle):
    g = torch.Generator().manual_seed(5)
    V = 5000
    cur = torch.randn(32, V, generator=g) * torch.linspace(0.1, 6.0, 32).unsqueeze(1)
    cur[::3, 77] += 15.0
    prev = cur + 0.7 * torch.randn(32, V, generator=g)
    out = oracle.step_stats(cur.to(torch.bfloat16), prev=prev.to(torch.bfloat16))
    H, kl, conf = out["entropy"], out["kl"], out["conf"]
    assert np.all(kl >= -1e-15)
    assert np.all(H >= -1e-15) and np.all(H <= math.log(V) + 1e-12)
    assert np.all(conf >= 1.0 / V - 1e-18) and np.all(conf <= 1.0)
    assert np.all(conf >= np.exp(-H) - 1e-15)  # max p >= exp(-H)


def test_shift_invariance_fp32(oracle):
    g = torch.Generator().manual_seed(3)
    # values on a 1/64 grid so that adding 0.5 is exact in fp32
    cur = torch.round(torch.randn(4, 2048, generator=g) * 128) / 64
    prev = torch.round(torch.randn(4, 2048, generator=g) * 128) / 64
    a = oracle.step_stats(cur, prev=prev)
    b = oracle.step_stats(cur + 0.5, prev=prev - 0.25)
    assert np.allclose(a["conf"], b["conf"], rtol=0, atol=1e-13)
    assert np.allclose(a["entropy"], b["entropy"], rtol=0, atol=1e-12)
    assert np.allclose(a["kl"], b["kl"], rtol=0, atol=1e-12)
    assert np.allclose(b["lse"] - a["lse"], 0.5, rtol=0, atol=1e-12)
    assert np.array_equal(a["argmax"], b["argmax"])


def test_bf16_widening_is_exact(oracle):
    g = torch.Generator().manual_seed(8)
    x = (torch.randn(3, 4096, generator=g) * 3).to(torch.bfloat16)
    a = oracle.step_stats(x)
    b = oracle.step_stats(x.float())
    for k in ("conf", "entropy", "lse"):
        assert np.array_equal(a[k], b[k])
    assert np.array_equal(a["argmax"], b["argmax"])


def test_row_index_and_leading_dimension(oracle):
    g = torch.Generator().manual_seed(9)
    full = torch.randn(10, 600, generator=g)
    full[:, 500:] = 1e4  # padding beyond the vocabulary must be ignored
    rows = np.array([7, 2, 2, 9], dtype=np.int64)
    out = oracle.step_stats(full, row_index=rows, vocab=500)
    ref = oracle.step_stats(full[rows.tolist(), :500].contiguous())
    for k in ("conf", "entropy", "lse", "argmax"):
        assert np.array_equal(out[k], ref[k])


def test_non_finite_rows(oracle):
    V = 256
    ninf = float("-inf")
    x = torch.randn(6, V, generator=torch.Generator().manual_seed(1))
    q = x.clone()
    x[0, 10] = float("nan")               # NaN -> NaN stats, argmax over non-NaN
    x[1, :] = ninf                         # all -inf -> NaN stats, argmax 0
    x[2, 100:] = ninf                      # -inf entries contribute 0
    q[3, 7] = ninf                         # q = 0 where p > 0 -> KL = +inf
    x[4, 5] = float("inf")                 # +inf -> NaN stats, argmax at the +inf
    x[5, :] = float("nan")                 # all NaN -> argmax 0
    out = oracle.step_stats(x, prev=q)
    ref_arg0 = int(torch.argmax(torch.nan_to_num(x[0], nan=-1e30)))
    assert np.isnan(out["conf"][0]) and np.isnan(out["entropy"][0]) and np.isnan(out["kl"][0])
    assert out["argmax"][0] == ref_arg0
    assert np.isnan(out["conf"][1]) and out["argmax"][1] == 0
    assert np.isnan(out["entropy"][1]) and np.isnan(out["kl"][1]) and np.isnan(out["lse"][1])
    lp = torch.log_softmax(x[2, :100].double(), -1)
    assert abs(out["entropy"][2] - float(-(lp.exp() * lp).sum())) < 1e-13
    assert out["kl"][3] == float("inf")
    assert np.isnan(out["conf"][4]) and out["argmax"][4] == 5
    assert np.isnan(out["lse"][5]) and out["argmax"][5] == 0
    assert np.isnan(out["entropy"][4]) and np.isnan(out["entropy"][5])
