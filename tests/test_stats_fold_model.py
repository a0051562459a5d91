"""CPU model of the statistics kernel's per-lane fold, checked against the
fp64 definitions (DepCap summary, Methodology: H_k = H(p_curr^k) and
I_k = KL(p_curr^k || p_prev^k); Fast-dLLM review, Method: the max-softmax
confidence).  The model follows the kernel's steps in fp32, one row at a time:
768 lanes, lane l folding chunks l, l + 768, ... of 8 elements; per chunk the
running max, and, when some lane of the wave has a max more than the margin
(8, in log2 units) above its integer reference, an exact power-of-two rescale
of that wave's running sums to h = ceil(max * log2 e); then the sums of
e = 2^t, e*t, e*t_y and 2^t_y with t = x*log2 e - h and t_y = y*log2 e - h,
each chunk's B as sum e*t - sum e*t_y; the lane totals moved to the row's
reference in fp64 and formed into the statistics.  It checks the claims the
kernel's numerics rest on: every exponent stays at or below the margin (no
overflow), equal rows give B = 0 and Z2 = Z bit for bit (KL exactly 0), and
the statistics stay well inside the 1e-5 tolerance of the definitions on rows
that move the reference many times or late, and a masked (-inf) entry leaves a
non-finite total, the kernel's signal for its element-wise path."""
import numpy as np
import pytest
import torch

F = np.float32
L2E = F(1.4426950408889634)
LN2F = F(0.69314718)
SLACK = F(8.0)
LOW = F(-1e30)
NT, VEC, WAVE = 768, 8, 64


def _fma(a, b, c):
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(F)


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def fold_row(x, y, lazy=True):
    """One row through the lane fold; returns (H, KL, lse, conf, max t, rescales per lane)."""
    V = x.size
    n_c = V // VEC
    segs = -(-n_c // NT)
    lanes = np.arange(NT)
    m = np.full(NT, LOW, F)
    h = np.full(NT, np.ceil(LOW * L2E), F)
    thr = np.full(NT, LOW, F)
    Z, A, B, Z2 = (np.zeros(NT, F) for _ in range(4))
    t_max = -np.inf
    rescales = np.zeros(NT, int)
    for s in range(segs):
        ch = s * NT + lanes
        val = ch < n_c
        idx = np.minimum(ch, n_c - 1)[:, None] * VEC + np.arange(VEC)
        xc, yc = x[idx], y[idx]
        cm = np.where(val, xc.max(axis=1), LOW).astype(F)
        m = np.maximum(m, cm)
        need = m > thr if lazy else np.ones(NT, bool)
        wave_need = need.reshape(-1, WAVE).any(axis=1).repeat(WAVE)
        if wave_need.any():
            hn = np.ceil(m * L2E).astype(F)
            dh = (h - hn).astype(F)
            di = np.maximum(dh, F(-256)).astype(np.int64)
            A = np.where(wave_need, np.ldexp(_fma(dh, Z, A), di).astype(F), A)
            Z = np.where(wave_need, np.ldexp(Z, di).astype(F), Z)
            B = np.where(wave_need, np.ldexp(B, di).astype(F), B)
            Z2 = np.where(wave_need, np.ldexp(Z2, di).astype(F), Z2)
            rescales += wave_need & (hn != h)
            h = np.where(wave_need, hn, h)
            thr = np.where(wave_need, ((hn + SLACK) * LN2F).astype(F), thr)
        t = _fma(xc, np.full_like(xc, L2E), -h[:, None])
        ty = _fma(yc, np.full_like(yc, L2E), -h[:, None])
        e = np.exp2(t).astype(F)
        if val.any():
            fin = np.isfinite(t[val])
            t_max = max(t_max, float(t[val][fin].max()) if fin.any() else -np.inf)
        z, a, ay, z2 = (np.full(NT, F(-0.0)) for _ in range(4))
        for k in range(VEC):
            z = (z + e[:, k]).astype(F)
            with np.errstate(invalid="ignore"):
                a = _fma(e[:, k], t[:, k], a)
                ay = _fma(e[:, k], ty[:, k], ay)
            z2 = (z2 + np.exp2(ty[:, k]).astype(F)).astype(F)
        Z = np.where(val, Z + z, Z).astype(F)
        A = np.where(val, A + a, A).astype(F)
        B = np.where(val, B + (a - ay).astype(F), B).astype(F)
        Z2 = np.where(val, Z2 + z2, Z2).astype(F)
    # lane totals to the row's integer reference, in fp64
    M = float(m.max())
    hr = float(np.ceil(F(M) * L2E))
    d = h.astype(np.float64) - hr
    sc = np.ldexp(1.0, np.maximum(d, -1100).astype(np.int64))
    Zr = float(np.sum(Z * sc))
    Ar = float(np.sum((A.astype(np.float64) + d * Z) * sc))
    Br = float(np.sum(B * sc))
    Z2r = float(np.sum(Z2 * sc))
    cM = hr - M * float(L2E)
    ln2 = np.log(2.0)
    H = ln2 * (np.log2(Zr) - Ar / Zr)
    KL = ln2 * (Br / Zr + np.log2(Z2r / Zr))
    lse = M + ln2 * (np.log2(Zr) + cM)
    conf = 2.0 ** (-cM) / Zr
    return H, KL, lse, conf, t_max, rescales, (Z, Z2, B)


def exact(x, y):
    x = x.astype(np.float64)
    y = y.astype(np.float64)
    lse = np.logaddexp.reduce(x)
    lp = x - lse
    lq = y - np.logaddexp.reduce(y)
    p = np.exp(lp)
    fin = p > 0
    H = -np.sum(p[fin] * lp[fin])
    KL = np.sum(p[fin] * (lp[fin] - lq[fin]))
    return H, KL, lse, float(np.exp(x.max() - lse))


def _rows(V, seed):
    g = np.random.default_rng(seed)
    v = np.arange(V, dtype=np.float64)
    noise = g.standard_normal(V) * 2.0
    spike = noise.copy()
    spike[g.integers(V)] += 12.0
    late = noise.copy()
    late[V - 1] = 40.0
    masked = noise.copy()
    masked[: V // 2] = -np.inf
    return {"planted peak": spike, "late spike": late, "masked half": masked,
            "ramp 60": 60.0 * v / V - 20.0, "ramp 200": 200.0 * v / V - 100.0,
            "falling ramp": 40.0 - 60.0 * v / V, "sawtooth": 30.0 * np.remainder(v, 4096.0) / 4096.0}


@pytest.mark.parametrize("name", ["planted peak", "late spike", "ramp 60", "ramp 200",
                                  "falling ramp", "sawtooth"])
def test_fold_model_matches_the_definitions(name):
    V = 126464
    x = _bf16(_rows(V, 7)[name])
    y = _bf16(x + np.random.default_rng(11).standard_normal(V) * 0.5)
    H, KL, lse, conf, t_max, resc, _ = fold_row(x, y)
    He, KLe, lsee, confe = exact(x, y)
    # every exponent at or below the margin: 2^t <= 256, no overflow
    assert t_max <= float(SLACK) + 1e-3, t_max
    for got, want, what in ((H, He, "entropy"), (KL, KLe, "kl"), (lse, lsee, "lse"),
                            (conf, confe, "conf")):
        assert abs(got - want) <= 2e-6 * max(1.0, abs(want)), (name, what, got, want)
    # against the per-chunk rescale (the reference always at ceil(max log2 e))
    H0, KL0, lse0, conf0, t0, _, _ = fold_row(x, y, lazy=False)
    assert t0 <= 1e-3
    assert abs(H - H0) <= 2e-6 and abs(KL - KL0) <= 2e-6, (name, H, H0, KL, KL0)
    print(f"[fold model] {name}: H err {abs(H - He):.1e} KL err {abs(KL - KLe):.1e} "
          f"max t {t_max:.2f} rescales per lane {resc.mean():.2f} (max {resc.max()})")


def test_fold_model_masked_entries_leave_a_non_finite_total():
    # a -inf logit makes e*t = 0 * -inf a NaN in the lane sums: the kernel's
    # finalize sees a non-finite total and sends the row to its element-wise
    # path, which applies 0 log 0 = 0 term by term
    V = 126464
    x = _bf16(_rows(V, 7)["masked half"])
    H, KL, lse, conf, *_ = fold_row(x, x)
    assert not np.isfinite(H) and not np.isfinite(KL)


def test_fold_model_equal_rows_give_exact_zero_kl():
    V = 126464
    for name, row in _rows(V, 3).items():
        if name == "masked half":
            continue
        x = _bf16(row)
        H, KL, lse, conf, t_max, resc, (Z, Z2, B) = fold_row(x, x)
        assert np.array_equal(Z.view(np.uint32), Z2.view(np.uint32)), name
        assert np.all(B == 0.0), name
        assert KL == 0.0, (name, KL)


def test_fold_model_rescales_rarely_on_gaussian_rows():
    # N(0, 2) logits with a planted peak: after a lane's first chunk, a
    # rescale needs its max to pass the reference by 8 log2 units (5.5 nats)
    V = 126464
    x = _bf16(_rows(V, 5)["planted peak"])
    *_, resc, _ = fold_row(x, x)
    assert resc.mean() <= 2.0, resc.mean()
    *_, resc0, _ = fold_row(x, x, lazy=False)
    assert resc0.mean() > 2.0 * resc.mean()
