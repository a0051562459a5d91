"""GPU parity of the schedule calls: dlm_topk_select, dlm_factor_select,
dlm_fixed_block_eligible and dlm_dapd_step (marked gpu).

Top-K, factor decoding and fixed-block eligibility are integer decisions taken
on the given fp32 confidences (the factor test in fp64 on both sides, where it
is exact), so they are compared bit for bit with the oracle on the same inputs.
So is the DAPD step's late stage and its stage flag.  Its graph stage must
equal the plain DAPD selection of the same call plus the pre-unmasked rows,
and is compared end to end with the oracle with near-tie flags, as the plain
selection is.
"""
import numpy as np
import pytest
import torch

import oracle
from _parity import Flags, dapd_explained, f64, host
from diffusion_lm_unmask_amd import api, synth

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("poisoned_outputs")]
DEV = "cuda"


def _csr(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _conf_mix(n, seed):
    """fp32 confidences with ties, NaN, exact 1.0 and values just below 1."""
    rng = np.random.default_rng(seed)
    c = rng.random(n).astype(np.float32)
    c[rng.random(n) < 0.3] = np.float32(np.round(rng.random() * 64) / 64)   # one shared value
    near1 = rng.random(n) < 0.3
    c[near1] = (1.0 - np.ldexp(1.0, -rng.integers(1, 24, near1.sum()))).astype(np.float32)
    c[rng.random(n) < 0.02] = np.nan
    c[rng.random(n) < 0.02] = 1.0
    ties = rng.random(n) < 0.2
    c[ties] = np.float32(0.75)
    return c


LENS = [1, 7, 32, 0, 256, 1024, 1025, 100, 3]   # 1025 exceeds the per-sequence limit


def _inputs(seed):
    so = _csr(LENS)
    n = int(so[-1])
    conf = _conf_mix(n, seed)
    el = (np.random.default_rng(seed + 1).random(n) < 0.85).astype(np.uint8)
    return so, conf, el


def _check_over_long(commit, n_commit, so):
    for b, m in enumerate(LENS):
        if m > 1024:
            assert int(n_commit[b]) == -1 and commit[so[b]:so[b + 1]].sum() == 0


@pytest.mark.parametrize("k", [1, 3, 8, 64, 2000])
@pytest.mark.parametrize("with_el", [False, True])
def test_topk_bit_exact(k, with_el):
    so, conf, el = _inputs(7)
    el_arg = el if with_el else None
    c_g, n_g = api.topk_select(torch.from_numpy(conf).to(DEV), torch.from_numpy(so).to(DEV), k,
                               eligible=torch.from_numpy(el).to(DEV) if with_el else None)
    c_g, n_g = host(c_g).numpy(), host(n_g).numpy()
    c_o, n_o = oracle.topk_select(conf.astype(np.float64), so, k, eligible=el_arg)
    for b, m in enumerate(LENS):
        lo, hi = so[b], so[b + 1]
        if m > 1024:
            continue
        assert np.array_equal(c_g[lo:hi], c_o[lo:hi]), f"k={k} seq {b}"
        assert n_g[b] == n_o[b]
    _check_over_long(c_g, n_g, so)


@pytest.mark.parametrize("f", [1.0, 0.5, 2.0, 1e-3, 30.0, 1.5])
@pytest.mark.parametrize("with_el", [False, True])
def test_factor_bit_exact(f, with_el):
    so, conf, el = _inputs(11)
    f32 = float(np.float32(f))
    c_g, n_g, ce_g = api.factor_select(torch.from_numpy(conf).to(DEV),
                                       torch.from_numpy(so).to(DEV), f,
                                       eligible=torch.from_numpy(el).to(DEV) if with_el else None)
    c_g, n_g, ce_g = host(c_g).numpy(), host(n_g).numpy(), host(ce_g).numpy()
    c_o, n_o, ce_o = oracle.factor_select(conf.astype(np.float64), so, f32,
                                          eligible=el if with_el else None)
    for b, m in enumerate(LENS):
        lo, hi = so[b], so[b + 1]
        if m > 1024:
            assert ce_g[b] == 0
            continue
        assert np.array_equal(c_g[lo:hi], c_o[lo:hi]), f"f={f} seq {b}"
        assert n_g[b] == n_o[b] and ce_g[b] == ce_o[b], f"f={f} seq {b}"
    _check_over_long(c_g, n_g, so)
    print(f"[factor] f={f}: n_commit {n_g.tolist()} certified {ce_g.tolist()}")


def test_factor_exact_equalities():
    # fp32-exact values where (n+1)(1 - c) hits the bound exactly
    cases = [([0.75, 0.75, 0.75], 1.0, 2, 1), ([0.75, 0.75, 0.75], 1.5, 3, 1), ([0.5], 1.0, 1, 1),
             ([0.4, 0.3], 1.0, 1, 0)]
    conf = np.concatenate([np.float32(c) for c, *_ in cases]).astype(np.float32)
    so = _csr([len(c) for c, *_ in cases])
    for j, (c, f, n_star, cert) in enumerate(cases):
        sub = torch.from_numpy(np.asarray(c, np.float32)).to(DEV)
        cg, ng, ceg = api.factor_select(sub, torch.tensor([0, len(c)], device=DEV,
                                                          dtype=torch.int32), f)
        assert int(host(ng)[0]) == n_star and int(host(ceg)[0]) == cert, (c, f)
    assert conf.size == int(so[-1])


def test_fixed_block_bit_exact():
    rng = np.random.default_rng(5)
    lens = [40, 0, 7, 256, 1, 300]
    gs = np.array([512, 0, 100, 512, 9, 0], np.int32)
    pos = []
    for m, g in zip(lens, gs):
        p = np.sort(rng.choice(np.arange(max(0, g - 20), g + 400), m, replace=False))
        pos.append(p)
    pos = np.concatenate(pos).astype(np.int32)
    so = _csr(lens)
    for L in (16, 32, 64, 1):
        for gen_start in (gs, None):
            el_g = api.fixed_block_eligible(torch.from_numpy(pos).to(DEV),
                                            torch.from_numpy(so).to(DEV), L,
                                            gen_start=None if gen_start is None
                                            else torch.from_numpy(gen_start).to(DEV))
            el_o = oracle.fixed_block_eligible(pos, so, L, gen_start=gen_start)
            assert np.array_equal(host(el_g).numpy(), el_o), (L, gen_start is None)


def test_fixed_block_then_threshold():
    # the baseline schedule: the active block's rows under the threshold rule
    pos, offs = synth.gen_positions("llada", DEV)
    conf = torch.from_numpy(_conf_mix(pos.numel(), 3)).to(DEV)
    for L in (16, 32, 64):
        el = api.fixed_block_eligible(pos, offs, L, gen_start=torch.tensor(
            [int(host(pos)[0])], device=DEV, dtype=torch.int32))
        assert int(host(el).sum()) == L
        c, n = api.fastdllm_select(conf, offs, 0.9, eligible=el)
        c_o, n_o = oracle.fastdllm_select(f64(conf), host(offs).numpy(), float(np.float32(0.9)),
                                          eligible=host(el).numpy())
        assert np.array_equal(host(c).numpy(), c_o) and int(host(n)[0]) == int(n_o[0])


# ------------------------------------------------------------- DAPD step

def _dapd_step_case(attn, pos, so, conf, gen_len, tau, m_max, tag, pre_unmask=True,
                    random_shape=False):
    out = api.dapd_step(attn, pos, so, conf, tau, gen_len=gen_len, pre_unmask=pre_unmask,
                        m_max=m_max, want_degree=True, want_key=True)
    plain = api.dapd_select(attn, pos, so, conf, tau, m_max=m_max, want_key=True, want_sym=True)
    torch.cuda.synchronize()
    so_h = host(so).numpy()
    conf_h = host(conf).numpy()
    gl = None if gen_len is None else host(gen_len).numpy()
    t32 = float(np.float32(tau))
    ref = oracle.dapd_step(host(attn), host(pos).numpy(), so_h, conf_h.astype(np.float64), t32,
                           gen_len=gl, pre_unmask=pre_unmask)
    ref_plain = oracle.dapd_select(host(attn), host(pos).numpy(), so_h,
                                   conf_h.astype(np.float64), t32, m_max=m_max)
    commit, stage = host(out["commit"]).numpy(), host(out["stage"]).numpy()
    assert np.array_equal(stage, ref["stage"]), f"{tag}: stage"
    pc = host(plain["commit"]).numpy()
    fl = Flags(f"dapd_step {tag}")
    for b in range(len(so_h) - 1):
        lo, hi = so_h[b], so_h[b + 1]
        pre = (conf_h[lo:hi] == np.float32(1.0)) if pre_unmask else np.zeros(hi - lo, bool)
        if stage[b]:
            # late stage: exact (threshold on the given fp32 confidences)
            assert np.array_equal(commit[lo:hi], ref["commit"][lo:hi]), f"{tag} seq {b}: late"
            assert np.all(np.isnan(f64(out["degree"])[lo:hi]))
        else:
            # graph stage: the plain selection of the same call, plus pre-unmask
            want = (pc[lo:hi].astype(bool) | pre).astype(np.uint8)
            assert np.array_equal(commit[lo:hi], want), f"{tag} seq {b}: graph stage"
            M = hi - lo
            so_ = ref_plain["sym"][b][:M, :M]
            fl.check(np.array_equal(commit[lo:hi], ref["commit"][lo:hi]), True,
                     lambda: dapd_explained(so_, ref_plain["key"][lo:hi], t32), f"seq {b}")
        assert int(host(out["n_commit"])[b]) == int(commit[lo:hi].sum())
    fl.report() if random_shape else fl.assert_none()
    print(f"[dapd_step] {tag}: stages {stage.tolist()} committed "
          f"{[int(commit[so_h[b]:so_h[b + 1]].sum()) for b in range(len(so_h) - 1)]}")
    return out


@pytest.mark.parametrize("variant", ["peak", "cov"])
def test_dapd_step_full(variant):
    spec = synth.SPECS["dapd"]
    cur, prev, so, ri = synth.logits("dapd", DEV)
    g = api.step_stats(cur)
    pos, offs = synth.gen_positions("dapd", DEV)
    attn = synth.attention("dapd", DEV, variant=variant, masked_pos=pos[:spec.rows])
    conf = g["conf"].clone()
    conf[5] = 1.0                      # graph-stage sequence 0: pre-unmasked
    conf[spec.rows + 9] = 1.0          # sequence 1
    conf[3 * spec.rows + 17] = 1.0     # a late-stage sequence
    # 256 masked rows each: late iff gen_len > 512 (512 itself stays in the graph stage)
    gen_len = torch.tensor([256, 300, 600, 512, 513, 400, 1000, 256], device=DEV,
                           dtype=torch.int32)[:offs.numel() - 1].contiguous()
    _dapd_step_case(attn, pos, offs, conf, gen_len, 0.01, 256, f"dapd/{variant}")


def test_dapd_step_without_policy_equals_select():
    cur, prev, so, ri = synth.logits("tiny", DEV)
    g = api.step_stats(cur)
    attn = synth.attention("tiny", DEV)
    pos, offs = synth.gen_positions("tiny", DEV)
    a = api.dapd_step(attn, pos, offs, g["conf"], 0.01, gen_len=None, pre_unmask=False, m_max=32)
    b = api.dapd_select(attn, pos, offs, g["conf"], 0.01, m_max=32)
    assert torch.equal(a["commit"], b["commit"]) and torch.equal(a["n_commit"], b["n_commit"])
    assert int(host(a["stage"]).sum()) == 0


def test_dapd_step_late_fallback_and_scattered():
    spec = synth.Spec("scat", 11, 3, 40, 512, torch.bfloat16, 2.0, 0.6, 12.0, None,
                      n_lh=6, seq_len=100, attn_sigma=3.0)
    attn = synth.attention(spec, DEV)
    gen = torch.Generator().manual_seed(3)
    pos = torch.cat([torch.randperm(100, generator=gen)[:40].sort().values for _ in range(3)])
    pos = pos.to(device=DEV, dtype=torch.int32)
    so = torch.tensor([0, 40, 40, 77], device=DEV, dtype=torch.int32)
    conf = torch.rand(77, generator=gen).to(DEV) * 0.8          # nothing above 0.9
    conf[50] = 1.0
    conf[60] = float("nan")
    # seq 0 (40 rows) graph stage, seq 1 empty, seq 2 (37 rows of 100) late
    gen_len = torch.tensor([60, 10, 100], device=DEV, dtype=torch.int32)
    for pre in (True, False):
        _dapd_step_case(attn, pos[:77].contiguous(), so, conf, gen_len, 0.02, 45,
                        f"scattered pre={pre}", pre_unmask=pre)


# ------------------------------------------------------------ random shapes

@pytest.mark.parametrize("seed", [71, 72, 73, 74, 75, 76])
def test_schedules_random_shapes(seed):
    # top-K, factor decoding and fixed-block eligibility on random sequence
    # lengths (empty, single rows, the 1024-row limit and past it), random
    # K, f, block length and eligibility: bit for bit against the oracle
    g = np.random.default_rng(seed)
    lens = [int(x) for x in g.choice([0, 1, 2, 31, 64, 65, 255, 511, 1023, 1024, 1025, 1300],
                                     int(g.integers(1, 9)))]
    so = _csr(lens)
    n = int(so[-1])
    conf = _conf_mix(n, seed)
    el = (g.random(n) < g.uniform(0.1, 1.0)).astype(np.uint8) if g.integers(0, 2) else None
    so_d, conf_d = torch.from_numpy(so).to(DEV), torch.from_numpy(conf).to(DEV)
    el_d = None if el is None else torch.from_numpy(el).to(DEV)
    over = [b for b, m in enumerate(lens) if m > 1024]
    ok = [b for b, m in enumerate(lens) if m <= 1024]
    k = int(g.integers(1, 1100))
    c_g, n_g = (host(x).numpy() for x in api.topk_select(conf_d, so_d, k, eligible=el_d))
    c_o, n_o = oracle.topk_select(conf.astype(np.float64), so, k, eligible=el)
    f = float(np.float32(g.choice([1e-3, 0.1, 0.5, 1.0, 2.0, 10.0, 100.0]) * g.uniform(0.5, 1.5)))
    fc_g, fn_g, ce_g = (host(x).numpy() for x in api.factor_select(conf_d, so_d, f,
                                                                   eligible=el_d))
    fc_o, fn_o, ce_o = oracle.factor_select(conf.astype(np.float64), so, f, eligible=el)
    tag = f"seed {seed}: lens {lens} k {k} f {f:.4g} eligible {el is not None}"
    for b in ok:
        lo, hi = so[b], so[b + 1]
        assert np.array_equal(c_g[lo:hi], c_o[lo:hi]) and n_g[b] == n_o[b], f"{tag} top-K seq {b}"
        assert np.array_equal(fc_g[lo:hi], fc_o[lo:hi]) and fn_g[b] == fn_o[b] and \
            ce_g[b] == ce_o[b], f"{tag} factor seq {b}"
    for b in over:
        lo, hi = so[b], so[b + 1]
        assert n_g[b] == -1 and c_g[lo:hi].sum() == 0, f"{tag} top-K over-long seq {b}"
        assert fn_g[b] == -1 and fc_g[lo:hi].sum() == 0 and ce_g[b] == 0, f"{tag} factor seq {b}"
    # fixed-block eligibility over sorted positions starting near gen_start
    gs = g.integers(0, 2000, len(lens)).astype(np.int32)
    pos = np.concatenate([np.sort(g.choice(np.arange(max(0, s - 30), s + 3 * m + 40), m,
                                           replace=False)) if m else np.zeros(0, np.int64)
                          for m, s in zip(lens, gs)]).astype(np.int32)
    L = int(g.choice([1, 16, 32, 64, 100]))
    for start in (gs, None):
        el_g = api.fixed_block_eligible(torch.from_numpy(pos).to(DEV), so_d, L,
                                        gen_start=None if start is None
                                        else torch.from_numpy(start).to(DEV))
        el_o = oracle.fixed_block_eligible(pos, so, L, gen_start=start)
        assert np.array_equal(host(el_g).numpy(), el_o), f"{tag} fixed block L {L}"
    print(f"[schedules] {tag}: top-K {n_g.tolist()} factor {fn_g.tolist()}")


@pytest.mark.parametrize("seed", [81, 82, 83, 84])
def test_dapd_step_random_shapes(seed):
    # the full DAPD step on random shapes: batch, rows, maps, S, attention
    # dtype, tau, generation lengths on both sides of the late-stage switch,
    # pre-unmask on and off, exact-1.0 confidences planted
    g = np.random.default_rng(seed)
    B, rows = int(g.integers(1, 5)), int(g.integers(2, 129))
    spec = synth.Spec(f"dsrand{seed}", seed, B, rows, 64, torch.bfloat16, 2.0, 0.5, 12.0, None,
                      n_lh=int(g.integers(1, 9)), seq_len=rows + int(g.integers(0, 40)),
                      attn_sigma=float(g.uniform(0.5, 3.0)),
                      attn_dtype=(torch.bfloat16, torch.float32)[int(g.integers(0, 2))])
    attn = synth.attention(spec, DEV)
    pos, offs = synth.gen_positions(spec, DEV)
    conf = torch.from_numpy(g.random(B * rows).astype(np.float32)).to(DEV)
    conf[torch.from_numpy(g.random(B * rows) < 0.05).to(DEV)] = 1.0
    gen_len = torch.from_numpy(g.integers(rows, 3 * rows + 2, B).astype(np.int32)).to(DEV)
    tau = float((0.005, 0.02, 0.1)[int(g.integers(0, 3))])
    m_max = rows + int(g.integers(0, 20))
    for pre in (True, False):
        _dapd_step_case(attn, pos, offs, conf, gen_len, tau, m_max,
                        f"random seed {seed} B {B} rows {rows} pre={pre}", pre_unmask=pre)


def test_every_rule_with_all_sequences_empty():
    # a batch whose sequences are all empty (nothing left to decode): the
    # per-row tensors have no storage, and every rule call still runs and
    # reports each sequence (nothing committed), as the oracle does
    so = torch.zeros(4, device=DEV, dtype=torch.int32)          # three empty sequences
    so_h = host(so).numpy()
    e32 = torch.empty(0, device=DEV, dtype=torch.float32)
    ei32 = torch.empty(0, device=DEV, dtype=torch.int32)
    c, n = api.fastdllm_select(e32, so, 0.9)
    assert c.numel() == 0 and host(n).tolist() == [0, 0, 0]
    c, n = api.topk_select(e32, so, 4)
    assert host(n).tolist() == list(oracle.topk_select(np.zeros(0), so_h, 4)[1]) == [0, 0, 0]
    c, n, ce = api.factor_select(e32, so, 1.0)
    _, n_o, ce_o = oracle.factor_select(np.zeros(0), so_h, 1.0)
    assert host(n).tolist() == list(n_o) and host(ce).tolist() == list(ce_o)
    L, S = api.depcap_boundary(e32, e32, so, l_min=8, l_max=128)
    assert host(L).tolist() == list(oracle.depcap_boundary(np.zeros(0), np.zeros(0), so_h, 128,
                                                           8, 1.2)[0]) == [0, 0, 0]
    logits = torch.randn(5, 64, device=DEV)
    r = api.cap_select(logits, torch.empty(0, device=DEV, dtype=torch.int64), so, e32, ei32, e32,
                       k_max=8)
    assert host(r["n_commit"]).tolist() == [0, 0, 0]
    el = api.fixed_block_eligible(ei32, so, 32)
    assert el.numel() == 0
    attn = torch.rand(3, 2, 16, 16, device=DEV)
    r = api.dapd_select(attn, ei32, so, e32, 0.01, m_max=16)
    assert host(r["n_commit"]).tolist() == [0, 0, 0]
    gen_len = torch.tensor([0, 4, 16], device=DEV, dtype=torch.int32)
    r = api.dapd_step(attn, ei32, so, e32, 0.01, gen_len=gen_len, m_max=16)
    ref = oracle.dapd_step(host(attn), np.zeros(0, np.int32), so_h, np.zeros(0), 0.01,
                           gen_len=host(gen_len).numpy())
    assert host(r["n_commit"]).tolist() == [0, 0, 0]
    assert np.array_equal(host(r["stage"]).numpy(), ref["stage"])


def test_schedule_parameters_at_their_extremes():
    # factor decoding with f <= 0 (no n satisfies the bound: the fallback),
    # a tiny f, f = 1e30 and +inf (every eligible row); top-K with the largest
    # k; a fixed block longer than any generation.  Bit-exact against the
    # oracle, with the over-long sequence reported
    so, conf, el = _inputs(19)
    conf_g, so_g, el_g = (torch.from_numpy(x).to(DEV) for x in (conf, so, el))
    for f in (0.0, -1.0, 1e-30, 1e30, float("inf")):
        f32 = float(np.float32(f))
        c_g, n_g, ce_g = (host(x).numpy() for x in api.factor_select(conf_g, so_g, f,
                                                                      eligible=el_g))
        c_o, n_o, ce_o = oracle.factor_select(conf.astype(np.float64), so, f32, eligible=el)
        for b, m in enumerate(LENS):
            lo, hi = so[b], so[b + 1]
            if m > 1024:
                continue
            assert np.array_equal(c_g[lo:hi], c_o[lo:hi]), f"f={f} seq {b}"
            assert n_g[b] == n_o[b] and ce_g[b] == ce_o[b], f"f={f} seq {b}"
        _check_over_long(c_g, n_g, so)
    k = 2 ** 31 - 1
    c_g, n_g = (host(x).numpy() for x in api.topk_select(conf_g, so_g, k, eligible=el_g))
    c_o, n_o = oracle.topk_select(conf.astype(np.float64), so, k, eligible=el)
    for b, m in enumerate(LENS):
        if m <= 1024:
            lo, hi = so[b], so[b + 1]
            assert np.array_equal(c_g[lo:hi], c_o[lo:hi]) and n_g[b] == n_o[b], f"k max seq {b}"
    _check_over_long(c_g, n_g, so)
    pos = np.concatenate([np.arange(m) * 3 + 7 for m in LENS]).astype(np.int32)
    for L in (2 ** 30, 2 ** 31 - 1):
        e_g = api.fixed_block_eligible(torch.from_numpy(pos).to(DEV), so_g, L)
        e_o = oracle.fixed_block_eligible(pos, so, L)
        assert np.array_equal(host(e_g).numpy(), e_o), L


def test_dapd_step_policy_at_its_extremes():
    # the late-stage switch and threshold at their limits: late_frac 0 or
    # below (no sequence is late), 1, a large value and +inf (every sequence
    # with masks left is late), late_tau -inf (every row passes), +inf (only
    # the fallback) and 0.  Stage per sequence and commits against the oracle
    spec = synth.Spec("scatx", 13, 3, 40, 512, torch.bfloat16, 2.0, 0.6, 12.0, None,
                      n_lh=6, seq_len=100, attn_sigma=3.0)
    attn = synth.attention(spec, DEV)
    gen = torch.Generator().manual_seed(5)
    pos = torch.cat([torch.randperm(100, generator=gen)[:40].sort().values for _ in range(3)])
    pos = pos[:77].to(device=DEV, dtype=torch.int32).contiguous()
    so = torch.tensor([0, 40, 40, 77], device=DEV, dtype=torch.int32)
    conf = torch.rand(77, generator=gen).to(DEV)
    conf[50] = 1.0
    gen_len = torch.tensor([60, 10, 100], device=DEV, dtype=torch.int32)
    so_h, conf_h = host(so).numpy(), host(conf).numpy().astype(np.float64)
    for lf, lt in ((0.0, 0.9), (-1.0, 0.9), (1.0, 0.9), (1e30, 0.9), (float("inf"), 0.9),
                   (float("inf"), float("-inf")), (float("inf"), float("inf")),
                   (float("inf"), 0.0)):
        out = api.dapd_step(attn, pos, so, conf, 0.02, gen_len=gen_len, late_frac=lf,
                            late_tau=lt, m_max=45)
        torch.cuda.synchronize()
        ref = oracle.dapd_step(host(attn), host(pos).numpy(), so_h, conf_h,
                               float(np.float32(0.02)), gen_len=host(gen_len).numpy(),
                               late_frac=float(np.float32(lf)), late_tau=float(np.float32(lt)))
        tag = f"late_frac={lf} late_tau={lt}"
        assert np.array_equal(host(out["stage"]).numpy(), ref["stage"]), tag
        assert np.array_equal(host(out["commit"]).numpy(), ref["commit"]), tag
        assert np.array_equal(host(out["n_commit"]).numpy(), ref["n_commit"]), tag
