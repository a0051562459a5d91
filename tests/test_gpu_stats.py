"""GPU parity of dlm_step_stats against the fp64 oracle (marked gpu).

Sizes span several chunks per lane, a ragged vocabulary tail, row gathers and
padded leading dimensions; the full LLaDA-shaped step is compared on every
row, the Dream- and stress-shaped launches (the bench's launch configuration)
on sampled rows the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
from _parity import assert_close, host
from diffusion_lm_unmask_amd import api, synth

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("poisoned_outputs")]
DEV = "cuda"


def _compare(cur, prev, row_index=None, vocab=None, tag="", split=True):
    out = api.step_stats(cur, prev, row_index=row_index, vocab=vocab, split=split)
    torch.cuda.synchronize()
    ri = None if row_index is None else host(row_index).numpy()
    ref = oracle.step_stats(host(cur), host(prev) if prev is not None else None, row_index=ri,
                            vocab=vocab)
    w = {}
    for k in ("conf", "entropy", "lse") + (("kl",) if prev is not None else ()):
        w[k] = assert_close(out[k], ref[k], f"{tag}{k}")
    assert np.array_equal(host(out["argmax"]).numpy(), ref["argmax"]), f"{tag}argmax"
    print(f"[stats] {tag} max err " + " ".join(f"{k}={v:.2e}" for k, v in w.items()))
    return out, ref


@pytest.mark.parametrize("with_prev", [True, False])
def test_tiny_fp32(with_prev):
    cur, prev, so, ri = synth.logits("tiny", DEV)
    _compare(cur, prev if with_prev else None, tag="tiny ")


@pytest.mark.parametrize("rows,vocab", [(37, 5000), (5, 7), (3, 8), (130, 32768 + 24), (2, 1)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_shapes(rows, vocab, dtype):
    spec = synth.Spec("ragged", 7, 1, rows, vocab, dtype, 2.0, 0.6, 12.0, 0.5)
    cur, prev, so, ri = synth.logits(spec, DEV)
    _compare(cur, prev, tag=f"{rows}x{vocab} {dtype} ")
    _compare(cur, None, tag=f"{rows}x{vocab} {dtype} noprev ")


def test_padded_ld_and_row_gather():
    spec = synth.Spec("pad", 8, 1, 64, 3000, torch.bfloat16, 2.0, 0.6, 12.0, 0.5)
    cur, prev, so, ri = synth.logits(spec, DEV, vocab=3008)
    cur[:, 3000:] = 50.0                               # beyond the vocabulary: ignored
    prev[:, 3000:] = -50.0
    idx = torch.tensor([5, 63, 0, 5, 17, 40], device=DEV, dtype=torch.int64)
    _compare(cur, prev, row_index=idx, vocab=3000, tag="ld-pad ")
    _compare(cur, prev, row_index=idx, vocab=3000, tag="ld-pad unsplit ", split=False)
    # leading dimension that breaks 16-byte row alignment -> element-wise path
    big = torch.zeros(64, 3003, device=DEV, dtype=torch.bfloat16)
    big2 = torch.zeros_like(big)
    big[:, :3000] = cur[:, :3000]
    big2[:, :3000] = prev[:, :3000]
    _compare(big, big2, row_index=idx, vocab=3000, tag="ld-unaligned ")
    _compare(big, big2, row_index=idx, vocab=3000, tag="ld-unaligned unsplit ", split=False)


def test_non_finite_rows():
    spec = synth.Spec("nf", 9, 1, 12, 4100, torch.float32, 2.0, 0.6, 12.0, 0.5)
    cur, prev, so, ri = synth.logits(spec, DEV)
    ninf, nan, inf = float("-inf"), float("nan"), float("inf")
    cur[0, 10] = nan
    cur[1, :] = ninf
    cur[2, 100:] = ninf
    prev[3, 7] = ninf
    cur[4, 5] = inf
    cur[5, :] = nan
    prev[6, 2000] = nan
    cur[7, :4000] = ninf
    prev[7, :4000] = ninf                           # p = 0 and q = 0 together
    cur[8, 3] = cur[8].max() + 1.0
    cur[8, 4099] = cur[8, 3]                        # tie across chunk and tail
    for dt in (torch.float32, torch.bfloat16):
        c = cur.to(dt)
        p = prev.to(dt)
        _compare(c, p, tag=f"non-finite {dt} ")
        # one workgroup per row: bf16 with prev takes the 768-thread rows
        _compare(c, p, tag=f"non-finite {dt} unsplit ", split=False)


def test_argmax_ties_lowest_index():
    x = torch.zeros(4, 126464, device=DEV, dtype=torch.bfloat16)
    x[0, [126463, 9, 70000]] = 3.0
    x[1, [4096, 4095]] = 2.0
    x[3] = torch.randn(126464, device=DEV).to(torch.bfloat16)
    out, ref = _compare(x, None, tag="ties ")
    assert list(host(out["argmax"]).numpy()[:3]) == [9, 4095, 0]


def test_llada_full_all_rows_and_determinism():
    cur, prev, so, ri = synth.logits("llada", DEV)
    out, ref = _compare(cur, prev, tag="llada ")
    again = api.step_stats(cur, prev)
    for k in ("conf", "entropy", "kl", "lse", "argmax"):
        assert torch.equal(out[k], again[k]), f"{k} not bitwise reproducible"


@pytest.mark.parametrize("name,sample", [("dream", 96), ("stress", 64)])
def test_full_size_sampled(name, sample):
    cur, prev, so, ri = synth.logits(name, DEV)
    out = api.step_stats(cur, prev)                       # the full launch
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(123)
    idx = torch.randperm(cur.shape[0], generator=g)[:sample].sort().values
    sub_c = host(cur[idx.to(DEV)])
    sub_p = host(prev[idx.to(DEV)]) if prev is not None else None
    ref = oracle.step_stats(sub_c, sub_p)
    for k in ("conf", "entropy", "lse") + (("kl",) if prev is not None else ()):
        w = assert_close(out[k][idx.to(DEV)], ref[k], f"{name} {k}")
        print(f"[stats] {name} sampled {k} max err {w:.2e}")
    assert np.array_equal(host(out["argmax"][idx.to(DEV)]).numpy(), ref["argmax"])
    # invariants on every row of the launch
    conf, H = out["conf"], out["entropy"]
    V = cur.shape[1]
    assert bool(torch.all(conf <= 1.0)) and bool(torch.all(conf >= 1.0 / V * (1 - 1e-5)))
    assert bool(torch.all(H >= -1e-5)) and bool(torch.all(H <= np.log(V) + 1e-5))
    if prev is not None:
        assert bool(torch.all(out["kl"] >= -1e-5))


@pytest.mark.parametrize("rows,vocab", [(1, 126464), (3, 126467), (37, 100003), (256, 126464)])
def test_split_rows_match_oracle_and_repeat(rows, vocab):
    # few rows over a wide vocabulary: each row is split over several
    # workgroups and merged by the last one to arrive
    spec = synth.Spec("split", 12, 1, rows, vocab, torch.bfloat16, 2.0, 0.6, 12.0, 0.5)
    cur, prev, so, ri = synth.logits(spec, DEV)
    out, ref = _compare(cur, prev, tag=f"split {rows}x{vocab} ")
    single = api.step_stats(cur, prev, split=False)
    for k in ("conf", "entropy", "kl", "lse"):
        assert_close(single[k], ref[k], f"single-workgroup {k}")
    assert torch.equal(single["argmax"], out["argmax"])
    for _ in range(3):                                    # arrival order must not matter
        again = api.step_stats(cur, prev)
        for k in ("conf", "entropy", "kl", "lse", "argmax"):
            assert torch.equal(out[k], again[k]), f"split {k} not bitwise reproducible"


def test_split_rows_non_finite():
    spec = synth.Spec("splitnf", 13, 1, 6, 126464, torch.float32, 2.0, 0.6, 12.0, 0.5)
    cur, prev, so, ri = synth.logits(spec, DEV)
    cur[0, 100000] = float("nan")                       # in a late split
    cur[1, 5:] = float("-inf")                          # -inf across every split
    prev[2, 120000] = float("-inf")                     # KL = +inf
    cur[3, 126463] = cur[3].max() + 2.0                 # max in the last element
    cur[4, 0] = cur[4].max() + 2.0                      # max in the first element
    _compare(cur.to(torch.bfloat16), prev.to(torch.bfloat16), tag="split non-finite bf16 ")
    _compare(cur, prev, tag="split non-finite f32 ")


def test_one_workspace_serves_any_row_count():
    # a 37-row call leaves its partials where a 256-row layout would put
    # counters if the layout depended on the row count; it must not
    outs = []
    for rows in (37, 256, 3, 256, 37):
        spec = synth.Spec("mix", 14 + rows, 1, rows, 126464, torch.bfloat16, 2.0, 0.6, 12.0, 0.5)
        cur, prev, so, ri = synth.logits(spec, DEV)
        outs.append(_compare(cur, prev, tag=f"shared workspace {rows} rows "))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("gap", [30.0, 120.0])
def test_stats_large_kl(dt, gap):
    # current and previous rows peaked on different tokens, the peak `gap`
    # above N(0, 1) noise: KL is about the gap (up to ~123 nats), where the
    # fp32 output spacing is largest; still within 1e-5 of the oracle
    g = np.random.default_rng(int(gap))
    n, V = 8, 126464
    cur = torch.from_numpy(g.normal(0, 1, (n, V)).astype(np.float32))
    prev = torch.from_numpy(g.normal(0, 1, (n, V)).astype(np.float32))
    for r in range(n):
        a, b = g.integers(0, V, 2)
        cur[r, a] += gap
        prev[r, b] += gap
    cur, prev = cur.to(dt), prev.to(dt)
    gs = api.step_stats(cur.to(DEV), prev.to(DEV))
    torch.cuda.synchronize()
    o = oracle.step_stats(cur, prev)
    assert float(np.min(o["kl"])) > gap - 15.0
    for k in ("conf", "entropy", "kl", "lse"):
        assert_close(gs[k], o[k], f"large KL gap {gap} {dt} {k}")


# ------------------------------------------------------------ closed forms
# Rows whose statistics have closed forms (DepCap, Methodology: H and KL of
# each position's distribution; Fast-dLLM review, Method: max-softmax
# confidence), on every path that computes statistics: the streaming path
# (512-thread workgroups; split rows with a workspace; 256-thread workgroups
# from 4096 rows up), the element-wise path (rows holding -inf), and the
# fused step's streaming launch.
#   uniform row (all logits c)       conf = 1/V, H = log V, lse = c + log V, argmax 0
#   one-hot row (1000 at j, 0 else)  conf = 1, H = 0, lse = 1000, argmax j
#   -inf except n equal entries      conf = 1/n, H = log n (element-wise path)
#   -inf except one entry            conf = 1, H = 0 exactly (element-wise path)
#   prev == cur                      KL = 0 exactly, on every row

def _closed_form_rows(n_rows, V, dtype):
    x = torch.zeros(n_rows, V, dtype=torch.float32)
    kind, want = [], []
    for r in range(n_rows):
        k = r % 5
        if k == 0:                                           # uniform at c
            c = (0.0, 3.5, -7.25)[(r // 5) % 3]
            x[r] = c
            want.append((1.0 / V, np.log(V), c + np.log(V), 0))
        elif k == 1:                                         # one-hot 1000
            j = (r * 7919) % V
            x[r, j] = 1000.0
            want.append((1.0, 0.0, 1000.0, j))
        elif k == 2:                                         # one-hot 1000 with negative rest
            j = (r * 104729) % V
            x[r] = -3.0
            x[r, j] = 1000.0
            want.append((1.0, 0.0, 1000.0, j))
        elif k == 3:                                         # n equal entries, -inf elsewhere
            n = 1 + (r * 31) % min(V, 97)
            x[r] = float("-inf")
            idx = torch.arange(n) * (V // n)
            x[r, idx] = 2.0
            want.append((1.0 / n, np.log(n), 2.0 + np.log(n), 0))
        else:                                                # a single finite entry
            j = (r * 13) % V
            x[r] = float("-inf")
            x[r, j] = -5.0
            want.append((1.0, 0.0, -5.0, j))
        kind.append(k)
    return x.to(dtype).to(DEV), np.array(kind), want


def _check_closed_forms(out, kind, want, tag):
    conf, ent, lse = (host(out[k]).double().numpy() for k in ("conf", "entropy", "lse"))
    kl, arg = host(out["kl"]).double().numpy(), host(out["argmax"]).numpy()
    for r, (c, h, l, j) in enumerate(want):
        assert arg[r] == j, f"{tag} row {r} (kind {kind[r]}): argmax {arg[r]} != {j}"
        assert kl[r] == 0.0, f"{tag} row {r} (kind {kind[r]}): KL {kl[r]!r} with prev == cur"
        assert abs(ent[r] - h) <= 1e-5, f"{tag} row {r}: entropy {ent[r]} vs {h}"
        assert abs(lse[r] - l) <= 1e-5 + 6.2e-5 * (abs(l) >= 512), f"{tag} row {r}: lse {lse[r]} vs {l}"
        if kind[r] in (0, 3):
            assert abs(conf[r] * (1.0 / c) - 1.0) <= 1e-5, f"{tag} row {r}: conf {conf[r]} vs {c}"
        else:
            assert abs(conf[r] - 1.0) <= 1e-6, f"{tag} row {r}: conf {conf[r]}"
            assert abs(ent[r]) <= 1e-6, f"{tag} row {r}: entropy {ent[r]}"
        if kind[r] == 4:                                     # element-wise path: exact
            assert conf[r] == 1.0 and ent[r] == 0.0, f"{tag} row {r}: {conf[r]!r} {ent[r]!r}"


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 126464), (torch.float32, 4099)])
@pytest.mark.parametrize("n_rows,split", [(40, True), (40, False), (300, False)])
def test_closed_forms(dtype, V, n_rows, split):
    cur, kind, want = _closed_form_rows(n_rows, V, dtype)
    out = api.step_stats(cur, cur, split=split)
    torch.cuda.synchronize()
    _check_closed_forms(out, kind, want, f"{dtype} V={V} rows={n_rows} split={split}")
    fused = api.decide_step(cur, cur)                        # the fused step's launch 1
    torch.cuda.synchronize()
    _check_closed_forms(fused, kind, want, f"fused {dtype} V={V} rows={n_rows}")


def test_closed_forms_256_thread_rows():
    # 4096 rows take the 256-thread workgroups
    cur, kind, want = _closed_form_rows(4096, 1000, torch.bfloat16)
    out = api.step_stats(cur, cur)
    torch.cuda.synchronize()
    _check_closed_forms(out, kind, want, "4096 x 1000 bf16")


@pytest.mark.parametrize("extra", [0, 1])
def test_thread_counts_at_the_compute_unit_count(extra):
    # bf16 rows with a previous row, at most one per compute unit, take the
    # 768-thread workgroups; one row more takes 512.  Both against the oracle
    # on a ragged vocabulary (a partial last segment and a tail element), and
    # the fused step's launch 1 bitwise equal to the call in both shapes
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    spec = synth.Spec("cus", 11, 1, cus + extra, 20011, torch.bfloat16, 2.0, 0.6, 12.0, 0.5)
    cur, prev, so, ri = synth.logits(spec, DEV)
    out, _ = _compare(cur, prev, tag=f"{cus + extra} rows ")
    fused = api.decide_step(cur, prev)
    solo = api.step_stats(cur, prev, split=False)
    torch.cuda.synchronize()
    for k in ("conf", "argmax", "entropy", "kl", "lse"):
        assert torch.equal(fused[k].view(torch.int32), solo[k].view(torch.int32)), k
        assert torch.equal(out[k].view(torch.int32), solo[k].view(torch.int32)), k


# Rows that move the lane reference: it trails the running max and moves
# (an exact power-of-two rescale) only once the max passes it by a margin, so
# rows whose max keeps rising across a lane's chunks, or jumps in the last
# chunk, rescale many times or late.  Kinds (r % 6):
#   0  rising ramp, 60 nats over the row (the max rises in every chunk)
#   1  falling ramp (the max sits in the first chunk)
#   2  N(0, 2) with a +40 spike on the last element (a rescale in the tail)
#   3  N(0, 2) with the first half of the vocabulary at -inf (masked)
#   4  sawtooth, 30 nats per 4096-element period
#   5  rising ramp, 200 nats over the row (rescales far apart in value)
# prev is cur plus N(0, 0.5) noise on every row.
def _trailing_reference_rows(n_rows, V, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    v = torch.arange(V, dtype=torch.float64)
    x = torch.empty(n_rows, V, dtype=torch.float64)
    for r in range(n_rows):
        k = r % 6
        if k == 0:
            x[r] = 60.0 * v / V - 20.0
        elif k == 1:
            x[r] = 40.0 - 60.0 * v / V
        elif k == 2:
            x[r] = torch.randn(V, generator=g, dtype=torch.float64) * 2.0
            x[r, V - 1] = 40.0
        elif k == 3:
            x[r] = torch.randn(V, generator=g, dtype=torch.float64) * 2.0
            x[r, : V // 2] = float("-inf")
        elif k == 4:
            x[r] = 30.0 * torch.remainder(v, 4096.0) / 4096.0
        else:
            x[r] = 200.0 * v / V - 100.0
    prev = x + torch.randn(n_rows, V, generator=g, dtype=torch.float64) * 0.5
    return x.to(dtype).to(DEV), prev.to(dtype).to(DEV)


@pytest.mark.parametrize("rows,vocab,dtype,with_prev,split", [
    (256, 126464, torch.bfloat16, True, False),   # 768-thread rows (the LLaDA shape)
    (300, 20011, torch.bfloat16, True, False),    # 512 threads, two segments in flight
    (300, 20011, torch.bfloat16, False, False),   # the same without a previous row
    (4096, 3001, torch.bfloat16, True, False),    # 256-thread rows
    (64, 20011, torch.float32, True, False),      # fp32 chunks
    (64, 20011, torch.float32, True, True),       # fp32 rows split over workgroups
    (12, 126464, torch.bfloat16, True, True),     # bf16 rows split over workgroups
])
def test_rows_that_move_the_lane_reference(rows, vocab, dtype, with_prev, split):
    cur, prev = _trailing_reference_rows(rows, vocab, dtype, seed=rows * 7 + vocab)
    prev = prev if with_prev else None
    tag = f"{rows} x {vocab} {dtype} prev={with_prev} split={split} "
    out = api.step_stats(cur, prev, split=split)
    torch.cuda.synchronize()
    ref = oracle.step_stats(host(cur), host(prev) if prev is not None else None)
    for k in ("conf", "entropy", "lse") + (("kl",) if with_prev else ()):
        assert_close(out[k], ref[k], f"{tag}{k}")
    assert np.array_equal(host(out["argmax"]).numpy(), ref["argmax"]), f"{tag}argmax"
    if with_prev and not split:
        # the fused step's launch 1 runs the same kernel: bitwise equal
        fused = api.decide_step(cur, prev)
        torch.cuda.synchronize()
        for k in ("conf", "argmax", "entropy", "kl", "lse"):
            assert torch.equal(fused[k].view(torch.int32), out[k].view(torch.int32)), f"{tag}{k}"


# Finite logits of extreme size: near the bf16 limit, and below the fold's
# running-max sentinel (-1e30).  Their exponents overflow the fold, so these
# rows reach the element-wise path, which must still give the definitions'
# values.  lse is stored in fp32, so it is compared to fp32 rounding of its
# own size; everything else at 1e-5 absolute, argmax exactly.
def _extreme_rows(V, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.empty(6, V, dtype=torch.float64)
    x[0] = -3.0e38                                   # all equal, below the sentinel
    x[1] = -2.0e38 - torch.rand(V, generator=g, dtype=torch.float64) * 1e38
    x[2] = 3.0e38                                    # all equal, near the top of the range
    x[3] = torch.randn(V, generator=g, dtype=torch.float64) * 2.0
    x[3, V // 3] = 1.0e30                            # one huge finite entry
    x[4] = -1.5e30 + torch.randn(V, generator=g, dtype=torch.float64) * 1e28
    x[5] = torch.randn(V, generator=g, dtype=torch.float64) * 1e20
    return x.to(dtype).to(DEV)


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 126464), (torch.float32, 4099)])
def test_extreme_finite_logits(dtype, V):
    cur = _extreme_rows(V, dtype, seed=V)
    for prev in (None, cur):
        tag = f"extreme {dtype} V={V} prev={'cur' if prev is not None else 'none'} "
        out = api.step_stats(cur, prev, split=False)
        torch.cuda.synchronize()
        ref = oracle.step_stats(host(cur), host(prev) if prev is not None else None)
        for k in ("conf", "entropy") + (("kl",) if prev is not None else ()):
            assert_close(out[k], ref[k], f"{tag}{k}")
        lse_g = host(out["lse"]).double().numpy()
        lse_o = np.asarray(ref["lse"], np.float64)
        tol = np.maximum(1e-5, np.abs(lse_o) * 2.0 ** -23)
        assert np.all(np.abs(lse_g - lse_o) <= tol), (tag, lse_g, lse_o)
        assert np.array_equal(host(out["argmax"]).numpy(), ref["argmax"]), f"{tag}argmax"
        if prev is not None:
            assert np.all(host(out["kl"]).numpy() == 0.0), f"{tag}KL with prev == cur"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_non_finite_padding_beyond_a_ragged_vocabulary(dtype):
    # rows padded past a vocabulary that is not a multiple of the 16-byte
    # chunk, the padding holding NaN and +-inf: nothing past `vocab` may be
    # read into the statistics (a leak would turn them NaN or inf), on the
    # split, unsplit and fused paths
    V, ld = 3001, 3024
    g = torch.Generator().manual_seed(3001)
    cur = torch.randn(40, ld, generator=g) * 2.0
    prev = cur + torch.randn(40, ld, generator=g) * 0.5
    cur[:, V:] = float("nan")
    cur[::3, V + 1] = float("inf")
    prev[:, V:] = float("-inf")
    prev[1::3, V + 2] = float("nan")
    cur, prev = cur.to(dtype).to(DEV), prev.to(dtype).to(DEV)
    out, _ = _compare(cur, prev, vocab=V, tag="nan padding ")
    _compare(cur, prev, vocab=V, tag="nan padding unsplit ", split=False)
    for k in ("conf", "entropy", "kl", "lse"):
        assert bool(torch.isfinite(out[k]).all()), k
    fused = api.decide_step(cur, prev, vocab=V)
    solo = api.step_stats(cur, prev, vocab=V, split=False)
    torch.cuda.synchronize()
    for k in ("conf", "argmax", "entropy", "kl", "lse"):
        assert torch.equal(fused[k].view(torch.int32), solo[k].view(torch.int32)), k
