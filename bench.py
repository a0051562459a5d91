#!/usr/bin/env python3
"""Benchmark of the per-denoising-step unmask decision on one MI355X.

A step is one pass of the whole decision path over one batch of synthetic
input.  The headline step is the LLaDA-shaped workload as configured: one
sequence of 256 masked generation rows, vocabulary 126464, bf16 current and
previous-step logits, with

  statistics   confidence / argmax / entropy / KL / lse of all 256 rows
  Fast-dLLM    threshold 0.9 on the active 32-token block (rows 0-31)
  DepCap       DepGA-Block boundary over the 128-row window (lambda 1.2,
               L_min 8, L_max 128)

issued as one dlm_decide_step call (two launches: the statistics kernel, then
the two rules), back to back on one stream.  `value` is rows decided per
second; `roofline` is that of the statistics kernel (launch 1), timed by HIP
events that the launch itself sets to the kernel's start and end.

The other workloads run in the same process under the same clock, each as
one dlm_decide_step per step (sub-results under "workloads"):
  llada_all_rules  the LLaDA step plus CAP on block 0 and a DAPD graph over
                   the 256 rows from [1, 320, 768, 768] attention
  dapd             8 x 256 rows (no prev) + DAPD over [8, 320, 768, 768]
                   attention (literal: no edge at tau 0.01), and the same step
                   on the partner-covariance attention (edge-rich greedy)
  stress           64 x 1024 rows, cur + prev (33.15 GB) + DepCap + CAP (K 128)
  dream            16 x 256 rows, V 151936 (no prev) + CAP (0.7, K 64)
  tiny             1 x 32 rows, fp32, every rule (latency)
For the three V = 126464 workloads the statistics kernel's achieved HBM
bandwidth is reported against the 8 TB/s peak ("stats_kernel").

Inputs are resident in HBM before timing starts; LLaDA-sized inputs rotate
over `--replicas` copies so that consecutive steps miss the 256 MB Infinity
Cache (the larger workloads exceed it by themselves).  The CPU oracle is timed
on the LLaDA step on the host's cores (and on one core, on an 8-sequence
sample of the stress step and on the DAPD step), and its decisions are
compared with the GPU's on the same inputs ("oracle_parity").
Prints one JSON line (N = 1).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "masked-row decisions/sec and achieved HBM GB/s (% of peak), V=126464 bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
# the device sources each timed kernel is built from: a counter reading is
# only reported while they are unchanged since it was taken
KERNEL_SOURCES = {
    "k_step_rows": ("fused.hip", "stats_impl.h", "dlm_device.h"),
    "k_step_stream": ("fused.hip", "stats_impl.h", "dapd_impl.h", "dlm_device.h"),
}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "diffusion_lm_unmask_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(key: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, copy-calibrated), or None when absent or taken
    on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(key, {})
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


class TimingEvents:
    """Pairs of HIP timing events created without the system-scope fence
    (hipEventDisableSystemFence), handed to dlm_decide_step, whose launch 1
    sets them to its kernel's start and end.  They come from the HIP runtime
    already loaded into the process (torch's), so they are valid on torch's
    streams."""

    NO_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int):
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.hip = ctypes.CDLL(path)
        self.pairs = []
        for _ in range(n):
            pair = []
            for _ in range(2):
                e = ctypes.c_void_p()
                if self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.NO_SYSTEM_FENCE):
                    raise RuntimeError("hipEventCreateWithFlags failed")
                pair.append(e.value)
            self.pairs.append(tuple(pair))

    def durations_us(self):
        """Each pair's interval in microseconds (call after the device is synchronized)."""
        ms, out = ctypes.c_float(), []
        for a, b in self.pairs:
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                            ctypes.c_void_p(b)):
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value * 1000.0)
        return out

    def mean_us(self):
        """Average interval in microseconds (call after the device is synchronized)."""
        d = self.durations_us()
        return sum(d) / len(d)

    def close(self):
        for pair in self.pairs:
            for e in pair:
                self.hip.hipEventDestroy(ctypes.c_void_p(e))
        self.pairs = []


def gbs(nbytes, us):
    return nbytes / (us * 1e-6) / 1e9


class Step:
    """One decision step as prebuilt dlm_decide_step descriptors, one per
    input replica (api.step_descriptor marshals them once; the timed loop only
    calls the C entry point)."""

    def __init__(self, name, rows, replicas, stream, launch1_bytes, **parts):
        """replicas: one dict of step_descriptor arguments per input replica;
        `parts` are added to each (a replica's own entries take precedence)."""
        from diffusion_lm_unmask_amd import _lib, api
        self.name, self.rows, self.launch1_bytes = name, rows, launch1_bytes
        self.stream = stream
        self.L = _lib.lib()
        self.check = _lib.check
        self.built = [api.step_descriptor(**dict(parts, **r)) for r in replicas]
        self.descs = [b[0] for b in self.built]
        self.refs = [ctypes.byref(d) for d in self.descs]

    def run(self, i, ev=None):
        d = self.descs[i % len(self.descs)]
        d.launch1_begin_event = ev[0] if ev is not None else None
        d.launch1_end_event = ev[1] if ev is not None else None
        st = self.L.dlm_decide_step(self.refs[i % len(self.refs)], self.stream)
        if st:
            self.check(st, f"dlm_decide_step ({self.name})")

    def out(self, i=0):
        return self.built[i % len(self.built)][1]


def time_step(step: Step, steps: int, warmup: int):
    """ms per step over `steps` back-to-back steps (events around the batch,
    device synchronized on both sides), then the average duration of launch 1
    over a second run of the same steps (events set by the launch itself)."""
    import torch
    torch.cuda.synchronize()
    for i in range(warmup):
        step.run(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s = torch.cuda.ExternalStream(step.stream)
    t0.record(s)
    for i in range(steps):
        step.run(i)
    t1.record(s)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    ev = TimingEvents(steps)
    torch.cuda.synchronize()
    for i in range(steps):
        step.run(i, ev.pairs[i])
    torch.cuda.synchronize()
    d = sorted(ev.durations_us())
    us = sum(d) / len(d)
    # the spread of the launches behind the average (reported beside it)
    step.launch1_spread = {"min_us": round(d[0], 3), "p50_us": round(d[len(d) // 2], 3),
                           "p90_us": round(d[min(len(d) - 1, (9 * len(d)) // 10)], 3),
                           "max_us": round(d[-1], 3)}
    ev.close()
    for d in step.descs:
        d.launch1_begin_event = d.launch1_end_event = None
    return ms, us


def result(step: Step, ms, us, kernel, extra=None):
    r = {"rows": step.rows, "ms_per_step": round(ms, 5),
         "decisions_per_s": round(step.rows / (ms * 1e-3), 1),
         "launch1": {"kernel": kernel, "avg_us": round(us, 3),
                     "algorithmic_bytes": step.launch1_bytes,
                     "GB/s": round(gbs(step.launch1_bytes, us), 1),
                     "frac_of_peak": round(gbs(step.launch1_bytes, us) / PEAK_HBM_GBS, 4),
                     **getattr(step, "launch1_spread", {})}}
    if extra:
        r.update(extra)
    return r


def replicas_of(x, n):
    return [x] + [x.clone() for _ in range(n - 1)]


def block_mask(n, lo, hi, dev):
    import torch
    m = torch.zeros(n, device=dev, dtype=torch.uint8)
    m[lo:hi] = 1
    return m


def cpu_model():
    """The host CPU as /proc/cpuinfo names it (model name, family / model /
    stepping, clock and cache of the first processor entry) and the logical
    CPUs this process may run on and the machine has."""
    info = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if not line.strip():
                    if info:
                        break
                    continue
                k, _, v = line.partition(":")
                info.setdefault(k.strip(), v.strip())
    except OSError:
        pass
    name = info.get("model name", "unknown")
    extra = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    if "cpu MHz" in info:
        extra.append(f"{float(info['cpu MHz']):.0f} MHz")
    if "cache size" in info:
        extra.append(f"cache {info['cache size']}")
    extra.append(f"{len(os.sched_getaffinity(0))} of {os.cpu_count()} logical CPUs usable")
    return f"{name} ({', '.join(extra)})"


def _timed_reps(fn, seconds, min_reps=1):
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds and reps >= min_reps:
            return reps, el


def f32(x):
    import numpy as np
    return float(np.float32(x))


# ---------------------------------------------------------------- workloads

def llada_workloads(dev, stream, args, res):
    """The headline step and the all-rules LLaDA step; returns the headline
    pieces (step, inputs, rules) for the CPU baseline."""
    from diffusion_lm_unmask_amd import api, synth
    R = synth.RULES["llada"]
    spec = synth.SPECS["llada"]
    cur, prev, so, ri = synth.logits("llada", dev)
    n = spec.rows
    block = block_mask(n, *R["fast_block"], dev)
    curs, prevs = replicas_of(cur, args.replicas), replicas_of(prev, args.replicas)
    # the rows are the logits' rows in order: no row-index array (NULL)
    reps = [dict(logits=c, prev=p, seq_offsets=so, row_index=None) for c, p in zip(curs, prevs)]
    fast = dict(eligible=block, tau=R["tau"])
    depcap = dict(lam=R["lam"], l_min=R["l_min"], l_max=R["l_max"])
    stats_bytes = n * spec.vocab * 2 * 2
    head = Step("llada", n, reps, stream, stats_bytes, fast=fast, depcap=depcap)
    ms, us = time_step(head, args.steps, args.warmup)
    res["llada"] = result(head, ms, us, "k_step_rows (the statistics kernel)",
                          {"workload": "1 x 256 rows, V=126464 bf16 cur+prev; statistics + "
                                       "Fast-dLLM 0.9 on block 0 + DepCap (lambda 1.2, L_min 8, "
                                       "L_max 128)"})
    # the statistics call on its own (no workspace: the same kernel), back to
    # back through the C entry point with preallocated outputs
    import torch
    from diffusion_lm_unmask_amd import _lib
    L = _lib.lib()
    o = head.out(0)
    outs = [o[k].data_ptr() for k in ("conf", "argmax", "entropy", "kl", "lse")]
    calls = [(c.data_ptr(), p.data_ptr()) for c, p in zip(curs, prevs)]

    def stats_call(i):
        c, p = calls[i % len(calls)]
        st = L.dlm_step_stats(c, p, _lib.BF16, spec.vocab, spec.vocab, None, n, *outs,
                              None, 0, stream)
        if st:
            _lib.check(st, "dlm_step_stats")

    torch.cuda.synchronize()
    for i in range(args.warmup):
        stats_call(i)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        stats_call(i)
    t1.record()
    torch.cuda.synchronize()
    call_us = t0.elapsed_time(t1) * 1000.0 / args.steps
    res["llada"]["stats_call_back_to_back_us"] = round(call_us, 3)
    print(f"[bench] llada: {res['llada']}", file=sys.stderr, flush=True)

    # every rule on the same rows, with DAPD over [1, 320, 768, 768] attention
    pos, offs = synth.gen_positions("llada", dev, batch=1)
    attns = [synth.attention("llada", dev, batch=1) for _ in range(args.replicas)]
    ws = torch.empty(api.dapd_workspace_bytes(1, n), device=dev, dtype=torch.uint8)
    cap = dict(eligible=block, tau_low=R["tau_low"], tau_high=R["tau_high"], gamma=R["gamma"],
               k_max=R["k_max"])
    avg_bytes = spec.n_lh * n * n * 2 + n * n * 4
    # the attention replica follows the logits replica
    reps_a = [dict(r, dapd=dict(attn=a, masked_pos=pos, m_max=n, tau=R["dapd_tau"],
                                workspace=ws)) for r, a in zip(reps, attns)]
    allr = Step("llada_all_rules", n, reps_a, stream, stats_bytes + avg_bytes, fast=fast,
                depcap=depcap, cap=cap)
    ms2, us2 = time_step(allr, args.steps, args.warmup)
    res["llada_all_rules"] = result(allr, ms2, us2, "k_step_stream (statistics rows + DAPD "
                                                    "attention tiles)",
                                    {"workload": "the llada step + CAP on block 0 (K 32) + DAPD "
                                                 "over 256 rows, [1, 320, 768, 768] bf16 "
                                                 "attention, tau 0.01"})
    print(f"[bench] llada_all_rules: {res['llada_all_rules']}", file=sys.stderr, flush=True)
    del attns, allr, ws
    return head, (cur, prev, so, ri, block, R)


def dapd_workloads(dev, stream, args, res, cpu):
    import torch
    from diffusion_lm_unmask_amd import api, synth
    spec = synth.SPECS["dapd"]
    cur, _, so, ri = synth.logits("dapd", dev)
    n = spec.n_rows
    pos, offs = synth.gen_positions("dapd", dev)
    attn = synth.attention("dapd", dev)
    ws = torch.empty(api.dapd_workspace_bytes(spec.batch, spec.rows), device=dev,
                     dtype=torch.uint8)
    stats_bytes = n * spec.vocab * 2
    avg_bytes = spec.batch * (spec.n_lh * spec.rows * spec.rows * 2 + spec.rows * spec.rows * 4)
    base = dict(logits=cur, prev=None, seq_offsets=so, row_index=None)
    st = Step("dapd_stats", n, [base], stream, stats_bytes)
    ms0, us0 = time_step(st, args.steps, args.warmup)
    stats_only = result(st, ms0, us0, "k_step_rows (the statistics kernel)")
    dp = dict(attn=attn, masked_pos=pos, m_max=spec.rows, tau=synth.RULES["dapd"]["dapd_tau"],
              workspace=ws)
    step = Step("dapd", n, [base], stream, stats_bytes + avg_bytes, dapd=dp)
    ms, us = time_step(step, args.steps, args.warmup)
    res["dapd"] = result(step, ms, us, "k_step_stream (statistics rows + DAPD attention tiles)",
                         {"workload": "8 x 256 rows, V=126464 bf16 (no prev) + DAPD over "
                                      "[8, 320, 768, 768] bf16 attention, 256 masked positions "
                                      "each, tau 0.01 (no edge: the graph is empty)",
                          "statistics_only": stats_only})
    print(f"[bench] dapd: {res['dapd']}", file=sys.stderr, flush=True)
    if cpu is not None:
        cpu["dapd"] = (step, cur, attn, pos, offs, so)
    # the same step on the edge-rich attention (partner covariance): the greedy runs
    attn_cov = synth.attention("dapd", dev, variant="cov", masked_pos=pos[:spec.rows])
    dpc = dict(dp, attn=attn_cov)
    stepc = Step("dapd_cov", n, [base], stream, stats_bytes + avg_bytes, dapd=dpc)
    msc, usc = time_step(stepc, args.steps, args.warmup)
    o = stepc.out()
    torch.cuda.synchronize()
    n_commit = o["dapd"][1].cpu().tolist()
    res["dapd_cov"] = result(stepc, msc, usc, "k_step_stream (statistics rows + DAPD attention "
                                              "tiles)",
                             {"workload": "the dapd step on the partner-covariance attention "
                                          "(3 masked partners per position, +4 logits): an "
                                          "edge-rich graph, so the Welsh-Powell greedy runs",
                              "dapd_committed_per_sequence": n_commit})
    print(f"[bench] dapd_cov: {res['dapd_cov']}", file=sys.stderr, flush=True)
    del attn_cov, stepc
    if cpu is None:
        del attn
    torch.cuda.empty_cache()


def stress_workload(dev, stream, args, res, cpu):
    import torch
    from diffusion_lm_unmask_amd import synth
    spec = synth.SPECS["stress"]
    R = synth.RULES["stress"]
    cur, prev, so, ri = synth.logits("stress", dev)
    n = spec.n_rows
    step = Step("stress", n, [dict(logits=cur, prev=prev, seq_offsets=so, row_index=None)], stream,
                n * spec.vocab * 2 * 2,
                depcap=dict(lam=R["lam"], l_min=R["l_min"], l_max=R["l_max"]),
                cap=dict(tau_low=R["tau_low"], tau_high=R["tau_high"], gamma=R["gamma"],
                         k_max=R["k_max"]))
    steps = max(3, min(args.steps, 10))
    ms, us = time_step(step, steps, min(args.warmup, 2))
    res["stress"] = result(step, ms, us, "k_step_rows (the statistics kernel)",
                           {"workload": "64 x 1024 rows, V=126464 bf16 cur+prev (33.15 GB) + "
                                        "DepCap (defaults) + CAP (0.8 / 0.95 / -16, K 128) over "
                                        "every row",
                            "steps": steps})
    print(f"[bench] stress: {res['stress']}", file=sys.stderr, flush=True)
    if cpu is not None:
        # the oracle's sample: every 8th sequence (8 of 64), copied to the host
        sample = list(range(0, spec.batch, 8))
        o = step.out()
        torch.cuda.synchronize()
        rows = [slice(b * spec.rows, (b + 1) * spec.rows) for b in sample]
        cpu["stress"] = dict(
            sample=sample,
            cur=torch.cat([cur[r].cpu() for r in rows]), prev=torch.cat([prev[r].cpu() for r in rows]),
            gpu={k: (None if o[k] is None else torch.cat([o[k][r].cpu() for r in rows]))
                 for k in ("conf", "entropy", "kl", "lse", "argmax")},
            depcap=o["depcap"][0][sample].cpu(),
            cap=torch.cat([o["cap"][0][r].cpu() for r in rows]), R=R, rows=spec.rows)
    del cur, prev, step
    torch.cuda.empty_cache()


def dream_workload(dev, stream, args, res):
    import torch
    from diffusion_lm_unmask_amd import synth
    spec = synth.SPECS["dream"]
    R = synth.RULES["dream"]
    cur, _, so, ri = synth.logits("dream", dev)
    n = spec.n_rows
    step = Step("dream", n, [dict(logits=cur, prev=None, seq_offsets=so, row_index=None)], stream,
                n * spec.vocab * 2,
                cap=dict(tau_low=R["tau_low"], tau_high=R["tau_high"], gamma=R["gamma"],
                         k_max=R["k_max"]))
    ms, us = time_step(step, args.steps, args.warmup)
    res["dream"] = result(step, ms, us, "k_step_rows (the statistics kernel)",
                          {"workload": "16 x 256 rows, V=151936 bf16 (no prev) + CAP (0.7 / 0.95 "
                                       "/ -16, K 64) over every row"})
    print(f"[bench] dream: {res['dream']}", file=sys.stderr, flush=True)
    del cur, step
    torch.cuda.empty_cache()


def tiny_workload(dev, stream, args, res):
    from diffusion_lm_unmask_amd import synth
    R = synth.RULES["tiny"]
    cur, prev, so, ri = synth.logits("tiny", dev)
    n = cur.shape[0]
    block = block_mask(n, 0, n, dev)
    attn = synth.attention("tiny", dev)
    pos, offs = synth.gen_positions("tiny", dev)
    step = Step("tiny", n, [dict(logits=cur, prev=prev, seq_offsets=so, row_index=None)], stream,
                cur.numel() * 4 * 2 + 32 * 32 * 4 + 32 * 32 * 4,
                fast=dict(eligible=block, tau=R["tau"]),
                depcap=dict(lam=R["lam"], l_min=R["l_min"], l_max=R["l_max"]),
                cap=dict(eligible=block, tau_low=R["tau_low"], tau_high=R["tau_high"],
                         gamma=R["gamma"], k_max=R["k_max"]),
                dapd=dict(attn=attn, masked_pos=pos, m_max=32, tau=R["dapd_tau"]))
    ms, us = time_step(step, args.steps, args.warmup)
    r = result(step, ms, us, "k_step_stream")
    r["workload"] = "1 x 32 rows, V=4096 fp32 cur+prev, every rule (latency-bound)"
    r["us_per_step"] = round(ms * 1000.0, 2)
    res["tiny"] = r
    print(f"[bench] tiny: {r}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- oracle leg

def _stats_err(g, o, keys):
    import numpy as np
    w = 0.0
    for k in keys:
        a = g[k].double().numpy() if hasattr(g[k], "double") else np.asarray(g[k], np.float64)
        b = np.asarray(o[k], np.float64)
        m = np.isfinite(b)
        if m.any():
            w = max(w, float(np.max(np.abs(a[m] - b[m]))))
    return w


def cpu_leg(head, head_inputs, cpu, seconds):
    """The oracle (as it stands) on host copies of the exact inputs: timed on
    the LLaDA step (all threads and one thread), on the DAPD step and on an
    8-of-64-sequence sample of the stress step; its decisions are compared
    with the GPU's."""
    import numpy as np
    import torch

    import oracle
    threads = oracle.default_threads()
    cur, prev, so, ri, block, R = head_inputs
    cur_h, prev_h = cur.cpu(), prev.cpu()
    so_h, block_h = so.cpu().numpy(), block.cpu().numpy()
    parity = {}
    baselines = {}

    def llada_once(nt):
        st = oracle.step_stats(cur_h, prev_h, n_threads=nt)
        c, _ = oracle.fastdllm_select(st["conf"], so_h, f32(R["tau"]), block_h)
        L, _ = oracle.depcap_boundary(st["kl"], st["entropy"], so_h, R["l_max"], R["l_min"],
                                      R["lam"])
        return st, c, L

    reps, el = _timed_reps(lambda: llada_once(threads), seconds)
    main = {"value": round(head.rows * reps / el, 1), "unit": "decisions/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the full llada step (statistics of 256 rows, Fast-dLLM, DepCap) repeated "
                      f"{reps} times in {el:.1f} s on {threads} threads; host CPU: {cpu_model()}"}
    reps1, el1 = _timed_reps(lambda: llada_once(1), min(seconds, 4.0))
    baselines["llada_1_thread"] = {"value": round(head.rows * reps1 / el1, 1),
                                   "unit": "decisions/s", "cores": 1,
                                   "sample": f"the same step, {reps1} repetitions in {el1:.1f} s"}
    # decisions against the GPU's (replica 0)
    head.run(0)
    torch.cuda.synchronize()
    g = head.out(0)
    st, c_o, L_o = llada_once(threads)
    gh = {k: g[k].cpu() for k in ("conf", "entropy", "kl", "lse", "argmax")}
    same = (np.array_equal(g["fast"][0].cpu().numpy(), c_o) and
            int(g["depcap"][0].cpu()[0]) == int(L_o[0]))
    parity["llada"] = {"sequences": 1, "identical": int(same), "flagged": int(not same),
                       "argmax_equal": bool(np.array_equal(gh["argmax"].numpy(), st["argmax"])),
                       "stats_max_abs_err": _stats_err(gh, st, ("conf", "entropy", "kl"))}

    if "dapd" in cpu:
        step, dcur, attn, pos, offs, dso = cpu["dapd"]
        step.run(0)
        torch.cuda.synchronize()
        g = step.out(0)
        dcur_h, attn_h = dcur.cpu(), attn.cpu()
        pos_h, offs_h = pos.cpu().numpy(), offs.cpu().numpy()
        t0 = time.perf_counter()
        st = oracle.step_stats(dcur_h, None, n_threads=threads)
        d_o = oracle.dapd_select(attn_h, pos_h, offs_h, st["conf"], f32(0.01), m_max=256,
                                 n_threads=threads)
        el = time.perf_counter() - t0
        baselines["dapd"] = {"value": round(step.rows / el, 1), "unit": "decisions/s",
                             "cores": threads,
                             "sample": f"the full dapd step (statistics of 2048 rows, DAPD over "
                                       f"8 sequences) once in {el:.2f} s"}
        gc = g["dapd"][0].cpu().numpy()
        ident = sum(int(np.array_equal(gc[offs_h[b]:offs_h[b + 1]],
                                       d_o["commit"][offs_h[b]:offs_h[b + 1]]))
                    for b in range(len(offs_h) - 1))
        gh = {k: g[k].cpu() for k in ("conf", "entropy", "argmax")}
        parity["dapd"] = {"sequences": len(offs_h) - 1, "identical": ident,
                          "flagged": len(offs_h) - 1 - ident,
                          "argmax_equal": bool(np.array_equal(gh["argmax"].numpy(),
                                                              st["argmax"])),
                          "stats_max_abs_err": _stats_err(gh, st, ("conf", "entropy"))}
        del attn_h, dcur_h

    if "stress" in cpu:
        s = cpu["stress"]
        Rs, M, B = s["R"], s["rows"], len(s["sample"])
        so_s = np.arange(0, (B + 1) * M, M, dtype=np.int32)
        ri_s = np.arange(B * M, dtype=np.int64)
        t0 = time.perf_counter()
        st = oracle.step_stats(s["cur"], s["prev"], n_threads=threads)
        L_o, _ = oracle.depcap_boundary(st["kl"], st["entropy"], so_s, Rs["l_max"], Rs["l_min"],
                                        Rs["lam"])
        c_o = oracle.cap_select(s["cur"], ri_s, so_s, st["conf"], st["argmax"], st["lse"],
                                f32(Rs["tau_low"]), f32(Rs["tau_high"]), f32(Rs["gamma"]),
                                Rs["k_max"], n_threads=threads)
        el = time.perf_counter() - t0
        baselines["stress_sample"] = {
            "value": round(B * M / el, 1), "unit": "decisions/s", "cores": threads,
            "sample": f"sequences {s['sample']} of 64 ({B * M} rows, statistics + DepCap + CAP) "
                      f"in {el:.2f} s",
            "extrapolated_full_step_s": round(el * 64 / B, 2),
            "extrapolation": f"x{64 // B}, labelled: the full 64-sequence step was not run"}
        gd = s["depcap"].numpy()
        gcap = s["cap"].numpy()
        ident = 0
        for b in range(B):
            r = slice(b * M, (b + 1) * M)
            ident += int(int(gd[b]) == int(L_o[b]) and
                         np.array_equal(gcap[r], c_o["commit"][r]))
        parity["stress_sample"] = {"sequences": B, "identical": ident, "flagged": B - ident,
                                   "argmax_equal": bool(np.array_equal(
                                       s["gpu"]["argmax"].numpy(), st["argmax"])),
                                   "stats_max_abs_err": _stats_err(s["gpu"], st,
                                                                   ("conf", "entropy", "kl"))}
    return main, baselines, parity


# ------------------------------------------------------------ per-call mode

def per_call(dev: str, iters: int) -> dict:
    """Time every entry point on the workloads it is defined on.  Each
    measurement captures `iters` calls (rotating input replicas where the
    inputs would fit in the 256 MB Infinity Cache) in a HIP graph and times
    replays with HIP events, so small kernels are timed on the GPU rather than
    through host launch latency.  HBM-bound calls also report GB/s."""
    import torch
    from diffusion_lm_unmask_amd import api, synth

    res = {}
    stream = torch.cuda.Stream(device=dev)

    def timed(name, fn, n_rep=1, nbytes=None, note=None):
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for i in range(2):
                fn(i % n_rep)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(iters):
                fn(i % n_rep)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        with torch.cuda.stream(stream):
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / (reps * iters)
        entry = {"us": round(us, 2)}
        if nbytes:
            entry["GB/s"] = round(nbytes / us / 1e3, 1)
            entry["frac_of_peak"] = round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)
        if note:
            entry["workload"] = note
        res[name] = entry
        print(f"[calls] {name}: {entry}", file=sys.stderr, flush=True)
        del g

    def stats_of(name, replicas):
        spec = synth.SPECS[name]
        cur, prev, so, ri = synth.logits(name, dev)
        curs = replicas_of(cur, replicas)
        prevs = None if prev is None else replicas_of(prev, replicas)
        nb = cur.numel() * cur.element_size() * (1 if prev is None else 2)
        timed(f"step_stats/{name}",
              lambda r: api.step_stats(curs[r], None if prevs is None else prevs[r]),
              replicas, nb, f"{cur.shape[0]} rows x V={spec.vocab} "
                            f"{'cur+prev' if prev is not None else 'cur'} {cur.dtype}")
        st = api.step_stats(cur, prev)
        return spec, cur, prev, so, ri, st, curs

    def schedules(tag, st, so, el, pos, offs):
        conf = st["conf"]
        gs = pos[offs[:-1].long()].contiguous()  # each sequence's first masked position
        timed(f"fastdllm_select/{tag}", lambda r: api.fastdllm_select(conf, so, 0.9, eligible=el))
        timed(f"topk_select/{tag}", lambda r: api.topk_select(conf, so, 2, eligible=el))
        timed(f"factor_select/{tag}", lambda r: api.factor_select(conf, so, 1.0, eligible=el))
        timed(f"fixed_block_eligible/{tag}",
              lambda r: api.fixed_block_eligible(pos, offs, 32, gen_start=gs))

    with torch.cuda.stream(stream):
        spec, cur, prev, so, ri, st, _ = stats_of("tiny", 4)
        del cur, prev, st
        spec, cur, prev, so, ri, st, curs = stats_of("llada", 4)
        R = synth.RULES["llada"]
        block = block_mask(cur.shape[0], *R["fast_block"], dev)
        pos, offs = synth.gen_positions("llada", dev)
        schedules("llada", st, so, block, pos, offs)
        timed("depcap_boundary/llada", lambda r: api.depcap_boundary(st["kl"], st["entropy"], so))
        timed("cap_select/llada", lambda r: api.cap_select(
            curs[r], None, so, st["conf"], st["argmax"], st["lse"], eligible=block,
            k_max=R["k_max"]), 4)
        attn = [synth.attention("llada", dev, batch=1) for _ in range(4)]
        ws = torch.empty(api.dapd_workspace_bytes(1, 256), device=dev, dtype=torch.uint8)
        nb = 320 * 256 * 256 * 2 + 256 * 256 * 4
        timed("dapd_select/llada", lambda r: api.dapd_select(attn[r], pos, offs, st["conf"], 0.01,
                                                             m_max=256, workspace=ws), 4, nb,
              "1 x [320, 768, 768] bf16 maps, 256 masked")
        timed("dapd_select_static/llada", lambda r: api.dapd_select_static(
            attn[r], pos, offs, st["conf"], 0.01, m_max=256), 4, nb,
              "the same with the library's static workspace")
        del cur, prev, curs, attn, st
        torch.cuda.empty_cache()
        spec, cur, prev, so, ri, st, _ = stats_of("dream", 1)
        Rd = synth.RULES["dream"]
        timed("cap_select/dream", lambda r: api.cap_select(
            cur, None, so, st["conf"], st["argmax"], st["lse"], tau_low=Rd["tau_low"],
            k_max=Rd["k_max"]))
        del cur, st
        torch.cuda.empty_cache()
        spec, cur, prev, so, ri, st, _ = stats_of("dapd", 2)
        pos, offs = synth.gen_positions("dapd", dev)
        attn = synth.attention("dapd", dev, variant="cov", masked_pos=pos[:spec.rows])
        ws = torch.empty(api.dapd_workspace_bytes(spec.batch, 256), device=dev,
                         dtype=torch.uint8)
        nb = spec.batch * (320 * 256 * 256 * 2 + 256 * 256 * 4)
        timed("dapd_select/dapd", lambda r: api.dapd_select(attn, pos, offs, st["conf"], 0.01,
                                                            m_max=256, workspace=ws), 1, nb,
              "8 x [320, 768, 768] bf16 maps, 256 masked each, partner-covariance variant")
        gen_len = torch.tensor([256, 384, 512, 600, 256, 700, 1000, 400], device=dev,
                               dtype=torch.int32)
        timed("dapd_step/dapd", lambda r: api.dapd_step(attn, pos, offs, st["conf"], 0.01,
                                                        gen_len=gen_len, m_max=256, workspace=ws),
              1, None, "same, 3 of 8 sequences in the late stage")
        del cur, attn, st
        torch.cuda.empty_cache()
        spec, cur, prev, so, ri, st, _ = stats_of("stress", 1)
        pos = (torch.arange(1024, device=dev, dtype=torch.int32) + 512).repeat(spec.batch)
        schedules("stress", st, so, None, pos, so)
        timed("depcap_boundary/stress", lambda r: api.depcap_boundary(st["kl"], st["entropy"],
                                                                      so))
        timed("cap_select/stress", lambda r: api.cap_select(cur, None, so, st["conf"],
                                                            st["argmax"], st["lse"], k_max=128))
        del cur, prev, st
        torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma-separated sub-workloads to run besides the headline "
                         "(llada_all_rules is always run): dapd,stress,dream,tiny; default all")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device-to-device copies of MIB MiB (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    ap.add_argument("--calls", action="store_true",
                    help="only time every entry point on its workloads and print one JSON line")
    ap.add_argument("--call-iters", type=int, default=20)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decision path shards by sequence with no "
              "exchange between GPUs, so one GPU's figure is the per-GPU rate (use --gpus 1).",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (no HIP device visible)", file=sys.stderr)
        return 2
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.randint(0, 255, (n,), device=dev, dtype=torch.uint8)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "copies": 10}), flush=True)
        return 0
    if args.calls:
        print(json.dumps({"calls": per_call(dev, args.call_iters), "n_gpus": 1,
                          "data": "synthetic"}), flush=True)
        return 0

    only = set(w for w in args.only.split(",") if w) or {"dapd", "stress", "dream", "tiny"}
    # every launch goes to this stream (default priority)
    ts = torch.cuda.Stream(device=dev)
    stream = ts.cuda_stream
    cpu = None if args.no_cpu_baseline else {}
    res = {}
    with torch.cuda.stream(ts):
        head, head_inputs = llada_workloads(dev, stream, args, res)
        if "tiny" in only:
            tiny_workload(dev, stream, args, res)
        if "dapd" in only:
            dapd_workloads(dev, stream, args, res, cpu)
        if "dream" in only:
            dream_workload(dev, stream, args, res)
        if "stress" in only:
            stress_workload(dev, stream, args, res, cpu)
    torch.cuda.synchronize()

    h = res["llada"]
    l1 = h["launch1"]
    stats_kernel = {w: {"kernel": "k_step_rows", "avg_us": r["launch1"]["avg_us"],
                        "algorithmic_bytes": r["launch1"]["algorithmic_bytes"],
                        "frac_of_peak": r["launch1"]["frac_of_peak"]}
                    for w, r in (("llada", h), ("stress", res.get("stress")),
                                 ("dream", res.get("dream"))) if r}
    if "dapd" in res:
        stats_kernel["dapd"] = {k: v for k, v in res["dapd"]["statistics_only"]["launch1"].items()
                                if k != "GB/s"}
        stats_kernel["dapd"]["kernel"] = "k_step_rows"
    v126 = [stats_kernel[w]["frac_of_peak"] for w in ("llada", "dapd", "stress")
            if w in stats_kernel]
    line = {
        "metric": METRIC,
        "value": h["decisions_per_s"],
        "unit": "decisions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llada-step: 1 seq x 256 masked rows, V=126464 bf16 cur+prev logits; "
                        "statistics + Fast-dLLM threshold 0.9 on block 0 + DepCap boundary "
                        "(lambda 1.2, L_min 8, L_max 128), one dlm_decide_step per step",
            "rows": 256, "vocab": 126464, "replicas": args.replicas,
        },
        "roofline": {
            "bound": "hbm", "kernel": "k_step_rows (dlm_decide_step launch 1: the statistics "
                                      "kernel of dlm_step_stats)",
            "achieved": l1["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": l1["frac_of_peak"],
            "traffic": measured_traffic("llada/k_step_rows", "k_step_rows"),
            "traffic_unit": "bytes/launch",
            "algorithmic_bytes_per_launch": l1["algorithmic_bytes"],
            "avg_launch_us": l1["avg_us"],
        },
        "stats_kernel": dict(stats_kernel, target_frac=0.70,
                             min_frac_over_v126464=min(v126) if v126 else None),
        "workloads": res,
    }
    if cpu is not None:
        main_b, baselines, parity = cpu_leg(head, head_inputs, cpu, args.cpu_seconds)
        line["cpu_baseline"] = main_b
        line["cpu_baselines"] = baselines
        line["oracle_parity"] = parity
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
