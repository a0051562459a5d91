#!/usr/bin/env python3
"""Benchmark of one per-denoising-step unmask decision on one MI355X.

A step is one pass of the whole decision path over one batch of synthetic
input, the LLaDA-shaped step (one sequence, 256 masked generation rows,
vocabulary 126464, bf16 current and previous-step logits):

  dlm_step_stats       confidence / argmax / entropy / KL / lse for 256 rows
  dlm_fastdllm_select  threshold 0.9 on the active 32-token block (rows 0-31)
  dlm_depcap_boundary  DepGA-Block scan over the 128-row window (lambda 1.2,
                       L_min 8, L_max 128)
  dlm_cap_select       CAP-Decoding on the same 32-token block (0.8 / 0.95 / -16)
  dlm_dapd_select      DAPD graph over the 256 rows from [1, 320, 768, 768] bf16
                       attention (prompt 512 + generation 256), tau 0.01

By default (`--mode fused`) the step is the one call dlm_decide_step, which
runs the same decisions in two launches (statistics rows and attention
averaging in one streaming kernel, then the four rules, with the DAPD
selection in the last of its scores workgroups), issued back to back on one
stream; the host stays ahead of the
GPU, so the launches queue without gaps (a graph per step measured slower:
each graph launch adds a few microseconds).  Its decisions equal the five
calls' (checked on every run and reported).

Inputs are resident in HBM before timing starts; `--replicas` independent
copies are rotated so that consecutive steps do not hit the 256 MB Infinity
Cache.  Prints one JSON line (rank 0, N = 1): decisions/s, ms/step, the
dominant kernel's achieved HBM bandwidth against the 8 TB/s peak (HIP events
on its launch stream, averaged over the timed steps), and the CPU oracle's
rate on the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "llada_step_traffic.json")
# the device sources each timed kernel is built from: a counter reading is
# only reported while they are unchanged since it was taken
KERNEL_SOURCES = {
    "k_step_stream": ("fused.hip", "stats_impl.h", "dapd_impl.h", "dlm_device.h"),
    "k_stats": ("stats.hip", "stats_impl.h", "dlm_device.h"),
}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "diffusion_lm_unmask_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    runs (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(kernel, {})
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


class TimingEvents:
    """Pairs of HIP timing events created without the system-scope fence
    (hipEventDisableSystemFence), so that recording one adds no cache
    write-back to the interval it brackets.  The fused step hands them to its
    streaming launch, which sets them to the kernel's start and end; the
    five-call step records them on the launch stream around the statistics
    call.  They come from the HIP runtime already loaded into the process
    (torch's), so they are valid on torch's streams."""

    NO_SYSTEM_FENCE = 0x20000000

    def __init__(self, n: int):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.ct = ctypes
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

    def record(self, ev, stream):
        if self.hip.hipEventRecord(self.ct.c_void_p(ev), self.ct.c_void_p(stream)):
            raise RuntimeError("hipEventRecord failed")

    def mean_us(self):
        """Average interval in microseconds (call after the device is synchronized)."""
        ms, acc = self.ct.c_float(), 0.0
        for a, b in self.pairs:
            if self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ct.c_void_p(a),
                                            self.ct.c_void_p(b)):
                raise RuntimeError("hipEventElapsedTime failed")
            acc += ms.value
        return acc / len(self.pairs) * 1000.0

    def close(self):
        for pair in self.pairs:
            for e in pair:
                self.hip.hipEventDestroy(self.ct.c_void_p(e))
        self.pairs = []


def torch_int_view(t):
    import torch
    return {torch.float32: torch.int32, torch.float64: torch.int64}.get(t.dtype, t.dtype)


class LladaStep:
    """Preallocated buffers and ctypes argument lists for the LLaDA-shaped step."""

    def __init__(self, replicas: int, dev: str):
        import torch
        from diffusion_lm_unmask_amd import _lib, synth

        self.torch = torch
        self.L = _lib.lib()
        self.check = _lib.check
        spec = synth.SPECS["llada"]
        self.R = synth.RULES["llada"]
        self.rows, self.V = spec.rows, spec.vocab
        cur, prev, so, ri = synth.logits("llada", dev)
        attn = synth.attention("llada", dev, batch=1)
        pos, offs = synth.gen_positions("llada", dev, batch=1)
        self.cur = [cur] + [cur.clone() for _ in range(replicas - 1)]
        self.prev = [prev] + [prev.clone() for _ in range(replicas - 1)]
        self.attn = [attn] + [attn.clone() for _ in range(replicas - 1)]
        self.so, self.ri, self.pos, self.offs = so, ri, pos, offs
        n = self.rows
        f32 = dict(device=dev, dtype=torch.float32)
        self.conf, self.ent, self.kl, self.lse = (torch.empty(n, **f32) for _ in range(4))
        self.arg = torch.empty(n, device=dev, dtype=torch.int32)
        self.block = torch.zeros(n, device=dev, dtype=torch.uint8)
        b0, b1 = self.R["fast_block"]
        self.block[b0:b1] = 1
        u8 = dict(device=dev, dtype=torch.uint8)
        i32 = dict(device=dev, dtype=torch.int32)
        self.commit_f, self.commit_c, self.commit_d = (torch.empty(n, **u8) for _ in range(3))
        self.nf, self.nc, self.nd, self.blen = (torch.empty(1, **i32) for _ in range(4))
        self.score = torch.empty(n, device=dev, dtype=torch.float64)
        self.sws_bytes = int(self.L.dlm_step_stats_workspace_bytes(n))
        self.sws = torch.zeros(self.sws_bytes, **u8)     # zero-filled once; kept zero by the library
        self.ws_bytes = int(self.L.dlm_dapd_workspace_bytes(1, n))
        self.ws = torch.empty(self.ws_bytes, **u8)
        # every call goes to this stream (default priority), eager or captured
        self.torch_stream = torch.cuda.Stream(device=dev)
        self.stream = self.torch_stream.cuda_stream
        self.n_lh, self.S = attn.shape[1], attn.shape[2]
        self.bytes_stats = n * self.V * 2 * 2          # cur + prev rows, bf16
        # the DAPD average reads the masked rows x masked columns of every
        # attention map (bf16) and writes the fp32 average a
        self.bytes_avg = self.n_lh * n * n * 2 + n * n * 4
        self.desc = [self._desc(r) for r in range(replicas)]

    def _desc(self, r):
        """dlm_decide_step descriptor of the same step on input replica r."""
        from diffusion_lm_unmask_amd import _lib
        R, d = self.R, _lib.StepDesc()
        d.logits, d.prev_logits, d.dtype = self.cur[r].data_ptr(), self.prev[r].data_ptr(), 0
        d.vocab, d.ld, d.row_index, d.n_rows = self.V, self.V, self.ri.data_ptr(), self.rows
        d.conf, d.argmax, d.entropy = self.conf.data_ptr(), self.arg.data_ptr(), self.ent.data_ptr()
        d.kl, d.lse, d.seq_offsets, d.n_seq = self.kl.data_ptr(), self.lse.data_ptr(), \
            self.so.data_ptr(), 1
        d.fast_eligible, d.fast_tau = self.block.data_ptr(), R["tau"]
        d.fast_commit, d.fast_n_commit = self.commit_f.data_ptr(), self.nf.data_ptr()
        d.depcap_lambda, d.depcap_l_min, d.depcap_l_max = R["lam"], R["l_min"], R["l_max"]
        d.depcap_radius, d.depcap_eps = 1, 1e-12
        d.depcap_block_len, d.depcap_score = self.blen.data_ptr(), self.score.data_ptr()
        d.cap_eligible, d.cap_tau_low, d.cap_tau_high = self.block.data_ptr(), R["tau_low"], \
            R["tau_high"]
        d.cap_gamma, d.cap_k_max = R["gamma"], R["k_max"]
        d.cap_commit, d.cap_n_commit = self.commit_c.data_ptr(), self.nc.data_ptr()
        d.attn, d.attn_dtype, d.n_lh, d.S = self.attn[r].data_ptr(), 0, self.n_lh, self.S
        d.batch_stride, d.masked_pos, d.m_max = self.n_lh * self.S * self.S, \
            self.pos.data_ptr(), self.rows
        d.dapd_tau, d.dapd_commit, d.dapd_n_commit = R["dapd_tau"], self.commit_d.data_ptr(), \
            self.nd.data_ptr()
        d.dapd_workspace, d.dapd_workspace_bytes = self.ws.data_ptr(), self.ws_bytes
        return d

    def fused(self, r, ev=None):
        """The same step as one dlm_decide_step call (two launches); with
        `ev` (a pair of raw HIP events), the library records them around its
        streaming launch."""
        import ctypes
        d = self.desc[r]
        d.launch1_begin_event = ev[0] if ev is not None else None
        d.launch1_end_event = ev[1] if ev is not None else None
        st = self.L.dlm_decide_step(ctypes.byref(d), self.stream)
        if st:
            self.check(st, "dlm_decide_step")

    def outputs(self):
        """Copies of every output, as raw bits (so NaN compares equal to NaN)."""
        out = []
        for t in (self.conf, self.arg, self.ent, self.kl, self.lse, self.commit_f, self.nf,
                  self.blen, self.score, self.commit_c, self.nc, self.commit_d, self.nd):
            out.append(t.view(torch_int_view(t)).clone())
        return out

    def stats(self, r):
        st = self.L.dlm_step_stats(self.cur[r].data_ptr(), self.prev[r].data_ptr(), 0, self.V,
                                   self.V, self.ri.data_ptr(), self.rows, self.conf.data_ptr(),
                                   self.arg.data_ptr(), self.ent.data_ptr(), self.kl.data_ptr(),
                                   self.lse.data_ptr(), self.sws.data_ptr(), self.sws_bytes,
                                   self.stream)
        if st:
            self.check(st, "dlm_step_stats")

    def fastdllm(self, r):
        st = self.L.dlm_fastdllm_select(self.conf.data_ptr(), self.block.data_ptr(),
                                        self.so.data_ptr(), 1, self.R["tau"],
                                        self.commit_f.data_ptr(), self.nf.data_ptr(), self.stream)
        if st:
            self.check(st, "dlm_fastdllm_select")

    def depcap(self, r):
        st = self.L.dlm_depcap_boundary(self.kl.data_ptr(), self.ent.data_ptr(), self.so.data_ptr(),
                                        1, None, self.R["lam"], self.R["l_min"], self.R["l_max"], 1,
                                        1e-12, self.blen.data_ptr(), self.score.data_ptr(),
                                        self.stream)
        if st:
            self.check(st, "dlm_depcap_boundary")

    def cap(self, r):
        R = self.R
        st = self.L.dlm_cap_select(self.cur[r].data_ptr(), 0, self.V, self.V, self.ri.data_ptr(),
                                   self.so.data_ptr(), 1, self.conf.data_ptr(), self.arg.data_ptr(),
                                   self.lse.data_ptr(), self.block.data_ptr(), R["tau_low"],
                                   R["tau_high"], R["gamma"], R["k_max"],
                                   self.commit_c.data_ptr(), self.nc.data_ptr(), None, None,
                                   self.stream)
        if st:
            self.check(st, "dlm_cap_select")

    def dapd(self, r):
        st = self.L.dlm_dapd_select(self.attn[r].data_ptr(), 0, self.n_lh, self.S,
                                    self.n_lh * self.S * self.S, self.pos.data_ptr(),
                                    self.offs.data_ptr(), 1, self.rows, self.conf.data_ptr(),
                                    self.R["dapd_tau"], self.commit_d.data_ptr(),
                                    self.nd.data_ptr(), None, None, None, self.ws.data_ptr(),
                                    self.ws_bytes, self.stream)
        if st:
            self.check(st, "dlm_dapd_select")

    def step(self, r, ev=None, events=None):
        if ev is not None:
            events.record(ev[0], self.stream)
        self.stats(r)
        if ev is not None:
            events.record(ev[1], self.stream)
        self.fastdllm(r)
        self.depcap(r)
        self.cap(r)
        self.dapd(r)


def cpu_baseline(step: LladaStep, seconds: float):
    """Time the CPU oracle (as it stands) on the same step, on host copies."""
    import numpy as np

    import oracle

    cur = step.cur[0].cpu()
    prev = step.prev[0].cpu()
    attn = step.attn[0].cpu()
    pos = step.pos.cpu().numpy()
    offs = step.offs.cpu().numpy()
    so = step.so.cpu().numpy()
    ri = step.ri.cpu().numpy()
    block = step.block.cpu().numpy()
    R = step.R
    threads = oracle.default_threads()
    f = lambda x: float(np.float32(x))  # noqa: E731  (the GPU receives f32 thresholds)

    def one():
        st = oracle.step_stats(cur, prev, n_threads=threads)
        oracle.fastdllm_select(st["conf"], so, f(R["tau"]), block)
        oracle.depcap_boundary(st["kl"], st["entropy"], so, R["l_max"], R["l_min"], R["lam"])
        oracle.cap_select(cur, ri, so, st["conf"], st["argmax"], st["lse"], f(R["tau_low"]),
                          f(R["tau_high"]), f(R["gamma"]), R["k_max"], eligible=block,
                          n_threads=threads)
        oracle.dapd_select(attn, pos, offs, st["conf"], f(R["dapd_tau"]), n_threads=threads)

    reps, t0 = 0, time.perf_counter()
    while True:
        one()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": step.rows * reps / el, "unit": "decisions/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the full step ({step.rows} rows, all five calls) repeated {reps} times "
                      f"in {el:.1f} s on {threads} threads; host CPU: {model}"}


def per_call(dev: str, iters: int) -> dict:
    """Time every entry point on the workloads it is defined on (the five
    workload shapes of the decision step).  Each measurement captures `iters`
    calls (rotating input replicas where the inputs would fit in the 256 MB
    Infinity Cache) in a HIP graph and times replays with HIP events, so small
    kernels are timed on the GPU rather than through host launch latency.
    HBM-bound calls also report GB/s against the 8 TB/s peak."""
    import torch
    from diffusion_lm_unmask_amd import api, synth

    res = {}
    stream = torch.cuda.Stream(device=dev)

    def timed(name, fn, n_rep=1, nbytes=None, note=None):
        # every input was produced on `stream` (see below); wait for it all
        # before the first use, and keep every launch on that one stream
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
        curs = [cur] + [cur.clone() for _ in range(replicas - 1)]
        prevs = None if prev is None else [prev] + [prev.clone() for _ in range(replicas - 1)]
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
        return _per_call_body(dev, timed, stats_of, schedules, res)


def _per_call_body(dev, timed, stats_of, schedules, res):
    """The workloads of per_call, run with its stream current: the inputs,
    the reference statistics the rules consume and every timed call are
    ordered on one stream."""
    import torch
    from diffusion_lm_unmask_amd import api, synth

    # tiny
    spec, cur, prev, so, ri, st, _ = stats_of("tiny", 4)
    del cur, prev, st
    # llada-shaped step inputs
    spec, cur, prev, so, ri, st, curs = stats_of("llada", 4)
    R = synth.RULES["llada"]
    block = torch.zeros(cur.shape[0], device=dev, dtype=torch.uint8)
    block[R["fast_block"][0]:R["fast_block"][1]] = 1
    pos, offs = synth.gen_positions("llada", dev)
    schedules("llada", st, so, block, pos, offs)
    timed("depcap_boundary/llada", lambda r: api.depcap_boundary(st["kl"], st["entropy"], so))
    timed("cap_select/llada", lambda r: api.cap_select(
        curs[r], ri, so, st["conf"], st["argmax"], st["lse"], eligible=block, k_max=R["k_max"]), 4)
    attn = [synth.attention("llada", dev, batch=1) for _ in range(4)]
    ws = torch.empty(api.dapd_workspace_bytes(1, 256), device=dev, dtype=torch.uint8)
    nb = 320 * 256 * 256 * 2 + 256 * 256 * 4
    timed("dapd_select/llada", lambda r: api.dapd_select(attn[r], pos, offs, st["conf"], 0.01,
                                                         m_max=256, workspace=ws), 4, nb,
          "1 x [320, 768, 768] bf16 maps, 256 masked")
    # the whole step as one call (two launches)
    prevs = [prev] + [prev.clone() for _ in range(3)]
    parts = dict(fast=dict(eligible=block, tau=R["tau"]),
                 depcap=dict(lam=R["lam"], l_min=R["l_min"], l_max=R["l_max"]),
                 cap=dict(eligible=block, tau_low=R["tau_low"], tau_high=R["tau_high"],
                          gamma=R["gamma"], k_max=R["k_max"]))
    timed("decide_step/llada", lambda r: api.decide_step(
        curs[r], prevs[r], so, row_index=ri, **parts,
        dapd=dict(attn=attn[r], masked_pos=pos, m_max=256, tau=R["dapd_tau"], workspace=ws)),
          4, cur.numel() * 2 * 2 + nb, "statistics, Fast-dLLM, DepCap, CAP and DAPD in one call")
    del cur, prev, curs, prevs, attn, st
    torch.cuda.empty_cache()
    # dream: CAP with K_max 64 over every row
    spec, cur, prev, so, ri, st, _ = stats_of("dream", 1)
    Rd = synth.RULES["dream"]
    timed("cap_select/dream", lambda r: api.cap_select(
        cur, ri, so, st["conf"], st["argmax"], st["lse"], tau_low=Rd["tau_low"],
        k_max=Rd["k_max"]))
    del cur, st
    torch.cuda.empty_cache()
    # dapd: 8 sequences, plain selection and the full step (half of them late)
    spec, cur, prev, so, ri, st, _ = stats_of("dapd", 2)
    pos, offs = synth.gen_positions("dapd", dev)
    attn = [synth.attention("dapd", dev, variant="cov", masked_pos=pos[:spec.rows])]
    ws = torch.empty(api.dapd_workspace_bytes(spec.batch, 256), device=dev, dtype=torch.uint8)
    nb = spec.batch * (320 * 256 * 256 * 2 + 256 * 256 * 4)
    timed("dapd_select/dapd", lambda r: api.dapd_select(attn[0], pos, offs, st["conf"], 0.01,
                                                        m_max=256, workspace=ws), 1, nb,
          "8 x [320, 768, 768] bf16 maps, 256 masked each, partner-covariance variant")
    gen_len = torch.tensor([256, 384, 512, 600, 256, 700, 1000, 400], device=dev,
                           dtype=torch.int32)
    timed("dapd_step/dapd", lambda r: api.dapd_step(attn[0], pos, offs, st["conf"], 0.01,
                                                    gen_len=gen_len, m_max=256, workspace=ws),
          1, None, "same, 3 of 8 sequences in the late stage")
    timed("decide_step/dapd", lambda r: api.decide_step(
        cur, None, offs, row_index=ri, fast=dict(tau=0.9), cap=dict(k_max=64),
        dapd=dict(attn=attn[0], masked_pos=pos, m_max=256, tau=0.01, workspace=ws)),
          1, cur.numel() * 2 + nb, "statistics, Fast-dLLM, CAP (every row) and DAPD, 8 sequences")
    del cur, attn, st
    torch.cuda.empty_cache()
    # stress: 64 x 1024 rows with prev (33 GB)
    spec, cur, prev, so, ri, st, _ = stats_of("stress", 1)
    pos = (torch.arange(1024, device=dev, dtype=torch.int32) + 512).repeat(spec.batch)
    schedules("stress", st, so, None, pos, so)
    timed("depcap_boundary/stress", lambda r: api.depcap_boundary(st["kl"], st["entropy"], so))
    timed("cap_select/stress", lambda r: api.cap_select(cur, ri, so, st["conf"], st["argmax"],
                                                        st["lse"], k_max=128))
    del cur, prev, st
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown-iters", type=int, default=200)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device-to-device copies of MIB MiB (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    ap.add_argument("--mode", choices=("fused", "fused-graph", "graph", "eager"),
                    default="fused",
                    help="fused: one dlm_decide_step call (two launches) per step; "
                         "fused-graph: that call captured once per input replica and "
                         "replayed; graph: the five individual calls captured and replayed; "
                         "eager: the five calls launched one by one")
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
    step = LladaStep(args.replicas, dev)
    R = args.replicas
    sm = step.torch_stream
    torch.cuda.synchronize()

    def timed_eager(n_steps, fused):
        """Eager run of n_steps steps with HIP events on the dominant launch
        of each step (set by the fused streaming launch itself, else recorded
        around the statistics call), on the launch stream."""
        events = TimingEvents(n_steps)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(sm):
            t0.record()
            for i in range(n_steps):
                if fused:
                    step.fused(i % R, events.pairs[i])
                else:
                    step.step(i % R, events.pairs[i], events)
            t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / n_steps
        us = events.mean_us()
        events.close()
        return ms, us

    fused = args.mode in ("fused", "fused-graph")
    run = step.fused if fused else step.step
    with torch.cuda.stream(sm):
        for i in range(args.warmup):
            run(i % R)
    torch.cuda.synchronize()

    # on replica 0: the fused step's decisions against the four rule calls run
    # on the fused statistics (bitwise), and its statistics against the
    # statistics call (argmax identical, floats to the last bits)
    with torch.cuda.stream(sm):
        step.fused(0)
    torch.cuda.synchronize()
    fused_out = step.outputs()
    with torch.cuda.stream(sm):
        for name in ("fastdllm", "depcap", "cap", "dapd"):
            getattr(step, name)(0)
    torch.cuda.synchronize()
    rules_out = step.outputs()
    decisions_idx = (5, 6, 7, 8, 9, 10, 11, 12)     # every commit, count, length and score
    fused_match = all(torch.equal(rules_out[i], fused_out[i]) for i in decisions_idx)
    with torch.cuda.stream(sm):
        step.stats(0)
    torch.cuda.synchronize()
    calls_out = step.outputs()
    fused_match = fused_match and torch.equal(calls_out[1], fused_out[1])
    stats_diff = max(float((calls_out[i].view(torch.float32).double() -
                            fused_out[i].view(torch.float32).double()).abs().max())
                     for i in (0, 2, 3, 4))

    def timed_plain(fn):
        """K steps back to back on the launch stream, bracketed by events."""
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(sm):
            t0.record()
            for i in range(args.steps):
                fn(i % R)
            t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    graph_ok = None
    if args.mode in ("graph", "fused-graph"):
        # one captured step per input replica; replays run its kernels back
        # to back without host launch overhead
        graphs = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=sm):
                run(r)
            graphs.append(g)
        torch.cuda.synchronize()
        # replay correctness: each replica's replay equals its eager step
        graph_ok = True
        for r in range(R):
            with torch.cuda.stream(sm):
                run(r)
            torch.cuda.synchronize()
            want = step.outputs()
            graphs[r].replay()
            torch.cuda.synchronize()
            got = step.outputs()
            graph_ok = graph_ok and all(torch.equal(a, b) for a, b in zip(want, got))
        for i in range(args.warmup):
            graphs[i % R].replay()
        ms_per_step = timed_plain(lambda r: graphs[r].replay())
    else:
        ms_per_step = timed_plain(run)
    # the dominant kernel's live duration over a second run of the same steps:
    # HIP events on its launch stream, which the fused step's launch sets to
    # the kernel's own start and end (the five-call step records them around
    # the statistics call instead)
    events_ms, dom_us = timed_eager(args.steps, fused)
    # the statistics call on its own (the five calls, eager), for reference
    calls_events_ms, stats_us = timed_eager(args.steps, False)

    # per-call breakdown (untimed region, same rotation)
    breakdown = {}
    for name in ("stats", "fastdllm", "depcap", "cap", "dapd"):
        fn = getattr(step, name)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(sm):
            for i in range(10):
                step.step(i % R)
            torch.cuda.synchronize()
            acc = 0.0
            for i in range(args.breakdown_iters):
                e0.record()
                fn(i % R)
                e1.record()
                e1.synchronize()
                acc += e0.elapsed_time(e1)
                step.step((i + 1) % R)          # keep the inputs cold in cache
        breakdown[name] = round(acc / args.breakdown_iters * 1000.0, 2)

    if fused:
        dom, dom_label = "k_step_stream", "dlm_decide_step launch 1 (k_step_stream)"
        dom_bytes = step.bytes_stats + step.bytes_avg
    else:
        dom, dom_label = "k_stats", "dlm_step_stats (k_stats)"
        dom_bytes = step.bytes_stats
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    st_achieved = step.bytes_stats / (stats_us * 1e-6) / 1e9
    decisions = step.rows
    value = decisions / (ms_per_step * 1e-3)
    line = {
        "metric": "masked-row decisions/sec and achieved HBM GB/s (% of peak), V=126464 bf16",
        "value": round(value, 1),
        "unit": "decisions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llada-step: 1 seq x 256 masked rows, V=126464 bf16 cur+prev logits; "
                        "Fast-dLLM + DepCap boundary + CAP on block 0 + DAPD over 256 rows",
            "rows": step.rows, "vocab": step.V, "attention": [1, step.n_lh, step.S, step.S],
            "replicas": args.replicas, "mode": args.mode,
        },
        "events_run_ms_per_step": round(events_ms, 5),
        "graph_replay_matches_eager": graph_ok,
        "fused_decisions_match_rule_calls": fused_match,
        "fused_stats_max_abs_diff_vs_stats_call": stats_diff,
        "calls_events_run_ms_per_step": round(calls_events_ms, 5),
        "roofline": {
            "bound": "hbm", "kernel": dom_label,
            "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(dom), "traffic_unit": "bytes/launch",
            "algorithmic_bytes_per_launch": dom_bytes,
            "avg_launch_us": round(dom_us, 3),
        },
        "stats_call_roofline": {
            "kernel": "dlm_step_stats (k_stats)", "achieved": round(st_achieved, 1),
            "frac": round(st_achieved / PEAK_HBM_GBS, 4), "avg_launch_us": round(stats_us, 3),
            "algorithmic_bytes_per_launch": step.bytes_stats,
            "traffic": measured_traffic("k_stats"),
        },
        "breakdown_us": breakdown,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(step, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
