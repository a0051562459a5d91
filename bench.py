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

Inputs are resident in HBM before timing starts; `--replicas` independent
copies are rotated so that consecutive steps do not hit the 256 MB Infinity
Cache.  Prints one JSON line (rank 0, N = 1): decisions/s, ms/step, the stats
kernel's achieved HBM bandwidth against the 8 TB/s peak (HIP events on the
launch stream, averaged over the timed steps), and the CPU oracle's rate on
the same step.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "stats_llada_traffic.json")
STATS_SOURCES = [os.path.join(ROOT, "diffusion_lm_unmask_amd", "csrc", f)
                 for f in ("stats.hip", "dlm_device.h")]


def stats_source_hash() -> str:
    h = hashlib.sha256()
    for p in STATS_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(nbytes_alg: int):
    """HBM bytes per stats launch from the committed rocprofv3 counter runs,
    only while the kernel source is unchanged since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != stats_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def torch_int_view(t):
    import torch
    return {torch.float32: torch.int32}.get(t.dtype, t.dtype)


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
        self.score = torch.empty(n, **f32)
        self.sws_bytes = int(self.L.dlm_step_stats_workspace_bytes(n))
        self.sws = torch.zeros(self.sws_bytes, **u8)     # zero-filled once; kept zero by the library
        self.ws_bytes = int(self.L.dlm_dapd_workspace_bytes(1, n))
        self.ws = torch.empty(self.ws_bytes, **u8)
        # every call goes to this stream (default priority), eager or captured
        self.torch_stream = torch.cuda.Stream(device=dev)
        self.stream = self.torch_stream.cuda_stream
        self.n_lh, self.S = attn.shape[1], attn.shape[2]
        self.bytes_stats = n * self.V * 2 * 2          # cur + prev rows, bf16

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

    def step(self, r, ev=None):
        if ev is not None:
            ev[0].record()
        self.stats(r)
        if ev is not None:
            ev[1].record()
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
    del cur, prev, curs, attn, st
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
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown-iters", type=int, default=200)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device-to-device copies of MIB MiB (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph",
                    help="graph: the step is captured once per input replica and replayed")
    ap.add_argument("--calls", action="store_true",
                    help="only time every entry point on its workloads and print one JSON line")
    ap.add_argument("--call-iters", type=int, default=20)
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decision path shards by sequence with no "
              "exchange, and this build runs on a single MI355X (use --gpus 1).", file=sys.stderr)
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

    def timed_eager(n_steps, with_stats_events):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_steps)] if with_stats_events else None
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(sm):
            t0.record()
            for i in range(n_steps):
                step.step(i % R, ev[i] if ev else None)
            t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / n_steps
        st_us = (sum(a.elapsed_time(b) for a, b in ev) / n_steps * 1000.0) if ev else None
        return ms, st_us

    with torch.cuda.stream(sm):
        for i in range(args.warmup):
            step.step(i % R)
    torch.cuda.synchronize()

    graph_ok = None
    if args.mode == "graph":
        # one captured step per input replica; replays run the seven kernels
        # back to back without host launch overhead
        graphs = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=sm):
                step.step(r)
            graphs.append(g)
        torch.cuda.synchronize()
        # replay correctness: each replica's replay equals its eager step
        graph_ok = True
        for r in range(R):
            with torch.cuda.stream(sm):
                step.step(r)
            torch.cuda.synchronize()
            want = step.outputs()
            graphs[r].replay()
            torch.cuda.synchronize()
            got = step.outputs()
            graph_ok = graph_ok and all(torch.equal(a, b) for a, b in zip(want, got))
        for i in range(args.warmup):
            graphs[i % R].replay()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(sm):
            t0.record()
            for i in range(args.steps):
                graphs[i % R].replay()
            t1.record()
        torch.cuda.synchronize()
        ms_per_step = t0.elapsed_time(t1) / args.steps
        # the stats kernel's live duration: HIP events on its launch stream over
        # an eager run of the same steps (events cannot sit inside the graphs)
        eager_ms, stats_us = timed_eager(args.steps, True)
    else:
        ms_per_step, stats_us = timed_eager(args.steps, True)
        eager_ms = ms_per_step

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

    achieved = step.bytes_stats / (stats_us * 1e-6) / 1e9
    traffic = measured_traffic(step.bytes_stats)
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
        "eager_ms_per_step": round(eager_ms, 5),
        "graph_replay_matches_eager": graph_ok,
        "roofline": {
            "bound": "hbm", "kernel": "dlm_step_stats (k_stats)",
            "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic, "traffic_unit": "bytes/launch",
            "algorithmic_bytes_per_launch": step.bytes_stats,
            "avg_launch_us": round(stats_us, 3),
        },
        "breakdown_us": breakdown,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(step, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
