"""The whole decision step captured as a HIP graph (marked gpu): the five
individual calls, and the fused call.

Replays are interleaved with unrelated eager work and synchronisations, and
every replay must reproduce the eager step bit for bit.  No memset node is
recorded: the statistics workspace is created and zero-filled eagerly, before
capture, and the kernels leave it zero-filled; the binding refuses to create
one under capture."""
import pytest
import torch

from diffusion_lm_unmask_amd import api, synth
from diffusion_lm_unmask_amd._lib import DLMError

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _llada(replicas):
    R = synth.RULES["llada"]
    cur, prev, so, ri = synth.logits("llada", DEV)
    n = cur.shape[0]
    block = torch.zeros(n, device=DEV, dtype=torch.uint8)
    block[R["fast_block"][0]:R["fast_block"][1]] = 1
    pos, offs = synth.gen_positions("llada", DEV, batch=1)
    ins = [(cur, prev, synth.attention("llada", DEV, batch=1))]
    for _ in range(replicas - 1):
        ins.append((cur.clone(), prev.clone(), synth.attention("llada", DEV, batch=1)))
    ws = torch.empty(api.dapd_workspace_bytes(1, n), device=DEV, dtype=torch.uint8)
    return R, ins, so, ri, block, pos, ws


def _five_calls(R, inp, so, ri, block, pos, ws):
    cur, prev, attn = inp
    st = api.step_stats(cur, prev, row_index=ri)
    f = api.fastdllm_select(st["conf"], so, R["tau"], block)
    d = api.depcap_boundary(st["kl"], st["entropy"], so, lam=R["lam"], l_min=R["l_min"],
                            l_max=R["l_max"])
    c = api.cap_select(cur, ri, so, st["conf"], st["argmax"], st["lse"], block,
                       tau_low=R["tau_low"], tau_high=R["tau_high"], gamma=R["gamma"],
                       k_max=R["k_max"])
    p = api.dapd_select(attn, pos, so, st["conf"], R["dapd_tau"], m_max=cur.shape[0],
                        workspace=ws)
    return [st["conf"], st["argmax"], st["entropy"], st["kl"], st["lse"], *f, *d,
            c["commit"], c["n_commit"], p["commit"], p["n_commit"]]


def _bits(t):
    return t.view({torch.float32: torch.int32, torch.float64: torch.int64}.get(t.dtype, t.dtype))


def test_llada_step_graph_replays_match_eager():
    R, ins, so, ri, block, pos, ws = _llada(2)
    sm = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(sm):
        _five_calls(R, ins[0], so, ri, block, pos, ws)      # the workspace exists before capture
    torch.cuda.synchronize()
    graphs, outs = [], []
    for r in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=sm):
            outs.append(_five_calls(R, ins[r], so, ri, block, pos, ws))
        graphs.append(g)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        r = rep % 2
        with torch.cuda.stream(sm):
            want = [t.clone() for t in _five_calls(R, ins[r], so, ri, block, pos, ws)]
        torch.cuda.synchronize()
        for t in outs[r]:
            t.view(torch.uint8).fill_(7)                     # clobber the captured outputs
        scratch.mul_(1.0001).add_(0.5)                       # unrelated eager work
        torch.cuda.synchronize()
        graphs[r].replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(want, outs[r])):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep}: output {k} differs from eager"


def test_fused_step_repeats_bitwise_and_graph_replays_match_eager():
    import ctypes

    from diffusion_lm_unmask_amd import _lib
    R, ins, so, ri, block, pos, ws = _llada(2)
    parts = dict(fast=dict(eligible=block, tau=R["tau"]),
                 depcap=dict(lam=R["lam"], l_min=R["l_min"], l_max=R["l_max"]),
                 cap=dict(eligible=block, tau_low=R["tau_low"], tau_high=R["tau_high"],
                          gamma=R["gamma"], k_max=R["k_max"]))
    built = [api.step_descriptor(cur, prev, so, row_index=ri, **parts,
                                 dapd=dict(attn=attn, masked_pos=pos, m_max=cur.shape[0],
                                           tau=R["dapd_tau"], workspace=ws))
             for cur, prev, attn in ins]
    sm = torch.cuda.Stream(device=DEV)
    L = _lib.lib()

    def run(r):
        assert L.dlm_decide_step(ctypes.byref(built[r][0]), sm.cuda_stream) == 0

    def outputs(r):
        o = built[r][1]
        ts = [o[k] for k in ("conf", "argmax", "entropy", "kl", "lse")]
        for part in ("fast", "depcap", "cap", "dapd"):
            ts += list(o[part])
        return ts

    torch.cuda.synchronize()
    run(0)
    torch.cuda.synchronize()
    first = [t.clone() for t in outputs(0)]
    run(1)
    run(0)
    torch.cuda.synchronize()
    for a, b in zip(first, outputs(0)):
        assert torch.equal(_bits(a), _bits(b)), "dlm_decide_step is not deterministic"
    graphs = []
    for r in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=sm):
            run(r)
        graphs.append(g)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        r = rep % 2
        run(r)
        torch.cuda.synchronize()
        want = [t.clone() for t in outputs(r)]
        for t in outputs(r):
            t.view(torch.uint8).fill_(7)                     # clobber the outputs
        scratch.mul_(1.0001).add_(0.5)                       # unrelated eager work
        torch.cuda.synchronize()
        graphs[r].replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(want, outputs(r))):
            assert torch.equal(_bits(a), _bits(b)), f"fused replay {rep}: output {k} differs"


def test_binding_refuses_to_create_a_workspace_under_capture(monkeypatch):
    # a split-row workspace first needed under capture is refused (its zero
    # fill would only be recorded): checked with the capture query forced on,
    # so no real capture is aborted; created eagerly first, a real capture of
    # the split call replays bit for bit
    x = torch.randn(40, 3000, device=DEV).to(torch.bfloat16)
    sm = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(sm):
        with monkeypatch.context() as m:
            m.setattr(torch.cuda, "is_current_stream_capturing", lambda: True)
            with pytest.raises(DLMError):
                api.step_stats(x, split=True)
        want = api.step_stats(x, split=True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=sm):
        got = api.step_stats(x, split=True)
    for _ in range(3):
        got["conf"].fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(got["conf"], want["conf"]) and torch.equal(got["argmax"], want["argmax"])
