"""The whole decision step (the five calls, and the fused call) captured as a
HIP graph (marked gpu).

Replays are interleaved with unrelated eager work and synchronisations, and
every replay must reproduce the eager step bit for bit (no memset nodes are
recorded: the stats workspace is zero-filled once, before capture, and the
kernels leave it zero-filled)."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_llada_step_graph_replays_match_eager():
    import bench
    step = bench.LladaStep(2, "cuda:0")
    sm = step.torch_stream
    torch.cuda.synchronize()
    graphs = []
    for r in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=sm):
            step.step(r)
        graphs.append(g)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        r = rep % 2
        with torch.cuda.stream(sm):
            step.step(r)
        torch.cuda.synchronize()
        want = step.outputs()
        for t in (step.conf, step.commit_d, step.blen):   # clobber the outputs
            t.fill_(7)
        scratch.mul_(1.0001).add_(0.5)                     # unrelated eager work
        torch.cuda.synchronize()
        graphs[r].replay()
        torch.cuda.synchronize()
        got = step.outputs()
        for a, b in zip(want, got):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"


def test_fused_step_repeats_bitwise_and_graph_replays_match_eager():
    import bench
    step = bench.LladaStep(2, "cuda:0")
    sm = step.torch_stream
    torch.cuda.synchronize()
    # eager repeats are bitwise identical
    with torch.cuda.stream(sm):
        step.fused(0)
    torch.cuda.synchronize()
    first = step.outputs()
    with torch.cuda.stream(sm):
        step.fused(1)
        step.fused(0)
    torch.cuda.synchronize()
    for a, b in zip(first, step.outputs()):
        assert torch.equal(a, b), "dlm_decide_step is not deterministic"
    graphs = []
    for r in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=sm):
            step.fused(r)
        graphs.append(g)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        r = rep % 2
        with torch.cuda.stream(sm):
            step.fused(r)
        torch.cuda.synchronize()
        want = step.outputs()
        for t in (step.conf, step.commit_d, step.nd, step.commit_c, step.nc, step.commit_f,
                  step.nf, step.blen):                                    # clobber the outputs
            t.fill_(7)
        scratch.mul_(1.0001).add_(0.5)                                    # unrelated eager work
        torch.cuda.synchronize()
        graphs[r].replay()
        torch.cuda.synchronize()
        for a, b in zip(want, step.outputs()):
            assert torch.equal(a, b), f"fused replay {rep} differs from the eager step"
