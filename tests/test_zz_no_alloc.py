"""GPU test of dlm_dapd_select_static, the DAPD selection whose workspace is
the library's static per-GPU array (for callers that cannot allocate).

It is called through the C ABI with caller-owned outputs and compared, bit
for bit, with dlm_dapd_select (caller workspace) on the same inputs: first on
the DAPD workload (8 sequences x 256 masked positions over [8, 320, 768, 768]
bf16 attention, the edge-rich partner variant), then, reusing the same static
array, on a smaller call (3 sequences of at most 40 positions, one empty, fp32
attention), so that anything left in the array by the first call would show.
"""
import ctypes

import numpy as np
import pytest
import torch

from diffusion_lm_unmask_amd import _lib, api, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _call(fn_name, attn, pos, so, conf, tau, m_max, workspace=None):
    L = _lib.lib()
    n, n_seq = conf.numel(), so.numel() - 1
    B, n_lh, S, _ = attn.shape
    outs = dict(commit=torch.full((n,), 0xA5, device=DEV, dtype=torch.uint8),
                n_commit=torch.full((n_seq,), -7, device=DEV, dtype=torch.int32),
                degree=torch.full((n,), 7.0, device=DEV),
                key=torch.full((n,), 7.0, device=DEV),
                sym=torch.full((n_seq, m_max, m_max), 7.0, device=DEV))
    dt = _lib.BF16 if attn.dtype == torch.bfloat16 else _lib.F32
    stream = torch.cuda.current_stream().cuda_stream
    args = [attn.data_ptr(), dt, n_lh, S, n_lh * S * S, pos.data_ptr(), so.data_ptr(), n_seq,
            m_max, conf.data_ptr(), ctypes.c_float(tau), outs["commit"].data_ptr(),
            outs["n_commit"].data_ptr(), outs["degree"].data_ptr(), outs["sym"].data_ptr(),
            outs["key"].data_ptr()]
    if workspace is not None:
        args += [workspace.data_ptr(), workspace.numel()]
    st = getattr(L, fn_name)(*args, stream)
    assert st == 0, (fn_name, _lib.lib().dlm_status_string(st))
    return outs


def _compare(attn, pos, so, conf, tau, m_max, tag):
    need = int(_lib.lib().dlm_dapd_workspace_bytes(so.numel() - 1, m_max))
    ws = torch.full((need,), 0x5A, device=DEV, dtype=torch.uint8)
    want = _call("dlm_dapd_select", attn, pos, so, conf, tau, m_max, ws)
    got = _call("dlm_dapd_select_static", attn, pos, so, conf, tau, m_max)
    torch.cuda.synchronize()
    for k in want:
        assert torch.equal(_bits(got[k]), _bits(want[k])), f"{tag}: {k} differs"
    return want


def test_static_workspace_matches_caller_workspace():
    print("[no-alloc] call 1: dapd workload, 8 x 256, cov attention", flush=True)
    spec = synth.SPECS["dapd"]
    cur, prev, so, ri = synth.logits("dapd", DEV)
    conf = api.step_stats(cur)["conf"]
    pos, offs = synth.gen_positions("dapd", DEV)
    attn = synth.attention("dapd", DEV, variant="cov", masked_pos=pos[:spec.rows])
    out = _compare(attn, pos, offs, conf, 0.01, 256, "dapd 8 x 256")
    n_commit = out["n_commit"].cpu().numpy()
    assert np.all(n_commit > 0) and np.all(n_commit < 256), n_commit   # real graphs, with edges
    del attn, cur
    torch.cuda.empty_cache()

    print("[no-alloc] call 2: 3 sequences (40, 0, 37 positions), fp32 attention", flush=True)
    small = synth.Spec("scat", 11, 3, 40, 512, torch.bfloat16, 2.0, 0.6, 12.0, None,
                       n_lh=6, seq_len=100, attn_sigma=3.0)
    cur2, _, _, _ = synth.logits(small, DEV)
    conf2 = api.step_stats(cur2)["conf"][:77].contiguous()
    gen = torch.Generator().manual_seed(3)
    pos2 = torch.cat([torch.randperm(100, generator=gen)[:40].sort().values for _ in range(3)])
    pos2 = pos2[:77].to(device=DEV, dtype=torch.int32).contiguous()
    attn2 = synth.attention(small, DEV).float().contiguous()
    so2 = torch.tensor([0, 40, 40, 77], device=DEV, dtype=torch.int32)
    for tau in (0.01, 0.02):
        _compare(attn2, pos2, so2, conf2, tau, 45, f"small tau={tau}")


def test_static_workspace_size_limit():
    # beyond the static array the call is refused before any launch
    L = _lib.lib()
    attn = torch.zeros(64, 1, 8, 8, device=DEV)
    pos = torch.zeros(64 * 1024, device=DEV, dtype=torch.int32)
    so = torch.arange(0, 65 * 1024, 1024, device=DEV, dtype=torch.int32)
    conf = torch.zeros(64 * 1024, device=DEV)
    commit = torch.zeros(64 * 1024, device=DEV, dtype=torch.uint8)
    n_commit = torch.full((64,), -7, device=DEV, dtype=torch.int32)
    st = L.dlm_dapd_select_static(attn.data_ptr(), _lib.F32, 1, 8, 64, pos.data_ptr(),
                                  so.data_ptr(), 64, 1024, conf.data_ptr(), ctypes.c_float(0.01),
                                  commit.data_ptr(), n_commit.data_ptr(), None, None, None,
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == _lib.ERR_UNSUPPORTED
    assert int(n_commit[0]) == -7                     # nothing was launched
