"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/dlm.h, and rejects bad arguments on the host (these
calls return before any HIP call, so nothing is enqueued)."""
import ctypes
import math

import pytest

from diffusion_lm_unmask_amd import _lib

FAKE = 0x100000  # a non-NULL, aligned pointer value; never dereferenced here


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_exports_every_declared_symbol(L):
    names = _lib.header_symbols()
    assert set(names) == set(_lib.SIGNATURES)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s, text in ((0, b"ok"), (1, b"invalid argument"), (3, b"HIP kernel launch failed")):
        assert L.dlm_status_string(s) == text
    assert L.dlm_status_string(99) == b"unknown status"


def test_step_stats_validation(L):
    f = L.dlm_step_stats
    args = [FAKE, None, _lib.BF16, 1000, 1000, FAKE, 4, FAKE, FAKE, FAKE, None, FAKE, None, 0,
            None]
    bad = list(args)
    bad[0] = None
    assert f(*bad) == _lib.ERR_ARG                      # NULL logits
    bad = list(args)
    bad[2] = 5
    assert f(*bad) == _lib.ERR_UNSUPPORTED              # unknown dtype
    bad = list(args)
    bad[4] = 999
    assert f(*bad) == _lib.ERR_ARG                      # ld < vocab
    bad = list(args)
    bad[6] = 0
    assert f(*bad) == _lib.ERR_ARG                      # no rows
    bad = list(args)
    bad[1] = FAKE
    assert f(*bad) == _lib.ERR_ARG                      # prev without kl
    bad = list(args)
    bad[0] = FAKE + 1
    assert f(*bad) == _lib.ERR_ARG                      # misaligned bf16 base
    bad = list(args)
    bad[3] = 2**31
    bad[4] = 2**31
    assert f(*bad) == _lib.ERR_UNSUPPORTED              # vocab >= 2^31
    need = L.dlm_step_stats_workspace_bytes(4)
    assert need > 0 and L.dlm_step_stats_workspace_bytes(0) == 0
    bad = list(args)
    bad[12], bad[13] = FAKE, need - 1
    assert f(*bad) == _lib.ERR_ARG                      # workspace too small
    bad[12], bad[13] = FAKE + 8, need
    assert f(*bad) == _lib.ERR_ARG                      # workspace misaligned


def test_rule_validation(L):
    assert L.dlm_fastdllm_select(FAKE, None, FAKE, 1, math.nan, FAKE, FAKE, None) == _lib.ERR_ARG
    assert L.dlm_fastdllm_select(None, None, FAKE, 1, 0.9, FAKE, FAKE, None) == _lib.ERR_ARG
    assert L.dlm_fastdllm_select(FAKE, None, FAKE, 0, 0.9, FAKE, FAKE, None) == _lib.ERR_ARG
    d = L.dlm_depcap_boundary
    ok = [FAKE, FAKE, FAKE, 1, None, 1.2, 8, 128, 1, 1e-12, FAKE, None, None]
    for i, v, code in ((6, 9, _lib.ERR_ARG), (7, 4, _lib.ERR_ARG), (7, 2048, _lib.ERR_UNSUPPORTED),
                       (8, -1, _lib.ERR_ARG), (5, math.nan, _lib.ERR_ARG), (9, -1.0, _lib.ERR_ARG),
                       (10, None, _lib.ERR_ARG)):
        bad = list(ok)
        bad[7] = 128
        bad[i] = v
        if i == 6:
            bad[7] = 8           # l_min > l_max
        assert d(*bad) == code, (i, v)
    c = L.dlm_cap_select
    ok = [FAKE, _lib.BF16, 1000, 1000, FAKE, FAKE, 1, FAKE, FAKE, FAKE, None, 0.8, 0.95, -16.0, 64,
          FAKE, FAKE, None, None, None]
    for i, v, code in ((14, 129, _lib.ERR_UNSUPPORTED), (14, 0, _lib.ERR_ARG),
                       (1, 3, _lib.ERR_UNSUPPORTED), (13, math.nan, _lib.ERR_ARG),
                       (9, None, _lib.ERR_ARG), (6, 0, _lib.ERR_ARG)):
        bad = list(ok)
        bad[i] = v
        assert c(*bad) == code, (i, v)


def test_dapd_validation(L):
    # the fp32 average a plus the adjacency bitsets, keys and edge flags
    assert L.dlm_dapd_workspace_bytes(8, 256) >= 8 * 256 * 256 * 4 + 8 * 256 * (32 + 8 + 1)
    assert L.dlm_dapd_workspace_bytes(8, 256) % 256 == 0
    assert L.dlm_dapd_workspace_bytes(1, 1025) == 0
    assert L.dlm_dapd_workspace_bytes(0, 10) == 0
    f = L.dlm_dapd_select
    need = L.dlm_dapd_workspace_bytes(2, 64)
    ok = [FAKE, _lib.BF16, 4, 96, 4 * 96 * 96, FAKE, FAKE, 2, 64, FAKE, 0.01, FAKE, FAKE, None,
          None, None, FAKE, need, None]
    for i, v, code in ((17, need - 1, _lib.ERR_ARG), (8, 1025, _lib.ERR_UNSUPPORTED),
                       (10, math.nan, _lib.ERR_ARG), (4, 10, _lib.ERR_ARG),
                       (16, None, _lib.ERR_ARG), (16, FAKE + 4, _lib.ERR_ARG),
                       (1, 9, _lib.ERR_UNSUPPORTED), (2, 0, _lib.ERR_ARG),
                       (3, 2**31, _lib.ERR_UNSUPPORTED),
                       (3, 2**31 - 1, _lib.ERR_UNSUPPORTED)):  # 4 maps of S*S overflow int64
        bad = list(ok)
        bad[i] = v
        assert f(*bad) == code, (i, v)
    # the static-workspace variant: the same checks (no workspace argument),
    # and sizes beyond its static array are refused before any HIP call
    g = L.dlm_dapd_select_static
    ok_s = ok[:16] + ok[18:]
    assert len(ok_s) == 17
    for i, v, code in ((8, 1025, _lib.ERR_UNSUPPORTED), (10, math.nan, _lib.ERR_ARG),
                       (4, 10, _lib.ERR_ARG), (1, 9, _lib.ERR_UNSUPPORTED), (2, 0, _lib.ERR_ARG),
                       (0, None, _lib.ERR_ARG), (11, None, _lib.ERR_ARG)):
        bad = list(ok_s)
        bad[i] = v
        assert g(*bad) == code, (i, v)
    big = list(ok_s)
    big[7], big[8] = 64, 1024                           # 277 MB of workspace: over the array
    assert L.dlm_dapd_workspace_bytes(64, 1024) > 16 << 20
    assert g(*big) == _lib.ERR_UNSUPPORTED


def test_schedule_validation(L):
    assert L.dlm_topk_select(FAKE, None, FAKE, 1, 0, FAKE, FAKE, None) == _lib.ERR_ARG      # k < 1
    assert L.dlm_topk_select(None, None, FAKE, 1, 2, FAKE, FAKE, None) == _lib.ERR_ARG
    assert L.dlm_topk_select(FAKE, None, FAKE, 0, 2, FAKE, FAKE, None) == _lib.ERR_ARG      # n_seq
    assert L.dlm_factor_select(FAKE, None, FAKE, 1, math.nan, FAKE, FAKE, None, None) == _lib.ERR_ARG
    assert L.dlm_factor_select(FAKE, None, FAKE, 1, 1.0, None, FAKE, None, None) == _lib.ERR_ARG
    assert L.dlm_fixed_block_eligible(FAKE, FAKE, 1, None, 0, FAKE, None) == _lib.ERR_ARG  # len 0
    assert L.dlm_fixed_block_eligible(FAKE, FAKE, 1, None, 32, None, None) == _lib.ERR_ARG
    need = L.dlm_dapd_workspace_bytes(2, 64)
    ok = [FAKE, _lib.BF16, 4, 96, 4 * 96 * 96, FAKE, FAKE, 2, 64, FAKE, 0.01, None, 0.5, 0.9, 1,
          FAKE, FAKE, None, None, None, None, FAKE, need, None]
    f = L.dlm_dapd_step
    for i, v, code in ((12, math.nan, _lib.ERR_ARG), (13, math.nan, _lib.ERR_ARG),
                       (22, need - 1, _lib.ERR_ARG), (8, 1025, _lib.ERR_UNSUPPORTED),
                       (15, None, _lib.ERR_ARG)):
        bad = list(ok)
        bad[i] = v
        assert f(*bad) == code, (i, v)


def test_step_desc_layout_matches_the_header(tmp_path):
    # compile the header with the host C compiler and compare every field's
    # offset and the struct size with the ctypes mirror used by the binding
    import os
    import subprocess
    fields = [f for f, _ in _lib.StepDesc._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "dlm.h"\nint main(void){\n' +
                   "".join(f'printf("%zu\\n", offsetof(dlm_step_desc, {f}));\n' for f in fields) +
                   'printf("%zu\\n", sizeof(dlm_step_desc));\nreturn 0;}\n')
    exe = tmp_path / "layout"
    inc = os.path.join(os.path.dirname(_lib.HEADER))
    subprocess.run(["gcc", "-std=c99", "-I", inc, str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    want = [getattr(_lib.StepDesc, f).offset for f in fields] + [ctypes.sizeof(_lib.StepDesc)]
    assert got == want


def test_decide_step_validation(L):
    d = _lib.StepDesc()
    assert L.dlm_decide_step(None, None) == _lib.ERR_ARG
    assert L.dlm_decide_step(ctypes.byref(d), None) == _lib.ERR_ARG     # no logits
    d.logits = d.row_index = d.conf = d.argmax = d.entropy = d.lse = FAKE
    d.dtype, d.vocab, d.ld, d.n_rows = _lib.BF16, 1000, 1000, 4
    d.fast_commit, d.fast_n_commit, d.fast_tau = FAKE, FAKE, math.nan
    d.seq_offsets, d.n_seq = FAKE, 1
    assert L.dlm_decide_step(ctypes.byref(d), None) == _lib.ERR_ARG     # NaN tau
    d.fast_tau = 0.9
    d.depcap_block_len, d.depcap_l_min, d.depcap_l_max = FAKE, 8, 128
    assert L.dlm_decide_step(ctypes.byref(d), None) == _lib.ERR_ARG     # DepCap without KL
    d.depcap_block_len = None
    d.dapd_commit, d.dapd_n_commit = FAKE, FAKE
    d.attn, d.attn_dtype, d.n_lh, d.S, d.masked_pos, d.m_max = FAKE, _lib.BF16, 4, 96, FAKE, 2000
    d.dapd_workspace = FAKE
    assert L.dlm_decide_step(ctypes.byref(d), None) == _lib.ERR_UNSUPPORTED  # m_max > 1024


def test_binding_fails_loudly_without_device_tensors():
    torch = pytest.importorskip("torch")
    import diffusion_lm_unmask_amd as d
    with pytest.raises(d.DLMError):
        d.step_stats(torch.zeros(2, 8))             # host tensor: refused, no CPU fallback
