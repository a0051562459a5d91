"""Thin torch-facing binding over the C ABI (include/dlm.h).

Each function checks device, dtype, shape and contiguity, allocates its
outputs as torch tensors on the input's device, and calls the library entry
point of the same name on torch's current HIP stream.  Argument marshalling
only: every step of the computation runs in the library's kernels.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import DLMError

DEFAULTS = dict(
    fastdllm_tau=0.9, fastdllm_block=32,
    depcap_lambda=1.2, depcap_l_min=8, depcap_l_max=128, depcap_radius=1, depcap_eps=1e-12,
    cap_tau_low=0.8, cap_tau_high=0.95, cap_gamma=-16.0,
    dapd_layer_frac=0.3, dapd_late_frac=0.5, dapd_late_tau=0.9, factor_f=1.0,
)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise DLMError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise DLMError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _vec(t, name, dtype, device):
    _dev(t, name, dtype)
    if t.device != device:
        raise DLMError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise DLMError(f"{name} must be contiguous")
    return t


def _opt(t, name, dtype, device):
    return None if t is None else _vec(t, name, dtype, device)


def _ptr(t):
    return None if t is None else t.data_ptr()


_PLACEHOLDER: dict = {}


def _rows(t):
    """Pointer to a per-row tensor.  A tensor with no rows has no storage
    (data_ptr 0), which the library refuses as a missing argument.  With no
    rows the kernels never dereference it, so the address of a small
    per-device placeholder stands in, and the launch still writes every
    sequence's outputs (an empty sequence commits nothing)."""
    if t is None:
        return None
    if t.numel():
        return t.data_ptr()
    ph = _PLACEHOLDER.get(t.device)
    if ph is None:
        ph = _PLACEHOLDER[t.device] = torch.zeros(64, device=t.device, dtype=torch.int64)
    return ph.data_ptr()


def _len(t, n, name):
    """Per-row (or per-sequence) tensors must match the count they go with:
    the kernels index them by row, and the library cannot see their sizes."""
    if t is not None and t.numel() != n:
        raise DLMError(f"{name} has {t.numel()} entries, expected {n}")


def _vocab(vocab, logits):
    vocab = logits.shape[1] if vocab is None else int(vocab)
    if not 1 <= vocab <= logits.shape[1]:
        raise DLMError(f"vocab must be in [1, {logits.shape[1]}] (the logits' row length)")
    return vocab


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return _lib.BF16
    if t.dtype == torch.float32:
        return _lib.F32
    raise DLMError(f"unsupported element type {t.dtype}")


def _rows2d(logits, name):
    _dev(logits, name)
    if logits.dim() != 2 or logits.stride(1) != 1:
        raise DLMError(f"{name} must be 2-D [rows, ld] with unit column stride")
    return logits.stride(0)


_WORKSPACES: dict = {}
_RETIRED: list = []


def stats_workspace(n_rows: int, device) -> torch.Tensor:
    """Zero-filled dlm_step_stats workspace for `n_rows` rows, cached per
    (device, current stream): the library leaves it zero-filled after every
    call, and calls on one stream never overlap.

    A workspace is never freed: when a call needs a larger one, the smaller
    one is kept alive (a HIP graph captured earlier may still point at it).
    A new workspace is never made during stream capture, where its zero fill
    would only be recorded: call once eagerly on the stream first, or pass
    split=False."""
    dev = torch.device(device)
    key = (dev.index, torch.cuda.current_stream(dev).cuda_stream)
    need = int(_lib.lib().dlm_step_stats_workspace_bytes(int(n_rows)))
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < need:
        if torch.cuda.is_current_stream_capturing():
            raise DLMError("the statistics workspace for this many rows does not exist yet and "
                           "cannot be created under graph capture: call step_stats once "
                           "eagerly on this stream first, or pass split=False")
        if ws is not None:
            _RETIRED.append(ws)
        ws = torch.zeros(max(need, 256), device=dev, dtype=torch.uint8)
        torch.cuda.synchronize(dev)          # zeroed before any kernel can use it
        _WORKSPACES[key] = ws
    return ws


def step_stats(logits: torch.Tensor, prev: torch.Tensor | None = None,
               row_index: torch.Tensor | None = None, vocab: int | None = None,
               split: bool = True):
    """dlm_step_stats.  logits: [N, >=vocab] (bf16 or f32, unit column
    stride); row_index: int64 rows to decide (default: all).  Returns a dict
    with conf, argmax, entropy, kl (None without prev), lse.  split=False
    runs one workgroup per row (no workspace)."""
    ld = _rows2d(logits, "logits")
    dev = logits.device
    vocab = _vocab(vocab, logits)
    if prev is not None:
        _rows2d(prev, "prev")
        if prev.dtype != logits.dtype or prev.stride(0) != ld or prev.shape != logits.shape:
            raise DLMError("prev must match logits in dtype, shape and strides")
    if row_index is not None:
        _vec(row_index, "row_index", torch.int64, dev)
    n = logits.shape[0] if row_index is None else row_index.numel()
    f = dict(device=dev, dtype=torch.float32)
    conf, ent, lse = torch.empty(n, **f), torch.empty(n, **f), torch.empty(n, **f)
    kl = torch.empty(n, **f) if prev is not None else None
    arg = torch.empty(n, device=dev, dtype=torch.int32)
    ws = stats_workspace(n, dev) if split else None
    st = _lib.lib().dlm_step_stats(logits.data_ptr(), _ptr(prev), _dtype_code(logits), vocab, ld,
                                   _ptr(row_index), n, conf.data_ptr(), arg.data_ptr(),
                                   ent.data_ptr(), _ptr(kl), lse.data_ptr(), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(logits))
    _lib.check(st, "dlm_step_stats")
    return {"conf": conf, "argmax": arg, "entropy": ent, "kl": kl, "lse": lse}


def fastdllm_select(conf, seq_offsets, tau=DEFAULTS["fastdllm_tau"], eligible=None):
    """dlm_fastdllm_select -> (commit u8 [rows], n_commit int32 [n_seq])."""
    dev = _vec(conf, "conf", torch.float32, conf.device).device
    _vec(seq_offsets, "seq_offsets", torch.int32, dev)
    _opt(eligible, "eligible", torch.uint8, dev)
    _len(eligible, conf.numel(), "eligible")
    n_seq = seq_offsets.numel() - 1
    commit = torch.empty(conf.numel(), device=dev, dtype=torch.uint8)
    n_commit = torch.empty(max(n_seq, 0), device=dev, dtype=torch.int32)
    st = _lib.lib().dlm_fastdllm_select(_rows(conf), _ptr(eligible), seq_offsets.data_ptr(),
                                        n_seq, float(tau), _rows(commit), n_commit.data_ptr(),
                                        _stream(conf))
    _lib.check(st, "dlm_fastdllm_select")
    return commit, n_commit


def depcap_boundary(kl, entropy, seq_offsets, has_prev=None, lam=DEFAULTS["depcap_lambda"],
                    l_min=DEFAULTS["depcap_l_min"], l_max=DEFAULTS["depcap_l_max"],
                    radius=DEFAULTS["depcap_radius"], eps=DEFAULTS["depcap_eps"],
                    want_score=True):
    """dlm_depcap_boundary -> (block_len int32 [n_seq], score f64 [rows] or None)."""
    dev = _vec(kl, "kl", torch.float32, kl.device).device
    _vec(entropy, "entropy", torch.float32, dev)
    _vec(seq_offsets, "seq_offsets", torch.int32, dev)
    _opt(has_prev, "has_prev", torch.uint8, dev)
    if entropy.numel() != kl.numel():
        raise DLMError("kl and entropy must have the same length")
    n_seq = seq_offsets.numel() - 1
    _len(has_prev, n_seq, "has_prev")
    block_len = torch.empty(max(n_seq, 0), device=dev, dtype=torch.int32)
    score = torch.empty(kl.numel(), device=dev, dtype=torch.float64) if want_score else None
    st = _lib.lib().dlm_depcap_boundary(_rows(kl), _rows(entropy), seq_offsets.data_ptr(),
                                        n_seq, _ptr(has_prev), float(lam), int(l_min), int(l_max),
                                        int(radius), float(eps), block_len.data_ptr(),
                                        _ptr(score), _stream(kl))
    _lib.check(st, "dlm_depcap_boundary")
    return block_len, score


def cap_select(logits, row_index, seq_offsets, conf, argmax, lse, eligible=None,
               tau_low=DEFAULTS["cap_tau_low"], tau_high=DEFAULTS["cap_tau_high"],
               gamma=DEFAULTS["cap_gamma"], k_max=64, vocab=None, want_cand=False,
               want_dmat=False):
    """dlm_cap_select -> dict(commit, n_commit, cand or None, dmat or None).
    row_index None: row r of logits is candidate row r."""
    ld = _rows2d(logits, "logits")
    dev = logits.device
    vocab = _vocab(vocab, logits)
    _opt(row_index, "row_index", torch.int64, dev)
    _vec(seq_offsets, "seq_offsets", torch.int32, dev)
    _vec(conf, "conf", torch.float32, dev)
    _vec(argmax, "argmax", torch.int32, dev)
    _vec(lse, "lse", torch.float32, dev)
    _opt(eligible, "eligible", torch.uint8, dev)
    for t, name in ((row_index, "row_index"), (argmax, "argmax"), (lse, "lse"),
                    (eligible, "eligible")):
        _len(t, conf.numel(), name)
    n_seq = seq_offsets.numel() - 1
    k_max = int(k_max)
    commit = torch.empty(conf.numel(), device=dev, dtype=torch.uint8)
    n_commit = torch.empty(max(n_seq, 0), device=dev, dtype=torch.int32)
    cand = torch.empty(max(n_seq, 0), k_max, device=dev, dtype=torch.int32) if want_cand else None
    dmat = (torch.empty(max(n_seq, 0), k_max, k_max, device=dev, dtype=torch.float32)
            if want_dmat else None)
    st = _lib.lib().dlm_cap_select(_rows(logits), _dtype_code(logits), vocab, ld,
                                   _ptr(row_index), seq_offsets.data_ptr(), n_seq,
                                   _rows(conf), _rows(argmax), _rows(lse),
                                   _ptr(eligible), float(tau_low), float(tau_high), float(gamma),
                                   k_max, _rows(commit), n_commit.data_ptr(), _ptr(cand),
                                   _ptr(dmat), _stream(logits))
    _lib.check(st, "dlm_cap_select")
    return {"commit": commit, "n_commit": n_commit, "cand": cand, "dmat": dmat}


def dapd_workspace_bytes(n_seq: int, m_max: int) -> int:
    return int(_lib.lib().dlm_dapd_workspace_bytes(int(n_seq), int(m_max)))


def _dapd_args(attn, masked_pos, seq_offsets, conf, m_max):
    """Checks shared by the DAPD selection bindings; returns (dev, n_lh, S, n_seq)."""
    _dev(attn, "attn")
    if attn.dim() != 4 or not attn.is_contiguous() or attn.shape[2] != attn.shape[3]:
        raise DLMError("attn must be a contiguous [B, n_lh, S, S] tensor")
    dev = attn.device
    B, n_lh, S, _ = attn.shape
    _vec(masked_pos, "masked_pos", torch.int32, dev)
    _vec(seq_offsets, "seq_offsets", torch.int32, dev)
    _vec(conf, "conf", torch.float32, dev)
    _len(masked_pos, conf.numel(), "masked_pos")
    n_seq = seq_offsets.numel() - 1
    if n_seq > B:
        raise DLMError("more sequences than attention batches")
    if m_max is None:
        raise DLMError("m_max (an upper bound on masked positions per sequence) is required")
    return dev, n_lh, S, n_seq


def _dapd_outputs(dev, n, n_seq, m_max, want_degree, want_key, want_sym):
    f = dict(device=dev, dtype=torch.float32)
    return (torch.empty(n, device=dev, dtype=torch.uint8),
            torch.empty(max(n_seq, 0), device=dev, dtype=torch.int32),
            torch.empty(n, **f) if want_degree else None,
            torch.empty(n, **f) if want_key else None,
            torch.empty(max(n_seq, 0), m_max, m_max, **f) if want_sym else None)


def dapd_select(attn, masked_pos, seq_offsets, conf, tau, m_max=None, workspace=None,
                want_degree=False, want_key=False, want_sym=False):
    """dlm_dapd_select.  attn: [B, n_lh, S, S] contiguous (bf16 or f32), the
    maps to average; masked_pos int32 CSR by seq_offsets; conf f32 per row.
    Returns dict(commit, n_commit, degree, key, sym)."""
    dev, n_lh, S, n_seq = _dapd_args(attn, masked_pos, seq_offsets, conf, m_max)
    need = dapd_workspace_bytes(n_seq, m_max)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    _vec(workspace, "workspace", torch.uint8, dev)
    commit, n_commit, degree, key, sym = _dapd_outputs(dev, conf.numel(), n_seq, m_max,
                                                       want_degree, want_key, want_sym)
    st = _lib.lib().dlm_dapd_select(attn.data_ptr(), _dtype_code(attn), n_lh, S, n_lh * S * S,
                                    _rows(masked_pos), seq_offsets.data_ptr(), n_seq,
                                    int(m_max), _rows(conf), float(tau), _rows(commit),
                                    n_commit.data_ptr(), _ptr(degree), _ptr(sym), _ptr(key),
                                    workspace.data_ptr(), workspace.numel(), _stream(attn))
    _lib.check(st, "dlm_dapd_select")
    return {"commit": commit, "n_commit": n_commit, "degree": degree, "key": key, "sym": sym}


def dapd_select_static(attn, masked_pos, seq_offsets, conf, tau, m_max=None,
                       want_degree=False, want_key=False, want_sym=False):
    """dlm_dapd_select_static: dlm_dapd_select with the library's static
    per-GPU workspace (no workspace argument; the library allocates nothing).
    Calls that overlap in time on one GPU race.  The outputs are allocated
    here, as for every binding; a caller that cannot allocate calls the C
    entry point with its own output buffers."""
    dev, n_lh, S, n_seq = _dapd_args(attn, masked_pos, seq_offsets, conf, m_max)
    commit, n_commit, degree, key, sym = _dapd_outputs(dev, conf.numel(), n_seq, m_max,
                                                       want_degree, want_key, want_sym)
    st = _lib.lib().dlm_dapd_select_static(attn.data_ptr(), _dtype_code(attn), n_lh, S,
                                           n_lh * S * S, _rows(masked_pos),
                                           seq_offsets.data_ptr(), n_seq, int(m_max),
                                           _rows(conf), float(tau), _rows(commit),
                                           n_commit.data_ptr(), _ptr(degree), _ptr(sym),
                                           _ptr(key), _stream(attn))
    _lib.check(st, "dlm_dapd_select_static")
    return {"commit": commit, "n_commit": n_commit, "degree": degree, "key": key, "sym": sym}


def dapd_step(attn, masked_pos, seq_offsets, conf, tau, gen_len=None,
              late_frac=DEFAULTS["dapd_late_frac"], late_tau=DEFAULTS["dapd_late_tau"],
              pre_unmask=True, m_max=None, workspace=None, want_degree=False, want_key=False,
              want_sym=False):
    """dlm_dapd_step: dlm_dapd_select plus the late-stage switch (gen_len int32
    per sequence, or None) and the conf = 1 pre-unmask.  Returns dict(commit,
    n_commit, stage, degree, key, sym)."""
    _dev(attn, "attn")
    if attn.dim() != 4 or not attn.is_contiguous() or attn.shape[2] != attn.shape[3]:
        raise DLMError("attn must be a contiguous [B, n_lh, S, S] tensor")
    dev = attn.device
    B, n_lh, S, _ = attn.shape
    _vec(masked_pos, "masked_pos", torch.int32, dev)
    _vec(seq_offsets, "seq_offsets", torch.int32, dev)
    _vec(conf, "conf", torch.float32, dev)
    _opt(gen_len, "gen_len", torch.int32, dev)
    _len(masked_pos, conf.numel(), "masked_pos")
    n_seq = seq_offsets.numel() - 1
    _len(gen_len, n_seq, "gen_len")
    if n_seq > B:
        raise DLMError("more sequences than attention batches")
    if m_max is None:
        raise DLMError("m_max (an upper bound on masked positions per sequence) is required")
    need = dapd_workspace_bytes(n_seq, m_max)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    _vec(workspace, "workspace", torch.uint8, dev)
    n = conf.numel()
    f = dict(device=dev, dtype=torch.float32)
    commit = torch.empty(n, device=dev, dtype=torch.uint8)
    n_commit = torch.empty(max(n_seq, 0), device=dev, dtype=torch.int32)
    stage = torch.empty(max(n_seq, 0), device=dev, dtype=torch.uint8)
    degree = torch.empty(n, **f) if want_degree else None
    key = torch.empty(n, **f) if want_key else None
    sym = torch.empty(max(n_seq, 0), m_max, m_max, **f) if want_sym else None
    st = _lib.lib().dlm_dapd_step(attn.data_ptr(), _dtype_code(attn), n_lh, S, n_lh * S * S,
                                  _rows(masked_pos), seq_offsets.data_ptr(), n_seq,
                                  int(m_max), _rows(conf), float(tau), _ptr(gen_len),
                                  float(late_frac), float(late_tau), int(bool(pre_unmask)),
                                  _rows(commit), n_commit.data_ptr(), stage.data_ptr(),
                                  _ptr(degree), _ptr(sym), _ptr(key), workspace.data_ptr(),
                                  workspace.numel(), _stream(attn))
    _lib.check(st, "dlm_dapd_step")
    return {"commit": commit, "n_commit": n_commit, "stage": stage, "degree": degree,
            "key": key, "sym": sym}


def _select_common(conf, seq_offsets, eligible):
    _dev(conf, "conf", torch.float32)
    dev = conf.device
    _vec(conf, "conf", torch.float32, dev)
    _vec(seq_offsets, "seq_offsets", torch.int32, dev)
    _opt(eligible, "eligible", torch.uint8, dev)
    _len(eligible, conf.numel(), "eligible")
    n_seq = seq_offsets.numel() - 1
    commit = torch.empty(conf.numel(), device=dev, dtype=torch.uint8)
    n_commit = torch.empty(max(n_seq, 0), device=dev, dtype=torch.int32)
    return dev, n_seq, commit, n_commit


def factor_select(conf, seq_offsets, f=DEFAULTS["factor_f"], eligible=None):
    """dlm_factor_select: returns commit, n_commit and the Theorem-1 certificate."""
    dev, n_seq, commit, n_commit = _select_common(conf, seq_offsets, eligible)
    cert = torch.empty(max(n_seq, 0), device=dev, dtype=torch.uint8)
    st = _lib.lib().dlm_factor_select(_rows(conf), _ptr(eligible), seq_offsets.data_ptr(),
                                      n_seq, float(f), _rows(commit), n_commit.data_ptr(),
                                      cert.data_ptr(), _stream(conf))
    _lib.check(st, "dlm_factor_select")
    return commit, n_commit, cert


def topk_select(conf, seq_offsets, k, eligible=None):
    """dlm_topk_select: the k most confident eligible rows per sequence."""
    dev, n_seq, commit, n_commit = _select_common(conf, seq_offsets, eligible)
    st = _lib.lib().dlm_topk_select(_rows(conf), _ptr(eligible), seq_offsets.data_ptr(),
                                    n_seq, int(k), _rows(commit), n_commit.data_ptr(),
                                    _stream(conf))
    _lib.check(st, "dlm_topk_select")
    return commit, n_commit


def fixed_block_eligible(masked_pos, seq_offsets, block_len, gen_start=None):
    """dlm_fixed_block_eligible: masked rows of each sequence's active fixed block."""
    _dev(masked_pos, "masked_pos", torch.int32)
    dev = masked_pos.device
    _vec(masked_pos, "masked_pos", torch.int32, dev)
    _vec(seq_offsets, "seq_offsets", torch.int32, dev)
    _opt(gen_start, "gen_start", torch.int32, dev)
    n_seq = seq_offsets.numel() - 1
    _len(gen_start, n_seq, "gen_start")
    el = torch.empty(masked_pos.numel(), device=dev, dtype=torch.uint8)
    st = _lib.lib().dlm_fixed_block_eligible(_rows(masked_pos), seq_offsets.data_ptr(), n_seq,
                                             _ptr(gen_start), int(block_len), _rows(el),
                                             _stream(masked_pos))
    _lib.check(st, "dlm_fixed_block_eligible")
    return el


def step_descriptor(logits, prev=None, seq_offsets=None, row_index=None, vocab=None, fast=None,
                    depcap=None, cap=None, dapd=None):
    """The dlm_step_desc of a dlm_decide_step call, without calling it.
    Returns (desc, out, keep): the filled descriptor, the output tensors it
    points into (the dict decide_step returns) and the input tensors it
    points into (keep both alive while the descriptor is used).  For callers
    that issue the same step many times (a decoding loop, the benchmark).

    Each rule part is None (off) or a dict of its parameters, named as in the
    individual wrappers:
      fast   = dict(eligible=None, tau=0.9)
      depcap = dict(has_prev=None, lam=1.2, l_min=8, l_max=128, radius=1, eps=1e-12)
      cap    = dict(eligible=None, tau_low=0.8, tau_high=0.95, gamma=-16.0, k_max=64)
      dapd   = dict(attn=..., masked_pos=..., m_max=..., tau=0.01, workspace=None)
    `out` holds the statistics (conf, argmax, entropy, kl, lse) and, per
    enabled part, its outputs (fast / depcap / cap / dapd)."""
    ld = _rows2d(logits, "logits")
    dev = logits.device
    vocab = _vocab(vocab, logits)
    if prev is not None:
        _rows2d(prev, "prev")
        if prev.dtype != logits.dtype or prev.stride(0) != ld or prev.shape != logits.shape:
            raise DLMError("prev must match logits in dtype, shape and strides")
    if row_index is not None:
        _vec(row_index, "row_index", torch.int64, dev)
    n = logits.shape[0] if row_index is None else row_index.numel()
    if seq_offsets is None:
        seq_offsets = torch.tensor([0, n], device=dev, dtype=torch.int32)
    _vec(seq_offsets, "seq_offsets", torch.int32, dev)
    n_seq = seq_offsets.numel() - 1
    f = dict(device=dev, dtype=torch.float32)
    i32 = dict(device=dev, dtype=torch.int32)
    u8 = dict(device=dev, dtype=torch.uint8)
    out = {"conf": torch.empty(n, **f), "argmax": torch.empty(n, **i32),
           "entropy": torch.empty(n, **f), "lse": torch.empty(n, **f),
           "kl": torch.empty(n, **f) if prev is not None else None}
    d = _lib.StepDesc()
    d.logits, d.prev_logits = logits.data_ptr(), _ptr(prev)
    d.dtype, d.vocab, d.ld = _dtype_code(logits), vocab, ld
    d.row_index, d.n_rows = _ptr(row_index), n
    d.conf, d.argmax = out["conf"].data_ptr(), out["argmax"].data_ptr()
    d.entropy, d.kl, d.lse = out["entropy"].data_ptr(), _ptr(out["kl"]), out["lse"].data_ptr()
    d.seq_offsets, d.n_seq = seq_offsets.data_ptr(), n_seq
    keep = [row_index, seq_offsets]
    if fast is not None:
        el = _opt(fast.get("eligible"), "eligible", torch.uint8, dev)
        _len(el, n, "eligible")
        out["fast"] = (torch.empty(n, **u8), torch.empty(max(n_seq, 0), **i32))
        d.fast_eligible, d.fast_tau = _ptr(el), float(fast.get("tau", DEFAULTS["fastdllm_tau"]))
        d.fast_commit, d.fast_n_commit = out["fast"][0].data_ptr(), out["fast"][1].data_ptr()
        keep.append(el)
    if depcap is not None:
        hp = _opt(depcap.get("has_prev"), "has_prev", torch.uint8, dev)
        _len(hp, n_seq, "has_prev")
        out["depcap"] = (torch.empty(max(n_seq, 0), **i32),
                         torch.empty(n, device=dev, dtype=torch.float64))
        d.depcap_has_prev = _ptr(hp)
        d.depcap_lambda = float(depcap.get("lam", DEFAULTS["depcap_lambda"]))
        d.depcap_l_min = int(depcap.get("l_min", DEFAULTS["depcap_l_min"]))
        d.depcap_l_max = int(depcap.get("l_max", DEFAULTS["depcap_l_max"]))
        d.depcap_radius = int(depcap.get("radius", DEFAULTS["depcap_radius"]))
        d.depcap_eps = float(depcap.get("eps", DEFAULTS["depcap_eps"]))
        d.depcap_block_len, d.depcap_score = (out["depcap"][0].data_ptr(),
                                              out["depcap"][1].data_ptr())
        keep.append(hp)
    if cap is not None:
        el = _opt(cap.get("eligible"), "eligible", torch.uint8, dev)
        _len(el, n, "eligible")
        out["cap"] = (torch.empty(n, **u8), torch.empty(max(n_seq, 0), **i32))
        d.cap_eligible = _ptr(el)
        d.cap_tau_low = float(cap.get("tau_low", DEFAULTS["cap_tau_low"]))
        d.cap_tau_high = float(cap.get("tau_high", DEFAULTS["cap_tau_high"]))
        d.cap_gamma = float(cap.get("gamma", DEFAULTS["cap_gamma"]))
        d.cap_k_max = int(cap.get("k_max", 64))
        d.cap_commit, d.cap_n_commit = out["cap"][0].data_ptr(), out["cap"][1].data_ptr()
        keep.append(el)
    if dapd is not None:
        attn = dapd["attn"]
        _dev(attn, "attn")
        if attn.dim() != 4 or not attn.is_contiguous() or attn.shape[2] != attn.shape[3]:
            raise DLMError("attn must be a contiguous [B, n_lh, S, S] tensor")
        if n_seq > attn.shape[0]:
            raise DLMError("more sequences than attention batches")
        pos = _vec(dapd["masked_pos"], "masked_pos", torch.int32, dev)
        _len(pos, n, "masked_pos")
        m_max = int(dapd["m_max"])
        ws = dapd.get("workspace")
        if ws is None:
            ws = torch.empty(max(dapd_workspace_bytes(n_seq, m_max), 1), **u8)
        _vec(ws, "workspace", torch.uint8, dev)
        B, n_lh, S, _ = attn.shape
        out["dapd"] = (torch.empty(n, **u8), torch.empty(max(n_seq, 0), **i32))
        d.attn, d.attn_dtype, d.n_lh, d.S = attn.data_ptr(), _dtype_code(attn), n_lh, S
        d.batch_stride, d.masked_pos, d.m_max = n_lh * S * S, pos.data_ptr(), m_max
        d.dapd_tau = float(dapd.get("tau", 0.01))
        d.dapd_commit, d.dapd_n_commit = out["dapd"][0].data_ptr(), out["dapd"][1].data_ptr()
        d.dapd_workspace, d.dapd_workspace_bytes = ws.data_ptr(), ws.numel()
        keep += [attn, pos, ws]
    keep += [logits, prev]
    return d, out, keep


def decide_step(logits, prev=None, seq_offsets=None, row_index=None, vocab=None, fast=None,
                depcap=None, cap=None, dapd=None):
    """dlm_decide_step: statistics plus the enabled rules in two launches.
    Arguments and the returned dict as for step_descriptor (see there)."""
    d, out, keep = step_descriptor(logits, prev, seq_offsets, row_index, vocab, fast, depcap, cap,
                                   dapd)
    st = _lib.lib().dlm_decide_step(ctypes.byref(d), _stream(logits))
    _lib.check(st, "dlm_decide_step")
    return out
