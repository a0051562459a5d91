"""fp64 CPU oracle for the per-step unmask decision — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding in ``diffusion_lm_unmask_amd``) never imports it and shares no code
with it.

The arithmetic lives in ``dlm_oracle.c`` (plain C11, IEEE double); this module
only marshals torch CPU tensors / numpy arrays into that library via ctypes.
Each wrapper names the C function it calls; the C file cites the passages of
the pages each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dlm_oracle.c")
# DLM_ORACLE_SANITIZED=1 selects the AddressSanitizer + UndefinedBehaviorSanitizer
# build (tests only; the process must preload the sanitizer runtimes)
_SANITIZED = os.environ.get("DLM_ORACLE_SANITIZED") == "1"
_LIB_PATH = os.path.join(_HERE, "liboracle_san.so" if _SANITIZED else "liboracle.so")

BF16 = 0
F32 = 1

_FLAGS = ["-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]
SANITIZE_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer"]


def build(force: bool = True, sanitized: bool | None = None) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, no FP contraction);
    `sanitized` builds the ASan + UBSan variant instead."""
    san = _SANITIZED if sanitized is None else sanitized
    path = os.path.join(_HERE, "liboracle_san.so" if san else "liboracle.so")
    if force or not os.path.exists(path):
        tmp = path + ".tmp%d" % os.getpid()
        opt = SANITIZE_FLAGS if san else ["-O2"]
        cmd = ["gcc", *opt, *_FLAGS, _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, path)
    return path


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_D = ctypes.c_double
_INT = ctypes.c_int


def _declare(L):
    L.dlmo_step_stats.argtypes = [_P, _P, _INT, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _INT]
    L.dlmo_fastdllm_select.argtypes = [_P, _P, _P, _I32, _D, _P, _P]
    L.dlmo_depcap_scores.argtypes = [_P, _P, _P, _I32, _I32, _P, _D, _I32, _D, _P]
    L.dlmo_depcap_decide.argtypes = [_P, _P, _I32, _I32, _P, _I32, _P]
    L.dlmo_cap_pool.argtypes = [_P, _P, _I32, _D, _I32, _P, _P, _P]
    L.dlmo_cap_dmatrix.argtypes = [_P, _INT, _I64, _I64, _P, _P, _P, _P, _I32, _P, _I32]
    L.dlmo_cap_greedy.argtypes = [_P, _P, _I32, _I32, _D, _D, _P]
    L.dlmo_cap_select.argtypes = [_P, _INT, _I64, _I64, _P, _P, _I32, _P, _P, _P, _P, _D, _D,
                                  _D, _I32, _P, _P, _P, _P, _INT]
    L.dlmo_dapd_average.argtypes = [_P, _INT, _I32, _I64, _P, _I32, _P]
    L.dlmo_dapd_graph.argtypes = [_P, _I32, _P, _P, _P, _P]
    L.dlmo_dapd_greedy.argtypes = [_P, _I32, _I64, _D, _P, _P]
    L.dlmo_dapd_select.argtypes = [_P, _INT, _I32, _I64, _I64, _P, _P, _I32, _P, _D, _P, _P, _P,
                                   _P, _I32, _P, _INT]
    L.dlmo_topk_select.argtypes = [_P, _P, _P, _I32, _I32, _P, _P]
    L.dlmo_factor_select.argtypes = [_P, _P, _P, _I32, _D, _P, _P, _P]
    L.dlmo_fixed_block_eligible.argtypes = [_P, _P, _I32, _P, _I32, _P]
    L.dlmo_dapd_step.argtypes = [_P, _INT, _I32, _I64, _I64, _P, _P, _I32, _P, _D, _P, _D, _D,
                                 _INT, _P, _P, _P, _INT]
    for name in ("dlmo_step_stats", "dlmo_fastdllm_select", "dlmo_depcap_scores",
                 "dlmo_depcap_decide", "dlmo_cap_pool", "dlmo_cap_dmatrix", "dlmo_cap_greedy",
                 "dlmo_cap_select", "dlmo_dapd_average", "dlmo_dapd_graph", "dlmo_dapd_greedy",
                 "dlmo_dapd_select", "dlmo_topk_select", "dlmo_factor_select",
                 "dlmo_fixed_block_eligible", "dlmo_dapd_step"):
        getattr(L, name).restype = _INT


# ------------------------------------------------------------------ marshal

def _host(t):
    """Contiguous CPU torch tensor or numpy array -> (keepalive, pointer)."""
    if t is None:
        return None, None
    if isinstance(t, torch.Tensor):
        t = t.detach()
        if t.device.type != "cpu":
            raise ValueError("oracle takes host tensors only")
        t = t.contiguous()
        return t, t.data_ptr()
    a = np.ascontiguousarray(t)
    return a, a.ctypes.data


def _f64(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i32(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _i64(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _u8(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.uint8))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported logits dtype {t.dtype}")


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: bad argument (oracle status {rc})")


# ------------------------------------------------------------------- calls

def step_stats(logits: torch.Tensor, prev: torch.Tensor | None = None, row_index=None,
               vocab: int | None = None, n_threads: int | None = None):
    """dlmo_step_stats over a 2-D [rows, ld] CPU tensor.  Returns a dict of
    numpy arrays: conf, argmax, entropy, kl (None without prev), lse."""
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D [rows, ld]")
    ld = logits.shape[1]
    vocab = ld if vocab is None else vocab
    if row_index is None:
        row_index = np.arange(logits.shape[0], dtype=np.int64)
    ri = _i64(row_index)
    n = ri.shape[0]
    lt, lp = _host(logits)
    if prev is not None:
        if prev.dtype != logits.dtype or prev.shape != logits.shape:
            raise ValueError("prev must match logits")
        pt, pp = _host(prev)
    else:
        pt, pp = None, None
    conf = np.empty(n, np.float64)
    arg = np.empty(n, np.int32)
    ent = np.empty(n, np.float64)
    kl = np.empty(n, np.float64) if prev is not None else None
    lse = np.empty(n, np.float64)
    rc = lib().dlmo_step_stats(lp, pp, _dtype_code(logits), vocab, ld, _ptr(ri), n, _ptr(conf),
                               _ptr(arg), _ptr(ent), _ptr(kl), _ptr(lse),
                               n_threads or default_threads())
    _check(rc, "step_stats")
    return {"conf": conf, "argmax": arg, "entropy": ent, "kl": kl, "lse": lse}


def fastdllm_select(conf, seq_offsets, tau, eligible=None):
    c = _f64(conf)
    so = _i32(seq_offsets)
    el = _u8(eligible)
    n_seq = so.shape[0] - 1
    commit = np.zeros(c.shape[0], np.uint8)
    n_commit = np.zeros(max(n_seq, 0), np.int32)
    rc = lib().dlmo_fastdllm_select(_ptr(c), _ptr(el), _ptr(so), n_seq, float(tau),
                                    _ptr(commit), _ptr(n_commit))
    _check(rc, "fastdllm_select")
    return commit, n_commit


def depcap_scores(kl, entropy, seq_offsets, l_max, lam, radius=1, eps=1e-12, has_prev=None):
    k = _f64(kl)
    h = _f64(entropy)
    so = _i32(seq_offsets)
    hp = _u8(has_prev)
    n_seq = so.shape[0] - 1
    score = np.empty(k.shape[0], np.float64)
    rc = lib().dlmo_depcap_scores(_ptr(k), _ptr(h), _ptr(so), n_seq, int(l_max), _ptr(hp),
                                  float(lam), int(radius), float(eps), _ptr(score))
    _check(rc, "depcap_scores")
    return score


def depcap_decide(score, seq_offsets, l_max, l_min, has_prev=None):
    s = _f64(score)
    so = _i32(seq_offsets)
    hp = _u8(has_prev)
    n_seq = so.shape[0] - 1
    out = np.zeros(max(n_seq, 0), np.int32)
    rc = lib().dlmo_depcap_decide(_ptr(s), _ptr(so), n_seq, int(l_max), _ptr(hp), int(l_min),
                                  _ptr(out))
    _check(rc, "depcap_decide")
    return out


def depcap_boundary(kl, entropy, seq_offsets, l_max, l_min, lam, radius=1, eps=1e-12,
                    has_prev=None):
    score = depcap_scores(kl, entropy, seq_offsets, l_max, lam, radius, eps, has_prev)
    return depcap_decide(score, seq_offsets, l_max, l_min, has_prev), score


def cap_pool(conf, tau_low, k_max, eligible=None):
    c = _f64(conf)
    el = _u8(eligible)
    cand = np.zeros(max(int(k_max), 1), np.int32)
    nc = np.zeros(1, np.int32)
    fb = np.zeros(1, np.int32)
    rc = lib().dlmo_cap_pool(_ptr(c), _ptr(el), c.shape[0], float(tau_low), int(k_max),
                             _ptr(cand), _ptr(nc), _ptr(fb))
    _check(rc, "cap_pool")
    return cand[: nc[0]].copy(), int(fb[0])


def cap_greedy(cand_conf, D, tau_high, gamma):
    cc = _f64(cand_conf)
    Dm = _f64(D)
    n = cc.shape[0]
    if Dm.ndim != 2 or Dm.shape[0] < n or Dm.shape[1] < n:
        raise ValueError("D must be at least [n, n]")
    take = np.zeros(max(n, 1), np.uint8)
    rc = lib().dlmo_cap_greedy(_ptr(cc), _ptr(Dm), Dm.shape[1], n, float(tau_high),
                               float(gamma), _ptr(take))
    _check(rc, "cap_greedy")
    return take[:n].copy()


def cap_dmatrix(logits: torch.Tensor, row_index, argmax, lse, cand_rows, vocab=None):
    ld = logits.shape[1]
    vocab = ld if vocab is None else vocab
    lt, lp = _host(logits)
    ri, am, ls, cr = _i64(row_index), _i32(argmax), _f64(lse), _i32(cand_rows)
    n = cr.shape[0]
    D = np.empty((max(n, 1), max(n, 1)), np.float64)
    rc = lib().dlmo_cap_dmatrix(lp, _dtype_code(logits), vocab, ld, _ptr(ri), _ptr(am),
                                _ptr(ls), _ptr(cr), n, _ptr(D), max(n, 1))
    _check(rc, "cap_dmatrix")
    return D[:n, :n].copy()


def cap_select(logits: torch.Tensor, row_index, seq_offsets, conf, argmax, lse, tau_low,
               tau_high, gamma, k_max, eligible=None, vocab=None, n_threads=None):
    ld = logits.shape[1]
    vocab = ld if vocab is None else vocab
    lt, lp = _host(logits)
    ri, so = _i64(row_index), _i32(seq_offsets)
    c, am, ls, el = _f64(conf), _i32(argmax), _f64(lse), _u8(eligible)
    n_seq = so.shape[0] - 1
    commit = np.zeros(c.shape[0], np.uint8)
    n_commit = np.zeros(max(n_seq, 0), np.int32)
    cand = np.full(max(n_seq, 0) * int(k_max), -1, np.int32)
    dmat = np.full(max(n_seq, 0) * int(k_max) * int(k_max), np.nan, np.float64)
    rc = lib().dlmo_cap_select(lp, _dtype_code(logits), vocab, ld, _ptr(ri), _ptr(so), n_seq,
                               _ptr(c), _ptr(am), _ptr(ls), _ptr(el), float(tau_low),
                               float(tau_high), float(gamma), int(k_max), _ptr(commit),
                               _ptr(n_commit), _ptr(cand), _ptr(dmat),
                               n_threads or default_threads())
    _check(rc, "cap_select")
    return {"commit": commit, "n_commit": n_commit,
            "cand": cand.reshape(max(n_seq, 0), int(k_max)),
            "dmat": dmat.reshape(max(n_seq, 0), int(k_max), int(k_max))}


def dapd_average(attn_maps: torch.Tensor, pos):
    """attn_maps: [n_lh, S, S] CPU tensor of one sequence."""
    n_lh, S, S2 = attn_maps.shape
    if S != S2:
        raise ValueError("maps must be square")
    at, ap = _host(attn_maps)
    p = _i32(pos)
    M = p.shape[0]
    a = np.empty((max(M, 1), max(M, 1)), np.float64)
    rc = lib().dlmo_dapd_average(ap, _dtype_code(attn_maps), n_lh, S, _ptr(p), M, _ptr(a))
    _check(rc, "dapd_average")
    return a[:M, :M].copy()


def dapd_graph(a, conf):
    am = _f64(a)
    c = _f64(conf)
    M = c.shape[0]
    s = np.empty((M, M), np.float64)
    deg = np.empty(M, np.float64)
    key = np.empty(M, np.float64)
    rc = lib().dlmo_dapd_graph(_ptr(am), M, _ptr(c), _ptr(s), _ptr(deg), _ptr(key))
    _check(rc, "dapd_graph")
    return s, deg, key


def dapd_greedy(s, tau, key):
    sm = _f64(s)
    k = _f64(key)
    M = k.shape[0]
    take = np.zeros(max(M, 1), np.uint8)
    rc = lib().dlmo_dapd_greedy(_ptr(sm), M, sm.shape[1] if sm.ndim == 2 else M, float(tau),
                                _ptr(k), _ptr(take))
    _check(rc, "dapd_greedy")
    return take[:M].copy()


def dapd_select(attn: torch.Tensor, masked_pos, seq_offsets, conf, tau, m_max=None,
                n_threads=None):
    """attn: [B, n_lh, S, S] CPU tensor.  Returns commit, n_commit, degree,
    key (per row) and sym [B, m_max, m_max]."""
    B, n_lh, S, S2 = attn.shape
    at, ap = _host(attn)
    mp, so, c = _i32(masked_pos), _i32(seq_offsets), _f64(conf)
    n_seq = so.shape[0] - 1
    if n_seq > B:
        raise ValueError("more sequences than attention batches")
    if m_max is None:
        m_max = int(np.max(np.diff(so))) if n_seq > 0 else 1
    n = c.shape[0]
    commit = np.zeros(n, np.uint8)
    n_commit = np.zeros(max(n_seq, 0), np.int32)
    degree = np.empty(n, np.float64)
    key = np.empty(n, np.float64)
    sym = np.empty(max(n_seq, 0) * m_max * m_max, np.float64)
    rc = lib().dlmo_dapd_select(ap, _dtype_code(attn), n_lh, S, n_lh * S * S, _ptr(mp), _ptr(so),
                                n_seq, _ptr(c), float(tau), _ptr(commit), _ptr(n_commit),
                                _ptr(degree), _ptr(sym), int(m_max), _ptr(key),
                                n_threads or default_threads())
    _check(rc, "dapd_select")
    return {"commit": commit, "n_commit": n_commit, "degree": degree, "key": key,
            "sym": sym.reshape(max(n_seq, 0), m_max, m_max)}


def topk_select(conf, seq_offsets, k, eligible=None):
    """dlmo_topk_select: the k most confident eligible rows per sequence."""
    c, so, el = _f64(conf), _i32(seq_offsets), _u8(eligible)
    n_seq = so.shape[0] - 1
    commit = np.zeros(c.shape[0], np.uint8)
    n_commit = np.zeros(max(n_seq, 0), np.int32)
    rc = lib().dlmo_topk_select(_ptr(c), _ptr(el), _ptr(so), n_seq, int(k), _ptr(commit),
                                _ptr(n_commit))
    _check(rc, "topk_select")
    return commit, n_commit


def factor_select(conf, seq_offsets, f=1.0, eligible=None):
    """dlmo_factor_select: returns commit, n_commit and the Theorem-1 certificate."""
    c, so, el = _f64(conf), _i32(seq_offsets), _u8(eligible)
    n_seq = so.shape[0] - 1
    commit = np.zeros(c.shape[0], np.uint8)
    n_commit = np.zeros(max(n_seq, 0), np.int32)
    cert = np.zeros(max(n_seq, 0), np.uint8)
    rc = lib().dlmo_factor_select(_ptr(c), _ptr(el), _ptr(so), n_seq, float(f), _ptr(commit),
                                  _ptr(n_commit), _ptr(cert))
    _check(rc, "factor_select")
    return commit, n_commit, cert


def fixed_block_eligible(masked_pos, seq_offsets, block_len, gen_start=None):
    """dlmo_fixed_block_eligible: masked rows of each sequence's active fixed block."""
    mp, so = _i32(masked_pos), _i32(seq_offsets)
    gs = None if gen_start is None else _i32(gen_start)
    n_seq = so.shape[0] - 1
    el = np.zeros(mp.shape[0], np.uint8)
    rc = lib().dlmo_fixed_block_eligible(_ptr(mp), _ptr(so), n_seq, _ptr(gs), int(block_len),
                                         _ptr(el))
    _check(rc, "fixed_block_eligible")
    return el


def dapd_step(attn: torch.Tensor, masked_pos, seq_offsets, conf, tau, gen_len=None,
              late_frac=0.5, late_tau=0.9, pre_unmask=True, n_threads=None):
    """dlmo_dapd_step: returns commit, n_commit and the per-sequence stage (1 = late)."""
    B, n_lh, S, S2 = attn.shape
    at, ap = _host(attn)
    mp, so, c = _i32(masked_pos), _i32(seq_offsets), _f64(conf)
    gl = None if gen_len is None else _i32(gen_len)
    n_seq = so.shape[0] - 1
    if n_seq > B:
        raise ValueError("more sequences than attention batches")
    commit = np.zeros(c.shape[0], np.uint8)
    n_commit = np.zeros(max(n_seq, 0), np.int32)
    stage = np.zeros(max(n_seq, 0), np.uint8)
    rc = lib().dlmo_dapd_step(ap, _dtype_code(attn), n_lh, S, n_lh * S * S, _ptr(mp), _ptr(so),
                              n_seq, _ptr(c), float(tau), _ptr(gl), float(late_frac),
                              float(late_tau), int(bool(pre_unmask)), _ptr(commit),
                              _ptr(n_commit), _ptr(stage), n_threads or default_threads())
    _check(rc, "dapd_step")
    return {"commit": commit, "n_commit": n_commit, "stage": stage}
