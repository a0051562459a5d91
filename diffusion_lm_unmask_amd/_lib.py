"""ctypes loader for libdlm.so — the C ABI declared in include/dlm.h.

No fallback: if the library is missing this raises.  Build it with
``python -m diffusion_lm_unmask_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdlm.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "dlm.h")

OK, ERR_ARG, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3
BF16, F32 = 0, 1

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_D = ctypes.c_double
_INT = ctypes.c_int
_SZ = ctypes.c_size_t

SIGNATURES = {
    "dlm_step_stats": (_INT, [_P, _P, _INT, _I64, _I64, _P, _I64, _P, _P, _P, _P, _P, _P, _SZ,
                              _P]),
    "dlm_step_stats_workspace_bytes": (_SZ, [_I64]),
    "dlm_fastdllm_select": (_INT, [_P, _P, _P, _I32, _F, _P, _P, _P]),
    "dlm_depcap_boundary": (_INT, [_P, _P, _P, _I32, _P, _D, _I32, _I32, _I32, _D, _P, _P, _P]),
    "dlm_cap_select": (_INT, [_P, _INT, _I64, _I64, _P, _P, _I32, _P, _P, _P, _P, _F, _F, _F,
                              _I32, _P, _P, _P, _P, _P]),
    "dlm_dapd_workspace_bytes": (_SZ, [_I32, _I32]),
    "dlm_dapd_select": (_INT, [_P, _INT, _I32, _I64, _I64, _P, _P, _I32, _I32, _P, _F, _P, _P, _P,
                               _P, _P, _P, _SZ, _P]),
    "dlm_dapd_select_static": (_INT, [_P, _INT, _I32, _I64, _I64, _P, _P, _I32, _I32, _P, _F, _P,
                                      _P, _P, _P, _P, _P]),
    "dlm_dapd_step": (_INT, [_P, _INT, _I32, _I64, _I64, _P, _P, _I32, _I32, _P, _F, _P, _F, _F,
                             _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "dlm_factor_select": (_INT, [_P, _P, _P, _I32, _F, _P, _P, _P, _P]),
    "dlm_topk_select": (_INT, [_P, _P, _P, _I32, _I32, _P, _P, _P]),
    "dlm_fixed_block_eligible": (_INT, [_P, _P, _I32, _P, _I32, _P, _P]),
    "dlm_decide_step": (_INT, [_P, _P]),
    "dlm_status_string": (ctypes.c_char_p, [_INT]),
}


class StepDesc(ctypes.Structure):
    """ctypes mirror of `dlm_step_desc` (include/dlm.h), field for field."""
    _fields_ = [
        ("logits", _P), ("prev_logits", _P), ("dtype", _I32), ("vocab", _I64), ("ld", _I64),
        ("row_index", _P), ("n_rows", _I64), ("conf", _P), ("argmax", _P), ("entropy", _P),
        ("kl", _P), ("lse", _P), ("seq_offsets", _P), ("n_seq", _I32),
        ("fast_eligible", _P), ("fast_tau", _F), ("fast_commit", _P), ("fast_n_commit", _P),
        ("depcap_has_prev", _P), ("depcap_lambda", _D), ("depcap_l_min", _I32),
        ("depcap_l_max", _I32), ("depcap_radius", _I32), ("depcap_eps", _D),
        ("depcap_block_len", _P), ("depcap_score", _P),
        ("cap_eligible", _P), ("cap_tau_low", _F), ("cap_tau_high", _F), ("cap_gamma", _F),
        ("cap_k_max", _I32), ("cap_commit", _P), ("cap_n_commit", _P),
        ("attn", _P), ("attn_dtype", _I32), ("n_lh", _I32), ("S", _I64), ("batch_stride", _I64),
        ("masked_pos", _P), ("m_max", _I32), ("dapd_tau", _F), ("dapd_commit", _P),
        ("dapd_n_commit", _P), ("dapd_workspace", _P), ("dapd_workspace_bytes", _SZ),
        ("launch1_begin_event", _P), ("launch1_end_event", _P),
    ]


class DLMError(RuntimeError):
    pass


_lib = None


def header_symbols() -> list[str]:
    """Function names declared in include/dlm.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(dlm_\w+)\s*\(", text,
                                 re.M)))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise DLMError(f"{LIB_PATH} is not built: run `python -m diffusion_lm_unmask_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int, name: str) -> None:
    if status != OK:
        msg = lib().dlm_status_string(status).decode()
        raise DLMError(f"{name} failed with status {status}: {msg}")
