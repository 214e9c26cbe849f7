"""CPU oracle for trellis-coded FP4 weights -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path
(``trellis_coded_fp4_amd``) never does.

The arithmetic lives in ``trellis_oracle.c`` (plain C, fp64, sequential);
this module builds it with gcc into ``liboracle.so`` and wraps it with ctypes.
Inputs are NumPy arrays; floating-point inputs are converted to float64,
which holds bf16 and fp32 values exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "trellis_oracle.c")
_LIB = os.environ.get("TRELLIS_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math, no vector ISA flags)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_palette_entry.argtypes = [ctypes.c_int, ctypes.c_int]
        L.oracle_palette_entry.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_code.argtypes = [ctypes.c_double]
        L.oracle_e2m1_code.restype = ctypes.c_int
        L.oracle_ue8m0_scale.argtypes = [ctypes.c_int]
        L.oracle_ue8m0_scale.restype = ctypes.c_double
        L.oracle_state_value.argtypes = [ctypes.c_uint32]
        L.oracle_state_value.restype = ctypes.c_double
        L.oracle_state_code.argtypes = [ctypes.c_uint32]
        L.oracle_state_code.restype = ctypes.c_int
        L.oracle_decode_codes.argtypes = [P, I64, I64, I64, P]
        L.oracle_decode_codes.restype = None
        L.oracle_decode_window.argtypes = [P, I64]
        L.oracle_decode_window.restype = ctypes.c_int
        L.oracle_decode_values.argtypes = [P, P, I64, I64, P]
        L.oracle_decode_values.restype = None
        L.oracle_expand.argtypes = [P, P, I64, I64, I64, P, P]
        L.oracle_expand.restype = None
        L.oracle_gemv.argtypes = [P, P, I64, I64, P, I64, P, P]
        L.oracle_gemv.restype = None
        L.oracle_moe_gemv.argtypes = [P, P, I64, I64, I64, P, ctypes.c_int, P, P, I64, I64, P, P]
        L.oracle_moe_gemv.restype = I64
        L.oracle_round_bf16.argtypes = [ctypes.c_double]
        L.oracle_round_bf16.restype = ctypes.c_double
        L.oracle_swiglu_bf16.argtypes = [P, I64, I64, P]
        L.oracle_swiglu_bf16.restype = None
        L.oracle_moe_ffn.argtypes = [P, P, P, P, I64, I64, I64, P, P, P, I64, I64, P, P, P]
        L.oracle_moe_ffn.restype = I64
        L.oracle_viterbi.argtypes = [P, P, ctypes.c_int, P]
        L.oracle_viterbi.restype = ctypes.c_double
        L.oracle_e5m3_scale.argtypes = [ctypes.c_int]
        L.oracle_e5m3_scale.restype = ctypes.c_double
        L.oracle_decode_values_fmt.argtypes = [P, P, I64, I64, ctypes.c_int, P]
        L.oracle_decode_values_fmt.restype = None
        L.oracle_moe_gemv_fmt.argtypes = [P, P, I64, I64, I64, ctypes.c_int, P, ctypes.c_int, P, P, I64, I64, P, P]
        L.oracle_moe_gemv_fmt.restype = I64
        L.oracle_moe_ffn_fmt.argtypes = [P, P, P, P, I64, I64, I64, ctypes.c_int, P, P, P, I64, I64, P, P, P]
        L.oracle_moe_ffn_fmt.restype = I64
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u32(a):
    return np.ascontiguousarray(a, dtype=np.uint32)


def _u8(a):
    return np.ascontiguousarray(a, dtype=np.uint8)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


# ---- scalar helpers ----

def palette_entry(palette: int, entry: int) -> float:
    return lib().oracle_palette_entry(int(palette), int(entry))



def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def e2m1_code(v: float) -> int:
    return lib().oracle_e2m1_code(float(v))


def ue8m0_scale(e: int) -> float:
    return lib().oracle_ue8m0_scale(int(e))


SCALE_FORMATS = {"ue8m0": 0, "e5m3": 1}


def e5m3_scale(byte: int) -> float:
    """Value of an E5M3 block-scale byte (reading R14 in the C source)."""
    return lib().oracle_e5m3_scale(int(byte))


def state_value(s: int) -> float:
    return lib().oracle_state_value(int(s))


def state_code(s: int) -> int:
    return lib().oracle_state_code(int(s))


def round_bf16(v: float) -> float:
    return lib().oracle_round_bf16(float(v))


# ---- array entry points ----

def decode_codes(syms: np.ndarray, cols: int) -> np.ndarray:
    """syms [..., rows, words_per_row] -> codes [..., rows, cols] (uint8, one per weight)."""
    s = _u32(syms)
    wpr = s.shape[-1]
    rows = int(np.prod(s.shape[:-1]))
    out = np.empty(s.shape[:-1] + (cols,), dtype=np.uint8)
    lib().oracle_decode_codes(_p(s), rows, cols, wpr, _p(out))
    return out


def decode_window(row_words: np.ndarray, k: int) -> int:
    w = _u32(row_words)
    return lib().oracle_decode_window(_p(w), int(k))


def decode_values(syms: np.ndarray, scales: np.ndarray, scale_fmt: str = "ue8m0") -> np.ndarray:
    """Dense fp64 weights [..., rows, cols] from symbols and block scales
    (UE8M0 bytes, or E5M3 bytes with scale_fmt="e5m3")."""
    s, e = _u32(syms), _u8(scales)
    cols = s.shape[-1] * 16
    rows = int(np.prod(s.shape[:-1]))
    out = np.empty(s.shape[:-1] + (cols,), dtype=np.float64)
    if scale_fmt == "ue8m0":
        lib().oracle_decode_values(_p(s), _p(e), rows, cols, _p(out))
    else:
        lib().oracle_decode_values_fmt(_p(s), _p(e), rows, cols, SCALE_FORMATS[scale_fmt], _p(out))
    return out


def expand(syms: np.ndarray, scales: np.ndarray):
    """syms [n_mat, rows, cols/16], scales [n_mat, rows, cols/32] -> (packed [n_mat, rows, cols/2], scales copy)."""
    s, e = _u32(syms), _u8(scales)
    n_mat, rows, wpr = s.shape
    cols = wpr * 16
    packed = np.empty((n_mat, rows, cols // 2), dtype=np.uint8)
    sc = np.empty_like(e)
    lib().oracle_expand(_p(s), _p(e), n_mat, rows, cols, _p(packed), _p(sc))
    return packed, sc


def gemv(syms: np.ndarray, scales: np.ndarray, x: np.ndarray):
    """One matrix [rows, cols/16] with x [nx, cols] -> (y [nx, rows], bound [nx, rows]) fp64."""
    s, e = _u32(syms), _u8(scales)
    rows, wpr = s.shape[-2], s.shape[-1]
    cols = wpr * 16
    xv = _f64(x).reshape(-1, cols)
    nx = xv.shape[0]
    y = np.empty((nx, rows))
    b = np.empty((nx, rows))
    lib().oracle_gemv(_p(s), _p(e), rows, cols, _p(xv), nx, _p(y), _p(b))
    return y, b


def moe_gemv(syms, scales, x, ids, gate_w=None, x_per_slot=False, scale_fmt="ue8m0"):
    """Routed GEMV; returns (y, bound, skipped). See oracle_moe_gemv in the C source."""
    s, e = _u32(syms), _u8(scales)
    n_exp, rows, wpr = s.shape
    cols = wpr * 16
    idv = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = idv.shape
    xv = _f64(x).reshape((T, k, cols) if x_per_slot else (T, cols))
    gw = None if gate_w is None else _f64(gate_w).reshape(T, k)
    shape = (T, rows) if gw is not None else (T, k, rows)
    y = np.empty(shape)
    b = np.empty(shape)
    if scale_fmt == "ue8m0":
        skipped = lib().oracle_moe_gemv(_p(s), _p(e), n_exp, rows, cols, _p(xv), int(bool(x_per_slot)),
                                        _p(idv), _p(gw), T, k, _p(y), _p(b))
    else:
        skipped = lib().oracle_moe_gemv_fmt(_p(s), _p(e), n_exp, rows, cols, SCALE_FORMATS[scale_fmt], _p(xv),
                                            int(bool(x_per_slot)), _p(idv), _p(gw), T, k, _p(y), _p(b))
    return y, b, int(skipped)


def swiglu_bf16(y_gu: np.ndarray, inter: int) -> np.ndarray:
    yv = _f64(y_gu).reshape(-1, 2 * inter)
    h = np.empty((yv.shape[0], inter))
    lib().oracle_swiglu_bf16(_p(yv), yv.shape[0], inter, _p(h))
    return h.reshape(y_gu.shape[:-1] + (inter,))


def moe_ffn(gu_syms, gu_scales, dn_syms, dn_scales, x, ids, gate_w, scale_fmt="ue8m0"):
    """Whole MoE layer; returns (y [T,H], bound [T,H], h [T,k,I], skipped).
    scale_fmt: both stacks' scale bytes as "ue8m0" or "e5m3"."""
    gs, ge, ds, de = _u32(gu_syms), _u8(gu_scales), _u32(dn_syms), _u8(dn_scales)
    n_exp, two_i, wpr = gs.shape
    hidden = wpr * 16
    inter = two_i // 2
    idv = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = idv.shape
    xv = _f64(x).reshape(T, hidden)
    gw = _f64(gate_w).reshape(T, k)
    h = np.empty((T, k, inter))
    y = np.empty((T, hidden))
    b = np.empty((T, hidden))
    skipped = lib().oracle_moe_ffn_fmt(_p(gs), _p(ge), _p(ds), _p(de), n_exp, hidden, inter,
                                       SCALE_FORMATS[scale_fmt], _p(xv), _p(idv), _p(gw), T, k, _p(h), _p(y), _p(b))
    return y, b, h, int(skipped)


def viterbi(target: np.ndarray, d: Optional[np.ndarray] = None):
    """Minimum-distortion symbol sequence for one row; returns (symbols uint8 [n], cost)."""
    t = _f64(target)
    n = t.shape[0]
    dv = _f64(np.ones(n) if d is None else d)
    out = np.empty(n, dtype=np.uint8)
    cost = lib().oracle_viterbi(_p(t), _p(dv), n, _p(out))
    return out, float(cost)


def router_topk(x: np.ndarray, w_router: np.ndarray, k: int):
    """Router in front of the layer: logits, top-k, gate weights.

    The pages leave routing unspecified; the reading taken is the usual
    mixture-of-experts router: logits[t, e] = sum_h x[t, h] * W_r[e, h] in
    float64 (a matmul of the exact float64 images of the inputs), the k
    largest logits of each token in descending order with ties going to the
    lower expert id, and gate weights = softmax over those k logits
    (float64: exp(l - l_max) / sum). Returns (ids int32 [T, k], gate weights
    float64 [T, k], logits float64 [T, E]).
    """
    xv = _f64(np.atleast_2d(x))
    wv = _f64(w_router)
    logits = xv @ wv.T
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    gw = np.empty((T, k))
    for t in range(T):
        picked = sorted(range(E), key=lambda e: (-logits[t, e], e))[:k]
        ids[t] = picked
        sel = logits[t, picked]
        ex = np.exp(sel - sel[0])
        gw[t] = ex / ex.sum()
    return ids, gw, logits
