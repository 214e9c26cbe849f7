"""trellis_coded_fp4_amd -- trellis-coded FP4 (MXFP4-grid) weights on MI355X.

Thin ctypes binding of libtrellis.so (HIP kernels for gfx950 behind the C ABI
declared in include/trellis.h). This module only marshals arguments: every
step of decoding and multiplication runs in the library's kernels. PyTorch
supplies device memory and the current HIP stream.

If the library has not been built, importing works but every call raises:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtrellis.so")

TRELLIS_F32 = 0
TRELLIS_BF16 = 1

ERRORS = {0: "TRELLIS_OK", -1: "TRELLIS_EINVAL", -2: "TRELLIS_ENULL", -3: "TRELLIS_EWORKSPACE",
          -4: "TRELLIS_EHIP", -5: "TRELLIS_EDEVICE"}

# Every symbol include/trellis.h declares.
EXPORTS = ["trellis_version", "trellis_strerror", "trellis_decode_expand",
           "trellis_moe_gemv_workspace_size", "trellis_moe_gemv_workspace", "trellis_moe_gemv",
           "trellis_moe_ffn_workspace_size", "trellis_moe_ffn", "trellis_moe_ffn_timed",
           "trellis_moe_ffn_noalloc", "trellis_moe_ffn_routed",
           "trellis_mxfp4_moe_gemv", "trellis_mxfp4_moe_ffn", "trellis_moe_gemv_e5m3", "trellis_moe_ffn_e5m3",
           "trellis_viterbi_workspace_size", "trellis_viterbi_encode", "trellis_router_workspace_size",
           "trellis_router_topk", "trellis_read_bandwidth"]


class TrellisError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {ERRORS.get(code, code)} ({strerror(code)})")


class Mat(ctypes.Structure):
    """trellis_mat_t"""
    _fields_ = [("syms", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("n_mat", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class MxMat(ctypes.Structure):
    """trellis_mx_t"""
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("n_mat", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libtrellis.so (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libtrellis.so not built at {LIB_PATH}; run "
                               "`python -m trellis_coded_fp4_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        MP = ctypes.POINTER(Mat)
        L.trellis_version.argtypes = []
        L.trellis_version.restype = ctypes.c_int
        L.trellis_strerror.argtypes = [ctypes.c_int]
        L.trellis_strerror.restype = ctypes.c_char_p
        L.trellis_decode_expand.argtypes = [P, MP, P, P]
        L.trellis_decode_expand.restype = ctypes.c_int
        L.trellis_moe_gemv_workspace_size.argtypes = [I32] * 5
        L.trellis_moe_gemv_workspace_size.restype = SZ
        L.trellis_moe_gemv_workspace.argtypes = [MP, I32, I32]
        L.trellis_moe_gemv_workspace.restype = SZ
        L.trellis_moe_gemv.argtypes = [P, MP, P, I32, I32, P, P, I32, I32, P, P, SZ]
        L.trellis_moe_gemv.restype = ctypes.c_int
        L.trellis_moe_ffn_workspace_size.argtypes = [I32] * 5
        L.trellis_moe_ffn_workspace_size.restype = SZ
        L.trellis_moe_ffn.argtypes = [P, MP, MP, P, I32, P, P, I32, I32, P, P, P, SZ]
        L.trellis_moe_ffn.restype = ctypes.c_int
        L.trellis_moe_ffn_timed.argtypes = [P, MP, MP, P, I32, P, P, I32, I32, P, P, P, SZ, P]
        L.trellis_moe_ffn_timed.restype = ctypes.c_int
        L.trellis_moe_ffn_routed.argtypes = [P, MP, MP, P, I32, P, I32, P, P, P, P, P, SZ, P]
        L.trellis_moe_ffn_routed.restype = ctypes.c_int
        L.trellis_moe_ffn_noalloc.argtypes = [P, MP, MP, P, I32, P, P, I32, I32, P, P]
        L.trellis_moe_ffn_noalloc.restype = ctypes.c_int
        L.trellis_moe_gemv_e5m3.argtypes = [P, MP, P, I32, I32, P, P, I32, I32, P, P, SZ]
        L.trellis_moe_gemv_e5m3.restype = ctypes.c_int
        L.trellis_moe_ffn_e5m3.argtypes = [P, MP, MP, P, I32, P, P, I32, I32, P, P, P, SZ]
        L.trellis_moe_ffn_e5m3.restype = ctypes.c_int
        XP = ctypes.POINTER(MxMat)
        L.trellis_mxfp4_moe_gemv.argtypes = [P, XP, P, I32, I32, P, P, I32, I32, P, P, SZ]
        L.trellis_mxfp4_moe_gemv.restype = ctypes.c_int
        L.trellis_mxfp4_moe_ffn.argtypes = [P, XP, XP, P, I32, P, P, I32, I32, P, P, P, SZ]
        L.trellis_mxfp4_moe_ffn.restype = ctypes.c_int
        L.trellis_viterbi_workspace_size.argtypes = [I32, I32]
        L.trellis_viterbi_workspace_size.restype = SZ
        L.trellis_viterbi_encode.argtypes = [P, P, P, I32, I32, P, P, P, SZ]
        L.trellis_viterbi_encode.restype = ctypes.c_int
        L.trellis_router_workspace_size.argtypes = [I32, I32]
        L.trellis_router_workspace_size.restype = SZ
        L.trellis_router_topk.argtypes = [P, P, I32, P, I32, I32, I32, I32, P, P, P, SZ]
        L.trellis_router_topk.restype = ctypes.c_int
        L.trellis_read_bandwidth.argtypes = [P, P, SZ, P]
        L.trellis_read_bandwidth.restype = ctypes.c_int
        _lib = L
    return _lib


def version() -> int:
    return lib().trellis_version()


def strerror(code: int) -> str:
    return lib().trellis_strerror(int(code)).decode()


# ---------------------------------------------------------------- torch helpers

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _on(stream):
    """Context in which temporaries are allocated (and zero-filled) on the
    stream the call is enqueued on, so that they are ordered before it and
    the caching allocator keeps them for that stream."""
    torch = _torch()
    if stream is None:
        import contextlib
        return contextlib.nullcontext()
    return torch.cuda.stream(stream)


class WorkspaceError(RuntimeError):
    """A call on this workspace found a wait that timed out (its status word
    is set); its outputs are NaN until the workspace is zero-filled again."""


def check_workspace(workspace, stream=None):
    """Synchronise `stream` (default: current) and raise WorkspaceError if a
    wait of a call on `workspace` timed out. Returns the number of routing
    slots the last call skipped (expert id >= n_mat)."""
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    s.synchronize()
    words = workspace[:8].view(torch.int32).cpu()
    if int(words[1]) != 0:
        raise WorkspaceError("a wait timed out in a call on this workspace (other work kept the kernel's "
                             "workgroups from being resident); zero-fill the workspace before reusing it")
    return int(words[0])


def _check(t, dtype, name, shape=None):
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


class Call:
    """One library call with its arguments marshalled ahead of time.

    ``fn(..., prepare=True)`` runs every check and builds the ctypes arguments
    once and returns a Call instead of launching; ``call()`` then only enters
    the C function (for loops that launch the same shapes many times).
    ``result`` is what the eager function returns (the output tensors)."""

    __slots__ = ("fn", "args", "name", "result", "keep")

    def __init__(self, fn, args, name, result, keep):
        self.fn, self.args, self.name, self.result, self.keep = fn, args, name, result, keep

    def __call__(self):
        rc = self.fn(*self.args)
        if rc:
            raise TrellisError(rc, self.name)
        return self.result


def _run(prepare, fn, args, name, result, keep=(), check=None, stream=None):
    """Enqueue the call (or return it prepared). ``check``: a workspace whose
    status word is read after the call (synchronising ``stream``);
    WorkspaceError is raised if a wait of the call timed out."""
    c = Call(fn, args, name, result, keep)
    if prepare:
        if check is not None:
            raise ValueError("check=True needs an eager call (prepare=False)")
        return c
    out = c()
    if check is not None:
        check_workspace(check, stream)
    return out


def mat(syms, scales) -> Mat:
    """trellis_mat_t for syms [n_mat, rows, cols/16] int32/uint32 and scales [n_mat, rows, cols/32] uint8."""
    torch = _torch()
    if syms.dim() == 2:
        syms = syms.unsqueeze(0)
    if scales.dim() == 2:
        scales = scales.unsqueeze(0)
    if syms.dtype not in (torch.int32, torch.uint32):
        raise ValueError("syms must be int32/uint32 words")
    _check(syms, syms.dtype, "syms")
    n_mat, rows, wpr = syms.shape
    _check(scales, torch.uint8, "scales", (n_mat, rows, wpr // 2))
    return Mat(syms.data_ptr(), scales.data_ptr(), n_mat, rows, wpr * 16)


def decode_expand(syms, scales, codes_out=None, scales_out=None, stream=None, prepare=False):
    """Expand to resident MXFP4: returns (codes [n_mat, rows, cols/2] uint8, scales copy)."""
    torch = _torch()
    m = mat(syms, scales)
    with _on(stream):
        if codes_out is None:
            codes_out = torch.empty((m.n_mat, m.rows, m.cols // 2), dtype=torch.uint8, device=syms.device)
        if scales_out is None:
            scales_out = torch.empty((m.n_mat, m.rows, m.cols // 32), dtype=torch.uint8, device=syms.device)
    _check(codes_out, torch.uint8, "codes_out", (m.n_mat, m.rows, m.cols // 2))
    _check(scales_out, torch.uint8, "scales_out", (m.n_mat, m.rows, m.cols // 32))
    return _run(prepare, lib().trellis_decode_expand,
                (_stream(stream), ctypes.byref(m), codes_out.data_ptr(), scales_out.data_ptr()),
                "trellis_decode_expand", (codes_out, scales_out), (m,))


def _x_dtype(x):
    torch = _torch()
    if x.dtype == torch.float32:
        return TRELLIS_F32
    if x.dtype == torch.bfloat16:
        return TRELLIS_BF16
    raise ValueError("x must be float32 or bfloat16")


def gemv_workspace(n_mat, rows, cols, T, k, device="cuda"):
    """A zero-filled workspace for trellis_moe_gemv (current stream)."""
    torch = _torch()
    n = lib().trellis_moe_gemv_workspace_size(n_mat, rows, cols, T, k)
    if n == 0:
        raise TrellisError(-1, "trellis_moe_gemv_workspace_size")
    return torch.zeros(n, dtype=torch.uint8, device=device)   # zero-filled before first use


def ffn_workspace(n_exp, hidden, inter, T, k, device="cuda"):
    """A zero-filled workspace for trellis_moe_ffn (current stream)."""
    torch = _torch()
    n = lib().trellis_moe_ffn_workspace_size(n_exp, hidden, inter, T, k)
    if n == 0:
        raise TrellisError(-1, "trellis_moe_ffn_workspace_size")
    return torch.zeros(n, dtype=torch.uint8, device=device)   # zero-filled before first use


def moe_gemv(syms, scales, x, topk_ids, topk_w=None, x_per_slot=False, y=None, workspace=None,
             stream=None, prepare=False, check=False):
    """Routed fused-decode GEMV. y is [T, k, rows] without topk_w, [T, rows] with it.

    check=True synchronises the stream after the call and raises
    WorkspaceError if a wait timed out (the workspace's sticky status word)."""
    return _moe_gemv("trellis_moe_gemv", syms, scales, x, topk_ids, topk_w, x_per_slot, y, workspace, stream,
                     prepare, check)


def moe_gemv_e5m3(syms, scales, x, topk_ids, topk_w=None, x_per_slot=False, y=None, workspace=None,
                  stream=None, prepare=False, check=False):
    """moe_gemv with the scale bytes read as E5M3 (trellis_moe_gemv_e5m3)."""
    return _moe_gemv("trellis_moe_gemv_e5m3", syms, scales, x, topk_ids, topk_w, x_per_slot, y, workspace,
                     stream, prepare, check)


def _moe_gemv(entry, syms, scales, x, topk_ids, topk_w, x_per_slot, y, workspace, stream, prepare, check):
    torch = _torch()
    m = mat(syms, scales)
    T, k = topk_ids.shape
    _check(topk_ids, torch.int32, "topk_ids")
    if topk_w is not None:
        _check(topk_w, torch.float32, "topk_w", (T, k))
    _check(x, x.dtype, "x", (T, k, m.cols) if x_per_slot else (T, m.cols))
    shape = (T, m.rows) if topk_w is not None else (T, k, m.rows)
    with _on(stream):
        if y is None:
            y = torch.empty(shape, dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = gemv_workspace(m.n_mat, m.rows, m.cols, T, k, x.device)
    _check(y, torch.float32, "y", shape)
    return _run(prepare, getattr(lib(), entry),
                (_stream(stream), ctypes.byref(m), x.data_ptr(), _x_dtype(x), int(bool(x_per_slot)),
                 topk_ids.data_ptr(), _ptr(topk_w), T, k, y.data_ptr(), workspace.data_ptr(), workspace.numel()),
                entry, y, (m,), workspace if check else None, stream)


def moe_ffn(gu_syms, gu_scales, dn_syms, dn_scales, x, topk_ids, topk_w=None, h=None, y=None,
            workspace=None, stream=None, events=None, prepare=False, check=False):
    """Whole fused MoE layer; returns (y [T, hidden] fp32, h [T, k, inter] bf16).

    ``events``: optional ctypes array of hipEvent_t; events[0] and events[1]
    are stamped with the start and the end of the layer kernel's execution
    (see trellis_moe_ffn_timed). check=True: as for moe_gemv."""
    return _moe_ffn(None, gu_syms, gu_scales, dn_syms, dn_scales, x, topk_ids, topk_w, h, y, workspace, stream,
                    events, prepare, check)


def moe_ffn_e5m3(gu_syms, gu_scales, dn_syms, dn_scales, x, topk_ids, topk_w=None, h=None, y=None,
                 workspace=None, stream=None, prepare=False, check=False):
    """moe_ffn with both stacks' scale bytes read as E5M3 (trellis_moe_ffn_e5m3)."""
    return _moe_ffn("trellis_moe_ffn_e5m3", gu_syms, gu_scales, dn_syms, dn_scales, x, topk_ids, topk_w, h, y,
                    workspace, stream, None, prepare, check)


def _moe_ffn(entry, gu_syms, gu_scales, dn_syms, dn_scales, x, topk_ids, topk_w, h, y, workspace, stream, events,
             prepare, check):
    torch = _torch()
    mg = mat(gu_syms, gu_scales)
    md = mat(dn_syms, dn_scales)
    T, k = topk_ids.shape
    _check(topk_ids, torch.int32, "topk_ids")
    if topk_w is not None:
        _check(topk_w, torch.float32, "topk_w", (T, k))
    hidden, inter = mg.cols, mg.rows // 2
    _check(x, x.dtype, "x", (T, hidden))
    with _on(stream):
        if h is None:
            h = torch.empty((T, k, inter), dtype=torch.bfloat16, device=x.device)
        if y is None:
            y = torch.empty((T, hidden), dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = ffn_workspace(mg.n_mat, hidden, inter, T, k, x.device)
    _check(h, torch.bfloat16, "h", (T, k, inter))
    _check(y, torch.float32, "y", (T, hidden))
    args = (_stream(stream), ctypes.byref(mg), ctypes.byref(md), x.data_ptr(), _x_dtype(x),
            topk_ids.data_ptr(), _ptr(topk_w), T, k, h.data_ptr(), y.data_ptr(), workspace.data_ptr(),
            workspace.numel())
    if entry is None:   # the UE8M0 layer, through the timed entry point (events may be None)
        return _run(prepare, lib().trellis_moe_ffn_timed, args + (events,), "trellis_moe_ffn", (y, h),
                    (mg, md, events), workspace if check else None, stream)
    return _run(prepare, getattr(lib(), entry), args, entry, (y, h), (mg, md), workspace if check else None,
                stream)


def moe_ffn_routed(gu_syms, gu_scales, dn_syms, dn_scales, x, w_router, k, topk_ids=None, topk_w=None, h=None,
                   y=None, workspace=None, stream=None, events=None, prepare=False, check=False):
    """Router and layer for one token in one launch (trellis_moe_ffn_routed):
    x [1, hidden], w_router bf16 [E, hidden]; returns (y, h, topk_ids, topk_w),
    the last two the routing the kernel computed."""
    torch = _torch()
    mg = mat(gu_syms, gu_scales)
    md = mat(dn_syms, dn_scales)
    hidden, inter = mg.cols, mg.rows // 2
    _check(x, x.dtype, "x", (1, hidden))
    _check(w_router, torch.bfloat16, "w_router", (mg.n_mat, hidden))
    with _on(stream):
        if topk_ids is None:
            topk_ids = torch.empty((1, k), dtype=torch.int32, device=x.device)
        if topk_w is None:
            topk_w = torch.empty((1, k), dtype=torch.float32, device=x.device)
        if h is None:
            h = torch.empty((1, k, inter), dtype=torch.bfloat16, device=x.device)
        if y is None:
            y = torch.empty((1, hidden), dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = ffn_workspace(mg.n_mat, hidden, inter, 1, k, x.device)
    _check(topk_ids, torch.int32, "topk_ids", (1, k))
    _check(topk_w, torch.float32, "topk_w", (1, k))
    _check(h, torch.bfloat16, "h", (1, k, inter))
    _check(y, torch.float32, "y", (1, hidden))
    args = (_stream(stream), ctypes.byref(mg), ctypes.byref(md), x.data_ptr(), _x_dtype(x), w_router.data_ptr(),
            k, topk_ids.data_ptr(), topk_w.data_ptr(), h.data_ptr(), y.data_ptr(), workspace.data_ptr(),
            workspace.numel(), events)
    return _run(prepare, lib().trellis_moe_ffn_routed, args, "trellis_moe_ffn_routed", (y, h, topk_ids, topk_w),
                (mg, md, events), workspace if check else None, stream)


NOALLOC_SCRATCH_BYTES = 8 << 20   # TRELLIS_NOALLOC_SCRATCH_BYTES


def moe_ffn_noalloc(gu_syms, gu_scales, dn_syms, dn_scales, x, topk_ids, topk_w, h, y, stream=None,
                    prepare=False):
    """moe_ffn on the library's own per-device scratch (trellis_moe_ffn_noalloc):
    the caller passes the outputs h [T, k, inter] bf16 and y [T, hidden] fp32,
    and nothing is allocated. Returns (y, h)."""
    torch = _torch()
    mg = mat(gu_syms, gu_scales)
    md = mat(dn_syms, dn_scales)
    T, k = topk_ids.shape
    _check(topk_ids, torch.int32, "topk_ids")
    if topk_w is not None:
        _check(topk_w, torch.float32, "topk_w", (T, k))
    hidden, inter = mg.cols, mg.rows // 2
    _check(x, x.dtype, "x", (T, hidden))
    _check(h, torch.bfloat16, "h", (T, k, inter))
    _check(y, torch.float32, "y", (T, hidden))
    need = lib().trellis_moe_ffn_workspace_size(mg.n_mat, hidden, inter, T, k)
    if need > NOALLOC_SCRATCH_BYTES:
        raise TrellisError(-3, f"trellis_moe_ffn_noalloc: this layer needs {need} bytes of "
                           f"workspace, the library's scratch holds {NOALLOC_SCRATCH_BYTES}")
    return _run(prepare, lib().trellis_moe_ffn_noalloc,
                (_stream(stream), ctypes.byref(mg), ctypes.byref(md), x.data_ptr(), _x_dtype(x),
                 topk_ids.data_ptr(), _ptr(topk_w), T, k, h.data_ptr(), y.data_ptr()),
                "trellis_moe_ffn_noalloc", (y, h), (mg, md))


# ---------------------------------------------------------------- expanded (MXFP4) weights

def mx_mat(codes, scales) -> MxMat:
    """trellis_mx_t for codes [n_mat, rows, cols/2] uint8 (as trellis_decode_expand writes
    them) and scales [n_mat, rows, cols/32] uint8; both 16-byte aligned."""
    torch = _torch()
    if codes.dim() == 2:
        codes = codes.unsqueeze(0)
    if scales.dim() == 2:
        scales = scales.unsqueeze(0)
    _check(codes, torch.uint8, "codes")
    n_mat, rows, half = codes.shape
    _check(scales, torch.uint8, "scales", (n_mat, rows, half // 16))
    return MxMat(codes.data_ptr(), scales.data_ptr(), n_mat, rows, half * 2)


def mxfp4_moe_gemv(codes, scales, x, topk_ids, topk_w=None, x_per_slot=False, y=None, workspace=None,
                   stream=None, prepare=False, check=False):
    """moe_gemv on expanded MXFP4 weights (trellis_mxfp4_moe_gemv)."""
    torch = _torch()
    m = mx_mat(codes, scales)
    T, k = topk_ids.shape
    _check(topk_ids, torch.int32, "topk_ids")
    if topk_w is not None:
        _check(topk_w, torch.float32, "topk_w", (T, k))
    _check(x, x.dtype, "x", (T, k, m.cols) if x_per_slot else (T, m.cols))
    shape = (T, m.rows) if topk_w is not None else (T, k, m.rows)
    with _on(stream):
        if y is None:
            y = torch.empty(shape, dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = gemv_workspace(m.n_mat, m.rows, m.cols, T, k, x.device)
    _check(y, torch.float32, "y", shape)
    return _run(prepare, lib().trellis_mxfp4_moe_gemv,
                (_stream(stream), ctypes.byref(m), x.data_ptr(), _x_dtype(x), int(bool(x_per_slot)),
                 topk_ids.data_ptr(), _ptr(topk_w), T, k, y.data_ptr(), workspace.data_ptr(), workspace.numel()),
                "trellis_mxfp4_moe_gemv", y, (m,), workspace if check else None, stream)


def mxfp4_moe_ffn(gu_codes, gu_scales, dn_codes, dn_scales, x, topk_ids, topk_w=None, h=None, y=None,
                  workspace=None, stream=None, prepare=False, check=False):
    """moe_ffn on expanded MXFP4 weights (trellis_mxfp4_moe_ffn); returns (y, h)."""
    torch = _torch()
    mg = mx_mat(gu_codes, gu_scales)
    md = mx_mat(dn_codes, dn_scales)
    T, k = topk_ids.shape
    _check(topk_ids, torch.int32, "topk_ids")
    if topk_w is not None:
        _check(topk_w, torch.float32, "topk_w", (T, k))
    hidden, inter = mg.cols, mg.rows // 2
    _check(x, x.dtype, "x", (T, hidden))
    with _on(stream):
        if h is None:
            h = torch.empty((T, k, inter), dtype=torch.bfloat16, device=x.device)
        if y is None:
            y = torch.empty((T, hidden), dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = ffn_workspace(mg.n_mat, hidden, inter, T, k, x.device)
    _check(h, torch.bfloat16, "h", (T, k, inter))
    _check(y, torch.float32, "y", (T, hidden))
    return _run(prepare, lib().trellis_mxfp4_moe_ffn,
                (_stream(stream), ctypes.byref(mg), ctypes.byref(md), x.data_ptr(), _x_dtype(x),
                 topk_ids.data_ptr(), _ptr(topk_w), T, k, h.data_ptr(), y.data_ptr(), workspace.data_ptr(),
                 workspace.numel()),
                "trellis_mxfp4_moe_ffn", (y, h), (mg, md), workspace if check else None, stream)


def viterbi_workspace(rows, n, device="cuda"):
    torch = _torch()
    nb = lib().trellis_viterbi_workspace_size(rows, n)
    if nb == 0:
        raise TrellisError(-1, "trellis_viterbi_workspace_size")
    return torch.empty(nb, dtype=torch.uint8, device=device)


def viterbi_encode(target, d=None, syms_out=None, cost_out=None, workspace=None, stream=None, prepare=False):
    """Curvature-aware Viterbi symbol search per row: target [rows, n] float64,
    d [rows, n] float64 or None (ones). Returns (symbols [rows, n] uint8, cost [rows] float64)."""
    torch = _torch()
    if target.dim() == 1:
        target = target.unsqueeze(0)
    _check(target, torch.float64, "target")
    rows, n = target.shape
    if d is not None:
        _check(d, torch.float64, "d", (rows, n))
    with _on(stream):
        if syms_out is None:
            syms_out = torch.empty((rows, n), dtype=torch.uint8, device=target.device)
        if cost_out is None:
            cost_out = torch.empty((rows,), dtype=torch.float64, device=target.device)
        if workspace is None:
            workspace = viterbi_workspace(rows, n, device=target.device)
    _check(syms_out, torch.uint8, "syms_out", (rows, n))
    _check(cost_out, torch.float64, "cost_out", (rows,))
    return _run(prepare, lib().trellis_viterbi_encode,
                (_stream(stream), target.data_ptr(), _ptr(d), rows, n, syms_out.data_ptr(), cost_out.data_ptr(),
                 workspace.data_ptr(), workspace.numel() * workspace.element_size()),
                "trellis_viterbi_encode", (syms_out, cost_out), (workspace,))


def router_workspace(E, T, device="cuda"):
    torch = _torch()
    n = lib().trellis_router_workspace_size(E, T)
    if n == 0:
        raise TrellisError(-1, "trellis_router_workspace_size")
    return torch.zeros(n, dtype=torch.uint8, device=device)   # zero-filled before first use


def router_topk(x, w_router, k, topk_ids=None, topk_w=None, workspace=None, stream=None, prepare=False):
    """Router: x [T, H] fp32/bf16, w_router [E, H] bf16 -> (topk_ids [T, k] int32, topk_w [T, k] fp32)."""
    torch = _torch()
    if x.dim() == 1:
        x = x.unsqueeze(0)
    _check(x, x.dtype, "x")
    _check(w_router, torch.bfloat16, "w_router")
    T, H = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise ValueError("w_router must be [E, H] with the same H as x")
    with _on(stream):
        if topk_ids is None:
            topk_ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
        if topk_w is None:
            topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = router_workspace(E, T, device=x.device)
    _check(topk_ids, torch.int32, "topk_ids", (T, k))
    _check(topk_w, torch.float32, "topk_w", (T, k))
    return _run(prepare, lib().trellis_router_topk,
                (_stream(stream), x.data_ptr(), _x_dtype(x), w_router.data_ptr(), E, H, T, k,
                 topk_ids.data_ptr(), topk_w.data_ptr(), workspace.data_ptr(),
                 workspace.numel() * workspace.element_size()),
                "trellis_router_topk", (topk_ids, topk_w), (workspace,))


def read_bandwidth(buf, sink, stream=None, prepare=False):
    """Read every byte of the device tensor `buf` once (trellis_read_bandwidth),
    XOR-folding its 32-bit words into `sink` (int32 device tensor of 256
    elements; the XOR of all of them is the checksum)."""
    torch = _torch()
    _check(sink, torch.int32, "sink", (256,))
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    return _run(prepare, lib().trellis_read_bandwidth,
                (_stream(stream), buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr()),
                "trellis_read_bandwidth", sink, (buf,))
