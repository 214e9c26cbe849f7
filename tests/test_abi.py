"""The C ABI without a GPU: the library loads, exports every function that
include/trellis.h declares, and rejects bad arguments on the host before
anything would be enqueued (these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

import trellis_coded_fp4_amd as tq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "trellis.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(trellis_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = tq.lib()
    names = declared_functions()
    assert names, "no declarations parsed"
    assert sorted(names) == sorted(tq.EXPORTS)
    for n in names:
        assert hasattr(lib, n), f"libtrellis.so does not export {n}"


def test_version_and_strerror():
    assert tq.version() >= 100
    for code in (0, -1, -2, -3, -4, -5):
        assert tq.strerror(code)
    assert tq.strerror(-99) == "unknown error"


def _mat(syms=1, scales=1, n_mat=1, rows=16, cols=64):
    return tq.Mat(syms, scales, n_mat, rows, cols)


FAKE = 0x1000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("m,code", [
    (None, -2),
    (dict(syms=0), -2),
    (dict(scales=0), -2),
    (dict(n_mat=0), -1),
    (dict(rows=0), -1),
    (dict(cols=48), -1),
    (dict(cols=0), -1),
])
def test_expand_rejects(m, code):
    lib = tq.lib()
    arg = None if m is None else ctypes.byref(_mat(**m))
    assert lib.trellis_decode_expand(None, arg, FAKE, FAKE) == code


def test_expand_rejects_null_outputs():
    lib = tq.lib()
    assert lib.trellis_decode_expand(None, ctypes.byref(_mat()), None, FAKE) == -2
    assert lib.trellis_decode_expand(None, ctypes.byref(_mat()), FAKE, None) == -2


def _gemv(lib, m=None, x=FAKE, dtype=0, per_slot=0, ids=FAKE, w=None, T=1, k=1, y=FAKE, ws=0x10000,
          wsb=1 << 30):
    m = _mat() if m is None else m
    return lib.trellis_moe_gemv(None, ctypes.byref(m), x, dtype, per_slot, ids, w, T, k, y, ws, wsb)


def test_gemv_argument_checks():
    lib = tq.lib()
    assert _gemv(lib, x=None) == -2
    assert _gemv(lib, ids=None) == -2
    assert _gemv(lib, y=None) == -2
    assert _gemv(lib, ws=None) == -2
    assert _gemv(lib, dtype=7) == -1
    assert _gemv(lib, per_slot=2) == -1
    assert _gemv(lib, T=0) == -1
    assert _gemv(lib, T=129) == -1                # T > 128
    assert _gemv(lib, k=0) == -1
    assert _gemv(lib, k=33) == -1
    assert _gemv(lib, m=_mat(rows=24)) == -1          # rows % 16
    assert _gemv(lib, m=_mat(n_mat=1025)) == -1
    assert _gemv(lib, ws=0x10010) == -3               # misaligned workspace
    assert _gemv(lib, wsb=16) == -3                   # too small


def test_ffn_argument_checks():
    lib = tq.lib()
    gu, dn = _mat(n_mat=2, rows=128, cols=64), _mat(n_mat=2, rows=64, cols=64)

    def call(gu=gu, dn=dn, x=FAKE, h=FAKE, y=FAKE, T=1, k=1, ws=0x10000, wsb=1 << 30):
        return lib.trellis_moe_ffn(None, ctypes.byref(gu), ctypes.byref(dn), x, 1, FAKE, None, T, k, h, y,
                                   ws, wsb)
    assert call(h=None) == -2
    assert call(x=None) == -2
    assert call(dn=_mat(n_mat=3, rows=64, cols=64)) == -1     # expert counts differ
    assert call(dn=_mat(n_mat=2, rows=32, cols=64)) == -1     # down rows != hidden
    assert call(dn=_mat(n_mat=2, rows=64, cols=32)) == -1     # down cols != inter
    assert call(gu=_mat(n_mat=2, rows=96, cols=64)) == -1     # 2*inter % 64
    assert call(wsb=100) == -3


def test_ffn_routed_argument_checks():
    lib = tq.lib()
    gu, dn = _mat(n_mat=4, rows=128, cols=64), _mat(n_mat=4, rows=64, cols=64)

    def call(gu=gu, dn=dn, x=FAKE, w=FAKE, k=2, ids=FAKE, gw=FAKE, h=FAKE, y=FAKE, ws=0x10000, wsb=1 << 30):
        return lib.trellis_moe_ffn_routed(None, ctypes.byref(gu), ctypes.byref(dn), x, 1, w, k, ids, gw, h, y,
                                          ws, wsb, None)
    assert call(w=None) == -2
    assert call(ids=None) == -2
    assert call(gw=None) == -2
    assert call(k=5) == -1                                    # k > number of experts
    assert call(k=0) == -1
    assert call(dn=_mat(n_mat=3, rows=64, cols=64)) == -1     # expert counts differ
    assert call(wsb=100) == -3


def test_ffn_noalloc_rejects_what_its_scratch_cannot_hold():
    """trellis_moe_ffn_noalloc checks the shape's workspace need against its
    fixed scratch before anything is enqueued."""
    lib = tq.lib()
    # 128 experts, hidden 4096, inter 4096, 128 tokens x top-8: ~9.8 MB
    gu, dn = _mat(n_mat=128, rows=8192, cols=4096), _mat(n_mat=128, rows=4096, cols=4096)
    assert lib.trellis_moe_ffn_workspace_size(128, 4096, 4096, 128, 8) > tq.NOALLOC_SCRATCH_BYTES
    rc = lib.trellis_moe_ffn_noalloc(None, ctypes.byref(gu), ctypes.byref(dn), FAKE, 1, FAKE, None, 128, 8,
                                     FAKE, FAKE)
    assert rc == -3
    assert lib.trellis_moe_ffn_noalloc(None, None, ctypes.byref(dn), FAKE, 1, FAKE, None, 1, 1, FAKE, FAKE) == -2
    assert lib.trellis_moe_ffn_noalloc(None, ctypes.byref(gu), ctypes.byref(dn), FAKE, 1, FAKE, None, 1, 0,
                                       FAKE, FAKE) == -1


def test_workspace_sizes():
    lib = tq.lib()
    a = lib.trellis_moe_gemv_workspace_size(32, 5760, 2880, 1, 4)
    b = lib.trellis_moe_gemv_workspace_size(32, 5760, 2880, 32, 4)
    assert 0 < a < b
    assert lib.trellis_moe_gemv_workspace_size(32, 5760, 2881, 1, 4) == 0
    assert lib.trellis_moe_gemv_workspace_size(32, 5760, 2880, 0, 4) == 0
    f = lib.trellis_moe_ffn_workspace_size(128, 4096, 1536, 32, 8)
    assert f > 0 and f % 256 == 0
    assert lib.trellis_moe_ffn_workspace_size(128, 4096, 1530, 32, 8) == 0


def test_mxfp4_argument_checks():
    lib = tq.lib()
    m = tq.MxMat(0x10000, 0x20000, 1, 16, 64)
    call = lambda mm, **kw: lib.trellis_mxfp4_moe_gemv(None, ctypes.byref(mm) if mm is not None else None,
                                                       kw.get("x", FAKE), 0, 0, FAKE, None, 1, 1, FAKE, 0x10000,
                                                       1 << 30)
    assert call(None) == -2
    assert call(tq.MxMat(0, 0x20000, 1, 16, 64)) == -2
    assert call(tq.MxMat(0x10008, 0x20000, 1, 16, 64)) == -1     # codes not 16-byte aligned
    assert call(tq.MxMat(0x10000, 0x20004, 1, 16, 64)) == -1     # scales not 16-byte aligned
    assert call(tq.MxMat(0x10000, 0x20000, 1, 24, 64)) == -1     # rows % 16
    assert call(m, x=None) == -2
    gu, dn = tq.MxMat(0x10000, 0x20000, 2, 128, 64), tq.MxMat(0x10000, 0x20000, 2, 64, 64)
    f = lambda g, d, h=FAKE: lib.trellis_mxfp4_moe_ffn(None, ctypes.byref(g), ctypes.byref(d), FAKE, 1, FAKE,
                                                       None, 1, 1, h, FAKE, 0x10000, 1 << 30)
    assert f(gu, dn, h=None) == -2
    assert f(gu, tq.MxMat(0x10000, 0x20000, 2, 64, 32)) == -1    # down cols != inter


def test_viterbi_argument_checks():
    lib = tq.lib()
    call = lambda t=FAKE, d=None, rows=4, n=16, s=FAKE, c=0x30000, ws=0x10000: lib.trellis_viterbi_encode(
        None, t, d, rows, n, s, c, ws, 1 << 30)
    assert call(t=None) == -2
    assert call(s=None) == -2
    assert call(c=None) == -2
    assert call(ws=None) == -2
    assert call(rows=0) == -1
    assert call(n=0) == -1
    assert call(t=FAKE + 4) == -1          # float64 target not 8-byte aligned
    assert call(d=FAKE + 4) == -1
    assert call(c=0x30004) == -1
    assert call(ws=0x10040) == -3          # workspace not 256-byte aligned
    assert lib.trellis_viterbi_workspace_size(0, 16) == 0
    assert lib.trellis_viterbi_workspace_size(4, 0) == 0


def test_router_argument_checks():
    lib = tq.lib()
    call = lambda x=FAKE, dt=1, w=0x20000, E=32, H=2880, T=1, k=4, i=0x30000, g=0x40000, ws=0x50000, wsb=1 << 20: \
        lib.trellis_router_topk(None, x, dt, w, E, H, T, k, i, g, ws, wsb)
    assert call(x=None) == -2
    assert call(w=None) == -2
    assert call(i=None) == -2
    assert call(g=None) == -2
    assert call(dt=7) == -1
    assert call(E=0) == -1
    assert call(E=1025) == -1
    assert call(k=0) == -1
    assert call(k=33, E=32) == -1          # k > E
    assert call(H=2884) == -1              # H % 8
    assert call(H=8200) == -1              # H > 8192
    assert call(T=0) == -1
    assert call(w=0x20008) == -1           # router rows not 16-byte aligned
    assert call(x=FAKE + 8) == -1          # x not 16-byte aligned
    assert call(ws=None) == -2
    assert call(ws=0x50040) == -3          # workspace not 256-byte aligned
    assert call(wsb=16) == -3              # workspace too small
    assert lib.trellis_router_workspace_size(32, 1) == 256 + 32 * 8
    assert lib.trellis_router_workspace_size(0, 1) == 0


def test_gemv_workspace_for_a_stack_matches_the_shape_query():
    """trellis_moe_gemv_workspace(w, T, k) is the shape query for w's own shape."""
    lib = tq.lib()
    for n_mat, rows, cols, T, k in [(1, 256, 1024, 1, 1), (32, 5760, 2880, 1, 4), (128, 3072, 4096, 32, 8),
                                    (3, 16, 32, 32, 8)]:
        m = _mat(n_mat=n_mat, rows=rows, cols=cols)
        assert lib.trellis_moe_gemv_workspace(ctypes.byref(m), T, k) == \
            lib.trellis_moe_gemv_workspace_size(n_mat, rows, cols, T, k) > 0
    assert lib.trellis_moe_gemv_workspace(None, 1, 1) == 0
    assert lib.trellis_moe_gemv_workspace(ctypes.byref(_mat(cols=48)), 1, 1) == 0
    assert lib.trellis_moe_gemv_workspace(ctypes.byref(_mat()), 0, 1) == 0


def test_ffn_workspace_covers_the_single_token_region():
    """The layer workspace holds the general kernel's layout and, after the
    status words, the single-token kernel's region; larger for more tokens."""
    lib = tq.lib()
    one = lib.trellis_moe_ffn_workspace_size(32, 2880, 2880, 1, 4)
    many = lib.trellis_moe_ffn_workspace_size(32, 2880, 2880, 8, 4)
    # region: call counter line + tagged h of up to 32 experts + a tag per 16 rows of y
    region = 256 + 32 * 2880 * 4 + (2880 // 16) * 4
    assert one >= 256 + region and many > one


def test_read_bandwidth_argument_checks():
    """The streaming-read reference rejects NULL pointers, a misaligned buffer
    and a byte count that is not a whole number of 32-bit words."""
    lib = tq.lib()
    buf, sink = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000)
    assert lib.trellis_read_bandwidth(None, None, 64, sink) == -2
    assert lib.trellis_read_bandwidth(None, buf, 64, None) == -2
    assert lib.trellis_read_bandwidth(None, ctypes.c_void_p(0x10004), 64, sink) == -1
    assert lib.trellis_read_bandwidth(None, buf, 66, sink) == -1
