"""Host build of the device decoder's integer arithmetic vs the oracle.

libtq_bitcheck.so is compiled from the same tq_decode.h the kernels use, so
these CPU tests check the bit-sliced decode (16 weights per word from funnel
shifts and XORs) and the activation layout without a GPU."""
import ctypes
import os

import numpy as np
import pytest

import workloads

HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(HERE, "trellis_coded_fp4_amd", "libtq_bitcheck.so")


@pytest.fixture(scope="module")
def bc():
    if not os.path.exists(LIB):
        pytest.fail("libtq_bitcheck.so not built (run python -m trellis_coded_fp4_amd.build)")
    L = ctypes.CDLL(LIB)
    U = ctypes.c_uint32
    PU = ctypes.POINTER(U)
    L.tq_bitcheck_decode_word.argtypes = [U, U, PU, PU]
    L.tq_bitcheck_natural.argtypes = [U, U, PU, PU]
    for f in ("tq_bitcheck_nibble_position", "tq_bitcheck_bchunk_offset"):
        getattr(L, f).argtypes = [ctypes.c_int]
        getattr(L, f).restype = ctypes.c_int
    L.tq_bitcheck_canonical_k.argtypes = [ctypes.c_int, ctypes.c_int]
    L.tq_bitcheck_canonical_k.restype = ctypes.c_int
    L.tq_bitcheck_e5m3_terms.argtypes = [U]
    L.tq_bitcheck_e5m3_terms.restype = U
    return L


def _decode_row(bc, words):
    """Per-weight codes of one row through the bit-sliced decoder."""
    out = []
    prev = 0
    e, o = ctypes.c_uint32(), ctypes.c_uint32()
    for w in words:
        bc.tq_bitcheck_decode_word(int(w), prev, ctypes.byref(e), ctypes.byref(o))
        for m in range(16):
            src = e.value if m % 2 == 0 else o.value
            out.append((src >> (4 * (m // 2))) & 0xF)
        prev = int(w)
    return np.array(out, dtype=np.uint8)


def test_bitsliced_decode_matches_oracle(bc, orc):
    g = workloads.rng(77, 0)
    syms = workloads.symbols(g, 1, 40, 256)[0]
    syms[0, :] = 0
    syms[1, :] = 0xFFFFFFFF
    ref = orc.decode_codes(syms, 256)
    for r in range(syms.shape[0]):
        assert (_decode_row(bc, syms[r]) == ref[r]).all(), f"row {r}"


def test_natural_order_matches_oracle_expand(bc, orc):
    g = workloads.rng(77, 1)
    syms = workloads.symbols(g, 1, 8, 128)
    sc = workloads.scales(g, 1, 8, 128)
    packed, _ = orc.expand(syms, sc)
    lo, hi = ctypes.c_uint32(), ctypes.c_uint32()
    for r in range(8):
        prev = 0
        got = bytearray()
        for w in syms[0, r]:
            bc.tq_bitcheck_natural(int(w), prev, ctypes.byref(lo), ctypes.byref(hi))
            got += int(lo.value).to_bytes(4, "little") + int(hi.value).to_bytes(4, "little")
            prev = int(w)
        assert bytes(got) == packed[0, r].tobytes()


def test_activation_layout_is_a_bijection(bc):
    # nibble n of the four decoded registers <-> weight position in the block
    pos = [bc.tq_bitcheck_nibble_position(n) for n in range(32)]
    assert sorted(pos) == list(range(32))
    # canonical K of (block, position) covers 0..127 once, and inverts nibble_position
    ks = [bc.tq_bitcheck_canonical_k(b, p) for b in range(4) for p in range(32)]
    assert sorted(ks) == list(range(128))
    for n in range(32):
        assert bc.tq_bitcheck_canonical_k(0, pos[n]) == n
    # byte offset of canonical K inside a 128-byte B chunk: bijective, 32 per lane group
    offs = [bc.tq_bitcheck_bchunk_offset(k) for k in range(128)]
    assert sorted(offs) == list(range(128))
    for k in range(128):
        lane_group, byte = divmod(offs[k], 32)
        # bytes 0..15 of lane group g hold k = 16g..16g+15, bytes 16..31 hold k = 64+16g..
        assert k == (16 * lane_group + byte if byte < 16 else 64 + 16 * lane_group + byte - 16)


def test_activation_column_layout(bc):
    """Physical block b of a row feeds matrix-core step 2*(b//8) + b%2 as K-block
    (b%8)//2, which is what lane-group g reads when it loads blocks 8j+2g, 8j+2g+1.
    Over a whole column the weight positions map one-to-one onto bytes."""
    bc.tq_bitcheck_act_offset.argtypes = [ctypes.c_int, ctypes.c_int]
    bc.tq_bitcheck_act_offset.restype = ctypes.c_int
    bc.tq_bitcheck_act_scale_index.argtypes = [ctypes.c_int]
    bc.tq_bitcheck_act_scale_index.restype = ctypes.c_int
    nb = 96
    offs = [bc.tq_bitcheck_act_offset(b, p) for b in range(nb) for p in range(32)]
    assert sorted(offs) == list(range(nb * 32))
    sidx = [bc.tq_bitcheck_act_scale_index(b) for b in range(nb)]
    assert sorted(sidx) == list(range(nb))
    for j in range(nb // 8):
        for g in range(4):
            for h in range(2):
                b = 8 * j + 2 * g + h
                step = 2 * j + h
                assert sidx[b] == 4 * step + g
                # the block's 32 bytes sit in lane-group g's halves of the step's chunk
                got = sorted(bc.tq_bitcheck_act_offset(b, p) - 128 * step for p in range(32))
                assert got == list(range(16 * g, 16 * g + 16)) + list(range(64 + 16 * g, 64 + 16 * g + 16)) or \
                    got == sorted(bc.tq_bitcheck_bchunk_offset(32 * g + n) for n in range(32))


def test_e5m3_terms_sum_to_the_oracle_scale(bc, orc):
    """The matrix-core path writes each E5M3 block scale as four UE8M0
    terms; their values sum to the oracle's E5M3 value for every byte, with
    0 marking the zero scale and four NaN bytes for exponent 31."""
    for c in range(256):
        t = bc.tq_bitcheck_e5m3_terms(c)
        want = orc.e5m3_scale(c)
        if not np.isfinite(want):
            assert t == 0xFFFFFFFF, c
        elif want == 0.0:
            assert t == 0, c
        else:
            b = [(t >> (8 * i)) & 0xFF for i in range(4)]
            assert all(1 <= x <= 254 for x in b), (c, b)
            assert sum(np.ldexp(1.0, x - 127) for x in b) == want, (c, b)
