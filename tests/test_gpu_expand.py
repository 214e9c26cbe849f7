"""Expand (HEPH's second serving mode) on the GPU: bit-exact against the oracle."""
import os

import numpy as np
import pytest

import workloads
from helpers import announce, dev

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decode_vectors.txt")


def _expand(tq, syms, scales):
    codes, sc = tq.decode_expand(dev(syms), dev(scales))
    return codes.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("n_mat,rows,cols", [
    (1, 256, 1024),      # single-matrix workload shape
    (2, 3, 32),          # two words per row: one-word-per-thread path
    (3, 7, 96),          # six words per row
    (1, 5, 2880),        # 180 words per row, 90 scale blocks
    (4, 64, 1536),       # expert matrix width of the 128-expert layer
    (1, 1, 64),
])
def test_expand_bit_exact(trellis_lib, orc, n_mat, rows, cols):
    announce(f"expand {n_mat}x{rows}x{cols}")
    g = workloads.rng(501, cols, rows, n_mat)
    syms = workloads.symbols(g, n_mat, rows, cols)
    sc = workloads.scales(g, n_mat, rows, cols)
    ref_codes, ref_sc = orc.expand(syms, sc)
    codes, sc2 = _expand(trellis_lib, syms, sc)
    assert (sc2 == ref_sc).all()
    mism = np.nonzero(codes != ref_codes)
    assert mism[0].size == 0, f"{mism[0].size} bytes differ, first at {[m[0] for m in mism]}"


def test_expand_golden_rows(trellis_lib):
    """Hand-derived vectors: each golden row padded to 32 weights with a zero word
    (the padding only follows the golden words, so their codes are unaffected)."""
    announce("expand golden rows")
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, words, _, packed = [f.strip() for f in line.split("|")]
        w = [int(t, 16) for t in words.split()]
        n_words = len(w) + (len(w) % 2)
        row = np.zeros((1, 1, n_words), dtype=np.uint32)
        row[0, 0, :len(w)] = w
        sc = np.full((1, 1, n_words // 2), 127, dtype=np.uint8)
        codes, _ = _expand(trellis_lib, row, sc)
        want = bytes.fromhex(packed)
        assert codes.tobytes()[:len(want)] == want, name


def test_expand_special_streams(trellis_lib, orc):
    announce("expand constant streams")
    rows = np.stack([np.zeros(64, np.uint32), np.full(64, 0xFFFFFFFF, np.uint32),
                     np.full(64, 0x55555555, np.uint32), np.full(64, 0xAAAAAAAA, np.uint32)])[None]
    sc = np.full((1, 4, 32), 127, np.uint8)
    sc[0, 1, :] = 255     # NaN exponents are copied, not interpreted
    sc[0, 2, :] = 0
    ref, _ = orc.expand(rows, sc)
    codes, sc2 = _expand(trellis_lib, rows, sc)
    assert (codes == ref).all() and (sc2 == sc).all()
    assert (codes[0, 0] == 0xFF).all()       # zero stream: -6 everywhere


def test_expand_full_128_experts_every_row(trellis_lib, orc):
    """All 128 experts x 3 matrices of 4096 x 1536 expanded in one call (the
    expand workload), every byte of codes and scales against the oracle's
    expand (matrices checked in parallel host threads)."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    announce("expand 128x3x4096x1536, every row")
    n_mat, rows, cols = 3 * 128, 4096, 1536
    g = workloads.rng(5, workloads.T_SYMS_UP)
    syms = workloads.symbols(g, n_mat, rows, cols)
    sc = workloads.scales(g, n_mat, rows, cols)
    ds, de = dev(syms), dev(sc)
    codes, sc2 = trellis_lib.decode_expand(ds, de)
    torch.cuda.synchronize()
    assert torch.equal(sc2, de)
    del ds, de, sc2
    got = codes.cpu().numpy()
    del codes
    torch.cuda.empty_cache()

    def differs(m):
        ref, _ = orc.expand(syms[m:m + 1], sc[m:m + 1])
        return not np.array_equal(ref[0], got[m])

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(threads) as ex:
        bad = [m for m, d in enumerate(ex.map(differs, range(n_mat))) if d]
    assert not bad, f"{len(bad)} of {n_mat} matrices differ, first {bad[:5]}"
