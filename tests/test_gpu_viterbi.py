"""The encoder's curvature-aware Viterbi search on the GPU against the
oracle's search (XOR-Trellis news article, bullet "Curvature-aware Viterbi
objective"): symbols bit-exact, minimum cost equal in float64."""
import numpy as np
import pytest

import workloads
from helpers import announce, dev

pytestmark = pytest.mark.gpu


def _gpu(tq, target, d):
    syms, cost = tq.viterbi_encode(dev(target), None if d is None else dev(d))
    return syms.cpu().numpy(), cost.cpu().numpy()


def _objective(orc, syms, target, d):
    """The objective of the given symbol rows, in position order (oracle decode)."""
    rows, n = syms.shape
    npad = (n + 15) // 16 * 16
    s = np.zeros((rows, npad), dtype=np.uint32)
    s[:, :n] = syms
    words = np.zeros((rows, npad // 16), dtype=np.uint32)
    for j in range(16):
        words |= s[:, j::16] << np.uint32(2 * j)
    codes = orc.decode_codes(words, npad)[:, :n]
    table = np.array([orc.e2m1_value(c) for c in range(16)])
    vals = table[codes]
    cost = np.zeros(rows)
    for k in range(n):
        err = target[:, k] - vals[:, k]
        cost = cost + d[:, k] * err * err
    return cost


@pytest.mark.parametrize("rows,n,weighted,seed", [
    (3, 1, False, 0),
    (4, 5, True, 1),
    (3, 64, True, 2),
    (2, 257, True, 3),     # crosses a 256-position staging chunk; ragged traceback chunk
    (2, 300, False, 4),
])
def test_viterbi_matches_oracle(trellis_lib, orc, rows, n, weighted, seed):
    announce(f"viterbi rows={rows} n={n} weighted={weighted}")
    target, d = workloads.encode_rows(900 + seed, rows, n)
    syms, cost = _gpu(trellis_lib, target, d if weighted else None)
    for r in range(rows):
        ref_syms, ref_cost = orc.viterbi(target[r], d[r] if weighted else None)
        assert cost[r] == ref_cost, (r, cost[r], ref_cost)
        assert np.array_equal(syms[r], ref_syms), r


def test_viterbi_more_rows_than_workgroups(trellis_lib, orc):
    """600 rows: more than the 2 x 256 workgroups of one launch, so
    workgroups search several rows each."""
    rows, n = 600, 3
    announce(f"viterbi rows={rows} n={n}")
    target, d = workloads.encode_rows(950, rows, n)
    syms, cost = _gpu(trellis_lib, target, d)
    for r in range(rows):
        ref_syms, ref_cost = orc.viterbi(target[r], d[r])
        assert cost[r] == ref_cost and np.array_equal(syms[r], ref_syms), r


def test_viterbi_encodable_target(trellis_lib, orc):
    """A target that is itself a decoded row is reached at zero cost by the
    symbols that produced it (the zero-cost path is unique)."""
    g = workloads.rng(951, 0)
    words = workloads.symbols(g, 1, 2, 160)[0]
    codes = orc.decode_codes(words, 160)
    table = np.array([orc.e2m1_value(c) for c in range(16)])
    target = table[codes]
    syms, cost = _gpu(trellis_lib, target, None)
    assert np.all(cost == 0.0)
    ref = np.stack([(words[:, j // 16] >> np.uint32(2 * (j % 16))) & np.uint32(3) for j in range(160)], axis=1)
    assert np.array_equal(syms, ref.astype(np.uint8))


def test_viterbi_zero_weights(trellis_lib):
    """d = 0: every path costs 0; the search keeps the smaller predecessor on
    ties and ends in the smallest state, which is the all-zero path."""
    target, _ = workloads.encode_rows(952, 2, 40)
    syms, cost = _gpu(trellis_lib, target, np.zeros_like(target))
    assert np.all(cost == 0.0)
    assert not syms.any()


def test_viterbi_full_size_sampled(trellis_lib, orc):
    """The benchmark shape (512 rows x 2880 positions): every row's symbols
    achieve the reported cost; two sampled rows match the oracle's search."""
    cfg = workloads.VITERBI
    rows, n = cfg["rows"], cfg["n"]
    announce(f"viterbi full size {rows}x{n}")
    target, d = workloads.encode_rows(cfg["config_id"], rows, n)
    syms, cost = _gpu(trellis_lib, target, d)
    assert syms.max() <= 3
    np.testing.assert_array_equal(_objective(orc, syms, target, d), cost)
    for r in (0, rows - 1):
        ref_syms, ref_cost = orc.viterbi(target[r], d[r])
        assert cost[r] == ref_cost and np.array_equal(syms[r], ref_syms), r
