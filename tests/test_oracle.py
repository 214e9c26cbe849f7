"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's decoder: each checks it against a value
printed on the pages, a closed form, an invariant, a hand derivation
(tests/golden), exact rational arithmetic, a library routine, or brute force.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decode_vectors.txt")

# XOR-Trellis article, bullet "XOR-Trellis FP4 decoder": the four palettes as
# printed (English page; the Chinese page prints the same lists).
PAGE_PALETTES = [[-6, -1.5, 0, 2], [-4, -1, 0.5, 3], [-3, -0.5, 1, 4], [-2, 0, 1.5, 6]]
# HEPH abstract: the codebook is "the 15 distinct E2M1 values".
# Tied Trit-Planes paper, section 2.3: fp4 magnitudes x2 are {0,1,2,3,4,6,8,12}.
DOUBLED_E2M1_MAGNITUDES = [0, 1, 2, 3, 4, 6, 8, 12]


def _e2m1_set():
    mags = [m / 2 for m in DOUBLED_E2M1_MAGNITUDES]
    return sorted(set(mags) | set(-m for m in mags))


def _parse_value(tok):
    return -0.0 if tok == "-0" else float(tok)


def _golden():
    out = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, words, vals, packed = [f.strip() for f in line.split("|")]
        w = np.array([int(t, 16) for t in words.split()], dtype=np.uint32)
        v = None if vals == "-" else [_parse_value(t) for t in vals.split()]
        out.append((name, w, v, bytes.fromhex(packed)))
    return out


# ---------------------------------------------------------------- tables

def test_palettes_equal_the_article(orc):
    for p in range(4):
        for e in range(4):
            assert orc.palette_entry(p, e) == PAGE_PALETTES[p][e]


def test_palette_zero_signs_make_palettes_disjoint(orc):
    """The article calls the palettes disjoint: with P3's 0 read as -0 the 16
    (palette, entry) pairs are 16 distinct E2M1 codes (reading R4)."""
    codes = [orc.e2m1_code(orc.palette_entry(p, e)) for p in range(4) for e in range(4)]
    assert sorted(codes) == list(range(16))
    assert math.copysign(1, orc.palette_entry(3, 1)) < 0
    assert math.copysign(1, orc.palette_entry(0, 2)) > 0


def test_e2m1_decode_matches_doubled_magnitudes(orc):
    assert [2 * orc.e2m1_value(c) for c in range(8)] == DOUBLED_E2M1_MAGNITUDES
    for c in range(8):
        assert orc.e2m1_value(c | 8) == -orc.e2m1_value(c)
        assert math.copysign(1, orc.e2m1_value(c | 8)) < 0
    assert orc.e2m1_code(0.25) == -1 and orc.e2m1_code(5.0) == -1


def test_ue8m0_scale(orc):
    assert orc.ue8m0_scale(127) == 1.0
    assert orc.ue8m0_scale(130) == 8.0
    assert orc.ue8m0_scale(124) == 0.125
    assert orc.ue8m0_scale(0) == 2.0 ** -127
    assert math.isnan(orc.ue8m0_scale(255))


def test_palette_union_is_e2m1_set(orc):
    vals = {orc.palette_entry(p, e) for p in range(4) for e in range(4)}
    assert sorted(vals) == sorted(set(_e2m1_set()))
    assert len(vals) == 15


# ---------------------------------------------------------------- invariants

def test_uniform_use_over_all_states(orc):
    """Every E2M1 code is produced by exactly 4096 of the 2^16 states
    (the article's 'uniform use' of four disjoint 4-entry palettes)."""
    counts = np.zeros(16, dtype=np.int64)
    for s in range(1 << 16):
        counts[orc.state_code(s)] += 1
    assert (counts == 4096).all()


def test_decoded_values_in_e2m1_set(orc):
    g = workloads.rng(99, 0)
    syms = workloads.symbols(g, 1, 64, 256)
    sc = np.full((1, 64, 8), 127, dtype=np.uint8)
    w = orc.decode_values(syms, sc)
    assert set(np.unique(w).tolist()) <= set(_e2m1_set())
    codes = orc.decode_codes(syms, 256)
    assert codes.max() < 16


def test_state_bits_14_15_never_matter(orc):
    """All masks live in bits 0..13, so states differing in bits 14..15 agree."""
    for s in range(0, 1 << 14, 7):
        c = orc.state_code(s)
        for hi in (1, 2, 3):
            assert orc.state_code(s | (hi << 14)) == c


def test_windowed_equals_sequential(orc):
    g = workloads.rng(99, 1)
    syms = workloads.symbols(g, 1, 8, 512)[0]
    codes = orc.decode_codes(syms, 512)
    rs = np.random.default_rng(5)
    for r in range(8):
        for k in list(range(0, 20)) + rs.integers(0, 512, size=40).tolist():
            assert orc.decode_window(syms[r], k) == codes[r, k]


def test_gf2_affinity(orc):
    """The code map is affine over GF(2) in the stream bits:
    code(a ^ b) = code(a) ^ code(b) ^ 0xF weight by weight."""
    g = workloads.rng(99, 2)
    a = workloads.symbols(g, 1, 16, 512)[0]
    b = workloads.symbols(g, 1, 16, 512)[0]
    ca, cb, cab = orc.decode_codes(a, 512), orc.decode_codes(b, 512), orc.decode_codes(a ^ b, 512)
    assert ((ca ^ cb ^ 0xF) == cab).all()


def test_rows_are_independent(orc):
    """State resets at every row: a row decodes the same alone or after others."""
    g = workloads.rng(99, 3)
    syms = workloads.symbols(g, 1, 5, 64)[0]
    all_codes = orc.decode_codes(syms, 64)
    for r in range(5):
        assert (orc.decode_codes(syms[r:r + 1], 64)[0] == all_codes[r]).all()


# ---------------------------------------------------------------- closed forms

def test_zero_stream_is_minus_six(orc):
    """s stays 0, all parities are 0: palette P0, entry 0 -> -6 everywhere."""
    syms = np.zeros((3, 64), dtype=np.uint32)
    codes = orc.decode_codes(syms, 1024)
    assert (codes == 0xF).all()
    g = workloads.rng(99, 4)
    sc = workloads.scales(g, 1, 3, 1024)[0]
    x = g.standard_normal((2, 1024))
    y, bound = orc.gemv(syms, sc, x)
    for t in range(2):
        for r in range(3):
            exp = sum(-6.0 * 2.0 ** (int(sc[r, b]) - 127) * x[t, 32 * b:32 * b + 32].sum()
                      for b in range(32))
            assert abs(y[t, r] - exp) <= 1e-12 * bound[t, r]


def test_all_ones_stream(orc):
    """b = 3 always: the state fills with ones and sticks at 0xFFFF."""
    codes = orc.decode_codes(np.full((1, 4), 0xFFFFFFFF, dtype=np.uint32), 64)[0]
    vals = [orc.e2m1_value(c) for c in codes]
    head = [-0.0, -3, -1.5, 3, 1.5, -0.0]
    for v, h in zip(vals[:6], head):
        assert v == h and math.copysign(1, v) == math.copysign(1, h)
    assert all(v == 2 for v in vals[6:])


# ---------------------------------------------------------------- golden vectors

@pytest.mark.parametrize("case", _golden(), ids=lambda c: c[0])
def test_golden_vectors(orc, case):
    name, words, values, packed = case
    cols = 16 * len(words)
    codes = orc.decode_codes(words[None, :], cols)[0]
    if values is not None:
        got = [orc.e2m1_value(c) for c in codes]
        for a, b in zip(got, values):
            assert a == b and math.copysign(1, a) == math.copysign(1, b)
    if cols % 32 == 0:
        p, sc = orc.expand(words[None, None, :], np.full((1, 1, cols // 32), 127, np.uint8))
        assert p.tobytes() == packed
    else:
        got = bytes((int(codes[2 * j]) | (int(codes[2 * j + 1]) << 4)) for j in range(cols // 2))
        assert got == packed


def test_expand_copies_scales_and_nibble_order(orc):
    g = workloads.rng(99, 5)
    syms = workloads.symbols(g, 2, 3, 96)
    sc = workloads.scales(g, 2, 3, 96)
    p, sc2 = orc.expand(syms, sc)
    assert (sc2 == sc).all()
    codes = orc.decode_codes(syms, 96)
    assert ((p & 0xF) == codes[..., 0::2]).all()
    assert ((p >> 4) == codes[..., 1::2]).all()


# ---------------------------------------------------------------- GEMV arithmetic

def test_gemv_exact_rational(orc):
    """Weights and x are dyadic, so the exact sum is a Fraction; the fp64
    sequential sum must be within cols * 2^-53 * sum|w||x| of it."""
    g = workloads.rng(99, 6)
    rows, cols = 4, 96
    syms = workloads.symbols(g, 1, rows, cols)[0]
    sc = workloads.scales(g, 1, rows, cols)[0]
    x = workloads.activations(g, 2, cols, bf16=True).astype(np.float64)
    y, bound = orc.gemv(syms, sc, x)
    codes = orc.decode_codes(syms, cols)
    for t in range(2):
        for r in range(rows):
            exact = Fraction(0)
            mag = Fraction(0)
            for k in range(cols):
                v = Fraction(orc.e2m1_value(int(codes[r, k]))) * Fraction(2) ** (int(sc[r, k // 32]) - 127)
                exact += v * Fraction(float(x[t, k]))
                mag += abs(v) * abs(Fraction(float(x[t, k])))
            assert abs(Fraction(y[t, r]) - exact) <= Fraction(cols) * Fraction(2) ** -53 * mag
            assert Fraction(bound[t, r]) == mag or abs(Fraction(bound[t, r]) - mag) <= Fraction(cols) * Fraction(2) ** -53 * mag


def test_decode_values_scale_blocks(orc):
    """Each block of 32 weights carries its own UE8M0 scale."""
    g = workloads.rng(99, 7)
    syms = workloads.symbols(g, 1, 2, 128)[0]
    sc = workloads.scales(g, 1, 2, 128)[0]
    w = orc.decode_values(syms, sc)
    codes = orc.decode_codes(syms, 128)
    for r in range(2):
        for k in range(128):
            assert w[r, k] == orc.e2m1_value(int(codes[r, k])) * 2.0 ** (int(sc[r, k // 32]) - 127)


def _dense(orc, syms, sc):
    return orc.decode_values(syms, sc)


def test_moe_gemv_matches_numpy(orc):
    g = workloads.rng(99, 8)
    E, rows, cols, T, k = 5, 24, 96, 3, 2
    syms = workloads.symbols(g, E, rows, cols)
    sc = workloads.scales(g, E, rows, cols)
    x = workloads.activations(g, T, cols, bf16=True).astype(np.float64)
    ids = np.array([[0, 3], [4, 4], [2, 1]], dtype=np.int32)
    gw = np.array([[0.25, 0.75], [0.5, 0.5], [1.0, -2.0]])
    W = _dense(orc, syms, sc)
    # per-slot outputs
    y, b, skipped = orc.moe_gemv(syms, sc, x, ids)
    assert skipped == 0
    for t in range(T):
        for j in range(k):
            ref = W[ids[t, j]] @ x[t]
            refb = np.abs(W[ids[t, j]]) @ np.abs(x[t])
            np.testing.assert_allclose(y[t, j], ref, rtol=1e-12, atol=1e-12 * refb.max())
            np.testing.assert_allclose(b[t, j], refb, rtol=1e-12)
    # combined outputs
    yc, bc, _ = orc.moe_gemv(syms, sc, x, ids, gate_w=gw)
    for t in range(T):
        ref = sum(gw[t, j] * (W[ids[t, j]] @ x[t]) for j in range(k))
        refb = sum(abs(gw[t, j]) * (np.abs(W[ids[t, j]]) @ np.abs(x[t])) for j in range(k))
        np.testing.assert_allclose(yc[t], ref, rtol=1e-11, atol=1e-12 * refb.max())
        np.testing.assert_allclose(bc[t], refb, rtol=1e-12)
    # per-slot inputs
    xs = workloads.activations(g, T * k, cols, bf16=True).astype(np.float64).reshape(T, k, cols)
    ys, _, _ = orc.moe_gemv(syms, sc, xs, ids, gate_w=gw, x_per_slot=True)
    for t in range(T):
        ref = sum(gw[t, j] * (W[ids[t, j]] @ xs[t, j]) for j in range(k))
        np.testing.assert_allclose(ys[t], ref, rtol=1e-11, atol=1e-11)


def test_moe_gemv_empty_and_out_of_range_ids(orc):
    g = workloads.rng(99, 9)
    E, rows, cols = 2, 8, 64
    syms = workloads.symbols(g, E, rows, cols)
    sc = workloads.scales(g, E, rows, cols)
    x = workloads.activations(g, 2, cols, bf16=True)
    ids = np.array([[0, -1], [7, 1]], dtype=np.int32)
    y, b, skipped = orc.moe_gemv(syms, sc, x, ids)
    assert skipped == 1
    assert (y[0, 1] == 0).all() and (y[1, 0] == 0).all() and (b[1, 0] == 0).all()
    W = _dense(orc, syms, sc)
    np.testing.assert_allclose(y[1, 1], W[1] @ x[1].astype(np.float64), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- bf16 and SwiGLU

def test_round_bf16_cases(orc):
    one = 1.0
    assert orc.round_bf16(one) == one
    assert orc.round_bf16(1 + 2 ** -8) == 1.0                  # tie -> even
    assert orc.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6       # tie -> even (up)
    assert orc.round_bf16(1 + 2 ** -8 + 2 ** -30) == 1 + 2 ** -7
    assert orc.round_bf16(-(1 + 2 ** -8 + 2 ** -30)) == -(1 + 2 ** -7)
    assert orc.round_bf16(0.0) == 0.0
    assert orc.round_bf16(3.0 * 2 ** 100) == 3.0 * 2 ** 100


def test_round_bf16_matches_fp32_path_on_fp32_values(orc):
    """For inputs that are exact fp32 values there is no double rounding, so the
    bf16 conversion of the generator module must agree exactly."""
    g = np.random.default_rng(11)
    x = (g.standard_normal(4000) * np.exp2(g.integers(-20, 20, 4000))).astype(np.float32)
    ref = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(x)).astype(np.float64)
    got = np.array([orc.round_bf16(float(v)) for v in x])
    assert (got == ref).all()


def test_ffn_matches_numpy(orc):
    g = workloads.rng(99, 10)
    E, H, I, T, k = 3, 64, 32, 2, 2
    gs = workloads.symbols(g, E, 2 * I, H)
    ge = workloads.scales(g, E, 2 * I, H)
    ds = workloads.symbols(g, E, H, I)
    de = workloads.scales(g, E, H, I)
    x = workloads.activations(g, T, H, bf16=True).astype(np.float64)
    ids = np.array([[2, 0], [1, 2]], dtype=np.int32)
    gw = np.array([[0.6, 0.4], [0.3, 0.7]])
    y, b, h, skipped = orc.moe_ffn(gs, ge, ds, de, x, ids, gw)
    assert skipped == 0
    Wg, Wd = _dense(orc, gs, ge), _dense(orc, ds, de)
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            e = ids[t, j]
            z = Wg[e] @ x[t]
            gate, up = z[:I], z[I:]
            hh = gate / (1 + np.exp(-gate)) * up
            hb = np.array([orc.round_bf16(v) for v in hh])
            # the bf16 step: within half an ulp of the fp64 value (2^-8 relative
            # for normal values; half the smallest subnormal, 2^-134, below)
            assert (np.abs(hb - hh) <= np.maximum(np.abs(hh) * 2.0 ** -8, 2.0 ** -134)).all()
            np.testing.assert_allclose(h[t, j], hb, rtol=0, atol=0)
            acc += gw[t, j] * (Wd[e] @ hb)
        np.testing.assert_allclose(y[t], acc, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------- Viterbi vs brute force

def _brute_force(orc, target, d):
    n = len(target)
    seqs = np.arange(4 ** n, dtype=np.uint64)
    words = np.zeros(4 ** n, dtype=np.uint32)
    for j in range(n):
        words |= (((seqs >> np.uint64(2 * j)) & np.uint64(3)).astype(np.uint32) << np.uint32(2 * j))
    codes = orc.decode_codes(words[:, None], n)
    table = np.array([orc.e2m1_value(c) for c in range(16)])
    vals = table[codes]
    cost = np.zeros(4 ** n)
    for j in range(n):                    # same order of additions as the DP
        err = target[j] - vals[:, j]
        cost = cost + d[j] * err * err
    return cost, words


@pytest.mark.parametrize("n,seed,weighted", [(6, 0, False), (6, 1, True), (6, 2, True),
                                             (9, 3, False), (10, 4, True)])
def test_viterbi_matches_brute_force(orc, n, seed, weighted):
    g = np.random.default_rng(seed)
    target = g.standard_normal(n) * 3
    d = g.uniform(0.1, 4.0, n) if weighted else np.ones(n)
    syms, cost = orc.viterbi(target, d)
    bf, words = _brute_force(orc, target, d)
    assert cost == bf.min()
    # the returned path achieves the minimum
    w = np.uint32(sum(int(s) << (2 * j) for j, s in enumerate(syms)))
    assert bf[np.nonzero(words == w)[0][0]] == cost
    # compare sequences only where the minimum is unique
    if (bf == bf.min()).sum() == 1:
        assert int(words[np.argmin(bf)]) == int(w)


def test_viterbi_reproduces_an_encodable_target(orc):
    """A target that is itself a decoded sequence is reached at zero cost."""
    g = workloads.rng(99, 11)
    word = workloads.symbols(g, 1, 1, 16)[0, 0]
    codes = orc.decode_codes(word[None, :], 12)[0]
    target = np.array([orc.e2m1_value(c) for c in codes])
    syms, cost = orc.viterbi(target)
    assert cost == 0.0


# ---------------------------------------------------------------- router (top-k, softmax)

@pytest.mark.parametrize("E,k,seed", [(6, 2, 0), (7, 3, 1), (8, 8, 2), (5, 1, 3)])
def test_router_topk_brute_force(orc, E, k, seed):
    """The picked experts are the k-subset with the largest logit sum (brute
    force over all subsets; logits distinct), listed in descending logit order."""
    import itertools
    g = np.random.default_rng(seed)
    x = g.standard_normal((3, 16))
    w = g.standard_normal((E, 16))
    ids, gw, logits = orc.router_topk(x, w, k)
    for t in range(3):
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(Fraction(logits[t, e]) for e in c))
        assert sorted(ids[t].tolist()) == sorted(best)
        assert all(logits[t, ids[t, j]] > logits[t, ids[t, j + 1]] for j in range(k - 1))


def test_router_one_hot_rows(orc):
    """Router rows that are unit vectors: logit e is exactly x[perm[e]], so
    the picks are the largest entries of x (a library sort)."""
    g = np.random.default_rng(5)
    H, E, k = 32, 12, 4
    perm = g.permutation(H)[:E]
    w = np.zeros((E, H))
    w[np.arange(E), perm] = 1.0
    x = g.standard_normal((2, H))
    ids, gw, logits = orc.router_topk(x, w, k)
    for t in range(2):
        assert np.array_equal(logits[t], x[t, perm])
        assert ids[t].tolist() == list(np.argsort(-x[t, perm], kind="stable")[:k])


def test_router_ties_go_to_the_lower_id(orc):
    g = np.random.default_rng(6)
    row = g.standard_normal(8)
    w = np.stack([row * 0.5, row, row * 0.5, row, -row])   # experts 1 and 3 tie, then 0 and 2
    x = row[None, :]
    ids, gw, _ = orc.router_topk(x, w, 4)
    assert ids[0].tolist() == [1, 3, 0, 2]
    assert gw[0, 0] == gw[0, 1] and gw[0, 2] == gw[0, 3]


def test_router_gate_weights_closed_form(orc):
    """Softmax over the picked logits: weights sum to 1, and
    w_i / w_j = exp(l_i - l_j)."""
    g = np.random.default_rng(7)
    x = g.standard_normal((4, 24))
    w = g.standard_normal((10, 24)) * 0.3
    ids, gw, logits = orc.router_topk(x, w, 3)
    for t in range(4):
        assert abs(gw[t].sum() - 1.0) < 1e-15
        l = logits[t, ids[t]]
        for i in range(3):
            for j in range(3):
                assert math.isclose(gw[t, i] / gw[t, j], math.exp(l[i] - l[j]), rel_tol=1e-13)


# ---------------------------------------------------------------- E5M3 block scales (reading R14)
#
# XOR-Trellis article, "So what", the paragraph on the grouping format: the
# paper groups E2M1 elements under E5M3 block scales. The article gives no
# encoding; the reading is an unsigned 8-bit float laid out like the upper
# byte of an IEEE binary16 number without its sign. numpy's float16 is an
# independent implementation of that number format.

def _binary16_of_byte(c):
    return float(np.array([int(c) << 7], dtype=np.uint16).view(np.float16)[0])


def test_e5m3_scale_is_the_upper_byte_of_a_binary16(orc):
    """All 256 bytes: bias 15, subnormals at exponent 0, infinity and NaN at 31."""
    for c in range(256):
        want, got = _binary16_of_byte(c), orc.e5m3_scale(c)
        assert (np.isnan(want) and np.isnan(got)) or got == want, (c, got, want)
    assert orc.e5m3_scale(0x78) == 1.0 and orc.e5m3_scale(0x01) == 2.0 ** -17


def test_e5m3_powers_of_two_match_ue8m0(orc):
    """An E5M3 byte with mantissa 0 and exponent E is 2^(E - 15): the same
    weights as the UE8M0 byte E + 112 (the two decoders agree where the
    formats overlap)."""
    g = workloads.rng(99, 20)
    syms = workloads.symbols(g, 1, 6, 256)[0]
    E = g.integers(1, 31, size=(6, 8))
    w5 = orc.decode_values(syms, (E << 3).astype(np.uint8), scale_fmt="e5m3")
    w8 = orc.decode_values(syms, (E + 112).astype(np.uint8))
    assert np.array_equal(w5, w8)


def test_e5m3_moe_gemv_exact_rational(orc):
    """Routed GEMV with E5M3 scales covering every mantissa, subnormals and
    a wide exponent range: within cols * 2^-53 * sum|w||x| of the exact
    Fraction sum of (E2M1 value x binary16 value of the scale byte) x x."""
    g = workloads.rng(99, 21)
    E, rows, cols, T, k = 3, 5, 96, 2, 2
    syms = workloads.symbols(g, E, rows, cols)
    sc = np.concatenate([g.integers(0, 8, size=(E, rows, 1)),           # subnormals
                         g.integers(8, 248, size=(E, rows, cols // 32 - 1))], axis=2).astype(np.uint8)
    x = workloads.activations(g, T, cols, bf16=True).astype(np.float64)
    ids = np.array([[0, 2], [1, 0]], np.int32)
    gw = np.array([[0.5, 0.25], [1.0, 2.0]])
    y, bound, skipped = orc.moe_gemv(syms, sc, x, ids, gate_w=gw, scale_fmt="e5m3")
    assert skipped == 0
    codes = orc.decode_codes(syms.reshape(E * rows, cols // 16), cols).reshape(E, rows, cols)
    for t in range(T):
        for r in range(rows):
            exact, mag = Fraction(0), Fraction(0)
            for j in range(k):
                e = int(ids[t, j])
                for c in range(cols):
                    v = Fraction(orc.e2m1_value(int(codes[e, r, c]))) * Fraction(_binary16_of_byte(sc[e, r, c // 32]))
                    exact += Fraction(gw[t, j]) * v * Fraction(float(x[t, c]))
                    mag += abs(Fraction(gw[t, j]) * v) * abs(Fraction(float(x[t, c])))
            assert abs(Fraction(y[t, r]) - exact) <= Fraction(2 * cols) * Fraction(2) ** -53 * mag


def _dense_e5m3(orc, syms, sc):
    """Weights rebuilt from the decoded E2M1 codes and numpy's binary16 value
    of each scale byte (independent of the oracle's E5M3 decoder)."""
    E, rows, wpr = syms.shape
    cols = wpr * 16
    codes = orc.decode_codes(syms.reshape(E * rows, wpr), cols).reshape(E, rows, cols)
    val = np.array([orc.e2m1_value(c) for c in range(16)])[codes]
    s16 = np.array([_binary16_of_byte(c) for c in range(256)])[sc]
    return val * np.repeat(s16, 32, axis=2)


def test_ffn_e5m3_matches_numpy(orc):
    """The layer with E5M3 scales (subnormal and normal blocks) against numpy
    on weights rebuilt with binary16 scale values."""
    g = workloads.rng(99, 22)
    E, H, I, T, k = 3, 64, 32, 2, 2
    gs = workloads.symbols(g, E, 2 * I, H)
    ge = g.integers(0x40, 0x90, size=(E, 2 * I, H // 32)).astype(np.uint8)
    ds = workloads.symbols(g, E, H, I)
    de = g.integers(0x60, 0x88, size=(E, H, I // 32)).astype(np.uint8)
    ge[0, :4, 0] = np.arange(4)   # subnormal and zero scales
    x = workloads.activations(g, T, H, bf16=True).astype(np.float64)
    ids = np.array([[2, 0], [1, 2]], dtype=np.int32)
    gw = np.array([[0.6, 0.4], [0.3, 0.7]])
    y, b, h, skipped = orc.moe_ffn(gs, ge, ds, de, x, ids, gw, scale_fmt="e5m3")
    assert skipped == 0
    Wg, Wd = _dense_e5m3(orc, gs, ge), _dense_e5m3(orc, ds, de)
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            e = ids[t, j]
            z = Wg[e] @ x[t]
            hh = z[:I] / (1 + np.exp(-z[:I])) * z[I:]
            hb = np.array([orc.round_bf16(v) for v in hh])
            np.testing.assert_allclose(h[t, j], hb, rtol=0, atol=0)
            acc += gw[t, j] * (Wd[e] @ hb)
        np.testing.assert_allclose(y[t], acc, rtol=1e-11, atol=1e-11)
