"""Bit-exact checks of the weights that the fused kernels decode.

These tests check decoded weights against the oracle's sequential decode
(XOR-Trellis article, bullet "XOR-Trellis FP4 decoder"; HEPH abstract,
UE8M0 block scales). The usual GEMV tolerance is too loose to catch a few
wrong weights in a row, so these checks are exact.

GEMV: with a one-hot activation x = e_c, every output row has a single
non-zero term.
  * The activation 1.0 reaches the matrix cores as an exact FP8 value, and
    the low term of its split is 0.
  * The FP4 x FP8 product is exact, and adding zeros is exact.
  * So y[m] equals the decoded weight W[m][c] = value x 2^(e-127) bit for
    bit. The only thing y cannot show is the sign of a zero weight.
  * Sweeping c over every column checks every weight.
With gate weights that are powers of two, every partial sum of a slot
combine is a float32 number, so y is exact there as well.

Layer: the layer kernels do not expose the gate/up GEMV outputs. They hand
h = bf16(silu(gate) x up) to the down projection. Three crafted layers make
the decoded weights visible through h and y:
  * Up rows set to the all-zero symbol stream, which decodes to
    -6 x 2^(e-127) at every column. h then depends on the gate weight
    alone. At a fixed block scale, the possible gate values give h values
    at least 0.9 % apart (silu(-0.75) and silu(-2) are the closest pair),
    and bf16 rounding moves h by at most 2^-9. So
    |h - h(true gate)| <= 2^-8 |h| holds exactly when the decoded gate
    weight is the true one.
  * Gate rows set to the all-zero stream. h is then linear in the up
    weight.
  * Gate rows whose 8-symbol windows are chosen so that, at the probed
    column, exactly one row r decodes to a non-zero value. h is then
    non-zero only at row r, and
    y = sum_j gw_j W_down_j[:, r] h_j[r] exactly. Every partial sum of
    those terms is a float32 number, so the order of the atomic adds does
    not matter. This exposes column r of every active down matrix.
"""
import numpy as np
import pytest

import workloads
from helpers import announce, dev, silu

pytestmark = pytest.mark.gpu


def _mismatch(got, want, what):
    bad = got != want
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outputs differ from the oracle's decoded "
                           f"weights; first at {tuple(int(i[0]) for i in np.nonzero(bad))}: "
                           f"{got[bad][0]!r} vs {want[bad][0]!r}")


def _eye(n):
    import torch
    return torch.eye(n, dtype=torch.bfloat16, device="cuda")


def _rows_of(eye, cols):
    import torch
    cols = np.asarray(cols)
    if cols.size == 1:
        c = int(cols.reshape(-1)[0])
        return eye[c:c + 1]
    return eye.index_select(0, torch.from_numpy(cols.reshape(-1).astype(np.int64)).cuda())


# ---------------------------------------------------------------- routed GEMV, one-hot sweeps

def _gemv_sweep(tq, orc, E, rows, cols, T, k, per_slot, weighted, seed, mx=False):
    """Every column of E matrices through moe_gemv (or mxfp4_moe_gemv on
    oracle-expanded weights), T*k or T one-hot columns per call."""
    import torch
    g = workloads.rng(611, seed, E * 100 + k, rows * 100000 + cols)
    syms = workloads.symbols(g, E, rows, cols)
    sc = workloads.scales(g, E, rows, cols)
    W = orc.decode_values(syms, sc)
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    gw = np.tile(np.ldexp(1.0, -np.arange(k)), (T, 1)).astype(np.float32) if weighted else None
    if mx:
        codes, sc2 = orc.expand(syms, sc)
        wd = (dev(codes), dev(sc2))
        call = tq.mxfp4_moe_gemv
    else:
        wd = (dev(syms), dev(sc))
        call = tq.moe_gemv
    dgw = dev(gw) if weighted else None
    eye = _eye(cols)
    ws = tq.gemv_workspace(E, rows, cols, T, k)
    n_per = T * k if per_slot else T
    starts = list(range(0, cols, n_per))
    # with per-slot activations each column reaches one slot, i.e. one
    # expert per call: E passes, the expert ids rotated by one each pass
    passes = [(ids + p) % E for p in range(E if per_slot else 1)]
    shape = (T, rows) if weighted else (T, k, rows)
    Y = torch.empty((len(passes), len(starts)) + shape, dtype=torch.float32, device="cuda")
    probe = np.empty((len(starts), n_per), np.int64)
    for p, ids_p in enumerate(passes):
        dids = dev(ids_p.astype(np.int32))
        for n, c0 in enumerate(starts):
            probe[n] = (c0 + np.arange(n_per)) % cols
            x = _rows_of(eye, probe[n]).reshape((T, k, cols) if per_slot else (T, cols))
            call(*wd, x, dids, dgw, x_per_slot=per_slot, y=Y[p, n], workspace=ws)
    Y = Y.cpu().numpy()
    assert int(ws[:8].view(torch.int32)[1].item()) == 0, "a wait timed out"
    C = probe.reshape(len(starts), T, k) if per_slot else np.repeat(probe[:, :, None], k, axis=2)
    covered = np.zeros((E, cols), bool)
    wants = []
    for ids_p in passes:
        want = W[ids_p[None, :, :], :, C]                 # [calls, T, k, rows]
        if weighted:
            want = (want * gw[None, :, :, None]).sum(axis=2)
        wants.append(want.astype(np.float32))
        covered[np.broadcast_to(ids_p[None], C.shape), C] = True
    return Y, np.stack(wants), covered


@pytest.mark.parametrize("E,rows,cols,T,k,per_slot,weighted,what", [
    (8, 64, 2880, 1, 8, False, False, "one resident token, aligned rows, K = 2880"),
    (8, 80, 2912, 1, 8, False, False, "one resident token, unaligned rows, partial row tile"),
    (8, 64, 4096, 1, 8, False, False, "one resident token at the window limit K = 4096"),
    (4, 32, 4128, 1, 4, False, False, "one token beyond one register window (per-item split)"),
    (8, 64, 2880, 128, 8, False, True, "128 tokens, split once per call, slot-order combine"),
    (8, 64, 4096, 128, 8, False, False, "128 tokens at K = 4096"),
    (32, 48, 2880, 32, 32, True, False, "per-slot activations, 1024 slots per call"),
    (4, 32, 8192, 128, 4, False, False, "K = 8192: two register windows, per-item split"),
    (4, 48, 8192, 32, 4, True, True, "K = 8192 per-slot with combine"),
])
def test_gemv_one_hot_every_column(trellis_lib, orc, E, rows, cols, T, k, per_slot, weighted, what):
    announce(f"exact gemv sweep: {what} (E={E} {rows}x{cols} T={T} k={k})")
    Y, want, covered = _gemv_sweep(trellis_lib, orc, E, rows, cols, T, k, per_slot, weighted, seed=cols + T)
    assert covered.all(), "the sweep must reach every column of every expert"
    _mismatch(Y, want, what)


@pytest.mark.parametrize("E,rows,cols,T,k,per_slot", [
    (32, 48, 2880, 32, 32, True),
    (8, 64, 2880, 1, 8, False),
])
def test_mxfp4_gemv_one_hot_every_column(trellis_lib, orc, E, rows, cols, T, k, per_slot):
    """The expanded-MXFP4 path reads the oracle's expanded nibbles as the matrix-core operand."""
    announce(f"exact mxfp4 gemv sweep E={E} {rows}x{cols} T={T} k={k} per_slot={per_slot}")
    Y, want, covered = _gemv_sweep(trellis_lib, orc, E, rows, cols, T, k, per_slot, False, seed=7 + T, mx=True)
    assert covered.all()
    _mismatch(Y, want, "mxfp4 gemv")


# ---------------------------------------------------------------- whole layer, crafted streams

def _state_halfword(S):
    """The 8 symbols (one half of a 32-bit word) after which the decoder's
    state is S: the last symbol is S's low two bits."""
    return sum(((S >> (14 - 2 * j)) & 3) << (2 * j) for j in range(8))


def _states(orc):
    """A state whose weight is 0 and one whose weight is 2 (at scale 1)."""
    vals = np.array([orc.state_value(s) for s in range(1 << 16)])
    return int(np.nonzero(vals == 0.0)[0][0]), int(np.nonzero(vals == 2.0)[0][0])


def _candidate_gap(orc):
    """Smallest relative gap between silu(v * 2^(e-127)) of distinct E2M1
    values v, over the scale bytes the workloads use."""
    vals = np.unique([orc.e2m1_value(c) for c in range(16)])
    gap = np.inf
    for e in range(workloads.SCALE_LO, workloads.SCALE_HI + 1):
        s = np.sort(silu(vals * 2.0 ** (e - 127)))
        d = np.diff(s) / np.maximum(np.abs(s[1:]), np.abs(s[:-1]))
        gap = min(gap, float(d.min()))
    return gap


def _ffn_dev(tq, L, orc=None, mx_experts=None):
    """The layer's weights on the device: trellis streams, or (mx_experts
    given) the MXFP4 codes and scales the oracle expands for those experts
    (the other experts are never read)."""
    if mx_experts is None:
        return [dev(L.gu_syms), dev(L.gu_scales), dev(L.dn_syms), dev(L.dn_scales)]
    from test_gpu_mxfp4 import _expand
    gc, gs = _expand(orc, L.gu_syms, L.gu_scales, mx_experts)
    dc, ds = _expand(orc, L.dn_syms, L.dn_scales, mx_experts)
    return [dev(gc), dev(gs), dev(dc), dev(ds)]


def _run_layer(tq, wd, eye, col_lists, ids, gw, I, H, ws, mx=False, fmt="ue8m0"):
    """One layer call per list of probe columns (one token each); returns h, y."""
    import torch
    n, T = len(col_lists), len(col_lists[0])
    k = ids.shape[1]
    Hh = torch.empty((n, T, k, I), dtype=torch.bfloat16, device="cuda")
    Yy = torch.empty((n, T, H), dtype=torch.float32, device="cuda")
    dids, dgw = dev(ids), dev(gw)
    fn = tq.mxfp4_moe_ffn if mx else tq.moe_ffn_e5m3 if fmt == "e5m3" else tq.moe_ffn
    for i, cs in enumerate(col_lists):
        fn(*wd, _rows_of(eye, cs), dids, dgw, h=Hh[i], y=Yy[i], workspace=ws)
    h = Hh.float().cpu().numpy()
    y = Yy.cpu().numpy()
    assert int(ws[:8].view(torch.int32)[1].item()) == 0, "a wait timed out"
    return h, y


# the scale byte whose value is 1 in each format (E5M3: exponent 15, mantissa 0)
ONE = {"ue8m0": 127, "e5m3": 15 << 3}


def _layer_setup(cfg, T, seed, fmt="ue8m0"):
    L = workloads.moe_layer(cfg, layer_id=seed)
    if fmt == "e5m3":
        g = workloads.rng(616, cfg.config_id, seed)
        E = L.gu_syms.shape[0]
        L.gu_scales = workloads.scales_e5m3(g, E, 2 * cfg.inter, cfg.hidden)
        L.dn_scales = workloads.scales_e5m3(g, E, cfg.hidden, cfg.inter)
    act = np.array(L.ids[0][:cfg.k], np.int32)           # k distinct experts
    ids = np.tile(act, (T, 1)).astype(np.int32)
    gw = np.full((T, cfg.k), 1.0 / cfg.k, np.float32)    # a power of two for k = 4, 8
    return L, act, ids, gw


def _stage1_probe(tq, orc, cfg, T, which, seed=0, mx=False, fmt="ue8m0"):
    """which = 'gate': up rows of the active experts are the all-zero stream;
    'up': gate rows are. h at every column identifies the other weight.
    mx: the same weights expanded to MXFP4 by the oracle, through the
    layer on expanded weights."""
    import torch
    H, I, k = cfg.hidden, cfg.inter, cfg.k
    L, act, ids, gw = _layer_setup(cfg, T, seed, fmt)
    zero_rows = slice(I, 2 * I) if which == "gate" else slice(0, I)
    for e in act:
        L.gu_syms[e, zero_rows] = 0
        if fmt == "e5m3":
            # E5M3 scales reach ~15: a zero-stream gate row would decode to
            # about -90, where silu's exp leaves the fp32 range; at scale 1
            # the constant gate is -6
            L.gu_scales[e, zero_rows] = ONE[fmt]
    if which == "gate":
        assert fmt == "ue8m0", "the gate probe's gap bound is derived for UE8M0 scales"
        assert _candidate_gap(orc) > 2.0 ** -7   # > 2^-8 (accepted) + 2^-9 (bf16 rounding) + margin
    wd = _ffn_dev(tq, L, orc, act if mx else None)
    eye = _eye(H)
    ws = tq.ffn_workspace(cfg.n_exp, H, I, T, k)
    lists = [(c0 + np.arange(T)) % H for c0 in range(0, H, T)]
    h, _ = _run_layer(tq, wd, eye, lists, ids, gw, I, H, ws, mx, fmt)
    probe = np.concatenate(lists)                       # column of each (call, token)
    h = h.reshape(-1, k, I)
    worst = 0.0
    for j, e in enumerate(act):
        Wgu = orc.decode_values(L.gu_syms[e], L.gu_scales[e], scale_fmt=fmt)   # [2I, H]
        g = Wgu[:I][:, probe].T                                     # [probes, I]
        u = Wgu[I:][:, probe].T
        ref = silu(g) * u
        got = h[:, j, :]
        zero = ref == 0
        assert (got[zero] == 0).all(), f"{which} probe, slot {j}: h not exactly 0 where the weight is 0"
        rel = np.abs(got[~zero] - ref[~zero]) / np.abs(ref[~zero])
        if rel.size:
            worst = max(worst, float(rel.max()))
            if rel.max() > 2.0 ** -8:
                i = np.argmax(rel)
                pos = np.argwhere(~zero)[i]
                raise AssertionError(f"{which} probe, expert {e}: decoded weight at row {pos[1]} column "
                                     f"{probe[pos[0]]} differs (h {got[tuple(pos)]!r}, expected "
                                     f"{ref[tuple(pos)]!r})")
    torch.cuda.empty_cache()
    print(f"{which}: {len(probe)} columns x {I} rows x {k} experts, worst relative h error {worst:.2e}")


def _down_probe(tq, orc, cfg, T, seed=0, mx=False, fmt="ue8m0"):
    """Crafted gate rows make h one-hot at one row r per token; y then exposes
    column r of every active down matrix exactly (mx: on the weights
    expanded to MXFP4 by the oracle)."""
    import torch
    H, I, k = cfg.hidden, cfg.inter, cfg.k
    L, act, ids, gw = _layer_setup(cfg, T, seed, fmt)
    s_zero, s_two = _states(orc)
    hw_zero, hw_two = _state_halfword(s_zero), _state_halfword(s_two)
    n_probe_cols = H // 8                               # windows of 8 symbols end at 8n + 7
    n_st = -(-I // n_probe_cols)                        # crafted stacks needed to cover all I rows
    P = -(-I // n_st)                                   # probes per stack
    for e in act:
        L.gu_syms[e, I:] = 0                            # up rows: -6 everywhere
        L.gu_scales[e] = ONE[fmt]
    wd = _ffn_dev(tq, L, orc, act if mx else None)
    eye = _eye(H)
    ws = tq.ffn_workspace(cfg.n_exp, H, I, T, k)
    Wdn = [orc.decode_values(L.dn_syms[e], L.dn_scales[e], scale_fmt=fmt) for e in act]   # [H, I] each
    h_two = orc.round_bf16(float(silu(2.0) * -6.0))
    r_all = np.arange(I)
    for sigma in range(n_st):
        half = np.full((I, n_probe_cols), hw_zero, np.uint16)
        mine = r_all % n_st == sigma
        half[r_all[mine], r_all[mine] // n_st] = hw_two
        gate = half.view(np.uint32)                     # [I, H/16], little-endian halves
        # the crafting itself, checked on the oracle: at column 8n+7 only row n*n_st+sigma is non-zero
        dec = orc.decode_values(gate[None], np.full((1, I, H // 32), ONE[fmt], np.uint8), scale_fmt=fmt)[0][:, 7::8]
        want_nz = np.zeros_like(dec, bool)
        want_nz[r_all[mine], r_all[mine] // n_st] = True
        assert np.array_equal(dec != 0, want_nz) and (dec[want_nz] == 2.0).all()
        g_dev = dev(orc.expand(gate[None], np.full((1, I, H // 32), 127, np.uint8))[0][0]) if mx else dev(gate)
        for e in act:
            wd[0][int(e), :I] = g_dev
        lists = [(p0 + np.arange(T)) % P for p0 in range(0, P, T)]
        h, y = _run_layer(tq, wd, eye, [8 * p + 7 for p in lists], ids, gw, I, H, ws, mx, fmt)
        n_of = np.concatenate(lists)
        r_of = n_of * n_st + sigma
        h = h.reshape(-1, k, I)
        y = y.reshape(-1, H)
        for q, r in enumerate(r_of):
            hq = h[q]
            if r >= I:
                assert (hq == 0).all() and (y[q] == 0).all()
                continue
            others = np.ones(I, bool)
            others[r] = False
            assert (hq[:, others] == 0).all(), f"stack {sigma}: h not one-hot at row {r}"
            assert (np.abs(hq[:, r] - h_two) <= 2.0 ** -8 * abs(h_two)).all(), f"h at row {r}: {hq[:, r]}"
        live = r_of < I
        rr = r_of[live]
        terms = np.stack([gw[0, j] * Wdn[j][:, rr].T * h[live, j, rr][:, None] for j in range(k)])  # [k, q, H]
        # every partial sum is a float32 number: all terms are multiples of
        # their smallest lowest set bit u and the sum of magnitudes is < 2^24 u
        m, ex = np.frexp(terms)
        M = np.abs(m * 2.0 ** 53).astype(np.int64)
        with np.errstate(divide="ignore"):
            lsb = np.where(M != 0, np.log2((M & -M).astype(np.float64)) + ex - 53, np.inf)
        u = lsb.min(axis=0)
        fits = np.abs(terms).sum(axis=0) < 2.0 ** (24 + np.where(np.isfinite(u), u, 0))
        assert fits.all(), "crafted probe terms too spread for an exact float32 sum"
        want = terms.sum(axis=0).astype(np.float32)
        _mismatch(y[live], want, f"down projection, stack {sigma}")
    torch.cuda.empty_cache()
    print(f"down: {n_st} stacks x {P} probes, {k} experts x {H} rows exact")


LAYERS = {
    "moe32": workloads.MOE_32E,
    "moe128": workloads.MoEConfig(4, "128 experts top-8 H=4096 I=1536", 128, 4096, 1536, 8, 1, True),
    # hidden and inter not multiples of 64: the general layer kernel's single-token path
    # (unaligned rows, pre-decoded down projection)
    "odd": workloads.MoEConfig(95, "8 experts top-4 H=2912 I=1440", 8, 2912, 1440, 4, 1, True),
    # one piece per row: waves of the single-token kernel without pieces of their own
    "small": workloads.MoEConfig(96, "8 experts top-4 H=256 I=128", 8, 256, 128, 4, 1, True),
}


@pytest.mark.parametrize("layer,T", [("moe32", 1), ("moe32", 128), ("moe128", 1), ("moe128", 32), ("odd", 1),
                                     ("small", 1)])
@pytest.mark.parametrize("which", ["gate", "up"])
def test_layer_gate_up_decode_exact(trellis_lib, orc, layer, T, which):
    cfg = LAYERS[layer]
    announce(f"exact layer stage-1 probe ({which}) {cfg.name} T={T}")
    _stage1_probe(trellis_lib, orc, cfg, T, which)


@pytest.mark.parametrize("layer,T", [("moe32", 1), ("moe32", 128), ("moe128", 1), ("moe128", 32), ("odd", 1),
                                     ("small", 1)])
def test_layer_down_decode_exact(trellis_lib, orc, layer, T):
    cfg = LAYERS[layer]
    announce(f"exact layer down probe {cfg.name} T={T}")
    _down_probe(trellis_lib, orc, cfg, T)


# Expanded MXFP4 weights (expand mode): the same probes through
# trellis_mxfp4_moe_ffn, on codes the oracle expands. One token runs the
# single-token kernel where it takes the shape (moe32, small), the general
# layer kernel otherwise (moe128 at eight slots, odd widths).
@pytest.mark.parametrize("layer,T", [("moe32", 1), ("small", 1), ("moe128", 1), ("odd", 1), ("moe32", 8)])
@pytest.mark.parametrize("which", ["gate", "up"])
def test_mxfp4_layer_gate_up_exact(trellis_lib, orc, layer, T, which):
    cfg = LAYERS[layer]
    announce(f"exact mxfp4 layer stage-1 probe ({which}) {cfg.name} T={T}")
    _stage1_probe(trellis_lib, orc, cfg, T, which, mx=True)


@pytest.mark.parametrize("layer,T", [("moe32", 1), ("small", 1), ("moe128", 1), ("odd", 1), ("moe32", 8)])
def test_mxfp4_layer_down_exact(trellis_lib, orc, layer, T):
    cfg = LAYERS[layer]
    announce(f"exact mxfp4 layer down probe {cfg.name} T={T}")
    _down_probe(trellis_lib, orc, cfg, T, mx=True)


# E5M3 block scales (the XOR-Trellis article's grouping format, read as an
# unsigned binary16 upper byte): the up and down probes through
# trellis_moe_ffn_e5m3. One token runs the single-token kernel (moe32,
# small), eight tokens the general layer kernel.
@pytest.mark.parametrize("layer,T", [("moe32", 1), ("small", 1), ("moe32", 8)])
def test_e5m3_layer_up_exact(trellis_lib, orc, layer, T):
    cfg = LAYERS[layer]
    announce(f"exact e5m3 layer stage-1 probe (up) {cfg.name} T={T}")
    _stage1_probe(trellis_lib, orc, cfg, T, "up", fmt="e5m3")


@pytest.mark.parametrize("layer,T", [("moe32", 1), ("small", 1), ("moe32", 8)])
def test_e5m3_layer_down_exact(trellis_lib, orc, layer, T):
    cfg = LAYERS[layer]
    announce(f"exact e5m3 layer down probe {cfg.name} T={T}")
    _down_probe(trellis_lib, orc, cfg, T, fmt="e5m3")
