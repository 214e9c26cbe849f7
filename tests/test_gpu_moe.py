"""Fused trellis-decode MoE GEMV / FFN on the GPU against the oracle.

Bar: every output within 2e-3 * sum |w| |x| of the oracle's fp64 result. For
the whole layer each stage is gated on its own: the gate_up/SwiGLU stage by
h, the down stage by the oracle fed the GPU's own h (so bf16 rounding flips
in h do not compound); the end-to-end difference is printed, not gated.
"""
import numpy as np
import pytest

import workloads
from helpers import TOL, announce, check_tol, dev, sigmoid, silu, x_dev

pytestmark = pytest.mark.gpu


def _gemv_case(tq, orc, E, rows, cols, T, k, bf16, weighted, per_slot, ids=None, seed=0):
    g = workloads.rng(601, seed, E * 1000 + rows, cols * 100 + T * 10 + k)
    syms = workloads.symbols(g, E, rows, cols)
    sc = workloads.scales(g, E, rows, cols)
    x = workloads.activations(g, T * (k if per_slot else 1), cols, bf16)
    x = x.reshape((T, k, cols) if per_slot else (T, cols))
    if ids is None:
        ids, gw = workloads.routing_topk(g, T, E, min(k, E))
        if ids.shape[1] < k:
            ids = np.concatenate([ids, -np.ones((T, k - ids.shape[1]), np.int32)], axis=1)
            gw = np.concatenate([gw, np.zeros((T, k - gw.shape[1]), np.float32)], axis=1)
    else:
        gw = g.uniform(0.1, 1.0, size=ids.shape).astype(np.float32)
    y = tq.moe_gemv(dev(syms), dev(sc), x_dev(x, bf16), dev(ids),
                    dev(gw) if weighted else None, x_per_slot=per_slot).cpu().numpy()
    y_ref, bound, skipped = orc.moe_gemv(syms, sc, x, ids, gate_w=gw if weighted else None,
                                        x_per_slot=per_slot)
    return y, y_ref, bound, skipped


def test_single_matrix_fp32(trellis_lib, orc):
    """The 256 x 1024 single-matrix workload: fp32 x, batch 1, one expert."""
    announce("gemv single matrix 256x1024 fp32")
    c = workloads.SINGLE_MATRIX
    g = workloads.rng(c["config_id"], 0)
    syms = workloads.symbols(g, 1, c["rows"], c["cols"])
    sc = workloads.scales(workloads.rng(c["config_id"], 1), 1, c["rows"], c["cols"])
    x = workloads.activations(workloads.rng(c["config_id"], workloads.T_X), 1, c["cols"], bf16=False)
    ids = np.zeros((1, 1), np.int32)
    y = trellis_lib.moe_gemv(dev(syms), dev(sc), x_dev(x, False), dev(ids)).cpu().numpy()
    y_ref, bound, _ = orc.moe_gemv(syms, sc, x, ids)
    r = check_tol(y, y_ref, bound, "single matrix")
    print(f"worst err/tol {r:.4f}")


@pytest.mark.parametrize("E,rows,cols,T,k,bf16,weighted,per_slot", [
    (5, 48, 96, 3, 2, True, False, False),      # partial 128-K chunk, 3 row tiles
    (5, 48, 96, 3, 2, True, True, False),
    (5, 48, 96, 3, 2, False, True, True),
    (4, 64, 2880, 1, 4, True, False, False),    # K = 2880: 90 blocks, ragged last chunk
    (4, 64, 2880, 1, 4, True, True, False),
    (16, 80, 256, 4, 4, True, True, False),
    (16, 64, 256, 8, 4, True, True, False),
    (16, 64, 256, 16, 4, True, False, False),
    (16, 64, 256, 16, 4, True, True, False),
    (16, 32, 512, 32, 4, True, True, False),
    (16, 32, 512, 32, 4, True, False, False),
    (3, 16, 32, 32, 8, False, True, True),      # one block per row; T*k = 256 slots over 3 experts
    # one token, shared x, per-slot outputs: the single-token GEMV kernel
    (5, 48, 192, 1, 3, True, False, False),     # three row tiles, one piece per row
    (40, 1024, 256, 1, 32, False, False, False),   # 32 slots: eight tiles per workgroup
    (1, 256, 1024, 1, 1, False, False, False),  # the single-matrix benchmark shape
])
def test_moe_gemv(trellis_lib, orc, E, rows, cols, T, k, bf16, weighted, per_slot):
    announce(f"gemv E={E} {rows}x{cols} T={T} k={k} bf16={bf16} w={weighted} per_slot={per_slot}")
    y, y_ref, bound, _ = _gemv_case(trellis_lib, orc, E, rows, cols, T, k, bf16, weighted, per_slot)
    check_tol(y, y_ref, bound, "moe_gemv")


def test_moe_gemv_dead_and_duplicate_slots(trellis_lib, orc):
    announce("gemv dead and duplicate slots")
    import torch
    E, rows, cols = 4, 32, 128
    ids = np.array([[0, -1, 2], [7, 1, 1], [3, 3, -5]], dtype=np.int32)   # 7 >= E is skipped
    for weighted in (False, True):
        for per_slot in (False, True):
            y, y_ref, bound, skipped = _gemv_case(trellis_lib, orc, E, rows, cols, 3, 3, True, weighted,
                                                  per_slot, ids=ids, seed=1)
            assert skipped == 1
            check_tol(y, y_ref, bound, f"dead/dup weighted={weighted} per_slot={per_slot}")
            if not weighted:
                assert (y[0, 1] == 0).all() and (y[1, 0] == 0).all() and (y[2, 2] == 0).all()
    # the skipped-slot count is reported in the first workspace word
    g = workloads.rng(602, 0)
    syms = workloads.symbols(g, E, rows, cols)
    sc = workloads.scales(g, E, rows, cols)
    ws = trellis_lib.gemv_workspace(E, rows, cols, 3, 3)
    trellis_lib.moe_gemv(dev(syms), dev(sc), x_dev(workloads.activations(g, 3, cols, True), True), dev(ids),
                         workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32)[0]) == 1


def test_moe_gemv_one_token_dead_duplicate_and_empty(trellis_lib, orc):
    """One token through the single-token GEMV kernel: a skipped id, an empty
    slot, a duplicated expert; then a call where no slot routes anywhere
    (every output row zero, y starting as garbage)."""
    announce("gemv one token: dead, duplicate and all-empty slots")
    import torch
    E, rows, cols = 4, 64, 512
    ids = np.array([[7, -1, 2, 2]], dtype=np.int32)
    y, y_ref, bound, skipped = _gemv_case(trellis_lib, orc, E, rows, cols, 1, 4, True, False, False, ids=ids,
                                          seed=3)
    assert skipped == 1
    check_tol(y, y_ref, bound, "one token dead/dup")
    assert (y[0, 0] == 0).all() and (y[0, 1] == 0).all() and np.array_equal(y[0, 2], y[0, 3])
    g = workloads.rng(604, 0)
    syms, sc = workloads.symbols(g, E, rows, cols), workloads.scales(g, E, rows, cols)
    ws = trellis_lib.gemv_workspace(E, rows, cols, 1, 2)
    yd = torch.full((1, 2, rows), 3.0, dtype=torch.float32, device="cuda")
    trellis_lib.moe_gemv(dev(syms), dev(sc), x_dev(workloads.activations(g, 1, cols, True), True),
                         dev(np.array([[-1, 9]], np.int32)), y=yd, workspace=ws)
    torch.cuda.synchronize()
    assert (yd.cpu().numpy() == 0).all()
    assert int(ws[:4].view(torch.int32)[0]) == 1


def test_moe_gemv_repeat_is_deterministic(trellis_lib, orc):
    announce("gemv determinism")
    import torch
    g = workloads.rng(603, 0)
    E, rows, cols, T, k = 8, 64, 1024, 4, 4
    syms, sc = dev(workloads.symbols(g, E, rows, cols)), dev(workloads.scales(g, E, rows, cols))
    x = x_dev(workloads.activations(g, T, cols, True), True)
    ids, gw = workloads.routing_topk(g, T, E, k)
    a = trellis_lib.moe_gemv(syms, sc, x, dev(ids), dev(gw))
    b = trellis_lib.moe_gemv(syms, sc, x, dev(ids), dev(gw))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---------------------------------------------------------------- whole layer

def _h_tolerance(g_ref, u_ref, bg, bu):
    """Bound on |h_gpu - silu(g)u| from the per-row GEMV bounds plus bf16 rounding."""
    sig = sigmoid(g_ref)
    dsilu = np.abs(sig * (1.0 + g_ref * (1.0 - sig)))
    tg, tu = TOL * bg, TOL * bu
    h = silu(g_ref) * u_ref
    return (dsilu + 0.6 * tg) * (np.abs(u_ref) + tu) * tg + (np.abs(silu(g_ref)) + tg) * tu \
        + np.abs(h) * 2.0 ** -7 + 1e-30


def _check_layer(tq, orc, layer, rows_gu=None, rows_dn=None, run=None):
    """Run the layer on the GPU (trellis weights, or run(layer) -> (y, h)); check h
    on sampled (slot, i) and y on sampled rows."""
    import torch
    cfg = layer.cfg
    E = layer.gu_syms.shape[0]
    I, H = cfg.inter, cfg.hidden
    T, k = layer.ids.shape
    if run is None:
        y, h = tq.moe_ffn(dev(layer.gu_syms), dev(layer.gu_scales), dev(layer.dn_syms), dev(layer.dn_scales),
                          x_dev(layer.x, cfg.x_bf16), dev(layer.ids), dev(layer.gate_w))
    else:
        y, h = run(layer)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    h = h.float().cpu().numpy()
    ii = np.arange(I) if rows_gu is None else rows_gu
    x64 = layer.x.astype(np.float64)
    worst = 0.0
    for t in range(T):
        for j in range(k):
            e = int(layer.ids[t, j])
            sel = np.concatenate([ii, I + ii])
            yg, bg = orc.gemv(layer.gu_syms[e][sel], layer.gu_scales[e][sel], x64[t])
            g_ref, u_ref = yg[0, :len(ii)], yg[0, len(ii):]
            bgg, bgu = bg[0, :len(ii)], bg[0, len(ii):]
            lim = _h_tolerance(g_ref, u_ref, bgg, bgu)
            err = np.abs(h[t, j, ii] - silu(g_ref) * u_ref)
            assert (err <= lim).all(), f"h slot ({t},{j}) worst {(err / lim).max():.3f}"
            worst = max(worst, float((err / lim).max()))
    # down stage fed the GPU's own h
    rr = np.arange(H) if rows_dn is None else rows_dn
    y_ref = np.zeros((T, len(rr)))
    bound = np.zeros((T, len(rr)))
    for t in range(T):
        for j in range(k):
            e = int(layer.ids[t, j])
            yd, bd = orc.gemv(layer.dn_syms[e][rr], layer.dn_scales[e][rr], h[t, j].astype(np.float64))
            y_ref[t] += layer.gate_w[t, j] * yd[0]
            bound[t] += abs(layer.gate_w[t, j]) * bd[0]
    r = check_tol(y[:, rr], y_ref, bound, "down + combine")
    print(f"h worst err/tol {worst:.4f}; y worst err/tol {r:.4f}")
    return y, h


def test_ffn_small_with_edge_routing(trellis_lib, orc):
    announce("ffn small, dead and duplicate slots")
    import torch
    cfg = workloads.MoEConfig(90, "small", 4, 96, 64, 3, 3, True)
    layer = workloads.moe_layer(cfg)
    layer.ids[:] = np.array([[0, 2, -1], [1, 1, 3], [9, 0, 0]], np.int32)
    layer.gate_w[:] = np.array([[0.5, 0.3, 0.2], [0.25, 0.25, 0.5], [0.1, 0.6, 0.3]], np.float32)
    y, h = trellis_lib.moe_ffn(dev(layer.gu_syms), dev(layer.gu_scales), dev(layer.dn_syms),
                               dev(layer.dn_scales), x_dev(layer.x, True), dev(layer.ids), dev(layer.gate_w))
    torch.cuda.synchronize()
    y, h = y.cpu().numpy(), h.float().cpu().numpy()
    assert (h[0, 2] == 0).all() and (h[2, 0] == 0).all()
    y_ref, bound, h_ref, skipped = orc.moe_ffn(layer.gu_syms, layer.gu_scales, layer.dn_syms, layer.dn_scales,
                                              layer.x, layer.ids, layer.gate_w)
    assert skipped == 1
    # the oracle's chain fed the GPU's h reproduces y within tolerance
    yg = np.zeros_like(y_ref)
    bg = np.zeros_like(y_ref)
    for t in range(3):
        for j in range(3):
            e = int(layer.ids[t, j])
            if e < 0 or e >= 4:
                continue
            yd, bd = orc.gemv(layer.dn_syms[e], layer.dn_scales[e], h[t, j].astype(np.float64))
            yg[t] += layer.gate_w[t, j] * yd[0]
            bg[t] += abs(layer.gate_w[t, j]) * bd[0]
    check_tol(y, yg, bg, "ffn small")
    print("end-to-end max |y - y_oracle| / bound:", float((np.abs(y - y_ref) / (bound + 1e-30)).max()))


def test_ffn_expert_ffn_full(trellis_lib, orc):
    """One expert FFN, batch 1: gate_up 5760 x 2880 and down 2880 x 2880, all rows."""
    announce("ffn one expert 5760x2880 + 2880x2880")
    layer = workloads.moe_layer(workloads.EXPERT_FFN)
    layer.ids[:] = 0
    layer.gate_w[:] = 1.0
    _check_layer(trellis_lib, orc, layer)


def test_ffn_32_experts_all_rows(trellis_lib, orc):
    """Full MoE layer, 32 experts, top-4, batch 1: every row of both stages."""
    announce("ffn 32 experts top-4 batch 1, all rows")
    layer = workloads.moe_layer(workloads.MOE_32E)
    _check_layer(trellis_lib, orc, layer)


@pytest.mark.parametrize("T", [1, 4, 8, 16, 32, 64, 128])
def test_ffn_128_experts_sweep_sampled(trellis_lib, orc, T):
    """128 experts, hidden 4096, intermediate 1536, top-8, Zipf(1.1) routing."""
    announce(f"ffn 128 experts top-8 T={T}")
    layer = workloads.moe_layer(workloads.moe_128e(T))
    rs = np.random.default_rng(T)
    n_gu = 48 if T <= 8 else 16
    _check_layer(trellis_lib, orc, layer, rows_gu=np.sort(rs.choice(1536, n_gu, replace=False)),
                 rows_dn=np.sort(rs.choice(4096, 64, replace=False)))


def test_single_token_calls_share_a_workspace(trellis_lib, orc):
    """One token (the split-once path): calls on one workspace, with a call
    whose slots are all empty in between, each see their own activations."""
    announce("single-token calls on one workspace, with an all-empty call between")
    import torch
    E, rows, cols, k = 4, 64, 2880, 4
    g = workloads.rng(604, 0)
    syms, sc = workloads.symbols(g, E, rows, cols), workloads.scales(g, E, rows, cols)
    ws = trellis_lib.gemv_workspace(E, rows, cols, 1, k)
    empty = -np.ones((1, k), np.int32)
    for i in range(3):
        x = workloads.activations(g, 1, cols, True)
        ids, gw = workloads.routing_topk(g, 1, E, k)
        y = trellis_lib.moe_gemv(dev(syms), dev(sc), x_dev(x, True), dev(ids), dev(gw), workspace=ws)
        y_ref, bound, _ = orc.moe_gemv(syms, sc, x, ids, gate_w=gw)
        check_tol(y.cpu().numpy(), y_ref, bound, f"gemv call {i}")
        torch.cuda.synchronize()
        assert int(ws[:8].view(torch.int32)[1]) == 0   # no wait timed out
        y0 = trellis_lib.moe_gemv(dev(syms), dev(sc), x_dev(x, True), dev(empty), dev(gw), workspace=ws)
        assert (y0.cpu().numpy() == 0).all()
        torch.cuda.synchronize()
        assert int(ws[:8].view(torch.int32)[1]) == 0

    cfg = workloads.MoEConfig(91, "small-1", 4, 256, 96, 3, 1, True)
    wsf = trellis_lib.ffn_workspace(cfg.n_exp, cfg.hidden, cfg.inter, 1, cfg.k)
    for i in range(3):
        layer = workloads.moe_layer(cfg, layer_id=i)
        run = lambda L: trellis_lib.moe_ffn(dev(L.gu_syms), dev(L.gu_scales), dev(L.dn_syms), dev(L.dn_scales),
                                            x_dev(L.x, True), dev(L.ids), dev(L.gate_w), workspace=wsf)
        _check_layer(trellis_lib, orc, layer, run=run)
        assert int(wsf[:8].view(torch.int32)[1]) == 0   # no wait timed out
        ye, he = trellis_lib.moe_ffn(dev(layer.gu_syms), dev(layer.gu_scales), dev(layer.dn_syms),
                                     dev(layer.dn_scales), x_dev(layer.x, True), dev(-np.ones((1, 3), np.int32)),
                                     dev(layer.gate_w), workspace=wsf)
        assert (ye.cpu().numpy() == 0).all() and (he.float().cpu().numpy() == 0).all()
        torch.cuda.synchronize()
        assert int(wsf[:8].view(torch.int32)[1]) == 0


def test_prepared_calls(trellis_lib, orc):
    """Calls checked and marshalled once (prepare=True) and entered many times
    give the eager results: a layer on two weight copies, alternated."""
    announce("prepared moe_ffn / moe_gemv calls, replayed")
    import torch
    cfg = workloads.MoEConfig(92, "small-prep", 4, 256, 96, 2, 1, True)
    layer = workloads.moe_layer(cfg, layer_id=0)
    w = [(dev(layer.gu_syms), dev(layer.gu_scales), dev(layer.dn_syms), dev(layer.dn_scales)) for _ in range(2)]
    x, ids, gw = x_dev(layer.x, True), dev(layer.ids), dev(layer.gate_w)
    ws = trellis_lib.ffn_workspace(cfg.n_exp, cfg.hidden, cfg.inter, 1, cfg.k)
    calls = [trellis_lib.moe_ffn(*w[i], x, ids, gw, workspace=ws, prepare=True) for i in range(2)]
    assert isinstance(calls[0], trellis_lib.Call)
    for r in range(4):
        y, h = calls[r % 2]()
        torch.cuda.synchronize()
        _check_layer(trellis_lib, orc, layer, run=lambda L, y=y, h=h: (y, h))
        assert int(ws[:8].view(torch.int32)[1]) == 0

    E, rows, cols, k = 4, 64, 512, 2
    g = workloads.rng(605, 0)
    syms, sc = workloads.symbols(g, E, rows, cols), workloads.scales(g, E, rows, cols)
    xg = workloads.activations(g, 1, cols, True)
    idg, gwg = workloads.routing_topk(g, 1, E, k)
    call = trellis_lib.moe_gemv(dev(syms), dev(sc), x_dev(xg, True), dev(idg), dev(gwg), prepare=True)
    y_ref, bound, _ = orc.moe_gemv(syms, sc, xg, idg, gate_w=gwg)
    for r in range(3):
        check_tol(call().cpu().numpy(), y_ref, bound, f"prepared gemv replay {r}")


def test_ffn_calls_share_a_workspace_varying_experts(trellis_lib, orc):
    """Layer calls on one workspace whose active-expert count changes (6, 1,
    2) and that leave tokens with no live slot: y starts from garbage each
    time, so every row must be written (the empty tokens' rows exactly 0),
    and no wait may time out (the stage-1 counts are cleared by their last
    readers, expert 0's by every down-projection item)."""
    announce("ffn calls on one workspace, varying active experts and empty tokens")
    import torch
    cfg = workloads.MoEConfig(93, "small-ws", 6, 128, 64, 2, 3, True)
    ws = trellis_lib.ffn_workspace(cfg.n_exp, cfg.hidden, cfg.inter, cfg.T, cfg.k)
    routings = [np.array([[0, 1], [2, 3], [4, 5]], np.int32),
                np.array([[-1, -1], [1, 1], [-1, -1]], np.int32),
                np.array([[5, -1], [9, 2], [-1, -1]], np.int32)]
    for i, ids in enumerate(routings):
        layer = workloads.moe_layer(cfg, layer_id=10 + i)
        layer.ids[:] = ids
        y = torch.full((cfg.T, cfg.hidden), 1e30, dtype=torch.float32, device="cuda")
        y, h = trellis_lib.moe_ffn(dev(layer.gu_syms), dev(layer.gu_scales), dev(layer.dn_syms),
                                   dev(layer.dn_scales), x_dev(layer.x, True), dev(layer.ids), dev(layer.gate_w),
                                   y=y, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:8].view(torch.int32)[1]) == 0, f"call {i}: a wait timed out"
        y, h = y.cpu().numpy(), h.float().cpu().numpy()
        yg, bg = np.zeros_like(y, dtype=np.float64), np.zeros_like(y, dtype=np.float64)
        for t in range(cfg.T):
            for j in range(cfg.k):
                e = int(ids[t, j])
                if e < 0 or e >= cfg.n_exp:
                    assert (h[t, j] == 0).all()
                    continue
                yd, bd = orc.gemv(layer.dn_syms[e], layer.dn_scales[e], h[t, j].astype(np.float64))
                yg[t] += layer.gate_w[t, j] * yd[0]
                bg[t] += abs(layer.gate_w[t, j]) * bd[0]
        for t in range(cfg.T):
            if all(int(e) < 0 or int(e) >= cfg.n_exp for e in ids[t]):
                assert (y[t] == 0).all(), f"call {i}: empty token {t} not zero"
        check_tol(y, yg, bg, f"shared workspace call {i}")


def test_timed_out_workspace_is_sticky_and_raises(trellis_lib, orc):
    """A workspace whose status word records a timed-out wait (written here
    from the host, as such a call leaves it): every later call on it writes
    NaN to y, the binding's check raises WorkspaceError, and once the
    workspace is zero-filled again the calls are correct. Covers the
    single-token layer kernel (T = 1), the general layer kernel (T = 2) and
    the routed GEMV."""
    announce("sticky timed-out status word: layer T=1, T=2, routed GEMV")
    import torch
    for T in (1, 2):
        cfg = workloads.MoEConfig(94, f"sticky T={T}", 4, 256, 128, 2, T, True)
        layer = workloads.moe_layer(cfg)
        args = (dev(layer.gu_syms), dev(layer.gu_scales), dev(layer.dn_syms), dev(layer.dn_scales),
                x_dev(layer.x, True), dev(layer.ids), dev(layer.gate_w))
        ws = trellis_lib.ffn_workspace(cfg.n_exp, cfg.hidden, cfg.inter, T, cfg.k)
        ws[:8].view(torch.int32)[1] = 1
        y, _ = trellis_lib.moe_ffn(*args, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isnan(y).all(), f"T={T}: y not marked invalid"
        with pytest.raises(trellis_lib.WorkspaceError):
            trellis_lib.check_workspace(ws)
        with pytest.raises(trellis_lib.WorkspaceError):
            trellis_lib.moe_ffn(*args, workspace=ws, check=True)
        assert int(ws[:8].view(torch.int32)[1]) == 1      # still set: sticky
        ws.zero_()
        _check_layer(trellis_lib, orc, layer,
                     run=lambda L: trellis_lib.moe_ffn(*args, workspace=ws, check=True))
    g = workloads.rng(606, 0)
    E, rows, cols, T, k = 4, 32, 256, 2, 2
    syms, sc = workloads.symbols(g, E, rows, cols), workloads.scales(g, E, rows, cols)
    x = workloads.activations(g, T, cols, True)
    ids, gw = workloads.routing_topk(g, T, E, k)
    ws = trellis_lib.gemv_workspace(E, rows, cols, T, k)
    ws[:8].view(torch.int32)[1] = 1
    with pytest.raises(trellis_lib.WorkspaceError):
        y = trellis_lib.moe_gemv(dev(syms), dev(sc), x_dev(x, True), dev(ids), dev(gw), workspace=ws, check=True)
    y = trellis_lib.moe_gemv(dev(syms), dev(sc), x_dev(x, True), dev(ids), dev(gw), workspace=ws)
    assert torch.isnan(y).all()
    ws.zero_()
    y = trellis_lib.moe_gemv(dev(syms), dev(sc), x_dev(x, True), dev(ids), dev(gw), workspace=ws, check=True)
    y_ref, bound, _ = orc.moe_gemv(syms, sc, x, ids, gate_w=gw)
    check_tol(y.cpu().numpy(), y_ref, bound, "gemv after re-zeroing")
