"""Grouped MoE GEMV / layer on expanded MXFP4 weights against the oracle.

Expand mode serves the codes that trellis_decode_expand writes; the same
routed GEMV and layer then run with the weights' nibbles fed to the matrix
cores as stored. The weights here are expanded by the oracle on the CPU
(only the experts a case routes to), so these tests share nothing with the
device expand kernel; the expected values are the oracle's trellis GEMV on
the original symbols (expansion is exact). Same bar as the fused path:
every output within 2e-3 * sum |w| |x|.
"""
import numpy as np
import pytest

import workloads
from helpers import announce, check_tol, dev, x_dev
from test_gpu_moe import _check_layer

pytestmark = pytest.mark.gpu


def _expand(orc, syms, sc, experts):
    """Expanded codes/scales for all experts; only `experts` are filled (the
    others are never read by a call routed to `experts`)."""
    E, rows, wpr = syms.shape
    codes = np.zeros((E, rows, wpr * 8), np.uint8)
    scales = np.zeros_like(sc)
    for e in sorted(set(int(v) for v in experts if 0 <= v < E)):
        c, s = orc.expand(syms[e:e + 1], sc[e:e + 1])
        codes[e], scales[e] = c[0], s[0]
    return codes, scales


def _mx_gemv_case(tq, orc, E, rows, cols, T, k, bf16, weighted, per_slot, seed=0):
    g = workloads.rng(611, seed, E * 1000 + rows, cols * 100 + T * 10 + k)
    syms = workloads.symbols(g, E, rows, cols)
    sc = workloads.scales(g, E, rows, cols)
    x = workloads.activations(g, T * (k if per_slot else 1), cols, bf16)
    x = x.reshape((T, k, cols) if per_slot else (T, cols))
    ids, gw = workloads.routing_topk(g, T, E, min(k, E))
    if ids.shape[1] < k:
        ids = np.concatenate([ids, -np.ones((T, k - ids.shape[1]), np.int32)], axis=1)
        gw = np.concatenate([gw, np.zeros((T, k - gw.shape[1]), np.float32)], axis=1)
    codes, mxs = _expand(orc, syms, sc, ids.ravel())
    y = tq.mxfp4_moe_gemv(dev(codes), dev(mxs), x_dev(x, bf16), dev(ids), dev(gw) if weighted else None,
                          x_per_slot=per_slot).cpu().numpy()
    y_ref, bound, _ = orc.moe_gemv(syms, sc, x, ids, gate_w=gw if weighted else None, x_per_slot=per_slot)
    return y, y_ref, bound


@pytest.mark.parametrize("E,rows,cols,T,k,bf16,weighted,per_slot", [
    (5, 48, 96, 3, 2, True, False, False),       # 3 blocks: a partial step
    (5, 48, 96, 3, 2, False, True, True),
    (4, 64, 1024, 1, 4, False, False, False),    # one window, single-token split
    (4, 64, 2880, 1, 4, True, True, False),      # 23 steps: two register windows
    (4, 32, 4096, 1, 2, True, False, False),     # 32 steps: two full windows
    (16, 64, 1536, 8, 4, True, True, False),
    (16, 32, 512, 32, 4, True, True, False),
    (3, 16, 32, 32, 8, False, True, True),       # one block per row
])
def test_mxfp4_gemv(trellis_lib, orc, E, rows, cols, T, k, bf16, weighted, per_slot):
    announce(f"mxfp4 gemv E={E} {rows}x{cols} T={T} k={k} bf16={bf16} w={weighted} per_slot={per_slot}")
    y, y_ref, bound = _mx_gemv_case(trellis_lib, orc, E, rows, cols, T, k, bf16, weighted, per_slot)
    check_tol(y, y_ref, bound, "mxfp4 gemv")


def test_mxfp4_gemv_matches_device_expand(trellis_lib, orc):
    """Codes from the device expand kernel give the same GEMV as the oracle's."""
    announce("mxfp4 gemv on device-expanded codes")
    import torch
    g = workloads.rng(612, 0)
    E, rows, cols, T, k = 8, 64, 2880, 2, 4
    syms, sc = workloads.symbols(g, E, rows, cols), workloads.scales(g, E, rows, cols)
    x = workloads.activations(g, T, cols, True)
    ids, gw = workloads.routing_topk(g, T, E, k)
    codes, mxs = trellis_lib.decode_expand(dev(syms), dev(sc))
    y = trellis_lib.mxfp4_moe_gemv(codes, mxs, x_dev(x, True), dev(ids), dev(gw))
    torch.cuda.synchronize()
    y_ref, bound, _ = orc.moe_gemv(syms, sc, x, ids, gate_w=gw)
    check_tol(y.cpu().numpy(), y_ref, bound, "mxfp4 gemv (device expand)")


def _mx_run(tq, orc, device_expand=False):
    """Layer on expanded weights. The large layers are expanded by the device
    kernel (bit-exact against the oracle in test_gpu_expand); the oracle
    would take minutes over hundreds of millions of weights."""
    def run(layer):
        cfg = layer.cfg
        if device_expand:
            gc, gs = tq.decode_expand(dev(layer.gu_syms), dev(layer.gu_scales))
            dc, ds = tq.decode_expand(dev(layer.dn_syms), dev(layer.dn_scales))
        else:
            gc, gs = (dev(a) for a in _expand(orc, layer.gu_syms, layer.gu_scales, layer.ids.ravel()))
            dc, ds = (dev(a) for a in _expand(orc, layer.dn_syms, layer.dn_scales, layer.ids.ravel()))
        return tq.mxfp4_moe_ffn(gc, gs, dc, ds, x_dev(layer.x, cfg.x_bf16), dev(layer.ids), dev(layer.gate_w))
    return run


def test_mxfp4_ffn_small_edge_routing(trellis_lib, orc):
    announce("mxfp4 ffn small, dead and duplicate slots")
    cfg = workloads.MoEConfig(91, "small", 4, 96, 64, 3, 3, True)
    layer = workloads.moe_layer(cfg)
    layer.ids[:] = np.array([[0, 2, -1], [1, 1, 3], [9, 0, 0]], np.int32)
    layer.gate_w[:] = np.array([[0.5, 0.3, 0.2], [0.25, 0.25, 0.5], [0.1, 0.6, 0.3]], np.float32)
    import torch
    y, h = _mx_run(trellis_lib, orc)(layer)
    torch.cuda.synchronize()
    y, h = y.cpu().numpy(), h.float().cpu().numpy()
    assert (h[0, 2] == 0).all() and (h[2, 0] == 0).all()
    yg = np.zeros((3, 96))
    bg = np.zeros((3, 96))
    for t in range(3):
        for j in range(3):
            e = int(layer.ids[t, j])
            if e < 0 or e >= 4:
                continue
            yd, bd = orc.gemv(layer.dn_syms[e], layer.dn_scales[e], h[t, j].astype(np.float64))
            yg[t] += layer.gate_w[t, j] * yd[0]
            bg[t] += abs(layer.gate_w[t, j]) * bd[0]
    check_tol(y, yg, bg, "mxfp4 ffn small")


def test_mxfp4_ffn_32_experts_sampled(trellis_lib, orc):
    """The 32-expert top-4 batch-1 layer on expanded weights (sampled rows)."""
    announce("mxfp4 ffn 32 experts top-4 batch 1")
    layer = workloads.moe_layer(workloads.MOE_32E)
    rs = np.random.default_rng(1)
    _check_layer(trellis_lib, orc, layer, rows_gu=np.sort(rs.choice(2880, 96, replace=False)),
                 rows_dn=np.sort(rs.choice(2880, 96, replace=False)), run=_mx_run(trellis_lib, orc))


@pytest.mark.parametrize("T", [1, 8, 32, 128])
def test_mxfp4_ffn_128_experts_sampled(trellis_lib, orc, T):
    """128 experts, hidden 4096, intermediate 1536, top-8 on expanded weights."""
    announce(f"mxfp4 ffn 128 experts top-8 T={T}")
    layer = workloads.moe_layer(workloads.moe_128e(T))
    rs = np.random.default_rng(100 + T)
    _check_layer(trellis_lib, orc, layer, rows_gu=np.sort(rs.choice(1536, 16, replace=False)),
                 rows_dn=np.sort(rs.choice(4096, 48, replace=False)), run=_mx_run(trellis_lib, orc, True))
