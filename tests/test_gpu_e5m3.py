"""E5M3 block scales on the GPU (trellis_moe_gemv_e5m3, trellis_moe_ffn_e5m3)
against the oracle's E5M3 reading (unsigned binary16 upper byte, bias 15,
subnormals at exponent 0).

Bars:
  * one-hot activations give every weight bit-exactly: value x scale is
    exact in fp32, and each scale enters the matrix cores as four exact
    power-of-two terms; every finite scale byte (zero and subnormals
    included) is covered;
  * random activations: within 2e-3 * sum |w| |x| of the oracle's fp64
    result, the UE8M0 calls' bound;
  * the layer: h and y gated stage by stage, as for the UE8M0 layer;
  * exponent-31 blocks make exactly their rows' outputs non-finite.
"""
import numpy as np
import pytest

import workloads
from helpers import TOL, announce, check_tol, dev, sigmoid, silu, x_dev

pytestmark = pytest.mark.gpu

FINITE = 0xF8   # bytes 0 .. 0xF7 are finite E5M3 values


def _all_finite_bytes(g, E, rows, nb):
    """Scale bytes in which every finite byte appears (rows * nb >= 248 per expert)."""
    assert rows * nb >= FINITE
    sc = np.empty((E, rows * nb), np.uint8)
    for e in range(E):
        sc[e] = np.concatenate([g.permutation(FINITE), g.integers(0, FINITE, rows * nb - FINITE)])
    return sc.reshape(E, rows, nb)


@pytest.mark.parametrize("E,rows,cols,T", [
    (2, 64, 256, 32),      # 8 blocks per row: every byte in 512 blocks per expert
    (3, 16, 1024, 1),      # one token, activations resident in LDS
    (2, 48, 2880, 32),     # K = 2880: ragged last chunk
    (1, 32, 4128, 1),      # one token, unaligned rows, K past one register window
])
def test_one_hot_every_weight_exact(trellis_lib, orc, E, rows, cols, T):
    announce(f"e5m3 one-hot E={E} {rows}x{cols} T={T}")
    import torch
    g = workloads.rng(611, E, rows, cols)
    syms = workloads.symbols(g, E, rows, cols)
    sc = _all_finite_bytes(g, E, rows, cols // 32)
    W = orc.decode_values(syms, sc, scale_fmt="e5m3")            # [E, rows, cols]
    ids = np.tile(np.arange(E, dtype=np.int32), (T, 1))
    dsyms, dsc, dids = dev(syms), dev(sc), dev(ids)
    ws = trellis_lib.gemv_workspace(E, rows, cols, T, E)
    eye = torch.eye(cols, dtype=torch.float32, device="cuda")
    for c0 in range(0, cols, T):
        cc = np.minimum(np.arange(c0, c0 + T), cols - 1)
        x = eye[torch.from_numpy(cc).cuda()].contiguous()
        y = trellis_lib.moe_gemv_e5m3(dsyms, dsc, x, dids, workspace=ws).cpu().numpy()   # [T, E, rows]
        want = np.transpose(W[:, :, cc], (2, 0, 1))
        assert np.array_equal(y, want.astype(np.float32)), f"columns {c0}..: {np.abs(y - want).max()}"


@pytest.mark.parametrize("E,rows,cols,T,k,bf16,weighted,per_slot", [
    (5, 48, 96, 3, 2, True, False, False),
    (5, 48, 96, 3, 2, True, True, False),
    (5, 48, 96, 3, 2, False, True, True),
    (4, 64, 2880, 1, 4, True, True, False),
    (16, 64, 256, 16, 4, True, True, False),
    (16, 32, 512, 32, 4, True, False, False),
    (16, 32, 1024, 128, 4, True, True, False),
])
def test_random_within_bound(trellis_lib, orc, E, rows, cols, T, k, bf16, weighted, per_slot):
    announce(f"e5m3 gemv E={E} {rows}x{cols} T={T} k={k} w={weighted} per_slot={per_slot}")
    g = workloads.rng(612, E * 1000 + rows, cols, T * 10 + k)
    syms = workloads.symbols(g, E, rows, cols)
    sc = workloads.scales_e5m3(g, E, rows, cols)
    sc[0, 0, :] = np.arange(sc.shape[2]) % 8          # zero and subnormal blocks in one row
    x = workloads.activations(g, T * (k if per_slot else 1), cols, bf16)
    x = x.reshape((T, k, cols) if per_slot else (T, cols))
    ids, gw = workloads.routing_topk(g, T, E, k)
    y = trellis_lib.moe_gemv_e5m3(dev(syms), dev(sc), x_dev(x, bf16), dev(ids), dev(gw) if weighted else None,
                                  x_per_slot=per_slot, check=True).cpu().numpy()
    y_ref, bound, _ = orc.moe_gemv(syms, sc, x, ids, gate_w=gw if weighted else None, x_per_slot=per_slot,
                                   scale_fmt="e5m3")
    r = check_tol(y, y_ref, bound, "moe_gemv_e5m3")
    print(f"worst err/tol {r:.4f}")


def test_exponent_31_blocks_make_their_rows_nan(trellis_lib, orc):
    announce("e5m3 exponent-31 scale bytes")
    E, rows, cols, T, k = 2, 32, 256, 2, 2
    g = workloads.rng(613, 0)
    syms = workloads.symbols(g, E, rows, cols)
    sc = workloads.scales_e5m3(g, E, rows, cols)
    sc[0, 3, 2] = 0xF8      # infinity
    sc[1, 17, 7] = 0xFB     # NaN
    x = workloads.activations(g, T, cols, True)
    x[:, :] = np.abs(x) + 0.25                  # no zero activations
    ids = np.array([[0, 1], [1, 0]], np.int32)
    y = trellis_lib.moe_gemv_e5m3(dev(syms), dev(sc), x_dev(x, True), dev(ids)).cpu().numpy()
    y_ref, _, _ = orc.moe_gemv(syms, sc, x, ids, scale_fmt="e5m3")
    bad = ~np.isfinite(y)
    assert np.array_equal(bad, ~np.isfinite(y_ref))
    assert bad.sum() == 4   # row 3 of expert 0 and row 17 of expert 1, for both tokens


def _check_layer_e5m3(tq, orc, layer, rows_gu=None, rows_dn=None):
    import torch
    cfg = layer.cfg
    I, H = cfg.inter, cfg.hidden
    T, k = layer.ids.shape
    y, h = tq.moe_ffn_e5m3(dev(layer.gu_syms), dev(layer.gu_scales), dev(layer.dn_syms), dev(layer.dn_scales),
                           x_dev(layer.x, cfg.x_bf16), dev(layer.ids), dev(layer.gate_w), check=True)
    torch.cuda.synchronize()
    y, h = y.cpu().numpy(), h.float().cpu().numpy()
    ii = np.arange(I) if rows_gu is None else rows_gu
    sel = np.concatenate([ii, I + ii])
    x64 = layer.x.astype(np.float64)
    one = np.zeros((1, 1), np.int32)
    worst = 0.0
    for t in range(T):
        for j in range(k):
            e = int(layer.ids[t, j])
            yg, bg, _ = orc.moe_gemv(layer.gu_syms[e][sel][None], layer.gu_scales[e][sel][None], x64[t][None],
                                     one, scale_fmt="e5m3")
            yg, bg = yg[0, 0], bg[0, 0]
            g_ref, u_ref, tg, tu = yg[:len(ii)], yg[len(ii):], TOL * bg[:len(ii)], TOL * bg[len(ii):]
            sig = sigmoid(g_ref)
            dsilu = np.abs(sig * (1.0 + g_ref * (1.0 - sig)))
            href = silu(g_ref) * u_ref
            lim = (dsilu + 0.6 * tg) * (np.abs(u_ref) + tu) * tg + (np.abs(silu(g_ref)) + tg) * tu \
                + np.abs(href) * 2.0 ** -7 + 1e-30
            err = np.abs(h[t, j, ii] - href)
            assert (err <= lim).all(), f"h slot ({t},{j}) worst {(err / lim).max():.3f}"
            worst = max(worst, float((err / lim).max()))
    rr = np.arange(H) if rows_dn is None else rows_dn
    y_ref = np.zeros((T, len(rr)))
    bound = np.zeros((T, len(rr)))
    for t in range(T):
        for j in range(k):
            e = int(layer.ids[t, j])
            yd, bd, _ = orc.moe_gemv(layer.dn_syms[e][rr][None], layer.dn_scales[e][rr][None],
                                     h[t, j].astype(np.float64)[None], one, scale_fmt="e5m3")
            y_ref[t] += layer.gate_w[t, j] * yd[0, 0]
            bound[t] += abs(layer.gate_w[t, j]) * bd[0, 0]
    r = check_tol(y[:, rr], y_ref, bound, "e5m3 down + combine")
    print(f"h worst err/tol {worst:.4f}; y worst err/tol {r:.4f}")


def _e5m3_layer(cfg, n_exp=None, seed=0):
    layer = workloads.moe_layer(cfg, n_exp=n_exp)
    g = workloads.rng(614, cfg.config_id, seed)
    E = layer.gu_syms.shape[0]
    layer.gu_scales = workloads.scales_e5m3(g, E, 2 * cfg.inter, cfg.hidden)
    layer.dn_scales = workloads.scales_e5m3(g, E, cfg.hidden, cfg.inter)
    return layer


def test_ffn_small(trellis_lib, orc):
    announce("e5m3 ffn small 4 experts 96x64 T=3 k=3")
    _check_layer_e5m3(trellis_lib, orc, _e5m3_layer(workloads.MoEConfig(90, "small", 4, 96, 64, 3, 3, True)))


@pytest.mark.parametrize("T", [1, 32])
def test_ffn_32_experts_sampled(trellis_lib, orc, T):
    """The 32-expert H = I = 2880 top-4 layer (single token, then 32 tokens),
    on sampled h and y rows."""
    announce(f"e5m3 ffn 32 experts 2880x2880 T={T}")
    import dataclasses
    cfg = dataclasses.replace(workloads.MOE_32E, T=T)
    g = np.random.default_rng(615)
    rows_gu = np.sort(g.choice(cfg.inter, 96, replace=False))
    rows_dn = np.sort(g.choice(cfg.hidden, 96, replace=False))
    _check_layer_e5m3(trellis_lib, orc, _e5m3_layer(cfg, seed=T), rows_gu, rows_dn)
