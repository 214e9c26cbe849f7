"""The router in front of the layer on the GPU against the oracle's router:
top-k ids equal (where the oracle's logits do not tie within the GPU's
float64 summation bound), gate weights within fp32 rounding; and the router
chained into the layer on one stream."""
import dataclasses

import numpy as np
import pytest

import workloads
from helpers import announce, dev

pytestmark = pytest.mark.gpu


def _router_inputs(seed, T, E, H, bf16):
    g = workloads.rng(960 + seed, 0)
    x = workloads.activations(g, T, H, bf16)
    w = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(
        workloads.rng(960 + seed, 1).standard_normal((E, H)).astype(np.float32) / np.sqrt(H)))
    return x, w


def _w_dev(w):
    import torch
    return dev(workloads.to_bf16_bits(w).view(np.int16)).view(torch.bfloat16)


def _x_dev(x, bf16):
    import torch
    t = dev(x)
    return t.to(torch.bfloat16) if bf16 else t


def _check(orc, x, w, k, ids, gw):
    ref_ids, ref_gw, logits = orc.router_topk(x, w, k)
    bound = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T * 1e-12
    for t in range(x.shape[0]):
        if not np.array_equal(ids[t], ref_ids[t]):
            # only a tie within the float64 summation bound may reorder
            for j in range(k):
                a, b = int(ids[t, j]), int(ref_ids[t, j])
                assert abs(logits[t, a] - logits[t, b]) <= bound[t, a] + bound[t, b], (t, j, a, b)
        # gate weights of the ids the GPU picked: softmax over the oracle's
        # float64 logits of those ids (equal to the oracle's own weights when
        # the ids agree), so weights are checked whether or not a tie reordered
        picked = logits[t, ids[t].astype(np.int64)]
        e = np.exp(picked - picked.max())
        want = (e / e.sum()).astype(np.float32)
        np.testing.assert_allclose(gw[t], want, rtol=1e-6, atol=0)
        if np.array_equal(ids[t], ref_ids[t]):
            np.testing.assert_allclose(gw[t], ref_gw[t], rtol=1e-6, atol=0)


@pytest.mark.parametrize("T,E,H,k,bf16", [
    (1, 32, 2880, 4, True),      # the 32-expert layer's router
    (32, 128, 4096, 8, False),   # the 128-expert layer's router, 32 tokens
    (3, 8, 64, 8, True),         # k = E
    (2, 1000, 200, 64, False),   # many experts: several per lane, the largest k
])
def test_router_matches_oracle(trellis_lib, orc, T, E, H, k, bf16):
    announce(f"router T={T} E={E} H={H} k={k} bf16={bf16}")
    x, w = _router_inputs(E + T, T, E, H, bf16)
    ids, gw = trellis_lib.router_topk(_x_dev(x, bf16), _w_dev(w), k)
    _check(orc, x, w, k, ids.cpu().numpy(), gw.cpu().numpy())


def test_router_ties_go_to_the_lower_id(trellis_lib, orc):
    x, w = _router_inputs(3, 2, 6, 64, False)
    w[4] = w[1]                       # experts 1 and 4 have equal logits
    w[5] = w[1]
    ids, gw = trellis_lib.router_topk(_x_dev(x, False), _w_dev(w), 6)
    ref_ids, ref_gw, _ = orc.router_topk(x, w, 6)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    pos = {e: j for j, e in enumerate(ref_ids[0])}
    assert pos[1] < pos[4] < pos[5]


def test_router_chained_into_the_layer(trellis_lib, orc):
    """Router then layer on one stream, the layer reading the router's device
    outputs; the layer is checked with the router's ids and weights."""
    import torch
    from test_gpu_moe import _check_layer
    cfg = workloads.MoEConfig(97, "router chain: 16 experts top-4 H=512 I=256 batch-2", 16, 512, 256, 4, 2, True)
    layer = workloads.moe_layer(cfg)
    _, w = _router_inputs(9, 2, 16, 512, True)
    xd = _x_dev(layer.x, True)
    ids, gw = trellis_lib.router_topk(xd, _w_dev(w), cfg.k)
    y, h = trellis_lib.moe_ffn(dev(layer.gu_syms), dev(layer.gu_scales), dev(layer.dn_syms), dev(layer.dn_scales),
                               xd, ids, gw)
    torch.cuda.synchronize()
    ids_h, gw_h = ids.cpu().numpy(), gw.cpu().numpy()
    _check(orc, layer.x, w, cfg.k, ids_h, gw_h)
    chained = dataclasses.replace(layer, ids=ids_h, gate_w=gw_h)
    _check_layer(trellis_lib, orc, chained, run=lambda L: (y, h))


def test_router_calls_share_a_workspace(trellis_lib, orc):
    """The per-token counters return to zero: one workspace serves calls of
    different shapes back to back."""
    ws = trellis_lib.router_workspace(128, 32)
    for i, (T, E, H, k) in enumerate([(32, 128, 4096, 8), (1, 32, 2880, 4), (5, 100, 256, 7), (32, 128, 4096, 8)]):
        x, w = _router_inputs(20 + i, T, E, H, False)
        ids, gw = trellis_lib.router_topk(_x_dev(x, False), _w_dev(w), k, workspace=ws)
        _check(orc, x, w, k, ids.cpu().numpy(), gw.cpu().numpy())


@pytest.mark.parametrize("cfg,bf16", [
    (workloads.MOE_32E, True),   # the 32-expert layer, bf16 x
    (workloads.MoEConfig(98, "routed: 16 experts top-4 H=512 I=256 batch-1", 16, 512, 256, 4, 1, False), False),
    (workloads.MoEConfig(99, "routed: 6 experts top-6 H=256 I=128 batch-1", 6, 256, 128, 6, 1, True), True),
])
def test_routed_layer_in_one_launch(trellis_lib, orc, cfg, bf16):
    """trellis_moe_ffn_routed: the routing the kernel computes equals the
    standalone router's bit for bit (and the oracle's, as the router tests
    check it); h equals the unrouted layer's fed that routing, bit for bit;
    the layer is checked against the oracle with that routing; a second call
    on the same workspace gives the same routing and h."""
    import torch
    from test_gpu_moe import _check_layer
    announce(f"routed layer in one launch: {cfg.name}")
    cfg = dataclasses.replace(cfg, x_bf16=bf16)
    layer = workloads.moe_layer(cfg)
    _, w = _router_inputs(cfg.config_id, 1, cfg.n_exp, cfg.hidden, bf16)
    xd, wd = _x_dev(layer.x, bf16), _w_dev(w)
    W = [dev(layer.gu_syms), dev(layer.gu_scales), dev(layer.dn_syms), dev(layer.dn_scales)]
    ws = trellis_lib.ffn_workspace(cfg.n_exp, cfg.hidden, cfg.inter, 1, cfg.k)
    y, h, ids, gw = trellis_lib.moe_ffn_routed(*W, xd, wd, cfg.k, workspace=ws, check=True)
    ids2, gw2 = trellis_lib.router_topk(xd, wd, cfg.k)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(gw, gw2), "fused routing differs from trellis_router_topk"
    ids_h, gw_h = ids.cpu().numpy(), gw.cpu().numpy()
    _check(orc, layer.x, w, cfg.k, ids_h, gw_h)
    y_u, h_u = trellis_lib.moe_ffn(*W, xd, ids, gw)
    torch.cuda.synchronize()
    assert torch.equal(h, h_u), "h differs from the unrouted layer fed the same routing"
    routed = dataclasses.replace(layer, ids=ids_h, gate_w=gw_h)
    _check_layer(trellis_lib, orc, routed, run=lambda L: (y, h))
    y3, h3, ids3, gw3 = trellis_lib.moe_ffn_routed(*W, xd, wd, cfg.k, workspace=ws, check=True)
    assert torch.equal(ids3, ids) and torch.equal(gw3, gw) and torch.equal(h3, h)


def test_routed_layer_rejects_other_shapes(trellis_lib):
    """Shapes the single-token kernel does not take are refused before
    anything is enqueued (more than 32 experts here)."""
    import torch
    cfg = workloads.MoEConfig(100, "routed: 40 experts", 40, 256, 128, 4, 1, True)
    layer = workloads.moe_layer(cfg)
    _, w = _router_inputs(5, 1, 40, 256, True)
    W = [dev(layer.gu_syms), dev(layer.gu_scales), dev(layer.dn_syms), dev(layer.dn_scales)]
    with pytest.raises(trellis_lib.TrellisError):
        trellis_lib.moe_ffn_routed(*W, _x_dev(layer.x, True), _w_dev(w), 4)
    torch.cuda.synchronize()
