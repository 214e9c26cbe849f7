"""trellis_moe_ffn_noalloc -- the layer on the library's own per-device
scratch -- against trellis_moe_ffn on a caller workspace (same kernels) and
against the oracle, on calls in a row whose shapes change: the 32-expert
single-token layer, then a smaller three-token layer, then the first again.

Bar: h (bf16, deterministic) bit-identical to the caller-workspace call; y
of both calls within the oracle bound of 2e-3 * sum |w| |x| (the down stage
fed the GPU's own h); the two y differ only in the order of the float
atomics that combine the slots."""
import numpy as np
import pytest

import workloads
from helpers import announce, dev, x_dev
from test_gpu_moe import _check_layer

pytestmark = pytest.mark.gpu


def _both(tq, orc, name, layer, **rows):
    import torch
    cfg = layer.cfg
    T, k = layer.ids.shape
    args = (dev(layer.gu_syms), dev(layer.gu_scales), dev(layer.dn_syms), dev(layer.dn_scales),
            x_dev(layer.x, cfg.x_bf16), dev(layer.ids), dev(layer.gate_w))
    # outputs start from garbage: every element must be written
    h = torch.full((T, k, cfg.inter), 3.0, dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, cfg.hidden), 7.0, dtype=torch.float32, device="cuda")
    y_n, h_n = tq.moe_ffn_noalloc(*args, h=h, y=y)
    assert y_n is y and h_n is h
    torch.cuda.synchronize()
    y_r, h_r = tq.moe_ffn(*args)
    torch.cuda.synchronize()
    assert torch.equal(h_n, h_r), f"{name}: h differs from the caller-workspace call"
    print(name, "no-alloc:")
    _check_layer(tq, orc, layer, run=lambda L: (y_n, h_n), **rows)
    print(name, "caller workspace:")
    _check_layer(tq, orc, layer, run=lambda L: (y_r, h_r), **rows)


def test_noalloc_layer_matches_the_workspace_call(trellis_lib, orc):
    announce("moe_ffn_noalloc: 32-expert batch-1 layer, a smaller 3-token layer, the first again")
    big = workloads.moe_layer(workloads.MOE_32E, layer_id=1)
    small = workloads.moe_layer(workloads.MoEConfig(93, "small-3", 4, 256, 96, 3, 3, True), layer_id=2)
    small.ids[:] = np.array([[0, 2, 1], [1, 1, 3], [3, 0, 2]], np.int32)   # a duplicate slot
    rs = np.random.default_rng(7)
    rows = dict(rows_gu=np.sort(rs.choice(2880, 96, replace=False)),
                rows_dn=np.sort(rs.choice(2880, 96, replace=False)))
    _both(trellis_lib, orc, "32e batch-1", big, **rows)
    _both(trellis_lib, orc, "small 3-token", small)
    _both(trellis_lib, orc, "32e batch-1 again", big, **rows)
