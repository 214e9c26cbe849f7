"""Seeded synthetic inputs for the trellis-coded FP4 MoE path.

This module only draws random inputs. It holds none of the decoding or
GEMV arithmetic, so that the CPU oracle (``oracle/``) and the HIP library
(``trellis_coded_fp4_amd``) can both be fed from it without sharing code.

Everything is NumPy on the host. Every tensor comes from its own
``numpy.random.default_rng(SeedSequence([config_id, tensor_id, layer_id, rep]))``
stream, so any tensor can be regenerated on its own.

Distributions (the pages give none; these are the stated synthetic
stand-ins for the gpt-oss-class MoE checkpoints the HEPH abstract evaluates):

* branch symbols: i.i.d. uniform 2-bit symbols, i.e. uniform uint32 words
  holding 16 symbols each, little-endian, row-major;
* UE8M0 block exponents: uniform integers in 124..130 inclusive, one per
  32 weights along a row;
* activations: float32 N(0, 1), rounded to bf16 (round-to-nearest-even)
  where the workload uses bf16 activations;
* routing: top-k of N(0, 1) logits (ties to the lower id) with softmax
  gate weights over the k selected logits; or, for the skewed sweep,
  Zipf(1.1) expert popularity sampled without replacement by Gumbel-top-k.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Tensor ids inside one configuration's seed sequence.
T_SYMS_GATE_UP = 0
T_SCALES_GATE_UP = 1
T_SYMS_DOWN = 2
T_SCALES_DOWN = 3
T_X = 4
T_ROUTE = 5
T_ROUTE_W = 6
T_SYMS_UP = 7          # third matrix of the expand workload
T_SCALES_UP = 8
T_ROUTER = 11          # router weights of the router-in-front workload

SCALE_LO = 124
SCALE_HI = 130


def rng(config_id: int, tensor_id: int, layer_id: int = 0, rep: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([config_id, tensor_id, layer_id, rep]))


def symbols(g: np.random.Generator, n_mat: int, rows: int, cols: int) -> np.ndarray:
    """Uniform 2-bit symbols packed 16 per uint32: shape [n_mat, rows, cols // 16]."""
    assert cols % 16 == 0
    return g.integers(0, 1 << 32, size=(n_mat, rows, cols // 16), dtype=np.uint64).astype(np.uint32)


def scales(g: np.random.Generator, n_mat: int, rows: int, cols: int,
           lo: int = SCALE_LO, hi: int = SCALE_HI) -> np.ndarray:
    """UE8M0 exponent bytes, one per 32 weights: shape [n_mat, rows, cols // 32]."""
    assert cols % 32 == 0
    return g.integers(lo, hi + 1, size=(n_mat, rows, cols // 32), dtype=np.int64).astype(np.uint8)


# E5M3 block-scale bytes (exponent bits 7..3, mantissa 2..0): exponents 12..18
# with every mantissa, the UE8M0 range above at eight steps per octave.
E5M3_LO = 0x60
E5M3_HI = 0x97


def scales_e5m3(g: np.random.Generator, n_mat: int, rows: int, cols: int,
                lo: int = E5M3_LO, hi: int = E5M3_HI) -> np.ndarray:
    """E5M3 scale bytes, one per 32 weights, uniform in [lo, hi]: shape [n_mat, rows, cols // 32]."""
    assert cols % 32 == 0
    return g.integers(lo, hi + 1, size=(n_mat, rows, cols // 32), dtype=np.int64).astype(np.uint8)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even); return the raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def activations(g: np.random.Generator, T: int, K: int, bf16: bool) -> np.ndarray:
    """x ~ N(0,1) as float32 [T, K]; if ``bf16`` the values are bf16-representable."""
    x = g.standard_normal(size=(T, K), dtype=np.float32)
    if bf16:
        x = bf16_bits_to_f32(to_bf16_bits(x))
    return x


def routing_topk(g: np.random.Generator, T: int, E: int, k: int):
    """Top-k of N(0,1) router logits; gate weights = softmax over the k picked logits."""
    logits = g.standard_normal(size=(T, E))
    # stable descending sort: equal logits keep the lower expert id first
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    picked = np.take_along_axis(logits, order, axis=1)
    e = np.exp(picked - picked.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def routing_zipf(g: np.random.Generator, T: int, E: int, k: int, s: float = 1.1):
    """k distinct experts per token with Zipf(s) popularity (expert id = rank).

    Sampling without replacement is Gumbel-top-k on log p; the gate weights
    are a softmax over independent N(0,1) logits of the k picked experts.
    """
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    gumbel = -np.log(-np.log(g.uniform(low=np.finfo(np.float64).tiny, high=1.0, size=(T, E))))
    order = np.argsort(-(logp[None, :] + gumbel), axis=1, kind="stable")[:, :k]
    logits = g.standard_normal(size=(T, k))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """Shape of one workload. A matrix is [rows = out features][cols = in features]."""
    config_id: int
    name: str
    n_exp: int
    hidden: int            # H: input width of gate_up, output width of down
    inter: int             # I: expert intermediate width (gate_up has 2*I rows)
    k: int
    T: int
    x_bf16: bool
    zipf: bool = False

    @property
    def gate_up_shape(self):
        return (self.n_exp, 2 * self.inter, self.hidden)

    @property
    def down_shape(self):
        return (self.n_exp, self.hidden, self.inter)


# The five synthetic workloads (the pages measure gpt-oss-class MoE layers in
# SGLang; these shapes stand in for them).
SINGLE_MATRIX = dict(config_id=1, name="single-matrix 256x1024 batch-1", rows=256, cols=1024)
EXPERT_FFN = MoEConfig(2, "one expert FFN 5760x2880 + 2880x2880 batch-1", 1, 2880, 2880, 1, 1, True)
MOE_32E = MoEConfig(3, "MoE layer 32 experts top-4 H=I=2880 batch-1", 32, 2880, 2880, 4, 1, True)


def moe_128e(T: int) -> MoEConfig:
    return MoEConfig(4, f"MoE layer 128 experts top-8 H=4096 I=1536 batch-{T} zipf1.1",
                     128, 4096, 1536, 8, T, True, zipf=True)


EXPAND_128E = dict(config_id=5, name="expand 128 experts x 3 matrices 4096x1536",
                   n_exp=128, rows=4096, cols=1536)


@dataclasses.dataclass
class MoELayer:
    """Host tensors of one MoE layer instance plus its routed batch."""
    cfg: MoEConfig
    gu_syms: np.ndarray
    gu_scales: np.ndarray
    dn_syms: np.ndarray
    dn_scales: np.ndarray
    x: np.ndarray            # float32 [T, H] (bf16-representable if cfg.x_bf16)
    ids: np.ndarray          # int32 [T, k]
    gate_w: np.ndarray       # float32 [T, k]


def moe_batch(cfg: MoEConfig, layer_id: int = 0, rep: int = 0, n_exp: Optional[int] = None):
    """The routed batch of one step: x [T, hidden], ids [T, k], gate weights [T, k]."""
    E = cfg.n_exp if n_exp is None else n_exp
    c = cfg.config_id
    x = activations(rng(c, T_X, layer_id, rep), cfg.T, cfg.hidden, cfg.x_bf16)
    if cfg.zipf:
        ids, w = routing_zipf(rng(c, T_ROUTE, layer_id, rep), cfg.T, E, min(cfg.k, E))
    else:
        ids, w = routing_topk(rng(c, T_ROUTE, layer_id, rep), cfg.T, E, min(cfg.k, E))
    return x, ids, w


def moe_layer(cfg: MoEConfig, layer_id: int = 0, rep: int = 0,
              n_exp: Optional[int] = None, route_rep: Optional[int] = None) -> MoELayer:
    """All tensors of one layer instance. ``n_exp`` may shrink the expert
    count (for oracle-sized tests); routing is drawn over the shrunk count."""
    E = cfg.n_exp if n_exp is None else n_exp
    c = cfg.config_id
    rr = rep if route_rep is None else route_rep
    gu_s = symbols(rng(c, T_SYMS_GATE_UP, layer_id, rep), E, 2 * cfg.inter, cfg.hidden)
    gu_e = scales(rng(c, T_SCALES_GATE_UP, layer_id, rep), E, 2 * cfg.inter, cfg.hidden)
    dn_s = symbols(rng(c, T_SYMS_DOWN, layer_id, rep), E, cfg.hidden, cfg.inter)
    dn_e = scales(rng(c, T_SCALES_DOWN, layer_id, rep), E, cfg.hidden, cfg.inter)
    x, ids, w = moe_batch(cfg, layer_id, rr, n_exp=E)
    return MoELayer(cfg, gu_s, gu_e, dn_s, dn_e, x, ids, w)



# ---------------------------------------------------------------- encoder search
#
# Rows to encode: targets are weights already divided by their block scale,
# N(0, 2^2), so that they span the palettes' range [-6, 6]; the per-position
# weights d (the curvature diagonal) are positive, lognormal(0, 0.5).
T_TARGET = 9
T_CURV = 10
VITERBI = dict(config_id=6, name="Viterbi encode 512 rows x 2880 positions", rows=512, n=2880)


def encode_rows(config_id: int, rows: int, n: int, rep: int = 0):
    """(target [rows, n] float64, d [rows, n] float64) for the encoder search."""
    target = rng(config_id, T_TARGET, 0, rep).standard_normal((rows, n)) * 2.0
    d = rng(config_id, T_CURV, 0, rep).lognormal(0.0, 0.5, (rows, n))
    return target, d
