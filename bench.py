"""Benchmark of the trellis-coded FP4 hot path on one MI355X.

Default (the headline): compressed-weight GB/s of the fused trellis-decode
MoE layer at batch 1 -- 32 experts, top-4, hidden = intermediate = 2880, one
token (gpt-oss-class layer shape) -- through the C ABI (trellis_moe_ffn):
routing, the activation split, the fused decode + FP4 matrix-core gate_up
GEMV with the SwiGLU epilogue, and the fused down GEMV with the gate-weighted
combine, all in one kernel launch. A step is one layer for one routed token.

Other workloads (--workload):
  ffn1      one expert FFN, gate_up 5760x2880 + down 2880x2880, batch 1
  gemv1     one 256x1024 matrix, fp32 x, batch 1 (trellis_moe_gemv)
  moe128:T  128 experts, top-8, hidden 4096, intermediate 1536, Zipf(1.1)
            routing, T tokens (batch sweep; T >= 16 is the matrix-core path)
  expand    expand mode: decode all 128 experts x 3 matrices (4096x1536)
            into resident MXFP4 (trellis_decode_expand)
  mx128:T   expand mode, second half: the 128-expert layer on the expanded
            MXFP4 weights (trellis_mxfp4_moe_ffn)
  mx32      the default layer shape on expanded MXFP4 weights
  moe32r    the default layer with the device-side router in front of it
            (trellis_router_topk then trellis_moe_ffn, one stream): the
            per-layer latency from activations to output
  moe32rf   the same in one launch (trellis_moe_ffn_routed: every workgroup
            computes the router, then the layer)
  viterbi   the encoder's curvature-aware Viterbi search: 512 rows x 2880
            positions per call (trellis_viterbi_encode), float64; reported
            in encoded weights/s against the fp64 vector ALU roofline

All data is synthetic (workloads.py) and resident in HBM before timing. To
keep the 256 MB Infinity Cache from serving repeated weights, steps walk a
ring of distinct copies of the weights totalling >= --ring-gb GiB, with at
least --reuse-mb MiB of other weights read between two reads of a copy.
Each step's activations, ids and gate weights are consecutive slices of one
device tensor each (--step-buffers packed), as a serving loop reuses its
buffers from layer to layer.

Printed: one JSON line with the whole-job throughput, a roofline entry for
the kernel (its average duration over launches of the timed region, from HIP
events on the stream it runs on: stamped by the kernel's dispatch for the
UE8M0 layer, recorded around the call otherwise), and the CPU oracle's rate
on a bounded sample as a reported baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

TRELLIS_BPW = 0.25 + 1.0 / 32.0           # 2-bit symbol + one UE8M0 byte per 32 weights
MX_BPW = 0.5 + 1.0 / 32.0                 # E2M1 nibble + UE8M0 byte per 32 weights
HBM_PEAK_GBS = 8000.0                     # MI355X HBM3E, published
FP4_PEAK_TFLOPS = 10100.0                 # MI355X dense FP4 matrix cores, published
FP64_PEAK_TFLOPS = 78.6                   # MI355X fp64 vector, published (an FMA counted as two)
FP64_OPS_PEAK_T = FP64_PEAK_TFLOPS / 2    # fp64 vector instructions of one operation each (add, min): 39.3 T/s
VALU_WAVE_INSTS_PER_S = 1024 * 2.4e9 / 4  # 256 CUs x 4 SIMDs, a wave64 VALU instruction every 4 cycles
# encoder search, per position and row: one add per candidate (4096 histories
# x 4 branches) and three minimums per history (the best of four)
VIT_OPS_PER_POSITION = 4096 * 4 + 4096 * 3
METRIC = "compressed-weight GB/s of fused trellis-decode MoE GEMV (batch 1) + % HBM peak"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="moe32",
                   help="moe32 (default) | ffn1 | gemv1 | moe128:T | expand | mx128:T | mx32 | moe32r | moe32rf | e5m3_32 | "
                        "e5m3_128:T | viterbi")
    p.add_argument("--ring-gb", type=float, default=1.0,
                   help="minimum total size of the ring of weight copies (GiB)")
    p.add_argument("--reuse-mb", type=float, default=512.0,
                   help="minimum MiB of other weight traffic between two reads of the same copy's bytes "
                        "(the Infinity Cache holds 256 MB): the ring gets enough copies for it")
    p.add_argument("--rounds", type=int, default=4,
                   help="after the timed region: this many interleaved rounds, cold ring / warm (one copy "
                        "repeated) / warm / cold ..., 50 steps each, reported as a spread check")
    p.add_argument("--step-buffers", choices=("packed", "separate"), default="packed",
                   help="layer workloads: each step's activations, ids and gate weights as consecutive slices of "
                        "one device tensor each (packed, as a serving loop reuses its buffers) or as tensors of "
                        "their own (separate)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="seconds of oracle work for each CPU-baseline leg (one thread, then all cores)")
    p.add_argument("--no-stage-events", action="store_true",
                   help="no events around each launch (time only the whole timed region)")
    p.add_argument("--event-every", type=int, default=8, metavar="N",
                   help="bracket every N-th launch of the timed region with a pair of events (each pair costs "
                        "the stream a few microseconds, so bracketing every launch slows the loop it measures)")
    p.add_argument("--event-release", choices=("device", "none", "system"), default="none",
                   help="memory release of the per-launch events: none (default: no system fence), device "
                        "scope, or HIP's default system scope, which writes back and invalidates the caches "
                        "each record")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB ten times (reference for the HBM "
                        "byte counters of a profiler) and exit")
    return p.parse_args()


def copy_calibration(mib):
    """A plain torch device-to-device copy of a known size: its profiler byte
    counters (FETCH_SIZE, WRITE_SIZE) per dispatch give the scale factor
    between counter readings and bytes moved."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4, "dispatches": 10}), flush=True)


# ---------------------------------------------------------------- HIP events on the launch stream

class Hip:
    def __init__(self):
        L = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch already loaded
        L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.L = L

    # hipEventDisableSystemFence, hipEventReleaseToDevice (hip_runtime_api.h)
    FLAGS = {"system": 0, "none": 0x20000000, "device": 0x40000000}

    def event(self, release="system"):
        e = ctypes.c_void_p()
        rc = self.L.hipEventCreateWithFlags(ctypes.byref(e), self.FLAGS[release])
        assert rc == 0, rc
        return e.value

    def record(self, ev, stream):
        rc = self.L.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        assert rc == 0, rc

    def bracket(self, call, events, stream):
        """call, or a callable that records events[0] / events[1] on stream around it."""
        if not events:
            return call
        rec, e0, e1, st = self.L.hipEventRecord, ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1]), \
            ctypes.c_void_p(stream)

        def run():
            rec(e0, st)
            call()
            rec(e1, st)
        return run

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.L.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        assert rc == 0, rc
        return ms.value


def dev(a):
    import torch
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int32) if a.dtype == np.uint32 else a).cuda()


def ring_copies(tensors, bytes_per_copy, ring_gb, step_bytes=None, reuse_mb=0.0):
    """Distinct device copies of `tensors`: enough to total >= ring_gb GiB and,
    when the bytes a step reads are given (the least of any step), enough
    that steps walking the copies in turn read >= reuse_mb MiB of other
    weights between two reads of the same copy. Returns (copies, reuse
    distance in bytes: (copies - 1) x the least bytes of a step)."""
    n = max(1, int(np.ceil(ring_gb * (1 << 30) / bytes_per_copy)))
    if step_bytes:
        n = max(n, int(np.ceil(reuse_mb * (1 << 20) / step_bytes)) + 1)
    ring = [tensors] + [tuple(t.clone() for t in tensors) for _ in range(n - 1)]
    return ring, ((n - 1) * step_bytes if step_bytes else None)


def cpu_run(fn, seconds, threads):
    """Call fn repeatedly on `threads` threads (the oracle's C calls release
    the GIL) for about `seconds`; returns (calls completed, elapsed s)."""
    import threading
    t0 = time.perf_counter()
    counts = [0] * threads

    def worker(i):
        while True:
            fn()
            counts[i] += 1
            if time.perf_counter() - t0 >= seconds:
                break
    ts = [threading.Thread(target=worker, args=(i,)) for i in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    return sum(counts), time.perf_counter() - t0


def host_cpu():
    """(usable hardware threads, CPU model) of this host."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return n, model


def stream_read_peak(nbytes, reuse_mb, steps=100):
    """GB/s of a plain streaming read (trellis_read_bandwidth: every byte read
    once with 16-byte vector loads) over nbytes per step, walking a ring of
    buffers as the layer steps do: the practical read rate at this size,
    launch gaps included, for comparison with the layer."""
    import torch
    import trellis_coded_fp4_amd as tq
    n = max(2, int(np.ceil(reuse_mb * (1 << 20) / nbytes)) + 1)
    nbytes = (nbytes + 15) // 16 * 16
    bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(n)]
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    calls = [tq.read_bandwidth(b, sink, prepare=True) for b in bufs]
    for i in range(10):
        calls[i % n]()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        calls[i % n]()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / steps
    del bufs
    return round(nbytes / (us * 1e-6) / 1e9, 1), round(us, 2)


# ---------------------------------------------------------------- workloads
#
# Each returns a dict: name/config, make(s, events) that returns a callable
# enqueueing step s (recording events[0] / events[1] around the launch when
# given) with its arguments already checked and marshalled, per-step
# algorithmic bytes, and optionally flops and a CPU-oracle sample.

def layer_workload(args, cfg, mx=False, router=False, e5m3=False, fused_router=False):
    import torch
    import trellis_coded_fp4_amd as tq
    E, H, I = cfg.n_exp, cfg.hidden, cfg.inter
    L0 = workloads.moe_layer(cfg)
    if e5m3:
        # the same streams under E5M3 block scales (same byte count)
        L0.gu_scales = workloads.scales_e5m3(workloads.rng(cfg.config_id, workloads.T_SCALES_GATE_UP), E,
                                             2 * I, H)
        L0.dn_scales = workloads.scales_e5m3(workloads.rng(cfg.config_id, workloads.T_SCALES_DOWN), E, H, I)
    w0 = (dev(L0.gu_syms), dev(L0.gu_scales), dev(L0.dn_syms), dev(L0.dn_scales))
    bpw = MX_BPW if mx else TRELLIS_BPW
    if mx:
        gc, gs = tq.decode_expand(w0[0], w0[1])
        dc, ds = tq.decode_expand(w0[2], w0[3])
        torch.cuda.synchronize()
        w0 = (gc, gs, dc, ds)
    expert_weights = 3 * H * I
    routes, uniq, slots = [], [], []
    n_steps = args.warmup + args.steps + 50 * max(args.rounds, 0)
    batches = [(L0.x, L0.ids, L0.gate_w) if s == 0 else workloads.moe_batch(cfg, 0, 1000 + s)
               for s in range(n_steps)]
    if args.step_buffers == "packed":
        # every step's activations, ids and gate weights are consecutive
        # slices of one tensor each, as a serving loop reuses its buffers
        X = dev(np.stack([b[0] for b in batches]))
        X = X.to(torch.bfloat16) if cfg.x_bf16 else X
        IDS, GW = dev(np.stack([b[1] for b in batches])), dev(np.stack([b[2] for b in batches]))
    for s, (x, ids, gw) in enumerate(batches):
        if args.step_buffers == "packed":
            routes.append((X[s], IDS[s], GW[s]))
        else:
            xs = dev(x).to(torch.bfloat16) if cfg.x_bf16 else dev(x)
            routes.append((xs, dev(ids), dev(gw)))
        live = ids[(ids >= 0) & (ids < E)]
        uniq.append(len(np.unique(live)))
        slots.append(len(live))
    ring, reuse = ring_copies(w0, E * expert_weights * bpw, args.ring_gb,
                              step_bytes=min(uniq) * expert_weights * bpw, reuse_mb=args.reuse_mb)
    T, k = cfg.T, cfg.k
    ws = tq.ffn_workspace(E, H, I, T, k)
    h = torch.empty((T, k, I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream
    if router:
        # the router (bf16 [E][H], N(0, 1/H)) picks each step's experts on the
        # device; the experts a step touches are read back once, before timing
        wr = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(
            workloads.rng(cfg.config_id, workloads.T_ROUTER).standard_normal((E, H)).astype(np.float32)
            / np.sqrt(H)))
        wr = dev(workloads.to_bf16_bits(wr).view(np.int16)).view(torch.bfloat16)
        r_ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        r_gw = torch.empty((T, k), dtype=torch.float32, device="cuda")
        r_ws = tq.router_workspace(E, T)
        for s in range(len(routes)):
            ids_s, _ = tq.router_topk(routes[s][0], wr, k, workspace=r_ws)
            live = ids_s.cpu().numpy()
            uniq[s], slots[s] = len(np.unique(live)), live.size

    def make(s, events=None, copy=None):
        a, b, c, d = ring[s % len(ring) if copy is None else copy]
        xs, ids, gw = routes[s]
        if router and fused_router:
            return tq.moe_ffn_routed(a, b, c, d, xs, wr, k, topk_ids=r_ids, topk_w=r_gw, h=h, y=y, workspace=ws,
                                     prepare=True,
                                     events=(ctypes.c_void_p * 4)(events[0], events[1], None, None) if events else None)
        if router:
            rcall = tq.router_topk(xs, wr, k, topk_ids=r_ids, topk_w=r_gw, workspace=r_ws, prepare=True)
            lcall = tq.moe_ffn(a, b, c, d, xs, r_ids, r_gw, h=h, y=y, workspace=ws, prepare=True,
                               events=(ctypes.c_void_p * 4)(events[0], events[1], None, None) if events else None)

            def step():
                rcall()
                lcall()
            return step
        if mx:
            return hip.bracket(tq.mxfp4_moe_ffn(a, b, c, d, xs, ids, gw, h=h, y=y, workspace=ws, prepare=True),
                               events, stream)
        if e5m3:
            return hip.bracket(tq.moe_ffn_e5m3(a, b, c, d, xs, ids, gw, h=h, y=y, workspace=ws, prepare=True),
                               events, stream)
        return tq.moe_ffn(a, b, c, d, xs, ids, gw, h=h, y=y, workspace=ws, prepare=True,
                          events=(ctypes.c_void_p * 4)(events[0], events[1], None, None) if events else None)

    def cpu_sample(seconds, threads=1):
        import oracle
        done, dt = cpu_run(lambda: oracle.moe_ffn(L0.gu_syms, L0.gu_scales, L0.dn_syms, L0.dn_scales, L0.x,
                                                  L0.ids, L0.gate_w, scale_fmt="e5m3" if e5m3 else "ue8m0"),
                           seconds, threads)
        return done * uniq[0] * expert_weights * TRELLIS_BPW / dt / 1e9, \
            f"{done} full layer step(s) of the same workload (routing of step 0" + \
            ("; the router itself is not part of the sample" if router else "") + \
            f"), C oracle on {threads} thread(s), {dt:.1f} s"

    if mx and T == 1:
        kernel = ("k_tok<MX> (single-token MoE layer on expanded MXFP4 weights: routing, FP4 matrix-core gate_up "
                  "+ SwiGLU, tagged h hand-off, down + gate-weighted atomic combine)")
    elif mx:
        kernel = "k_layer<FmtMx> (whole MoE layer on expanded MXFP4 weights)"
    elif e5m3 and T == 1:
        kernel = ("k_tok<E5M3> (single-token MoE layer, E5M3 block scales: each matrix-core step issued once per "
                  "power-of-two term of its scale, four terms)")
    elif e5m3:
        kernel = ("k_layer<FmtTrellisE5M3> (whole MoE layer, E5M3 block scales: each matrix-core step issued "
                  "once per power-of-two term of its scale, four terms)")
    elif T == 1:
        kernel = ("k_tok (single-token MoE layer: routing, fused decode + FP4 matrix-core gate_up + SwiGLU, "
                  "tagged h hand-off, down + gate-weighted atomic combine)")
    else:
        kernel = ("k_layer<FmtTrellis> (whole MoE layer: routing, activation split, fused decode + FP4 "
                  "matrix-core gate_up + SwiGLU, down + combine)")
    if router and fused_router:
        kernel = ("k_tok<routed> (router computed by every workgroup, then the single-token MoE layer, one launch "
                  "per step)")
    elif router:
        kernel += "; each step is k_router then k_layer, the events time k_layer"
    return dict(
        name=("router + " if router else "") + ("(one launch) " if fused_router else "") + cfg.name + (" [expanded MXFP4]" if mx else "")
        + (" [E5M3 scales]" if e5m3 else ""), make=make, hip=hip,
        stream=stream,
        bytes=lambda s: uniq[s] * expert_weights * bpw,
        flops=lambda s: 2.0 * slots[s] * expert_weights,
        tokens=T, kernel=kernel, cpu=cpu_sample, workspace=ws, ring=len(ring),
        # the UE8M0 layer's events are stamped by the kernel's dispatch
        # (trellis_moe_ffn_timed); the other calls are bracketed by events
        dispatch_events=not (mx or e5m3),
        config={"n_experts": E, "top_k": k, "hidden": H, "intermediate": I, "tokens": T,
                "bytes_per_weight": bpw,
                "weights": "expanded MXFP4" if mx else "trellis-coded" + (", E5M3 scales" if e5m3 else ""),
                "ring_copies": len(ring), "reuse_distance_mb": round(reuse / (1 << 20), 1)})


def gemv_workload(args):
    import torch
    import trellis_coded_fp4_amd as tq
    c = workloads.SINGLE_MATRIX
    rows, cols = c["rows"], c["cols"]
    syms = workloads.symbols(workloads.rng(c["config_id"], 0), 1, rows, cols)
    sc = workloads.scales(workloads.rng(c["config_id"], 1), 1, rows, cols)
    x = workloads.activations(workloads.rng(c["config_id"], workloads.T_X), 1, cols, bf16=False)
    w0 = (dev(syms), dev(sc))
    ring, reuse = ring_copies(w0, rows * cols * TRELLIS_BPW, args.ring_gb, step_bytes=rows * cols * TRELLIS_BPW,
                              reuse_mb=args.reuse_mb)
    xs, ids = dev(x), dev(np.zeros((1, 1), np.int32))
    ws = tq.gemv_workspace(1, rows, cols, 1, 1)
    y = torch.empty((1, 1, rows), dtype=torch.float32, device="cuda")
    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream

    def make(s, events=None, copy=None):
        a, b = ring[s % len(ring) if copy is None else copy]
        return hip.bracket(tq.moe_gemv(a, b, xs, ids, y=y, workspace=ws, prepare=True), events, stream)

    def cpu_sample(seconds, threads=1):
        import oracle
        done, dt = cpu_run(lambda: oracle.moe_gemv(syms, sc, x, np.zeros((1, 1), np.int32)), seconds, threads)
        return done * rows * cols * TRELLIS_BPW / dt / 1e9, f"{done} GEMV(s), C oracle on {threads} thread(s), {dt:.1f} s"

    return dict(name=c["name"], make=make, hip=hip, stream=stream, bytes=lambda s: rows * cols * TRELLIS_BPW,
                flops=lambda s: 2.0 * rows * cols, tokens=1, cpu=cpu_sample, workspace=ws, ring=len(ring),
                kernel="k_tok_gemv (single-token routed GEMV: one 16-row tile per workgroup, K split over its waves)",
                config={"rows": rows, "cols": cols, "tokens": 1, "x": "fp32", "ring_copies": len(ring),
                        "reuse_distance_mb": round(reuse / (1 << 20), 3)})


def expand_workload(args):
    import torch
    import trellis_coded_fp4_amd as tq
    c = workloads.EXPAND_128E
    n, rows, cols = 3 * c["n_exp"], c["rows"], c["cols"]
    # 384 matrices of uniform symbols and scales in 124..130, drawn on the device
    gen = torch.Generator(device="cuda")
    gen.manual_seed(c["config_id"])
    syms = torch.randint(-2**31, 2**31 - 1, (n, rows, cols // 16), dtype=torch.int32, device="cuda", generator=gen)
    sc = torch.randint(workloads.SCALE_LO, workloads.SCALE_HI + 1, (n, rows, cols // 32), dtype=torch.uint8,
                       device="cuda", generator=gen)
    codes = torch.empty((n, rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales_out = torch.empty((n, rows, cols // 32), dtype=torch.uint8, device="cuda")
    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream
    weights = n * rows * cols

    def make(s, events=None, copy=None):
        return hip.bracket(tq.decode_expand(syms, sc, codes_out=codes, scales_out=scales_out, prepare=True),
                           events, stream)

    g = workloads.rng(c["config_id"], 0)
    small = (workloads.symbols(g, 1, 64, cols), workloads.scales(g, 1, 64, cols))

    def cpu_sample(seconds, threads=1):
        import oracle
        done, dt = cpu_run(lambda: oracle.expand(*small), seconds, threads)
        return done * 64 * cols * TRELLIS_BPW / dt / 1e9, \
            f"{done} expand(s) of a 64x{cols} matrix, C oracle on {threads} thread(s), {dt:.1f} s"

    return dict(name=c["name"], make=make, hip=hip, stream=stream, bytes=lambda s: weights * TRELLIS_BPW,
                flops=None, tokens=None, cpu=cpu_sample, traffic_bytes=weights * (TRELLIS_BPW + MX_BPW),
                kernel="k_expand_quads (decode to packed E2M1 + scale copy)",
                config={"matrices": n, "rows": rows, "cols": cols, "read_bytes": weights * TRELLIS_BPW,
                        "write_bytes": weights * MX_BPW})


def viterbi_workload(args):
    import torch
    import trellis_coded_fp4_amd as tq
    c = workloads.VITERBI
    rows, n = c["rows"], c["n"]
    target_h, d_h = workloads.encode_rows(c["config_id"], rows, n)
    target, d = dev(target_h), dev(d_h)
    syms = torch.empty((rows, n), dtype=torch.uint8, device="cuda")
    cost = torch.empty((rows,), dtype=torch.float64, device="cuda")
    ws = tq.viterbi_workspace(rows, n)
    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream

    def make(s, events=None, copy=None):
        return hip.bracket(tq.viterbi_encode(target, d, syms_out=syms, cost_out=cost, workspace=ws, prepare=True),
                           events, stream)

    def cpu_sample(seconds, threads=1):
        import oracle
        counter = iter(range(1 << 30))
        done, dt = cpu_run(lambda: (lambda i: oracle.viterbi(target_h[i % rows], d_h[i % rows]))(next(counter)),
                           seconds, threads)
        return done * n / dt, f"{done} row(s) of {n} positions of the same workload, C oracle on {threads} " \
                              f"thread(s) (65536 states x 4 branches per position), {dt:.1f} s"

    return dict(name=c["name"], make=make, hip=hip, stream=stream, bytes=lambda s: rows * n,
                units="weights/s", scale=1.0,
                metric="Viterbi-encoded weights/s (curvature-aware search, 4096 histories x 4 branches, fp64)",
                alu_ops=rows * n * VIT_OPS_PER_POSITION,
                flops=None, tokens=None, cpu=cpu_sample,
                kernel="k_viterbi (one workgroup per row, fp64 add-compare-select in LDS)",
                config={"rows": rows, "positions": n, "histories": 4096, "branches": 4})


def pick(args):
    w = args.workload
    if w == "moe32":
        return layer_workload(args, workloads.MOE_32E)
    if w == "mx32":
        return layer_workload(args, workloads.MOE_32E, mx=True)
    if w == "moe32r":
        return layer_workload(args, workloads.MOE_32E, router=True)
    if w == "moe32rf":
        return layer_workload(args, workloads.MOE_32E, router=True, fused_router=True)
    if w == "ffn1":
        return layer_workload(args, workloads.EXPERT_FFN)
    if w == "gemv1":
        return gemv_workload(args)
    if w == "expand":
        return expand_workload(args)
    if w == "viterbi":
        return viterbi_workload(args)
    if w.startswith("moe128:"):
        return layer_workload(args, workloads.moe_128e(int(w.split(":")[1])))
    if w == "e5m3_32":
        return layer_workload(args, workloads.MOE_32E, e5m3=True)
    if w.startswith("e5m3_128:"):
        return layer_workload(args, workloads.moe_128e(int(w.split(":")[1])), e5m3=True)
    if w.startswith("mx128:"):
        return layer_workload(args, workloads.moe_128e(int(w.split(":")[1])), mx=True)
    raise SystemExit(f"unknown workload {w}")


# The device sources each workload's kernel is compiled from: a recorded
# traffic figure stays valid while these are unchanged. One token of the
# 32-expert shape (trellis, expanded or E5M3) and the single-matrix GEMV run
# the single-token kernels (tq_tok.hip); the other layer workloads the
# general layer kernel.
KERNEL_SOURCES = {
    "tok": ["tq_tok.hip", "tq_tok.h", "tq_common.h", "tq_decode.h"],
    "layer": ["tq_layer.hip", "tq_layer_mx.hip", "tq_layer_e5m3.hip", "tq_layer.h", "tq_tok.h", "tq_common.h",
              "tq_decode.h"],
    "expand": ["tq_expand.hip", "tq_common.h", "tq_decode.h"],
    "viterbi": ["tq_viterbi.hip", "tq_common.h", "tq_decode.h"],
}
TOK_WORKLOADS = ("moe32", "mx32", "moe32r", "moe32rf", "ffn1", "e5m3_32", "gemv1")


def kernel_sha(workload="moe32"):
    kind = workload if workload in KERNEL_SOURCES else "tok" if workload in TOK_WORKLOADS else "layer"
    h = hashlib.sha256()
    d = os.path.join(ROOT, "trellis_coded_fp4_amd", "csrc")
    for f in sorted(KERNEL_SOURCES[kind]):
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path runs on a single MI355X and has no multi-GPU "
              f"mode (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import torch
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    W = pick(args)
    hip, stream = W["hip"], W["stream"]
    every = max(1, args.event_every)
    evs = [(hip.event(args.event_release), hip.event(args.event_release)) if s % every == 0 else None
           for s in range(args.steps)] if not args.no_stage_events else None
    t0e, t1e = hip.event(), hip.event()

    # Every step's call is checked and marshalled here, before the timed region:
    # inside it each step is one entry into the C library.
    warm = [W["make"](s) for s in range(args.warmup)]
    calls = [W["make"](args.warmup + s, evs[s] if evs else None) for s in range(args.steps)]
    for c in warm:
        c()
    torch.cuda.synchronize()
    hip.record(t0e, stream)
    w0 = time.perf_counter()
    for c in calls:
        c()
    hip.record(t1e, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = hip.elapsed_ms(t0e, t1e)
    # a wait that timed out in any call makes every result invalid (sticky status word)
    status_error = None
    if W.get("workspace") is not None:
        status_error = int(W["workspace"][:8].view(torch.int32)[1].item())
        if status_error:
            raise SystemExit("bench.py: a wait timed out in the timed region (workspace status word set); "
                             "the measurement is invalid")
    ms_per_step = total_ms / args.steps
    timed = range(args.warmup, args.warmup + args.steps)
    total_bytes = sum(W["bytes"](s) for s in timed)
    scale = W.get("scale", 1e-9)   # bytes -> GB by default
    value = total_bytes / (total_ms * 1e-3) * scale

    roofline, launch = None, None
    if evs:
        d = np.array([hip.elapsed_ms(*e) for e in evs if e])
        launch = {"kernel_us_mean": float(d.mean() * 1e3), "kernel_us_min": float(d.min() * 1e3),
                  "step_us": float(ms_per_step * 1e3), "launches_bracketed": len(d), "every": every,
                  "event_release": args.event_release}
        per_launch = float(np.mean([W["bytes"](s) for s, e in zip(timed, evs) if e]))
        achieved = per_launch / (d.mean() * 1e-3) / 1e9
        traffic, valu_insts = None, None
        if os.path.exists(PROFILE_TRAFFIC):
            try:
                tr = json.load(open(PROFILE_TRAFFIC)).get(args.workload, {})
                if tr.get("kernel_source_sha") == kernel_sha(args.workload):
                    traffic = tr.get("bytes_per_launch")
                    valu_insts = tr.get("valu_insts_per_launch")
            except (OSError, ValueError):
                traffic, valu_insts = None, None
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": W["kernel"],
                    "bytes_per_launch": per_launch,
                    "duration_us": round(float(d.mean() * 1e3), 3),
                    "duration_source": (f"mean over every {every}th launch of the timed region of HIP events "
                                        "stamped with the kernel's start and end by its dispatch "
                                        "(trellis_moe_ffn_timed)") if W.get("dispatch_events") else
                                       (f"mean of HIP event pairs recorded around every {every}th launch of the "
                                        "timed region, on the launch stream")}
        if valu_insts:
            # the decode's vector-ALU bound: the kernel's VALU wave instructions
            # (profiler count for these sources) at the chip's issue rate
            issue_us = valu_insts / VALU_WAVE_INSTS_PER_S * 1e6
            roofline["valu"] = {"insts_per_launch": valu_insts,
                                "lane_ops_per_weight": round(valu_insts * 64 / (per_launch / TRELLIS_BPW), 3),
                                "issue_us": round(issue_us, 3),
                                "issue_bound_GBs": round(per_launch / (issue_us * 1e-6) / 1e9, 1),
                                "issue_frac": round(issue_us / (d.mean() * 1e3), 4),
                                "peak": "1024 SIMDs x 2.4 GHz / 4 cycles per wave64 instruction"}
        if W.get("traffic_bytes"):
            roofline["read_plus_write_GBs"] = round(W["traffic_bytes"] / (d.mean() * 1e-3) / 1e9, 1)
        if W.get("alu_ops"):
            # adds and minimums, one fp64 vector operation each, against the
            # chip's fp64 vector issue rate for such operations (half the
            # FMA-counted 78.6 TFLOP/s)
            tf = W["alu_ops"] / (d.mean() * 1e-3) / 1e12
            roofline = {"bound": "alu", "achieved": round(tf, 3), "peak": FP64_OPS_PEAK_T,
                        "unit": "T fp64 ops/s (add, min)",
                        "frac": round(tf / FP64_OPS_PEAK_T, 4), "traffic": traffic, "kernel": W["kernel"],
                        "ops_per_launch": W["alu_ops"],
                        "peak_note": "78.6 TFLOP/s fp64 vector counts an FMA as two operations; adds and "
                                     "minimums issue at half that"}
        if W.get("flops"):
            fl = float(np.mean([W["flops"](s) for s, e in zip(timed, evs) if e]))
            tf = fl / (d.mean() * 1e-3) / 1e12
            roofline["matrix_core"] = {"useful_tflops": round(tf, 3), "fp4_dense_peak_tflops": FP4_PEAK_TFLOPS,
                                       "frac": round(tf / FP4_PEAK_TFLOPS, 6), "flops_per_launch": fl}

    # interleaved rounds after the timed region (cold ring, warm = one copy
    # repeated): A B B A ..., 50 steps each, with their spread
    rounds = None
    if args.rounds > 0 and W.get("ring"):
        base = args.warmup + args.steps
        vals = {"cold": [], "warm": []}
        for r in range(args.rounds):
            kind = "cold" if r % 4 in (0, 3) else "warm"
            cs = [W["make"](base + 50 * r + i, copy=None if kind == "cold" else 0) for i in range(50)]
            torch.cuda.synchronize()
            hip.record(t0e, stream)
            for c in cs:
                c()
            hip.record(t1e, stream)
            torch.cuda.synchronize()
            ms = hip.elapsed_ms(t0e, t1e)
            vals[kind].append(sum(W["bytes"](base + 50 * r + i) for i in range(50)) / (ms * 1e-3) * scale)
        rounds = {k: [round(v, 1) for v in vs] for k, vs in vals.items() if vs}
        if vals["cold"]:
            c = np.array(vals["cold"])
            rounds["cold_median"] = round(float(np.median(c)), 1)
            rounds["cold_spread_pct"] = round(100 * float((c.max() - c.min()) / np.median(c)), 2)
            rounds["spread_over_5pct"] = bool(rounds["cold_spread_pct"] > 5.0)
        if vals["warm"]:
            rounds["warm_median"] = round(float(np.median(vals["warm"])), 1)
        if W.get("status_check", True) and W.get("workspace") is not None:
            if int(W["workspace"][:8].view(torch.int32)[1].item()):
                raise SystemExit("bench.py: a wait timed out in the rounds (workspace status word set)")

    # the practical read rate at this size: a plain device reduction over
    # the same bytes per step, ring-walked like the steps
    stream_peak = None
    if "units" not in W and W.get("ring"):
        gbs, us = stream_read_peak(int(np.mean([W["bytes"](s) for s in timed])), args.reuse_mb)
        stream_peak = {"GBs": gbs, "us_per_step": us,
                       "kernel": "trellis_read_bandwidth over the step's bytes (ring of buffers, launch gaps included)",
                       "value_frac": round(value / gbs, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        n_cores, model = host_cpu()
        v1, s1 = W["cpu"](args.cpu_seconds, 1)
        vn, sn = W["cpu"](args.cpu_seconds, n_cores)
        cpu = {"value": round(vn, 6), "unit": W.get("units", "GB/s"), "cores": n_cores, "kind": "oracle",
               "sample": sn, "single_thread_value": round(v1, 6), "single_thread_sample": s1,
               "cpu_model": model}

    if W.get("metric"):
        metric = W["metric"]
    elif args.workload == "moe32":
        metric = METRIC
    elif args.workload == "expand":
        metric = "decode GB/s (compressed bytes read) of expand to MXFP4"
    else:
        metric = f"compressed-weight GB/s, {W['name']}"
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": W.get("units", "GB/s"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"expand": "u32 -> u8", "viterbi": "f64"}.get(args.workload, "u32 decode, e2m1 x e4m3(hi+lo) -> f32"),
        "data": "synthetic",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2) if "units" not in W else None,
        "tokens_per_s": round(W["tokens"] / (ms_per_step * 1e-3), 1) if W.get("tokens") else None,
        "config": dict({"workload": W["name"]}, **W["config"],
                       **{"wall_s": round(wall, 4)}),
        "launch": launch,
        "roofline": roofline,
        "rounds": rounds,
        "stream_read_peak": stream_peak,
        "status_error": status_error,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
