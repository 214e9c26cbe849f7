"""Benchmark: compressed-weight GB/s of the fused trellis-decode MoE layer at batch 1.

One step = one whole MoE layer through the C ABI (trellis_moe_ffn): routing
and activation prep, the fused decode + FP4 matrix-core gate_up GEMV with the
SwiGLU epilogue, and the fused down GEMV with the gate-weighted combine.

Default workload: 32 experts, top-4, hidden = intermediate = 2880, one token
(gpt-oss-class layer shape; synthetic symbols, scales, activations and
routing from workloads.py). Weights are resident in HBM before timing. To
keep the 256 MB Infinity Cache from serving repeated weights, the steps walk
a ring of distinct layer instances totalling >= --ring-gb GiB.

Printed: one JSON line with the throughput (algorithmic compressed bytes of
the experts each step touches / wall time), a roofline entry for the
dominant kernel (its average duration from HIP events recorded around it in
the timed region, on the stream it runs on), and the CPU oracle's rate on a
bounded sample as a reported baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

BYTES_PER_WEIGHT = 0.25 + 1.0 / 32.0      # 2-bit symbol + one UE8M0 byte per 32 weights
HBM_PEAK_GBS = 8000.0                     # MI355X HBM3E, published
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="moe32",
                   help="moe32 (default) | ffn1 | moe128:T")
    p.add_argument("--ring-gb", type=float, default=1.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-stage-events", action="store_true",
                   help="time only the whole step (no events between kernels)")
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


def workload_cfg(name):
    if name == "moe32":
        return workloads.MOE_32E
    if name == "ffn1":
        return workloads.EXPERT_FFN
    if name.startswith("moe128:"):
        return workloads.moe_128e(int(name.split(":")[1]))
    raise SystemExit(f"unknown workload {name}")


def hip():
    L = ctypes.CDLL("libamdhip64.so.7")   # the runtime torch already loaded
    L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    L.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return L


def new_event(H):
    e = ctypes.c_void_p()
    rc = H.hipEventCreate(ctypes.byref(e))
    assert rc == 0, rc
    return e.value


def elapsed_ms(H, a, b):
    ms = ctypes.c_float()
    rc = H.hipEventElapsedTime(ctypes.byref(ms), a, b)
    assert rc == 0, rc
    return ms.value


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
    import trellis_coded_fp4_amd as tq

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    cfg = workload_cfg(args.workload)
    E, H_, I = cfg.n_exp, cfg.hidden, cfg.inter
    layer_weights = E * (2 * I * H_ + H_ * I)
    layer_bytes = layer_weights * BYTES_PER_WEIGHT
    n_layers = max(1, int(np.ceil(args.ring_gb * (1 << 30) / layer_bytes)))

    def dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int32) if a.dtype == np.uint32 else a).cuda()

    ring = []
    for li in range(n_layers):
        L = workloads.moe_layer(cfg, layer_id=li)
        ring.append((dev(L.gu_syms), dev(L.gu_scales), dev(L.dn_syms), dev(L.dn_scales)))
        if li == 0:
            layer0 = L
    # one routed batch per step, drawn up front and resident on the device
    n_route = args.warmup + args.steps
    routes = []
    uniq = []
    for s in range(n_route):
        if s:
            x_np, ids_np, gw_np = workloads.moe_batch(cfg, layer_id=0, rep=1000 + s)
        else:
            x_np, ids_np, gw_np = layer0.x, layer0.ids, layer0.gate_w
        xs = dev(x_np).to(torch.bfloat16) if cfg.x_bf16 else dev(x_np)
        routes.append((xs, dev(ids_np), dev(gw_np)))
        uniq.append(len(np.unique(ids_np[(ids_np >= 0) & (ids_np < E)])))
    T, k = cfg.T, cfg.k
    ws = tq.ffn_workspace(E, H_, I, T, k)
    h = torch.empty((T, k, I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, H_), dtype=torch.float32, device="cuda")
    Hl = hip()
    stream = torch.cuda.current_stream()
    ev_arrays = []
    for s in range(args.steps):
        arr = (ctypes.c_void_p * 4)()
        if not args.no_stage_events:
            for i in range(2):
                arr[i] = new_event(Hl)
        ev_arrays.append(arr)
    t0e, t1e = new_event(Hl), new_event(Hl)

    def step(s, events=None):
        gs, ge, ds, de = ring[s % n_layers]
        xs, ids, gw = routes[s]
        tq.moe_ffn(gs, ge, ds, de, xs, ids, gw, h=h, y=y, workspace=ws, events=events)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    Hl.hipEventRecord(t0e, ctypes.c_void_p(stream.cuda_stream))
    w0 = time.perf_counter()
    for s in range(args.steps):
        step(args.warmup + s, None if args.no_stage_events else ev_arrays[s])
    Hl.hipEventRecord(t1e, ctypes.c_void_p(stream.cuda_stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = elapsed_ms(Hl, t0e, t1e)
    ms_per_step = total_ms / args.steps

    expert_bytes = (2 * I * H_ + H_ * I) * BYTES_PER_WEIGHT
    timed_uniq = uniq[args.warmup:]
    total_bytes = sum(u * expert_bytes for u in timed_uniq)
    value = total_bytes / (total_ms * 1e-3) / 1e9

    roofline = None
    stages = None
    if not args.no_stage_events:
        d = np.array([elapsed_ms(Hl, ev[0], ev[1]) for ev in ev_arrays])
        stages = {"layer_kernel_us": float(d.mean() * 1e3), "layer_kernel_us_min": float(d.min() * 1e3),
                  "step_us": float(ms_per_step * 1e3)}
        launch_bytes = float(np.mean([u * expert_bytes for u in timed_uniq]))
        achieved = launch_bytes / (d.mean() * 1e-3) / 1e9
        traffic = None
        if os.path.exists(PROFILE_TRAFFIC):
            try:
                tr = json.load(open(PROFILE_TRAFFIC))
                if tr.get("workload") == args.workload and tr.get("kernel_source_sha") == _kernel_sha():
                    traffic = tr.get("bytes_per_launch")
            except Exception:
                traffic = None
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": "k_layer (whole MoE layer: routing, activation split, fused decode + FP4 MFMA "
                              "gate_up + SwiGLU, down + combine)",
                    "bytes_per_launch": launch_bytes}

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        L0 = layer0
        done = 0
        bytes_done = 0.0
        c0 = time.perf_counter()
        while True:
            oracle.moe_ffn(L0.gu_syms, L0.gu_scales, L0.dn_syms, L0.dn_scales, L0.x, L0.ids, L0.gate_w)
            done += 1
            bytes_done += uniq[0] * expert_bytes
            if time.perf_counter() - c0 >= args.cpu_seconds:
                break
        cdt = time.perf_counter() - c0
        cpu = {"value": round(bytes_done / cdt / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} full layer step(s) of the same workload (routing of step 0), "
                         f"single-threaded C oracle, {cdt:.1f} s"}

    out = {
        "metric": "compressed-weight GB/s of fused trellis-decode MoE GEMV (batch 1) + % HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32 decode, e2m1 x e4m3(hi+lo) -> f32",
        "data": "synthetic",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "config": {"workload": cfg.name, "n_experts": E, "top_k": k, "hidden": H_, "intermediate": I,
                   "tokens": T, "bytes_per_weight": BYTES_PER_WEIGHT, "ring_layers": n_layers,
                   "ring_gib": round(n_layers * layer_bytes / (1 << 30), 3),
                   "stage_events": not args.no_stage_events, "wall_s": round(wall, 4)},
        "stages": stages,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def _kernel_sha():
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "trellis_coded_fp4_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
