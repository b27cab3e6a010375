"""Benchmark of the quantized gated Delta-rule decode step on one MI355X.

Workload: GDN serving pool, B=512 requests x H=32 heads, d_k=d_v=128, the
6-bit nominal mix {4-bit: 9, 6-bit: 16, 8-bit: 6, FP16 pivot: 1 head} of
heads, state resident in HBM.  One step = one decode token of one layer
(stq_decode_step over all 16,384 (request, head) tiles).  L independent
layer pools are stepped round-robin, as a model does, so the working set
(L x 214 MB) exceeds the 256 MB Infinity Cache and the timing is HBM-bound.

Prints one JSON line with throughput, the dominant kernel's roofline figure
(algorithmic bytes / average kernel duration, from HIP events on the launch
stream) and the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(bits, H, dk, dv, B, gate_per_row=False):
    """Bytes the method must move per step: packed state read + write, the
    q/k/v/a/b inputs and the readout.  Per-head metadata is excluded."""
    tile = 0
    for n in bits:
        tile += 2 * (dk * dv * n // 8 + (0 if n == 16 else 2 * (dk + dv)))
    io = 4 * (2 * dk + dv) + 4 * (dk if gate_per_row else 1) + 4 + 4 * dv
    return B * (tile + H * io)


def kernel_source_hash():
    """sha256[:16] of the decode-step kernel sources, as the profile summaries record it."""
    h = hashlib.sha256()
    for f in ("stq.hip", "stq_device.h"):
        with open(os.path.join(ROOT, "quantized_linear_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per step launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary (counters scaled by a plain-copy calibration), or None when the kernel
    sources differ from the ones that were measured."""
    path = os.path.join(ROOT, "profiles", "k_tile_step_C3_hbm_traffic.txt")
    try:
        with open(path) as fh:
            txt = fh.read()
    except OSError:
        return None
    h = re.search(r"kernel source sha256\[:16\] \(stq.hip \+ stq_device.h\): (\w+)", txt)
    t = re.search(r"traffic_bytes_per_launch: (\d+)", txt)
    if not h or not t or h.group(1) != kernel_source_hash():
        return None
    return int(t.group(1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": src.numel() * 4, "copies": 3}))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the decode step has no cross-GPU exchange and this "
              "build runs on a single MI355X (requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_linear_attention_amd as stq
    from workloads import Workload

    dev = torch.device("cuda:0")
    wl = Workload("C3")
    B, H, dk, dv = wl.B, wl.H, wl.dk, wl.dv
    T = B * H
    L = args.layers
    desc = stq.make_desc(B, H, dk, dv, wl.bits, wl.row_weight)
    nbytes = stq.stq_pool_bytes(desc)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    pools, bufs = [], []
    r_prof = torch.as_tensor(wl.r_prof, dtype=torch.float32, device=dev)
    c_prof = torch.as_tensor(wl.c_prof, dtype=torch.float32, device=dev)
    for layer in range(L):
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        pool = stq.stq_pool_create(desc, buf)
        gen.manual_seed(wl.seed * 100 + layer)
        for c0 in range(0, B, 64):     # same recipe as workloads.Workload.state, drawn on the GPU
            z = torch.randn((64, H, dk, dv), generator=gen, device=dev)
            S0 = (0.1 * z * r_prof[None, :, :, None] * c_prof[None, :, None, :]).contiguous()
            stq.stq_pool_store(pool, slots[c0:c0 + 64].contiguous(), S0)
        pools.append(pool)
        bufs.append(buf)
    NTOK = 8
    toks = []
    for t in range(NTOK):
        q, k, v, a, b = wl.token(t)
        toks.append([torch.as_tensor(x, device=dev) for x in (q, k, v, a, b)])
    o = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(s):
        q, k, v, a, b = toks[(s // L) % NTOK]
        stq.stq_decode_step(pools[s % L], slots, q, k, v, a, b, o)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for s in range(K):
        ev[s].record()
        step(args.warmup + s)
    ev[K].record()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    per = np.array([ev[s].elapsed_time(ev[s + 1]) for s in range(K)])
    avg_ms = float(per.mean())
    bytes_step = int(algorithmic_bytes([int(n) for n in wl.bits], H, dk, dv, B))
    achieved = bytes_step / (avg_ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build()
        ns = 32                                    # slots per oracle call (1,024 tiles)
        P = oracle.OraclePool(ns, H, dk, dv, wl.bits, wl.row_weight)
        sl = np.arange(ns)
        P.store(sl, wl.state(sl))
        q, k, v, a, b = wl.token(0, ns)
        calls = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            P.step(sl, q, k, v, a, b)
            calls += 1
        el = time.perf_counter() - t0
        cpu = {"value": calls * ns * H / el, "unit": "request-head steps/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": "%d calls x %d tiles of the same workload (B=%d slots, all 32 heads), %.1f s"
                         % (calls, ns * H, ns, el)}

    traffic = measured_traffic()
    line = {
        "metric": "request-head decode steps/s (B=512, H=32, d=128, 6-bit nominal GDN pool)",
        "value": T * K / (total_ms * 1e-3),
        "unit": "request-head steps/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": total_ms / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 update, 4/6/8-bit + f16 state",
        "data": "synthetic (seeded; pool states drawn on the GPU with the workload recipe)",
        "config": {"workload": "GDN serving pool B=512 H=32 d_k=d_v=128, heads {4b:9, 6b:16, 8b:6, "
                               "fp16:1}, %d layer pools round-robin" % L,
                   "global_batch": B, "heads": H, "d_k": dk, "d_v": dv, "layers": L},
        "hbm_gbs": achieved, "hbm_frac": achieved / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "traffic_gbs": None if traffic is None else traffic / (avg_ms * 1e-3) / 1e9,
                     "kernel": "k_tile<128,128,step>", "bytes_per_launch": bytes_step,
                     "avg_launch_ms": avg_ms, "p10_ms": float(np.percentile(per, 10)),
                     "p90_ms": float(np.percentile(per, 90))},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
