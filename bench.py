"""Benchmark of the quantized gated Delta-rule decode step on one MI355X.

Default workload (C3): GDN serving pool, B=512 requests x H=32 heads,
d_k=d_v=128, the 6-bit nominal mix {4-bit: 9, 6-bit: 16, 8-bit: 6, FP16
pivot: 1 head} of heads, state resident in HBM.  One step = one decode token
of one layer (stq_decode_step over all 16,384 (request, head) tiles).  L
independent layer pools are stepped round-robin, as a model does, so the
working set exceeds the 256 MB Infinity Cache and the timing is HBM-bound.
`--workload C4` times the per-channel-gate, per-key-row-width pool (B=256)
and `--workload C5` the windowed 4-bit pool (W=16, whole windows timed);
`--workload P3` times the prefill ingest of a batch of prompts into the C3
pool (stq_prefill; one step = one call over all prompts).

Prints one JSON line with throughput, the dominant kernel's roofline figure
(algorithmic bytes / average kernel duration, from HIP events on the launch
stream, one event per round over the layer pools; p10/p90 are over those
rounds) and the CPU oracle timed on a bounded sample of the same workload.
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


def tile_bytes(bits, dk, dv):
    """Packed bytes of one tile: codes, then the bf16 row and column scales.
    `bits` is the tile's width (unit = head) or its per-key-row widths (unit =
    key row); a binary16 pivot head carries no scales."""
    b = np.atleast_1d(np.asarray(bits, np.int64))
    if b.size == 1:
        n = int(b[0])
        return dk * dv * n // 8 + (0 if n == 16 else 2 * (dk + dv))
    return int((dv * b // 8).sum()) + 2 * (dk + dv)


def io_bytes(dk, dv, gate_per_row):
    """q, k, v, a, b read and o written, per tile and token (binary32)."""
    return 4 * (2 * dk + dv) + 4 * (dk if gate_per_row else 1) + 4 + 4 * dv


def algorithmic_bytes(wl, pos=0, n_comp=0):
    """Bytes the method must move in one launch over all B x H tiles.

    Per-head and per-key-row modes: the packed state read and written once,
    plus the per-token inputs and readout.  Window mode at window position
    `pos` (tokens already cached): the frozen base read, the pos cached
    (Gamma, k, u) entries read, the new entry and the count written, the
    inputs and readout, and at the window's last token the base written by
    the fold.  With n_comp compensator rows per tile a quantized tile's
    readout also reads them (values and row indices), and the fold reads
    and rewrites them (a binary16 pivot tile only has its empty slots
    rewritten).  Per-head metadata is excluded."""
    c, H, dk, dv = wl.cfg, wl.H, wl.dk, wl.dv
    per_row = wl.bits.ndim == 2
    tiles = [tile_bytes(wl.bits[h], dk, dv) for h in range(H)]
    io = io_bytes(dk, dv, c.gate == 1)
    if c.window == 0:
        return wl.B * sum(2 * t + io for t in tiles)
    ent = 4 * (dk + dv + 1)
    fold = pos + 1 == c.window
    comp = n_comp * (4 * dv + 4)
    quant = [np.atleast_1d(wl.bits[h])[0] != 16 for h in range(H)]
    per = [t + 8 + pos * ent + ent + io + (t if fold else 0)
           + (comp if q else 0) + ((2 * comp if q else comp) if fold else 0) for t, q in zip(tiles, quant)]
    assert not per_row
    return wl.B * sum(per)


def kernel_source_hash():
    """sha256[:16] of the decode-step kernel sources, as the profile summaries record it."""
    h = hashlib.sha256()
    for f in ("stq.hip", "stq_device.h"):
        with open(os.path.join(ROOT, "quantized_linear_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(key):
    """HBM bytes per step launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary of the workload's step kernel (counters scaled by a plain-copy
    calibration), or None when there is none or the kernel sources differ from
    the ones that were measured."""
    path = os.path.join(ROOT, "profiles", "%s_%s_hbm_traffic.txt" % (BENCH[key]["prof"], key))
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


# Timed workloads.  C3 is the headline line; C4 (per-channel gate, per-key-row
# widths) and C5 (windowed 4-bit) time the other step kernels the same way.
# `layers` independent pools are stepped round-robin so that the working set
# exceeds the 256 MB Infinity Cache (one layer's pool: C3 214 MB, C4 103 MB,
# C5 415 MB with its window caches).
BENCH = {
    "C3": {"layers": 4, "kernel": "k_tile<128, 128, 0>", "prof": "k_tile_step",
           "metric": "request-head decode steps/s (B=512, H=32, d=128, 6-bit nominal GDN pool)",
           "workload": "GDN serving pool B=512 H=32 d_k=d_v=128, heads {4b:9, 6b:16, 8b:6, fp16:1}",
           "dtype": "f32 update and refit; the two matvecs on matrix cores with each f32 operand split into "
                    "f16 hi + lo (f32 accumulation); 4/6/8-bit + f16 state"},
    "C4": {"layers": 8, "kernel": "k_rows_mf<128, 4>", "prof": "k_rows_mf_step",
           "metric": "request-head decode steps/s (B=256, H=32, d=128, KDA per-channel gate, "
                     "per-key-row widths)",
           "workload": "KDA pool B=256 H=32 d_k=d_v=128, per-channel gate, key rows "
                       "{4b:30%, 6b:50%, 8b:19%, fp16:1%}",
           "dtype": "f32 update and refit; the two matvecs on matrix cores with each f32 operand split into "
                    "f16 hi + lo (f32 accumulation), the rank-one update on f32 matrix cores; per-key-row "
                    "4/6/8-bit + f16 state"},
    "C5": {"layers": 2,
           "kernel": "k_window_read<128, 128, false, true> + k_window_fold<128, 128, true, false, 16>",
           "regex": "k_window_(read<128, 128, false, true>|fold<128, 128, true, false, 16>)",
           "prof": "k_window_step",
           "metric": "request-head decode steps/s (B=512, H=32, d=128, 4-bit GDN, window W=16)",
           "workload": "windowed GDN pool B=512 H=32 d_k=d_v=128, all heads 4-bit, W=16 "
                       "(binary32 window caches, one fold per 16 tokens)",
           "dtype": "f32 update and window cache; the base matvecs on matrix cores with each f32 operand "
                    "split into f16 hi + lo (f32 accumulation); 4-bit base state"},
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 512; P3: 8)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 32; P3: 2)")
    ap.add_argument("--workload", choices=sorted(BENCH) + ["P3", "P4", "P5"], default="C3")
    ap.add_argument("--prompt-len", type=int, default=1024, help="P3: tokens per prompt")
    ap.add_argument("--prompts", type=int, default=64, help="P3: prompts per prefill call")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="P3/P4: seconds of oracle prefill timing")
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="after the --warmup steps, keep stepping untimed until this much time has passed "
                         "(clocks and caches settle; the count done is reported as warmup)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--n-comp", type=int, default=0,
                    help="window workloads: compensator rows per tile (0 = the workload as specified)")
    ap.add_argument("--graph", action="store_true",
                    help="C workloads: capture one pass over every (layer, token) step in a HIP graph and replay it")
    ap.add_argument("--split", action="store_true",
                    help="C3: time the step split into readout and commit, the commit on a second stream")
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

    key = args.workload
    if key in ("P3", "P4", "P5"):
        return prefill_bench(args)
    spec = BENCH[key]
    dev = torch.device("cuda:0")
    wl = Workload(key)
    c = wl.cfg
    B, H, dk, dv = wl.B, wl.H, wl.dk, wl.dv
    T = B * H
    L = spec["layers"] if args.layers is None else args.layers
    K = 512 if args.steps is None else args.steps
    Wu = 32 if args.warmup is None else args.warmup
    if c.window:
        # whole windows in the warm-up and in the timed region, so every pool
        # enters the timed region with an empty window
        span = L * c.window
        K = max(span, -(-K // span) * span)
        Wu = -(-Wu // span) * span
    C = args.n_comp
    if C and not c.window:
        print("--n-comp needs a window workload", file=sys.stderr)
        sys.exit(2)
    desc = stq.make_desc(B, H, dk, dv, wl.bits, wl.row_weight, c.gate, c.unit, c.window, C)
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
            n = min(64, B - c0)
            z = torch.randn((n, H, dk, dv), generator=gen, device=dev)
            S0 = (0.1 * z * r_prof[None, :, :, None] * c_prof[None, :, None, :]).contiguous()
            stq.stq_pool_store(pool, slots[c0:c0 + n].contiguous(), S0)
        pools.append(pool)
        bufs.append(buf)
    NTOK = 8
    toks = []
    for t in range(NTOK):
        q, k, v, a, b = wl.token(t)
        toks.append([torch.as_tensor(x, device=dev) for x in (q, k, v, a, b)])
    o = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    if args.split:
        if c.window or c.unit:
            print("--split: per-head pools without a window (C1-C3)", file=sys.stderr)
            sys.exit(2)
        return split_timing(stq, torch, pools, slots, toks, o, L, K, Wu, wl, spec)

    def step(s):
        q, k, v, a, b = toks[(s // L) % NTOK]
        stq.stq_decode_step(pools[s % L], slots, q, k, v, a, b, o)

    # untimed: the requested steps, then whole rounds over the layer pools (whole
    # windows) until --warmup-seconds have passed
    rnd = L * max(c.window, 16)
    for s in range(Wu):
        step(s)
    torch.cuda.synchronize()
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < args.warmup_seconds:
        for s in range(Wu, Wu + rnd):
            step(s)
        Wu += rnd
        torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    if args.graph:
        # one pass over every (layer pool, token) pair and whole windows, captured once
        G = L * max(NTOK, c.window)
        K = -(-K // G) * G
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for s in range(G):
                step(Wu + s)
        graph.replay()
        torch.cuda.synchronize()
        R = K // G
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
        start.record()
        for r in range(R):
            ev[r].record()
            graph.replay()
        ev[R].record()
        stop.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(stop)
        per = np.array([ev[r].elapsed_time(ev[r + 1]) / G for r in range(R)])
        Wu += G
    else:
        # one event per round over the layer pools (at least 4 launches): an
        # event between every two launches adds a packet and a gap that a
        # serving loop does not have (about 6 us per C3 launch)
        M = max(L, 4)
        K = -(-K // M) * M
        R = K // M
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
        torch.cuda.synchronize()
        start.record()
        for r in range(R):
            ev[r].record()
            for s in range(r * M, (r + 1) * M):
                step(Wu + s)
        ev[R].record()
        stop.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(stop)
        per = np.array([ev[r].elapsed_time(ev[r + 1]) / M for r in range(R)])
    avg_ms = float(per.mean())
    if c.window:
        # launch s is token (Wu + s) // L of its pool: window position that mod W
        pos = [((Wu + s) // L) % c.window for s in range(K)]
        bytes_step = float(np.mean([algorithmic_bytes(wl, p, C) for p in pos]))
    else:
        bytes_step = float(algorithmic_bytes(wl))
    achieved = bytes_step / (avg_ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, bufs[0].cpu().numpy(), C, bytes_step)

    traffic = measured_traffic(key) if C == 0 else None
    line = {
        "metric": spec["metric"],
        "value": T * K / (total_ms * 1e-3),
        "unit": "request-head steps/s",
        "n_gpus": 1, "steps": K, "warmup": Wu,
        "ms_per_step": total_ms / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": spec["dtype"],
        "data": "synthetic (seeded; pool states drawn on the GPU with the workload recipe)",
        "config": {"workload": spec["workload"] + (", %d compensator rows per tile" % C if C else "")
                   + ", %d layer pools round-robin" % L + (", replayed from a HIP graph" if args.graph else ""),
                   "global_batch": B, "heads": H, "d_k": dk, "d_v": dv, "layers": L},
        "hbm_gbs": achieved, "hbm_frac": achieved / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "traffic_gbs": None if traffic is None else traffic / (avg_ms * 1e-3) / 1e9,
                     "kernel": spec["kernel"].replace("read<128, 128, false,", "read<128, 128, true,")
                                             .replace("fold<128, 128, true, false>", "fold<128, 128, true, true>")
                               if C else spec["kernel"],
                     "bytes_per_launch": bytes_step,
                     "avg_launch_ms": avg_ms, "p10_ms": float(np.percentile(per, 10)),
                     "p90_ms": float(np.percentile(per, 90))},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def cpu_baseline(wl, image, C, bytes_step):
    """The oracle on the full step of the same workload: every (request, head)
    tile of one layer pool, starting from the GPU pool's own bytes (layer 0 as
    the timed run left it).  All host threads: 1 untimed + 3 timed steps (a
    window workload: one whole window of W steps, its fold included); then one
    core: 1 timed step.  The oracle computes the update in binary64; the
    figure is a reported baseline, not a target."""
    import oracle
    oracle.build()
    c, B, H = wl.cfg, wl.B, wl.H
    P = oracle.OraclePool(B, H, wl.dk, wl.dv, wl.bits, wl.row_weight, c.gate, c.unit, c.window,
                          image=image, n_comp=C)
    sl = np.arange(B)
    n_timed = c.window if c.window else 3
    tk = [wl.token(t) for t in range(min(n_timed + 1, 4))]
    cores = oracle.num_threads()
    P.step(sl, *tk[0])
    t0 = time.perf_counter()
    for t in range(n_timed):
        P.step(sl, *tk[1 + t % (len(tk) - 1)])
    el = time.perf_counter() - t0
    oracle.set_num_threads(1)
    t1 = time.perf_counter()
    P.step(sl, *tk[1])
    el1 = time.perf_counter() - t1
    oracle.set_num_threads(cores)
    rate = n_timed * B * H / el
    return {"value": rate, "unit": "request-head steps/s", "cores": cores, "kind": "oracle",
            "gbs": rate / (B * H) * bytes_step / 1e9,
            "one_core": {"value": B * H / el1, "unit": "request-head steps/s", "seconds": el1,
                         "steps": 1},
            "sample": "the full step: %d steps x %d tiles (B=%d, all %d heads%s) on %d threads in %.1f s "
                      "after 1 untimed step; one core: 1 step in %.1f s"
                      % (n_timed, B * H, B, H, ", one whole window" if c.window else "", cores, el, el1)}


def split_timing(stq, torch, pools, slots, toks, o, L, K, Wu, wl, spec):
    """The decode step as readout (stream 1) + commit (stream 2, after the
    readout of the same layer; the next readout of a layer waits for its
    commit), layers round-robin as in the fused timing."""
    B, H, dk, dv = wl.B, wl.H, wl.dk, wl.dv
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    done = [None] * L
    rt, ct = [], []

    def step(s, timed):
        lay = s % L
        q, k, v, a, b = toks[(s // L) % len(toks)]
        if done[lay] is not None:
            sa.wait_event(done[lay])
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(sa)
        stq.stq_decode_readout(pools[lay], slots, q, k, v, a, b, o, stream=sa)
        e[1].record(sa)
        sb.wait_event(e[1])
        e[2].record(sb)
        stq.stq_decode_commit(pools[lay], slots, q, k, v, a, b, stream=sb)
        e[3].record(sb)
        done[lay] = e[3]
        if timed:
            rt.append((e[0], e[1]))
            ct.append((e[2], e[3]))

    for s in range(Wu):
        step(s, False)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(sa)
    sb.wait_event(start)
    for s in range(K):
        step(Wu + s, True)
    for d in done:
        sa.wait_event(d)
    stop.record(sa)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    r_ms = float(np.mean([x.elapsed_time(y) for x, y in rt]))
    c_ms = float(np.mean([x.elapsed_time(y) for x, y in ct]))
    T = B * H
    state = B * sum(tile_bytes(wl.bits[h], dk, dv) for h in range(H))
    inputs = T * 4 * (2 * dk + dv + 2)
    r_bytes, c_bytes = state + inputs + T * 4 * dv, 2 * state + inputs
    achieved = c_bytes / (c_ms * 1e-3) / 1e9
    line = {
        "metric": spec["metric"],
        "value": T * K / (total_ms * 1e-3),
        "unit": "request-head steps/s",
        "n_gpus": 1, "steps": K, "warmup": Wu, "ms_per_step": total_ms / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": spec["dtype"],
        "data": "synthetic (seeded; pool states drawn on the GPU with the workload recipe)",
        "config": {"workload": spec["workload"] + ", %d layer pools round-robin; step split into readout "
                   "(stream 1) and commit (stream 2)" % L,
                   "global_batch": B, "heads": H, "d_k": dk, "d_v": dv, "layers": L},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "k_tile<128, 128, 3> (commit)",
                     "bytes_per_launch": c_bytes, "avg_launch_ms": c_ms},
        "split": {"readout_ms": r_ms, "readout_bytes": r_bytes,
                  "readout_gbs": r_bytes / (r_ms * 1e-3) / 1e9, "commit_ms": c_ms, "commit_bytes": c_bytes},
        "cpu_baseline": None,
    }
    print(json.dumps(line))


PL = 32                     # tokens per chunk of the prefill kernel
MFMA_F32_PEAK = 157.3       # TFLOP/s, dense binary32 matrix cores


def method_flops(n_tok, H, dk, dv, per_channel):
    """Flops the gated delta rule itself needs per token and head: u = S^T k,
    o = S^T q and the rank-one update (2 d_k d_v each), plus the per-channel
    gate's d_k d_v multiplies (a scalar gate folds into the products)."""
    return n_tok * H * (6 + (1 if per_channel else 0)) * dk * dv


def prefill_flops(n_tok, H, dk, dv):
    """Matrix-core flops of the chunkwise prefill per token and head, counting
    each product at the extent the chunk form needs: the three state products
    (S^T K^T, S^T Q^T, K^T Delta) 6 dk dv, the strictly lower K K^T and the
    lower Q K^T dk L, the two lower-triangular products with Delta 2 dv (L + 1)."""
    return n_tok * H * (6 * dk * dv + dk * PL + 2 * dv * (PL + 1))


def prefill_setup(key, B, Lp, dev):
    """Pool and prompts of the prefill workloads, drawn on the GPU: P3 the C3
    pool (GDN head mix, H = 32, d = 128) with GDN half-life gates; P4 per-channel
    (KDA) gates of C4's half-life law on per-head widths of the same mix; P5 P4's
    prompts into the C4 pool (per-key-row widths).  B prompts of Lp tokens each,
    one per slot; the pool's states are stored first.  Returns the workload, the
    pool and its buffer, and the prefill call's tensors."""
    import dataclasses

    import torch

    import quantized_linear_attention_amd as stq
    from workloads import Workload
    kda = key in ("P4", "P5")
    rows = key == "P5"
    wl = Workload("C4" if kda else "C3", B=B)
    if kda and not rows:
        wl.cfg = dataclasses.replace(wl.cfg, unit=0)
        wl.bits = Workload("C3").bits
    c, H, dk, dv = wl.cfg, wl.H, wl.dk, wl.dv
    T = B * Lp
    desc = stq.make_desc(B, H, dk, dv, np.asarray(wl.bits).reshape(-1), wl.row_weight, c.gate, c.unit, 0, 0)
    buf = torch.empty(stq.stq_pool_bytes(desc), dtype=torch.uint8, device=dev)
    pool = stq.stq_pool_create(desc, buf)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed * 100 + 77)
    r_prof = torch.as_tensor(wl.r_prof, dtype=torch.float32, device=dev)
    c_prof = torch.as_tensor(wl.c_prof, dtype=torch.float32, device=dev)
    z = torch.randn((B, H, dk, dv), generator=gen, device=dev)
    stq.stq_pool_store(pool, slots, (0.1 * z * r_prof[None, :, :, None] * c_prof[None, :, None, :]).contiguous())
    del z
    # prompts: the per-token law of workloads.Workload (normalised q, k with the
    # persistent row profile, v with the column profile, GDN half-life gates), drawn on the GPU
    rbar = r_prof / torch.exp(torch.log(r_prof).mean(dim=1, keepdim=True))
    cbar = c_prof / torch.exp(torch.log(c_prof).mean(dim=1, keepdim=True))
    q = torch.randn((T, H, dk), generator=gen, device=dev)
    k = torch.randn((T, H, dk), generator=gen, device=dev) * torch.sqrt(rbar)[None]
    v = torch.randn((T, H, dv), generator=gen, device=dev) * cbar[None]
    q = (q / q.norm(dim=-1, keepdim=True)).contiguous()
    k = (k / k.norm(dim=-1, keepdim=True)).contiguous()
    b = (0.05 + 0.9 * torch.rand((T, H), generator=gen, device=dev)).contiguous()
    hl = torch.as_tensor(wl.half_life, dtype=torch.float32, device=dev)
    if kda:
        hp = hl[None] * torch.exp(0.1 * torch.randn((T, H, dk), generator=gen, device=dev))
        a = (2.0 ** (-1.0 / hp)).contiguous()
    else:
        hp = hl[None, :] * torch.exp(0.1 * torch.randn((T, H), generator=gen, device=dev))
        a = torch.clamp(2.0 ** (-1.0 / hp), 0.9, 0.9999).contiguous()
    ss = torch.arange(0, T + 1, Lp, dtype=torch.int32, device=dev)
    o = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
    return {"wl": wl, "desc": desc, "buf": buf, "pool": pool, "slots": slots, "ss": ss, "o": o, "T": T,
            "q": q, "k": k, "v": v, "a": a, "b": b}


def prefill_bench(args):
    """P3: prefill ingest of a batch of prompts into the C3 pool (GDN head mix,
    H = 32, d = 128): one step = one stq_prefill call over all prompts.  P4: the
    same with per-channel (KDA) gates of C4's half-life law on per-head widths
    of the same mix (the chunkwise form with the gate products folded into the
    keys and queries).  P5: P4's prompts into the C4 pool itself (per-key-row
    widths: records decoded and refitted on chip)."""
    import torch

    import quantized_linear_attention_amd as stq
    dev = torch.device("cuda:0")
    B, Lp = args.prompts, args.prompt_len
    kda = args.workload in ("P4", "P5")
    rows = args.workload == "P5"
    st = prefill_setup(args.workload, B, Lp, dev)
    wl, pool, slots, ss, o = st["wl"], st["pool"], st["slots"], st["ss"], st["o"]
    q, k, v, a, b = (st[x] for x in "qkvab")
    c, H, dk, dv, T = wl.cfg, wl.H, wl.dk, wl.dv, st["T"]
    K = 8 if args.steps is None else args.steps
    Wu = 2 if args.warmup is None else args.warmup
    torch.cuda.synchronize()
    for _ in range(Wu):
        stq.stq_prefill(pool, slots, ss, q, k, v, a, b, o)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    for s in range(K):
        ev[s].record()
        stq.stq_prefill(pool, slots, ss, q, k, v, a, b, o)
    ev[K].record()
    torch.cuda.synchronize()
    per = np.array([ev[s].elapsed_time(ev[s + 1]) for s in range(K)])
    total_ms = float(ev[0].elapsed_time(ev[K]))
    avg_ms = float(per.mean())
    # the method's own work (the chunk form issues more on the matrix cores:
    # flops_issued; with per-channel gates the gate is a per-chunk scaling of
    # the keys and queries on the vector ALUs)
    flops = method_flops(T, H, dk, dv, kda)
    issued = prefill_flops(T, H, dk, dv)
    tflops = flops / (avg_ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build()
        ns, Ls = 2, 64
        P = oracle.OraclePool(ns, H, dk, dv, np.asarray(wl.bits).reshape(-1), wl.row_weight, c.gate, c.unit, 0)
        P.store(np.arange(ns), wl.state(np.arange(ns)))
        pr = wl.prompts([Ls] * ns)
        calls = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            P.prefill(np.arange(ns), *pr)
            calls += 1
        el = time.perf_counter() - t0
        cpu = {"value": calls * ns * Ls * H / el, "unit": "request-head prompt tokens/s",
               "cores": oracle.num_threads(), "kind": "oracle",
               "sample": "%d calls x %d prompts of %d tokens, all %d heads, %.1f s" % (calls, ns, Ls, H, el)}
    gname = "KDA per-channel gates" if kda else "GDN"
    mix = ("per-key-row widths {4b:30%, 6b:50%, 8b:19%, fp16:1%}" if rows
           else "heads {4b:9, 6b:16, 8b:6, fp16:1}")
    line = {
        "metric": "request-head prompt tokens/s (prefill ingest, B=%d prompts x %d tokens, H=32, d=128, "
                  "6-bit nominal %s pool%s)" % (B, Lp, gname, ", per-key-row widths" if rows else ""),
        "value": T * H * K / (total_ms * 1e-3),
        "unit": "request-head prompt tokens/s",
        "n_gpus": 1, "steps": K, "warmup": Wu, "ms_per_step": total_ms / K,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 state and products, 4/6/8-bit + f16 final state",
        "data": "synthetic (seeded; states and prompts drawn on the GPU with the workload recipe)",
        "config": {"workload": "prefill of %d prompts x %d tokens into the %s pool H=32 d_k=d_v=128, %s"
                               % (B, Lp, gname, mix),
                   "global_batch": B, "prompt_len": Lp, "heads": H, "d_k": dk, "d_v": dv},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_F32_PEAK, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_F32_PEAK, "traffic": None,
                     "kernel": "%s<128, 128, %s>" % ("k_prefill_rows" if rows else "k_prefill", "true" if kda else "false"),
                     "flops_per_launch": flops, "flops_issued_per_launch": issued,
                     "issued_tflops": issued / (avg_ms * 1e-3) / 1e12, "avg_launch_ms": avg_ms,
                     "p10_ms": float(np.percentile(per, 10)), "p90_ms": float(np.percentile(per, 90)),
                     "hbm_gbs": (T * H * (4 * (2 * dk + 2 * dv) + 8)) / (avg_ms * 1e-3) / 1e9},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
