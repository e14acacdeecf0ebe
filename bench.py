#!/usr/bin/env python3
"""Benchmark of the block-FP8 routed MoE layer on one MI355X.

One step = one moe_forward call (router, top-k, permutation, gate/up+SwiGLU,
down, combine) over one batch of synthetic tokens already resident in HBM.
Successive steps rotate over R input batches and C device copies of the
expert bank, so that repeated calls cannot be served from the 256 MB MALL.

Prints one JSON line: MoE-layer tokens/s, plus
  roofline:     the dominant kernel (gate/up expert pass) timed with HIP events
                attached to its own dispatch (the library launches it with
                hipExtLaunchKernel when the caller passes them): on every timed
                step of a prefill-sized workload, on every 21st step of a
                decode-sized one (recording them costs the stream about 1 us,
                which a ~20-80 us decode step would feel), and always on at
                least the last timed step; algorithmic bytes = the bytes of the
                experts the step's routing touches (E4M3 weights + fp32
                scales), or algorithmic FLOPs for MFMA-bound workloads;
  cpu_baseline: the CPU oracle (fp64 NumPy) timed on a bounded sample of the
                same workload on this host (consecutive token chunks of the
                input batches, for about --cpu-seconds);
  roofline.traffic: HBM bytes per launch of that kernel, from rocprofv3 PMC
                runs (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by
                the bytes a plain copy kernel of known size moves per KiB the
                same counter reports), read from profiles/traffic.json when its
                recorded hash of the kernel code (comments and whitespace left
                out) matches the current sources; null otherwise.

The default workload is the 512-expert, 4096-token prefill layer (hidden 4096,
top-10 + 1 shared expert, skewed routing): the largest one-GPU configuration.
After the W warm-up steps, further untimed steps run until --settle-seconds
have passed, so that the K timed steps see the steady clock the chip settles
at under load rather than the first steps' ramp.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c4] [--tokens T]
                       [--path auto|gemv|mfma|mfma_fp8]
       (mfma_fp8: the variant with E4M3 operands in both expert contractions;
        its roofline takes the FP8 peak, 5.0 PFLOP/s, and its ridge)
       python bench.py --stream-slots N [--config c3]  (routed experts streamed from pinned
                                      host memory through an LRU cache of N device slots)
       python bench.py --copy-calibration            (the copy kernel for the counters)
       python bench.py --gemm-calibration --config c4  (library bf16 GEMMs at the expert shapes)
       python bench.py --traffic-report FETCH.csv WRITE.csv COPYF.csv COPYW.csv --config c1
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
EV_EVERY = 21                  # decode default: timed steps per step that records the gate/up
                               # events (coprime with the input batches and bank copies)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Hip:
    """The few HIP runtime calls the timing needs (the process's own runtime)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def record(self, ev, stream):
        assert self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                            ctypes.c_void_p(b)) == 0
        return ms.value


def expert_bytes(shape):
    return shape.expert_bytes()


def cpu_baseline(shape, host, x_batches, seconds, chunk=64):
    """Time the CPU oracle on consecutive chunks of at most `chunk` tokens of
    the input batches (in order) for about `seconds` (at least one chunk)."""
    import numpy as np
    import oracle
    import workloads as W
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    bank, shared = host
    sh = W.bank_expert(shared, 0) if shape.shared else None
    wr, b = W.gen_router(shape), W.gen_bias(shape)
    chunks = [xb[lo:lo + chunk] for xb in x_batches for lo in range(0, len(xb), chunk)]
    done, t0, i = 0, time.perf_counter(), 0
    while True:
        x = chunks[i % len(chunks)]
        oracle.moe_layer(x, wr, b, lambda e: W.bank_expert(bank, e), shape.top_k, shape.inter,
                         shape.block, shared=sh)
        done += len(x)
        i += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": done / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": (f"{i} oracle forwards of {len(chunks[0])} tokens ({done} tokens, "
                   f"{el:.1f} s): consecutive chunks of the timed workload's input batches, "
                   f"same bank and router; fp64 NumPy, "
                   f"BLAS may use {cores} threads, decode and dequantisation single-threaded; "
                   f"host CPU: {model}"),
    }


# sources that define each dominant kernel (its traffic is void once they change)
KERNEL_SOURCES = {
    "gemv": ["expert_gemv.hip", "gemv_body.hpp", "device.hpp", "layer.hpp"],
    "gemv_fused": ["decode_fused.hip", "gemv_body.hpp", "router_decode.hpp", "select.hpp",
                   "permute.hpp", "device.hpp", "layer.hpp"],
    "mfma": ["expert_mfma.hip", "device.hpp", "layer.hpp"],
    "mfma_fp8": ["expert_mfma.hip", "device.hpp", "layer.hpp"],
}
# the dominant kernel of each path: the gate/up kernel, or the launch that
# holds it (the decode layer's single launch; the grouped paths' gate/up +
# down launch)
KERNEL_MATCH = {"gemv": "gemv_gate_up<", "gemv_fused": "decode_fused<", "mfma": "mfma_layer<",
                "mfma_fp8": "mfma_layer_f8<"}
COPY_MATCH = "MulFunctor"  # the copy kernel of --copy-calibration (dst = src * 1)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COPY_MIB = 512


def code_text(src):
    """Kernel source without its comments and with whitespace collapsed, so
    that a recorded traffic figure survives edits that change no code."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def sources_sha(family):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "block_fp8_routed_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()


def traffic_key(config, tokens, family):
    return f"{config}:T{tokens}:{family}"


def copy_calibration():
    """The plain copy kernel the counters are calibrated on: an elementwise
    kernel reading COPY_MIB MiB and writing as many, five times."""
    import torch
    n = COPY_MIB * 2**20 // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda")  # contents do not matter
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 5}))


def gemm_calibration(shape):
    """The vendor library's bf16 GEMM (torch.matmul -> hipBLASLt) at one
    expert's gate/up (rows x H -> 2I) and down (rows x I -> H) shapes for
    several group sizes, plus a large square product: a reference for what
    a dense bf16 contraction of these sizes reaches on this chip, with bf16
    weights (no dequantisation) and one launch per expert."""
    import torch
    torch.manual_seed(0)
    H, I = shape.hidden, shape.inter

    def rate(M, N, K, what, reps=50):
        a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(N, K, device="cuda", dtype=torch.bfloat16)
        bt = b.t()  # weights stored row-major [N][K], as the experts are
        for _ in range(5):
            c = a @ bt
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            c = a @ bt
        e1.record()
        torch.cuda.synchronize()
        del c
        us = e0.elapsed_time(e1) / reps * 1e3
        tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
        print(json.dumps({"what": what, "M": M, "N": N, "K": K, "us": round(us, 2),
                          "TFLOPs": round(tf, 1), "frac_of_2.5PF": round(tf / 2500, 4)}), flush=True)

    for rows in (64, 256, 1024, 2048, 4096):
        rate(rows, 2 * I, H, "gate/up")
        rate(rows, H, I, "down")
    rate(8192, 8192, 8192, "square")


def counter_means(path, match):
    """Mean counter value (KiB) per dispatch of the kernels whose name holds match."""
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path)) if match in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no dispatch of {match!r} in {path}")
    return sum(vals) / len(vals), len(vals)


def traffic_report(args):
    fetch_csv, write_csv, copy_f_csv, copy_w_csv = args.traffic_report
    import workloads as W
    shape = W.CONFIGS[args.config]
    T = args.tokens if args.tokens is not None else shape.tokens
    import torch
    import block_fp8_routed_amd as moe
    xdt = torch.bfloat16 if shape.x_dtype == "bf16" else torch.float32
    cfg = moe.make_config(T, shape.hidden, shape.experts, shape.inter, shape.top_k,
                          shape.block, shape.shared, xdt, torch.float32, args.path)
    # the family the library takes for this call (the grouped ones keep h's
    # exponent bytes)
    grouped = moe.workspace_region(cfg, moe.MOE_WS_H_EXPS)[1] > 0
    family = args.path if args.path in ("mfma", "mfma_fp8") else "mfma" if grouped else "gemv"
    if family == "gemv":  # the single-launch decode layer where the library takes it
        if moe.workspace_region(cfg, moe.MOE_WS_STATUS)[1] > 0:
            family = "gemv_fused"
    f_kib, nf = counter_means(fetch_csv, KERNEL_MATCH[family])
    w_kib, nw = counter_means(write_csv, KERNEL_MATCH[family])
    cf_kib, _ = counter_means(copy_f_csv, COPY_MATCH)
    cw_kib, _ = counter_means(copy_w_csv, COPY_MATCH)
    copy_bytes = COPY_MIB * 2**20
    fetch_scale, write_scale = copy_bytes / (cf_kib * 1024), copy_bytes / (cw_kib * 1024)
    entry = {
        "kernel": KERNEL_MATCH[family], "config": args.config, "tokens": T,
        "sources_sha256": sources_sha(family),
        "fetch_kib_per_dispatch": round(f_kib, 1), "write_kib_per_dispatch": round(w_kib, 1),
        "dispatches": [nf, nw],
        "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_kib": round(cf_kib, 1),
                             "write_kib": round(cw_kib, 1), "fetch_bytes_per_kib": fetch_scale,
                             "write_bytes_per_kib": write_scale},
        "traffic_bytes_per_launch": round(f_kib * 1024 * fetch_scale + w_kib * 1024 * write_scale),
    }
    table = {}
    if os.path.exists(TRAFFIC_FILE):
        table = json.load(open(TRAFFIC_FILE))
    table[traffic_key(args.config, T, family)] = entry
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(entry))


def recorded_traffic(config, tokens, family):
    """Traffic per launch from profiles/traffic.json, if taken on the current sources."""
    try:
        entry = json.load(open(TRAFFIC_FILE)).get(traffic_key(config, tokens, family))
    except (OSError, ValueError):
        return None
    if not entry or entry.get("sources_sha256") != sources_sha(family):
        return None
    return entry["traffic_bytes_per_launch"]


def stream_main(args):
    """moe_forward_streamed on the workload: every step routes a new input
    batch (batches rotate), brings its missing experts from pinned host
    memory into the least recently used device slots, and runs the layer.
    Each call returns once its work is done, so steps are timed on the host
    clock. Reports tokens/s, the cache's hit rate and the host-to-device
    expert rate."""
    import numpy as np
    import torch
    import workloads as W
    import block_fp8_routed_amd as moe

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    moe.load()
    dev = torch.device("cuda:0")
    shape = W.CONFIGS[args.config]
    T = args.tokens if args.tokens is not None else shape.tokens
    H, E, I, B, k = shape.hidden, shape.experts, shape.inter, shape.block, shape.top_k
    xdt = torch.bfloat16 if shape.x_dtype == "bf16" else torch.float32
    log(f"generating {args.config} bank (E={E}) into pinned host memory")
    bank_h = W.gen_bank(shape)
    host = moe.Bank.pinned_from_numpy(bank_h)
    del bank_h
    shared = moe.Bank.from_numpy(W.gen_bank(shape, shared=True), dev) if shape.shared else None
    slots = args.stream_slots
    cache = moe.ExpertCache(slots)
    slot_bank = moe.Bank.empty_slots(slots, H, I, B, dev)
    router = torch.from_numpy(W.gen_router(shape)).to(dev)
    bias_h = W.gen_bias(shape)
    bias = None if bias_h is None else torch.from_numpy(bias_h).to(dev)
    xs = [torch.from_numpy(W.gen_x(shape, T, batch=r)).to(xdt).to(dev) for r in range(args.batches)]
    cfg = moe.make_config(T, H, E, I, k, B, shape.shared, xdt, torch.float32, args.path)
    ws = moe.make_workspace(cfg, dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)

    def call(i):
        moe.moe_forward_streamed(xs[i % len(xs)], router, host, slot_bank, cache, k, B,
                                 shared=shared, router_bias=bias, path=args.path, out=out,
                                 workspace=ws)

    log(f"warmup {args.warmup} streamed steps (T={T}, slots={slots})")
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    h0, m0, b0 = cache.hits, cache.misses, cache.bytes_in
    rounds = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(args.warmup + i)
        rounds.append(cache.rounds_last)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    hits, misses, bytes_in = cache.hits - h0, cache.misses - m0, cache.bytes_in - b0
    res = {
        "metric": "MoE-layer tokens/s, routed experts streamed host->HBM through an LRU cache",
        "value": round(T * args.steps / el, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(el / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if args.path == "mfma_fp8" else "bf16" if xdt == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.config} {shape.name}: hidden {H}, {E} experts top-{k}"
                               f"{' + 1 shared (resident)' if shape.shared else ''}, inter {I}, "
                               f"{T} tokens per step, routed experts in pinned host memory, "
                               f"{slots} device expert slots (LRU)",
                   "tokens": T, "slots": slots, "input_batches": len(xs), "path": args.path},
        "stream": {
            "hit_rate": round(hits / max(hits + misses, 1), 4),
            "experts_needed_per_step": round((hits + misses) / args.steps, 2),
            "experts_copied_per_step": round(misses / args.steps, 2),
            "bytes_in_per_step": round(bytes_in / args.steps),
            "host_to_device_GBps": round(bytes_in / el / 1e9, 2),
            "rounds_per_step": round(sum(rounds) / len(rounds), 2),
        },
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c4", choices=["c0", "c1", "c2", "c3", "c4"])
    ap.add_argument("--tokens", type=int, default=None, help="tokens per step (default: config)")
    ap.add_argument("--path", default="auto",
                    choices=["auto", "gemv", "gemv_fused", "mfma", "mfma_fp8"],
                    help="expert family; mfma_fp8 runs both expert contractions on E4M3 "
                         "operands (a numerics variant, never chosen by auto); gemv_fused "
                         "the whole decode layer in one launch (never chosen by auto)")
    ap.add_argument("--batches", type=int, default=8, help="distinct input batches rotated")
    ap.add_argument("--copies", type=int, default=0, help="device copies of the bank (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-chunk", type=int, default=64,
                    help="tokens per oracle call in the cpu_baseline sample")
    ap.add_argument("--settle-seconds", type=float, default=2.0,
                    help="untimed steps after the warm-up until this much time has passed")
    ap.add_argument("--event-every", type=int, default=None,
                    help="record the gate/up kernel events on every N-th timed step "
                         "(default: 1 above 16 tokens per step, else 21; always at least the "
                         "last timed step; 0: none, no roofline figure)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stream-slots", type=int, default=0,
                    help="run moe_forward_streamed: routed experts in pinned host memory, "
                         "an LRU cache of this many device expert slots")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the copy kernel the PMC counters are calibrated on")
    ap.add_argument("--gemm-calibration", action="store_true",
                    help="time the library bf16 GEMM at the workload's expert shapes")
    ap.add_argument("--traffic-report", nargs=4, metavar="CSV",
                    help="FETCH_SIZE, WRITE_SIZE, copy FETCH_SIZE, copy WRITE_SIZE counter CSVs: "
                         "record the dominant kernel's traffic in profiles/traffic.json")
    args = ap.parse_args()
    if args.traffic_report:
        traffic_report(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gemm_calibration:
        import workloads as W
        gemm_calibration(W.CONFIGS[args.config])
        return
    if args.stream_slots:
        if args.gpus != 1:
            print("bench.py measures one GPU only", file=sys.stderr)
            sys.exit(2)
        stream_main(args)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(this layer is built and measured on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as W
    import block_fp8_routed_amd as moe

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    lib = moe.load()
    hip = Hip()
    dev = torch.device("cuda:0")
    shape = W.CONFIGS[args.config]
    T = args.tokens if args.tokens is not None else shape.tokens
    H, E, I, B, k = shape.hidden, shape.experts, shape.inter, shape.block, shape.top_k
    xdt = torch.bfloat16 if shape.x_dtype == "bf16" else torch.float32

    log(f"generating {args.config} bank (E={E}, H={H}, I={I})")
    t0 = time.perf_counter()
    bank_h = W.gen_bank(shape)
    shared_h = W.gen_bank(shape, shared=True) if shape.shared else None
    log(f"bank generated in {time.perf_counter() - t0:.1f} s")
    bank_bytes = (E + int(shape.shared)) * expert_bytes(shape)
    copies = args.copies or max(1, min(8, math.ceil(2.5e9 / bank_bytes)))
    banks = [moe.Bank.from_numpy(bank_h, dev)]
    for _ in range(copies - 1):
        b0 = banks[0]
        banks.append(moe.Bank(b0.w_gate_up.clone(), b0.s_gate_up.clone(), b0.w_down.clone(),
                              b0.s_down.clone()))
    shared = moe.Bank.from_numpy(shared_h, dev) if shape.shared else None
    router = torch.from_numpy(W.gen_router(shape)).to(dev)
    bias_h = W.gen_bias(shape)
    bias = None if bias_h is None else torch.from_numpy(bias_h).to(dev)
    x_host = [W.gen_x(shape, T, batch=r) for r in range(args.batches)]
    xs = [torch.from_numpy(x).to(xdt).to(dev) for x in x_host]

    cfg = moe.make_config(T, H, E, I, k, B, shape.shared, xdt, torch.float32, args.path)
    ws = moe.make_workspace(cfg, dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    f8 = args.path == "mfma_fp8"
    # the family the library takes (the grouped ones keep h's exponent bytes)
    mfma = moe.workspace_region(cfg, moe.MOE_WS_H_EXPS)[1] > 0
    # the single-launch decode layer has a status region (so have the grouped
    # paths, whose gate/up and down passes share one launch)
    fused = not mfma and moe.workspace_region(cfg, moe.MOE_WS_STATUS)[1] > 0
    one_launch = mfma
    family_key = "mfma_fp8" if f8 else "mfma" if mfma else "gemv_fused" if fused else "gemv"

    # routing of each batch: which experts a step touches (outside the timed region)
    uniq = []
    for x in xs:
        idx, _ = moe.moe_route(x, router, k, I, B, router_bias=bias)
        uniq.append(len(np.unique(idx.cpu().numpy())) + int(shape.shared))
    gu_bytes_per_expert = 2 * I * H + 4 * (2 * I // B) * (H // B)
    all_bytes_per_expert = expert_bytes(shape)

    def call(i, evs=None):
        r, c = i % len(xs), i % len(banks)
        st = lib.moe_forward(ctypes.c_void_p(xs[r].data_ptr()), ctypes.c_void_p(router.data_ptr()),
                             None if bias is None else ctypes.c_void_p(bias.data_ptr()),
                             ctypes.byref(banks[c].c),
                             ctypes.byref(shared.c) if shared is not None else None, k,
                             ctypes.c_void_p(out.data_ptr()), ctypes.byref(cfg),
                             ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                             ctypes.byref(evs) if evs is not None else None, ctypes.c_void_p(sp))
        if st != 0:
            raise moe.MoeError(st, "moe_forward")

    # the gate/up kernel's own start and end (PERMUTED -> GATE_UP, attached to
    # its dispatch) on every EV_EVERY-th timed step: recording them costs the
    # stream about a microsecond, so recording on every step would slow the
    # steps being timed
    K, Wm = args.steps, args.warmup
    every = args.event_every if args.event_every is not None else (1 if T > 16 else EV_EVERY)
    every = min(every, K)
    # (with every > 1 the first sample is step every-1: the first timed step
    # follows the settling phase's synchronize and can start at a lower clock)
    sampled = list(range(every - 1, K, every)) if every > 0 else []
    ev_pairs = [(hip.event(), hip.event()) for _ in sampled]
    ev_structs = {}
    for i, (a, b) in zip(sampled, ev_pairs):
        s = moe.MoePhaseEvents()
        s.ev[moe.MOE_EV_PERMUTED] = a
        s.ev[moe.MOE_EV_GATE_UP] = b
        ev_structs[i] = s
    start, stop = hip.event(), hip.event()

    log(f"warmup {Wm} steps (T={T}, copies={copies}, batches={len(xs)}, path={family_key})")
    for i in range(Wm):
        call(i)
    torch.cuda.synchronize()
    # settle: untimed steps until the clock has had settle_seconds under load
    settle, t_settle = 0, time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_seconds:
        for _ in range(8):
            call(Wm + settle)
            settle += 1
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle
    # keep the timed steps on the same rotation of batches and bank copies
    Wm_eff = Wm + settle
    log(f"settled for {settle} untimed steps ({settle_s:.1f} s); timing {K} steps")
    hip.record(start, sp)
    for i in range(K):
        call(Wm_eff + i, ev_structs.get(i))
    hip.record(stop, sp)
    torch.cuda.synchronize()
    total_ms = hip.elapsed_ms(start, stop)
    ms = total_ms / K
    gu_ms = [hip.elapsed_ms(a, b) for a, b in ev_pairs]
    if not gu_ms:  # --event-every 0: time the steps only
        print(json.dumps({"ms_per_step": round(ms, 5), "steps": K, "tokens_per_s": T / (ms / 1e3)}))
        return
    gu_avg_ms = sum(gu_ms) / len(gu_ms)
    # the bytes of the sampled steps (for the kernel) and of all steps (for the layer)
    gu_bytes = sum(uniq[(Wm_eff + i) % len(xs)] for i in sampled) / len(sampled) * gu_bytes_per_expert
    mean_uniq = sum(uniq[(Wm_eff + i) % len(xs)] for i in range(K)) / K
    layer_bytes = mean_uniq * all_bytes_per_expert

    # phase breakdown (outside the timed region): all phase events on a few
    # steps. Each stream-marker event costs the stream ~3 us, and the kernel-
    # attached pair starts ~6-10 us after a preceding marker, so "permute"
    # (ROUTED marker -> gate/up kernel start) carries that overhead; the
    # rocprofv3 kernel traces give the per-kernel times.
    phase = {n: [] for n in ("route", "permute", "gate_up", "down", "combine")}
    for i in range(0 if fused else min(20, K)):  # one kernel: no phases to split
        evs = [hip.event() for _ in range(moe.MOE_EV_COUNT)]
        s = moe.MoePhaseEvents()
        for j, e in enumerate(evs):
            s.ev[j] = e
        call(i, s)
        torch.cuda.synchronize()
        for j, n in enumerate(phase):
            phase[n].append(hip.elapsed_ms(evs[j], evs[j + 1]) * 1e3)
    phases_us = {n: round(sorted(v)[len(v) // 2], 2) for n, v in phase.items() if v}
    if one_launch and phases_us:  # the gate/up kernel's events span both passes
        phases_us["gate_up+down"] = round(phases_us.pop("gate_up") + phases_us.pop("down"), 2)

    tokens_per_s = T / (ms / 1e3)
    rows = T * k + T * int(shape.shared)
    flops = rows * 6 * H * I
    gu_flops = rows * 4 * H * I
    if fused or one_launch:  # the timed kernel runs both contractions: all expert bytes and products
        gu_bytes = gu_bytes / gu_bytes_per_expert * all_bytes_per_expert
        gu_flops = flops
    gu_s = gu_avg_ms / 1e3
    gbps = gu_bytes / gu_s / 1e9
    tflops = gu_flops / gu_s / 1e12
    # the gate/up kernel's bound: HBM unless its arithmetic intensity passes
    # the bf16 ridge point (peak FLOP/s over peak bytes/s)
    # (the fp8 ridge for the FP8 variant, whose products are fp8)
    peak = FP8_PEAK_TFLOPS if f8 else BF16_PEAK_TFLOPS
    ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    family = ("grouped FP8 MFMA, E4M3 x and h" if f8 else
              "grouped bf16 MFMA" if mfma else "wavefront GEMV")
    what = ("the whole decode layer in one launch (router, selection, permutation, gate/up + "
            "SwiGLU, down, combine; wavefront GEMV)" if fused else
            f"expert gate/up + SwiGLU and down in one launch ({family})" if one_launch else
            f"expert gate/up + SwiGLU ({family})")
    if gu_flops / gu_bytes > ridge:
        roof = {"bound": "mfma", "kernel": what,
                "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4), "traffic": None,
                "algorithmic_per_launch": gu_flops,
                "hbm_GBps": round(gbps, 1)}
    else:
        roof = {"bound": "hbm", "kernel": what,
                "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBS, 4), "traffic": None,
                "algorithmic_per_launch": round(gu_bytes),
                "mfma_TFLOPs": round(tflops, 2)}
    roof["avg_launch_us"] = round(gu_avg_ms * 1e3, 2)
    roof["launch_samples"] = len(sampled)
    roof["traffic"] = recorded_traffic(args.config, T, family_key)

    res = {
        "metric": "MoE-layer tokens/s; decode HBM GB/s vs peak, prefill MFMA util",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "settle": {"untimed_steps": settle, "seconds": round(settle_s, 2)},
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # arithmetic of the dominant gate/up pass: bf16 activations meet the
        # (exact) bf16 form of the E4M3 weights on both families, fp32
        # activations (the tiny layer) take fp32 products, the fp8 variant
        # E4M3 x E4M3 products (in both passes); accumulation is fp32
        # throughout (the down products of the other paths are fp16 x fp16)
        "dtype": "fp8" if f8 else "bf16" if xdt == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{args.config} {shape.name}: hidden {H}, {E} experts top-{k}"
                         f"{' + 1 shared' if shape.shared else ''}, inter {I}, E4M3 weights "
                         f"with {B}x{B} fp32 block scales, {T} tokens per step, "
                         f"{shape.x_dtype} activations"
                         f"{' (E4M3, one power-of-two scale per 128 columns, in both expert contractions, h likewise)' if f8 else ''}"
                         ", fp32 output"),
            "tokens": T, "hidden": H, "experts": E, "top_k": k, "inter": I, "block": B,
            "shared": shape.shared,
            "path": family_key,
            "bank_copies": copies, "input_batches": len(xs),
        },
        "roofline": roof,
        "layer": {
            "unique_experts_per_step": round(mean_uniq, 2),
            "expert_bytes_per_step": round(layer_bytes),
            "expert_GBps": round(layer_bytes / (ms / 1e3) / 1e9, 1),
            "expert_GBps_frac": round(layer_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "flops_per_step": flops,
            "mfma_util": round(flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 5),
            "phases_us_median": phases_us,
        },
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle for ~{args.cpu_seconds:.0f} s")
        res["cpu_baseline"] = cpu_baseline(shape, (bank_h, shared_h), x_host, args.cpu_seconds,
                                           args.cpu_chunk)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
