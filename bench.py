#!/usr/bin/env python3
"""Benchmark of the W1.58A8 BitLinear forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--tokens M]

A step is one pass of the per-token hot path over one batch of synthetic
input: per-token absmax int8 quantization, load + unpack of the packed
ternary weights, the int32 contraction, the float rescale (and ReLU^2 where
the workload has it) for every linear of the workload.  Weights are quantized
and packed once, before timing (offline, as the packed form is what a model
stores); that offline pass is timed separately and reported as
``offline_weight_quant_ms``.

Default workload: the decode GEMV pair at M=1 (up 2560->6912, ReLU^2, down
6912->2560, bf16 activations).  Its 8.85 MB of packed weights would sit in
the 256 MB Infinity Cache, so steps rotate over enough weight copies that
the weights stream from HBM.

The K timed steps run as one HIP graph replay on torch's stream, bracketed
by synchronizations; the JSON line carries whole-step throughput (``value``),
the roofline of the dominant kernel (timed with HIP events around a graph of
back-to-back launches of that kernel alone), and the CPU oracle timed on a
bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("ternary GEMV HBM GB/s (% of peak), µs/token for all linears; "
          "prefill int8 TOPS")
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, 5.0 POP/s
MALL_BYTES = 256 * 1024 * 1024  # Infinity Cache
# Sources of each measured kernel: a committed counter summary applies only
# to the kernel version it was taken on (matched by their hash).
GEMV_SOURCES = ["gemv.hip", "gemv_tile.hpp", "common.hpp"]
GEMM_SOURCES = ["gemm.hip", "group.hpp", "common.hpp"]
GROUP_SOURCES = ["group.hip", "group.hpp", "gemv_tile.hpp", "quant_row.hpp", "common.hpp"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_gemv_pair_m1")
    p.add_argument("--tokens", type=int, default=None, help="M for multi-M workloads")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="time budget of the CPU oracle sample")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--kernel-launches", type=int, default=400,
                   help="launches of the dominant kernel timed for the roofline")
    p.add_argument("--glu", action="store_true",
                   help="gated FFN: pack each gate+up linear (N = 2 x the down projection's K) "
                        "for the gated squared-ReLU epilogue (output N/2)")
    p.add_argument("--subln", action="store_true",
                   help="give every linear a subln gain (RMSNorm fused into its quantization)")
    p.add_argument("--grouped", action="store_true",
                   help="run all linears of a step as one grouped forward (M <= 4)")
    p.add_argument("--probes", action="store_true",
                   help="only run the context probes: streaming-read bandwidth (1 GiB, a "
                        "2B decode step's 521 MB, one 4.4 MB GEMV's worth) and the int8 "
                        "matrix-core rate (both MFMA shapes)")
    p.add_argument("--copy-probe", action="store_true",
                   help="only time a plain 1 GiB device-to-device copy (achievable HBM "
                        "bandwidth, and the known-size kernel for counter calibration)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# Workload runners: allocate everything up front; step(i) only launches.
# ---------------------------------------------------------------------------
class Linear:
    def __init__(self, bl, torch, dev, N, K, M, x_dtype, seed, sparse, copies, subln=False,
                 glu=False):
        self.N, self.K, self.M = N, K, M
        self.epi = "relu2_glu" if glu else None
        gen = torch.Generator(device=dev)
        self.packed, self.gamma = [], []
        t0 = time.perf_counter()
        for c in range(copies):
            gen.manual_seed(seed * 131 + c)
            W = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32) * 0.02
            if sparse > 0:
                mask = torch.rand((N, K), generator=gen, device=dev) < sparse
                W = torch.where(mask, W * 1e-3, W)
            p, g = bl.quantize_weights(W, glu=glu)
            self.packed.append(p)
            self.gamma.append(g)
            del W
        torch.cuda.synchronize()
        self.quant_s = time.perf_counter() - t0
        gen.manual_seed(seed * 131 + 7777)
        X = torch.randn((M, K), generator=gen, device=dev, dtype=torch.float32)
        self.X = X.to(x_dtype) if x_dtype is not None else X
        self.Y = torch.empty((M, N // 2 if glu else N), dtype=torch.float32, device=dev)
        self.gain = None
        if subln:  # gains uniform on [0.5, 1.5)
            gen.manual_seed(seed * 131 + 8888)
            self.gain = torch.rand(K, generator=gen, device=dev, dtype=torch.float32) + 0.5
        ws = bl.workspace_bytes(M, K, N)
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev) if ws > 0 else None

    def bytes(self):
        """Algorithmic bytes of one forward: packed W + X in + Y out + gamma
        (+ the subln gain)."""
        return (self.N * self.K // 4 + self.X.numel() * self.X.element_size()
                + self.Y.numel() * 4 + 4 + (self.K * 4 if self.gain is not None else 0))

    def ops(self):
        return 2 * self.M * self.N * self.K


def build_runner(args, bl, torch, wl, dev):
    wk = wl.WORKLOADS[args.workload]
    M = args.tokens if args.tokens is not None else wk.tokens[0]
    if M not in wk.tokens:
        log(f"note: M={M} is not one of the workload's token counts {wk.tokens}")
    x_dtype = torch.bfloat16 if wk.x_kind.endswith("bf16") else None
    packed_per_step = wk.weights_per_step // 4
    # weight copies: enough that the bytes cycled through exceed 2x the MALL
    copies = max(1, -(-2 * MALL_BYTES // packed_per_step))
    copies = min(copies, 64)
    lins = []
    downs_k = {l.K for l in wk.linears}
    for layer, li, shape in wl.step_linears(wk):
        glu = bool(args.glu) and shape.N % 2 == 0 and shape.N // 2 in downs_k and \
            shape.N // 2 != shape.K
        lins.append(Linear(bl, torch, dev, shape.N, shape.K, M, x_dtype,
                           wl.weight_seed(wk.key, layer, li), wk.weight_sparse_frac, copies,
                           subln=args.subln, glu=glu))
    if wk.chain_relu2:
        # up (ReLU^2) feeds down: down's input is up's float output
        up, down = lins
        down.X = up.Y

    groups = None
    if args.grouped:
        if wk.chain_relu2:
            raise SystemExit("--grouped needs independent linears")
        groups = [bl.Group([(l.X, l.packed[c], l.gamma[c], l.N, l.epi, l.Y, l.gain)
                            for l in lins])
                  for c in range(copies)]

    def step(i):
        c = i % copies
        if groups is not None:
            groups[c].forward()
            return
        if wk.chain_relu2:
            up, down = lins
            bl.forward(up.X, up.packed[c], up.gamma[c], up.N, epilogue="relu2", out=up.Y,
                       workspace=up.ws, norm_gain=up.gain)
            bl.forward(down.X, down.packed[c], down.gamma[c], down.N, out=down.Y,
                       workspace=down.ws, norm_gain=down.gain)
        else:
            for lin in lins:
                bl.forward(lin.X, lin.packed[c], lin.gamma[c], lin.N, epilogue=lin.epi,
                           out=lin.Y, workspace=lin.ws, norm_gain=lin.gain)

    return wk, M, lins, copies, step, groups


def capture(torch, fn, count):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)  # one eager pass to settle any lazy initialisation
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(count):
            fn(i)
    return g


def time_graph(torch, fn, count):
    """Microseconds per call of fn(i), i < count, replayed as one graph."""
    g = capture(torch, fn, count)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / count


def roofline_single(args, torch, bl, wk, M, lins, metric_kind):
    """The linear with the most packed bytes, launched alone back to back
    (rotating its weight copies) in a graph bracketed by HIP events."""
    dom = max(lins, key=lambda l: l.N * l.K)
    epi = "relu2" if (wk.chain_relu2 and dom is lins[0]) else dom.epi
    n = args.kernel_launches
    copies = len(dom.packed)
    gemm = metric_kind == "tops" and dom.ws is not None
    if gemm:
        # The GEMM launch alone, from activations quantized beforehand (the
        # forward's other launch, the per-token quantization, is not the
        # contraction being measured).
        Xq, sx, rs = bl.quantize_acts(dom.X, norm_gain=dom.gain)
        qws = bl.forward_q_workspace(dom.M, dom.K, dom.N, dom.X.device)

    def dom_step(i):
        c = i % copies
        if gemm:
            bl.forward_q(Xq, sx, rs, dom.packed[c], dom.gamma[c], dom.N, epilogue=epi,
                         out=dom.Y, workspace=qws)
        else:
            bl.forward(dom.X, dom.packed[c], dom.gamma[c], dom.N, epilogue=epi, out=dom.Y,
                       workspace=dom.ws, norm_gain=dom.gain)

    us = time_graph(torch, dom_step, n)
    if metric_kind == "tops":
        achieved = dom.ops() / (us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": INT8_PEAK_TOPS,
                "unit": "TFLOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4)}
        key = f"gemm_q_{dom.K}x{dom.N}_m{M}"
        src = source_hash(GEMM_SOURCES)
    else:
        achieved = dom.bytes() / (us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        key = f"gemv_{dom.K}x{dom.N}_m{M}"
        src = source_hash(GEMV_SOURCES)
    roof["traffic"] = traffic_from_profile(src, key)
    roof["kernel"] = key
    roof["kernel_us"] = round(us, 3)
    roof["launches_timed"] = "gemm only (forward_q)" if gemm else (
        "quantization + gemm" if dom.ws is not None else "one fused launch")
    log(f"dominant forward {key}: {us:.3f} us per call")
    return roof


def roofline_grouped(args, torch, step, bytes_step, ops_step, wk, M, n_lin, metric_kind):
    """The grouped forward of a whole step (quantization included).  Up to 16
    tokens it streams the weights (HBM roof); above, it is one tiled int8 GEMM
    over all linears, and from 128 tokens on (where the step's ops per weight
    byte pass the chip's 625) the matrix cores bound it."""
    n = max(4, args.kernel_launches // 20)
    us = time_graph(torch, step, n)
    if metric_kind == "tops":
        achieved = ops_step / (us * 1e-6) / 1e12
        key = f"group_gemm_{wk.key}_m{M}"
        roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": INT8_PEAK_TOPS,
                "unit": "TFLOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4),
                "traffic": traffic_from_profile(source_hash(GEMM_SOURCES), key)}
    else:
        achieved = bytes_step / (us * 1e-6) / 1e9
        key = f"group_gemv_{wk.key}_m{M}"
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile(source_hash(GROUP_SOURCES), key)}
    roof.update({"kernel": key, "kernel_us": round(us, 3),
                 "launches_per_forward": 1 if M <= 4 else 2})
    log(f"grouped forward: {us:.3f} us per step ({n_lin} linears)")
    return roof


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample)
# ---------------------------------------------------------------------------
def cpu_baseline(args, wk, M, lins_shapes, metric_kind, budget_s, subln=False):
    import numpy as np

    import oracle
    from w1_a8_matmul_amd import workloads as wl

    orc = oracle.get()
    threads = orc.max_threads()
    rng_seed = 424242
    # one layer's linears (the sample); weights quantized by the oracle itself
    shapes = list(wk.linears)
    Ms = M if metric_kind != "tops" else min(M, 16)  # prefill: a sample of token rows
    prepared = []
    for li, lin in enumerate(shapes):
        W = wl.gen_weight(rng_seed + li, lin.N, lin.K, wk.weight_sparse_frac)
        _, gc, qw = orc.quantize_weights(W)
        del W
        X, is_bf16 = wl.gen_acts(rng_seed + 100 + li, Ms, lin.K, wk.x_kind)
        g = wl.gen_gain(rng_seed + 200 + li, lin.K) if subln else None
        prepared.append((lin, qw, gc, X, is_bf16, g))

    def fwd(X, qw, gc, bf16, g):
        if g is None:
            y, *_ = orc.forward(X, qw, gc, bf16=bf16)
            return y
        q, s, _ = orc.quant_acts_rmsnorm(X, g, 1e-5, bf16=bf16)
        return orc.rescale(orc.int_matmul(q, qw), s, gc)

    def one_pass():
        if wk.chain_relu2:
            (lu, qu, gu, Xu, bu, guu), (ld, qd, gd, _, _, gdd) = prepared
            h = orc.relu2(fwd(Xu, qu, gu, bu, guu))
            fwd(h, qd, gd, False, gdd)
        else:
            for lin, qw, gc, X, is_bf16, g in prepared:
                fwd(X, qw, gc, is_bf16, g)

    one_pass()
    n = 0
    t0 = time.perf_counter()
    while True:
        one_pass()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 100000:
            break
    per_pass = el / n
    layer_bytes = sum(lin.N * lin.K // 4 + Ms * lin.K * (2 if is_bf16 else 4) + Ms * lin.N * 4 + 4
                      for lin, _, _, _, is_bf16, _ in prepared)
    layer_ops = sum(2 * Ms * lin.N * lin.K for lin, *_ in prepared)
    if subln:
        layer_bytes += sum(lin.K * 4 for lin, *_ in prepared)
    if metric_kind == "tops":
        value, unit = layer_ops / per_pass / 1e12, "TOPS"
    else:
        value, unit = layer_bytes / per_pass / 1e9, "GB/s"
    sample = (f"{n} passes over one layer's linears ({', '.join(f'{l.K}->{l.N}' for l in shapes)})"
              f" at M={Ms}, {el:.1f} s; oracle on unpacked int8 weights, OpenMP over outputs")
    return {"value": round(value, 4), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": sample, "us_per_layer_pass": round(per_pass * 1e6, 1)}


def traffic_from_profile(kernel_src_hash, kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on another version of the kernel."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get(kernel_key)
    if not ent or ent.get("source_sha1") != kernel_src_hash:
        return None
    return ent.get("hbm_bytes_per_launch")


def source_hash(names):
    h = hashlib.sha1()
    for n in names:
        with open(os.path.join(ROOT, "w1_a8_matmul_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def copy_probe(torch, nbytes=1 << 30, reps=10):
    """A plain device copy of known size: reads and writes nbytes each."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"probe": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "ms": round(ms, 4), "GBps_read_plus_write": round(2 * nbytes / ms / 1e6, 1)}),
          flush=True)


def context_probes(torch):
    """Achievable streaming-read bandwidth and int8 MFMA rate on this GPU.

    Context for the roofline fractions (which use the published peaks)."""
    import ctypes

    from w1_a8_matmul_amd.build import PROBES_LIBRARY

    L = ctypes.CDLL(PROBES_LIBRARY)
    L.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_void_p]
    L.probe_mfma_i8.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    st = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731
    out = {"probe": "context", "compute_units": cus}

    # streaming read: sizes x buffer copies (copies rotate so that the small
    # sizes stream from HBM rather than the 256 MB Infinity Cache)
    for label, nbytes, copies in (("1GiB", 1 << 30, 1), ("2b_step_521MB", 521011200, 1),
                                  ("gemv_4.4MB", 4423680, 61)):
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(copies)]
        best = None
        for wg_per_cu in (2, 3, 4, 8):
            grid = wg_per_cu * cus

            def fn(i):
                b = bufs[i % copies]
                rc = L.probe_stream_read(b.data_ptr(), nbytes, sink.data_ptr(), grid, st())
                assert rc == 0, rc

            us = time_graph(torch, fn, 4 if copies == 1 else 200)
            gbs = nbytes / (us * 1e-6) / 1e9
            if best is None or gbs > best[0]:
                best = (round(gbs, 1), round(us, 3), wg_per_cu)
        out[f"read_{label}"] = {"GBps": best[0], "us": best[1], "wg_per_cu": best[2]}
        del bufs
    # int8 matrix cores: random operand bytes, then operands shaped like the
    # GEMM's (A: quantized N(0,1) activations, B: codes 0/1/2 with 35% zeros)
    src = torch.randint(-2**31, 2**31 - 1, (4096,), dtype=torch.int32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    a_bytes = torch.clamp(torch.round(torch.randn(8192, device="cuda", generator=gen) * 28.0),
                          -127, 127).to(torch.int8)
    u = torch.rand(8192, device="cuda", generator=gen)
    b_codes = torch.where(u < 0.35, 1, torch.where(u < 0.675, 0, 2)).to(torch.int8)
    src_t = torch.cat([a_bytes, b_codes]).view(torch.int32).contiguous()
    for shape, label, macs, operands in (
            (0, "mfma_i32_16x16x64_i8", 8 * 16 * 16 * 64, src),
            (1, "mfma_i32_32x32x32_i8", 4 * 32 * 32 * 32, src),
            (1, "mfma_i32_32x32x32_i8_ternary_operands", 4 * 32 * 32 * 32, src_t)):
        src = operands
        best = None
        for wg_per_cu in (1, 2, 4):
            grid, iters = wg_per_cu * cus, 2000

            def fn(i):
                rc = L.probe_mfma_i8(shape, src.data_ptr(), iters, sink.data_ptr(), grid, st())
                assert rc == 0, rc

            us = time_graph(torch, fn, 5)
            tops = 2 * macs * iters * grid * 4 / (us * 1e-6) / 1e12
            if best is None or tops > best[0]:
                best = (round(tops, 1), wg_per_cu * 4)
        out[label] = {"TOPS": best[0], "waves_per_cu": best[1]}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; "
                                   f"--gpus {args.gpus} is not supported (the forward is "
                                   "single-GPU; see the sharding note in the design notes)"}))
        sys.exit(2)
    import torch

    from w1_a8_matmul_amd import bitlinear as bl
    from w1_a8_matmul_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_probe:
        copy_probe(torch)
        return
    if args.probes:
        context_probes(torch)
        return
    bl.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wk, M, lins, copies, step, groups = build_runner(args, bl, torch, wl, dev)
    quant_s = sum(l.quant_s for l in lins)
    n_weights = sum(l.N * l.K for l in lins) * copies
    log(f"workload {wk.key} M={M}: {len(lins)} linears, {copies} weight copies, "
        f"offline quantization {quant_s*1e3:.1f} ms for {n_weights/1e6:.1f} M weights")

    # In the ReLU^2 chain the hidden vector h counts twice: written by the up
    # projection and read by the down projection, as it is on the device.
    bytes_step = sum(l.bytes() for l in lins)
    ops_step = sum(l.ops() for l in lins)
    metric_kind = "tops" if M >= 128 else "hbm"

    # warmup
    if args.warmup > 0:
        gw = capture(torch, step, args.warmup)
        gw.replay()
        torch.cuda.synchronize()
        log(f"warmup {args.warmup} steps done")
    g = capture(torch, step, args.steps)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / args.steps
    log(f"timed {args.steps} steps: wall {wall*1e3:.3f} ms, events {gpu_ms:.3f} ms")

    if groups is not None:
        roof = roofline_grouped(args, torch, step, bytes_step, ops_step, wk, M, len(lins),
                                metric_kind)
    else:
        roof = roofline_single(args, torch, bl, wk, M, lins, metric_kind)

    step_s = ms_per_step / 1e3
    if metric_kind == "tops":
        value, unit = ops_step / step_s / 1e12, "TOPS"
    else:
        value, unit = bytes_step / step_s / 1e9, "GB/s"

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(args, wk, M, wk.linears, metric_kind, args.cpu_seconds,
                           subln=args.subln)
        log(f"cpu oracle: {cpu}")

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": wk.key,
            "description": wk.description,
            "tokens": M,
            "linears_per_step": len(lins),
            "weight_copies_rotated": copies,
            "bytes_per_step": bytes_step,
            "ops_per_step": ops_step,
            "us_per_token": round(ms_per_step * 1e3 / M, 3),
            "gpu_event_ms_per_step": round(gpu_ms / args.steps, 6),
            "offline_weight_quant_ms": round(quant_s * 1e3 / copies, 3),
            "grouped": groups is not None,
            "subln": bool(args.subln),
            "glu": bool(args.glu),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
