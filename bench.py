#!/usr/bin/env python3
"""Benchmark of the W1.58A8 BitLinear forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--tokens M] [--grouped | --per-linear] [--b3] [--lut] [--no-sub]
                    [--no-cpu]

A step is one pass of the per-token hot path over one batch of synthetic
input: per-token absmax int8 quantization, load + unpack of the packed
ternary weights, the int32 contraction, the float rescale (and ReLU^2 where
the workload has it) for every linear of the workload.  Weights are quantized
and packed once, before timing (offline: the packed form is what a model
stores); that pass is timed separately (``offline_weight_quant_ms``).

Default line: the whole decode step of the 2B-shape model at M = 1 -- 30
layers of QKV 2560->3840, O 2560->2560, gate+up 2560->13824 and down
6912->2560, 120 linears, 521 MB of packed weights -- run as one grouped
forward per step ("µs/token for all linears").  Two weight sets alternate, so
no step finds its weights in the 256 MB Infinity Cache.  The same JSON line
carries keyed sub-records (``sub``) for the decode GEMV pair (M = 1, up ->
ReLU^2 -> down, 61 rotating weight copies), the 2B step at M = 4 and 16, and
the prefill GEMMs at M = 2048 (int8 TOPS), the 2B step at M = 1 with its
weights in the base-3 layout (five codes per byte), the 7B-like step (32
layers, 128 linears) at M = 1, 64 and 512 (int8 TOPS at 512), and the decode
pair by table lookup instead of multiplies.

Timing: W warm-up steps, then exactly K steps, each as one HIP graph replay
on torch's stream, bracketed by synchronizations; HIP events around the
timed replay give ``ms_per_step``, the host clock gives the wall time
(reported beside it).  Weight copies are indexed from the warm-up's end, so
the timed steps read copies the warm-up did not.  The ``roofline`` object is
that of the dominant kernel: for the default line the grouped decode kernel
(one launch per step, so its average launch time is the event time of the
timed region divided by K).  ``cpu_baseline`` is the CPU oracle timed on a
bounded sample of the same workload on this host, with all the host's
threads and with one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
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
LUT_SOURCES = ["lut.hip", "gemv_tile.hpp", "common.hpp"]
GROUP_SOURCES = ["group.hip", "group.hpp", "gemv_tile.hpp", "quant_row.hpp", "common.hpp"]
# Up to this many tokens the grouped decode quantizes inside its one launch;
# above, a quantization launch precedes it.
GROUP_INLINE_MAX_M = 3


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="decode_step_2b")
    p.add_argument("--tokens", type=int, default=None, help="M for multi-M workloads")
    mode = p.add_mutually_exclusive_group()
    mode.add_argument("--grouped", dest="grouped", action="store_true", default=None,
                      help="run all linears of a step as one grouped forward (the default "
                           "for the multi-layer decode steps)")
    mode.add_argument("--per-linear", dest="grouped", action="store_false",
                      help="one forward call per linear")
    p.add_argument("--no-sub", action="store_true",
                   help="only the main line: skip the keyed sub-records")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="time budget of each CPU oracle sample")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--kernel-launches", type=int, default=400,
                   help="launches of the dominant kernel timed for a per-linear roofline")
    p.add_argument("--glu", action="store_true",
                   help="gated FFN: pack each gate+up linear (N = 2 x the down projection's K) "
                        "for the gated squared-ReLU epilogue (output N/2)")
    p.add_argument("--lut", action="store_true",
                   help="one-token linears by table lookup (bitlinear_forward_lut; per linear)")
    p.add_argument("--b3", action="store_true",
                   help="weights in the base-3 layout (five codes per byte; grouped, M <= 16)")
    p.add_argument("--subln", action="store_true",
                   help="give every linear a subln gain (RMSNorm fused into its quantization)")
    p.add_argument("--probes", action="store_true",
                   help="only run the context probes: streaming-read bandwidth (1 GiB, a "
                        "2B decode step's 521 MB, one 4.4 MB GEMV's worth) and the int8 "
                        "matrix-core rate (both MFMA shapes)")
    p.add_argument("--copy-probe", action="store_true",
                   help="only time a plain 1 GiB device-to-device copy (achievable HBM "
                        "bandwidth, and the known-size kernel for counter calibration)")
    return p.parse_args()


# ---------------------------------------------------------------------------
# Workloads: allocate everything up front; step(i) only launches.
# ---------------------------------------------------------------------------
def weight_copies(packed_bytes_per_step):
    """Weight sets to rotate: enough that the bytes between two reads of one
    set exceed twice the Infinity Cache (at least two sets)."""
    return int(min(64, max(2, -(-2 * MALL_BYTES // packed_bytes_per_step))))


class Linear:
    """One linear of a step: `copies` packed weight sets, its activations
    (the workload's distribution), its output and workspace."""

    def __init__(self, bl, torch, wl, dev, wk, layer, li, shape, M, copies, subln=False,
                 glu=False, fmt=None):
        self.N, self.K, self.M = shape.N, shape.K, M
        self.epi = "relu2_glu" if glu else None
        self.packed_bytes = (bl.packed_bytes_b3(self.N, self.K) if fmt == "b3"
                             else self.N * self.K // 4)
        self.packed, self.gamma = [], []
        t0 = time.perf_counter()
        for c in range(copies):
            # copy 0 uses the seed the parity tests use; the others differ
            seed = wl.weight_seed(wk.key, layer, li) + 100003 * c
            W = wl.gen_weight_device(seed, self.N, self.K, wk.weight_sparse_frac, dev)
            if fmt == "b3":
                p, g = bl.quantize_weights_b3(W, glu=glu)
            else:
                p, g = bl.quantize_weights(W, glu=glu)
            self.packed.append(p)
            self.gamma.append(g)
            del W
        torch.cuda.synchronize()
        self.quant_s = time.perf_counter() - t0
        self.seed_x = wl.act_seed(wk.key, layer, li)
        self.X = make_acts(torch, wl, self.seed_x, M, self.K, wk.x_kind, dev)
        self.Y = torch.empty((M, self.N // 2 if glu else self.N), dtype=torch.float32,
                             device=dev)
        self.gain = None
        if subln:  # gains uniform on [0.5, 1.5)
            self.gain = torch.from_numpy(wl.gen_gain(self.seed_x + 1, self.K)).to(dev)
        ws = bl.workspace_bytes(M, self.K, self.N)
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev) if ws > 0 else None

    def bytes(self):
        """Algorithmic bytes of one forward: packed W (in its layout) + X in +
        Y out + gamma (+ the subln gain)."""
        return (self.packed_bytes + self.X.numel() * self.X.element_size()
                + self.Y.numel() * 4 + 4 + (self.K * 4 if self.gain is not None else 0))

    def ops(self):
        return 2 * self.M * self.N * self.K


def make_acts(torch, wl, seed, M, K, x_kind, dev):
    """Activations of the workload's kind (bf16 as torch.bfloat16)."""
    X, is_bf16 = wl.gen_acts(seed, M, K, x_kind)
    t = torch.from_numpy(X).to(dev)
    return t.view(torch.bfloat16) if is_bf16 else t


class Runner:
    """A workload at M tokens: its linears and a step function."""

    def __init__(self, bl, torch, wl, dev, key, M, grouped, copies=None, subln=False,
                 glu=False, share_weights=None, fmt=None, lut=False):
        wk = wl.WORKLOADS[key]
        self.wk, self.M, self.fmt, self.lut = wk, M, fmt, lut
        if lut and (grouped or M != 1 or subln):
            raise SystemExit("the lookup-table GEMV runs one linear per launch at M = 1")
        if fmt == "b3" and (not grouped or M > 16):
            raise SystemExit("base-3 weights run in the grouped decode forward (M <= 16)")
        self.copies = copies or weight_copies(wk.weights_per_step // 4)
        downs_k = {l.K for l in wk.linears}
        self.lins = []
        for idx, (layer, li, shape) in enumerate(wl.step_linears(wk)):
            g = bool(glu) and shape.N % 2 == 0 and shape.N // 2 in downs_k and \
                shape.N // 2 != shape.K
            if share_weights is not None:
                lin = Linear.__new__(Linear)
                src = share_weights.lins[idx]
                lin.N, lin.K, lin.M, lin.epi = src.N, src.K, M, src.epi
                lin.packed_bytes = src.packed_bytes
                lin.packed, lin.gamma, lin.quant_s = src.packed, src.gamma, 0.0
                lin.seed_x = src.seed_x + 100 * M
                lin.X = make_acts(torch, wl, lin.seed_x, M, lin.K, wk.x_kind, dev)
                lin.Y = torch.empty((M, src.Y.shape[1]), dtype=torch.float32, device=dev)
                lin.gain = None
                if src.gain is not None:
                    lin.gain = src.gain
                ws = bl.workspace_bytes(M, lin.K, lin.N)
                lin.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device=dev) if ws > 0 else None
            else:
                lin = Linear(bl, torch, wl, dev, wk, layer, li, shape, M, self.copies,
                             subln=subln, glu=g, fmt=fmt)
            self.lins.append(lin)
        if share_weights is not None:
            self.copies = share_weights.copies
        if wk.chain_relu2:
            up, down = self.lins  # up's float output feeds down
            down.X = up.Y
        self.groups = None
        if grouped:
            if wk.chain_relu2:
                raise SystemExit("a grouped forward needs independent linears")
            self.groups = [bl.Group([(l.X, l.packed[c], l.gamma[c], l.N, l.epi, l.Y, l.gain)
                                     for l in self.lins], fmt=fmt)
                           for c in range(self.copies)]
        self.bl = bl
        self.offset = 0  # first copy of the timed region

    def step(self, i):
        bl = self.bl
        c = (i + self.offset) % self.copies
        if self.groups is not None:
            self.groups[c].forward()
        elif self.lut:
            for lin in self.lins:  # in order, so the chain's down reads up's output
                epi = "relu2" if (self.wk.chain_relu2 and lin is self.lins[0]) else lin.epi
                bl.forward_lut(lin.X, lin.packed[c], lin.gamma[c], lin.N, epilogue=epi,
                               out=lin.Y)
        elif self.wk.chain_relu2:
            up, down = self.lins
            bl.forward(up.X, up.packed[c], up.gamma[c], up.N, epilogue="relu2", out=up.Y,
                       workspace=up.ws, norm_gain=up.gain)
            bl.forward(down.X, down.packed[c], down.gamma[c], down.N, out=down.Y,
                       workspace=down.ws, norm_gain=down.gain)
        else:
            for lin in self.lins:
                bl.forward(lin.X, lin.packed[c], lin.gamma[c], lin.N, epilogue=lin.epi,
                           out=lin.Y, workspace=lin.ws, norm_gain=lin.gain)

    def bytes_step(self):
        # In the ReLU^2 chain the hidden vector counts twice: written by the up
        # projection and read by the down projection, as on the device.
        return sum(l.bytes() for l in self.lins)

    def ops_step(self):
        return sum(l.ops() for l in self.lins)

    def quant_ms(self):
        return sum(l.quant_s for l in self.lins) * 1e3 / self.copies


def capture(torch, fn, count, first=0):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(first)  # one eager pass to settle any lazy initialisation
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(first, first + count):
            fn(i)
    return g


def time_steps(torch, runner, steps, warmup):
    """W warm-up steps (copies 0..W-1), then exactly K timed steps (copies
    from W on) as one graph replay between synchronizations.  Returns
    (event ms per step, wall ms per step)."""
    runner.offset = 0
    if warmup > 0:
        gw = capture(torch, runner.step, warmup)
        gw.replay()
        torch.cuda.synchronize()
        del gw
    runner.offset = warmup
    g = capture(torch, runner.step, steps)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / steps, wall * 1e3 / steps


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


def hbm_roof(bytes_, us, key, src):
    achieved = bytes_ / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile(source_hash(src), key), "kernel": key,
            "kernel_us": round(us, 3)}


def mfma_roof(ops, us, key, src):
    achieved = ops / (us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 3), "peak": INT8_PEAK_TOPS,
            "unit": "TFLOP/s", "frac": round(achieved / INT8_PEAK_TOPS, 4),
            "traffic": traffic_from_profile(source_hash(src), key), "kernel": key,
            "kernel_us": round(us, 3)}


def roofline_single(args, torch, bl, runner, metric_kind):
    """The linear with the most packed bytes, launched alone back to back
    (rotating its weight copies) in a graph bracketed by HIP events.  For the
    MFMA-bound case, the GEMM launch alone (activations quantized
    beforehand)."""
    wk, lins, M = runner.wk, runner.lins, runner.M
    dom = max(lins, key=lambda l: l.N * l.K)
    epi = "relu2" if (wk.chain_relu2 and dom is lins[0]) else dom.epi
    copies = len(dom.packed)
    gemm = metric_kind == "tops" and dom.ws is not None
    if gemm:
        Xq, sx, rs = bl.quantize_acts(dom.X, norm_gain=dom.gain)
        qws = bl.forward_q_workspace(dom.M, dom.K, dom.N, dom.X.device)

    def dom_step(i):
        c = i % copies
        if gemm:
            bl.forward_q(Xq, sx, rs, dom.packed[c], dom.gamma[c], dom.N, epilogue=epi,
                         out=dom.Y, workspace=qws)
        elif runner.lut:
            bl.forward_lut(dom.X, dom.packed[c], dom.gamma[c], dom.N, epilogue=epi, out=dom.Y)
        else:
            bl.forward(dom.X, dom.packed[c], dom.gamma[c], dom.N, epilogue=epi, out=dom.Y,
                       workspace=dom.ws, norm_gain=dom.gain)

    us = time_graph(torch, dom_step, args.kernel_launches)
    if metric_kind == "tops":
        roof = mfma_roof(dom.ops(), us, f"gemm_q_{dom.K}x{dom.N}_m{M}", GEMM_SOURCES)
        roof["launches_timed"] = "gemm only (forward_q)"
    elif runner.lut:
        roof = hbm_roof(dom.bytes(), us, f"lut_gemv_{dom.K}x{dom.N}_m{M}", LUT_SOURCES)
        roof["launches_timed"] = "one fused launch (lookup tables)"
    else:
        roof = hbm_roof(dom.bytes(), us, f"gemv_{dom.K}x{dom.N}_m{M}", GEMV_SOURCES)
        roof["launches_timed"] = "one fused launch" if dom.ws is None else \
            "quantization + gemm"
    log(f"dominant forward {roof['kernel']}: {us:.3f} us per call")
    return roof


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded samples, all threads and one)
# ---------------------------------------------------------------------------
def host_description():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    threads = affinity
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        threads = min(threads, int(env))  # the host share this process may use
    return model, affinity, threads


def cpu_sample(orc, wl, wk, Ms, budget_s, subln, seed0=424242):
    """One layer's linears of the workload at Ms token rows, on the oracle
    (weights quantized by the oracle itself).  Returns (pass_fn, bytes, ops)."""
    prepared = []
    for li, lin in enumerate(wk.linears):
        W = wl.gen_weight(seed0 + li, lin.N, lin.K, wk.weight_sparse_frac)
        _, gc = orc.absmean(W)
        qw = orc.ternarize(W, gc)
        del W
        X, is_bf16 = wl.gen_acts(seed0 + 100 + li, Ms, lin.K, wk.x_kind)
        g = wl.gen_gain(seed0 + 200 + li, lin.K) if subln else None
        prepared.append((lin, qw, gc, X, is_bf16, g))

    def fwd(X, qw, gc, bf16, g):
        if g is None:
            return orc.forward(X, qw, gc, bf16=bf16)[0]
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

    nbytes = sum(lin.N * lin.K // 4 + Ms * lin.K * (2 if is_bf16 else 4) + Ms * lin.N * 4 + 4
                 + (lin.K * 4 if subln else 0) for lin, _, _, _, is_bf16, _ in prepared)
    if wk.chain_relu2:  # h written and read, as on the device
        nbytes = sum(lin.N * lin.K // 4 + 4 for lin, *_ in prepared) + \
            Ms * prepared[0][0].K * 2 + 2 * Ms * prepared[0][0].N * 4 + Ms * prepared[1][0].N * 4
    ops = sum(2 * Ms * lin.N * lin.K for lin, *_ in prepared)
    return one_pass, nbytes, ops


def time_cpu(one_pass, budget_s):
    one_pass()
    n, t0 = 0, time.perf_counter()
    while True:
        one_pass()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 100000:
            return el / n, n, el


def cpu_baseline(wl, wk, M, metric_kind, budget_s, subln=False):
    """The oracle as it stands on this host: all the threads this process may
    use, then one thread.  Decode: one layer's linears at M; prefill (TOPS):
    the full M with all threads, a 128-row sample with one thread."""
    import oracle

    orc = oracle.get()
    model, affinity, threads = host_description()
    out = {"kind": "oracle", "cpu_model": model, "host_cpus_in_affinity": affinity}
    layers = wk.layers
    runs = []
    for nthreads in (threads, 1):
        Ms = M if (metric_kind != "tops" or nthreads > 1) else min(M, 128)
        orc.set_threads(nthreads)
        one_pass, nbytes, ops = cpu_sample(orc, wl, wk, Ms, budget_s, subln)
        per, n, el = time_cpu(one_pass, budget_s)
        if metric_kind == "tops":
            value, unit = ops / per / 1e12, "TOPS"
        else:
            value, unit = nbytes / per / 1e9, "GB/s"
        rec = {"value": round(value, 4), "unit": unit, "cores": nthreads,
               "sample": (f"{n} passes over one layer's linears "
                          f"({', '.join(f'{l.K}->{l.N}' for l in wk.linears)}) at M={Ms}, "
                          f"{el:.1f} s; oracle on unpacked int8 weights"
                          + (", OpenMP over outputs" if nthreads > 1 else "")),
               "us_per_layer_pass": round(per * 1e6, 1)}
        if metric_kind != "tops":
            rec["us_per_token_all_linears"] = round(per * 1e6 * layers / Ms, 1)
        runs.append(rec)
    orc.set_threads(threads)
    out.update(runs[0])
    out["one_thread"] = runs[1]
    return out


# ---------------------------------------------------------------------------
# Counter summaries, probes
# ---------------------------------------------------------------------------
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
    """Hash of a kernel's sources with comments and blank space removed, so
    that a counter record stays valid across edits that leave the code as
    it was."""
    h = hashlib.sha1()
    for n in names:
        with open(os.path.join(ROOT, "w1_a8_matmul_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(" ".join(text.split()).encode())
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
    for fn_name in ("probe_stream_read", "probe_stream_read_nt"):
        getattr(L, fn_name).argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_void_p]
    L.probe_mfma_i8.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    st = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731
    out = {"probe": "context", "compute_units": cus}

    # streaming read: sizes x buffer copies (copies rotate so that the small
    # sizes stream from HBM rather than the 256 MB Infinity Cache, and the
    # 521 MB read alternates two buffers as the decode bench does), with the
    # default and the non-temporal load policy
    for label, nbytes, copies, read in (
            ("1GiB", 1 << 30, 1, L.probe_stream_read),
            ("2b_step_521MB", 521011200, 1, L.probe_stream_read),
            ("2b_step_521MB_2buf_nt", 521011200, 2, L.probe_stream_read_nt),
            ("gemv_4.4MB", 4423680, 61, L.probe_stream_read),
            ("gemv_4.4MB_nt", 4423680, 61, L.probe_stream_read_nt)):
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(copies)]
        best = None
        for wg_per_cu in (2, 3, 4, 8):
            grid = wg_per_cu * cus

            def fn(i):
                b = bufs[i % copies]
                rc = read(b.data_ptr(), nbytes, sink.data_ptr(), grid, st())
                assert rc == 0, rc

            us = time_graph(torch, fn, 4 if copies == 1 else (40 if copies == 2 else 200))
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


# ---------------------------------------------------------------------------
# Records
# ---------------------------------------------------------------------------
def ffn_record(torch, bl, wl, dev, launches):
    """The 2B model's gated FFN for one token (layer 0's gate+up and down
    weights of the 2B step): gate+up 2560 -> 13824 (fused,
    gated ReLU^2) then down 6912 -> 2560, three ways -- two plain forwards (the
    down launch quantizes h itself); forward_glu_quant (h quantized by the
    gate+up launch's last workgroup) then forward_q from the codes; and
    ffn_chain (both projections in one launch).  Weight
    sets rotate past the Infinity Cache; graph-timed, HIP events."""
    K, N, Kd, Nd = 2560, 13824, 6912, 2560
    copies = weight_copies(N * K // 4 + Nd * Kd // 4)
    gu, dn = [], []
    for c in range(copies):
        W = wl.gen_weight_device(wl.weight_seed("decode_step_2b", 0, 2) + 100003 * c, N, K, 0.0, dev)
        gu.append(bl.quantize_weights(W, glu=True))
        W = wl.gen_weight_device(wl.weight_seed("decode_step_2b", 0, 3) + 100003 * c, Nd, Kd, 0.0, dev)
        dn.append(bl.quantize_weights(W))
        del W
    X = make_acts(torch, wl, wl.act_seed("decode_step_2b", 0, 2), 1, K, "normal_bf16", dev)
    H = torch.empty((1, N // 2), dtype=torch.float32, device=dev)
    Y = torch.empty((1, Nd), dtype=torch.float32, device=dev)
    ws = bl.forward_glu_quant_workspace(dev)
    wc = bl.ffn_chain_workspace(N, dev)

    def plain(i):
        c = i % copies
        bl.forward(X, gu[c][0], gu[c][1], N, epilogue="relu2_glu", out=H)
        bl.forward(H, dn[c][0], dn[c][1], Nd, out=Y)

    def fused(i):
        c = i % copies
        _, hq, hs, hr = bl.forward_glu_quant(X, gu[c][0], gu[c][1], N, workspace=ws, out=H)
        bl.forward_q(hq, hs, hr, dn[c][0], dn[c][1], Nd, out=Y, split_remainder=False)

    def chain(i):
        c = i % copies
        bl.ffn_chain(X, gu[c][0], gu[c][1], N, dn[c][0], dn[c][1], Nd, glu=True, workspace=wc,
                     H=H, out=Y)

    t_plain = time_graph(torch, plain, max(launches, copies))
    t_fused = time_graph(torch, fused, max(launches, copies))
    t_chain = time_graph(torch, chain, max(launches, copies))
    return {"us_two_forwards": round(t_plain, 3), "us_glu_quant_then_forward_q": round(t_fused, 3),
            "us_one_launch_chain": round(t_chain, 3),
            "weight_copies_rotated": copies, "tokens": 1,
            "note": "gate+up 2560->13824 with the gated ReLU^2, down 6912->2560"}


def step_record(runner, ev_ms, wall_ms, metric_kind):
    """Throughput of one workload line from its per-step event time."""
    bytes_step, ops_step = runner.bytes_step(), runner.ops_step()
    step_s = ev_ms / 1e3
    if metric_kind == "tops":
        value, unit = ops_step / step_s / 1e12, "TOPS"
    else:
        value, unit = bytes_step / step_s / 1e9, "GB/s"
    return {"value": round(value, 3), "unit": unit, "ms_per_step": round(ev_ms, 6),
            "wall_ms_per_step": round(wall_ms, 6), "us_per_step": round(ev_ms * 1e3, 3),
            "us_per_token": round(ev_ms * 1e3 / runner.M, 3), "bytes_per_step": bytes_step,
            "ops_per_step": ops_step, "linears_per_step": len(runner.lins),
            "weight_copies_rotated": runner.copies,
            "frac_of_hbm_peak" if metric_kind != "tops" else "frac_of_int8_peak":
                round(value / (HBM_PEAK_GBS if metric_kind != "tops" else INT8_PEAK_TOPS), 4)}


def sub_records(args, torch, bl, wl, dev, main_runner):
    """Keyed sub-records: decode GEMV pair; the 2B step at M = 4 and 16 (on the
    main line's weights when it is the 2B step); the 7B-like step at M = 1, 64
    and 512; prefill GEMMs at M = 2048."""
    subs = {}
    steps, warmup = max(20, args.steps // 2), max(5, args.warmup // 2)

    # decode GEMV pair, M = 1 (two launches: up with ReLU^2, then down)
    r = Runner(bl, torch, wl, dev, "decode_gemv_pair_m1", 1, grouped=False, copies=61)
    ev, wall = time_steps(torch, r, max(steps, 61), warmup)
    rec = step_record(r, ev, wall, "hbm")
    rec["roofline"] = roofline_single(args, torch, bl, r, "hbm")
    rec["launches_per_step"] = 2
    subs["decode_gemv_pair_m1"] = rec
    del r

    # the same pair in one launch (bitlinear_ffn_chain)
    r = Runner(bl, torch, wl, dev, "decode_gemv_pair_m1", 1, grouped=False, copies=61)
    up, down = r.lins
    wc = bl.ffn_chain_workspace(up.N, dev)

    def chain_step(i):
        c = i % r.copies
        bl.ffn_chain(up.X, up.packed[c], up.gamma[c], up.N, down.packed[c], down.gamma[c],
                     down.N, workspace=wc, H=up.Y, out=down.Y)

    us = time_graph(torch, chain_step, max(steps, 61))
    subs["decode_gemv_pair_m1_chain"] = {"us_per_step": round(us, 3),
                                         "value": round(r.bytes_step() / (us * 1e-6) / 1e9, 3),
                                         "unit": "GB/s", "launches_per_step": 1,
                                         "weight_copies_rotated": r.copies}
    log(f"decode pair in one launch: {us:.3f} us")
    del r

    # the same pair by table lookup (bitlinear_forward_lut)
    r = Runner(bl, torch, wl, dev, "decode_gemv_pair_m1", 1, grouped=False, copies=61, lut=True)
    ev, wall = time_steps(torch, r, max(steps, 61), warmup)
    rec = step_record(r, ev, wall, "hbm")
    rec["roofline"] = roofline_single(args, torch, bl, r, "hbm")
    rec["launches_per_step"] = 2
    subs["decode_gemv_pair_m1_lut"] = rec
    log(f"decode pair by table lookup: {rec['us_per_step']} us")
    del r

    # the 2B gated FFN at one token, with and without the fused quantization of h
    subs["decode_ffn_2b_m1"] = ffn_record(torch, bl, wl, dev, max(steps, 61))
    log(f"gated FFN, one token: {subs['decode_ffn_2b_m1']}")
    torch.cuda.empty_cache()

    # 2B step at M = 4 and 16, grouped
    share = main_runner if (main_runner.wk.key == "decode_step_2b" and
                            main_runner.groups is not None and
                            main_runner.fmt is None) else None
    for M in (4, 16):
        r = Runner(bl, torch, wl, dev, "decode_step_2b", M, grouped=True, share_weights=share)
        ev, wall = time_steps(torch, r, steps, warmup)
        rec = step_record(r, ev, wall, "hbm")
        rec["launches_per_step"] = 1 if M <= GROUP_INLINE_MAX_M else 2
        subs[f"decode_step_2b_m{M}"] = rec
        del r
    torch.cuda.empty_cache()

    # 2B step at M = 1 with the weights in the base-3 layout (five codes per
    # byte, 418.8 MB instead of 521.0 MB); GB/s counts the bytes it reads
    if main_runner.fmt is None:
        r = Runner(bl, torch, wl, dev, "decode_step_2b", 1, grouped=True, fmt="b3")
        ev, wall = time_steps(torch, r, steps, warmup)
        rec = step_record(r, ev, wall, "hbm")
        rec["weight_format"] = "b3"
        rec["launches_per_step"] = 1
        subs["decode_step_2b_m1_b3"] = rec
        log(f"2B step M=1, base-3 weights: {rec['us_per_step']} us, {rec['value']} GB/s")
        del r
        torch.cuda.empty_cache()

    # the 7B-like step (32 layers, 128 linears, 1.62 GB packed) at M = 1, 64
    # and 512 on one weight set pair, grouped; M = 512 in int8 TOPS
    r7 = Runner(bl, torch, wl, dev, "decode_prefill_7b", 1, grouped=True)
    for M in (1, 64, 512):
        r = r7 if M == 1 else Runner(bl, torch, wl, dev, "decode_prefill_7b", M, grouped=True,
                                     share_weights=r7)
        kind = "tops" if M >= 128 else "hbm"
        ev, wall = time_steps(torch, r, steps, warmup)
        rec = step_record(r, ev, wall, kind)
        rec["launches_per_step"] = 1 if M <= GROUP_INLINE_MAX_M else 2
        subs[f"decode_prefill_7b_m{M}"] = rec
        log(f"7B step M={M}: {rec['us_per_step']} us, {rec['value']} {rec['unit']}")
        if r is not r7:
            del r
    del r7
    torch.cuda.empty_cache()

    # prefill, M = 2048: the whole step (two quantizations + two GEMMs) and each
    # GEMM launch alone
    r = Runner(bl, torch, wl, dev, "prefill_m2048", 2048, grouped=False, copies=2)
    ev, wall = time_steps(torch, r, steps, warmup)
    rec = step_record(r, ev, wall, "tops")
    for lin in r.lins:
        Xq, sx, rs = bl.quantize_acts(lin.X)
        qws = bl.forward_q_workspace(lin.M, lin.K, lin.N, dev)

        def one(i, lin=lin, Xq=Xq, sx=sx, rs=rs, qws=qws):
            c = i % len(lin.packed)
            bl.forward_q(Xq, sx, rs, lin.packed[c], lin.gamma[c], lin.N, out=lin.Y,
                         workspace=qws)

        us = time_graph(torch, one, 100)
        rec[f"gemm_{lin.K}x{lin.N}"] = mfma_roof(lin.ops(), us, f"gemm_q_{lin.K}x{lin.N}_m2048",
                                                 GEMM_SOURCES)
    subs["prefill_m2048"] = rec
    if not args.no_cpu:
        cpu = cpu_baseline(wl, r.wk, 2048, "tops", args.cpu_seconds / 2)
        rec["cpu_baseline"] = cpu
        log(f"cpu oracle (prefill): {cpu}")
    del r
    torch.cuda.empty_cache()
    return subs


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

    wk = wl.WORKLOADS[args.workload]
    M = args.tokens if args.tokens is not None else wk.tokens[0]
    if M not in wk.tokens:
        log(f"note: M={M} is not one of the workload's token counts {wk.tokens}")
    grouped = args.grouped
    if grouped is None:  # default: grouped for the multi-layer decode steps
        grouped = wk.layers > 1 and M <= 64 and not wk.chain_relu2
    if args.lut:
        grouped = False
    runner = Runner(bl, torch, wl, dev, args.workload, M, grouped, subln=args.subln,
                    glu=args.glu, fmt="b3" if args.b3 else None, lut=args.lut)
    log(f"workload {wk.key} M={M}: {len(runner.lins)} linears, {runner.copies} weight "
        f"copies, offline quantization {runner.quant_ms():.1f} ms per weight set")
    metric_kind = "tops" if M >= 128 else "hbm"

    ev_ms, wall_ms = time_steps(torch, runner, args.steps, args.warmup)
    log(f"timed {args.steps} steps: events {ev_ms * 1e3:.3f} us/step, wall "
        f"{wall_ms * 1e3:.3f} us/step")
    rec = step_record(runner, ev_ms, wall_ms, metric_kind)

    if runner.groups is not None:
        # The dominant kernel is the grouped kernel; up to four tokens it is
        # the step's only launch, so its average duration is the timed
        # region's event time per step.
        key = (f"group_gemm_{wk.key}_m{M}" if M > 16 else f"group_gemv_{wk.key}_m{M}")
        key += "_b3" if args.b3 else ""
        if metric_kind == "tops":
            roof = mfma_roof(runner.ops_step(), ev_ms * 1e3, key, GEMM_SOURCES)
        else:
            roof = hbm_roof(runner.bytes_step(), ev_ms * 1e3, key,
                            GEMM_SOURCES if M > 16 else GROUP_SOURCES)
        roof["launches_per_step"] = 1 if M <= GROUP_INLINE_MAX_M else 2
        if args.b3:
            roof["note"] = ("base-3 weights: the digit extraction makes the kernel VALU-bound; "
                            "the HBM fraction is kept for comparison with the 2-bit layout")
        roof["timed_over"] = (f"the timed region: {args.steps} steps, HIP events on torch's "
                              "stream" + ("" if M <= GROUP_INLINE_MAX_M else "; includes the quantization "
                                          "launch"))
    else:
        roof = roofline_single(args, torch, bl, runner, metric_kind)

    subs = None
    if not args.no_sub:
        subs = sub_records(args, torch, bl, wl, dev, runner)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, wk, M, metric_kind, args.cpu_seconds, subln=args.subln)
        log(f"cpu oracle: {cpu}")

    out = {
        "metric": METRIC,
        "value": rec["value"],
        "unit": rec["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": wk.key,
            "description": wk.description,
            "tokens": M,
            "grouped": runner.groups is not None,
            "us_per_token": rec["us_per_token"],
            "wall_ms_per_step": rec["wall_ms_per_step"],
            "linears_per_step": rec["linears_per_step"],
            "weight_copies_rotated": runner.copies,
            "bytes_per_step": rec["bytes_per_step"],
            "ops_per_step": rec["ops_per_step"],
            "offline_weight_quant_ms": round(runner.quant_ms(), 3),
            "subln": bool(args.subln),
            "glu": bool(args.glu),
            "weight_format": "b3" if args.b3 else "2bit",
            "lookup_tables": bool(args.lut),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "sub": subs,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
