#!/usr/bin/env python3
"""Benchmark of the NF4 + LoRA linear layer hot path on one MI355X.

Default workload (block65b): one LLaMA-65B-shaped transformer block's seven NF4
linears (q, k, v, o 8192 -> 8192; gate, up 8192 -> 22016; down 22016 -> 8192),
LoRA rank 64 on each, s = 0.25, 2048 tokens.  One step is one pass of the whole
hot path on one batch:
  - codec: each float32 base weight quantized to NF4, its block scales
    double-quantized, and the weight dequantized to bf16;
  - forward: q, k, v, gate and up read the block input X; o reads a seeded
    stand-in for the attention output (attention itself is not a QLoRA linear);
    H = SiLU(gate) * up; down reads H;
  - backward: down from a seeded output gradient; the SiLU gate's backward; gate
    and up; o from a seeded output gradient; q, k, v from seeded stand-ins for
    attention's backward; the block input's gradient is the sum of the five dX.
All inputs are resident in HBM before timing starts.  mlp7b is the same step on
a LLaMA-7B feed-forward (gate, up 4096 -> 11008, down 11008 -> 4096, 4096 tokens,
r = 64, s = 0.25); attn_proj is one 4096 x 4096 linear (2048 tokens, r = 16, s = 2).

`value` is the algorithmic forward+backward FLOP of the linears divided by the
whole step's time (codec and glue are inside the step).  The `roofline` object
reports the dominant kernel: the fused dequant-GEMM direction (forward or dX)
with the larger total time, timed inside the timed steps with events the library
records right around one launch (each step times one linear's forward GEMM and
one linear's dX GEMM, in rotation).  Every event recorded between two kernels
holds the stream about 4.5 us, also without the system-scope fence (all events
here are created with hipEventDisableSystemFence), so per-stage times come from
a second pass of the same steps with HIP events between the stages.
`cpu_baseline` times the CPU oracle on a bounded sample of the same step.

Other workloads (not the default line): --workload codec (quantize + double
quant + dequantize of 4e9 bf16 weights), gemv (few-token forward on an
8192 x 28672 weight at 1, 4 and 16 tokens), small (1024 x 1024, 16 tokens),
merge (the r = 64 adapters of a LLaMA-65B-shaped block's seven linears merged
into bf16 weights, then merged and re-quantized to NF4), adamw (one AdamW step
on those seven adapters' 10.0 M parameters, moments in HBM, then with the
moments in pinned host memory), codebooks (NF4 / INT4 / FP4 with and without
double quantization: reconstruction MSE on 2^26 N(0, 1) and Student-t(4)
weights, and quantize + dequantize throughput per codebook), stream (the plain
HBM streaming ceilings the bandwidth-bound kernels are compared with: a pure
read, 4 bytes read per byte written and 1 read per 4 written, on 8 GiB and on
four rotating GEMV-sized 117 MiB buffers).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QLoRA linear fwd+bwd TFLOP/s & quantize/dequant GB/s, % of MI355X roofline"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.txt")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 14 for the block workloads, 20 otherwise)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 3 / 5)")
    ap.add_argument("--workload", default="block65b",
                    choices=["block65b", "mlp7b", "attn_proj", "codec", "gemv", "small", "merge", "adamw",
                             "codebooks", "stream"])
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU work for the oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy (a known-size kernel whose "
                         "FETCH_SIZE / WRITE_SIZE counters calibrate the HBM traffic figures)")
    return ap.parse_args()


def linear_flops(M, h, o, r):
    fwd = 2 * M * h * o + 2 * M * r * (h + o)
    bwd = 2 * M * h * o + 4 * M * r * (h + o)
    return fwd, bwd


def codec_bytes(n, src_bytes, out_bytes):
    nb = (n + 63) // 64
    nch = (nb + 255) // 256
    quant = n * src_bytes + (n + 1) // 2 + 4 * nb
    dq = 4 * nb + nb + 4 * nch + 4
    deq = (n + 1) // 2 + nb + 4 * nch + 4 + n * out_bytes
    return quant, dq, deq


class HipEvents:
    """hipEvent_t handles from the HIP runtime PyTorch already loaded.  The library
    records them around a kernel launch; torch.cuda.Event refuses to time events it
    did not record itself, so they are created and read here directly."""

    def __init__(self, torch):
        import ctypes
        self.ct = ctypes
        path = None
        for line in open("/proc/self/maps"):
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
        self.hip = ctypes.CDLL(path or os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.live = []

    # hipEventDisableSystemFence: the events only time kernels (read after a full
    # synchronize), so recording them skips the system-scope cache writeback and
    # invalidation (a kernel trace shows the stream held 4.5 us per event with it
    # against 5.7 us without)
    DISABLE_SYSTEM_FENCE = 0x20000000

    def create(self):
        ev = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.live.append(ev)
        return ev

    def elapsed_ms(self, a, b) -> float:
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def record(self, ev, torch):
        """Record ev on torch's current stream."""
        rc = self.hip.hipEventRecord(ev, self.ct.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def event(self, enable_timing=True):
        """A stand-in for torch.cuda.Event(enable_timing=True) built on these events."""
        return _Event(self)

    def close(self):
        for ev in self.live:
            self.hip.hipEventDestroy(ev)
        self.live = []


class _Event:
    def __init__(self, hev):
        import torch
        self.hev, self.torch, self.ev = hev, torch, hev.create()

    def record(self):
        self.hev.record(self.ev, self.torch)

    def elapsed_time(self, other) -> float:
        return self.hev.elapsed_ms(self.ev, other.ev)


def read_traffic(key: str):
    """HBM bytes per launch ("<workload>.<kernel>") from the committed rocprofv3 counter
    summary, or None when absent or when that kernel's source file changed since the
    counters were taken."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = {}
    for line in open(TRAFFIC_FILE):
        line = line.strip()
        if not line or line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        rec[k.strip()] = v.strip()
    src = rec.get(f"{key}.source")
    if src is None or f"{key}.bytes_per_launch" not in rec:
        return None
    path = os.path.join(ROOT, "bit_quantized_fine_nf4_amd", "csrc", src)
    if not os.path.exists(path):
        return None
    sha = hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]
    if rec.get(f"source.{src}") != sha:
        return None
    return round(float(rec[f"{key}.bytes_per_launch"]))


def cpu_oracle_attn_proj(wl_mod, target_s):
    """Time the oracle on the whole default workload, repeated until target_s of work."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    c = wl_mod.C2
    ls = c.linears[0]
    w = wl_mod.base_weight(c, 0).numpy().ravel()
    l1, l2 = wl_mod.lora_factors(c, 0)
    L1, L2 = l1.float().numpy(), l2.float().numpy()
    X = wl_mod.activations(c, 0).float().numpy().astype(np.float64)
    DY = wl_mod.activations(c, 0, tensor=wl_mod.TENSOR_DY).float().numpy().astype(np.float64)
    reps, t_total = 0, 0.0
    while t_total < target_s and reps < 50:
        t0 = time.perf_counter()
        p, a = oracle.quantize(w)
        q, s2, mean = oracle.double_quant(a)
        oracle.dequantize(p, q, s2, mean, w.size, out="bf16")
        wh = oracle.dequantized_weight(p, q, s2, mean, ls.h, ls.o)
        oracle.linear_fwd(wh, X, L1, L2, ls.s)
        oracle.linear_bwd(wh, X, DY, L1, L2, ls.s)
        t_total += time.perf_counter() - t0
        reps += 1
    fwd, bwd = linear_flops(c.tokens, ls.h, ls.o, ls.r)
    return {"value": round((fwd + bwd) * reps / t_total / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": f"whole workload (one full step: quantize, double quant, dequant, fp64 fwd+bwd) x {reps} "
                      f"reps, {t_total:.1f} s; codec single-threaded NumPy, fp64 GEMMs on {threads} BLAS threads",
            "s_per_step": round(t_total / reps, 4)}


def bench_attn_proj(args, torch, nf4, wl):
    dev = "cuda:0"
    c = wl.C2
    ls = c.linears[0]
    M, h, o, r, s = c.tokens, ls.h, ls.o, ls.r, ls.s
    n = h * o
    w = wl.base_weight(c, 0).to(dev)
    l1, l2 = (t.to(dev) for t in wl.lora_factors(c, 0))
    X = wl.activations(c, 0).to(dev)
    dY = wl.activations(c, 0, tensor=wl.TENSOR_DY).to(dev)
    codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
    absmax = torch.empty(n // 64, dtype=torch.float32, device=dev)
    qa = torch.empty(n // 64, dtype=torch.int8, device=dev)
    s2 = torch.empty((n // 64 + 255) // 256, dtype=torch.float32, device=dev)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    dq_ws = torch.empty(nf4.workspace_size(nf4.QLORA_OP_DOUBLE_QUANT, n // 64), dtype=torch.uint8, device=dev)
    wdeq = torch.empty(n, dtype=torch.bfloat16, device=dev)
    Y = torch.empty(M, o, dtype=torch.bfloat16, device=dev)
    T = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, h, dtype=torch.bfloat16, device=dev)
    dL1 = torch.empty(h, r, dtype=torch.float32, device=dev)
    dL2 = torch.empty(r, o, dtype=torch.float32, device=dev)
    fws = torch.empty(nf4.workspace_size(nf4.QLORA_OP_LINEAR_FWD, M, h, o, r), dtype=torch.uint8, device=dev)
    bws = torch.empty(nf4.workspace_size(nf4.QLORA_OP_LINEAR_BWD, M, h, o, r), dtype=torch.uint8, device=dev)
    W = nf4.NF4Weight(codes, qa, s2, mean, h, o)
    stages = ["quantize", "double_quant", "dequantize", "fwd", "bwd"]
    E = HipEvents(torch).event  # fence-free timing events

    def step(ev=None, kev=None, which=(True, True)):
        if kev is not None:
            nf4.qlora_set_timing_events(nf4.TIMED_GEMM_FWD, *(kev[0:2] if which[0] else (None, None)))
            nf4.qlora_set_timing_events(nf4.TIMED_GEMM_DX, *(kev[2:4] if which[1] else (None, None)))
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        nf4.qlora_quantize(w, codes, absmax)
        rec(1)
        nf4.qlora_double_quant(absmax, qa, s2, mean, dq_ws)
        rec(2)
        nf4.qlora_dequantize(codes, qa, s2, mean, n, torch.bfloat16, out=wdeq)
        rec(3)
        nf4.qlora_linear_fwd(W, X, l1, l2, s, Y, T, fws)
        rec(4)
        nf4.qlora_linear_bwd(W, X, T, dY, l1, l2, s, dX, dL1, dL2, bws)
        rec(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    hev = HipEvents(torch)
    kevs = [[hev.create() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    # Timed region: K steps; the only events in it are the pairs the library records
    # around a fused GEMM launch: the forward GEMM in even steps, the dX GEMM in odd
    # ones (every event pair holds the stream a few microseconds; with one step,
    # both).
    timed = [(i % 2 == 0, i % 2 == 1) if args.steps > 1 else (True, True) for i in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(None, kevs[i], timed[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nf4.qlora_set_timing_events(nf4.TIMED_GEMM_FWD, None, None)
    nf4.qlora_set_timing_events(nf4.TIMED_GEMM_DX, None, None)
    # Stage breakdown from a second pass: an event recorded between two kernels
    # holds the stream a few microseconds, so it stays out of the timed steps.
    evs = [[E(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()

    ms_per_step = wall * 1e3 / args.steps
    # median over the steps: a host-side hiccup in one step of this untimed pass would
    # otherwise dominate its stage
    st_ms = {k: statistics.median(e[i].elapsed_time(e[i + 1]) for e in evs) for i, k in enumerate(stages)}
    gemm_fwd_ms = statistics.mean(hev.elapsed_ms(k[0], k[1]) for k, w in zip(kevs, timed) if w[0])
    gemm_dx_ms = statistics.mean(hev.elapsed_ms(k[2], k[3]) for k, w in zip(kevs, timed) if w[1])
    hev.close()
    fwd_f, bwd_f = linear_flops(M, h, o, r)
    qb, dqb, deqb = codec_bytes(n, 4, 2)
    stages_out = {
        "quantize": {"ms": st_ms["quantize"], "GB/s": qb / st_ms["quantize"] / 1e6},
        "double_quant": {"ms": st_ms["double_quant"], "GB/s": dqb / st_ms["double_quant"] / 1e6},
        "dequantize_bf16": {"ms": st_ms["dequantize"], "GB/s": deqb / st_ms["dequantize"] / 1e6},
        "linear_fwd": {"ms": st_ms["fwd"], "TFLOP/s": fwd_f / st_ms["fwd"] / 1e9},
        "linear_bwd": {"ms": st_ms["bwd"], "TFLOP/s": bwd_f / st_ms["bwd"] / 1e9},
        "gemm_fwd_kernel": {"ms": gemm_fwd_ms, "TFLOP/s": (2 * M * h * o + 2 * M * r * o) / gemm_fwd_ms / 1e9},
        "gemm_dx_kernel": {"ms": gemm_dx_ms, "TFLOP/s": (2 * M * h * o + 2 * M * r * h) / gemm_dx_ms / 1e9},
    }
    for v in stages_out.values():
        for k in list(v):
            v[k] = round(v[k], 4)
    # 4096 x 4096 with 2048 tokens: 256x128 tiles, the forward on the four-wave kernel,
    # dX on the eight-wave one
    if gemm_dx_ms >= gemm_fwd_ms:
        dom, dom_ms, dom_flops = "nf4_gemm_kernel<256,128,true>", gemm_dx_ms, 2 * M * h * o + 2 * M * r * h
        tkey = "gemm_dx"
    else:
        dom, dom_ms, dom_flops = "nf4_gemm_wide_fwd_kernel<1>", gemm_fwd_ms, 2 * M * h * o + 2 * M * r * o
        tkey = "gemm_fwd"
    achieved = dom_flops / dom_ms / 1e9
    roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": read_traffic(f"{c.name}.{tkey}"),
                "kernel": dom, "kernel_ms": round(dom_ms, 5), "flop_per_launch": dom_flops}
    value = (fwd_f + bwd_f) / (ms_per_step * 1e-3) / 1e12
    line = {"metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": c.name, "h": h, "o": o, "tokens": M, "r": r, "s": s,
                       "step": "quantize(fp32 W) + double_quant + dequantize(bf16) + linear_fwd + linear_bwd"},
            "tokens_per_s": round(M / (ms_per_step * 1e-3), 1), "roofline": roofline, "stages": stages_out}
    return line


class BlockPlan:
    """The linears of a transformer block, what each one reads and where its output
    gradient comes from (the workload's seeded tensors, or the glue)."""

    def __init__(self, wl, c):
        self.c = c
        names = [ls.name for ls in c.linears]
        self.names = names
        self.ffn = ("gate" in names and "up" in names and "down" in names)
        self.x_readers = [i for i, n in enumerate(names) if n in ("q", "k", "v", "gate", "up")]
        self.li = {n: i for i, n in enumerate(names)}
        h0 = c.linears[self.x_readers[0]].h
        self.h_in = h0
        # seeded inputs: X for the readers of the block input, a stand-in for the
        # attention output (o), gradients from outside the block for o, down and the
        # attention backward into q, k, v
        self.stand_in_inputs = {i: wl.TENSOR_AUX for i, n in enumerate(names) if n == "o"}
        self.seeded_grads = [i for i, n in enumerate(names) if n in ("q", "k", "v", "o", "down")]

    def order_fwd(self):
        return [i for i, n in enumerate(self.names) if n != "down"] + [self.li["down"]]

    def order_bwd(self):
        first = [self.li["down"]]
        rest = [self.li["gate"], self.li["up"]] + [i for i, n in enumerate(self.names) if n in ("o", "q", "k", "v")]
        return first + rest


def block_flops(c):
    f = b = 0
    for ls in c.linears:
        fw, bw = linear_flops(c.tokens, ls.h, ls.o, ls.r)
        f += fw
        b += bw
    return f, b


def bench_block(args, torch, nf4, wl, c):
    dev = "cuda:0"
    M = c.tokens
    plan = BlockPlan(wl, c)
    L = len(c.linears)
    host_w, w32, Ws, Ls = [], [], [], []
    codec_bufs = []
    for li, ls in enumerate(c.linears):
        w = wl.base_weight(c, li)
        host_w.append(w)
        w32.append(w.to(dev))
        n = ls.h * ls.o
        nb = n // 64
        codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
        absmax = torch.empty(nb, dtype=torch.float32, device=dev)
        qa = torch.empty(nb, dtype=torch.int8, device=dev)
        s2 = torch.empty((nb + 255) // 256, dtype=torch.float32, device=dev)
        mean = torch.empty(1, dtype=torch.float32, device=dev)
        codec_bufs.append((codes, absmax, qa, s2, mean))
        Ws.append(nf4.NF4Weight(codes, qa, s2, mean, ls.h, ls.o))
        Ls.append(tuple(t.to(dev) for t in wl.lora_factors(c, li)))
    nmax = max(ls.h * ls.o for ls in c.linears)
    wdeq = torch.empty(nmax, dtype=torch.bfloat16, device=dev)
    dq_ws = torch.empty(nf4.workspace_size(nf4.QLORA_OP_DOUBLE_QUANT, nmax // 64), dtype=torch.uint8, device=dev)
    fws = torch.empty(max(nf4.workspace_size(nf4.QLORA_OP_LINEAR_FWD, M, ls.h, ls.o, ls.r) for ls in c.linears),
                      dtype=torch.uint8, device=dev)
    bws = torch.empty(max(nf4.workspace_size(nf4.QLORA_OP_LINEAR_BWD, M, ls.h, ls.o, ls.r) for ls in c.linears),
                      dtype=torch.uint8, device=dev)
    X = wl.activations(c, plan.x_readers[0]).to(dev)
    inputs, grads = {}, {}
    for li, ls in enumerate(c.linears):
        if li in plan.x_readers:
            inputs[li] = X
        elif li in plan.stand_in_inputs:
            inputs[li] = wl.activations(c, li, width=ls.h, tensor=wl.TENSOR_AUX).to(dev)
    for li in plan.seeded_grads:
        grads[li] = wl.activations(c, li, tensor=wl.TENSOR_DY).to(dev)
    gi, ui, di = plan.li["gate"], plan.li["up"], plan.li["down"]
    f_mid = c.linears[gi].o
    Hbuf = torch.empty(M, f_mid, dtype=torch.bfloat16, device=dev)
    inputs[di] = Hbuf
    Y = {li: torch.empty(M, ls.o, dtype=torch.bfloat16, device=dev) for li, ls in enumerate(c.linears)}
    T = {li: torch.empty(M, ls.r, dtype=torch.bfloat16, device=dev) for li, ls in enumerate(c.linears)}
    dXs = {li: torch.empty(M, ls.h, dtype=torch.bfloat16, device=dev) for li, ls in enumerate(c.linears)}
    dL1 = {li: torch.empty(ls.h, ls.r, dtype=torch.float32, device=dev) for li, ls in enumerate(c.linears)}
    dL2 = {li: torch.empty(ls.r, ls.o, dtype=torch.float32, device=dev) for li, ls in enumerate(c.linears)}
    dG = torch.empty(M, f_mid, dtype=torch.bfloat16, device=dev)
    dU = torch.empty(M, f_mid, dtype=torch.bfloat16, device=dev)
    grads[gi], grads[ui] = dG, dU
    dX_block = torch.empty(M, plan.h_in, dtype=torch.bfloat16, device=dev)
    E = HipEvents(torch).event  # fence-free timing events

    def step(ev=None, kev=None, timed=None):
        """One pass of the whole hot path.  ev: stage events (second pass); kev/timed:
        the GEMM launches bracketed by the library's timing hook in this step."""
        marks = []
        rec = (lambda name: (ev[len(marks)].record(), marks.append(name))) if ev is not None else (lambda name: None)

        def hook(kind, li, on):
            if kev is None or timed is None or timed[kind] != li:
                return
            slot = nf4.TIMED_GEMM_FWD if kind == 0 else nf4.TIMED_GEMM_DX
            nf4.qlora_set_timing_events(slot, *((kev[2 * kind], kev[2 * kind + 1]) if on else (None, None)))

        rec("start")
        for li, ls in enumerate(c.linears):
            codes, absmax, qa, s2, mean = codec_bufs[li]
            n = ls.h * ls.o
            nf4.qlora_quantize(w32[li], codes, absmax)
            nf4.qlora_double_quant(absmax, qa, s2, mean, dq_ws)
            nf4.qlora_dequantize(codes, qa, s2, mean, n, torch.bfloat16, out=wdeq[:n])
        rec("codec")
        for li in plan.order_fwd():
            if li == di:
                nf4.qlora_silu_gate_fwd(Y[gi], Y[ui], Hbuf)
                rec("glue_fwd")
            ls = c.linears[li]
            hook(0, li, True)
            nf4.qlora_linear_fwd(Ws[li], inputs[li], Ls[li][0], Ls[li][1], ls.s, Y[li], T[li], fws)
            hook(0, li, False)
            rec("fwd_" + ls.name)
        for li in plan.order_bwd():
            ls = c.linears[li]
            hook(1, li, True)
            nf4.qlora_linear_bwd(Ws[li], inputs[li], T[li], grads[li], Ls[li][0], Ls[li][1], ls.s, dXs[li],
                                 dL1[li], dL2[li], bws)
            hook(1, li, False)
            rec("bwd_" + ls.name)
            if li == di:
                nf4.qlora_silu_gate_bwd(Y[gi], Y[ui], dXs[di], dG, dU)
                rec("glue_bwd")
        nf4.qlora_grad_sum([dXs[li] for li in plan.x_readers], out=dX_block)
        rec("grad_sum")
        return marks

    steps, warmup = args.steps, args.warmup
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    hev = HipEvents(torch)
    kevs = [[hev.create() for _ in range(4)] for _ in range(steps)]
    # step i times linear i % L's forward GEMM and linear (i + i // L) % L's dX GEMM
    timed = [(i % L, (i + i // L) % L) for i in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(None, kevs[i], timed[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nf4.qlora_set_timing_events(nf4.TIMED_GEMM_FWD, None, None)
    nf4.qlora_set_timing_events(nf4.TIMED_GEMM_DX, None, None)
    gemm_ms = {0: {}, 1: {}}
    for k, (lf, ld) in zip(kevs, timed):
        gemm_ms[0].setdefault(lf, []).append(hev.elapsed_ms(k[0], k[1]))
        gemm_ms[1].setdefault(ld, []).append(hev.elapsed_ms(k[2], k[3]))
    hev.close()
    # stage breakdown from a second pass (events between stages stall the stream)
    nstage = 2 + 2 * L + 3
    evs = [[E(enable_timing=True) for _ in range(nstage)] for _ in range(steps)]
    torch.cuda.synchronize()
    names = None
    for i in range(steps):
        names = step(evs[i])
    torch.cuda.synchronize()
    st_ms = {}
    for j in range(1, len(names)):
        st_ms[names[j]] = statistics.median(e[j - 1].elapsed_time(e[j]) for e in evs)  # robust to one slow step

    ms_per_step = wall * 1e3 / steps
    fwd_f, bwd_f = block_flops(c)
    stages = {"codec": {"ms": st_ms["codec"]}}
    for li, ls in enumerate(c.linears):
        fw, bw = linear_flops(M, ls.h, ls.o, ls.r)
        stages["fwd_" + ls.name] = {"ms": st_ms["fwd_" + ls.name], "TFLOP/s": fw / st_ms["fwd_" + ls.name] / 1e9}
        stages["bwd_" + ls.name] = {"ms": st_ms["bwd_" + ls.name], "TFLOP/s": bw / st_ms["bwd_" + ls.name] / 1e9}
    nmid = M * f_mid
    stages["glue_fwd"] = {"ms": st_ms["glue_fwd"], "GB/s": 6 * nmid / st_ms["glue_fwd"] / 1e6}
    stages["glue_bwd"] = {"ms": st_ms["glue_bwd"], "GB/s": 10 * nmid / st_ms["glue_bwd"] / 1e6}
    nsum = M * plan.h_in
    stages["grad_sum"] = {"ms": st_ms["grad_sum"],
                          "GB/s": 2 * nsum * (len(plan.x_readers) + 1) / st_ms["grad_sum"] / 1e6}
    gem = {}
    for kind, label in ((0, "fwd"), (1, "dx")):
        # rate over the timed launches; a linear no step timed (fewer steps than
        # linears) is counted at that rate in the per-step estimate
        flop = lambda ls: 2 * M * ls.h * ls.o + 2 * M * ls.r * (ls.o if kind == 0 else ls.h)
        t_f = sum(flop(c.linears[li]) * len(v) for li, v in gemm_ms[kind].items())
        t_ms = sum(sum(v) for v in gemm_ms[kind].values())
        rate = t_f / t_ms  # FLOP per ms
        tot_ms = tot_f = 0.0
        per = {}
        for li, ls in enumerate(c.linears):
            f = flop(ls)
            v = gemm_ms[kind].get(li, [])
            ms = statistics.mean(v) if v else f / rate
            per[ls.name] = {"ms": round(ms, 5), "TFLOP/s": round(f / ms / 1e9, 2), "launches_timed": len(v)}
            tot_ms += ms
            tot_f += f
        gem[label] = {"ms_per_step": tot_ms, "flop_per_step": tot_f, "per_linear": per,
                      "timed_flop": t_f, "timed_ms": t_ms}
    for v in stages.values():
        for k in list(v):
            v[k] = round(v[k], 4)
    dom = "dx" if gem["dx"]["ms_per_step"] >= gem["fwd"]["ms_per_step"] else "fwd"
    achieved = gem[dom]["timed_flop"] / gem[dom]["timed_ms"] / 1e9
    # 256x256 tiles: both directions run the four-wave kernels
    kname = "nf4_gemm_wide_dx_kernel" if dom == "dx" else "nf4_gemm_wide_fwd_kernel"
    roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": read_traffic(f"{c.name}.gemm_{dom}"),
                "kernel": kname, "kernel_ms_mean": round(gem[dom]["ms_per_step"] / L, 5),
                "flop_per_launch_mean": gem[dom]["flop_per_step"] / L,
                "launches_per_step": L}
    value = (fwd_f + bwd_f) / (ms_per_step * 1e-3) / 1e12
    line = {"metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps,
            "warmup": warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": c.name, "linears": {ls.name: [ls.h, ls.o] for ls in c.linears},
                       "tokens": M, "r": c.linears[0].r, "s": c.linears[0].s,
                       "step": "codec (quantize fp32 W + double_quant + dequantize bf16) of every linear + block "
                               "forward (with SiLU gate) + block backward (with SiLU gate, input-gradient sum)"},
            "tokens_per_s": round(M / (ms_per_step * 1e-3), 1), "roofline": roofline,
            "gemm": {k: {"TFLOP/s": round(v["timed_flop"] / v["timed_ms"] / 1e9, 2),
                         "ms_per_step": round(v["ms_per_step"], 4), "per_linear": v["per_linear"]}
                     for k, v in gem.items()},
            "stages": stages}
    line["_cpu_sample_host"] = host_w  # consumed by the CPU baseline (removed before printing)
    return line


def cpu_oracle_block(wl, c, host_w, target_s, ns=128):
    """The oracle on a bounded sample of the block step: every linear restricted to
    its first `ns` outputs (rows [0, ns) of the [o][h] weight, columns [0, ns) of L2)
    with all tokens, so the codec and the matmuls shrink by the same factor.  The SiLU
    gate runs on the sampled gate/up columns; down reads a seeded stand-in for its
    full-width input, q/k/v/o and down take seeded output gradients and gate/up the
    glue's.  Repeated to at least target_s seconds; value = the sample's linear FLOP
    per second."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    plan = BlockPlan(wl, c)
    M = c.tokens
    f64 = lambda t: t.float().numpy().astype(np.float64)
    X = f64(wl.activations(c, plan.x_readers[0]))
    gi, ui, di = plan.li["gate"], plan.li["up"], plan.li["down"]
    per = []
    for li, ls in enumerate(c.linears):
        w = host_w[li][:ns].numpy().ravel()
        l1, l2 = wl.lora_factors(c, li)
        L1, L2 = l1.float().numpy(), l2.float().numpy()[:, :ns]
        if li in plan.x_readers:
            xin = X
        elif li == di:
            xin = f64(wl.activations(c, li, width=ls.h, tensor=wl.TENSOR_AUX))
        else:
            xin = f64(wl.activations(c, li, width=ls.h, tensor=wl.TENSOR_AUX))
        dy = f64(wl.activations(c, li, tensor=wl.TENSOR_DY))[:, :ns] if li in plan.seeded_grads else None
        per.append((ls, w, L1, L2, xin, dy))
    dH = f64(wl.activations(c, di, width=c.linears[gi].o, tensor=wl.TENSOR_DY))[:, :ns]
    reps, t_total = 0, 0.0
    while t_total < target_s and reps < 50:
        t0 = time.perf_counter()
        outs = {}
        for li, (ls, w, L1, L2, xin, dy) in enumerate(per):
            p, a = oracle.quantize(w)
            q, s2, mean = oracle.double_quant(a)
            oracle.dequantize(p, q, s2, mean, w.size, out="bf16")
            wh = oracle.dequantized_weight(p, q, s2, mean, ls.h, ns)
            outs[li] = (wh, oracle.linear_fwd(wh, xin, L1, L2, ls.s)[0])
        oracle.silu_gate_fwd(outs[gi][1], outs[ui][1])
        dG, dU = oracle.silu_gate_bwd(outs[gi][1], outs[ui][1], dH)
        dxs = []
        for li, (ls, w, L1, L2, xin, dy) in enumerate(per):
            g = dG if li == gi else (dU if li == ui else dy)
            dx, _, _ = oracle.linear_bwd(outs[li][0], xin, g, L1, L2, ls.s)
            if li in plan.x_readers:
                dxs.append(dx)
        oracle.grad_sum(dxs)
        t_total += time.perf_counter() - t0
        reps += 1
    flops = sum(sum(linear_flops(M, ls.h, ns, ls.r)) for ls in c.linears)
    return {"value": round(flops * reps / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the whole step restricted to each linear's first {ns} outputs (all {M} tokens; codec of "
                      f"{ns} weight rows per linear, fp64 forward and backward, SiLU gate on the sampled columns, "
                      f"input-gradient sum) x {reps} reps, {t_total:.1f} s; codec single-threaded NumPy, fp64 "
                      f"matmuls on {threads} BLAS threads; value = sampled linear FLOP / time",
            "s_per_sample": round(t_total / reps, 4)}


STREAM_SHAPES = [(d, b) for d in (1, 2, 4, 8) for b in (1024, 2048, 4096, 8192, 16384)]


def stream_rate(torch, nf4, rd, wr, srcs, dst, tiles, reps, shapes=STREAM_SHAPES, warmup=2):
    """Best GB/s (bytes read + written) of the stream probe over `tiles` tiles across the launch
    shapes (tiles per wave and pass, workgroups), rotating over the source buffers `srcs`; each
    shape's rate is the median of `reps` launches timed with fence-free events.
    Returns (GB/s, ms, {"depth": d, "blocks": b})."""
    E = HipEvents(torch).event
    best = None
    for depth, blocks in shapes:
        for i in range(warmup):
            nf4.qlora_stream_probe(rd, wr, srcs[i % len(srcs)], dst, tiles, depth=depth, blocks=blocks)
        torch.cuda.synchronize()
        ev = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            ev[i][0].record()
            nf4.qlora_stream_probe(rd, wr, srcs[i % len(srcs)], dst, tiles, depth=depth, blocks=blocks)
            ev[i][1].record()
        torch.cuda.synchronize()
        ms = statistics.median(a.elapsed_time(b) for a, b in ev)
        if best is None or ms < best[1]:
            best = (tiles * 1024 * (rd + wr) / ms / 1e6, ms, {"depth": depth, "blocks": blocks})
    return best


def bench_stream(args, torch, nf4, wl):
    """Plain streaming ceilings: the stream probe at the codec's byte mixes on an 8 GiB source,
    and a pure read over four rotating buffers of the GEMV weight's code size (4 x 117 MiB, more
    than the last-level cache).  Not a step of the method: the reference rate for the HBM-bound
    kernels."""
    dev = "cuda:0"
    reps = max(args.steps, 8)
    big = torch.full((1 << 31,), 0x5A5A5A5A, dtype=torch.int32, device=dev)  # 8 GiB source
    out = torch.empty(1 << 31, dtype=torch.int32, device=dev)  # 8 GiB destination
    res = {}
    for rd, wr in ((1, 0), (4, 1), (1, 4)):
        tiles = (8 << 30) // (1024 * max(rd, wr))  # the larger side spans the 8 GiB buffer
        gbs, ms, shape = stream_rate(torch, nf4, rd, wr, [big], out, tiles, reps)
        res[f"read{rd}_write{wr}_8GiB"] = {"ms": round(ms, 4), "GB/s": round(gbs, 2),
                                            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "shape": shape}
    del big, out
    c = wl.C4_GEMV
    nbytes = c.linears[0].h * c.linears[0].o // 2
    srcs = [torch.full((nbytes // 4,), 0x3C3C3C3C, dtype=torch.int32, device=dev) for _ in range(4)]
    sink = torch.empty(4, dtype=torch.int32, device=dev)
    gbs, ms, shape = stream_rate(torch, nf4, 1, 0, srcs, sink, nbytes // 1024, reps)
    res["read1_write0_gemv_codes_x4"] = {"ms": round(ms, 5), "GB/s": round(gbs, 2),
                                         "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes,
                                         "shape": shape}
    top = res["read1_write0_8GiB"]
    return {"metric": METRIC, "value": top["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": reps,
            "warmup": 2, "ms_per_step": top["ms"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "u32", "data": "synthetic",
            "config": {"workload": "stream_probe", "tile_kb_read_write": [[1, 0], [4, 1], [1, 4]],
                       "source": "8 GiB, and 4 rotating buffers of the 8192 x 28672 NF4 codes"},
            "roofline": {"bound": "hbm", "achieved": top["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": top["frac_hbm"], "traffic": None,
                         "kernel": f"stream_probe_kernel<1, 0, {top['shape']['depth']}>"},
            "stages": res}


def bench_codec(args, torch, nf4, wl):
    dev = "cuda:0"
    n = wl.C4_CODEC_N
    w = wl.codec_weights_device(n, seed=0, device=dev)
    nb = n // 64
    codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
    absmax = torch.empty(nb, dtype=torch.float32, device=dev)
    qa = torch.empty(nb, dtype=torch.int8, device=dev)
    s2 = torch.empty((nb + 255) // 256, dtype=torch.float32, device=dev)
    mean = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(nf4.workspace_size(nf4.QLORA_OP_DOUBLE_QUANT, nb), dtype=torch.uint8, device=dev)
    out = torch.empty(n, dtype=torch.bfloat16, device=dev)
    E = HipEvents(torch).event  # fence-free timing events

    def step(ev=None):
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        nf4.qlora_quantize(w, codes, absmax)
        rec(1)
        nf4.qlora_double_quant(absmax, qa, s2, mean, ws)
        rec(2)
        nf4.qlora_dequantize(codes, qa, s2, mean, n, torch.bfloat16, out=out)
        rec(3)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[E(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [statistics.mean(e[i].elapsed_time(e[i + 1]) for e in evs) for i in range(3)]
    qb, dqb, deqb = codec_bytes(n, 2, 2)
    gbs = [qb / ms[0] / 1e6, dqb / ms[1] / 1e6, deqb / ms[2] / 1e6]
    # the plain stream ceilings of the same byte mixes (after the timed steps; the probe
    # overwrites `out`): read 2n, write n/2 like quantize; read n/2, write 2n like dequantize
    ceil_q = stream_rate(torch, nf4, 4, 1, [w], out, (2 * n) // 4096, 5)[0]
    ceil_d = stream_rate(torch, nf4, 1, 4, [codes], out, (n // 2) // 1024, 5)[0]
    dom = max(range(3), key=lambda i: ms[i])
    names = ["quantize_kernel<bf16>", "double_quant", "dequantize_kernel<bf16>"]
    total_bytes = qb + dqb + deqb
    ms_step = wall * 1e3 / args.steps
    return {"metric": METRIC, "value": round(total_bytes / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "codec_4e9_bf16", "n": n, "step": "quantize(bf16) + double_quant + dequantize(bf16)"},
            "roofline": {"bound": "hbm", "achieved": round(gbs[dom], 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs[dom] / PEAK_HBM_GBS, 4), "traffic": None, "kernel": names[dom]},
            "stages": {"quantize": {"ms": round(ms[0], 4), "GB/s": round(gbs[0], 2),
                                    "frac_hbm": round(gbs[0] / PEAK_HBM_GBS, 4),
                                    "stream_ceiling_GB/s": round(ceil_q, 2),
                                    "frac_of_ceiling": round(gbs[0] / ceil_q, 4)},
                       "double_quant": {"ms": round(ms[1], 4), "GB/s": round(gbs[1], 2)},
                       "dequantize_bf16": {"ms": round(ms[2], 4), "GB/s": round(gbs[2], 2),
                                           "frac_hbm": round(gbs[2] / PEAK_HBM_GBS, 4),
                                           "stream_ceiling_GB/s": round(ceil_d, 2),
                                           "frac_of_ceiling": round(gbs[2] / ceil_d, 4)}}}


def bench_gemv(args, torch, nf4, wl):
    dev = "cuda:0"
    c = wl.C4_GEMV
    ls = c.linears[0]
    h, o = ls.h, ls.o
    copies = 4  # 4 x 121 MB > the 256 MB last-level cache: every launch streams from HBM
    w = wl.base_weight(c, 0).to(dev)
    Ws = [nf4.quantize_weight(w) for _ in range(copies)]
    del w
    res = {}
    hev = HipEvents(torch)
    for m in wl.C4_GEMV_TOKENS:
        X = wl.activations(c, 0, tokens=m).to(dev)
        Y = torch.empty(m, o, dtype=torch.bfloat16, device=dev)
        for i in range(args.warmup):
            nf4.qlora_linear_fwd(Ws[i % copies], X, None, None, 1.0, Y)
        torch.cuda.synchronize()
        reps = max(args.steps, 8)
        kev = [[hev.create(), hev.create()] for _ in range(reps)]
        for i in range(reps):
            nf4.qlora_set_timing_events(nf4.TIMED_GEMV, kev[i][0], kev[i][1])
            nf4.qlora_linear_fwd(Ws[i % copies], X, None, None, 1.0, Y)
        torch.cuda.synchronize()
        nf4.qlora_set_timing_events(nf4.TIMED_GEMV, None, None)
        ms = statistics.median(hev.elapsed_ms(k[0], k[1]) for k in kev)
        nb = h * o // 64
        bytes_ = h * o // 2 + nb + 4 * ((nb + 255) // 256) + 2 * m * h + 2 * m * o
        res[m] = {"ms": round(ms, 5), "GB/s": round(bytes_ / ms / 1e6, 2),
                  "frac_hbm": round(bytes_ / ms / 1e6 / PEAK_HBM_GBS, 4), "bytes": bytes_}
    # few-token backward dX = dY·W_hat^T (no adapter): the dX GEMV kernel timed by the library's
    # hook, and the whole call (GEMV + the partial-sum finish) by events on the stream
    bwd = {}
    E = HipEvents(torch).event  # fence-free timing events
    for m in wl.C4_GEMV_TOKENS:
        dY = wl.activations(c, 0, tokens=m, tensor=wl.TENSOR_DY).to(dev)
        dX = torch.empty(m, h, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(nf4.workspace_size(nf4.QLORA_OP_LINEAR_BWD, m, h, o, 0), dtype=torch.uint8, device=dev)
        for i in range(args.warmup):
            nf4.qlora_linear_bwd(Ws[i % copies], None, None, dY, None, None, 1.0, dX=dX, workspace=ws)
        torch.cuda.synchronize()
        reps = max(args.steps, 8)
        kev = [[hev.create(), hev.create()] for _ in range(reps)]
        tev = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            nf4.qlora_set_timing_events(nf4.TIMED_GEMM_DX, kev[i][0], kev[i][1])
            tev[i][0].record()
            nf4.qlora_linear_bwd(Ws[i % copies], None, None, dY, None, None, 1.0, dX=dX, workspace=ws)
            tev[i][1].record()
        torch.cuda.synchronize()
        nf4.qlora_set_timing_events(nf4.TIMED_GEMM_DX, None, None)
        ms = statistics.median(hev.elapsed_ms(k[0], k[1]) for k in kev)
        call_ms = statistics.median(a.elapsed_time(b) for a, b in tev)
        nb = h * o // 64
        bytes_ = h * o // 2 + nb + 4 * ((nb + 255) // 256) + 2 * m * o + 2 * m * h
        bwd[m] = {"kernel_ms": round(ms, 5), "call_ms": round(call_ms, 5), "GB/s": round(bytes_ / ms / 1e6, 2),
                  "frac_hbm": round(bytes_ / ms / 1e6 / PEAK_HBM_GBS, 4), "bytes": bytes_}
    worst = min(res, key=lambda k: res[k]["GB/s"])
    # read-only stream ceiling over the same four rotating code buffers
    sink = torch.empty(4, dtype=torch.int32, device=dev)
    ceil_r = stream_rate(torch, nf4, 1, 0, [W.codes for W in Ws], sink, Ws[0].codes.numel() // 1024,
                         max(args.steps, 8))[0]
    for v in res.values():
        v["frac_of_read_ceiling"] = round(v["GB/s"] / ceil_r, 4)
    return {"metric": METRIC, "value": res[16]["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": res[16]["ms"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": c.name, "h": h, "o": o, "tokens": list(wl.C4_GEMV_TOKENS), "weight_copies": copies},
            "roofline": {"bound": "hbm", "achieved": res[worst]["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": res[worst]["frac_hbm"], "traffic": read_traffic(f"{c.name}.gemv_m{worst}"),
                         "kernel": GEMV_KERNEL[worst]},
            "stages": {f"M={k}": v for k, v in res.items()},
            "read_stream_ceiling_GB/s": round(ceil_r, 2),
            "backward_dx": {f"M={k}": v for k, v in bwd.items()}}


# the few-token forward kernel each token count of the GEMV workload runs (K = 8192)
GEMV_KERNEL = {1: "nf4_gemv1_kernel<4>", 4: "nf4_gemv_kernel<4>", 16: "nf4_gemv_kernel<16>"}


def bench_small(args, torch, nf4, wl):
    dev = "cuda:0"
    c = wl.C1
    ls = c.linears[0]
    M, h, o, r, s = c.tokens, ls.h, ls.o, ls.r, ls.s
    W = nf4.quantize_weight(wl.base_weight(c, 0).to(dev))
    l1, l2 = (t.to(dev) for t in wl.lora_factors(c, 0))
    X = wl.activations(c, 0).to(dev)
    dY = wl.activations(c, 0, tensor=wl.TENSOR_DY).to(dev)
    Y, T = nf4.qlora_linear_fwd(W, X, l1, l2, s)
    for _ in range(args.warmup):
        nf4.qlora_linear_fwd(W, X, l1, l2, s, Y, T)
        nf4.qlora_linear_bwd(W, X, T, dY, l1, l2, s)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        nf4.qlora_linear_fwd(W, X, l1, l2, s, Y, T)
        nf4.qlora_linear_bwd(W, X, T, dY, l1, l2, s)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    fwd_f, bwd_f = linear_flops(M, h, o, r)
    return {"metric": METRIC, "value": round((fwd_f + bwd_f) / ms / 1e9, 4), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": c.name, "h": h, "o": o, "tokens": M, "r": r, "s": s, "step": "linear_fwd + linear_bwd"},
            "roofline": None}


def merge_bytes(h, o, r, out_bytes_per_weight):
    """Algorithmic HBM bytes of one merge: codes, int8 scales, second-level scales,
    the mean, both factors once, and the output."""
    n = h * o
    nb = n // 64
    return n // 2 + nb + 4 * ((nb + 255) // 256) + 4 + 2 * r * (h + o) + int(n * out_bytes_per_weight)


def bench_merge(args, torch, nf4, wl):
    dev = "cuda:0"
    c = wl.C5
    Ws, Ls, outs, reqs = [], [], [], []
    for li, ls in enumerate(c.linears):
        Ws.append(nf4.quantize_weight(wl.base_weight(c, li).to(dev)))
        Ls.append(tuple(t.to(dev) for t in wl.lora_factors(c, li)))
        outs.append(torch.empty(ls.o, ls.h, dtype=torch.bfloat16, device=dev))
        n = ls.h * ls.o
        reqs.append((torch.empty(n // 2, dtype=torch.uint8, device=dev),
                     torch.empty(n // 64, dtype=torch.float32, device=dev)))
    E = HipEvents(torch).event  # fence-free timing events
    nl = len(c.linears)

    def step(ev=None):
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        for li, ls in enumerate(c.linears):
            nf4.qlora_merge_adapter(Ws[li], Ls[li][0], Ls[li][1], ls.s, torch.bfloat16, out=outs[li])
        rec(1)
        for li, ls in enumerate(c.linears):
            nf4.qlora_merge_requantize(Ws[li], Ls[li][0], Ls[li][1], ls.s, reqs[li][0], reqs[li][1])
        rec(2)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[E(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [statistics.mean(e[i].elapsed_time(e[i + 1]) for e in evs) for i in range(2)]
    b_bf16 = sum(merge_bytes(ls.h, ls.o, ls.r, 2.0) for ls in c.linears)
    b_req = sum(merge_bytes(ls.h, ls.o, ls.r, 0.5 + 4 / 64) for ls in c.linears)
    gbs = [b_bf16 / ms[0] / 1e6, b_req / ms[1] / 1e6]
    ms_step = wall * 1e3 / args.steps
    return {"metric": METRIC, "value": round((b_bf16 + b_req) / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "merge_" + c.name, "linears": nl, "weights": sum(ls.h * ls.o for ls in c.linears),
                       "step": "merge to bf16 + merge and re-quantize, all seven linears"},
            "roofline": {"bound": "hbm", "achieved": round(gbs[0], 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs[0] / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "merge_kernel<bf16>"},
            "stages": {"merge_bf16": {"ms": round(ms[0], 4), "GB/s": round(gbs[0], 2),
                                      "frac_hbm": round(gbs[0] / PEAK_HBM_GBS, 4), "bytes": b_bf16},
                       "merge_requantize": {"ms": round(ms[1], 4), "GB/s": round(gbs[1], 2),
                                            "frac_hbm": round(gbs[1] / PEAK_HBM_GBS, 4), "bytes": b_req}}}


def bench_adamw(args, torch, nf4, wl):
    dev = "cuda:0"
    c = wl.C5
    n = sum(ls.r * (ls.h + ls.o) for ls in c.linears)  # L1 and L2 of every linear, flat
    g = torch.Generator(device=dev).manual_seed(0)
    # three independent copies of (p, g, m, v, bf16 p), 540 MB, used in turn: more than the
    # 256 MB Infinity Cache, so every step streams from HBM
    copies = [(torch.randn(n, device=dev, generator=g) * 0.01, torch.randn(n, device=dev, generator=g) * 1e-3,
               torch.zeros(n, device=dev), torch.zeros(n, device=dev),
               torch.empty(n, dtype=torch.bfloat16, device=dev)) for _ in range(3)]
    mh = torch.zeros(n, pin_memory=True)
    vh = torch.zeros(n, pin_memory=True)
    hp = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    E = HipEvents(torch).event  # fence-free timing events
    bytes_step = n * (4 * 4 + 3 * 4 + 2)  # read p, g, m, v; write p, m, v and the bf16 copy
    res = {}
    for name in ("hbm", "host_state"):
        def args_for(i):
            p, grad, m, v, pbf = copies[i % 3]
            return (p, grad, m, v, pbf) if name == "hbm" else (p, grad, mh, vh, pbf)
        for t in range(1, args.warmup + 1):
            p, grad, M, V, pbf = args_for(t)
            nf4.qlora_adamw_step(p, grad, M, V, t, param_bf16=pbf, **hp)
        torch.cuda.synchronize()
        ev = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(args.steps)]
        for i in range(args.steps):
            p, grad, M, V, pbf = args_for(i)
            ev[i][0].record()
            nf4.qlora_adamw_step(p, grad, M, V, args.warmup + 1 + i, param_bf16=pbf, **hp)
            ev[i][1].record()
        torch.cuda.synchronize()
        ms = statistics.median(a.elapsed_time(b) for a, b in ev)
        res[name] = {"ms": round(ms, 5), "GB/s": round(bytes_step / ms / 1e6, 2),
                     "frac_hbm": round(bytes_step / ms / 1e6 / PEAK_HBM_GBS, 4)}
    h = res["hbm"]
    return {"metric": METRIC, "value": h["GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": h["ms"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "adamw_" + c.name, "params": n, "state": "float32 m, v", "copies": 3,
                       "step": "one AdamW step on all seven adapters (flat), bf16 copy written"},
            "roofline": {"bound": "hbm", "achieved": h["GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": h["frac_hbm"], "traffic": None, "kernel": "adamw_kernel"},
            "stages": res}


def bench_codebooks(args, torch, nf4, wl):
    """Reconstruction-MSE study (stands in for the pages' quality-vs-bits comparison with
    synthetic weights) and per-codebook codec throughput, all on the GPU."""
    dev = "cuda:0"
    n = 1 << 26
    g = torch.Generator(device=dev).manual_seed(0)
    data = {"normal": torch.randn(n, device=dev, generator=g)}
    # Student-t(4) = N / sqrt(chi2_4 / 4)
    chi = sum(torch.randn(n, device=dev, generator=g) ** 2 for _ in range(4)) / 4
    data["student_t4"] = torch.randn(n, device=dev, generator=g) / chi.sqrt()
    del chi
    mse = {}
    for dname, w in data.items():
        w64 = w.double()
        for cname, c in nf4.CODEBOOKS.items():
            codes, absmax = nf4.qlora_quantize(w, codebook=c)
            qa, s2, mean = nf4.qlora_double_quant(absmax)
            for dq in (True, False):
                rec = (nf4.qlora_dequantize(codes, qa, s2, mean, n, torch.float32, codebook=c) if dq else
                       nf4.qlora_dequantize_nodq(codes, absmax, n, torch.float32, codebook=c))
                mse[f"{dname}/{cname}/{'dq' if dq else 'no_dq'}"] = float(((rec.double() - w64) ** 2).mean())
        del w64
    w = data["normal"].to(torch.bfloat16)
    out = torch.empty(n, dtype=torch.bfloat16, device=dev)
    E = HipEvents(torch).event  # fence-free timing events
    rates = {}
    qb, dqb, deqb = codec_bytes(n, 2, 2)
    for cname, c in nf4.CODEBOOKS.items():
        codes = torch.empty(n // 2, dtype=torch.uint8, device=dev)
        absmax = torch.empty(n // 64, dtype=torch.float32, device=dev)
        for _ in range(args.warmup):
            nf4.qlora_quantize(w, codes, absmax, codebook=c)
        qa, s2, mean = nf4.qlora_double_quant(absmax)
        torch.cuda.synchronize()
        ev = [[E(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for e in ev:
            e[0].record()
            nf4.qlora_quantize(w, codes, absmax, codebook=c)
            e[1].record()
            nf4.qlora_dequantize(codes, qa, s2, mean, n, torch.bfloat16, out=out, codebook=c)
            e[2].record()
        torch.cuda.synchronize()
        tq = statistics.median(e[0].elapsed_time(e[1]) for e in ev)
        td = statistics.median(e[1].elapsed_time(e[2]) for e in ev)
        rates[cname] = {"quantize_ms": round(tq, 4), "quantize_GB/s": round(qb / tq / 1e6, 1),
                        "dequantize_ms": round(td, 4), "dequantize_GB/s": round(deqb / td / 1e6, 1)}
    q = rates["nf4"]
    return {"metric": METRIC, "value": q["quantize_GB/s"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(q["quantize_ms"] + q["dequantize_ms"], 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": "codebooks_2e26", "n": n, "codebooks": list(nf4.CODEBOOKS),
                       "inputs": ["N(0,1)", "Student-t(4)"]},
            "roofline": {"bound": "hbm", "achieved": q["quantize_GB/s"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(q["quantize_GB/s"] / PEAK_HBM_GBS, 4), "traffic": None,
                         "kernel": "quantize_kernel<bf16> (NF4)"},
            "stages": rates, "mse": mse}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        return 1
    import bit_quantized_fine_nf4_amd as nf4
    import workloads as wl
    block = args.workload in ("block65b", "mlp7b")
    if args.steps is None:
        args.steps = 14 if block else 20
    if args.warmup is None:
        args.warmup = 3 if block else 5
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    fn = {"attn_proj": bench_attn_proj, "codec": bench_codec, "gemv": bench_gemv, "small": bench_small,
          "merge": bench_merge, "adamw": bench_adamw, "codebooks": bench_codebooks, "stream": bench_stream,
          "block65b": lambda *a: bench_block(*a, wl.C5), "mlp7b": lambda *a: bench_block(*a, wl.C3)}[args.workload]
    line = fn(args, torch, nf4, wl)
    host_w = line.pop("_cpu_sample_host", None)
    if args.no_cpu_baseline:
        line["cpu_baseline"] = None
    elif args.workload == "attn_proj":
        line["cpu_baseline"] = cpu_oracle_attn_proj(wl, args.cpu_seconds)
    elif block:
        line["cpu_baseline"] = cpu_oracle_block(wl, wl.C5 if args.workload == "block65b" else wl.C3, host_w,
                                                args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
