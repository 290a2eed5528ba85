#!/usr/bin/env python3
"""Benchmark: batch-1 k-quant decode FFN at Gemma-3-4B shape on one MI355X.

One step = one pass of the decode hot path over one token, one qffn_decode
call, which launches:
  qffn_gate_up_act   RMS-norm(x) -> gate/up GEMV (Q4_K, 10240 x 2560 each)
                     -> GELU-tanh(gate) * up = h
  qgemv_q6k          down GEMV (Q6_K, 2560 x 10240) on h
Weights are seeded synthetic tensors with the workload's field distributions
(no checkpoint is available); they rotate through enough distinct copies
(>= 1 GiB) that neither the L2 nor the 256 MB Infinity Cache serves them.
Inputs are resident in HBM before the timed region.

Prints ONE JSON line on stdout.  `value` is weight GB/s of the whole step
(the step's launches replayed as a HIP graph); `roofline` is for the dominant
kernel (the gate/up GEMV), timed with HIP events on the stream it runs on, in
an eager pass that makes the same two launches through their own entry
points; `cpu_baseline` is the C oracle on the host cores.  Other workloads
(--workload) are for profiling and sweeps; gemma4_prefill reports TFLOP/s of
the 512-token prefill GEMMs against the bf16 MFMA peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
METRIC = "batch-1 k-quant GEMV µs and weight GB/s (% of HBM peak), Gemma-3-4B FFN"
ROTATE_BYTES = 1 << 30
FFN_WORKLOADS = ("gemma3_ffn", "gemma3_ffn_2k", "gemma4_ffn", "gemma4_ffn_2k", "gemma4_ffn_b8")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="gemma3_ffn",
                   choices=["gemma3_ffn", "gemma3_ffn_2k", "gemma4_ffn", "gemma4_ffn_2k",
                            "gemma4_ffn_b8", "gemma4_prefill", "gemma3_qkv", "gemma3_qkv_q8_0",
                            "moe_decode", "q4k_512x512",
                            "lm_head_q4k",
                            "lm_head_q8_0", "lm_head_q8_0_q8act", "down_q6k", "gate_up_q4k", "copy"])
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate CPU time budget of the oracle baseline (0 = skip)")
    p.add_argument("--seed", type=int, default=0x5EED)
    p.add_argument("--rotate-mib", type=int, default=1024,
                   help="distinct weight copies totalling at least this many MiB rotate through "
                        "the steps (0 = one copy: warm caches)")
    p.add_argument("--override", default="",
                   help="p_in,p_out,nr launch-shape override (tuning only)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_decode_q4k_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key: str, alg_bytes: float):
    """HBM bytes per launch from the committed PMC summary, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None
    e = d.get(kernel_key)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


class Workload:
    """Weights (rotating copies), activations and the per-step launches."""

    def __init__(self, name, seed, dev, rotate_bytes=ROTATE_BYTES):
        import torch
        import synth
        import quantized_decode_q4k_amd as qd
        self.qd, self.torch, self.name = qd, torch, name
        t = lambda a: torch.from_numpy(a).to(dev)
        self.batch = 1
        if name in FFN_WORKLOADS + ("gate_up_q4k", "down_q6k"):
            hidden, ff = (2560, 10240) if name in ("gemma3_ffn", "gemma3_ffn_2k", "gate_up_q4k",
                                                   "down_q6k") else (5376, 21504)
            self.batch = 8 if name == "gemma4_ffn_b8" else 1
            self.hidden, self.ff = hidden, ff
            mats = {}
            if name != "down_q6k":
                mats["gate"] = synth.quant_weights("q4_k", ff, hidden, seed, tensor_id=41)
                mats["up"] = synth.quant_weights("q4_k", ff, hidden, seed, tensor_id=42)
            if name != "gate_up_q4k":
                mats["down"] = synth.quant_weights("q6_k", hidden, ff, seed, tensor_id=45)
            self.weight_bytes = sum(m.size for m in mats.values())
            x = synth.normal((self.batch, hidden), seed, tensor_id=43)
            nw = synth.normal((hidden,), seed, tensor_id=44, mean=1.0, std=0.1)
            self.x = t(x)
            self.nw = t(nw)
            self.h = torch.empty((self.batch, ff), device=dev)
            self.hin = t(synth.normal((self.batch, ff), seed, tensor_id=46))
            self.y = torch.empty((self.batch, hidden), device=dev)
            base = {k: t(v) for k, v in mats.items()}
            self.hidden = hidden
        elif name == "gemma4_prefill":
            M, hidden, ff = 512, synth.GEMMA4_HIDDEN, synth.GEMMA4_FF
            self.M, self.hidden, self.ff = M, hidden, ff
            mats = {"gate": synth.quant_weights("q4_k", ff, hidden, seed, tensor_id=71),
                    "up": synth.quant_weights("q4_k", ff, hidden, seed, tensor_id=72),
                    "down": synth.quant_weights("q6_k", hidden, ff, seed, tensor_id=74)}
            self.weight_bytes = sum(m.size for m in mats.values())
            self.X = t(synth.normal_bf16((M, hidden), seed, tensor_id=73).view("int16"))
            self.H = torch.empty((M, ff), dtype=torch.bfloat16, device=dev)
            self.Y = torch.empty((M, hidden), device=dev)
            self.flops_gate_up = 2 * 2 * M * ff * hidden
            self.flops = self.flops_gate_up + 2 * M * hidden * ff
            base = {k: t(v) for k, v in mats.items()}
        elif name == "q4k_512x512":
            # the small parity configuration: one Q4_K GEMV, 512 rows x K = 512
            W = synth.quant_weights("q4_k", 512, 512, seed, tensor_id=1)
            self.weight_bytes = W.size
            self.x = t(synth.normal((1, 512), seed, tensor_id=2))
            self.y = torch.empty((1, 512), device=dev)
            base = {"W": t(W)}
        elif name == "moe_decode":
            # 8 of 128 experts per token, hidden 2560, expert FF 1024 (Q4_K
            # gate/up, Q6_K down); the routed ids differ from step to step,
            # so the experts a step reads rotate through all 128 (653 MB)
            self.n_exp, self.n_sel, hidden, ff = 128, 8, 2560, 1024
            self.hidden, self.ff = hidden, ff
            Wg = synth.quant_weights("q4_k", self.n_exp * ff, hidden, seed, tensor_id=101)
            Wu = synth.quant_weights("q4_k", self.n_exp * ff, hidden, seed, tensor_id=102)
            Wd = synth.quant_weights("q6_k", self.n_exp * hidden, ff, seed, tensor_id=103)
            self.moe_w = (t(Wg), t(Wu), t(Wd))
            self.weight_bytes = self.n_sel * (Wg.size + Wu.size + Wd.size) // self.n_exp
            self.x = t(synth.normal((hidden,), seed, tensor_id=104))
            self.nw = t(synth.normal((hidden,), seed, tensor_id=105, mean=1.0, std=0.1))
            self.y = torch.empty((hidden,), device=dev)
            import numpy as np
            rng = np.random.default_rng(seed)
            nsteps = 4096
            ids = np.stack([rng.choice(self.n_exp, self.n_sel, replace=False) for _ in range(nsteps)])
            coef = rng.dirichlet(np.ones(self.n_sel), size=nsteps)
            self.moe_ids = t(ids.astype(np.int32))
            self.moe_coef = t(coef.astype(np.float32))
            base = {}
        elif name in ("gemma3_qkv", "gemma3_qkv_q8_0"):
            self.qkv_fmts = ("q4_k", "q4_k", "q6_k") if name == "gemma3_qkv" else ("q8_0",) * 3
            hidden = 2560
            mats = {"q": synth.quant_weights(self.qkv_fmts[0], 2048, hidden, seed, tensor_id=61),
                    "k": synth.quant_weights(self.qkv_fmts[1], 1024, hidden, seed, tensor_id=62),
                    "v": synth.quant_weights(self.qkv_fmts[2], 1024, hidden, seed, tensor_id=63)}
            self.weight_bytes = sum(m.size for m in mats.values())
            self.x = t(synth.normal((1, hidden), seed, tensor_id=64))
            self.nw = t(synth.normal((hidden,), seed, tensor_id=65, mean=1.0, std=0.1))
            self.qkv_out = [torch.empty((1, n), device=dev) for n in (2048, 1024, 1024)]
            base = {k: t(v) for k, v in mats.items()}
        elif name in ("lm_head_q4k", "lm_head_q8_0", "lm_head_q8_0_q8act"):
            fmt = "q4_k" if name == "lm_head_q4k" else "q8_0"
            self.fmt = fmt
            W = synth.quant_weights(fmt, 262144, 2560, seed, tensor_id=10)
            self.weight_bytes = W.size
            self.x = t(synth.normal((1, 2560), seed, tensor_id=5))
            self.y = torch.empty((1, 262144), device=dev)
            if name == "lm_head_q8_0_q8act":
                self.xq = qd.qquantize_q8_act(self.x)   # the dominant-kernel timing runs the GEMV alone
            base = {"W": t(W)}
        else:  # copy: plain device copy of 512 MiB, to calibrate counters
            self.weight_bytes = 512 << 20
            base = {"src": torch.empty(self.weight_bytes // 4, device=dev).fill_(1.0)}
            self.dst = torch.empty_like(base["src"])
        ncopy = max(2, math.ceil(rotate_bytes / max(1, self.weight_bytes))) if name not in ("copy", "moe_decode") else 1
        if rotate_bytes == 0:
            ncopy = 1
        if name == "moe_decode":
            ncopy = self.moe_ids.shape[0]   # one routed id set per step
            self.copies = [base] * ncopy
            self.ncopy = ncopy
            self.i = 0
            return
        self.copies = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(ncopy - 1)]
        self.ncopy = ncopy
        self.i = 0

    def alg_bytes(self):
        """(dominant kernel name, algorithmic bytes per launch of it)."""
        b, n = self.batch, self.name
        if n == "gemma4_prefill":
            return "qgemm_prefill_gate_up_act", self.flops_gate_up
        if n in ("gemma3_ffn", "gemma4_ffn", "gemma3_ffn_2k", "gemma4_ffn_2k", "gemma4_ffn_b8",
                 "gate_up_q4k"):
            w = 2 * self.ff * (self.hidden // 256) * 144
            return "qffn_gate_up_act", w + 4 * (b * self.hidden + self.hidden + b * self.ff)
        if n == "down_q6k":
            return "qgemv_q6k", self.hidden * (self.ff // 256) * 210 + 4 * b * (self.ff + self.hidden)
        if n.startswith("gemma3_qkv"):
            return "qqkv_proj", self.weight_bytes + 4 * (2 * 2560 + 4096)
        if n == "q4k_512x512":
            return "qgemv_q4k", self.weight_bytes + 4 * (512 + 512)
        if n == "moe_decode":
            return "qmoe_ffn_decode", self.weight_bytes + 4 * (3 * self.hidden + 2 * self.n_sel * self.ff)
        if n == "lm_head_q8_0_q8act":
            return "qgemv_q8_0_preq", self.weight_bytes + 2560 + 4 * (80 + 262144)
        if n.startswith("lm_head"):
            return "qgemv", self.weight_bytes + 4 * (2560 + 262144)
        return "copy", 2 * self.weight_bytes

    def step(self):
        """One step: every launch of the workload, weights rotating."""
        c = self.copies[self.i]
        self.i = (self.i + 1) % self.ncopy
        qd, n = self.qd, self.name
        if n in ("gemma3_ffn", "gemma4_ffn", "gemma4_ffn_b8"):
            qd.qffn_decode("q4_k", c["gate"], c["up"], "q6_k", c["down"], self.x, self.nw, 1e-6,
                           "gelu_tanh", y=self.y)
        elif n == "gemma4_prefill":
            qd.qgemm_prefill_gate_up_act("q4_k", c["gate"], c["up"], self.X, "gelu_tanh", H=self.H)
            qd.qgemm_prefill("q6_k", c["down"], self.H, Y=self.Y)
        elif n in ("gemma3_ffn_2k", "gemma4_ffn_2k", "gate_up_q4k"):
            qd.qffn_gate_up_act("q4_k", c["gate"], c["up"], self.x, self.nw, 1e-6, "gelu_tanh", h=self.h)
            if n != "gate_up_q4k":
                qd.qgemv_q6k(c["down"], self.h, self.y)
        elif n == "down_q6k":
            qd.qgemv_q6k(c["down"], self.hin, self.y)
        elif n == "lm_head_q8_0_q8act":
            qd.qgemv_q8_0_q8act(c["W"], self.x, self.y)
        elif n.startswith("lm_head"):
            qd.qgemv(self.fmt, c["W"], self.x, self.y)
        elif n.startswith("gemma3_qkv"):
            self.qkv(c)
        elif n == "moe_decode":
            self.moe()
        elif n == "q4k_512x512":
            qd.qgemv_q4k(c["W"], self.x, self.y)
        else:
            self.dst.copy_(c["src"])

    def moe(self):
        j = self.i  # already advanced: the step's own routed set
        Wg, Wu, Wd = self.moe_w
        self.qd.qmoe_ffn_decode("q4_k", Wg, Wu, "q6_k", Wd, self.n_exp, self.moe_ids[j], self.moe_coef[j],
                                self.x, self.nw, 1e-6, "gelu_tanh", y=self.y)

    def qkv(self, c):
        o = self.qkv_out
        self.qd.qqkv_proj(self.qkv_fmts, c["q"], c["k"], c["v"], self.x, self.nw, 1e-6,
                          q=o[0], k=o[1], v=o[2])


def _dominant(self):
    """One launch of the workload's dominant kernel (the roofline's kernel)."""
    c = self.copies[self.i]
    self.i = (self.i + 1) % self.ncopy
    qd, n = self.qd, self.name
    if n == "gemma4_prefill":
        qd.qgemm_prefill_gate_up_act("q4_k", c["gate"], c["up"], self.X, "gelu_tanh", H=self.H)
    elif n in ("gemma3_ffn", "gemma4_ffn", "gemma3_ffn_2k", "gemma4_ffn_2k", "gemma4_ffn_b8",
               "gate_up_q4k"):
        qd.qffn_gate_up_act("q4_k", c["gate"], c["up"], self.x, self.nw, 1e-6, "gelu_tanh", h=self.h)
    elif n == "down_q6k":
        qd.qgemv_q6k(c["down"], self.hin, self.y)
    elif n == "lm_head_q8_0_q8act":
        qd.qgemv_q8_0_preq(c["W"], *self.xq, self.y)
    elif n.startswith("lm_head"):
        qd.qgemv(self.fmt, c["W"], self.x, self.y)
    elif n.startswith("gemma3_qkv"):
        self.qkv(c)
    elif n == "moe_decode":
        self.moe()
    elif n == "q4k_512x512":
        qd.qgemv_q4k(c["W"], self.x, self.y)
    else:
        self.dst.copy_(c["src"])


Workload.dominant = _dominant


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(seed, budget_s):
    """The C oracle on one FFN step of the same workload (RMS-norm, gate/up,
    GELU-tanh, down; every row), timed as the median of whole steps: on one
    thread and with rows split over the host's cores (at most 16 threads).
    About budget_s seconds in all."""
    import numpy as np
    import oracle
    import synth
    hidden, ff = 2560, 10240
    Wg = synth.quant_weights("q4_k", ff, hidden, seed, tensor_id=41)
    Wu = synth.quant_weights("q4_k", ff, hidden, seed, tensor_id=42)
    Wd = synth.quant_weights("q6_k", hidden, ff, seed, tensor_id=45)
    x = synth.normal((1, hidden), seed, tensor_id=43)
    nw = synth.normal((hidden,), seed, tensor_id=44, mean=1.0, std=0.1)
    host_cores = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = host_cores
    threads = max(1, min(16, affinity))
    wbytes = Wg.size + Wu.size + Wd.size

    def one(th):
        xn = oracle.rmsnorm(x, nw, 1e-6).astype(np.float32)
        g, _ = oracle.gemv_threaded("q4_k", Wg, xn, ff, hidden, th)
        u, _ = oracle.gemv_threaded("q4_k", Wu, xn, ff, hidden, th)
        h = (oracle.act_vec(oracle.ACT_GELU_TANH, g) * u).astype(np.float32)
        oracle.gemv_threaded("q6_k", Wd, h, hidden, ff, th)

    def timed(th, budget):
        t0 = time.perf_counter()
        one(th)                                   # untimed warm-up
        first = time.perf_counter() - t0
        reps = max(3, int(budget / max(first, 1e-3)))
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            one(th)
            ts.append(time.perf_counter() - t0)
        ts.sort()
        return ts[len(ts) // 2], reps

    t1, r1 = timed(1, 0.3 * budget_s)
    tn, rn = timed(threads, 0.7 * budget_s)
    return {"value": round(wbytes / tn / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "threads": threads, "host_cores": host_cores, "affinity_cores": affinity,
            "cpu_model": _cpu_model(),
            "ms_per_step_all": round(tn * 1e3, 3), "ms_per_step_1t": round(t1 * 1e3, 3),
            "value_1t": round(wbytes / t1 / 1e9, 4),
            "sample": f"median of {rn} full FFN steps on {threads} threads (value) and of {r1} on one "
                      f"thread, each after one untimed step: all 10240+10240+2560 rows, RMS-norm, "
                      f"GELU-tanh, fp64 accumulation; rows split over the threads"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    import quantized_decode_q4k_amd as qd
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    qd.lib()
    if args.override:
        p_in, p_out, nr = (int(v) for v in args.override.split(","))
        qd.set_launch_override(p_in, p_out, nr)

    log(f"[bench] workload={args.workload} steps={args.steps} warmup={args.warmup}")
    wl = Workload(args.workload, args.seed, dev, rotate_bytes=args.rotate_mib << 20)
    log(f"[bench] weight bytes/step={wl.weight_bytes} rotating copies={wl.ncopy}")
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()

    K = args.steps
    stream = torch.cuda.Stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            wl.step()
        stream.synchronize()
        # Timed region 1 (value, ms_per_step): the K steps captured once as a
        # HIP graph and replayed, so host launch overhead is not measured.
        graph = torch.cuda.CUDAGraph()
        wl.i = 0
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(K):
                wl.step()
        for _ in range(3):          # untimed: the first replays (clocks and weight pages warm up)
            graph.replay()
        stream.synchronize()
        start.record(stream)
        graph.replay()
        end.record(stream)
        stream.synchronize()
        total_ms = start.elapsed_time(end)
        ms_per_step = total_ms / K
        # Timed region 2 (roofline): the dominant kernel alone, launched K
        # times back to back (weights rotating as in the step) between one
        # pair of HIP events on its stream; a GPU spin first lets the host
        # queue every launch before the GPU reaches them, so the average is
        # kernel time, as a kernel trace reports it.
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        wl.i = 0
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(int(2e6 + 4e4 * K))
        ev0.record(stream)
        for _ in range(K):
            wl.dominant()
        ev1.record(stream)
        stream.synchronize()
    kern_avg = ev0.elapsed_time(ev1) / K
    kname, alg = wl.alg_bytes()
    prefill = args.workload == "gemma4_prefill"
    scale = 1e12 if prefill else 1e9                  # TFLOP/s or GB/s
    achieved = alg / (kern_avg * 1e-3) / scale
    log(f"[bench] step {ms_per_step * 1e3:.2f} us (graph replay); {kname} avg {kern_avg * 1e3:.2f} us "
        f"over {K} back-to-back launches -> {achieved:.0f} {'TFLOP/s' if prefill else 'GB/s'}")

    if prefill:
        value = wl.flops / (ms_per_step * 1e-3) / 1e12
        metric, unit, peak, bound = ("prefill TFLOP/s, Gemma-4-31B FFN, 512 tokens", "TFLOP/s",
                                     MFMA_BF16_PEAK_TFLOPS, "mfma")
    else:
        value = wl.weight_bytes / (ms_per_step * 1e-3) / 1e9
        metric = METRIC if args.workload == "gemma3_ffn" else f"weight GB/s, {args.workload}"
        unit, peak, bound = "GB/s", HBM_PEAK_GBS, "hbm"
    workloads = {
        "gemma3_ffn": "Gemma-3-4B FFN decode step, batch 1: RMS-norm + gate/up Q4_K 10240x2560 + "
                      "GELU-tanh + down Q6_K 2560x10240 (one qffn_decode call)",
        "gemma3_qkv": "Gemma-3-4B attention input projections, batch 1: RMS-norm + Q Q4_K 2048x2560, "
                      "K Q4_K 1024x2560, V Q6_K 1024x2560 (one qqkv_proj call)",
        "gemma3_qkv_q8_0": "Gemma-3-4B attention input projections in Q8_0, batch 1: RMS-norm + Q "
                           "2048x2560, K 1024x2560, V 1024x2560 (one qqkv_proj call)",
        "moe_decode": "MoE decode FFN, batch 1: 8 of 128 experts (hidden 2560, expert FF 1024; Q4_K "
                      "gate/up + GELU-tanh, Q6_K down), routed ids and weights on the device, new ids "
                      "every step (one qmoe_ffn_decode call)",
        "gemma4_prefill": "Gemma-4-31B FFN prefill, 512 tokens: gate/up Q4_K 21504x5376 + "
                          "GELU-tanh -> bf16 h, down Q6_K 5376x21504 (bf16 MFMA, fp32 accumulate)",
    }
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # arithmetic of the path: prefill bf16 MFMA with fp32 accumulation;
        # decode: exact int8 x int8 -> int32 products of quants and activation
        # digits (v_dot4 at batch 1-2, int8 MFMA from batch 3 on), block
        # scales in fp64 (Q4_K) / fp32 (Q6_K, Q8_0)
        "dtype": "bf16-mfma/f32" if prefill else ("i8-dot-i32/f64-f32" if wl.batch <= 2 else "i8-mfma-i32/f64-f32"),
        "data": "synthetic",
        "config": {
            "workload": workloads.get(args.workload, args.workload),
            "batch": wl.M if prefill else wl.batch,
            "weight_bytes_per_step": wl.weight_bytes,
            "us_per_step": round(ms_per_step * 1e3, 3),
            "rotating_weight_copies": wl.ncopy,
            "rotate_mib": args.rotate_mib,
            "timing": "value/ms_per_step: K steps in one HIP graph replay; roofline: K eager "
                      "back-to-back launches of the dominant kernel between one HIP event pair",
            "seed": args.seed,
        },
        "roofline": {
            "kernel": kname,
            "bound": bound,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": None if prefill else traffic_from_profiles(f"{args.workload}:{kname}", alg),
            ("alg_flops_per_launch" if prefill else "alg_bytes_per_launch"): alg,
            "avg_launch_us": round(kern_avg * 1e3, 3),
        },
        "context": "pages' figure: ~1670 ms/token CPU-fallback decode of Gemma-4-E2B (larql); not a target",
    }
    if not prefill:
        out["config"]["pct_hbm_peak"] = round(100 * value / HBM_PEAK_GBS, 2)
    if args.cpu_seconds > 0 and args.workload == "gemma3_ffn":
        log("[bench] cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(args.seed, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
