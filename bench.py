"""Benchmark of the PRISM memory-writing forward pass (libprism, one MI355X).

One step = the whole hot path over one batch of the 130M-LM-shaped layer
(B=8 sequences x T=2048 tokens, H=6 heads, dk=dv=128, L=4, bf16 inputs,
fp32 state): the prologue kernel (ShortConv anchor, closed-form residual
chain, write keys) followed by the chunkwise WY/UT scan kernel, i.e. the two
launches prism_fwd makes, issued through the C ABI as prism_prologue then
prism_scan on the current stream.  Inputs are synthetic, seeded and already
resident in HBM; several input copies are rotated so that the 256 MB Infinity
Cache cannot hold a step's working set from the previous step.

Prints ONE JSON line.  Per-kernel durations come from HIP events recorded on
the launch stream inside the timed region (around every fourth step's
launches).  The CPU baseline is the fp64
oracle (plain C, OpenMP over chains) on the same workload, timed on the host
cores; its outputs double as a parity check of the last timed step.

The line also carries a "decode" object: the single-token decode step
(prism_decode_step, state and convolution history carried in place) timed
on serving batches shaped like the recommendation and language-model layers,
each against its HBM roofline, and a "backward" object: prism_bwd (the
gradients of every input for an upstream dO) on the same workload, with a
"training_pair" inside it where the chunkwise backward serves the shape:
prism_fwd_ckpt then prism_bwd_ckpt, the forward keeping every chunk's start
state for the backward (and the same step through the torch.autograd
wrapper).  Both are measured after the forward pass and are not
part of "value".
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

METRIC = "PRISM fwd tokens/sec at 1 GPU (L=4) + % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
FP32_MFMA_PEAK_TFLOPS = 157.3
FP32_VALU_PEAK_TFLOPS = 157.3    # MI355X fp32 vector (packed FMA); unpacked: 256 CU x 64 lanes x 2 x 2.4 GHz = 78.6
_CSRC = "gated_delta_rule_prologue_amd/csrc/"
# Sources that determine each kernel as launched (kernel body, shared helpers,
# dispatch): a committed counter figure is only reported while they are unchanged.
KERNEL_SOURCES = {
    "prologue": [_CSRC + f for f in ("prologue.hip", "prologue_kernel.h", "prologue_bf16.hip",
                                      "prologue_f32.hip", "prologue_bf16_ext.hip",
                                      "prologue_f32_ext.hip", "common.h", "kernels.h",
                                      "prism_api.hip")],
    "scan": [_CSRC + f for f in ("chunk_scan_bf16.hip", "chunk_scan.hip", "long_seq.hip", "common.h",
                                  "kernels.h", "prism_api.hip", "mfma_bf16.h")],
    "decode": [_CSRC + f for f in ("decode.hip", "common.h", "kernels.h", "prism_api.hip")],
}
# Decode batches: (name, sequences, heads, dk, dv, L), one new token per sequence.
DECODE_BATCHES = [
    ("recsys-serving-512x8", 512, 8, 64, 64, 8),
    ("lm-130m-serving-256x6", 256, 6, 128, 128, 4),
    ("lm-130m-serving-8x6", 8, 6, 128, 128, 4),        # small batch: launch-latency bound
]


def algorithmic_work(w, n_seqs, T, esize):
    """Algorithmic HBM bytes and MFMA flops of one step.

    Per head-token (ht):
      prologue bytes = e [dk (k) + 2 (L-1) dk (u, a) + max(L-2, 0) dk (h slots read) + 1 (b) + dk (kw)]
      scan bytes     = e [3 dk (q, k, kw) + dv (v) + 2 (g, b) + dv (o)]  + S_final (fp32) per chain
      scan flops     = the chunkwise WY/UT form with C = 64 counted with dense C x C tiles:
                       10 C dk + 8 C dv + 8 dk dv + 2 C^2 / 3 per head-token (four Gram tiles
                       and the UT-transformed keys T (b gamma K), the three C x C-by-V/X products
                       and T R, K S0 and Q S0, the state update, the C x C inverse)
    """
    H, dk, dv, L = w.heads, w.dk, w.dv, w.L
    ht = T * H
    pro = esize * (dk + 2 * (L - 1) * dk + max(L - 2, 0) * dk + 1 + dk) * ht
    scan = esize * (3 * dk + dv + 2 + dv) * ht + 4 * n_seqs * H * dk * dv
    return {"prologue_bytes": pro, "scan_bytes": scan, "scan_flops": scan_flops_ht(w) * ht,
            "head_tokens": ht}


def scan_flops_ht(w):
    """Dense MFMA flops of the chunkwise scan per head-token (C = 64; see
    algorithmic_work)."""
    C, dk, dv = 64, w.dk, w.dv
    return 10 * C * dk + 8 * C * dv + 8 * dk * dv + round(2 * C * C / 3)


def source_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    s = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    if not m or not s or s.group(1) != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return float(m.group(1))


def measured_mfma(kernel, workload):
    """MFMA utilisation per launch from the committed rocprofv3 counter summary
    (profiles/<kernel>_<workload>_mfma.md): (busy fraction of all SIMD cycles,
    MFMA flops executed), or None when there is none or the kernel's sources
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_mfma.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    b = re.search(r"mfma_busy_frac:\s*([0-9.eE+-]+)", text)
    f = re.search(r"mfma_flops_per_launch:\s*([0-9.eE+-]+)", text)
    s = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    if not b or not f or not s or s.group(1) != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return float(b.group(1)), float(f.group(1))


def cpu_baseline(inp, o_gpu, s_gpu):
    """fp64 oracle on the host cores over the whole workload; also a parity check."""
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    # repeat the whole-workload pass until about 10 s of host time has been
    # measured (at most 100 passes), so the figure is not a single short run
    reps, spent = 0, 0.0
    while reps == 0 or (spent < 10.0 and reps < 100):
        t0 = time.perf_counter()
        o_ref, s_ref = oracle.fwd(inp, threads=threads)
        spent += time.perf_counter() - t0
        reps += 1
    dt = spent / reps
    o = o_gpu.float().cpu().numpy().astype(np.float64)
    s = s_gpu.cpu().numpy().astype(np.float64)
    eo = float(np.max(np.abs(o - o_ref)) / np.max(np.abs(o_ref)))
    es = float(np.max(np.abs(s - s_ref)) / np.max(np.abs(s_ref)))
    try:
        cpu = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                   if l.startswith("model name"))
    except (OSError, StopIteration):
        cpu = "unknown"
    return ({"value": inp.total_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
             "sample": f"whole workload: all {inp.n_seqs * inp.heads} (sequence, head) chains, "
                       f"{inp.total_tokens} tokens, fp64, OpenMP over chains; mean of {reps} passes",
             "seconds": dt, "passes": reps, "cpu_model": cpu},
            {"o_max_rel_err": eo, "S_max_rel_err": es, "tolerance": 1e-2,
             "checked": "last timed step, every element"})


def oracle_timed(fn, units, unit, sample, min_seconds=2.0, max_passes=50):
    """The fp64 oracle as it is, timed on the host cores beside a GPU row: fn()
    repeated until about min_seconds have been measured; units of work per call."""
    import oracle
    reps, spent = 0, 0.0
    while reps == 0 or (spent < min_seconds and reps < max_passes):
        t0 = time.perf_counter()
        fn()
        spent += time.perf_counter() - t0
        reps += 1
    dt = spent / reps
    return {"value": units / dt, "unit": unit, "cores": oracle.default_threads(), "kind": "oracle",
            "sample": f"{sample}; mean of {reps} passes", "seconds": dt, "passes": reps}


def decode_bytes(n, H, dk, dv, L, esize):
    """Algorithmic HBM bytes of one decode step over n sequences: the fp32 state
    read and written (8 dk dv per chain) plus, per chain, e [q, k (2 dk), v (dv),
    u, a (2 (L-1) dk), h slots read (max(L-2, 0) dk), g, b (2), history read and
    written (6 dk), o (dv)], plus the conv taps once per head (4 dk e)."""
    chains = n * H
    per = 8 * dk * dv + esize * (2 * dk + dv + 2 * (L - 1) * dk + max(L - 2, 0) * dk + 2 + 6 * dk + dv)
    return chains * per + H * 4 * dk * esize


_HIP = None


def _hip_runtime():
    """The HIP runtime this process already runs on (the libamdhip64 torch
    loaded, which libprism's calls resolve to as well), bound through ctypes."""
    global _HIP
    if _HIP is None:
        import ctypes
        import torch
        torch.cuda.init()
        path = next(line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line)
        h = ctypes.CDLL(path)
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        for f in (h.hipEventCreateWithFlags, h.hipEventRecord, h.hipEventElapsedTime, h.hipEventDestroy):
            f.restype = ctypes.c_int
        _HIP = h
    return _HIP


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: its
    record makes no system-scope release, so it neither writes back nor
    invalidates the caches between the launches it brackets (a default event
    does both, which lengthens the interval it closes and slows the launch
    after it).  Same use as TimingEvent(): record on
    the launch stream, synchronize, then elapsed_time in ms."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self._h = _hip_runtime()
        self._e = ctypes.c_void_p()
        st = self._h.hipEventCreateWithFlags(ctypes.byref(self._e), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self, stream):
        st = self._h.hipEventRecord(self._e, ctypes_stream(stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        st = self._h.hipEventElapsedTime(ctypes.byref(ms), self._e, end._e)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        if getattr(self, "_e", None) is not None and self._e.value:
            self._h.hipEventDestroy(self._e)


def ctypes_stream(stream):
    """A torch stream (or None: the current one) as the hipStream_t value."""
    import torch
    return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream


def raw_args(*xs):
    """Arguments of one C-ABI call, marshalled once: tensors as device pointers.
    A timed loop of short kernels calls the library with these directly, so
    that the binding's per-call shape checks (tens of microseconds of Python)
    do not leave the GPU idle between the events around each launch; every
    loop is preceded by a checked call through the binding with the same
    tensors."""
    return [None if x is None else (x.data_ptr() if hasattr(x, "data_ptr") else x) for x in xs]


def decode_bench(steps, warmup, with_oracle=False):
    """Time prism_decode_step on each serving batch.  Inputs, states and
    histories are rotated over enough copies that a step's working set is not
    left in the 256 MB Infinity Cache by the step before."""
    import ctypes
    import torch
    from gated_delta_rule_prologue_amd import binding
    from gated_delta_rule_prologue_amd.configs import Workload
    from gated_delta_rule_prologue_amd.inputs import make_inputs

    out = {}
    stream = torch.cuda.current_stream()
    for name, n, H, dk, dv, L in DECODE_BATCHES:
        w = Workload(name, heads=H, dk=dk, dv=dv, L=L, dtype="bf16", seed=2000,
                     lengths=[1] * n)
        step = make_inputs(w)
        nbytes = decode_bytes(n, H, dk, dv, L, 2)
        ncopy = max(2, min(16, -(-(640 << 20) // nbytes)))
        base = binding.to_device(step)
        copies = []
        for i in range(ncopy):
            c = {k: (v.clone() if v is not None else None) for k, v in base.items()}
            c["S"] = torch.zeros((n, H, dk, dv), dtype=torch.float32, device="cuda")
            c["hist"] = torch.zeros((n, H, 3, dk), dtype=torch.bfloat16, device="cuda")
            c["o"] = torch.empty_like(c["v"])
            copies.append(c)

        for c in copies:                   # checked calls through the binding
            binding.decode_step(c["q"], c["k"], c["v"], c["u"], c["g"], c["b"], c["a"], c["h"],
                                c["conv_w"], L, c["S"], c["hist"], o=c["o"], stream=stream)
        lib = binding.lib()
        dims = binding.Dims(n, n, H, dk, dv, binding.PRISM_BF16)
        args = [[ctypes.byref(dims)] + raw_args(c["q"], c["k"], c["v"], c["u"], c["g"], c["b"],
                                                 c["a"], c["h"], c["conv_w"], L, 0, c["S"],
                                                 c["hist"], c["o"], stream.cuda_stream)
                for c in copies]
        for i in range(warmup):
            lib.prism_decode_step(*args[i % ncopy])
        torch.cuda.synchronize()
        ev = [[TimingEvent() for _ in range(2)] for _ in range(steps)]
        status = 0
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record(stream)
            status |= lib.prism_decode_step(*args[i % ncopy])
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        assert status == 0, binding.status_str(status)
        ms = sum(a.elapsed_time(b) for a, b in ev) / steps
        ach = nbytes / (ms * 1e-3) / 1e9
        # the same steps replayed from a HIP graph (captured once; no launch
        # overhead between steps): the per-step time a serving loop would see
        G, R = 16, 4
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(G):
                lib.prism_decode_step(*(args[i % ncopy][:-1] + [side.cuda_stream]))
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream().cuda_stream
            for i in range(G):
                lib.prism_decode_step(*(args[i % ncopy][:-1] + [cap]))
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = TimingEvent(), TimingEvent()
        g0.record(stream)
        for _ in range(R):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_us = g0.elapsed_time(g1) * 1e3 / (R * G)
        out[name] = {
            "sequences": n, "heads": H, "dk": dk, "dv": dv, "L": L, "dtype": "bf16",
            "tokens_per_s": steps * n / elapsed, "us_per_step": elapsed / steps * 1e6,
            "tokens_per_s_kernel": n / (ms * 1e-3),
            "graph_us_per_step": graph_us, "tokens_per_s_graph": n / (graph_us * 1e-6),
            "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic("decode", name),
                         "kernel": "decode", "avg_launch_us": ms * 1e3,
                         "algorithmic_bytes": nbytes},
            "state_copies": ncopy,
        }
        if with_oracle:
            import numpy as np
            import oracle
            S0 = np.zeros((n, H, dk, dv))
            h0 = np.zeros((n, H, 3, dk), dtype=np.uint16)
            out[name]["cpu_baseline"] = oracle_timed(
                lambda: oracle.decode_step(step, S0, h0), n, "tokens/s",
                f"the whole batch: one decode step of all {n * H} (sequence, head) chains, fp64")
    return out


def bwd_bytes(w, n_seqs, T, esize):
    """Algorithmic HBM bytes of one backward pass: the inputs read (q, k, v,
    u, a, h slots read, g, b, conv taps and dO, input dtype) and every gradient
    written once (fp32), per head-token, plus dS_init (fp32) per chain."""
    H, dk, dv, L = w.heads, w.dk, w.dv, w.L
    ht = T * H
    reads = esize * (2 * dk + dv + 2 * (L - 1) * dk + max(L - 2, 0) * dk + 2 + dv)
    writes = 4 * (2 * dk + dv + 3 * (L - 1) * dk + 2)
    return ht * (reads + writes) + 4 * n_seqs * H * dk * dv + H * dk * 4 * (esize + 4)


def bwd_flops(w, T):
    """fp32 vector flops of one backward pass in its token-recurrent form, per
    element of the dk x dv state and head-token: the forward token twice (the
    checkpoint sweep and the recomputation; p = S^T k 2, the update 5) and the
    reverse token (G += q dO^T 2, dq 2, dkw 2, dv 2, p 2, dg 4, G *= g 1,
    y 2, dk 4, G -= b k y^T 2): 37 in all."""
    return 37 * T * w.heads * w.dk * w.dv


def bwd_chunk_flops(w, T):
    """Dense MFMA flops of one backward pass in its chunkwise form (C = 64), per
    head-token: the forward's chunk algebra recomputed (scan_flops), the
    reverse state pass (K dS1, A_qk^T dO, T^T dX, Q^T dO, K^T dR:
    6 dk dv + 4 C dv), the state-dependent gradients (K S0, A_kkw V, T R, K dS1,
    A_qk^T dO, T^T dX, KW dS1, A_qkw^T dO, A_kkw^T dR, then dO S0^T, dR S0^T,
    X dS1^T, V dS1^T: 14 dk dv + 12 C dv) and the Gram-side gradients (four Gram
    products, four dA products, eight M products: 24 C dk + 8 C dv)."""
    C, dk, dv = 64, w.dk, w.dv
    per = 20 * dk * dv + 24 * C * dk + 24 * C * dv
    return (per + scan_flops_ht(w)) * T * w.heads


def training_pair_bench(w, inp, dims, dev_copies, steps, warmup, bwd_args):
    """Time a training step's pair: prism_fwd_ckpt (the forward, keeping the
    write keys and every chunk's start state) then prism_bwd_ckpt (every
    gradient, reading those instead of recomputing them; the token-sized
    gradients in bf16, as a bf16 training loop takes them), HIP events around
    each call; and the same loop of prism_fwd then prism_bwd (recomputing,
    fp32 gradients) on the same input copies, so both pairs see the same cache
    state."""
    import ctypes
    import torch
    from gated_delta_rule_prologue_amd import binding
    stream = torch.cuda.current_stream()
    lib = binding.lib()
    T = inp.total_tokens
    cb = binding.checkpoint_bytes(dims)
    fneed = binding.workspace_bytes(dims, w.L)
    lin = binding.RESIDUAL["linear"]
    fargs, bargs, pargs = [], [], []
    for c in dev_copies:
        c["ck"] = torch.empty(cb, dtype=torch.uint8, device="cuda")
        c["fws"] = torch.empty(fneed, dtype=torch.uint8, device="cuda")
        o, S, _ = binding.fwd_ckpt(c["q"], c["k"], c["v"], c["u"], c["g"], c["b"], c["a"], c["h"],
                                   c["conv_w"], c["cu_seqlens"], w.L, checkpoints=c["ck"])
        out = binding.bwd(c["q"], c["k"], c["v"], c["u"], c["g"], c["b"], c["a"], c["h"],
                          c["conv_w"], c["cu_seqlens"], w.L, c["dO"], want_dS_init=True,
                          workspace=c["bws"], checkpoints=c["ck"], grad_dtype=torch.bfloat16)
        fargs.append([ctypes.byref(dims)] + raw_args(
            c["q"], c["k"], c["v"], c["u"], c["g"], c["b"], c["a"], c["h"], c["conv_w"],
            c["cu_seqlens"], w.L, lin, None, o, S, c["ck"], None, 0, stream.cuda_stream))
        bargs.append([ctypes.byref(dims)] + raw_args(
            c["q"], c["k"], c["v"], c["u"], c["g"], c["b"], c["a"], c["h"], c["conv_w"],
            c["cu_seqlens"], w.L, lin, binding.PRISM_BF16, None, c["dO"], None, out["q"], out["k"], out["v"],
            out["u"], out["g"], out["b"], out["a"], out["h"], out["conv_w"], out["S_init"],
            c["ck"], c["bws"], c["bws"].numel(), stream.cuda_stream))
        pargs.append([ctypes.byref(dims)] + raw_args(
            c["q"], c["k"], c["v"], c["u"], c["g"], c["b"], c["a"], c["h"], c["conv_w"],
            c["cu_seqlens"], w.L, o, S, c["fws"], fneed, stream.cuda_stream))

    def pair(fwd, bwd, fa, ba):
        for i in range(warmup):
            fwd(*fa[i % len(fa)])
            bwd(*ba[i % len(ba)])
        torch.cuda.synchronize()
        ev = [[TimingEvent() for _ in range(3)] for _ in range(steps)]
        status = 0
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record(stream)
            status |= fwd(*fa[i % len(fa)])
            ev[i][1].record(stream)
            status |= bwd(*ba[i % len(ba)])
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        assert status == 0, binding.status_str(status)
        f_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
        b_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
        return steps * T / elapsed, f_ms * 1e3, b_ms * 1e3

    tps, f_us, b_us = pair(lib.prism_fwd_ckpt, lib.prism_bwd_ckpt, fargs, bargs)
    _, rf_us, rb_us = pair(lib.prism_fwd, lib.prism_bwd, pargs, bwd_args)

    # the same step through the torch.autograd wrapper (which makes the same two
    # calls, plus its own allocations and the casts of the fp32 gradients dg, db,
    # dconv_w), gradients of <dO, o> with respect to every input
    from gated_delta_rule_prologue_amd.autograd import prism
    names = ("q", "k", "v", "u", "g", "b", "a", "h", "conv_w")
    leaves = [{n: c[n].detach().requires_grad_(True) for n in names} for c in dev_copies]

    def ag_step(i):
        c, x = dev_copies[i % len(dev_copies)], leaves[i % len(leaves)]
        o, _ = prism(*(x[n] for n in names), c["cu_seqlens"], w.L)
        return torch.autograd.grad(o, [x[n] for n in names], grad_outputs=c["dO"])

    for i in range(warmup):
        ag_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ag_step(i)
    torch.cuda.synchronize()
    ag_us = (time.perf_counter() - t0) / steps * 1e6
    return {"tokens_per_s": tps, "us_per_step": f_us + b_us,
            "fwd_ckpt_us": f_us, "bwd_ckpt_us": b_us, "checkpoint_bytes": cb,
            "autograd_us_per_step": ag_us,
            "recompute_pair": {"us_per_step": rf_us + rb_us, "fwd_us": rf_us, "bwd_us": rb_us}}


def bwd_bench(w, inp, dev_copies, steps, warmup, with_oracle=False):
    """Time prism_bwd (gradients of every input) on the workload, with the
    upstream gradient dO and no carried state."""
    import ctypes
    import torch
    from gated_delta_rule_prologue_amd import binding
    stream = torch.cuda.current_stream()
    esize = 2 if w.dtype == "bf16" else 4
    T, H = inp.total_tokens, inp.heads
    dims = binding.Dims(inp.n_seqs, T, H, w.dk, w.dv, binding.PRISM_BF16 if esize == 2 else 0)
    lib = binding.lib()
    need = int(lib.prism_bwd_workspace_bytes(ctypes.byref(dims), w.L))
    args = []
    for c in dev_copies:
        g = torch.Generator(device="cuda").manual_seed(7)
        c["dO"] = torch.randn(c["v"].shape, device="cuda", generator=g).to(c["v"].dtype)
        out = binding.bwd(c["q"], c["k"], c["v"], c["u"], c["g"], c["b"], c["a"], c["h"],
                          c["conv_w"], c["cu_seqlens"], w.L, c["dO"], want_dS_init=True)
        c["grads"] = out
        c["bws"] = torch.empty(need, dtype=torch.uint8, device="cuda")
        args.append([ctypes.byref(dims)] + raw_args(
            c["q"], c["k"], c["v"], c["u"], c["g"], c["b"], c["a"], c["h"], c["conv_w"],
            c["cu_seqlens"], w.L, None, c["dO"], None, out["q"], out["k"], out["v"], out["u"],
            out["g"], out["b"], out["a"], out["h"], out["conv_w"], out["S_init"], c["bws"], need,
            stream.cuda_stream))
    for i in range(warmup):
        lib.prism_bwd(*args[i % len(args)])
    torch.cuda.synchronize()
    ev = [[TimingEvent() for _ in range(2)] for _ in range(steps)]
    status = 0
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        status |= lib.prism_bwd(*args[i % len(args)])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert status == 0, binding.status_str(status)
    ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    nbytes = bwd_bytes(w, inp.n_seqs, T, esize)
    flops = bwd_flops(w, T)
    ach = nbytes / (ms * 1e-3) / 1e9
    tf = flops / (ms * 1e-3) / 1e12
    # bf16 runs the chunkwise form (MFMA products; its floor is the HBM traffic
    # of the inputs and gradients), fp32 or PRISM_BWD_CHUNKED=0 the token walk
    # (fp32 vector arithmetic)
    chunked = esize == 2 and os.environ.get("PRISM_BWD_CHUNKED", "1") == "1"
    hbm = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": ach / HBM_PEAK_GBS, "traffic": None, "kernel": "backward (all launches)",
           "avg_launch_us": ms * 1e3, "algorithmic_bytes": nbytes}
    alu = {"bound": "alu", "achieved": tf, "peak": FP32_VALU_PEAK_TFLOPS,
           "unit": "TFLOP/s", "frac": tf / FP32_VALU_PEAK_TFLOPS, "traffic": None,
           "kernel": "backward (all launches)", "avg_launch_us": ms * 1e3,
           "algorithmic_flops": flops}
    res = {"tokens_per_s": steps * T / elapsed, "us_per_call": ms * 1e3,
           "path": "chunkwise" if chunked else "token walk",
           "roofline": hbm if chunked else alu, "hbm": hbm}
    if chunked:
        mf = bwd_chunk_flops(w, T)
        tfm = mf / (ms * 1e-3) / 1e12
        res["mfma"] = {"achieved": tfm, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                       "frac": tfm / BF16_PEAK_TFLOPS, "algorithmic_flops": mf}
        if binding.checkpoint_bytes(dims) > 0:
            res["training_pair"] = training_pair_bench(w, inp, dims, dev_copies, steps, warmup,
                                                       args)
    if with_oracle:
        # a bounded sample: as many whole (sequence, head) chains as host threads
        # (the oracle keeps every state of a chain), scaled to tokens/s of the
        # workload by the chains' share of its head-tokens
        import numpy as np
        import oracle
        nch = min(inp.n_seqs * H, oracle.default_threads())
        chains = list(range(nch))
        lens = np.diff(inp.cu_seqlens)
        ht = int(sum(lens[c // H] for c in chains))
        d_o = np.random.default_rng(7).standard_normal((T, H, w.dv))
        res["cpu_baseline"] = oracle_timed(
            lambda: oracle.bwd(inp, d_o, chains=chains), ht / H, "tokens/s",
            f"{nch} whole (sequence, head) chains ({ht} head-tokens) of the workload, fp64, one "
            f"thread per chain; tokens/s = head-tokens/s / H", min_seconds=1.0, max_passes=5)
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="workload name (default: lm-130m-layer)")
    ap.add_argument("--copies", type=int, default=3, help="input copies rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode steps (profiling runs); prints their JSON object")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after the timed region, run torch copies of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (--gpus {args.gpus} requested); "
              "the operator's (sequence, head) chains shard across GPUs without communication, "
              "so the per-GPU figure is the one reported", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_prologue_amd import binding
    from gated_delta_rule_prologue_amd.configs import BENCH_WORKLOAD, BY_NAME
    from gated_delta_rule_prologue_amd.inputs import make_inputs

    torch.cuda.set_device(0)
    binding.lib()
    if args.decode_only:
        print(json.dumps({"decode": decode_bench(args.steps, args.warmup)}), flush=True)
        return
    w = BY_NAME[args.workload or BENCH_WORKLOAD]
    inp = make_inputs(w)
    esize = 2 if w.dtype == "bf16" else 4
    n_seqs, T = inp.n_seqs, inp.total_tokens

    base = binding.to_device(inp)
    copies = [base] + [{k: (v.clone() if v is not None else None) for k, v in base.items()}
                       for _ in range(max(1, args.copies) - 1)]
    # the scan's segment buffers (few long sequences only; see prism_scan_ex)
    dims = binding.Dims(n_seqs, T, w.heads, w.dk, w.dv, binding.PRISM_BF16 if esize == 2 else 0)
    split_bytes = binding.scan_workspace_bytes(dims)
    for c in copies:
        c["kw"] = torch.empty_like(c["k"])
        c["o"] = torch.empty_like(c["v"])
        c["S"] = torch.empty((n_seqs, w.heads, w.dk, w.dv), dtype=torch.float32, device="cuda")
        c["ws"] = torch.empty(split_bytes, dtype=torch.uint8, device="cuda") if split_bytes else None
    stream = torch.cuda.current_stream()

    # one step = the launches prism_fwd makes: the prologue, then the scan
    def scan(c):
        binding.scan_ex(c["q"], c["k"], c["kw"], c["v"], c["g"], c["b"], c["cu_seqlens"],
                        o=c["o"], S_final=c["S"], workspace=c["ws"], stream=stream)

    def launch(c):
        binding.prologue(c["k"], c["u"], c["a"], c["h"], c["b"], c["conv_w"], c["cu_seqlens"],
                         w.L, kw=c["kw"], stream=stream)
        scan(c)

    # warmup through the checked binding calls; the timed loop then calls the C ABI
    # with the same tensors, marshalled once (raw_args)
    for i in range(args.warmup):
        launch(copies[i % len(copies)])
    torch.cuda.synchronize()
    import ctypes
    lib = binding.lib()
    pargs, sargs = [], []
    for c in copies:
        pargs.append([ctypes.byref(dims)] + raw_args(c["k"], c["u"], c["a"], c["h"], c["b"], c["conv_w"],
                                                      c["cu_seqlens"], w.L, c["kw"], stream.cuda_stream))
        sargs.append([ctypes.byref(dims)] + raw_args(c["q"], c["k"], c["kw"], c["v"], c["g"], c["b"],
                                                      c["cu_seqlens"], None, c["o"], c["S"], c["ws"],
                                                      split_bytes, stream.cuda_stream))

    K = args.steps
    # Launch durations come from HIP events on the launch stream (TimingEvent:
    # no cache writeback or invalidation at a record), recorded around both
    # launches of every EV_EVERY-th step of the timed region: each event is
    # still a packet of its own in the queue, so sampling keeps the
    # instrumentation from weighing on the timed throughput.
    EV_EVERY = 4
    sampled = [i for i in range(K) if i % EV_EVERY == 0]
    ev = {i: [TimingEvent() for _ in range(3)] for i in sampled}
    torch.cuda.synchronize()
    status = 0
    t0 = time.perf_counter()
    for i in range(K):
        j = i % len(copies)
        e = ev.get(i)
        if e:
            e[0].record(stream)
        status |= lib.prism_prologue(*pargs[j])
        if e:
            e[1].record(stream)
        status |= lib.prism_scan_ex(*sargs[j])
        if e:
            e[2].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert status == 0, binding.status_str(status)
    last = copies[(K - 1) % len(copies)]

    pro_ms = sum(e[0].elapsed_time(e[1]) for e in ev.values()) / len(ev)
    scan_ms = sum(e[1].elapsed_time(e[2]) for e in ev.values()) / len(ev)
    work = algorithmic_work(w, n_seqs, T, esize)

    def hbm(kernel, nbytes, ms):
        a = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": a / HBM_PEAK_GBS, "traffic": measured_traffic(kernel, w.name),
                "kernel": kernel, "avg_launch_us": ms * 1e3, "algorithmic_bytes": nbytes}

    # the non-linear refinement variant of the prologue (GELU residual chain), same
    # inputs and bytes, timed on its own after the forward steps
    gargs = []
    for c in copies:                       # checked calls through the binding
        binding.prologue_ex(c["k"], c["u"], c["a"], c["h"], c["b"], c["conv_w"], c["cu_seqlens"],
                            w.L, residual="gelu", kw=c["kw"], stream=stream)
        gargs.append([ctypes.byref(dims)] + raw_args(c["k"], c["u"], c["a"], c["h"], c["b"],
                                                      c["conv_w"], None, c["cu_seqlens"], w.L, 1,
                                                      c["kw"], stream.cuda_stream))
    gev = [[TimingEvent() for _ in range(2)] for _ in range(K)]
    status = 0
    for i in range(K):
        gev[i][0].record(stream)
        status |= lib.prism_prologue_ex(*gargs[i % len(copies)])
        gev[i][1].record(stream)
    torch.cuda.synchronize()
    assert status == 0, binding.status_str(status)
    gelu_ms = sum(a.elapsed_time(b) for a, b in gev) / K

    pro = hbm("prologue", work["prologue_bytes"], pro_ms)
    scn = hbm("scan", work["scan_bytes"], scan_ms)
    scn["mfma_tflops"] = work["scan_flops"] / (scan_ms * 1e-3) / 1e12
    scn["mfma_frac"] = scn["mfma_tflops"] / (BF16_PEAK_TFLOPS if esize == 2 else FP32_MFMA_PEAK_TFLOPS)
    scn["algorithmic_flops"] = work["scan_flops"]
    # the same from rocprofv3 counters (committed summary, same source-hash rule
    # as traffic): MFMA-busy share of all SIMD cycles, and the flops the MFMA
    # units executed (redundant work included) over this run's launch time
    mc = measured_mfma("scan", w.name)
    scn["mfma_counters"] = None if mc is None else {
        "busy_frac": mc[0], "flops_per_launch": mc[1],
        "tflops_executed": mc[1] / (scan_ms * 1e-3) / 1e12,
        "frac_of_peak": mc[1] / (scan_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
    dominant = scn if scan_ms >= pro_ms else pro

    out = {
        "metric": METRIC,
        "value": K * T / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": elapsed / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; shapes and distributions of the workload, inputs resident in HBM)",
        "config": {"workload": w.name, "n_seqs": n_seqs, "seq_len": T // n_seqs, "heads": w.heads,
                   "dk": w.dk, "dv": w.dv, "L": w.L, "tokens_per_step": T,
                   "head_tokens_per_step": work["head_tokens"], "input_copies": len(copies),
                   "scan_segments_workspace_bytes": split_bytes},
        "head_tokens_per_s": K * work["head_tokens"] / elapsed,
        "roofline": {k: dominant[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "kernels": {"prologue": pro, "scan": scn,
                    "prologue_gelu": dict(hbm("prologue", work["prologue_bytes"], gelu_ms),
                                          kernel="prologue (GELU residual chain)", traffic=None),
                    "pipeline_frac_hbm": (work["prologue_bytes"] + work["scan_bytes"]) / HBM_PEAK_GBS
                    / 1e9 / ((pro_ms + scan_ms) * 1e-3)},
    }
    out["roofline"]["kernel"] = dominant["kernel"]
    if not args.no_backward:
        out["backward"] = bwd_bench(w, inp, copies[:2], max(5, K // 5), 2,
                                    with_oracle=not args.no_cpu_baseline)
    if not args.no_decode:
        out["decode"] = decode_bench(max(20, K), max(5, args.warmup),
                                     with_oracle=not args.no_cpu_baseline)
    # last copy kernels of the run: the reference for the counter calibration
    if args.calibrate_copy_mib:
        nb = args.calibrate_copy_mib << 20
        src = torch.empty(nb // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        cb, parity = cpu_baseline(inp, last["o"], last["S"])
        out["cpu_baseline"] = cb
        import oracle
        out["kernels"]["prologue_gelu"]["cpu_baseline"] = oracle_timed(
            lambda: oracle.prologue(inp, residual="gelu"), T, "tokens/s",
            f"whole workload: write keys of all {T} tokens x {w.heads} heads, fp64")
        out["parity"] = parity
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
