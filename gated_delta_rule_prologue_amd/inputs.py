"""Seeded synthetic inputs for the PRISM memory-writing operator.

This module draws random tensors with the shapes and value distributions of
the workloads in ``configs.py``.  It holds none of the operator's arithmetic:
it only samples, squashes samples through a sigmoid or L2-normalises them (the
input recipe), and rounds them to bf16.  Both the GPU path and the fp64 oracle
consume exactly the arrays returned here.

Layout (row-major, ``T`` = total packed tokens, ``H`` = heads):

    q, k        [T, H, dk]            unit L2 norm per (token, head)
    v           [T, H, dv]
    u           [T, H, L-1, dk]       unit L2 norm per (token, head, level)
    a           [T, H, L-1, dk]       0.5 * sigmoid(N(0, 1))
    h           [T, H, L-1, dk]       sigmoid(N(0, 1))
    g, b        [T, H]                sigmoid(N(g_mu, 1)), sigmoid(N(0, 1))
    conv_w      [H, dk, 4]            N(0, 0.5^2); tap 3 multiplies the current token
    cu_seqlens  [n_seqs + 1] int32

bf16 tensors are returned as ``uint16`` arrays holding the raw bf16 bits
(round-to-nearest-even from fp32); fp32 tensors as ``float32``.

Reproducibility: every tensor gets its own child of ``SeedSequence(seed)``
(draw order: lengths, q, k, v, u, a, h, g, b, conv_w) and is filled in blocks,
each block with its own grandchild seed, so the values do not depend on the
number of threads used to fill them.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

from .configs import Workload

_BLOCK_ROWS = 1 << 15            # rows of the last axis per independently seeded block
_ORDER = ("lengths", "q", "k", "v", "u", "a", "h", "g", "b", "conv_w")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the raw uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits to fp32."""
    return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_float(x: np.ndarray) -> np.ndarray:
    """fp32 view of an input array, whichever of the two storage types it uses."""
    if x is None:
        return None
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x)
    return np.asarray(x, dtype=np.float32)


@dataclass
class Inputs:
    dtype: str                 # "f32" | "bf16"
    L: int
    heads: int
    dk: int
    dv: int
    cu_seqlens: np.ndarray     # int32 [n_seqs + 1]
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    u: Optional[np.ndarray]
    a: Optional[np.ndarray]
    h: Optional[np.ndarray]
    g: np.ndarray
    b: np.ndarray
    conv_w: np.ndarray

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def n_seqs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    def arrays(self) -> Dict[str, np.ndarray]:
        return {n: getattr(self, n) for n in ("q", "k", "v", "u", "g", "b", "a", "h", "conv_w")}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:          # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill(seq: np.random.SeedSequence, rows: int, width: int, transform, out_dtype: str,
          pool: ThreadPoolExecutor) -> np.ndarray:
    """Draw a [rows, width] tensor block by block; ``transform`` maps N(0,1) fp32 rows."""
    n_blocks = max(1, -(-rows // _BLOCK_ROWS))
    children = seq.spawn(n_blocks)
    out = np.empty((rows, width), dtype=np.uint16 if out_dtype == "bf16" else np.float32)

    def work(i):
        lo = i * _BLOCK_ROWS
        hi = min(rows, lo + _BLOCK_ROWS)
        if hi <= lo:
            return
        gen = np.random.Generator(np.random.PCG64(children[i]))
        x = gen.standard_normal((hi - lo, width), dtype=np.float32)
        x = transform(x)
        out[lo:hi] = f32_to_bf16_bits(x) if out_dtype == "bf16" else x

    list(pool.map(work, range(n_blocks)))
    return out


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x, dtype=np.float32))).astype(np.float32)


def _l2norm_rows(x):
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=1, keepdims=True))
    n[n == 0] = 1.0
    return (x / n).astype(np.float32)


def lengths_of(w: Workload, seq: Optional[np.random.SeedSequence] = None) -> np.ndarray:
    if w.lengths is not None:
        return np.asarray(w.lengths, dtype=np.int64)
    if w.lognormal is not None:
        n, mu, sigma, lo, hi = w.lognormal
        if seq is None:
            seq = np.random.SeedSequence(w.seed).spawn(len(_ORDER))[0]
        gen = np.random.Generator(np.random.PCG64(seq))
        x = gen.lognormal(mean=mu, sigma=sigma, size=int(n))
        return np.clip(np.rint(x), lo, hi).astype(np.int64)
    return np.full(w.n_seqs, w.seq_len, dtype=np.int64)


def make_inputs(w: Workload, threads: Optional[int] = None) -> Inputs:
    """Seeded synthetic inputs of workload ``w`` (see the module docstring)."""
    seqs = dict(zip(_ORDER, np.random.SeedSequence(w.seed).spawn(len(_ORDER))))
    lens = lengths_of(w, seqs["lengths"])
    cu = np.zeros(lens.shape[0] + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    if cu[-1] >= 2 ** 31:
        raise ValueError("total token count does not fit int32")
    cu = cu.astype(np.int32)
    T, H, dk, dv, L, dt = int(cu[-1]), w.heads, w.dk, w.dv, w.L, w.dtype
    ident = lambda x: x
    with ThreadPoolExecutor(max_workers=threads or _threads()) as pool:
        q = _fill(seqs["q"], T * H, dk, _l2norm_rows, dt, pool).reshape(T, H, dk)
        k = _fill(seqs["k"], T * H, dk, _l2norm_rows, dt, pool).reshape(T, H, dk)
        v = _fill(seqs["v"], T * H, dv, ident, dt, pool).reshape(T, H, dv)
        if L > 1:
            u = _fill(seqs["u"], T * H * (L - 1), dk, _l2norm_rows, dt, pool).reshape(T, H, L - 1, dk)
            a = _fill(seqs["a"], T * H * (L - 1), dk, lambda x: (0.5 * _sigmoid(x)).astype(np.float32),
                      dt, pool).reshape(T, H, L - 1, dk)
            h = _fill(seqs["h"], T * H * (L - 1), dk, _sigmoid, dt, pool).reshape(T, H, L - 1, dk)
        else:
            u = a = h = None
        g_mu = np.float32(w.g_mu)
        g = _fill(seqs["g"], T, H, lambda x: _sigmoid(x + g_mu), dt, pool).reshape(T, H)
        b = _fill(seqs["b"], T, H, _sigmoid, dt, pool).reshape(T, H)
        conv_w = _fill(seqs["conv_w"], H * dk, 4, lambda x: (0.5 * x).astype(np.float32),
                       dt, pool).reshape(H, dk, 4)
    return Inputs(dt, L, H, dk, dv, cu, q, k, v, u, a, h, g, b, conv_w)
