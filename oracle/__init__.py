"""fp64 CPU oracle for the PRISM memory-writing operator (forward pass).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never loads it, and it shares no code with the GPU library.

The arithmetic lives in ``prism_oracle.c`` (plain C, double precision,
token-by-token recurrence; the definition and the readings it follows are in
that file's header).  This module only compiles it with gcc, marshals numpy
arrays through ctypes and returns double-precision numpy results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "prism_oracle.c")
_LIB = os.path.join(_HERE, "libprism_oracle.so")
_lib = None


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("n_seqs", "total_tokens", "heads", "dk", "dv", "L", "dtype", "residual")]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libprism_oracle.so``."""
    global _lib
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
                        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.prism_oracle_prologue.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P, P, P,
                                              ctypes.c_int]
        lib.prism_oracle_prologue.restype = ctypes.c_int
        lib.prism_oracle_fwd.argtypes = [ctypes.POINTER(_Dims), P, P, P, P, P, P, P, P, P, P, P, P,
                                         P, ctypes.c_int64, P, P, ctypes.c_int]
        lib.prism_oracle_fwd.restype = ctypes.c_int
        lib.prism_oracle_k_history.argtypes = [ctypes.POINTER(_Dims), P, P, P, P]
        lib.prism_oracle_k_history.restype = ctypes.c_int
        lib.prism_oracle_bwd.argtypes = [ctypes.POINTER(_Dims)] + [P] * 14 + [ctypes.c_int64] + \
            [P] * 10 + [ctypes.c_int]
        lib.prism_oracle_bwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:      # pragma: no cover
        return os.cpu_count() or 1


def _ptr(x: Optional[np.ndarray]):
    if x is None:
        return None
    assert x.flags["C_CONTIGUOUS"]
    return x.ctypes.data


RESIDUAL = {"linear": 0, "gelu": 1}


def _dims(inp, dtype_code: int, residual: str = "linear") -> _Dims:
    return _Dims(inp.n_seqs, inp.total_tokens, inp.heads, inp.dk, inp.dv, inp.L, dtype_code,
                 RESIDUAL[residual])


def _check(inp):
    code = {"f32": 0, "bf16": 1}[inp.dtype]
    want = np.float32 if code == 0 else np.uint16
    for name, arr in inp.arrays().items():
        if arr is None:
            continue
        if arr.dtype != want or not arr.flags["C_CONTIGUOUS"]:
            raise TypeError(f"oracle input {name}: expected contiguous {want.__name__}")
    cu = np.ascontiguousarray(inp.cu_seqlens, dtype=np.int32)
    return code, cu


def _hist(inp, k_hist):
    """Carried conv history [n_seqs, H, 3, dk] in the inputs' storage type, or None."""
    if k_hist is None:
        return None
    want = np.float32 if inp.dtype == "f32" else np.uint16
    k_hist = np.ascontiguousarray(k_hist)
    if k_hist.dtype != want or k_hist.shape != (inp.n_seqs, inp.heads, 3, inp.dk):
        raise TypeError(f"k_hist: expected {want.__name__} [{inp.n_seqs}, {inp.heads}, 3, {inp.dk}]")
    return k_hist


def _state(inp, S_init):
    if S_init is None:
        return None
    S_init = np.ascontiguousarray(S_init, dtype=np.float64)
    if S_init.shape != (inp.n_seqs, inp.heads, inp.dk, inp.dv):
        raise ValueError("S_init: expected [n_seqs, H, dk, dv]")
    return S_init


def prologue(inp, threads: Optional[int] = None, k_hist=None, residual: str = "linear") -> np.ndarray:
    """Write keys kw [T, H, dk] in float64 (``k_hist``: carried conv history;
    ``residual``: "linear" closed form or "gelu" refinement chain)."""
    code, cu = _check(inp)
    hist = _hist(inp, k_hist)
    out = np.zeros((inp.total_tokens, inp.heads, inp.dk), dtype=np.float64)
    d = _dims(inp, code, residual)
    rc = _load().prism_oracle_prologue(ctypes.byref(d), _ptr(cu), _ptr(inp.k), _ptr(inp.u),
                                       _ptr(inp.a), _ptr(inp.h), _ptr(inp.b), _ptr(inp.conv_w),
                                       _ptr(hist), _ptr(out), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"prism_oracle_prologue failed ({rc})")
    return out


def fwd(inp, chains: Optional[Sequence[int]] = None, threads: Optional[int] = None,
        S_init=None, k_hist=None, residual: str = "linear"):
    """Forward pass.  Returns (o [T, H, dv], S_final [n_seqs, H, dk, dv]) in float64.

    ``chains`` restricts the evaluation to the listed (sequence * H + head)
    chains; rows of other chains are left at zero.  ``S_init`` [n_seqs, H, dk,
    dv] is the state each sequence starts from and ``k_hist`` [n_seqs, H, 3,
    dk] (input storage type) the three k rows before each sequence's first
    token; both default to zero.  ``residual``: "linear" (closed-form chain) or
    "gelu" (non-linear refinement chain).
    """
    code, cu = _check(inp)
    hist, s0 = _hist(inp, k_hist), _state(inp, S_init)
    o = np.zeros((inp.total_tokens, inp.heads, inp.dv), dtype=np.float64)
    s = np.zeros((inp.n_seqs, inp.heads, inp.dk, inp.dv), dtype=np.float64)
    ch = None if chains is None else np.ascontiguousarray(np.asarray(chains, dtype=np.int64))
    if ch is not None and ch.size and (ch.min() < 0 or ch.max() >= inp.n_seqs * inp.heads):
        raise ValueError("chain index out of range")
    d = _dims(inp, code, residual)
    rc = _load().prism_oracle_fwd(ctypes.byref(d), _ptr(cu), _ptr(inp.q), _ptr(inp.k),
                                  _ptr(inp.v), _ptr(inp.u), _ptr(inp.g), _ptr(inp.b),
                                  _ptr(inp.a), _ptr(inp.h), _ptr(inp.conv_w), _ptr(s0),
                                  _ptr(hist), _ptr(ch), 0 if ch is None else int(ch.size),
                                  _ptr(o), _ptr(s), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"prism_oracle_fwd failed ({rc})")
    return o, s


def k_history(inp, k_hist=None) -> np.ndarray:
    """The conv history to carry past the end of each sequence: [n_seqs, H, 3,
    dk] float64, slot m = k at position (sequence end - 3 + m), read from
    ``k_hist`` (or zero) for positions before the sequence start."""
    code, cu = _check(inp)
    hist = _hist(inp, k_hist)
    out = np.zeros((inp.n_seqs, inp.heads, 3, inp.dk), dtype=np.float64)
    rc = _load().prism_oracle_k_history(ctypes.byref(_dims(inp, code)), _ptr(cu), _ptr(inp.k),
                                        _ptr(hist), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"prism_oracle_k_history failed ({rc})")
    return out


def decode_step(step, S, k_hist, threads: Optional[int] = None, residual: str = "linear"):
    """One token of every sequence: the recurrence itself with the state and
    conv history carried in.  ``step`` holds one token per sequence
    (cu_seqlens = 0, 1, ..., n_seqs).  Returns (o [n_seqs, H, dv], S_new,
    k_hist_new [n_seqs, H, 3, dk]) in float64."""
    if not np.array_equal(step.cu_seqlens, np.arange(step.n_seqs + 1)):
        raise ValueError("a decode step holds exactly one token per sequence")
    o, s = fwd(step, threads=threads, S_init=S, k_hist=k_hist, residual=residual)
    return o, s, k_history(step, k_hist)


def bwd(inp, d_o, dS_final=None, S_init=None, chains: Optional[Sequence[int]] = None,
        threads: Optional[int] = None, residual: str = "linear"):
    """Backward pass (``residual``: "linear" closed-form chain or "gelu") for the loss
    sum <d_o, o> + <dS_final, S_final>: a dict of float64 gradients for q, k,
    v [T, H, d], u, a, h [T, H, L-1, dk] (L > 1), g, b [T, H], conv_w [H, dk, 4]
    and S_init [n_seqs, H, dk, dv].  ``chains`` restricts the evaluation (rows of
    other chains stay zero; conv_w sums over the listed chains only)."""
    code, cu = _check(inp)
    T, H, dk, dv, L = inp.total_tokens, inp.heads, inp.dk, inp.dv, inp.L
    d_o = np.ascontiguousarray(d_o, dtype=np.float64)
    if d_o.shape != (T, H, dv):
        raise ValueError("d_o: expected [T, H, dv]")
    dsf = None if dS_final is None else np.ascontiguousarray(dS_final, dtype=np.float64)
    s0 = _state(inp, S_init)
    out = {"q": np.zeros((T, H, dk)), "k": np.zeros((T, H, dk)), "v": np.zeros((T, H, dv)),
           "g": np.zeros((T, H)), "b": np.zeros((T, H)), "conv_w": np.zeros((H, dk, 4)),
           "S_init": np.zeros((inp.n_seqs, H, dk, dv))}
    lv = (T, H, max(L - 1, 0), dk)
    for n in ("u", "a", "h"):
        out[n] = np.zeros(lv) if L > 1 else None
    ch = None if chains is None else np.ascontiguousarray(np.asarray(chains, dtype=np.int64))
    rc = _load().prism_oracle_bwd(
        ctypes.byref(_dims(inp, code, residual)), _ptr(cu), _ptr(inp.q), _ptr(inp.k), _ptr(inp.v),
        _ptr(inp.u), _ptr(inp.g), _ptr(inp.b), _ptr(inp.a), _ptr(inp.h), _ptr(inp.conv_w),
        _ptr(s0), _ptr(d_o), _ptr(dsf), _ptr(ch), 0 if ch is None else int(ch.size),
        _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]), _ptr(out["u"]), _ptr(out["g"]),
        _ptr(out["b"]), _ptr(out["a"]), _ptr(out["h"]), _ptr(out["conv_w"]), _ptr(out["S_init"]),
        threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"prism_oracle_bwd failed ({rc})")
    return out
