"""ctypes binding of libprism (C ABI in ``include/prism.h``).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the operator runs in the library's HIP kernels.  The
functions raise if the library is not built -- there is no fallback path.

Names follow the C ABI: ``fwd`` -> prism_fwd, ``fwd_resume`` ->
prism_fwd_resume, ``fwd_noalloc`` -> prism_fwd_noalloc, ``decode_step`` -> prism_decode_step, ``prologue`` ->
prism_prologue, ``prologue_ex`` -> prism_prologue_ex, ``scan`` -> prism_scan,
``scan_ex`` -> prism_scan_ex, ``workspace_bytes`` -> prism_workspace_bytes,
``scan_workspace_bytes`` -> prism_scan_workspace_bytes, ``fwd_ckpt`` -> prism_fwd_ckpt,
``checkpoint_bytes`` -> prism_checkpoint_bytes, ``bwd`` -> prism_bwd_ex or prism_bwd_ckpt (prism_bwd
with a residual choice), ``scan_wait_giveups`` -> prism_scan_wait_giveups.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libprism.so")
_lib = None

PRISM_OK, PRISM_EINVAL, PRISM_EUNSUPPORTED, PRISM_EHIP, PRISM_ENOSPACE = 0, 1, 2, 3, 4
NOALLOC_MAX_BYTES = 64 << 20                 # PRISM_NOALLOC_MAX_BYTES
PRISM_F32, PRISM_BF16 = 0, 1
RESIDUAL = {"linear": 0, "gelu": 1}          # prism_residual
MAX_LEVELS = 16


class PrismError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("n_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("heads", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libprism.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built: run __graft_entry__.build() "
                               "(or python -m gated_delta_rule_prologue_amd.build)")
        L = ctypes.CDLL(_LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        D = ctypes.POINTER(Dims)
        L.prism_workspace_bytes.argtypes = [D, I]
        L.prism_workspace_bytes.restype = S
        L.prism_fwd.argtypes = [D, P, P, P, P, P, P, P, P, P, P, I, P, P, P, S, P]
        L.prism_fwd.restype = I
        L.prism_fwd_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P, I, P, P, P]
        L.prism_fwd_noalloc.restype = I
        L.prism_prologue.argtypes = [D, P, P, P, P, P, P, P, I, P, P]
        L.prism_prologue.restype = I
        L.prism_scan.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
        L.prism_scan.restype = I
        L.prism_scan_ex.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, S, P]
        L.prism_scan_ex.restype = I
        L.prism_scan_workspace_bytes.argtypes = [D]
        L.prism_scan_workspace_bytes.restype = S
        L.prism_prologue_ex.argtypes = [D, P, P, P, P, P, P, P, P, I, I, P, P]
        L.prism_prologue_ex.restype = I
        L.prism_fwd_resume.argtypes = [D, P, P, P, P, P, P, P, P, P, P, I, I, P, P, P, P, P, P, S, P]
        L.prism_fwd_resume.restype = I
        L.prism_decode_step.argtypes = [D, P, P, P, P, P, P, P, P, P, I, I, P, P, P, P]
        L.prism_bwd_workspace_bytes.argtypes = [D, I]
        L.prism_bwd_workspace_bytes.restype = S
        L.prism_bwd.argtypes = [D] + [P] * 10 + [I] + [P] * 14 + [S, P]
        L.prism_bwd.restype = I
        L.prism_bwd_ex.argtypes = [D] + [P] * 10 + [I, I] + [P] * 14 + [S, P]
        L.prism_bwd_ex.restype = I
        L.prism_checkpoint_bytes.argtypes = [D]
        L.prism_checkpoint_bytes.restype = S
        L.prism_fwd_ckpt.argtypes = [D] + [P] * 10 + [I, I] + [P] * 5 + [S, P]
        L.prism_fwd_ckpt.restype = I
        L.prism_bwd_ckpt.argtypes = [D] + [P] * 10 + [I, I, I] + [P] * 15 + [S, P]
        L.prism_bwd_ckpt.restype = I
        L.prism_decode_step.restype = I
        L.prism_status_str.argtypes = [I]
        L.prism_status_str.restype = ctypes.c_char_p
        L.prism_scan_wait_giveups.argtypes = [ctypes.POINTER(ctypes.c_uint), I]
        L.prism_scan_wait_giveups.restype = I
        L.prism_abi_version.argtypes = []
        L.prism_abi_version.restype = I
        _lib = L
    return _lib


def status_str(s: int) -> str:
    return lib().prism_status_str(int(s)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return PRISM_BF16
    if t.dtype == torch.float32:
        return PRISM_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libprism takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libprism takes contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def make_dims(n_seqs: int, total_tokens: int, heads: int, dk: int, dv: int, dtype: int) -> Dims:
    return Dims(n_seqs, total_tokens, heads, dk, dv, dtype)


def _dims_of(q_or_k: torch.Tensor, v: Optional[torch.Tensor], cu_seqlens: torch.Tensor) -> Dims:
    if q_or_k.dim() != 3:
        raise ValueError("q / k must be [T, H, dk]")
    T, H, dk = q_or_k.shape
    dv = v.shape[2] if v is not None else dk
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be int32 [n_seqs + 1] with n_seqs >= 1")
    return Dims(cu_seqlens.numel() - 1, T, H, dk, dv, _dtype_code(q_or_k))


def _expect(name: str, t: Optional[torch.Tensor], shape, dtype):
    """Shape / dtype check so that the kernels never index past a caller's buffer."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


def _check_write_branch(d: Dims, dt, k, u, a, h, b, conv_w, L: int):
    T, H, dk = d.total_tokens, d.heads, d.dk
    _expect("k", k, (T, H, dk), dt)
    _expect("b", b, (T, H), dt)
    _expect("conv_w", conv_w, (H, dk, 4), dt)
    if not 1 <= int(L) <= MAX_LEVELS:
        raise ValueError(f"L must be in 1..{MAX_LEVELS}")
    if L > 1:
        for name, x in (("u", u), ("a", a), ("h", h)):
            _expect(name, x, (T, H, L - 1, dk), dt)


def _check_scan(d: Dims, dt, q, k, kw, v, g, b):
    T, H = d.total_tokens, d.heads
    for name, x in (("q", q), ("k", k), ("kw", kw)):
        _expect(name, x, (T, H, d.dk), dt)
    _expect("v", v, (T, H, d.dv), dt)
    _expect("g", g, (T, H), dt)
    _expect("b", b, (T, H), dt)


def workspace_bytes(dims: Dims, L: int) -> int:
    return int(lib().prism_workspace_bytes(ctypes.byref(dims), int(L)))


def _check(fn: str, status: int):
    if status != PRISM_OK:
        raise PrismError(fn, status)


def prologue(k, u, a, h, b, conv_w, cu_seqlens, L: int, kw=None, stream=None) -> torch.Tensor:
    """Write keys kw [T, H, dk] (prism_prologue)."""
    d = _dims_of(k, None, cu_seqlens)
    _check_write_branch(d, k.dtype, k, u, a, h, b, conv_w, L)
    if kw is None:
        kw = torch.empty_like(k)
    _expect("kw", kw, k.shape, k.dtype)
    _check("prism_prologue", lib().prism_prologue(
        ctypes.byref(d), _ptr(k), _ptr(u), _ptr(a), _ptr(h), _ptr(b), _ptr(conv_w),
        _ptr(cu_seqlens), int(L), _ptr(kw), _stream(stream)))
    return kw


def prologue_ex(k, u, a, h, b, conv_w, cu_seqlens, L: int, k_hist=None, residual="linear",
                kw=None, stream=None) -> torch.Tensor:
    """Write keys with a carried history and a choice of residual chain
    (prism_prologue_ex; ``residual`` is "linear" or "gelu")."""
    d = _dims_of(k, None, cu_seqlens)
    _check_write_branch(d, k.dtype, k, u, a, h, b, conv_w, L)
    if k_hist is not None:
        _expect("k_hist", k_hist, (d.n_seqs, d.heads, 3, d.dk), k.dtype)
    if kw is None:
        kw = torch.empty_like(k)
    _expect("kw", kw, k.shape, k.dtype)
    _check("prism_prologue_ex", lib().prism_prologue_ex(
        ctypes.byref(d), _ptr(k), _ptr(u), _ptr(a), _ptr(h), _ptr(b), _ptr(conv_w), _ptr(k_hist),
        _ptr(cu_seqlens), int(L), RESIDUAL[residual], _ptr(kw), _stream(stream)))
    return kw


def scan(q, k, kw, v, g, b, cu_seqlens, o=None, S_final=None, stream=None):
    """Chunkwise scan from precomputed write keys (prism_scan).  Returns (o, S_final)."""
    d = _dims_of(q, v, cu_seqlens)
    _check_scan(d, q.dtype, q, k, kw, v, g, b)
    if o is None:
        o = torch.empty_like(v)
    if S_final is None:
        S_final = torch.empty((d.n_seqs, d.heads, d.dk, d.dv), dtype=torch.float32, device=q.device)
    _expect("o", o, v.shape, v.dtype)
    _expect("S_final", S_final, (d.n_seqs, d.heads, d.dk, d.dv), torch.float32)
    _check("prism_scan", lib().prism_scan(
        ctypes.byref(d), _ptr(q), _ptr(k), _ptr(kw), _ptr(v), _ptr(g), _ptr(b), _ptr(cu_seqlens),
        _ptr(o), _ptr(S_final), _stream(stream)))
    return o, S_final


def scan_workspace_bytes(dims: Dims) -> int:
    return int(lib().prism_scan_workspace_bytes(ctypes.byref(dims)))


def scan_ex(q, k, kw, v, g, b, cu_seqlens, S_init=None, o=None, S_final=None, workspace=None,
            stream=None):
    """Scan with a start state and the segment split for few long sequences
    (prism_scan_ex).  Returns (o, S_final)."""
    d = _dims_of(q, v, cu_seqlens)
    _check_scan(d, q.dtype, q, k, kw, v, g, b)
    if S_init is not None:
        _expect("S_init", S_init, (d.n_seqs, d.heads, d.dk, d.dv), torch.float32)
    need = scan_workspace_bytes(d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(v)
    if S_final is None:
        S_final = torch.empty((d.n_seqs, d.heads, d.dk, d.dv), dtype=torch.float32, device=q.device)
    _expect("o", o, v.shape, v.dtype)
    _expect("S_final", S_final, (d.n_seqs, d.heads, d.dk, d.dv), torch.float32)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace needs {need} bytes")
    _check("prism_scan_ex", lib().prism_scan_ex(
        ctypes.byref(d), _ptr(q), _ptr(k), _ptr(kw), _ptr(v), _ptr(g), _ptr(b), _ptr(cu_seqlens),
        _ptr(S_init), _ptr(o), _ptr(S_final), _ptr(workspace), nbytes, _stream(stream)))
    return o, S_final


def fwd(q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L: int, o=None, S_final=None,
        workspace=None, stream=None):
    """Full forward pass (prism_fwd).  Returns (o, S_final)."""
    d = _dims_of(q, v, cu_seqlens)
    _check_write_branch(d, q.dtype, k, u, a, h, b, conv_w, L)
    _check_scan(d, q.dtype, q, k, k, v, g, b)
    need = workspace_bytes(d, L)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(v)
    if S_final is None:
        S_final = torch.empty((d.n_seqs, d.heads, d.dk, d.dv), dtype=torch.float32, device=q.device)
    _expect("o", o, v.shape, v.dtype)
    _expect("S_final", S_final, (d.n_seqs, d.heads, d.dk, d.dv), torch.float32)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    _check("prism_fwd", lib().prism_fwd(
        ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(g), _ptr(b), _ptr(a), _ptr(h),
        _ptr(conv_w), _ptr(cu_seqlens), int(L), _ptr(o), _ptr(S_final), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, S_final


def fwd_noalloc(q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L: int, o, S_final, stream=None):
    """Forward pass with the library's static scratch as workspace
    (prism_fwd_noalloc): the caller passes the outputs o and S_final, and
    nothing is allocated.  Returns (o, S_final)."""
    d = _dims_of(q, v, cu_seqlens)
    _check_write_branch(d, q.dtype, k, u, a, h, b, conv_w, L)
    _check_scan(d, q.dtype, q, k, k, v, g, b)
    _expect("o", o, v.shape, v.dtype)
    _expect("S_final", S_final, (d.n_seqs, d.heads, d.dk, d.dv), torch.float32)
    _check("prism_fwd_noalloc", lib().prism_fwd_noalloc(
        ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(g), _ptr(b), _ptr(a), _ptr(h),
        _ptr(conv_w), _ptr(cu_seqlens), int(L), _ptr(o), _ptr(S_final), _stream(stream)))
    return o, S_final


def fwd_resume(q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L: int, S_init=None, k_hist=None,
               o=None, S_final=None, k_hist_out=None, workspace=None, stream=None,
               residual="linear"):
    """Forward pass continuing from a carried state and conv history
    (prism_fwd_resume).  ``S_init`` fp32 [n_seqs, H, dk, dv] and ``k_hist``
    [n_seqs, H, 3, dk] default to zero; ``k_hist_out`` (optional, may be
    ``k_hist``) receives the history to carry on; ``residual`` is "linear"
    or "gelu".  Returns (o, S_final, k_hist_out)."""
    d = _dims_of(q, v, cu_seqlens)
    _check_write_branch(d, q.dtype, k, u, a, h, b, conv_w, L)
    _check_scan(d, q.dtype, q, k, k, v, g, b)
    n, H = d.n_seqs, d.heads
    if S_init is not None:
        _expect("S_init", S_init, (n, H, d.dk, d.dv), torch.float32)
    for name, x in (("k_hist", k_hist), ("k_hist_out", k_hist_out)):
        if x is not None:
            _expect(name, x, (n, H, 3, d.dk), q.dtype)
    need = workspace_bytes(d, L)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(v)
    if S_final is None:
        S_final = torch.empty((n, H, d.dk, d.dv), dtype=torch.float32, device=q.device)
    _expect("o", o, v.shape, v.dtype)
    _expect("S_final", S_final, (n, H, d.dk, d.dv), torch.float32)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    _check("prism_fwd_resume", lib().prism_fwd_resume(
        ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(g), _ptr(b), _ptr(a), _ptr(h),
        _ptr(conv_w), _ptr(cu_seqlens), int(L), RESIDUAL[residual], _ptr(S_init), _ptr(k_hist), _ptr(o),
        _ptr(S_final), _ptr(k_hist_out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, S_final, k_hist_out


def decode_step(q, k, v, u, g, b, a, h, conv_w, L: int, S, k_hist, o=None, stream=None,
                residual="linear"):
    """One new token per sequence (prism_decode_step): q, k [N, H, dk], v [N, H,
    dv], u/a/h [N, H, L-1, dk], g/b [N, H].  ``S`` fp32 [N, H, dk, dv] and
    ``k_hist`` [N, H, 3, dk] are updated in place.  Returns o [N, H, dv]."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q / v must be [N, H, d]")
    N, H, dk = q.shape
    d = Dims(N, N, H, dk, v.shape[2], _dtype_code(q))
    _check_write_branch(d, q.dtype, k, u, a, h, b, conv_w, L)
    _expect("q", q, (N, H, dk), q.dtype)
    _expect("v", v, (N, H, d.dv), q.dtype)
    _expect("g", g, (N, H), q.dtype)
    _expect("S", S, (N, H, dk, d.dv), torch.float32)
    _expect("k_hist", k_hist, (N, H, 3, dk), q.dtype)
    if o is None:
        o = torch.empty_like(v)
    _expect("o", o, v.shape, v.dtype)
    _check("prism_decode_step", lib().prism_decode_step(
        ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(g), _ptr(b), _ptr(a), _ptr(h),
        _ptr(conv_w), int(L), RESIDUAL[residual], _ptr(S), _ptr(k_hist), _ptr(o), _stream(stream)))
    return o


def checkpoint_bytes(dims: Dims) -> int:
    """Bytes of prism_fwd_ckpt's chunk-start states for the shape (0: none)."""
    return int(lib().prism_checkpoint_bytes(ctypes.byref(dims)))


def fwd_ckpt(q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L: int, S_init=None, o=None,
             S_final=None, checkpoints=None, workspace=None, stream=None, residual="linear"):
    """Forward pass that keeps every chunk's start state and the write keys for
    the backward (prism_fwd_ckpt; it uses no workspace, ``workspace`` is passed
    through if given).  Returns (o, S_final, checkpoints), the last a uint8
    device tensor of checkpoint_bytes(dims) bytes to pass to bwd()."""
    d = _dims_of(q, v, cu_seqlens)
    _check_write_branch(d, q.dtype, k, u, a, h, b, conv_w, L)
    _check_scan(d, q.dtype, q, k, k, v, g, b)
    n, H = d.n_seqs, d.heads
    if S_init is not None:
        _expect("S_init", S_init, (n, H, d.dk, d.dv), torch.float32)
    cb = checkpoint_bytes(d)
    if checkpoints is None:
        checkpoints = torch.empty(max(cb, 1), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty_like(v)
    if S_final is None:
        S_final = torch.empty((n, H, d.dk, d.dv), dtype=torch.float32, device=q.device)
    _expect("o", o, v.shape, v.dtype)
    _expect("S_final", S_final, (n, H, d.dk, d.dv), torch.float32)
    if checkpoints.numel() * checkpoints.element_size() < cb:
        raise ValueError(f"checkpoints need {cb} bytes")
    _check("prism_fwd_ckpt", lib().prism_fwd_ckpt(
        ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(g), _ptr(b), _ptr(a), _ptr(h),
        _ptr(conv_w), _ptr(cu_seqlens), int(L), RESIDUAL[residual], _ptr(S_init), _ptr(o),
        _ptr(S_final), _ptr(checkpoints), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, S_final, checkpoints


def bwd(q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L: int, dO, dS_final=None, S_init=None,
        want_dS_init: bool = True, workspace=None, stream=None, residual="linear",
        checkpoints=None, grad_dtype=None) -> dict:
    """Gradients of sum <dO, o> + <dS_final, S_final> (prism_bwd_ex, or
    prism_bwd_ckpt with the ``checkpoints`` of fwd_ckpt on the same inputs;
    ``residual`` "linear" closed-form chain or "gelu"): a dict of tensors q, k,
    v, u, a, h, g, b, conv_w and S_init (the last when ``want_dS_init``), all
    fp32, except that with checkpoints ``grad_dtype=torch.bfloat16`` stores q,
    k, v, u, a, h in bf16 (each the fp32 value rounded to nearest even)."""
    if residual not in RESIDUAL:
        raise ValueError(f"residual must be one of {sorted(RESIDUAL)}")
    d = _dims_of(q, v, cu_seqlens)
    _check_write_branch(d, q.dtype, k, u, a, h, b, conv_w, L)
    _check_scan(d, q.dtype, q, k, k, v, g, b)
    _expect("dO", dO, v.shape, v.dtype)
    n, T, H, dk, dv = d.n_seqs, d.total_tokens, d.heads, d.dk, d.dv
    for name, x in (("dS_final", dS_final), ("S_init", S_init)):
        if x is not None:
            _expect(name, x, (n, H, dk, dv), torch.float32)
    if grad_dtype not in (None, torch.float32, torch.bfloat16):
        raise ValueError("grad_dtype must be torch.float32 or torch.bfloat16")
    if grad_dtype == torch.bfloat16 and checkpoints is None:
        raise ValueError("bf16 gradients need the checkpoints of fwd_ckpt")
    f32 = dict(dtype=torch.float32, device=q.device)
    gt = dict(dtype=grad_dtype or torch.float32, device=q.device)
    out = {"q": torch.empty((T, H, dk), **gt), "k": torch.empty((T, H, dk), **gt),
           "v": torch.empty((T, H, dv), **gt), "g": torch.empty((T, H), **f32),
           "b": torch.empty((T, H), **f32), "conv_w": torch.empty((H, dk, 4), **f32),
           "S_init": torch.empty((n, H, dk, dv), **f32) if want_dS_init else None}
    for name in ("u", "a", "h"):
        out[name] = torch.empty((T, H, L - 1, dk), **gt) if L > 1 else None
    need = int(lib().prism_bwd_workspace_bytes(ctypes.byref(d), int(L)))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    grads = (_ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]), _ptr(out["u"]), _ptr(out["g"]),
             _ptr(out["b"]), _ptr(out["a"]), _ptr(out["h"]), _ptr(out["conv_w"]), _ptr(out["S_init"]))
    head = (ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(u), _ptr(g), _ptr(b), _ptr(a), _ptr(h),
            _ptr(conv_w), _ptr(cu_seqlens), int(L), RESIDUAL[residual])
    state = (_ptr(S_init), _ptr(dO), _ptr(dS_final))
    tail = (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if checkpoints is not None:
        cb = checkpoint_bytes(d)
        if checkpoints.numel() * checkpoints.element_size() < cb:
            raise ValueError(f"checkpoints need {cb} bytes")
        gd = PRISM_BF16 if grad_dtype == torch.bfloat16 else PRISM_F32
        _check("prism_bwd_ckpt", lib().prism_bwd_ckpt(*head, gd, *state, *grads, _ptr(checkpoints),
                                                       *tail))
    else:
        _check("prism_bwd_ex", lib().prism_bwd_ex(*head, *state, *grads, *tail))
    return out


def scan_wait_giveups(reset: bool = True) -> int:
    """Bounded in-kernel waits that gave up since the last reset
    (prism_scan_wait_giveups, synchronous); 0 when every scan ran as designed."""
    n = ctypes.c_uint(0)
    _check("prism_scan_wait_giveups", lib().prism_scan_wait_giveups(ctypes.byref(n), int(reset)))
    return int(n.value)


def to_device(inp, device="cuda") -> dict:
    """Upload an ``inputs.Inputs`` to device tensors (bf16 bits reinterpreted, no rounding)."""
    out = {}
    for name, arr in inp.arrays().items():
        if arr is None:
            out[name] = None
            continue
        t = torch.from_numpy(arr)
        if arr.dtype.name == "uint16":
            t = t.view(torch.bfloat16)
        out[name] = t.to(device).contiguous()
    out["cu_seqlens"] = torch.from_numpy(inp.cu_seqlens).to(device)
    return out
