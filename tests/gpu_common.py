"""Helpers shared by the GPU parity tests: upload, run through the C ABI, compare."""
from __future__ import annotations

import numpy as np

# Tolerances on max|x_gpu - x_ref| / max|x_ref| (o and S_final separately):
# 1e-4 for fp32 inputs, 1e-2 for bf16 inputs with an fp32 state.
TOL = {"f32": 1e-4, "bf16": 1e-2}
# Write keys straight out of the prologue: fp32 arithmetic only (fp32), plus one
# round-to-nearest to bf16 (bf16, relative error <= 2^-9 per element).
TOL_KW = {"f32": 1e-5, "bf16": 2.0 ** -8}


def max_rel(x, ref, mask=None):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        x, ref = x[mask], ref[mask]
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(x - ref)))
    if den == 0.0:
        return num
    return num / den


def chain_row_mask(inp, chains):
    """Boolean mask [T, H] of the (token, head) rows that belong to the given chains."""
    m = np.zeros((inp.total_tokens, inp.heads), dtype=bool)
    for c in chains:
        n, e = divmod(int(c), inp.heads)
        m[inp.cu_seqlens[n]:inp.cu_seqlens[n + 1], e] = True
    return m


def to_host(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def gpu_fwd(inp, dev=None):
    import torch
    from gated_delta_rule_prologue_amd import binding
    dev = dev or binding.to_device(inp)
    o, s = binding.fwd(dev["q"], dev["k"], dev["v"], dev["u"], dev["g"], dev["b"], dev["a"],
                       dev["h"], dev["conv_w"], dev["cu_seqlens"], inp.L)
    torch.cuda.synchronize()
    return to_host(o), to_host(s)


def gpu_prologue(inp, dev=None):
    import torch
    from gated_delta_rule_prologue_amd import binding
    dev = dev or binding.to_device(inp)
    kw = binding.prologue(dev["k"], dev["u"], dev["a"], dev["h"], dev["b"], dev["conv_w"],
                          dev["cu_seqlens"], inp.L)
    torch.cuda.synchronize()
    return to_host(kw)


def say(msg):
    print(msg, flush=True)
