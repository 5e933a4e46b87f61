"""Pins of the oracle's non-linear refinement variant (residual = "gelu").

The gist.science summary of arXiv 2602.10796, section 2.2, refines the
residual with delta = GELU(gain * residual); the WeChat PRISM page, section
消除 Step 间串行, linearises it into the closed-form chain that the default
path uses.  The variant keeps the GELU: r_{l+1} = r_l - a_l GELU(h_l r_l).
Each test checks it against a route that does not share its code.
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle
from gated_delta_rule_prologue_amd.configs import Workload
from gated_delta_rule_prologue_amd.inputs import make_inputs
from tests import refs


def small(L=4, lengths=(37, 1, 2, 3, 70), H=2, dk=16, dv=12, dtype="f32", seed=13):
    return make_inputs(Workload("small", heads=H, dk=dk, dv=dv, L=L, dtype=dtype, seed=seed,
                                lengths=list(lengths)))


def rel(x, ref):
    return float(np.max(np.abs(np.asarray(x) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def test_gelu_reference_values():
    """The reference GELU: 0 at 0, Phi(1) at 1, -Phi(-1) at -1, odd part x/2."""
    x = np.array([0.0, 1.0, -1.0, 3.0])
    g = refs.gelu_cdf(x)
    assert g[0] == 0.0
    assert abs(g[1] - 0.5 * (1 + math.erf(1 / math.sqrt(2)))) < 1e-15
    assert abs(g[2] + 0.5 * (1 - math.erf(1 / math.sqrt(2)))) < 1e-15
    assert abs((g[3] - refs.gelu_cdf(-3.0)) - 3.0) < 1e-14          # GELU(x) - GELU(-x) = x


@pytest.mark.parametrize("L", [3, 4, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gelu_chain_matches_reference(L, dtype):
    """Write keys of the variant equal the level-by-level numpy chain with
    Phi from scipy (history included)."""
    inp = small(L=L, dtype=dtype)
    rng = np.random.default_rng(2)
    hist = rng.standard_normal((inp.n_seqs, inp.heads, 3, inp.dk)).astype(np.float32)
    if dtype == "bf16":
        from gated_delta_rule_prologue_amd.inputs import f32_to_bf16_bits
        hist = f32_to_bf16_bits(hist)
    kw = oracle.prologue(inp, residual="gelu", k_hist=hist)
    assert rel(kw, refs.write_key_gelu(inp, hist)) < 1e-13


def test_gelu_amplified_residual_matters():
    """With large gains the variant differs from the closed form by a lot, so a
    variant that silently fell back to the linear chain fails the test above."""
    inp = small(L=5)
    inp.h[:] = inp.h * np.float32(8.0)
    inp.u[:] = inp.u * np.float32(4.0)
    lin = oracle.prologue(inp)
    gel = oracle.prologue(inp, residual="gelu")
    assert rel(gel, lin) > 1e-2


@pytest.mark.parametrize("L", [1, 2])
def test_gelu_equals_linear_without_residual_updates(L):
    """L <= 2: no residual update reaches the write key, so both variants agree exactly."""
    inp = small(L=L)
    assert np.array_equal(oracle.prologue(inp, residual="gelu"), oracle.prologue(inp))
    o1, s1 = oracle.fwd(inp, residual="gelu")
    o2, s2 = oracle.fwd(inp)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_small_gain_limit_is_the_closed_form():
    """GELU(x) = x/2 + x^2/sqrt(2 pi) + O(x^4): with gains eps * h, the variant
    equals the closed form with gains eps * h / 2 up to O(eps^2)."""
    inp = small(L=6)
    for eps in (1e-2, 1e-3):
        gel = oracle.prologue(dataclasses.replace(inp, h=(inp.h * np.float32(eps)).astype(np.float32)),
                              residual="gelu")
        lin = oracle.prologue(dataclasses.replace(inp, h=(inp.h * np.float32(eps / 2)).astype(np.float32)))
        assert rel(gel, lin) < 3 * eps ** 2


def test_gelu_scan_is_unchanged():
    """Only the write key changes: the forward pass of the variant equals the
    linear-chain forward pass fed with the variant's write keys (g = 1, b = 0
    makes the scan causal linear attention, pinned by brute force)."""
    inp = small(L=4, lengths=(30, 4))
    inp.g[:] = 1
    inp.b[:] = 0
    kw = refs.write_key_gelu(inp)
    o, _ = oracle.fwd(inp, residual="gelu")
    assert rel(o, refs.linear_attention_bruteforce(inp.q, kw, inp.v, inp.cu_seqlens)) < 1e-12


def test_gelu_decode_steps_equal_one_call():
    inp = small(L=4, lengths=(6, 6), dtype="bf16")
    o, s = oracle.fwd(inp, residual="gelu")
    S = np.zeros((2, inp.heads, inp.dk, inp.dv))
    hist = np.zeros((2, inp.heads, 3, inp.dk), dtype=np.uint16)
    from gated_delta_rule_prologue_amd.inputs import f32_to_bf16_bits
    for t in range(6):
        rows = inp.cu_seqlens[:-1] + t
        step = dataclasses.replace(
            inp, cu_seqlens=np.arange(3, dtype=np.int32),
            **{f: np.ascontiguousarray(getattr(inp, f)[rows])
               for f in ("q", "k", "v", "u", "a", "h", "g", "b")})
        ot, S, h64 = oracle.decode_step(step, S, hist, residual="gelu")
        hist = f32_to_bf16_bits(h64.astype(np.float32))
        assert rel(ot, o[rows]) < 1e-12
    assert rel(S, s) < 1e-12
