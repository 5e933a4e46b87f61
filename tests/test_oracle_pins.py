"""Pins of the fp64 oracle against facts fixed by the PRISM pages and by mathematics.

Every test here checks ``oracle`` (token-by-token fp64 recurrence in C)
against something other than itself: a textbook routine, a closed form, an
invariant, a special case that reduces to a known model, or an exact-rational
brute force.  See ``tests/refs.py`` for the independent references.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from gated_delta_rule_prologue_amd.configs import Workload
from gated_delta_rule_prologue_amd.inputs import make_inputs, to_float, f32_to_bf16_bits
from tests import refs


def small(L=3, lengths=(37, 1, 2, 3, 70), H=2, dk=16, dv=12, dtype="f32", seed=7, g_mu=3.0):
    return make_inputs(Workload("small", heads=H, dk=dk, dv=dv, L=L, dtype=dtype, seed=seed,
                                lengths=list(lengths), g_mu=g_mu))


def rel(x, ref):
    return float(np.max(np.abs(np.asarray(x) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def as_f32(inp):
    """Same values as fp32 arrays (exact widening of bf16)."""
    conv = {}
    for n in ("q", "k", "v", "u", "a", "h", "g", "b", "conv_w"):
        x = getattr(inp, n)
        conv[n] = None if x is None else np.ascontiguousarray(to_float(x))
    return dataclasses.replace(inp, dtype="f32", **conv)


# --------------------------------------------------------------------------- input decoding
def test_bf16_inputs_widen_exactly():
    """bf16 inputs give bit-identical results to their exact fp32 widening."""
    inp = small(dtype="bf16", L=4)
    o1, s1 = oracle.fwd(inp)
    o2, s2 = oracle.fwd(as_f32(inp))
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    assert np.array_equal(oracle.prologue(inp), oracle.prologue(as_f32(inp)))


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.140625, 1e-3], dtype=np.float32)
    got = to_float(f32_to_bf16_bits(x))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even mantissa (1.0);
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6 -> 1 + 2^-6.
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == 1.0 + 2 ** -6
    assert got[3] == -2.5 and got[4] == 3.140625
    assert abs(got[5] - 1e-3) <= 1e-3 * 2 ** -8


# --------------------------------------------------------------------------- write branch
def test_anchor_is_causal_convolution():
    """With b = 0, a = 1, u = 1 and L = 2 the write key is the ShortConv anchor itself.

    Pinned against numpy.convolve per (sequence, channel): taps t-3..t, tap 3 on
    the current token, zero before each sequence start (PRISM anchor: WeChat
    page section 消除 Token 间串行; poster abstract).
    """
    inp = small(L=2)
    inp.b[:] = 0
    inp.a[:] = 1
    inp.u[:] = 1
    kw = oracle.prologue(inp)
    r0 = refs.anchor_convolve(inp.k, inp.conv_w, inp.cu_seqlens)
    assert rel(kw, r0) < 1e-14


def test_anchor_single_token_uses_tap3():
    inp = small(L=2, lengths=(1,))
    inp.b[:] = 0
    inp.a[:] = 1
    inp.u[:] = 1
    kw = oracle.prologue(inp)
    want = inp.conv_w[None, :, :, 3].astype(np.float64) * inp.k.astype(np.float64)
    assert np.array_equal(kw, want)


@pytest.mark.parametrize("L", [1, 2, 3, 5, 8])
def test_closed_form_equals_iterative_residual_chain(L):
    """Closed-form residual (WeChat page, 消除 Step 间串行) = repeated subtraction
    r <- r - (a h) r (gist.science section 2.2 with the GELU linearised)."""
    inp = small(L=L)
    assert rel(oracle.prologue(inp), refs.write_key_iterative(inp)) < 1e-13


def test_write_key_special_cases():
    inp = small(L=4)
    k = inp.k.astype(np.float64)
    bk = inp.b[:, :, None].astype(np.float64) * k
    # a = 0: only the GDN write key b k remains
    z = dataclasses.replace(inp, a=np.zeros_like(inp.a))
    assert np.array_equal(oracle.prologue(z), bk)
    # h = 0: no decay along the chain, kw = b k + r0 * sum_l a_l u_l
    z = dataclasses.replace(inp, h=np.zeros_like(inp.h))
    r0 = refs.anchor_convolve(inp.k, inp.conv_w, inp.cu_seqlens)
    want = bk + r0 * np.sum(inp.a.astype(np.float64) * inp.u.astype(np.float64), axis=2)
    assert rel(oracle.prologue(z), want) < 1e-14
    # a_1 h_1 = 1: levels 2.. see a zero residual
    a2 = inp.a.copy()
    h2 = inp.h.copy()
    a2[:, :, 0] = 0.5
    h2[:, :, 0] = 2.0
    z = dataclasses.replace(inp, a=a2, h=h2)
    want = bk + 0.5 * r0 * inp.u[:, :, 0].astype(np.float64)
    assert rel(oracle.prologue(z), want) < 1e-14


def test_last_h_slot_is_never_read():
    """With L-1 levels the chain multiplies only h_1..h_{L-2} into later levels."""
    inp = small(L=4)
    h2 = inp.h.copy()
    h2[:, :, -1] = 123.0
    z = dataclasses.replace(inp, h=h2)
    assert np.array_equal(oracle.prologue(z), oracle.prologue(inp))


# --------------------------------------------------------------------------- recurrence
def test_L1_is_gated_deltanet():
    """L = 1 reduces exactly to Gated DeltaNet (WeChat page 架构形式), checked
    against GDN written in prediction-error form."""
    inp = small(L=1, dk=16, dv=16)
    o, s = oracle.fwd(inp)
    o2, s2 = refs.gdn_delta_form(inp)
    assert rel(o, o2) < 1e-12 and rel(s, s2) < 1e-12


def test_ungated_no_erase_is_linear_attention():
    """g = 1, b = 0: causal linear attention with the PRISM write key, by O(T^2) sums."""
    inp = small(L=3, lengths=(40, 5, 1))
    inp.g[:] = 1
    inp.b[:] = 0
    kw = refs.write_key_iterative(inp)
    o, s = oracle.fwd(inp)
    o2 = refs.linear_attention_bruteforce(inp.q, kw, inp.v, inp.cu_seqlens)
    assert rel(o, o2) < 1e-12
    # the final state is sum_s kw_s v_s^T
    for n in range(inp.n_seqs):
        lo, hi = inp.cu_seqlens[n], inp.cu_seqlens[n + 1]
        for e in range(inp.heads):
            want = kw[lo:hi, e].T @ inp.v[lo:hi, e].astype(np.float64)
            assert np.max(np.abs(s[n, e] - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_linear_in_v():
    """o and S are linear in v: o(v1 + 2 v2) = o(v1) + 2 o(v2); o(0) = 0."""
    inp = small(L=4)
    rng = np.random.default_rng(3)
    v1 = to_float(f32_to_bf16_bits(rng.standard_normal(inp.v.shape).astype(np.float32)))
    v2 = to_float(f32_to_bf16_bits(rng.standard_normal(inp.v.shape).astype(np.float32)))
    mix = (v1 + np.float32(2.0) * v2).astype(np.float32)
    # bf16-valued operands: the fp32 mix is exact, so the identity holds to fp64 round-off
    assert np.array_equal(mix.astype(np.float64), v1.astype(np.float64) + 2.0 * v2.astype(np.float64))
    o1, s1 = oracle.fwd(dataclasses.replace(inp, v=v1))
    o2, s2 = oracle.fwd(dataclasses.replace(inp, v=v2))
    o3, s3 = oracle.fwd(dataclasses.replace(inp, v=mix))
    assert rel(o3, o1 + 2.0 * o2) < 1e-12
    assert rel(s3, s1 + 2.0 * s2) < 1e-12
    o0, s0 = oracle.fwd(dataclasses.replace(inp, v=np.zeros_like(inp.v)))
    assert not o0.any() and not s0.any()


def test_linear_in_v_exact_scaling():
    """Scaling v by a power of two scales o and S exactly."""
    inp = small(L=3)
    o1, s1 = oracle.fwd(inp)
    o2, s2 = oracle.fwd(dataclasses.replace(inp, v=(inp.v * np.float32(4.0))))
    assert np.array_equal(o2, 4.0 * o1) and np.array_equal(s2, 4.0 * s1)


@pytest.mark.parametrize("C", [1, 16, 64])
def test_chunkwise_ut_form(C):
    """Dense chunkwise WY/UT evaluation equals the token-by-token recurrence
    (the write depends on inputs only, so any chunking of the scan agrees:
    gist.science section 2.2, WeChat page 背景 on parallel scans)."""
    inp = small(L=4, lengths=(203, 64, 1, 65))
    kw = refs.write_key_iterative(inp)
    o, s = oracle.fwd(inp)
    o2, s2 = refs.chunkwise_ut(inp, kw, C)
    assert rel(o, o2) < 1e-12 and rel(s, s2) < 1e-12


def test_chunkwise_ut_small_gates():
    """Strong decay (g ~ sigmoid(N(-2,1))) exercises the masked exponentials."""
    inp = small(L=3, lengths=(150,), g_mu=-2.0)
    kw = refs.write_key_iterative(inp)
    o, s = oracle.fwd(inp)
    o2, s2 = refs.chunkwise_ut(inp, kw, 64)
    assert np.isfinite(o2).all()
    assert rel(o, o2) < 1e-10 and rel(s, s2) < 1e-10


def test_delta_rule_exact_retrieval():
    """L = 1, g = 1, b = 1, q = k, |k| = 1: the delta rule writes v_t exactly, o_t = v_t."""
    inp = small(L=1, lengths=(30,), dk=16, dv=8)
    inp.g[:] = 1
    inp.b[:] = 1
    kk = inp.k.astype(np.float64)
    kk /= np.linalg.norm(kk, axis=2, keepdims=True)
    inp = dataclasses.replace(inp, q=inp.k.copy())
    o, _ = oracle.fwd(inp)
    # |k| = 1 up to fp32 rounding of the normalised inputs
    assert np.max(np.abs(o - inp.v.astype(np.float64))) < 1e-5


def test_single_token():
    """T = 1: S = kw v^T and o = (q . kw) v."""
    inp = small(L=3, lengths=(1,))
    kw = oracle.prologue(inp)
    o, s = oracle.fwd(inp)
    v = inp.v.astype(np.float64)
    q = inp.q.astype(np.float64)
    for e in range(inp.heads):
        assert rel(s[0, e], np.outer(kw[0, e], v[0, e])) < 1e-15
        assert rel(o[0, e], np.dot(q[0, e], kw[0, e]) * v[0, e]) < 1e-14


def test_no_write_no_erase_gives_zero():
    """b = 0 and L = 1: the write key is zero, so o = 0 and S = 0."""
    inp = small(L=1)
    inp.b[:] = 0
    o, s = oracle.fwd(inp)
    assert not o.any() and not s.any()


def test_varlen_is_concatenation():
    """Packing sequences with cu_seqlens equals running each one alone (state and
    conv halo restart at every sequence boundary)."""
    inp = small(L=4, lengths=(37, 1, 2, 3, 70))
    o, s = oracle.fwd(inp)
    cu = inp.cu_seqlens
    for n in range(inp.n_seqs):
        lo, hi = int(cu[n]), int(cu[n + 1])
        one = dataclasses.replace(
            inp, cu_seqlens=np.array([0, hi - lo], dtype=np.int32),
            **{f: np.ascontiguousarray(getattr(inp, f)[lo:hi])
               for f in ("q", "k", "v", "u", "a", "h", "g", "b")})
        o1, s1 = oracle.fwd(one)
        assert np.array_equal(o1, o[lo:hi]) and np.array_equal(s1[0], s[n])


def test_empty_sequences():
    inp = small(L=3, lengths=(0, 5, 0, 3, 0))
    o, s = oracle.fwd(inp)
    assert not s[0].any() and not s[2].any() and not s[4].any()
    assert s[1].any() and s[3].any()
    o2, s2 = refs.gdn_delta_form(dataclasses.replace(inp, L=1, u=None, a=None, h=None))
    assert o.shape == o2.shape


def test_chain_selection_matches_full_run():
    inp = small(L=3)
    o, s = oracle.fwd(inp)
    chains = [1, 4, 9]
    o2, s2 = oracle.fwd(inp, chains=chains)
    for c in chains:
        n, e = divmod(c, inp.heads)
        lo, hi = inp.cu_seqlens[n], inp.cu_seqlens[n + 1]
        assert np.array_equal(o2[lo:hi, e], o[lo:hi, e]) and np.array_equal(s2[n, e], s[n, e])


def test_exact_rational_bruteforce():
    """Tiny case against exact rational arithmetic through explicit transition
    matrices A_t = g_t (I - b_t k_t k_t^T) (S_t = A_t S_{t-1} + kw_t v_t^T,
    gist.science section 2.1) and an exact residual chain."""
    inp = small(L=3, lengths=(4, 2), H=1, dk=3, dv=2, seed=11)
    kw = refs.write_key_exact(inp)
    o_ex, s_ex = refs.transition_products_exact(inp, kw)
    o, s = oracle.fwd(inp)
    kw_o = oracle.prologue(inp)
    kw_f = np.array([[[float(x) for x in row] for row in tok] for tok in kw])
    assert rel(kw_o, kw_f) < 1e-15
    o_f = np.array([[[float(x) for x in row] for row in tok] for tok in o_ex])
    s_f = np.array([[[[float(x) for x in r] for r in head] for head in seq] for seq in s_ex])
    assert rel(o, o_f) < 1e-14 and rel(s, s_f) < 1e-14


def test_reading_of_chain_start_is_discriminated():
    """The rejected reading of the residual chain (product starting at j = 0, so
    the anchor is shrunk by (1 - a_1 h_1) before the first level) moves the
    write key by far more than the fp32 tolerance: parity at 1e-4 therefore
    fixes which reading the kernels implement."""
    inp = small(L=3, lengths=(64,), dk=16, dv=16)
    kw = refs.write_key_iterative(inp)
    r0 = refs.anchor_convolve(inp.k, inp.conv_w, inp.cu_seqlens)
    a, h, u = (inp.a.astype(np.float64), inp.h.astype(np.float64), inp.u.astype(np.float64))
    alt = inp.b[:, :, None] * inp.k.astype(np.float64)
    r = r0 * (1 - a[:, :, 0] * h[:, :, 0])
    for s_ in range(inp.L - 1):
        alt = alt + a[:, :, s_] * r * u[:, :, s_]
        r = r - a[:, :, s_] * h[:, :, s_] * r
    assert rel(alt, kw) > 1e-3
    assert rel(oracle.prologue(inp), kw) < 1e-13
