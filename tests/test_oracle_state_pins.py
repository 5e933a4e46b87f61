"""Pins of the oracle's carried state: an initial state S_init, a carried
convolution history k_hist, and the single-token decode step.

The state matrix of the operator holds the whole history of a sequence in a
fixed size and is updated one token at a time (WeChat ICML 2026 PRISM page,
section 背景：无限背包 vs 有限背包; poster page, lay summary), so a sequence
may be processed in pieces.  Each test checks the oracle's new arguments
against a route that does not use them: the zero-state path pinned in
``test_oracle_pins.py``, a textbook convolution over the concatenated rows,
GDN in prediction-error form, causal linear attention by brute force, or the
dense chunkwise formulation started from a given state.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from gated_delta_rule_prologue_amd.configs import Workload
from gated_delta_rule_prologue_amd.inputs import make_inputs, f32_to_bf16_bits
from tests import refs

PER_TOKEN = ("q", "k", "v", "u", "a", "h", "g", "b")


def small(L=3, lengths=(37, 1, 2, 3, 70), H=2, dk=16, dv=12, dtype="f32", seed=11, g_mu=3.0):
    return make_inputs(Workload("small", heads=H, dk=dk, dv=dv, L=L, dtype=dtype, seed=seed,
                                lengths=list(lengths), g_mu=g_mu))


def rel(x, ref):
    return float(np.max(np.abs(np.asarray(x) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def random_state(inp, seed=5, scale=0.3):
    rng = np.random.default_rng(seed)
    return scale * rng.standard_normal((inp.n_seqs, inp.heads, inp.dk, inp.dv))


def random_hist(inp, seed=6):
    rng = np.random.default_rng(seed)
    x = (0.25 * rng.standard_normal((inp.n_seqs, inp.heads, 3, inp.dk))).astype(np.float32)
    return f32_to_bf16_bits(x) if inp.dtype == "bf16" else x


def pieces(inp, cut):
    """Split every sequence at min(cut, len): (first pieces, second pieces)."""
    cu = inp.cu_seqlens
    lo_rows, hi_rows, c1, c2 = [], [], [0], [0]
    for n in range(inp.n_seqs):
        a, b = int(cu[n]), int(cu[n + 1])
        m = min(cut, b - a)
        lo_rows.extend(range(a, a + m))
        hi_rows.extend(range(a + m, b))
        c1.append(c1[-1] + m)
        c2.append(c2[-1] + (b - a - m))

    def take(rows, c):
        idx = np.asarray(rows, dtype=np.int64)
        sub = {f: np.ascontiguousarray(getattr(inp, f)[idx]) for f in PER_TOKEN
               if getattr(inp, f) is not None}
        return dataclasses.replace(inp, cu_seqlens=np.asarray(c, dtype=np.int32), **sub)

    return take(lo_rows, c1), take(hi_rows, c2), np.asarray(hi_rows, dtype=np.int64)


def as_storage(inp, x):
    """fp64 values that are exactly representable in the inputs' storage type."""
    x = np.asarray(x, dtype=np.float32)
    return f32_to_bf16_bits(x) if inp.dtype == "bf16" else x


# --------------------------------------------------------------------------- history
def test_history_prepends_rows_to_the_convolution():
    """With b = 0, a = 1, u = 1, L = 2 the write key is the anchor: numpy.convolve
    over the three history rows followed by the sequence (oldest first)."""
    inp = small(L=2, lengths=(9, 1, 2, 0, 5))
    inp.b[:] = 0
    inp.a[:] = 1
    inp.u[:] = 1
    hist = random_hist(inp)
    kw = oracle.prologue(inp, k_hist=hist)
    want = refs.anchor_convolve(inp.k, inp.conv_w, inp.cu_seqlens, hist)
    assert rel(kw, want) < 1e-14
    # and the history changes only the first three tokens of each sequence
    kw0 = oracle.prologue(inp)
    cu = inp.cu_seqlens
    for n in range(inp.n_seqs):
        lo, hi = int(cu[n]), int(cu[n + 1])
        assert np.array_equal(kw[lo + 3:hi], kw0[lo + 3:hi])


def test_history_one_token_closed_form():
    """One token with a history: r_0 = w3 k_t + w2 hist[2] + w1 hist[1] + w0 hist[0]."""
    inp = small(L=2, lengths=(1,))
    inp.b[:] = 0
    inp.a[:] = 1
    inp.u[:] = 1
    hist = random_hist(inp).astype(np.float64)
    w = inp.conv_w.astype(np.float64)
    want = w[None, :, :, 3] * inp.k.astype(np.float64)
    for m in range(3):
        want = want + w[None, :, :, m] * hist[:, :, m]
    kw = oracle.prologue(inp, k_hist=random_hist(inp))
    assert rel(kw, want) < 1e-15


def test_history_full_write_key():
    """Every level of the write key sees the history through the anchor only."""
    inp = small(L=5, lengths=(4, 1, 7))
    hist = random_hist(inp)
    assert rel(oracle.prologue(inp, k_hist=hist), refs.write_key_iterative(inp, hist)) < 1e-13


def test_k_history_is_last_three_rows():
    """The carried history is the last three k rows of each sequence, with the
    incoming history filling in for sequences shorter than three tokens."""
    inp = small(lengths=(6, 2, 1, 0, 3))
    hist = random_hist(inp)
    out = oracle.k_history(inp, hist)
    k, h = inp.k.astype(np.float64), hist.astype(np.float64)
    cu = inp.cu_seqlens
    for n in range(inp.n_seqs):
        lo, hi = int(cu[n]), int(cu[n + 1])
        rows = np.concatenate([h[n].transpose(1, 0, 2), k[lo:hi]], axis=0)[-3:]   # [3, H, dk]
        assert np.array_equal(out[n], rows.transpose(1, 0, 2))
    assert not oracle.k_history(inp)[3].any()          # empty sequence, no history: zero


# --------------------------------------------------------------------------- initial state
def test_initial_state_L1_is_gated_deltanet():
    """L = 1 from a given state equals GDN in prediction-error form from that state."""
    inp = small(L=1, dk=16, dv=16)
    S0 = random_state(inp)
    o, s = oracle.fwd(inp, S_init=S0)
    o2, s2 = refs.gdn_delta_form(inp, S0)
    assert rel(o, o2) < 1e-12 and rel(s, s2) < 1e-12


def test_initial_state_linear_attention():
    """g = 1, b = 0: o_t = S_init^T q_t + causal linear attention, S_T = S_init + sum kw v^T."""
    inp = small(L=3, lengths=(20, 3, 1))
    inp.g[:] = 1
    inp.b[:] = 0
    S0 = random_state(inp)
    hist = random_hist(inp)
    kw = refs.write_key_iterative(inp, hist)
    o, s = oracle.fwd(inp, S_init=S0, k_hist=hist)
    o2 = refs.linear_attention_bruteforce(inp.q, kw, inp.v, inp.cu_seqlens)
    cu = inp.cu_seqlens
    q, v = inp.q.astype(np.float64), inp.v.astype(np.float64)
    for n in range(inp.n_seqs):
        lo, hi = int(cu[n]), int(cu[n + 1])
        for e in range(inp.heads):
            o2[lo:hi, e] += q[lo:hi, e] @ S0[n, e]
            want = S0[n, e] + kw[lo:hi, e].T @ v[lo:hi, e]
            assert np.max(np.abs(s[n, e] - want)) <= 1e-12 * np.max(np.abs(want))
    assert rel(o, o2) < 1e-12


@pytest.mark.parametrize("C", [16, 64])
def test_initial_state_chunkwise_ut(C):
    """The dense chunkwise (WY/UT) form started from S_init equals the recurrence."""
    inp = small(L=4, lengths=(90, 64, 1, 17))
    S0 = random_state(inp)
    hist = random_hist(inp)
    o, s = oracle.fwd(inp, S_init=S0, k_hist=hist)
    o2, s2 = refs.chunkwise_ut(inp, refs.write_key_iterative(inp, hist), C, S0)
    assert rel(o, o2) < 1e-12 and rel(s, s2) < 1e-12


def test_empty_sequence_passes_state_through():
    inp = small(lengths=(0, 4, 0))
    S0 = random_state(inp)
    _, s = oracle.fwd(inp, S_init=S0)
    assert np.array_equal(s[0], S0[0]) and np.array_equal(s[2], S0[2])


# --------------------------------------------------------------------------- resume
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cut", [0, 1, 2, 3, 5, 64, 1000])
def test_resume_equals_one_call(dtype, cut):
    """Processing each sequence in two pieces, carrying S_final and the last three
    k rows from the first piece into the second, reproduces one call over the
    whole sequence (zero start state and history, pinned independently)."""
    inp = small(L=4, lengths=(70, 1, 2, 3, 6, 0), dtype=dtype)
    o, s = oracle.fwd(inp)
    first, second, rows = pieces(inp, cut)
    o1, s1 = oracle.fwd(first)
    hist = as_storage(inp, oracle.k_history(first))
    o2, s2 = oracle.fwd(second, S_init=s1, k_hist=hist)
    assert rel(o2, o[rows]) < 1e-12 if rows.size else True
    assert rel(s2, s) < 1e-12


def test_decode_steps_equal_one_call():
    """Running every sequence token by token through decode_step (state and
    history carried from each step to the next) reproduces one call."""
    inp = small(L=3, lengths=(9, 9, 9), dtype="bf16")
    o, s = oracle.fwd(inp)
    H, dk, dv = inp.heads, inp.dk, inp.dv
    S = np.zeros((inp.n_seqs, H, dk, dv))
    hist = as_storage(inp, np.zeros((inp.n_seqs, H, 3, dk)))
    cu = inp.cu_seqlens
    for t in range(9):
        rows = cu[:-1] + t
        step = dataclasses.replace(
            inp, cu_seqlens=np.arange(inp.n_seqs + 1, dtype=np.int32),
            **{f: np.ascontiguousarray(getattr(inp, f)[rows]) for f in PER_TOKEN})
        ot, S, h64 = oracle.decode_step(step, S, hist)
        hist = as_storage(inp, h64)
        assert rel(ot, o[rows]) < 1e-12
    assert rel(S, s) < 1e-12


def test_decode_step_rejects_multi_token_sequences():
    inp = small(lengths=(2, 1))
    with pytest.raises(ValueError):
        oracle.decode_step(inp, np.zeros((2, inp.heads, inp.dk, inp.dv)),
                           np.zeros((2, inp.heads, 3, inp.dk), dtype=np.float32))


def test_planted_history_mistakes_fail():
    """Reversed history slots, or a history offset by one row, change the write key."""
    inp = small(L=2, lengths=(5, 2))
    hist = random_hist(inp)
    kw = oracle.prologue(inp, k_hist=hist)
    rev = np.ascontiguousarray(hist[:, :, ::-1])
    assert rel(oracle.prologue(inp, k_hist=rev), kw) > 1e-3
    shifted = np.ascontiguousarray(np.concatenate([np.zeros_like(hist[:, :, :1]), hist[:, :, :2]], axis=2))
    assert rel(oracle.prologue(inp, k_hist=shifted), kw) > 1e-3
