"""Pins of the oracle's backward pass (closed-form residual chain, and the
non-linear refinement chain r_{l+1} = r_l - a_l GELU(h_l r_l)).

The backward is reverse-mode differentiation of the forward recurrence; it is
checked against (1) central finite differences of the fp64 forward oracle,
input by input, and (2) torch autograd through an independent token-by-token
forward written with torch fp64 CPU operations (not the oracle's code).  The
loss is sum <d_o, o> + <dS_final, S_final> for random d_o, dS_final.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from gated_delta_rule_prologue_amd.configs import Workload
from gated_delta_rule_prologue_amd.inputs import make_inputs

FIELDS = ("q", "k", "v", "u", "g", "b", "a", "h", "conv_w")


def small(L=3, lengths=(6, 1, 4), H=2, dk=4, dv=3, seed=17, g_mu=1.0):
    return make_inputs(Workload("bwd", heads=H, dk=dk, dv=dv, L=L, dtype="f32", seed=seed,
                                lengths=list(lengths), g_mu=g_mu))


def upstream(inp, seed=3):
    rng = np.random.default_rng(seed)
    d_o = rng.standard_normal((inp.total_tokens, inp.heads, inp.dv))
    dsf = rng.standard_normal((inp.n_seqs, inp.heads, inp.dk, inp.dv))
    return d_o, dsf


def loss(inp, d_o, dsf, S_init=None, residual="linear"):
    o, s = oracle.fwd(inp, S_init=S_init, residual=residual)
    return float(np.sum(o * d_o) + np.sum(s * dsf))


@pytest.mark.parametrize("L,residual", [(1, "linear"), (2, "linear"), (4, "linear"),
                                        (3, "gelu"), (4, "gelu")])
def test_backward_matches_finite_differences(L, residual):
    """Every input element, central differences with steps of 2^-10 (exact in
    fp32 for these magnitudes), against the fp64 forward."""
    inp = small(L=L)
    d_o, dsf = upstream(inp)
    rng = np.random.default_rng(8)
    S0 = 0.3 * rng.standard_normal((inp.n_seqs, inp.heads, inp.dk, inp.dv))
    grads = oracle.bwd(inp, d_o, dS_final=dsf, S_init=S0, residual=residual)
    hstep = 2.0 ** -10
    for name in FIELDS:
        x = getattr(inp, name)
        if x is None:
            continue
        fd = np.zeros(x.shape)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += np.float32(hstep)
            xm[idx] -= np.float32(hstep)
            lp = loss(dataclasses.replace(inp, **{name: xp}), d_o, dsf, S0, residual)
            lm = loss(dataclasses.replace(inp, **{name: xm}), d_o, dsf, S0, residual)
            fd[idx] = (lp - lm) / (2 * hstep)
        err = np.max(np.abs(fd - grads[name])) / max(np.max(np.abs(fd)), 1e-12)
        assert err < 1e-4, (name, err)
    # the start state: the loss is linear in it, so differences are exact
    for idx in list(np.ndindex(S0.shape))[::7]:
        sp, sm = S0.copy(), S0.copy()
        sp[idx] += 0.5
        sm[idx] -= 0.5
        fd = loss(inp, d_o, dsf, sp, residual) - loss(inp, d_o, dsf, sm, residual)
        assert abs(fd - grads["S_init"][idx]) < 1e-9 * max(1.0, abs(fd))


def torch_forward(inp, tensors, S0, residual="linear"):
    """Token-by-token forward in torch fp64 (either chain; torch's exact erf
    GELU), independent of the oracle."""
    import torch
    q, k, v, u, g, b, a, h, w = (tensors[n] for n in FIELDS)
    cu = inp.cu_seqlens
    outs, finals = [], []
    for n in range(inp.n_seqs):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        for e in range(inp.heads):
            S = S0[n, e]
            for t in range(t0, t1):
                r = w[e, :, 3] * k[t, e]
                for m in range(3):
                    tau = t - 3 + m
                    if tau >= t0:
                        r = r + w[e, :, m] * k[tau, e]
                kw = b[t, e] * k[t, e]
                for s in range(inp.L - 1):
                    kw = kw + a[t, e, s] * r * u[t, e, s]
                    if residual == "gelu":
                        r = r - a[t, e, s] * torch.nn.functional.gelu(h[t, e, s] * r)
                    else:
                        r = r * (1 - a[t, e, s] * h[t, e, s])
                p = S.T @ k[t, e]
                S = g[t, e] * (S - b[t, e] * torch.outer(k[t, e], p)) + torch.outer(kw, v[t, e])
                outs.append(((t, e), S.T @ q[t, e]))
            finals.append(((n, e), S))
    return outs, finals


@pytest.mark.parametrize("L,residual", [(1, "linear"), (3, "linear"), (5, "linear"),
                                        (3, "gelu"), (5, "gelu")])
def test_backward_matches_torch_autograd(L, residual):
    torch = pytest.importorskip("torch")
    inp = small(L=L, lengths=(9, 2, 5), dk=5, dv=4)
    d_o, dsf = upstream(inp, seed=5)
    rng = np.random.default_rng(9)
    S0 = 0.2 * rng.standard_normal((inp.n_seqs, inp.heads, inp.dk, inp.dv))
    tensors = {}
    for n in FIELDS:
        x = getattr(inp, n)
        tensors[n] = None if x is None else torch.tensor(x.astype(np.float64), requires_grad=True)
    if L == 1:
        for n in ("u", "a", "h"):
            tensors[n] = torch.zeros((inp.total_tokens, inp.heads, 0, inp.dk), dtype=torch.float64)
    S0t = torch.tensor(S0, requires_grad=True)
    outs, finals = torch_forward(inp, tensors, S0t, residual)
    total = sum((o * torch.tensor(d_o[te])).sum() for te, o in outs)
    total = total + sum((s * torch.tensor(dsf[ne])).sum() for ne, s in finals)
    total.backward()
    grads = oracle.bwd(inp, d_o, dS_final=dsf, S_init=S0, residual=residual)
    for n in FIELDS:
        if getattr(inp, n) is None:
            continue
        gr = tensors[n].grad                     # None: the loss does not depend on it
        ref = np.zeros(getattr(inp, n).shape) if gr is None else gr.numpy()
        err = np.max(np.abs(ref - grads[n])) / max(np.max(np.abs(ref)), 1e-30)
        assert err < 1e-12, (n, err)
    assert np.max(np.abs(S0t.grad.numpy() - grads["S_init"])) < 1e-12 * np.max(np.abs(grads["S_init"]))


def test_backward_chain_subset():
    inp = small(L=3, lengths=(5, 3, 4))
    d_o, dsf = upstream(inp)
    full = oracle.bwd(inp, d_o, dS_final=dsf)
    part = oracle.bwd(inp, d_o, dS_final=dsf, chains=[1, 4])
    for c in (1, 4):
        n, e = divmod(c, inp.heads)
        lo, hi = inp.cu_seqlens[n], inp.cu_seqlens[n + 1]
        for name in ("q", "k", "v", "g", "b"):
            assert np.array_equal(part[name][lo:hi, e], full[name][lo:hi, e])
