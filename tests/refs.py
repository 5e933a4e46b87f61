"""Independent numpy / exact-rational references used to pin the fp64 oracle.

Each function below reaches the operator's result by a route other than the
oracle's token-by-token recurrence, so that a dropped term, a wrong sign, a
wrong index or a transposed operand in the oracle disagrees with at least one
of them.  None of them is used by the GPU library.

Sources are the PRISM pages:
  * ICML 2026 PRISM summary (WeChat article), sections 核心迭代形式,
    消除 Token 间串行, 消除 Step 间串行 and 架构形式;
  * gist.science technical summary of arXiv 2602.10796, sections 2.1-2.2;
  * the linear-attention ancestor cited on the WeChat page (Katharopoulos et
    al., reference [3]) for the g = 1, b = 0 special case.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def f64(x):
    from gated_delta_rule_prologue_amd.inputs import to_float
    return None if x is None else to_float(x).astype(np.float64)


# ---------------------------------------------------------------------------
# write branch
# ---------------------------------------------------------------------------
def anchor_convolve(k, conv_w, cu, hist=None):
    """ShortConv anchor r_0 by numpy.convolve, one channel and sequence at a time.

    ``np.convolve(x, w[::-1])[n] = sum_m w[m] x[n - 3 + m]`` with x read as
    zero before the sequence start: the causal width-4 depthwise convolution.
    With ``hist`` [n_seqs, H, 3, dk], the three rows before each sequence are
    prepended to it (oldest first) and the first three outputs dropped.
    """
    k = f64(k)
    w = f64(conv_w)
    hist = f64(hist)
    T, H, dk = k.shape
    r0 = np.zeros_like(k)
    for n in range(len(cu) - 1):
        lo, hi = int(cu[n]), int(cu[n + 1])
        if hi == lo:
            continue
        for e in range(H):
            for i in range(dk):
                x = k[lo:hi, e, i]
                if hist is not None:
                    x = np.concatenate([hist[n, e, :, i], x])
                full = np.convolve(x, w[e, i, ::-1])[: len(x)]
                r0[lo:hi, e, i] = full[len(x) - (hi - lo):]
    return r0


def write_key_iterative(inp, hist=None):
    """kw by running the residual chain as repeated subtraction.

    Linearised refinement step of the gist.science summary, section 2.2:
    r^(l+1) = r^(l) - delta^(l) with delta^(l) = (a_l * h_l) * r^(l) (the
    GELU absorbed, WeChat page section 消除 Step 间串行), starting from the
    anchor r^(1) = r_0; level l contributes a_l * r^(l) * u_l to the key.
    """
    k = f64(inp.k)
    b = f64(inp.b)
    kw = b[:, :, None] * k
    if inp.L == 1:
        return kw
    r = anchor_convolve(inp.k, inp.conv_w, inp.cu_seqlens, hist)
    a, h, u = f64(inp.a), f64(inp.h), f64(inp.u)
    for s in range(inp.L - 1):
        kw = kw + a[:, :, s] * r * u[:, :, s]
        r = r - (a[:, :, s] * h[:, :, s]) * r
    return kw


def gelu_cdf(x):
    """GELU(x) = x Phi(x) with Phi from scipy's normal distribution."""
    from scipy.stats import norm
    return x * norm.cdf(x)


def write_key_gelu(inp, hist=None):
    """kw with the non-linear refinement chain of the gist.science summary,
    section 2.2: r^(1) = anchor, r^(l+1) = r^(l) - a_l * GELU(h_l * r^(l)); level
    l contributes a_l * r^(l) * u_l to the key."""
    k = f64(inp.k)
    b = f64(inp.b)
    kw = b[:, :, None] * k
    if inp.L == 1:
        return kw
    r = anchor_convolve(inp.k, inp.conv_w, inp.cu_seqlens, hist)
    a, h, u = f64(inp.a), f64(inp.h), f64(inp.u)
    for s in range(inp.L - 1):
        kw = kw + a[:, :, s] * r * u[:, :, s]
        r = r - a[:, :, s] * gelu_cdf(h[:, :, s] * r)
    return kw


# ---------------------------------------------------------------------------
# state recurrence
# ---------------------------------------------------------------------------
def gdn_delta_form(inp, S0=None):
    """L = 1 reference: Gated DeltaNet in prediction-error form.

    S <- g S + b k (v - g S^T k)^T, o = S^T q.  Algebraically equal to
    g (I - b k k^T) S + b k v^T but evaluated differently.  ``S0``
    [n_seqs, H, dk, dv]: start states (zero by default).
    """
    q, k, v, g, b = (f64(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.b))
    T, H, dk = k.shape
    dv = v.shape[2]
    cu = inp.cu_seqlens
    o = np.zeros((T, H, dv))
    S_fin = np.zeros((len(cu) - 1, H, dk, dv))
    for n in range(len(cu) - 1):
        for e in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[n, e], dtype=np.float64)
            for t in range(int(cu[n]), int(cu[n + 1])):
                pred = g[t, e] * (S.T @ k[t, e])
                S = g[t, e] * S + b[t, e] * np.outer(k[t, e], v[t, e] - pred)
                o[t, e] = S.T @ q[t, e]
            S_fin[n, e] = S
    return o, S_fin


def linear_attention_bruteforce(q, kw, v, cu):
    """g = 1, b = 0: causal linear attention, o_t = sum_{s<=t} (q_t . kw_s) v_s, by O(T^2) sums."""
    q, v = f64(q), f64(v)
    T, H, dv = v.shape
    o = np.zeros((T, H, dv))
    for n in range(len(cu) - 1):
        lo, hi = int(cu[n]), int(cu[n + 1])
        for e in range(H):
            for t in range(lo, hi):
                acc = np.zeros(dv)
                for s in range(lo, t + 1):
                    acc += float(np.dot(q[t, e], kw[s, e])) * v[s, e]
                o[t, e] = acc
    return o


def chunkwise_ut(inp, kw, C, S0=None):
    """Dense chunkwise (WY/UT) evaluation of the recurrence, chunk size C.

    Inside a chunk with incoming state S0, cumulative log-gates lam and
    gamma = exp(lam), decay matrix D[t, s] = exp(lam_t - lam_s) (s <= t):
      X     = (I + B (D . tril_-1(K K^T)))^{-1} (B Gamma K S0 + B (D . tril_-1(K KW^T)) V)
      O     = Gamma Q S0 + (D . tril_0(Q KW^T)) V - (D . tril_0(Q K^T)) X
      S_out = gamma_n S0 + (diag(gamma_n/gamma) KW)^T V - (diag(gamma_n/gamma) K)^T X
    X holds the per-token erase rows w_t = g_t b_t S_{t-1}^T k_t.
    """
    q, k, v, g, b = (f64(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.b))
    T, H, dk = k.shape
    dv = v.shape[2]
    cu = inp.cu_seqlens
    o = np.zeros((T, H, dv))
    S_fin = np.zeros((len(cu) - 1, H, dk, dv))
    for n in range(len(cu) - 1):
        for e in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[n, e], dtype=np.float64)
            for c0 in range(int(cu[n]), int(cu[n + 1]), C):
                c1 = min(c0 + C, int(cu[n + 1]))
                m = c1 - c0
                Q, K, KW, V = q[c0:c1, e], k[c0:c1, e], kw[c0:c1, e], v[c0:c1, e]
                B = b[c0:c1, e]
                lam = np.cumsum(np.log(g[c0:c1, e]))
                gam = np.exp(lam)
                diff = lam[:, None] - lam[None, :]
                low0 = np.tril(np.ones((m, m), dtype=bool))
                low1 = np.tril(np.ones((m, m), dtype=bool), -1)
                D = np.where(low0, np.exp(np.where(low0, diff, 0.0)), 0.0)
                A_kk = B[:, None] * np.where(low1, D * (K @ K.T), 0.0)
                A_kkw = B[:, None] * np.where(low1, D * (K @ KW.T), 0.0)
                Tm = np.linalg.inv(np.eye(m) + A_kk)
                X = Tm @ ((B * gam)[:, None] * (K @ S) + A_kkw @ V)
                O = gam[:, None] * (Q @ S) + np.where(low0, D * (Q @ KW.T), 0.0) @ V \
                    - np.where(low0, D * (Q @ K.T), 0.0) @ X
                tail = gam[-1] / gam
                S = gam[-1] * S + (tail[:, None] * KW).T @ V - (tail[:, None] * K).T @ X
                o[c0:c1, e] = O
            S_fin[n, e] = S
    return o, S_fin


# ---------------------------------------------------------------------------
# exact rational brute force (tiny inputs only)
# ---------------------------------------------------------------------------
def _F(x):
    return Fraction(float(x))


def transition_products_exact(inp, kw):
    """Exact-rational evaluation through explicit transition matrices.

    A_t = g_t (I - b_t k_t k_t^T) as a dense dk x dk matrix, and
    S_t = sum_{s<=t} (A_t A_{t-1} ... A_{s+1}) kw_s v_s^T,  o_t = S_t^T q_t,
    i.e. the unrolled linear recurrence S_t = A_t S_{t-1} + B_t of the
    gist.science summary, section 2.1, with B_t = kw_t v_t^T.  ``kw`` must be
    given as exact Fractions (or floats that are converted exactly).
    Pure Python; only for a handful of tokens and channels.
    """
    q, k, v, g, b = (f64(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.b))
    T, H, dk = k.shape
    dv = v.shape[2]
    cu = inp.cu_seqlens

    def matmul(A, B):
        return [[sum(A[i][r] * B[r][j] for r in range(len(B))) for j in range(len(B[0]))]
                for i in range(len(A))]

    o = [[[None] * dv for _ in range(H)] for _ in range(T)]
    S_fin = []
    for n in range(len(cu) - 1):
        lo, hi = int(cu[n]), int(cu[n + 1])
        per_head = []
        for e in range(H):
            A = {}
            for t in range(lo, hi):
                kk = [_F(x) for x in k[t, e]]
                gt, bt = _F(g[t, e]), _F(b[t, e])
                A[t] = [[gt * ((1 if i == j else 0) - bt * kk[i] * kk[j]) for j in range(dk)]
                        for i in range(dk)]
            S = [[Fraction(0)] * dv for _ in range(dk)]
            for t in range(lo, hi):
                S = [[Fraction(0)] * dv for _ in range(dk)]
                for s in range(lo, t + 1):
                    Phi = [[Fraction(1 if i == j else 0) for j in range(dk)] for i in range(dk)]
                    for r in range(t, s, -1):
                        Phi = matmul(Phi, A[r])
                    kws = [kw[s][e][i] if isinstance(kw[s][e][i], Fraction) else _F(kw[s][e][i])
                           for i in range(dk)]
                    vs = [_F(x) for x in v[s, e]]
                    Bs = [[kws[i] * vs[j] for j in range(dv)] for i in range(dk)]
                    PB = matmul(Phi, Bs)
                    S = [[S[i][j] + PB[i][j] for j in range(dv)] for i in range(dk)]
                qt = [_F(x) for x in q[t, e]]
                for j in range(dv):
                    o[t][e][j] = sum(S[i][j] * qt[i] for i in range(dk))
            per_head.append(S)
        S_fin.append(per_head)
    return o, S_fin


def write_key_exact(inp):
    """kw as exact Fractions, residual chain by repeated subtraction (see write_key_iterative)."""
    k, b, w = f64(inp.k), f64(inp.b), f64(inp.conv_w)
    a_, h_, u_ = f64(inp.a), f64(inp.h), f64(inp.u)
    T, H, dk = k.shape
    cu = inp.cu_seqlens
    kw = [[[None] * dk for _ in range(H)] for _ in range(T)]
    for n in range(len(cu) - 1):
        lo, hi = int(cu[n]), int(cu[n + 1])
        for t in range(lo, hi):
            for e in range(H):
                for i in range(dk):
                    r = sum((_F(w[e, i, m]) * _F(k[t - 3 + m, e, i])
                             for m in range(4) if t - 3 + m >= lo), Fraction(0))
                    acc = _F(b[t, e]) * _F(k[t, e, i])
                    for s in range(inp.L - 1):
                        al, hl, ul = _F(a_[t, e, s, i]), _F(h_[t, e, s, i]), _F(u_[t, e, s, i])
                        acc += al * r * ul
                        r = r - al * hl * r
                    kw[t][e][i] = acc
    return kw
