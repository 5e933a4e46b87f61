/*
 * prism_oracle.c -- plain fp64 CPU oracle for the forward pass of PRISM's
 * memory-writing operator.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition the GPU kernels are checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header or constant with the GPU library.
 *
 * What it computes (one reading of the pages, fixed once for all code):
 *
 *   Per (sequence n, head e) chain, state S in R^{dk x dv}, S = S_init[n, e]
 *   at the sequence start (zero when no S_init is given).  For every token t
 *   of the sequence, in order:
 *
 *     r_0[i]  = sum_{m=0..3} w[e,i,m] * k[t-3+m, e, i]        causal depthwise
 *               (taps before the sequence start read the       ShortConv, width 4
 *                carried history, zero when none is given)
 *     r_1     = r_0
 *     r_l     = r_0 * prod_{j=1..l-1} (1 - a_j * h_j)          closed-form residual
 *     kw      = b_t k_t + sum_{l=1..L-1} a_l * r_l * u_l        write key
 *     S       = g_t (I - b_t k_t k_t^T) S + kw v_t^T            GDN forget/erase + write
 *     o_t     = S^T q_t
 *
 *   where a_l, h_l, u_l are slot l-1 of the [T, H, L-1, dk] inputs and
 *   "*" is element-wise over the dk channel.  At L = 1 this is exactly the
 *   Gated DeltaNet recurrence.
 *
 *   Non-linear refinement variant (residual = ORACLE_RESIDUAL_GELU): the
 *   residual chain keeps its GELU instead of the closed form,
 *
 *     r_1 = r_0,   r_{l+1} = r_l - a_l * GELU(h_l * r_l),   GELU(x) = x Phi(x),
 *
 *   with the same write key sum.  It reduces to the closed form when GELU is
 *   replaced by the identity, and equals it for L <= 2 (no residual update is
 *   used before the last level).
 *
 * Sources (PRISM pages):
 *   - ICML 2026 PRISM summary (WeChat article), section 核心迭代形式: the
 *     step-size x residual x direction write, sum over L levels.
 *   - same page, section 消除 Token 间串行: forget term kept identical to GDN,
 *     all non-linearity confined to the write; ShortConv local anchor.
 *   - same page, section 消除 Step 间串行: the residual chain becomes an
 *     element-wise linear recurrence with a closed form.
 *   - same page, section 架构形式: first step is the standard GDN write;
 *     L = 1 reduces exactly to GDN.
 *   - gist.science technical summary of arXiv 2602.10796, section 2.1
 *     (S_t = S_{t-1} A_t + B_t with an input-only write) and section 2.2
 *     (ShortConv anchor, refinement steps l = 1..L with r^(1) the anchor,
 *     residual update r^(l+1) = r^(l) - delta^(l), delta^(l) the GELU of the
 *     predicted gain times the residual, a step-size gate per level).
 *   - ICML 2026 poster abstract: a short convolution anchors the initial
 *     residual.
 *   - WeChat page, section 背景：无限背包 vs 有限背包, and the poster page's
 *     lay summary: the whole history lives in a fixed-size state matrix
 *     updated one token at a time (an RNN recurrence), so a sequence can be
 *     processed in pieces by carrying S (and the convolution's last three
 *     inputs) from one piece to the next.
 *
 * Readings where the pages are silent or garbled (all code follows them):
 *   - the product in the residual closed form runs over j = 1..l-1, so the
 *     first refinement level uses the raw anchor; h's last slot is unused;
 *   - conv tap 3 multiplies the current token, taps 0..2 the three before it;
 *     no bias and no activation after the convolution;
 *   - g and b are per (token, head) scalars; g is a linear-space gate;
 *   - no query scaling; the initial state is zero unless S_init is given;
 *   - GELU variant: the gain of the gist page's delta is h_l and the step-size
 *     gate a_l scales the subtracted GELU, so that the linearised chain
 *     (GELU -> identity) is the closed form above; GELU is the exact erf form;
 *   - carried conv history k_hist [n_seqs, H, 3, dk]: slot m holds k at
 *     position (sequence start - 3 + m), i.e. slot 2 is the token just before
 *     the first one; zero when no history is given.
 *
 * Precision: all arithmetic in double.  Inputs are fp32 or bf16 (raw 16-bit
 * patterns) and are widened exactly.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <math.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_RESIDUAL_LINEAR 0
#define ORACLE_RESIDUAL_GELU 1

typedef struct {
    int64_t n_seqs;
    int64_t total_tokens;
    int64_t heads;
    int64_t dk;
    int64_t dv;
    int64_t L;
    int64_t dtype;      /* ORACLE_F32 or ORACLE_BF16 */
    int64_t residual;   /* ORACLE_RESIDUAL_LINEAR or ORACLE_RESIDUAL_GELU */
} oracle_dims;

/* GELU(x) = x * Phi(x), Phi the standard normal CDF, in its erf form. */
static double gelu(double x)
{
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

/* GELU'(x) = Phi(x) + x phi(x), phi the standard normal density. */
static double gelu_prime(double x)
{
    return 0.5 * (1.0 + erf(x / sqrt(2.0))) + x * exp(-0.5 * x * x) / sqrt(2.0 * 3.14159265358979323846);
}

/* Exact widening of element i of an fp32 or bf16 array. */
static double elem(const void* p, int64_t dtype, int64_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float*)p)[i];
    uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* k at position tau, channel i, of sequence n (first token seq_start), head e:
 * the token's own row, or the carried history before the sequence start. */
static double k_at(const oracle_dims* d, const void* k, const void* k_hist, int64_t n,
                   int64_t seq_start, int64_t tau, int64_t e, int64_t i)
{
    const int64_t H = d->heads, dk = d->dk;
    if (tau >= seq_start)
        return elem(k, d->dtype, (tau * H + e) * dk + i);
    if (!k_hist || tau < seq_start - 3)
        return 0.0;
    return elem(k_hist, d->dtype, ((n * H + e) * 3 + (tau - seq_start + 3)) * dk + i);
}

/* Write key of token t, head e into kw[0..dk).  t belongs to sequence n, whose
 * first token is seq_start (conv taps before it read the carried history, or
 * zero without one). */
static void write_key(const oracle_dims* d, const void* k, const void* u, const void* a,
                      const void* h, const void* b, const void* conv_w, const void* k_hist,
                      int64_t n, int64_t seq_start, int64_t t, int64_t e, double* kw)
{
    const int64_t H = d->heads, dk = d->dk, L = d->L, dt = d->dtype;
    const double bt = elem(b, dt, t * H + e);
    for (int64_t i = 0; i < dk; ++i) {
        /* r_0: causal depthwise convolution over k along the token axis. */
        double r0 = 0.0;
        for (int64_t m = 0; m < 4; ++m) {
            r0 += elem(conv_w, dt, (e * dk + i) * 4 + m) *
                  k_at(d, k, k_hist, n, seq_start, t - 3 + m, e, i);
        }
        double acc = bt * elem(k, dt, (t * H + e) * dk + i);
        if (d->residual == ORACLE_RESIDUAL_GELU) {
            /* r_{l+1} = r_l - a_l GELU(h_l r_l), level by level */
            double r = r0;
            for (int64_t l = 1; l <= L - 1; ++l) {
                int64_t sl = ((t * H + e) * (L - 1) + (l - 1)) * dk + i;
                acc += elem(a, dt, sl) * r * elem(u, dt, sl);
                if (l <= L - 2)
                    r -= elem(a, dt, sl) * gelu(elem(h, dt, sl) * r);
            }
            kw[i] = acc;
            continue;
        }
        for (int64_t l = 1; l <= L - 1; ++l) {
            /* closed form r_l = r_0 * prod_{j=1..l-1} (1 - a_j h_j) */
            double prod = 1.0;
            for (int64_t j = 1; j <= l - 1; ++j) {
                int64_t sj = ((t * H + e) * (L - 1) + (j - 1)) * dk + i;
                prod *= 1.0 - elem(a, dt, sj) * elem(h, dt, sj);
            }
            int64_t sl = ((t * H + e) * (L - 1) + (l - 1)) * dk + i;
            acc += elem(a, dt, sl) * (r0 * prod) * elem(u, dt, sl);
        }
        kw[i] = acc;
    }
}

/* kw for every token and head: out[T, H, dk] (double).  k_hist may be NULL. */
int prism_oracle_prologue(const oracle_dims* d, const int32_t* cu_seqlens,
                          const void* k, const void* u, const void* a, const void* h,
                          const void* b, const void* conv_w, const void* k_hist,
                          double* kw_out, int nthreads)
{
    if (!d || !cu_seqlens || !k || !b || !conv_w || !kw_out || d->L < 1)
        return 1;
    if (d->L > 1 && (!u || !a || !h))
        return 1;
    const int64_t H = d->heads, dk = d->dk;
    int64_t n_items = d->n_seqs * H;
    (void)nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t item = 0; item < n_items; ++item) {
        int64_t n = item / H, e = item % H;
        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t)
            write_key(d, k, u, a, h, b, conv_w, k_hist, n, cu_seqlens[n], t, e,
                      kw_out + (t * H + e) * dk);
    }
    return 0;
}

/*
 * Full forward.  chains: optional list of (sequence * heads + head) indices to
 * evaluate (NULL = all).  Only the selected chains' rows of o_out [T, H, dv]
 * and blocks of s_out [n_seqs, H, dk, dv] are written.  s_init
 * [n_seqs, H, dk, dv] and k_hist [n_seqs, H, 3, dk] (input dtype) may be NULL
 * (zero state, zero history).
 */
int prism_oracle_fwd(const oracle_dims* d, const int32_t* cu_seqlens,
                     const void* q, const void* k, const void* v, const void* u,
                     const void* g, const void* b, const void* a, const void* h,
                     const void* conv_w, const double* s_init, const void* k_hist,
                     const int64_t* chains, int64_t n_chains,
                     double* o_out, double* s_out, int nthreads)
{
    if (!d || !cu_seqlens || !q || !k || !v || !g || !b || !conv_w || !o_out || !s_out || d->L < 1)
        return 1;
    if (d->L > 1 && (!u || !a || !h))
        return 1;
    const int64_t H = d->heads, dk = d->dk, dv = d->dv, dt = d->dtype;
    const int64_t n_items = chains ? n_chains : d->n_seqs * H;
    int status = 0;
    (void)nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t item = 0; item < n_items; ++item) {
        int64_t c = chains ? chains[item] : item;
        int64_t n = c / H, e = c % H;
        double* S = (double*)calloc((size_t)(dk * dv), sizeof(double));
        double* kw = (double*)malloc((size_t)dk * sizeof(double));
        double* kt = (double*)malloc((size_t)dk * sizeof(double));
        double* p = (double*)malloc((size_t)dv * sizeof(double));
        double* qt = (double*)malloc((size_t)dk * sizeof(double));
        double* vt = (double*)malloc((size_t)dv * sizeof(double));
        if (!S || !kw || !kt || !p || !qt || !vt) {
#pragma omp atomic write
            status = 2;
            free(S); free(kw); free(kt); free(p); free(qt); free(vt);
            continue;
        }
        if (s_init)
            memcpy(S, s_init + c * dk * dv, (size_t)(dk * dv) * sizeof(double));
        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            write_key(d, k, u, a, h, b, conv_w, k_hist, n, cu_seqlens[n], t, e, kw);
            const double gt = elem(g, dt, t * H + e);
            const double bt = elem(b, dt, t * H + e);
            for (int64_t i = 0; i < dk; ++i) {
                kt[i] = elem(k, dt, (t * H + e) * dk + i);
                qt[i] = elem(q, dt, (t * H + e) * dk + i);
            }
            for (int64_t j = 0; j < dv; ++j)
                vt[j] = elem(v, dt, (t * H + e) * dv + j);
            /* p = S^T k_t, so (I - b k k^T) S = S - b k p^T */
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk; ++i)
                    acc += S[i * dv + j] * kt[i];
                p[j] = acc;
            }
            /* S = g (S - b k p^T) + kw v^T */
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j)
                    S[i * dv + j] = gt * (S[i * dv + j] - bt * kt[i] * p[j]) + kw[i] * vt[j];
            /* o_t = S^T q_t */
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk; ++i)
                    acc += S[i * dv + j] * qt[i];
                o_out[(t * H + e) * dv + j] = acc;
            }
        }
        memcpy(s_out + c * dk * dv, S, (size_t)(dk * dv) * sizeof(double));
        free(S); free(kw); free(kt); free(p); free(qt); free(vt);
    }
    return status;
}

/*
 * The convolution history to carry into the next piece of each sequence:
 * out[n, e, m, :] = k at position (sequence end - 3 + m), taken from the
 * carried history k_hist (may be NULL: zero) where that position lies before
 * the sequence start.  out is [n_seqs, H, 3, dk] (double).
 */
int prism_oracle_k_history(const oracle_dims* d, const int32_t* cu_seqlens, const void* k,
                           const void* k_hist, double* out)
{
    if (!d || !cu_seqlens || !out || (d->total_tokens > 0 && !k))
        return 1;
    const int64_t H = d->heads, dk = d->dk;
    for (int64_t n = 0; n < d->n_seqs; ++n)
        for (int64_t e = 0; e < H; ++e)
            for (int64_t m = 0; m < 3; ++m)
                for (int64_t i = 0; i < dk; ++i)
                    out[((n * H + e) * 3 + m) * dk + i] =
                        k_at(d, k, k_hist, n, cu_seqlens[n], cu_seqlens[n + 1] - 3 + m, e, i);
    return 0;
}

/*
 * Backward pass of the forward above (either residual chain, L >= 1), for
 * the loss  sum_t <do_t, o_t> + <dS_final, S_final>  of given upstream
 * gradients.  Reverse-mode differentiation of the token recurrence, written
 * out step by step:
 *
 *   G <- dS_final (or 0);  for t = last .. first of the sequence:
 *     G     += q_t do_t^T                       (o_t = S_t^T q_t)
 *     dq_t   = S_t do_t,  dv_t = G^T kw_t,  dkw_t = G v_t
 *     P      = S_{t-1} - b_t k_t p^T,  p = S_{t-1}^T k_t
 *     dg_t   = <G, P>,  dP = g_t G,  y = dP^T k_t
 *     db_t  += -(y . p),  dk_t += -b_t (dP p + S_{t-1} y)
 *     G      = dP - b_t k_t y^T                 (S_t = g_t P + kw_t v_t^T)
 *   dS_init = G
 *
 * then through the write key kw_t = b_t k_t + sum_l a_l r_l u_l with
 * r_{l+1} = r_l (1 - a_l h_l), r_1 = r_0 = sum_m w_m k_{t-3+m}: the residual
 * chain in reverse (dr_l = dkw a_l u_l + dr_{l+1} (1 - a_l h_l)); with the
 * GELU chain r_{l+1} = r_l - a_l GELU(h_l r_l) the factor (1 - a_l h_l)
 * becomes 1 - a_l h_l GELU'(h_l r_l), da_l takes -dr_{l+1} GELU(h_l r_l) and
 * dh_l = -dr_{l+1} a_l r_l GELU'(h_l r_l); then the convolution (dw_m += dr_0 k_{t-3+m}, dk_{t-3+m} += w_m dr_0 inside the
 * sequence).  Taps that read a carried history contribute to no input
 * gradient here.  All outputs are double; chains, when given, restrict the
 * evaluation like prism_oracle_fwd (dconv_w then sums over those chains only).
 * The per-chain states are kept in full, so this is for small inputs or a few
 * chains.
 */
int prism_oracle_bwd(const oracle_dims* d, const int32_t* cu_seqlens,
                     const void* q, const void* k, const void* v, const void* u,
                     const void* g, const void* b, const void* a, const void* h,
                     const void* conv_w, const double* s_init, const double* d_o,
                     const double* d_sfinal, const int64_t* chains, int64_t n_chains,
                     double* dq, double* dk, double* dv, double* du, double* dg, double* db,
                     double* da, double* dh, double* dconv_w, double* ds_init, int nthreads)
{
    if (!d || !cu_seqlens || !q || !k || !v || !g || !b || !conv_w || !d_o || !dq || !dk ||
        !dv || !dg || !db || !dconv_w || d->L < 1 ||
        (d->residual != ORACLE_RESIDUAL_LINEAR && d->residual != ORACLE_RESIDUAL_GELU))
        return 1;
    if (d->L > 1 && (!u || !a || !h || !du || !da || !dh))
        return 1;
    const int64_t H = d->heads, dk_ = d->dk, dv_ = d->dv, dt = d->dtype, L = d->L;
    const int64_t n_items = chains ? n_chains : d->n_seqs * H;
    int status = 0;
    (void)nthreads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t item = 0; item < n_items; ++item) {
        const int64_t c = chains ? chains[item] : item;
        const int64_t n = c / H, e = c % H;
        const int64_t t0 = cu_seqlens[n], len = cu_seqlens[n + 1] - cu_seqlens[n];
        const int64_t SZ = dk_ * dv_;
        double* Ss = (double*)calloc((size_t)((len + 1) * SZ), sizeof(double));
        double* kw = (double*)malloc((size_t)((len > 0 ? len : 1) * dk_) * sizeof(double));
        double* dkw = (double*)calloc((size_t)((len > 0 ? len : 1) * dk_), sizeof(double));
        double* G = (double*)calloc((size_t)SZ, sizeof(double));
        double* P = (double*)malloc((size_t)SZ * sizeof(double));
        double* p = (double*)malloc((size_t)dv_ * sizeof(double));
        double* y = (double*)malloc((size_t)dv_ * sizeof(double));
        double* r = (double*)malloc((size_t)(L > 1 ? L : 2) * sizeof(double));
        double* dwc = (double*)calloc((size_t)(dk_ * 4), sizeof(double));
        if (!Ss || !kw || !dkw || !G || !P || !p || !y || !r || !dwc) {
#pragma omp atomic write
            status = 2;
            free(Ss); free(kw); free(dkw); free(G); free(P); free(p); free(y); free(r); free(dwc);
            continue;
        }
        if (s_init)
            memcpy(Ss, s_init + c * SZ, (size_t)SZ * sizeof(double));
        /* forward: S_{t} at Ss[(t - t0 + 1) SZ] */
        for (int64_t j = 0; j < len; ++j) {
            const int64_t t = t0 + j;
            write_key(d, k, u, a, h, b, conv_w, NULL, n, t0, t, e, kw + j * dk_);
            const double gt = elem(g, dt, t * H + e), bt = elem(b, dt, t * H + e);
            const double* S0 = Ss + j * SZ;
            double* S1 = Ss + (j + 1) * SZ;
            for (int64_t jj = 0; jj < dv_; ++jj) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk_; ++i)
                    acc += S0[i * dv_ + jj] * elem(k, dt, (t * H + e) * dk_ + i);
                p[jj] = acc;
            }
            for (int64_t i = 0; i < dk_; ++i) {
                const double ki = elem(k, dt, (t * H + e) * dk_ + i);
                for (int64_t jj = 0; jj < dv_; ++jj)
                    S1[i * dv_ + jj] = gt * (S0[i * dv_ + jj] - bt * ki * p[jj]) +
                                       kw[j * dk_ + i] * elem(v, dt, (t * H + e) * dv_ + jj);
            }
        }
        /* reverse through the state recurrence */
        if (d_sfinal)
            memcpy(G, d_sfinal + c * SZ, (size_t)SZ * sizeof(double));
        for (int64_t j = len - 1; j >= 0; --j) {
            const int64_t t = t0 + j;
            const double gt = elem(g, dt, t * H + e), bt = elem(b, dt, t * H + e);
            const double* Sm = Ss + j * SZ;           /* S_{t-1} */
            const double* St = Ss + (j + 1) * SZ;     /* S_t */
            const double* dot = d_o + (t * H + e) * dv_;
            for (int64_t i = 0; i < dk_; ++i) {
                const double qi = elem(q, dt, (t * H + e) * dk_ + i);
                for (int64_t jj = 0; jj < dv_; ++jj)
                    G[i * dv_ + jj] += qi * dot[jj];
            }
            for (int64_t i = 0; i < dk_; ++i) {
                double aq = 0.0, aw = 0.0;
                for (int64_t jj = 0; jj < dv_; ++jj) {
                    aq += St[i * dv_ + jj] * dot[jj];
                    aw += G[i * dv_ + jj] * elem(v, dt, (t * H + e) * dv_ + jj);
                }
                dq[(t * H + e) * dk_ + i] = aq;
                dkw[j * dk_ + i] = aw;
            }
            for (int64_t jj = 0; jj < dv_; ++jj) {
                double acc = 0.0, pk = 0.0;
                for (int64_t i = 0; i < dk_; ++i) {
                    acc += G[i * dv_ + jj] * kw[j * dk_ + i];
                    pk += Sm[i * dv_ + jj] * elem(k, dt, (t * H + e) * dk_ + i);
                }
                dv[(t * H + e) * dv_ + jj] = acc;
                p[jj] = pk;
            }
            double dgt = 0.0;
            for (int64_t i = 0; i < dk_; ++i) {
                const double ki = elem(k, dt, (t * H + e) * dk_ + i);
                for (int64_t jj = 0; jj < dv_; ++jj) {
                    P[i * dv_ + jj] = Sm[i * dv_ + jj] - bt * ki * p[jj];
                    dgt += G[i * dv_ + jj] * P[i * dv_ + jj];
                }
            }
            dg[t * H + e] = dgt;
            /* dP = g G (in place), y = dP^T k */
            for (int64_t x = 0; x < SZ; ++x)
                G[x] *= gt;
            for (int64_t jj = 0; jj < dv_; ++jj) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk_; ++i)
                    acc += G[i * dv_ + jj] * elem(k, dt, (t * H + e) * dk_ + i);
                y[jj] = acc;
            }
            double yp = 0.0;
            for (int64_t jj = 0; jj < dv_; ++jj)
                yp += y[jj] * p[jj];
            db[t * H + e] = -yp;
            for (int64_t i = 0; i < dk_; ++i) {
                double a1 = 0.0, a2 = 0.0;
                for (int64_t jj = 0; jj < dv_; ++jj) {
                    a1 += G[i * dv_ + jj] * p[jj];
                    a2 += Sm[i * dv_ + jj] * y[jj];
                }
                dk[(t * H + e) * dk_ + i] = -bt * (a1 + a2);
            }
            for (int64_t i = 0; i < dk_; ++i) {
                const double ki = elem(k, dt, (t * H + e) * dk_ + i);
                for (int64_t jj = 0; jj < dv_; ++jj)
                    G[i * dv_ + jj] -= bt * ki * y[jj];
            }
        }
        if (ds_init)
            memcpy(ds_init + c * SZ, G, (size_t)SZ * sizeof(double));
        /* through the write key, token by token (the conv spreads over 4 tokens,
         * so dk of earlier tokens is accumulated here after their own rows) */
        for (int64_t j = 0; j < len; ++j) {
            const int64_t t = t0 + j;
            const double bt = elem(b, dt, t * H + e);
            for (int64_t i = 0; i < dk_; ++i) {
                const double kt = elem(k, dt, (t * H + e) * dk_ + i);
                const double dkwi = dkw[j * dk_ + i];
                db[t * H + e] += dkwi * kt;
                dk[(t * H + e) * dk_ + i] += bt * dkwi;
                if (L == 1)
                    continue;
                double r0 = 0.0;
                for (int64_t m = 0; m < 4; ++m)
                    r0 += elem(conv_w, dt, (e * dk_ + i) * 4 + m) *
                          k_at(d, k, NULL, n, t0, t - 3 + m, e, i);
                /* r[l] for l = 1 .. L-1 */
                const int gel = d->residual == ORACLE_RESIDUAL_GELU;
                r[1] = r0;
                for (int64_t l = 1; l < L - 1; ++l) {
                    const int64_t sl = ((t * H + e) * (L - 1) + (l - 1)) * dk_ + i;
                    const double al = elem(a, dt, sl), hl = elem(h, dt, sl);
                    r[l + 1] = gel ? r[l] - al * gelu(hl * r[l]) : r[l] * (1.0 - al * hl);
                }
                double dr_next = 0.0;                  /* dr_{l+1} */
                for (int64_t l = L - 1; l >= 1; --l) {
                    const int64_t sl = ((t * H + e) * (L - 1) + (l - 1)) * dk_ + i;
                    const double al = elem(a, dt, sl), ul = elem(u, dt, sl), hl = elem(h, dt, sl);
                    du[sl] = dkwi * al * r[l];
                    double dal = dkwi * ul * r[l];
                    double dhl = 0.0, drl = dkwi * al * ul;
                    if (l <= L - 2) {
                        if (gel) {                     /* r_{l+1} = r_l - a_l GELU(h_l r_l) */
                            const double x = hl * r[l], gp = gelu_prime(x);
                            dal -= dr_next * gelu(x);
                            dhl = -dr_next * al * r[l] * gp;
                            drl += dr_next * (1.0 - al * hl * gp);
                        } else {                       /* r_{l+1} = r_l (1 - a_l h_l) */
                            dal -= dr_next * hl * r[l];
                            dhl = -dr_next * al * r[l];
                            drl += dr_next * (1.0 - al * hl);
                        }
                    }
                    da[sl] = dal;
                    dh[sl] = dhl;
                    dr_next = drl;
                }
                /* dr_next is now dr_1 = dr_0 */
                for (int64_t m = 0; m < 4; ++m) {
                    const int64_t tau = t - 3 + m;
                    if (tau < t0)
                        continue;
                    dwc[i * 4 + m] += dr_next * elem(k, dt, (tau * H + e) * dk_ + i);
                    dk[(tau * H + e) * dk_ + i] += elem(conv_w, dt, (e * dk_ + i) * 4 + m) * dr_next;
                }
            }
        }
#pragma omp critical
        for (int64_t x = 0; x < dk_ * 4; ++x)
            dconv_w[e * dk_ * 4 + x] += dwc[x];
        free(Ss); free(kw); free(dkw); free(G); free(P); free(p); free(y); free(r); free(dwc);
    }
    return status;
}
