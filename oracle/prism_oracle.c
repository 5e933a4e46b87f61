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
 *   Per (sequence n, head e) chain, state S in R^{dk x dv}, S = 0 at the
 *   sequence start.  For every token t of the sequence, in order:
 *
 *     r_0[i]  = sum_{m=0..3} w[e,i,m] * k[t-3+m, e, i]        causal depthwise
 *               (taps before the sequence start read zero)      ShortConv, width 4
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
 *     residual update r^(l+1) = r^(l) - delta^(l)).
 *   - ICML 2026 poster abstract: a short convolution anchors the initial
 *     residual.
 *
 * Readings where the pages are silent or garbled (all code follows them):
 *   - the product in the residual closed form runs over j = 1..l-1, so the
 *     first refinement level uses the raw anchor; h's last slot is unused;
 *   - conv tap 3 multiplies the current token, taps 0..2 the three before it;
 *     no bias and no activation after the convolution;
 *   - g and b are per (token, head) scalars; g is a linear-space gate;
 *   - no query scaling; the initial state is zero.
 *
 * Precision: all arithmetic in double.  Inputs are fp32 or bf16 (raw 16-bit
 * patterns) and are widened exactly.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

typedef struct {
    int64_t n_seqs;
    int64_t total_tokens;
    int64_t heads;
    int64_t dk;
    int64_t dv;
    int64_t L;
    int64_t dtype;      /* ORACLE_F32 or ORACLE_BF16 */
} oracle_dims;

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

/* Write key of token t, head e into kw[0..dk).  seq_start is the first token
 * of t's sequence (conv taps before it read zero). */
static void write_key(const oracle_dims* d, const void* k, const void* u, const void* a,
                      const void* h, const void* b, const void* conv_w,
                      int64_t seq_start, int64_t t, int64_t e, double* kw)
{
    const int64_t H = d->heads, dk = d->dk, L = d->L, dt = d->dtype;
    const double bt = elem(b, dt, t * H + e);
    for (int64_t i = 0; i < dk; ++i) {
        /* r_0: causal depthwise convolution over k along the token axis. */
        double r0 = 0.0;
        for (int64_t m = 0; m < 4; ++m) {
            int64_t tau = t - 3 + m;
            if (tau < seq_start)
                continue;
            r0 += elem(conv_w, dt, (e * dk + i) * 4 + m) * elem(k, dt, (tau * H + e) * dk + i);
        }
        double acc = bt * elem(k, dt, (t * H + e) * dk + i);
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

/* kw for every token and head: out[T, H, dk] (double). */
int prism_oracle_prologue(const oracle_dims* d, const int32_t* cu_seqlens,
                          const void* k, const void* u, const void* a, const void* h,
                          const void* b, const void* conv_w, double* kw_out, int nthreads)
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
            write_key(d, k, u, a, h, b, conv_w, cu_seqlens[n], t, e, kw_out + (t * H + e) * dk);
    }
    return 0;
}

/*
 * Full forward.  chains: optional list of (sequence * heads + head) indices to
 * evaluate (NULL = all).  Only the selected chains' rows of o_out [T, H, dv]
 * and blocks of s_out [n_seqs, H, dk, dv] are written.
 */
int prism_oracle_fwd(const oracle_dims* d, const int32_t* cu_seqlens,
                     const void* q, const void* k, const void* v, const void* u,
                     const void* g, const void* b, const void* a, const void* h,
                     const void* conv_w, const int64_t* chains, int64_t n_chains,
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
        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            write_key(d, k, u, a, h, b, conv_w, cu_seqlens[n], t, e, kw);
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
