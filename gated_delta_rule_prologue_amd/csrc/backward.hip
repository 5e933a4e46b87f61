// backward.hip -- gradients of PRISM's memory-writing operator (closed-form
// residual chain) for the loss sum <dO, o> + <dS_final, S_final>.
//
// Reverse-mode differentiation of the token recurrence (WeChat ICML 2026
// PRISM summary, sections 核心迭代形式, 消除 Token 间串行 and 消除 Step 间串行;
// gist.science summary section 2.1, S_t = S_{t-1} A_t + B_t).  With
// G = dL/dS_t and, for each token from the last,
//   G += q_t dO_t^T;  dq_t = S_t dO_t;  dv_t = G^T kw_t;  dkw_t = G v_t
//   P = S_{t-1} - b k p^T, p = S_{t-1}^T k;  dg_t = <G, P>;  dP = g G
//   y = dP^T k;  db_t -= y . p;  dk_t -= b (dP p + S_{t-1} y);  G = dP - b k y^T
// and dS_init = G at the sequence start; then the write key backwards through
// the residual chain and the ShortConv taps.
//
// Design: correct first, a plain token-by-token form (the chunkwise form of
// the forward is the faster route; see the forward scan for its algebra).
//   * scan_bwd_kernel: one 256-thread workgroup per (sequence, head, 32 value
//     columns); thread (rg, cg) holds rows rg + 32 r, columns 4 cg .. 4 cg + 3
//     of S and G in registers.  A first sweep stores S at every chunk start
//     (64 tokens); then, chunk by chunk from the last, the chunk's states are
//     recomputed into a per-workgroup scratch and the chunk is walked
//     backwards.  Column sums (over the dk rows) go through LDS; row sums (over
//     the 32 columns) through lane shuffles, then fp32 atomics into dq, dk and
//     dkw, which the value slices of a chain share.
//   * write_key_bwd_kernel: one thread per (head, channel, block of 64 tokens):
//     the residual chain backwards (du, da, dh written, dr_0 formed), b and
//     the taps (dk, db through atomics; dconv_w summed over the block first).
#include "common.h"
#include "kernels.h"

namespace prism {
namespace bwd {

constexpr int kC = 64;                           // chunk of the checkpoint sweep
constexpr int kCols = 32;                        // value columns per workgroup

// checkpoint slot of the chunk starting at token s of sequence n (unique, < T/64 + n_seqs + 1)
__device__ __forceinline__ int64_t ckpt_slot(int s, int n) { return (int64_t)(s / kC) + n; }

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) { return to_f32(p[i]); }

// Sum over the lanes of a wavefront that share lane % 8 (the eight row groups
// of one column group in a wavefront).
__device__ __forceinline__ float sum_rows8(float x)
{
    x += __shfl_xor(x, 8);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}
// Sum over the eight consecutive lanes of one row group (its 8 column groups).
__device__ __forceinline__ float sum_cols8(float x)
{
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    return x;
}

template <typename T, int DK>
__global__ __launch_bounds__(256) void scan_bwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ kw,
    const T* __restrict__ v, const T* __restrict__ g, const T* __restrict__ b,
    const T* __restrict__ dO, const int32_t* __restrict__ cu, int H, int DV,
    const float* __restrict__ S_init, const float* __restrict__ dS_final,
    float* __restrict__ ckpt, float* __restrict__ scr,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dkw,
    float* __restrict__ dv, float* __restrict__ dg, float* __restrict__ db,
    float* __restrict__ dS_init)
{
    constexpr int RPT = DK / 32;                 // rows per thread
    constexpr int EL = RPT * 4;                  // state elements per thread
    __shared__ float red[2][4][3][kCols];        // per wavefront column partials, double-buffered
    __shared__ float redg[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid & 7, rg = tid >> 3;       // column group, row group (0..31)
    const int slices = DV / kCols;
    const int slice = blockIdx.x % slices;
    const int chain = blockIdx.x / slices;
    const int n = chain / H, e = chain % H;
    const int j0 = slice * kCols + cg * 4;       // first of this thread's 4 columns
    const int seq0 = cu[n], seq1 = cu[n + 1];
    const int64_t wg = blockIdx.x;
    // this thread's elements of a dk x 32 slice, stored thread-major in scratch
    const int64_t SL = (int64_t)DK * kCols;
    auto st_idx = [&](int r, int c) { return (int64_t)(r * 4 + c) * 256 + tid; };

    float S[EL], G[EL];
    const int64_t sbase = ((int64_t)chain * DK) * DV;    // [n, e] block of S_init / dS_final
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int64_t x = sbase + (int64_t)(rg + 32 * r) * DV + j0 + c;
            S[r * 4 + c] = S_init ? S_init[x] : 0.f;
            G[r * 4 + c] = dS_final ? dS_final[x] : 0.f;
        }
    int buf = 0;
    // column sums of up to three vectors of this thread's 4 columns over the dk rows
    auto colsum = [&](float (&x)[3][4], int nv, float gpart, float& gsum) {
#pragma unroll
        for (int vv = 0; vv < 3; ++vv)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (vv < nv)
                    x[vv][c] = sum_rows8(x[vv][c]);
        float gw = gpart;
        for (int o = 32; o > 0; o >>= 1)
            gw += __shfl_xor(gw, o);
        if (lane < 8) {
#pragma unroll
            for (int vv = 0; vv < 3; ++vv)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (vv < nv)
                        red[buf][wave][vv][cg * 4 + c] = x[vv][c];
        }
        if (lane == 0)
            redg[buf][wave] = gw;
        __syncthreads();
#pragma unroll
        for (int vv = 0; vv < 3; ++vv)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (vv < nv)
                    x[vv][c] = red[buf][0][vv][cg * 4 + c] + red[buf][1][vv][cg * 4 + c] +
                               red[buf][2][vv][cg * 4 + c] + red[buf][3][vv][cg * 4 + c];
        gsum = redg[buf][0] + redg[buf][1] + redg[buf][2] + redg[buf][3];
        buf ^= 1;
    };
    // one forward token: S <- g (S - b k p^T) + kw v^T
    auto step_fwd = [&](int t) {
        const int64_t rk = ((int64_t)t * H + e) * DK, rv = ((int64_t)t * H + e) * DV + j0;
        float kk[RPT], ww[RPT], vv4[4];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            kk[r] = ld(k, rk + rg + 32 * r);
            ww[r] = ld(kw, rk + rg + 32 * r);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
            vv4[c] = ld(v, rv + c);
        const float gt = ld(g, (int64_t)t * H + e), bt = ld(b, (int64_t)t * H + e);
        float x[3][4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < RPT; ++r)
                acc += S[r * 4 + c] * kk[r];
            x[0][c] = acc;
        }
        float gs;
        colsum(x, 1, 0.f, gs);
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                S[r * 4 + c] = gt * (S[r * 4 + c] - bt * kk[r] * x[0][c]) + ww[r] * vv4[c];
    };

    // sweep 1: S at every chunk start
    for (int t = seq0; t < seq1; ++t) {
        if ((t - seq0) % kC == 0) {
            float* cp = ckpt + (ckpt_slot(t, n) * H * (DV / kCols) + (int64_t)e * slices + slice) * SL;
#pragma unroll
            for (int r = 0; r < RPT; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    cp[st_idx(r, c)] = S[r * 4 + c];
        }
        step_fwd(t);
    }

    // sweep 2: chunks from the last, states recomputed into scratch, then walked back
    float* sc = scr + wg * (int64_t)(kC + 1) * SL;
    const int nch = (seq1 - seq0 + kC - 1) / kC;
    for (int ch = nch - 1; ch >= 0; --ch) {
        const int c0 = seq0 + ch * kC, c1 = min(seq1, c0 + kC);
        const float* cp = ckpt + (ckpt_slot(c0, n) * H * (DV / kCols) + (int64_t)e * slices + slice) * SL;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                S[r * 4 + c] = cp[st_idx(r, c)];
                sc[st_idx(r, c)] = S[r * 4 + c];
            }
        for (int t = c0; t < c1; ++t) {
            step_fwd(t);
            float* so = sc + (int64_t)(t - c0 + 1) * SL;
#pragma unroll
            for (int r = 0; r < RPT; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    so[st_idx(r, c)] = S[r * 4 + c];
        }
        // S holds S_{c1 - 1}
        for (int t = c1 - 1; t >= c0; --t) {
            const float* sp = sc + (int64_t)(t - c0) * SL;
            float Sm[EL];
#pragma unroll
            for (int r = 0; r < RPT; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    Sm[r * 4 + c] = sp[st_idx(r, c)];
            const int64_t rk = ((int64_t)t * H + e) * DK, rv = ((int64_t)t * H + e) * DV + j0;
            float kk[RPT], qq[RPT], ww[RPT], vv4[4], do4[4];
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                kk[r] = ld(k, rk + rg + 32 * r);
                qq[r] = ld(q, rk + rg + 32 * r);
                ww[r] = ld(kw, rk + rg + 32 * r);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                vv4[c] = ld(v, rv + c);
                do4[c] = ld(dO, rv + c);
            }
            const float gt = ld(g, (int64_t)t * H + e), bt = ld(b, (int64_t)t * H + e);
            // G += q dO^T; dq = S_t dO and dkw = G v (row sums: lanes, then atomics)
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                float aq = 0.f, aw = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    G[r * 4 + c] += qq[r] * do4[c];
                    aq += S[r * 4 + c] * do4[c];
                    aw += G[r * 4 + c] * vv4[c];
                }
                aq = sum_cols8(aq);
                aw = sum_cols8(aw);
                if (cg == 0) {
                    atomicAdd(dq + rk + rg + 32 * r, aq);
                    atomicAdd(dkw + rk + rg + 32 * r, aw);
                }
            }
            // column sums: dv = G^T kw and p = S_{t-1}^T k
            float x[3][4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float a1 = 0.f, a2 = 0.f;
#pragma unroll
                for (int r = 0; r < RPT; ++r) {
                    a1 += G[r * 4 + c] * ww[r];
                    a2 += Sm[r * 4 + c] * kk[r];
                }
                x[0][c] = a1;
                x[1][c] = a2;
            }
            float gs;
            colsum(x, 2, 0.f, gs);
            if (rg == 0)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    dv[rv + c] = x[0][c];
            float p4[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
                p4[c] = x[1][c];
            // dg = <G, P>, P = S_{t-1} - b k p^T; dP = g G; y = dP^T k
            float dgp = 0.f;
#pragma unroll
            for (int r = 0; r < RPT; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    dgp += G[r * 4 + c] * (Sm[r * 4 + c] - bt * kk[r] * p4[c]);
                    G[r * 4 + c] *= gt;
                }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float a1 = 0.f;
#pragma unroll
                for (int r = 0; r < RPT; ++r)
                    a1 += G[r * 4 + c] * kk[r];
                x[0][c] = a1;
            }
            float dgs;
            colsum(x, 1, dgp, dgs);
            float y4[4];
#pragma unroll
            for (int c = 0; c < 4; ++c)
                y4[c] = x[0][c];
            if (tid == 0)
                atomicAdd(dg + (int64_t)t * H + e, dgs);
            if (rg == 0) {                       // db -= y . p over this slice's columns
                float yp = y4[0] * p4[0] + y4[1] * p4[1] + y4[2] * p4[2] + y4[3] * p4[3];
                yp = sum_cols8(yp);
                if (cg == 0)
                    atomicAdd(db + (int64_t)t * H + e, -yp);
            }
            // dk -= b (dP p + S_{t-1} y); G = dP - b k y^T
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                float a1 = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    a1 += G[r * 4 + c] * p4[c] + Sm[r * 4 + c] * y4[c];
                    G[r * 4 + c] -= bt * kk[r] * y4[c];
                }
                a1 = sum_cols8(a1);
                if (cg == 0)
                    atomicAdd(dk + rk + rg + 32 * r, -bt * a1);
            }
#pragma unroll
            for (int x2 = 0; x2 < EL; ++x2)
                S[x2] = Sm[x2];
        }
    }
    if (dS_init) {
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                dS_init[sbase + (int64_t)(rg + 32 * r) * DV + j0 + c] = G[r * 4 + c];
    }
}

// One thread per (head e, channel i, block of 64 tokens): for each token of the
// block, the write key backwards.  dkw (fp32) comes from the scan backward.
template <typename T>
__global__ __launch_bounds__(256) void write_key_bwd_kernel(
    const T* __restrict__ k, const T* __restrict__ u, const T* __restrict__ a,
    const T* __restrict__ h, const T* __restrict__ b, const T* __restrict__ conv_w,
    const int32_t* __restrict__ cu, int n_seqs, int T_total, int H, int DK, int L,
    const float* __restrict__ dkw, float* __restrict__ dk, float* __restrict__ du,
    float* __restrict__ da, float* __restrict__ dh, float* __restrict__ db,
    float* __restrict__ dconv_w)
{
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int i = (int)(gid % DK);
    const int e = (int)((gid / DK) % H);
    const int64_t blk = gid / ((int64_t)DK * H);
    const int t_lo = (int)(blk * kC);
    if (t_lo >= T_total)
        return;
    const int t_hi = min(T_total, t_lo + kC);
    float w[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        w[m] = ld(conv_w, ((int64_t)e * DK + i) * 4 + m);
    // sequence of t_lo
    int lo = 0, hi = n_seqs;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= t_lo) lo = mid; else hi = mid;
    }
    int sn = lo;
    float dw[4] = {0.f, 0.f, 0.f, 0.f};
    const int64_t lrow = (int64_t)H * (L - 1) * DK;
    for (int t = t_lo; t < t_hi; ++t) {
        while (cu[sn + 1] <= t)
            ++sn;                                // the sequence holding t (skips empty ones)
        const int s0 = cu[sn];
        const int64_t rk = ((int64_t)t * H + e) * DK + i;
        const float g_kw = dkw[rk];
        const float kt = ld(k, rk), bt = ld(b, (int64_t)t * H + e);
        // b k part of the key
        atomicAdd(dk + rk, bt * g_kw);
        float dbp = g_kw * kt;
        for (int o = 32; o > 0; o >>= 1)         // one atomic per wavefront: its lanes are
            dbp += __shfl_xor(dbp, o);           // 64 channels of one (token, head) when DK >= 64
        if (DK >= 64) {
            if ((threadIdx.x & 63) == 0)
                atomicAdd(db + (int64_t)t * H + e, dbp);
        } else {
            atomicAdd(db + (int64_t)t * H + e, g_kw * kt);
        }
        if (L == 1)
            continue;
        float kx[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int tau = t - 3 + m;
            kx[m] = tau >= s0 ? ld(k, ((int64_t)tau * H + e) * DK + i) : 0.f;
        }
        const float r0 = w[0] * kx[0] + w[1] * kx[1] + w[2] * kx[2] + w[3] * kx[3];
        // residuals r_l, l = 1 .. L-1 (closed form as a running product)
        float r[16];
        r[1] = r0;
        const int64_t lb = (int64_t)t * lrow + (int64_t)e * (L - 1) * DK + i;
        for (int l = 1; l < L - 1; ++l)
            r[l + 1] = r[l] * (1.f - ld(a, lb + (int64_t)(l - 1) * DK) * ld(h, lb + (int64_t)(l - 1) * DK));
        float dr_next = 0.f;
        for (int l = L - 1; l >= 1; --l) {
            const int64_t sl = lb + (int64_t)(l - 1) * DK;
            const float al = ld(a, sl), ul = ld(u, sl), hl = ld(h, sl);
            du[sl] = g_kw * al * r[l];
            float dal = g_kw * ul * r[l], dhl = 0.f, drl = g_kw * al * ul;
            if (l <= L - 2) {
                dal -= dr_next * hl * r[l];
                dhl = -dr_next * al * r[l];
                drl += dr_next * (1.f - al * hl);
            }
            da[sl] = dal;
            dh[sl] = dhl;
            dr_next = drl;
        }
        // the taps: dw_m += dr_0 k_{t-3+m}, dk_{t-3+m} += w_m dr_0 inside the sequence
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int tau = t - 3 + m;
            if (tau < s0)
                continue;
            dw[m] += dr_next * kx[m];
            atomicAdd(dk + ((int64_t)tau * H + e) * DK + i, w[m] * dr_next);
        }
    }
    if (L > 1)
#pragma unroll
        for (int m = 0; m < 4; ++m)
            atomicAdd(dconv_w + ((int64_t)e * DK + i) * 4 + m, dw[m]);
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, int64_t n)
{
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256)
        p[x] = 0.f;
}

}  // namespace bwd

size_t bwd_workspace_floats(int n_seqs, int total_tokens, int heads, int dk, int dv)
{
    const int64_t slots = total_tokens / bwd::kC + n_seqs + 1;
    const int64_t wgs = (int64_t)n_seqs * heads * (dv / bwd::kCols);
    return (size_t)(slots * heads * dk * dv)                      // chunk-start states
         + (size_t)(wgs * (bwd::kC + 1) * dk * bwd::kCols)       // one chunk of states per workgroup
         + (size_t)total_tokens * heads * dk;                     // dkw
}

bool bwd_supported(int dk, int dv) { return (dk == 64 || dk == 128) && (dv == 64 || dv == 128); }

template <typename T, int DK>
static hipError_t launch_bwd_T(const BwdArgs& p, hipStream_t s)
{
    const int H = p.heads, T_ = p.total_tokens;
    const int64_t slots = T_ / bwd::kC + p.n_seqs + 1;
    float* ckpt = p.ws;
    float* scr = ckpt + slots * H * DK * p.dv;
    const int64_t wgs = (int64_t)p.n_seqs * H * (p.dv / bwd::kCols);
    float* dkw = scr + wgs * (bwd::kC + 1) * DK * bwd::kCols;
    // accumulators start at zero (a fill kernel: no memset node under graph capture)
    auto zero = [&](float* x, int64_t n) {
        if (n > 0)
            hipLaunchKernelGGL(bwd::zero_kernel, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)),
                               dim3(256), 0, s, x, n);
    };
    zero(p.gq, (int64_t)T_ * H * DK);
    zero(p.gk, (int64_t)T_ * H * DK);
    zero(dkw, (int64_t)T_ * H * DK);
    zero(p.gg, (int64_t)T_ * H);
    zero(p.gb, (int64_t)T_ * H);
    zero(p.gconv, (int64_t)H * DK * 4);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || wgs == 0)
        return err;
    hipLaunchKernelGGL((bwd::scan_bwd_kernel<T, DK>), dim3((unsigned)wgs), dim3(256), 0, s,
                       (const T*)p.q, (const T*)p.k, (const T*)p.kw, (const T*)p.v, (const T*)p.g,
                       (const T*)p.b, (const T*)p.dO, p.cu_seqlens, H, p.dv, p.s_init, p.ds_final,
                       ckpt, scr, p.gq, p.gk, dkw, p.gv, p.gg, p.gb, p.gs_init);
    if ((err = hipGetLastError()) != hipSuccess || T_ == 0)
        return err;
    const int64_t threads = ((int64_t)(T_ + bwd::kC - 1) / bwd::kC) * H * DK;
    hipLaunchKernelGGL((bwd::write_key_bwd_kernel<T>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, s, (const T*)p.k, (const T*)p.u, (const T*)p.a,
                       (const T*)p.h, (const T*)p.b, (const T*)p.conv_w, p.cu_seqlens, p.n_seqs,
                       T_, H, DK, p.L, dkw, p.gk, p.gu, p.ga, p.gh, p.gb, p.gconv);
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& p, hipStream_t s)
{
    if (!bwd_supported(p.dk, p.dv) || p.L < 1 || p.L > 16)
        return hipErrorInvalidValue;
    if (p.bf16)
        return p.dk == 64 ? launch_bwd_T<uint16_t, 64>(p, s) : launch_bwd_T<uint16_t, 128>(p, s);
    return p.dk == 64 ? launch_bwd_T<float, 64>(p, s) : launch_bwd_T<float, 128>(p, s);
}

}  // namespace prism
