// decode.hip -- one token of every sequence through PRISM's memory-writing
// operator, with the state S and the convolution history carried in device
// memory and updated in place (serving: one call per generated or arriving
// token).
//
// Per (sequence n, head e), for the sequence's one new token:
//   r_0  = w3 k + w2 hist[2] + w1 hist[1] + w0 hist[0]     ShortConv anchor
//   kw   = b k + sum_{l=1..L-1} a_l r_l u_l,  r_{l+1} = r_l (1 - a_l h_l)
//          (or r_{l+1} = r_l - a_l GELU(h_l r_l), the non-linear refinement chain)
//   p    = S^T k
//   S   <- g (S - b k p^T) + kw v^T                         = g (I - b k k^T) S + kw v^T
//   o    = S^T q
//   hist <- (hist[1], hist[2], k)
// PRISM pages: WeChat ICML 2026 summary, sections 背景：无限背包 vs 有限背包
// (a fixed-size state updated by an RNN recurrence), 核心迭代形式, 消除 Token 间串行
// and 消除 Step 间串行 (the write key); gist.science summary of arXiv
// 2602.10796, section 2.1 (S_t = S_{t-1} A_t + B_t).
//
// Design (HBM-bound: the fp32 state is read and written once per token, every
// other operand is a few hundred bytes per chain):
//   * one workgroup per chain (256 threads), so the in-place updates of S and
//     of the history need no ordering between workgroups;
//   * thread (rg, cg) owns the 4 columns cg*4..cg*4+3 of rows rg, rg + RG,
//     ...; a wavefront's loads for one row index cover whole contiguous rows
//     of S (16-byte accesses);
//   * the state is loaded and stored with the nontemporal hint: it is touched
//     once per step, and keeping it out of the caches let the step run about
//     17 % faster on both serving batches measured (recsys 512 x 8 heads,
//     dk = dv = 64; LM 256 x 6 heads, dk = dv = 128);
//   * every load of the step is issued before the first wait: the state rows,
//     then the chain's u, a, h slots (contiguous, (L-1) dk elements each),
//     fetched by the whole workgroup as 16-byte vectors and parked in LDS, so
//     the write key costs one memory round trip whatever L is;
//   * the write key is then computed by one thread per channel from LDS and
//     kept in fp32 (never rounded to the input type);
//   * the two column reductions (S^T k before the update, S^T q after it) go
//     through LDS, one partial per row group.
#include "common.h"
#include "kernels.h"

namespace prism {

template <typename T, int DK, int DV, int NTH>
__global__ __launch_bounds__(NTH) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ u, const T* __restrict__ a, const T* __restrict__ h,
    const T* __restrict__ g, const T* __restrict__ b, const T* __restrict__ conv_w, int H, int L,
    bool gelu, float* __restrict__ S, T* __restrict__ k_hist, T* __restrict__ o)
{
    constexpr int CG = DV / 4;                   // 4-column groups
    constexpr int RG = NTH / CG;                 // row groups
    constexpr int RPT = DK / RG;                 // rows per thread
    static_assert(NTH % CG == 0 && DK % RG == 0 && DK <= NTH, "thread layout");
    __shared__ float sK[DK], sQ[DK], sKW[DK];
    __shared__ f32x4_t sRed[2][RG][CG];
    extern __shared__ uint4 sLev[];              // raw a | u | h slots of the chain
    constexpr int VE = 16 / (int)sizeof(T);      // elements per 16-byte vector

    const int tid = threadIdx.x;
    const int64_t chain = blockIdx.x;            // n * H + e
    const int e = (int)(chain % H);
    const int cg = tid % CG, rg = tid / CG;
    float* Sc = S + chain * DK * DV + cg * 4;

    f32x4_t x[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        x[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(Sc + (int64_t)(rg + r * RG) * DV));
    float vv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        vv[c] = to_f32(v[chain * DV + cg * 4 + c]);
    const float gt = to_f32(g[chain]), bt = to_f32(b[chain]);

    // the chain's level slots: a and u have L - 1, h's last one is never read
    const int nv = (L - 1) * DK / VE, nh = (L > 2 ? L - 2 : 0) * DK / VE;
    const int64_t lvb = chain * (L - 1) * DK / VE;
    for (int j = tid; j < nv; j += NTH) {
        const uint4 av = reinterpret_cast<const uint4*>(a)[lvb + j];
        const uint4 uv = reinterpret_cast<const uint4*>(u)[lvb + j];
        uint4 hv = make_uint4(0u, 0u, 0u, 0u);
        if (j < nh)
            hv = reinterpret_cast<const uint4*>(h)[lvb + j];
        sLev[j] = av;
        sLev[nv + j] = uv;
        sLev[2 * nv + j] = hv;
    }
    T kraw = T(0), h0 = T(0), h1 = T(0), h2 = T(0), qraw = T(0), w[4];
    T* hp = k_hist + chain * 3 * DK + tid;
    if (tid < DK) {
        kraw = k[chain * DK + tid];
        qraw = q[chain * DK + tid];
        h0 = hp[0];
        h1 = hp[DK];
        h2 = hp[2 * DK];
#pragma unroll
        for (int m = 0; m < 4; ++m)
            w[m] = conv_w[((int64_t)e * DK + tid) * 4 + m];
    }
    __syncthreads();

    if (tid < DK) {
        const int i = tid;
        const float kt = to_f32(kraw);
        float r = to_f32(w[3]) * kt + to_f32(w[2]) * to_f32(h2) + to_f32(w[1]) * to_f32(h1) +
                  to_f32(w[0]) * to_f32(h0);
        float acc = bt * kt;
        const T* la = reinterpret_cast<const T*>(sLev);
        const T* lu = la + nv * VE;
        const T* lh = lu + nv * VE;
        for (int s = 0; s < L - 1; ++s) {        // level l = s + 1
            const float av = to_f32(la[s * DK + i]);
            acc += av * r * to_f32(lu[s * DK + i]);
            if (s < L - 2) {
                const float hv = to_f32(lh[s * DK + i]);
                if (gelu)                        // r - a GELU(h r)
                    r -= av * gelu_as(hv * r);
                else
                    r *= 1.f - av * hv;
            }
        }
        sKW[i] = acc;
        sK[i] = kt;
        sQ[i] = to_f32(qraw);
        hp[0] = h1;
        hp[DK] = h2;
        hp[2 * DK] = kraw;
    }
    __syncthreads();

    // p = S^T k
    f32x4_t pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        pp += x[r] * sK[rg + r * RG];
    sRed[0][rg][cg] = pp;
    __syncthreads();
    f32x4_t p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RG; ++j)
        p += sRed[0][j][cg];

    // S <- g (S - b k p^T) + kw v^T, then the partial o = S^T q
    f32x4_t po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int i = rg + r * RG;
        const float ki = sK[i], kwi = sKW[i];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            x[r][c] = gt * (x[r][c] - bt * ki * p[c]) + kwi * vv[c];
        __builtin_nontemporal_store(x[r], reinterpret_cast<f32x4_t*>(Sc + (int64_t)i * DV));
        po += x[r] * sQ[i];
    }
    sRed[1][rg][cg] = po;
    __syncthreads();
    if (rg == 0) {
        f32x4_t ov = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < RG; ++j)
            ov += sRed[1][j][cg];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            o[chain * DV + cg * 4 + c] = from_f32<T>(ov[c]);
    }
}

bool decode_supported(int dk, int dv)
{
    return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

template <typename T, int DK, int DV, int NTH = 256>
static hipError_t launch_dec(const DecodeArgs& p, hipStream_t stream)
{
    const int64_t blocks = (int64_t)p.n_seqs * p.heads;
    if (blocks == 0)
        return hipSuccess;
    const size_t lev = 3 * (size_t)(p.L - 1) * DK * sizeof(T);    // raw a | u | h slots
    hipLaunchKernelGGL((decode_kernel<T, DK, DV, NTH>), dim3((unsigned)blocks), dim3(NTH), lev, stream,
                       (const T*)p.q, (const T*)p.k, (const T*)p.v, (const T*)p.u, (const T*)p.a,
                       (const T*)p.h, (const T*)p.g, (const T*)p.b, (const T*)p.conv_w, p.heads,
                       p.L, p.gelu, p.S, (T*)p.k_hist, (T*)p.o);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_dec_T(const DecodeArgs& p, hipStream_t s)
{
    if (p.dk == 64)
        return p.dv == 64 ? launch_dec<T, 64, 64>(p, s) : launch_dec<T, 64, 128>(p, s);
    return p.dv == 64 ? launch_dec<T, 128, 64>(p, s) : launch_dec<T, 128, 128>(p, s);
}

hipError_t launch_decode(const DecodeArgs& p, hipStream_t stream)
{
    if (!decode_supported(p.dk, p.dv) || p.L < 1)
        return hipErrorInvalidValue;
    return p.bf16 ? launch_dec_T<uint16_t>(p, stream) : launch_dec_T<float>(p, stream);
}

}  // namespace prism
