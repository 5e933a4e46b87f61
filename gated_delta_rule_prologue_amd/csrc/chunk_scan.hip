// chunk_scan.hip -- chunkwise WY/UT scan of the gated delta-rule state recurrence
//
//   S_t = g_t (I - b_t k_t k_t^T) S_{t-1} + kw_t v_t^T,     o_t = S_t^T q_t
//
// (PRISM pages: WeChat ICML 2026 summary, section 消除 Token 间串行 -- the
// forget/erase term is the Gated DeltaNet one and the write depends on the
// inputs only; gist.science summary of arXiv 2602.10796, section 2.1 --
// S_t = S_{t-1} A_t + B_t with input-only A_t, B_t, which is what makes a
// chunked / parallel evaluation exact.)
//
// Chunk algebra (64 tokens, incoming state S0, in-chunk cumulative log2-gates
// lam_t, gamma_t = 2^lam_t, decay D[t,s] = 2^(lam_t - lam_s) for s <= t):
//   A_kk  = diag(b) (D . tril_-1(K K^T))          A_kkw = diag(b) (D . tril_-1(K KW^T))
//   A_qk  = D . tril_0(Q K^T)                     A_qkw = D . tril_0(Q KW^T)
//   Tm    = (I + A_kk)^-1                          (UT transform, fp32)
//   R     = diag(b gamma) K S0 + A_kkw V
//   X     = Tm R                                   rows x_t = g_t b_t S_{t-1}^T k_t
//   O     = diag(gamma) Q S0 + A_qkw V - A_qk X
//   S_out = gamma_C S0 + (diag(gamma_C/gamma) KW)^T V - (diag(gamma_C/gamma) K)^T X
// The masks are applied before the exponentials, so every factor used is
// <= 1 and strong decay cannot overflow.
//
// Mapping to gfx950:
//   * one workgroup (4 wavefronts) per (sequence, head, value slice): the value
//     columns of S are independent, so a chain's dv columns are split over
//     several workgroups to occupy the 256 CUs when chains are few;
//   * the state slice (dk x dv_slice) lives in MFMA accumulator registers in
//     fp32 for the whole sequence; it is rounded to the operand type only as an
//     operand of the chunk products;
//   * every contraction is a 16x16 MFMA tile product with both operands staged
//     in LDS with the contraction index contiguous (bf16: v_mfma_f32_16x16x32_bf16,
//     fp32: v_mfma_f32_16x16x4_f32); K and KW are staged twice (row-major for
//     the Gram products, transposed and decay-scaled for the state update);
//   * the 64x64 unit-lower-triangular inverse is done in fp32: the four 16x16
//     diagonal blocks by substitution, then three levels of off-diagonal
//     blocks with fp32 MFMA;
//   * varlen: chunks restart at every cu_seqlens entry; a ragged last chunk is
//     zero-padded (k = kw = q = v = 0, g = 1, b = 0), which leaves S unchanged.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace prism {

constexpr int kC = 64;          // chunk length
constexpr int kThreads = 256;   // 4 wavefronts
constexpr int kFLd = 65;        // row stride of the fp32 inverse scratch
constexpr int kPLd = 17;        // row stride of the 16x16 fp32 level scratch

template <typename Op> struct Mfma;
template <> struct Mfma<uint16_t> {          // bf16 operands
    static constexpr int KB = 32, KPL = 8;
    using Frag = bf16x8_t;
    __device__ static Frag load(const uint16_t* p)
    {
        return __builtin_bit_cast(Frag, *reinterpret_cast<const uint4*>(p));
    }
    __device__ static f32x4_t mma(Frag a, Frag b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {             // fp32 operands
    static constexpr int KB = 4, KPL = 1;
    using Frag = float;
    __device__ static Frag load(const float* p) { return *p; }
    __device__ static f32x4_t mma(float a, float b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ f32x4_t mma_f32(float a, float b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc += A[0:16, 0:K] B[0:K, 0:16].  A is stored [m][k] at `a` (row stride lda),
// B is stored transposed, [n][k], at `bt` (row stride ldb).  Accumulator
// layout: lane l holds C[4 (l >> 4) + r][l & 15], r = 0..3.
template <typename Op, int K>
__device__ __forceinline__ f32x4_t tile_mma(f32x4_t acc, const Op* a, int lda, const Op* bt,
                                            int ldb, int lane)
{
    using M = Mfma<Op>;
    const Op* pa = a + (lane & 15) * lda + (lane >> 4) * M::KPL;
    const Op* pb = bt + (lane & 15) * ldb + (lane >> 4) * M::KPL;
#pragma unroll
    for (int k = 0; k < K; k += M::KB)
        acc = M::mma(M::load(pa + k), M::load(pb + k), acc);
    return acc;
}

template <typename Op>
__device__ __forceinline__ f32x4_t tile_mma_n(f32x4_t acc, const Op* a, int lda, const Op* bt,
                                              int ldb, int K, int lane)
{
    using M = Mfma<Op>;
    const Op* pa = a + (lane & 15) * lda + (lane >> 4) * M::KPL;
    const Op* pb = bt + (lane & 15) * ldb + (lane >> 4) * M::KPL;
    for (int k = 0; k < K; k += M::KB)
        acc = M::mma(M::load(pa + k), M::load(pb + k), acc);
    return acc;
}

// Store four consecutive fp32 values as the operand type (8 or 16 bytes).
__device__ __forceinline__ void store4(uint16_t* p, f32x4_t x)
{
    uint32_t w0 = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
    uint32_t w1 = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
    *reinterpret_cast<uint2*>(p) = make_uint2(w0, w1);
}
__device__ __forceinline__ void store4(float* p, f32x4_t x)
{
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// LDS carve-up (byte offsets, all multiples of 16).
template <typename Op, int D, int DVS>
struct Layout {
    static constexpr bool kBf = sizeof(Op) == 2;
    static constexpr int PAD = 16 / (int)sizeof(Op);
    static constexpr int LDD = D + PAD;          // row stride of [64][D] and [DVS][D] tiles
    static constexpr int LDC = kC + PAD;         // row stride of [*][64] tiles
    static constexpr int E = (int)sizeof(Op);
    static constexpr int szRowD = kC * LDD * E;
    static constexpr int szKt = kBf ? D * LDC * E : 0;
    static constexpr int szVt = DVS * LDC * E;
    static constexpr int szM = kC * LDC * E;
    static constexpr int szT = kBf ? szM : 0;
    static constexpr int szS0t = DVS * LDD * E;
    static constexpr int szRt = DVS * LDC * E;
    static constexpr int szF = kC * kFLd * 4;
    static constexpr int szWork = szS0t + 2 * szRt;
    // bf16: the fp32 inverse scratch is dead before S0t/Rt/Xt are written, so they share bytes
    static constexpr int szU = kBf ? (szWork > szF ? szWork : szF) : szWork;
    static constexpr int szFsep = kBf ? 0 : szF;
    static constexpr int szP = 3 * 16 * kPLd * 4;
    static constexpr int szG = 2 * kC * 4;

    static constexpr int oQ = 0;
    static constexpr int oK = oQ + szRowD;
    static constexpr int oKW = oK + szRowD;
    static constexpr int oKt = oKW + szRowD;
    static constexpr int oKWt = oKt + szKt;
    static constexpr int oVt = oKWt + szKt;
    static constexpr int oAkkw = oVt + szVt;
    static constexpr int oAqkw = oAkkw + szM;
    static constexpr int oAqk = oAqkw + szM;
    static constexpr int oT = oAqk + szM;
    static constexpr int oU = oT + szT;
    static constexpr int oS0t = oU;
    static constexpr int oRt = oS0t + szS0t;
    static constexpr int oXt = oRt + szRt;
    static constexpr int oFsep = oU + szU;
    static constexpr int oF = kBf ? oU : oFsep;
    static constexpr int oP = oFsep + szFsep;
    static constexpr int oG = oP + szP;
    static constexpr int total = oG + szG;
};

template <typename T, int D, int DVS>
__global__ __launch_bounds__(kThreads) void chunk_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ kw,
    const T* __restrict__ v, const T* __restrict__ g, const T* __restrict__ b,
    const int32_t* __restrict__ cu, int H, int DV, int n_slices, T* __restrict__ o,
    float* __restrict__ s_final)
{
    using Ly = Layout<T, D, DVS>;
    using M = Mfma<T>;
    constexpr bool kBf = Ly::kBf;
    constexpr int LDD = Ly::LDD, LDC = Ly::LDC;
    constexpr int NJ = DVS / 16;                 // 16-column tiles of the value slice
    constexpr int NS = (D / 16) * NJ;            // state tiles
    constexpr int NSW = NS / 4;                  // state tiles owned by one wavefront
    static_assert(NS % 4 == 0, "state tiles must split over 4 wavefronts");
    static_assert(Ly::total <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(16))) unsigned char smem[Ly::total];
    T* sQ = reinterpret_cast<T*>(smem + Ly::oQ);
    T* sK = reinterpret_cast<T*>(smem + Ly::oK);
    T* sKW = reinterpret_cast<T*>(smem + Ly::oKW);
    T* sKt = reinterpret_cast<T*>(smem + Ly::oKt);       // -diag(gamma_C/gamma) K, transposed (bf16)
    T* sKWt = reinterpret_cast<T*>(smem + Ly::oKWt);     //  diag(gamma_C/gamma) KW, transposed (bf16)
    T* sVt = reinterpret_cast<T*>(smem + Ly::oVt);       // V slice, transposed [j][t]
    T* sAkkw = reinterpret_cast<T*>(smem + Ly::oAkkw);   // [t][s]
    T* sAqkw = reinterpret_cast<T*>(smem + Ly::oAqkw);   // [t][s]
    T* sAqk = reinterpret_cast<T*>(smem + Ly::oAqk);     // -A_qk, [t][s]
    T* sT = reinterpret_cast<T*>(smem + Ly::oT);         // UT inverse [t][s] (bf16)
    T* sS0t = reinterpret_cast<T*>(smem + Ly::oS0t);     // S0 transposed [j][i]
    T* sRt = reinterpret_cast<T*>(smem + Ly::oRt);       // R transposed [j][t]
    T* sXt = reinterpret_cast<T*>(smem + Ly::oXt);       // X transposed [j][t]
    float* sF = reinterpret_cast<float*>(smem + Ly::oF); // A_kk (strict lower) / Tm^T (strict upper)
    float* sP = reinterpret_cast<float*>(smem + Ly::oP);
    float* sLam = reinterpret_cast<float*>(smem + Ly::oG);
    float* sBv = sLam + kC;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slice = (int)(blockIdx.x % (unsigned)n_slices);
    const int chain = (int)(blockIdx.x / (unsigned)n_slices);
    const int n = chain / H, e = chain % H;
    const int j0 = slice * DVS;
    const int seq0 = cu[n], seq1 = cu[n + 1];
    const int nchunks = (seq1 - seq0 + kC - 1) / kC;
    const int64_t rowQK = (int64_t)H * D, rowV = (int64_t)H * DV;

    f32x4_t S[NSW];
#pragma unroll
    for (int i = 0; i < NSW; ++i)
        S[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int tb = wave;                         // token block handled in the R / X / O products
    const int kTri = ((tb + 1) * 16 + M::KB - 1) / M::KB * M::KB;

    for (int ch = 0; ch < nchunks; ++ch) {
        const int c0 = seq0 + ch * kC;
        const int nt = min(kC, seq1 - c0);

        // ---- gates: cumulative log2 decay, erase strength ----
        if (wave == 0) {
            float gv = 1.f, bv = 0.f;
            if (lane < nt) {
                gv = to_f32(g[(int64_t)(c0 + lane) * H + e]);
                bv = to_f32(b[(int64_t)(c0 + lane) * H + e]);
            }
            float lam = __log2f(fmaxf(gv, 1e-30f));
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                float y = __shfl_up(lam, d, 64);
                if (lane >= d)
                    lam += y;
            }
            sLam[lane] = lam;
            sBv[lane] = bv;
        }
        __syncthreads();
        const float lamC = sLam[kC - 1];

        // ---- stage the chunk into LDS ----
        {
            constexpr int V = Vec16<T>::N;
            constexpr int GPR = D / V;
            for (int idx = tid; idx < kC * GPR; idx += kThreads) {
                const int t = idx / GPR, c = (idx % GPR) * V;
                float xq[V], xk[V], xw[V];
                if (t < nt) {
                    const int64_t off = (int64_t)(c0 + t) * rowQK + (int64_t)e * D + c;
                    Vec16<T>::load(q + off, xq);
                    Vec16<T>::load(k + off, xk);
                    Vec16<T>::load(kw + off, xw);
                } else {
#pragma unroll
                    for (int i = 0; i < V; ++i) { xq[i] = 0.f; xk[i] = 0.f; xw[i] = 0.f; }
                }
                Vec16<T>::store(sQ + t * LDD + c, xq);
                Vec16<T>::store(sK + t * LDD + c, xk);
                Vec16<T>::store(sKW + t * LDD + c, xw);
                if constexpr (kBf) {
                    const float fac = exp2f(lamC - sLam[t]);
#pragma unroll
                    for (int i = 0; i < V; ++i) {
                        sKt[(c + i) * LDC + t] = f32_to_bf16(-xk[i] * fac);
                        sKWt[(c + i) * LDC + t] = f32_to_bf16(xw[i] * fac);
                    }
                }
            }
            constexpr int GPV = DVS / V;
            for (int idx = tid; idx < kC * GPV; idx += kThreads) {
                const int t = idx / GPV, jj = (idx % GPV) * V;
                float xv[V];
                if (t < nt) {
                    Vec16<T>::load(v + (int64_t)(c0 + t) * rowV + (int64_t)e * DV + j0 + jj, xv);
                } else {
#pragma unroll
                    for (int i = 0; i < V; ++i) xv[i] = 0.f;
                }
#pragma unroll
                for (int i = 0; i < V; ++i)
                    sVt[(jj + i) * LDC + t] = from_f32<T>(xv[i]);
            }
        }
        __syncthreads();

        // ---- Gram tiles with masks and decays: wavefront w builds matrix w ----
        //   w0: A_kk (fp32 scratch)  w1: A_kkw  w2: A_qkw  w3: -A_qk
        {
            const T* X = (wave < 2) ? sK : sQ;                    // supplies the row index t
            const T* Y = (wave == 0 || wave == 3) ? sK : sKW;     // supplies the column index s
            const bool strict = wave < 2;
            T* dstM = (wave == 1) ? sAkkw : (wave == 2) ? sAqkw : sAqk;
            for (int tb2 = 0; tb2 < 4; ++tb2) {
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
                    const int t = tb2 * 16 + (lane & 15);
                    const int s0 = sb * 16 + (lane >> 4) * 4;
                    f32x4_t val = {0.f, 0.f, 0.f, 0.f};
                    if (sb <= tb2) {
                        // transposed tile: C[s][t] = sum_i Y[s][i] X[t][i]
                        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                        acc = tile_mma<T, D>(acc, Y + sb * 16 * LDD, LDD, X + tb2 * 16 * LDD, LDD,
                                             lane);
                        const float lt = sLam[t];
                        const float sc = (wave < 2) ? sBv[t] : ((wave == 3) ? -1.f : 1.f);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int s = s0 + r;
                            const bool keep = strict ? (s < t) : (s <= t);
                            const float dec = exp2f(keep ? (lt - sLam[s]) : -200.f);
                            val[r] = keep ? acc[r] * sc * dec : 0.f;
                        }
                    }
                    if (wave == 0) {
                        if (sb <= tb2) {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                sF[t * kFLd + s0 + r] = val[r];
                        }
                    } else {
                        store4(dstM + t * LDC + s0, val);
                    }
                }
            }
        }
        __syncthreads();

        // ---- UT transform Tm = (I + A_kk)^-1 in fp32 ----
        // sF: A_kk[t][s] in the strict lower triangle; Tm[t][s] (s < t) is written
        // transposed into the strict upper triangle, Tm[t][t] = 1 implicit.
        if (wave == 0) {                                   // diagonal 16x16 blocks
            const int bi = lane >> 4, j = lane & 15;
            const float* A = sF + (bi * 16) * kFLd + bi * 16;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int c = 0; c < r; ++c)
                    acc -= A[r * kFLd + c] * x[c];
                x[r] = acc;
            }
            float* dst = sF + (bi * 16 + j) * kFLd + bi * 16;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (r > j)
                    dst[r] = x[r];
        }
        __syncthreads();
        for (int d = 1; d < 4; ++d) {                      // off-diagonal blocks, by distance
            const int bi = wave + d, bj = wave;            // block (bi, bj)
            const bool active = wave < 4 - d;
            float* Pw = sP + wave * 16 * kPLd;
            if (active) {                                  // P = sum_{m=bj}^{bi-1} A_{bi,m} Tm_{m,bj}
                f32x4_t p = {0.f, 0.f, 0.f, 0.f};
                const int tcol = bj * 16 + (lane & 15);
                for (int kk = 0; kk < 16 * d; kk += 4) {
                    const int kc = bj * 16 + kk + (lane >> 4);
                    const float av = sF[(bi * 16 + (lane & 15)) * kFLd + kc];
                    const float tv = kc > tcol ? sF[tcol * kFLd + kc] : (kc == tcol ? 1.f : 0.f);
                    p = mma_f32(av, tv, p);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Pw[((lane >> 4) * 4 + r) * kPLd + (lane & 15)] = p[r];
            }
            __syncthreads();
            if (active) {                                  // Tm_{bi,bj} = -Tm_{bi,bi} P
                f32x4_t ta = {0.f, 0.f, 0.f, 0.f};
                const int rr = lane & 15;
#pragma unroll
                for (int kk = 0; kk < 16; kk += 4) {
                    const int kc = kk + (lane >> 4);
                    const float av = rr > kc ? sF[(bi * 16 + kc) * kFLd + bi * 16 + rr]
                                             : (rr == kc ? 1.f : 0.f);
                    const float bv = Pw[kc * kPLd + (lane & 15)];
                    ta = mma_f32(av, bv, ta);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sF[(bj * 16 + (lane & 15)) * kFLd + bi * 16 + (lane >> 4) * 4 + r] = -ta[r];
            }
            __syncthreads();
        }
        if constexpr (kBf) {                               // Tm as a bf16 operand [t][s]
            for (int idx = tid; idx < kC * kC; idx += kThreads) {
                const int t = idx >> 6, s = idx & 63;
                const float tv = s < t ? sF[s * kFLd + t] : (s == t ? 1.f : 0.f);
                sT[t * LDC + s] = f32_to_bf16(tv);
            }
            __syncthreads();
        }

        // ---- incoming state as an operand: S0^T [j][i] ----
#pragma unroll
        for (int qd = 0; qd < NSW; ++qd) {
            const int sidx = wave * NSW + qd, ib = sidx / NJ, jb = sidx % NJ;
            store4(sS0t + (jb * 16 + (lane & 15)) * LDD + ib * 16 + (lane >> 4) * 4, S[qd]);
        }
        __syncthreads();

        // ---- R = diag(b gamma) K S0 + A_kkw V ----
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            acc = tile_mma<T, D>(acc, sK + tb * 16 * LDD, LDD, sS0t + jb * 16 * LDD, LDD, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = tb * 16 + (lane >> 4) * 4 + r;
                acc[r] *= sBv[t] * exp2f(sLam[t]);
            }
            acc = tile_mma_n<T>(acc, sAkkw + tb * 16 * LDC, LDC, sVt + jb * 16 * LDC, LDC, kTri, lane);
            store4(sRt + (jb * 16 + (lane & 15)) * LDC + tb * 16 + (lane >> 4) * 4, acc);
        }
        __syncthreads();

        // ---- X = Tm R ----
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            if constexpr (kBf) {
                acc = tile_mma_n<T>(acc, sT + tb * 16 * LDC, LDC, sRt + jb * 16 * LDC, LDC, kTri,
                                    lane);
            } else {
                const int t = tb * 16 + (lane & 15);
                for (int kk = 0; kk < 16 * (tb + 1); kk += 4) {
                    const int s = kk + (lane >> 4);
                    const float tv = s < t ? sF[s * kFLd + t] : (s == t ? 1.f : 0.f);
                    const float rv = to_f32(sRt[(jb * 16 + (lane & 15)) * LDC + s]);
                    acc = mma_f32(tv, rv, acc);
                }
            }
            store4(sXt + (jb * 16 + (lane & 15)) * LDC + tb * 16 + (lane >> 4) * 4, acc);
        }
        __syncthreads();

        // ---- O = diag(gamma) Q S0 + A_qkw V - A_qk X ----
#pragma unroll
        for (int jb = 0; jb < NJ; ++jb) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            acc = tile_mma<T, D>(acc, sQ + tb * 16 * LDD, LDD, sS0t + jb * 16 * LDD, LDD, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[r] *= exp2f(sLam[tb * 16 + (lane >> 4) * 4 + r]);
            acc = tile_mma_n<T>(acc, sAqkw + tb * 16 * LDC, LDC, sVt + jb * 16 * LDC, LDC, kTri, lane);
            acc = tile_mma_n<T>(acc, sAqk + tb * 16 * LDC, LDC, sXt + jb * 16 * LDC, LDC, kTri, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = tb * 16 + (lane >> 4) * 4 + r;
                if (t < nt)
                    o[(int64_t)(c0 + t) * rowV + (int64_t)e * DV + j0 + jb * 16 + (lane & 15)] =
                        from_f32<T>(acc[r]);
            }
        }

        // ---- S <- gamma_C S0 + (diag(gamma_C/gamma) KW)^T V - (diag(gamma_C/gamma) K)^T X ----
        const float gC = exp2f(lamC);
#pragma unroll
        for (int qd = 0; qd < NSW; ++qd) {
            const int sidx = wave * NSW + qd, ib = sidx / NJ, jb = sidx % NJ;
            f32x4_t acc = S[qd];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[r] *= gC;
            if constexpr (kBf) {
                acc = tile_mma<T, kC>(acc, sKWt + ib * 16 * LDC, LDC, sVt + jb * 16 * LDC, LDC, lane);
                acc = tile_mma<T, kC>(acc, sKt + ib * 16 * LDC, LDC, sXt + jb * 16 * LDC, LDC, lane);
            } else {
                const int i = ib * 16 + (lane & 15);
                for (int kk = 0; kk < kC; kk += 4) {
                    const int s = kk + (lane >> 4);
                    const float fac = exp2f(lamC - sLam[s]);
                    const float akw = to_f32(sKW[s * LDD + i]) * fac;
                    const float ak = -to_f32(sK[s * LDD + i]) * fac;
                    const float bv = to_f32(sVt[(jb * 16 + (lane & 15)) * LDC + s]);
                    const float bx = to_f32(sXt[(jb * 16 + (lane & 15)) * LDC + s]);
                    acc = mma_f32(akw, bv, acc);
                    acc = mma_f32(ak, bx, acc);
                }
            }
            S[qd] = acc;
        }
        __syncthreads();
    }

    // ---- final state, fp32 [n_seqs, H, dk, dv] ----
#pragma unroll
    for (int qd = 0; qd < NSW; ++qd) {
        const int sidx = wave * NSW + qd, ib = sidx / NJ, jb = sidx % NJ;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ib * 16 + (lane >> 4) * 4 + r;
            s_final[(((int64_t)n * H + e) * D + i) * DV + j0 + jb * 16 + (lane & 15)] = S[qd][r];
        }
    }
}

template <typename T, int D, int DVS>
static hipError_t launch(const ScanArgs& p, hipStream_t stream)
{
    const int n_slices = p.dv / DVS;
    const int64_t blocks = (int64_t)p.n_seqs * p.heads * n_slices;
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL((chunk_scan_kernel<T, D, DVS>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, (const T*)p.q, (const T*)p.k, (const T*)p.kw, (const T*)p.v,
                       (const T*)p.g, (const T*)p.b, p.cu_seqlens, p.heads, p.dv, n_slices,
                       (T*)p.o, p.s_final);
    return hipGetLastError();
}

bool scan_supported(bool bf16, int dk, int dv, int dvs)
{
    if (dv % dvs != 0 || (dv != 64 && dv != 128))
        return false;
    if (bf16) {
        if (dk == 64) return dvs == 16 || dvs == 32 || dvs == 64;
        if (dk == 128) return dvs == 16 || dvs == 32;
        return false;
    }
    return dk == 64 && (dvs == 16 || dvs == 32);
}

hipError_t launch_scan(const ScanArgs& p, hipStream_t s)
{
    if (!scan_supported(p.bf16, p.dk, p.dv, p.dv_slice))
        return hipErrorInvalidValue;
    if (p.bf16) {
        if (p.dk == 64) {
            if (p.dv_slice == 16) return launch<uint16_t, 64, 16>(p, s);
            if (p.dv_slice == 32) return launch<uint16_t, 64, 32>(p, s);
            return launch<uint16_t, 64, 64>(p, s);
        }
        if (p.dv_slice == 16) return launch<uint16_t, 128, 16>(p, s);
        return launch<uint16_t, 128, 32>(p, s);
    }
    if (p.dv_slice == 16) return launch<float, 64, 16>(p, s);
    return launch<float, 64, 32>(p, s);
}

}  // namespace prism
