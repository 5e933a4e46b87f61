// chunk_scan_bf16.hip -- bf16 chunkwise scan with a register-resident state path
//
// Same recurrence and chunk algebra as chunk_scan.hip (gated delta rule,
// chunks of 64 tokens, WY/UT form; PRISM pages: WeChat ICML 2026 summary,
// section 消除 Token 间串行; gist.science summary of arXiv 2602.10796,
// section 2.1).  This variant evaluates the UT system blockwise:
//
//   (I + A_kk) X = R,  A_kk strictly lower, split into 16x16 blocks A_ij:
//   X_i = T_ii (R_i - sum_{j<i} A_ij X_j),   T_ii = (I + A_ii)^-1,
//
// so only the four 16x16 diagonal inverses are formed (one per wavefront,
// by substitution in fp32) and the off-diagonal coupling is applied on the
// state path itself.
//
// Per chunk there are three barriers:
//   1. stage q, k, kw, v (prefetched into registers during the previous
//      chunk) and the gates into LDS;
//   2. Gram blocks with masks and decays (every wavefront takes its diagonal
//      (t, s) block pair and one or two off-diagonal pairs), then each
//      wavefront inverts the diagonal block it built;
//   3. the state path.  Wavefront jb owns 16 value columns of S (fp32, in
//      MFMA accumulators) and carries them through
//        S <- gamma_C S + KW^T diag(gamma_C/gamma) V
//        R  = diag(b gamma) K S0 + A_kkw V
//        X  = blockwise UT solve (above)
//        O  = diag(gamma) Q S0 + A_qkw V - A_qk X
//        S <- S - K^T diag(gamma_C/gamma) X
//      entirely in registers: products whose right operand is an
//      intermediate (X, R - A X) use v_mfma_f32_16x16x16_bf16, whose B
//      operand layout is exactly the accumulator layout of a 16x16 tile, so
//      no intermediate is written to LDS.  S0^T for the next chunk's K S0 and
//      Q S0 products goes to LDS rows private to the wavefront.
#include "common.h"
#include "kernels.h"

namespace prism {
namespace bf16scan {

constexpr int kC = 64;
constexpr int kThreads = 256;

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef short v8s_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

__device__ __forceinline__ v4s_t lds_read_tr(const uint16_t* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(const_cast<uint16_t*>(p)));
}

// 16x16x32 operand fragments (row m = lane % 16, k = 8 (lane / 16) + 0..7).
//   row(p, ld): element (m, k) at p[m * ld + k]
//   col(p, ld): element (m, k) at p[k * ld + m]   (two transposed LDS reads)
__device__ __forceinline__ bf16x8_t frag_row(const uint16_t* p, int ld, int lane)
{
    return __builtin_bit_cast(bf16x8_t,
                              *reinterpret_cast<const uint4*>(p + (lane & 15) * ld + (lane >> 4) * 8));
}
__device__ __forceinline__ bf16x8_t frag_col(const uint16_t* p, int ld, int lane)
{
    const int i = lane & 15;
    const uint16_t* a = p + ((lane >> 4) * 8 + (i >> 2)) * ld + (i & 3) * 4;
    v8s_t x = __builtin_shufflevector(lds_read_tr(a), lds_read_tr(a + 4 * ld), 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, x);
}
// 16x16x16 operand fragments (row m = lane % 16, k = 4 (lane / 16) + 0..3).
__device__ __forceinline__ v4s_t frag4_row(const uint16_t* p, int ld, int lane)
{
    return *reinterpret_cast<const v4s_t*>(p + (lane & 15) * ld + (lane >> 4) * 4);
}
__device__ __forceinline__ v4s_t frag4_col(const uint16_t* p, int ld, int lane)
{
    const int i = lane & 15;
    return lds_read_tr(p + ((lane >> 4) * 4 + (i >> 2)) * ld + (i & 3) * 4);
}

// Inclusive prefix sum over the 64 lanes with DPP row shifts and row
// broadcasts (no LDS round trips).
__device__ __forceinline__ float dpp_add(float v, int t) { return v + __int_as_float(t); }
__device__ __forceinline__ float wave_inclusive_sum(float v)
{
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));
    v = dpp_add(v, __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));
    return v;
}

// Scale the eight k-entries of a 16x16x32 fragment (k = 8 (lane / 16) + e)
// by f[k]: used to fold diag(gamma_C / gamma) into the V operand.
__device__ __forceinline__ bf16x8_t scale_k(bf16x8_t x, const float* f, int lane)
{
    const float4 f0 = *reinterpret_cast<const float4*>(f + (lane >> 4) * 8);
    const float4 f1 = *reinterpret_cast<const float4*>(f + (lane >> 4) * 8 + 4);
    const uint4 w = __builtin_bit_cast(uint4, x);
    const float fv[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = pack_bf16x2(__uint_as_float(wv[i] << 16) * fv[2 * i],
                           __uint_as_float(wv[i] & 0xffff0000u) * fv[2 * i + 1]);
    return __builtin_bit_cast(bf16x8_t, make_uint4(r[0], r[1], r[2], r[3]));
}

__device__ __forceinline__ f32x4_t mma32(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma16(v4s_t a, v4s_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// An accumulator tile as the B operand of a 16x16x16 product (bf16, scaled).
__device__ __forceinline__ v4s_t as_b16(f32x4_t x, float s0, float s1, float s2, float s3)
{
    return __builtin_bit_cast(v4s_t, make_uint2(pack_bf16x2(x[0] * s0, x[1] * s1),
                                                pack_bf16x2(x[2] * s2, x[3] * s3)));
}

__device__ __forceinline__ void st4(uint16_t* p, f32x4_t x)
{
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
}

template <int D, int DVS>
struct Layout {
    static constexpr int LDD = D + 8;            // [64][D] tiles and S0^T [DVS][D]
    static constexpr int LDC = kC + 8;           // [64][64] matrices
    static constexpr int LDV = DVS + 8;          // [64][DVS] value tiles
    static constexpr int LDT = 16 + 8;           // diagonal inverse blocks [4][16][16]
    static constexpr int szRowD = kC * LDD * 2;
    static constexpr int szV = kC * LDV * 2;
    static constexpr int szM = kC * LDC * 2;
    static constexpr int szTd = kC * LDT * 2;
    static constexpr int szS0t = DVS * LDD * 2;
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + szRowD;
    static constexpr int oKW = oK + szRowD;
    static constexpr int oV = oKW + szRowD;
    static constexpr int oAkk = oV + szV;        // four matrices, then S0^T: zeroed once
    static constexpr int oAkkw = oAkk + szM;
    static constexpr int oAqkw = oAkkw + szM;
    static constexpr int oAqk = oAqkw + szM;
    static constexpr int oS0t = oAqk + szM;
    static constexpr int oTd = oS0t + szS0t;
    static constexpr int oG = oTd + szTd;
    static constexpr int total = oG + 4 * kC * 4;
    static_assert(oAkk % 16 == 0 && oS0t % 16 == 0 && oTd % 16 == 0 && oG % 16 == 0, "alignment");
};

// Off-diagonal (t-block, s-block) pairs; wavefront w takes kOff[w] and kOff[w + 4].
__constant__ const int kOffT[6] = {1, 2, 2, 3, 3, 3};
__constant__ const int kOffS[6] = {0, 0, 1, 0, 1, 2};

template <int D, int DVS>
__global__ __launch_bounds__(kThreads) void scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ kw, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ b,
    const int32_t* __restrict__ cu, int H, int DV, int n_slices, uint16_t* __restrict__ o,
    float* __restrict__ s_final)
{
    using Ly = Layout<D, DVS>;
    constexpr int LDD = Ly::LDD, LDC = Ly::LDC, LDV = Ly::LDV, LDT = Ly::LDT;
    constexpr int NJ = DVS / 16;                 // state wavefronts (one per 16 value columns)
    constexpr int NI = D / 16;                   // 16-row blocks of S
    constexpr int NQ = kC * D / 8 / kThreads;    // q / k / kw 16-byte vectors per thread
    constexpr int NVV = kC * DVS / 8;            // v vectors per chunk
    constexpr int NVT = (NVV + kThreads - 1) / kThreads;
    static_assert(NJ >= 1 && NJ <= 4, "value slice");
    static_assert(Ly::total <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(16))) unsigned char smem[Ly::total];
    uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + Ly::oQ);
    uint16_t* sK = reinterpret_cast<uint16_t*>(smem + Ly::oK);
    uint16_t* sKW = reinterpret_cast<uint16_t*>(smem + Ly::oKW);
    uint16_t* sV = reinterpret_cast<uint16_t*>(smem + Ly::oV);
    uint16_t* sAkk = reinterpret_cast<uint16_t*>(smem + Ly::oAkk);
    uint16_t* sAkkw = reinterpret_cast<uint16_t*>(smem + Ly::oAkkw);
    uint16_t* sAqkw = reinterpret_cast<uint16_t*>(smem + Ly::oAqkw);
    uint16_t* sAqk = reinterpret_cast<uint16_t*>(smem + Ly::oAqk);   // holds -A_qk
    uint16_t* sS0t = reinterpret_cast<uint16_t*>(smem + Ly::oS0t);
    uint16_t* sTd = reinterpret_cast<uint16_t*>(smem + Ly::oTd);
    float* sLam = reinterpret_cast<float*>(smem + Ly::oG);
    float* sBv = sLam + kC;
    float* sGam = sBv + kC;
    float* sFac = sGam + kC;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const int slice = (int)(blockIdx.x % (unsigned)n_slices);
    const int chain = (int)(blockIdx.x / (unsigned)n_slices);
    const int n = chain / H, e = chain % H;
    const int j0 = slice * DVS;
    const int seq0 = cu[n], seq1 = cu[n + 1];
    const int nchunks = (seq1 - seq0 + kC - 1) / kC;
    const int64_t rowQK = (int64_t)H * D, rowV = (int64_t)H * DV;

    {
        constexpr int nz = (4 * Ly::szM + Ly::szS0t) / 16;
        uint4* z = reinterpret_cast<uint4*>(smem + Ly::oAkk);
        for (int i = tid; i < nz; i += kThreads)
            z[i] = make_uint4(0u, 0u, 0u, 0u);
    }

    f32x4_t S[NI];                               // S[:, 16 jb : 16 jb + 16] of wavefront jb
#pragma unroll
    for (int i = 0; i < NI; ++i)
        S[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // ---- register prefetch (per-thread offsets fixed across chunks) ----
    int offq[NQ], tq[NQ], offv[NVT], tv[NVT];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int idx = tid + j * kThreads;
        tq[j] = idx / (D / 8);
        offq[j] = tq[j] * H * D + e * D + (idx % (D / 8)) * 8;
    }
#pragma unroll
    for (int j = 0; j < NVT; ++j) {
        const int idx = tid + j * kThreads;
        tv[j] = idx < NVV ? idx / (DVS / 8) : kC;
        offv[j] = (idx / (DVS / 8)) * H * DV + e * DV + j0 + (idx % (DVS / 8)) * 8;
    }
    uint4 pq[NQ], pk[NQ], pw[NQ], pv[NVT];
    uint16_t pg = 0x3f80u, pb = 0u;              // bf16 1.0 and 0.0
    auto prefetch = [&](int ch) {
        const int c0 = seq0 + ch * kC;
        const int nt = min(kC, seq1 - c0);
        const uint16_t* bq = q + (int64_t)c0 * rowQK;
        const uint16_t* bk = k + (int64_t)c0 * rowQK;
        const uint16_t* bw = kw + (int64_t)c0 * rowQK;
        const uint16_t* bv = v + (int64_t)c0 * rowV;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            pq[j] = pk[j] = pw[j] = make_uint4(0u, 0u, 0u, 0u);
            if (tq[j] < nt) {
                pq[j] = *reinterpret_cast<const uint4*>(bq + offq[j]);
                pk[j] = *reinterpret_cast<const uint4*>(bk + offq[j]);
                pw[j] = *reinterpret_cast<const uint4*>(bw + offq[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NVT; ++j) {
            pv[j] = make_uint4(0u, 0u, 0u, 0u);
            if (tv[j] < nt)
                pv[j] = *reinterpret_cast<const uint4*>(bv + offv[j]);
        }
        pg = 0x3f80u;                            // kept raw: no wait on this prefetch now
        pb = 0u;
        if (lane < nt) {
            pg = g[(int64_t)(c0 + lane) * H + e];
            pb = b[(int64_t)(c0 + lane) * H + e];
        }
    };
    if (nchunks > 0)
        prefetch(0);
    __syncthreads();

    for (int ch = 0; ch < nchunks; ++ch) {
        const int c0 = seq0 + ch * kC;
        const int nt = min(kC, seq1 - c0);

        // ================= 1. gates (every wavefront, lane = token) and staging =================
        const float lam = wave_inclusive_sum(__log2f(fmaxf(bf16_to_f32(pg), 1e-30f)));
        const float lamC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), 63));
        if (wave == 0) {
            sLam[lane] = lam;
            sBv[lane] = bf16_to_f32(pb);
            sGam[lane] = __builtin_amdgcn_exp2f(lam);
            sFac[lane] = __builtin_amdgcn_exp2f(lamC - lam);      // gamma_C / gamma_t <= 1
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int idx = tid + j * kThreads;
            const int t = idx / (D / 8), c = (idx % (D / 8)) * 8;
            *reinterpret_cast<uint4*>(sQ + t * LDD + c) = pq[j];
            *reinterpret_cast<uint4*>(sK + t * LDD + c) = pk[j];
            *reinterpret_cast<uint4*>(sKW + t * LDD + c) = pw[j];
        }
#pragma unroll
        for (int j = 0; j < NVT; ++j) {
            const int idx = tid + j * kThreads;
            const int t = idx / (DVS / 8), c = (idx % (DVS / 8)) * 8;
            if (idx < NVV)
                *reinterpret_cast<uint4*>(sV + t * LDV + c) = pv[j];
        }
        if (ch + 1 < nchunks)
            prefetch(ch + 1);
        __syncthreads();

        // ================= 2. Gram blocks, masks; diagonal inverse of block `wave` =================
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            int tb, sb;
            if (u < 2) {
                const int p = wave + 4 * u;
                if (p >= 6)
                    continue;
                tb = kOffT[p];
                sb = kOffS[p];
            } else {
                tb = sb = wave;                  // diagonal pair last: its inverse follows
            }
            f32x4_t gkk = {0.f, 0.f, 0.f, 0.f}, gkw = gkk, gqk = gkk, gqw = gkk;
            const uint16_t* yk = sK + sb * 16 * LDD;
            const uint16_t* yw = sKW + sb * 16 * LDD;
            const uint16_t* xk = sK + tb * 16 * LDD;
            const uint16_t* xq = sQ + tb * 16 * LDD;
#pragma unroll
            for (int kk = 0; kk < D; kk += 32) {
                bf16x8_t ak = frag_row(yk + kk, LDD, lane), aw = frag_row(yw + kk, LDD, lane);
                bf16x8_t bk = frag_row(xk + kk, LDD, lane), bq = frag_row(xq + kk, LDD, lane);
                gkk = mma32(ak, bk, gkk);        // transposed blocks: element (s, t)
                gkw = mma32(aw, bk, gkw);
                gqk = mma32(ak, bq, gqk);
                gqw = mma32(aw, bq, gqw);
            }
            const int t = tb * 16 + li;
            const int s0 = sb * 16 + lg * 4;
            const float lt = sLam[t], bt = sBv[t];
            const float4 ls = *reinterpret_cast<const float4*>(sLam + s0);
            const float lsv[4] = {ls.x, ls.y, ls.z, ls.w};
            f32x4_t vkk, vkw, vqk, vqw;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = s0 + r;
                const float dec = __builtin_amdgcn_exp2f(fminf(lt - lsv[r], 0.f));
                const float mi = s <= t ? dec : 0.f;
                const float ms = s < t ? dec * bt : 0.f;
                vkk[r] = ms * gkk[r];
                vkw[r] = ms * gkw[r];
                vqk[r] = -mi * gqk[r];
                vqw[r] = mi * gqw[r];
            }
            st4(sAkk + t * LDC + s0, vkk);
            st4(sAkkw + t * LDC + s0, vkw);
            st4(sAqk + t * LDC + s0, vqk);
            st4(sAqkw + t * LDC + s0, vqw);
        }
        {
            // T_ww = (I + A_ww)^-1 for the diagonal block this wavefront just wrote
            // (same-wavefront LDS ordering).  Column j = lane % 16 by substitution;
            // lane group g stores rows 4 g .. 4 g + 3.
            const uint16_t* A = sAkk + (wave * 16) * LDC + wave * 16;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint4 w0 = *reinterpret_cast<const uint4*>(A + r * LDC);
                const uint4 w1 = *reinterpret_cast<const uint4*>(A + r * LDC + 8);
                const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
                float acc = (r == li) ? 1.f : 0.f;
#pragma unroll
                for (int c = 0; c < r; ++c) {
                    const uint32_t h2 = wv[c >> 1];
                    const float a = __uint_as_float((c & 1) ? (h2 & 0xffff0000u) : (h2 << 16));
                    acc -= a * x[c];
                }
                x[r] = acc;
            }
            uint16_t* Td = sTd + (wave * 16) * LDT + li;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if ((r >> 2) == lg)
                    Td[r * LDT] = f32_to_bf16(x[r]);
        }
        __syncthreads();

        // ================= 3. state path: wavefront jb, value columns 16 jb .. 16 jb + 15 =================
        if (wave < NJ) {
            const int jb = wave;
            const float gC = __builtin_amdgcn_exp2f(lamC);
            const uint16_t* s0t = sS0t + jb * 16 * LDD;

            // a. S <- gamma_C S + KW^T diag(fac) V
            bf16x8_t vf[2], vs[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                vf[h2] = frag_col(sV + h2 * 32 * LDV + jb * 16, LDV, lane);
                vs[h2] = scale_k(vf[h2], sFac + h2 * 32, lane);
            }
#pragma unroll
            for (int ib = 0; ib < NI; ++ib) {
                f32x4_t acc = S[ib];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[r] *= gC;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                    acc = mma32(frag_col(sKW + h2 * 32 * LDD + ib * 16, LDD, lane), vs[h2], acc);
                S[ib] = acc;
            }

            // b. R_tb = diag(b gamma) (K S0)_tb + A_kkw V ;  O partial = diag(gamma) (Q S0)_tb + A_qkw V
            bf16x8_t sf[D / 32];
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                sf[kk] = frag_row(s0t + kk * 32, LDD, lane);
            f32x4_t R[4], O[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                f32x4_t ra = {0.f, 0.f, 0.f, 0.f}, oa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < D / 32; ++kk) {
                    ra = mma32(frag_row(sK + tb * 16 * LDD + kk * 32, LDD, lane), sf[kk], ra);
                    oa = mma32(frag_row(sQ + tb * 16 * LDD + kk * 32, LDD, lane), sf[kk], oa);
                }
                const float4 gm = *reinterpret_cast<const float4*>(sGam + tb * 16 + lg * 4);
                const float4 bb = *reinterpret_cast<const float4*>(sBv + tb * 16 + lg * 4);
                const float gmv[4] = {gm.x, gm.y, gm.z, gm.w}, bbv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ra[r] *= bbv[r] * gmv[r];
                    oa[r] *= gmv[r];
                }
#pragma unroll
                for (int h2 = 0; h2 < (tb + 2) / 2; ++h2) {
                    ra = mma32(frag_row(sAkkw + tb * 16 * LDC + h2 * 32, LDC, lane), vf[h2], ra);
                    oa = mma32(frag_row(sAqkw + tb * 16 * LDC + h2 * 32, LDC, lane), vf[h2], oa);
                }
                R[tb] = ra;
                O[tb] = oa;
            }

            // c. X_i = T_ii (R_i - sum_{j<i} A_ij X_j)   (16x16x16, B operands from registers)
            f32x4_t X[4];
            v4s_t nX[4];                         // -X_j as bf16 B operands
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f32x4_t y = R[i];
#pragma unroll
                for (int j = 0; j < i; ++j)
                    y = mma16(frag4_row(sAkk + i * 16 * LDC + j * 16, LDC, lane), nX[j], y);
                f32x4_t x = {0.f, 0.f, 0.f, 0.f};
                x = mma16(frag4_row(sTd + i * 16 * LDT, LDT, lane), as_b16(y, 1.f, 1.f, 1.f, 1.f), x);
                X[i] = x;
                nX[i] = as_b16(x, -1.f, -1.f, -1.f, -1.f);
            }

            // d. O_tb += -A_qk X  (sAqk holds -A_qk); rows past the chunk's last
            //    token fall outside the buffer range and are dropped by the hardware
            const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                o + (int64_t)c0 * rowV, 0, nt * (int)rowV * 2, 0x00020000);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                f32x4_t oa = O[tb];
#pragma unroll
                for (int sb = 0; sb <= tb; ++sb)
                    oa = mma16(frag4_row(sAqk + tb * 16 * LDC + sb * 16, LDC, lane),
                               as_b16(X[sb], 1.f, 1.f, 1.f, 1.f), oa);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = tb * 16 + lg * 4 + r;
                    __builtin_amdgcn_raw_buffer_store_b16(
                        f32_to_bf16(oa[r]), orsrc, (t * (int)rowV + e * DV + j0 + jb * 16 + li) * 2, 0, 0);
                }
            }

            // e. S <- S - K^T diag(fac) X ;  f. S0^T for the next chunk (rows private to jb)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float4 fv = *reinterpret_cast<const float4*>(sFac + tb * 16 + lg * 4);
                const v4s_t bx = as_b16(X[tb], -fv.x, -fv.y, -fv.z, -fv.w);
#pragma unroll
                for (int ib = 0; ib < NI; ++ib)
                    S[ib] = mma16(frag4_col(sK + tb * 16 * LDD + ib * 16, LDD, lane), bx, S[ib]);
            }
#pragma unroll
            for (int ib = 0; ib < NI; ++ib)
                st4(sS0t + (jb * 16 + li) * LDD + ib * 16 + lg * 4, S[ib]);
        }
        __syncthreads();
    }

    if (wave < NJ) {
        const int jb = wave;
#pragma unroll
        for (int ib = 0; ib < NI; ++ib) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ib * 16 + lg * 4 + r;
                s_final[(((int64_t)n * H + e) * D + i) * DV + j0 + jb * 16 + li] = S[ib][r];
            }
        }
    }
}

template <int D, int DVS>
static hipError_t launch(const ScanArgs& p, hipStream_t stream)
{
    const int n_slices = p.dv / DVS;
    const int64_t blocks = (int64_t)p.n_seqs * p.heads * n_slices;
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL((scan_kernel<D, DVS>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.kw,
                       (const uint16_t*)p.v, (const uint16_t*)p.g, (const uint16_t*)p.b,
                       p.cu_seqlens, p.heads, p.dv, n_slices, (uint16_t*)p.o, p.s_final);
    return hipGetLastError();
}

}  // namespace bf16scan

bool scan_bf16_supported(int dk, int dv, int dvs)
{
    if (dv % dvs != 0 || (dv != 64 && dv != 128))
        return false;
    return (dk == 64 || dk == 128) && (dvs == 16 || dvs == 32 || dvs == 64);
}

hipError_t launch_scan_bf16(const ScanArgs& p, hipStream_t s)
{
    if (!scan_bf16_supported(p.dk, p.dv, p.dv_slice))
        return hipErrorInvalidValue;
    if (p.dk == 64) {
        if (p.dv_slice == 16) return bf16scan::launch<64, 16>(p, s);
        if (p.dv_slice == 32) return bf16scan::launch<64, 32>(p, s);
        return bf16scan::launch<64, 64>(p, s);
    }
    if (p.dv_slice == 16) return bf16scan::launch<128, 16>(p, s);
    if (p.dv_slice == 32) return bf16scan::launch<128, 32>(p, s);
    return bf16scan::launch<128, 64>(p, s);
}

}  // namespace prism
