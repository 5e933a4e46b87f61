// chunk_scan_bf16.hip -- bf16 chunkwise scans with a register-resident state path
//
// Same recurrence and chunk algebra as chunk_scan.hip (gated delta rule,
// chunks of 64 tokens, WY/UT form; PRISM pages: WeChat ICML 2026 summary,
// section 消除 Token 间串行; gist.science summary of arXiv 2602.10796,
// section 2.1).  The UT system is evaluated blockwise:
//
//   (I + A_kk) X = R,  A_kk strictly lower, split into 16x16 blocks A_ij:
//   X_i = T_ii (R_i - sum_{j<i} A_ij X_j),   T_ii = (I + A_ii)^-1,
//
// so only the four 16x16 diagonal inverses are formed (by substitution in
// fp32) and the off-diagonal coupling is applied on the state path itself.
//
// The state path: wavefront jb owns 16 value columns of S (fp32, in MFMA
// accumulators) and carries them through
//   S <- gamma_C S + KW^T diag(gamma_C/gamma) V
//   R  = diag(b gamma) K S0 + A_kkw V
//   X  = blockwise UT solve (above)
//   O  = diag(gamma) Q S0 + A_qkw V - A_qk X
//   S <- S - K^T diag(gamma_C/gamma) X
// entirely in registers: products with an intermediate operand (S0, X,
// R - A X) use v_mfma_f32_16x16x16_bf16, whose B operand layout (and, read
// transposed, whose A operand layout) is exactly the accumulator layout of a
// 16x16 tile, so no intermediate goes through LDS.
//
// Two kernels:
//   scan_kernel     every wavefront stages rows, builds Gram blocks and
//                   inverses, then the state wavefronts run the state path
//                   (three barriers per chunk); any value slice up to 64.
//   scan_ws_kernel  wavefront-specialised (slices of 16 or 32 columns):
//                   helper wavefronts prepare chunk c + 1 while the state
//                   wavefronts run chunk c (two barriers per chunk); four
//                   wavefronts, or eight (two per SIMD) for 32 columns.
#include "common.h"
#include "kernels.h"
#include "mfma_bf16.h"

namespace prism {
namespace bf16scan {

constexpr int kC = 64;
constexpr int kThreads = 256;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
// Cache-policy operand of a buffer access that is coherent at device scope
// (gfx950 sc1): written where, and read from where, every compute unit of
// every XCD sees the same data, whichever L2 it sits behind.
constexpr int kScopeDevice = 16;
constexpr int kNontemporal = 2;                  // cache-policy operand: streaming (nt)
constexpr int kProducerWaves = 8;                // wavefronts of a write-key producer block

using namespace mfma;

template <int D, int DVS>
struct Layout {
    static constexpr int LDD = D + 8;            // [64][D] tiles
    static constexpr int LDC = kC + 8;           // [64][64] matrices
    static constexpr int LDV = DVS + 8;          // [64][DVS] value tiles
    static constexpr int LDT = 16 + 8;           // diagonal inverse blocks [4][16][16]
    static constexpr int szRowD = kC * LDD * 2;
    static constexpr int szV = kC * LDV * 2;
    static constexpr int szM = kC * LDC * 2;
    static constexpr int szTd = kC * LDT * 2;
    static constexpr int oQ = 0;
    static constexpr int oK = oQ + szRowD;
    static constexpr int oKW = oK + szRowD;
    static constexpr int oV = oKW + szRowD;
    static constexpr int oAkk = oV + szV;        // four matrices: zeroed once
    static constexpr int oAkkw = oAkk + szM;
    static constexpr int oAqkw = oAkkw + szM;
    static constexpr int oAqk = oAqkw + szM;
    static constexpr int oTd = oAqk + szM;
    static constexpr int oG = oTd + szTd;
    static constexpr int total = oG + 5 * kC * 4;
    static_assert(oAkk % 16 == 0 && oTd % 16 == 0 && oG % 16 == 0, "alignment");
};


// The per-chunk state path of one wavefront (value columns 16 jb .. 16 jb + 15):
//   a. S <- gamma_C S + KW^T diag(fac) V
//   b. R = diag(b gamma) K S0 + A_kkw V;   O^T = (diag(gamma) Q S0 + A_qkw V)^T
//   c. X_i = T_ii (R_i - sum_{j<i} A_kk{ij} X_j)
//   d. O^T += -(A_qk X)^T (the tile holds -A_qk), stored as bf16
//   e. S <- S - K^T diag(fac) X
// S0, the state at the chunk start, enters b straight from the accumulators: a
// 16x16 fp32 accumulator tile converted to bf16 is both the B operand and the
// transposed A operand of a 16x16x16 product.  O is produced transposed, so a
// lane holds four consecutive value columns of one token (8-byte stores).
// All tiles are bf16 in LDS with the strides of Layout; S is fp32 in accumulators.
// T_ii is read from sTd, or with TD_IN_AKK from the diagonal blocks of A_kk
// (which the state path never needs otherwise), which then hold T_ii transposed.
// a. S <- gamma_C S + KW^T diag(fac) V for value columns 16 jb .. 16 jb + 15;
// first captures S0 (the state before the update) as bf16 16x16x16 operands in
// s0b and leaves the V fragments in vf for b.
template <int D, int DVS>
__device__ __forceinline__ void a_step(f32x4_t (&S)[D / 16], v4s_t (&s0b)[D / 16], bf16x8_t (&vf)[2],
                                       const uint16_t* sKW, const uint16_t* sV, const float* sFac,
                                       float gC, int jb, int lane)
{
    using Ly = Layout<D, DVS>;
    constexpr int LDD = Ly::LDD, LDV = Ly::LDV;
    constexpr int NI = D / 16;
    const int lg = lane >> 4;
#pragma unroll
    for (int ib = 0; ib < NI; ++ib)
        s0b[ib] = as_b16(S[ib], 1.f, 1.f, 1.f, 1.f);

    // LDS reads run a short, fixed distance ahead of their MFMAs: a wavefront
    // can wait precisely only for the oldest of at most 15 outstanding reads,
    // so each batch is kept small and issued a few steps before its use.
    bf16x8_t kwf[2][NI];
    float4 fc[4];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        vf[h2] = frag_col(sV + h2 * 32 * LDV + jb * 16, LDV, lane);
        fc[2 * h2] = *reinterpret_cast<const float4*>(sFac + h2 * 32 + lg * 8);
        fc[2 * h2 + 1] = *reinterpret_cast<const float4*>(sFac + h2 * 32 + lg * 8 + 4);
    }
    auto load_kw = [&](int ib) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
            kwf[h2][ib] = frag_col(sKW + h2 * 32 * LDD + ib * 16, LDD, lane);
    };
    // two 16-row blocks per step, so that each accumulator's second product is
    // not issued right behind its first (a dependent 16x16x32 product waits for
    // its predecessor's result)
    load_kw(0);
    load_kw(1);
    load_kw(2);
    load_kw(3);
    SCHED_FENCE();
    bf16x8_t vs[2];
    vs[0] = scale8(vf[0], fc[0], fc[1]);
    vs[1] = scale8(vf[1], fc[2], fc[3]);
#pragma unroll
    for (int ib = 0; ib < NI; ib += 2) {
        if (ib + 4 < NI) {
            load_kw(ib + 4);
            load_kw(ib + 5);
        }
        SCHED_FENCE();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            S[ib][r] *= gC;
            S[ib + 1][r] *= gC;
        }
        S[ib] = mma32(kwf[0][ib], vs[0], S[ib]);
        S[ib + 1] = mma32(kwf[0][ib + 1], vs[0], S[ib + 1]);
        S[ib] = mma32(kwf[1][ib], vs[1], S[ib]);
        S[ib + 1] = mma32(kwf[1][ib + 1], vs[1], S[ib + 1]);
        SCHED_FENCE();
    }
}

// With SPLIT the a-step has already run (a_step, which filled s0b and vf);
// otherwise state_path runs it first.
template <int D, int DVS, bool TD_IN_AKK = false, bool SPLIT = false>
__device__ __forceinline__ void state_path(
    f32x4_t (&S)[D / 16], v4s_t (&s0b)[D / 16], bf16x8_t (&vf)[2], const uint16_t* sQ,
    const uint16_t* sK, const uint16_t* sKW,
    const uint16_t* sV, const uint16_t* sAkk, const uint16_t* sAkkw, const uint16_t* sAqkw,
    const uint16_t* sAqk, const uint16_t* sTd, const float* sBG, const float* sGam,
    const float* sFac, float gC, uint16_t* o, int c0, int nt, int64_t rowV, int e, int DV,
    int j0, int jb, int lane)
{
    using Ly = Layout<D, DVS>;
    constexpr int LDD = Ly::LDD, LDC = Ly::LDC, LDT = Ly::LDT;
    constexpr int NI = D / 16;
    const int li = lane & 15, lg = lane >> 4;
    if constexpr (!SPLIT)
        a_step<D, DVS>(S, s0b, vf, sKW, sV, sFac, gC, jb, lane);

    // ---- b, one unit (two 16-token blocks 2 tp, 2 tp + 1; 32-channel step kp) at a
    //      time: four independent accumulator chains (R and O^T of both blocks)
    constexpr int NKP = NI / 2;
    constexpr int NU = 2 * NKP;                     // units
    // S0 as 16x16x32 operands pairing with 16-byte row reads of K and Q
    bf16x8_t s0q[NKP];
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp)
        s0q[kp] = pair_rows(s0b[2 * kp], s0b[2 * kp + 1]);
    bf16x8_t kf[NU][2], qf[NU][2];
    bf16x8_t akw[4][2], aqw[4][2];
    float4 bg[4];
    float go[4];
    v4s_t akk[6], td[4], aqk[10];
    auto load_unit = [&](int u) {
        const int tp = u / NKP, kp = u % NKP;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int tb = 2 * tp + h;
            kf[u][h] = frag_row(sK + tb * 16 * LDD + kp * 32, LDD, lane);
            qf[u][h] = frag_row(sQ + tb * 16 * LDD + kp * 32, LDD, lane);
        }
        if (kp == 0) {                              // per-block operands and gates
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tb = 2 * tp + h;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    if (h2 < (tb + 2) / 2) {
                        akw[tb][h2] = frag_row(sAkkw + tb * 16 * LDC + h2 * 32, LDC, lane);
                        aqw[tb][h2] = frag_row(sAqkw + tb * 16 * LDC + h2 * 32, LDC, lane);
                    }
                }
                bg[tb] = *reinterpret_cast<const float4*>(sBG + tb * 16 + lg * 4);
                go[tb] = sGam[tb * 16 + li];
            }
        }
        // the operands of c, spread over the last three units
        const int w = u - (NU - 3);
        if (w >= 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int idx = w * 4 + q;          // 0 .. 9: akk 0..5, td 6..9
                if (idx < 6) {
                    const int i2 = idx < 1 ? 1 : idx < 3 ? 2 : 3;
                    const int j2 = idx - (i2 * (i2 - 1)) / 2;
                    akk[idx] = frag4_row(sAkk + i2 * 16 * LDC + j2 * 16, LDC, lane);
                } else if (idx < 10) {
                    const int i2 = idx - 6;
                    td[i2] = TD_IN_AKK ? frag4_col(sAkk + i2 * 16 * LDC + i2 * 16, LDC, lane)
                                       : frag4_row(sTd + i2 * 16 * LDT, LDT, lane);
                }
            }
        }
    };
    // the operands of d, read while c runs
    auto load_aqk = [&]() {
#pragma unroll
        for (int n2 = 0; n2 < 10; ++n2) {
            const int i2 = n2 < 1 ? 0 : n2 < 3 ? 1 : n2 < 6 ? 2 : 3;
            const int j2 = n2 - (i2 * (i2 + 1)) / 2;
            aqk[n2] = frag4_row(sAqk + i2 * 16 * LDC + j2 * 16, LDC, lane);
        }
    };
    f32x4_t R[4], OT[4];
    constexpr int AHEAD_B = 1;                      // 4 reads per unit (+ per-block extras)
#pragma unroll
    for (int u = 0; u < AHEAD_B; ++u)
        load_unit(u);
    SCHED_FENCE();
    f32x4_t ra[2], oa[2];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int tp = u / NKP, kp = u % NKP;
        if (u + AHEAD_B < NU)
            load_unit(u + AHEAD_B);
        SCHED_FENCE();
        if (kp == 0) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                ra[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                oa[h] = ra[h];
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
            ra[h] = mma32(kf[u][h], s0q[kp], ra[h]);          // (K S0)[t][j]
#pragma unroll
        for (int h = 0; h < 2; ++h)
            oa[h] = mma32(s0q[kp], qf[u][h], oa[h]);          // (Q S0)^T[j][t]
        if (kp == NKP - 1) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tb = 2 * tp + h;
                const float bgv[4] = {bg[tb].x, bg[tb].y, bg[tb].z, bg[tb].w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    ra[h][r] *= bgv[r];
                    oa[h][r] *= go[tb];
                }
            }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int tb = 2 * tp + h;
                    if (h2 < (tb + 2) / 2)
                        ra[h] = mma32(akw[tb][h2], vf[h2], ra[h]);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int tb = 2 * tp + h;
                    if (h2 < (tb + 2) / 2)
                        oa[h] = mma32(vf[h2], aqw[tb][h2], oa[h]);   // (A_qkw V)^T
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                R[2 * tp + h] = ra[h];
                OT[2 * tp + h] = oa[h];
            }
        }
        SCHED_FENCE();
    }

    // reads for e (first 32 tokens) and its scales: K^T fragments with tokens
    // 8g .. 8g+7 of each 32-token pair in lane group g
    bf16x8_t ke[2][NI];
    float4 fe[4];
    auto load_e = [&](int tp) {
#pragma unroll
        for (int ib = 0; ib < NI; ++ib)
            ke[tp][ib] = frag_col(sK + tp * 32 * LDD + ib * 16, LDD, lane);
        fe[2 * tp] = *reinterpret_cast<const float4*>(sFac + tp * 32 + lg * 4);
        fe[2 * tp + 1] = *reinterpret_cast<const float4*>(sFac + tp * 32 + 16 + lg * 4);
    };
    load_e(0);
    load_aqk();
    SCHED_FENCE();

    // ---- c. X_i = T_ii (R_i - sum_{j<i} A_ij X_j)   (16x16x16, B operands from registers)
    f32x4_t X[4];
    v4s_t nX[4];                         // -X_j as bf16 B operands
#pragma unroll
    for (int i = 0, n = 0; i < 4; ++i) {
        f32x4_t y = R[i];
#pragma unroll
        for (int j = 0; j < i; ++j, ++n)
            y = mma16(akk[n], nX[j], y);
        f32x4_t x = {0.f, 0.f, 0.f, 0.f};
        x = mma16(td[i], as_b16(y, 1.f, 1.f, 1.f, 1.f), x);
        X[i] = x;
        nX[i] = as_b16(x, -1.f, -1.f, -1.f, -1.f);
    }
    SCHED_FENCE();
    load_e(1);
    SCHED_FENCE();

    // ---- d. O^T += X^T (-A_qk)^T; token rows past the chunk's last token fall
    //      outside the buffer range and are dropped by the hardware
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        o + (int64_t)c0 * rowV, 0, nt * (int)rowV * 2, 0x00020000);
    v4s_t xb[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
        xb[sb] = as_b16(X[sb], 1.f, 1.f, 1.f, 1.f);
    const v4s_t zero4 = {0, 0, 0, 0};
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int n = tb * (tb + 1) / 2;             // aqk[n + sb] is block (tb, sb)
        f32x4_t oa = OT[tb];
        // every product of the chain is 16x16x32 (an odd block is paired with a
        // zero block): a dependent 16x16x16 and 16x16x32 pair whose results the
        // compiler places two registers apart corrupts the accumulator
#pragma unroll
        for (int sb = 0; sb <= tb; sb += 2) {
            if (sb + 1 <= tb)
                oa = mma32(cat8(xb[sb], xb[sb + 1]), cat8(aqk[n + sb], aqk[n + sb + 1]), oa);
            else
                oa = mma32(cat8(xb[sb], zero4), cat8(aqk[n + sb], zero4), oa);
        }
        // lane (li, lg): token tb * 16 + li, value columns 4 lg .. 4 lg + 3 of block jb
        const int t = tb * 16 + li;
        typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t w = {pack_bf16x2(oa[0], oa[1]), pack_bf16x2(oa[2], oa[3])};
        __builtin_amdgcn_raw_buffer_store_b64(w, orsrc, (t * (int)rowV + e * DV + j0 + jb * 16 + lg * 4) * 2,
                                              0, 0);
    }

    // ---- e. S <- S - K^T diag(fac) X   (NI independent accumulators per block)
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
        const bf16x8_t bx = pair_rows(
            as_b16(X[2 * tp], -fe[2 * tp].x, -fe[2 * tp].y, -fe[2 * tp].z, -fe[2 * tp].w),
            as_b16(X[2 * tp + 1], -fe[2 * tp + 1].x, -fe[2 * tp + 1].y, -fe[2 * tp + 1].z,
                   -fe[2 * tp + 1].w));
#pragma unroll
        for (int ib = 0; ib < NI; ++ib)
            S[ib] = mma32(ke[tp][ib], bx, S[ib]);
    }
}

// Off-diagonal (t-block, s-block) pairs; wavefront w takes kOff[w] and kOff[w + 4].
__constant__ const int kOffT[6] = {1, 2, 2, 3, 3, 3};
// Start state of one state wavefront: S[ib][r] = S_init[ib * 16 + lg * 4 + r][li]
// relative to base (the wavefront's first column of the chain's fp32 state,
// row pitch DV), or zero without a start state.
template <int D>
__device__ __forceinline__ void load_state(f32x4_t (&S)[D / 16], const float* s_init, int64_t base,
                                           int DV, int lane, bool active)
{
    const int li = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int ib = 0; ib < D / 16; ++ib) {
        S[ib] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (s_init && active) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[ib][r] = s_init[base + (int64_t)(ib * 16 + lg * 4 + r) * DV + li];
        }
    }
}

__constant__ const int kOffS[6] = {0, 0, 1, 0, 1, 2};

template <int D, int DVS>
__global__ __launch_bounds__(kThreads) void scan_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ kw, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ b,
    const int32_t* __restrict__ cu, int H, int DV, int n_slices,
    const float* __restrict__ s_init, uint16_t* __restrict__ o, float* __restrict__ s_final)
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
    uint16_t* sTd = reinterpret_cast<uint16_t*>(smem + Ly::oTd);
    float* sLam = reinterpret_cast<float*>(smem + Ly::oG);
    float* sBv = sLam + kC;
    float* sGam = sBv + kC;
    float* sFac = sGam + kC;
    float* sBG = sFac + kC;                      // b gamma

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
        constexpr int nz = 4 * Ly::szM / 16;
        uint4* z = reinterpret_cast<uint4*>(smem + Ly::oAkk);
        for (int i = tid; i < nz; i += kThreads)
            z[i] = make_uint4(0u, 0u, 0u, 0u);
    }

    f32x4_t S[NI];                               // S[:, 16 jb : 16 jb + 16] of wavefront jb
    load_state<D>(S, s_init, (((int64_t)n * H + e) * D) * DV + j0 + wave * 16, DV, lane,
                  wave < NJ);

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
    lds_barrier();

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
            sBG[lane] = bf16_to_f32(pb) * __builtin_amdgcn_exp2f(lam);
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
        lds_barrier();

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
        lds_barrier();

        // ================= 3. state path: wavefront jb, value columns 16 jb .. 16 jb + 15 =================
        if (wave < NJ) {
            v4s_t s0b[D / 16];
            bf16x8_t vf[2];
            state_path<D, DVS>(S, s0b, vf, sQ, sK, sKW, sV, sAkk, sAkkw, sAqkw, sAqk, sTd, sBG, sGam,
                               sFac, __builtin_amdgcn_exp2f(lamC), o, c0, nt, rowV, e, DV, j0, wave,
                               lane);
        }
        lds_barrier();
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


// ---------------------------------------------------------------------------
// Wavefront-specialised variant (value slices of 16 or 32 columns).
//
// NJ = DVS / 16 state wavefronts run the state path of chunk c while the
// other NH = 4 - NJ helper wavefronts prepare chunk c + 1.  The q, k, kw, v
// rows are double-buffered in LDS; the chunk matrices are single-buffered and
// carried in helper registers until the state path has finished with them.
// Per chunk:
//   phase A: state path of chunk c (rows buffer c % 2, matrices of c)
//            helpers: start loading the rows of chunk c + 2 (registers);
//            Gram blocks, masks and diagonal inverses of chunk c + 1 from the
//            rows buffer (c + 1) % 2, into registers
//   barrier
//   phase B: helpers write the matrices and gates of chunk c + 1, and store
//            the rows of chunk c + 2 into buffer c % 2
//   barrier
// so each load has a whole state path to arrive.
// ---------------------------------------------------------------------------
// Workgroups are dispatched to the eight XCDs round-robin (workgroup w runs
// on XCD w % 8), and each XCD has its own L2.  When the chains split evenly
// over the XCDs, all value slices of a chain go to one XCD, so its q, k, kw
// rows come from HBM once and from that L2 for the other slices.
constexpr int kXcds = 8;
constexpr int kDiagRowBlocks = 2;               // four wavefronts: row blocks moved by the diagonal helper
__device__ __forceinline__ void xcd_map(unsigned w, unsigned n_blocks, int n_slices, int& slice,
                                        int& chain)
{
    const unsigned n_chains = n_blocks / (unsigned)n_slices;
    if (n_chains % kXcds == 0) {
        const unsigned x = w % kXcds, j = w / kXcds;
        chain = (int)((j / (unsigned)n_slices) * kXcds + x);
        slice = (int)(j % (unsigned)n_slices);
    } else {
        slice = (int)(w % (unsigned)n_slices);
        chain = (int)(w / (unsigned)n_slices);
    }
}

template <int D, int DVS>
struct LayoutWS {
    using L = Layout<D, DVS>;
    static constexpr int szRows = 3 * L::szRowD + L::szV;   // q, k, kw, v of one chunk
    static constexpr int oRows = 0;                          // two row buffers
    static constexpr int oAkk = oRows + 2 * szRows;          // diagonal blocks hold T_ii
    static constexpr int oAkkw = oAkk + L::szM;
    static constexpr int oAqkw = oAkkw + L::szM;
    static constexpr int oAqk = oAqkw + L::szM;              // holds -A_qk
    static constexpr int oG = oAqk + L::szM;                 // b gamma, gamma, gamma_C / gamma; two chunks
    static constexpr int oScr = oG + 2 * 3 * kC * 4;         // A_ii rows for the inverses
    static constexpr int oLam = oScr + 4 * 16 * 16 * 2;      // log2 decay sums, one slot per helper
    static constexpr int oFlag = oLam + 4 * kC * 4;          // scratch-ready flags (eight waves)
    static constexpr int total = oFlag + 16;
    static_assert(szRows % 16 == 0 && oAkk % 16 == 0 && oG % 16 == 0 && oScr % 16 == 0 &&
                  oLam % 16 == 0, "alignment");
};

// Per-workgroup context shared by the two wavefront roles.
struct WsCtx {
    unsigned char* smem;
    const uint16_t *q, *k, *kw, *v, *g, *b;
    const uint16_t *u, *a, *h, *cw;              // prologue inputs (fused write keys only)
    uint16_t* o;
    const float* s_init;
    float* s_final;
    int n, e, H, DV, j0, seq0, seq1, nchunks, lane;
    bool s_identity;                             // start from S = I (the transition-only job)
    int64_t rowQK, rowV;
    const int* kw_ready;                         // write keys made by producer blocks: one flag
                                                 // per (virtual chunk, head), counted once stored
    uint16_t *ck, *ckT;                          // chunk-start states for the backward, or null
};

template <int D, int DVS>
struct WsBuf {
    using L = Layout<D, DVS>;
    using Ly = LayoutWS<D, DVS>;
    unsigned char* base;
    __device__ unsigned char* rows(int c) const { return base + Ly::oRows + (c & 1) * Ly::szRows; }
    __device__ uint16_t* Q(int c) const { return reinterpret_cast<uint16_t*>(rows(c)); }
    __device__ uint16_t* K(int c) const { return reinterpret_cast<uint16_t*>(rows(c) + L::szRowD); }
    __device__ uint16_t* KW(int c) const { return reinterpret_cast<uint16_t*>(rows(c) + 2 * L::szRowD); }
    __device__ uint16_t* V(int c) const { return reinterpret_cast<uint16_t*>(rows(c) + 3 * L::szRowD); }
    __device__ uint16_t* Akk() const { return reinterpret_cast<uint16_t*>(base + Ly::oAkk); }
    __device__ uint16_t* Akkw() const { return reinterpret_cast<uint16_t*>(base + Ly::oAkkw); }
    __device__ uint16_t* Aqkw() const { return reinterpret_cast<uint16_t*>(base + Ly::oAqkw); }
    __device__ uint16_t* Aqk() const { return reinterpret_cast<uint16_t*>(base + Ly::oAqk); }
    __device__ float* G(int c) const { return reinterpret_cast<float*>(base + Ly::oG) + (c & 1) * 3 * kC; }
    __device__ uint16_t* Scr() const { return reinterpret_cast<uint16_t*>(base + Ly::oScr); }
    __device__ float* Lam(int slot) const { return reinterpret_cast<float*>(base + Ly::oLam) + slot * kC; }
    // volatile LDS words (explicitly in the LDS address space: volatile accesses
    // through a generic pointer would become flat accesses)
    __device__ volatile lds_int_t* Flag(int i) const
    {
        return (volatile lds_int_t*)(reinterpret_cast<int*>(base + Ly::oFlag) + i);
    }
};

// Gram pairs (t-block, s-block) of each helper role, ordered by t-block.  With
// four wavefronts, role 0 takes the four diagonal pairs (their A_kk blocks go
// to the inverse scratch) and (1, 0); the other off-diagonal pairs go to one
// helper (role 1) or are split over two (roles 2, 3).  With eight wavefronts
// the ten pairs are split over roles 4, 6, 5 and 3, and role 7 (no pairs) only
// moves rows.
template <int ROLE> struct Pairs;
template <> struct Pairs<0> {
    static constexpr int n = 5;
    static constexpr int t[5] = {0, 1, 1, 2, 3}, s[5] = {0, 0, 1, 2, 3};
};
template <> struct Pairs<1> {
    static constexpr int n = 5;
    static constexpr int t[5] = {2, 2, 3, 3, 3}, s[5] = {0, 1, 0, 1, 2};
};
template <> struct Pairs<2> {
    static constexpr int n = 2;
    static constexpr int t[2] = {2, 2}, s[2] = {0, 1};
};
template <> struct Pairs<3> {
    static constexpr int n = 3;
    static constexpr int t[3] = {3, 3, 3}, s[3] = {0, 1, 2};
};
template <> struct Pairs<4> {
    static constexpr int n = 2;
    static constexpr int t[2] = {0, 1}, s[2] = {0, 1};
};
template <> struct Pairs<5> {
    static constexpr int n = 2;
    static constexpr int t[2] = {2, 3}, s[2] = {2, 3};
};
template <> struct Pairs<6> {
    static constexpr int n = 3;
    static constexpr int t[3] = {1, 2, 2}, s[3] = {0, 0, 1};
};
template <> struct Pairs<7> {
    static constexpr int n = 0;
    static constexpr int t[1] = {0}, s[1] = {0};
};

// Count of bounded LDS-flag waits (eight-wavefront scan) that gave up before
// their flags were raised.  Every writer reaches its flag before the phase
// barrier, so this stays zero; a give-up would leave the inverse built from
// whatever the scratch held, so it is counted here (global atomic) for the
// host to check (read_wait_giveups).
__device__ unsigned int g_wait_giveups = 0;

// Column li of (I + A)^-1 for a strictly lower 16x16 block A whose row li (16
// bf16) is at `row`; lanes 16 g .. 16 g + 15 must hold the rows of one block.
__device__ __forceinline__ void invert_cols(const uint16_t* row, float (&x)[16], int li)
{
    const uint4 w0 = *reinterpret_cast<const uint4*>(row);
    const uint4 w1 = *reinterpret_cast<const uint4*>(row + 8);
    const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float a[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[2 * j] = __uint_as_float(wv[j] << 16);
        a[2 * j + 1] = __uint_as_float(wv[j] & 0xffff0000u);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
        x[r] = (r == li) ? 1.f : 0.f;
    subst<0>(x, a);
}

// Column i of a block inverse as row i of the transposed block (two 16-byte stores).
__device__ __forceinline__ void store_trow(uint16_t* p, const float (&x)[16])
{
    uint32_t w[8];
#pragma unroll
    for (int r = 0; r < 8; ++r)
        w[r] = pack_bf16x2(x[2 * r], x[2 * r + 1]);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(p + 8) = make_uint4(w[4], w[5], w[6], w[7]);
}

// T_g = (I + A_g)^-1 for the four diagonal blocks of A_kk: scr holds the strictly
// lower blocks A_g row-major (rows of 16 bf16, block g at row 16 g); T_g goes
// transposed into the diagonal block g of Akk (row stride LDC).  One wavefront.
template <int LDC>
__device__ __forceinline__ void invert_diag(const uint16_t* scr, uint16_t* Akk, int lane)
{
    const int li = lane & 15, lg = lane >> 4;
    float x[16];
    invert_cols(scr + lane * 16, x, li);
    store_trow(Akk + (lg * 16 + li) * LDC + lg * 16, x);
}

// ---- Fused write keys (LF = L levels): a chunk's kw rows computed in place of
// being read from memory, with the prologue's arithmetic (PRISM pages: WeChat
// ICML 2026 summary, sections 消除 Token 间串行 and 消除 Step 间串行;
// gist.science summary of arXiv 2602.10796, section 2.2):
//   r_1  = sum_m w[e,i,m] k[t-3+m]   (ShortConv, taps before the sequence start read 0)
//   r_{l+1} = r_l (1 - a_l h_l),  kw = b k + sum_{l=1..L-1} a_l r_l u_l.
// NWV wavefronts (r = 0 .. NWV - 1) share a chunk: lane (channel piece
// p = lane % (D/8), token strip) walks ST consecutive tokens of 8 channels, so
// the conv taps stay in registers; with L <= 4 the inputs of token j + 1 are
// loaded while token j is computed.
// Every load is a bounded buffer load: taps before the sequence start and
// tokens past the chunk's end read zeros (a zero kw row there).
// The rows go to an LDS tile (row stride D + 8), or with GLOBAL to the kw rows
// of the chunk in device memory through a buffer range that ends at the chunk's
// last token (rows past it are dropped), stored coherently at device scope
// (sc1) for readers on other compute units.
template <int D>
__device__ __forceinline__ void load_taps(const WsCtx& c, float (&w)[8][4])
{
    const int pc = (c.lane % (D / 8)) * 8;
    const uint16_t* p = c.cw + ((int64_t)c.e * D + pc) * 4;    // conv_w [H][D][4]
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const uint4 v = *reinterpret_cast<const uint4*>(p + 8 * x);
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int lo = 8 * x + 2 * i, hi = lo + 1;
            w[lo / 4][lo % 4] = __uint_as_float(wv[i] << 16);
            w[hi / 4][hi % 4] = __uint_as_float(wv[i] & 0xffff0000u);
        }
    }
}

template <int D, int LF, int NWV = 4, bool GLOBAL = false>
__device__ __forceinline__ void fused_kw(const WsCtx& c, uint16_t* sKW, int ch, int r, const float (&w)[8][4])
{
    constexpr int LDD = D + 8;
    constexpr int NPC = D / 8;                   // 16-byte channel pieces per row
    constexpr int SPW = 64 / NPC;                // token strips per wavefront
    constexpr int ST = kC / (NWV * SPW);         // tokens per strip
    static_assert(ST >= 1 && ST * NWV * SPW == kC, "strips cover the chunk");
    constexpr int NS = LF - 1;                   // u, a slots (levels 1 .. L-1)
    constexpr int NH = LF > 2 ? LF - 2 : 1;      // h slots read (the last one never is)
    constexpr uint32_t fl = 0x00020000;
    const int lane = c.lane;
    const int pc = (lane % NPC) * 8;
    const int tl0 = (r * SPW + lane / NPC) * ST; // first token of the strip, chunk-relative
    const int c0 = c.seq0 + ch * kC;
    const int nt = __builtin_amdgcn_readfirstlane(max(0, min(kC, c.seq1 - c0)));
    const int hb = max(c.seq0, c0 - 3);          // first k row a tap may read
    const int rowQK = (int)c.rowQK, lrow = c.H * NS * D;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.k + (int64_t)hb * rowQK + c.e * D),
                                                      0, (c0 + nt - hb) * rowQK * 2, fl);
    const int64_t lbase = (int64_t)c0 * lrow + (int64_t)c.e * NS * D;
    const auto ru = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.u + lbase), 0, nt * lrow * 2, fl);
    const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.a + lbase), 0, nt * lrow * 2, fl);
    const auto rh = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.h + lbase), 0, nt * lrow * 2, fl);
    const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.b + (int64_t)c0 * c.H + c.e), 0,
                                                      nt * c.H * 2, fl);
    // GLOBAL: sKW is the kw array [T, H, D]; the range ends at the chunk's last token
    const auto rkw = __builtin_amdgcn_make_buffer_rsrc(sKW + (GLOBAL ? (int64_t)c0 * rowQK + c.e * D : 0), 0,
                                                       GLOBAL ? nt * rowQK * 2 : 0, fl);
    auto ld = [&](__amdgpu_buffer_rsrc_t rs, int off) {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    };
    auto unpack = [](const uint4& v, float* out) {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(wv[i] << 16);
            out[2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
        }
    };
    // k row of chunk-relative token tl (negative offsets: before the range, zero)
    auto koff = [&](int tl) { return ((c0 + tl - hb) * rowQK + pc) * 2; };
    struct In {
        uint4 k, u[NS], a[NS], h[NH];
        uint16_t b;
    };
    auto fetch = [&](int tl, In& x) {
        x.k = ld(rk, koff(tl));
        const int lo = (tl * lrow + pc) * 2;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            x.u[s] = ld(ru, lo + s * D * 2);
            x.a[s] = ld(ra, lo + s * D * 2);
            if (s < LF - 2)
                x.h[s] = ld(rh, lo + s * D * 2);
        }
        x.b = __builtin_amdgcn_raw_buffer_load_b16(rb, tl * c.H * 2, 0, 0);
    };
    // two input sets (token j + 1 in flight while token j is computed) where
    // they fit the registers (L <= 4); one otherwise
    constexpr bool PIPE = LF <= 4;
    float x1[8], x2[8], x3[8];                   // k at t - 1, t - 2, t - 3
    {
        const uint4 h1 = ld(rk, koff(tl0 - 1)), h2 = ld(rk, koff(tl0 - 2)), h3 = ld(rk, koff(tl0 - 3));
        unpack(h1, x1);
        unpack(h2, x2);
        unpack(h3, x3);
    }
    In X[PIPE ? 2 : 1];
    fetch(tl0, X[0]);
#pragma unroll
    for (int j = 0; j < ST; ++j) {
        if constexpr (PIPE) {
            if (j + 1 < ST)
                fetch(tl0 + j + 1, X[(j + 1) & 1]);
        } else if (j > 0) {
            SCHED_FENCE();
            fetch(tl0 + j, X[0]);
        }
        const In& x = X[PIPE ? (j & 1) : 0];
        float kt[8], rr[8], acc[8];
        unpack(x.k, kt);
        const float bt = bf16_to_f32(x.b);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            rr[i] = w[i][3] * kt[i] + w[i][2] * x1[i] + w[i][1] * x2[i] + w[i][0] * x3[i];
            acc[i] = bt * kt[i];
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            float av[8], uv[8];
            unpack(x.a[s], av);
            unpack(x.u[s], uv);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] += av[i] * rr[i] * uv[i];
            if (s < LF - 2) {
                float hv[8];
                unpack(x.h[s], hv);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    rr[i] *= 1.f - av[i] * hv[i];
            }
        }
        const uint4 out = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
        if constexpr (GLOBAL)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, out), rkw,
                                                   ((tl0 + j) * rowQK + pc) * 2, 0, kScopeDevice);
        else
            *reinterpret_cast<uint4*>(sKW + (tl0 + j) * LDD + pc) = out;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            x3[i] = x2[i];
            x2[i] = x1[i];
            x1[i] = kt[i];
        }
    }
}

// Helper wavefront: loads and stores the 16-token row blocks LB0 .. LB0 + NLB - 1
// of q, k, kw, v (NLB may be 0), and builds the Gram pairs of its role from the
// rows in LDS (role 7 has none).  With GATES it also publishes the gate vectors.
// Eight wavefronts: the two helpers with the diagonal pairs build the A_kk part
// of those pairs first and raise flag SIG once their A_tt rows are in the
// scratch; the INV wavefront (a row mover) waits for both flags (a bounded
// wait: both writers reach them before the phase barrier), inverts the four
// diagonal blocks in one pass and stores T_tt with the phase-B stores.
// SLOT: this wavefront's row of decay sums in LDS.
// LF > 0: the write keys are fused (computed, not read): the row movers leave
// kw alone, and the Gram helper with KWR = r >= 0 computes its quarter of every
// chunk's kw rows (fused_kw) in phase B, two chunks ahead, where the kw rows
// would otherwise have been stored.
// KWP: the write keys are made during the scan by producer blocks of the same
// launch.  Before a chunk's kw rows are loaded, its readiness count is read
// (issued ahead of the chunk's other loads, so that waiting for it waits for
// nothing else) and, until all kProducerWaves producer wavefronts have counted
// their parts, polled; a bounded wait.  The flag and
// the kw rows are read coherently at device scope, like the producers wrote
// them.
template <int D, int DVS, int ROLE, int LB0, int NLB, bool GATES, int SLOT, bool INV = false,
          int SIG = -1, int LF = 0, int KWR = -1, bool KWP = false>
__device__ __forceinline__ void helper_loop(const WsCtx& c)
{
    static_assert(KWR < 0 || (LF > 0 && NLB == 0), "fused write keys: Gram helpers only");
    using L = Layout<D, DVS>;
    using P = Pairs<ROLE>;
    constexpr int LDD = L::LDD, LDC = L::LDC, LDV = L::LDV;
    constexpr int KS = D / 32;
    constexpr int NP = P::n;
    constexpr int NPA = NP > 0 ? NP : 1;         // array extents
    constexpr int NLBA = NLB > 0 ? NLB : 1;
    constexpr bool DIAG = GATES;
    float tinv[16];                              // column li of T_(lane / 16)
    constexpr int VL = DVS / 8;                  // 16-byte v vectors per token row
    const WsBuf<D, DVS> m{c.smem};
    const int lane = c.lane, li = lane & 15, lg = lane >> 4;

    // ---- rows of one chunk in flight (this wavefront's blocks), 16-byte pieces.
    // Each load instruction covers whole token rows (RPI rows of D channels), so
    // every cache line it touches is used in full; buffer loads bounded at the
    // chunk's last token return zeros past it.
    constexpr int PPR = D / 8;                   // 16-byte pieces per row
    constexpr int RPI = 64 / PPR;                // rows per instruction
    constexpr uint32_t kRsrcFlags = 0x00020000;
    const int pr = lane / PPR, pc = (lane % PPR) * 8;
    uint4 rq[NLBA][KS], rk[NLBA][KS], rw[NLBA][KS], rv[NLBA];
    uint16_t ng = 0x3f80u, nb = 0u;              // gates in flight (b reads 0 past the chunk end)
    bool nin = false;                            // token `lane` inside the chunk in flight
    // Loads of one chunk, issued in NLB + 1 groups (the gates, then one row
    // block each) so that they can be spread over the Gram computation.
    struct Src {
        __amdgpu_buffer_rsrc_t k, kw, q, v, g, b;
        int nt;
    };
    auto src = [&](int ch) {
        const int c0 = c.seq0 + ch * kC;
        const int nt = min(kC, c.seq1 - c0);
        const int64_t base = (int64_t)c0 * c.rowQK + (int64_t)c.e * D;
        const int nqk = nt * (int)c.rowQK * 2;   // rows past the chunk end read as zero
        Src r;
        r.k = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.k + base), 0, nqk, kRsrcFlags);
        // a null kw or v reads as zero (an empty buffer range): the transition-only
        // scan, whose write term kw v^T vanishes
        r.kw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.kw ? c.kw + base : c.k), 0,
                                                 c.kw ? nqk : 0, kRsrcFlags);
        r.q = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.q + base), 0, nqk, kRsrcFlags);
        r.v = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(c.v ? c.v + (int64_t)c0 * c.rowV + (int64_t)c.e * c.DV + c.j0 : c.k),
            0, c.v ? nt * (int)c.rowV * 2 : 0, kRsrcFlags);
        r.g = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.g + (int64_t)c0 * c.H + c.e), 0,
                                                nt * c.H * 2, kRsrcFlags);
        r.b = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.b + (int64_t)c0 * c.H + c.e), 0,
                                                nt * c.H * 2, kRsrcFlags);
        r.nt = nt;
        return r;
    };
    auto load_gates = [&](const Src& r) {
        ng = __builtin_amdgcn_raw_buffer_load_b16(r.g, lane * c.H * 2, 0, 0);
        nb = __builtin_amdgcn_raw_buffer_load_b16(r.b, lane * c.H * 2, 0, 0);
        nin = lane < r.nt;                       // decay 1 past the chunk end, applied once the
    };                                           // gates are taken over (no wait here)
    auto load_block = [&](const Src& r, int u) {
        const int rowQK = (int)c.rowQK, rowV = (int)c.rowV;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int off = (((LB0 + u) * 16 + ks * RPI + pr) * rowQK + pc) * 2;
            rk[u][ks] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r.k, off, 0, 0));
            if constexpr (LF == 0 && !KWP)
                rw[u][ks] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r.kw, off, 0, 0));
            rq[u][ks] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r.q, off, 0, 0));
        }
        const int offv = (((LB0 + u) * 16 + lane / VL) * rowV + (lane % VL) * 8) * 2;
        rv[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r.v, offv, 0, 0));
    };
    auto load_kw_block = [&](const Src& r, int u) {
        const int rowQK = (int)c.rowQK;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int off = (((LB0 + u) * 16 + ks * RPI + pr) * rowQK + pc) * 2;
            rw[u][ks] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r.kw, off, 0,
                                                                                        kScopeDevice));
        }
    };
    auto load = [&](int ch) {
        const Src r = src(ch);
        if constexpr (KWP) {
            const int* fp = c.kw_ready + ((int64_t)(c.seq0 / kC + c.n + ch)) * c.H + c.e;
            int ready = __hip_atomic_load(fp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            SCHED_FENCE();
            load_gates(r);
#pragma unroll
            for (int u = 0; u < NLB; ++u)
                load_block(r, u);
            SCHED_FENCE();
            // the first test outside the polling loop, so that it waits for the
            // flag load alone (a loop head would wait for every load)
            if (__builtin_amdgcn_readfirstlane(ready) < kProducerWaves) {
                for (int spin = 0; spin < (1 << 16); ++spin) {
                    __builtin_amdgcn_s_sleep(2);
                    ready = __hip_atomic_load(fp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (__builtin_amdgcn_readfirstlane(ready) >= kProducerWaves)
                        break;
                }
                // a wait that gives up is counted (the kw rows read may then be stale)
                if (__builtin_amdgcn_readfirstlane(ready) < kProducerWaves && lane == 0)
                    atomicAdd(&g_wait_giveups, 1u);
            }
            asm volatile("" ::: "memory");       // the kw loads stay below the wait
#pragma unroll
            for (int u = 0; u < NLB; ++u)
                load_kw_block(r, u);
        } else {
            load_gates(r);
#pragma unroll
            for (int u = 0; u < NLB; ++u)
                load_block(r, u);
        }
    };
    uint16_t cg = 0x3f80u, cb = 0u;              // gates of the chunk being prepared
    // the rows in flight into the row buffer of chunk ch (and the gates taken over)
    auto store_rows = [&](int ch) {
        uint16_t *sQ = m.Q(ch), *sK = m.K(ch), *sKW = m.KW(ch), *sV = m.V(ch);
#pragma unroll
        for (int u = 0; u < NLB; ++u) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int off = ((LB0 + u) * 16 + ks * RPI + pr) * LDD + pc;
                *reinterpret_cast<uint4*>(sK + off) = rk[u][ks];
                *reinterpret_cast<uint4*>(sQ + off) = rq[u][ks];
                if constexpr (LF == 0)
                    *reinterpret_cast<uint4*>(sKW + off) = rw[u][ks];
            }
            if (lane < 16 * VL)
                *reinterpret_cast<uint4*>(sV + ((LB0 + u) * 16 + lane / VL) * LDV + (lane % VL) * 8) = rv[u];
        }
        cg = nin ? ng : (uint16_t)0x3f80u;
        cb = nb;
    };

    // ---- one chunk's matrices in registers (bf16 pairs, accumulator layout)
    uint2 mkk[NPA], mkw[NPA], mqk[NPA], mqw[NPA];
    // prep(ch, lch): matrices of chunk ch; the loads of chunk lch (if >= 0) are
    // issued between its Gram pairs
    auto prep = [&](int ch, int lch) {
        if constexpr (NP == 0) {                 // rows (and the inverses)
            if (lch >= 0)
                load(lch);
            if constexpr (INV) {
                volatile lds_int_t* f0 = m.Flag(0);
                volatile lds_int_t* f1 = m.Flag(1);
                bool ready = false;
                for (int spin = 0; spin < (1 << 20) && !ready; ++spin) {
                    ready = *f0 == ch + 1 && *f1 == ch + 1;
                    if (!ready)
                        __builtin_amdgcn_s_sleep(1);
                }
                // a wait that gives up is counted (the result may then be wrong);
                // prism_scan_wait_giveups reports the count to the host
                if (!ready && lane == 0)
                    atomicAdd(&g_wait_giveups, 1u);
                asm volatile("" ::: "memory");   // the scratch reads stay below the wait
                __builtin_amdgcn_s_setprio(2);
                invert_cols(m.Scr() + lane * 16, tinv, li);
                __builtin_amdgcn_s_setprio(0);
            }
            return;
        }
        Src lsrc;
        if (lch >= 0) {
            lsrc = src(lch);
            load_gates(lsrc);
        }
        const float lam = wave_inclusive_sum(__log2f(fmaxf(bf16_to_f32(cg), 1e-30f)));
        const float bv = bf16_to_f32(cb);
        if constexpr (DIAG) {
            // gates of chunk ch, in the buffer the state path of chunk ch - 1 does not read
            const float lamC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), 63));
            float* G = m.G(ch);
            G[lane] = bv * __builtin_amdgcn_exp2f(lam);
            G[kC + lane] = __builtin_amdgcn_exp2f(lam);
            G[2 * kC + lane] = __builtin_amdgcn_exp2f(lamC - lam);
        }
        const uint16_t *sQ = m.Q(ch), *sK = m.K(ch), *sKW = m.KW(ch);
        float* sLam = m.Lam(SLOT);
        sLam[lane] = lam;
        // operands of pair p (t-block rows taken over from `prev` when pair p - 1
        // has the same t-block) and its decay sums
        struct Ops {
            bf16x8_t bk[KS], bq[KS], ak[KS], aw[KS];
            float lt, bt, le;
            float4 ls4;
        };
        // what the A_kk block of a diagonal pair needs (K rows, decay sums), and the rest
        auto read_kk = [&](int p, Ops& o) {
            const int tb = P::t[p];
            const int t = tb * 16 + li;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                o.bk[ks] = frag_row(sK + tb * 16 * LDD + ks * 32, LDD, lane);
                o.ak[ks] = o.bk[ks];
            }
            o.lt = sLam[t];
            o.bt = __shfl(bv, t, 64);
            o.ls4 = *reinterpret_cast<const float4*>(sLam + tb * 16 + lg * 4);
            o.le = 0.f;
        };
        auto read_rest = [&](int p, Ops& o) {
            const int tb = P::t[p];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                o.bq[ks] = frag_row(sQ + tb * 16 * LDD + ks * 32, LDD, lane);
                o.aw[ks] = frag_row(sKW + tb * 16 * LDD + ks * 32, LDD, lane);
            }
        };
        auto read_ops = [&](int p, Ops& o, const Ops& prev) {
            const int tb = P::t[p], sb = P::s[p];
            const int t = tb * 16 + li;
            if (p > 0 && P::t[p > 0 ? p - 1 : 0] == tb) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    o.bk[ks] = prev.bk[ks];
                    o.bq[ks] = prev.bq[ks];
                }
                o.lt = prev.lt;
                o.bt = prev.bt;
            } else {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    o.bk[ks] = frag_row(sK + tb * 16 * LDD + ks * 32, LDD, lane);
                    o.bq[ks] = frag_row(sQ + tb * 16 * LDD + ks * 32, LDD, lane);
                }
                o.lt = sLam[t];
                o.bt = __shfl(bv, t, 64);
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                o.ak[ks] = sb == tb ? o.bk[ks] : frag_row(sK + sb * 16 * LDD + ks * 32, LDD, lane);
                o.aw[ks] = frag_row(sKW + sb * 16 * LDD + ks * 32, LDD, lane);
            }
            o.ls4 = *reinterpret_cast<const float4*>(sLam + sb * 16 + lg * 4);
            o.le = sb == tb ? 0.f : sLam[sb * 16 + 15];
        };
        // part 0: the four matrices of pair p; 1: its A_kk block only; 2: the other three
        auto compute = [&](int p, const Ops& o, int part) {
            const int tb = P::t[p], sb = P::s[p];
            const int t = tb * 16 + li;
            f32x4_t gkk = {0.f, 0.f, 0.f, 0.f}, gkw = gkk, gqk = gkk, gqw = gkk;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (part != 2)
                    gkk = mma32(o.ak[ks], o.bk[ks], gkk); // transposed blocks: element (s, t)
                if (part != 1) {
                    gkw = mma32(o.aw[ks], o.bk[ks], gkw);
                    gqk = mma32(o.ak[ks], o.bq[ks], gqk);
                    gqw = mma32(o.aw[ks], o.bq[ks], gqw);
                }
            }
            const int s0 = sb * 16 + lg * 4;
            const float lsv[4] = {o.ls4.x, o.ls4.y, o.ls4.z, o.ls4.w};
            const float lt = o.lt, bt = o.bt;
            f32x4_t vkk, vkw, vqk, vqw;
            if (sb == tb) {
                // diagonal block: causal masks, decay 2^(lam_t - lam_s) per element
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
            } else {
                // s-block entirely before t: 2^(lam_t - lam_s) = 2^(lam_t - lam_e) 2^(lam_e - lam_s)
                // with lam_e the last token of the s-block; both factors are <= 1
                // because lam never increases along the chunk
                const float le = o.le;
                const float et = __builtin_amdgcn_exp2f(lt - le), bet = bt * et;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float fs = __builtin_amdgcn_exp2f(le - lsv[r]);
                    const float mi = et * fs, ms = bet * fs;
                    vkk[r] = ms * gkk[r];
                    vkw[r] = ms * gkw[r];
                    vqk[r] = -mi * gqk[r];
                    vqw[r] = mi * gqw[r];
                }
            }
            if (part != 2) {
                mkk[p] = make_uint2(pack_bf16x2(vkk[0], vkk[1]), pack_bf16x2(vkk[2], vkk[3]));
                if (tb == sb)                            // A_tt row li, columns 4 lg .. 4 lg + 3
                    *reinterpret_cast<uint2*>(m.Scr() + (tb * 16 + li) * 16 + lg * 4) = mkk[p];
            }
            if (part != 1) {
                mkw[p] = make_uint2(pack_bf16x2(vkw[0], vkw[1]), pack_bf16x2(vkw[2], vkw[3]));
                mqk[p] = make_uint2(pack_bf16x2(vqk[0], vqk[1]), pack_bf16x2(vqk[2], vqk[3]));
                mqw[p] = make_uint2(pack_bf16x2(vqw[0], vqw[1]), pack_bf16x2(vqw[2], vqw[3]));
            }
        };
        if constexpr (SIG >= 0) {
            // two diagonal pairs: both A_tt blocks first, then the flag, then the rest
            static_assert(NP == 2 && NLB == 0 && P::t[0] == P::s[0] && P::t[1] == P::s[1],
                          "SIG: two diagonal pairs, no rows");
            // (raised issue priority until the flag: the inverse waits on it)
            __builtin_amdgcn_s_setprio(2);
            Ops ops[2];
            read_kk(0, ops[0]);
            read_kk(1, ops[1]);
            SCHED_FENCE();
            read_rest(0, ops[0]);
            compute(0, ops[0], 1);
            compute(1, ops[1], 1);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            *m.Flag(SIG) = ch + 1;
            __builtin_amdgcn_s_setprio(0);
            read_rest(1, ops[1]);
            compute(0, ops[0], 2);
            compute(1, ops[1], 2);
        } else if constexpr (NLB == 0) {
            // no rows to move: the operands of pair p + 1 are read while pair p computes
            Ops ops[2];
            read_ops(0, ops[0], ops[0]);
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                if (p + 1 < NP)
                    read_ops(p + 1, ops[(p + 1) & 1], ops[p & 1]);
                SCHED_FENCE();
                compute(p, ops[p & 1], 0);
                SCHED_FENCE();
            }
        } else {
            // the row loads of chunk lch are spread between the pairs
            Ops o;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
#pragma unroll
                for (int u = 0; u < NLB; ++u) {
                    if (p == u * NP / NLB && lch >= 0) {
                        SCHED_FENCE();
                        load_block(lsrc, u);
                        SCHED_FENCE();
                    }
                }
                read_ops(p, o, o);
                compute(p, o, 0);
            }
        }
    };
    auto write_mats = [&]() {
        uint16_t *Akk = m.Akk(), *Akkw = m.Akkw(), *Aqkw = m.Aqkw(), *Aqk = m.Aqk();
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int off = (P::t[p] * 16 + li) * LDC + P::s[p] * 16 + lg * 4;
            if (P::t[p] != P::s[p])              // the diagonal blocks of A_kk hold T_tt
                *reinterpret_cast<uint2*>(Akk + off) = mkk[p];
            *reinterpret_cast<uint2*>(Akkw + off) = mkw[p];
            *reinterpret_cast<uint2*>(Aqk + off) = mqk[p];
            *reinterpret_cast<uint2*>(Aqkw + off) = mqw[p];
        }
        if constexpr (INV)                       // T_tt transposed
            store_trow(Akk + (lg * 16 + li) * LDC + lg * 16, tinv);
    };

    float taps[8][4];
    if constexpr (KWR >= 0)
        load_taps<D>(c, taps);
    const int nch = c.nchunks;
    if (nch > 0)
        load(0);
    lds_barrier();                               // LDS cleared
    if (nch > 0) {
        store_rows(0);
        if (nch > 1)
            load(1);
        if constexpr (KWR >= 0)
            fused_kw<D, LF>(c, m.KW(0), 0, KWR, taps);
    }
    lds_barrier();                               // rows of chunk 0 visible
    if (nch > 0) {
        prep(0, -1);
        write_mats();
        if (nch > 1) {
            store_rows(1);
            if constexpr (KWR >= 0)
                fused_kw<D, LF>(c, m.KW(1), 1, KWR, taps);
        }
    }
    lds_barrier();                               // matrices of chunk 0 (A_ii in the scratch)
    lds_barrier();                               // T_ii of chunk 0 (four wavefronts: a state wavefront)
    for (int ch = 0; ch < nch; ++ch) {
        // phase A (beside the state path of chunk ch): matrices of chunk ch + 1,
        // with the loads of chunk ch + 2 spread between its Gram pairs
        if (ch + 1 < nch)
            prep(ch + 1, ch + 2 < nch ? ch + 2 : -1);
        lds_barrier();
        // phase B
        if (ch + 1 < nch)
            write_mats();
        if (ch + 2 < nch) {
            store_rows(ch + 2);
            // kw rows of chunk ch + 2 into the buffer whose kw chunk ch no longer needs
            if constexpr (KWR >= 0)
                fused_kw<D, LF>(c, m.KW(ch + 2), ch + 2, KWR, taps);
        }
        lds_barrier();
    }
}

// State wavefront jb: value columns 16 jb .. 16 jb + 15 of the slice.
// INV: wavefront 0 inverts the diagonal blocks (in phase B).  SPLIT: the a-step
// of chunk ch + 1 runs in phase B of chunk ch, beside the helpers' stores.
template <int D, int DVS, bool INV, bool SPLIT, bool CK = false>
__device__ __forceinline__ void state_loop(const WsCtx& c, int jb)
{
    constexpr int NI = D / 16;
    const WsBuf<D, DVS> m{c.smem};
    const int lane = c.lane, li = lane & 15, lg = lane >> 4;
    f32x4_t S[NI];
    load_state<D>(S, c.s_init, (((int64_t)c.n * c.H + c.e) * D) * c.DV + c.j0 + jb * 16, c.DV,
                  lane, true);
    if (c.s_identity) {
#pragma unroll
        for (int ib = 0; ib < NI; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[ib][r] = (ib * 16 + lg * 4 + r == c.j0 + jb * 16 + li) ? 1.f : 0.f;
    }
    lds_barrier();
    lds_barrier();
    lds_barrier();
    // the helpers have built the matrices of chunk 0; invert its diagonal blocks
    if (INV && jb == 0 && c.nchunks > 0)
        invert_diag<Layout<D, DVS>::LDC>(m.Scr(), m.Akk(), lane);
    v4s_t s0b[NI];
    bf16x8_t vf[2];
    // a-step of chunk ch from the gates G(ch): gamma_C = gamma of the last token
    // (gates past the chunk end are 1)
    auto a_of = [&](int ch) {
        const float* G = m.G(ch);
        a_step<D, DVS>(S, s0b, vf, m.KW(ch), m.V(ch), G + 2 * kC, G[2 * kC - 1], jb, lane);
        if constexpr (CK) {
            // the chunk's start state (s0b: bf16 of S before the a-step) as rows
            // [dk][dv] and transposed [dv][dk] per (virtual chunk, head).  A lane
            // holds four consecutive rows of one column: one 8-byte store into the
            // transposed copy; for the rows, the four lanes of each quad transpose
            // their 4 x 4 block (QuadTranspose) so that a lane stores four
            // consecutive columns of one row.
            const int64_t vc = ((int64_t)(c.seq0 / kC + c.n + ch)) * c.H + c.e;
            const int col = c.j0 + jb * 16 + li;
            const int qp = li & 3;               // position in the quad
            const QuadTranspose qt(qp);
            uint16_t* rows = c.ck + (vc * D + lg * 4 + qp) * c.DV + col - qp;
#pragma unroll
            for (int ib = 0; ib < D / 16; ++ib) {
                *reinterpret_cast<v4s_t*>(c.ckT + (vc * c.DV + col) * D + ib * 16 + lg * 4) = s0b[ib];
                // row ib * 16 + lg * 4 + qp, columns col - qp .. col - qp + 3
                *reinterpret_cast<uint2*>(rows + (int64_t)ib * 16 * c.DV) = qt(__builtin_bit_cast(uint2, s0b[ib]));
            }
        }
    };
    if (SPLIT && c.nchunks > 0)
        a_of(0);
    lds_barrier();
    for (int ch = 0; ch < c.nchunks; ++ch) {
        const int c0 = c.seq0 + ch * kC;
        const int nt = min(kC, c.seq1 - c0);
        const float* G = m.G(ch);
        state_path<D, DVS, true, SPLIT>(S, s0b, vf, m.Q(ch), m.K(ch), m.KW(ch), m.V(ch), m.Akk(),
                                        m.Akkw(), m.Aqkw(), m.Aqk(), nullptr, G, G + kC, G + 2 * kC,
                                        G[2 * kC - 1], c.o, c0, nt, c.rowV, c.e, c.DV, c.j0, jb,
                                        lane);
        lds_barrier();
        // phase B: the diagonal inverses of chunk ch + 1 (their A_ii were built in
        // phase A) or the a-step of chunk ch + 1, beside the helpers' stores
        if (INV && jb == 0 && ch + 1 < c.nchunks)
            invert_diag<Layout<D, DVS>::LDC>(m.Scr(), m.Akk(), lane);
        if (SPLIT && ch + 1 < c.nchunks)
            a_of(ch + 1);
        lds_barrier();
    }
#pragma unroll
    for (int ib = 0; ib < NI; ++ib) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ib * 16 + lg * 4 + r;
            c.s_final[(((int64_t)c.n * c.H + c.e) * D + i) * c.DV + c.j0 + jb * 16 + li] = S[ib][r];
        }
    }
}

// Write-key producers: blocks 0 .. n_prod - 1 of a scan launch whose other
// blocks run the scan on the remaining compute units.  They form the kw rows
// of every (chunk, sequence, head) item with the prologue's arithmetic (the
// same steps as fused_kw), in chunk-major order so that every chain's chunk c
// is ready about when its scan reaches it, store them coherently at device
// scope, and count each wavefront's part into the item's flag once its
// stores have completed.  Eight wavefronts share an item (lane: 8 channels of
// a strip of ST tokens).  The loads of the next item are issued before the wait for the
// current item's stores, so the two latencies overlap.  Producers wait for
// nothing but their own memory operations, so the scan blocks that wait for
// them (a bounded wait) cannot stall them.
template <int D, int LF>
__device__ __forceinline__ void produce_kw(const WsCtx& c, const int32_t* __restrict__ cu, int n_seqs,
                                           int n_prod, uint16_t* kw_out, int* ready)
{
    constexpr int NPC = D / 8;                   // 16-byte channel pieces per row
    constexpr int SPW = 64 / NPC;                // token strips per wavefront
    constexpr int ST = kC / (kProducerWaves * SPW);   // tokens per strip
    constexpr int NS = LF - 1;                   // u, a slots (levels 1 .. L-1)
    constexpr int NH = LF > 2 ? LF - 2 : 1;      // h slots read (the last one never is)
    constexpr uint32_t fl = 0x00020000;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pc = (lane % NPC) * 8;
    const int tl0 = (wave * SPW + lane / NPC) * ST;          // first token of the strip, chunk-relative
    const int H = c.H, rowQK = (int)c.rowQK, lrow = H * NS * D;

    int* sMax = reinterpret_cast<int*>(c.smem);  // the longest sequence's chunk count
    if (tid == 0)
        *sMax = 0;
    __syncthreads();
    for (int n = tid; n < n_seqs; n += blockDim.x)
        atomicMax(sMax, (cu[n + 1] - cu[n] + kC - 1) / kC);
    __syncthreads();
    const int n_chains = n_seqs * H;
    const int64_t items = (int64_t)*sMax * n_chains;

    struct Item {
        int ch, n, e, s0, s1;
    };
    // the first item with tokens at index >= i (stride n_prod), or `items`
    auto next_item = [&](int64_t i, Item& it) {
        for (; i < items; i += n_prod) {
            const int ch = (int)(i / n_chains), chain = (int)(i % n_chains);
            const int n = chain / H;
            const int s0 = cu[n], s1 = cu[n + 1];
            if (ch * kC < s1 - s0) {
                it.ch = ch; it.n = n; it.e = chain % H; it.s0 = s0; it.s1 = s1;
                return i;
            }
        }
        return items;
    };
    struct In {
        uint4 w[4];                              // conv taps of the lane's channels (bf16)
        uint4 hk[3];                             // k at tl0 - 1, tl0 - 2, tl0 - 3
        uint4 k[ST], u[ST][NS], a[ST][NS], h[ST][NH];
        uint16_t b[ST];
    };
    auto ld = [](__amdgpu_buffer_rsrc_t rs, int off) {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    };
    // u, a, h are read once: nontemporal, so they do not displace the rows the
    // scan blocks share through L2
    auto ldn = [](__amdgpu_buffer_rsrc_t rs, int off) {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNontemporal));
    };
    // Bounded buffer loads: taps before the sequence start and tokens past the
    // chunk's end read zeros.
    auto fetch = [&](const Item& it, In& x) {
        const int c0 = it.s0 + it.ch * kC;
        const int nt = min(kC, it.s1 - c0);
        const int hb = max(it.s0, c0 - 3);       // first k row a tap may read
        const auto rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(c.k + (int64_t)hb * rowQK + it.e * D), 0, (c0 + nt - hb) * rowQK * 2, fl);
        const int64_t lbase = (int64_t)c0 * lrow + (int64_t)it.e * NS * D;
        const auto ru = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.u + lbase), 0, nt * lrow * 2, fl);
        const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.a + lbase), 0, nt * lrow * 2, fl);
        const auto rh = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.h + lbase), 0, nt * lrow * 2, fl);
        const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(c.b + (int64_t)c0 * H + it.e), 0,
                                                          nt * H * 2, fl);
        const uint4* wp = reinterpret_cast<const uint4*>(c.cw + ((int64_t)it.e * D + pc) * 4);   // [H][D][4]
#pragma unroll
        for (int x4 = 0; x4 < 4; ++x4)
            x.w[x4] = wp[x4];
        auto koff = [&](int tl) { return ((c0 + tl - hb) * rowQK + pc) * 2; };   // negative: before the range
#pragma unroll
        for (int m = 0; m < 3; ++m)
            x.hk[m] = ld(rk, koff(tl0 - 1 - m));
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            x.k[j] = ld(rk, koff(tl0 + j));
            const int lo = ((tl0 + j) * lrow + pc) * 2;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                x.u[j][s] = ldn(ru, lo + s * D * 2);
                x.a[j][s] = ldn(ra, lo + s * D * 2);
                if (s < LF - 2)
                    x.h[j][s] = ldn(rh, lo + s * D * 2);
            }
            x.b[j] = __builtin_amdgcn_raw_buffer_load_b16(rb, (tl0 + j) * H * 2, 0, 0);
        }
    };
    auto unpack = [](const uint4& v, float* out) {
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(wv[i] << 16);
            out[2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
        }
    };
    // kw rows of the item (rows past the chunk's end dropped by the range)
    auto emit = [&](const Item& it, const In& x) {
        const int c0 = it.s0 + it.ch * kC;
        const int nt = min(kC, it.s1 - c0);
        const auto rkw = __builtin_amdgcn_make_buffer_rsrc(kw_out + (int64_t)c0 * rowQK + it.e * D, 0,
                                                           nt * rowQK * 2, fl);
        float w[8][4];                           // tap m of channel pc + i
#pragma unroll
        for (int x4 = 0; x4 < 4; ++x4) {
            const uint32_t wv[4] = {x.w[x4].x, x.w[x4].y, x.w[x4].z, x.w[x4].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int lo = 8 * x4 + 2 * i, hi = lo + 1;
                w[lo / 4][lo % 4] = __uint_as_float(wv[i] << 16);
                w[hi / 4][hi % 4] = __uint_as_float(wv[i] & 0xffff0000u);
            }
        }
        float x1[8], x2[8], x3[8];               // k at t - 1, t - 2, t - 3
        unpack(x.hk[0], x1);
        unpack(x.hk[1], x2);
        unpack(x.hk[2], x3);
#pragma unroll
        for (int j = 0; j < ST; ++j) {
            float kt[8], rr[8], acc[8];
            unpack(x.k[j], kt);
            const float bt = bf16_to_f32(x.b[j]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                rr[i] = w[i][3] * kt[i] + w[i][2] * x1[i] + w[i][1] * x2[i] + w[i][0] * x3[i];
                acc[i] = bt * kt[i];
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                float av[8], uv[8];
                unpack(x.a[j][s], av);
                unpack(x.u[j][s], uv);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[i] += av[i] * rr[i] * uv[i];
                if (s < LF - 2) {
                    float hv[8];
                    unpack(x.h[j][s], hv);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        rr[i] *= 1.f - av[i] * hv[i];
                }
            }
            const uint4 out = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                         pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, out), rkw,
                                                   ((tl0 + j) * rowQK + pc) * 2, 0, kScopeDevice);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                x3[i] = x2[i];
                x2[i] = x1[i];
                x1[i] = kt[i];
            }
        }
    };
    // Once every memory operation of this wavefront has completed (the stores
    // of the item just emitted, the loads of the next), its part of the item is
    // visible at device scope: count it in the item's flag.  No workgroup
    // barrier: the wavefronts run out of step, so one's wait overlaps the
    // others' loads.  The item is ready when all kProducerWaves have counted.
    auto finish = [&](const Item& it) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);
        asm volatile("" ::: "memory");
        if (lane == 0)
            __hip_atomic_fetch_add(ready + (int64_t)(it.s0 / kC + it.n + it.ch) * H + it.e, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    };

    Item cur, nxt;
    In X;
    int64_t i = next_item(blockIdx.x, cur);
    if (i < items)
        fetch(cur, X);
    while (i < items) {
        const int64_t j = next_item(i + n_prod, nxt);
        emit(cur, X);
        SCHED_FENCE();
        if (j < items)
            fetch(nxt, X);
        finish(cur);
        i = j;
        cur = nxt;
    }
}

__global__ __launch_bounds__(256) void clear_ready_kernel(int* __restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0;
}

// NW wavefronts: 4 (one per SIMD) or 8 (two per SIMD; slices of 32 columns).
// Wavefront w runs on SIMD w % 4: with eight, the two state wavefronts share
// their SIMDs with the two row movers, and each remaining SIMD runs two Gram
// helpers (five pairs per SIMD).
// LF > 0: the write keys are computed in the kernel from u, a, h and the conv
// taps cw (L = LF levels, closed form, no carried history) instead of read from kw.
// PK > 0: the first n_prod blocks are write-key producers (produce_kw, L = PK
// levels) that write kw and raise kw_ready flags; the scan blocks after them
// read kw once flagged.
// CK: the state wavefronts also write every chunk's start state (ck, ckT).
template <int D, int DVS, int NW, int LF = 0, int PK = 0, bool CK = false>
__global__ __launch_bounds__(NW * 64) void scan_ws_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ kw, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ b,
    const int32_t* __restrict__ cu, int H, int DV, int n_slices,
    const float* __restrict__ s_init, uint16_t* __restrict__ o,
    float* __restrict__ s_final, int split_block, int DV1, int n_slices1, uint16_t* __restrict__ o1,
    float* __restrict__ s_final1, int skip1, const uint16_t* __restrict__ u = nullptr,
    const uint16_t* __restrict__ a = nullptr, const uint16_t* __restrict__ h = nullptr,
    const uint16_t* __restrict__ cw = nullptr, int n_prod = 0, int* kw_ready = nullptr,
    uint16_t* kw_out = nullptr, uint16_t* __restrict__ ck = nullptr, uint16_t* __restrict__ ckT = nullptr)
{
    static_assert(LF == 0 || NW == 8, "fused write keys: the eight-wavefront kernel");
    static_assert(PK == 0 || (NW == 8 && LF == 0), "write-key producers: the eight-wavefront kernel");
    static_assert(!CK || (NW == 8 && LF == 0 && PK == 0), "checkpoints: the eight-wavefront kernel");
    using Ly = LayoutWS<D, DVS>;
    constexpr int NJ = DVS / 16;
    static_assert(NJ == 1 || NJ == 2, "one or two state wavefronts");
    static_assert(NW == 4 || (NW == 8 && NJ == 2), "four, or eight with two state wavefronts");
    static_assert(Ly::total <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(16))) unsigned char smem[Ly::total];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Blocks from split_block on run a second scan over the same sequences: the
    // transitions alone (start S = I with DV1 = D columns, no write term),
    // writing o1 and s_final1.  One launch keeps both on the chip at once.
    // With skip1 = P > 1 the second scan leaves out sequences 0, P, 2P, ...
    // (first segments started from zero need no transition).
    if constexpr (PK > 0) {
        if ((int)blockIdx.x < n_prod) {
            WsCtx pc;
            pc.smem = smem;
            pc.k = k; pc.b = b; pc.u = u; pc.a = a; pc.h = h; pc.cw = cw;
            pc.H = H;
            pc.rowQK = (int64_t)H * D;
            const int n_seqs = (int)((gridDim.x - (unsigned)n_prod) / (unsigned)n_slices) / H;
            produce_kw<D, PK>(pc, cu, n_seqs, n_prod, kw_out, kw_ready);
            return;
        }
    }
    // scan blocks are numbered from 0 after the producers (n_prod is a multiple
    // of the XCD count, so the XCD of a block is unchanged by the renumbering)
    const unsigned bid = blockIdx.x - (unsigned)(PK > 0 ? n_prod : 0);
    const unsigned nbk = gridDim.x - (unsigned)(PK > 0 ? n_prod : 0);
    const bool job1 = (int)bid >= split_block;
    int slice, chain;
    if (job1) {
        xcd_map(bid - (unsigned)split_block, nbk - (unsigned)split_block, n_slices1,
                slice, chain);
        if (skip1 > 1) {
            const int s1 = chain / H;
            chain = ((s1 / (skip1 - 1)) * skip1 + 1 + s1 % (skip1 - 1)) * H + chain % H;
        }
    } else {
        xcd_map(bid, min(nbk, (unsigned)split_block), n_slices, slice, chain);
    }

    WsCtx c;
    c.smem = smem;
    c.q = q; c.k = k; c.g = g; c.b = b;
    c.u = u; c.a = a; c.h = h; c.cw = cw;
    c.kw = job1 ? nullptr : kw;
    c.v = job1 ? nullptr : v;
    c.o = job1 ? o1 : o;
    c.s_init = job1 ? nullptr : s_init;
    c.s_identity = job1;
    c.s_final = job1 ? s_final1 : s_final;
    c.n = chain / H;
    c.e = chain % H;
    c.H = H;
    c.DV = job1 ? DV1 : DV;
    c.j0 = slice * DVS;
    c.seq0 = cu[c.n];
    c.seq1 = cu[c.n + 1];
    c.nchunks = (c.seq1 - c.seq0 + kC - 1) / kC;
    c.lane = tid & 63;
    c.rowQK = (int64_t)H * D;
    c.rowV = (int64_t)H * c.DV;              // the second job's rows are DV1 wide
    c.kw_ready = kw_ready;
    c.ck = ck;
    c.ckT = ckT;

    {
        // matrices (their upper blocks are never written), gates, scratch
        constexpr int nz = (Ly::total - Ly::oAkk) / 16;
        uint4* z = reinterpret_cast<uint4*>(smem + Ly::oAkk);
        for (int i = tid; i < nz; i += NW * 64)
            z[i] = make_uint4(0u, 0u, 0u, 0u);
    }

    // Every role passes the same number of barriers: 4 + 2 per chunk.
    if (wave < NJ) {
        state_loop<D, DVS, NW == 4, NW == 8, CK>(c, wave);
    } else if constexpr (NW == 8) {
        constexpr int K0 = LF ? 0 : -1, K1 = LF ? 1 : -1, K2 = LF ? 2 : -1, K3 = LF ? 3 : -1;
        switch (wave) {
        case 2: helper_loop<D, DVS, 4, 0, 0, true, 0, false, 0, LF, K0>(c); break;   // (0,0) (1,1), gates
        case 3: helper_loop<D, DVS, 6, 0, 0, false, 1, false, -1, LF, K1>(c); break; // (1,0) (2,0) (2,1)
        case 4: helper_loop<D, DVS, 7, 0, 2, false, 0, true, -1, LF, -1, (PK > 0)>(c); break;  // rows 0, 1; T_tt
        case 5: helper_loop<D, DVS, 7, 2, 2, false, 0, false, -1, LF, -1, (PK > 0)>(c); break; // rows of blocks 2, 3
        case 6: helper_loop<D, DVS, 5, 0, 0, false, 2, false, 1, LF, K2>(c); break;  // (2,2) (3,3)
        default: helper_loop<D, DVS, 3, 0, 0, false, 3, false, -1, LF, K3>(c); break; // (3,0) (3,1) (3,2)
        }
    } else if constexpr (NJ == 2) {              // diagonal pairs | six off-diagonal pairs
        if (wave == 2)
            helper_loop<D, DVS, 0, 0, kDiagRowBlocks, true, 0>(c);
        else
            helper_loop<D, DVS, 1, kDiagRowBlocks, 4 - kDiagRowBlocks, false, 1>(c);
    } else {                                     // diagonal | three | three
        if (wave == 1)
            helper_loop<D, DVS, 0, 0, 1, true, 0>(c);
        else if (wave == 2)
            helper_loop<D, DVS, 2, 1, 1, false, 1>(c);
        else
            helper_loop<D, DVS, 3, 2, 2, false, 2>(c);
    }
}

template <int D, int DVS, int NW, bool CK = false>
static hipError_t launch_ws(const ScanArgs& p, hipStream_t stream)
{
    const int n_slices = p.dv / DVS;
    const int64_t blocks = (int64_t)p.n_seqs * p.heads * n_slices;
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL((scan_ws_kernel<D, DVS, NW, 0, 0, CK>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream,
                       (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.kw,
                       (const uint16_t*)p.v, (const uint16_t*)p.g, (const uint16_t*)p.b,
                       p.cu_seqlens, p.heads, p.dv, n_slices, p.s_init, (uint16_t*)p.o,
                       p.s_final, 0x7fffffff, 0, 1, nullptr, nullptr, 0, nullptr, nullptr, nullptr,
                       nullptr, 0, nullptr, nullptr, (uint16_t*)p.ck, (uint16_t*)p.ckT);
    return hipGetLastError();
}

template <int D, int LF>
static hipError_t launch_fused(const ScanArgs& p, hipStream_t stream)
{
    const int n_slices = p.dv / 32;
    const int64_t blocks = (int64_t)p.n_seqs * p.heads * n_slices;
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL((scan_ws_kernel<D, 32, 8, LF>), dim3((unsigned)blocks), dim3(512), 0, stream,
                       (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.kw,
                       (const uint16_t*)p.v, (const uint16_t*)p.g, (const uint16_t*)p.b,
                       p.cu_seqlens, p.heads, p.dv, n_slices, p.s_init, (uint16_t*)p.o,
                       p.s_final, 0x7fffffff, 0, 1, nullptr, nullptr, 0, (const uint16_t*)p.u,
                       (const uint16_t*)p.a, (const uint16_t*)p.h, (const uint16_t*)p.conv_w);
    return hipGetLastError();
}

// The scan with write-key producers: the readiness flags cleared (a fill
// kernel, so the pair can be captured into a HIP graph), then one launch of
// p.kw_producers producer blocks followed by the scan blocks.
template <int D, int L>
static hipError_t launch_prod(const ScanArgs& p, hipStream_t stream)
{
    const int n_slices = p.dv / 32;
    const int64_t blocks = (int64_t)p.n_seqs * p.heads * n_slices;
    if (blocks == 0)
        return hipSuccess;
    const int64_t nflags = ((int64_t)p.total_tokens / kC + p.n_seqs) * p.heads;
    const int64_t cb = (nflags + 255) / 256;
    hipLaunchKernelGGL(clear_ready_kernel, dim3((unsigned)(cb < 1024 ? cb : 1024)), dim3(256), 0, stream,
                       p.kw_ready, nflags);
    hipLaunchKernelGGL((scan_ws_kernel<D, 32, 8, 0, L>), dim3((unsigned)(blocks + p.kw_producers)), dim3(512),
                       0, stream, (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.kw,
                       (const uint16_t*)p.v, (const uint16_t*)p.g, (const uint16_t*)p.b,
                       p.cu_seqlens, p.heads, p.dv, n_slices, p.s_init, (uint16_t*)p.o,
                       p.s_final, 0x7fffffff, 0, 1, nullptr, nullptr, 0, (const uint16_t*)p.u,
                       (const uint16_t*)p.a, (const uint16_t*)p.h, (const uint16_t*)p.conv_w,
                       p.kw_producers, p.kw_ready, const_cast<uint16_t*>((const uint16_t*)p.kw));
    return hipGetLastError();
}

// Two scans in one launch of the eight-wavefront kernel: `a` as given, and
// `m`, the transitions alone over the same sequences (kw = v = null, start
// S = I, m.dv = D columns) except every skip-th one from the first (skip > 1),
// in the blocks after a's.
template <int D>
static hipError_t launch_pair(const ScanArgs& a, const ScanArgs& m, int skip, hipStream_t stream)
{
    const int na = a.dv / 32, nm = m.dv / 32;
    const int m_seqs = skip > 1 ? m.n_seqs / skip * (skip - 1) : m.n_seqs;
    const int64_t ba = (int64_t)a.n_seqs * a.heads * na, bm = (int64_t)m_seqs * m.heads * nm;
    if (ba + bm == 0)
        return hipSuccess;
    hipLaunchKernelGGL((scan_ws_kernel<D, 32, 8>), dim3((unsigned)(ba + bm)), dim3(512), 0, stream,
                       (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.kw,
                       (const uint16_t*)a.v, (const uint16_t*)a.g, (const uint16_t*)a.b,
                       a.cu_seqlens, a.heads, a.dv, na, a.s_init, (uint16_t*)a.o, a.s_final,
                       (int)ba, m.dv, nm, (uint16_t*)m.o, m.s_final, skip);
    return hipGetLastError();
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
                       p.cu_seqlens, p.heads, p.dv, n_slices, p.s_init, (uint16_t*)p.o,
                       p.s_final);
    return hipGetLastError();
}

}  // namespace bf16scan

bool scan_bf16_supported(int dk, int dv, int dvs)
{
    if (dv % dvs != 0 || (dv != 64 && dv != 128))
        return false;
    return (dk == 64 || dk == 128) && (dvs == 16 || dvs == 32 || dvs == 64);
}

hipError_t launch_scan_bf16_pair(const ScanArgs& a, const ScanArgs& m, int skip, hipStream_t s)
{
    if (!scan_bf16_supported(a.dk, a.dv, 32) || m.dv != a.dk || !a.specialised || a.ws_waves != 8 ||
        m.n_seqs != a.n_seqs || m.cu_seqlens != a.cu_seqlens || (skip > 1 && a.n_seqs % skip != 0))
        return hipErrorInvalidValue;
    return a.dk == 64 ? bf16scan::launch_pair<64>(a, m, skip, s)
                      : bf16scan::launch_pair<128>(a, m, skip, s);
}

hipError_t read_wait_giveups(unsigned int* count, bool reset)
{
    hipError_t e = hipMemcpyFromSymbol(count, HIP_SYMBOL(bf16scan::g_wait_giveups), sizeof(unsigned int),
                                       0, hipMemcpyDeviceToHost);
    if (e == hipSuccess && reset) {
        const unsigned int zero = 0;
        e = hipMemcpyToSymbol(HIP_SYMBOL(bf16scan::g_wait_giveups), &zero, sizeof(unsigned int), 0,
                              hipMemcpyHostToDevice);
    }
    return e;
}

// dk = 128 with L = 8 does not fit the Gram helpers' registers (it would spill)
bool scan_fused_kw_supported(int dk, int dv, int L)
{
    return scan_bf16_supported(dk, dv, 32) && (L == 4 || (L == 8 && dk == 64));
}

hipError_t launch_scan_bf16(const ScanArgs& p, hipStream_t s)
{
    if (!scan_bf16_supported(p.dk, p.dv, p.dv_slice))
        return hipErrorInvalidValue;
    if (p.ck || p.ckT) {                         // checkpoints: the eight-wavefront kernel only
        if (!p.ck || !p.ckT || p.fused_L > 0 || !p.specialised || p.ws_waves != 8 || p.dv_slice != 32)
            return hipErrorInvalidValue;
        return p.dk == 64 ? bf16scan::launch_ws<64, 32, 8, true>(p, s)
                          : bf16scan::launch_ws<128, 32, 8, true>(p, s);
    }
    if (p.fused_L > 0) {
        if (!scan_fused_kw_supported(p.dk, p.dv, p.fused_L) || !p.specialised || p.ws_waves != 8 ||
            p.dv_slice != 32 || !p.u || !p.a || !p.h || !p.conv_w)
            return hipErrorInvalidValue;
        if (p.kw_producers > 0) {
            if (p.kw_producers % bf16scan::kXcds != 0 || !p.kw_ready)
                return hipErrorInvalidValue;
            if (p.dk == 64)
                return p.fused_L == 4 ? bf16scan::launch_prod<64, 4>(p, s) : bf16scan::launch_prod<64, 8>(p, s);
            return bf16scan::launch_prod<128, 4>(p, s);
        }
        if (p.dk == 64)
            return p.fused_L == 4 ? bf16scan::launch_fused<64, 4>(p, s) : bf16scan::launch_fused<64, 8>(p, s);
        return bf16scan::launch_fused<128, 4>(p, s);
    }
    if (p.specialised) {
        const bool w8 = p.ws_waves == 8;
        if (p.dk == 64) {
            if (p.dv_slice == 16) return bf16scan::launch_ws<64, 16, 4>(p, s);
            return w8 ? bf16scan::launch_ws<64, 32, 8>(p, s) : bf16scan::launch_ws<64, 32, 4>(p, s);
        }
        if (p.dv_slice == 16) return bf16scan::launch_ws<128, 16, 4>(p, s);
        return w8 ? bf16scan::launch_ws<128, 32, 8>(p, s) : bf16scan::launch_ws<128, 32, 4>(p, s);
    }
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
