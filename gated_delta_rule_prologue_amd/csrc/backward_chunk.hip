// backward_chunk.hip -- chunkwise backward of the bf16 scan (WY/UT form), the
// MFMA counterpart of the token-recurrent scan_bwd_kernel
//
// Gradients of L = sum <dO, o> + <dS_final, S_final> for the gated delta-rule
// recurrence S_t = g_t (I - b_t k_t k_t^T) S_{t-1} + kw_t v_t^T, o_t = S_t^T q_t
// (PRISM pages: WeChat ICML 2026 summary, sections 核心迭代形式 and
// 消除 Token 间串行; gist.science summary of arXiv 2602.10796, section 2.1),
// differentiated through the chunk form of the forward (chunks of 64 tokens,
// gamma the in-chunk cumulative decay, fac = gamma_C / gamma, T = (I + A_kk)^-1):
//
//   X  = T (diag(b gamma) K S0 + A_kkw V)
//   O  = diag(gamma) Q S0 + A_qkw V - A_qk X
//   S1 = gamma_C S0 + KW^T diag(fac) V - K^T diag(fac) X
//
// The gradient dS1 of a chunk's end state is carried from the last chunk to the
// first (pass B, this file):
//
//   dX = -A_qk^T dO - diag(fac) K dS1,   dR = T^T dX,
//   dS0 = gamma_C dS1 + Q^T diag(gamma) dO + K^T diag(b gamma) dR,
//
// and stored per chunk, so that every chunk's input gradients can then be
// formed independently (passes C1, C2) from its start state S0 (stored by the
// forward, chunk_scan_state.hip) and dS1.
#include "common.h"
#include "gram.h"
#include "kernels.h"
#include "mfma_bf16.h"

namespace prism {
namespace bwdc {

using namespace mfma;
using gram::kC;

constexpr int kDVS = 32;                         // value columns per workgroup of pass B
constexpr int kXcds = 8;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// blocks (i, j), i >= j, of a 64x64 lower-triangular matrix in blk_index order
__device__ __forceinline__ constexpr int blk_i(int idx) { return idx < 1 ? 0 : idx < 3 ? 1 : idx < 6 ? 2 : 3; }
__device__ __forceinline__ constexpr int blk_j(int idx) { return idx - blk_i(idx) * (blk_i(idx) + 1) / 2; }

// Workgroups are dispatched to the eight XCDs round-robin; with the chains a
// multiple of eight, all slices of a chain go to one XCD (one L2).
__device__ __forceinline__ void xcd_map(unsigned w, unsigned n_blocks, int n_slices, int& slice, int& chain)
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

// ---------------------------------------------------------------------------
// Pass B: one workgroup per (sequence, head, 32 value columns), four
// wavefronts.  Wavefronts 0 and 1 hold 16 columns of dS each in fp32 MFMA
// accumulators and run the recurrence above chunk by chunk from the last;
// wavefronts 2 and 3 stage chunk c - 1 (k and q rows, the dO slice, T and -A_qk
// expanded to full 64x64 matrices so their transposes are transposed LDS
// reads, and the gates) into the other LDS buffer meanwhile.
// ---------------------------------------------------------------------------
template <int D>
struct LayB {
    static constexpr int LDD = D + 8, LDV = kDVS + 8, LDC = kC + 8;
    static constexpr int szRow = kC * LDD * 2, szV = kC * LDV * 2, szM = kC * LDC * 2;
    static constexpr int oK = 0, oQ = szRow, oO = 2 * szRow, oT = oO + szV, oN = oT + szM;
    static constexpr int oG = oN + szM;          // gamma, b gamma, fac (64 each), gamma_C
    static constexpr int szBuf = oG + 3 * kC * 4 + 16;
    static constexpr int total = 2 * szBuf;
    static_assert(szRow % 16 == 0 && oT % 16 == 0 && oG % 16 == 0 && szBuf % 16 == 0, "alignment");
    static_assert(total <= 160 * 1024, "LDS budget");
};

struct CtxB {
    const uint16_t *q, *k, *dO, *g, *b, *mats;
    int n, e, H, DV, j0, seq0, seq1, nchunks, lane;
    int64_t rowQK, rowV, vbase;
};

// mover m (0, 1): tokens 32 m .. 32 m + 31 of chunk ch (q, k rows, the dO slice),
// and the chunk's T (mover 0, with the gates) or -A_qk (mover 1).  The loads of a
// chunk go to registers (load) one chunk before they are stored into an LDS
// buffer (store), so each has a whole chunk period to arrive.
template <int D>
struct StageB {
    static constexpr int PPR = D / 8, NPQ = D / 16;
    uint4 vk[NPQ], vq[NPQ], vo[2], vm[5];
    uint16_t gv, bv;
    int nt;

    __device__ __forceinline__ void load(const CtxB& c, int ch, int m)
    {
        const int lane = c.lane;
        const int c0 = c.seq0 + ch * kC;
        nt = __builtin_amdgcn_readfirstlane(max(0, min(kC, c.seq1 - c0)));
        const auto rk = rsrc(c.k + (int64_t)c0 * c.rowQK + (int64_t)c.e * D, nt * (int)c.rowQK * 2);
        const auto rq = rsrc(c.q + (int64_t)c0 * c.rowQK + (int64_t)c.e * D, nt * (int)c.rowQK * 2);
        const auto ro = rsrc(c.dO + (int64_t)c0 * c.rowV + (int64_t)c.e * c.DV + c.j0, nt * (int)c.rowV * 2);
#pragma unroll
        for (int x = 0; x < NPQ; ++x) {
            const int p = lane + 64 * x;
            const int off = ((32 * m + p / PPR) * (int)c.rowQK + (p % PPR) * 8) * 2;
            vk[x] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
            vq[x] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
        }
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int p = lane + 64 * x;
            vo[x] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  ro, ((32 * m + p / 4) * (int)c.rowV + (p % 4) * 8) * 2, 0, 0));
        }
        // the chunk's stored matrix (T for mover 0, -A_qk for mover 1): ten 16x16 blocks
        const int mat = m == 0 ? gram::kMatT : gram::kMatNAqk;
        const auto rm = rsrc(c.mats + ((c.vbase + ch) * c.H + c.e) * (int64_t)gram::kChunkElems +
                                 mat * gram::kMatElems,
                             gram::kMatElems * 2);
#pragma unroll
        for (int x = 0; x < 5; ++x) {
            const int idx = lane + 64 * x, blk = idx / 32, p = idx % 32;
            const int r = p / 2, hh = p % 2;
            vm[x] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rm, (blk * gram::kBlockElems + gram::swz(r, 8 * hh)) * 2, 0, 0));
        }
        gv = 0;
        bv = 0;
        if (m == 0) {
            const auto rg = rsrc(c.g + (int64_t)c0 * c.H + c.e, nt * c.H * 2);
            const auto rb = rsrc(c.b + (int64_t)c0 * c.H + c.e, nt * c.H * 2);
            gv = __builtin_amdgcn_raw_buffer_load_b16(rg, lane * c.H * 2, 0, 0);
            bv = __builtin_amdgcn_raw_buffer_load_b16(rb, lane * c.H * 2, 0, 0);
        }
    }

    __device__ __forceinline__ void store(const CtxB& c, unsigned char* buf, int m) const
    {
        using Ly = LayB<D>;
        const int lane = c.lane;
        uint16_t* sK = reinterpret_cast<uint16_t*>(buf + Ly::oK);
        uint16_t* sQ = reinterpret_cast<uint16_t*>(buf + Ly::oQ);
        uint16_t* sO = reinterpret_cast<uint16_t*>(buf + Ly::oO);
        uint16_t* sM = reinterpret_cast<uint16_t*>(buf + (m == 0 ? Ly::oT : Ly::oN));
#pragma unroll
        for (int x = 0; x < NPQ; ++x) {
            const int p = lane + 64 * x;
            const int off = (32 * m + p / PPR) * Ly::LDD + (p % PPR) * 8;
            *reinterpret_cast<uint4*>(sK + off) = vk[x];
            *reinterpret_cast<uint4*>(sQ + off) = vq[x];
        }
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int p = lane + 64 * x;
            *reinterpret_cast<uint4*>(sO + (32 * m + p / 4) * Ly::LDV + (p % 4) * 8) = vo[x];
        }
#pragma unroll
        for (int x = 0; x < 5; ++x) {
            const int idx = lane + 64 * x, blk = idx / 32, p = idx % 32;
            const int r = p / 2, hh = p % 2;
            *reinterpret_cast<uint4*>(sM + (16 * blk_i(blk) + r) * Ly::LDC + 16 * blk_j(blk) + 8 * hh) = vm[x];
        }
        if (m == 0) {
            float* G = reinterpret_cast<float*>(buf + Ly::oG);
            const float l2 = lane < nt ? __log2f(fmaxf(bf16_to_f32(gv), 1e-30f)) : 0.f;
            const float lam = wave_inclusive_sum(l2);
            const float lamC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), 63));
            const float gam = __builtin_amdgcn_exp2f(lam);
            G[lane] = gam;
            G[kC + lane] = bf16_to_f32(bv) * gam;
            G[2 * kC + lane] = __builtin_amdgcn_exp2f(lamC - lam);
            if (lane == 0)
                G[3 * kC] = __builtin_amdgcn_exp2f(lamC);
        }
    }
};

// state wavefront jb: one chunk of the recurrence for value columns j0 + 16 jb ..
template <int D>
__device__ __forceinline__ void dstate_chunk(f32x4_t (&dS)[D / 16], const unsigned char* buf, const CtxB& c, int jb)
{
    using Ly = LayB<D>;
    constexpr int LDD = Ly::LDD, LDV = Ly::LDV, LDC = Ly::LDC;
    constexpr int NI = D / 16, NKP = NI / 2;
    const int lane = c.lane, lg = lane >> 4;
    const uint16_t* sK = reinterpret_cast<const uint16_t*>(buf + Ly::oK);
    const uint16_t* sQ = reinterpret_cast<const uint16_t*>(buf + Ly::oQ);
    const uint16_t* sO = reinterpret_cast<const uint16_t*>(buf + Ly::oO);
    const uint16_t* sT = reinterpret_cast<const uint16_t*>(buf + Ly::oT);
    const uint16_t* sN = reinterpret_cast<const uint16_t*>(buf + Ly::oN);
    const float* sGam = reinterpret_cast<const float*>(buf + Ly::oG);
    const float* sBG = sGam + kC;
    const float* sFac = sGam + 2 * kC;

    // dS1 as 16x16x32 operands (channels 32 kp + 8 g .. in lane group g)
    bf16x8_t s1q[NKP];
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp)
        s1q[kp] = pair_rows(as_b16(dS[2 * kp], 1.f, 1.f, 1.f, 1.f), as_b16(dS[2 * kp + 1], 1.f, 1.f, 1.f, 1.f));
    // dO (tokens 32 h2 + 8 g .., this wavefront's columns)
    bf16x8_t of[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
        of[h2] = frag_col(sO + h2 * 32 * LDV + jb * 16, LDV, lane);
    SCHED_FENCE();

    // Y = K dS1 (four chains), Xl = (-A_qk)^T dO
    f32x4_t Y[4], Xl[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        Y[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        Xl[tb] = Y[tb];
    }
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
            Y[tb] = mma32(frag_row(sK + tb * 16 * LDD + kp * 32, LDD, lane), s1q[kp], Y[tb]);
    }
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
        for (int h2 = sb / 2; h2 < 2; ++h2)
            Xl[sb] = mma32(frag_col(sN + h2 * 32 * LDC + sb * 16, LDC, lane), of[h2], Xl[sb]);
    }
    // dX = Xl - diag(fac) Y;  dR = T^T dX
    bf16x8_t dxq[2];
    {
        v4s_t xb[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const float4 f = *reinterpret_cast<const float4*>(sFac + sb * 16 + lg * 4);
            const f32x4_t dx = {Xl[sb][0] - f.x * Y[sb][0], Xl[sb][1] - f.y * Y[sb][1],
                                Xl[sb][2] - f.z * Y[sb][2], Xl[sb][3] - f.w * Y[sb][3]};
            xb[sb] = as_b16(dx, 1.f, 1.f, 1.f, 1.f);
        }
        dxq[0] = pair_rows(xb[0], xb[1]);
        dxq[1] = pair_rows(xb[2], xb[3]);
    }
    f32x4_t dR[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
        dR[sb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h2 = sb / 2; h2 < 2; ++h2)
            dR[sb] = mma32(frag_col(sT + h2 * 32 * LDC + sb * 16, LDC, lane), dxq[h2], dR[sb]);
    }
    SCHED_FENCE();

    // dS <- gamma_C dS + Q^T diag(gamma) dO + K^T diag(b gamma) dR
    const float gC = sGam[3 * kC];
#pragma unroll
    for (int ib = 0; ib < NI; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dS[ib][r] *= gC;
    bf16x8_t og[2], drq[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        const float4 g0 = *reinterpret_cast<const float4*>(sGam + h2 * 32 + lg * 8);
        const float4 g1 = *reinterpret_cast<const float4*>(sGam + h2 * 32 + lg * 8 + 4);
        og[h2] = scale8(of[h2], g0, g1);
        const float4 b0 = *reinterpret_cast<const float4*>(sBG + h2 * 32 + lg * 4);
        const float4 b1 = *reinterpret_cast<const float4*>(sBG + h2 * 32 + 16 + lg * 4);
        drq[h2] = pair_rows(as_b16(dR[2 * h2], b0.x, b0.y, b0.z, b0.w),
                            as_b16(dR[2 * h2 + 1], b1.x, b1.y, b1.z, b1.w));
    }
#pragma unroll
    for (int ib = 0; ib < NI; ++ib) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            dS[ib] = mma32(frag_col(sQ + h2 * 32 * LDD + ib * 16, LDD, lane), og[h2], dS[ib]);
            dS[ib] = mma32(frag_col(sK + h2 * 32 * LDD + ib * 16, LDD, lane), drq[h2], dS[ib]);
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_state_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ b, const int32_t* __restrict__ cu,
    int H, int DV, int n_slices, const uint16_t* __restrict__ mats, const float* __restrict__ dS_final,
    uint16_t* __restrict__ dck, uint16_t* __restrict__ dckT, float* __restrict__ dS_init)
{
    using Ly = LayB<D>;
    constexpr int NI = D / 16;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Ly::total];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int slice, chain;
    xcd_map(blockIdx.x, gridDim.x, n_slices, slice, chain);
    CtxB c;
    c.q = q; c.k = k; c.dO = dO; c.g = g; c.b = b; c.mats = mats;
    c.n = chain / H;
    c.e = chain % H;
    c.H = H;
    c.DV = DV;
    c.j0 = slice * kDVS;
    c.seq0 = cu[c.n];
    c.seq1 = cu[c.n + 1];
    c.nchunks = (c.seq1 - c.seq0 + kC - 1) / kC;
    c.lane = tid & 63;
    c.rowQK = (int64_t)H * D;
    c.rowV = (int64_t)H * DV;
    c.vbase = c.seq0 / kC + c.n;
    const int li = c.lane & 15, lg = c.lane >> 4;

    // the full matrices' blocks above the diagonal are never written: zero them once
    for (int i = tid; i < 2 * Ly::szM / 16; i += 256) {
#pragma unroll
        for (int bsel = 0; bsel < 2; ++bsel)
            *reinterpret_cast<uint4*>(smem + bsel * Ly::szBuf + Ly::oT + 16 * i) = make_uint4(0u, 0u, 0u, 0u);
    }
    lds_barrier();

    if (wave < 2) {
        const int jb = wave;
        f32x4_t dS[NI];
        const int64_t sb = (((int64_t)c.n * H + c.e) * D) * DV + c.j0 + jb * 16;
#pragma unroll
        for (int ib = 0; ib < NI; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dS[ib][r] = dS_final ? dS_final[sb + (int64_t)(ib * 16 + lg * 4 + r) * DV + li] : 0.f;
        lds_barrier();                           // the last chunk staged
        for (int ch = c.nchunks - 1; ch >= 0; --ch) {
            // dS at the end of chunk ch, bf16, as rows [dk][dv] and transposed [dv][dk]
            const int64_t vc = (c.vbase + ch) * H + c.e;
            const int col = c.j0 + jb * 16 + li;
#pragma unroll
            for (int ib = 0; ib < NI; ++ib) {
                const int r0 = ib * 16 + lg * 4;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dck[(vc * D + r0 + r) * DV + col] = (uint16_t)(pack_bf16x2(dS[ib][r], 0.f) & 0xffffu);
                *reinterpret_cast<uint2*>(dckT + (vc * DV + col) * D + r0) =
                    make_uint2(pack_bf16x2(dS[ib][0], dS[ib][1]), pack_bf16x2(dS[ib][2], dS[ib][3]));
            }
            dstate_chunk<D>(dS, smem + (ch & 1) * Ly::szBuf, c, jb);
            lds_barrier();
        }
        if (dS_init) {
#pragma unroll
            for (int ib = 0; ib < NI; ++ib)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dS_init[sb + (int64_t)(ib * 16 + lg * 4 + r) * DV + li] = dS[ib][r];
        }
    } else {
        // chunk ch - 1 is stored while chunk ch - 2 loads (past the first chunk the
        // ranges are empty and nothing is stored)
        const int m = wave - 2;
        StageB<D> st;
        if (c.nchunks > 0) {
            st.load(c, c.nchunks - 1, m);
            st.store(c, smem + ((c.nchunks - 1) & 1) * Ly::szBuf, m);
        }
        if (c.nchunks > 1)
            st.load(c, c.nchunks - 2, m);
        lds_barrier();
        for (int ch = c.nchunks - 1; ch >= 0; --ch) {
            if (ch >= 1) {
                st.store(c, smem + ((ch - 1) & 1) * Ly::szBuf, m);
                if (ch >= 2)
                    st.load(c, ch - 2, m);
            }
            lds_barrier();
        }
    }
}

// ---------------------------------------------------------------------------
// The chunk-parallel gradients: one workgroup per (virtual chunk, head), eight
// wavefronts (two per SIMD); wavefront w owns the chunk's tokens 16 (w & 3) ..
// + 15 and column half w >> 2 of every output, so every gradient element is
// written once, by one workgroup (no global atomics).  In order:
//   X = T (diag(b gamma) K S0 + A_kkw V), dX, dR = T^T dX (as in pass B),
//   dV = diag(fac) KW dS1 + A_qkw^T dO + A_kkw^T dR;
//   the Gram matrices and their gradients dA_qkw = tril0(dO V^T),
//   dA_qk = -tril0(dO X^T), dA_kk = -tril-1(dR X^T), dA_kkw = tril-1(dR V^T),
//   M = dA (.) D (b by row for the kk pair), with the row and column sums the
//   decay gradient needs;
//   dQ = diag(gamma) dO S0^T + M_qk K + M_qkw KW,
//   dK = diag(b gamma) dR S0^T - diag(fac) X dS1^T + (M_kk + M_kk^T) K + M_kkw KW + M_qk^T Q,
//   dKW = diag(fac) V dS1^T + M_kkw^T K + M_qkw^T Q, with the per-token dot
//   products the decay and b gradients need; then db and dg (d/d ln gamma
//   summed backwards over the chunk).
// S0 and dS1 come from the bf16 checkpoints, whose two layouts give every
// MFMA fragment as one 16-byte read.
// ---------------------------------------------------------------------------
struct CtxC {
    const uint16_t *g, *b;
    int H, DV, c0, nt, lane, e;
    int64_t rowQK, rowV, vcid;                   // vcid: (virtual chunk) * H + head
};

// the sequence of virtual chunk vch (chunks numbered floor(cu[n] / 64) + n + i)
// and the chunk's first token and token count; false for a slot no chunk uses
__device__ __forceinline__ bool locate(const int32_t* cu, int n_seqs, int vch, int& c0, int& nt)
{
    int lo = 0, hi = n_seqs;                     // largest n with floor(cu[n]/64) + n <= vch
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] / kC + mid <= vch) lo = mid; else hi = mid;
    }
    const int n = lo;
    const int ch = vch - (cu[n] / kC + n);
    c0 = cu[n] + ch * kC;
    nt = min(kC, cu[n + 1] - c0);
    return ch >= 0 && nt > 0;
}

// sum over the 16 lanes of a lane group (all of them get it)
__device__ __forceinline__ float sum16(float x)
{
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    return x;
}

__device__ __forceinline__ bf16x8_t ldg16(const uint16_t* p)
{
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

// Staging of the chunk-parallel kernels (kNW wavefronts): every load of a
// tensor's 64 x W tile is issued into registers before any LDS store, so the
// workgroup waits for memory once.  Rows past the chunk's nt tokens read as zero.
constexpr int kNW = 8;

template <int W>
struct StageRows {
    static constexpr int PPR = W / 8, N = kC * PPR / (kNW * 64);
    uint4 x[N];
    __device__ __forceinline__ void load(const uint16_t* src, int64_t row, int nt, int tid)
    {
        const auto rs = rsrc(src, nt * (int)row * 2);
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int p = tid + kNW * 64 * j;
            x[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rs, ((p / PPR) * (int)row + (p % PPR) * 8) * 2, 0, 0));
        }
    }
    template <int LD>
    __device__ __forceinline__ void store(uint16_t* dst, int tid) const
    {
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int p = tid + kNW * 64 * j;
            *reinterpret_cast<uint4*>(dst + (p / PPR) * LD + (p % PPR) * 8) = x[j];
        }
    }
};

// one stored lower-triangular matrix (ten blocks) as a full 64 x 64 matrix,
// zeros above the diagonal blocks: thread tid moves one 16-byte half row
struct StageMat {
    uint4 x;
    __device__ __forceinline__ void load(const uint16_t* m, int tid)
    {
        const int bi = tid / 128, bj = (tid / 32) % 4, p = tid % 32;
        x = make_uint4(0u, 0u, 0u, 0u);
        if (bj <= bi)
            x = *reinterpret_cast<const uint4*>(m + gram::blk_index(bi, bj) * gram::kBlockElems +
                                                gram::swz(p / 2, 8 * (p % 2)));
    }
    template <int LDC>
    __device__ __forceinline__ void store(uint16_t* dst, int tid) const
    {
        const int bi = tid / 128, bj = (tid / 32) % 4, p = tid % 32;
        *reinterpret_cast<uint4*>(dst + (16 * bi + p / 2) * LDC + 16 * bj + 8 * (p % 2)) = x;
    }
};

// gates of the chunk (wavefront 0, lane = token): gamma, b gamma, fac, lambda
// (log2 of gamma), g, b (64 each), then gamma_C
__device__ __forceinline__ void gates_c(float* G, const CtxC& c)
{
    const int lane = c.lane;
    const auto rg = rsrc(c.g + (int64_t)c.c0 * c.H + c.e, c.nt * c.H * 2);
    const auto rb = rsrc(c.b + (int64_t)c.c0 * c.H + c.e, c.nt * c.H * 2);
    const float gv = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rg, lane * c.H * 2, 0, 0));
    const float bv = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rb, lane * c.H * 2, 0, 0));
    const float l2 = lane < c.nt ? __log2f(fmaxf(gv, 1e-30f)) : 0.f;
    const float lam = wave_inclusive_sum(l2);
    const float lamC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), 63));
    const float gam = __builtin_amdgcn_exp2f(lam);
    G[lane] = gam;
    G[kC + lane] = bv * gam;
    G[2 * kC + lane] = __builtin_amdgcn_exp2f(lamC - lam);
    G[3 * kC + lane] = lam;
    G[4 * kC + lane] = lane < c.nt ? gv : 1.f;
    G[5 * kC + lane] = bv;
    if (lane == 0)
        G[6 * kC] = __builtin_amdgcn_exp2f(lamC);
}
constexpr int kGateBytes = 6 * kC * 4 + 16;

__device__ __forceinline__ void st_rows(uint16_t* dst, int ld, int t0, const f32x4_t& x, int col)
{
#pragma unroll
    for (int r = 0; r < 4; ++r)
        dst[(t0 + r) * ld + col] = (uint16_t)(pack_bf16x2(x[r], 0.f) & 0xffffu);
}

// block pairs (t-block, s-block), s <= t, in order (0,0) (1,0) (1,1) (2,0) ..
__device__ __forceinline__ constexpr int pair_t(int p) { return p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3; }
__device__ __forceinline__ constexpr int pair_s(int p) { return p - pair_t(p) * (pair_t(p) + 1) / 2; }

template <int D, int DV>
struct LayG {
    static constexpr int LDD = D + 8, LDV = DV + 8, LDC = kC + 8;
    static constexpr int szD = kC * LDD * 2, szV = kC * LDV * 2, szM = kC * LDC * 2;
    static constexpr int oK = 0, oKW = szD, oQ = 2 * szD, oV = 3 * szD, oO = oV + szV;
    static constexpr int oT = oO + szV, oAkw = oT + szM, oNqk = oAkw + szM, oAqw = oNqk + szM;
    static constexpr int oR = oAqw + szM, oX = oR + szV, oG = oX + szV;
    static constexpr int oSc = oG + kGateBytes;  // per-token dot products (3 x 64), then the
    static constexpr int oL = oSc + 3 * kC * 4;  // decay gradient l and db's Gram part (64 each)
    static constexpr int oRed = oL + 2 * kC * 4;
    static constexpr int total = oRed + kNW * 4;
    static_assert(total <= 160 * 1024, "LDS budget");
};

// The chunk-parallel gradients of one (chunk, head).  Wavefront w: token rows
// 16 (w & 3) .., value (or key) column half w >> 2; in the block-pair stage,
// pairs w and w + 8.  The stored T, A_kkw, -A_qk and A_qkw tiles are dead after
// dV, and their LDS holds M_qk, M_qkw, M_kk and M_kkw from there on.
template <int D, int DV, typename GT>
__global__ __launch_bounds__(kNW * 64) void bwd_grads_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ kw,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO, const uint16_t* __restrict__ g,
    const uint16_t* __restrict__ b, const int32_t* __restrict__ cu, int n_seqs, int H,
    const uint16_t* __restrict__ mats, const uint16_t* __restrict__ ck, const uint16_t* __restrict__ ckT,
    const uint16_t* __restrict__ dck, const uint16_t* __restrict__ dckT, GT* __restrict__ gq,
    float* __restrict__ gk, float* __restrict__ gkw, GT* __restrict__ gv, float* __restrict__ gg,
    float* __restrict__ gb)
{
    using Ly = LayG<D, DV>;
    constexpr int LDD = Ly::LDD, LDV = Ly::LDV, LDC = Ly::LDC;
    constexpr int NKD = D / 32, NKV = DV / 32;
    constexpr int HV = DV / 32, HD = D / 32;     // 16-column tiles of a column half
    __shared__ __attribute__((aligned(16))) unsigned char smem[Ly::total];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tb = wave & 3, nh = wave >> 2;
    const int vch = blockIdx.x / H, e = blockIdx.x % H;
    CtxC c;
    if (!locate(cu, n_seqs, vch, c.c0, c.nt))
        return;
    c.g = g; c.b = b;
    c.H = H; c.DV = DV; c.e = e; c.lane = tid & 63;
    c.rowQK = (int64_t)H * D;
    c.rowV = (int64_t)H * DV;
    c.vcid = (int64_t)vch * H + e;
    const int lane = c.lane, li = lane & 15, lg = lane >> 4;
    uint16_t* sK = reinterpret_cast<uint16_t*>(smem + Ly::oK);
    uint16_t* sKW = reinterpret_cast<uint16_t*>(smem + Ly::oKW);
    uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + Ly::oQ);
    uint16_t* sV = reinterpret_cast<uint16_t*>(smem + Ly::oV);
    uint16_t* sO = reinterpret_cast<uint16_t*>(smem + Ly::oO);
    uint16_t* sT = reinterpret_cast<uint16_t*>(smem + Ly::oT);
    uint16_t* sAkw = reinterpret_cast<uint16_t*>(smem + Ly::oAkw);
    uint16_t* sNqk = reinterpret_cast<uint16_t*>(smem + Ly::oNqk);
    uint16_t* sAqw = reinterpret_cast<uint16_t*>(smem + Ly::oAqw);
    uint16_t* sR = reinterpret_cast<uint16_t*>(smem + Ly::oR);
    uint16_t* sX = reinterpret_cast<uint16_t*>(smem + Ly::oX);
    float* G = reinterpret_cast<float*>(smem + Ly::oG);
    float* sSc = reinterpret_cast<float*>(smem + Ly::oSc);
    float* sL = reinterpret_cast<float*>(smem + Ly::oL);   // d/d ln gamma per token
    float* sDB = sL + kC;                                  // db (Gram part) per token
    float* sRed = reinterpret_cast<float*>(smem + Ly::oRed);
    const int t0 = tb * 16 + lg * 4;             // this lane's first token row of a tile
    const uint16_t* ckT0 = ckT + c.vcid * (int64_t)DV * D;
    const uint16_t* ck0 = ck + c.vcid * (int64_t)D * DV;
    const uint16_t* dckT0 = dckT + c.vcid * (int64_t)DV * D;
    const uint16_t* dck0 = dck + c.vcid * (int64_t)D * DV;
    const int v0c = nh * (DV / 2), d0c = nh * (D / 2);   // first column of this wavefront's half
    // B fragments of S0 (the first product) and of dS1 (dX and dV), read ahead
    bf16x8_t fS[NKD][HV];

    {
        const int64_t r0 = (int64_t)c.c0 * c.rowQK + (int64_t)e * D, v0 = (int64_t)c.c0 * c.rowV + (int64_t)e * DV;
        const uint16_t* m = mats + c.vcid * (int64_t)gram::kChunkElems;
        StageRows<D> xk, xkw, xq;
        StageRows<DV> xv, xo;
        StageMat mt, makw, mnqk, maqw;
        xk.load(k + r0, c.rowQK, c.nt, tid);
        xkw.load(kw + r0, c.rowQK, c.nt, tid);
        xq.load(q + r0, c.rowQK, c.nt, tid);
        xv.load(v + v0, c.rowV, c.nt, tid);
        xo.load(dO + v0, c.rowV, c.nt, tid);
        mt.load(m + gram::kMatT * gram::kMatElems, tid);
        makw.load(m + gram::kMatAkkw * gram::kMatElems, tid);
        mnqk.load(m + gram::kMatNAqk * gram::kMatElems, tid);
        maqw.load(m + gram::kMatAqkw * gram::kMatElems, tid);
        // S0 fragments of the first product, in flight with the staging
#pragma unroll
        for (int kp = 0; kp < NKD; ++kp)
#pragma unroll
            for (int n = 0; n < HV; ++n)
                fS[kp][n] = ldg16(ckT0 + (v0c + n * 16 + li) * D + kp * 32 + lg * 8);
        if (wave == 0)
            gates_c(G, c);
        xk.template store<LDD>(sK, tid);
        xkw.template store<LDD>(sKW, tid);
        xq.template store<LDD>(sQ, tid);
        xv.template store<LDV>(sV, tid);
        xo.template store<LDV>(sO, tid);
        mt.template store<LDC>(sT, tid);
        makw.template store<LDC>(sAkw, tid);
        mnqk.template store<LDC>(sNqk, tid);
        maqw.template store<LDC>(sAqw, tid);
        if (tid < 5 * kC)
            sSc[tid] = 0.f;                      // sSc, sL and sDB
    }
    lds_barrier();
    const float* sBG = G + kC;
    const float* sFac = G + 2 * kC;

    // ---- R = diag(b gamma) K S0 + A_kkw V -> sR
    {
        f32x4_t acc[HV];
#pragma unroll
        for (int n = 0; n < HV; ++n)
            acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < NKD; ++kp) {
            const bf16x8_t a = frag_row(sK + tb * 16 * LDD + kp * 32, LDD, lane);
#pragma unroll
            for (int n = 0; n < HV; ++n)
                acc[n] = mma32(a, fS[kp][n], acc[n]);
        }
        // dS1 fragments for dX and dV, in flight from here
#pragma unroll
        for (int kp = 0; kp < NKD; ++kp)
#pragma unroll
            for (int n = 0; n < HV; ++n)
                fS[kp][n] = ldg16(dckT0 + (v0c + n * 16 + li) * D + kp * 32 + lg * 8);
        const float4 bg = *reinterpret_cast<const float4*>(sBG + t0);
#pragma unroll
        for (int n = 0; n < HV; ++n) {
            acc[n][0] *= bg.x; acc[n][1] *= bg.y; acc[n][2] *= bg.z; acc[n][3] *= bg.w;
        }
#pragma unroll
        for (int h2 = 0; h2 <= 1; ++h2) {
            if (h2 <= tb / 2) {
                const bf16x8_t a = frag_row(sAkw + tb * 16 * LDC + h2 * 32, LDC, lane);
#pragma unroll
                for (int n = 0; n < HV; ++n)
                    acc[n] = mma32(a, frag_col(sV + h2 * 32 * LDV + v0c + n * 16, LDV, lane), acc[n]);
            }
        }
#pragma unroll
        for (int n = 0; n < HV; ++n)
            st_rows(sR, LDV, t0, acc[n], v0c + n * 16 + li);
    }
    lds_barrier();
    // ---- X = T R -> sX
    {
        f32x4_t acc[HV];
#pragma unroll
        for (int n = 0; n < HV; ++n)
            acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h2 = 0; h2 <= 1; ++h2) {
            if (h2 <= tb / 2) {
                const bf16x8_t a = frag_row(sT + tb * 16 * LDC + h2 * 32, LDC, lane);
#pragma unroll
                for (int n = 0; n < HV; ++n)
                    acc[n] = mma32(a, frag_col(sR + h2 * 32 * LDV + v0c + n * 16, LDV, lane), acc[n]);
            }
        }
#pragma unroll
        for (int n = 0; n < HV; ++n)
            st_rows(sX, LDV, t0, acc[n], v0c + n * 16 + li);
    }
    lds_barrier();
    // ---- dX = (-A_qk)^T dO - diag(fac) K dS1 -> sR
    {
        f32x4_t y[HV], xl[HV];
#pragma unroll
        for (int n = 0; n < HV; ++n) {
            y[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            xl[n] = y[n];
        }
#pragma unroll
        for (int kp = 0; kp < NKD; ++kp) {
            const bf16x8_t a = frag_row(sK + tb * 16 * LDD + kp * 32, LDD, lane);
#pragma unroll
            for (int n = 0; n < HV; ++n)
                y[n] = mma32(a, fS[kp][n], y[n]);
        }
#pragma unroll
        for (int h2 = 0; h2 <= 1; ++h2) {
            if (h2 >= tb / 2) {
                const bf16x8_t a = frag_col(sNqk + h2 * 32 * LDC + tb * 16, LDC, lane);
#pragma unroll
                for (int n = 0; n < HV; ++n)
                    xl[n] = mma32(a, frag_col(sO + h2 * 32 * LDV + v0c + n * 16, LDV, lane), xl[n]);
            }
        }
        const float4 f = *reinterpret_cast<const float4*>(sFac + t0);
#pragma unroll
        for (int n = 0; n < HV; ++n) {
            const f32x4_t dx = {xl[n][0] - f.x * y[n][0], xl[n][1] - f.y * y[n][1], xl[n][2] - f.z * y[n][2],
                                xl[n][3] - f.w * y[n][3]};
            st_rows(sR, LDV, t0, dx, v0c + n * 16 + li);
        }
    }
    lds_barrier();
    // ---- dR = T^T dX -> sR (after every wavefront has read dX)
    {
        f32x4_t acc[HV];
#pragma unroll
        for (int n = 0; n < HV; ++n)
            acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h2 = 0; h2 <= 1; ++h2) {
            if (h2 >= tb / 2) {
                const bf16x8_t a = frag_col(sT + h2 * 32 * LDC + tb * 16, LDC, lane);
#pragma unroll
                for (int n = 0; n < HV; ++n)
                    acc[n] = mma32(a, frag_col(sR + h2 * 32 * LDV + v0c + n * 16, LDV, lane), acc[n]);
            }
        }
        lds_barrier();
#pragma unroll
        for (int n = 0; n < HV; ++n)
            st_rows(sR, LDV, t0, acc[n], v0c + n * 16 + li);
    }
    lds_barrier();

    const float4 gam4 = *reinterpret_cast<const float4*>(G + t0);
    const float4 bg4 = *reinterpret_cast<const float4*>(sBG + t0);
    const float4 fac4 = *reinterpret_cast<const float4*>(sFac + t0);
    const float gam[4] = {gam4.x, gam4.y, gam4.z, gam4.w}, bgm[4] = {bg4.x, bg4.y, bg4.z, bg4.w},
                fac[4] = {fac4.x, fac4.y, fac4.z, fac4.w};
    auto row_ok = [&](int r) { return t0 + r < c.nt; };
    auto gidx = [&](int r, int64_t rowlen, int wdt, int col) {
        return (int64_t)(c.c0 + t0 + r) * rowlen + (int64_t)e * wdt + col;
    };

    // B fragments of S0^T and dS1^T for the last products (rows of the checkpoints),
    // two 16-row tiles ahead, the first two in flight from here
    bf16x8_t f0[2][NKV], f1[2][NKV];
    auto load_fin = [&](int n, int slot) {
        const int col = d0c + n * 16 + li;
#pragma unroll
        for (int kp = 0; kp < NKV; ++kp) {
            f0[slot][kp] = ldg16(ck0 + col * DV + kp * 32 + lg * 8);
            f1[slot][kp] = ldg16(dck0 + col * DV + kp * 32 + lg * 8);
        }
    };
    load_fin(0, 0);
    if (HD > 1)
        load_fin(1, 1);

    // ---- dV = diag(fac) KW dS1 + A_qkw^T dO + A_kkw^T dR
    {
        f32x4_t acc[HV];
#pragma unroll
        for (int n = 0; n < HV; ++n)
            acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kp = 0; kp < NKD; ++kp) {
            const bf16x8_t a = frag_row(sKW + tb * 16 * LDD + kp * 32, LDD, lane);
#pragma unroll
            for (int n = 0; n < HV; ++n)
                acc[n] = mma32(a, fS[kp][n], acc[n]);
        }
#pragma unroll
        for (int n = 0; n < HV; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[n][r] *= fac[r];
#pragma unroll
        for (int h2 = 0; h2 <= 1; ++h2) {
            if (h2 >= tb / 2) {
                const bf16x8_t a1 = frag_col(sAqw + h2 * 32 * LDC + tb * 16, LDC, lane);
                const bf16x8_t a2 = frag_col(sAkw + h2 * 32 * LDC + tb * 16, LDC, lane);
#pragma unroll
                for (int n = 0; n < HV; ++n) {
                    acc[n] = mma32(a1, frag_col(sO + h2 * 32 * LDV + v0c + n * 16, LDV, lane), acc[n]);
                    acc[n] = mma32(a2, frag_col(sR + h2 * 32 * LDV + v0c + n * 16, LDV, lane), acc[n]);
                }
            }
        }
#pragma unroll
        for (int n = 0; n < HV; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (row_ok(r))
                    gv[gidx(r, c.rowV, DV, v0c + n * 16 + li)] = from_f32<GT>(acc[n][r]);
    }

    // the four matrices are dead from here: their LDS holds M
    lds_barrier();
    uint16_t* sMqk = sT;
    uint16_t* sMqw = sAkw;
    uint16_t* sMkk = sNqk;
    uint16_t* sMkw = sAqw;
    // the M matrices' blocks above the diagonal stay zero
    for (int idx = tid; idx < 4 * 16 * 32; idx += kNW * 64) {
        const int mtx = idx / 512, bi = (idx / 128) % 4, bj = (idx / 32) % 4, p = idx % 32;
        if (bj > bi) {
            uint16_t* M = mtx == 0 ? sMqk : mtx == 1 ? sMqw : mtx == 2 ? sMkk : sMkw;
            *reinterpret_cast<uint4*>(M + (16 * bi + p / 2) * LDC + 16 * bj + 8 * (p % 2)) =
                make_uint4(0u, 0u, 0u, 0u);
        }
    }
    const float* sLam = G + 3 * kC;
    const float* sB = G + 5 * kC;

    // ---- block pairs: Gram products and their gradients
    for (int p = wave; p < 10; p += kNW) {
        const int tb = pair_t(p), sb = pair_s(p);
        f32x4_t gkk = {0.f, 0.f, 0.f, 0.f}, gkw2 = gkk, aqk = gkk, aqw = gkk;
        f32x4_t dqw = gkk, dqk = gkk, dkk = gkk, dkw2 = gkk;
#pragma unroll
        for (int kp = 0; kp < NKD; ++kp) {
            const bf16x8_t ak = frag_row(sK + tb * 16 * LDD + kp * 32, LDD, lane);
            const bf16x8_t aq = frag_row(sQ + tb * 16 * LDD + kp * 32, LDD, lane);
            const bf16x8_t bk = frag_row(sK + sb * 16 * LDD + kp * 32, LDD, lane);
            const bf16x8_t bw = frag_row(sKW + sb * 16 * LDD + kp * 32, LDD, lane);
            gkk = mma32(ak, bk, gkk);
            gkw2 = mma32(ak, bw, gkw2);
            aqk = mma32(aq, bk, aqk);
            aqw = mma32(aq, bw, aqw);
        }
#pragma unroll
        for (int kp = 0; kp < NKV; ++kp) {
            const bf16x8_t ao = frag_row(sO + tb * 16 * LDV + kp * 32, LDV, lane);
            const bf16x8_t ar = frag_row(sR + tb * 16 * LDV + kp * 32, LDV, lane);
            const bf16x8_t bv = frag_row(sV + sb * 16 * LDV + kp * 32, LDV, lane);
            const bf16x8_t bx = frag_row(sX + sb * 16 * LDV + kp * 32, LDV, lane);
            dqw = mma32(ao, bv, dqw);
            dqk = mma32(ao, bx, dqk);
            dkk = mma32(ar, bx, dkk);
            dkw2 = mma32(ar, bv, dkw2);
        }
        // element (t, s): t = 16 tb + 4 lg + r, s = 16 sb + li
        const int s = sb * 16 + li;
        const float ls = sLam[s];
        float rowsum[4], dbs[4], colsum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tb * 16 + lg * 4 + r;
            const float bt = sB[t];
            const float dec = __builtin_amdgcn_exp2f(fminf(sLam[t] - ls, 0.f));
            const float m0 = s <= t ? dec : 0.f, m1 = s < t ? dec : 0.f;
            const float Aqk = m0 * aqk[r], Aqw = m0 * aqw[r], Gkk = m1 * gkk[r], Gkw = m1 * gkw2[r];
            const float dAqw = s <= t ? dqw[r] : 0.f, dAqk = s <= t ? -dqk[r] : 0.f;
            const float dAkk = s < t ? -dkk[r] : 0.f, dAkw = s < t ? dkw2[r] : 0.f;
            dbs[r] = dAkk * Gkk + dAkw * Gkw;
            const float cc = dAkk * bt * Gkk + dAkw * bt * Gkw + dAqk * Aqk + dAqw * Aqw;
            rowsum[r] = cc;
            colsum += cc;
            sMqk[t * LDC + s] = (uint16_t)(pack_bf16x2(dAqk * m0, 0.f) & 0xffffu);
            sMqw[t * LDC + s] = (uint16_t)(pack_bf16x2(dAqw * m0, 0.f) & 0xffffu);
            sMkk[t * LDC + s] = (uint16_t)(pack_bf16x2(dAkk * bt * m1, 0.f) & 0xffffu);
            sMkw[t * LDC + s] = (uint16_t)(pack_bf16x2(dAkw * bt * m1, 0.f) & 0xffffu);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            rowsum[r] = sum16(rowsum[r]);
            dbs[r] = sum16(dbs[r]);
            if (li == 0) {
                atomicAdd(sL + tb * 16 + lg * 4 + r, rowsum[r]);
                atomicAdd(sDB + tb * 16 + lg * 4 + r, dbs[r]);
            }
        }
        colsum += __shfl_xor(colsum, 16, 64);
        colsum += __shfl_xor(colsum, 32, 64);
        if (lg == 0)
            atomicAdd(sL + s, -colsum);
    }
    lds_barrier();

    // ---- dQ, dK, dKW (key column half), with the dot products of each token row;
    //      the wavefronts of token block 0 also sum S0 . dS1 over their half of the
    //      rows from the same fragments (every element exactly once)
    float kd[4] = {0.f, 0.f, 0.f, 0.f}, qd[4] = {0.f, 0.f, 0.f, 0.f}, fd[4] = {0.f, 0.f, 0.f, 0.f};
    float sd = 0.f;
#pragma unroll
    for (int n = 0; n < HD; ++n) {
        const int col = d0c + n * 16 + li;
        f32x4_t zq = {0.f, 0.f, 0.f, 0.f}, z1 = zq, z2 = zq, z3 = zq;
#pragma unroll
        for (int kp = 0; kp < NKV; ++kp) {
            const bf16x8_t s0r = f0[n & 1][kp];
            const bf16x8_t s1r = f1[n & 1][kp];
            zq = mma32(frag_row(sO + tb * 16 * LDV + kp * 32, LDV, lane), s0r, zq);   // dO S0^T
            z1 = mma32(frag_row(sR + tb * 16 * LDV + kp * 32, LDV, lane), s0r, z1);   // dR S0^T
            z2 = mma32(frag_row(sX + tb * 16 * LDV + kp * 32, LDV, lane), s1r, z2);   // X dS1^T
            z3 = mma32(frag_row(sV + tb * 16 * LDV + kp * 32, LDV, lane), s1r, z3);   // V dS1^T
            if (tb == 0) {
                const uint4 a4 = __builtin_bit_cast(uint4, s0r), b4 = __builtin_bit_cast(uint4, s1r);
                const uint32_t ua[4] = {a4.x, a4.y, a4.z, a4.w}, ub[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    sd += __uint_as_float(ua[x] << 16) * __uint_as_float(ub[x] << 16) +
                          __uint_as_float(ua[x] & 0xffff0000u) * __uint_as_float(ub[x] & 0xffff0000u);
            }
        }
        if (n + 2 < HD)
            load_fin(n + 2, n & 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float kv = bf16_to_f32(sK[(t0 + r) * LDD + col]);
            const float qv = bf16_to_f32(sQ[(t0 + r) * LDD + col]);
            const float wv = bf16_to_f32(sKW[(t0 + r) * LDD + col]);
            kd[r] += kv * z1[r];
            qd[r] += qv * zq[r];
            fd[r] += wv * z3[r] - kv * z2[r];
        }
        // dQ = diag(gamma) dO S0^T + M_qk K + M_qkw KW,
        // dK = diag(b gamma) dR S0^T - diag(fac) X dS1^T + (M_kk + M_kk^T) K + M_kkw KW + M_qk^T Q,
        // dKW = diag(fac) V dS1^T + M_kkw^T K + M_qkw^T Q
        f32x4_t aq, ak, aw;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            aq[r] = gam[r] * zq[r];
            ak[r] = bgm[r] * z1[r] - fac[r] * z2[r];
            aw[r] = fac[r] * z3[r];
        }
        const int nc = d0c + n * 16;
#pragma unroll
        for (int h2 = 0; h2 <= 1; ++h2) {
            const bf16x8_t bK = frag_col(sK + h2 * 32 * LDD + nc, LDD, lane);
            const bf16x8_t bW = frag_col(sKW + h2 * 32 * LDD + nc, LDD, lane);
            const bf16x8_t bQ = frag_col(sQ + h2 * 32 * LDD + nc, LDD, lane);
            if (h2 <= tb / 2) {                // s <= t: rows of M
                aq = mma32(frag_row(sMqk + tb * 16 * LDC + h2 * 32, LDC, lane), bK, aq);
                aq = mma32(frag_row(sMqw + tb * 16 * LDC + h2 * 32, LDC, lane), bW, aq);
                ak = mma32(frag_row(sMkk + tb * 16 * LDC + h2 * 32, LDC, lane), bK, ak);
                ak = mma32(frag_row(sMkw + tb * 16 * LDC + h2 * 32, LDC, lane), bW, ak);
            }
            if (h2 >= tb / 2) {                // s >= t: columns of M (transposes)
                ak = mma32(frag_col(sMkk + h2 * 32 * LDC + tb * 16, LDC, lane), bK, ak);
                ak = mma32(frag_col(sMqk + h2 * 32 * LDC + tb * 16, LDC, lane), bQ, ak);
                aw = mma32(frag_col(sMkw + h2 * 32 * LDC + tb * 16, LDC, lane), bK, aw);
                aw = mma32(frag_col(sMqw + h2 * 32 * LDC + tb * 16, LDC, lane), bQ, aw);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (row_ok(r)) {
                const int64_t o = gidx(r, c.rowQK, D, col);
                gq[o] = from_f32<GT>(aq[r]);
                gk[o] = ak[r];
                gkw[o] = aw[r];
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        kd[r] = sum16(kd[r]);
        qd[r] = sum16(qd[r]);
        fd[r] = sum16(fd[r]);
        if (li == 0) {                           // the two column halves meet in LDS
            atomicAdd(sSc + t0 + r, kd[r]);
            atomicAdd(sSc + kC + t0 + r, qd[r]);
            atomicAdd(sSc + 2 * kC + t0 + r, fd[r]);
        }
    }

    // ---- <S0, dS1>: the two halves from the token-block-0 wavefronts
    if (tb == 0) {
        sd = sum16(sd);
        sd += __shfl_xor(sd, 16, 64);
        sd += __shfl_xor(sd, 32, 64);
        if (lane == 0)
            sRed[nh] = sd;
    }
    lds_barrier();

    // ---- db and dg (wavefront 0, lane = token)
    if (wave == 0) {
        const int t = lane;
        const bool ok = t < c.nt;
        const int64_t o = (int64_t)(c.c0 + t) * H + e;
        const float kS = sSc[t], qS = sSc[kC + t], fdv = sSc[2 * kC + t];
        const float gmt = G[t], bgt = G[kC + t], fct = G[2 * kC + t], gt = G[4 * kC + t];
        if (ok)
            gb[o] = sDB[t] + gmt * kS;
        const float ffd = fct * fdv;
        float l = sL[t] + bgt * kS + gmt * qS - ffd;
        // the chunk's last token: gamma_C carries sum fac dfac and <S0, dS1>
        float tot = ffd;
        for (int x = 1; x < 64; x <<= 1)
            tot += __shfl_xor(tot, x, 64);
        if (t == 63)
            l += tot + G[6 * kC] * (sRed[0] + sRed[1]);
        // d ln g_t = sum of l over t' >= t: a prefix sum over reversed lanes
        const float rev = __shfl(l, 63 - t, 64);
        const float cs = wave_inclusive_sum(rev);
        const float dl = __shfl(cs, 63 - t, 64);
        if (ok)
            gg[o] = dl / gt;
    }
}

}  // namespace bwdc

using bwdc::kC;

template <int D, int DV, typename G>
static void launch_g_TG(const ScanArgs& p, const BwdChunkBufs& w, int64_t blocks, hipStream_t stream)
{
    hipLaunchKernelGGL((bwdc::bwd_grads_kernel<D, DV, G>), dim3((unsigned)blocks), dim3(bwdc::kNW * 64), 0,
                       stream, (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.kw,
                       (const uint16_t*)p.v, (const uint16_t*)w.dO, (const uint16_t*)p.g,
                       (const uint16_t*)p.b, p.cu_seqlens, p.n_seqs, p.heads, (const uint16_t*)w.mats,
                       (const uint16_t*)w.ck, (const uint16_t*)w.ckT, (const uint16_t*)w.dck,
                       (const uint16_t*)w.dckT, static_cast<G*>(w.gq), w.gk, w.gkw, static_cast<G*>(w.gv),
                       w.gg, w.gb);
}

template <int D, int DV>
static hipError_t launch_g_T(const ScanArgs& p, const BwdChunkBufs& w, hipStream_t stream)
{
    const int64_t blocks = (int64_t)(p.total_tokens / kC + p.n_seqs) * p.heads;
    if (blocks == 0)
        return hipSuccess;
    if (w.grad_bf16)
        launch_g_TG<D, DV, uint16_t>(p, w, blocks, stream);
    else
        launch_g_TG<D, DV, float>(p, w, blocks, stream);
    return hipGetLastError();
}

hipError_t launch_bwd_grads(const ScanArgs& p, const BwdChunkBufs& w, hipStream_t stream)
{
    if (!p.bf16)
        return hipErrorInvalidValue;
    if (p.dk == 64)
        return p.dv == 64 ? launch_g_T<64, 64>(p, w, stream) : p.dv == 128 ? launch_g_T<64, 128>(p, w, stream)
                                                                           : hipErrorInvalidValue;
    if (p.dk == 128)
        return p.dv == 64 ? launch_g_T<128, 64>(p, w, stream) : p.dv == 128 ? launch_g_T<128, 128>(p, w, stream)
                                                                            : hipErrorInvalidValue;
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_state(const ScanArgs& p, const void* dO, const void* mats, const float* dS_final,
                            void* dck, void* dckT, float* dS_init, hipStream_t stream)
{
    if (!p.bf16 || !(p.dk == 64 || p.dk == 128) || p.dv % bwdc::kDVS != 0)
        return hipErrorInvalidValue;
    const int n_slices = p.dv / bwdc::kDVS;
    const int64_t blocks = (int64_t)p.n_seqs * p.heads * n_slices;
    if (blocks == 0)
        return hipSuccess;
    auto kern = p.dk == 64 ? bwdc::bwd_state_kernel<64> : bwdc::bwd_state_kernel<128>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, stream, (const uint16_t*)p.q,
                       (const uint16_t*)p.k, (const uint16_t*)dO, (const uint16_t*)p.g,
                       (const uint16_t*)p.b, p.cu_seqlens, p.heads, p.dv, n_slices,
                       (const uint16_t*)mats, dS_final, (uint16_t*)dck, (uint16_t*)dckT, dS_init);
    return hipGetLastError();
}

}  // namespace prism
