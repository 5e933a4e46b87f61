// chunk_scan.hip -- chunkwise WY/UT scan of the gated delta-rule state recurrence
//
//   S_t = g_t (I - b_t k_t k_t^T) S_{t-1} + kw_t v_t^T,     o_t = S_t^T q_t
//
// (PRISM pages: WeChat ICML 2026 summary, section 消除 Token 间串行 -- the
// forget/erase term is the Gated DeltaNet one and the write depends on the
// inputs only; gist.science summary of arXiv 2602.10796, section 2.1 --
// S_t = S_{t-1} A_t + B_t with input-only A_t, B_t, which is what makes a
// chunked evaluation exact.)
//
// Chunk algebra (64 tokens, incoming state S0, in-chunk cumulative log2-gates
// lam_t, gamma_t = 2^lam_t, decay D[t,s] = 2^(lam_t - lam_s) for s <= t):
//   A_kk  = diag(b) (D . tril_-1(K K^T))          A_kkw = diag(b) (D . tril_-1(K KW^T))
//   A_qk  = D . tril_0(Q K^T)                     A_qkw = D . tril_0(Q KW^T)
//   Tm    = (I + A_kk)^-1                          (UT transform)
//   R     = diag(b gamma) K S0 + A_kkw V
//   X     = Tm R                                   rows x_t = g_t b_t S_{t-1}^T k_t
//   O     = diag(gamma) Q S0 + A_qkw V - A_qk X
//   S_out = gamma_C S0 + KW^T diag(gamma_C/gamma) V - K^T diag(gamma_C/gamma) X
// The masks are applied before the exponentials, so every factor used is
// <= 1 and strong decay cannot overflow.
//
// Mapping to gfx950:
//   * one workgroup (4 wavefronts) per (sequence, head, value slice): the value
//     columns of S are independent, so a chain's dv columns are split over
//     several workgroups when chains are too few to occupy the 256 CUs;
//   * the state slice (dk x dv_slice) lives in MFMA accumulators in fp32 for the
//     whole sequence and is rounded to the operand type only as an operand;
//   * every contraction is a 16x16 MFMA tile product (bf16: 16x16x32, fp32:
//     16x16x4) on tiles staged row-major in LDS.  Operands whose contraction
//     index is the tile's row index (token-contracted products K^T X, KW^T V
//     and A V) are fetched with the LDS transpose read ds_read_b64_tr_b16, so
//     no tile is ever stored twice;
//   * the next chunk's q, k, kw, v, g, b are loaded into registers while the
//     current chunk computes (software pipelining of the HBM latency);
//   * Gram tiles: each wavefront builds all four masked 16x16 blocks of its
//     (t-block, s-block) pairs, so one operand fetch feeds two MFMAs;
//   * the 64x64 unit-lower-triangular inverse: wavefront 0 inverts the four
//     16x16 diagonal blocks by substitution in fp32 while the other three
//     compute the S0-dependent parts of R and O; the off-diagonal blocks follow
//     by distance with 16x16x16 MFMAs whose intermediate stays in registers
//     (bf16 operands, fp32 accumulation; fp32 MFMA on the fp32 path);
//   * varlen: chunks restart at every cu_seqlens entry; a ragged last chunk is
//     zero-padded (k = kw = q = v = 0, g = 1, b = 0), which leaves S unchanged.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace prism {

constexpr int kC = 64;          // chunk length
constexpr int kThreads = 256;   // 4 wavefronts
constexpr int kPLd = 17;        // row stride of the fp32 level scratch

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef short v8s_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

// Transposed 16-bit LDS read (gfx950): within each group of 16 lanes, lane i
// receives element (i % 4) of the 8-byte chunk addressed by lane 4 e + i / 4,
// for e = 0..3.
__device__ __forceinline__ v4s_t lds_read_tr(const uint16_t* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(const_cast<uint16_t*>(p)));
}

// MFMA operand fetch.  A fragment covers a 16 x KB block (row m, contraction k).
//   row(p, ld): element (m, k) at p[m * ld + k]   (k contiguous)
//   col(p, ld): element (m, k) at p[k * ld + m]   (m contiguous)
template <typename Op> struct Mfma;
template <> struct Mfma<uint16_t> {              // bf16: v_mfma_f32_16x16x32_bf16
    static constexpr int KB = 32;
    using Frag = bf16x8_t;
    __device__ static Frag row(const uint16_t* p, int ld, int lane)
    {
        return __builtin_bit_cast(
            Frag, *reinterpret_cast<const uint4*>(p + (lane & 15) * ld + (lane >> 4) * 8));
    }
    __device__ static Frag col(const uint16_t* p, int ld, int lane)
    {
        const int i = lane & 15;
        const uint16_t* a = p + ((lane >> 4) * 8 + (i >> 2)) * ld + (i & 3) * 4;
        v4s_t lo = lds_read_tr(a);
        v4s_t hi = lds_read_tr(a + 4 * ld);
        v8s_t x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(Frag, x);
    }
    __device__ static f32x4_t mma(Frag a, Frag b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {                 // fp32: v_mfma_f32_16x16x4_f32
    static constexpr int KB = 4;
    using Frag = float;
    __device__ static Frag row(const float* p, int ld, int lane)
    {
        return p[(lane & 15) * ld + (lane >> 4)];
    }
    __device__ static Frag col(const float* p, int ld, int lane)
    {
        return p[(lane >> 4) * ld + (lane & 15)];
    }
    __device__ static f32x4_t mma(float a, float b, f32x4_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ f32x4_t mma_f32(float a, float b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc += A B over `steps` contraction blocks of KB.  Suffix letters give the
// fetch form of A then B (B is fetched as the 16 x K block B^T, i.e. its
// fragment row index is n).
template <typename Op>
__device__ __forceinline__ f32x4_t mm_rr(f32x4_t acc, const Op* a, int lda, const Op* b, int ldb,
                                         int steps, int lane)
{
    using M = Mfma<Op>;
    for (int s = 0; s < steps; ++s)
        acc = M::mma(M::row(a + s * M::KB, lda, lane), M::row(b + s * M::KB, ldb, lane), acc);
    return acc;
}
template <typename Op>
__device__ __forceinline__ f32x4_t mm_rc(f32x4_t acc, const Op* a, int lda, const Op* b, int ldb,
                                         int steps, int lane)
{
    using M = Mfma<Op>;
    for (int s = 0; s < steps; ++s)
        acc = M::mma(M::row(a + s * M::KB, lda, lane), M::col(b + s * M::KB * ldb, ldb, lane), acc);
    return acc;
}
template <typename Op>
__device__ __forceinline__ f32x4_t mm_cc(f32x4_t acc, const Op* a, int lda, const Op* b, int ldb,
                                         int steps, int lane)
{
    using M = Mfma<Op>;
    for (int s = 0; s < steps; ++s)
        acc = M::mma(M::col(a + s * M::KB * lda, lda, lane), M::col(b + s * M::KB * ldb, ldb, lane),
                     acc);
    return acc;
}
template <typename Op>
__device__ __forceinline__ f32x4_t mm_cr(f32x4_t acc, const Op* a, int lda, const Op* b, int ldb,
                                         int steps, int lane)
{
    using M = Mfma<Op>;
    for (int s = 0; s < steps; ++s)
        acc = M::mma(M::col(a + s * M::KB * lda, lda, lane), M::row(b + s * M::KB, ldb, lane), acc);
    return acc;
}

// Four consecutive fp32 values -> operand type at p (8-byte store for bf16).
__device__ __forceinline__ void st4(uint16_t* p, f32x4_t x)
{
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
}
__device__ __forceinline__ void st4(float* p, f32x4_t x)
{
    p[0] = x[0]; p[1] = x[1]; p[2] = x[2]; p[3] = x[3];
}

__device__ __forceinline__ v4s_t pack_bf16x4(f32x4_t x)
{
    return __builtin_bit_cast(v4s_t, make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])));
}

// 16 bytes of staged input (8 bf16 or 4 fp32) -> LDS row segment.
__device__ __forceinline__ void put16(uint16_t* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ void put16(float* p, uint4 v)
{
    p[0] = __uint_as_float(v.x); p[1] = __uint_as_float(v.y);
    p[2] = __uint_as_float(v.z); p[3] = __uint_as_float(v.w);
}
// Same, scaled by f.
__device__ __forceinline__ void put16_scaled(uint16_t* p, uint4 v, float f)
{
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        w[i] = pack_bf16x2(__uint_as_float(w[i] << 16) * f, __uint_as_float(w[i] & 0xffff0000u) * f);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void put16_scaled(float* p, uint4 v, float f)
{
    p[0] = __uint_as_float(v.x) * f; p[1] = __uint_as_float(v.y) * f;
    p[2] = __uint_as_float(v.z) * f; p[3] = __uint_as_float(v.w) * f;
}

// LDS carve-up (byte offsets).  bf16 tiles use rows padded by 16 bytes
// (16-byte aligned rows for vector and transpose reads); fp32 tiles use an
// odd row stride (scalar fragment reads, conflict-free).
template <typename Op, int D, int DVS>
struct Layout {
    static constexpr bool kBf = sizeof(Op) == 2;
    static constexpr int E = (int)sizeof(Op);
    static constexpr int PAD = kBf ? 8 : 1;
    static constexpr int LDD = D + PAD;          // [64][D] tiles, S0^T [DVS][D]
    static constexpr int LDC = kC + PAD;         // [64][64] matrices, [DVS][64] transposed tiles
    static constexpr int LDV = DVS + PAD;        // [64][DVS] value tiles
    static constexpr int szRowD = kC * LDD * E;
    static constexpr int szV = kC * LDV * E;
    static constexpr int szM = kC * LDC * E;
    static constexpr int szS0t = DVS * LDD * E;
    static constexpr int szJt = DVS * LDC * E;
    static constexpr int szP = kBf ? 0 : 3 * 16 * kPLd * 4;
    static constexpr int szG = 4 * kC * 4;

    static constexpr int oQ = 0;
    static constexpr int oK = oQ + szRowD;
    static constexpr int oKW = oK + szRowD;
    static constexpr int oV = oKW + szRowD;
    static constexpr int oVs = oV + szV;
    static constexpr int oAkk = oVs + szV;       // five 64x64 matrices, contiguous
    static constexpr int oAkkw = oAkk + szM;
    static constexpr int oAqkw = oAkkw + szM;
    static constexpr int oAqk = oAqkw + szM;
    static constexpr int oT = oAqk + szM;
    static constexpr int oS0t = oT + szM;
    static constexpr int oRt = oS0t + szS0t;
    static constexpr int oXt = oRt + szJt;
    static constexpr int oXst = oXt + szJt;
    static constexpr int oP = oXst + szJt;
    static constexpr int oG = oP + szP;
    static constexpr int total = oG + szG;
    static_assert(oAkk % 16 == 0 && oS0t % 16 == 0 && oRt % 16 == 0 && oP % 16 == 0,
                  "LDS alignment");
};

// Unordered (t-block, s-block) pairs of the lower-triangular 16x16 tiling of a
// 64x64 matrix, dealt round-robin to the 4 wavefronts (at most 3 each).
__constant__ const int kPairT[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ const int kPairS[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

template <typename T, int D, int DVS>
__global__ __launch_bounds__(kThreads) void chunk_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ kw,
    const T* __restrict__ v, const T* __restrict__ g, const T* __restrict__ b,
    const int32_t* __restrict__ cu, int H, int DV, int n_slices,
    const float* __restrict__ s_init, T* __restrict__ o, float* __restrict__ s_final)
{
    using Ly = Layout<T, D, DVS>;
    using M = Mfma<T>;
    constexpr bool kBf = Ly::kBf;
    constexpr int LDD = Ly::LDD, LDC = Ly::LDC, LDV = Ly::LDV;
    constexpr int KB = M::KB;
    constexpr int NJ = DVS / 16;                 // 16-column tiles of the value slice
    constexpr int NS = (D / 16) * NJ;            // state tiles
    constexpr int NSW = NS / 4;                  // state tiles per wavefront
    constexpr int NRT = 4 * NJ;                  // tiles of R, X and O
    constexpr int NOW = (NRT + 2) / 3;           // O tiles per wavefront 1..3
    constexpr int VE = 16 / (int)sizeof(T);      // elements per 16-byte vector
    constexpr int NQ = kC * D / VE / kThreads;   // q / k / kw vectors per thread
    constexpr int NVV = kC * DVS / VE;           // v vectors per chunk
    constexpr int NVT = (NVV + kThreads - 1) / kThreads;
    static_assert(NS % 4 == 0, "state tiles must split over 4 wavefronts");
    static_assert(kC * D / VE % kThreads == 0, "staging split");
    static_assert(Ly::total <= 160 * 1024, "LDS budget");

    __shared__ __attribute__((aligned(16))) unsigned char smem[Ly::total];
    T* sQ = reinterpret_cast<T*>(smem + Ly::oQ);
    T* sK = reinterpret_cast<T*>(smem + Ly::oK);
    T* sKW = reinterpret_cast<T*>(smem + Ly::oKW);
    T* sV = reinterpret_cast<T*>(smem + Ly::oV);         // V slice [t][j]
    T* sVs = reinterpret_cast<T*>(smem + Ly::oVs);       // diag(gamma_C/gamma) V [t][j]
    T* sAkk = reinterpret_cast<T*>(smem + Ly::oAkk);     // [t][s]
    T* sAkkw = reinterpret_cast<T*>(smem + Ly::oAkkw);
    T* sAqkw = reinterpret_cast<T*>(smem + Ly::oAqkw);
    T* sAqk = reinterpret_cast<T*>(smem + Ly::oAqk);     // holds -A_qk
    T* sT = reinterpret_cast<T*>(smem + Ly::oT);         // Tm [t][s]
    T* sS0t = reinterpret_cast<T*>(smem + Ly::oS0t);     // S0^T [j][i]
    T* sRt = reinterpret_cast<T*>(smem + Ly::oRt);       // R^T [j][t]
    T* sXt = reinterpret_cast<T*>(smem + Ly::oXt);       // X^T [j][t]
    T* sXst = reinterpret_cast<T*>(smem + Ly::oXst);     // -(diag(gamma_C/gamma) X)^T [j][t]
    float* sP = reinterpret_cast<float*>(smem + Ly::oP);
    float* sLam = reinterpret_cast<float*>(smem + Ly::oG);
    float* sBv = sLam + kC;
    float* sGam = sBv + kC;
    float* sFac = sGam + kC;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int slice = (int)(blockIdx.x % (unsigned)n_slices);
    const int chain = (int)(blockIdx.x / (unsigned)n_slices);
    const int n = chain / H, e = chain % H;
    const int j0 = slice * DVS;
    const int seq0 = cu[n], seq1 = cu[n + 1];
    const int nchunks = (seq1 - seq0 + kC - 1) / kC;
    const int64_t rowQK = (int64_t)H * D, rowV = (int64_t)H * DV;

    // zero the 64x64 matrices (their upper blocks are never written) and S0^T
    {
        constexpr int nz = (5 * Ly::szM + Ly::szS0t) / 16;
        uint4* z = reinterpret_cast<uint4*>(smem + Ly::oAkk);
        for (int i = tid; i < nz; i += kThreads)
            z[i] = make_uint4(0u, 0u, 0u, 0u);
    }

    // state tile qd of this wavefront: rows ib * 16 + (lane >> 4) * 4 + r, column
    // jb * 16 + (lane & 15) of the slice; start state from s_init (or zero), also
    // kept transposed in LDS as the b-step operand S0^T
    f32x4_t S[NSW];
#pragma unroll
    for (int qd = 0; qd < NSW; ++qd) {
        S[qd] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (s_init) {
            const int sidx = wave * NSW + qd, ib = sidx / NJ, jb = sidx % NJ;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = ib * 16 + (lane >> 4) * 4 + r;
                S[qd][r] = s_init[(((int64_t)n * H + e) * D + i) * DV + j0 + jb * 16 + (lane & 15)];
            }
        }
    }
    if (s_init) {
        __syncthreads();                         // after the zeroing of S0^T above
#pragma unroll
        for (int qd = 0; qd < NSW; ++qd) {
            const int sidx = wave * NSW + qd, ib = sidx / NJ, jb = sidx % NJ;
            st4(sS0t + (jb * 16 + (lane & 15)) * LDD + ib * 16 + (lane >> 4) * 4, S[qd]);
        }
    }

    // ---- register prefetch of one chunk ----
    // Per-thread element offsets inside a chunk do not change from chunk to
    // chunk: they are computed once, and each chunk only adds a scalar base.
    int offq[NQ], tq[NQ], offv[NVT], tv[NVT];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int idx = tid + j * kThreads;
        tq[j] = idx / (D / VE);
        offq[j] = tq[j] * H * D + e * D + (idx % (D / VE)) * VE;
    }
#pragma unroll
    for (int j = 0; j < NVT; ++j) {
        const int idx = tid + j * kThreads;
        tv[j] = idx < NVV ? idx / (DVS / VE) : kC;
        offv[j] = (idx / (DVS / VE)) * H * DV + e * DV + j0 + (idx % (DVS / VE)) * VE;
    }
    uint4 pq[NQ], pk[NQ], pw[NQ], pv[NVT];
    const T one = from_f32<T>(1.f), zero = from_f32<T>(0.f);
    T pg = one, pb = zero;
    auto prefetch = [&](int ch) {
        const int c0 = seq0 + ch * kC;
        const int nt = min(kC, seq1 - c0);
        const T* bq = q + (int64_t)c0 * rowQK;
        const T* bk = k + (int64_t)c0 * rowQK;
        const T* bw = kw + (int64_t)c0 * rowQK;
        const T* bv = v + (int64_t)c0 * rowV;
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
        // raw values: converting here would make the compiler wait for every
        // load of this prefetch right away
        pg = one;
        pb = zero;
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

        // ======== phase 1: gates (every wavefront, lane = token) and staging ========
        const float bv_lane = to_f32(pb);
        float lam = __log2f(fmaxf(to_f32(pg), 1e-30f));
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            float y = __shfl_up(lam, d, 64);
            if (lane >= d)
                lam += y;
        }
        const float lamC = __shfl(lam, 63, 64);
        const float fac = exp2f(lamC - lam);            // gamma_C / gamma_t <= 1
        if (wave == 0) {
            sLam[lane] = lam;
            sBv[lane] = bv_lane;
            sGam[lane] = exp2f(lam);
            sFac[lane] = fac;
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int idx = tid + j * kThreads;
            const int t = idx / (D / VE), c = (idx % (D / VE)) * VE;
            put16(sQ + t * LDD + c, pq[j]);
            put16(sK + t * LDD + c, pk[j]);
            put16(sKW + t * LDD + c, pw[j]);
        }
#pragma unroll
        for (int j = 0; j < NVT; ++j) {
            const int idx = tid + j * kThreads;
            const int t = idx / (DVS / VE), c = (idx % (DVS / VE)) * VE;
            const float ft = __shfl(fac, t & 63, 64);
            if (idx < NVV) {
                put16(sV + t * LDV + c, pv[j]);
                put16_scaled(sVs + t * LDV + c, pv[j], ft);
            }
        }
        if (ch + 1 < nchunks)
            prefetch(ch + 1);
        __syncthreads();

        // ======== phase 2: masked Gram blocks; S <- gamma_C S + KW^T diag(fac) V ========
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int p = wave + 4 * u;
            if (p >= 10)
                break;
            const int tb = kPairT[p], sb = kPairS[p];
            f32x4_t gkk = {0.f, 0.f, 0.f, 0.f}, gkw = gkk, gqk = gkk, gqw = gkk;
            const T* yk = sK + sb * 16 * LDD;
            const T* yw = sKW + sb * 16 * LDD;
            const T* xk = sK + tb * 16 * LDD;
            const T* xq = sQ + tb * 16 * LDD;
#pragma unroll
            for (int kk = 0; kk < D; kk += KB) {
                auto ak = M::row(yk + kk, LDD, lane);
                auto aw = M::row(yw + kk, LDD, lane);
                auto bk = M::row(xk + kk, LDD, lane);
                auto bq = M::row(xq + kk, LDD, lane);
                gkk = M::mma(ak, bk, gkk);     // (K K^T)^T block: element (s, t)
                gkw = M::mma(aw, bk, gkw);     // (K KW^T)^T
                gqk = M::mma(ak, bq, gqk);     // (Q K^T)^T
                gqw = M::mma(aw, bq, gqw);     // (Q KW^T)^T
            }
            const int t = tb * 16 + (lane & 15);
            const int s0 = sb * 16 + (lane >> 4) * 4;
            const float lt = sLam[t], bt = sBv[t];
            const float4 ls = *reinterpret_cast<const float4*>(sLam + s0);
            const float lsv[4] = {ls.x, ls.y, ls.z, ls.w};
            f32x4_t vkk, vkw, vqk, vqw;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = s0 + r;
                // lam is non-increasing in t, so lt - ls <= 0 wherever s <= t
                const float dec = __builtin_amdgcn_exp2f(fminf(lt - lsv[r], 0.f));
                const float mi = s <= t ? dec : 0.f;     // inclusive mask
                const float ms = s < t ? dec * bt : 0.f; // strict mask, times b_t
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
            const float gC = exp2f(lamC);
#pragma unroll
            for (int qd = 0; qd < NSW; ++qd) {
                const int sidx = wave * NSW + qd, ib = sidx / NJ, jb = sidx % NJ;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[qd][r] *= gC;
                S[qd] = mm_cc<T>(S[qd], sKW + ib * 16, LDD, sVs + jb * 16, LDV, kC / KB, lane);
            }
        }
        __syncthreads();

        // ======== phase 3: diagonal blocks of Tm (wave 0) | R and O partials (waves 1-3) ========
        f32x4_t oacc[NOW];
        if (wave == 0) {
            const int bi = lane >> 4, j = lane & 15;
            const T* A = sAkk + (bi * 16) * LDC + bi * 16;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
                for (int c = 0; c < r; ++c)
                    acc -= to_f32(A[r * LDC + c]) * x[c];
                x[r] = acc;
            }
            T* Td = sT + (bi * 16) * LDC + bi * 16 + j;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                Td[r * LDC] = from_f32<T>(x[r]);
        } else {
#pragma unroll
            for (int u = 0; u < NOW; ++u) {
                const int qt = (wave - 1) + 3 * u;
                if (qt < NRT) {
                    const int tb = qt / NJ, jb = qt % NJ;
                    const int steps = (16 * (tb + 1) + KB - 1) / KB;
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                    acc = mm_rr<T>(acc, sK + tb * 16 * LDD, LDD, sS0t + jb * 16 * LDD, LDD, D / KB,
                                   lane);
                    f32x4_t oa = {0.f, 0.f, 0.f, 0.f};
                    oa = mm_rr<T>(oa, sQ + tb * 16 * LDD, LDD, sS0t + jb * 16 * LDD, LDD, D / KB,
                                  lane);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = tb * 16 + (lane >> 4) * 4 + r;
                        acc[r] *= sBv[t] * sGam[t];
                        oa[r] *= sGam[t];
                    }
                    acc = mm_rc<T>(acc, sAkkw + tb * 16 * LDC, LDC, sV + jb * 16, LDV, steps, lane);
                    st4(sRt + (jb * 16 + (lane & 15)) * LDC + tb * 16 + (lane >> 4) * 4, acc);
                    oacc[u] = mm_rc<T>(oa, sAqkw + tb * 16 * LDC, LDC, sV + jb * 16, LDV, steps,
                                       lane);
                }
            }
        }
        __syncthreads();

        // ======== phase 4: off-diagonal blocks of Tm, by distance ========
        //   Tm_{bi,bj} = -Tm_{bi,bi} sum_{m=bj}^{bi-1} A_kk{bi,m} Tm_{m,bj}
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            const int bi = wave + d, bj = wave;
            const bool active = wave < 4 - d;
            if constexpr (kBf) {
                if (active) {
                    f32x4_t p = {0.f, 0.f, 0.f, 0.f};
                    const int i = lane & 15, gq = lane >> 4;
                    for (int m = bj; m < bi; ++m) {
                        v4s_t a = *reinterpret_cast<const v4s_t*>(sAkk + (bi * 16 + i) * LDC +
                                                                  m * 16 + gq * 4);
                        v4s_t bt = lds_read_tr(sT + (m * 16 + gq * 4 + (i >> 2)) * LDC + bj * 16 +
                                               (i & 3) * 4);
                        p = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bt, p, 0, 0, 0);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        p[r] = -p[r];
                    v4s_t a = *reinterpret_cast<const v4s_t*>(sT + (bi * 16 + i) * LDC + bi * 16 +
                                                              gq * 4);
                    f32x4_t tij = {0.f, 0.f, 0.f, 0.f};
                    tij = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pack_bf16x4(p), tij, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sT[(bi * 16 + gq * 4 + r) * LDC + bj * 16 + i] = f32_to_bf16(tij[r]);
                }
                __syncthreads();
            } else {
                float* Pw = sP + wave * 16 * kPLd;
                if (active) {
                    f32x4_t p = {0.f, 0.f, 0.f, 0.f};
                    for (int kk = 0; kk < 16 * d; kk += 4) {
                        const int kc = bj * 16 + kk + (lane >> 4);
                        p = mma_f32(sAkk[(bi * 16 + (lane & 15)) * LDC + kc],
                                    sT[kc * LDC + bj * 16 + (lane & 15)], p);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        Pw[((lane >> 4) * 4 + r) * kPLd + (lane & 15)] = p[r];
                }
                __syncthreads();
                if (active) {
                    f32x4_t ta = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 16; kk += 4) {
                        const int kc = kk + (lane >> 4);
                        ta = mma_f32(sT[(bi * 16 + (lane & 15)) * LDC + bi * 16 + kc],
                                     Pw[kc * kPLd + (lane & 15)], ta);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sT[(bi * 16 + (lane >> 4) * 4 + r) * LDC + bj * 16 + (lane & 15)] = -ta[r];
                }
                __syncthreads();
            }
        }

        // ======== phase 5: X = Tm R ========
        for (int qt = wave; qt < NRT; qt += 4) {
            const int tb = qt / NJ, jb = qt % NJ;
            const int steps = (16 * (tb + 1) + KB - 1) / KB;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            acc = mm_rr<T>(acc, sT + tb * 16 * LDC, LDC, sRt + jb * 16 * LDC, LDC, steps, lane);
            f32x4_t xs;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                xs[r] = -acc[r] * sFac[tb * 16 + (lane >> 4) * 4 + r];
            const int off = (jb * 16 + (lane & 15)) * LDC + tb * 16 + (lane >> 4) * 4;
            st4(sXt + off, acc);
            st4(sXst + off, xs);
        }
        __syncthreads();

        // ======== phase 6: O = O' - A_qk X (waves 1-3); S <- S - K^T diag(fac) X ========
        if (wave > 0) {
#pragma unroll
            for (int u = 0; u < NOW; ++u) {
                const int qt = (wave - 1) + 3 * u;
                if (qt < NRT) {
                    const int tb = qt / NJ, jb = qt % NJ;
                    const int steps = (16 * (tb + 1) + KB - 1) / KB;
                    f32x4_t acc = mm_rr<T>(oacc[u], sAqk + tb * 16 * LDC, LDC, sXt + jb * 16 * LDC,
                                           LDC, steps, lane);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = tb * 16 + (lane >> 4) * 4 + r;
                        if (t < nt)
                            o[(int64_t)(c0 + t) * rowV + (int64_t)e * DV + j0 + jb * 16 +
                              (lane & 15)] = from_f32<T>(acc[r]);
                    }
                }
            }
        }
#pragma unroll
        for (int qd = 0; qd < NSW; ++qd) {
            const int sidx = wave * NSW + qd, ib = sidx / NJ, jb = sidx % NJ;
            S[qd] = mm_cr<T>(S[qd], sK + ib * 16, LDD, sXst + jb * 16 * LDC, LDC, kC / KB, lane);
            st4(sS0t + (jb * 16 + (lane & 15)) * LDD + ib * 16 + (lane >> 4) * 4, S[qd]);
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
                       p.s_init, (T*)p.o, p.s_final);
    return hipGetLastError();
}

bool scan_supported(bool bf16, int dk, int dv, int dvs)
{
    if (dv % dvs != 0 || (dv != 64 && dv != 128))
        return false;
    if (bf16)
        return (dk == 64 || dk == 128) && (dvs == 16 || dvs == 32 || dvs == 64);
    return dk == 64 && dvs == 16;
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
        if (p.dv_slice == 32) return launch<uint16_t, 128, 32>(p, s);
        return launch<uint16_t, 128, 64>(p, s);
    }
    return launch<float, 64, 16>(p, s);
}

}  // namespace prism
