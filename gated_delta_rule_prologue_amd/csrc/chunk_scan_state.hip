// chunk_scan_state.hip -- the sequential part of the bf16 chunk scan, in WY
// form, from per-chunk matrices formed beforehand
//
// Gated delta-rule recurrence S_t = g_t (I - b_t k_t k_t^T) S_{t-1} + kw_t v_t^T,
// o_t = S_t^T q_t (PRISM pages: WeChat ICML 2026 summary, section
// 消除 Token 间串行; gist.science summary of arXiv 2602.10796, section 2.1:
// A_t and B_t depend on the inputs only, so any chunking is exact), in chunks
// of 64 tokens.  With S0 the state entering a chunk, gamma the in-chunk
// cumulative decay, fac = gamma_C / gamma and T = (I + A_kk)^-1, A_kkw, A_qkw,
// A_qk the chunk's matrices (chunk_gram.hip), the chunk is
//
//   X = T (diag(b gamma) K S0 + A_kkw V)       (rows x_t = g_t b_t S_{t-1}^T k_t)
//   O = diag(gamma) Q S0 + A_qkw V - A_qk X
//   S = gamma_C S0 + KW^T diag(fac) V - K^T diag(fac) X
//
// and, splitting off everything that does not involve S0,
//
//   W  = T diag(b gamma) K,            U     = T A_kkw V
//   Q' = diag(gamma) Q - A_qk W,       O_loc = A_qkw V - A_qk U
//   X  = W S0 + U,   O = Q' S0 + O_loc,   S = gamma_C S0 + KW^T diag(fac) V - K^T diag(fac) X.
//
// Only the last line depends on the previous chunk: one product of S0 feeds
// the state update directly, and O hangs off S0 beside it.
//
// One workgroup per (sequence, head, 32 value columns), four wavefronts, one
// per SIMD.  Wavefronts 0 and 1 (state) hold 16 value columns of S each in
// fp32 MFMA accumulators and run the last line for every chunk in turn.
// Wavefronts 2 and 3 (helpers) prepare chunk c + 1 while the state wavefronts
// run chunk c: each stores half of the chunk's k and kw rows (its half of the
// channels) and half of the value slice into an LDS buffer, forms its channel
// half of W and Q' (as transposed tiles, written as rows) and its 16 columns
// of U and O_loc (in the state wavefronts' accumulator layout), and issues the
// loads of chunk c + 2.  Neither helper reads what the other wrote, so they
// need no synchronisation of their own; one barrier per chunk hands a buffer
// over.  All products are bf16 16x16x32 MFMA with fp32 accumulation.
#include "common.h"
#include "gram.h"
#include "kernels.h"
#include "mfma_bf16.h"

namespace prism {
namespace stscan {

using namespace mfma;
using gram::kC;

constexpr int kWaves = 4;
constexpr int kDVS = 32;                         // value columns per workgroup
constexpr int kXcds = 8;
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// One LDS buffer per chunk parity (double-buffered), then the helpers' gates.
template <int D>
struct Lay {
    static constexpr int LDD = D + 8;            // k, kw rows (read transposed)
    static constexpr int LDV = kDVS + 8;         // rows of the value slice
    static constexpr int szRow = kC * LDD * 2;
    static constexpr int szV = kC * LDV * 2;
    static constexpr int szWY = kC * D * 2;      // W, Q' rows (16-byte pieces swizzled)
    static constexpr int szLane = 2 * 4 * 64 * 8;    // U, O_loc: [wavefront][token block][lane] x 4 bf16
    static constexpr int oK = 0, oKW = szRow, oV = 2 * szRow;
    static constexpr int oW = oV + szV, oQp = oW + szWY;
    static constexpr int oU = oQp + szWY, oO = oU + szLane;
    static constexpr int oFac = oO + szLane;     // gamma_C / gamma (64), then gamma_C
    static constexpr int szBuf = oFac + kC * 4 + 16;
    static constexpr int oScr = 2 * szBuf;       // per helper: b gamma (64), gamma (64)
    static constexpr int total = oScr + 2 * 2 * kC * 4;
    static_assert(szRow % 16 == 0 && szV % 16 == 0 && oW % 16 == 0 && oU % 16 == 0 &&
                      szBuf % 16 == 0,
                  "alignment");
    static_assert(total <= 160 * 1024, "LDS budget");
};

// Element (t, ch) of a W or Q' row block: the 16-byte pieces of row t are
// permuted by t, so that the sixteen rows of a fragment read (one piece of
// each) fall in distinct banks.
template <int D>
__device__ __forceinline__ int wy_off(int t, int ch)
{
    return t * D + ((((ch >> 3) ^ t) & (D / 8 - 1)) << 3) + (ch & 7);
}

// 16x16x32 A fragment of the transpose of a swizzled row block: element (m, k)
// = rows r0 + k, column ch0 + m (two transposed LDS reads, as frag_col).
template <int D>
__device__ __forceinline__ bf16x8_t wy_col(const uint16_t* p, int r0, int ch0, int lane)
{
    const int i = lane & 15;
    const int r = r0 + (lane >> 4) * 8 + (i >> 2), ch = ch0 + (i & 3) * 4;
    const v8s_t x = __builtin_shufflevector(lds_read_tr(p + wy_off<D>(r, ch)),
                                            lds_read_tr(p + wy_off<D>(r + 4, ch)), 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, x);
}

__device__ __forceinline__ f32x4_t unpack4(u32x2_t w)
{
    return f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                   __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
}
__device__ __forceinline__ u32x2_t pack4(f32x4_t x)
{
    return u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
}

// Workgroups are dispatched to the eight XCDs round-robin (workgroup w on XCD
// w % 8), each with its own L2: when the chains split evenly over the XCDs,
// all slices of a chain go to one XCD, so its rows and matrices come from HBM
// once and from that L2 for the other slices.
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

// 16x16x32 fragment (rows of block-row i, the 32 columns of blocks 2h, 2h + 1)
// of one of the chunk's stored lower-triangular matrices, through a bounded
// buffer rs over the chunk's matrices.  A block above the diagonal is read
// past the end of the buffer, which returns zeros: no arithmetic touches the
// loaded value, so the load can stay in flight until the fragment is used.
__device__ __forceinline__ bf16x8_t mat32(__amdgpu_buffer_rsrc_t rs, int mat, int i, int h, int lane)
{
    const int li = lane & 15, lg = lane >> 4;
    const int j = 2 * h + (lg >> 1);
    const int jj = min(j, i);
    const int past = (j > i) * (gram::kChunkElems * 2);   // arithmetic, not a select: no branch
    const int off = (mat * gram::kMatElems + gram::blk_index(i, jj) * gram::kBlockElems +
                     gram::swz(li, 8 * (lg & 1))) * 2 + past;
    return __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

// The (16-token block, 32-token half) pairs of a lower-triangular product:
// pair index pidx(tb, h2) for h2 <= tb / 2.
constexpr int kPairs = 6;
__device__ __forceinline__ constexpr int pidx(int tb, int h2) { return (tb < 2 ? tb : 2 * tb - 2) + h2; }
__device__ __forceinline__ constexpr int pair_tb(int p) { return p < 2 ? p : (p + 2) / 2; }
__device__ __forceinline__ constexpr int pair_h2(int p) { return p < 2 ? 0 : p % 2; }

struct Ctx {
    const uint16_t *q, *k, *kw, *v, *g, *b, *mats;
    uint16_t* o;
    int n, e, H, DV, j0, seq0, seq1, nchunks, lane;
    int64_t rowQK, rowV, vbase;                  // vbase: first matrix chunk of the chain
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint16_t* p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p), 0, bytes, 0x00020000);
}

// Tokens of chunk ch that exist (0 past the chain's end; readfirstlane: med3
// has no scalar form, and a range the compiler cannot prove uniform turns
// every load into a waterfall loop).
__device__ __forceinline__ int chunk_tokens(const Ctx& c, int ch)
{
    return __builtin_amdgcn_readfirstlane(max(0, min(kC, c.seq1 - (c.seq0 + ch * kC))));
}

// ---- What a helper loads ahead of preparing a chunk: the rows (issued as
// soon as the previous chunk's rows are stored) and the matrix fragments and q
// tiles (each group issued right after its last use for the previous chunk).
// Every load is a bounded buffer load; past the chain's last chunk the ranges
// are empty (all zeros), so no branch guards them.
template <int D>
struct Rows {
    static constexpr int HALF = D / 2;           // channels of this helper
    static constexpr int NPK = D / 16;           // 16-byte pieces per lane of a half row block
    uint4 rk[NPK], rw[NPK], rv[2];
    uint16_t gv, bv;

    __device__ void load(const Ctx& c, int ch, int h)
    {
        const int lane = c.lane;
        const int c0 = c.seq0 + ch * kC;
        const int nt = chunk_tokens(c, ch);
        const int64_t base = (int64_t)c0 * c.rowQK + (int64_t)c.e * D + h * HALF;
        const int nqk = nt * (int)c.rowQK * 2;
        const auto sk = rsrc(c.k + base, nqk), sw = rsrc(c.kw + base, nqk);
        constexpr int PPR = HALF / 8;
#pragma unroll
        for (int x = 0; x < NPK; ++x) {
            const int p = lane + 64 * x;
            const int off = ((p / PPR) * (int)c.rowQK + (p % PPR) * 8) * 2;
            rk[x] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(sk, off, 0, 0));
            rw[x] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(sw, off, 0, 0));
        }
        const auto sv = rsrc(c.v + (int64_t)c0 * c.rowV + (int64_t)c.e * c.DV + c.j0 + 16 * h,
                             nt * (int)c.rowV * 2);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int p = lane + 64 * x;
            rv[x] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  sv, ((p / 2) * (int)c.rowV + (p % 2) * 8) * 2, 0, 0));
        }
        const auto sg = rsrc(c.g + (int64_t)c0 * c.H + c.e, nt * c.H * 2);
        const auto sb = rsrc(c.b + (int64_t)c0 * c.H + c.e, nt * c.H * 2);
        gv = __builtin_amdgcn_raw_buffer_load_b16(sg, lane * c.H * 2, 0, 0);
        bv = __builtin_amdgcn_raw_buffer_load_b16(sb, lane * c.H * 2, 0, 0);
    }
};

template <int D>
struct Frags {
    static constexpr int HALF = D / 2;
    static constexpr int NT = HALF / 16;         // channel tiles of a half
    u32x2_t q[NT][4];                            // q (token block, channel tile), accumulator layout
    bf16x8_t t[kPairs], akw[kPairs], aqw[kPairs], naqk[kPairs];

    __device__ static __amdgpu_buffer_rsrc_t mats(const Ctx& c, int ch)
    {
        const bool in = ch < c.nchunks;
        return rsrc(c.mats + ((c.vbase + (in ? ch : 0)) * c.H + c.e) * (int64_t)gram::kChunkElems,
                    in ? gram::kChunkElems * 2 : 0);
    }
    // T and A_kkw (last used by U)
    __device__ void load_t(const Ctx& c, int ch)
    {
        const auto rs = mats(c, ch);
#pragma unroll
        for (int p = 0; p < kPairs; ++p) {
            t[p] = mat32(rs, gram::kMatT, pair_tb(p), pair_h2(p), c.lane);
            akw[p] = mat32(rs, gram::kMatAkkw, pair_tb(p), pair_h2(p), c.lane);
        }
    }
    // -A_qk and A_qkw (last used by O_loc)
    __device__ void load_qk(const Ctx& c, int ch)
    {
        const auto rs = mats(c, ch);
#pragma unroll
        for (int p = 0; p < kPairs; ++p) {
            naqk[p] = mat32(rs, gram::kMatNAqk, pair_tb(p), pair_h2(p), c.lane);
            aqw[p] = mat32(rs, gram::kMatAqkw, pair_tb(p), pair_h2(p), c.lane);
        }
    }
    // q tiles of this helper's channels (last used by Q')
    __device__ void load_q(const Ctx& c, int ch, int h)
    {
        const int li = c.lane & 15, lg = c.lane >> 4;
        const int c0 = c.seq0 + ch * kC;
        const int nt = chunk_tokens(c, ch);
        const auto sq = rsrc(c.q + (int64_t)c0 * c.rowQK + (int64_t)c.e * D + h * HALF,
                             nt * (int)c.rowQK * 2);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                q[n][tb] = __builtin_bit_cast(
                    u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
                                 sq, ((tb * 16 + li) * (int)c.rowQK + n * 16 + 4 * lg) * 2, 0, 0));
        }
    }
    template <bool WO>
    __device__ void load(const Ctx& c, int ch, int h)
    {
        load_t(c, ch);
        if constexpr (WO) {
            load_qk(c, ch);
            load_q(c, ch, h);
        }
    }
};

// ---- helper h: chunk ch into buffer buf (rows, gates, W, Q', U, O_loc) from
// st (rows of ch) and fr (fragments of ch), loading each for chunk ch + 1 as
// soon as chunk ch is done with it.  Reads only what this wavefront wrote.
// WO false (no outputs wanted: the states alone): Q' and O_loc are skipped.
template <int D, bool WO>
__device__ __forceinline__ void prepare(Rows<D>& st, Frags<D>& fr, unsigned char* buf, float* scr,
                                        const Ctx& c, int ch, int h)
{
    using Ly = Lay<D>;
    using St = Rows<D>;
    constexpr int LDD = Ly::LDD, LDV = Ly::LDV, HALF = St::HALF, NT = Frags<D>::NT;
    const int lane = c.lane, li = lane & 15, lg = lane >> 4;
    uint16_t* sK = reinterpret_cast<uint16_t*>(buf + Ly::oK);
    uint16_t* sKW = reinterpret_cast<uint16_t*>(buf + Ly::oKW);
    uint16_t* sV = reinterpret_cast<uint16_t*>(buf + Ly::oV);
    uint16_t* sW = reinterpret_cast<uint16_t*>(buf + Ly::oW);
    uint16_t* sQp = reinterpret_cast<uint16_t*>(buf + Ly::oQp);
    u32x2_t* sU = reinterpret_cast<u32x2_t*>(buf + Ly::oU) + h * 4 * 64;
    u32x2_t* sO = reinterpret_cast<u32x2_t*>(buf + Ly::oO) + h * 4 * 64;
    float* sFac = reinterpret_cast<float*>(buf + Ly::oFac);

    // rows of chunk ch: channels h * HALF .., value columns 16 h ..
    {
        constexpr int PPR = HALF / 8;
#pragma unroll
        for (int x = 0; x < St::NPK; ++x) {
            const int p = lane + 64 * x;
            const int off = (p / PPR) * LDD + h * HALF + (p % PPR) * 8;
            *reinterpret_cast<uint4*>(sK + off) = st.rk[x];
            *reinterpret_cast<uint4*>(sKW + off) = st.rw[x];
        }
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int p = lane + 64 * x;
            *reinterpret_cast<uint4*>(sV + (p / 2) * LDV + 16 * h + (p % 2) * 8) = st.rv[x];
        }
    }
    // gates of chunk ch (lane = token; decay 1 past the chunk's end)
    {
        const int nt = chunk_tokens(c, ch);
        const float l2 = lane < nt ? __log2f(fmaxf(bf16_to_f32(st.gv), 1e-30f)) : 0.f;
        const float lam = wave_inclusive_sum(l2);
        const float lamC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lam), 63));
        const float gam = __builtin_amdgcn_exp2f(lam);
        scr[lane] = bf16_to_f32(st.bv) * gam;
        scr[kC + lane] = gam;
        if (h == 0) {
            sFac[lane] = __builtin_amdgcn_exp2f(lamC - lam);
            if (lane == 0)
                sFac[kC] = __builtin_amdgcn_exp2f(lamC);
        }
    }
    SCHED_FENCE();
    st.load(c, ch + 1, h);
    SCHED_FENCE();

    // K^T fragments of this half and V fragments of these columns; b gamma by token pieces
    bf16x8_t kf[NT][2], vf[2];
    float4 bg[2][2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
        for (int n = 0; n < NT; ++n)
            kf[n][h2] = frag_col(sK + h2 * 32 * LDD + h * HALF + n * 16, LDD, lane);
        vf[h2] = frag_col(sV + h2 * 32 * LDV + 16 * h, LDV, lane);
        bg[h2][0] = *reinterpret_cast<const float4*>(scr + h2 * 32 + lg * 8);
        bg[h2][1] = *reinterpret_cast<const float4*>(scr + h2 * 32 + lg * 8 + 4);
    }
    SCHED_FENCE();

    // W^T (channels of tile n, tokens of block tb) = K^T diag(b gamma) T^T: all
    // products first, then the stores, so no store waits on a product just issued
    {
        bf16x8_t ts[kPairs];
#pragma unroll
        for (int p = 0; p < kPairs; ++p)
            ts[p] = scale8(fr.t[p], bg[pair_h2(p)][0], bg[pair_h2(p)][1]);
        f32x4_t w[4][NT];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
            for (int tb = 2 * h2; tb < 4; ++tb) {
#pragma unroll
                for (int n = 0; n < NT; ++n)
                    w[tb][n] = mma32(kf[n][h2], ts[pidx(tb, h2)],
                                     h2 == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : w[tb][n]);
            }
        }
        // lane (li, lg): token tb * 16 + li, channels 4 lg .. 4 lg + 3 of tile n
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
            for (int n = 0; n < NT; ++n)
                *reinterpret_cast<u32x2_t*>(sW + wy_off<D>(tb * 16 + li, h * HALF + n * 16 + 4 * lg)) =
                    pack4(w[tb][n]);
        }
    }
    // U = T (A_kkw V), columns 16 h .. 16 h + 15, accumulator layout (lane: column li, tokens 4 lg ..)
    f32x4_t u[4];
    {
        f32x4_t up[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
            for (int tb = 2 * h2; tb < 4; ++tb)
                up[tb] = mma32(fr.akw[pidx(tb, h2)], vf[h2], h2 == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : up[tb]);
        }
        bf16x8_t upp[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
            upp[h2] = pair_rows(as_b16(up[2 * h2], 1.f, 1.f, 1.f, 1.f), as_b16(up[2 * h2 + 1], 1.f, 1.f, 1.f, 1.f));
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
            for (int tb = 2 * h2; tb < 4; ++tb)
                u[tb] = mma32(fr.t[pidx(tb, h2)], upp[h2], h2 == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : u[tb]);
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
            sU[tb * 64 + lane] = pack4(u[tb]);
    }
    SCHED_FENCE();
    fr.load_t(c, ch + 1);
    SCHED_FENCE();
    if constexpr (!WO)
        return;

    // Q'^T = diag(gamma) Q^T - W^T A_qk^T (the stored matrix is -A_qk); W^T read back
    {
        bf16x8_t wf[NT][2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
            for (int n = 0; n < NT; ++n)
                wf[n][h2] = wy_col<D>(sW, h2 * 32, h * HALF + n * 16, lane);
        }
        float gq[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
            gq[tb] = scr[kC + tb * 16 + li];
        SCHED_FENCE();
        f32x4_t w[4][NT];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                w[tb][n] = unpack4(fr.q[n][tb]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    w[tb][n][r] *= gq[tb];
            }
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
            for (int tb = 2 * h2; tb < 4; ++tb) {
#pragma unroll
                for (int n = 0; n < NT; ++n)
                    w[tb][n] = mma32(wf[n][h2], fr.naqk[pidx(tb, h2)], w[tb][n]);
            }
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
            for (int n = 0; n < NT; ++n)
                *reinterpret_cast<u32x2_t*>(sQp + wy_off<D>(tb * 16 + li, h * HALF + n * 16 + 4 * lg)) =
                    pack4(w[tb][n]);
        }
    }
    SCHED_FENCE();
    fr.load_q(c, ch + 1, h);
    // O_loc^T = V^T A_qkw^T - U^T A_qk^T, lane (li, lg): token li of block tb, columns 4 lg ..
    {
        bf16x8_t uq[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
            uq[h2] = pair_rows(as_b16(u[2 * h2], 1.f, 1.f, 1.f, 1.f), as_b16(u[2 * h2 + 1], 1.f, 1.f, 1.f, 1.f));
        f32x4_t o[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
            for (int tb = 2 * h2; tb < 4; ++tb)
                o[tb] = mma32(vf[h2], fr.aqw[pidx(tb, h2)], h2 == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : o[tb]);
#pragma unroll
            for (int tb = 2 * h2; tb < 4; ++tb)
                o[tb] = mma32(uq[h2], fr.naqk[pidx(tb, h2)], o[tb]);
        }
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
            sO[tb * 64 + lane] = pack4(o[tb]);
    }
    SCHED_FENCE();
    fr.load_qk(c, ch + 1);
}

// ---- state wavefront jb: value columns j0 + 16 jb .. + 15, one chunk:
//   X = W S0 + U,  O^T = (Q' S0)^T + O_loc^T,
//   S <- gamma_C S0 + KW^T diag(fac) V - K^T diag(fac) X.
// S0 enters the products as a 16x16x32 operand built from the accumulators.
// The LDS reads of each step are issued one step ahead (SCHED_FENCE keeps the
// scheduler from sinking them next to their uses: a wavefront alone on its
// SIMD has nothing else to hide the LDS latency with).  WO false: no O.
template <int D, bool WO>
__device__ __forceinline__ void state_chunk(f32x4_t (&S)[D / 16], const unsigned char* buf, const Ctx& c,
                                            int ch, int jb)
{
    using Ly = Lay<D>;
    constexpr int LDD = Ly::LDD, LDV = Ly::LDV;
    constexpr int NI = D / 16, NKP = NI / 2;
    const int lane = c.lane, li = lane & 15, lg = lane >> 4;
    const uint16_t* sK = reinterpret_cast<const uint16_t*>(buf + Ly::oK);
    const uint16_t* sKW = reinterpret_cast<const uint16_t*>(buf + Ly::oKW);
    const uint16_t* sV = reinterpret_cast<const uint16_t*>(buf + Ly::oV);
    const uint16_t* sW = reinterpret_cast<const uint16_t*>(buf + Ly::oW);
    const uint16_t* sQp = reinterpret_cast<const uint16_t*>(buf + Ly::oQp);
    const u32x2_t* sU = reinterpret_cast<const u32x2_t*>(buf + Ly::oU) + jb * 4 * 64;
    const u32x2_t* sO = reinterpret_cast<const u32x2_t*>(buf + Ly::oO) + jb * 4 * 64;
    const float* sFac = reinterpret_cast<const float*>(buf + Ly::oFac);

    // W row fragments and U
    bf16x8_t wf[4][NKP];
    u32x2_t ub[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
        for (int kp = 0; kp < NKP; ++kp)
            wf[tb][kp] = *reinterpret_cast<const bf16x8_t*>(sW + wy_off<D>(tb * 16 + li, kp * 32 + lg * 8));
        ub[tb] = sU[tb * 64 + lane];
    }
    // S0 as 16x16x32 operands (channels 32 kp + 8 g .. in lane group g)
    bf16x8_t s0q[NKP];
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp)
        s0q[kp] = pair_rows(as_b16(S[2 * kp], 1.f, 1.f, 1.f, 1.f), as_b16(S[2 * kp + 1], 1.f, 1.f, 1.f, 1.f));
    SCHED_FENCE();
    // Q' row fragments and O_loc, read while X runs
    bf16x8_t qf[4][NKP];
    u32x2_t ob[4];
    if constexpr (WO) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
            for (int kp = 0; kp < NKP; ++kp)
                qf[tb][kp] = *reinterpret_cast<const bf16x8_t*>(sQp + wy_off<D>(tb * 16 + li, kp * 32 + lg * 8));
            ob[tb] = sO[tb * 64 + lane];
        }
    }
    SCHED_FENCE();

    // ---- X = W S0 + U: four independent accumulator chains
    f32x4_t X[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
        X[tb] = unpack4(ub[tb]);
#pragma unroll
    for (int kp = 0; kp < NKP; ++kp) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
            X[tb] = mma32(wf[tb][kp], s0q[kp], X[tb]);
    }
    SCHED_FENCE();

    // reads for the KW^T V part of the update (first two row blocks), V and fac
    const float gC = sFac[kC];
    bf16x8_t vf[2], kwf[2][NI];
    float4 fc[4];
    auto load_kw = [&](int ib) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
            kwf[h2][ib] = frag_col(sKW + h2 * 32 * LDD + ib * 16, LDD, lane);
    };
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        vf[h2] = frag_col(sV + h2 * 32 * LDV + jb * 16, LDV, lane);
        fc[2 * h2] = *reinterpret_cast<const float4*>(sFac + h2 * 32 + lg * 8);
        fc[2 * h2 + 1] = *reinterpret_cast<const float4*>(sFac + h2 * 32 + lg * 8 + 4);
    }
    load_kw(0);
    load_kw(1);
    SCHED_FENCE();

    // ---- O^T = (Q' S0)^T + O_loc^T
    f32x4_t OT[4];
    if constexpr (WO) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
            OT[tb] = unpack4(ob[tb]);
#pragma unroll
        for (int kp = 0; kp < NKP; ++kp) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
                OT[tb] = mma32(s0q[kp], qf[tb][kp], OT[tb]);
        }
    }
    SCHED_FENCE();

    // ---- S <- gamma_C S + KW^T diag(fac) V, two 16-row blocks of S per step
    {
        load_kw(2);
        load_kw(3);
        SCHED_FENCE();
        const bf16x8_t vs0 = scale8(vf[0], fc[0], fc[1]);
        const bf16x8_t vs1 = scale8(vf[1], fc[2], fc[3]);
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
            S[ib] = mma32(kwf[0][ib], vs0, S[ib]);
            S[ib + 1] = mma32(kwf[0][ib + 1], vs0, S[ib + 1]);
            S[ib] = mma32(kwf[1][ib], vs1, S[ib]);
            S[ib + 1] = mma32(kwf[1][ib + 1], vs1, S[ib + 1]);
            SCHED_FENCE();
        }
    }

    // K^T fragments (tokens 8g .. 8g+7 of each 32-token half in lane group g) and scales
    bf16x8_t ke[2][NI];
    float4 fe[4];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
#pragma unroll
        for (int ib = 0; ib < NI; ++ib)
            ke[tp][ib] = frag_col(sK + tp * 32 * LDD + ib * 16, LDD, lane);
        fe[2 * tp] = *reinterpret_cast<const float4*>(sFac + tp * 32 + lg * 4);
        fe[2 * tp + 1] = *reinterpret_cast<const float4*>(sFac + tp * 32 + 16 + lg * 4);
    }
    SCHED_FENCE();

    // ---- S <- S - K^T diag(fac) X   (NI independent accumulators per half)
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

    // ---- O rows (lane (li, lg): token tb * 16 + li, value columns 4 lg .. of block jb);
    //      rows past the chunk's last token fall outside the buffer range
    if constexpr (!WO)
        return;
    const int c0 = c.seq0 + ch * kC;
    const int nt = chunk_tokens(c, ch);
    const __amdgpu_buffer_rsrc_t orsrc = rsrc(c.o + (int64_t)c0 * c.rowV, nt * (int)c.rowV * 2);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int t = tb * 16 + li;
        __builtin_amdgcn_raw_buffer_store_b64(pack4(OT[tb]), orsrc,
                                              (t * (int)c.rowV + c.e * c.DV + c.j0 + jb * 16 + lg * 4) * 2, 0, 0);
    }
}

template <int D, bool WO>
__global__ __launch_bounds__(kWaves * 64) void scan_state_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ kw, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ b,
    const int32_t* __restrict__ cu, int H, int DV, int n_slices, const float* __restrict__ s_init,
    const uint16_t* __restrict__ mats, uint16_t* __restrict__ o, float* __restrict__ s_final,
    uint16_t* __restrict__ ck = nullptr, uint16_t* __restrict__ ckT = nullptr)
{
    using Ly = Lay<D>;
    constexpr int NI = D / 16;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Ly::total];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int slice, chain;
    xcd_map(blockIdx.x, gridDim.x, n_slices, slice, chain);

    Ctx c;
    c.q = q; c.k = k; c.kw = kw; c.v = v; c.g = g; c.b = b; c.mats = mats; c.o = o;
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
    c.vbase = c.seq0 / kC + c.n;                 // the chain's first virtual chunk
    const int li = c.lane & 15, lg = c.lane >> 4;

    if (wave < 2) {
        const int jb = wave;
        f32x4_t S[NI];
        const int64_t sb = (((int64_t)c.n * H + c.e) * D) * DV + c.j0 + jb * 16;
#pragma unroll
        for (int ib = 0; ib < NI; ++ib) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[ib][r] = s_init ? s_init[sb + (int64_t)(ib * 16 + lg * 4 + r) * DV + li] : 0.f;
        }
        lds_barrier();                           // chunk 0 prepared
        for (int ch = 0; ch < c.nchunks; ++ch) {
            if (ck) {
                // the chunk's start state, bf16, as rows [dk][dv] and transposed [dv][dk]
                // per (virtual chunk, head) (the chunkwise backward reads both)
                const int64_t vc = (c.vbase + ch) * H + c.e;
                const int col = c.j0 + jb * 16 + li;
#pragma unroll
                for (int ib = 0; ib < NI; ++ib) {
                    const int r0 = ib * 16 + lg * 4;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        ck[(vc * D + r0 + r) * DV + col] = (uint16_t)(pack_bf16x2(S[ib][r], 0.f) & 0xffffu);
                    *reinterpret_cast<uint2*>(ckT + (vc * DV + col) * D + r0) =
                        make_uint2(pack_bf16x2(S[ib][0], S[ib][1]), pack_bf16x2(S[ib][2], S[ib][3]));
                }
            }
            state_chunk<D, WO>(S, smem + (ch & 1) * Ly::szBuf, c, ch, jb);
            lds_barrier();
        }
        if (s_final) {
#pragma unroll
            for (int ib = 0; ib < NI; ++ib) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s_final[sb + (int64_t)(ib * 16 + lg * 4 + r) * DV + li] = S[ib][r];
            }
        }
    } else {
        const int h = wave - 2;
        float* scr = reinterpret_cast<float*>(smem + Ly::oScr) + h * 2 * kC;
        Rows<D> rows;
        Frags<D> fr;
        rows.load(c, 0, h);
        fr.template load<WO>(c, 0, h);
        prepare<D, WO>(rows, fr, smem, scr, c, 0, h);
        lds_barrier();
        // chunk ch + 1 into the buffer the state wavefronts are not reading
        // (past the last chunk this prepares an empty chunk no one reads)
        for (int ch = 0; ch < c.nchunks; ++ch) {
            prepare<D, WO>(rows, fr, smem + ((ch + 1) & 1) * Ly::szBuf, scr, c, ch + 1, h);
            lds_barrier();
        }
    }
}

}  // namespace stscan

bool scan_state_supported(int dk, int dv)
{
    return (dk == 64 || dk == 128) && dv > 0 && dv % stscan::kDVS == 0;
}

hipError_t launch_scan_state(const ScanArgs& p, const void* mats, hipStream_t stream, void* ck, void* ckT)
{
    if (!p.bf16 || !scan_state_supported(p.dk, p.dv))
        return hipErrorInvalidValue;
    const int n_slices = p.dv / stscan::kDVS;
    const int64_t blocks = (int64_t)p.n_seqs * p.heads * n_slices;
    if (blocks == 0)
        return hipSuccess;
    // without o (the backward's recomputation of the states) the output terms are skipped
    auto kern = p.o ? (p.dk == 64 ? stscan::scan_state_kernel<64, true> : stscan::scan_state_kernel<128, true>)
                    : (p.dk == 64 ? stscan::scan_state_kernel<64, false> : stscan::scan_state_kernel<128, false>);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(stscan::kWaves * 64), 0, stream,
                       (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.kw,
                       (const uint16_t*)p.v, (const uint16_t*)p.g, (const uint16_t*)p.b,
                       p.cu_seqlens, p.heads, p.dv, n_slices, p.s_init, (const uint16_t*)mats,
                       (uint16_t*)p.o, p.s_final, (uint16_t*)ck, (uint16_t*)ckT);
    return hipGetLastError();
}

}  // namespace prism
