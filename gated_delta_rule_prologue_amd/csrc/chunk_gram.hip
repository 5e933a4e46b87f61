// chunk_gram.hip -- per-chunk matrices of the WY/UT scan, all chunks in parallel
//
// The chunk algebra of the gated delta-rule scan (chunks of 64 tokens; see
// chunk_scan.hip for the derivation; PRISM pages: WeChat ICML 2026 summary,
// section 消除 Token 间串行; gist.science summary of arXiv 2602.10796,
// section 2.1, S_t = S_{t-1} A_t + B_t with input-only A_t, B_t) needs, per
// chunk, four 64x64 matrices that depend on the chunk's inputs only:
//
//   T     = (I + A_kk)^-1,   A_kk = diag(b) (D . tril_-1(K K^T))      UT transform
//   A_kkw = diag(b) (D . tril_-1(K KW^T))
//   A_qkw = D . tril_0(Q KW^T)
//   -A_qk = -(D . tril_0(Q K^T))
//
// with D[t, s] = 2^(lam_t - lam_s) for s <= t (lam the in-chunk cumulative
// log2 of the forget gates).  No chunk depends on another, so they are formed
// here for every (chunk, head) at once, one workgroup each, and the state
// scan (chunk_scan_state.hip) reads them back; the sequential part of the scan
// then carries only the state products.
//
// Per workgroup (four wavefronts): the q, k, kw rows of the chunk are staged
// in LDS; each wavefront builds its Gram block pairs on 16x16x32 bf16 MFMA
// with the masks and decays applied (the same factorised decays as the
// single-kernel scan); A_kkw, A_qkw and -A_qk go to the workspace from
// registers; A_kk goes to LDS in fp32, where the four diagonal 16x16 inverses
// are formed by substitution in fp32 and the off-diagonal blocks of T by the
// block recursion T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj on fp32 MFMA
// (16x16x4), level by level.  T is rounded to bf16 once, at the end.
//
// Output layout per (virtual chunk v, head e), 20 KB: matrices T, A_kkw,
// A_qkw, -A_qk, each as the ten 16x16 blocks (i, j), i >= j, at index
// i (i + 1) / 2 + j, 256 bf16 per block, rows of 16 elements whose two
// 16-byte halves are swapped in rows 8..15 (so that a 16-byte fragment read
// of a block by 32 lanes touches each LDS bank once).  Virtual chunks number
// the chunks of all sequences without a table: sequence n owns virtual chunks
// vstart(n) = floor(cu[n] / 64) + n onwards, which leaves room for its
// ceil(len / 64) chunks before vstart(n + 1).
#include "common.h"
#include "gram.h"
#include "kernels.h"
#include "mfma_bf16.h"

namespace prism {
namespace gram {

using namespace mfma;

constexpr int kThreads = 256;

template <int D>
struct GLayout {
    static constexpr int LDD = D + 8;
    static constexpr int szRow = kC * LDD * 2;
    static constexpr int oQ = 0, oK = szRow, oKW = 2 * szRow;
    // after the Gram phase the row tiles are dead: fp32 A_kk, T and one 16x16
    // scratch block per wavefront take their place
    static constexpr int LDF = kC + 1;
    static constexpr int oAkk = 0;
    static constexpr int oT = oAkk + kC * LDF * 4;
    static constexpr int oY = oT + kC * LDF * 4;
    static constexpr int endF = oY + 4 * 16 * 17 * 4;
    static constexpr int oLam = ((3 * szRow > endF ? 3 * szRow : endF) + 15) / 16 * 16;  // lam, b
    static constexpr int total = oLam + 2 * kC * 4;
};

// The pairs (t-block, s-block) of each wavefront (ten lower-triangle pairs;
// 3, 3, 2, 2 per wavefront).
__constant__ const int kPairT[4][3] = {{3, 3, 3}, {2, 2, 2}, {3, 1, -1}, {1, 0, -1}};
__constant__ const int kPairS[4][3] = {{0, 1, 2}, {0, 1, 2}, {3, 0, -1}, {1, 0, -1}};

// Product of two 16x16 fp32 blocks in LDS (row strides lda, ldb) on
// v_mfma_f32_16x16x4_f32, added to acc: lane (j, g) gets rows 4g .. 4g + 3 of
// column j.
__device__ __forceinline__ f32x4_t mm16_f32(const float* a, int lda, const float* b, int ldb,
                                             f32x4_t acc, int lane)
{
    const int i = lane & 15, g = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i * lda + 4 * s + g], b[(4 * s + g) * ldb + i],
                                                  acc, 0, 0, 0);
    return acc;
}

// Largest sequence n with vstart(n) = floor(cu[n] / 64) + n <= v (64-ary
// search over the wavefront; vstart strictly increases with n and vstart(0) = 0).
__device__ __forceinline__ int find_seq(const int32_t* cu, int n_seqs, int v, int lane)
{
    int lo = 0, hi = n_seqs;
    while (hi - lo > 1) {
        const int step = (hi - lo + 63) / 64;
        const int idx = lo + lane * step;
        const bool ok = idx < hi && cu[idx] / kC + idx <= v;
        const int cnt = __popcll(__ballot(ok));
        lo += (cnt - 1) * step;
        hi = min(lo + step, hi);
    }
    return lo;
}

template <int D>
__global__ __launch_bounds__(kThreads) void gram_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ kw,
    const uint16_t* __restrict__ g, const uint16_t* __restrict__ b, const int32_t* __restrict__ cu,
    int n_seqs, int H, uint16_t* __restrict__ out)
{
    using Ly = GLayout<D>;
    constexpr int LDD = Ly::LDD, LDF = Ly::LDF;
    constexpr int KS = D / 32;
    __shared__ __attribute__((aligned(16))) unsigned char smem[Ly::total];
    uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + Ly::oQ);
    uint16_t* sK = reinterpret_cast<uint16_t*>(smem + Ly::oK);
    uint16_t* sKW = reinterpret_cast<uint16_t*>(smem + Ly::oKW);
    float* sLam = reinterpret_cast<float*>(smem + Ly::oLam);
    float* sB = sLam + kC;
    float* fA = reinterpret_cast<float*>(smem + Ly::oAkk);
    float* fT = reinterpret_cast<float*>(smem + Ly::oT);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const int e = (int)(blockIdx.x % (unsigned)H);
    const int v = (int)(blockIdx.x / (unsigned)H);
    const int n = find_seq(cu, n_seqs, v, lane);
    const int seq0 = cu[n], seq1 = cu[n + 1];
    const int c0 = seq0 + (v - (seq0 / kC + n)) * kC;
    const int nt = min(kC, seq1 - c0);
    if (nt <= 0)
        return;                                  // a virtual chunk past the sequence's last

    // ---- stage the rows and the gates: every load issued before any LDS store;
    // bounded buffer loads return zeros for rows past the chunk end
    const int rowQK = H * D;
    const int64_t base = (int64_t)c0 * rowQK + (int64_t)e * D;
    constexpr int PPR = D / 8;                   // 16-byte pieces per row
    constexpr int NX = kC * PPR / kThreads;
    constexpr uint32_t fl = 0x00020000;
    const int nbytes = nt * rowQK * 2;
    const auto rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(q + base), 0, nbytes, fl);
    const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(k + base), 0, nbytes, fl);
    const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kw + base), 0, nbytes, fl);
    const auto rg = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(g + (int64_t)c0 * H + e), 0,
                                                     nt * H * 2, fl);
    const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(b + (int64_t)c0 * H + e), 0,
                                                     nt * H * 2, fl);
    const uint16_t graw = __builtin_amdgcn_raw_buffer_load_b16(rg, lane * H * 2, 0, 0);
    const uint16_t braw = __builtin_amdgcn_raw_buffer_load_b16(rb, lane * H * 2, 0, 0);
    uint4 vq[NX], vk[NX], vw[NX];
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        const int p = tid + x * kThreads;
        const int off = ((p / PPR) * rowQK + (p % PPR) * 8) * 2;
        vq[x] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
        vk[x] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
        vw[x] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
    }
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        const int p = tid + x * kThreads;
        const int t = p / PPR, c = (p % PPR) * 8;
        *reinterpret_cast<uint4*>(sQ + t * LDD + c) = vq[x];
        *reinterpret_cast<uint4*>(sK + t * LDD + c) = vk[x];
        *reinterpret_cast<uint4*>(sKW + t * LDD + c) = vw[x];
    }
    if (wave == 0) {
        // decay 1 and no erase past the chunk end
        const float gv = lane < nt ? bf16_to_f32(graw) : 1.f;
        sLam[lane] = wave_inclusive_sum(__log2f(fmaxf(gv, 1e-30f)));
        sB[lane] = bf16_to_f32(braw);
    }
    lds_barrier();

    // ---- Gram pairs of this wavefront, masked and decayed, in registers
    // (transposed blocks: lane (li, lg) holds element (t = tb 16 + li, s = sb 16 + 4 lg + r))
    f32x4_t mkk[3], mkw[3], mqk[3], mqw[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const int tb = kPairT[wave][p], sb = kPairS[wave][p];
        if (tb < 0)
            continue;
        f32x4_t gkk = {0.f, 0.f, 0.f, 0.f}, gkw = gkk, gqk = gkk, gqw = gkk;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8_t ak = frag_row(sK + sb * 16 * LDD + ks * 32, LDD, lane);
            const bf16x8_t aw = frag_row(sKW + sb * 16 * LDD + ks * 32, LDD, lane);
            const bf16x8_t bk = frag_row(sK + tb * 16 * LDD + ks * 32, LDD, lane);
            const bf16x8_t bq = frag_row(sQ + tb * 16 * LDD + ks * 32, LDD, lane);
            gkk = mma32(ak, bk, gkk);
            gkw = mma32(aw, bk, gkw);
            gqk = mma32(ak, bq, gqk);
            gqw = mma32(aw, bq, gqw);
        }
        const int t = tb * 16 + li, s0 = sb * 16 + lg * 4;
        const float lt = sLam[t], bt = sB[t];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int s = s0 + r;
            float mi, ms;
            if (sb == tb) {
                // diagonal block: causal masks, decay 2^(lam_t - lam_s) per element
                const float dec = __builtin_amdgcn_exp2f(fminf(lt - sLam[s], 0.f));
                mi = s <= t ? dec : 0.f;
                ms = s < t ? dec * bt : 0.f;
            } else {
                // s-block before t: 2^(lam_t - lam_e) 2^(lam_e - lam_s), lam_e the
                // s-block's last token, both factors <= 1 (lam never increases)
                const float le = sLam[sb * 16 + 15];
                mi = __builtin_amdgcn_exp2f(lt - le) * __builtin_amdgcn_exp2f(le - sLam[s]);
                ms = mi * bt;
            }
            mkk[p][r] = ms * gkk[r];
            mkw[p][r] = ms * gkw[r];
            mqk[p][r] = -mi * gqk[r];
            mqw[p][r] = mi * gqw[r];
        }
    }

    // ---- A_kkw, A_qkw, -A_qk straight to the workspace (bf16, 8-byte pieces)
    uint16_t* o = out + ((int64_t)v * H + e) * kChunkElems;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const int tb = kPairT[wave][p], sb = kPairS[wave][p];
        if (tb < 0)
            continue;
        const int off = blk_index(tb, sb) * kBlockElems + swz(li, lg * 4);
        st4(o + 1 * kMatElems + off, mkw[p]);
        st4(o + 2 * kMatElems + off, mqw[p]);
        st4(o + 3 * kMatElems + off, mqk[p]);
    }
    lds_barrier();                               // row tiles dead from here

    // ---- A_kk in fp32 (lower blocks; the diagonal blocks strictly lower)
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const int tb = kPairT[wave][p], sb = kPairS[wave][p];
        if (tb < 0)
            continue;
        const int t = tb * 16 + li, s0 = sb * 16 + lg * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            fA[t * LDF + s0 + r] = mkk[p][r];
    }
    lds_barrier();

    // ---- diagonal inverses: lane (16 g + i) holds row i of A_gg, returns column i of T_gg
    if (wave == 0) {
        float a[16], x[16];
#pragma unroll
        for (int c = 0; c < 16; ++c)
            a[c] = fA[(lg * 16 + li) * LDF + lg * 16 + c];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            x[r] = (r == li) ? 1.f : 0.f;
        subst<0>(x, a);
#pragma unroll
        for (int r = 0; r < 16; ++r)
            fT[(lg * 16 + r) * LDF + lg * 16 + li] = x[r];
    }
    lds_barrier();

    // ---- off-diagonal blocks of T, by distance d = i - j:
    //      Y = sum_{k=j}^{i-1} A_ik T_kj,  T_ij = -T_ii Y
    float* fY = reinterpret_cast<float*>(smem + Ly::oY) + wave * 16 * 17;
    auto block = [&](int i, int j) {
        f32x4_t y = {0.f, 0.f, 0.f, 0.f};
        for (int kk = j; kk < i; ++kk)
            y = mm16_f32(fA + (i * 16) * LDF + kk * 16, LDF, fT + (kk * 16) * LDF + j * 16, LDF, y,
                         lane);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            fY[(lg * 4 + r) * 17 + li] = y[r];
        // same-wavefront LDS write then read: ordered by the wavefront itself
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        f32x4_t t = {0.f, 0.f, 0.f, 0.f};
        t = mm16_f32(fT + (i * 16) * LDF + i * 16, LDF, fY, 17, t, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            fT[(i * 16 + lg * 4 + r) * LDF + j * 16 + li] = -t[r];
    };
    if (wave < 3)
        block(wave + 1, wave);                   // d = 1: (1,0) (2,1) (3,2)
    lds_barrier();
    if (wave < 2)
        block(wave + 2, wave);                   // d = 2: (2,0) (3,1)
    lds_barrier();
    if (wave == 0)
        block(3, 0);                             // d = 3: (3,0)
    lds_barrier();

    // ---- T (bf16) to the workspace: 10 blocks x 16 rows x 2 halves of 8 elements
    for (int p = tid; p < kBlocks * 32; p += kThreads) {
        const int bi = p >> 5, r = (p >> 1) & 15, h = p & 1;
        int i = 0;
        while ((i + 1) * (i + 2) / 2 <= bi)
            ++i;
        const int j = bi - i * (i + 1) / 2;
        const float* src = fT + (i * 16 + r) * LDF + j * 16 + h * 8;
        uint32_t w[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
            w[x] = pack_bf16x2(src[2 * x], src[2 * x + 1]);
        *reinterpret_cast<uint4*>(o + bi * kBlockElems + swz(r, h * 8)) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

}  // namespace gram

size_t gram_workspace_bytes(int n_seqs, int total_tokens, int heads)
{
    const int64_t nv = (int64_t)total_tokens / gram::kC + n_seqs;
    return (size_t)(nv * heads) * gram::kChunkElems * 2;
}

hipError_t launch_gram(const ScanArgs& p, void* ws, hipStream_t stream)
{
    if (!p.bf16 || (p.dk != 64 && p.dk != 128))
        return hipErrorInvalidValue;
    const int64_t blocks = ((int64_t)p.total_tokens / gram::kC + p.n_seqs) * p.heads;
    if (blocks == 0 || p.total_tokens == 0)
        return hipSuccess;
    auto kern = p.dk == 64 ? gram::gram_kernel<64> : gram::gram_kernel<128>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(gram::kThreads), 0, stream,
                       (const uint16_t*)p.q, (const uint16_t*)p.k, (const uint16_t*)p.kw,
                       (const uint16_t*)p.g, (const uint16_t*)p.b, p.cu_seqlens, p.n_seqs, p.heads,
                       (uint16_t*)ws);
    return hipGetLastError();
}

}  // namespace prism
