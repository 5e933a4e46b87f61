// long_seq.hip -- the chunk scan of few, long sequences, split into segments
// that are scanned side by side.
//
// The recurrence is affine in the state: over a segment p of a sequence,
// S_end = M_p S_in + S_loc, where M_p is the product of the segment's
// transitions g_t (I - b_t k_t k_t^T) and S_loc the end state of the segment
// run from S = 0 (WeChat page section 背景：无限背包 vs 有限背包 on linear
// recurrences and parallel scans; gist.science summary section 2.1,
// S_t = S_{t-1} A_t + B_t with input-only A_t, B_t).  With few chains the scan
// leaves most compute units idle while it walks every chunk of a chain in
// order, so each sequence is cut into P segments and:
//   1. one scan launch over all segments as separate sequences: its first
//      blocks run them from S = 0 (local outputs o_loc, end states S_loc), the
//      rest scan the transitions alone (start S = I with dv = dk, no write
//      term), giving M_p and o'_t = M_{start->t}^T q_t;
//   2. combine_kernel, once per segment in order, chains them: S_in(0) = S_init
//      (or 0), S_in(p + 1) = M_p S_in(p) + S_loc(p), S_final = S_in(P);
//   3. correct_kernel adds the carried state to the outputs,
//      o_t += S_in(p)^T o'_t, a (tokens x dk) by (dk x dv) product on MFMA.
// The segment boundaries are planned on the device from cu_seqlens (no host
// synchronisation): segment p of sequence n starts p * ceil(len / P / 64) * 64
// tokens into it (whole chunks), clamped to its end.
#include "common.h"
#include "kernels.h"

namespace prism {
namespace longseq {

typedef unsigned v4u_t __attribute__((ext_vector_type(4)));

// seg_cu[n P + p] = start of segment p of sequence n; seg_cu[n_seqs P] = T.
__global__ __launch_bounds__(256) void plan_kernel(const int32_t* __restrict__ cu, int n_seqs, int P,
                                                   int32_t* __restrict__ seg_cu)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i > n_seqs * P)
        return;
    if (i == n_seqs * P) {
        seg_cu[i] = cu[n_seqs];
        return;
    }
    const int n = i / P, p = i % P;
    const int len = cu[n + 1] - cu[n];
    const int seg = (len + P * 64 - 1) / (P * 64) * 64;     // whole chunks per segment
    seg_cu[i] = cu[n] + min(p * seg, len);
}

// One step of the chain over segments: S_next = M_p S_prev + S_loc(p) for
// every (sequence, head), one workgroup per 32 x 32 output block, M_p rows
// and S_prev columns staged in LDS.  S_prev is the start state of segment p
// (S_init or zero for p = 0, else the S_in slot of segment p); S_next is the
// S_in slot of segment p + 1, or S_final after the last segment; both are
// addressed per (sequence n, head e) as base + n * nstride + e * dk * dv.
template <int D, int DV>
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ M, const float* __restrict__ S_loc, const float* S_prev,
    int64_t prev_nstride, int H, int P, int p, float* S_next, int64_t next_nstride)
{
    constexpr int B = 32;
    __shared__ float sM[B][D + 1];
    __shared__ float sP[D][B];
    const int tid = threadIdx.x;
    const int jj = tid % B, rr = tid / B;        // column; row group of 4 rows
    const int blk = blockIdx.x % ((D / B) * (DV / B));
    const int chain = blockIdx.x / ((D / B) * (DV / B));
    const int rb = blk / (DV / B), cb = blk % (DV / B);
    const int n = chain / H, e = chain % H;
    const int64_t seg = ((int64_t)n * P + p) * H + e;
    const float* Mp = M + seg * D * D + (int64_t)rb * B * D;
    if (S_prev)                                  // (no M_p for a first segment from zero)
        for (int x = tid; x < B * D; x += 256)
            sM[x / D][x % D] = Mp[x];
    const float* prev = S_prev ? S_prev + n * prev_nstride + (int64_t)e * D * DV : nullptr;
    for (int x = tid; x < D * B; x += 256)
        sP[x / B][x % B] = prev ? prev[(int64_t)(x / B) * DV + cb * B + x % B] : 0.f;
    __syncthreads();
    const int j = cb * B + jj;
    const float* loc = S_loc + seg * D * DV;
    float acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        acc[r] = loc[(int64_t)(rb * B + rr * 4 + r) * DV + j];
    // a zero start state skips the product (M_p of such a first segment is never computed)
    for (int k = 0; prev && k < D; ++k) {
        const float pk = sP[k][jj];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            acc[r] += sM[rr * 4 + r][k] * pk;
    }
    float* out = S_next + n * next_nstride + (int64_t)e * D * DV;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        out[(int64_t)(rb * B + rr * 4 + r) * DV + j] = acc[r];
}

// o[t] += S_in(p)^T o'[t].  Grid: (heads, segment x group of kTPW tiles of 64
// tokens counted from the segment start).  The segment's start state is
// staged once as S_in^T in bf16 (LDS); wave w computes rows 16 w .. 16 w + 15
// of a tile on 16x16x32 bf16 MFMA (A = o' rows straight from HBM, B = S_in^T
// from LDS) and the fp32 tile goes through LDS for a 16-byte read-modify-write
// of o.  The o' and o rows of tile i + 1 are loaded while tile i is computed.
constexpr int kTPW = 8;
template <int D, int DV>
__global__ __launch_bounds__(256) void correct_kernel(
    const uint16_t* __restrict__ op, const float* __restrict__ S_in, const float* __restrict__ S_init,
    const int32_t* __restrict__ seg_cu, int P, int groups, int H, uint16_t* __restrict__ o)
{
    constexpr int LDB = D + 8;                   // bf16 pitch of S_in^T rows
    constexpr int LDC = DV + 4;                  // fp32 pitch of the result tile
    constexpr int KS = D / 32, NB = DV / 16;
    constexpr int OV = 64 * DV / 8 / 256;        // 16-byte pieces of o per thread per tile
    __shared__ __attribute__((aligned(16))) uint16_t sB[DV * LDB];
    __shared__ __attribute__((aligned(16))) float sC[64 * LDC];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int sg = blockIdx.y / groups, grp = blockIdx.y % groups;
    const int e = blockIdx.x;                    // heads fastest: the rows of one token are
                                                 // read by workgroups dispatched together
    if (sg % P == 0 && !S_init)
        return;                                  // a first segment started from zero
    const int start = seg_cu[sg], end = seg_cu[sg + 1];
    const int t_first = start + grp * kTPW * 64;
    if (t_first >= end)
        return;
    const int ntiles = min(kTPW, (end - t_first + 63) / 64);
    const float* Sp = sg % P == 0 ? S_init + ((int64_t)(sg / P) * H + e) * D * DV
                                  : S_in + ((int64_t)sg * H + e) * D * DV;
    // consecutive lanes take consecutive rows k, so the transposed 2-byte LDS
    // writes of a wavefront fall in consecutive banks
    for (int x = tid; x < D * DV / 4; x += 256) {
        const int k = x % D, j = (x / D) * 4;
        const float4 v4 = *reinterpret_cast<const float4*>(Sp + (int64_t)k * DV + j);
        sB[(j + 0) * LDB + k] = f32_to_bf16(v4.x);
        sB[(j + 1) * LDB + k] = f32_to_bf16(v4.y);
        sB[(j + 2) * LDB + k] = f32_to_bf16(v4.z);
        sB[(j + 3) * LDB + k] = f32_to_bf16(v4.w);
    }
    // buffer ranges that end at the segment's last token: loads past it read
    // zero and stores past it are dropped, with no branch (a branch around a
    // load makes the compiler wait for every load in flight)
    constexpr uint32_t kRsrcFlags = 0x00020000;
    const int rows = min(end - t_first, kTPW * 64);   // this workgroup's tokens
    const __amdgpu_buffer_rsrc_t rop = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(op + ((int64_t)t_first * H + e) * D), 0, rows * H * D * 2, kRsrcFlags);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        o + ((int64_t)t_first * H + e) * DV, 0, rows * H * DV * 2, kRsrcFlags);
    auto fetch = [&](int i, uint4 (&a)[KS], uint4 (&ov)[OV]) {
        const int r0 = i * 64;                   // tile rows from t_first
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            a[ks] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rop, ((r0 + wave * 16 + m) * H * D + ks * 32 + g * 8) * 2, 0, 0));
#pragma unroll
        for (int r = 0; r < OV; ++r) {
            const int x = tid + r * 256, row = x / (DV / 8), c8 = (x % (DV / 8)) * 8;
            ov[r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                ro, ((r0 + row) * H * DV + c8) * 2, 0, 0));
        }
    };
    // tile i from (a, ov), with the loads of tile i + 1 issued into (an, ovn)
    // first.  Two named register sets used alternately (the loop below is
    // unrolled by two), so that the loads land where they are used: a runtime
    // buffer index made the compiler copy, and so wait for, every load at once.
    // No branch around a load either: past the last tile the buffer ranges read
    // zeros and drop the stores, so the loop runs whole pairs of tiles.
    auto tile = [&](int i, const uint4 (&a)[KS], const uint4 (&ov)[OV], uint4 (&an)[KS], uint4 (&ovn)[OV]) {
        fetch(i + 1, an, ovn);
        f32x4_t acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8_t af = __builtin_bit_cast(bf16x8_t, a[ks]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const bf16x8_t bfr = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const uint4*>(sB + (nb * 16 + m) * LDB + ks * 32 + g * 8));
                acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr, acc[nb], 0, 0, 0);
            }
        }
        // C layout: lane holds rows 4 g + 0..3 of the wave's 16, column nb * 16 + m
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sC[(wave * 16 + g * 4 + r) * LDC + nb * 16 + m] = acc[nb][r];
        lds_barrier();
#pragma unroll
        for (int r = 0; r < OV; ++r) {
            const int x = tid + r * 256, row = x / (DV / 8), c8 = (x % (DV / 8)) * 8;
            const uint32_t w[4] = {ov[r].x, ov[r].y, ov[r].z, ov[r].w};
            uint32_t res[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo_f = __uint_as_float(w[q] << 16) + sC[row * LDC + c8 + 2 * q];
                const float hi_f = __uint_as_float(w[q] & 0xffff0000u) + sC[row * LDC + c8 + 2 * q + 1];
                res[q] = pack_bf16x2(lo_f, hi_f);
            }
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(v4u_t, make_uint4(res[0], res[1], res[2], res[3])), ro,
                ((i * 64 + row) * H * DV + c8) * 2, 0, 0);
        }
        lds_barrier();                           // sC consumed
    };
    uint4 A0[KS], O0[OV], A1[KS], O1[OV];
    fetch(0, A0, O0);
    lds_barrier();                               // sB staged
    for (int i = 0; i < ntiles; i += 2) {
        tile(i, A0, O0, A1, O1);
        tile(i + 1, A1, O1, A0, O0);
    }
}

}  // namespace longseq

// Segments per sequence for the split scan (1 = no split): as many as keep
// both scan launches within one workgroup per compute unit, up to 8, and only
// while every segment keeps at least 8 chunks on average.
int split_segments(int n_seqs, int heads, int dk, int dv, int total_tokens, int cus)
{
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128) || n_seqs < 1)
        return 1;
    const long per_seg = (long)n_seqs * heads * (dv / 32 + dk / 32);   // workgroups per segment
    int P = (int)(cus / per_seg);
    P = P > 8 ? 8 : P;
    while (P >= 2 && (long)total_tokens < (long)n_seqs * P * 64 * 8)
        --P;
    return P >= 2 ? P : 1;
}

size_t split_workspace_bytes(int n_seqs, int heads, int dk, int dv, int total_tokens, int P)
{
    if (P < 2)
        return 0;
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t segs = (size_t)n_seqs * P;
    return up((size_t)total_tokens * heads * dk * 2)          // o' (bf16)
         + up(segs * heads * dk * dv * 4)                     // S_loc
         + up(segs * heads * dk * dv * 4)                     // S_in
         + up(segs * heads * dk * dk * 4)                     // M
         + up((segs + 1) * 4);                                // segment offsets
}

hipError_t launch_split_scan(const ScanArgs& p, int P, void* ws, hipStream_t s)
{
    auto up = [](size_t x) { return (x + 255) / 256 * 256; };
    const int H = p.heads, dk = p.dk, dv = p.dv, T = p.total_tokens;
    const int segs = p.n_seqs * P;
    unsigned char* w = static_cast<unsigned char*>(ws);
    uint16_t* op = reinterpret_cast<uint16_t*>(w);
    w += up((size_t)T * H * dk * 2);
    float* S_loc = reinterpret_cast<float*>(w);
    w += up((size_t)segs * H * dk * dv * 4);
    float* S_in = reinterpret_cast<float*>(w);
    w += up((size_t)segs * H * dk * dv * 4);
    float* M = reinterpret_cast<float*>(w);
    w += up((size_t)segs * H * dk * dk * 4);
    int32_t* seg_cu = reinterpret_cast<int32_t*>(w);

    hipLaunchKernelGGL(longseq::plan_kernel, dim3((segs + 1 + 255) / 256), dim3(256), 0, s,
                       p.cu_seqlens, p.n_seqs, P, seg_cu);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    // 1. local scans of all segments and, in the same launch, their transitions alone
    ScanArgs a = p;
    a.n_seqs = segs;
    a.cu_seqlens = seg_cu;
    a.s_init = nullptr;
    a.s_final = S_loc;
    ScanArgs m = a;
    m.dv = dk;
    m.kw = nullptr;
    m.v = nullptr;
    m.o = op;
    m.s_final = M;
    // a first segment started from zero needs neither its transition nor o'
    if ((err = launch_scan_bf16_pair(a, m, p.s_init ? 0 : P, s)) != hipSuccess)
        return err;
    // 2. chain the segments (all but the last step), 3. add the carried states
    // to the outputs, 4. the last step, which writes S_final: the correction
    // reads S_init for the first segments, and S_final may be that buffer
    const int64_t stride = (int64_t)dk * dv;
    const dim3 cgrid((unsigned)(p.n_seqs * H * (dk / 32) * (dv / 32)));
    auto combine = [&](int q) {
        // S_prev: S_init (or zero) for segment 0, else the S_in slot of segment q
        const float* prev = q == 0 ? p.s_init : S_in + (int64_t)q * H * stride;
        const int64_t prev_nstride = (q == 0 ? 1 : P) * (int64_t)H * stride;
        float* next = q + 1 < P ? S_in + (int64_t)(q + 1) * H * stride : p.s_final;
        const int64_t next_nstride = (q + 1 < P ? P : 1) * (int64_t)H * stride;
#define PRISM_COMBINE(DK_, DV_)                                                                  \
        hipLaunchKernelGGL((longseq::combine_kernel<DK_, DV_>), cgrid, dim3(256), 0, s, M, S_loc,  \
                           prev, prev_nstride, H, P, q, next, next_nstride)
        if (dk == 64 && dv == 64)
            PRISM_COMBINE(64, 64);
        else if (dk == 64)
            PRISM_COMBINE(64, 128);
        else if (dv == 64)
            PRISM_COMBINE(128, 64);
        else
            PRISM_COMBINE(128, 128);
#undef PRISM_COMBINE
        return hipGetLastError();
    };
    for (int q = 0; q + 1 < P; ++q)
        if ((err = combine(q)) != hipSuccess)
            return err;
    if (T > 0) {
        // no segment is longer than ceil(T / P / 64) chunks of 64 tokens
        const int tiles = (T + P * 64 - 1) / (P * 64);
        const int groups = (tiles + longseq::kTPW - 1) / longseq::kTPW;
        const dim3 grid((unsigned)H, (unsigned)(segs * groups));
#define PRISM_CORRECT(DK_, DV_)                                                                   \
        hipLaunchKernelGGL((longseq::correct_kernel<DK_, DV_>), grid, dim3(256), 0, s, op, S_in,   \
                           p.s_init, seg_cu, P, groups, H, (uint16_t*)p.o)
        if (dk == 64 && dv == 64)
            PRISM_CORRECT(64, 64);
        else if (dk == 64)
            PRISM_CORRECT(64, 128);
        else if (dv == 64)
            PRISM_CORRECT(128, 64);
        else
            PRISM_CORRECT(128, 128);
#undef PRISM_CORRECT
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
    }
    return combine(P - 1);
}

}  // namespace prism
