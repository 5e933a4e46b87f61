// scan_f32_recurrent.hip -- fp32 scan at dk = 128, token by token
//
// The recurrence itself, one token at a time, in fp32:
//
//   p   = S^T k_t
//   S  <- g_t (S - b_t k_t p^T) + kw_t v_t^T        (= g_t (I - b_t k_t k_t^T) S + kw_t v_t^T)
//   o_t = S^T q_t
//
// (PRISM pages: WeChat ICML 2026 summary, section 消除 Token 间串行 -- the
// forget/erase term is the Gated DeltaNet one and the write is kw_t v_t^T;
// gist.science summary of arXiv 2602.10796, section 2.1 -- S_t = S_{t-1} A_t
// + B_t.)  This serves fp32 inputs at dk = 128, where the chunkwise fp32 form
// needs 64-row fp32 tiles of q, k and kw plus five 64x64 fp32 matrices, more
// than the 160 KB of LDS of a compute unit; fp32 exists for the strict
// tolerance, so the exact token order of the recurrence is kept here.
//
// Mapping: one wavefront per (sequence, head, 8 value columns), four per
// workgroup (32 columns).  Lane (c, r) = (lane / 8, lane % 8) holds rows
// r * D/8 .. r * D/8 + D/8 - 1 of value column c in registers; the column sums
// p and o are finished across the eight lanes of a column with three xor
// shuffles, so the recurrence needs no LDS and no barrier.  The next token's
// rows are loaded while the current token is processed.
#include "common.h"
#include "kernels.h"

namespace prism {
namespace f32rec {

constexpr int kWaves = 4;
constexpr int kCols = 8 * kWaves;                // value columns per workgroup

template <int D>
struct Rows {
    float k[D / 8], q[D / 8], w[D / 8];
    float v, g, b;
};

template <int D>
__device__ __forceinline__ void load_rows(Rows<D>& r, const float* q, const float* k,
                                          const float* kw, const float* v, const float* g,
                                          const float* b, int64_t t, int e, int H, int DV, int j,
                                          int i0)
{
    constexpr int R = D / 8;
    const int64_t rq = (t * H + e) * D + i0;
#pragma unroll
    for (int x = 0; x < R; x += 4) {
        const float4 a = *reinterpret_cast<const float4*>(k + rq + x);
        const float4 c = *reinterpret_cast<const float4*>(q + rq + x);
        const float4 w = *reinterpret_cast<const float4*>(kw + rq + x);
        r.k[x] = a.x; r.k[x + 1] = a.y; r.k[x + 2] = a.z; r.k[x + 3] = a.w;
        r.q[x] = c.x; r.q[x + 1] = c.y; r.q[x + 2] = c.z; r.q[x + 3] = c.w;
        r.w[x] = w.x; r.w[x + 1] = w.y; r.w[x + 2] = w.z; r.w[x + 3] = w.w;
    }
    r.v = v[(t * H + e) * DV + j];
    r.g = g[t * H + e];
    r.b = b[t * H + e];
}

// Sum over the eight lanes of a value column (lane % 8 = row group).
__device__ __forceinline__ float col_sum(float x)
{
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    return x;
}

template <int D>
__global__ __launch_bounds__(64 * kWaves) void scan_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ kw,
    const float* __restrict__ v, const float* __restrict__ g, const float* __restrict__ b,
    const int32_t* __restrict__ cu, int H, int DV, int n_groups, const float* __restrict__ s_init,
    float* __restrict__ o, float* __restrict__ s_final)
{
    constexpr int R = D / 8;                     // rows per lane
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int grp = (int)(blockIdx.x % (unsigned)n_groups);
    const int chain = (int)(blockIdx.x / (unsigned)n_groups);
    const int n = chain / H, e = chain % H;
    const int c = lane >> 3, rg = lane & 7;
    const int j = grp * kCols + wave * 8 + c;    // value column
    const int i0 = rg * R;                       // first row of this lane
    const int seq0 = cu[n], seq1 = cu[n + 1];

    float S[R];
    const int64_t sbase = (((int64_t)n * H + e) * D + i0) * DV + j;
#pragma unroll
    for (int r = 0; r < R; ++r)
        S[r] = s_init ? s_init[sbase + (int64_t)r * DV] : 0.f;

    Rows<D> cur, nxt;
    if (seq0 < seq1)
        load_rows<D>(cur, q, k, kw, v, g, b, seq0, e, H, DV, j, i0);
    for (int t = seq0; t < seq1; ++t) {
        if (t + 1 < seq1)
            load_rows<D>(nxt, q, k, kw, v, g, b, t + 1, e, H, DV, j, i0);
        float p = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r)
            p = fmaf(S[r], cur.k[r], p);
        p = col_sum(p);
        const float bp = cur.b * p;
#pragma unroll
        for (int r = 0; r < R; ++r)
            S[r] = cur.g * (S[r] - cur.k[r] * bp) + cur.w[r] * cur.v;
        float y = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r)
            y = fmaf(S[r], cur.q[r], y);
        y = col_sum(y);
        if (rg == 0)
            o[((int64_t)t * H + e) * DV + j] = y;
        cur = nxt;
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
        s_final[sbase + (int64_t)r * DV] = S[r];
}

}  // namespace f32rec

bool scan_f32_recurrent_supported(int dk, int dv)
{
    return (dk == 64 || dk == 128) && dv % f32rec::kCols == 0 && dv > 0;
}

hipError_t launch_scan_f32_recurrent(const ScanArgs& p, hipStream_t stream)
{
    if (p.bf16 || !scan_f32_recurrent_supported(p.dk, p.dv))
        return hipErrorInvalidValue;
    const int n_groups = p.dv / f32rec::kCols;
    const int64_t blocks = (int64_t)p.n_seqs * p.heads * n_groups;
    if (blocks == 0)
        return hipSuccess;
    auto kern = p.dk == 64 ? f32rec::scan_kernel<64> : f32rec::scan_kernel<128>;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * f32rec::kWaves), 0, stream,
                       (const float*)p.q, (const float*)p.k, (const float*)p.kw, (const float*)p.v,
                       (const float*)p.g, (const float*)p.b, p.cu_seqlens, p.heads, p.dv, n_groups,
                       p.s_init, (float*)p.o, p.s_final);
    return hipGetLastError();
}

}  // namespace prism
