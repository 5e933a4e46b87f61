// backward.hip -- gradients of PRISM's memory-writing operator (closed-form
// residual chain, or the GELU refinement chain) for the loss
// sum <dO, o> + <dS_final, S_final>.
//
// Reverse-mode differentiation of the token recurrence (WeChat ICML 2026
// PRISM summary, sections 核心迭代形式, 消除 Token 间串行 and 消除 Step 间串行;
// gist.science summary section 2.1, S_t = S_{t-1} A_t + B_t).  With
// G = dL/dS_t and, for each token from the last,
//   G += q_t dO_t^T;  dq_t = S_t dO_t;  dv_t = G^T kw_t;  dkw_t = G v_t
//   P = S_{t-1} - b k p^T, p = S_{t-1}^T k;  dg_t = <G, P>;  dP = g G
//   y = dP^T k;  db_t -= y . p;  dk_t -= b (dP p + S_{t-1} y);  G = dP - b k y^T
// and dS_init = G at the sequence start; then the write key backwards through
// the residual chain and the ShortConv taps.
//
// Design: a token-by-token form (the chunkwise form of the forward is the
// faster route; see the forward scan for its algebra).
//   * scan_bwd_kernel: one wavefront per (sequence, head, 8 value columns).
//     The columns of S and G evolve independently, so all column sums stay
//     in the wavefront (DPP and row swaps, no LDS barrier on the recurrence).
//     A first launch stores S every 4 tokens (16 at dk = 64) and, beside it,
//     runs G alone backwards to store the gradient at the ends of P segments
//     per sequence; a second walks all segments side by side: sub-chunk by
//     sub-chunk from a segment's last, the sub-chunk's states are recomputed
//     into registers from its checkpoint and walked backwards with every
//     gradient output.  A sub-chunk's inputs are fetched one sub-chunk ahead
//     with 16-byte loads and staged in LDS as fp32.  Row sums (over the 8
//     columns) go to fp32 buffer atomics into dq, dk and dkw, which the value
//     slices of a chain share.
//   * write_key_bwd_kernel: one thread per (head, channel, block of 16 tokens),
//     the level count a template parameter: the residual chain backwards (du,
//     da, dh written, dr_0 formed), then dk's write-key part (b k and the taps)
//     summed in registers and added once; db and dconv_w through atomics.
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace prism {
namespace bwd {

constexpr int kC = 16;                           // tokens of one wavefront of the write-key backward
constexpr int kWkBlock = 64;                     // tokens of one workgroup of the write-key backward
constexpr int kWkRows = 16;                      // token blocks per slab of the dconv_w reduction
constexpr int kCols = 8;                         // value columns per wavefront of the scan backward
constexpr int kMaxSeg = 8;                       // segments per sequence of the scan backward

// tokens per checkpoint of the scan backward: one sub-chunk's states stay in
// registers (4 x 16 floats per lane at dk = 128, 16 x 8 at dk = 64), few enough
// for two wavefronts per SIMD in the segment walk
__host__ __device__ constexpr int sub_len(int dk) { return dk == 128 ? 4 : 16; }

// checkpoint slot of the sub-chunk starting at token s of sequence n (unique, < T/SUB + n_seqs + 1)
template <int SUB>
__device__ __forceinline__ int64_t ckpt_slot(int s, int n) { return (int64_t)(s / SUB) + n; }

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) { return to_f32(p[i]); }

// Cross-lane sums without LDS: DPP quad permutations and row rotations within
// rows of 16 lanes, and the gfx950 row swaps (v_permlane16_swap exchanges the
// odd rows of one operand with the even rows of the other, v_permlane32_swap
// the halves) across rows; each step adds a lane's partner to it.
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float add_xor16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// sum over the four lanes of a quad (lane bits 0-1: the column pairs)
__device__ __forceinline__ float sum_quad(float x)
{
    x += dpp<0xB1>(x);                           // quad_perm [1,0,3,2]
    return x + dpp<0x4E>(x);                     // quad_perm [2,3,0,1]
}
// sum over the sixteen lanes that share lane % 4 (lane bits 2-5: the row groups)
__device__ __forceinline__ float sum_rowgroups(float x)
{
    x += dpp<0x124>(x);                          // row_ror:4
    x += dpp<0x128>(x);                          // row_ror:8
    return add_xor32(add_xor16(x));
}

// One wavefront per (sequence n, head e, 8 value columns).  The columns of S
// and of G evolve independently, so every column sum stays inside the
// wavefront.  Lane (rg, cp) = (lane >> 2, lane & 3) holds rows rg + 16 r and
// the two columns 2 cp, 2 cp + 1 of the slice.
// Two launches, MODE 0 then MODE 1.  Each sequence is cut into P segments of
// whole sub-chunks.  MODE 0 runs two roles side by side over whole sequences:
// the forward sweep that stores S at every sub-chunk start (workgroups
// [0, nw)), and the reverse sweep of G alone (G += q dO^T, G <- A_t^T G), which
// stores the gradient flowing into each segment's last state from the tokens
// after it (workgroups [nw, 2 nw), P > 1 only).  MODE 1 then walks all segments
// of every chain side by side (workgroup p nw + w: segment p), each from its
// stored G, with every gradient output.
template <typename T, int DK, int MODE>
__global__ __launch_bounds__(64) void scan_bwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ kw,
    const T* __restrict__ v, const T* __restrict__ g, const T* __restrict__ b,
    const T* __restrict__ dO, const int32_t* __restrict__ cu, int H, int DV,
    const float* __restrict__ S_init, const float* __restrict__ dS_final,
    float* __restrict__ ckpt, float* __restrict__ gbuf, int P, int nw,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dkw,
    float* __restrict__ dv, float* __restrict__ dg, float* __restrict__ db,
    float* __restrict__ dS_init)
{
    constexpr int RPT = DK / 16;                 // rows per lane
    constexpr int EL = 2 * RPT;                  // state elements per lane
    constexpr int SUB = sub_len(DK);
    // tokens staged at once: the sub-chunk in the segment walk; 16 in the two
    // sweeps of the first launch, which keep no per-token states
    constexpr int NST = MODE == 0 && SUB < 16 ? 16 : SUB;
    constexpr int VE = 16 / (int)sizeof(T);      // elements per 16-byte vector
    constexpr int KV = NST * DK / VE;            // 16-byte vectors of one [NST, DK] tile
    constexpr int KPL = KV / 64;                 // ... per lane
    constexpr int VPT = kCols / VE;              // 16-byte vectors of one token's 8 columns
    constexpr int VV = NST * VPT;                // ... of the staged tokens
    static_assert(KV % 64 == 0 && 2 * VV <= 64 && NST % SUB == 0, "staging layout");
    // the staged rows, widened to fp32 once
    __shared__ __attribute__((aligned(16))) float sK[NST * DK], sW[NST * DK], sQ[NST * DK];
    __shared__ __attribute__((aligned(16))) float sV[NST * kCols], sD[NST * kCols];
    __shared__ float sG[NST], sB[NST];

    const int lane = threadIdx.x;
    const int cp = lane & 3, rg = lane >> 2;
    const int slices = DV / kCols;
    int wid = blockIdx.x, seg = 0;
    bool grole = false;                          // MODE 0: the G sweep
    if constexpr (MODE == 0) {
        grole = wid >= nw;
        if (grole)
            wid -= nw;
    } else {
        seg = wid / nw;
        wid -= seg * nw;
    }
    const int slice = wid % slices;
    const int chain = wid / slices;
    const int n = chain / H, e = chain % H;
    const int j0 = slice * kCols + cp * 2;       // first of this lane's 2 columns
    const int seq0 = cu[n], seq1 = cu[n + 1];
    // segment width: whole sub-chunks, at least one
    const int W = max(SUB, ((seq1 - seq0 + P - 1) / P + SUB - 1) / SUB * SUB);

    float S[EL], G[EL];
    const int64_t sbase = ((int64_t)chain * DK) * DV;    // [n, e] block of S_init / dS_final
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int64_t x = sbase + (int64_t)(rg + 16 * r) * DV + j0 + c;
            S[r * 2 + c] = S_init ? S_init[x] : 0.f;
            G[r * 2 + c] = dS_final ? dS_final[x] : 0.f;
        }
    auto ckpt_at = [&](int s) {
        return ckpt + ((ckpt_slot<SUB>(s, n) * H + e) * slices + slice) * (int64_t)(EL * 64) + lane;
    };
    // gradient into the last state of segment p from the tokens after it
    auto gbuf_at = [&](int p) {
        return gbuf + ((((int64_t)n * P + p) * H + e) * slices + slice) * (int64_t)(EL * 64) + lane;
    };

    // ---- a sub-chunk's inputs, loaded a sub-chunk ahead into registers, then staged in LDS
    struct Pre {
        uint4 k[KPL], w[KPL], q[KPL], vd;
        float gb;
    };
    auto pre_load = [&](int c, bool back, Pre& P) {
        const int last = seq1 - 1;               // tokens past the sequence end read its last one
#pragma unroll
        for (int x = 0; x < KPL; ++x) {
            const int idx = lane + 64 * x;
            const int t = min(c + idx / (DK / VE), last);
            const int64_t o = ((int64_t)t * H + e) * DK / VE + idx % (DK / VE);
            P.k[x] = reinterpret_cast<const uint4*>(k)[o];
            P.w[x] = reinterpret_cast<const uint4*>(kw)[o];
            if (back)
                P.q[x] = reinterpret_cast<const uint4*>(q)[o];
        }
        const int vl = lane < VV ? lane : lane - VV;
        const int t = min(c + vl / VPT, last);
        const int64_t ov = (((int64_t)t * H + e) * DV + slice * kCols) / VE + vl % VPT;
        P.vd = make_uint4(0u, 0u, 0u, 0u);
        if (lane < VV)
            P.vd = reinterpret_cast<const uint4*>(v)[ov];
        else if (back && lane < 2 * VV)
            P.vd = reinterpret_cast<const uint4*>(dO)[ov];
        const int tg = min(c + (lane % NST), last);
        P.gb = lane < 2 * NST ? ld(lane < NST ? g : b, (int64_t)tg * H + e) : 0.f;
    };
    // 16 bytes of T at element idx * VE of dst, as fp32
    auto put = [](float* dst, int idx, const uint4& raw) {
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        float4* d4 = reinterpret_cast<float4*>(dst + idx * VE);
        if constexpr (sizeof(T) == 2) {
            d4[0] = make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u));
            d4[1] = make_float4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                                __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u));
        } else {
            d4[0] = make_float4(__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]),
                                __uint_as_float(w[3]));
        }
    };
    auto pre_store = [&](const Pre& P, bool back) {
#pragma unroll
        for (int x = 0; x < KPL; ++x) {
            put(sK, lane + 64 * x, P.k[x]);
            put(sW, lane + 64 * x, P.w[x]);
            if (back)
                put(sQ, lane + 64 * x, P.q[x]);
        }
        if (lane < VV)
            put(sV, lane, P.vd);
        else if (back && lane < 2 * VV)
            put(sD, lane - VV, P.vd);
        if (lane < NST)
            sG[lane] = P.gb;
        else if (lane < 2 * NST)
            sB[lane - NST] = P.gb;
    };
    auto at = [](const float* base, int i) { return base[i]; };

    // ---- forward token j of the staged sub-chunk: So <- g (Si - b k p^T) + kw v^T
    // (So may be Si)
    auto fapply = [&](int j, const float (&Si)[EL], float (&So)[EL]) {
        float kk[RPT], ww[RPT], vv[2];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            kk[r] = at(sK, j * DK + rg + 16 * r);
            ww[r] = at(sW, j * DK + rg + 16 * r);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c)
            vv[c] = at(sV, j * kCols + cp * 2 + c);
        const float gt = sG[j], bt = sB[j];
        float p[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < RPT; ++r)
                acc += Si[r * 2 + c] * kk[r];
            p[c] = sum_rowgroups(acc);
        }
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                So[r * 2 + c] = gt * (Si[r * 2 + c] - bt * kk[r] * p[c]) + ww[r] * vv[c];
    };

    // fp32 atomics into one token's row of dk floats: a buffer resource over the
    // row and a fixed lane offset, so no per-atomic address arithmetic
    auto row_rsrc = [&](float* base, int64_t rk) {
        return __builtin_amdgcn_make_buffer_rsrc(base + rk, 0, DK * 4, 0x00020000);
    };
    const int aoff = rg * 4;

    // ---- backward token t = c + j of the staged sub-chunk; St = S_t, Sm = S_{t-1}
    auto bapply = [&](int c0, int j, const float (&St)[EL], const float (&Sm)[EL]) {
        const int t = c0 + j;
        const int64_t rk = ((int64_t)t * H + e) * DK, rv = ((int64_t)t * H + e) * DV + j0;
        const auto rq = row_rsrc(dq, rk), rw = row_rsrc(dkw, rk), rkk = row_rsrc(dk, rk);
        float kk[RPT], qq[RPT], ww[RPT], vv[2], dd[2];
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            kk[r] = at(sK, j * DK + rg + 16 * r);
            qq[r] = at(sQ, j * DK + rg + 16 * r);
            ww[r] = at(sW, j * DK + rg + 16 * r);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            vv[c] = at(sV, j * kCols + cp * 2 + c);
            dd[c] = at(sD, j * kCols + cp * 2 + c);
        }
        const float gt = sG[j], bt = sB[j];
        // G += q dO^T; dq = S_t dO and dkw = G v over this slice's columns
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            float aq = 0.f, aw = 0.f;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                G[r * 2 + c] += qq[r] * dd[c];
                aq += St[r * 2 + c] * dd[c];
                aw += G[r * 2 + c] * vv[c];
            }
            aq = sum_quad(aq);
            aw = sum_quad(aw);
            if (cp == 0) {
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(aq, rq, aoff + 64 * r, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(aw, rw, aoff + 64 * r, 0, 0);
            }
        }
        // dv = G^T kw; p = S_{t-1}^T k (column sums over the dk rows)
        float p[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float a1 = 0.f, a2 = 0.f;
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                a1 += G[r * 2 + c] * ww[r];
                a2 += Sm[r * 2 + c] * kk[r];
            }
            a1 = sum_rowgroups(a1);
            p[c] = sum_rowgroups(a2);
            if (rg == 0)
                dv[rv + c] = a1;
        }
        // dg = <G, P>, P = S_{t-1} - b k p^T; dP = g G; y = dP^T k
        float dgp = 0.f;
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                dgp += G[r * 2 + c] * (Sm[r * 2 + c] - bt * kk[r] * p[c]);
                G[r * 2 + c] *= gt;
            }
        dgp = sum_rowgroups(sum_quad(dgp));
        float y[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            float a1 = 0.f;
#pragma unroll
            for (int r = 0; r < RPT; ++r)
                a1 += G[r * 2 + c] * kk[r];
            y[c] = sum_rowgroups(a1);
        }
        const float yp = sum_quad(y[0] * p[0] + y[1] * p[1]);
        if (lane == 0) {
            atomicAdd(dg + (int64_t)t * H + e, dgp);
            atomicAdd(db + (int64_t)t * H + e, -yp);   // db -= y . p
        }
        // dk -= b (dP p + S_{t-1} y); G = dP - b k y^T
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            float a1 = 0.f;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                a1 += G[r * 2 + c] * p[c] + Sm[r * 2 + c] * y[c];
                G[r * 2 + c] -= bt * kk[r] * y[c];
            }
            a1 = sum_quad(a1);
            if (cp == 0)
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(-bt * a1, rkk, aoff + 64 * r, 0, 0);
        }
    };

    Pre P_;
    if constexpr (MODE == 0) {
        if (!grole) {
            // S at every sub-chunk start, into the checkpoints
            const int nst = (seq1 - seq0 + NST - 1) / NST;
            if (nst > 0)
                pre_load(seq0, false, P_);
            for (int m = 0; m < nst; ++m) {
                const int c0 = seq0 + m * NST, len = min(NST, seq1 - c0);
                lds_barrier();                   // the previous tokens' LDS reads are done
                pre_store(P_, false);
                lds_barrier();
                if (m + 1 < nst)
                    pre_load(c0 + NST, false, P_);
#pragma unroll
                for (int j = 0; j < NST; ++j) {
                    if (j < len) {
                        if (j % SUB == 0) {      // a sub-chunk start: checkpoint
                            float* cpt = ckpt_at(c0 + j);
#pragma unroll
                            for (int x = 0; x < EL; ++x)
                                cpt[x * 64] = S[x];
                        }
                        fapply(j, S, S);
                    }
                }
            }
            return;
        }
        // the G sweep: per token from the last, G += q dO^T, then G <- g (G - b k (G^T k)^T);
        // after a segment's first token t the result is the gradient into S_{t-1}
        auto gstep = [&](int j) {
            float kk[RPT], qq[RPT], dd[2];
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                kk[r] = at(sK, j * DK + rg + 16 * r);
                qq[r] = at(sQ, j * DK + rg + 16 * r);
            }
#pragma unroll
            for (int c = 0; c < 2; ++c)
                dd[c] = at(sD, j * kCols + cp * 2 + c);
            const float gt = sG[j], bt = sB[j];
            float y[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                float acc = 0.f;
#pragma unroll
                for (int r = 0; r < RPT; ++r) {
                    G[r * 2 + c] += qq[r] * dd[c];
                    acc += G[r * 2 + c] * kk[r];
                }
                y[c] = sum_rowgroups(acc);
            }
#pragma unroll
            for (int r = 0; r < RPT; ++r)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    G[r * 2 + c] = gt * (G[r * 2 + c] - bt * kk[r] * y[c]);
        };
        const int nst = (seq1 - seq0 + NST - 1) / NST;
        if (nst > 0)
            pre_load(seq0 + (nst - 1) * NST, true, P_);
        for (int m = nst - 1; m >= 0; --m) {
            const int c0 = seq0 + m * NST, len = min(NST, seq1 - c0);
            lds_barrier();
            pre_store(P_, true);
            lds_barrier();
            if (m > 0)
                pre_load(c0 - NST, true, P_);
#pragma unroll
            for (int j = NST - 1; j >= 0; --j) {
                if (j < len) {
                    gstep(j);
                    const int off = c0 + j - seq0;
                    if (off > 0 && off % W == 0) {
                        float* gp = gbuf_at(off / W - 1);
#pragma unroll
                        for (int x = 0; x < EL; ++x)
                            gp[x * 64] = G[x];
                    }
                }
            }
        }
        return;
    }

    // MODE 1: segment seg of the sequence, sub-chunk by sub-chunk from its last;
    // each sub-chunk's states recomputed into registers from its checkpoint,
    // then walked backwards
    const int a0 = seq0 + seg * W, a1 = min(seq1, a0 + W);
    if (a0 < seq1 && a1 < seq1) {                // not the last segment: G from the G sweep
        const float* gp = gbuf_at(seg);
#pragma unroll
        for (int x = 0; x < EL; ++x)
            G[x] = gp[x * 64];
    }
    const int m_lo = (a0 - seq0) / SUB, m_hi = a0 < seq1 ? (a1 - seq0 + SUB - 1) / SUB : m_lo;
    float Cn[EL];
    if (m_hi > m_lo) {
        pre_load(seq0 + (m_hi - 1) * SUB, true, P_);
        const float* cpt = ckpt_at(seq0 + (m_hi - 1) * SUB);
#pragma unroll
        for (int x = 0; x < EL; ++x)
            Cn[x] = cpt[x * 64];
    }
    for (int m = m_hi - 1; m >= m_lo; --m) {
        const int c0 = seq0 + m * SUB, len = min(SUB, seq1 - c0);
        lds_barrier();
        pre_store(P_, true);
        lds_barrier();
        float Ss[SUB + 1][EL];                   // Ss[j] = S before token c0 + j
#pragma unroll
        for (int x = 0; x < EL; ++x)
            Ss[0][x] = Cn[x];
        if (m > m_lo) {
            pre_load(c0 - SUB, true, P_);
            const float* cpt = ckpt_at(c0 - SUB);
#pragma unroll
            for (int x = 0; x < EL; ++x)
                Cn[x] = cpt[x * 64];
        }
#pragma unroll
        for (int j = 0; j < SUB; ++j)
            if (j < len)
                fapply(j, Ss[j], Ss[j + 1]);
#pragma unroll
        for (int j = SUB - 1; j >= 0; --j)
            if (j < len)
                bapply(c0, j, Ss[j + 1], Ss[j]);
    }
    if (seg == 0 && dS_init) {                   // G is now the gradient of the start state
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c)
                dS_init[sbase + (int64_t)(rg + 16 * r) * DV + j0 + c] = G[r * 2 + c];
    }
}

// The write key backwards.  One workgroup per (block of 64 tokens, head, 64
// channels): lane = channel, wavefront w = the block's tokens 16 w .. 16 w + 15.
// dkw (fp32) comes from the scan backward.  Each wavefront also runs the chain
// backward for the three tokens after its own, so every contribution to dk of
// its tokens (b k and the four taps of the tokens that read them) is summed in
// registers and added to dk, which already holds the scan's part, with one
// read-modify-write: no other wavefront touches those elements.  The keys of
// the taps slide through registers (one load per token), the next token's
// loads are issued before this token's arithmetic (the token loop is unrolled
// and every load is bounded, so the code is straight-line), db takes one
// atomic per (token, head, 64 channels), and the taps' gradients are summed
// over the workgroup and stored per token block (reduced by wk_reduce_kernel:
// no atomics on the 4 x H x dk weights).
template <typename T, int L>
struct WkTok {
    float gkw, kt, bt;
    float a[L > 1 ? L - 1 : 1], u[L > 1 ? L - 1 : 1], h[L > 1 ? L - 1 : 1];
};

// One element through a bounded buffer resource (zero outside its range).
__device__ __forceinline__ float bld(__amdgpu_buffer_rsrc_t r, int i, const uint16_t*)
{
    return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, i * 2, 0, 0));
}
__device__ __forceinline__ float bld(__amdgpu_buffer_rsrc_t r, int i, const float*)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, i * 4, 0, 0));
}

// Buffer resources over the rows [rb, re) of the tensors a wavefront reads:
// element offsets relative to row rb; rows outside the range read as zero, so
// no load needs a branch.
template <typename T>
struct WkSrc {
    __amdgpu_buffer_rsrc_t k, u, a, h, b, dkw, dk;
};

template <typename T, int L>
__device__ __forceinline__ void wk_load(WkTok<T, L>& x, const WkSrc<T>& r, int tr, int H, int DK, int e, int i)
{
    const int rk = (tr * H + e) * DK + i;
    x.gkw = bld(r.dkw, rk, (const float*)nullptr);
    x.kt = bld(r.k, rk, (const T*)nullptr);
    x.bt = bld(r.b, tr * H + e, (const T*)nullptr);
    if constexpr (L > 1) {
        const int lb = (tr * H + e) * (L - 1) * DK + i;
#pragma unroll
        for (int l = 0; l < L - 1; ++l) {
            x.a[l] = bld(r.a, lb + l * DK, (const T*)nullptr);
            x.u[l] = bld(r.u, lb + l * DK, (const T*)nullptr);
            x.h[l] = bld(r.h, lb + l * DK, (const T*)nullptr);
        }
    }
}

// G: the storage type of dk, du, da, dh (fp32, or bf16 rounded to nearest even
// from the same fp32 values).  dk_in holds the scan's part of dk in fp32; it is
// dk itself when G is fp32 (hence no __restrict__ on either).
template <typename T, int L, typename G>
__global__ __launch_bounds__(256) void write_key_bwd_kernel(
    const T* __restrict__ k, const T* __restrict__ u, const T* __restrict__ a,
    const T* __restrict__ h, const T* __restrict__ b, const T* __restrict__ conv_w,
    const int32_t* __restrict__ cu, int n_seqs, int T_total, int H, int DK, bool gelu,
    const float* __restrict__ dkw, const float* dk_in, G* dk, G* __restrict__ du,
    G* __restrict__ da, G* __restrict__ dh, float* __restrict__ db,
    float* __restrict__ dconv_part)
{
    constexpr int NIT = kC + 3;                  // own tokens and the three after them
    __shared__ float4 red[4][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ng = DK / 64;
    const int cg = blockIdx.x % ng, e = (blockIdx.x / ng) % H;
    const int tb = blockIdx.x / (ng * H);
    const int i = cg * 64 + lane;
    const int t_lo = tb * kWkBlock + wave * kC;
    const int t_hi = min(T_total, t_lo + kC);
    float w[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        w[m] = ld(conv_w, ((int64_t)e * DK + i) * 4 + m);
    float dw[4] = {0.f, 0.f, 0.f, 0.f};
    if (t_lo < T_total) {
        // sequence bounds of token t_lo - 3 + j in lane j (a token outside [0, T)
        // gets the end -1, which matches no token's)
        int sq0 = 0, sq1 = -1;
        {
            const int tt = t_lo - 3 + lane;
            if (lane < NIT + 3 && tt >= 0 && tt < T_total) {
                int lo = 0, hi = n_seqs;             // largest n with cu[n] <= tt
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (cu[mid] <= tt) lo = mid; else hi = mid;
                }
                sq0 = cu[lo];
                sq1 = cu[lo + 1];
            }
        }
        const int rb = max(0, t_lo - 3), re = min(T_total, t_lo + NIT);
        const int nr = re - rb;
        const int64_t rowK = (int64_t)H * DK, rowL = rowK * (L > 1 ? L - 1 : 1);
        auto mk = [](const void* p, int64_t bytes) {
            return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
        };
        WkSrc<T> r;
        r.k = mk(k + rb * rowK, nr * rowK * sizeof(T));
        r.dkw = mk(dkw + rb * rowK, nr * rowK * 4);
        r.dk = mk(dk_in + rb * rowK, nr * rowK * 4);
        r.b = mk(b + (int64_t)rb * H, (int64_t)nr * H * sizeof(T));
        if constexpr (L > 1) {
            r.u = mk(u + rb * rowL, nr * rowL * sizeof(T));
            r.a = mk(a + rb * rowL, nr * rowL * sizeof(T));
            r.h = mk(h + rb * rowL, nr * rowL * sizeof(T));
        }
        const int t0r = t_lo - rb;               // row of t_lo in the ranges
        // keys of tokens t-3 .. t (raw: the sequence start masks them per token)
        float kwin[4];
#pragma unroll
        for (int m = 0; m < 3; ++m)
            kwin[m + 1] = bld(r.k, (t0r - 3 + m) * (int)rowK + e * DK + i, (const T*)nullptr);
        // dr_0 of tokens t-3 .. t with the end of the sequence each belongs to, and
        // the dkw and b of those tokens (dk of token t-3 is completed at token t)
        float dr[4] = {0.f, 0.f, 0.f, 0.f}, gh[4] = {0.f, 0.f, 0.f, 0.f}, bh[4] = {0.f, 0.f, 0.f, 0.f};
        int se[4] = {-1, -1, -1, -1};
        // the next two tokens' loads in flight while a token is computed (up to
        // L = 4: beyond, the second set of registers costs more occupancy than it hides)
        constexpr int AHEAD = L <= 4 ? 2 : 1;
        WkTok<T, L> nx, nx2;
        wk_load<T, L>(nx, r, t0r, H, DK, e, i);
        if constexpr (AHEAD == 2)
            wk_load<T, L>(nx2, r, t0r + 1, H, DK, e, i);
        // fully unrolled: straight-line code, so every wait counts exactly the
        // loads it needs (a loop would wait for all of them at its head)
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int t = t_lo + it;
#pragma unroll
            for (int x = 0; x < 3; ++x) {
                dr[x] = dr[x + 1];
                se[x] = se[x + 1];
                gh[x] = gh[x + 1];
                bh[x] = bh[x + 1];
                kwin[x] = kwin[x + 1];
            }
            const int tau = t - 3;
            float dk_old = 0.f;
            if (it >= 3)
                dk_old = bld(r.dk, (tau - rb) * (int)rowK + e * DK + i, (const float*)nullptr);
            const WkTok<T, L> cur = nx;
            if constexpr (AHEAD == 2) {
                nx = nx2;
                if (it + 2 < NIT)
                    wk_load<T, L>(nx2, r, t0r + it + 2, H, DK, e, i);
            } else if (it + 1 < NIT) {
                wk_load<T, L>(nx, r, t0r + it + 1, H, DK, e, i);
            }
            const int s0 = __builtin_amdgcn_readlane(sq0, it + 3);
            se[3] = __builtin_amdgcn_readlane(sq1, it + 3);
            gh[3] = cur.gkw;
            bh[3] = cur.bt;
            kwin[3] = cur.kt;
            const bool own = t < t_hi;
            if (own) {                           // db from the b k part of the key: one
                float dbp = cur.gkw * cur.kt;     // atomic per wavefront (64 channels)
                for (int o = 32; o > 0; o >>= 1)
                    dbp += __shfl_xor(dbp, o);
                if (lane == 0)
                    atomicAdd(db + (int64_t)t * H + e, dbp);
            }
            dr[3] = 0.f;
            if constexpr (L > 1) {
                float kx[4];
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    kx[m] = t - 3 + m >= s0 ? kwin[m] : 0.f;
                const float r0 = w[0] * kx[0] + w[1] * kx[1] + w[2] * kx[2] + w[3] * kx[3];
                // residuals r_l, l = 1 .. L-1 (the closed form as a running product, or
                // the GELU refinement chain)
                float rr[L];
                rr[1] = r0;
#pragma unroll
                for (int l = 1; l < L - 1; ++l) {
                    const float al = cur.a[l - 1], hl = cur.h[l - 1];
                    rr[l + 1] = gelu ? rr[l] - al * gelu_as(hl * rr[l]) : rr[l] * (1.f - al * hl);
                }
                float dr_next = 0.f;
                const int64_t lb = ((int64_t)t * H + e) * (L - 1) * DK + i;
#pragma unroll
                for (int l = L - 1; l >= 1; --l) {
                    const float al = cur.a[l - 1], ul = cur.u[l - 1], hl = cur.h[l - 1];
                    const float g_kw = cur.gkw;
                    float dal = g_kw * ul * rr[l], dhl = 0.f, drl = g_kw * al * ul;
                    if (l <= L - 2) {
                        if (gelu) {              // r_{l+1} = r_l - a_l GELU(h_l r_l)
                            float gp;
                            const float gv = gelu_as_grad(hl * rr[l], gp);
                            dal -= dr_next * gv;
                            dhl = -dr_next * al * rr[l] * gp;
                            drl += dr_next * (1.f - al * hl * gp);
                        } else {                 // r_{l+1} = r_l (1 - a_l h_l)
                            dal -= dr_next * hl * rr[l];
                            dhl = -dr_next * al * rr[l];
                            drl += dr_next * (1.f - al * hl);
                        }
                    }
                    if (own) {
                        const int64_t sl = lb + (int64_t)(l - 1) * DK;
                        du[sl] = from_f32<G>(g_kw * al * rr[l]);
                        da[sl] = from_f32<G>(dal);
                        dh[sl] = from_f32<G>(dhl);
                    }
                    dr_next = drl;
                }
                dr[3] = dr_next;                 // dr_0 of token t
                if (own) {                       // the taps: dw_m += dr_0 k_{t-3+m}
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        dw[m] += dr_next * kx[m];
                }
            }
            // dk of token tau = t - 3: b dkw, and w_{3-d} dr_0 of token tau + d in its sequence
            if (it >= 3 && tau < t_hi) {
                float acc = bh[0] * gh[0] + w[3] * dr[0];
#pragma unroll
                for (int dd = 1; dd < 4; ++dd)
                    if (se[dd] == se[0])
                        acc += w[3 - dd] * dr[dd];
                dk[((int64_t)tau * H + e) * DK + i] = from_f32<G>(dk_old + acc);
            }
        }
    }
    red[wave][lane] = make_float4(dw[0], dw[1], dw[2], dw[3]);
    __syncthreads();
    if (wave == 0) {
        float4 sum = red[0][lane];
#pragma unroll
        for (int x = 1; x < 4; ++x) {
            const float4 y = red[x][lane];
            sum.x += y.x; sum.y += y.y; sum.z += y.z; sum.w += y.w;
        }
        *reinterpret_cast<float4*>(dconv_part + (((int64_t)tb * H + e) * DK + i) * 4) = sum;
    }
}

// dconv_w = the sum over token blocks of the per-block partials [nb][n], in two
// passes: slabs of kWkRows blocks into [slabs][n], then the slabs (rows = nb)
__global__ __launch_bounds__(256) void wk_reduce_kernel(const float* __restrict__ part, int nb, int n,
                                                        int rows, float* __restrict__ out)
{
    const int o = blockIdx.x * 256 + threadIdx.x;
    const int s = blockIdx.y;
    if (o >= n)
        return;
    const int b0 = s * rows, b1 = min(nb, b0 + rows);
    float acc = 0.f;
#pragma unroll 8
    for (int bb = b0; bb < b1; ++bb)
        acc += part[(int64_t)bb * n + o];
    out[(int64_t)s * n + o] = acc;
}

__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ p, int64_t n)
{
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256)
        p[x] = 0.f;
}

}  // namespace bwd

size_t wk_workspace_floats(int total_tokens, int heads, int dk)
{
    const int64_t nb = (total_tokens + bwd::kWkBlock - 1) / bwd::kWkBlock;
    const int64_t slabs = (nb + bwd::kWkRows - 1) / bwd::kWkRows;
    return (size_t)((nb + slabs) * heads * dk * 4);
}

size_t bwd_workspace_floats(int n_seqs, int total_tokens, int heads, int dk, int dv)
{
    const int64_t slots = total_tokens / bwd::sub_len(dk) + n_seqs + 1;
    return (size_t)(slots * heads * dk * dv)                      // sub-chunk start states
         + (size_t)n_seqs * bwd::kMaxSeg * heads * dk * dv        // segment-boundary gradients
         + (size_t)total_tokens * heads * dk                      // dkw
         + wk_workspace_floats(total_tokens, heads, dk);          // dconv_w partials
}

// Segments per sequence for the scan backward.  The segment walk holds two
// wavefronts per SIMD (2048 on the chip): with at least that many (chain,
// value slice) wavefronts one segment is best; below it, kMaxSeg short
// segments (measured at the LM layer, 768 wavefronts: 4.0 ms at P = 8, 4.1 at
// 5, 4.2 at 4, 4.5 at 2, 5.7 at 1; at the recommendation workload, 2048
// wavefronts: 2.9 ms at P = 1, 3.1 at 2 to 8).  PRISM_BWD_SEGMENTS=P forces P.
int bwd_segments(int n_seqs, int heads, int dv)
{
    const char* env = getenv("PRISM_BWD_SEGMENTS");
    if (env && *env) {
        const int f = atoi(env);
        if (f >= 1 && f <= bwd::kMaxSeg)
            return f;
    }
    const int64_t nw = (int64_t)n_seqs * heads * (dv / bwd::kCols);
    return nw >= 2048 ? 1 : bwd::kMaxSeg;
}

bool bwd_supported(int dk, int dv) { return (dk == 64 || dk == 128) && (dv == 64 || dv == 128); }

template <typename T, int L, typename G>
static void launch_wk_kernel(const BwdArgs& p, const float* dkw, float* part, int64_t nb, hipStream_t s)
{
    // with bf16 gradients gk, gu, ga, gh hold bf16 and the scan's fp32 part of dk
    // is in gk_part; otherwise gk holds that part on entry
    const float* dk_in = p.grad_bf16 ? p.gk_part : p.gk;
    hipLaunchKernelGGL((bwd::write_key_bwd_kernel<T, L, G>), dim3((unsigned)(nb * p.heads * (p.dk / 64))),
                       dim3(256), 0, s, (const T*)p.k, (const T*)p.u, (const T*)p.a, (const T*)p.h,
                       (const T*)p.b, (const T*)p.conv_w, p.cu_seqlens, p.n_seqs, p.total_tokens,
                       p.heads, p.dk, p.gelu, dkw, dk_in, reinterpret_cast<G*>(p.gk),
                       reinterpret_cast<G*>(p.gu), reinterpret_cast<G*>(p.ga), reinterpret_cast<G*>(p.gh),
                       p.gb, part);
}

template <typename T, int L>
static hipError_t launch_wk_L(const BwdArgs& p, const float* dkw, float* part, hipStream_t s)
{
    const int64_t nb = (p.total_tokens + bwd::kWkBlock - 1) / bwd::kWkBlock;
    const int n = p.heads * p.dk * 4;
    if (nb > 0) {
        if (p.grad_bf16)
            launch_wk_kernel<T, L, uint16_t>(p, dkw, part, nb, s);
        else
            launch_wk_kernel<T, L, float>(p, dkw, part, nb, s);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || n == 0)
        return err;
    // the partials [nb][n] -> slabs [ns][n] -> dconv_w (every element written)
    const int ns = (int)((nb + bwd::kWkRows - 1) / bwd::kWkRows);
    float* slabs = part + nb * n;
    const unsigned gx = (unsigned)((n + 255) / 256);
    if (ns > 0) {
        hipLaunchKernelGGL(bwd::wk_reduce_kernel, dim3(gx, (unsigned)ns), dim3(256), 0, s, part, (int)nb, n,
                           bwd::kWkRows, slabs);
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
    }
    hipLaunchKernelGGL(bwd::wk_reduce_kernel, dim3(gx, 1), dim3(256), 0, s, slabs, ns, n, ns, p.gconv);
    return hipGetLastError();
}

// The level count as a template parameter: the chain loops unroll and each
// token's loads issue together.
template <typename T>
static hipError_t launch_wk(const BwdArgs& p, const float* dkw, float* part, hipStream_t s)
{
    switch (p.L) {
    case 1: return launch_wk_L<T, 1>(p, dkw, part, s);
    case 2: return launch_wk_L<T, 2>(p, dkw, part, s);
    case 3: return launch_wk_L<T, 3>(p, dkw, part, s);
    case 4: return launch_wk_L<T, 4>(p, dkw, part, s);
    case 5: return launch_wk_L<T, 5>(p, dkw, part, s);
    case 6: return launch_wk_L<T, 6>(p, dkw, part, s);
    case 7: return launch_wk_L<T, 7>(p, dkw, part, s);
    case 8: return launch_wk_L<T, 8>(p, dkw, part, s);
    case 9: return launch_wk_L<T, 9>(p, dkw, part, s);
    case 10: return launch_wk_L<T, 10>(p, dkw, part, s);
    case 11: return launch_wk_L<T, 11>(p, dkw, part, s);
    case 12: return launch_wk_L<T, 12>(p, dkw, part, s);
    case 13: return launch_wk_L<T, 13>(p, dkw, part, s);
    case 14: return launch_wk_L<T, 14>(p, dkw, part, s);
    case 15: return launch_wk_L<T, 15>(p, dkw, part, s);
    case 16: return launch_wk_L<T, 16>(p, dkw, part, s);
    default: return hipErrorInvalidValue;
    }
}

template <typename T, int DK>
static hipError_t launch_bwd_T(const BwdArgs& p, hipStream_t s)
{
    const int H = p.heads, T_ = p.total_tokens;
    const int64_t slots = T_ / bwd::sub_len(DK) + p.n_seqs + 1;
    float* ckpt = p.ws;
    float* gbuf = ckpt + slots * H * DK * p.dv;
    float* dkw = gbuf + (int64_t)p.n_seqs * bwd::kMaxSeg * H * DK * p.dv;
    const int64_t wgs = (int64_t)p.n_seqs * H * (p.dv / bwd::kCols);
    const int P = bwd_segments(p.n_seqs, H, p.dv);
    // accumulators start at zero (a fill kernel: no memset node under graph capture)
    auto zero = [&](float* x, int64_t n) {
        if (n > 0)
            hipLaunchKernelGGL(bwd::zero_kernel, dim3((unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)),
                               dim3(256), 0, s, x, n);
    };
    zero(p.gq, (int64_t)T_ * H * DK);
    zero(p.gk, (int64_t)T_ * H * DK);
    zero(dkw, (int64_t)T_ * H * DK);
    zero(p.gg, (int64_t)T_ * H);
    zero(p.gb, (int64_t)T_ * H);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    if (wgs == 0)
        return launch_wk<T>(p, dkw, dkw + (int64_t)T_ * H * DK, s);
    // checkpoints and (P > 1) the segment-boundary gradients, then the segments
    hipLaunchKernelGGL((bwd::scan_bwd_kernel<T, DK, 0>), dim3((unsigned)(wgs * (P > 1 ? 2 : 1))),
                       dim3(64), 0, s, (const T*)p.q, (const T*)p.k, (const T*)p.kw,
                       (const T*)p.v, (const T*)p.g, (const T*)p.b, (const T*)p.dO, p.cu_seqlens,
                       H, p.dv, p.s_init, p.ds_final, ckpt, gbuf, P, (int)wgs, p.gq, p.gk, dkw,
                       p.gv, p.gg, p.gb, p.gs_init);
    if ((err = hipGetLastError()) != hipSuccess)
        return err;
    hipLaunchKernelGGL((bwd::scan_bwd_kernel<T, DK, 1>), dim3((unsigned)(wgs * P)), dim3(64), 0, s,
                       (const T*)p.q, (const T*)p.k, (const T*)p.kw, (const T*)p.v,
                       (const T*)p.g, (const T*)p.b, (const T*)p.dO, p.cu_seqlens, H, p.dv,
                       p.s_init, p.ds_final, ckpt, gbuf, P, (int)wgs, p.gq, p.gk, dkw, p.gv,
                       p.gg, p.gb, p.gs_init);
    if ((err = hipGetLastError()) != hipSuccess)
        return err;
    return launch_wk<T>(p, dkw, dkw + (int64_t)T_ * H * DK, s);
}

hipError_t launch_write_key_bwd(const BwdArgs& p, const float* dkw, float* part, hipStream_t s)
{
    if (!bwd_supported(p.dk, p.dv) || p.L < 1 || p.L > 16 || (p.grad_bf16 && (!p.bf16 || !p.gk_part)))
        return hipErrorInvalidValue;
    return p.bf16 ? launch_wk<uint16_t>(p, dkw, part, s) : launch_wk<float>(p, dkw, part, s);
}

hipError_t launch_bwd(const BwdArgs& p, hipStream_t s)
{
    if (!bwd_supported(p.dk, p.dv) || p.L < 1 || p.L > 16)
        return hipErrorInvalidValue;
    if (p.bf16)
        return p.dk == 64 ? launch_bwd_T<uint16_t, 64>(p, s) : launch_bwd_T<uint16_t, 128>(p, s);
    return p.dk == 64 ? launch_bwd_T<float, 64>(p, s) : launch_bwd_T<float, 128>(p, s);
}

}  // namespace prism
