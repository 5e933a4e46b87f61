// prologue_kernel.h -- fused write-key prologue of PRISM's memory-writing
// operator: the kernel template and its launch dispatch, instantiated once per
// input type (prologue_bf16.hip, prologue_f32.hip) so the two compile in
// parallel.
//
// For every token t and head e (all channels i independent):
//   r_0  = sum_{m=0..3} w[e,i,m] * k[t-3+m]     causal depthwise ShortConv, width 4,
//                                               taps before the sequence start read 0
//   r_1  = r_0,  r_{l+1} = r_l * (1 - a_l h_l)  closed-form residual chain
//   kw   = b_t k_t + sum_{l=1..L-1} a_l r_l u_l
// PRISM pages: WeChat ICML 2026 summary, sections 消除 Token 间串行 (ShortConv
// anchor) and 消除 Step 间串行 (residual chain linearised to an element-wise
// recurrence with a closed form); gist.science summary of arXiv 2602.10796,
// section 2.2 (anchor, then refinement levels l = 1..L, r^(1) = anchor).
//
// Design (HBM-bound streaming, ~0.5 flop/byte):
//   * one thread owns 16 (or 8) bytes of channels of one head and walks a
//     strip of consecutive tokens, so the 3-token conv halo lives in registers
//     and every k element is read from HBM once (plus a 3-token halo per
//     strip);
//   * consecutive threads own consecutive channel groups, so every wavefront
//     load instruction covers whole 256-byte rows of k, u, a, h;
//   * k, u, a, h are streamed with nontemporal loads (read exactly once);
//     the write keys are stored normally because the scan reads them next;
//   * L and the strip length are template parameters: the level loop and the
//     token loop unroll completely, h's last slot (never read by the closed
//     form) is never loaded, and the inputs of token t + 1 are loaded while
//     token t is computed (two register sets, alternating);
//   * sequence boundaries come from cu_seqlens on the device (binary search
//     once per strip, then a forward walk that marks the sequence starts in
//     the strip), so no host synchronisation and no reads inside the loop;
//   * a carried history (HIST: the three k rows before each sequence's first
//     token, from an earlier piece of the same sequences) replaces the zero
//     taps before a sequence start; it is read only where a sequence starts;
//   * GELU: the non-linear refinement chain r_{l+1} = r_l - a_l GELU(h_l r_l)
//     (gist.science summary, section 2.2: delta = GELU(gain * residual)) in
//     place of the closed form (gelu_as in common.h).  It changes nothing for
//     L <= 2, which take the closed-form kernels.
#pragma once
#include "common.h"
#include "kernels.h"

namespace prism {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// Raw 8- or 16-byte loads; the streaming form carries the nontemporal hint
// (inputs read exactly once should not displace cached lines).
template <int B, bool NT> struct Raw;
template <bool NT> struct Raw<16, NT> {
    using V = u32x4_t;
    __device__ static V ld(const void* p)
    {
        const V* q = reinterpret_cast<const V*>(p);
        if constexpr (NT) return __builtin_nontemporal_load(q);
        else return *q;
    }
};
template <bool NT> struct Raw<8, NT> {
    using V = u32x2_t;
    __device__ static V ld(const void* p)
    {
        const V* q = reinterpret_cast<const V*>(p);
        if constexpr (NT) return __builtin_nontemporal_load(q);
        else return *q;
    }
};

// N elements of T (8 or 16 bytes) <-> fp32.
template <typename T, int N> struct Lane {
    static constexpr int B = N * (int)sizeof(T);
    template <bool NT = false>
    __device__ static void load(const T* p, float* out)
    {
        auto v = Raw<B, NT>::ld(p);
        constexpr int W = B / 4;
#pragma unroll
        for (int i = 0; i < W; ++i) {
            if constexpr (sizeof(T) == 2) {
                out[2 * i] = __uint_as_float(v[i] << 16);
                out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
            } else {
                out[i] = __uint_as_float(v[i]);
            }
        }
    }
    __device__ static void store(T* p, const float* in)
    {
        if constexpr (sizeof(T) == 2) {
            if constexpr (N == 8)
                *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]),
                                                          pack_bf16x2(in[4], in[5]), pack_bf16x2(in[6], in[7]));
            else
                *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]));
        } else {
            if constexpr (N == 4)
                *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
            else
                *reinterpret_cast<float2*>(p) = make_float2(in[0], in[1]);
        }
    }
};

template <typename T, int L, int V, int STRIP, bool HIST, bool GELU>
__global__ __launch_bounds__(256) void prologue_kernel(
    const T* __restrict__ k, const T* __restrict__ u, const T* __restrict__ a,
    const T* __restrict__ h, const T* __restrict__ b, const T* __restrict__ conv_w,
    const T* __restrict__ k_hist, const int32_t* __restrict__ cu, int n_seqs, int T_total,
    int H, int dk, T* __restrict__ kw)
{
    constexpr int strip = STRIP;
    using LV = Lane<T, V>;
    const int groups = H * dk / V;                       // channel groups per token row
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cg = (int)(gid % groups);
    const int64_t t0_64 = (gid / groups) * strip;
    if (t0_64 >= T_total)
        return;
    const int t0 = (int)t0_64;
    const int t1 = min(T_total, t0 + strip);
    const int e = (cg * V) / dk;
    const int i0 = (cg * V) % dk;

    const int64_t row = (int64_t)H * dk;                 // elements per token of k / kw
    const int64_t lrow = (int64_t)H * (L - 1) * dk;      // elements per token of u / a / h
    const int64_t koff = (int64_t)e * dk + i0;
    const int64_t loff = (int64_t)e * (L - 1) * dk + i0;

    // Software pipeline over the strip: the raw inputs of token t + 1 are in
    // flight while token t is computed, so a thread always has two tokens of
    // loads outstanding.
    using R = Raw<LV::B, true>;
    using RV = typename R::V;
    struct In {
        RV k, a[L > 1 ? L - 1 : 1], u[L > 1 ? L - 1 : 1], h[L > 2 ? L - 2 : 1];
        T b;
    };
    auto fetch = [&](int t, In& x) {
        x.k = R::ld(k + (int64_t)t * row + koff);
        x.b = b[(int64_t)t * H + e];
        const T* ub = u + (int64_t)t * lrow + loff;
        const T* ab = a + (int64_t)t * lrow + loff;
        const T* hb = h + (int64_t)t * lrow + loff;
#pragma unroll
        for (int s = 0; s < L - 1; ++s) {
            x.a[s] = R::ld(ab + s * dk);
            x.u[s] = R::ld(ub + s * dk);
            if (s < L - 2)
                x.h[s] = R::ld(hb + s * dk);
        }
    };
    // the strip's first token is loaded before anything else, so that its loads
    // are in flight during the sequence lookup and the history loads
    In X[2];
    fetch(t0, X[0]);

    // conv taps for this thread's channels: w[e][i0 + c][m]
    float w[V][4];
#pragma unroll
    for (int c = 0; c < V; ++c) {
        const T* wp = conv_w + ((int64_t)e * dk + i0 + c) * 4;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            w[c][m] = to_f32(wp[m]);
    }

    // sequence containing t0: the largest n with cu[n] <= t0 (then t0 < cu[n+1]).
    // Binary searches on wavefront-uniform values (scalar loads, which wait on
    // their own counter, not behind the token loads in flight): one for the
    // wavefront's first live strip, one for its last.  Where both lie in the
    // same sequence, so does every lane's strip; otherwise each lane walks
    // forward from the first one's sequence.
    auto seq_of = [&](int t) {
        int lo = 0, hi = n_seqs;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (cu[mid] <= t) lo = mid; else hi = mid;
        }
        return lo;
    };
    const int t0w = __builtin_amdgcn_readfirstlane(t0);
    // the first live lane's gid + 63 bounds every lane's gid: its strip (clamped)
    // is at or past every lane's strip; uniform, so it is computed once, in SALU
    const int64_t gw = ((int64_t)__builtin_amdgcn_readfirstlane((int)(gid >> 32)) << 32) |
                       (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)gid);
    const int t0l = (int)min(((gw + 63) / groups) * strip, (int64_t)T_total - 1);
    const int nw = seq_of(t0w);
    int n, seq_start, next_start;
    if (nw == seq_of(t0l)) {
        n = nw;
        seq_start = cu[nw];
        next_start = cu[nw + 1];
    } else {
        n = nw;
        while (cu[n + 1] <= t0)                      // t0 < cu[n_seqs]: ends by n_seqs - 1
            ++n;
        seq_start = cu[n];
        next_start = cu[n + 1];
    }

    // conv history: x1 = k[t-1], x2 = k[t-2], x3 = k[t-3]; before the sequence
    // start the carried history of sequence n (slot 2 = the token just before
    // it) or zero
    float x1[V], x2[V], x3[V];
#pragma unroll
    for (int c = 0; c < V; ++c) { x1[c] = 0.f; x2[c] = 0.f; x3[c] = 0.f; }
    auto tap = [&](int tau, int start, int seq, float* x) {
        if constexpr (HIST) {
            // one unconditional load from the row chosen per lane: k inside the
            // sequence, the carried history before it (tau >= start - 3 here)
            const T* src = tau >= start
                               ? k + (int64_t)max(tau, 0) * row + koff
                               : k_hist + ((int64_t)seq * H * 3 + (int64_t)e * 3 + (tau - start + 3)) * dk + i0;
            LV::load(src, x);
        } else {
            // unconditional (a clamped row, zeroed before the sequence start), so
            // the three history loads issue together instead of one per branch
            LV::load(k + (int64_t)max(tau, 0) * row + koff, x);
            const bool in = tau >= start;
#pragma unroll
            for (int c = 0; c < V; ++c)
                x[c] = in ? x[c] : 0.f;
        }
    };
    tap(t0 - 1, seq_start, n, x1);
    tap(t0 - 2, seq_start, n, x2);
    tap(t0 - 3, seq_start, n, x3);
    int hseq = n;                                        // sequence of the latest reset (HIST)

    auto unpack = [&](const RV& v, float* out) {
        constexpr int W = LV::B / 4;
#pragma unroll
        for (int i = 0; i < W; ++i) {
            if constexpr (sizeof(T) == 2) {
                out[2 * i] = __uint_as_float(v[i] << 16);
                out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
            } else {
                out[i] = __uint_as_float(v[i]);
            }
        }
    };

    // tokens of the strip where a new sequence starts (bit t - t0), found before
    // the token loop so that the loop itself reads nothing but the inputs
    uint32_t resets = 0;
    for (int ns = next_start; ns < t1;) {               // ns > t0: t0 < cu[n + 1]
        resets |= 1u << (ns - t0);
        ++n;
        while (cu[n + 1] <= ns) ++n;                     // skips empty sequences; n+1 <= n_seqs
        ns = cu[n + 1];
    }

    auto step = [&](int t, const In& x) {
        if ((resets >> (t - t0)) & 1u) {                 // a new sequence starts at t
#pragma unroll
            for (int c = 0; c < V; ++c) { x1[c] = 0.f; x2[c] = 0.f; x3[c] = 0.f; }
            if constexpr (HIST) {
                while (cu[hseq + 1] <= t) ++hseq;        // the non-empty sequence starting at t
                tap(t - 1, t, hseq, x1);
                tap(t - 2, t, hseq, x2);
                tap(t - 3, t, hseq, x3);
            }
        }
        float kt[V];
        unpack(x.k, kt);
        const float bt = to_f32(x.b);
        float acc[V], r[V];
#pragma unroll
        for (int c = 0; c < V; ++c) {
            r[c] = w[c][3] * kt[c] + w[c][2] * x1[c] + w[c][1] * x2[c] + w[c][0] * x3[c];
            acc[c] = bt * kt[c];
        }
#pragma unroll
        for (int s = 0; s < L - 1; ++s) {                // level l = s + 1
            float av[V], uv[V];
            unpack(x.a[s], av);
            unpack(x.u[s], uv);
#pragma unroll
            for (int c = 0; c < V; ++c)
                acc[c] += av[c] * r[c] * uv[c];
            if (s < L - 2) {                             // residual for the next level
                float hv[V];
                unpack(x.h[s], hv);
#pragma unroll
                for (int c = 0; c < V; ++c) {
                    if constexpr (GELU)
                        r[c] -= av[c] * gelu_as(hv[c] * r[c]);
                    else
                        r[c] *= 1.f - av[c] * hv[c];
                }
            }
        }
        LV::store(kw + (int64_t)t * row + koff, acc);
#pragma unroll
        for (int c = 0; c < V; ++c) { x3[c] = x2[c]; x2[c] = x1[c]; x1[c] = kt[c]; }
    };

    // Two register sets used alternately over the fully unrolled strip: no
    // loop-carried copies (which would wait for the loads just issued), and the
    // prefetches are unconditional (past a short strip's end they re-read its
    // last token), so every wait is for the older set only.
#pragma unroll
    for (int i = 0; i < STRIP; ++i) {
        if (i + 1 < STRIP)
            fetch(min(t0 + i + 1, t1 - 1), X[(i + 1) & 1]);
        if (t0 + i < t1)
            step(t0 + i, X[i & 1]);
    }
}

template <typename T, int L, int V, int S, bool HIST = false, bool GELU = false>
static hipError_t launch_LVS(const PrologueArgs& p, hipStream_t stream)
{
    const int64_t groups = (int64_t)p.heads * p.dk / V;
    const int64_t strips = (p.total_tokens + S - 1) / S;
    const int64_t threads = groups * strips;
    if (threads == 0)
        return hipSuccess;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL((prologue_kernel<T, L, V, S, HIST, GELU>), dim3((unsigned)blocks), dim3(256), 0,
                       stream, (const T*)p.k, (const T*)p.u, (const T*)p.a, (const T*)p.h,
                       (const T*)p.b, (const T*)p.conv_w, (const T*)p.k_hist, p.cu_seqlens,
                       p.n_seqs, p.total_tokens, p.heads, p.dk, (T*)p.kw);
    return hipGetLastError();
}

// Tokens per thread: 4 (default: 2-3 % faster than 8 on the LM layer, where the
// 8-token strips leave a half-empty second round of workgroups), 8 or 16.
template <typename T, int L, int V>
static hipError_t launch_LV(const PrologueArgs& p, hipStream_t stream)
{
    if (p.strip == 4)
        return launch_LVS<T, L, V, 4>(p, stream);
    if (p.strip == 16)
        return launch_LVS<T, L, V, 16>(p, stream);
    return launch_LVS<T, L, V, 8>(p, stream);
}

// Channels per thread: 16-byte or 8-byte accesses (the narrow form halves the
// registers a thread holds, which doubles the wavefronts in flight).  With a
// carried history or the GELU chain: 16-byte groups, strips of 4 (the default) or 8.
// EXT: the history / GELU kernels (their own translation units).
template <typename T, int L, bool EXT>
static hipError_t launch_L(const PrologueArgs& p, hipStream_t stream)
{
    constexpr int wide = 16 / (int)sizeof(T), narrow = 8 / (int)sizeof(T);
    if constexpr (EXT) {
        if (p.strip == 4) {
            if (p.gelu && L > 2)
                return p.k_hist ? launch_LVS<T, L, wide, 4, true, true>(p, stream)
                                : launch_LVS<T, L, wide, 4, false, true>(p, stream);
            return launch_LVS<T, L, wide, 4, true>(p, stream);
        }
        if (p.gelu && L > 2)
            return p.k_hist ? launch_LVS<T, L, wide, 8, true, true>(p, stream)
                            : launch_LVS<T, L, wide, 8, false, true>(p, stream);
        return launch_LVS<T, L, wide, 8, true>(p, stream);
    } else {
        if (p.narrow)
            return launch_LV<T, L, narrow>(p, stream);
        return launch_LV<T, L, wide>(p, stream);
    }
}




template <typename T, bool EXT>
static hipError_t launch_T(const PrologueArgs& p, hipStream_t s)
{
    switch (p.L) {
    case 1: return launch_L<T, 1, EXT>(p, s);
    case 2: return launch_L<T, 2, EXT>(p, s);
    case 3: return launch_L<T, 3, EXT>(p, s);
    case 4: return launch_L<T, 4, EXT>(p, s);
    case 5: return launch_L<T, 5, EXT>(p, s);
    case 6: return launch_L<T, 6, EXT>(p, s);
    case 7: return launch_L<T, 7, EXT>(p, s);
    case 8: return launch_L<T, 8, EXT>(p, s);
    case 9: return launch_L<T, 9, EXT>(p, s);
    case 10: return launch_L<T, 10, EXT>(p, s);
    case 11: return launch_L<T, 11, EXT>(p, s);
    case 12: return launch_L<T, 12, EXT>(p, s);
    case 13: return launch_L<T, 13, EXT>(p, s);
    case 14: return launch_L<T, 14, EXT>(p, s);
    case 15: return launch_L<T, 15, EXT>(p, s);
    case 16: return launch_L<T, 16, EXT>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace prism
