// mfma_bf16.h -- bf16 MFMA operand fragments and small wavefront helpers for
// gfx950, shared by the chunk-scan kernels (one 64-lane wavefront per tile
// product; 16x16x32 and 16x16x16 bf16 MFMA with fp32 accumulators).
#pragma once

#include "common.h"

namespace prism {
namespace mfma {

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef short v8s_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
typedef __attribute__((address_space(3))) int lds_int_t;

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

// Two 16x16x16 operand fragments side by side as one 16x16x32 fragment: the
// contraction index of the wider product runs over both halves (k slots
// 8 g + 0..3 from lo, 8 g + 4..7 from hi).  Pairing A and B fragments the
// same way makes a 16x16x32 product equal to the sum of the two 16x16x16
// products, at the 16x16x32 rate.
__device__ __forceinline__ bf16x8_t cat8(v4s_t lo, v4s_t hi)
{
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Two 16x16x16 operand fragments of consecutive 16-row blocks (rows 4g .. 4g+3
// of `lo` and of `hi` in lane group g = lane / 16) as one 16x16x32 fragment
// holding rows 8g .. 8g+7 of the 32-row pair in lane group g, so that it pairs
// with a plain 16-byte row read of the other operand.  Per dword:
// v_permlane32_swap exchanges lane groups 2, 3 of lo with groups 0, 1 of hi,
// giving (lo0 lo1 hi0 hi1 | lo2 lo3 hi2 hi3); v_permlane16_swap then exchanges
// the odd groups of the first with the even groups of the second, giving
// (lo0 lo2 hi0 hi2 | lo1 lo3 hi1 hi3): rows 8g .. 8g+3 and 8g+4 .. 8g+7.
__device__ __forceinline__ bf16x8_t pair_rows(v4s_t lo, v4s_t hi)
{
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    const auto x0 = __builtin_amdgcn_permlane32_swap(a.x, b.x, false, false);
    const auto y0 = __builtin_amdgcn_permlane16_swap(x0[0], x0[1], false, false);
    const auto x1 = __builtin_amdgcn_permlane32_swap(a.y, b.y, false, false);
    const auto y1 = __builtin_amdgcn_permlane16_swap(x1[0], x1[1], false, false);
    return __builtin_bit_cast(bf16x8_t, make_uint4(y0[0], y1[0], y0[1], y1[1]));
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

// Scale the eight k-entries of a 16x16x32 fragment by f0 (k = 8 (lane / 16) + 0..3)
// and f1 (+ 4..7): folds diag(gamma_C / gamma) into a V operand.
__device__ __forceinline__ bf16x8_t scale8(bf16x8_t x, float4 f0, float4 f1)
{
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

// Keeps the compiler from moving instructions across this point: the state
// path issues each batch of LDS reads one computation ahead of its use, and
// the scheduler would otherwise sink every read next to its MFMA (one
// wavefront per SIMD leaves nothing else to hide the LDS latency).
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// Unit lower-triangular 16x16 inverse, four blocks per wavefront: lane
// (16 g + i) holds row i of the strictly lower block A_g in a[] and returns
// column i of (I + A_g)^-1 in x[] (right-looking substitution in fp32).  Step c
// updates x[r] -= A_g[r][c] x[c] for r > c with one v_fmac_f32 each, the entry
// A_g[r][c] coming from lane 16 g + r through a DPP row broadcast of a[c]
// (`row_newbcast`, which the compiler does not fuse into the FMA by itself).
// A DPP read needs two wait states after a VALU write of its source, and the
// hardware does not enforce them; the compiler does not see into the asm, so
// the first FMA of each step carries its own s_nop in the same statement (the
// compiler may place the write of a[c] right before it).  The later FMAs of the
// step read the same register.
template <int C, int R>
__device__ __forceinline__ void subst_col(float (&x)[16], float ac, float xc)
{
    if constexpr (R < 16) {
        if constexpr (R == C + 1)
            asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %1, -%2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                         : "+v"(x[R])
                         : "v"(ac), "v"(xc), "i"(R));
        else
            asm volatile("v_fmac_f32_dpp %0, %1, -%2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                         : "+v"(x[R])
                         : "v"(ac), "v"(xc), "i"(R));
        subst_col<C, R + 1>(x, ac, xc);
    }
}
template <int C>
__device__ __forceinline__ void subst(float (&x)[16], const float (&a)[16])
{
    if constexpr (C < 15) {
        subst_col<C, C + 1>(x, a[C], x[C]);
        subst<C + 1>(x, a);
    }
}

}  // namespace mfma

// A 4 x 4 block of bf16 spread over the four lanes of a quad (four consecutive
// columns): lane p holds rows 0 .. 3 of column p as w (w.x rows 0 and 1, w.y
// rows 2 and 3, low halves first).  operator() returns row p of columns 0 .. 3
// in the same packing, so that a lane can store four consecutive columns of one
// row with one 8-byte store.  An exchange with lane p ^ 2 (DPP quad_perm) gives
// lanes 0, 1 the row pairs (0, 1) and lanes 2, 3 the pairs (2, 3) of the
// partner's column; an exchange with lane p ^ 1 then interleaves the 16-bit
// halves.  The lane-dependent choices are byte permutes with per-lane selectors
// (v_perm_b32: selector bytes 0-3 take the second operand's bytes, 4-7 the
// first's), not branches.
struct QuadTranspose {
    uint32_t sel_lo, sel_hi, sel_pair;
    __device__ __forceinline__ explicit QuadTranspose(int p)
    {
        constexpr uint32_t kFirst = 0x07060504u, kSecond = 0x03020100u;
        sel_lo = p < 2 ? kFirst : kSecond;
        sel_hi = p < 2 ? kSecond : kFirst;
        // even lanes: low halves of (own, partner); odd lanes: high halves of (partner, own)
        sel_pair = (p & 1) ? 0x03020706u : 0x05040100u;
    }
    __device__ __forceinline__ uint2 operator()(uint2 w) const
    {
        const uint32_t send = __builtin_amdgcn_perm(w.y, w.x, sel_lo);
        const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4e, 0xf, 0xf, false);
        const uint32_t a0 = __builtin_amdgcn_perm(recv, w.x, sel_hi);
        const uint32_t a1 = __builtin_amdgcn_perm(recv, w.y, sel_lo);
        const uint32_t b0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)a0, 0xb1, 0xf, 0xf, false);
        const uint32_t b1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)a1, 0xb1, 0xf, 0xf, false);
        return make_uint2(__builtin_amdgcn_perm(b0, a0, sel_pair), __builtin_amdgcn_perm(b1, a1, sel_pair));
    }
};

}  // namespace prism
