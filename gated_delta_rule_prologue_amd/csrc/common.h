// common.h -- small device helpers shared by the libprism kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prism {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// bf16 is carried as raw 16-bit patterns (uint16_t) everywhere in device code.
__device__ __forceinline__ float bf16_to_f32(uint16_t x)
{
    return __uint_as_float(((uint32_t)x) << 16);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    bf16x2_t h;
    h[0] = (__bf16)lo;
    h[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, h);
}

// Workgroup barrier that orders LDS accesses only.  Every exchange between the
// wavefronts of one workgroup in these kernels goes through LDS, so global
// loads (prefetches) and stores stay in flight across it; a full
// __syncthreads() would wait for all of them first.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// GELU(x) = x Phi(x) = x (1 + erf(x / sqrt 2)) / 2, with erf from the rational
// approximation of Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (after Hastings): for z >= 0,
//   erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),  t = 1 / (1 + p z),
// absolute error <= 1.5e-7, and erf is odd.  Branch-free: one reciprocal, one
// exp2, a degree-5 polynomial (the library erff costs several times as much and
// branches on |x|).  Relative error of the result about 2e-7.
__device__ __forceinline__ float gelu_as(float x)
{
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(1.f + 0.3275911f * z);
    const float poly =
        t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float e = 1.f - poly * __builtin_amdgcn_exp2f(-z * z * 1.44269504088896341f);
    return 0.5f * x * (1.f + __builtin_copysignf(e, x));
}

// GELU(x) and GELU'(x) = Phi(x) + x phi(x), phi(x) = exp(-x^2 / 2) / sqrt(2 pi):
// Phi from the same erf approximation as gelu_as, phi from one exp2.
__device__ __forceinline__ float gelu_as_grad(float x, float& dgelu)
{
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(1.f + 0.3275911f * z);
    const float poly =
        t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float ez = __builtin_amdgcn_exp2f(-z * z * 1.44269504088896341f);   // exp(-x^2 / 2)
    const float phi_cdf = 0.5f * (1.f + __builtin_copysignf(1.f - poly * ez, x));
    dgelu = phi_cdf + x * ez * 0.39894228040143268f;
    return x * phi_cdf;
}

// Element conversions for the two input storage types.
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float f) { return f32_to_bf16(f); }
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }

// 16-byte vector of the storage type: 8 bf16 or 4 fp32 elements.
template <typename T> struct Vec16;
template <> struct Vec16<uint16_t> {
    static constexpr int N = 8;
    __device__ static void load(const uint16_t* p, float* out)
    {
        uint4 v = *reinterpret_cast<const uint4*>(p);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ static void store(uint16_t* p, const float* in)
    {
        *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]),
                                                  pack_bf16x2(in[4], in[5]), pack_bf16x2(in[6], in[7]));
    }
};
template <> struct Vec16<float> {
    static constexpr int N = 4;
    __device__ static void load(const float* p, float* out)
    {
        float4 v = *reinterpret_cast<const float4*>(p);
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    }
    __device__ static void store(float* p, const float* in)
    {
        *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
    }
};

}  // namespace prism
