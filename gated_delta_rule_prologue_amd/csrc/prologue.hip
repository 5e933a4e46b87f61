// prologue.hip -- dispatch of the write-key prologue (kernels in
// prologue_kernel.h, instantiated per input type) and the kernel that writes
// the convolution history to carry past the end of each sequence.
#include "common.h"
#include "kernels.h"

namespace prism {

hipError_t launch_prologue_bf16(const PrologueArgs& p, hipStream_t stream);
hipError_t launch_prologue_f32(const PrologueArgs& p, hipStream_t stream);
hipError_t launch_prologue_bf16_ext(const PrologueArgs& p, hipStream_t stream);
hipError_t launch_prologue_f32_ext(const PrologueArgs& p, hipStream_t stream);

hipError_t launch_prologue(const PrologueArgs& p, hipStream_t stream)
{
    if (p.k_hist || (p.gelu && p.L > 2))         // history or GELU-chain kernels
        return p.bf16 ? launch_prologue_bf16_ext(p, stream) : launch_prologue_f32_ext(p, stream);
    return p.bf16 ? launch_prologue_bf16(p, stream) : launch_prologue_f32(p, stream);
}

// One thread per (sequence, head, 4 channels): reads its old history and k
// rows first, then writes, so k_hist_out may be k_hist itself.
template <typename T>
__global__ __launch_bounds__(256) void k_history_kernel(
    const T* __restrict__ k, const T* k_hist, const int32_t* __restrict__ cu, int n_seqs,
    int H, int dk, T* k_hist_out)
{
    const int groups = dk / 4;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= (int64_t)n_seqs * H * groups)
        return;
    const int i0 = (int)(gid % groups) * 4;
    const int e = (int)((gid / groups) % H);
    const int n = (int)(gid / groups / H);
    const int start = cu[n], end = cu[n + 1];
    T rows[3][4];
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        const int tau = end - 3 + m;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            T x = from_f32<T>(0.f);
            if (tau >= start)
                x = k[((int64_t)tau * H + e) * dk + i0 + c];
            else if (k_hist)
                x = k_hist[(((int64_t)n * H + e) * 3 + (tau - start + 3)) * dk + i0 + c];
            rows[m][c] = x;
        }
    }
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            k_hist_out[(((int64_t)n * H + e) * 3 + m) * dk + i0 + c] = rows[m][c];
}

hipError_t launch_k_history(bool bf16, int n_seqs, int heads, int dk, const void* k,
                            const void* k_hist, const int32_t* cu_seqlens, void* k_hist_out,
                            hipStream_t stream)
{
    if (dk % 4 != 0)
        return hipErrorInvalidValue;
    const int64_t threads = (int64_t)n_seqs * heads * (dk / 4);
    if (threads == 0)
        return hipSuccess;
    const unsigned blocks = (unsigned)((threads + 255) / 256);
    if (bf16)
        hipLaunchKernelGGL((k_history_kernel<uint16_t>), dim3(blocks), dim3(256), 0, stream,
                           (const uint16_t*)k, (const uint16_t*)k_hist, cu_seqlens, n_seqs, heads,
                           dk, (uint16_t*)k_hist_out);
    else
        hipLaunchKernelGGL((k_history_kernel<float>), dim3(blocks), dim3(256), 0, stream,
                           (const float*)k, (const float*)k_hist, cu_seqlens, n_seqs, heads, dk,
                           (float*)k_hist_out);
    return hipGetLastError();
}

}  // namespace prism
