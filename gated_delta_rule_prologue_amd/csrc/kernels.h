// kernels.h -- internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prism {

struct PrologueArgs {
    bool bf16;
    int n_seqs, total_tokens, heads, dk, L;
    int strip;                      // tokens walked by one thread: 4, 8 or 16
    bool narrow;                    // 8-byte instead of 16-byte channel groups
    const void *k, *u, *a, *h, *b, *conv_w;
    const int32_t* cu_seqlens;
    void* kw;
};

struct ScanArgs {
    bool bf16;
    int n_seqs, total_tokens, heads, dk, dv;
    int dv_slice;                   // value columns owned by one workgroup
    bool specialised;               // bf16: helper wavefronts prepare the next chunk (dv_slice <= 32)
    int ws_waves;                   // wavefronts of the specialised kernel: 4, or 8 (dv_slice 32)
    const void *q, *k, *kw, *v, *g, *b;
    const int32_t* cu_seqlens;
    void* o;
    float* s_final;
};

hipError_t launch_prologue(const PrologueArgs& p, hipStream_t stream);

// Generic chunk scan (fp32 and bf16 operands), LDS-staged intermediates.
// Returns hipErrorInvalidValue when (dtype, dk, dv_slice) has no kernel.
hipError_t launch_scan(const ScanArgs& p, hipStream_t stream);
bool scan_supported(bool bf16, int dk, int dv, int dv_slice);

// bf16 chunk scan with the register-resident state path.
hipError_t launch_scan_bf16(const ScanArgs& p, hipStream_t stream);
bool scan_bf16_supported(int dk, int dv, int dv_slice);

}  // namespace prism
