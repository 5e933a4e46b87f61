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
    bool gelu;                      // residual chain r - a GELU(h r) instead of the closed form
    const void *k, *u, *a, *h, *b, *conv_w;
    const void* k_hist;             // [n_seqs, H, 3, dk] carried conv history, or null (zero)
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
    const float* s_init;            // [n_seqs, H, dk, dv] start states, or null (zero)
    void* o;
    float* s_final;
};

hipError_t launch_prologue(const PrologueArgs& p, hipStream_t stream);

// k_hist_out[n, e, m, :] = k at position (end of sequence n) - 3 + m, read from
// k_hist (or zero) before the sequence start.  k_hist_out may equal k_hist.
hipError_t launch_k_history(bool bf16, int n_seqs, int heads, int dk, const void* k,
                            const void* k_hist, const int32_t* cu_seqlens, void* k_hist_out,
                            hipStream_t stream);

struct DecodeArgs {
    bool bf16;
    int n_seqs, heads, dk, dv, L;
    bool gelu;                      // residual chain r - a GELU(h r) instead of the closed form
    const void *q, *k, *v, *u, *a, *h, *g, *b, *conv_w;
    float* S;                       // [n_seqs, H, dk, dv], updated in place
    void* k_hist;                   // [n_seqs, H, 3, dk], updated in place
    void* o;
};

// Few long sequences: the scan split into P segments per sequence, scanned
// side by side and chained (long_seq.hip).  split_segments gives P (1 = no
// split) for the shape and the number of compute units; the launch needs
// split_workspace_bytes of device scratch.  Specialised bf16 kernels only.
int split_segments(int n_seqs, int heads, int dk, int dv, int total_tokens, int cus);
size_t split_workspace_bytes(int n_seqs, int heads, int dk, int dv, int total_tokens, int P);
hipError_t launch_split_scan(const ScanArgs& p, int P, void* ws, hipStream_t stream);

// Backward pass (closed-form residual chain): fp32 gradients of the loss
// sum <dO, o> + <dS_final, S_final>; kw from the prologue (input dtype).
struct BwdArgs {
    bool bf16;
    int n_seqs, total_tokens, heads, dk, dv, L;
    bool gelu;                      // residual chain r - a GELU(h r) instead of the closed form
    const void *q, *k, *v, *kw, *u, *a, *h, *g, *b, *conv_w, *dO;
    const int32_t* cu_seqlens;
    const float* s_init;            // or null (zero)
    const float* ds_final;          // or null (zero)
    float *gq, *gk, *gv, *gu, *ga, *gh, *gg, *gb, *gconv;
    float* gs_init;                 // or null (not written)
    float* ws;                      // bwd_workspace_floats(...) floats
};
size_t bwd_workspace_floats(int n_seqs, int total_tokens, int heads, int dk, int dv);
bool bwd_supported(int dk, int dv);
hipError_t launch_bwd(const BwdArgs& p, hipStream_t stream);

// One token per sequence through the recurrence (state and history in place).
hipError_t launch_decode(const DecodeArgs& p, hipStream_t stream);
bool decode_supported(int dk, int dv);

// Generic chunk scan (fp32 and bf16 operands), LDS-staged intermediates.
// Returns hipErrorInvalidValue when (dtype, dk, dv_slice) has no kernel.
hipError_t launch_scan(const ScanArgs& p, hipStream_t stream);
bool scan_supported(bool bf16, int dk, int dv, int dv_slice);

// bf16 chunk scan with the register-resident state path.
hipError_t launch_scan_bf16(const ScanArgs& p, hipStream_t stream);
// `a` on the eight-wavefront kernel (32-column slices) and, in the same launch,
// `m`: the transitions alone over the same sequences (m.dv = dk, start S = I,
// no write term), writing m.o and m.s_final; with skip > 1 the sequences
// 0, skip, 2 skip, ... are left out of `m`.
hipError_t launch_scan_bf16_pair(const ScanArgs& a, const ScanArgs& m, int skip, hipStream_t stream);
bool scan_bf16_supported(int dk, int dv, int dv_slice);

}  // namespace prism
