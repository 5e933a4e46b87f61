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
    // fused write keys (bf16, eight-wavefront kernel): fused_L = L > 0 computes kw
    // from k, u, a, h, b and conv_w inside the scan (closed form, no carried
    // history) instead of reading kw; 0 reads kw
    int fused_L = 0;
    const void *u = nullptr, *a = nullptr, *h = nullptr, *conv_w = nullptr;
    // with fused_L > 0 and kw_producers > 0 (a multiple of 8): that many
    // producer blocks in the scan launch write kw (the workspace array) and
    // count their eight wavefronts into one flag per (virtual chunk
    // floor(cu[n] / 64) + n + c, head) in kw_ready ((T / 64 + n_seqs) * H ints,
    // cleared by the launch) instead
    int kw_producers = 0;
    int* kw_ready = nullptr;
    // chunk-start states for the chunkwise backward (bf16 [nv, H, dk, dv] and
    // transposed [nv, H, dv, dk], nv = T / 64 + n_seqs), or null: the
    // eight-wavefront kernel
    void *ck = nullptr, *ckT = nullptr;
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
    // the chunkwise path only: gq, gk, gv, gu, ga, gh hold bf16 (round to nearest
    // even) instead of fp32, and the scan's fp32 part of dk is in gk_part
    bool grad_bf16 = false;
    const float* gk_part = nullptr;
    float* gs_init;                 // or null (not written)
    float* ws;                      // bwd_workspace_floats(...) floats
};
size_t bwd_workspace_floats(int n_seqs, int total_tokens, int heads, int dk, int dv);

// Chunkwise backward (bf16, backward_chunk.hip).  Pass B: the carried gradient
// of every chunk's end state, from the last chunk to the first, as bf16
// [virtual chunk][H][dk][dv] (dck) and [virtual chunk][H][dv][dk] (dckT), and
// dS_init (fp32, optional).  p holds q, k, g, b, cu_seqlens and the shape.
hipError_t launch_bwd_state(const ScanArgs& p, const void* dO, const void* mats, const float* dS_final,
                            void* dck, void* dckT, float* dS_init, hipStream_t stream);
struct BwdChunkBufs {
    const void *dO, *mats, *ck, *ckT, *dck, *dckT;
    void *gq, *gv;                               // fp32, or bf16 when grad_bf16
    float *gk, *gkw, *gg, *gb;                   // fp32 (gk: the scan's part of dk)
    bool grad_bf16 = false;
};
// The chunk-parallel gradients: every gradient of the scan's inputs (q, k, kw,
// v, g, b) from the checkpoints, in one launch; p.kw holds the write keys.
// Stores (no accumulation): dq, dk, dkw, dv, dg, db are written whole; dq and dv
// in bf16 (round to nearest even) when w.grad_bf16, the rest in fp32.
hipError_t launch_bwd_grads(const ScanArgs& p, const BwdChunkBufs& w, hipStream_t stream);

// The write-key part of the backward pass alone (backward.hip): from dkw (fp32
// [T][H][dk]) it writes du, da, dh, adds the write-key terms to dk and db (both
// hold the scan's gradients on entry), and writes dconv_w; part holds
// wk_workspace_floats(T, H, dk) floats of scratch (per-block partials).
size_t wk_workspace_floats(int total_tokens, int heads, int dk);
hipError_t launch_write_key_bwd(const BwdArgs& p, const float* dkw, float* part, hipStream_t stream);
bool bwd_supported(int dk, int dv);
hipError_t launch_bwd(const BwdArgs& p, hipStream_t stream);

// One token per sequence through the recurrence (state and history in place).
hipError_t launch_decode(const DecodeArgs& p, hipStream_t stream);
bool decode_supported(int dk, int dv);

// Generic chunk scan (fp32 and bf16 operands), LDS-staged intermediates.
// Returns hipErrorInvalidValue when (dtype, dk, dv_slice) has no kernel.
hipError_t launch_scan(const ScanArgs& p, hipStream_t stream);
bool scan_supported(bool bf16, int dk, int dv, int dv_slice);

// Two-pass bf16 scan: the per-chunk matrices of every (chunk, head) at once
// (chunk_gram.hip, into gram_workspace_bytes of device memory), then the
// sequential state products from them (chunk_scan_state.hip).
size_t gram_workspace_bytes(int n_seqs, int total_tokens, int heads);
hipError_t launch_gram(const ScanArgs& p, void* ws, hipStream_t stream);
// ck / ckT (optional): every chunk's start state, bf16, [virtual chunk][H][dk][dv]
// and [virtual chunk][H][dv][dk]; p.o and p.s_final may be null (not written)
hipError_t launch_scan_state(const ScanArgs& p, const void* mats, hipStream_t stream, void* ck = nullptr,
                             void* ckT = nullptr);
bool scan_state_supported(int dk, int dv);

// fp32 scan token by token (fp32 inputs at dk = 128, whose chunkwise tiles
// exceed the LDS); any dk in {64, 128}, dv a multiple of 32.
hipError_t launch_scan_f32_recurrent(const ScanArgs& p, hipStream_t stream);
bool scan_f32_recurrent_supported(int dk, int dv);

// bf16 chunk scan with the register-resident state path.
hipError_t launch_scan_bf16(const ScanArgs& p, hipStream_t stream);
bool scan_fused_kw_supported(int dk, int dv, int L);
// `a` on the eight-wavefront kernel (32-column slices) and, in the same launch,
// `m`: the transitions alone over the same sequences (m.dv = dk, start S = I,
// no write term), writing m.o and m.s_final; with skip > 1 the sequences
// 0, skip, 2 skip, ... are left out of `m`.
hipError_t launch_scan_bf16_pair(const ScanArgs& a, const ScanArgs& m, int skip, hipStream_t stream);
bool scan_bf16_supported(int dk, int dv, int dv_slice);
// Bounded in-kernel waits of the bf16 scan that gave up (synchronous read of
// a device counter on the current device; reset sets it back to zero).
hipError_t read_wait_giveups(unsigned int* count, bool reset);

}  // namespace prism
