// prism_api.hip -- C ABI of libprism (declared in include/prism.h): argument
// validation, kernel selection and launches on the caller's stream.
#include <mutex>
#include <stdint.h>
#include <stdlib.h>

#include "prism.h"
#include "kernels.h"

// Workspace of prism_fwd_noalloc: a file-scope device array, one copy per GPU
// for the life of the process.  Host code never passes `scratch` itself (in
// host code the name is only a stand-in for the device symbol); it passes the
// device address hipGetSymbolAddress returned on that device.
static __device__ __align__(256) unsigned char scratch[PRISM_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept; null if the lookup fails.
void* scratch_ptr()
{
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess)
            return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool dims_ok(const prism_dims* d)
{
    return d && d->n_seqs >= 1 && d->total_tokens >= 0 && d->heads >= 1 && d->dk >= 1 &&
           d->dv >= 1 && (d->dtype == PRISM_F32 || d->dtype == PRISM_BF16);
}

size_t elem_bytes(const prism_dims* d) { return d->dtype == PRISM_BF16 ? 2 : 4; }

// Pointer must be non-null and 16-byte aligned.
bool ptr_ok(const void* p) { return p && aligned16(p); }

// Per-token arrays may be NULL when there are no tokens at all.
bool tok_ok(const prism_dims* d, const void* p)
{
    return d->total_tokens == 0 ? aligned16(p) : ptr_ok(p);
}

int env_int(const char* name, int fallback)
{
    const char* s = getenv(name);
    if (!s || !*s)
        return fallback;
    char* end = nullptr;
    long v = strtol(s, &end, 10);
    return (end && *end == 0 && v >= 0 && v < (1 << 20)) ? (int)v : fallback;
}

// Which scan kernel runs: the register-resident bf16 kernel unless the
// generic one is requested (PRISM_SCAN_GENERIC=1) or the shape needs it.
bool use_bf16_kernel(const prism_dims* d, int dvs)
{
    return d->dtype == PRISM_BF16 && env_int("PRISM_SCAN_GENERIC", 0) == 0 &&
           prism::scan_bf16_supported(d->dk, d->dv, dvs);
}

bool slice_supported(const prism_dims* d, int dvs)
{
    const bool bf16 = d->dtype == PRISM_BF16;
    if (bf16 && env_int("PRISM_SCAN_GENERIC", 0) == 0)
        return prism::scan_bf16_supported(d->dk, d->dv, dvs);
    return prism::scan_supported(bf16, d->dk, d->dv, dvs);
}

bool ws8_enabled()
{
    return env_int("PRISM_SCAN_SPECIALISED", 1) != 0 && env_int("PRISM_SCAN_WAVES", 8) != 4;
}

// Value columns per scan workgroup: split the dv columns of each chain until
// there are enough workgroups for the 256 CUs (columns of S are independent).
// bf16 takes 32-column slices whenever the eight-wavefront kernel serves them:
// its per-chunk latency is the lowest, so it wins even where 64-column slices
// would fill the chip (measured on the recsys, varlen and 64k workloads).
int pick_dv_slice(const prism_dims* d)
{
    const int forced = env_int("PRISM_DV_SLICE", 0);
    if (forced && slice_supported(d, forced))
        return forced;
    if (d->dtype == PRISM_BF16 && env_int("PRISM_SCAN_GENERIC", 0) == 0 && ws8_enabled() &&
        slice_supported(d, 32))
        return 32;
    const long chains = (long)d->n_seqs * d->heads;
    const int cands[3] = {64, 32, 16};
    int best = 0;
    for (int c : cands) {
        if (!slice_supported(d, c))
            continue;
        best = c;                                   // smallest supported so far
        if (chains * (d->dv / c) >= 192)
            return c;                               // largest slice that fills the chip
    }
    return best;
}

// fp32 takes the token-recurrent scan at dk = 128 (its chunkwise tiles do not
// fit the LDS there), and anywhere with PRISM_SCAN_RECURRENT=1.
bool use_f32_recurrent(const prism_dims* d)
{
    return d->dtype == PRISM_F32 && prism::scan_f32_recurrent_supported(d->dk, d->dv) &&
           (d->dk == 128 || env_int("PRISM_SCAN_RECURRENT", 0) != 0);
}

prism_status check_scan_shape(const prism_dims* d)
{
    if (use_f32_recurrent(d))
        return PRISM_OK;
    for (int c : {64, 32, 16})
        if (slice_supported(d, c))
            return PRISM_OK;
    return PRISM_EUNSUPPORTED;
}

prism_status from_hip(hipError_t e) { return e == hipSuccess ? PRISM_OK : PRISM_EHIP; }

int device_cus()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return n;
}

// Segments per sequence of the split scan for a forward pass (1 = one scan
// launch over whole sequences).  The split serves few, long sequences on the
// eight-wavefront bf16 kernel; PRISM_SPLIT=0 turns it off, PRISM_SPLIT=P >= 2
// forces P segments.
int split_for(const prism_dims* d)
{
    if (d->dtype != PRISM_BF16 || env_int("PRISM_SCAN_GENERIC", 0) != 0 || !ws8_enabled() ||
        pick_dv_slice(d) != 32 || d->total_tokens == 0)
        return 1;
    const int forced = env_int("PRISM_SPLIT", -1);
    if (forced == 0)
        return 1;
    if (forced >= 2 && forced <= 64)
        return (d->dk == 64 || d->dk == 128) && (d->dv == 64 || d->dv == 128) ? forced : 1;
    return prism::split_segments(d->n_seqs, d->heads, d->dk, d->dv, d->total_tokens, device_cus());
}

// The two-pass bf16 scan (per-chunk matrices of all chunks at once, then the
// WY state kernel) is opt-in with PRISM_SCAN_TWOPASS=1 (and a workspace): on
// MI355X it is slower than the single fused kernel (the matrices make a round
// trip through HBM, and the state kernel's helpers bound its chunk rate).
bool use_two_pass(const prism_dims* d)
{
    return d->dtype == PRISM_BF16 && env_int("PRISM_SCAN_GENERIC", 0) == 0 &&
           env_int("PRISM_SCAN_TWOPASS", 0) == 1 && prism::scan_state_supported(d->dk, d->dv) &&
           d->total_tokens > 0;
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

size_t kw_bytes(const prism_dims* d)
{
    size_t n = (size_t)d->total_tokens * (size_t)d->heads * (size_t)d->dk * elem_bytes(d);
    n = (n + 255) / 256 * 256;
    return n < 256 ? 256 : n;
}

// Optional pointer: null, or 16-byte aligned.
bool opt_ok(const void* p) { return aligned16(p); }

bool residual_ok(int r) { return r == PRISM_RESIDUAL_LINEAR || r == PRISM_RESIDUAL_GELU; }

prism_status prologue_impl(const prism_dims* d, const void* k, const void* u, const void* a,
                           const void* h, const void* b, const void* conv_w, const void* k_hist,
                           const int32_t* cu_seqlens, int L, int residual, void* kw, void* stream)
{
    if (!dims_ok(d) || L < 1 || L > PRISM_MAX_LEVELS || !residual_ok(residual))
        return PRISM_EINVAL;
    if (!tok_ok(d, k) || !tok_ok(d, b) || !ptr_ok(conv_w) || !ptr_ok(cu_seqlens) ||
        !tok_ok(d, kw) || !opt_ok(k_hist))
        return PRISM_EINVAL;
    if (L > 1 && (!tok_ok(d, u) || !tok_ok(d, a) || !tok_ok(d, h)))
        return PRISM_EINVAL;
    const int vec = d->dtype == PRISM_BF16 ? 8 : 4;
    if (d->dk % vec != 0)
        return PRISM_EUNSUPPORTED;
    prism::PrologueArgs p;
    p.bf16 = d->dtype == PRISM_BF16;
    p.n_seqs = d->n_seqs;
    p.total_tokens = d->total_tokens;
    p.heads = d->heads;
    p.dk = d->dk;
    p.L = L;
    p.strip = env_int("PRISM_PROLOGUE_STRIP", 4);      // 4, 8 or 16 tokens per thread
    if (p.strip != 8 && p.strip != 16)
        p.strip = 4;
    p.narrow = env_int("PRISM_PROLOGUE_NARROW", 0) != 0;
    p.gelu = residual == PRISM_RESIDUAL_GELU;
    p.k = k; p.u = u; p.a = a; p.h = h; p.b = b; p.conv_w = conv_w;
    p.k_hist = k_hist;
    p.cu_seqlens = cu_seqlens;
    p.kw = kw;
    return from_hip(prism::launch_prologue(p, (hipStream_t)stream));
}

// Fused write keys (PRISM_FUSED_KW=1): prism_fwd computes kw inside the scan
// (the eight-wavefront kernel's Gram helpers) instead of launching the prologue,
// where that kernel serves the shape: bf16, L = 4 or 8, the closed-form chain,
// no carried history, 32-column slices, no segment split or two-pass scan.
bool use_fused_kw(const prism_dims* d, int L, int residual, const void* k_hist)
{
    return env_int("PRISM_FUSED_KW", 0) == 1 && d->dtype == PRISM_BF16 &&
           residual == PRISM_RESIDUAL_LINEAR && !k_hist &&
           prism::scan_fused_kw_supported(d->dk, d->dv, L) && use_bf16_kernel(d, 32) &&
           pick_dv_slice(d) == 32 && ws8_enabled() && split_for(d) < 2 && !use_two_pass(d) &&
           d->total_tokens > 0;
}

// Write-key producers (opt-in, PRISM_KW_PRODUCERS=1): prism_fwd runs no
// prologue launch; the scan launch carries producer blocks on the compute units
// its own blocks leave idle, which form kw chunk by chunk while the scan runs
// and flag each chunk's rows for it.  Same shapes as the fused write keys, and
// the scan must leave at least eight compute units idle (one producer per XCD).
// Returns the producer count (a multiple of 8, at most 128), or 0.  On MI355X
// the one launch is slower than the prologue and scan launches (the producers
// and the scan slow each other down), so it is off by default.
bool kw_producers_requested() { return env_int("PRISM_KW_PRODUCERS", 0) == 1; }

int kw_producers_for(const prism_dims* d, int L, int residual, const void* k_hist)
{
    if (!kw_producers_requested() || d->dtype != PRISM_BF16 ||
        residual != PRISM_RESIDUAL_LINEAR || k_hist ||
        !prism::scan_fused_kw_supported(d->dk, d->dv, L) || !use_bf16_kernel(d, 32) ||
        pick_dv_slice(d) != 32 || !ws8_enabled() || env_int("PRISM_SCAN_SPECIALISED", 1) == 0 ||
        env_int("PRISM_SCAN_WAVES", 8) == 4 || split_for(d) >= 2 || use_two_pass(d) ||
        d->total_tokens == 0)
        return 0;
    const int64_t blocks = (int64_t)d->n_seqs * d->heads * (d->dv / 32);
    const int64_t idle = (int64_t)device_cus() - blocks;
    if (idle < 8)
        return 0;
    return (int)(idle / 8 * 8 < 128 ? idle / 8 * 8 : 128);
}

// Bytes of the producers' readiness flags (one int per virtual chunk and head),
// reserved in the forward workspace when the producers are requested, for every
// shape they can serve, whichever way the call goes.
size_t kw_ready_bytes(const prism_dims* d, int L)
{
    if (!kw_producers_requested() || d->dtype != PRISM_BF16 || d->total_tokens == 0 ||
        !prism::scan_fused_kw_supported(d->dk, d->dv, L))
        return 0;
    return round256(((size_t)d->total_tokens / 64 + (size_t)d->n_seqs) * (size_t)d->heads * 4);
}

struct FusedKw {
    int L = 0;
    const void *u = nullptr, *a = nullptr, *h = nullptr, *conv_w = nullptr;
    int producers = 0;                           // > 0: producer blocks (kw written, flags raised)
    int* ready = nullptr;
};

prism_status scan_impl(const prism_dims* d, const void* q, const void* k, const void* kw,
                       const void* v, const void* g, const void* b, const int32_t* cu_seqlens,
                       const float* S_init, void* o, float* S_final, void* split_ws, void* stream,
                       const FusedKw& fk = FusedKw())
{
    if (!dims_ok(d))
        return PRISM_EINVAL;
    if (!tok_ok(d, q) || !tok_ok(d, k) || !tok_ok(d, kw) || !tok_ok(d, v) || !tok_ok(d, g) ||
        !tok_ok(d, b) || !ptr_ok(cu_seqlens) || !tok_ok(d, o) || !ptr_ok(S_final) ||
        !opt_ok(S_init))
        return PRISM_EINVAL;
    prism_status st = check_scan_shape(d);
    if (st != PRISM_OK)
        return st;
    prism::ScanArgs p;
    p.bf16 = d->dtype == PRISM_BF16;
    p.n_seqs = d->n_seqs;
    p.total_tokens = d->total_tokens;
    p.heads = d->heads;
    p.dk = d->dk;
    p.dv = d->dv;
    p.dv_slice = pick_dv_slice(d);
    p.specialised = p.bf16 && p.dv_slice <= 32 && env_int("PRISM_SCAN_SPECIALISED", 1) != 0;
    p.ws_waves = env_int("PRISM_SCAN_WAVES", 8) == 4 ? 4 : 8;
    p.q = q; p.k = k; p.kw = kw; p.v = v; p.g = g; p.b = b;
    p.cu_seqlens = cu_seqlens;
    p.s_init = S_init;
    p.o = o;
    p.s_final = S_final;
    if (fk.L > 0) {
        p.fused_L = fk.L;
        p.u = fk.u; p.a = fk.a; p.h = fk.h; p.conv_w = fk.conv_w;
        p.kw_producers = fk.producers;
        p.kw_ready = fk.ready;
        return from_hip(prism::launch_scan_bf16(p, (hipStream_t)stream));
    }
    if (use_f32_recurrent(d))
        return from_hip(prism::launch_scan_f32_recurrent(p, (hipStream_t)stream));
    const int P = split_ws ? split_for(d) : 1;
    if (P >= 2)
        return from_hip(prism::launch_split_scan(p, P, split_ws, (hipStream_t)stream));
    if (split_ws && use_two_pass(d)) {
        hipError_t e = prism::launch_gram(p, split_ws, (hipStream_t)stream);
        if (e == hipSuccess)
            e = prism::launch_scan_state(p, split_ws, (hipStream_t)stream);
        return from_hip(e);
    }
    if (use_bf16_kernel(d, p.dv_slice))
        return from_hip(prism::launch_scan_bf16(p, (hipStream_t)stream));
    return from_hip(prism::launch_scan(p, (hipStream_t)stream));
}

prism_status fwd_impl(const prism_dims* d, const void* q, const void* k, const void* v,
                      const void* u, const void* g, const void* b, const void* a, const void* h,
                      const void* conv_w, const int32_t* cu_seqlens, int L, int residual,
                      const float* S_init, const void* k_hist, void* o, float* S_final,
                      void* k_hist_out, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!dims_ok(d) || L < 1 || L > PRISM_MAX_LEVELS || !residual_ok(residual))
        return PRISM_EINVAL;
    if (!tok_ok(d, q) || !tok_ok(d, k) || !tok_ok(d, v) || !tok_ok(d, g) || !tok_ok(d, b) ||
        !ptr_ok(conv_w) || !ptr_ok(cu_seqlens) || !tok_ok(d, o) || !ptr_ok(S_final) ||
        !ptr_ok(workspace) || !opt_ok(S_init) || !opt_ok(k_hist) || !opt_ok(k_hist_out))
        return PRISM_EINVAL;
    if (L > 1 && (!tok_ok(d, u) || !tok_ok(d, a) || !tok_ok(d, h)))
        return PRISM_EINVAL;
    if (workspace_bytes < prism_workspace_bytes(d, L))
        return PRISM_EINVAL;
    prism_status st = check_scan_shape(d);
    if (st != PRISM_OK)
        return st;
    const int producers = use_fused_kw(d, L, residual, k_hist) ? 0 : kw_producers_for(d, L, residual, k_hist);
    if (use_fused_kw(d, L, residual, k_hist) || producers > 0) {
        FusedKw fk;
        fk.L = L;
        fk.u = u; fk.a = a; fk.h = h; fk.conv_w = conv_w;
        fk.producers = producers;
        fk.ready = reinterpret_cast<int*>(static_cast<unsigned char*>(workspace) + kw_bytes(d) +
                                          prism_scan_workspace_bytes(d));
        st = scan_impl(d, q, k, workspace, v, g, b, cu_seqlens, S_init, o, S_final,
                       static_cast<unsigned char*>(workspace) + kw_bytes(d), stream, fk);
    } else {
        st = prologue_impl(d, k, u, a, h, b, conv_w, k_hist, cu_seqlens, L, residual, workspace,
                           stream);
        if (st != PRISM_OK)
            return st;
        st = scan_impl(d, q, k, workspace, v, g, b, cu_seqlens, S_init, o, S_final,
                       static_cast<unsigned char*>(workspace) + kw_bytes(d), stream);
    }
    if (st != PRISM_OK || !k_hist_out)
        return st;
    // after the prologue on the same stream: k_hist_out may be k_hist itself
    return from_hip(prism::launch_k_history(d->dtype == PRISM_BF16, d->n_seqs, d->heads, d->dk,
                                            k, k_hist, cu_seqlens, k_hist_out,
                                            (hipStream_t)stream));
}

}  // namespace

extern "C" {

int prism_abi_version(void) { return PRISM_ABI_VERSION; }

const char* prism_status_str(prism_status s)
{
    switch (s) {
    case PRISM_OK: return "ok";
    case PRISM_EINVAL: return "invalid argument";
    case PRISM_EUNSUPPORTED: return "unsupported shape or dtype";
    case PRISM_EHIP: return "HIP launch failed";
    case PRISM_ENOSPACE: return "workspace needed exceeds the library's static scratch";
    }
    return "unknown status";
}

size_t prism_scan_workspace_bytes(const prism_dims* d)
{
    if (!dims_ok(d))
        return 0;
    const int P = split_for(d);
    if (P >= 2)
        return prism::split_workspace_bytes(d->n_seqs, d->heads, d->dk, d->dv, d->total_tokens, P);
    if (use_two_pass(d))
        return round256(prism::gram_workspace_bytes(d->n_seqs, d->total_tokens, d->heads));
    return 0;
}

size_t prism_workspace_bytes(const prism_dims* d, int L)
{
    if (!dims_ok(d) || L < 1 || L > PRISM_MAX_LEVELS)
        return 0;
    return kw_bytes(d) + prism_scan_workspace_bytes(d) + kw_ready_bytes(d, L);
}

prism_status prism_prologue(const prism_dims* d, const void* k, const void* u, const void* a,
                            const void* h, const void* b, const void* conv_w,
                            const int32_t* cu_seqlens, int L, void* kw, void* stream)
{
    return prologue_impl(d, k, u, a, h, b, conv_w, nullptr, cu_seqlens, L, PRISM_RESIDUAL_LINEAR,
                         kw, stream);
}

prism_status prism_prologue_ex(const prism_dims* d, const void* k, const void* u, const void* a,
                               const void* h, const void* b, const void* conv_w,
                               const void* k_hist, const int32_t* cu_seqlens, int L, int residual,
                               void* kw, void* stream)
{
    return prologue_impl(d, k, u, a, h, b, conv_w, k_hist, cu_seqlens, L, residual, kw, stream);
}

prism_status prism_scan(const prism_dims* d, const void* q, const void* k, const void* kw,
                        const void* v, const void* g, const void* b, const int32_t* cu_seqlens,
                        void* o, float* S_final, void* stream)
{
    return scan_impl(d, q, k, kw, v, g, b, cu_seqlens, nullptr, o, S_final, nullptr, stream);
}

prism_status prism_scan_ex(const prism_dims* d, const void* q, const void* k, const void* kw,
                           const void* v, const void* g, const void* b, const int32_t* cu_seqlens,
                           const float* S_init, void* o, float* S_final, void* workspace,
                           size_t workspace_bytes, void* stream)
{
    if (!dims_ok(d))
        return PRISM_EINVAL;
    const size_t need = prism_scan_workspace_bytes(d);
    if (need > 0 && (!ptr_ok(workspace) || workspace_bytes < need))
        return PRISM_EINVAL;
    return scan_impl(d, q, k, kw, v, g, b, cu_seqlens, S_init, o, S_final,
                     need > 0 ? workspace : nullptr, stream);
}

prism_status prism_fwd(const prism_dims* d, const void* q, const void* k, const void* v,
                       const void* u, const void* g, const void* b, const void* a,
                       const void* h, const void* conv_w, const int32_t* cu_seqlens, int L,
                       void* o, float* S_final, void* workspace, size_t workspace_bytes,
                       void* stream)
{
    return fwd_impl(d, q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L, PRISM_RESIDUAL_LINEAR,
                    nullptr, nullptr, o, S_final, nullptr, workspace, workspace_bytes, stream);
}

prism_status prism_fwd_noalloc(const prism_dims* d, const void* q, const void* k, const void* v,
                               const void* u, const void* g, const void* b, const void* a,
                               const void* h, const void* conv_w, const int32_t* cu_seqlens,
                               int L, void* o, float* S_final, void* stream)
{
    if (!dims_ok(d) || L < 1 || L > PRISM_MAX_LEVELS)
        return PRISM_EINVAL;
    const size_t need = prism_workspace_bytes(d, L);
    if (need > (size_t)PRISM_NOALLOC_MAX_BYTES)
        return PRISM_ENOSPACE;
    void* ws = scratch_ptr();
    if (!ws)
        return PRISM_EHIP;
    return fwd_impl(d, q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L, PRISM_RESIDUAL_LINEAR,
                    nullptr, nullptr, o, S_final, nullptr, ws, (size_t)PRISM_NOALLOC_MAX_BYTES,
                    stream);
}

prism_status prism_fwd_resume(const prism_dims* d, const void* q, const void* k, const void* v,
                              const void* u, const void* g, const void* b, const void* a,
                              const void* h, const void* conv_w, const int32_t* cu_seqlens,
                              int L, int residual, const float* S_init, const void* k_hist,
                              void* o, float* S_final, void* k_hist_out, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    return fwd_impl(d, q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L, residual, S_init, k_hist, o,
                    S_final, k_hist_out, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Chunkwise backward (bf16, dk and dv in {64, 128}; PRISM_BWD_CHUNKED=0 selects
// the token walk instead): the forward state products again with every chunk's
// start state kept (bf16), the carried state gradient backwards chunk by chunk,
// then every input gradient of all chunks at once on MFMA, then the write-key
// chain backwards.  At the LM layer (B=8, T=2048, H=6, d=128) 0.64 ms against
// 3.5 ms for the token walk.
bool use_bwd_chunked(const prism_dims* d)
{
    return env_int("PRISM_BWD_CHUNKED", 1) == 1 && d->dtype == PRISM_BF16 &&
           (d->dk == 64 || d->dk == 128) && (d->dv == 64 || d->dv == 128) && d->total_tokens > 0;
}

// Workspace of the chunkwise backward after kw, each part 256-byte aligned.
struct BwdChunkLayout {
    size_t mats, ck, ckT, dck, dckT, dkw, wk, total;
};

// Bytes of one of the two checkpoint arrays (bf16 chunk-start states [nv, H, dk, dv]
// and their transposes), 256-byte rounded; 0 where the chunkwise backward does not
// serve the shape (it is bf16 with dk, dv in {64, 128}).
size_t checkpoint_half(const prism_dims* d)
{
    if (d->dtype != PRISM_BF16 || !prism::bwd_supported(d->dk, d->dv))
        return 0;
    return round256((size_t)(d->total_tokens / 64 + d->n_seqs) * d->heads * d->dk * d->dv * 2);
}

// The checkpoints of prism_fwd_ckpt: the chunk-start states, their transposes
// and the write keys kw, each part 256-byte aligned; 0 where they do not serve.
size_t checkpoint_total(const prism_dims* d)
{
    const size_t half = checkpoint_half(d);
    return half ? 2 * half + kw_bytes(d) : 0;
}

BwdChunkLayout bwd_chunk_layout(const prism_dims* d)
{
    BwdChunkLayout w;
    const size_t nv = (size_t)(d->total_tokens / 64 + d->n_seqs) * d->heads;    // (virtual chunk, head)
    const size_t st = round256(nv * d->dk * d->dv * 2);
    size_t o = kw_bytes(d);
    w.mats = o; o += round256(prism::gram_workspace_bytes(d->n_seqs, d->total_tokens, d->heads));
    w.ck = o; o += st;
    w.ckT = o; o += st;
    w.dck = o; o += st;
    w.dckT = o; o += st;
    w.dkw = o; o += round256((size_t)d->total_tokens * d->heads * d->dk * 4);
    w.wk = o; o += round256(prism::wk_workspace_floats(d->total_tokens, d->heads, d->dk) * 4);
    w.total = o;
    return w;
}

}  // namespace

extern "C" {

size_t prism_bwd_workspace_bytes(const prism_dims* d, int L)
{
    if (!dims_ok(d) || L < 1 || L > PRISM_MAX_LEVELS)
        return 0;
    if (use_bwd_chunked(d))
        return bwd_chunk_layout(d).total;
    return kw_bytes(d) + prism::bwd_workspace_floats(d->n_seqs, d->total_tokens, d->heads, d->dk,
                                                     d->dv) * sizeof(float);
}

}  // extern "C"

namespace {

// The backward pass; with ckpt (prism_fwd_ckpt's chunk-start states and write
// keys of the same inputs) the chunkwise form reads them instead of recomputing
// them, and may store dq, dk, dv, du, da, dh in bf16 (grad_dtype PRISM_BF16).
prism_status bwd_impl(const prism_dims* d, const void* q, const void* k, const void* v,
                      const void* u, const void* g, const void* b, const void* a, const void* h,
                      const void* conv_w, const int32_t* cu_seqlens, int L, int residual,
                      int grad_dtype, const float* S_init, const void* dO, const float* dS_final,
                      void* dq, void* dk, void* dv, void* du, float* dg, float* db, void* da,
                      void* dh, float* dconv_w, float* dS_init, const void* ckpt, void* workspace,
                      size_t workspace_bytes, void* stream)
{
    if (!dims_ok(d) || L < 1 || L > PRISM_MAX_LEVELS || !residual_ok(residual) ||
        (grad_dtype != PRISM_F32 && grad_dtype != PRISM_BF16))
        return PRISM_EINVAL;
    if (!tok_ok(d, q) || !tok_ok(d, k) || !tok_ok(d, v) || !tok_ok(d, g) || !tok_ok(d, b) ||
        !tok_ok(d, dO) || !ptr_ok(conv_w) || !ptr_ok(cu_seqlens) || !tok_ok(d, dq) ||
        !tok_ok(d, dk) || !tok_ok(d, dv) || !tok_ok(d, dg) || !tok_ok(d, db) || !ptr_ok(dconv_w) ||
        !ptr_ok(workspace) || !opt_ok(S_init) || !opt_ok(dS_final) || !opt_ok(dS_init))
        return PRISM_EINVAL;
    if (L > 1 && (!tok_ok(d, u) || !tok_ok(d, a) || !tok_ok(d, h) || !tok_ok(d, du) ||
                  !tok_ok(d, da) || !tok_ok(d, dh)))
        return PRISM_EINVAL;
    if (!prism::bwd_supported(d->dk, d->dv))
        return PRISM_EUNSUPPORTED;
    if (workspace_bytes < prism_bwd_workspace_bytes(d, L))
        return PRISM_EINVAL;
    if (ckpt && !use_bwd_chunked(d))             // checkpoints serve the chunkwise form only
        return PRISM_EUNSUPPORTED;
    // bf16 gradients: the chunkwise form with checkpoints, whose unused state
    // region of the workspace then holds the scan's fp32 part of dk
    const bool grad_bf16 = grad_dtype == PRISM_BF16;
    if (grad_bf16 && !ckpt)
        return PRISM_EUNSUPPORTED;
    // the write keys: prism_fwd_ckpt's, after the two state arrays, or recomputed
    // into the workspace
    void* kwp = ckpt ? static_cast<unsigned char*>(const_cast<void*>(ckpt)) + 2 * checkpoint_half(d)
                     : workspace;
    if (!ckpt) {
        const prism_status st = prologue_impl(d, k, u, a, h, b, conv_w, nullptr, cu_seqlens, L,
                                              residual, workspace, stream);
        if (st != PRISM_OK)
            return st;
    }
    prism::BwdArgs p;
    p.bf16 = d->dtype == PRISM_BF16;
    p.n_seqs = d->n_seqs;
    p.total_tokens = d->total_tokens;
    p.heads = d->heads;
    p.dk = d->dk;
    p.dv = d->dv;
    p.L = L;
    p.gelu = residual == PRISM_RESIDUAL_GELU;
    p.q = q; p.k = k; p.v = v; p.kw = kwp; p.u = u; p.a = a; p.h = h; p.g = g; p.b = b;
    p.conv_w = conv_w;
    p.dO = dO;
    p.cu_seqlens = cu_seqlens;
    p.s_init = S_init;
    p.ds_final = dS_final;
    // typed fp32 here; they hold bf16 when grad_bf16 (the chunkwise path only)
    p.gq = static_cast<float*>(dq); p.gk = static_cast<float*>(dk); p.gv = static_cast<float*>(dv);
    p.gu = static_cast<float*>(du); p.ga = static_cast<float*>(da); p.gh = static_cast<float*>(dh);
    p.gg = dg; p.gb = db;
    p.gconv = dconv_w;
    p.gs_init = dS_init;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    if (!use_bwd_chunked(d)) {
        p.ws = reinterpret_cast<float*>(ws + kw_bytes(d));
        return from_hip(prism::launch_bwd(p, (hipStream_t)stream));
    }
    const BwdChunkLayout w = bwd_chunk_layout(d);
    prism::ScanArgs sp;
    sp.bf16 = true;
    sp.n_seqs = d->n_seqs;
    sp.total_tokens = d->total_tokens;
    sp.heads = d->heads;
    sp.dk = d->dk;
    sp.dv = d->dv;
    sp.dv_slice = 32;
    sp.specialised = false;
    sp.ws_waves = 8;
    sp.q = q; sp.k = k; sp.kw = kwp; sp.v = v; sp.g = g; sp.b = b;
    sp.cu_seqlens = cu_seqlens;
    sp.s_init = S_init;
    sp.o = nullptr;
    sp.s_final = nullptr;
    prism::BwdChunkBufs cb;
    cb.dO = dO;
    cb.mats = ws + w.mats;
    // the chunk-start states: recomputed below, or prism_fwd_ckpt's checkpoints
    const unsigned char* ckb = static_cast<const unsigned char*>(ckpt);
    cb.ck = ckpt ? (const void*)ckb : (const void*)(ws + w.ck);
    cb.ckT = ckpt ? (const void*)(ckb + checkpoint_half(d)) : (const void*)(ws + w.ckT);
    cb.dck = ws + w.dck; cb.dckT = ws + w.dckT;
    cb.gq = dq; cb.gv = dv;
    cb.gk = grad_bf16 ? reinterpret_cast<float*>(ws + w.ck) : static_cast<float*>(dk);
    cb.gkw = reinterpret_cast<float*>(ws + w.dkw);
    cb.gg = dg; cb.gb = db;
    cb.grad_bf16 = grad_bf16;
    p.grad_bf16 = grad_bf16;
    p.gk_part = cb.gk;
    const hipStream_t s = (hipStream_t)stream;
    hipError_t e = prism::launch_gram(sp, ws + w.mats, s);
    if (e == hipSuccess && !ckpt)
        e = prism::launch_scan_state(sp, ws + w.mats, s, ws + w.ck, ws + w.ckT);
    if (e == hipSuccess)
        e = prism::launch_bwd_state(sp, dO, ws + w.mats, dS_final, ws + w.dck, ws + w.dckT, dS_init, s);
    if (e == hipSuccess)
        e = prism::launch_bwd_grads(sp, cb, s);
    if (e == hipSuccess)
        e = prism::launch_write_key_bwd(p, cb.gkw, reinterpret_cast<float*>(ws + w.wk), s);
    return from_hip(e);
}

// The forward pass that also keeps every chunk's start state and the write keys
// for the chunkwise backward: the prologue (kw into the checkpoints), then the
// eight-wavefront bf16 scan over whole sequences (no segment split: its segments
// start from zero), whose state wavefronts store the chunk-start states.  The
// workspace is not used.
prism_status fwd_ckpt_impl(const prism_dims* d, const void* q, const void* k, const void* v,
                           const void* u, const void* g, const void* b, const void* a, const void* h,
                           const void* conv_w, const int32_t* cu_seqlens, int L, int residual,
                           const float* S_init, void* o, float* S_final, void* ckpt,
                           void* workspace, size_t workspace_bytes, void* stream)
{
    if (!dims_ok(d) || L < 1 || L > PRISM_MAX_LEVELS || !residual_ok(residual))
        return PRISM_EINVAL;
    if (!tok_ok(d, q) || !tok_ok(d, k) || !tok_ok(d, v) || !tok_ok(d, g) || !tok_ok(d, b) ||
        !ptr_ok(conv_w) || !ptr_ok(cu_seqlens) || !tok_ok(d, o) || !ptr_ok(S_final) ||
        !ptr_ok(ckpt) || !opt_ok(S_init))
        return PRISM_EINVAL;
    if (L > 1 && (!tok_ok(d, u) || !tok_ok(d, a) || !tok_ok(d, h)))
        return PRISM_EINVAL;
    (void)workspace;
    (void)workspace_bytes;
    if (checkpoint_half(d) == 0 || !use_bf16_kernel(d, 32) || !ws8_enabled() ||
        env_int("PRISM_SCAN_SPECIALISED", 1) == 0 || env_int("PRISM_SCAN_WAVES", 8) == 4)
        return PRISM_EUNSUPPORTED;
    unsigned char* ckb = static_cast<unsigned char*>(ckpt);
    void* kwp = ckb + 2 * checkpoint_half(d);
    prism_status st = prologue_impl(d, k, u, a, h, b, conv_w, nullptr, cu_seqlens, L, residual,
                                    kwp, stream);
    if (st != PRISM_OK)
        return st;
    prism::ScanArgs p;
    p.bf16 = true;
    p.n_seqs = d->n_seqs;
    p.total_tokens = d->total_tokens;
    p.heads = d->heads;
    p.dk = d->dk;
    p.dv = d->dv;
    p.dv_slice = 32;
    p.specialised = true;
    p.ws_waves = 8;
    p.q = q; p.k = k; p.kw = kwp; p.v = v; p.g = g; p.b = b;
    p.cu_seqlens = cu_seqlens;
    p.s_init = S_init;
    p.o = o;
    p.s_final = S_final;
    p.ck = ckb;
    p.ckT = ckb + checkpoint_half(d);
    return from_hip(prism::launch_scan_bf16(p, (hipStream_t)stream));
}

}  // namespace

extern "C" {

size_t prism_checkpoint_bytes(const prism_dims* d)
{
    return dims_ok(d) ? checkpoint_total(d) : 0;
}

prism_status prism_fwd_ckpt(const prism_dims* d, const void* q, const void* k, const void* v,
                            const void* u, const void* g, const void* b, const void* a,
                            const void* h, const void* conv_w, const int32_t* cu_seqlens, int L,
                            int residual, const float* S_init, void* o, float* S_final,
                            void* checkpoints, void* workspace, size_t workspace_bytes, void* stream)
{
    return fwd_ckpt_impl(d, q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L, residual, S_init, o,
                         S_final, checkpoints, workspace, workspace_bytes, stream);
}

prism_status prism_bwd_ckpt(const prism_dims* d, const void* q, const void* k, const void* v,
                            const void* u, const void* g, const void* b, const void* a, const void* h,
                            const void* conv_w, const int32_t* cu_seqlens, int L, int residual,
                            int grad_dtype, const float* S_init, const void* dO,
                            const float* dS_final, void* dq, void* dk, void* dv, void* du,
                            float* dg, float* db, void* da, void* dh, float* dconv_w,
                            float* dS_init, const void* checkpoints, void* workspace,
                            size_t workspace_bytes, void* stream)
{
    if (!ptr_ok(checkpoints))
        return PRISM_EINVAL;
    if (checkpoint_half(d) == 0)
        return PRISM_EUNSUPPORTED;
    return bwd_impl(d, q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L, residual, grad_dtype, S_init,
                    dO, dS_final, dq, dk, dv, du, dg, db, da, dh, dconv_w, dS_init, checkpoints,
                    workspace, workspace_bytes, stream);
}

prism_status prism_bwd_ex(const prism_dims* d, const void* q, const void* k, const void* v,
                          const void* u, const void* g, const void* b, const void* a, const void* h,
                          const void* conv_w, const int32_t* cu_seqlens, int L, int residual,
                          const float* S_init, const void* dO, const float* dS_final, float* dq,
                          float* dk, float* dv, float* du, float* dg, float* db, float* da,
                          float* dh, float* dconv_w, float* dS_init, void* workspace,
                          size_t workspace_bytes, void* stream)
{
    return bwd_impl(d, q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L, residual, PRISM_F32, S_init, dO,
                    dS_final, dq, dk, dv, du, dg, db, da, dh, dconv_w, dS_init, nullptr, workspace,
                    workspace_bytes, stream);
}

prism_status prism_bwd(const prism_dims* d, const void* q, const void* k, const void* v,
                       const void* u, const void* g, const void* b, const void* a, const void* h,
                       const void* conv_w, const int32_t* cu_seqlens, int L, const float* S_init,
                       const void* dO, const float* dS_final, float* dq, float* dk, float* dv,
                       float* du, float* dg, float* db, float* da, float* dh, float* dconv_w,
                       float* dS_init, void* workspace, size_t workspace_bytes, void* stream)
{
    return prism_bwd_ex(d, q, k, v, u, g, b, a, h, conv_w, cu_seqlens, L, PRISM_RESIDUAL_LINEAR,
                        S_init, dO, dS_final, dq, dk, dv, du, dg, db, da, dh, dconv_w, dS_init,
                        workspace, workspace_bytes, stream);
}

prism_status prism_scan_wait_giveups(unsigned int* count, int reset)
{
    if (!count)
        return PRISM_EINVAL;
    return from_hip(prism::read_wait_giveups(count, reset != 0));
}

prism_status prism_decode_step(const prism_dims* d, const void* q, const void* k, const void* v,
                               const void* u, const void* g, const void* b, const void* a,
                               const void* h, const void* conv_w, int L, int residual, float* S,
                               void* k_hist, void* o, void* stream)
{
    if (!dims_ok(d) || L < 1 || L > PRISM_MAX_LEVELS || d->total_tokens != d->n_seqs ||
        !residual_ok(residual))
        return PRISM_EINVAL;
    if (!ptr_ok(q) || !ptr_ok(k) || !ptr_ok(v) || !ptr_ok(g) || !ptr_ok(b) || !ptr_ok(conv_w) ||
        !ptr_ok(S) || !ptr_ok(k_hist) || !ptr_ok(o))
        return PRISM_EINVAL;
    if (L > 1 && (!ptr_ok(u) || !ptr_ok(a) || !ptr_ok(h)))
        return PRISM_EINVAL;
    if (!prism::decode_supported(d->dk, d->dv))
        return PRISM_EUNSUPPORTED;
    prism::DecodeArgs p;
    p.bf16 = d->dtype == PRISM_BF16;
    p.n_seqs = d->n_seqs;
    p.heads = d->heads;
    p.dk = d->dk;
    p.dv = d->dv;
    p.L = L;
    p.gelu = residual == PRISM_RESIDUAL_GELU;
    p.q = q; p.k = k; p.v = v; p.u = u; p.a = a; p.h = h; p.g = g; p.b = b;
    p.conv_w = conv_w;
    p.S = S;
    p.k_hist = k_hist;
    p.o = o;
    return from_hip(prism::launch_decode(p, (hipStream_t)stream));
}

}  // extern "C"
