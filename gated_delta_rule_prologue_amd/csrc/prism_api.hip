// prism_api.hip -- C ABI of libprism (declared in include/prism.h): argument
// validation, kernel selection and launches on the caller's stream.
#include <stdint.h>
#include <stdlib.h>

#include "prism.h"
#include "kernels.h"

namespace {

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

prism_status check_scan_shape(const prism_dims* d)
{
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

prism_status scan_impl(const prism_dims* d, const void* q, const void* k, const void* kw,
                       const void* v, const void* g, const void* b, const int32_t* cu_seqlens,
                       const float* S_init, void* o, float* S_final, void* split_ws, void* stream)
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
    const int P = split_ws ? split_for(d) : 1;
    if (P >= 2)
        return from_hip(prism::launch_split_scan(p, P, split_ws, (hipStream_t)stream));
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
    st = prologue_impl(d, k, u, a, h, b, conv_w, k_hist, cu_seqlens, L, residual, workspace,
                       stream);
    if (st != PRISM_OK)
        return st;
    st = scan_impl(d, q, k, workspace, v, g, b, cu_seqlens, S_init, o, S_final,
                   static_cast<unsigned char*>(workspace) + kw_bytes(d), stream);
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
    }
    return "unknown status";
}

size_t prism_scan_workspace_bytes(const prism_dims* d)
{
    if (!dims_ok(d))
        return 0;
    return prism::split_workspace_bytes(d->n_seqs, d->heads, d->dk, d->dv, d->total_tokens,
                                        split_for(d));
}

size_t prism_workspace_bytes(const prism_dims* d, int L)
{
    if (!dims_ok(d) || L < 1 || L > PRISM_MAX_LEVELS)
        return 0;
    return kw_bytes(d) + prism_scan_workspace_bytes(d);
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

size_t prism_bwd_workspace_bytes(const prism_dims* d, int L)
{
    if (!dims_ok(d) || L < 1 || L > PRISM_MAX_LEVELS)
        return 0;
    return kw_bytes(d) + prism::bwd_workspace_floats(d->n_seqs, d->total_tokens, d->heads, d->dk,
                                                     d->dv) * sizeof(float);
}

prism_status prism_bwd_ex(const prism_dims* d, const void* q, const void* k, const void* v,
                          const void* u, const void* g, const void* b, const void* a, const void* h,
                          const void* conv_w, const int32_t* cu_seqlens, int L, int residual,
                          const float* S_init, const void* dO, const float* dS_final, float* dq,
                          float* dk, float* dv, float* du, float* dg, float* db, float* da,
                          float* dh, float* dconv_w, float* dS_init, void* workspace,
                          size_t workspace_bytes, void* stream)
{
    if (!dims_ok(d) || L < 1 || L > PRISM_MAX_LEVELS || !residual_ok(residual))
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
    prism_status st = prologue_impl(d, k, u, a, h, b, conv_w, nullptr, cu_seqlens, L, residual,
                                    workspace, stream);
    if (st != PRISM_OK)
        return st;
    prism::BwdArgs p;
    p.bf16 = d->dtype == PRISM_BF16;
    p.n_seqs = d->n_seqs;
    p.total_tokens = d->total_tokens;
    p.heads = d->heads;
    p.dk = d->dk;
    p.dv = d->dv;
    p.L = L;
    p.gelu = residual == PRISM_RESIDUAL_GELU;
    p.q = q; p.k = k; p.v = v; p.kw = workspace; p.u = u; p.a = a; p.h = h; p.g = g; p.b = b;
    p.conv_w = conv_w;
    p.dO = dO;
    p.cu_seqlens = cu_seqlens;
    p.s_init = S_init;
    p.ds_final = dS_final;
    p.gq = dq; p.gk = dk; p.gv = dv; p.gu = du; p.ga = da; p.gh = dh; p.gg = dg; p.gb = db;
    p.gconv = dconv_w;
    p.gs_init = dS_init;
    p.ws = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + kw_bytes(d));
    return from_hip(prism::launch_bwd(p, (hipStream_t)stream));
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
