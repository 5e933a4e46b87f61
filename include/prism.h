/*
 * prism.h -- C ABI of libprism: the forward pass of PRISM's memory-writing
 * operator on AMD Instinct MI355X (gfx950).
 *
 * The operator (PRISM: Parallel Residual Iterative Sequence Model) keeps, per
 * (sequence, head), a state S in R^{dk x dv} that starts at zero (or at a
 * carried state, prism_fwd_resume and prism_decode_step) and, for each token t
 * of the sequence,
 *
 *   r_0   = causal depthwise ShortConv(width 4) of k at t       (local anchor)
 *   r_1   = r_0,  r_l = r_0 * prod_{j=1..l-1} (1 - a_j * h_j)   (residual chain, closed form)
 *   kw_t  = b_t k_t + sum_{l=1..L-1} a_l * r_l * u_l             (write key)
 *   S_t   = g_t (I - b_t k_t k_t^T) S_{t-1} + kw_t v_t^T         (GDN forget/erase + write)
 *   o_t   = S_t^T q_t
 *
 * ("*" is element-wise over the dk channel.)  Sources, all on the PRISM
 * pages: ICML 2026 PRISM summary (WeChat article), sections 核心迭代形式
 * (multi-step write), 消除 Token 间串行 (GDN forget, ShortConv anchor),
 * 消除 Step 间串行 (closed-form residual chain) and 架构形式 (L = 1 is GDN);
 * gist.science technical summary of arXiv 2602.10796, sections 2.1-2.2;
 * ICML 2026 poster abstract (the short convolution anchors the initial
 * residual).  Readings where the pages are silent: the residual product runs
 * over j = 1..l-1 (so h's last slot is never read); conv tap 3 multiplies the
 * current token, taps before a sequence start read zero, no bias, no
 * activation; g and b are per (token, head) scalars, g in linear space; no
 * query scaling; zero initial state.
 *
 * Conventions for every entry point
 *   - Tensors are dense, row-major, DEVICE pointers owned by the caller; the
 *     library never allocates, frees or retains them.  They must stay valid
 *     until the work queued on `stream` has finished.
 *   - Float inputs share one dtype (prism_dims.dtype): IEEE fp32, or bf16 as
 *     raw 16-bit patterns.  Outputs o and kw use that dtype; S_final is fp32.
 *   - Every pointer must be non-null and 16-byte aligned, except that the per-token
 *     arrays (q, k, v, u, a, h, g, b, o, kw) may be NULL when total_tokens == 0.
 *     cu_seqlens is int32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous: they enqueue kernels and return; no host synchronisation
 *     and no device-to-host copy happens inside.
 *   - Errors are return codes; nothing is thrown across the boundary.  All
 *     argument checks happen before any launch, so an error return means that
 *     nothing was enqueued.  A failed launch returns PRISM_EHIP.
 *   - Preconditions not checked (they live in device memory): cu_seqlens is
 *     non-decreasing, cu_seqlens[0] = 0 and cu_seqlens[n_seqs] = total_tokens.
 *   - The library keeps no state between calls and is re-entrant; calls on
 *     different streams may overlap if their output buffers do not.
 */
#ifndef PRISM_H
#define PRISM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Other shapes return PRISM_EUNSUPPORTED.  Gates: 0 <= g <= 1 (values below
 * 1e-30 act as 1e-30: the scan works with log2 g). */
typedef enum {
    PRISM_OK = 0,
    PRISM_EINVAL = 1,          /* null/misaligned pointer, bad size, L out of range */
    PRISM_EUNSUPPORTED = 2,    /* valid but not implemented here (e.g. dk not in {64, 128}) */
    PRISM_EHIP = 3,            /* a HIP launch failed */
    PRISM_ENOSPACE = 4         /* prism_fwd_noalloc: the shape needs more than the static scratch */
} prism_status;

typedef enum { PRISM_F32 = 0, PRISM_BF16 = 1 } prism_dtype;

/* Form of the residual chain of the write key (the `residual` argument).
 *   PRISM_RESIDUAL_LINEAR  r_l = r_0 * prod_{j=1..l-1} (1 - a_j * h_j): the GELU of the
 *                          refinement step absorbed into the gain, giving an element-wise
 *                          linear recurrence with a closed form (WeChat page section
 *                          消除 Step 间串行).  This is what prism_fwd computes.
 *   PRISM_RESIDUAL_GELU    r_1 = r_0, r_{l+1} = r_l - a_l * GELU(h_l * r_l), GELU(x) = x Phi(x):
 *                          the refinement step with its non-linearity kept (gist.science
 *                          summary, section 2.2: delta = GELU(gain * residual), one step-size
 *                          gate per level).  Identical to the linear form for L <= 2. */
typedef enum { PRISM_RESIDUAL_LINEAR = 0, PRISM_RESIDUAL_GELU = 1 } prism_residual;

typedef struct {
    int32_t n_seqs;        /* number of packed sequences, >= 1 */
    int32_t total_tokens;  /* T = cu_seqlens[n_seqs], >= 0 */
    int32_t heads;         /* H >= 1 */
    int32_t dk;            /* key width   (prism_fwd / prism_scan: 64 or 128) */
    int32_t dv;            /* value width (prism_fwd / prism_scan: 64 or 128) */
    int32_t dtype;         /* prism_dtype of every float input */
} prism_dims;

#define PRISM_MAX_LEVELS 16

/* Bytes of device workspace prism_fwd (and prism_fwd_resume) needs: the write
 * keys kw [T, H, dk] in the input dtype, rounded up to 256 bytes, plus
 * prism_scan_workspace_bytes(d), plus, when the in-scan write-key producers
 * are requested (PRISM_KW_PRODUCERS=1 in the environment of the size query and
 * of the call), for bf16 inputs with T > 0 at the shapes they serve (dk and dv
 * 64 or 128, L = 4; also L = 8 at dk = 64), their readiness flags:
 * 4 (floor(T / 64) + n_seqs) H bytes rounded up to 256.  Returns 0 for
 * invalid dims or L. */
size_t prism_workspace_bytes(const prism_dims* d, int L);

/*
 * Full forward pass: prologue then chunkwise scan, both on `stream`.  With
 * PRISM_KW_PRODUCERS=1, for bf16 inputs with the closed-form chain at the
 * shapes above, when the scan's workgroups leave at least eight compute units
 * idle, the prologue runs inside the scan launch instead: producer workgroups
 * on the idle compute units form the write keys chunk by chunk while the scan
 * runs, and the scan reads each chunk's keys once they are flagged.  Both
 * evaluate the same formulas; results agree up to rounding order.
 *
 *   q, k         [T, H, dk]
 *   v            [T, H, dv]
 *   u, a, h      [T, H, L-1, dk]  slot s holds level l = s + 1; NULL allowed iff L == 1
 *   g, b         [T, H]           forget gate (linear space) and erase/write strength
 *   conv_w       [H, dk, 4]       ShortConv taps; tap 3 multiplies token t, tap m token t-3+m
 *   cu_seqlens   [n_seqs + 1]     int32 device array of sequence offsets
 *   L            levels, 1..PRISM_MAX_LEVELS; L == 1 is exactly Gated DeltaNet
 *   o            out [T, H, dv], input dtype
 *   S_final      out fp32 [n_seqs, H, dk, dv], the state after each sequence's last token
 *                (zero for an empty sequence)
 *   workspace    device buffer of at least prism_workspace_bytes(d, L) bytes
 *
 * Sources: see the header comment above.
 */
prism_status prism_fwd(const prism_dims* d,
                       const void* q, const void* k, const void* v,
                       const void* u, const void* g, const void* b,
                       const void* a, const void* h, const void* conv_w,
                       const int32_t* cu_seqlens, int L,
                       void* o, float* S_final,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * prism_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace prism_fwd would take lives instead in
 * a static device array of PRISM_NOALLOC_MAX_BYTES inside the library, one
 * per GPU, held from the first call on that GPU until the process ends; its
 * device address is looked up once per GPU on the first call there (that
 * first call is not capturable; later ones are).  The call itself allocates
 * nothing.
 *
 *   Arguments, layouts and results as in prism_fwd (the caller still provides
 *   every input and output buffer).
 *   PRISM_ENOSPACE when prism_workspace_bytes(d, L) exceeds
 *   PRISM_NOALLOC_MAX_BYTES (e.g. the LM layer B=8, T=2048, H=6, d=128 needs
 *   about 25 MB and fits; one 65,536-token sequence of 16 heads does not).
 *   PRISM_EHIP if the scratch address cannot be looked up.
 * Every call on one GPU uses the same scratch: calls that overlap on one GPU
 * (different streams, or host threads) race and must be serialised by the
 * caller.  The scratch keeps the last call's contents; every byte a call reads
 * from it is written earlier in the same call.
 */
#define PRISM_NOALLOC_MAX_BYTES (64u << 20)
prism_status prism_fwd_noalloc(const prism_dims* d,
                               const void* q, const void* k, const void* v,
                               const void* u, const void* g, const void* b,
                               const void* a, const void* h, const void* conv_w,
                               const int32_t* cu_seqlens, int L,
                               void* o, float* S_final, void* stream);

/*
 * Prologue only: the write keys kw [T, H, dk] (input dtype, rounded to
 * nearest-even for bf16), i.e. the ShortConv anchor, the closed-form
 * residual chain and the write-key sum (WeChat page sections 消除 Token 间串行
 * and 消除 Step 间串行; gist.science section 2.2).  Arguments as in prism_fwd.
 * dk may be any multiple of 8 (bf16) or 4 (fp32) here.
 */
prism_status prism_prologue(const prism_dims* d,
                            const void* k, const void* u, const void* a,
                            const void* h, const void* b, const void* conv_w,
                            const int32_t* cu_seqlens, int L,
                            void* kw, void* stream);

/*
 * Prologue with the options of the carried-state path: k_hist [n_seqs, H, 3, dk]
 * (or NULL = zero) supplies the three k rows before each sequence's first token
 * (see prism_fwd_resume), and `residual` (prism_residual) selects the form of
 * the residual chain.  Other arguments as in prism_prologue; a residual value
 * outside prism_residual returns PRISM_EINVAL.
 */
prism_status prism_prologue_ex(const prism_dims* d,
                               const void* k, const void* u, const void* a,
                               const void* h, const void* b, const void* conv_w,
                               const void* k_hist, const int32_t* cu_seqlens, int L,
                               int residual, void* kw, void* stream);

/*
 * Scan only, from precomputed write keys kw [T, H, dk] (input dtype): the
 * gated delta-rule state recurrence S_t = g_t (I - b_t k_t k_t^T) S_{t-1} +
 * kw_t v_t^T, o_t = S_t^T q_t (WeChat page section 消除 Token 间串行: forget
 * identical to GDN; gist.science section 2.1: S_t = S_{t-1} A_t + B_t with an
 * input-only write), evaluated in chunks of 64 tokens (fp32 inputs at
 * dk = 128: token by token, whose fp32 chunk tiles would not fit the on-chip
 * memory).  Other arguments as in prism_fwd.
 */
prism_status prism_scan(const prism_dims* d,
                        const void* q, const void* k, const void* kw, const void* v,
                        const void* g, const void* b, const int32_t* cu_seqlens,
                        void* o, float* S_final, void* stream);

/*
 * Forward pass that continues sequences from an earlier call: the same
 * operator as prism_fwd, started from a carried state and convolution history
 * instead of zeros.  The state matrix holds a sequence's whole history in a
 * fixed size and is updated one token at a time (WeChat page section
 * 背景：无限背包 vs 有限背包; poster page, lay summary), so a sequence split into
 * pieces and run piece by piece, carrying S_final and k_hist_out of one call
 * into S_init and k_hist of the next, gives the outputs of one call over the
 * whole sequence (up to rounding).
 *
 *   S_init      fp32 [n_seqs, H, dk, dv] state before each sequence's first token,
 *               or NULL (zero).  May be the same buffer as S_final (in-place update).
 *   k_hist      [n_seqs, H, 3, dk] input dtype: the three k rows before each
 *               sequence's first token, oldest first (slot 2 is the token just
 *               before it); the ShortConv taps before the sequence start read
 *               them instead of zero.  NULL = zero.
 *   k_hist_out  [n_seqs, H, 3, dk] or NULL (not written): the history to carry
 *               on, i.e. the last three k rows of each sequence, with k_hist
 *               (or zero) filling in for sequences shorter than three tokens.
 *               May be the same buffer as k_hist.
 *   residual    prism_residual: the closed-form chain of prism_fwd or the GELU chain.
 * Other arguments, shapes and errors as in prism_fwd; the optional pointers
 * must be 16-byte aligned when given.
 */
prism_status prism_fwd_resume(const prism_dims* d,
                              const void* q, const void* k, const void* v,
                              const void* u, const void* g, const void* b,
                              const void* a, const void* h, const void* conv_w,
                              const int32_t* cu_seqlens, int L, int residual,
                              const float* S_init, const void* k_hist,
                              void* o, float* S_final, void* k_hist_out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step: exactly one new token for each of the n_seqs sequences
 * (d->total_tokens must equal d->n_seqs; no cu_seqlens), run through the
 * recurrence in its token-by-token form with the state and the convolution
 * history updated in place (WeChat page sections 背景：无限背包 vs 有限背包 and
 * 消除 Token 间串行; gist.science section 2.1, S_t = S_{t-1} A_t + B_t).
 *
 *   q, k        [n_seqs, H, dk]       the new token of each sequence
 *   v           [n_seqs, H, dv]
 *   u, a, h     [n_seqs, H, L-1, dk]  NULL allowed iff L == 1
 *   g, b        [n_seqs, H]
 *   conv_w      [H, dk, 4]
 *   S           fp32 [n_seqs, H, dk, dv], in/out: the state before the token,
 *               replaced by the state after it
 *   k_hist      [n_seqs, H, 3, dk] input dtype, in/out: the three k rows before
 *               the token (oldest first), replaced by the three ending with it
 *   o           out [n_seqs, H, dv], input dtype
 *   residual    prism_residual (form of the residual chain)
 * All pointers non-null and 16-byte aligned (u, a, h may be NULL when L == 1).
 * dk and dv in {64, 128}, else PRISM_EUNSUPPORTED.  The write key is kept in
 * fp32 here (prism_fwd rounds it to the input dtype between its two kernels).
 * A sequence of decode steps equals prism_fwd_resume over the same tokens.
 */
prism_status prism_decode_step(const prism_dims* d,
                               const void* q, const void* k, const void* v,
                               const void* u, const void* g, const void* b,
                               const void* a, const void* h, const void* conv_w, int L,
                               int residual, float* S, void* k_hist, void* o, void* stream);

/*
 * Scan only, with the options of the full forward pass: a start state S_init
 * (fp32 [n_seqs, H, dk, dv], NULL = zero; may be S_final) and a device
 * workspace of prism_scan_workspace_bytes(d) bytes (NULL allowed when that is
 * 0).  With few, long sequences (too few (sequence, head) chains to occupy
 * the GPU) each sequence is cut into segments that are scanned side by side
 * from zero, together with scans of their transitions alone; the segments are
 * then chained through the transitions and the carried state is added to
 * the outputs.  The recurrence is affine in the state (gist.science section
 * 2.1: S_t = S_{t-1} A_t + B_t with input-only A_t, B_t), so this changes the
 * result only by rounding.  The workspace holds those segment buffers.
 * prism_fwd and prism_fwd_resume run this scan.  Other arguments as in
 * prism_scan.
 */
prism_status prism_scan_ex(const prism_dims* d,
                           const void* q, const void* k, const void* kw, const void* v,
                           const void* g, const void* b, const int32_t* cu_seqlens,
                           const float* S_init, void* o, float* S_final,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace prism_scan_ex needs for the shape (0: no segment
 * split for it).  Depends on the current device's compute-unit count and on
 * PRISM_SPLIT (0 = never split, P >= 2 = always P segments).  Returns 0 for
 * invalid dims. */
size_t prism_scan_workspace_bytes(const prism_dims* d);

/*
 * Backward pass of prism_fwd with the closed-form residual chain: the fp32
 * gradients of the loss  sum_t <dO_t, o_t> + <dS_final, S_final>  with respect
 * to every input, by reverse-mode differentiation of the token recurrence
 * (WeChat page sections 核心迭代形式, 消除 Token 间串行, 消除 Step 间串行;
 * gist.science section 2.1).  The write keys are recomputed by the prologue.
 * bf16 inputs: the gradients come from the chunkwise (UT / WY) form of the
 * recurrence that the forward evaluates (WeChat page section 消除 Token 间串行):
 * the per-chunk products are recomputed with every 64-token chunk's start
 * state kept in bf16, the state gradient is carried backwards chunk by chunk,
 * and every other gradient of all chunks is formed at once on the matrix
 * cores; the workspace holds about H * (20 KB + 8 B * dk * dv) per chunk and
 * H * (6 dk + 4 dv + 12) bytes per token.  fp32 inputs (and bf16 with
 * PRISM_BWD_CHUNKED=0): the scan is walked backwards token by token, in up to
 * 8 segments per sequence side by side, from states checkpointed every 4
 * tokens (16 at dk = 64) and gradients stored at the segment ends, which the
 * workspace holds (about 4 B * H * dk * dv * (T / 4 + 9 n_seqs)).  The
 * workspace size depends on PRISM_BWD_CHUNKED at the time of the query.
 *
 *   inputs as in prism_fwd; S_init as in prism_fwd_resume (NULL = zero)
 *   dO          [T, H, dv], input dtype
 *   dS_final    fp32 [n_seqs, H, dk, dv] or NULL (zero)
 *   dq, dk      out fp32 [T, H, dk]          dv  out fp32 [T, H, dv]
 *   du, da, dh  out fp32 [T, H, L-1, dk] (NULL allowed iff L == 1; h's last
 *               slot, which the forward never reads, gets zero)
 *   dg, db      out fp32 [T, H]              dconv_w  out fp32 [H, dk, 4]
 *   dS_init     out fp32 [n_seqs, H, dk, dv] or NULL (not written)
 *   workspace   prism_bwd_workspace_bytes(d, L) bytes
 * On the chunkwise form dg is (dL/d ln g) / g: a forget gate of exactly 0 gives a
 * non-finite dg there (the token walk has no such limit).
 * dk, dv in {64, 128}, else PRISM_EUNSUPPORTED.  Some gradients are summed
 * with fp32 atomics (db over channel groups; on the token walk also over value
 * slices), so the last bits may differ from run to run.
 */
size_t prism_bwd_workspace_bytes(const prism_dims* d, int L);
prism_status prism_bwd(const prism_dims* d,
                       const void* q, const void* k, const void* v,
                       const void* u, const void* g, const void* b,
                       const void* a, const void* h, const void* conv_w,
                       const int32_t* cu_seqlens, int L, const float* S_init,
                       const void* dO, const float* dS_final,
                       float* dq, float* dk, float* dv, float* du, float* dg, float* db,
                       float* da, float* dh, float* dconv_w, float* dS_init,
                       void* workspace, size_t workspace_bytes, void* stream);

/* prism_bwd with a choice of residual chain (prism_residual): the closed form
 * (PRISM_RESIDUAL_LINEAR, as prism_bwd) or the non-linear refinement chain
 * r_{l+1} = r_l - a_l GELU(h_l r_l) of the gist.science summary, section 2.2
 * (PRISM_RESIDUAL_GELU; forward as in prism_fwd_resume).  Any other value:
 * PRISM_EINVAL.  Other arguments, layouts and errors as in prism_bwd. */
prism_status prism_bwd_ex(const prism_dims* d,
                          const void* q, const void* k, const void* v,
                          const void* u, const void* g, const void* b,
                          const void* a, const void* h, const void* conv_w,
                          const int32_t* cu_seqlens, int L, int residual, const float* S_init,
                          const void* dO, const float* dS_final,
                          float* dq, float* dk, float* dv, float* du, float* dg, float* db,
                          float* da, float* dh, float* dconv_w, float* dS_init,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training pair: a forward pass that keeps every 64-token chunk's start state,
 * and a backward pass that reads those checkpoints instead of recomputing them
 * (the chunkwise form of the recurrence, WeChat page section 消除 Token 间串行:
 * within a chunk the outputs and the next state follow from the chunk's start
 * state, so the backward needs the start state of every chunk).
 *
 * prism_checkpoint_bytes: bytes of the checkpoints for the shape, three bf16
 * arrays, each rounded up to 256 bytes: the start states [nv, H, dk, dv], the
 * same states transposed [nv, H, dv, dk], nv = floor(T / 64) + n_seqs, chunk c
 * of sequence n at slot floor(cu_seqlens[n] / 64) + n + c (slots of no chunk
 * are not written), then the write keys kw [T, H, dk] (at least 256 bytes).
 * 0 where the chunkwise backward does not serve the shape (dtype not bf16, dk
 * or dv not 64 or 128) or the dims are invalid.
 */
size_t prism_checkpoint_bytes(const prism_dims* d);

/* prism_fwd_resume without carried history (k_hist = NULL) that also writes
 * the checkpoints, a device buffer of prism_checkpoint_bytes(d) bytes
 * (caller-owned; the call writes it and keeps nothing).  The scan runs over
 * whole sequences (no segment split, whose segments start from zero), on the
 * eight-wavefront bf16 kernel; outputs as in prism_fwd_resume.  The write
 * keys go into the checkpoints, so the workspace is neither read nor written
 * (it may be NULL with workspace_bytes 0; the arguments keep the call shape of
 * the other forward entry points).
 * PRISM_EUNSUPPORTED for shapes with no checkpoints (see above) or when the
 * environment selects another scan kernel (PRISM_SCAN_GENERIC=1,
 * PRISM_SCAN_SPECIALISED=0, PRISM_SCAN_WAVES=4); PRISM_EINVAL for invalid
 * arguments, a null checkpoint buffer included. */
prism_status prism_fwd_ckpt(const prism_dims* d,
                            const void* q, const void* k, const void* v,
                            const void* u, const void* g, const void* b,
                            const void* a, const void* h, const void* conv_w,
                            const int32_t* cu_seqlens, int L, int residual, const float* S_init,
                            void* o, float* S_final, void* checkpoints,
                            void* workspace, size_t workspace_bytes, void* stream);

/* prism_bwd_ex on the chunkwise form with the chunk-start states read from
 * `checkpoints` (written by prism_fwd_ckpt for the same inputs, S_init and
 * residual chain; read only) and the write keys read from there too, instead
 * of recomputed: two launches fewer (the prologue and the state recompute).
 * grad_dtype (a prism_dtype) is the storage type of the six token-sized
 * gradients dq, dk, dv [T, H, d] and du, da, dh [T, H, L-1, dk]: PRISM_F32, or
 * PRISM_BF16 for each of them rounded to nearest even from the fp32 value the
 * PRISM_F32 call stores (half the bytes written, and no cast for a bf16
 * training loop).  dg, db, dconv_w and dS_init are fp32 either way.
 * Arguments, layouts, workspace and errors otherwise as in prism_bwd_ex;
 * PRISM_EUNSUPPORTED where the chunkwise form does not run (shapes with no
 * checkpoints, PRISM_BWD_CHUNKED=0); PRISM_EINVAL for a null checkpoint
 * buffer or another grad_dtype. */
prism_status prism_bwd_ckpt(const prism_dims* d,
                            const void* q, const void* k, const void* v,
                            const void* u, const void* g, const void* b,
                            const void* a, const void* h, const void* conv_w,
                            const int32_t* cu_seqlens, int L, int residual, int grad_dtype,
                            const float* S_init, const void* dO, const float* dS_final,
                            void* dq, void* dk, void* dv, void* du, float* dg, float* db,
                            void* da, void* dh, float* dconv_w, float* dS_init,
                            const void* checkpoints, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Diagnostic: the number of bounded in-kernel waits that gave up since the
 * last reset, on the current device.  The eight-wavefront bf16 scan has one
 * bounded LDS-flag wait per chunk (the workgroup's diagonal-inverse handoff);
 * every writer raises its flag before the next barrier, so the count stays
 * 0, and a nonzero count means some output of a scan since the reset may be
 * wrong.  Writes the count to *count (host pointer, non-null); reset != 0
 * sets it back to zero.  Unlike every other entry point this call is
 * synchronous: it reads (and with reset writes) a device word with a blocking
 * copy, so call it outside graph capture.  PRISM_EINVAL for a null pointer,
 * PRISM_EHIP if the copy fails.
 */
prism_status prism_scan_wait_giveups(unsigned int* count, int reset);

/* Static description of a status code. */
const char* prism_status_str(prism_status s);

/* ABI version of this header (bumped on any signature change). */
int prism_abi_version(void);
#define PRISM_ABI_VERSION 2

#ifdef __cplusplus
}
#endif
#endif /* PRISM_H */
