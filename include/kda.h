/*
 * kda.h — C ABI of the MI355X (gfx950) Kimi Delta Attention hot path.
 *
 * The operation (Kimi K3 blog, section "Kimi Delta Attention"; the
 * trillion-scale architecture page, section 4 "The KDA update, in plain
 * words"), per batch b and head h, for tokens t = 0..T-1:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,            alpha_t = exp(log_alpha_t) (per key channel)
 *
 * with state S in R^{dk x dv} per head. No scale factor is applied to q, and
 * q, k are not normalised here (the Kimi Linear layer L2-normalises them
 * before the op: "Kimi K3: the manos...", section "Kimi Linear").
 *
 * Layouts (row-major, contiguous, device memory):
 *     q, k, log_alpha   [B, T, H, dk]   q, k in `dtype`; log_alpha fp32 (natural log)
 *     v, o              [B, T, H, dv]   in `dtype`
 *     beta              [B, T, H]       fp32, used as given (no clamp)
 *     S0, S_final, S    [B, H, dk, dv]  fp32, dv contiguous
 * Decode drops the T axis.
 *
 * Ownership: the caller owns every buffer. The library allocates no device
 * memory in these calls, never frees and never synchronises; work is
 * enqueued on `stream` (a hipStream_t; NULL = the default stream) and runs
 * asynchronously, so a device fault surfaces at the caller's next
 * synchronisation. Every pointer must be memory of the calling thread's
 * current HIP device, and `stream` a stream of that device: kernels launch
 * there (and kda_prefill_fwd_noalloc uses that device's scratch array). The
 * library keeps no state between calls apart from that array and its
 * cached address, and is reentrant.
 *
 * Errors: every argument is validated on the host before anything is
 * launched; a rejected call has no side effect. KDA_ERR_HIP reports a launch
 * failure (hipGetLastError after the launch).
 *
 * Supported on the GPU: dk, dv in {16, 32, 64, 128}; chunk in {0 (=64), 16,
 * 32, 64}; dtype fp32 or bf16. All device pointers must be 16-byte aligned.
 * The log-decay is meant to lie in [-5, 0] per step (the bound stated on the
 * trillion-scale page, section 4). The fp32 paths take any value exactly.
 * The bf16 matrix-core paths clamp each log-decay first, so their results
 * are finite for every input: the prefill (dk = dv = 128, chunk 64) into
 * [-5, 0], kda_decode_multi drafts of 2..8 tokens into [-10, 0]. A step that
 * decays harder than the floor keeps exp(floor) of the old state (0.7% for
 * the prefill) instead of less; its error is that fraction of the old
 * state's contribution. The bf16 matrix-core prefill runs for up to 65536
 * heads; calls with more take the generic bf16 kernels (same results up to
 * rounding, slower).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, misalignment, aliasing */
    KDA_ERR_UNSUPPORTED = 2,   /* dk, dv, chunk or dtype outside the supported set */
    KDA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    KDA_ERR_HIP = 4,           /* a HIP call or kernel launch failed */
    KDA_ERR_SCRATCH = 5        /* kda_prefill_fwd_noalloc: the call needs more than
                                  the static scratch buffer holds */
} kda_status;

typedef enum {
    KDA_F32 = 0,               /* q, k, v, o are fp32 */
    KDA_BF16 = 1               /* q, k, v, o are bf16 (fp32 state and accumulation) */
} kda_dtype;

/*
 * Bytes of device workspace kda_prefill_fwd needs for these sizes (0 if
 * none). Returns 0 also for arguments it would reject.
 */
size_t kda_prefill_workspace_size(int B, int T, int H, int dk, int dv,
                                  kda_dtype dtype, int chunk);

/*
 * Chunk-parallel prefill ("Kimi K3: the manos...", section "FlashKDA
 * Algorithm": chunk-local cumulative decay, K/Q decay scaling, the UT
 * transform U = (I + L)^{-1} Diag(beta)(V - K_decay S_in), the causal
 * M_qk = tril(Q_decay K_inv^T) output term and the S_in -> S_out carry).
 *
 *   q, k, v, log_alpha, beta   inputs (required when T > 0)
 *   S0       initial state, or NULL for zeros
 *   o        output [B,T,H,dv] in `dtype` (required when T > 0); must not
 *            overlap any input
 *   S_final  final state, or NULL to skip; may be the same buffer as S0
 *            (in-place continuation), must not partially overlap it
 *   chunk    tokens per chunk, 0 = 64. It selects the blocking only; the
 *            result is the same recurrence for any value.
 *   ws, ws_bytes  device workspace of at least kda_prefill_workspace_size()
 *            bytes (may be NULL/0 when that size is 0)
 * T = 0 writes S_final = S0 (or zeros) and no o.
 */
kda_status kda_prefill_fwd(const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta,
                           const float* S0, void* o, float* S_final,
                           int B, int T, int H, int dk, int dv,
                           kda_dtype dtype, int chunk,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Bytes of device workspace kda_prefill_varlen needs for these sizes (never 0
 * for N, H > 0: it always holds the sequence table). Returns 0 for arguments
 * it would reject. For bf16 with 256 or more sequence-heads, fewer than 256
 * heads and at most 1024 sequences it also holds the split schedule's
 * tables, end states and operand records (at most 16384 chunk-heads of
 * 72,192 B: about 1.2 GB).
 */
size_t kda_prefill_varlen_workspace_size(int N, int T_total, int H, int dk, int dv,
                                         kda_dtype dtype, int chunk);

/*
 * Packed variable-length prefill with state checkpoints. Serving packs the
 * prompts of N requests along one token axis and keeps each request's state
 * at its prompt end and at coarse token intervals, since a state per token
 * would grow with the length ("Kimi K3: the manos...", section "KDA Prefix
 * Cache Management"; the trillion-scale architecture page, section 6:
 * checkpoints on a 512-token hash grid).
 *
 *   q, k, log_alpha [T_total,H,dk]; v, o [T_total,H,dv]; beta [T_total,H]
 *            (the kda_prefill_fwd layout with B = 1)
 *   cu_seqlens  device int32 [N+1], 4-byte aligned: sequence i is tokens
 *            [cu[i], cu[i+1]). The recurrence restarts at each sequence from
 *            S0[i]. Offsets are read on the device and not validated on the
 *            host: they are meant to be non-decreasing from cu[0] = 0 to
 *            cu[N] = T_total. Otherwise each is clamped into [0, T_total] and
 *            raised to the running maximum, which keeps every access inside
 *            the buffers (output rows outside all sequences are not written).
 *            Empty sequences are allowed: S_final[i] = S0[i] (or 0).
 *   S0, S_final [N,H,dk,dv] fp32: as in kda_prefill_fwd (NULL S0 = zeros,
 *            NULL S_final = skip, S_final may be exactly S0).
 *   ckpt_every  0, or a multiple of 64: the state after every ckpt_every
 *            tokens of each sequence (counted from its start) is stored to
 *            S_ckpt [ckpt_slots,H,dk,dv] fp32. Sequence i's checkpoints j = 1
 *            .. len_i / ckpt_every take slots c_i + j - 1, where c_i is the
 *            sum of len / ckpt_every over the sequences before i. Slots
 *            at or past ckpt_slots are not written, nor are the slots past
 *            the last checkpoint (sum over all sequences of len /
 *            ckpt_every), which keep their contents. T_total / ckpt_every
 *            slots always suffice. With ckpt_every = 0, S_ckpt and
 *            ckpt_slots are ignored.
 *   ws, ws_bytes  device workspace, 256-byte aligned, at least
 *            kda_prefill_varlen_workspace_size() bytes (required).
 * Outputs (o, S_final, S_ckpt, ws) must not overlap each other or an input.
 * The result for each sequence equals kda_prefill_fwd on that sequence alone,
 * up to rounding: with many sequence-heads (bf16, N * H >= 256), a sequence
 * much longer than the rest runs its first chunks in the fused kernel and the
 * others through the chunk-parallel prep and the state walk, decided on the
 * device from the offsets, so that it does not set the call's length alone.
 */
kda_status kda_prefill_varlen(const void* q, const void* k, const void* v,
                              const float* log_alpha, const float* beta,
                              const float* S0, void* o, float* S_final,
                              const int* cu_seqlens, int N, int T_total, int H, int dk, int dv,
                              kda_dtype dtype, int chunk,
                              float* S_ckpt, int ckpt_every, int ckpt_slots,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * One-token decode step (the recurrence above for a single t, the form
 * "Kimi K3: the manos..." section "FlashKDA Algorithm" gives as
 * u = beta (v - (D S)^T k), S = D S + k u^T, o^T = q^T S), updating S in
 * place. q, k, log_alpha [B,H,dk]; v, o [B,H,dv]; beta [B,H]; S [B,H,dk,dv].
 * Each state element is read once and written once.
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta,
                           float* S, void* o,
                           int B, int H, int dk, int dv,
                           kda_dtype dtype, void* stream);

/*
 * Multi-token decode from a live state, for verifying a drafted continuation
 * (the trillion-scale architecture page, section 6: a one-layer draft
 * proposes up to seven tokens that the model checks in one pass) and for
 * short multi-token steps. For each sequence b the recurrence runs over its
 * T tokens in order from S[b]:
 *   q, k, log_alpha [B,T,H,dk]; v, o [B,T,H,dv]; beta [B,T,H]; S [B,H,dk,dv]
 *   o         o_t for every token t, read from the state after token t of the
 *             T-token run (as in prefill)
 *   n_commit  device int32 [B] (4-byte aligned) or NULL: S[b] is overwritten
 *             with the state after its first n_commit[b] tokens, the accepted
 *             prefix; values are clamped to [0, T]; NULL means T. With 0, S[b]
 *             is left untouched (a verify pass), so a rejected draft needs no
 *             rollback copy.
 * Each state element is read once and written at most once. o must not
 * overlap an input, S or n_commit; S must not overlap an input. T = 0 is a
 * no-op. T is meant to be small (a draft); long sequences belong to
 * kda_prefill_fwd.
 */
kda_status kda_decode_multi(const void* q, const void* k, const void* v,
                            const float* log_alpha, const float* beta,
                            float* S, void* o, const int* n_commit,
                            int B, int T, int H, int dk, int dv,
                            kda_dtype dtype, void* stream);

/*
 * Layer form: the weight-free operations around the op, fused into its
 * kernels ("Kimi K3: the manos...", section "Kimi Linear": q and k are
 * L2-normalised, the decay gate comes from a projection, and the output is
 * normalised per head and scaled by an output gate; the trillion-scale
 * architecture page, section 4: the log-decay is bounded to (-5, 0)). The
 * projections themselves need trained weights and stay with the caller,
 * who passes their outputs.
 *
 * Gate input by mode (`gate` argument of the layer calls):
 *   KDA_GATE_LOG      fp32 natural log-decay [.., dk], as log_alpha above
 *   KDA_GATE_BOUNDED  pre-activation g [.., dk] in `dtype`:
 *                     log_alpha = -decay_bound * sigmoid(g), inside (-decay_bound, 0)
 *   KDA_GATE_SCALAR   fp32 log-decay per token and head [..] (no dk axis),
 *                     applied to every key channel: the Gated DeltaNet gate
 */
typedef enum {
    KDA_GATE_LOG = 0,
    KDA_GATE_BOUNDED = 1,
    KDA_GATE_SCALAR = 2
} kda_gate;

typedef struct {
    kda_gate gate;
    float decay_bound;         /* KDA_GATE_BOUNDED; 0 selects 5. Above 5 is
                                  KDA_ERR_UNSUPPORTED on the bf16 matrix-core
                                  prefill (bf16, dk = dv = 128, chunk 64), whose
                                  log-decay range is [-5, 0] */
    int l2norm_qk;             /* nonzero: q, k arrive raw and are divided by
                                  sqrt(sum of squares + l2_eps) per token and head */
    float l2_eps;              /* 0 selects 1e-6 */
    const void* out_gate;      /* z [.., dv] in `dtype` (16-byte aligned), or NULL: no
                                  epilogue. Otherwise o = w * o / sqrt(mean(o^2) + out_eps)
                                  * sigmoid(z), the mean over each token-head's dv values */
    const float* out_weight;   /* w [dv] fp32, or NULL for ones */
    float out_eps;             /* 0 selects 1e-6 */
} kda_layer_opts;

/*
 * kda_prefill_fwd in the layer form: the same layouts, workspace and rules,
 * with `gate` in place of log_alpha (its layout follows opts->gate) and the
 * prologue and epilogue of `opts` (NULL: the plain op). Negative bounds or
 * eps values and unknown gate modes are rejected; z and w count as inputs
 * for the overlap rules. With an epilogue, o is written once by the prefill
 * and then rewritten in place.
 */
kda_status kda_prefill_layer(const void* q, const void* k, const void* v, const void* gate,
                             const float* beta, const float* S0, void* o, float* S_final,
                             int B, int T, int H, int dk, int dv, kda_dtype dtype, int chunk,
                             const kda_layer_opts* opts, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * kda_decode_step in the layer form (gate as above, one token: [B,H,dk] or
 * [B,H] for KDA_GATE_SCALAR; z [B,H,dv]). The prologue and the epilogue run
 * inside the decode kernel: the state is still read once and written once.
 */
kda_status kda_decode_layer(const void* q, const void* k, const void* v, const void* gate,
                            const float* beta, float* S, void* o, int B, int H, int dk, int dv,
                            kda_dtype dtype, const kda_layer_opts* opts, void* stream);

/*
 * kda_prefill_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without the workspace, which instead lives in a static
 * device array inside the library, KDA_NOALLOC_SCRATCH_BYTES (80 MiB) on each
 * GPU the library runs on, held until the process ends. A call whose usual
 * workspace (kda_prefill_workspace_size()) is larger runs the few-head path
 * in pieces short enough for one piece's records to fit the array: the same
 * kernels on the same chunks, so the results are those of kda_prefill_fwd,
 * at some speed (the usual pieces keep the records of 3072 chunk-heads,
 * 222 MB, in the last-level cache). A call that could not fit even one chunk
 * per piece returns KDA_ERR_SCRATCH and launches nothing; with fewer than
 * 128 sequence-heads on that path, none does. The call itself allocates
 * nothing: no hipMalloc, no hipFree, no allocating library routine.
 * Every call on one GPU shares that GPU's array, and it keeps the last
 * call's contents: calls that overlap on one GPU (on different streams, or
 * from different host threads without ordering) race and must be avoided.
 * Calls ordered on one stream are safe.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)80 << 20)
kda_status kda_prefill_fwd_noalloc(const void* q, const void* k, const void* v,
                                   const float* log_alpha, const float* beta,
                                   const float* S0, void* o, float* S_final,
                                   int B, int T, int H, int dk, int dv,
                                   kda_dtype dtype, int chunk, void* stream);

/* Static description of a status code; never NULL. */
const char* kda_status_string(kda_status status);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
