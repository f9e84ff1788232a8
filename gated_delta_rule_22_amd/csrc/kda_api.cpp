// C ABI of the KDA hot path: argument validation on the host, then dispatch
// to the HIP kernels on the caller's stream. Nothing here allocates,
// synchronises or keeps state between calls.
#include "../../include/kda.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <cstring>
#include <mutex>

#include "kda_launch.h"

namespace {

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool chunk_ok(int c) { return c == 0 || c == 16 || c == 32 || c == 64; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

constexpr int kChunk = 64;   // chunk numbering of the MFMA path and checkpoint granularity

// Chunks in the numbering of a packed call: sum_i ceil(len_i / 64) over N
// sequences of T tokens in all is at most (T + 63 N) / 64.
size_t varlen_chunk_bound(int N, int T) {
    return ((size_t)T + (size_t)N * (kChunk - 1)) / kChunk;
}
size_t varlen_table_bytes(int N) { return align256((3 * (size_t)N + 3) * sizeof(int)); }

struct Range {
    uintptr_t lo = 0, hi = 0;  // [lo, hi)
    Range() = default;
    Range(const void* p, size_t bytes) : lo((uintptr_t)p), hi((uintptr_t)p + bytes) {}
    bool empty() const { return lo == hi; }
};
bool overlap(const Range& a, const Range& b) {
    return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

// a * b * ... without size_t overflow; false on overflow
bool mul_ok(size_t& acc, size_t x) {
    if (x != 0 && acc > SIZE_MAX / x) return false;
    acc *= x;
    return true;
}

// kda_prefill_fwd with the workspace capped at max_ws bytes: the piecewise
// split path then runs pieces short enough for one to fit (kda_prefill_fwd
// itself passes no cap; the allocation-free entry point its static array).
size_t prefill_workspace_capped(int B, int T, int H, int dk, int dv, kda_dtype dtype, int chunk,
                                size_t max_ws) {
    if (B <= 0 || T <= 0 || H <= 0 || dtype != KDA_BF16) return 0;
    if (!kda::prefill_mfma_supported(dk, dv, chunk, H)) return 0;
    return kda::prefill_mfma_workspace_fixed(B, H, ((long)T + kChunk - 1) / kChunk, max_ws);
}

kda_status prefill_fwd_capped(const void* q, const void* k, const void* v,
                              const float* log_alpha, const float* beta,
                              const float* S0, void* o, float* S_final,
                              int B, int T, int H, int dk, int dv,
                              kda_dtype dtype, int chunk,
                              void* ws, size_t ws_bytes, size_t max_ws, void* stream) {
    if (B < 0 || T < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv) || !chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return KDA_OK;

    const size_t elt = dtype == KDA_BF16 ? 2 : 4;
    size_t tok = 1;
    if (!mul_ok(tok, (size_t)B) || !mul_ok(tok, (size_t)T) || !mul_ok(tok, (size_t)H))
        return KDA_ERR_INVALID_ARG;
    size_t nk = tok, nv = tok, ns = (size_t)B * (size_t)H;
    if (!mul_ok(nk, (size_t)dk) || !mul_ok(nv, (size_t)dv) || !mul_ok(ns, (size_t)dk * dv))
        return KDA_ERR_INVALID_ARG;
    if (nk > (SIZE_MAX >> 3) || nv > (SIZE_MAX >> 3) || ns > (SIZE_MAX >> 3))
        return KDA_ERR_INVALID_ARG;

    if (T > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, log_alpha, beta, S0, o, S_final};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_INVALID_ARG;
    const size_t ws_need = prefill_workspace_capped(B, T, H, dk, dv, dtype, chunk, max_ws);
    if (ws_need > 0 && (ws == nullptr || ws_bytes < ws_need)) return KDA_ERR_WORKSPACE;
    if (ws_need > 0 && !aligned16(ws)) return KDA_ERR_INVALID_ARG;

    const Range rq(q, T ? nk * elt : 0), rk(k, T ? nk * elt : 0), rv(v, T ? nv * elt : 0);
    const Range rla(log_alpha, T ? nk * 4 : 0), rb(beta, T ? tok * 4 : 0);
    const Range rs0(S0, S0 ? ns * 4 : 0), ro(o, T ? nv * elt : 0);
    const Range rsf(S_final, S_final ? ns * 4 : 0);
    const Range inputs[] = {rq, rk, rv, rla, rb, rs0};
    for (const Range& in : inputs)
        if (overlap(ro, in) || overlap(rsf, in)) {
            // the only permitted overlap: S_final is exactly S0
            if (&in == &inputs[5] && rsf.lo == rs0.lo && !overlap(ro, in)) continue;
            return KDA_ERR_INVALID_ARG;
        }
    if (overlap(ro, rsf)) return KDA_ERR_INVALID_ARG;
    if (ws_need > 0) {
        const Range rws(ws, ws_need);
        for (const Range& in : inputs)
            if (overlap(rws, in)) return KDA_ERR_INVALID_ARG;
        if (overlap(rws, ro) || overlap(rws, rsf)) return KDA_ERR_INVALID_ARG;
    }

    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    const kda::SeqLayout sq{nullptr, B, T, kChunk, 0, T};
    if (dtype == KDA_BF16 && T > 0 && kda::prefill_mfma_supported(dk, dv, chunk, H)) {
        const size_t nch = (size_t)B * (((size_t)T + kChunk - 1) / kChunk);
        if (nch > (size_t)INT32_MAX) return KDA_ERR_INVALID_ARG;
        bool epi_done;
        e = kda::launch_prefill_mfma(q, k, v, log_alpha, beta, S0, o, S_final, sq, H, (int)nch,
                                     ws, nullptr, 0, 0, kda::Prologue{}, kda::Epilogue{},
                                     &epi_done, st, max_ws);
    } else {
        e = kda::launch_prefill_generic(dtype == KDA_BF16, q, k, v, log_alpha, beta, S0, o,
                                        S_final, sq, H, dk, dv, chunk ? chunk : 64, nullptr, 0,
                                        0, kda::Prologue{}, st);
    }
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARG: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported shape, chunk or dtype";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
        case KDA_ERR_HIP: return "HIP launch failed";
        case KDA_ERR_SCRATCH:
            return "the call needs more device scratch than the library's static buffer "
                   "holds (kda_prefill_fwd_noalloc; use kda_prefill_fwd with a workspace)";
    }
    return "unknown status";
}

size_t kda_prefill_workspace_size(int B, int T, int H, int dk, int dv, kda_dtype dtype,
                                  int chunk) {
    return prefill_workspace_capped(B, T, H, dk, dv, dtype, chunk, SIZE_MAX);
}

kda_status kda_prefill_fwd(const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta,
                           const float* S0, void* o, float* S_final,
                           int B, int T, int H, int dk, int dv,
                           kda_dtype dtype, int chunk,
                           void* ws, size_t ws_bytes, void* stream) {
    return prefill_fwd_capped(q, k, v, log_alpha, beta, S0, o, S_final, B, T, H, dk, dv, dtype,
                              chunk, ws, ws_bytes, SIZE_MAX, stream);
}

size_t kda_prefill_varlen_workspace_size(int N, int T_total, int H, int dk, int dv,
                                         kda_dtype dtype, int chunk) {
    if (N <= 0 || T_total < 0 || H <= 0) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    if (!dim_ok(dk) || !dim_ok(dv) || !chunk_ok(chunk)) return 0;
    size_t need = varlen_table_bytes(N);
    if (dtype == KDA_BF16 && kda::prefill_mfma_supported(dk, dv, chunk, H)) {
        need += kda::prefill_mfma_workspace((long)N * H, varlen_chunk_bound(N, T_total), H);
        const kda::SplitPlan plan = kda::prefill_split_plan(N, T_total, H, need);
        if (plan.n2 > 0) need = plan.end;
    }
    return need;
}

kda_status kda_prefill_varlen(const void* q, const void* k, const void* v,
                              const float* log_alpha, const float* beta,
                              const float* S0, void* o, float* S_final,
                              const int* cu_seqlens, int N, int T_total, int H, int dk, int dv,
                              kda_dtype dtype, int chunk,
                              float* S_ckpt, int ckpt_every, int ckpt_slots,
                              void* ws, size_t ws_bytes, void* stream) {
    if (N < 0 || T_total < 0 || H < 0 || ckpt_every < 0 || ckpt_slots < 0)
        return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv) || !chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    if (ckpt_every % kChunk != 0) return KDA_ERR_INVALID_ARG;
    if (ckpt_every > 0 && (S_ckpt == nullptr || ckpt_slots == 0)) return KDA_ERR_INVALID_ARG;
    if (ckpt_every == 0) {   // no checkpoints: S_ckpt and ckpt_slots are ignored
        S_ckpt = nullptr;
        ckpt_slots = 0;
    }
    if (N == 0 || H == 0) return KDA_OK;
    if (!cu_seqlens || ((uintptr_t)cu_seqlens & 3u)) return KDA_ERR_INVALID_ARG;
    if (N > INT32_MAX / 4 || varlen_chunk_bound(N, T_total) > (size_t)INT32_MAX)
        return KDA_ERR_INVALID_ARG;

    const size_t elt = dtype == KDA_BF16 ? 2 : 4;
    size_t tok = (size_t)T_total;
    if (!mul_ok(tok, (size_t)H)) return KDA_ERR_INVALID_ARG;
    size_t nk = tok, nv = tok, ns = (size_t)N * (size_t)H, nc = (size_t)ckpt_slots * (size_t)H;
    if (!mul_ok(nk, (size_t)dk) || !mul_ok(nv, (size_t)dv) || !mul_ok(ns, (size_t)dk * dv) ||
        !mul_ok(nc, (size_t)dk * dv))
        return KDA_ERR_INVALID_ARG;
    if (nk > (SIZE_MAX >> 3) || nv > (SIZE_MAX >> 3) || ns > (SIZE_MAX >> 3) ||
        nc > (SIZE_MAX >> 3))
        return KDA_ERR_INVALID_ARG;

    if (T_total > 0 && (!q || !k || !v || !log_alpha || !beta || !o)) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, log_alpha, beta, S0, o, S_final, S_ckpt};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_INVALID_ARG;
    const size_t ws_need = kda_prefill_varlen_workspace_size(N, T_total, H, dk, dv, dtype, chunk);
    if (ws == nullptr || ws_bytes < ws_need) return KDA_ERR_WORKSPACE;
    if (((uintptr_t)ws & 255u) != 0) return KDA_ERR_INVALID_ARG;

    const bool has_t = T_total > 0;
    const Range rq(q, has_t ? nk * elt : 0), rk(k, has_t ? nk * elt : 0),
        rv(v, has_t ? nv * elt : 0);
    const Range rla(log_alpha, has_t ? nk * 4 : 0), rb(beta, has_t ? tok * 4 : 0);
    const Range rs0(S0, S0 ? ns * 4 : 0), rcu(cu_seqlens, ((size_t)N + 1) * 4);
    const Range ro(o, has_t ? nv * elt : 0), rsf(S_final, S_final ? ns * 4 : 0),
        rck(S_ckpt, S_ckpt ? nc * 4 : 0), rws(ws, ws_need);
    const Range inputs[] = {rq, rk, rv, rla, rb, rs0, rcu};
    const Range outputs[] = {ro, rsf, rck, rws};
    for (const Range& out : outputs)
        for (const Range& in : inputs)
            if (overlap(out, in)) {
                // the only permitted overlap: S_final is exactly S0
                if (&out == &outputs[1] && &in == &inputs[5] && rsf.lo == rs0.lo) continue;
                return KDA_ERR_INVALID_ARG;
            }
    for (int a = 0; a < 4; ++a)
        for (int b = a + 1; b < 4; ++b)
            if (overlap(outputs[a], outputs[b])) return KDA_ERR_INVALID_ARG;

    hipStream_t st = (hipStream_t)stream;
    int* tab = (int*)ws;
    hipError_t e = kda::launch_varlen_table(cu_seqlens, N, T_total, kChunk, ckpt_every, tab, st);
    if (e != hipSuccess) return KDA_ERR_HIP;
    const kda::SeqLayout sq{tab, N, T_total, kChunk, ckpt_every, T_total};
    // With no tokens every sequence is empty and only S_final = S0 remains:
    // the generic kernel does that without touching a chunk record.
    bool epi_done;
    const bool mfma = dtype == KDA_BF16 && T_total > 0 && kda::prefill_mfma_supported(dk, dv, chunk, H);
    const kda::SplitPlan plan =
        mfma ? kda::prefill_split_plan(N, T_total, H, varlen_table_bytes(N)) : kda::SplitPlan{};
    if (plan.n2 > 0)
        // many sequence-heads, lengths decided on the device: sequences far
        // longer than the rest are split between the fused kernel and the
        // prep + state walk
        e = kda::launch_prefill_split(q, k, v, log_alpha, beta, S0, o, S_final, tab, N, T_total,
                                      ckpt_every, H, plan, (char*)ws, S_ckpt, ckpt_slots, st);
    else if (mfma)
        e = kda::launch_prefill_mfma(q, k, v, log_alpha, beta, S0, o, S_final, sq, H,
                                     (int)varlen_chunk_bound(N, T_total),
                                     (char*)ws + varlen_table_bytes(N), S_ckpt, ckpt_slots, 0,
                                     kda::Prologue{}, kda::Epilogue{}, &epi_done, st);
    else
        e = kda::launch_prefill_generic(dtype == KDA_BF16, q, k, v, log_alpha, beta, S0, o,
                                        S_final, sq, H, dk, dv, chunk ? chunk : 64, S_ckpt,
                                        ckpt_slots, 0, kda::Prologue{}, st);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_step(const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta,
                           float* S, void* o,
                           int B, int H, int dk, int dv,
                           kda_dtype dtype, void* stream) {
    if (B < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return KDA_OK;
    if (!q || !k || !v || !log_alpha || !beta || !S || !o) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, log_alpha, beta, S, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return KDA_ERR_INVALID_ARG;
    const size_t elt = dtype == KDA_BF16 ? 2 : 4;
    size_t bh = 1;
    if (!mul_ok(bh, (size_t)B) || !mul_ok(bh, (size_t)H)) return KDA_ERR_INVALID_ARG;
    if (bh > (size_t)INT32_MAX / 4) return KDA_ERR_INVALID_ARG;
    const size_t nk = bh * dk, nv = bh * dv, ns = bh * dk * dv;
    const Range rq(q, nk * elt), rk(k, nk * elt), rv(v, nv * elt), rla(log_alpha, nk * 4),
        rb(beta, bh * 4), rS(S, ns * 4), ro(o, nv * elt);
    const Range ins[] = {rq, rk, rv, rla, rb};
    for (const Range& in : ins)
        if (overlap(ro, in) || overlap(rS, in)) return KDA_ERR_INVALID_ARG;
    if (overlap(ro, rS)) return KDA_ERR_INVALID_ARG;

    kda::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.gate = log_alpha; a.beta = beta; a.S = S; a.o = o;
    a.BH = (int)bh;
    const hipError_t e = kda::launch_decode(dtype == KDA_BF16, dk, dv, a, (hipStream_t)stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_multi(const void* q, const void* k, const void* v,
                            const float* log_alpha, const float* beta,
                            float* S, void* o, const int* n_commit,
                            int B, int T, int H, int dk, int dv,
                            kda_dtype dtype, void* stream) {
    if (B < 0 || T < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || T == 0) return KDA_OK;
    if (!q || !k || !v || !log_alpha || !beta || !S || !o) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, log_alpha, beta, S, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return KDA_ERR_INVALID_ARG;
    if (n_commit && ((uintptr_t)n_commit & 3u)) return KDA_ERR_INVALID_ARG;
    const size_t elt = dtype == KDA_BF16 ? 2 : 4;
    size_t bh = 1, tok = 1;
    if (!mul_ok(bh, (size_t)B) || !mul_ok(bh, (size_t)H)) return KDA_ERR_INVALID_ARG;
    if (bh > (size_t)INT32_MAX / 4) return KDA_ERR_INVALID_ARG;
    if (!mul_ok(tok, bh) || !mul_ok(tok, (size_t)T) || tok > (SIZE_MAX >> 10))
        return KDA_ERR_INVALID_ARG;
    const size_t nk = tok * dk, nv = tok * dv, ns = bh * dk * dv;
    const Range rq(q, nk * elt), rk(k, nk * elt), rv(v, nv * elt), rla(log_alpha, nk * 4),
        rb(beta, tok * 4), rS(S, ns * 4), ro(o, nv * elt), rn(n_commit, n_commit ? (size_t)B * 4 : 0);
    const Range ins[] = {rq, rk, rv, rla, rb, rn};
    for (const Range& in : ins)
        if (overlap(ro, in) || overlap(rS, in)) return KDA_ERR_INVALID_ARG;
    if (overlap(ro, rS)) return KDA_ERR_INVALID_ARG;

    const hipError_t e = kda::launch_decode_multi(dtype == KDA_BF16, dk, dv, q, k, v, log_alpha,
                                                  beta, S, o, n_commit, (int)bh, H, T,
                                                  (hipStream_t)stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Layer form: the weight-free prologue and epilogue around the op.

namespace {

struct LayerCfg {
    int pro = 0;                 // kGate* | kProL2
    kda::Prologue pr{1e-6f, 5.f};
    const void* z = nullptr;
    const float* w = nullptr;
    float out_eps = 1e-6f;
};

// Validates opts (NULL = the plain op) and fills cfg. The gate input of
// each mode has its own element size and per-token count.
kda_status layer_cfg(const kda_layer_opts* opts, LayerCfg& cfg) {
    if (!opts) return KDA_OK;
    // the mode is read as an int: a C caller may store any value in the field
    int gate;
    std::memcpy(&gate, &opts->gate, sizeof gate);
    if (gate != KDA_GATE_LOG && gate != KDA_GATE_BOUNDED && gate != KDA_GATE_SCALAR)
        return KDA_ERR_INVALID_ARG;
    if (!(opts->decay_bound >= 0.f) || !(opts->l2_eps >= 0.f) || !(opts->out_eps >= 0.f))
        return KDA_ERR_INVALID_ARG;   // negative or NaN
    cfg.pro = gate | (opts->l2norm_qk ? kda::kProL2 : 0);
    if (opts->decay_bound > 0.f) cfg.pr.bound = opts->decay_bound;
    if (opts->l2_eps > 0.f) cfg.pr.l2_eps = opts->l2_eps;
    cfg.z = opts->out_gate;
    cfg.w = opts->out_weight;
    if (opts->out_eps > 0.f) cfg.out_eps = opts->out_eps;
    if (cfg.w && ((uintptr_t)cfg.w & 3u)) return KDA_ERR_INVALID_ARG;
    if (cfg.z && !aligned16(cfg.z)) return KDA_ERR_INVALID_ARG;
    return KDA_OK;
}

}  // namespace

kda_status kda_prefill_layer(const void* q, const void* k, const void* v, const void* gate,
                             const float* beta, const float* S0, void* o, float* S_final,
                             int B, int T, int H, int dk, int dv, kda_dtype dtype, int chunk,
                             const kda_layer_opts* opts, void* ws, size_t ws_bytes,
                             void* stream) {
    LayerCfg cfg;
    const kda_status ls = layer_cfg(opts, cfg);
    if (ls != KDA_OK) return ls;
    if (B < 0 || T < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv) || !chunk_ok(chunk)) return KDA_ERR_UNSUPPORTED;
    // the matrix-core path's log-decay range is [-5, 0]: a wider bounded
    // gate would be clamped there
    if (dtype == KDA_BF16 && kda::prefill_mfma_supported(dk, dv, chunk, H) &&
        (cfg.pro & 3) == KDA_GATE_BOUNDED && cfg.pr.bound > 5.f)
        return KDA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return KDA_OK;

    const size_t elt = dtype == KDA_BF16 ? 2 : 4;
    size_t tok = 1;
    if (!mul_ok(tok, (size_t)B) || !mul_ok(tok, (size_t)T) || !mul_ok(tok, (size_t)H))
        return KDA_ERR_INVALID_ARG;
    size_t nk = tok, nv = tok, ns = (size_t)B * (size_t)H;
    if (!mul_ok(nk, (size_t)dk) || !mul_ok(nv, (size_t)dv) || !mul_ok(ns, (size_t)dk * dv))
        return KDA_ERR_INVALID_ARG;
    if (nk > (SIZE_MAX >> 3) || nv > (SIZE_MAX >> 3) || ns > (SIZE_MAX >> 3))
        return KDA_ERR_INVALID_ARG;

    if (T > 0 && (!q || !k || !v || !gate || !beta || !o)) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, gate, beta, S0, o, S_final};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return KDA_ERR_INVALID_ARG;
    const size_t ws_need = kda_prefill_workspace_size(B, T, H, dk, dv, dtype, chunk);
    if (ws_need > 0 && (ws == nullptr || ws_bytes < ws_need)) return KDA_ERR_WORKSPACE;
    if (ws_need > 0 && !aligned16(ws)) return KDA_ERR_INVALID_ARG;

    const int gm = cfg.pro & 3;
    const size_t gate_bytes = gm == KDA_GATE_SCALAR ? tok * 4 : nk * (gm == KDA_GATE_LOG ? 4 : elt);
    const bool has_t = T > 0;
    const Range rq(q, has_t ? nk * elt : 0), rk(k, has_t ? nk * elt : 0),
        rv(v, has_t ? nv * elt : 0), rg(gate, has_t ? gate_bytes : 0),
        rb(beta, has_t ? tok * 4 : 0), rs0(S0, S0 ? ns * 4 : 0),
        rz(cfg.z, (has_t && cfg.z) ? nv * elt : 0), rw(cfg.w, cfg.w ? (size_t)dv * 4 : 0);
    const Range ro(o, has_t ? nv * elt : 0), rsf(S_final, S_final ? ns * 4 : 0),
        rws(ws, ws_need);
    const Range inputs[] = {rq, rk, rv, rg, rb, rs0, rz, rw};
    const Range outputs[] = {ro, rsf, rws};
    for (const Range& out : outputs)
        for (const Range& in : inputs)
            if (overlap(out, in)) {
                // the only permitted overlap: S_final is exactly S0
                if (&out == &outputs[1] && &in == &inputs[5] && rsf.lo == rs0.lo) continue;
                return KDA_ERR_INVALID_ARG;
            }
    if (overlap(ro, rsf) || overlap(ro, rws) || overlap(rsf, rws)) return KDA_ERR_INVALID_ARG;

    hipStream_t st = (hipStream_t)stream;
    const kda::SeqLayout sq{nullptr, B, T, kChunk, 0, T};
    hipError_t e;
    bool epi_done = false;
    if (dtype == KDA_BF16 && T > 0 && kda::prefill_mfma_supported(dk, dv, chunk, H)) {
        const size_t nch = (size_t)B * (((size_t)T + kChunk - 1) / kChunk);
        if (nch > (size_t)INT32_MAX) return KDA_ERR_INVALID_ARG;
        const kda::Epilogue ep{cfg.z, cfg.w, cfg.out_eps};
        e = kda::launch_prefill_mfma(q, k, v, gate, beta, S0, o, S_final, sq, H, (int)nch, ws,
                                     nullptr, 0, cfg.pro, cfg.pr, ep, &epi_done, st);
    } else {
        e = kda::launch_prefill_generic(dtype == KDA_BF16, q, k, v, gate, beta, S0, o, S_final,
                                        sq, H, dk, dv, chunk ? chunk : 64, nullptr, 0, cfg.pro,
                                        cfg.pr, st);
    }
    if (e == hipSuccess && cfg.z && T > 0 && !epi_done)
        e = kda::launch_norm_gate(dtype == KDA_BF16, o, cfg.z, cfg.w, cfg.out_eps, o, (long)tok,
                                  dv, st);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_layer(const void* q, const void* k, const void* v, const void* gate,
                            const float* beta, float* S, void* o, int B, int H, int dk, int dv,
                            kda_dtype dtype, const kda_layer_opts* opts, void* stream) {
    LayerCfg cfg;
    const kda_status ls = layer_cfg(opts, cfg);
    if (ls != KDA_OK) return ls;
    if (B < 0 || H < 0) return KDA_ERR_INVALID_ARG;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return KDA_OK;
    if (!q || !k || !v || !gate || !beta || !S || !o) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, gate, beta, S, o};
    for (const void* p : ptrs)
        if (!aligned16(p)) return KDA_ERR_INVALID_ARG;
    const size_t elt = dtype == KDA_BF16 ? 2 : 4;
    size_t bh = 1;
    if (!mul_ok(bh, (size_t)B) || !mul_ok(bh, (size_t)H)) return KDA_ERR_INVALID_ARG;
    if (bh > (size_t)INT32_MAX / 4) return KDA_ERR_INVALID_ARG;
    const int gm = cfg.pro & 3;
    const size_t nk = bh * dk, nv = bh * dv, ns = bh * dk * dv;
    const size_t gate_bytes = gm == KDA_GATE_SCALAR ? bh * 4 : nk * (gm == KDA_GATE_LOG ? 4 : elt);
    const Range rq(q, nk * elt), rk(k, nk * elt), rv(v, nv * elt), rg(gate, gate_bytes),
        rb(beta, bh * 4), rS(S, ns * 4), ro(o, nv * elt), rz(cfg.z, cfg.z ? nv * elt : 0),
        rw(cfg.w, cfg.w ? (size_t)dv * 4 : 0);
    const Range ins[] = {rq, rk, rv, rg, rb, rz, rw};
    for (const Range& in : ins)
        if (overlap(ro, in) || overlap(rS, in)) return KDA_ERR_INVALID_ARG;
    if (overlap(ro, rS)) return KDA_ERR_INVALID_ARG;

    kda::DecodeArgs a{};
    a.q = q; a.k = k; a.v = v; a.gate = gate; a.beta = beta; a.S = S; a.o = o;
    a.BH = (int)bh;
    a.layer = true;
    a.pro = cfg.pro;
    a.pr = cfg.pr;
    a.z = cfg.z;
    a.w = cfg.w;
    a.out_eps = cfg.out_eps;
    const hipError_t e = kda::launch_decode(dtype == KDA_BF16, dk, dv, a, (hipStream_t)stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}


// ---------------------------------------------------------------------------
// Prefill without any allocation: the workspace of kda_prefill_fwd lives in a
// file-scope device array instead of a caller buffer. Each GPU the library
// runs on holds its own copy (KDA_NOALLOC_SCRATCH_BYTES) until the process
// ends. The host-side name `scratch` only stands in for that memory: its
// device address comes from hipGetSymbolAddress, once per device, with that
// device current, and only that address is ever passed to a kernel.

}  // extern "C"

namespace {

static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (null on failure).
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

kda_status kda_prefill_fwd_noalloc(const void* q, const void* k, const void* v,
                                   const float* log_alpha, const float* beta,
                                   const float* S0, void* o, float* S_final,
                                   int B, int T, int H, int dk, int dv,
                                   kda_dtype dtype, int chunk, void* stream) {
    // the workspace capped at the array: a long few-head call runs its
    // pieces short enough for one to fit (slower than with the usual pieces,
    // which keep the records of 3072 chunk-heads in the last-level cache)
    const size_t need = prefill_workspace_capped(B, T, H, dk, dv, dtype, chunk,
                                                 KDA_NOALLOC_SCRATCH_BYTES);
    if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0) {
        ws = scratch_for_current_device();
        if (!ws) return KDA_ERR_HIP;
    }
    // every other rule (and every launch) is kda_prefill_fwd's; its kernels
    // write each record of the workspace before they read it, so the array
    // needs no clearing between calls
    return prefill_fwd_capped(q, k, v, log_alpha, beta, S0, o, S_final, B, T, H, dk, dv, dtype,
                              chunk, ws, need > 0 ? KDA_NOALLOC_SCRATCH_BYTES : 0,
                              KDA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
