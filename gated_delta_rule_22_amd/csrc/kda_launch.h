// Internal launchers behind the C ABI (shapes already validated by the caller).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kda_common.h"

namespace kda {

// Decode step over BH heads; layer = false is the plain op (gate = fp32
// log-decay, pro and the epilogue fields unused).
struct DecodeArgs {
    const void *q, *k, *v, *gate;
    const float* beta;
    float* S;
    void* o;
    int BH;
    bool layer;
    int pro;              // kGate* | kProL2
    Prologue pr;
    const void* z;        // epilogue gate input [BH, dv] or null
    const float* w;       // epilogue norm weight [dv] or null (ones)
    float out_eps;
};
hipError_t launch_decode(bool bf16_io, int dk, int dv, const DecodeArgs& a, hipStream_t st);

// Multi-token decode over B*H heads, T = ntok tokens each; S advanced by the
// first n_commit[b] tokens (all when n_commit is null).
hipError_t launch_decode_multi(bool bf16_io, int dk, int dv, const void* q, const void* k,
                               const void* v, const float* la, const float* beta, float* S,
                               void* o, const int* n_commit, int BH, int H, int ntok,
                               hipStream_t st);

// Sequence table of a packed variable-length call (layout: SeqLayout) from
// device offsets cu[0..N], into tab (3N + 3 ints of device memory).
hipError_t launch_varlen_table(const int* cu, int N, int T, int C, int K, int* tab,
                               hipStream_t st);

// Split schedule of a packed call (kda_varlen.hip): from the table of
// launch_varlen_table, the fused view of every sequence and a second table
// of the long sequences' second segments, into `out` (SplitPlan::sp).
hipError_t launch_varlen_split(const int* tab, int N, int T, int C, int K, int H, int n2,
                               int cap2, int* out, hipStream_t st);

// Multi-token decode on the matrix cores (bf16, dk = dv = 128, 2 <= ntok <= 8).
bool decode_multi_mfma_supported(bool bf16_io, int dk, int dv, int ntok);
hipError_t launch_decode_multi_mfma(const void* q, const void* k, const void* v, const float* la,
                                    const float* beta, float* S, void* o, const int* n_commit,
                                    int BH, int H, int ntok, hipStream_t st);

// Generic chunked prefill (fp32 arithmetic, any supported dk/dv/chunk, fp32 or
// bf16 I/O) over the sequences of `sq`; checkpoints when S_ckpt and sq.K are
// set; layer prologue `pro` (kGate* | kProL2, 0 = plain op).
hipError_t launch_prefill_generic(bool bf16_io, const void* q, const void* k, const void* v,
                                  const void* gate, const float* beta, const float* S0,
                                  void* o, float* S_final, const SeqLayout& sq, int H, int dk,
                                  int dv, int chunk, float* S_ckpt, int ck_slots, int pro,
                                  const Prologue& pr, hipStream_t st);

// bf16 MFMA chunked prefill for dk = dv = 128, chunk 64, over the sequences
// of `sq` (sq.C = 64). Below 128 sequence-heads it runs a chunk-parallel prep
// kernel and a state kernel that communicate through `ws`
// (prefill_mfma_workspace() bytes for nch_all chunks in the numbering);
// otherwise one fused kernel. With ep.z set, the 128-column fused kernel
// applies the layer epilogue itself and *epi_done says so; otherwise the
// caller runs launch_norm_gate afterwards.
// Heads at most kMfmaMaxHeads (above: the generic path).
constexpr long kMfmaMaxHeads = 65536;
bool prefill_mfma_supported(int dk, int dv, int chunk, long H);
bool prefill_mfma_split(long pairs);
size_t prefill_mfma_workspace(long pairs, size_t nch_all, int H);
// Fixed-length batches (B sequences of nch_seq chunks): the workspace of the
// split path, which for long sequences holds one piece of records (the
// launcher then walks the sequence piece by piece) plus a carried state.
// max_ws caps it: pieces shrink until one fits (SIZE_MAX: not even a piece
// of one chunk fits).
size_t prefill_mfma_workspace_fixed(int B, int H, long nch_seq, size_t max_ws = SIZE_MAX);
// Chunks per sequence of one piece of the piecewise split path, 0 = none,
// -1 = no piece fits max_ws.
long prefill_mfma_piece(long pairs, long nch_seq, size_t max_ws = SIZE_MAX);
// max_ws: the workspace bound the call's workspace size was computed with
// (prefill_mfma_workspace_fixed), which fixes the piece length.
hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, const void* gate,
                               const float* beta, const float* S0, void* o, float* S_final,
                               const SeqLayout& sq, int H, int nch_all, void* ws,
                               float* S_ckpt, int ck_slots, int pro, const Prologue& pr,
                               const Epilogue& ep, bool* epi_done, hipStream_t st,
                               size_t max_ws = SIZE_MAX);

// Split schedule of a packed call with many sequence-heads (N * H >= 256,
// N <= 1024): workspace layout after the sequence table (at byte `base`):
//   sp   ints: ord, lens1, mslot [N]; tab2 [3 n2 + 3]; lens2, fin2 [n2]
//   mid  first-segment end states, [n2][H][128][128] fp32
//   rec  operand records of the second segments, H * cap2 of them
// n2 == 0: the schedule does not apply (plain fused kernel).
struct SplitPlan {
    int n2 = 0;       // second-table entries, at most
    int cap2 = 0;     // second-segment chunks in all, at most
    int G = 0;        // prep workgroups per head
    size_t sp = 0, mid = 0, rec = 0, end = 0;
};
SplitPlan prefill_split_plan(int N, int T_total, int H, size_t base);
// Runs the schedule: the mixed fused + prep kernel, then the state walk of
// the second segments. tab = the sequence table, sp = SplitPlan::sp.
hipError_t launch_prefill_split(const void* q, const void* k, const void* v, const float* la,
                                const float* beta, const float* S0, void* o, float* S_final,
                                const int* tab, int N, int T_total, int K, int H,
                                const SplitPlan& plan, char* ws, float* S_ckpt, int ck_slots,
                                hipStream_t st);

// Layer epilogue over rows of dv values (one token and head each), in place
// allowed: out = w * o / sqrt(mean(o^2) + eps) * sigmoid(z); w may be null.
hipError_t launch_norm_gate(bool bf16_io, const void* o, const void* z, const float* w,
                            float eps, void* out, long rows, int dv, hipStream_t st);

}  // namespace kda
