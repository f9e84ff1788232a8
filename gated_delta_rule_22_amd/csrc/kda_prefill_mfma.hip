// Chunk-parallel KDA prefill for dk = dv = 128, chunk 64: bf16 MFMA
// contractions, fp32 state.
//
// Method ("Kimi K3: the manos...", section "FlashKDA Algorithm"): inside a
// chunk of C = 64 tokens with starting state S_in,
//   U     = (I + L)^{-1} Diag(beta)(V - K_decay S_in),  L = StrictTril(Diag(beta) K_decay K_inv^T)
//   O     = Q_decay S_in + M_qk U,                      M_qk = tril(Q_decay K_inv^T)
//   S_out = Diag(a_last) S_in + K_restore^T U
// a_t being the inclusive cumulative decay from the chunk start.
//
// Restated for the MI355X (every step below is exact algebra of the above):
//  * U is affine in S_in: U = U0 - W S_in with U0 = INV Diag(beta) V and
//    W = INV Diag(beta) K_decay, INV = (I + L)^{-1}. U0 and W are built by
//    forward substitution over four 16-token blocks (fp32 inverses of the
//    16x16 diagonal blocks, bf16 MFMA elsewhere). Only three MFMA passes then
//    depend on the state: U, then O and S_out.
//  * Decay factors never overflow. In a chunk whose every 8-token range
//    decays by at most exp(-8) per channel (all but extreme inputs), the Gram
//    entry for key s <= query t is  sum_d (k_t a_t)[d] (k_s / a_s)[d]  with a
//    the decay from the chunk start: 1/a_s <= exp(64). Otherwise the chunk
//    takes the 16-token block factorisation: with b_t the decay from the
//    start of t's block, the entry for t in block I and s in block J <= I is
//    sum_d (k_t b_t)[d] (k_s / b_s)[d] G_IJ[d], G_IJ the decay over blocks
//    J..I-1 (1 on the diagonal); every factor is <= 1 except 1/b_s <=
//    exp(80) for log-decays in [-5, 0] (the bound on the trillion-scale
//    architecture page, section 4). Both stay inside fp32/bf16 range, and
//    K_decay, Q_decay and K_restore are products of factors <= 1.
//
// Kernels:
//  * fused_kernel: one workgroup per (batch*head, 16*NW value columns); walks
//    the whole sequence. The state block lives in MFMA accumulators (wave w
//    owns 16 columns x 128 rows) and feeds the next chunk's MFMAs directly as
//    the B operand: the K index of each 32-deep step is permuted identically
//    on both operands, so no LDS round trip is needed. The next chunk's
//    inputs are loaded into registers while the current one computes.
//  * prep_kernel + state_kernel: for few heads. The prep kernel runs the
//    state-independent work of many chunks in parallel and writes, per
//    chunk-head, -W, Q_decay, K_restore^T, M_qk (bf16, in MFMA operand
//    register order), U0 and a_last to a workspace. The state
//    kernel then walks the chunks in order doing only the three state
//    passes, twelve waves per 16 value columns: four compute U, four
//    update the state, four form the output rows; each loads only its
//    operands, straight into MFMA registers, while the other passes run.
#include <algorithm>
#include <type_traits>

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace mf {

constexpr int DK = 128;
constexpr int C = 64;
constexpr int KS = 136;            // padded row stride (bf16) of [64][128] tiles
constexpr int TS = 72;             // padded row stride (bf16) of [*][64] tiles
constexpr int LDT = 16 * 16 + 4;   // fp32 stride of one diagonal L block
// A chunk whose token ranges all decay by at most exp(-kRangeDecay) per
// channel uses the chunk-level decay reference (1/a <= exp(8 * kRangeDecay)).
constexpr float kRangeDecay = 8.f;
constexpr float kLog2e = 1.4426950408889634f;
// Per-step log-decays are clamped into [-5, 0], the supported range (the
// bound on the trillion-scale architecture page, section 4; a decay never
// exceeds 1). A 16-token block then needs 1/b <= exp(80), inside fp32 and
// bf16, so every input gives finite results; a step that decays harder than
// exp(-5) keeps exp(-5) of the old state instead of less (within about 0.7%
// of the exact step for that channel).
constexpr float kLogDecayFloor = -5.f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// Per-chunk operands prepared in LDS.
struct Prep {
    bf16 Kd[C * KS];     // k_t b_t                  Gram left (L), K_decay = Kd * P
    bf16 Qd[C * KS];     // q_t b_t                  Gram left (M); then Q_decay in place
    bf16 Ki[C * KS];     // k_s / b_s                Gram right; then -W in place
    bf16 KrT[DK * TS];   // K_restore^T [channel][token]
    bf16 RkT[DK * TS];   // (Diag(beta) K_decay)^T [channel][token]: substitution input
    bf16x8 NWop[16][64]; // -W as A operands (I, kk), operand-record order
    bf16x8 Mop[6][64];   // M_qk as A operands (0,0),(1,0),(2,0),(3,0),(2,1),(3,1)
    bf16x4 NLt[6][64];   // -L_IJ, J < I, as 16x16x16 A operands, pair I(I-1)/2 + J
    bf16x4 Dt[4][64];    // (I + L_II)^{-1} as 16x16x16 A operands
    float Lt[4 * LDT];   // diagonal blocks of L, fp32, row-major [t][s]
    float P[4 * DK];     // decay from the chunk start to the start of block I
    float G[6 * DK];     // decay over blocks J..I-1 for the 6 pairs J < I
    float alast[DK];     // decay over the whole chunk
    float Tot[8 * DK];   // log-decay sums of the 8-or-4 token ranges
    float beta[C];
    float qs[C], ks[C];  // layer prologue: per-token L2 factors of q and k
    int strong[8];       // per token range: some channel decays by more than kRangeDecay
};

// Operand record written by the prep kernel, read by the state kernel, in
// MFMA register order: each A operand of a 16x16x32 step is 1 KB, 16 bytes
// per lane in lane order, so a wave loads it with one coalesced dwordx4
// load straight into the registers the MFMA reads.
//   NW  : -W      operands (I, kk), I, kk in 0..3          16 KB
//   QD  : Q_decay operands (I, kk)                          16 KB
//   M   : M_qk    operands (0,0),(1,0),(2,0),(3,0),(2,1),(3,1)  6 KB
//   KR  : K_restore^T operands (m, kk), m in 0..7, kk in 0..1  16 KB
//   AL  : a_last, 128 fp32
//   U0  : U0 tiles (I, value tile ct) in accumulator order, bf16   16 KB
constexpr int OPB = 1024;
constexpr int REC_NW = 0;
constexpr int REC_QD = REC_NW + 16 * OPB;
constexpr int REC_M = REC_QD + 16 * OPB;
constexpr int REC_KR = REC_M + 6 * OPB;
constexpr int REC_AL = REC_KR + 16 * OPB;
constexpr int REC_U0 = REC_AL + DK * 4;
constexpr int REC_BYTES = REC_U0 + C * 128 * 2;
static_assert(REC_BYTES % 256 == 0, "record alignment");

// The 10 lower block pairs (I, J), row-major, 2 bits per entry.
constexpr uint32_t kPairI = (0u << 0) | (1u << 2) | (1u << 4) | (2u << 6) | (2u << 8) |
                            (2u << 10) | (3u << 12) | (3u << 14) | (3u << 16) | (3u << 18);
constexpr uint32_t kPairJ = (0u << 0) | (0u << 2) | (1u << 4) | (0u << 6) | (1u << 8) |
                            (2u << 10) | (0u << 12) | (1u << 14) | (2u << 16) | (3u << 18);

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ s16x4 ld4(const bf16* p) { return *reinterpret_cast<const s16x4*>(p); }

// A operand of a 32-deep step whose K index follows the accumulator-pair
// permutation: slots 0..3 <- k0 + 4g + (0..3), slots 4..7 <- k0 + 16 + 4g + (0..3).
__device__ __forceinline__ bf16x8 ldA_perm(const bf16* rowp, int k0, int g) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(rowp + k0 + 4 * g);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(rowp + k0 + 16 + 4 * g);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ __forceinline__ f32x2 unpack2(uint32_t u) {
    return __builtin_convertvector(__builtin_bit_cast(bf16x2, u), f32x2);
}

// Multiply eight bf16 operand values by per-channel factors.
__device__ __forceinline__ bf16x8 scale8(bf16x8 v, f32x4 g0, f32x4 g1) {
    f32x8 f = __builtin_convertvector(v, f32x8);
    f32x8 gg = __builtin_shufflevector(g0, g1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_convertvector(f * gg, bf16x8);
}

// ---------------------------------------------------------------------------
// Chunk inputs held in registers between the load and the elementwise stage.
template <int NW>
struct Inputs {
    static constexpr int TPT = C / NW;        // tokens per thread (16 or 8)
    uint32_t k[TPT], q[TPT];                  // two channels, bf16 pair
    f32x2 la[TPT];                            // two channels' log-decay (raw gate bits
                                              // in .x for kGateBounded until converted)
    uint4 v[2];                               // two 16-byte pieces of the value block
    float beta;
};

// Load chunk c of a sequence's inputs. Thread (wave = token range, lane =
// channel pair).
// Loads are unconditional (tail tokens re-read the last token) and the raw
// values are kept as loaded: tail tokens are zeroed where they are consumed,
// so no instruction waits on a load before the next chunk is needed.
// Buffer loads: the chunk's first row of head h is the (scalar) base of each
// resource, a token's row a scalar offset and the lane's channels a vector
// offset fixed for the whole call, so issuing a load costs no vector address
// arithmetic. Offsets inside one chunk stay far below 2^31; each resource
// ends after the chunk's last real row, so nothing past it is ever read.
template <int NW, int DVB, int PRO, bool NT = false>
__device__ __forceinline__ void load_inputs(Inputs<NW>& in, const bf16* __restrict__ q,
                                            const bf16* __restrict__ k,
                                            const bf16* __restrict__ v,
                                            const void* __restrict__ gate,
                                            const float* __restrict__ beta, long tok0, int len,
                                            int h, int H, int c, int col0)
{
    constexpr int GM = PRO & 3;
    constexpr int TPT = C / NW;
    constexpr int VPR = DVB / 8;   // 16-byte pieces per value row
    constexpr int AUX = NT ? 2 : 0;   // cache policy: non-temporal
    constexpr int RSRC3 = 0x00020000;
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int t0 = wave * TPT;
    const int last = min(C, len - c * C) - 1;             // last real token of the chunk
    const size_t row0 = ((size_t)tok0 + (size_t)c * C) * H + h;
    const int rs2 = H * (DK * 2);                         // token stride of q, k (bytes)
    const int n2 = last * rs2 + DK * 2;
    const auto rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + row0 * DK), 0, n2, RSRC3);
    const auto rq = __builtin_amdgcn_make_buffer_rsrc((void*)(q + row0 * DK), 0, n2, RSRC3);
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
        const int tok = min(t0 + j, last);
        in.k[j] = __builtin_amdgcn_raw_buffer_load_b32(rk, 4 * lane, tok * rs2, AUX);
        in.q[j] = __builtin_amdgcn_raw_buffer_load_b32(rq, 4 * lane, tok * rs2, AUX);
    }
    if constexpr (GM == kGateLog) {
        const int rs4 = H * (DK * 4);
        const auto rg = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(static_cast<const float*>(gate) + row0 * DK), 0, last * rs4 + DK * 4, RSRC3);
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rg, 8 * lane, min(t0 + j, last) * rs4, AUX);
            in.la[j] = __builtin_bit_cast(f32x2, x);
        }
    } else if constexpr (GM == kGateBounded) {
        const auto rg = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(static_cast<const bf16*>(gate) + row0 * DK), 0, n2, RSRC3);
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const uint32_t bits = __builtin_amdgcn_raw_buffer_load_b32(rg, 4 * lane, min(t0 + j, last) * rs2, AUX);
            in.la[j] = f32x2{__builtin_bit_cast(float, bits), 0.f};
        }
    } else {
        const auto rg = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(static_cast<const float*>(gate) + row0), 0, last * H * 4 + 4, RSRC3);
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const float a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                rg, 0, min(t0 + j, last) * (H * 4), AUX));
            in.la[j] = f32x2{a, a};
        }
    }
    const int rsv = H * 256;                              // token stride of v (bytes)
    const auto rv = __builtin_amdgcn_make_buffer_rsrc((void*)(v + row0 * 128), 0, last * rsv + 256, RSRC3);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int piece = tid + p * NW * 64;
        const int t = piece / VPR, c8 = piece - t * VPR;
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(
            rv, min(t, last) * rsv + (col0 + 8 * c8) * 2, 0, AUX);
        in.v[p] = make_uint4(x[0], x[1], x[2], x[3]);
    }
    if (tid < C) {
        const auto rb = __builtin_amdgcn_make_buffer_rsrc((void*)(beta + row0), 0, last * H * 4 + 4, RSRC3);
        in.beta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, min(tid, last) * (H * 4), 0, AUX));
    }
}

// Layer prologue on a chunk's inputs, before stage 1a: the bounded gate's
// log-decay -bound * sigmoid(g) in fp32, and with kProL2 the per-token
// factors 1 / sqrt(|q|^2 + eps), 1 / sqrt(|k|^2 + eps) to LDS (stage 1b
// scales q and k by them, so each operand is rounded to bf16 once).
template <int NW, int PRO>
__device__ __forceinline__ void prologue(Prep& sm, Inputs<NW>& in, const Prologue& pr) {
    constexpr int TPT = C / NW;
    if constexpr ((PRO & 3) == kGateBounded) {
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const f32x2 g = unpack2(__builtin_bit_cast(u32x2, in.la[j])[0]);   // raw gate bits in .x
            in.la[j] = f32x2{-pr.bound * sigmoid_f(g[0]), -pr.bound * sigmoid_f(g[1])};
        }
    }
    // (the host rejects a bounded gate past the floor: that form is always
    // inside the range)
    if constexpr ((PRO & 3) != kGateBounded) {
#pragma unroll
        for (int j = 0; j < TPT; ++j)
            in.la[j] = f32x2{__builtin_amdgcn_fmed3f(in.la[j][0], kLogDecayFloor, 0.f),
                             __builtin_amdgcn_fmed3f(in.la[j][1], kLogDecayFloor, 0.f)};
    }
    if constexpr ((PRO & kProL2) != 0) {
        // squared norms by packed bf16 dot products (v_dot2: no unpacked
        // copies that could stay live until stage 1b), summed over the wave
        // without LDS; lane 0 stores the factors of the range's tokens
        const int lane = threadIdx.x & 63, wave = wave_id();
        float fq[TPT], fk[TPT];
#pragma unroll
        for (int j = 0; j < TPT; ++j) {
            const bf16x2 qq = __builtin_bit_cast(bf16x2, in.q[j]);
            const bf16x2 kk = __builtin_bit_cast(bf16x2, in.k[j]);
            fq[j] = __builtin_amdgcn_rsqf(
                wave_sum_uniform(__builtin_amdgcn_fdot2_f32_bf16(qq, qq, 0.f, false)) + pr.l2_eps);
            fk[j] = __builtin_amdgcn_rsqf(
                wave_sum_uniform(__builtin_amdgcn_fdot2_f32_bf16(kk, kk, 0.f, false)) + pr.l2_eps);
        }
        if (lane == 0) {
#pragma unroll
            for (int j = 0; j < TPT; j += 4) {
                *reinterpret_cast<f32x4*>(&sm.qs[wave * TPT + j]) = f32x4{fq[j], fq[j + 1], fq[j + 2], fq[j + 3]};
                *reinterpret_cast<f32x4*>(&sm.ks[wave * TPT + j]) = f32x4{fk[j], fk[j + 1], fk[j + 2], fk[j + 3]};
            }
        }
    }
}

// Stage 1a: per-range log-decay sums; values and beta to LDS. Tokens at or
// past ntok are padding: zero decay, value and beta (exact, the recurrence
// leaves the state unchanged for them). Each range also records whether some
// channel decays by more than kRangeDecay over it.
template <int NW, int DVB>
__device__ __forceinline__ void stage1a(Prep& sm, bf16* sV, const Inputs<NW>& in, int ntok) {
    constexpr int TPT = C / NW;
    constexpr int VPR = DVB / 8;
    constexpr int VS = DVB + 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int t0 = wave * TPT;
    f32x2 sum = {0.f, 0.f};
#pragma unroll
    for (int j = 0; j < TPT; ++j) sum += (t0 + j < ntok) ? in.la[j] : f32x2{0.f, 0.f};
    *reinterpret_cast<f32x2*>(&sm.Tot[wave * DK + 2 * lane]) = sum;
    const bool strong = __builtin_amdgcn_ballot_w64(fminf(sum[0], sum[1]) < -kRangeDecay) != 0;
    if (lane == 0) sm.strong[wave] = strong;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int piece = tid + p * NW * 64;
        const int t = piece / VPR, c8 = piece - t * VPR;
        *reinterpret_cast<uint4*>(&sV[t * VS + 8 * c8]) = (t < ntok) ? in.v[p] : make_uint4(0u, 0u, 0u, 0u);
    }
    if (tid < C) sm.beta[tid] = (tid < ntok) ? in.beta : 0.f;
}

// True when no token range of the chunk has a strongly decaying channel:
// the chunk then uses the chunk-level decay reference. Wave-uniform.
template <int NW>
__device__ __forceinline__ bool chunk_is_mild(const Prep& sm) {
    int any = 0;
#pragma unroll
    for (int s = 0; s < NW; ++s) any |= sm.strong[s];
    return __builtin_amdgcn_readfirstlane(any) == 0;
}

// Stage 1b: decay-scaled operands. Thread (range = wave, channels 2*lane, +1).
// The decay reference is the chunk start when `fast`, else the start of the
// token's 16-token block. FULL: every token of the chunk is real.
template <int NW, bool FULL, int PRO, bool FAST>
__device__ __forceinline__ void stage1b(Prep& sm, const Inputs<NW>& in, int ntok) {
    constexpr bool fast = FAST;
    constexpr int TPT = C / NW;
    constexpr int SPB = NW / 4;      // token ranges per 16-token block
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int t0 = wave * TPT;
    const int blk = t0 >> 4;
    const int d0 = 2 * lane;

    f32x2 tau[4];                    // per-block log-decay totals, both channels
    f32x2 offb = {0.f, 0.f};         // log-decay from the block start to this range
    f32x2 offc = {0.f, 0.f};         // log-decay from the chunk start to this range
#pragma unroll
    for (int m = 0; m < 4; ++m) tau[m] = f32x2{0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NW; ++s) {
        const float2 v = *reinterpret_cast<const float2*>(&sm.Tot[s * DK + d0]);
        const f32x2 vv = {v.x, v.y};
        tau[s / SPB] += vv;
        if (s < wave) offc += vv;
        if (s / SPB == blk && s < wave) offb += vv;
    }
    const f32x2 all = tau[0] + tau[1] + tau[2] + tau[3];
    f32x2 head = {0.f, 0.f};         // chunk start to the start of this block
#pragma unroll
    for (int m = 0; m < 4; ++m) if (m < blk) head += tau[m];
    // K_restore factor: decay from the reference point to the chunk end;
    // Diag(beta) K_decay factor: decay from the chunk start to the reference
    const f32x2 tail = fast ? all : all - head;
    const f32x2 eR = {exp_e(tail[0]), exp_e(tail[1])};
    const f32x2 eP = fast ? f32x2{1.f, 1.f} : f32x2{exp_e(head[0]), exp_e(head[1])};

    // chunk-level factors, spread over the first four token ranges (the
    // block decays P and G serve the block reference only)
    if (!fast && wave == 0) {
        f32x2 acc = {0.f, 0.f};
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            *reinterpret_cast<float2*>(&sm.P[I * DK + d0]) = make_float2(exp_e(acc[0]), exp_e(acc[1]));
            acc += tau[I];
        }
    } else if (!fast && (wave == 1 || wave == 2)) {
        // G for pairs (1,0),(2,0),(2,1) on range 1 and (3,0),(3,1),(3,2) on range 2
#pragma unroll
        for (int e = 0; e < 3; ++e) {
            const int I = (wave == 1) ? (e == 0 ? 1 : 2) : 3;
            const int J = (wave == 1) ? (e == 2 ? 1 : 0) : e;
            f32x2 sum = {0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; ++m) if (m >= J && m < I) sum += tau[m];
            const int pidx = I * (I - 1) / 2 + J;
            *reinterpret_cast<float2*>(&sm.G[pidx * DK + d0]) = make_float2(exp_e(sum[0]), exp_e(sum[1]));
        }
    } else if (wave == 3) {
        *reinterpret_cast<float2*>(&sm.alast[d0]) = make_float2(exp_e(all[0]), exp_e(all[1]));
    }

    // running log2-decay from the reference point; b_t = 2^run, 1/b_t = 2^-run
    f32x2 run = (fast ? offc : offb) * kLog2e;
    float kr0[TPT], kr1[TPT], rk0[TPT], rk1[TPT];
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
        const int t = t0 + j;
        const bool ok = FULL || t < ntok;
        const f32x2 la = ok ? in.la[j] : f32x2{0.f, 0.f};
        run = la * kLog2e + run;
        const f32x2 bt = {__builtin_amdgcn_exp2f(run[0]), __builtin_amdgcn_exp2f(run[1])};    // <= 1
        const f32x2 ib = {__builtin_amdgcn_exp2f(-run[0]), __builtin_amdgcn_exp2f(-run[1])};  // bounded above
        f32x2 kk = ok ? unpack2(in.k[j]) : f32x2{0.f, 0.f};
        f32x2 qq = ok ? unpack2(in.q[j]) : f32x2{0.f, 0.f};
        if constexpr ((PRO & kProL2) != 0) {
            kk *= sm.ks[t];
            qq *= sm.qs[t];
        }
        const f32x2 kd = kk * bt;
        const f32x2 ki = kk * ib;
        *reinterpret_cast<uint32_t*>(&sm.Kd[t * KS + d0]) = pack2(kd[0], kd[1]);
        *reinterpret_cast<uint32_t*>(&sm.Qd[t * KS + d0]) = pack2(qq[0] * bt[0], qq[1] * bt[1]);
        *reinterpret_cast<uint32_t*>(&sm.Ki[t * KS + d0]) = pack2(ki[0], ki[1]);
        kr0[j] = ki[0] * eR[0];                              // decay t+1 .. chunk end
        kr1[j] = ki[1] * eR[1];
        const float bta = sm.beta[t];
        if constexpr (fast) {                                // beta_t k_t decay(start .. t)
            rk0[j] = bta * kd[0];
            rk1[j] = bta * kd[1];
        } else {
            rk0[j] = bta * kd[0] * eP[0];
            rk1[j] = bta * kd[1] * eP[1];
        }
    }
    auto put8 = [&](bf16* dst, const float* x) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(pack2(x[0], x[1]), pack2(x[2], x[3]),
                                                    pack2(x[4], x[5]), pack2(x[6], x[7]));
    };
#pragma unroll
    for (int p = 0; p < TPT / 8; ++p) {
        put8(&sm.KrT[d0 * TS + t0 + 8 * p], kr0 + 8 * p);
        put8(&sm.KrT[(d0 + 1) * TS + t0 + 8 * p], kr1 + 8 * p);
        put8(&sm.RkT[d0 * TS + t0 + 8 * p], rk0 + 8 * p);
        put8(&sm.RkT[(d0 + 1) * TS + t0 + 8 * p], rk1 + 8 * p);
    }
}

// Stage 2: Gram blocks -> -L, M_qk, computed transposed: for the pair (I, J),
// J <= I, A = K_inv rows of block J (times G_IJ off the diagonal, block
// reference only) and B =
// K_decay or Q_decay rows of block I leave lane (g, r) holding the entries
// (t = 16I + r, s = 16J + 4g + i): row r of the block, which is the A
// operand of a 16x16x16 step and one half of a 16x16x32 one, so each block
// is stored with a single 8-byte write per lane. The wave owning a diagonal
// block then forms rows of (I + L_II)^{-1} in fp32.
template <int NW>
__device__ __forceinline__ void stage2(Prep& sm, bool fast) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, r = lane & 15;
    // Work list per wave, 4 bits per pair index (15 = none), at most 3 pairs.
    // 8 waves: the diagonal blocks on waves 0-3 (each followed by its
    // inverse), off-diagonal pairs 2+2+1+1 on waves 4-7. 4 waves: each takes a
    // diagonal block plus off-diagonal pairs 2, 2, 1, 1.
    // Pair indices: 0 (0,0) 1 (1,0) 2 (1,1) 3 (2,0) 4 (2,1) 5 (2,2) 6 (3,0) 7 (3,1) 8 (3,2) 9 (3,3).
    constexpr uint32_t kList8[8] = {0xFF0u, 0xFF2u, 0xFF5u, 0xFF9u, 0xF31u, 0xF64u, 0xFF7u, 0xFF8u};
    constexpr uint32_t kList4[4] = {0x310u, 0x642u, 0xF75u, 0xF89u};
    const uint32_t list = (NW == 8) ? kList8[wave] : kList4[wave];
#pragma unroll
    for (int slot = 0; slot < 3; ++slot) {
        const int p = (list >> (4 * slot)) & 15;
        if (p == 15) break;
        const int I = (kPairI >> (2 * p)) & 3, J = (kPairJ >> (2 * p)) & 3;
        const bool diag = I == J;
        const bf16* ap = sm.Ki + (16 * J + r) * KS + 8 * g;
        bf16x8 Ak[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) Ak[kk] = ld8(ap + 32 * kk);
        if (!diag && !fast) {
            const float* gp = sm.G + (I * (I - 1) / 2 + J) * DK + 8 * g;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                Ak[kk] = scale8(Ak[kk], *reinterpret_cast<const f32x4*>(gp + 32 * kk),
                                *reinterpret_cast<const f32x4*>(gp + 32 * kk + 4));
        }
        const bf16* kp = sm.Kd + (16 * I + r) * KS + 8 * g;
        const bf16* qp = sm.Qd + (16 * I + r) * KS + 8 * g;
        const float bt = sm.beta[16 * I + r];
        f32x4 aK = zero4(), aQ = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            aK = mma32(Ak[kk], ld8(kp + 32 * kk), aK);
            aQ = mma32(Ak[kk], ld8(qp + 32 * kk), aQ);
        }
        f32x4 lv, mv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = 4 * g + i;                 // key token inside block J
            lv[i] = (!diag || s < r) ? bt * aK[i] : 0.f;
            mv[i] = (!diag || s <= r) ? aQ[i] : 0.f;
        }
        // M_qk operand (I, J / 2) takes this block as its half J % 2; the
        // halves above the diagonal, (0, 1) and (2, 3), are zero
        bf16x4* mop = reinterpret_cast<bf16x4*>(&sm.Mop[(J < 2) ? I : I + 2][lane]);
        mop[J & 1] = __builtin_convertvector(mv, bf16x4);
        if (diag && (I & 1) == 0) mop[1] = bf16x4{};
        if (!diag) {
            sm.NLt[I * (I - 1) / 2 + J][lane] = __builtin_convertvector(-lv, bf16x4);
        } else {
            float* Lr = sm.Lt + I * LDT;
            *reinterpret_cast<f32x4*>(&Lr[r * 16 + 4 * g]) = lv;          // row-major [t][s]
            lds_fence_wave();
            // row r of (I + L)^{-1}: y (I + L) = e_r. Right-looking over the
            // rows i = 15..0 of L: y_i = [i == r] + p_i, then p_j -= y_i L[i][j]
            // for j < i, so each step is one dependent add plus independent
            // updates (y is zero above r). Rows of L are read two steps ahead
            // so their LDS latency overlaps the updates.
            float y[16], p[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) p[j] = 0.f;
            f32x4 row[3][4];
            auto load_row = [&](f32x4 (&dst)[4], int i) {
#pragma unroll
                for (int j4 = 0; j4 < 16; j4 += 4)
                    if (j4 < i) dst[j4 / 4] = *reinterpret_cast<const f32x4*>(&Lr[i * 16 + j4]);
            };
            load_row(row[15 % 3], 15);
            load_row(row[14 % 3], 14);
#pragma unroll
            for (int i = 15; i >= 0; --i) {
                if (i >= 2) load_row(row[(i - 2) % 3], i - 2);
                y[i] = ((i == r) ? 1.f : 0.f) + p[i];
#pragma unroll
                for (int j = 0; j < i; ++j) p[j] -= y[i] * row[i % 3][j / 4][j % 4];
            }
            // lane (g, r) keeps y[4g .. 4g + 3], picked with bit masks:
            // conditionals here compile to divergent branches or to an
            // indexed copy of y in scratch memory
            f32x4 d;
            const uint32_t m1 = (g & 1) ? ~0u : 0u, m2 = (g & 2) ? ~0u : 0u;
            auto pick = [](uint32_t m, float a, float b) {   // m ? b : a
                return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, a) & ~m) |
                                                     (__builtin_bit_cast(uint32_t, b) & m));
            };
#pragma unroll
            for (int i = 0; i < 4; ++i)
                d[i] = pick(m2, pick(m1, y[i], y[4 + i]), pick(m1, y[8 + i], y[12 + i]));
            sm.Dt[I][lane] = __builtin_convertvector(d, bf16x4);
        }
    }
}

// Stage 3: Q_decay in place (block reference only: with the chunk reference
// Qd already is Q_decay); forward substitution for -W and U0.
// Tiles: W channel tiles wave, wave + NW (< 8), then the U0 tile at u0col.
// Block I: Y_I -= sum_{J<I} L_IJ X_J, then X_I = D_I Y_I (accumulator order,
// feeds later blocks as the B operand) and, for W, X_I^T = Y_I^T D_I^T: its
// accumulator holds W rows in A-operand order, stored straight into NWop.
struct NoHook { __device__ void operator()(int) const {} };

// NWG: -W goes straight from registers to the operand record at nw_rec
// (each wave its own 8-byte half of each operand) instead of to sm.NWop.
template <int NW, int DVB, typename Hook = NoHook, bool NWG = false>
__device__ __forceinline__ void stage3(Prep& sm, const bf16* sV, int u0col, f32x4 (&U0)[4], bool fast,
                                       Hook hook = Hook(), char* nw_rec = nullptr) {
    constexpr int VS = DVB + 8;
    constexpr int NWT = 8 / NW;
    constexpr int NTILE = NWT + 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int g = lane >> 4, r = lane & 15;

    for (int idx = tid; !fast && idx < C * 64; idx += NW * 64) {
        const int t = idx >> 6, d = 2 * (idx & 63);
        uint32_t* p = reinterpret_cast<uint32_t*>(&sm.Qd[t * KS + d]);
        const f32x2 a = unpack2(*p);
        const float2 f = *reinterpret_cast<const float2*>(&sm.P[(t >> 4) * DK + d]);
        *p = pack2(a[0] * f.x, a[1] * f.y);
    }
    // a hook that reads Q_decay needs the scaling above from every thread
    if constexpr (!std::is_same<Hook, NoHook>::value)
        if (!fast) lds_barrier();

    f32x4 X[NTILE][4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        f32x4 Y[NTILE];
#pragma unroll
        for (int tl = 0; tl < NTILE; ++tl) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * I + 4 * g + i;
                if (tl == NWT) Y[tl][i] = sm.beta[t] * (float)sV[t * VS + u0col + r];
            }
            if (tl < NWT) {
                const int d = 16 * (wave + tl * NW) + r;
                const bf16x4 rk = *reinterpret_cast<const bf16x4*>(&sm.RkT[d * TS + 16 * I + 4 * g]);
                Y[tl] = __builtin_convertvector(rk, f32x4);
            }
        }
#pragma unroll
        for (int J = 0; J < I; ++J) {
            const s16x4 a = __builtin_bit_cast(s16x4, sm.NLt[I * (I - 1) / 2 + J][lane]);
#pragma unroll
            for (int tl = 0; tl < NTILE; ++tl) Y[tl] = mma16(a, pack4(X[tl][J]), Y[tl]);
        }
        const s16x4 dI = __builtin_bit_cast(s16x4, sm.Dt[I][lane]);
#pragma unroll
        for (int tl = 0; tl < NTILE; ++tl) {
            const s16x4 yb = pack4(Y[tl]);
            X[tl][I] = mma16(dI, yb, zero4());
            if (tl < NWT) {
                const f32x4 xt = mma16(yb, dI, zero4());
                const int dt = wave + tl * NW;                // channel tile
                const bf16x4 nw = __builtin_convertvector(-xt, bf16x4);
                if constexpr (NWG)
                    *reinterpret_cast<bf16x4*>(nw_rec + REC_NW + (I * 4 + (dt >> 1)) * OPB + lane * 16 + (dt & 1) * 8) = nw;
                else
                    reinterpret_cast<bf16x4*>(&sm.NWop[I * 4 + (dt >> 1)][lane])[dt & 1] = nw;
            }
        }
        hook(I);
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) U0[I] = X[NWT][I];
}

// The three state passes for one chunk and this wave's 16 value columns:
// U = U0 - W S, O = Q_decay S + M_qk U, S = Diag(a_last) S + K_restore^T U.
// Every A operand comes from LDS in operand order (one 16-byte read per lane:
// -W (I, kk), Q_decay (I, kk) at 4 I + kk, M_qk, K_restore^T (m, kk) at 2 m + kk).
// O[I] receives rows 16I + 4g + (0..3) of column r (MFMA accumulator layout).
// PRELOAD reads all LDS operands of a pass before its MFMAs so the reads
// overlap (needs ~130 more registers); otherwise the reads run a few MFMA
// steps ahead of their use.
// `between(k)` is called after the k-th of four MFMA groups (k = 0..3) so a
// caller can slot other instructions (the next chunk's loads) under the MFMAs.
struct NoOp { __device__ void operator()(int) const {} };

template <bool PRELOAD, typename Between = NoOp>
__device__ __forceinline__ void state_pass(f32x4 (&Sacc)[8], const f32x4 (&U0)[4],
                                           const bf16x8 (*nW)[64], const bf16x8 (*Qop)[64],
                                           const bf16x8 (*M)[64], const bf16x8 (*Krop)[64],
                                           const float* alast, f32x4 (&O)[4],
                                           Between between = Between())
{
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, r = lane & 15;
    bf16x8 SB[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) SB[kk] = pack8(Sacc[2 * kk], Sacc[2 * kk + 1]);

    f32x4 accU[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        accU[I] = U0[I];
        O[I] = zero4();
    }
    if (PRELOAD) {
        bf16x8 aW[4][4], aQ[4][4];
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                aW[I][kk] = nW[I * 4 + kk][lane];
                aQ[I][kk] = Qop[I * 4 + kk][lane];
            }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                accU[I] = mma32(aW[I][kk], SB[kk], accU[I]);
                O[I] = mma32(aQ[I][kk], SB[kk], O[I]);
            }
            __builtin_amdgcn_sched_barrier(0);
            between(kk);
            __builtin_amdgcn_sched_barrier(0);
        }
    } else {
        // LDS operand reads run D steps ahead of their MFMAs (step s = kk * 4
        // + I: consecutive steps feed independent accumulators); the M_qk
        // operands are read in the last steps, when no W/Q reads remain
        constexpr int D = 3;
        bf16x8 bw[D], bq[D], mop[6];
        auto ld_wq = [&](int s, bf16x8& w, bf16x8& q) {
            const int I = s & 3, kk = s >> 2;
            w = nW[I * 4 + kk][lane];
            q = Qop[I * 4 + kk][lane];
        };
#pragma unroll
        for (int s = 0; s < D; ++s) ld_wq(s, bw[s], bq[s]);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
            const int I = s & 3, kk = s >> 2;
            const bf16x8 w = bw[s % D], q = bq[s % D];
            if (s + D < 16) {
                ld_wq(s + D, bw[s % D], bq[s % D]);
            } else {
                const int j = 2 * (s + D - 16);       // 0, 2, 4
                mop[j] = M[j][lane];
                mop[j + 1] = M[j + 1][lane];
            }
            __builtin_amdgcn_sched_barrier(0);
            accU[I] = mma32(w, SB[kk], accU[I]);
            O[I] = mma32(q, SB[kk], O[I]);
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 UB[2];
        UB[0] = pack8(accU[0], accU[1]);
        UB[1] = pack8(accU[2], accU[3]);
        // K_restore^T pairs, two ahead
        bf16x8 bk[2][2];
        f32x4 bal[2];
        auto ld_k = [&](int m, bf16x8 (&kb)[2], f32x4& al) {
            kb[0] = Krop[2 * m][lane];
            kb[1] = Krop[2 * m + 1][lane];
            al = *reinterpret_cast<const f32x4*>(&alast[16 * m + 4 * g]);
        };
        ld_k(0, bk[0], bal[0]);
        ld_k(1, bk[1], bal[1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int I = 0; I < 4; ++I) O[I] = mma32(mop[I], UB[0], O[I]);
        O[2] = mma32(mop[4], UB[1], O[2]);
        O[3] = mma32(mop[5], UB[1], O[3]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const bf16x8 k0 = bk[m & 1][0], k1 = bk[m & 1][1];
            const f32x4 al = bal[m & 1];
            if (m + 2 < 8) ld_k(m + 2, bk[m & 1], bal[m & 1]);
            __builtin_amdgcn_sched_barrier(0);
            Sacc[m] *= al;
            Sacc[m] = mma32(k0, UB[0], Sacc[m]);
            Sacc[m] = mma32(k1, UB[1], Sacc[m]);
            __builtin_amdgcn_sched_barrier(0);
        }
        return;
    }
    bf16x8 UB[2];
    UB[0] = pack8(accU[0], accU[1]);
    UB[1] = pack8(accU[2], accU[3]);

#pragma unroll
    for (int I = 0; I < 4; ++I) O[I] = mma32(M[I][lane], UB[0], O[I]);
    O[2] = mma32(M[4][lane], UB[1], O[2]);
    O[3] = mma32(M[5][lane], UB[1], O[3]);
    {
        bf16x8 aK[8][2];
        f32x4 al[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            aK[m][0] = Krop[2 * m][lane];
            aK[m][1] = Krop[2 * m + 1][lane];
            al[m] = *reinterpret_cast<const f32x4*>(&alast[16 * m + 4 * g]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            Sacc[m] *= al[m];
            Sacc[m] = mma32(aK[m][0], UB[0], Sacc[m]);
            Sacc[m] = mma32(aK[m][1], UB[1], Sacc[m]);
        }
    }
}

// Store a 64 x 16 output tile (accumulator layout) as bf16, tokens < ntok.
// The tile goes through `stage` (this wave's 64 x 24 bf16 slot of an LDS
// buffer that is dead during the state pass) so that each lane stores one
// token's 16 columns with two 16-byte stores. Lanes past ntok store a copy of
// the last real token's row to that row (same data, same address), so every
// lane stores and the compiler sees a fixed number of stores.
constexpr int OTS = 24;   // staging row stride (bf16): 16-byte aligned, conflict-free reads
__device__ __forceinline__ void store_o(const f32x4 (&O)[4], bf16* stage, bf16* __restrict__ o,
                                        size_t row0, size_t rstride, int col0, int ntok) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int i = 0; i < 4; ++i) stage[(16 * I + 4 * g + i) * OTS + r] = (bf16)O[I][i];
    lds_fence_wave();
    const int t = min(lane, ntok - 1);
    const uint4 lo = *reinterpret_cast<const uint4*>(&stage[t * OTS]);
    const uint4 hi = *reinterpret_cast<const uint4*>(&stage[t * OTS + 8]);
    bf16* dst = o + (row0 + (size_t)t * rstride) * 128 + col0;
    *reinterpret_cast<uint4*>(dst) = lo;
    *reinterpret_cast<uint4*>(dst + 8) = hi;
}

// store_o for the layer epilogue: O (fp32, already normalised and weighted)
// goes through an fp32 staging slot, and lane t multiplies token t's 16
// values by sigmoid(z) (zv: its 16 gate values) before the one bf16 rounding.
constexpr int OTSF = 20;  // fp32 staging row stride: 16-byte aligned rows
__device__ __forceinline__ void store_o_gated(const f32x4 (&O)[4], float* stage, const uint4 (&zv)[2],
                                              bf16* __restrict__ o, size_t row0, size_t rstride,
                                              int col0, int ntok) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int i = 0; i < 4; ++i) stage[(16 * I + 4 * g + i) * OTSF + r] = O[I][i];
    lds_fence_wave();
    const int t = min(lane, ntok - 1);
    const uint32_t zw[8] = {zv[0].x, zv[0].y, zv[0].z, zv[0].w, zv[1].x, zv[1].y, zv[1].z, zv[1].w};
    uint32_t packed[8];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(&stage[t * OTSF + 4 * p]);
        const f32x2 za = unpack2(zw[2 * p]), zb = unpack2(zw[2 * p + 1]);
        packed[2 * p] = pack2(x[0] * sigmoid_f(za[0]), x[1] * sigmoid_f(za[1]));
        packed[2 * p + 1] = pack2(x[2] * sigmoid_f(zb[0]), x[3] * sigmoid_f(zb[1]));
    }
    bf16* dst = o + (row0 + (size_t)t * rstride) * 128 + col0;
    *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    *reinterpret_cast<uint4*>(dst + 8) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
}

}  // namespace mf

// ---------------------------------------------------------------------------
// Store this wave's part of a state block (Sacc[m][i] = row 16m + 4g + i,
// column ncol) to the [128][128] fp32 block at dst.
__device__ __forceinline__ void store_state(float* dst, const f32x4 (&Sacc)[8], int g, int ncol) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(size_t)(16 * m + 4 * g + i) * 128 + ncol] = Sacc[m][i];
}

// Fused kernel: one workgroup per (sequence*head, value block of 16*NW
// columns). With CKPT it also stores the state after every sq.K tokens of the
// sequence to checkpoint slot sq.ckpt0(i) + j - 1 (slots >= ck_slots are
// dropped). PRO selects the layer prologue (plain op: 0). EPI (128-column
// workgroups only, which hold a whole head's output row) applies the layer
// epilogue before the output store: per token the sum of o^2 over the
// row's columns is reduced inside each wave's 16 columns by DPP and across
// the eight waves through LDS, and z, fetched at the chunk start in the
// accumulator layout, gates the result.
// The body takes the LDS blocks and its block index from the kernel that
// runs it (the fused kernel, or the split schedule's mixed kernel). With
// sq.ord the j-th group of H workgroups takes sequence sq.ord[j]; with
// sq.mslot a split sequence leaves its end state in sq.mid instead of S_final.
template <int NW, bool CKPT, int PRO, bool EPI = false>
__device__ __forceinline__ void fused_body(
    mf::Prep& sm, bf16* sV, int blk,
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const void* __restrict__ gate, const float* __restrict__ beta,
    const float* S0, bf16* __restrict__ o, float* S_final, const SeqLayout& sq, int H, int NVB,
    float* __restrict__ S_ckpt, int ck_slots, const Prologue& pr, const Epilogue& ep)
{
    static_assert(!EPI || NW == 8, "the fused epilogue needs the whole row in one workgroup");
    using namespace mf;
    constexpr int DVB = NW * 16;

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int g = lane >> 4, r = lane & 15;
    const int vb = blk % NVB;
    const int bh0 = blk / NVB;
    const int j = bh0 / H, h = bh0 - j * H;
    const int b = sq.ord ? sq.ord[j] : j;
    const int bh = b * H + h;
    const int col0 = vb * DVB;
    const int ncol = col0 + 16 * wave + r;
    const long tok0 = sq.start(b);
    const int len = sq.len(b);

    f32x4 Sacc[8];
    const size_t sbase = (size_t)bh * DK * 128;
    if (S0) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sacc[m][i] = S0[sbase + (size_t)(16 * m + 4 * g + i) * 128 + ncol];
    } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) Sacc[m] = zero4();
    }

    Inputs<NW> in;
    const int nchunks = (len + C - 1) / C;
    const int ck_every = CKPT ? sq.K / C : 1;   // chunks per checkpoint
    const long ck0 = CKPT ? sq.ckpt0(b) : 0;
    if (nchunks > 0) load_inputs<NW, DVB, PRO>(in, q, k, v, gate, beta, tok0, len, h, H, 0, col0);
    const float epi_w = (EPI && ep.w) ? ep.w[ncol] : 1.f;

    for (int c = 0; c < nchunks; ++c) {
        const int ntok = len - c * C;
        lds_barrier();
        prologue<NW, PRO>(sm, in, pr);
        stage1a<NW, DVB>(sm, sV, in, ntok);
        lds_barrier();
        const bool fast = chunk_is_mild<NW>(sm);
        if (fast) {
            if (ntok >= C) stage1b<NW, true, PRO, true>(sm, in, ntok);
            else stage1b<NW, false, PRO, true>(sm, in, ntok);
        } else {
            if (ntok >= C) stage1b<NW, true, PRO, false>(sm, in, ntok);
            else stage1b<NW, false, PRO, false>(sm, in, ntok);
        }
        // next chunk's inputs; with 8 waves, waves 4-7 (lighter Gram work)
        // fetch after stage 2, so their fetches queue while the inverses finish
        const bool early_fetch = NW < 8 || wave < 4;
        if (c + 1 < nchunks && early_fetch) load_inputs<NW, DVB, PRO>(in, q, k, v, gate, beta, tok0, len, h, H, c + 1, col0);
        lds_barrier();
        stage2<NW>(sm, fast);
        if (c + 1 < nchunks && !early_fetch) load_inputs<NW, DVB, PRO>(in, q, k, v, gate, beta, tok0, len, h, H, c + 1, col0);
        lds_barrier();
        // Q_decay and K_restore^T to A-operand order in the slots of K_decay
        // and K_inv (dead since stage 2), one or two operands per wave after
        // each block of the substitution, under its matrix work: each wave
        // then reads every operand of the state pass with one conflict-free
        // 16-byte load per lane, where reading the row-major tiles takes two
        // 8-byte loads that collide in the LDS banks
        bf16x8 (*Qop)[64] = reinterpret_cast<bf16x8 (*)[64]>(sm.Kd);
        bf16x8 (*Krop)[64] = reinterpret_cast<bf16x8 (*)[64]>(sm.Ki);
        auto to_operands = [&](int I) {
#pragma unroll
            for (int u = 0; u < 8 / NW; ++u) {
                const int e = u * 4 * NW + I * NW + wave;   // 0 .. 31 over blocks and waves
                if (e < 16) {
                    Qop[e][lane] = ldA_perm(sm.Qd + (16 * (e >> 2) + r) * KS, 32 * (e & 3), g);
                } else {
                    const int jj = e - 16;
                    Krop[jj][lane] = ldA_perm(sm.KrT + (16 * (jj >> 1) + r) * TS, 32 * (jj & 1), g);
                }
            }
        };
        f32x4 U0[4];
        stage3<NW, DVB, decltype(to_operands)>(sm, sV, 16 * wave, U0, fast, to_operands);
        lds_barrier();
        // epilogue gate of this chunk in the output store's layout (lane t:
        // token t, this wave's 16 columns), fetched while the state pass runs
        uint4 zv[2];
        if constexpr (EPI) {
            const int t = min(lane, ntok - 1);
            const bf16* zp = static_cast<const bf16*>(ep.z) +
                             (((size_t)tok0 + (size_t)c * C + t) * H + h) * 128 + 16 * wave;
            zv[0] = *reinterpret_cast<const uint4*>(zp);
            zv[1] = *reinterpret_cast<const uint4*>(zp + 8);
        }
        f32x4 O[4];
        state_pass<(NW < 8)>(Sacc, U0, sm.NWop, Qop, sm.Mop, Krop, sm.alast, O);
        if constexpr (EPI) {
            __shared__ f32x4 epi_part[NW][C / 4];   // per wave: sum of o^2 over its 16 columns
            float s2[4][4];
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int i = 0; i < 4; ++i) s2[I][i] = row_sum16(O[I][i] * O[I][i]);
            if (r == 0)
#pragma unroll
                for (int I = 0; I < 4; ++I)
                    epi_part[wave][4 * I + g] = f32x4{s2[I][0], s2[I][1], s2[I][2], s2[I][3]};
            lds_barrier();
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                f32x4 tot = epi_part[0][4 * I + g];
#pragma unroll
                for (int w2 = 1; w2 < NW; ++w2) tot += epi_part[w2][4 * I + g];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    O[I][i] *= __builtin_amdgcn_rsqf(tot[i] * (1.f / 128) + ep.eps) * epi_w;
            }
            // fp32 staging (slots of 64 x OTSF floats: waves 0-2 in Kd, 3-5 in
            // Ki, 6-7 in RkT, all dead until the next chunk), so o is rounded
            // to bf16 once, after the gate
            float* stf = wave < 3 ? reinterpret_cast<float*>(sm.Kd) + wave * (C * OTSF)
                       : wave < 6 ? reinterpret_cast<float*>(sm.Ki) + (wave - 3) * (C * OTSF)
                                  : reinterpret_cast<float*>(sm.RkT) + (wave - 6) * (C * OTSF);
            store_o_gated(O, stf, zv, o, ((size_t)tok0 + (size_t)c * C) * H + h, (size_t)H,
                          16 * wave, ntok);
        } else {
            // staging slots: waves 0-5 in RkT, 6-7 in sV (both dead since stage 3;
            // other waves may still read Kd and Ki in their state pass)
            bf16* stage = (wave < 6) ? sm.RkT + wave * (C * OTS) : sV + (wave - 6) * (C * OTS);
            store_o(O, stage, o, ((size_t)tok0 + (size_t)c * C) * H + h, (size_t)H, col0 + 16 * wave, ntok);
        }
        if (CKPT && ntok >= C && (c + 1) % ck_every == 0) {
            const long slot = ck0 + (c + 1) / ck_every - 1;
            if (slot < ck_slots) store_state(S_ckpt + ((size_t)slot * H + h) * DK * 128, Sacc, g, ncol);
        }
    }

    const int ms = sq.mslot ? sq.mslot[b] : -1;
    if (ms >= 0) store_state(sq.mid + ((size_t)ms * H + h) * DK * 128, Sacc, g, ncol);
    else if (S_final) store_state(S_final + sbase, Sacc, g, ncol);
}

template <int NW, bool CKPT, int PRO, bool EPI = false>
__global__ __launch_bounds__(NW * 64, 1) void prefill_fused_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const void* __restrict__ gate, const float* __restrict__ beta,
    const float* S0, bf16* __restrict__ o, float* S_final, SeqLayout sq, int H, int NVB,
    float* __restrict__ S_ckpt, int ck_slots, Prologue pr, Epilogue ep)
{
    __shared__ mf::Prep sm;
    __shared__ __attribute__((aligned(16))) bf16 sV[mf::C * (NW * 16 + 8)];
    fused_body<NW, CKPT, PRO, EPI>(sm, sV, blockIdx.x, q, k, v, gate, beta, S0, o, S_final, sq, H,
                                   NVB, S_ckpt, ck_slots, pr, ep);
}

// Chunk numbering of the prep kernel, for fewer than 128 sequences: chunk gc
// of all chunks -> first token and length of its sequence, chunk within it.
struct ChunkPos {
    long tok0;
    int len, c;
};
template <bool kTable>
struct ChunkMap {
    SeqLayout sq;
    int nch;              // without a table: chunks per sequence
    int off[2], cst[2];   // with a table: offset and first chunk of entries lane, 64 + lane
    int ln[2];            // with explicit lengths (sq.lens): their lengths
    __device__ explicit ChunkMap(const SeqLayout& s) : sq(s), nch((s.T + mf::C - 1) / mf::C) {
        if (kTable) {
            const int lane = threadIdx.x & 63;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int j = min(lane + 64 * u, s.N);   // entries past N repeat entry N
                off[u] = s.tab[j];
                cst[u] = (lane + 64 * u <= s.N) ? s.tab[s.N + 1 + j] : 0x7fffffff;
                ln[u] = s.lens ? s.lens[min(j, s.N - 1)] : 0;
            }
        }
    }
    // entry j (wave-uniform) of a lane-distributed array
    __device__ int entry(const int (&x)[2], int j) const {
        return j < 64 ? __builtin_amdgcn_readlane(x[0], j) : __builtin_amdgcn_readlane(x[1], j - 64);
    }
    __device__ int total() const { return kTable ? entry(cst, sq.N) : sq.N * nch; }
    __device__ ChunkPos at(int gc) const {
        if (!kTable) {
            const int i = gc / nch;
            return {sq.start(i), sq.T, gc - i * nch};
        }
        // the sequence is the last entry whose first chunk is <= gc
        const int i = __builtin_popcountll(__builtin_amdgcn_ballot_w64(cst[0] <= gc)) +
                      __builtin_popcountll(__builtin_amdgcn_ballot_w64(cst[1] <= gc)) - 1;
        const int o0 = entry(off, i);
        const int len = sq.lens ? entry(ln, i) : entry(off, i + 1) - o0;
        return {(long)o0, len, gc - entry(cst, i)};
    }
    // position of chunk gc + 1 given that of chunk gc
    __device__ ChunkPos next(const ChunkPos& p, int gc) const {
        if (!kTable) {
            if (p.c + 1 < nch) return {p.tok0, p.len, p.c + 1};
            return {p.tok0 + sq.S, p.len, 0};
        }
        return at(gc + 1);
    }
};

// Prep kernel: chunks [gc0, gc0 + cpw) of the chunk numbering, head h;
// writes the operand record of chunk gc at record h * nch_all + gc. kTable:
// the sequences come from a device table (fewer than 128 of them). NT: the
// inputs are read non-temporally, so that streaming a long sequence through
// leaves the last-level cache to the records.
// The body runs chunks [gc0, gc0 + cpw) of head h (clamped to the
// numbering's end); the kernel that runs it passes the LDS blocks.
template <bool kTable, int PRO, bool NT>
__device__ __forceinline__ void prep_body(
    mf::Prep& sm, bf16* sV, int h, int gc0, int cpw,
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const void* __restrict__ gate, const float* __restrict__ beta,
    char* __restrict__ ws, const SeqLayout& sq, int H, int nch_all, const Prologue& pr)
{
    using namespace mf;
    constexpr int NW = 8, DVB = 128;

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const ChunkMap<kTable> map(sq);
    const int gc1 = min(gc0 + cpw, map.total());

    Inputs<NW> in;
    ChunkPos p{0, 1, 0};
    if (gc0 < gc1) {
        p = map.at(gc0);
        load_inputs<NW, DVB, PRO, NT>(in, q, k, v, gate, beta, p.tok0, p.len, h, H, p.c, 0);
    }
    for (int gc = gc0; gc < gc1; ++gc) {
        const int ntok = p.len - p.c * C;
        const bool more = gc + 1 < gc1;
        const ChunkPos pn = more ? map.next(p, gc) : p;
        lds_barrier();
        prologue<NW, PRO>(sm, in, pr);
        stage1a<NW, DVB>(sm, sV, in, ntok);
        lds_barrier();
        const bool fast = chunk_is_mild<NW>(sm);
        if (fast) {
            if (ntok >= C) stage1b<NW, true, PRO, true>(sm, in, ntok);
            else stage1b<NW, false, PRO, true>(sm, in, ntok);
        } else {
            if (ntok >= C) stage1b<NW, true, PRO, false>(sm, in, ntok);
            else stage1b<NW, false, PRO, false>(sm, in, ntok);
        }
        // next chunk's inputs: waves 0-3 now; waves 4-7 (lighter Gram work)
        // after stage 2, so their fetches queue while the inverses finish
        if (more && wave < 4) load_inputs<NW, DVB, PRO, NT>(in, q, k, v, gate, beta, pn.tok0, pn.len, h, H, pn.c, 0);
        lds_barrier();
        char* rec = ws + ((size_t)h * nch_all + gc) * REC_BYTES;
        const int g = lane >> 4, r = lane & 15;
        stage2<NW>(sm, fast);
        // Q_decay operands 4(w - 4) .. + 3 (block I = w - 4): on the chunk
        // reference they are final since stage 1, and waves 4-7 store them
        // here, in their slack while the inverses finish; otherwise (scaled
        // in stage 3) after the substitution's block 0
        auto store_qd = [&]() {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int j = 4 * (wave - 4) + kk;
                *reinterpret_cast<bf16x8*>(rec + REC_QD + j * OPB + lane * 16) =
                    ldA_perm(sm.Qd + (16 * (j >> 2) + r) * KS, 32 * kk, g);
            }
        };
        if (fast && wave >= 4) store_qd();
        // K_restore^T (final since stage 1 on either reference): waves 6, 7,
        // the two with a single Gram pair, store its 16 operands here
        if (wave >= 6) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int jj = 8 * (wave - 6) + e;   // m = jj / 2, kk = jj % 2
                *reinterpret_cast<bf16x8*>(rec + REC_KR + jj * OPB + lane * 16) =
                    ldA_perm(sm.KrT + (16 * (jj >> 1) + r) * TS, 32 * (jj & 1), g);
            }
        }
        if (more && wave >= 4) load_inputs<NW, DVB, PRO, NT>(in, q, k, v, gate, beta, pn.tok0, pn.len, h, H, pn.c, 0);
        lds_barrier();
        // Operand record stores (16 B per lane per A operand), each placed
        // where it overlaps other work:
        //   K_restore^T (16): waves 6-7, during stage 2 (above);
        //   Q_decay (16): waves 4-7, during stage 2 on the chunk reference
        //     (above), else after the substitution's block 0 (below);
        //   M_qk (6): waves 0-5, one each, after block 0 (below);
        //   -W (16): every wave, straight from the registers that form it in
        //     the substitution, its 8-byte half of the four operands of its
        //     channel tile;
        //   a_last and U0: from registers after the substitution.
        // Which stores a wave issues depends only on its index and the
        // chunk's decay reference, both wave-uniform.
        auto early = [&](int I) {
            // M_qk: one operand each for waves 0-5 after block 0
            if (I == 0 && wave < 6)
                *reinterpret_cast<bf16x8*>(rec + REC_M + wave * OPB + lane * 16) = sm.Mop[wave][lane];
            if (I == 0 && !fast && wave >= 4) store_qd();
        };
        f32x4 U0[4];
        stage3<NW, DVB, decltype(early), true>(sm, sV, 16 * wave, U0, fast, early, rec);
        p = pn;
        if (wave == 0)   // lanes 32-63 repeat lanes 0-31
            *reinterpret_cast<f32x4*>(rec + REC_AL + (lane & 31) * 16) =
                *reinterpret_cast<const f32x4*>(&sm.alast[4 * (lane & 31)]);
        // U0 tile (I, wave) in accumulator order: 4 bf16 per lane
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            uint2 u;
            u.x = pack2(U0[I][0], U0[I][1]);
            u.y = pack2(U0[I][2], U0[I][3]);
            *reinterpret_cast<uint2*>(rec + REC_U0 + ((I * 8 + wave) * 64 + lane) * 8) = u;
        }
    }
}

template <bool kTable, int PRO, bool NT>
__global__ __launch_bounds__(512, 1) void prefill_prep_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const void* __restrict__ gate, const float* __restrict__ beta,
    char* __restrict__ ws, SeqLayout sq, int H, int cpw, int nch_all, Prologue pr)
{
    __shared__ mf::Prep sm;
    __shared__ __attribute__((aligned(16))) bf16 sV[mf::C * (128 + 8)];
    const int ngrp = (nch_all + cpw - 1) / cpw;
    const int h = blockIdx.x / ngrp;
    const int gc0 = (blockIdx.x - h * ngrp) * cpw;
    prep_body<kTable, PRO, NT>(sm, sV, h, gc0, cpw, q, k, v, gate, beta, ws, sq, H, nch_all, pr);
}

// State kernel: one workgroup of twelve waves per (sequence*head, 16 value
// columns). Each wave has one role, so the chunk-to-chunk chain is two short
// MFMA passes and every wave loads only the few operands it uses:
//   waves 0-3  (U): U = U0 - W S for token tile w                 (-W: 4 KB)
//   waves 4-7  (S): S = Diag(a_last) S + K_restore^T U for state rows
//                   32s .. 32s + 31, s = w - 4           (K_restore^T: 4 KB)
//   waves 8-11 (O): O = Q_decay S + M_qk U for token tile w - 8
// S (bf16, B-operand order) and U pass between waves through LDS, two
// barriers per chunk: [S_c ready] U and Q_decay S; [U_c ready] S update and
// M_qk U. Operands arrive straight into registers from the operand record,
// which comes from HBM or the last-level cache: every wave keeps a ring of
// PF operand sets and fetches several chunks ahead. A wave issues its
// fetches in the phase where it is off the chain (one 1 KB load takes a wave
// tens of cycles to issue): the S waves and output tiles 0, 1 in phase 1,
// the U waves and output tiles 2, 3 in phase 2. The column tiles of a head
// run on one XCD (block ids sharing id % 8) and share its L2; when the
// workspace streams from HBM a thirteenth wave prefetches records into that
// L2 ahead of the role waves. The U and S waves run at raised priority so the
// output waves sharing their SIMDs do not delay the chain.
namespace mf {
constexpr int PF = 4;   // operand sets in flight per wave
}

// With CKPT the S waves also store the state after every sq.K tokens of the
// sequence to checkpoint slot sq.ckpt0(i) + j - 1 (slots >= ck_slots are dropped).
// NCT: 16-column tiles per workgroup (1 or 2). With 2, each workgroup covers
// 32 value columns and applies every operand it fetches to both tiles, so a
// head takes four workgroups instead of eight: half the workgroups for the
// same call, each fetching about the same bytes per chunk. That form runs
// without the L2-touch wave (twelve waves, up to 168 registers per lane: the
// two tiles' accumulators and operand sets do not fit in 128).
template <bool CKPT, int NCT>
__global__ __launch_bounds__(NCT == 1 ? 832 : 768, 1) void prefill_state_kernel(
    const char* __restrict__ ws, const float* S0, bf16* __restrict__ o, float* S_final,
    SeqLayout sq, int H, int BH, int nch_all, float* __restrict__ S_ckpt, int ck_slots)
{
    using namespace mf;
    static_assert(NCT == 1 || NCT == 2, "16 or 32 value columns per workgroup");
    constexpr int NT = 8 / NCT;            // workgroups per head
    // operand sets in flight per wave: one more with two tiles, which fetch
    // from HBM more often (fewer workgroups share each record through L2)
    constexpr int PF = NCT == 2 ? mf::PF + 1 : mf::PF;
    constexpr int CW = 16 * NCT;           // value columns per workgroup
    __shared__ bf16x8 sSB[NCT][4][64];     // S as four B operands (32-deep steps), per tile
    __shared__ bf16x4 sUB[NCT][2][64][2];  // U as two B operands, halves by token tile
    __shared__ __attribute__((aligned(16))) bf16 sO[4][16 * CW];   // output tiles, token-major

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int g = lane >> 4, r = lane & 15;
    const int grp = blockIdx.x / (8 * NT);
    const int bh = grp * 8 + (blockIdx.x & 7);
    const int ct = (blockIdx.x >> 3) % NT;         // value column tile of CW columns
    if (bh >= BH) return;                          // whole workgroup: uniform
    const int b = bh / H, h = bh - b * H;          // sequence b, head h
    if (sq.fin && sq.fin[b] < 0) return;           // unused entry of a split schedule
    auto ncol = [&](int u) { return CW * ct + 16 * u + r; };
    const long tok0 = sq.start(b);
    const int T = sq.len(b);
    const int nchunks = (T + C - 1) / C;
    const size_t sbase = (size_t)bh * DK * 128;
    // S_final row: the entry's own, or that of the sequence it continues
    const size_t fbase = sq.fin ? ((size_t)sq.fin[b] * H + h) * DK * 128 : sbase;
    // An empty sequence walks no chunk: its waves fetch record 0 of the
    // workspace (unused) and the S waves store S_final = S0.
    const size_t rbase = nchunks > 0 ? (size_t)h * nch_all + sq.chunk0(b) : 0;
    const int clast = max(nchunks - 1, 0);

    // record of chunk c, clamped: fetches past the end reload the last one
    auto rec = [&](int c) -> const char* {
        return ws + (rbase + min(c, clast)) * REC_BYTES;
    };
    auto op = [&](const char* rp, int off) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(rp + off + lane * 16);
    };
    // Runs step(set, prev, c, full) for every chunk with set = operand set
    // c % PF and prev = set (c - 1) % PF, unrolled so that each set is a
    // distinct register array. Whole groups of PF full chunks run unguarded
    // (so the compiler can count the loads in flight across the loop); the
    // remaining chunks follow, with `full` false for a chunk that may end
    // before 64 tokens.
    const int nfull = T / C;
    auto walk = [&](auto& sets, auto&& step) {
        int c = 0;
        for (; c + PF <= nfull; c += PF) {
#pragma unroll
            for (int k = 0; k < PF; ++k) step(sets[k], sets[(k + PF - 1) % PF], c + k, std::true_type{});
        }
#pragma unroll
        for (int k = 0; k < PF; ++k)
            if (c + k < nchunks) step(sets[k], sets[(k + PF - 1) % PF], c + k, std::false_type{});
    };

    if (wave < 4) {
        // ---- U = U0 - W S, token tile I (fetches in phase 2, PF ahead) ----
        __builtin_amdgcn_s_setprio(2);
        const int I = wave;
        struct Ops { bf16x8 w[4]; uint2 u0[NCT]; };
        auto load = [&](Ops& x, int c) {
            const char* rp = rec(c);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) x.w[kk] = op(rp, REC_NW + (I * 4 + kk) * OPB);
#pragma unroll
            for (int u = 0; u < NCT; ++u)
                x.u0[u] = *reinterpret_cast<const uint2*>(rp + REC_U0 + ((I * 8 + NCT * ct + u) * 64 + lane) * 8);
        };
        Ops sets[PF];
#pragma unroll
        for (int k = 0; k < PF; ++k) load(sets[k], k);
        walk(sets, [&](Ops& x, Ops&, int c, auto) {
            lds_barrier();                                   // S_c ready
#pragma unroll
            for (int u = 0; u < NCT; ++u) {
                const f32x2 lo = unpack2(x.u0[u].x), hi = unpack2(x.u0[u].y);
                f32x4 acc = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mma32(x.w[kk], sSB[u][kk][lane], acc);
                sUB[u][I >> 1][lane][I & 1] = __builtin_convertvector(acc, bf16x4);
            }
            lds_barrier();                                   // U_c ready
            load(x, c + PF);
        });
    } else if (wave < 8) {
        // ---- S = Diag(a_last) S + K_restore^T U, state rows 32s .. 32s + 31
        //      (fetches in phase 1, PF - 1 ahead) ----
        __builtin_amdgcn_s_setprio(2);
        const int s = wave - 4, m0 = 2 * s;
        f32x4 Sacc[NCT][2];
#pragma unroll
        for (int u = 0; u < NCT; ++u) {
            if (S0) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Sacc[u][m][i] = S0[sbase + (size_t)(16 * (m0 + m) + 4 * g + i) * 128 + ncol(u)];
            } else {
                Sacc[u][0] = zero4();
                Sacc[u][1] = zero4();
            }
        }
        const int ck_every = CKPT ? sq.K / C : 1;   // chunks per checkpoint
        int ck_left = ck_every;                      // chunks until the next one
        int ck_slot = CKPT ? (int)sq.ckpt0(b) : 0;   // its slot
        // a_last of rows 32s .. 32s + 31: one dword per lane (lanes 32-63
        // repeat 0-31), spread to the accumulator layout by lane shuffles,
        // instead of 16-byte loads that return the same bytes to 16 lanes
        struct Ops { bf16x8 k[4]; float al; };
        auto load = [&](Ops& x, int c) {
            const char* rp = rec(c);
#pragma unroll
            for (int j = 0; j < 4; ++j) x.k[j] = op(rp, REC_KR + (2 * m0 + j) * OPB);
            x.al = *reinterpret_cast<const float*>(rp + REC_AL + (32 * s + (lane & 31)) * 4);
        };
        Ops sets[PF];
#pragma unroll
        for (int k = 0; k < PF - 1; ++k) load(sets[k], k);
#pragma unroll
        for (int u = 0; u < NCT; ++u) sSB[u][s][lane] = pack8(Sacc[u][0], Sacc[u][1]);
        walk(sets, [&](Ops& x, Ops& px, int c, auto) {
            lds_barrier();                                   // S_c ready
            load(px, c + PF - 1);
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float a = __shfl(x.al, 16 * m + 4 * g + i);
#pragma unroll
                    for (int u = 0; u < NCT; ++u) Sacc[u][m][i] *= a;
                }
            lds_barrier();                                   // U_c ready
#pragma unroll
            for (int u = 0; u < NCT; ++u) {
                const bf16x8 UB0 = *reinterpret_cast<const bf16x8*>(&sUB[u][0][lane][0]);
                const bf16x8 UB1 = *reinterpret_cast<const bf16x8*>(&sUB[u][1][lane][0]);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    Sacc[u][m] = mma32(x.k[2 * m], UB0, Sacc[u][m]);
                    Sacc[u][m] = mma32(x.k[2 * m + 1], UB1, Sacc[u][m]);
                }
                sSB[u][s][lane] = pack8(Sacc[u][0], Sacc[u][1]);
            }
            if (CKPT && --ck_left == 0) {                   // checkpoint after chunk c
                ck_left = ck_every;
                if ((c + 1) * C <= T && ck_slot < ck_slots) {
#pragma unroll
                    for (int u = 0; u < NCT; ++u) {
                        float* dst = S_ckpt + ((size_t)ck_slot * H + h) * DK * 128 +
                                     (16 * m0 + 4 * g) * 128 + ncol(u);
#pragma unroll
                        for (int m = 0; m < 2; ++m)
#pragma unroll
                            for (int i = 0; i < 4; ++i) dst[(16 * m + i) * 128] = Sacc[u][m][i];
                    }
                }
                ++ck_slot;
            }
        });
        if (S_final) {
#pragma unroll
            for (int u = 0; u < NCT; ++u)
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S_final[fbase + (size_t)(16 * (m0 + m) + 4 * g + i) * 128 + ncol(u)] = Sacc[u][m][i];
        }
    } else if (wave == 12) {
        // ---- L2 prefetch (launched only for workspaces that stream from HBM):
        //      this workgroup's share of the record eight chunks ahead, one
        //      dword per 128-byte line, so that the role waves of the head's
        //      column tiles (one XCD, one L2) hit L2 ----
        constexpr int kAhead = PF + 2;
        constexpr int kSlice = REC_BYTES / NT;
        constexpr int kTouch = 2 * NCT;             // lines per lane (64 x 128 B each)
        uint32_t ring[3][kTouch] = {};
        uint32_t acc = 0;
        auto touch = [&](uint32_t (&dst)[kTouch], int c) {
            const char* rp = rec(c);
#pragma unroll
            for (int u = 0; u < kTouch; ++u) {
                const int off = min(ct * kSlice + (u * 64 + lane) * 128, REC_BYTES - 4);
                dst[u] = *reinterpret_cast<const uint32_t*>(rp + off);
            }
        };
        touch(ring[0], kAhead);
        touch(ring[1], kAhead + 1);
        for (int c = 0; c < nchunks; c += 3) {
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                if (c + k < nchunks) {
                    lds_barrier();                           // S_c ready
#pragma unroll
                    for (int u = 0; u < kTouch; ++u) acc ^= ring[(k + 2) % 3][u];   // oldest set: long arrived
                    touch(ring[(k + 2) % 3], c + k + kAhead + 2);
                    lds_barrier();                           // U_c ready
                }
            }
        }
        // keep the fetches alive; never true for a real call
        if (acc == 0x9e3779b9u && T < 0) o[lane] = (bf16)(float)acc;
    } else {
        // ---- O = Q_decay S + M_qk U, token tile I ----
        const int I = wave - 8;
        // M_qk operands of row tile I: against U rows 0-31 (record entry I)
        // and, for I >= 2, against U rows 32-63 (entry I + 2)
        struct Ops { bf16x8 q[4]; bf16x8 m0, m1; };
        auto load = [&](Ops& x, int c) {
            const char* rp = rec(c);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) x.q[kk] = op(rp, REC_QD + (I * 4 + kk) * OPB);
            x.m0 = op(rp, REC_M + I * OPB);
            if (I >= 2) x.m1 = op(rp, REC_M + (I + 2) * OPB);
        };
        // the tile leaves through LDS so that each lane stores 4 * NCT
        // columns of one token (8 * NCT bytes) instead of 4 tokens of one column
        bf16* tile = sO[I];
        constexpr int LC = 4 * NCT;                  // columns per lane in the store
        const int tt = lane >> 2, tc = LC * (lane & 3);
        // separate loops for the two fetch phases, so that each has one
        // load pattern the compiler can count across iterations
        auto run = [&](auto early) {
            constexpr bool kEarly = decltype(early)::value;   // fetch in phase 1
            Ops sets[PF];
#pragma unroll
            for (int k = 0; k < PF - 1; ++k) load(sets[k], k);
            walk(sets, [&](Ops& x, Ops& px, int c, auto full) {
                // fetches go first in their phase, into the set the previous
                // chunk freed, so they drain while this wave computes
                lds_barrier();                               // S_c ready
                if (kEarly) load(px, c + PF - 1);
                f32x4 Oa[NCT], Ob[NCT];
#pragma unroll
                for (int u = 0; u < NCT; ++u) {
                    Oa[u] = mma32(x.q[0], sSB[u][0][lane], zero4());
                    Ob[u] = mma32(x.q[1], sSB[u][1][lane], zero4());
                    Oa[u] = mma32(x.q[2], sSB[u][2][lane], Oa[u]);
                    Ob[u] = mma32(x.q[3], sSB[u][3][lane], Ob[u]);
                }
                lds_barrier();                               // U_c ready
                if (!kEarly) load(px, c + PF - 1);
#pragma unroll
                for (int u = 0; u < NCT; ++u) {
                    f32x4 O = mma32(x.m0, *reinterpret_cast<const bf16x8*>(&sUB[u][0][lane][0]), Oa[u]);
                    if (I >= 2) Ob[u] = mma32(x.m1, *reinterpret_cast<const bf16x8*>(&sUB[u][1][lane][0]), Ob[u]);
                    O += Ob[u];
#pragma unroll
                    for (int e = 0; e < 4; ++e) tile[(4 * g + e) * CW + 16 * u + r] = (bf16)O[e];
                }
                lds_fence_wave();
                // In a ragged last chunk, rows past the sequence end repeat the
                // tile's last real row (same data, same address); a tile wholly
                // past the end stores nothing. Full chunks store unconditionally.
                const int nt = T - c * C;
                if (decltype(full)::value || 16 * I < nt) {
                    const int t = decltype(full)::value ? 16 * I + tt : min(16 * I + tt, nt - 1);
                    bf16* dst = o + (((size_t)tok0 + (size_t)c * C + t) * H + h) * 128 + CW * ct + tc;
                    const bf16* src = &tile[(t - 16 * I) * CW + tc];
                    if constexpr (NCT == 1) {
                        const uint2 v = *reinterpret_cast<const uint2*>(src);
                        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                        __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(dst));
                    } else {
                        const uint4 v = *reinterpret_cast<const uint4*>(src);
                        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
                        __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
                    }
                }
            });
        };
        if (I < 2) run(std::true_type{});
        else run(std::false_type{});
    }
}

// Split schedule of a packed call, first launch: workgroups [0, nfused) run
// the fused kernel on every sequence (sq1: longest first, split sequences on
// their first segment, whose end state goes to sq1.mid); the other G per
// head prepare the records of the second segments (table sq2), each a
// consecutive share of that head's second-segment chunks. Both halves hold
// the same LDS blocks, so the grid mixes them freely. The prep shares are
// issued from the numbering's end back to its start, so the records of the
// first entries (the walk's first and longest chains) are written last and
// are the likeliest still in the last-level cache when the walk reads them;
// the prep reads its inputs non-temporally to leave that cache to them.
template <bool CKPT>
__global__ __launch_bounds__(512, 1) void prefill_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ la, const float* __restrict__ beta, const float* S0,
    bf16* __restrict__ o, float* S_final, SeqLayout sq1, SeqLayout sq2, int H, int nfused,
    int G, char* __restrict__ ws, int nrec, float* __restrict__ S_ckpt, int ck_slots)
{
    __shared__ mf::Prep sm;
    __shared__ __attribute__((aligned(16))) bf16 sV[mf::C * (128 + 8)];
    const int blk = blockIdx.x;
    if (blk < nfused) {
        fused_body<8, CKPT, 0>(sm, sV, blk, q, k, v, la, beta, S0, o, S_final, sq1, H, 1, S_ckpt,
                               ck_slots, Prologue{}, Epilogue{});
        return;
    }
    const int p = blk - nfused, grp = G - 1 - p / H, h = p % H;
    const int total2 = sq2.tab[2 * sq2.N + 1];
    const int cpw = (total2 + G - 1) / G;
    if (grp * cpw >= total2) return;                 // whole workgroup: uniform
    prep_body<true, 0, true>(sm, sV, h, grp * cpw, cpw, q, k, v, la, beta, ws, sq2, H, nrec,
                              Prologue{});
}

// ---------------------------------------------------------------------------
namespace {
constexpr size_t DK_STATE_BYTES = size_t(128) * 128 * 4;   // one fp32 state
}

namespace {
constexpr long kSplitBelowHeads = 128;   // fewer heads than this: prep + state kernels
// Piecewise split path: fixed-length batches whose records would outgrow the
// last-level cache run prep and state walk piece by piece along the
// sequence, about kPieceWork chunk-heads at a time: 3072 records are 221.8 MB,
// which the walk reads back from the 256 MB last-level cache (the prep reads
// its inputs non-temporally to leave it to them).
constexpr size_t kPieceAbove = size_t(192) << 20;
constexpr long kPieceWork = 3072;
}

bool prefill_mfma_supported(int dk, int dv, int chunk, long H) {
    // H: the chunk loads address one chunk of all heads with 32-bit offsets
    return dk == 128 && dv == 128 && (chunk == 64 || chunk == 0) && H <= kMfmaMaxHeads;
}

bool prefill_mfma_split(long pairs) { return pairs < kSplitBelowHeads; }

size_t prefill_mfma_workspace(long pairs, size_t nch_all, int H) {
    if (!prefill_mfma_split(pairs)) return 0;
    return (size_t)H * nch_all * mf::REC_BYTES;
}

long prefill_mfma_piece(long pairs, long nch_seq, size_t max_ws) {
    if (!prefill_mfma_split(pairs)) return 0;
    const size_t rec = (size_t)pairs * mf::REC_BYTES;        // one chunk of every sequence
    const size_t state = (size_t)pairs * DK_STATE_BYTES;
    long L = (size_t)nch_seq * rec > kPieceAbove ? std::max(1L, kPieceWork / pairs) : nch_seq;
    // the workspace holds the whole call's records, or one piece of them and
    // the carried state: pieces shrink until that fits max_ws
    const size_t need = L >= nch_seq ? (size_t)nch_seq * rec : (size_t)L * rec + state;
    if (need > max_ws) {
        const size_t room = max_ws > state ? max_ws - state : 0;
        L = std::min(L, (long)std::min(room / rec, (size_t)nch_seq));
        if (L < 1) return -1;
    }
    return L < nch_seq ? L : 0;
}

size_t prefill_mfma_workspace_fixed(int B, int H, long nch_seq, size_t max_ws) {
    const long pairs = (long)B * H;
    const long L = prefill_mfma_piece(pairs, nch_seq, max_ws);
    if (L < 0) return SIZE_MAX;
    if (L == 0) return prefill_mfma_workspace(pairs, (size_t)B * (size_t)nch_seq, H);
    // one piece of records, then the carried state (used when the caller
    // wants no S_final)
    return (size_t)pairs * (size_t)L * mf::REC_BYTES + (size_t)pairs * DK_STATE_BYTES;
}

namespace {

// Kernel instances by prologue: the plain op (with or without checkpoints)
// and the six layer forms (gate mode x L2), without checkpoints.
template <int NW, int PRO>
auto fused_kernel_for(bool ck, bool epi) {
    if constexpr (NW == 8) {
        if (epi) return prefill_fused_kernel<8, false, PRO, true>;
    }
    if constexpr (PRO == 0)
        return ck ? prefill_fused_kernel<NW, true, 0> : prefill_fused_kernel<NW, false, 0>;
    else
        return prefill_fused_kernel<NW, false, PRO>;
}

// Column tiles per state-walk workgroup: 16-column tiles put 8 workgroups
// on a sequence-head; when the walk's sequence-heads need more than one
// round of workgroups on the 256 compute units that way, 32-column tiles
// (4 per sequence-head) halve the rounds, at a higher time per chunk.
int state_tiles(long pairs) { return pairs * 8 > 256 ? 2 : 1; }

// State walk of `pairs` sequence-heads: groups of 8 sequence-heads, each on
// 8 / nct workgroups of 16 * nct value columns; the workgroups of one
// sequence-head have block ids equal mod 8 (one XCD, one L2).
hipError_t launch_state(bool ck, int nct, unsigned threads, const char* ws, const float* S0,
                        bf16* o, float* S_final, const SeqLayout& sq, int H, long pairs,
                        int nch_all, float* S_ckpt, int ck_slots, hipStream_t st)
{
    const long groups = (pairs + 7) / 8;
    const dim3 grid((unsigned)(groups * 64 / nct)), block(nct == 2 ? 768u : threads);
    auto kern = nct == 2 ? (ck ? prefill_state_kernel<true, 2> : prefill_state_kernel<false, 2>)
                         : (ck ? prefill_state_kernel<true, 1> : prefill_state_kernel<false, 1>);
    hipLaunchKernelGGL(kern, grid, block, 0, st, ws, S0, o, S_final, sq, H, (int)pairs, nch_all,
                       S_ckpt, ck_slots);
    return hipGetLastError();
}

// Piecewise split path (fixed-length batch, sq.tab == nullptr): for each
// piece of L chunks of every sequence, the prep kernel writes its records
// (one piece of the workspace, reused) and the state kernel walks them,
// reading the state the previous piece left in `carry` (S_final, or the
// state buffer after the records when the caller wants none). Records are
// read back while they are still in the last-level cache.
template <int PRO>
hipError_t launch_mfma_pieces(const void* q, const void* k, const void* v, const void* gate,
                              const float* beta, const float* S0, void* o, float* S_final,
                              const SeqLayout& sq, int H, int nch_all, void* ws, long L,
                              const Prologue& pr, hipStream_t st)
{
    constexpr int GM = PRO & 3;
    const int B = sq.N;
    const long pairs = (long)B * H;
    const long nch_seq = nch_all / B;
    char* rec = (char*)ws;
    float* carry = S_final ? S_final : (float*)(rec + (size_t)pairs * L * mf::REC_BYTES);
    // the records were just written and sit in the last-level cache: no
    // L2-touch wave (it measured slower here)
    const unsigned threads = 768u;
    const int nct = state_tiles(pairs);
    for (long c0 = 0; c0 < nch_seq; c0 += L) {
        const long Lc = std::min(L, nch_seq - c0);
        const long t0 = c0 * mf::C;
        const int Tp = (int)std::min(Lc * mf::C, (long)sq.T - t0);
        const SeqLayout sp{nullptr, B, Tp, mf::C, 0, sq.S};
        const size_t row = (size_t)t0 * H;        // first (token, head) row of the piece
        const bf16* qp = (const bf16*)q + row * mf::DK;
        const bf16* kp = (const bf16*)k + row * mf::DK;
        const bf16* vp = (const bf16*)v + row * 128;
        const float* bp = beta + row;
        const void* gp = GM == kGateLog ? (const void*)((const float*)gate + row * mf::DK)
                       : GM == kGateBounded ? (const void*)((const bf16*)gate + row * mf::DK)
                       : (const void*)((const float*)gate + row);
        bf16* op = (bf16*)o + row * 128;
        const int nch_piece = (int)(B * Lc);
        const long work = (long)H * nch_piece;
        int cpw = (int)((work + 255) / 256);
        if (cpw < 1) cpw = 1;
        const long ngrp = (nch_piece + cpw - 1) / cpw;
        hipLaunchKernelGGL((prefill_prep_kernel<false, PRO, true>), dim3((unsigned)(H * ngrp)), dim3(512),
                           0, st, qp, kp, vp, gp, bp, rec, sp, H, cpw, nch_piece, pr);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        e = launch_state(false, nct, threads, (const char*)rec, c0 == 0 ? S0 : (const float*)carry,
                         op, carry, sp, H, pairs, nch_piece, nullptr, 0, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int PRO>
hipError_t launch_mfma_pro(const void* q, const void* k, const void* v, const void* gate,
                           const float* beta, const float* S0, void* o, float* S_final,
                           const SeqLayout& sq, int H, int nch_all, void* ws, float* S_ckpt,
                           int ck_slots, const Prologue& pr, const Epilogue& ep,
                           bool* epi_done, size_t max_ws, hipStream_t st)
{
    const long pairs = (long)sq.N * H;
    const bool ck = S_ckpt != nullptr && sq.K > 0 && ck_slots > 0;
    *epi_done = false;
    if (!prefill_mfma_split(pairs)) {
        const bool wide = pairs >= 256;   // one 8-wave workgroup per pair, else two of 4 waves
        const dim3 grid((unsigned)(wide ? pairs : pairs * 2)), block(wide ? 512 : 256);
        const int nvb = wide ? 1 : 2;
        const bool epi = wide && ep.z != nullptr;
        auto kern = wide ? fused_kernel_for<8, PRO>(ck, epi) : fused_kernel_for<4, PRO>(ck, false);
        hipLaunchKernelGGL(kern, grid, block, 0, st, (const bf16*)q, (const bf16*)k,
                           (const bf16*)v, gate, beta, S0, (bf16*)o, S_final, sq, H, nvb,
                           S_ckpt, ck_slots, pr, ep);
        *epi_done = epi;
        return hipGetLastError();
    }
    // few sequence-heads, long sequences: prep and state walk piece by piece
    const long L = sq.tab ? 0 : prefill_mfma_piece(pairs, (long)nch_all / sq.N, max_ws);
    if (L < 0) return hipErrorInvalidValue;
    if (L > 0) return launch_mfma_pieces<PRO>(q, k, v, gate, beta, S0, o, S_final, sq, H,
                                              nch_all, ws, L, pr, st);
    // few sequence-heads: chunk-parallel prep, then the state walk
    if (nch_all > 0) {
        const long work = (long)H * nch_all;
        int cpw = (int)((work + 255) / 256);          // about one workgroup per CU
        if (cpw < 1) cpw = 1;
        const long ngrp = (nch_all + cpw - 1) / cpw;
        // (the layer forms take fixed-length batches only: no table variant)
        // (cached input loads: with the records of the whole call under the
        // piecewise threshold they measure faster here than non-temporal ones)
        auto prep = prefill_prep_kernel<false, PRO, false>;
        if constexpr (PRO == 0)
            if (sq.tab) prep = prefill_prep_kernel<true, 0, false>;
        hipLaunchKernelGGL(prep, dim3((unsigned)(H * ngrp)), dim3(512), 0, st, (const bf16*)q,
                           (const bf16*)k, (const bf16*)v, gate, beta, (char*)ws, sq, H, cpw,
                           nch_all, pr);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // A workspace that outgrows the last-level cache (256 MB) streams from
    // HBM: add the L2 prefetch wave (thirteenth wave) for it.
    const size_t ws_bytes = prefill_mfma_workspace(pairs, (size_t)nch_all, H);
    const unsigned threads = ws_bytes > (size_t(128) << 20) ? 832u : 768u;
    return launch_state(ck, state_tiles(pairs), threads, (const char*)ws, S0, (bf16*)o, S_final,
                        sq, H, pairs, nch_all, S_ckpt, ck_slots, st);
}

}  // namespace

SplitPlan prefill_split_plan(int N, int T_total, int H, size_t base) {
    SplitPlan p;
    // the fused part runs one 8-wave workgroup per (sequence, head); the
    // split table is built by one workgroup of 1024 threads
    if ((long)N * H < 256 || N > 1024 || T_total <= 0) return p;
    // a split sequence has more than total * H / 256 chunks, so fewer than
    // 256 / H of them exist (none at 256 heads or more); the prep's chunk
    // map holds up to 127 entries
    p.n2 = std::min(std::min(N, 127), (256 + H - 1) / H - 1);
    if (p.n2 <= 0) {
        p.n2 = 0;
        return p;
    }
    const long nb = ((long)T_total + (long)N * (mf::C - 1)) / mf::C;   // chunks, at most
    // records of at most 16384 chunk-heads (1.18 GB)
    p.cap2 = (int)std::min(nb, std::max(64L, 16384L / H));
    p.G = std::max(1, 512 / H);
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    p.sp = al(base);
    p.mid = al(p.sp + (3 * (size_t)N + 5 * (size_t)p.n2 + 3) * sizeof(int));
    p.rec = al(p.mid + (size_t)p.n2 * H * DK_STATE_BYTES);
    p.end = p.rec + (size_t)H * p.cap2 * mf::REC_BYTES;
    return p;
}

hipError_t launch_prefill_split(const void* q, const void* k, const void* v, const float* la,
                                const float* beta, const float* S0, void* o, float* S_final,
                                const int* tab, int N, int T_total, int K, int H,
                                const SplitPlan& plan, char* ws, float* S_ckpt, int ck_slots,
                                hipStream_t st)
{
    const int n2 = plan.n2;
    int* sp = reinterpret_cast<int*>(ws + plan.sp);
    hipError_t e = launch_varlen_split(tab, N, T_total, mf::C, K, H, n2, plan.cap2, sp, st);
    if (e != hipSuccess) return e;
    float* mid = reinterpret_cast<float*>(ws + plan.mid);
    char* rec = ws + plan.rec;
    SeqLayout sq1{tab, N, T_total, mf::C, K, T_total};
    sq1.lens = sp + N;
    sq1.ord = sp;
    sq1.mslot = sp + 2 * N;
    sq1.mid = mid;
    const int* tab2 = sp + 3 * N;
    SeqLayout sq2{tab2, n2, T_total, mf::C, K, T_total};
    sq2.lens = tab2 + 3 * n2 + 3;
    sq2.fin = sq2.lens + n2;
    const bool ck = S_ckpt != nullptr && K > 0 && ck_slots > 0;
    const int nfused = N * H;
    const long grid = (long)nfused + (long)H * plan.G;
    hipLaunchKernelGGL(ck ? prefill_split_kernel<true> : prefill_split_kernel<false>,
                       dim3((unsigned)grid), dim3(512), 0, st, (const bf16*)q, (const bf16*)k,
                       (const bf16*)v, la, beta, S0, (bf16*)o, S_final, sq1, sq2, H, nfused,
                       plan.G, rec, plan.cap2, S_ckpt, ck_slots);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long BH2 = (long)n2 * H;
    // records that may outgrow half the last-level cache: L2-touch wave
    const size_t rec_bytes = (size_t)H * plan.cap2 * mf::REC_BYTES;
    const unsigned threads = rec_bytes > (size_t(128) << 20) ? 832u : 768u;
    // column tiles as for two split sequences (how many entries the device
    // takes is not known here; entries are ordered longest first)
    const int nct = state_tiles((long)std::min(n2, 2) * H);
    return launch_state(ck, nct, threads, (const char*)rec, (const float*)mid, (bf16*)o, S_final,
                        sq2, H, BH2, plan.cap2, S_ckpt, ck_slots, st);
}

hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, const void* gate,
                               const float* beta, const float* S0, void* o, float* S_final,
                               const SeqLayout& sq, int H, int nch_all, void* ws,
                               float* S_ckpt, int ck_slots, int pro, const Prologue& pr,
                               const Epilogue& ep, bool* epi_done, hipStream_t st,
                               size_t max_ws)
{
#define KDA_PRO_CASE(P)                                                                     \
    case P:                                                                                 \
        return launch_mfma_pro<P>(q, k, v, gate, beta, S0, o, S_final, sq, H, nch_all, ws,  \
                                  S_ckpt, ck_slots, pr, ep, epi_done, max_ws, st);
    switch (pro) {
        KDA_PRO_CASE(0)
        KDA_PRO_CASE(kGateBounded)
        KDA_PRO_CASE(kGateScalar)
        KDA_PRO_CASE(kProL2)
        KDA_PRO_CASE(kProL2 | kGateBounded)
        KDA_PRO_CASE(kProL2 | kGateScalar)
    }
#undef KDA_PRO_CASE
    return hipErrorInvalidValue;
}

}  // namespace kda
