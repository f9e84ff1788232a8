// Multi-token decode on the matrix cores: a draft of 2..8 tokens verified
// (and an accepted prefix committed) from a live fp32 state, bf16 q/k/v,
// dk = dv = 128.
//
// The T tokens form one small chunk of the chunk algebra ("Kimi K3: the
// manos...", section "FlashKDA Algorithm"), with a_t the inclusive cumulative
// decay from the draft start:
//   W = [K_decay; Q_decay] S                (one 16-row MFMA tile: T <= 8 rows each)
//   (I + L) U = Diag(beta)(V - K_decay S),  L_ts = beta_t sum_d k_t[d] (a_t/a_s)[d] k_s[d], s < t
//   O = Q_decay S + M U,                    M_ts = sum_d q_t[d] (a_t/a_s)[d] k_s[d],       s <= t
//   S_n = Diag(a_{n-1}) S + sum_{t<n} Diag(a_{n-1}/a_t) k_t u_t^T   (the accepted prefix n)
// One workgroup per head, four waves, wave w owning value columns 32w..32w+31.
// The state slice is loaded once, at the start, in MFMA accumulator layout
// (lane (g, r) of a 16x16 tile: rows 4g..4g+3, column r), and used directly
// as the B operand of the W product with the K index of each 32-deep step
// permuted the same way on both operands. A committing pass then
// adds K_restore^T U to each 16-row tile in fp32 on the matrix cores and
// writes it back once; a verify pass (n = 0) only reads the state.
// Each log-decay is clamped into [-10, 0], so 1/a_t <= e^80 stays inside
// fp32 for any input. That holds the supported range (-5, 0) of the
// trillion-scale architecture page, section 4, exactly; a step that decays
// harder than exp(-10) keeps exp(-10) of the old state instead of less.
#include <type_traits>

#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int D = 128;
constexpr int TM = 8;             // most draft tokens
constexpr float kLogDecayFloor = -10.f;   // TM * 10 = 80 < 88 (fp32 exp range)
constexpr int AS = D + 8;         // bf16 row stride of [16][D] operand tiles
constexpr int RS = 16 + 8;        // bf16 row stride of K_restore^T [D][16 token slots]
constexpr int RT = 32 + 4;        // fp32 row stride of a wave's [16][32] commit staging block
constexpr int kStageFloats = 4 * 16 * RT;   // four waves

// Buffer resource word 3 for raw 32-bit accesses on CDNA, and the cache
// policy bit of a streaming (non-temporal) access. The b32 buffer builtins
// move raw bits (uint32): floats go through bit casts.
constexpr int kBufWord3 = 0x00020000;
constexpr int kNT = 2;

// 4x4 transpose across the four lanes of a quad: lane p holds x = M[p][0..3]
// and receives M[0..3][p]. Two butterfly steps, each taking the partner
// lane's element through a DPP quad permute (partners p ^ 1, then p ^ 2) for
// the positions whose index bit differs from the lane's.
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x) {
    const int p = threadIdx.x & 3;
    float a[4], b[4], v[4] = {x[0], x[1], x[2], x[3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float t = dpp_f<0xB1>(v[e ^ 1]);   // quad_perm [1,0,3,2]
        a[e] = ((e ^ p) & 1) ? t : v[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float t = dpp_f<0x4E>(a[e ^ 2]);   // quad_perm [2,3,0,1]
        b[e] = ((e ^ p) & 2) ? t : a[e];
    }
    return f32x4{b[0], b[1], b[2], b[3]};
}

// Swap of 16-lane rows between two registers (v_permlane16_swap): a keeps
// its rows 0 and 2 and takes b's rows 0 and 2 as its rows 1 and 3; b keeps
// its rows 1 and 3 and takes a's rows 1 and 3 as its rows 0 and 2. It is its
// own inverse.
__device__ __forceinline__ void row_swap(f32x4& a, f32x4& b) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 ua = __builtin_bit_cast(u32x4, a), ub = __builtin_bit_cast(u32x4, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const auto sw = __builtin_amdgcn_permlane16_swap(ua[e], ub[e], false, false);
        ua[e] = sw[0];
        ub[e] = sw[1];
    }
    a = __builtin_bit_cast(f32x4, ua);
    b = __builtin_bit_cast(f32x4, ub);
}

// Two 8-row loads (lane rows: 16-column tile 0 and 1 of rows +0..3, then the
// same of rows +4..7) -> the two accumulator tiles of those 16 rows.
__device__ __forceinline__ void tiles_from_rows(f32x4& a, f32x4& b) {
    a = quad_transpose(a);
    b = quad_transpose(b);
    row_swap(a, b);
}

__device__ __forceinline__ bf16x8 ldA_perm8(const bf16* rowp, int k0, int g) {
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(rowp + k0 + 4 * g);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(rowp + k0 + 16 + 4 * g);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// (four workgroups per CU: 123 registers, the accumulators in VGPRs; it took
// the verify pass from 111 to 101 us at B256 H32)
__global__ __launch_bounds__(256, 4) void decode_multi_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    float* __restrict__ S, bf16* __restrict__ o, const int* __restrict__ n_commit,
    int H, int T)
{
    // (16-byte aligned: operand rows are read as 8- and 16-byte vectors)
#define KDA_LDS __shared__ __attribute__((aligned(16)))
    KDA_LDS bf16 sA[16 * AS];      // rows 0..7: K_decay_t, rows 8..15: Q_decay_t (zero past T)
    KDA_LDS bf16 sKrT[D * RS];     // K_restore^T [channel][token slot], zero for slots >= n
    KDA_LDS bf16 sU[16 * AS];      // U (bf16) [token slot][column], zero for slots >= T
    KDA_LDS float sKd[TM * D];
    KDA_LDS float sQd[TM * D];
    KDA_LDS float sKi[TM * D];
    // [K_decay; Q_decay] S; once U and O are formed, the committing pass's
    // per-wave [16][RT] row-major staging of the updated tiles
    KDA_LDS float sW[kStageFloats > 16 * D ? kStageFloats : 16 * D];
    KDA_LDS float sL[TM * TM];
    KDA_LDS float sM[TM * TM];
    KDA_LDS float sDal[D];
    KDA_LDS float sBeta[TM];
#undef KDA_LDS

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int g = lane >> 4, r = lane & 15;
    const int head = blockIdx.x;
    const int bb = head / H, hh = head - bb * H;
    int n = n_commit ? n_commit[bb] : T;
    n = __builtin_amdgcn_readfirstlane(min(max(n, 0), T));

    // ---- state slice: this wave's 32 columns c0 .. c0 + 31 of all 128 rows.
    // It moves in whole 128-byte row pieces: load j brings rows 8j .. 8j + 7,
    // lane (hh = l / 32, cq = (l / 4) % 8, p = l % 4) holding row 8j + 4hh + p,
    // columns c0 + 4cq .. + 3. A transpose within each quad of lanes then
    // gives every lane four rows of one column, and a row swap between the
    // loads 2m and 2m + 1 (v_permlane16_swap) gathers each 16-column tile, so
    // that st[m][ct] is an MFMA accumulator tile: lane (g, r) holds column
    // c0 + 16ct + r of rows 16m + 4 sig(g) + i, sig(g) = (0, 2, 1, 3)[g]
    // (the A operands below index their rows with the same permutation). The
    // committed tiles return to the row pieces through LDS for the store.
    // Buffer accesses: a per-head resource, one per-lane byte offset and a
    // uniform offset per 8-row load.
    float* Sh = S + (size_t)head * D * D;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(Sh, 0, D * D * 4, kBufWord3);
    const int c0 = 32 * wave;
    const int off = ((4 * (lane >> 5) + (lane & 3)) * D + c0 + 4 * ((lane >> 2) & 7)) * 4;
    const int sig = ((g & 1) << 1) | (g >> 1);   // row quarter held by lane group g
    // ---- token side: one thread per channel d; threads 0-127 the key side
    //      (k, and the value column d), 128-255 the query side. All token
    //      loads are issued first.
    const int d = tid & (D - 1);
    const bool kside = tid < D;
    auto row = [&](int t) -> size_t { return ((size_t)bb * T + t) * H + hh; };
    const bf16* kq = kside ? k : q;
    // (raw bf16 bits, converted only after every load is issued; both sides
    // load the value column, used by the key side only)
    float la_t[TM];
    uint16_t x_raw[TM], v_raw[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const size_t e = row(min(t, T - 1)) * D + d;   // past T: re-read the last token, masked below
        la_t[t] = log_alpha[e];
        x_raw[t] = reinterpret_cast<const uint16_t*>(kq)[e];
        v_raw[t] = reinterpret_cast<const uint16_t*>(v)[e];
    }
    const float beta_d = d < TM ? beta[row(min(d, T - 1))] : 0.f;
    // The whole state slice is fetched next (64 registers per lane), after
    // the token loads and before any of them is used, so that the fetch
    // overlaps the token-side work; the W pass and the commit then use it
    // from registers. Streaming (nt) accesses: each element is read once and
    // written at most once.
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    f32x4 st[8][2];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int h = 0; h < 2; ++h)   // loads 2m + h, gathered into tiles below
            st[m][h] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(srs, off, (2 * m + h) * 8 * D * 4, kNT));
    float x_t[TM], vcol[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        x_t[t] = __builtin_bit_cast(float, (uint32_t)x_raw[t] << 16);
        vcol[t] = kside ? __builtin_bit_cast(float, (uint32_t)v_raw[t] << 16) : 0.f;
    }
    {
        float c = 0.f, cn = 0.f;
        float cum[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            if (t < T) c += __builtin_amdgcn_fmed3f(la_t[t], kLogDecayFloor, 0.f);
            cum[t] = c;
            if (t + 1 == n) cn = c;
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const float xt = t < T ? x_t[t] : 0.f;
            const float xd = xt * exp_e(cum[t]);
            if (kside) {
                sKd[t * D + d] = xd;
                sKi[t * D + d] = xt * exp_e(-cum[t]);
                sA[t * AS + d] = (bf16)xd;
                sKrT[d * RS + t] = (bf16)(t < n ? xt * exp_e(cn - cum[t]) : 0.f);
                sKrT[d * RS + 8 + t] = (bf16)0.f;
            } else {
                sQd[t * D + d] = xd;
                sA[(8 + t) * AS + d] = (bf16)xd;
            }
        }
        if (kside) sDal[d] = exp_e(cn);
        else if (d < TM) sBeta[d] = d < T ? beta_d : 0.f;
    }
    __syncthreads();

    // ---- L and M: the 8 x 8 dot products over the channels, all at once:
    //      thread (pair p = tid / 4, quarter j = tid % 4) sums channels
    //      32j .. 32j + 31 of k_t.Ki_s and q_t.Ki_s, then a quad reduction
    {
        const int p = tid >> 2, j = tid & 3;
        const int t = p >> 3, s = p & 7;
        const f32x4* kd4 = reinterpret_cast<const f32x4*>(sKd + t * D + 32 * j);
        const f32x4* qd4 = reinterpret_cast<const f32x4*>(sQd + t * D + 32 * j);
        const f32x4* ki4 = reinterpret_cast<const f32x4*>(sKi + s * D + 32 * j);
        f32x4 ak = zero4(), aq = zero4();
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const f32x4 ki = ki4[c];
            ak += kd4[c] * ki;
            aq += qd4[c] * ki;
        }
        float dk = ak[0] + ak[1] + ak[2] + ak[3];
        float dq = aq[0] + aq[1] + aq[2] + aq[3];
        dk += dpp_f<0xB1>(dk);   // quad_perm [1,0,3,2]
        dq += dpp_f<0xB1>(dq);
        dk += dpp_f<0x4E>(dk);   // quad_perm [2,3,0,1]
        dq += dpp_f<0x4E>(dq);
        if (j == 0) {
            const bool live = t < T && s < T;
            sL[p] = (live && s < t) ? sBeta[t] * dk : 0.f;
            sM[p] = (live && s <= t) ? dq : 0.f;
        }
    }

    // ---- W = [K_decay; Q_decay] S on the matrix cores, 32 state rows per
    //      step: the B operand of step kk is this lane's part of the tiles
    //      2kk and 2kk + 1 (rows 32kk + 4g + i and 32kk + 16 + 4g + i)
    // (row pieces to accumulator tiles, once the loads are in)
#pragma unroll
    for (int m = 0; m < 8; ++m) tiles_from_rows(st[m][0], st[m][1]);
    f32x4 Wc[2] = {zero4(), zero4()};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a = ldA_perm8(sA + r * AS, 32 * kk, sig);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) Wc[ct] = mma32(a, pack8(st[2 * kk][ct], st[2 * kk + 1][ct]), Wc[ct]);
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) sW[(4 * g + i) * D + c0 + 16 * ct + r] = Wc[ct][i];
    __syncthreads();

    // ---- U by forward substitution and O, one value column per key-side thread
    if (kside) {
        float u[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            float x = 0.f;
            if (t < T) {
                x = sBeta[t] * (vcol[t] - sW[t * D + d]);
#pragma unroll
                for (int s = 0; s < t; ++s) x -= sL[t * TM + s] * u[s];
            }
            u[t] = x;
            sU[t * AS + d] = (bf16)x;
            sU[(8 + t) * AS + d] = (bf16)0.f;
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            if (t < T) {
                float y = sW[(8 + t) * D + d];
#pragma unroll
                for (int s = 0; s <= t; ++s) y += sM[t * TM + s] * u[s];
                o[row(t) * D + d] = (bf16)y;
            }
        }
    }

    // ---- commit the accepted prefix: S = Diag(a_{n-1}) S + K_restore^T U,
    //      one 16-row tile at a time from the registers loaded at the start:
    //      decayed, updated on the matrix cores in fp32 and written back
    if (n == 0) return;   // verify pass: the state is only read (uniform)
    __syncthreads();
    s16x4 b[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) b[ct][i] = __builtin_bit_cast(short, sU[(4 * g + i) * AS + c0 + 16 * ct + r]);
    // The updated tiles go back to the row pieces of the loads through a
    // per-wave LDS block (sW is dead after the barrier above) rather than by
    // lane permutes: v_permlane16_swap on matrix-core results, followed by
    // the quad transposes, left stale values in the last lane of a 16-lane
    // row now and then on gfx950 (about 7 of 8192 heads per call).
    float* tb = sW + wave * (16 * RT);
    const int prow = 4 * (lane >> 5) + (lane & 3), pcol = 4 * ((lane >> 2) & 7);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        // (accumulator row 4g + i is state row 16m + 4 sig(g) + i; the A
        // operand's row r likewise stands for state row 16m + 4 sig(r / 4) + r % 4)
        const f32x4 dal = *reinterpret_cast<const f32x4*>(&sDal[16 * m + 4 * sig]);
        const int ar = 4 * (((r >> 2) & 1) << 1 | (r >> 3)) + (r & 3);
        const s16x4 a = *reinterpret_cast<const s16x4*>(&sKrT[(16 * m + ar) * RS + 4 * g]);
        const f32x4 t[2] = {mma16(a, b[0], st[m][0] * dal), mma16(a, b[1], st[m][1] * dal)};
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) tb[(4 * sig + i) * RT + 16 * ct + r] = t[ct][i];
        lds_fence_wave();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f32x4 y = *reinterpret_cast<const f32x4*>(&tb[(8 * h + prow) * RT + pcol]);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), srs, off,
                                                   (2 * m + h) * 8 * D * 4, kNT);
        }
        lds_fence_wave();   // the block's reads are done before the next tile's writes
    }
}

}  // namespace

bool decode_multi_mfma_supported(bool bf16_io, int dk, int dv, int ntok) {
    return bf16_io && dk == D && dv == D && ntok >= 2 && ntok <= TM;
}

hipError_t launch_decode_multi_mfma(const void* q, const void* k, const void* v, const float* la,
                                    const float* beta, float* S, void* o, const int* n_commit,
                                    int BH, int H, int ntok, hipStream_t st)
{
    hipLaunchKernelGGL(decode_multi_mfma_kernel, dim3((unsigned)BH), dim3(256), 0, st,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, la, beta, S, (bf16*)o,
                       n_commit, H, ntok);
    return hipGetLastError();
}

}  // namespace kda
