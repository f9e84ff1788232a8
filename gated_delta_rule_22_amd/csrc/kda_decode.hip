// One-token KDA decode step, streaming each fp32 state once from HBM.
//
// Per head ("Kimi K3: the manos...", section "FlashKDA Algorithm", the
// per-token form; Kimi K3 blog, "Decay Old Memory" / "Apply Delta-Rule
// Update"):
//     Sbar = Diag(alpha) S            alpha = exp(log_alpha), per key channel (row)
//     w    = Sbar^T k,  p = Sbar^T q  (reductions over the dk rows)
//     u    = beta (v - w)
//     S    = Sbar + k u^T             (written back in place)
//     o    = S^T q = p + u (k . q)    (same pass: no second read of S)
// The section's complexity analysis counts ~7 dk*dv flops and 8 dk*dv bytes
// (fp32 read + write) per head: the kernel is HBM-bound, so the design goal is
// exactly one coalesced read and one write of every state element.
//
// Mapping: one wave owns one head and a slice of NC (<= 32) columns. Lane
// (cg, rg) holds a float4 of columns and RPL consecutive rows, so each load
// instruction of the wave covers NRG rows x NC*4 bytes. The column reductions
// over rows are xor-shuffles across the NRG lanes sharing a column group.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

// N consecutive row values of one lane, with 16-byte loads where the row
// count allows (the row offset is a multiple of N, so the vectors are aligned).
template <typename T, int N>
__device__ __forceinline__ void load_row_vals(const T* __restrict__ p, float (&out)[N]) {
    if constexpr (sizeof(T) == 2 && N % 8 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 8) {
            const bf16x8 x = *reinterpret_cast<const bf16x8*>(p + i);
#pragma unroll
            for (int j = 0; j < 8; ++j) out[i + j] = (float)x[j];
        }
    } else if constexpr (sizeof(T) == 4 && N % 4 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(p + i);
#pragma unroll
            for (int j = 0; j < 4; ++j) out[i + j] = x[j];
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) out[i] = to_f32(p[i]);
    }
}

// LAYER: the layer form. The log-decay comes from `gate` as `pro` says
// (kGateLog / kGateBounded / kGateScalar), q and k are L2-normalised when
// pro has kProL2, and when z is given the output leaves as
// w * o / sqrt(mean(o^2) + out_eps) * sigmoid(z), the mean taken over the
// head's DV columns (the waves of one head share a workgroup).
template <int DK, int DV, typename T, bool LAYER>
__global__ __launch_bounds__(256) void decode_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const void* __restrict__ gate, const float* __restrict__ beta,
    float* __restrict__ S, T* __restrict__ o, int BH, int pro, Prologue pr,
    const T* __restrict__ z, const float* __restrict__ ow, float out_eps)
{
    constexpr int NC = DV < 32 ? DV : 32;   // columns per wave
    constexpr int NCG = NC / 4;             // float4 column groups
    constexpr int NRG = kWave / NCG;        // row groups
    constexpr int RPL = DK / NRG;           // rows per lane
    constexpr int SLICES = DV / NC;
    static_assert(RPL >= 1 && RPL * NRG == DK, "dk must cover every row group");

    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int head = gw / SLICES;
    // every wave reaches the workgroup barriers (and the layer epilogue's
    // reduction across the waves of a head): no early exit
    const bool live = head < BH;
    const int hd = live ? head : BH - 1;    // idle waves re-read the last head
    const int slice = gw - head * SLICES;
    const int cg = lane % NCG;
    const int rg = lane / NCG;
    const int col = slice * NC + cg * 4;
    const int row0 = rg * RPL;

    // (plain loads measured about 2% faster here than streaming ones; the
    // stores below stream)
    float* Sh = S + (size_t)hd * DK * DV;
    f32x4 s[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r)
        s[r] = *reinterpret_cast<const f32x4*>(Sh + (size_t)(row0 + r) * DV + col);

    float kr[RPL], qr[RPL], lar[RPL];
    load_row_vals<T, RPL>(k + (size_t)hd * DK + row0, kr);
    load_row_vals<T, RPL>(q + (size_t)hd * DK + row0, qr);
    const int gm = LAYER ? (pro & 3) : kGateLog;
    if (gm == kGateLog) {
        load_row_vals<float, RPL>(static_cast<const float*>(gate) + (size_t)hd * DK + row0, lar);
    } else if (gm == kGateBounded) {
        load_row_vals<T, RPL>(static_cast<const T*>(gate) + (size_t)hd * DK + row0, lar);
#pragma unroll
        for (int r = 0; r < RPL; ++r) lar[r] = -pr.bound * sigmoid_f(lar[r]);
    } else {
        const float a = static_cast<const float*>(gate)[hd];
#pragma unroll
        for (int r = 0; r < RPL; ++r) lar[r] = a;
    }
    float vv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) vv[c] = to_f32(v[(size_t)hd * DV + col + c]);
    const float b = beta[hd];
    // The waves of the workgroup (the column slices of one head, or of
    // neighbouring heads when dv < 128) meet here once their loads are in, so
    // that they go on to stream the rows of their states together rather than
    // drifting apart: 162 us per B256 H32 step against 187 us without it.
    __builtin_amdgcn_s_barrier();

    // Decay rows, then the two column reductions and k.q over this lane's rows.
    // (With L2 normalisation the per-head factors of k and q are applied to
    // the reduced sums: S^T k_hat = (S^T k) / |k|.)
    f32x4 w = zero4(), p = zero4();
    float kq = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
        const float a = exp_e(lar[r]);
        s[r] *= a;
        w += s[r] * kr[r];
        p += s[r] * qr[r];
        kq += kr[r] * qr[r];
        if (LAYER) {
            kk += kr[r] * kr[r];
            qq += qr[r] * qr[r];
        }
    }
#pragma unroll
    for (int off = NCG; off < kWave; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            w[c] += __shfl_xor(w[c], off);
            p[c] += __shfl_xor(p[c], off);
        }
        kq += __shfl_xor(kq, off);
        if (LAYER) {
            kk += __shfl_xor(kk, off);
            qq += __shfl_xor(qq, off);
        }
    }
    if (LAYER && (pro & kProL2)) {
        const float ks = __builtin_amdgcn_rsqf(kk + pr.l2_eps);
        const float qs = __builtin_amdgcn_rsqf(qq + pr.l2_eps);
        w *= ks;
        p *= qs;
        kq *= ks * qs;
#pragma unroll
        for (int r = 0; r < RPL; ++r) kr[r] *= ks;
    }

    f32x4 u;
#pragma unroll
    for (int c = 0; c < 4; ++c) u[c] = b * (vv[c] - w[c]);

    if (live) {
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            const f32x4 sn = s[r] + kr[r] * u;
            __builtin_nontemporal_store(sn, reinterpret_cast<f32x4*>(Sh + (size_t)(row0 + r) * DV + col));
        }
    }

    f32x4 ov;
#pragma unroll
    for (int c = 0; c < 4; ++c) ov[c] = p[c] + u[c] * kq;
    if (LAYER && z != nullptr) {
        // mean of o^2 over the head's columns: this wave's column groups
        // (lanes 0 .. NCG-1 of every row group hold the same values), then
        // the SLICES waves of the head through LDS
        __shared__ float part[4];
        float sq = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
#pragma unroll
        for (int off = 1; off < NCG; off <<= 1) sq += __shfl_xor(sq, off);
        const int wv = threadIdx.x >> 6;
        if (lane == 0) part[wv] = sq;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int j = 0; j < SLICES; ++j) tot += part[(wv / SLICES) * SLICES + j];
        const float rs = __builtin_amdgcn_rsqf(tot / DV + out_eps);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float g = sigmoid_f(to_f32(z[(size_t)hd * DV + col + c]));
            const float wc = ow ? ow[col + c] : 1.f;
            ov[c] = wc * ov[c] * rs * g;
        }
    }
    if (live && rg == 0) {
        T* oh = o + (size_t)hd * DV + col;
#pragma unroll
        for (int c = 0; c < 4; ++c) oh[c] = from_f32<T>(ov[c]);
    }
}

// Multi-token decode from a live state: T tokens per sequence applied in
// order with the same per-token step, the state slice staying in registers,
// o written for every token, and the state written back once, right after
// token n = n_commit[b] (clamped to [0, T]; none when n = 0). A verify pass
// (n = 0) thus reads each state element once and writes none; a commit or a
// plain multi-token step reads and writes it once.
template <int DK, int DV, typename T>
__global__ __launch_bounds__(256) void decode_multi_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    float* __restrict__ S, T* __restrict__ o, const int* __restrict__ n_commit,
    int BH, int H, int ntok)
{
    constexpr int NC = DV < 32 ? DV : 32;
    constexpr int NCG = NC / 4;
    constexpr int NRG = kWave / NCG;
    constexpr int RPL = DK / NRG;
    constexpr int SLICES = DV / NC;
    static_assert(RPL >= 1 && RPL * NRG == DK, "dk must cover every row group");

    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int head = gw / SLICES;
    if (head >= BH) return;
    const int slice = gw - head * SLICES;
    const int cg = lane % NCG;
    const int rg = lane / NCG;
    const int col = slice * NC + cg * 4;
    const int row0 = rg * RPL;
    const int bb = head / H, hh = head - bb * H;
    int n = n_commit ? n_commit[bb] : ntok;
    n = __builtin_amdgcn_readfirstlane(min(max(n, 0), ntok));

    float* Sh = S + (size_t)head * DK * DV;
    f32x4 s[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r)
        s[r] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(Sh + (size_t)(row0 + r) * DV + col));

    for (int t = 0; t < ntok; ++t) {
        const size_t tok = ((size_t)bb * ntok + t) * H + hh;
        float kr[RPL], qr[RPL], lar[RPL];
        load_row_vals<T, RPL>(k + tok * DK + row0, kr);
        load_row_vals<T, RPL>(q + tok * DK + row0, qr);
        load_row_vals<float, RPL>(log_alpha + tok * DK + row0, lar);
        float vv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) vv[c] = to_f32(v[tok * DV + col + c]);
        const float b = beta[tok];

        f32x4 w = zero4(), p = zero4();
        float kq = 0.f;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
            s[r] *= exp_e(lar[r]);
            w += s[r] * kr[r];
            p += s[r] * qr[r];
            kq += kr[r] * qr[r];
        }
#pragma unroll
        for (int off = NCG; off < kWave; off <<= 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                w[c] += __shfl_xor(w[c], off);
                p[c] += __shfl_xor(p[c], off);
            }
            kq += __shfl_xor(kq, off);
        }
        f32x4 u;
#pragma unroll
        for (int c = 0; c < 4; ++c) u[c] = b * (vv[c] - w[c]);
#pragma unroll
        for (int r = 0; r < RPL; ++r) s[r] += kr[r] * u;
        if (rg == 0) {
            T* ot = o + tok * DV + col;
#pragma unroll
            for (int c = 0; c < 4; ++c) ot[c] = from_f32<T>(p[c] + u[c] * kq);
        }
        if (t + 1 == n) {
#pragma unroll
            for (int r = 0; r < RPL; ++r)
                __builtin_nontemporal_store(s[r], reinterpret_cast<f32x4*>(Sh + (size_t)(row0 + r) * DV + col));
        }
    }
}

template <int DK, int DV, typename T>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st)
{
    constexpr int NC = DV < 32 ? DV : 32;
    const long waves = (long)a.BH * (DV / NC);
    const int threads = 256;
    const long blocks = (waves + 3) / 4;
    if (a.layer)
        hipLaunchKernelGGL((decode_kernel<DK, DV, T, true>), dim3((unsigned)blocks), dim3(threads),
                           0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.gate, a.beta,
                           a.S, (T*)a.o, a.BH, a.pro, a.pr, (const T*)a.z, a.w, a.out_eps);
    else
        hipLaunchKernelGGL((decode_kernel<DK, DV, T, false>), dim3((unsigned)blocks), dim3(threads),
                           0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.gate, a.beta,
                           a.S, (T*)a.o, a.BH, 0, a.pr, (const T*)nullptr, nullptr, 0.f);
    return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_dv(int dk, int dv, const DecodeArgs& a, hipStream_t st)
{
#define KDA_DEC_CASE(DKV, DVV) \
    if (dk == DKV && dv == DVV) return launch_decode_t<DKV, DVV, T>(a, st);
    KDA_DEC_CASE(16, 16) KDA_DEC_CASE(16, 32) KDA_DEC_CASE(16, 64) KDA_DEC_CASE(16, 128)
    KDA_DEC_CASE(32, 16) KDA_DEC_CASE(32, 32) KDA_DEC_CASE(32, 64) KDA_DEC_CASE(32, 128)
    KDA_DEC_CASE(64, 16) KDA_DEC_CASE(64, 32) KDA_DEC_CASE(64, 64) KDA_DEC_CASE(64, 128)
    KDA_DEC_CASE(128, 16) KDA_DEC_CASE(128, 32) KDA_DEC_CASE(128, 64) KDA_DEC_CASE(128, 128)
#undef KDA_DEC_CASE
    return hipErrorInvalidValue;
}

template <int DK, int DV, typename T>
static hipError_t launch_decode_multi_t(const void* q, const void* k, const void* v,
                                        const float* la, const float* beta, float* S, void* o,
                                        const int* n_commit, int BH, int H, int ntok,
                                        hipStream_t st)
{
    constexpr int NC = DV < 32 ? DV : 32;
    const long waves = (long)BH * (DV / NC);
    const long blocks = (waves + 3) / 4;
    hipLaunchKernelGGL((decode_multi_kernel<DK, DV, T>), dim3((unsigned)blocks), dim3(256), 0, st,
                       (const T*)q, (const T*)k, (const T*)v, la, beta, S, (T*)o, n_commit, BH,
                       H, ntok);
    return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_multi(int dk, int dv, const void* q, const void* k, const void* v,
                                 const float* la, const float* beta, float* S, void* o,
                                 const int* n_commit, int BH, int H, int ntok, hipStream_t st)
{
#define KDA_DEC_CASE(DKV, DVV) \
    if (dk == DKV && dv == DVV) \
        return launch_decode_multi_t<DKV, DVV, T>(q, k, v, la, beta, S, o, n_commit, BH, H, ntok, st);
    KDA_DEC_CASE(16, 16) KDA_DEC_CASE(16, 32) KDA_DEC_CASE(16, 64) KDA_DEC_CASE(16, 128)
    KDA_DEC_CASE(32, 16) KDA_DEC_CASE(32, 32) KDA_DEC_CASE(32, 64) KDA_DEC_CASE(32, 128)
    KDA_DEC_CASE(64, 16) KDA_DEC_CASE(64, 32) KDA_DEC_CASE(64, 64) KDA_DEC_CASE(64, 128)
    KDA_DEC_CASE(128, 16) KDA_DEC_CASE(128, 32) KDA_DEC_CASE(128, 64) KDA_DEC_CASE(128, 128)
#undef KDA_DEC_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode_multi(bool bf16_io, int dk, int dv, const void* q, const void* k,
                               const void* v, const float* la, const float* beta, float* S,
                               void* o, const int* n_commit, int BH, int H, int ntok,
                               hipStream_t st)
{
    // drafts of 2..8 tokens in bf16 at d = 128 run on the matrix cores
    if (decode_multi_mfma_supported(bf16_io, dk, dv, ntok))
        return launch_decode_multi_mfma(q, k, v, la, beta, S, o, n_commit, BH, H, ntok, st);
    if (bf16_io) return dispatch_multi<bf16>(dk, dv, q, k, v, la, beta, S, o, n_commit, BH, H, ntok, st);
    return dispatch_multi<float>(dk, dv, q, k, v, la, beta, S, o, n_commit, BH, H, ntok, st);
}

hipError_t launch_decode(bool bf16_io, int dk, int dv, const DecodeArgs& a, hipStream_t st)
{
    if (bf16_io) return dispatch_dv<bf16>(dk, dv, a, st);
    return dispatch_dv<float>(dk, dv, a, st);
}

}  // namespace kda
