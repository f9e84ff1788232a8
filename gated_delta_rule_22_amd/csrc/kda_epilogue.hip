// Output epilogue of the KDA layer ("Kimi K3: the manos...", section "Kimi
// Linear"): the output of each head is normalised and scaled by an output
// gate. Per token and head, over the d_v values of the row:
//     out = w * o / sqrt(mean(o^2) + eps) * sigmoid(z)
// Used after the prefill paths whose workgroups do not hold a whole head's
// output row. Every value is read once and written once (HBM-bound:
// 3 x d_v x elt bytes per row). out may be o (in place).
//
// Layout of the work: a lane moves 16 bytes of a row (8 bf16 or 4 fp32), so
// LPR = d_v / VEC lanes cover one row and a wave covers 64 / LPR rows per
// load instruction; each wave keeps kUnroll such row groups in flight. The
// row reduction is an xor-butterfly over the LPR lanes of the row.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kEpiWaves = 4;
constexpr int kUnroll = 4;

template <typename T, int DV>
__global__ __launch_bounds__(kEpiWaves * 64) void norm_gate_kernel(
    const T* o, const T* __restrict__ z, const float* __restrict__ w, float eps, T* out,
    long rows)
{
    constexpr int VEC = 16 / sizeof(T);
    constexpr int LPR = DV / VEC;           // lanes per row
    constexpr int RPW = 64 / LPR;           // rows per wave and load
    static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "row split");
    typedef T vecT __attribute__((ext_vector_type(VEC)));

    const int lane = threadIdx.x & 63;
    const int sub = lane / LPR, c0 = (lane % LPR) * VEC;
    float wv[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) wv[e] = w ? w[c0 + e] : 1.f;

    // The workgroup walks the rows in blocks of kEpiWaves * RPW * kUnroll, all
    // its waves taking the same number of steps, and the waves meet once
    // their loads are in so that they stream neighbouring rows together.
    constexpr long kBlockRows = (long)kEpiWaves * RPW * kUnroll;
    const long wave_rows = (long)(threadIdx.x >> 6) * (RPW * kUnroll);
    for (long b0 = (long)blockIdx.x * kBlockRows; b0 < rows; b0 += (long)gridDim.x * kBlockRows) {
        const long r0 = b0 + wave_rows;
        vecT x[kUnroll], g[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const long row = min(r0 + u * RPW + sub, rows - 1);   // tail rows re-read the last
            x[u] = *reinterpret_cast<const vecT*>(o + row * DV + c0);
            g[u] = *reinterpret_cast<const vecT*>(z + row * DV + c0);
        }
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float xf[VEC], sq = 0.f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                xf[e] = to_f32(x[u][e]);
                sq += xf[e] * xf[e];
            }
#pragma unroll
            for (int off = 1; off < LPR; off <<= 1) sq += __shfl_xor(sq, off);
            const float rs = __builtin_amdgcn_rsqf(sq * (1.f / DV) + eps);
            vecT y;
#pragma unroll
            for (int e = 0; e < VEC; ++e) y[e] = from_f32<T>(wv[e] * xf[e] * rs * sigmoid_f(to_f32(g[u][e])));
            const long row = r0 + u * RPW + sub;
            if (row < rows) *reinterpret_cast<vecT*>(out + row * DV + c0) = y;
        }
    }
}

template <typename T, int DV>
hipError_t launch_dv(const void* o, const void* z, const float* w, float eps, void* out,
                     long rows, hipStream_t st)
{
    constexpr int RPW = 64 / (DV / (16 / sizeof(T)));
    const long per_wave = (long)RPW * kUnroll;
    long blocks = (rows + per_wave * kEpiWaves - 1) / (per_wave * kEpiWaves);
    if (blocks > 8192) blocks = 8192;   // then grid-stride
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL((norm_gate_kernel<T, DV>), dim3((unsigned)blocks), dim3(kEpiWaves * 64),
                       0, st, (const T*)o, (const T*)z, w, eps, (T*)out, rows);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const void* o, const void* z, const float* w, float eps, void* out,
                    long rows, int dv, hipStream_t st)
{
    switch (dv) {
        case 16: return launch_dv<T, 16>(o, z, w, eps, out, rows, st);
        case 32: return launch_dv<T, 32>(o, z, w, eps, out, rows, st);
        case 64: return launch_dv<T, 64>(o, z, w, eps, out, rows, st);
        case 128: return launch_dv<T, 128>(o, z, w, eps, out, rows, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_norm_gate(bool bf16_io, const void* o, const void* z, const float* w,
                            float eps, void* out, long rows, int dv, hipStream_t st)
{
    if (bf16_io) return launch_t<bf16>(o, z, w, eps, out, rows, dv, st);
    return launch_t<float>(o, z, w, eps, out, rows, dv, st);
}

}  // namespace kda
