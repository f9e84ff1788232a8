// Sequence table of a packed variable-length prefill.
//
// Serving packs the prompts of several requests along one token axis and
// keeps the KDA state of each request at its prompt end and at coarse token
// intervals (the trillion-scale architecture page, section 6, and "Kimi K3:
// the manos...", section "KDA Prefix Cache Management": states exist only at
// chosen boundaries, since storing one per token would grow with the length).
// The caller describes the packing by cumulative offsets cu[0..N] on the
// device; one small workgroup turns them into the table the prefill kernels
// read (layout: SeqLayout in kda_common.h):
//   offsets       m_j = max(clamp(cu[0..j], 0, T)), so sequence i covers
//                 [m_i, m_{i+1}); equal to cu for valid (non-decreasing,
//                 in-range) offsets, and never out of bounds or overlapping
//                 otherwise
//   chunk starts  exclusive prefix sum of ceil(len_i / C)
//   ckpt starts   exclusive prefix sum of floor(len_i / K) (0 when K = 0)
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kTabThreads = 1024;
constexpr int kTabWaves = kTabThreads / kWave;

// Inclusive scan (running max, or running sum) of one value per thread over
// the workgroup; `total` receives the workgroup-wide result. `sh` holds one
// int per wave and may be reused after the next __syncthreads.
template <bool kMax>
__device__ __forceinline__ int block_scan(int x, int* sh, int& total) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane >= d) x = kMax ? max(x, y) : x + y;
    }
    if (lane == kWave - 1) sh[w] = x;
    __syncthreads();
    int pre = 0;
    total = 0;
#pragma unroll
    for (int j = 0; j < kTabWaves; ++j) {
        const int s = sh[j];
        if (j < w) pre = kMax ? max(pre, s) : pre + s;
        total = kMax ? max(total, s) : total + s;
    }
    return kMax ? max(pre, x) : pre + x;
}

__device__ __forceinline__ int clamp_tok(int x, int T) { return min(max(x, 0), T); }

__global__ __launch_bounds__(kTabThreads) void varlen_table_kernel(
    const int* __restrict__ cu, int N, int T, int C, int K, int* __restrict__ tab)
{
    __shared__ int sh[3][kTabWaves];
    int carry_m = 0, carry_ch = 0, carry_ck = 0;
    for (int base = 0; base < N; base += kTabThreads) {
        const int i = base + (int)threadIdx.x;
        const bool live = i < N;
        const int a = live ? clamp_tok(cu[i], T) : 0;
        const int b = live ? clamp_tok(cu[i + 1], T) : 0;
        int tm, tch, tck;
        const int m = max(carry_m, block_scan<true>(a, sh[0], tm));   // m_i
        const int len = live ? max(m, b) - m : 0;                      // m_{i+1} - m_i
        const int ch = len / C + (len % C != 0);
        const int ck = K > 0 ? len / K : 0;
        const int ich = block_scan<false>(ch, sh[1], tch);
        const int ick = block_scan<false>(ck, sh[2], tck);
        if (live) {
            tab[i] = m;
            tab[N + 1 + i] = carry_ch + ich - ch;
            tab[2 * N + 2 + i] = carry_ck + ick - ck;
        }
        carry_m = max(carry_m, tm);
        carry_ch += tch;
        carry_ck += tck;
        __syncthreads();   // sh is reused by the next tile
    }
    if (threadIdx.x == 0) {
        tab[N] = max(carry_m, clamp_tok(cu[N], T));
        tab[2 * N + 1] = carry_ch;
        tab[3 * N + 2] = carry_ck;
    }
}

}  // namespace

hipError_t launch_varlen_table(const int* cu, int N, int T, int C, int K, int* tab,
                               hipStream_t st) {
    hipLaunchKernelGGL(varlen_table_kernel, dim3(1), dim3(kTabThreads), 0, st, cu, N, T, C, K,
                       tab);
    return hipGetLastError();
}

}  // namespace kda
