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
constexpr int kSplitCUs = 256;   // compute units of the GPU (MI355X)

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

// Split schedule of a packed call (the many-head fused path): a sequence
// whose chunk count exceeds what one compute unit would get with the work
// spread evenly (M = ceil(total chunks * H / 256)) would alone set the
// call's length, since the fused kernel walks each (sequence, head) in one
// workgroup. Such a sequence keeps its first m chunks in the fused kernel
// (m = M rounded down to whole checkpoint intervals) and hands the rest to
// the chunk-parallel prep and the state walk, as an entry of a second table.
// Candidates (at least 8 chunks beyond m) are taken in index order while at
// most n2 of them and at most cap2 second-segment chunks in all are taken;
// the candidate that reaches cap2 is cut shorter (its first segment grows).
// Fused workgroups take the sequences longest first (by first-segment
// length), so the longest chains start at once. Output (ints, layout of
// SplitTables in kda_launch.h): ord, lens1, mslot [N]; tab2 [3 n2 + 3];
// lens2, fin2 [n2].
__global__ __launch_bounds__(kTabThreads) void varlen_split_kernel(
    const int* __restrict__ tab, int N, int T, int C, int K, int H, int n2, int cap2,
    int* __restrict__ out)
{
    __shared__ int sh[2][kTabWaves];
    __shared__ int key[kTabThreads];
    const int i = threadIdx.x;
    const bool live = i < N;
    const int total = tab[2 * N + 1];
    const int M = (int)(((long long)total * H + kSplitCUs - 1) / kSplitCUs);
    const int kc = K > 0 ? K / C : 1;                       // chunks per checkpoint interval
    const int mA = max(kc, (M / kc) * kc);
    const int st = live ? tab[i] : 0;
    const int len = live ? tab[i + 1] - st : 0;
    const int nch = len / C + (len % C != 0);
    const bool cand = live && nch >= mA + 8;
    const int want = cand ? nch - mA : 0;
    int tw, tc;
    const int pw = block_scan<false>(want, sh[0], tw);       // inclusive
    const int pc = block_scan<false>(cand ? 1 : 0, sh[1], tc);
    const int before = pw - want;                            // second-segment chunks taken before i
    int m = nch;                                             // first-segment chunks
    bool taken = cand && pc <= n2 && before < cap2;
    if (taken) {
        const int n2c = min(want, cap2 - before);
        m = ((nch - n2c + kc - 1) / kc) * kc;
        if (nch - m < 8) {
            taken = false;
            m = nch;
        }
    }
    const int len1 = taken ? m * C : len;
    int* ord = out;
    int* lens1 = out + N;
    int* mslot = out + 2 * N;
    int* tab2 = out + 3 * N;
    int* lens2 = tab2 + 3 * n2 + 3;
    int* fin2 = lens2 + n2;
    // Entries of the second table go longest first (by second-segment
    // chunks, ties by index), so the state walk starts its longest chains
    // first; entry j's chunks follow those of entries 0 .. j-1.
    const int nch2 = taken ? nch - m : 0;
    key[i] = nch2;
    __syncthreads();
    int j = 0, c2 = 0, total2 = 0, nl = 0;
    for (int u = 0; u < N; ++u) {
        const int ku = key[u];
        const bool ahead = ku > nch2 || (ku == nch2 && u < i);
        j += ku > 0 && ahead;
        c2 += ahead ? ku : 0;
        total2 += ku;
        nl += ku > 0;
    }
    if (live) {
        lens1[i] = len1;
        mslot[i] = taken ? j : -1;
    }
    if (taken) {
        tab2[j] = st + m * C;
        tab2[n2 + 1 + j] = c2;
        tab2[2 * n2 + 2 + j] = K > 0 ? tab[2 * N + 2 + i] + m * C / K : 0;
        lens2[j] = len - m * C;
        fin2[j] = i;
    }
    for (int e = nl + i; e < n2; e += kTabThreads) {         // unused entries
        tab2[e] = T;
        tab2[n2 + 1 + e] = total2;
        tab2[2 * n2 + 2 + e] = 0;
        lens2[e] = 0;
        fin2[e] = -1;
    }
    if (i == 0) {
        tab2[n2] = T;
        tab2[2 * n2 + 1] = total2;
        tab2[3 * n2 + 2] = 0;
    }
    __syncthreads();
    // longest first: rank by first-segment length, ties by index
    key[i] = live ? len1 : -1;
    __syncthreads();
    if (live) {
        int rank = 0;
        for (int u = 0; u < N; ++u) {
            const int ku = key[u];
            rank += (ku > len1) || (ku == len1 && u < i);
        }
        ord[rank] = i;
    }
}

}  // namespace

hipError_t launch_varlen_split(const int* tab, int N, int T, int C, int K, int H, int n2,
                               int cap2, int* out, hipStream_t st) {
    if (N > kTabThreads) return hipErrorInvalidValue;
    hipLaunchKernelGGL(varlen_split_kernel, dim3(1), dim3(kTabThreads), 0, st, tab, N, T, C, K, H,
                       n2, cap2, out);
    return hipGetLastError();
}

hipError_t launch_varlen_table(const int* cu, int N, int T, int C, int K, int* tab,
                               hipStream_t st) {
    hipLaunchKernelGGL(varlen_table_kernel, dim3(1), dim3(kTabThreads), 0, st, cu, N, T, C, K,
                       tab);
    return hipGetLastError();
}

}  // namespace kda
