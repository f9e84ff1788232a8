// Shared device helpers for the KDA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    bf16 b = (bf16)x;
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ float bf16_from_bits(uint16_t u) {
    return __builtin_bit_cast(float, (uint32_t)u << 16);
}

// Pack four fp32 into the 4 x bf16 operand of v_mfma_f32_16x16x16_bf16.
__device__ __forceinline__ s16x4 pack4(f32x4 v) {
    s16x4 r;
    r[0] = (short)bf16_bits(v[0]);
    r[1] = (short)bf16_bits(v[1]);
    r[2] = (short)bf16_bits(v[2]);
    r[3] = (short)bf16_bits(v[3]);
    return r;
}

// Pack 2 x 4 fp32 into the 8 x bf16 operand of v_mfma_f32_16x16x32_bf16.
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
    bf16x8 r;
    r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
    r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
    return r;
}

// D(16x16,f32) += A(16x32) * B(32x16), bf16 operands.
// Lane l holds A[l%16][8(l/16)..+7], B[8(l/16)..+7][l%16], D[4(l/16)..+3][l%16].
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// D(16x16,f32) += A(16x16) * B(16x16), bf16 operands.
// Lane l holds A[l%16][4(l/16)..+3], B[4(l/16)..+3][l%16], D[4(l/16)..+3][l%16].
__device__ __forceinline__ f32x4 mma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Wave index inside the workgroup, as a wave-uniform (scalar) value. Control
// flow that depends on it is then a scalar branch: MFMA instructions ignore
// the EXEC mask, so they must never sit under a lane-masked branch.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Sequence layout of a prefill call. Tokens are packed along one axis
// ([tokens, H, d] row-major); sequence i covers tokens
// [start(i), start(i) + len(i)) and is cut into chunks of C tokens from its
// own start. Either N sequences of T tokens each (tab == nullptr), or a table
// built on the device from cumulative offsets (launch_varlen_table):
//   tab[0 .. N]           offsets, non-decreasing, inside [0, T]
//   tab[N+1 .. 2N+1]      first chunk of each sequence in a numbering of all
//                         chunks (exclusive prefix sum; tab[2N+1] = total)
//   tab[2N+2 .. 3N+2]     first checkpoint slot of each sequence
// K is the checkpoint interval in tokens (a multiple of C), 0 for none:
// sequence i has len(i) / K checkpoints, the states after K, 2K, ... tokens.
// Without a table, sequence i starts at token i * S (S >= T: a window of T
// tokens of longer sequences, as the piecewise prefill walks them).
//
// Split schedule of a packed call (all null otherwise; see varlen_split in
// kda_varlen.hip): a long sequence runs its first segment in the fused
// kernel and the rest as an entry of a second table that the prep and state
// kernels walk.
//   lens  explicit entry lengths: entry i covers [tab[i], tab[i] + lens[i])
//         (the entries need not tile the token axis)
//   ord   fused kernel: sequence of the j-th group of workgroups (longest first)
//   mslot fused kernel: slot of sequence i's first-segment end state in mid,
//         -1 when it is not split
//   fin   state kernel: original sequence of entry i (its S_final row), -1 for
//         an unused entry (its workgroups exit at once)
struct SeqLayout {
    const int* tab;
    int N;   // sequences
    int T;   // tokens per sequence (no table) or in all (table)
    int C;   // chunk length of the chunk numbering
    int K;   // checkpoint interval, 0 = none
    long S;  // tokens between sequence starts (no table)
    const int* lens = nullptr;
    const int* ord = nullptr;
    const int* mslot = nullptr;
    const int* fin = nullptr;
    float* mid = nullptr;
    __device__ long start(int i) const { return tab ? (long)tab[i] : (long)i * S; }
    __device__ int len(int i) const {
        return lens ? lens[i] : (tab ? tab[i + 1] - tab[i] : T);
    }
    __device__ long chunk0(int i) const {
        return tab ? (long)tab[N + 1 + i] : (long)i * ((T + C - 1) / C);
    }
    __device__ long ckpt0(int i) const {
        return tab ? (long)tab[2 * N + 2 + i] : (K ? (long)i * (T / K) : 0);
    }
};

// Natural exponential through the hardware exp2 (v_exp_f32).
__device__ __forceinline__ float exp_e(float x) { return __expf(x); }

// Weight-free prologue of the layer form ("Kimi K3: the manos...", section
// "Kimi Linear"): where the per-channel log-decay comes from, and whether q
// and k arrive raw and are L2-normalised here.
//   kGateLog      log-decay given, fp32 [.., dk]
//   kGateBounded  gate pre-activation g in the q/k dtype, [.., dk]:
//                 log_alpha = -bound * sigmoid(g), inside (-bound, 0)
//   kGateScalar   one fp32 log-decay per token and head, [..]: the Gated
//                 DeltaNet gate, broadcast over the key channels
// Kernels that take the prologue as a template argument encode it as
// PRO = gate | (l2 ? 4 : 0); PRO = 0 is the plain op.
enum : int { kGateLog = 0, kGateBounded = 1, kGateScalar = 2, kProL2 = 4 };
struct Prologue {
    float l2_eps;   // q_hat = q / sqrt(sum q^2 + l2_eps)
    float bound;    // kGateBounded
};

// sigmoid through v_exp_f32 and v_rcp_f32 (about 1 ulp each)
__device__ __forceinline__ float sigmoid_f(float x) {
    return __builtin_amdgcn_rcpf(1.f + exp_e(-x));
}

// One DPP move (dpp_ctrl CTRL, rows ROWS) of a float; lanes of rows outside
// ROWS read 0.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false));
}

// Sum over each 16-lane row (lanes 16j .. 16j+15), left in every lane of the
// row: quad permutes [1,0,3,2] and [2,3,0,1], then row rotates by 4 and 8.
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp_f<0xB1>(x);
    x += dpp_f<0x4E>(x);
    x += dpp_f<0x124>(x);
    x += dpp_f<0x128>(x);
    return x;
}

// Layer epilogue inputs: o = w * o / sqrt(mean(o^2) + eps) * sigmoid(z).
struct Epilogue {
    const void* z;    // [tokens, H, dv] in the output dtype
    const float* w;   // [dv] or null (ones)
    float eps;
};

// Sum over the 64 lanes of a wave as a wave-uniform value, without LDS:
// DPP adds inside each 16-lane row (quad permutes [1,0,3,2] and [2,3,0,1],
// then row rotates by 4 and 8 lanes leave the row sum in every lane), then
// row_bcast:15 into rows 1 and 3 and row_bcast:31 into rows 2 and 3 leave
// the total in row 3, read from lane 63.
__device__ __forceinline__ float wave_sum_uniform(float x) {
    x = row_sum16(x);
    x += dpp_f<0x142, 0xA>(x);   // row_bcast:15
    x += dpp_f<0x143, 0xC>(x);   // row_bcast:31
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Workgroup barrier for LDS hazards only: waits for this wave's LDS (and
// scalar) operations, not for outstanding global loads, so register
// prefetches stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until this wave's LDS operations have completed.
__device__ __forceinline__ void lds_fence_wave() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

}  // namespace kda
