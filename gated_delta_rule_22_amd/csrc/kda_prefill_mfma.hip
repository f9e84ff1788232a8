// Fused chunk-parallel KDA prefill, bf16 MFMA contractions with fp32 state.
//
// Method ("Kimi K3: the manos...", section "FlashKDA Algorithm"): the
// sequence is cut into chunks of C = 64 tokens. Inside a chunk with starting
// state S_in,
//   B      = Diag(beta)(V - K_decay S_in),  L = StrictTril(Diag(beta) K_decay K_inv^T)
//   U      = (I + L)^{-1} B                   (UT transform, pseudo-values)
//   O      = Q_decay S_in + M_qk U,           M_qk = tril(Q_decay K_inv^T)
//   S_out  = Diag(a_last) S_in + K_restore^T U
// with a_t the inclusive cumulative decay from the chunk start.
//
// MI355X design (one workgroup per (batch, head, value block of DVB columns),
// the whole sequence processed in order, state never leaves the chip):
//  * The state block S (128 x DVB fp32) lives in MFMA accumulator registers:
//    wave w owns value columns [16w, 16w+16) and all 128 key rows, as eight
//    16x16 tiles. It feeds MFMAs directly as the B operand (the K index of a
//    32-deep step is permuted identically on both operands, so the
//    accumulator layout needs no LDS round trip).
//  * U does not depend on S_in except linearly: U = U0 - W S_in with
//    U0 = INV Diag(beta) V and W = INV Diag(beta) K_decay. U0 and W are
//    formed by blocked forward substitution on 16-token blocks (fp32 inverses
//    of the four 16x16 diagonal blocks, bf16 MFMA for the rest), so the
//    state-dependent chain per chunk is three MFMA passes: U, then O and S.
//  * Decay factors never overflow: the Gram matrices are built per 16x16
//    token block, factoring the decay at a block boundary so that every
//    factor is <= 1 except the within-block inverse decay, which is bounded by
//    exp(5 * 16) for log-decays in [-5, 0] (the bound stated on the
//    trillion-scale architecture page, section 4) and fits fp32/bf16 range.
//  * The next chunk's q, k, log-decay, v and beta are loaded into registers
//    while the current chunk computes.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace mf {

constexpr int DK = 128;
constexpr int C = 64;
constexpr int KS = 136;   // padded row stride (bf16) of [64][128] tiles
constexpr int TS = 72;    // padded row stride (bf16) of [*][64] tiles
constexpr int LDS_ = 16 * 16 + 4;  // fp32 diagonal block stride

template <int DVB>
struct Smem {
    static constexpr int VS = DVB + 8;
    bf16 Kd[C * KS];        // k_t * exp(c_t - c_{blockstart-1}): Gram left (L)
    bf16 Qd[C * KS];        // q_t * same: Gram left (M_qk)
    bf16 Ki[C * KS];        // k_s * exp(c_{blockstart-1} - c_s): diagonal-block right; later -W
    bf16 Ke[96 * KS];       // k_s * exp(c_{blockend} - c_s), blocks 0..2 + gap copies; later Q_decay
    bf16 KrT[DK * TS];      // K_restore^T [channel][token]
    bf16 V[C * VS];         // this workgroup's value columns
    bf16 nL[C * TS];        // -L (strictly lower; upper blocks stay zero)
    bf16 M[C * TS];         // M_qk (lower incl. diagonal; upper blocks stay zero)
    float Ld[4 * LDS_];     // diagonal blocks of L, fp32
    bf16 D[4 * 256];        // (I + L_II)^{-1}, bf16
    float P[4 * DK];        // exp(c_{blockstart-1}) per block, channel
    float Tot[4 * DK];      // per-block sums of log-decay
    float alast[DK];        // exp(c_63)
    float beta[C];
};

// Gram products: 10 lower block pairs (I, J) x {KK, QK}.
__constant__ int kPairI[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kPairJ[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

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
    return (uint32_t)bf16_bits(a) | ((uint32_t)bf16_bits(b) << 16);
}
__device__ __forceinline__ float lo_bf(uint32_t u) { return bf16_from_bits((uint16_t)(u & 0xffffu)); }
__device__ __forceinline__ float hi_bf(uint32_t u) { return bf16_from_bits((uint16_t)(u >> 16)); }

}  // namespace mf

template <int DVB>
__global__ __launch_bounds__(DVB / 16 * 64) void prefill_mfma_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    const float* S0, bf16* __restrict__ o, float* S_final, int T, int H, int NVB)
{
    using namespace mf;
    constexpr int NW = DVB / 16;
    constexpr int NT = NW * 64;
    constexpr int VS = Smem<DVB>::VS;
    constexpr int VPR = DVB / 8;                 // 16-byte pieces per value row
    static_assert((C * VPR) % NT == 0, "value pieces per thread");
    constexpr int VPT = C * VPR / NT;            // value pieces per thread

    __shared__ Smem<DVB> sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int r = lane & 15;

    const int bid = blockIdx.x;
    const int vb = bid % NVB;
    const int bh = bid / NVB;
    const int b = bh / H;
    const int h = bh - b * H;
    const int col0 = vb * DVB;                   // first value column of this workgroup
    const int ncol = col0 + 16 * wave + r;       // this lane's value column in P4

    auto tokrow = [&](int tok) -> size_t { return ((size_t)b * T + tok) * H + h; };

    // zero the triangular buffers once: their upper blocks are never written
    for (int i = tid; i < C * TS; i += NT) {
        sm.nL[i] = (bf16)0.f;
        sm.M[i] = (bf16)0.f;
    }

    // state tiles: Sacc[m] holds S[16m + 4g + i][ncol]
    f32x4 Sacc[8];
    const size_t sbase = (size_t)bh * DK * 128;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            Sacc[m][i] = S0 ? S0[sbase + (size_t)(16 * m + 4 * g + i) * 128 + ncol] : 0.f;

    // ---- register prefetch of one chunk's inputs
    const bool p1 = tid < 256;              // threads doing the elementwise chunk prep
    const int dp = tid & 63;                // channel pair 2dp, 2dp+1
    const int blk = (tid >> 6) & 3;         // 16-token block
    uint32_t pk[16], pq[16];
    float pla0[16], pla1[16];
    uint4 pv[VPT];
    float pb = 0.f;

    auto prefetch = [&](int c) {
        if (p1) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int tok = c * C + blk * 16 + j;
                if (tok < T) {
                    const size_t base = tokrow(tok) * DK + 2 * dp;
                    pk[j] = *reinterpret_cast<const uint32_t*>(k + base);
                    pq[j] = *reinterpret_cast<const uint32_t*>(q + base);
                    const float2 l2 = *reinterpret_cast<const float2*>(log_alpha + base);
                    pla0[j] = l2.x;
                    pla1[j] = l2.y;
                } else {
                    pk[j] = 0u; pq[j] = 0u; pla0[j] = 0.f; pla1[j] = 0.f;
                }
            }
        }
#pragma unroll
        for (int p = 0; p < VPT; ++p) {
            const int piece = tid + p * NT;
            const int t = piece / VPR, c8 = piece - t * VPR;
            const int tok = c * C + t;
            pv[p] = tok < T ? *reinterpret_cast<const uint4*>(v + tokrow(tok) * 128 + col0 + 8 * c8)
                            : make_uint4(0u, 0u, 0u, 0u);
        }
        if (tid < C) {
            const int tok = c * C + tid;
            pb = tok < T ? beta[tokrow(tok)] : 0.f;
        }
    };

    const int nchunks = (T + C - 1) / C;
    if (nchunks > 0) prefetch(0);

    for (int c = 0; c < nchunks; ++c) {
        __syncthreads();  // previous chunk's readers are done with every buffer

        // ---- P1a: block sums of the log-decay; values and beta to LDS
        if (p1) {
            float run0 = 0.f, run1 = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) { run0 += pla0[j]; run1 += pla1[j]; }
            sm.Tot[blk * DK + 2 * dp] = run0;
            sm.Tot[blk * DK + 2 * dp + 1] = run1;
        }
#pragma unroll
        for (int p = 0; p < VPT; ++p) {
            const int piece = tid + p * NT;
            const int t = piece / VPR, c8 = piece - t * VPR;
            *reinterpret_cast<uint4*>(&sm.V[t * VS + 8 * c8]) = pv[p];
        }
        if (tid < C) sm.beta[tid] = pb;
        __syncthreads();

        // ---- P1b: decay-scaled operands (block-local cumulative log-decay c_t)
        if (p1) {
            float tot[2][4];
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                tot[0][J] = sm.Tot[J * DK + 2 * dp];
                tot[1][J] = sm.Tot[J * DK + 2 * dp + 1];
            }
            float fP[2], fT[2], fR[2], g1[2], g2[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float logP = 0.f, total = 0.f, myT = 0.f;
#pragma unroll
                for (int J = 0; J < 4; ++J) {
                    if (J < blk) logP += tot[e][J];
                    if (J == blk) myT = tot[e][J];
                    total += tot[e][J];
                }
                const int d = 2 * dp + e;
                fP[e] = exp_e(logP);
                if (blk == 3) sm.alast[d] = exp_e(total);
                sm.P[blk * DK + d] = fP[e];
                fT[e] = exp_e(myT);                    // decay over the whole block
                fR[e] = exp_e(total - logP - myT);     // block end -> chunk end
                g1[e] = blk == 0 ? exp_e(tot[e][1]) : (blk == 1 ? exp_e(tot[e][2]) : 0.f);
                g2[e] = blk == 0 ? exp_e(tot[e][1] + tot[e][2]) : 0.f;
            }
            float run0 = 0.f, run1 = 0.f;
            uint32_t kr0[8], kr1[8];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                run0 += pla0[j];
                run1 += pla1[j];
                const float b0 = exp_e(run0), b1 = exp_e(run1);      // <= 1
                const float i0 = exp_e(-run0), i1 = exp_e(-run1);    // <= exp(80) in range
                const float k0 = lo_bf(pk[j]), k1 = hi_bf(pk[j]);
                const float q0 = lo_bf(pq[j]), q1 = hi_bf(pq[j]);
                const int t = blk * 16 + j;
                const float ki0 = k0 * i0, ki1 = k1 * i1;
                const float ke0 = ki0 * fT[0], ke1 = ki1 * fT[1];    // decay t+1 .. block end
                *reinterpret_cast<uint32_t*>(&sm.Kd[t * KS + 2 * dp]) = pack2(k0 * b0, k1 * b1);
                *reinterpret_cast<uint32_t*>(&sm.Qd[t * KS + 2 * dp]) = pack2(q0 * b0, q1 * b1);
                *reinterpret_cast<uint32_t*>(&sm.Ki[t * KS + 2 * dp]) = pack2(ki0, ki1);
                if (blk < 3)
                    *reinterpret_cast<uint32_t*>(&sm.Ke[t * KS + 2 * dp]) = pack2(ke0, ke1);
                if (blk == 0) {
                    *reinterpret_cast<uint32_t*>(&sm.Ke[(48 + j) * KS + 2 * dp]) =
                        pack2(ke0 * g1[0], ke1 * g1[1]);   // pair (2,0)
                    *reinterpret_cast<uint32_t*>(&sm.Ke[(64 + j) * KS + 2 * dp]) =
                        pack2(ke0 * g2[0], ke1 * g2[1]);   // pair (3,0)
                }
                if (blk == 1)
                    *reinterpret_cast<uint32_t*>(&sm.Ke[(80 + j) * KS + 2 * dp]) =
                        pack2(ke0 * g1[0], ke1 * g1[1]);   // pair (3,1)
                // K_restore: decay t+1 .. chunk end, two tokens per 32-bit word
                const float r0 = ke0 * fR[0], r1 = ke1 * fR[1];
                if (j & 1) {
                    kr0[j >> 1] |= (uint32_t)bf16_bits(r0) << 16;
                    kr1[j >> 1] |= (uint32_t)bf16_bits(r1) << 16;
                } else {
                    kr0[j >> 1] = bf16_bits(r0);
                    kr1[j >> 1] = bf16_bits(r1);
                }
            }
            uint4* d0 = reinterpret_cast<uint4*>(&sm.KrT[(2 * dp) * TS + blk * 16]);
            uint4* d1 = reinterpret_cast<uint4*>(&sm.KrT[(2 * dp + 1) * TS + blk * 16]);
            d0[0] = make_uint4(kr0[0], kr0[1], kr0[2], kr0[3]);
            d0[1] = make_uint4(kr0[4], kr0[5], kr0[6], kr0[7]);
            d1[0] = make_uint4(kr1[0], kr1[1], kr1[2], kr1[3]);
            d1[1] = make_uint4(kr1[4], kr1[5], kr1[6], kr1[7]);
        }
        // the registers are free again: start loading the next chunk
        if (c + 1 < nchunks) prefetch(c + 1);
        __syncthreads();

        // ---- P2: intra-chunk Gram blocks -> -L (bf16), L diag blocks (fp32), M_qk
        for (int p = wave; p < 20; p += NW) {
            const int pi = p % 10;
            const bool isK = p < 10;
            const int I = kPairI[pi], J = kPairJ[pi];
            const bf16* left = (isK ? sm.Kd : sm.Qd) + (16 * I + r) * KS;
            const bf16* right;
            if (J == I) right = sm.Ki + (16 * I + r) * KS;
            else if (J == I - 1) right = sm.Ke + (16 * J + r) * KS;
            else right = sm.Ke + ((I == 2 ? 48 : (J == 0 ? 64 : 80)) + r) * KS;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = mma32(ld8(left + 32 * kk + 8 * g), ld8(right + 32 * kk + 8 * g), acc);
            const int s = 16 * J + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * I + 4 * g + i;
                if (isK) {
                    const float val = (J < I || s < t) ? sm.beta[t] * acc[i] : 0.f;
                    sm.nL[t * TS + s] = (bf16)(-val);
                    if (J == I) sm.Ld[I * LDS_ + (4 * g + i) * 16 + r] = val;
                } else {
                    sm.M[t * TS + s] = (bf16)((J < I || s <= t) ? acc[i] : 0.f);
                }
            }
        }
        __syncthreads();

        // ---- P2b: inverses of the diagonal blocks (wave 0), Q_decay (everyone)
        if (wave == 0) {
            // lane (g, r): column r of (I + L_gg)^{-1} by forward substitution
            const float* Lb = sm.Ld + g * LDS_;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = (i == r) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) acc -= Lb[i * 16 + m] * x[m];
                x[i] = acc;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.D[g * 256 + i * 16 + r] = (bf16)x[i];
        }
        bf16* Qdec = sm.Ke;  // Gram right operands are dead now
        for (int idx = tid; idx < C * 64; idx += NT) {
            const int t = idx >> 6, d = 2 * (idx & 63);
            const int I = t >> 4;
            const uint32_t u = *reinterpret_cast<const uint32_t*>(&sm.Qd[t * KS + d]);
            const float a0 = mf::lo_bf(u) * sm.P[I * DK + d];
            const float a1 = mf::hi_bf(u) * sm.P[I * DK + d + 1];
            *reinterpret_cast<uint32_t*>(&Qdec[t * KS + d]) = mf::pack2(a0, a1);
        }
        __syncthreads();

        // ---- P3: W = INV Diag(beta) K_decay (stored negated) and U0 = INV Diag(beta) V
        bf16* nW = sm.Ki;   // Gram right operands are dead now
        f32x4 U0[4];
        constexpr int NWT = 8 / NW;   // W channel tiles per wave
        static_assert(NWT * NW == 8, "waves must divide the 8 key-channel tiles");
#pragma unroll
        for (int rep = 0; rep <= NWT; ++rep) {
            // tiles: W channel tiles wave, wave+NW (< 8), then this wave's U0 tile
            const bool isU = rep == NWT;
            const int ct = wave + rep * NW;
            f32x4 X[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                f32x4 Y;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * I + 4 * g + i;
                    Y[i] = isU ? sm.beta[t] * (float)sm.V[t * VS + 16 * wave + r]
                               : sm.beta[t] * (float)sm.Kd[t * KS + 16 * ct + r] *
                                     sm.P[I * DK + 16 * ct + r];
                }
#pragma unroll
                for (int J = 0; J < I; ++J)
                    Y = mma16(ld4(sm.nL + (16 * I + r) * TS + 16 * J + 4 * g), pack4(X[J]), Y);
                X[I] = mma16(ld4(sm.D + I * 256 + r * 16 + 4 * g), pack4(Y), zero4());
            }
            if (isU) {
#pragma unroll
                for (int I = 0; I < 4; ++I) U0[I] = X[I];
            } else {
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        nW[(16 * I + 4 * g + i) * KS + 16 * ct + r] = (bf16)(-X[I][i]);
            }
        }
        __syncthreads();

        // ---- P4: state-dependent chain for this wave's 16 value columns
        bf16x8 SB[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) SB[kk] = pack8(Sacc[2 * kk], Sacc[2 * kk + 1]);

        f32x4 accU[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            accU[I] = U0[I];
            const bf16* rowp = nW + (16 * I + r) * KS;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) accU[I] = mma32(mf::ldA_perm(rowp, 32 * kk, g), SB[kk], accU[I]);
        }
        bf16x8 UB[2];
        UB[0] = pack8(accU[0], accU[1]);
        UB[1] = pack8(accU[2], accU[3]);

#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 acc = zero4();
            const bf16* qrow = Qdec + (16 * I + r) * KS;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mma32(mf::ldA_perm(qrow, 32 * kk, g), SB[kk], acc);
            const bf16* mrow = sm.M + (16 * I + r) * TS;
            acc = mma32(mf::ldA_perm(mrow, 0, g), UB[0], acc);
            if (I >= 2) acc = mma32(mf::ldA_perm(mrow, 32, g), UB[1], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = c * C + 16 * I + 4 * g + i;
                if (tok < T) o[tokrow(tok) * 128 + ncol] = (bf16)acc[i];
            }
        }

#pragma unroll
        for (int m = 0; m < 8; ++m) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Sacc[m][i] *= sm.alast[16 * m + 4 * g + i];
            const bf16* krow = sm.KrT + (16 * m + r) * TS;
            Sacc[m] = mma32(mf::ldA_perm(krow, 0, g), UB[0], Sacc[m]);
            Sacc[m] = mma32(mf::ldA_perm(krow, 32, g), UB[1], Sacc[m]);
        }
    }

    if (S_final) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S_final[sbase + (size_t)(16 * m + 4 * g + i) * 128 + ncol] = Sacc[m][i];
    }
}

bool prefill_mfma_supported(int dk, int dv, int chunk) {
    return dk == 128 && dv == 128 && (chunk == 64 || chunk == 0);
}

hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, const float* la,
                               const float* beta, const float* S0, void* o, float* S_final,
                               int B, int T, int H, hipStream_t st)
{
    const long heads = (long)B * H;
    // One workgroup per head when that fills the chip; otherwise split the
    // value columns in two to double the workgroup count.
    if (heads >= 256) {
        hipLaunchKernelGGL(prefill_mfma_kernel<128>, dim3((unsigned)heads), dim3(512), 0, st,
                           (const bf16*)q, (const bf16*)k, (const bf16*)v, la, beta, S0,
                           (bf16*)o, S_final, T, H, 1);
    } else {
        hipLaunchKernelGGL(prefill_mfma_kernel<64>, dim3((unsigned)(heads * 2)), dim3(256), 0, st,
                           (const bf16*)q, (const bf16*)k, (const bf16*)v, la, beta, S0,
                           (bf16*)o, S_final, T, H, 2);
    }
    return hipGetLastError();
}

}  // namespace kda
