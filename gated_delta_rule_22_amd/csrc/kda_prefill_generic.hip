// Generic chunked KDA prefill with fp32 arithmetic on the vector ALUs.
//
// Serves the fp32-input path (where a 1e-5 match to the fp64 recurrence is
// required, so no bf16 rounding may enter) and any dk/dv/chunk the bf16 MFMA
// kernel does not implement. One workgroup per (batch, head); the state lives
// in LDS for the whole sequence. Sequences follow a SeqLayout (fixed-length
// batches or a packed variable-length table), and the state after every K
// tokens of a sequence can be stored as a checkpoint.
//
// Per chunk of n tokens with starting state S ("Kimi K3: the manos...",
// section "FlashKDA Algorithm"; cum_t is the inclusive sum of log-decays from
// the chunk start, so D_{t:s+1} = Diag(exp(cum_t - cum_s))):
//   L_ts   = beta_t k_t^T D_{t:s+1} k_s        (s < t, strictly lower)
//   Mqk_ts = q_t^T D_{t:s+1} k_s               (s <= t, lower incl. diagonal)
//   U      = (I + L)^{-1} Diag(beta)(V - K_decay S),  K_decay_t = exp(cum_t) k_t
//   O      = Q_decay S + Mqk U,                      Q_decay_t = exp(cum_t) q_t
//   S      = Diag(exp(cum_last)) S + K_restore^T U,  K_restore_t = exp(cum_last - cum_t) k_t
// Every decay factor is formed as exp of a non-positive log difference, so no
// intermediate can overflow whatever the chunk length. The triangular system
// is solved by forward substitution, one value column per thread.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

namespace gen {
constexpr int kThreads = 256;
constexpr int kTile = 2048;      // max n * max(dk, dv) elements per tile
constexpr int kMaxC = 64;
constexpr int kMaxD = 128;
}  // namespace gen

template <typename T>
__global__ __launch_bounds__(gen::kThreads) void prefill_generic_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const void* __restrict__ gate, const float* __restrict__ beta,
    const float* S0, T* __restrict__ o, float* S_final,
    SeqLayout sq, int H, int dk, int dv, int C, float* __restrict__ S_ckpt, int ck_slots,
    int pro, Prologue pr)
{
    __shared__ float sS[gen::kMaxD * gen::kMaxD];
    __shared__ float sQ[gen::kTile], sK[gen::kTile], sCum[gen::kTile], sKd[gen::kTile];
    __shared__ float sV[gen::kTile], sU[gen::kTile];
    __shared__ float sL[gen::kMaxC * gen::kMaxC], sM[gen::kMaxC * gen::kMaxC];
    __shared__ float sBeta[gen::kMaxC], sAlast[gen::kMaxD], sScale[2 * gen::kMaxC];

    const int tid = threadIdx.x;
    const int NT = blockDim.x;
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;   // sequence b, head h
    const size_t soff = (size_t)bh * dk * dv;
    const long tok0 = sq.start(b);
    const int Tlen = sq.len(b);
    const bool ckpt = S_ckpt != nullptr && sq.K > 0;
    const long ck0 = ckpt ? sq.ckpt0(b) : 0;

    for (int i = tid; i < dk * dv; i += NT) sS[i] = S0 ? S0[soff + i] : 0.f;
    __syncthreads();

    for (int c0 = 0; c0 < Tlen; c0 += C) {
        const int n = min(C, Tlen - c0);
        // token-head row index of token t of this chunk
        auto row = [&](int t) -> size_t { return ((size_t)tok0 + c0 + t) * H + h; };

        const int gm = pro & 3;
        for (int i = tid; i < n * dk; i += NT) {
            const int t = i / dk, d = i - t * dk;
            const size_t g = row(t) * dk + d;
            sQ[i] = to_f32(q[g]);
            sK[i] = to_f32(k[g]);
            // log-decay from the gate input (plain op: given)
            if (gm == kGateLog) sCum[i] = static_cast<const float*>(gate)[g];
            else if (gm == kGateBounded) sCum[i] = -pr.bound / (1.f + expf(-to_f32(static_cast<const T*>(gate)[g])));
            else sCum[i] = static_cast<const float*>(gate)[row(t)];
        }
        for (int i = tid; i < n * dv; i += NT) {
            const int t = i / dv, j = i - t * dv;
            sV[i] = to_f32(v[row(t) * dv + j]);
        }
        for (int t = tid; t < n; t += NT) sBeta[t] = beta[row(t)];
        __syncthreads();

        // layer prologue: q, k L2-normalised per token
        if (pro & kProL2) {
            for (int t = tid; t < 2 * n; t += NT) {
                float* x = (t < n ? sQ : sK) + (t % n) * dk;
                float ss = 0.f;
                for (int d = 0; d < dk; ++d) ss += x[d] * x[d];
                sScale[t] = 1.f / sqrtf(ss + pr.l2_eps);
            }
            __syncthreads();
            for (int i = tid; i < n * dk; i += NT) {
                const int t = i / dk;
                sQ[i] *= sScale[t];
                sK[i] *= sScale[n + t];
            }
            __syncthreads();
        }

        // chunk-local inclusive cumulative log-decay, one channel per thread
        for (int d = tid; d < dk; d += NT) {
            float run = 0.f;
            for (int t = 0; t < n; ++t) { run += sCum[t * dk + d]; sCum[t * dk + d] = run; }
        }
        __syncthreads();

        // intra-chunk interactions with exact per-channel decay ratios
        for (int i = tid; i < n * n; i += NT) {
            const int t = i / n, s = i - t * n;
            float lk = 0.f, mq = 0.f;
            if (s <= t) {
                for (int d = 0; d < dk; ++d) {
                    const float e = exp_e(sCum[t * dk + d] - sCum[s * dk + d]);
                    const float ks = sK[s * dk + d] * e;
                    lk += sK[t * dk + d] * ks;
                    mq += sQ[t * dk + d] * ks;
                }
            }
            sL[t * gen::kMaxC + s] = (s < t) ? sBeta[t] * lk : 0.f;
            sM[t * gen::kMaxC + s] = mq;
        }
        __syncthreads();

        // decay-scaled operands: K_decay, Q_decay (in place of q), K_restore (in place of k)
        for (int i = tid; i < n * dk; i += NT) {
            const int t = i / dk, d = i - t * dk;
            const float cm = sCum[i];
            const float cl = sCum[(n - 1) * dk + d];
            const float a = exp_e(cm);
            const float kv = sK[i];
            sKd[i] = a * kv;
            sQ[i] = a * sQ[i];
            sK[i] = exp_e(cl - cm) * kv;
        }
        for (int d = tid; d < dk; d += NT) sAlast[d] = exp_e(sCum[(n - 1) * dk + d]);
        __syncthreads();

        // right-hand side Diag(beta)(V - K_decay S)
        for (int i = tid; i < n * dv; i += NT) {
            const int t = i / dv, j = i - t * dv;
            float acc = 0.f;
            for (int d = 0; d < dk; ++d) acc += sKd[t * dk + d] * sS[d * dv + j];
            sU[i] = sBeta[t] * (sV[i] - acc);
        }
        __syncthreads();

        // (I + L) U = rhs by forward substitution; columns are independent
        for (int j = tid; j < dv; j += NT) {
            for (int t = 1; t < n; ++t) {
                float acc = sU[t * dv + j];
                for (int s = 0; s < t; ++s) acc -= sL[t * gen::kMaxC + s] * sU[s * dv + j];
                sU[t * dv + j] = acc;
            }
        }
        __syncthreads();

        // outputs from the chunk's starting state plus the causal intra-chunk term
        for (int i = tid; i < n * dv; i += NT) {
            const int t = i / dv, j = i - t * dv;
            float acc = 0.f;
            for (int d = 0; d < dk; ++d) acc += sQ[t * dk + d] * sS[d * dv + j];
            for (int s = 0; s <= t; ++s) acc += sM[t * gen::kMaxC + s] * sU[s * dv + j];
            o[row(t) * dv + j] = from_f32<T>(acc);
        }
        __syncthreads();

        // state carry to the end of the chunk
        for (int i = tid; i < dk * dv; i += NT) {
            const int d = i / dv, j = i - d * dv;
            float acc = sAlast[d] * sS[i];
            for (int s = 0; s < n; ++s) acc += sK[s * dk + d] * sU[s * dv + j];
            sS[i] = acc;
        }
        __syncthreads();

        // checkpoint j after j * K tokens (C divides K, so chunk ends meet it)
        if (ckpt && (c0 + n) % sq.K == 0) {
            const long slot = ck0 + (c0 + n) / sq.K - 1;
            if (slot < ck_slots) {
                float* dst = S_ckpt + ((size_t)slot * H + h) * dk * dv;
                for (int i = tid; i < dk * dv; i += NT) dst[i] = sS[i];
            }
        }
    }

    if (S_final)
        for (int i = tid; i < dk * dv; i += NT) S_final[soff + i] = sS[i];
}

hipError_t launch_prefill_generic(bool bf16_io, const void* q, const void* k, const void* v,
                                  const void* gate, const float* beta, const float* S0,
                                  void* o, float* S_final, const SeqLayout& sq, int H, int dk,
                                  int dv, int chunk, float* S_ckpt, int ck_slots, int pro,
                                  const Prologue& pr, hipStream_t st)
{
    // Largest chunk whose tiles fit the LDS budget; the chunk length changes
    // only the blocking, never the result.
    int C = chunk;
    const int dmax = dk > dv ? dk : dv;
    while (C > 1 && C * dmax > gen::kTile) C >>= 1;
    if (C > gen::kMaxC) C = gen::kMaxC;
    const dim3 grid((unsigned)((long)sq.N * H));
    if (bf16_io)
        hipLaunchKernelGGL(prefill_generic_kernel<bf16>, grid, dim3(gen::kThreads), 0, st,
                           (const bf16*)q, (const bf16*)k, (const bf16*)v, gate, beta, S0,
                           (bf16*)o, S_final, sq, H, dk, dv, C, S_ckpt, ck_slots, pro, pr);
    else
        hipLaunchKernelGGL(prefill_generic_kernel<float>, grid, dim3(gen::kThreads), 0, st,
                           (const float*)q, (const float*)k, (const float*)v, gate, beta, S0,
                           (float*)o, S_final, sq, H, dk, dv, C, S_ckpt, ck_slots, pro, pr);
    return hipGetLastError();
}

}  // namespace kda
