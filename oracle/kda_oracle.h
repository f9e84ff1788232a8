/*
 * KDA fp64 reference oracle — TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library. The product path never calls it and shares no code with it.
 *
 * It computes the Kimi Delta Attention recurrence token by token, exactly as
 * its definition reads (Kimi K3 blog, section "Kimi Delta Attention",
 * subsections "Decay Old Memory" and "Apply Delta-Rule Update"):
 *     Sbar   = Diag(alpha_t) S_{t-1},   alpha_t = exp(log_alpha_t)
 *     S_t    = Sbar + beta_t k_t (v_t - Sbar^T k_t)^T
 *     o_t    = S_t^T q_t
 * which is the single-matrix form S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
 * + beta_t k_t v_t^T of the same section and of "LLM architecture at trillion
 * scale" section 4.
 *
 * Layouts (row-major, contiguous), all fp64:
 *   q, k, log_alpha [B,T,H,dk]; v, o [B,T,H,dv]; beta [B,T,H];
 *   S0, S_final [B,H,dk,dv]. S0 == NULL means a zero initial state.
 * Returns 0 on success, -1 on a bad argument.
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

int kda_oracle_prefill_f64(const double* q, const double* k, const double* v,
                           const double* log_alpha, const double* beta,
                           const double* S0, double* o, double* S_final,
                           long B, long T, long H, long dk, long dv, int nthreads);

/* One decode step on S[B,H,dk,dv] in place; q,k,log_alpha [B,H,dk]; v,o [B,H,dv]; beta [B,H]. */
int kda_oracle_decode_f64(const double* q, const double* k, const double* v,
                          const double* log_alpha, const double* beta,
                          double* S, double* o,
                          long B, long H, long dk, long dv, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
