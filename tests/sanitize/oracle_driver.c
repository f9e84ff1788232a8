/* Host sanitizer run of the fp64 oracle (built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers.py): random problems of
 * several shapes, including no tokens and no initial state, and one exact
 * invariant per shape (a prefill split at any token continues exactly, since
 * the token loop carries only the state). Exit status 0 = clean. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kda_oracle.h"

static unsigned long long rng = 88172645463325252ull;
static double urand(void) {
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) * (1.0 / 9007199254740992.0);
}

static double* fill(long n, double lo, double hi) {
    double* p = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (long i = 0; i < n; ++i) p[i] = lo + (hi - lo) * urand();
    return p;
}

/* pointer to token t of a [B,T,H,d] tensor, batch b */
static int check(long B, long T, long H, long dk, long dv, int with_s0, long cut) {
    const long nk = B * T * H * dk, nv = B * T * H * dv, nt = B * T * H, ns = B * H * dk * dv;
    double *q = fill(nk, -0.3, 0.3), *k = fill(nk, -0.3, 0.3), *v = fill(nv, -1, 1);
    double *la = fill(nk, -0.2, 0.0), *beta = fill(nt, 0, 1);
    double *S0 = with_s0 ? fill(ns, -0.5, 0.5) : NULL;
    double *o = fill(nv, 0, 0), *S = fill(ns, 0, 0);
    int rc = kda_oracle_prefill_f64(q, k, v, la, beta, S0, o, S, B, T, H, dk, dv, 2);
    if (rc != 0) { printf("prefill rejected B%ld T%ld H%ld\n", B, T, H); return 1; }
    int bad = 0;
    if (B == 1 && cut > 0 && cut < T) {
        /* tokens [0, cut) then [cut, T) from the first part's state */
        const long t1 = T - cut;
        double *S1 = fill(ns, 0, 0), *S2 = fill(ns, 0, 0), *o1 = fill(cut * H * dv, 0, 0),
               *o2 = fill(t1 * H * dv, 0, 0);
        rc = kda_oracle_prefill_f64(q, k, v, la, beta, S0, o1, S1, 1, cut, H, dk, dv, 1);
        rc |= kda_oracle_prefill_f64(q + cut * H * dk, k + cut * H * dk, v + cut * H * dv,
                                     la + cut * H * dk, beta + cut * H, S1, o2, S2, 1, t1, H,
                                     dk, dv, 1);
        if (rc != 0) bad = 1;
        if (memcmp(S2, S, (size_t)ns * sizeof(double)) != 0) bad = 1;
        if (memcmp(o1, o, (size_t)cut * H * dv * sizeof(double)) != 0) bad = 1;
        if (memcmp(o2, o + cut * H * dv, (size_t)t1 * H * dv * sizeof(double)) != 0) bad = 1;
        free(S1); free(S2); free(o1); free(o2);
    }
    /* one decode step from the final state */
    if (T > 0) {
        double* Sd = fill(ns, 0, 0);
        memcpy(Sd, S, (size_t)ns * sizeof(double));
        double* od = fill(B * H * dv, 0, 0);
        rc = kda_oracle_decode_f64(q, k, v, la, beta, Sd, od, B, H, dk, dv, 2);
        if (rc != 0) bad = 1;
        free(Sd); free(od);
    }
    printf("B%ld T%ld H%ld dk%ld dv%ld s0=%d: %s\n", B, T, H, dk, dv, with_s0, bad ? "MISMATCH" : "ok");
    free(q); free(k); free(v); free(la); free(beta); free(S0); free(o); free(S);
    return bad;
}

int main(void) {
    int bad = 0;
    bad |= check(1, 37, 2, 8, 5, 1, 11);
    bad |= check(2, 16, 3, 16, 16, 0, 0);
    bad |= check(1, 0, 2, 4, 4, 1, 0);      /* no tokens: S_final = S0 */
    bad |= check(3, 1, 1, 3, 7, 1, 0);
    bad |= check(1, 64, 1, 32, 8, 0, 63);
    return bad;
}
