/*
 * CPU oracle for the Mamba-2 SSD selective scan -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  It shares no code, header, table or helper with the
 * GPU library, and the GPU library never calls it.
 *
 * What it computes (plain fp64, one token at a time, no chunking):
 *   "Engineering hybrid state-space models" (innvotechnologies blog), section 2
 *   ("Mathematical Formalization"): the per-token recurrence h_t = Abar_t h_{t-1}
 *   + Bbar_t x_t, y_t = C_t h_t, with Abar_t = exp(Delta_t A).  Mamba-2 keeps A
 *   scalar per head ("Compiler-First State Space Duality...", abstract:
 *   "diagonal per-head dynamics"), so for head h with group g:
 *       a        = exp(dt[t,h] * A[h])
 *       S[p][n]  = a * S[p][n] + (dt[t,h] * x[t,h,p]) * B[t,g,n]
 *       y[t,h,p] = sum_n S[p][n] * C[t,g,n]  +  D[h] * x[t,h,p]
 *   The input term uses Bbar_t x_t = dt_t * B_t * x_t (the Euler form that the
 *   blog's TypeScript decode step, section 4, also uses: bBar = delta * x),
 *   and D is the scalar skip term of the continuous SSM (lesty.tech Mamba
 *   explainer, section 2).  y uses the state AFTER token t is absorbed.
 *   The state layout is (batch, heads, head_dim, state_dim), as the blog's
 *   section 3 "Fixed Memory State Buffering" gives it.
 *
 * Layouts (row-major, innermost last), all fp64:
 *   x [T,H,P], dt [T,H], A [H], B,C [T,G,N], D [H],
 *   init/final [nseq,H,P,N]; sequence s owns tokens [cu[s], cu[s+1]).
 *   Head h uses group g = h / (H/G).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int ssd_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One (sequence, head) pair, token by token. S is P*N scratch. */
static void run_sequence_head(int64_t t0, int64_t t1, int32_t h, int32_t H, int32_t P,
                              int32_t N, int32_t G, const double* x, const double* dt,
                              const double* A, const double* B, const double* C,
                              const double* D, double* S, double* y) {
    const int32_t g = h / (H / G);
    for (int64_t t = t0; t < t1; ++t) {
        const double d = dt[t * H + h];
        const double a = exp(d * A[h]);
        const double* xt = x + (t * H + h) * (int64_t)P;
        const double* Bt = B + (t * G + g) * (int64_t)N;
        const double* Ct = C + (t * G + g) * (int64_t)N;
        double* yt = y + (t * H + h) * (int64_t)P;
        for (int32_t p = 0; p < P; ++p) {
            double* Sp = S + (int64_t)p * N;
            const double u = d * xt[p];
            double acc = 0.0;
            for (int32_t n = 0; n < N; ++n) {
                Sp[n] = a * Sp[n] + u * Bt[n];
                acc += Sp[n] * Ct[n];
            }
            yt[p] = acc + D[h] * xt[p];
        }
    }
}

/*
 * Prefill: y for every token of every sequence and the state after each
 * sequence's last token.  init == NULL means zero initial states;
 * final_state == NULL means it is not written.  Returns 0, or -1 on a bad
 * argument (G not dividing H, decreasing cu).
 */
int ssd_oracle_scan(int64_t nseq, const int64_t* cu, int32_t H, int32_t P, int32_t N,
                    int32_t G, const double* x, const double* dt, const double* A,
                    const double* B, const double* C, const double* D, const double* init,
                    double* y, double* final_state, int32_t nthreads) {
    if (nseq < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return -1;
    for (int64_t s = 0; s < nseq; ++s)
        if (cu[s + 1] < cu[s]) return -1;
    const int64_t pairs = nseq * (int64_t)H;
    const int64_t state_elems = (int64_t)P * N;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
#endif
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)state_elems);
        if (!S) bad = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t i = 0; i < pairs; ++i) {
            if (!S) continue;
            const int64_t s = i / H;
            const int32_t h = (int32_t)(i % H);
            const int64_t off = (s * H + h) * state_elems;
            if (init)
                memcpy(S, init + off, sizeof(double) * (size_t)state_elems);
            else
                memset(S, 0, sizeof(double) * (size_t)state_elems);
            run_sequence_head(cu[s], cu[s + 1], h, H, P, N, G, x, dt, A, B, C, D, S, y);
            if (final_state) memcpy(final_state + off, S, sizeof(double) * (size_t)state_elems);
        }
        free(S);
    }
    (void)nthreads;
    return bad ? -1 : 0;
}

/*
 * Cached decode: one step of the same recurrence applied to a stored state,
 * in place ("Compiler-First State Space Duality...", abstract: O(1) cached
 * decode).  state [batch,H,P,N], x [batch,H,P], dt [batch,H], B,C [batch,G,N],
 * y [batch,H,P].
 */
int ssd_oracle_decode(int64_t batch, int32_t H, int32_t P, int32_t N, int32_t G,
                      double* state, const double* x, const double* dt, const double* A,
                      const double* B, const double* C, const double* D, double* y,
                      int32_t nthreads) {
    if (batch < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return -1;
    const int64_t pairs = batch * (int64_t)H;
    const int64_t state_elems = (int64_t)P * N;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for num_threads(nthreads) schedule(static)
#endif
    for (int64_t i = 0; i < pairs; ++i) {
        const int64_t b = i / H;
        const int32_t h = (int32_t)(i % H);
        /* A decode step is the recurrence body for a single token: treat the
         * batch row as a one-token sequence whose state lives in `state`. */
        run_sequence_head(b, b + 1, h, H, P, N, G, x, dt, A, B, C, D,
                          state + (b * H + h) * state_elems, y);
    }
    (void)nthreads;
    return 0;
}
