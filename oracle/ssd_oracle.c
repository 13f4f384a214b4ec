/*
 * CPU oracle for the Mamba2 SSD varlen scan and the MTP selective state update.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * reference that the GPU library is checked against. Only the test suite, the
 * smoke entry point and the benchmark's CPU-baseline leg may build, load or
 * call it. The GPU library shares no code with it and never calls it.
 *
 * Arithmetic: float64 throughout, on the exact input values the GPU sees
 * (bf16 / fp32 inputs widened exactly by the Python caller).
 *
 * What it computes is the selective state-space recurrence, one token at a
 * time, per (sequence, head):
 *
 *     h_t = exp(dt_t * A_h) * h_{t-1} + dt_t * x_t (outer) B_t     h: [P x N]
 *     y_t = h_t . C_t + D_h * x_t                                 (sum over N)
 *
 * The pages name this recurrent state and its FP32 recurrence (vLLM PR
 * #52928 "[Mamba] Add FlashInfer ReplaySSM support for MTP", section
 * "Summary"; vLLM PR #62922, section "Details") without writing it out; the
 * formula is the standard Mamba2 selective SSM. Head h reads group
 * g = h / (H / G) of B and C.
 *
 * Varlen packing (vLLM PR #61501, section "Details": packed-varlen cu_seqlens;
 * chunk metadata per sequence): sequence s owns tokens cu[s] .. cu[s+1]-1 and
 * never sees another sequence's tokens. Its chunks of Q tokens start at its
 * first token; the last one may be partial. The oracle has no chunking in its
 * arithmetic: chunk size only decides where checkpoint states are recorded
 * (the exit state of every chunk, used by prefix caching, vLLM PR #61501,
 * section "Details", "Prefills that store Mamba checkpoints need every chunk
 * state").
 *
 * Cache slots, snapshot semantics and rounding to storage dtypes are done by
 * the Python wrapper around these functions (oracle/__init__.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of chunks of sequence with `len` tokens at chunk size Q. */
static int64_t n_chunks(int64_t len, int64_t Q) { return (len + Q - 1) / Q; }

/*
 * Prefill over a packed varlen batch.
 *
 *   x [T,H,P], dt [T,H], A [H], B [T,G,N], C [T,G,N], D [H] or NULL (= 0)
 *   cu_seqlens [S+1] (int32, cu[0] = 0, non-decreasing, cu[S] = T)
 *   init [S,H,P,N] or NULL; has_init [S] (uint8) or NULL (NULL = all from zero
 *     when init is NULL, all from init when init is given)
 *   y [T,H,P] out; final_state [S,H,P,N] out
 *   ckpt [nc,H,P,N] out or NULL: row chunk_cu[s] + k holds the state after the
 *     last token of chunk k of sequence s, chunk_cu = exclusive prefix sum of
 *     ceil(L_s / Q).
 *
 * Returns 0, or -1 on a bad argument.
 */
int ssd_oracle_prefill(int64_t T, int64_t S, int64_t H, int64_t P, int64_t N, int64_t G, int64_t Q,
                       const double *x, const double *dt, const double *A, const double *B,
                       const double *C, const double *D, const int32_t *cu_seqlens,
                       const double *init, const uint8_t *has_init, double *y,
                       double *final_state, double *ckpt, int nthreads)
{
    if (T < 0 || S < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || Q <= 0 || H % G != 0)
        return -1;
    if (cu_seqlens[0] != 0 || cu_seqlens[S] != T)
        return -1;
    for (int64_t s = 0; s < S; ++s)
        if (cu_seqlens[s + 1] < cu_seqlens[s])
            return -1;

    int64_t *chunk_cu = (int64_t *)malloc(sizeof(int64_t) * (size_t)(S + 1));
    if (!chunk_cu)
        return -1;
    chunk_cu[0] = 0;
    for (int64_t s = 0; s < S; ++s)
        chunk_cu[s + 1] = chunk_cu[s] + n_chunks(cu_seqlens[s + 1] - cu_seqlens[s], Q);

    const int64_t heads_per_group = H / G;
    const int64_t PN = P * N;
    const int64_t pairs = S * H;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *h = (double *)malloc(sizeof(double) * (size_t)PN);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t pair = 0; pair < pairs; ++pair) {
            const int64_t s = pair / H, hd = pair % H, g = hd / heads_per_group;
            const int64_t t0 = cu_seqlens[s], len = cu_seqlens[s + 1] - t0;
            const int use_init = init != NULL && (has_init == NULL || has_init[s] != 0);

            if (use_init)
                memcpy(h, init + (s * H + hd) * PN, sizeof(double) * (size_t)PN);
            else
                for (int64_t e = 0; e < PN; ++e)
                    h[e] = 0.0;

            const double Ah = A[hd];
            const double Dh = D ? D[hd] : 0.0;
            for (int64_t k = 0; k < len; ++k) {
                const int64_t t = t0 + k;
                const double dtt = dt[t * H + hd];
                const double decay = exp(dtt * Ah);
                const double *xt = x + (t * H + hd) * P;
                const double *Bt = B + (t * G + g) * N;
                const double *Ct = C + (t * G + g) * N;
                double *yt = y + (t * H + hd) * P;
                for (int64_t p = 0; p < P; ++p) {
                    double *hp = h + p * N;
                    const double u = dtt * xt[p];
                    for (int64_t n = 0; n < N; ++n)
                        hp[n] = decay * hp[n] + u * Bt[n];
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n)
                        acc += Ct[n] * hp[n];
                    yt[p] = acc + Dh * xt[p];
                }
                if (ckpt && ((k + 1) % Q == 0 || k + 1 == len)) {
                    const int64_t row = chunk_cu[s] + k / Q;
                    memcpy(ckpt + (row * H + hd) * PN, h, sizeof(double) * (size_t)PN);
                }
            }
            memcpy(final_state + (s * H + hd) * PN, h, sizeof(double) * (size_t)PN);
        }
        free(h);
    }
    free(chunk_cu);
    return 0;
}

/*
 * Decode / MTP verify state update: R requests with T tokens each, the same
 * recurrence continued from each request's initial state (vLLM PR #52928,
 * section "Summary": one target token plus several draft tokens per request;
 * section "Design": (batch, tokens, ...) inputs).
 *
 *   init [R,H,P,N]; x [R,T,H,P]; dt [R,T,H]; A [H]; B, C [R,T,G,N]; D [H] or NULL
 *   y [R,T,H,P] out
 *   states [R,T,H,P,N] out or NULL: the state after token t of request r, the
 *     per-draft-token intermediate state a rollback to t accepted drafts uses.
 *   final_state [R,H,P,N] out or NULL: the state after all T tokens.
 */
int ssd_oracle_state_update(int64_t R, int64_t T, int64_t H, int64_t P, int64_t N, int64_t G,
                            const double *init, const double *x, const double *dt,
                            const double *A, const double *B, const double *C, const double *D,
                            double *y, double *states, double *final_state, int nthreads)
{
    if (R < 0 || T < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0)
        return -1;
    const int64_t heads_per_group = H / G;
    const int64_t PN = P * N;
    const int64_t pairs = R * H;

#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
    {
        double *h = (double *)malloc(sizeof(double) * (size_t)PN);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t pair = 0; pair < pairs; ++pair) {
            const int64_t r = pair / H, hd = pair % H, g = hd / heads_per_group;
            memcpy(h, init + (r * H + hd) * PN, sizeof(double) * (size_t)PN);
            const double Ah = A[hd];
            const double Dh = D ? D[hd] : 0.0;
            for (int64_t t = 0; t < T; ++t) {
                const int64_t rt = r * T + t;
                const double dtt = dt[rt * H + hd];
                const double decay = exp(dtt * Ah);
                const double *xt = x + (rt * H + hd) * P;
                const double *Bt = B + (rt * G + g) * N;
                const double *Ct = C + (rt * G + g) * N;
                double *yt = y + (rt * H + hd) * P;
                for (int64_t p = 0; p < P; ++p) {
                    double *hp = h + p * N;
                    const double u = dtt * xt[p];
                    for (int64_t n = 0; n < N; ++n)
                        hp[n] = decay * hp[n] + u * Bt[n];
                    double acc = 0.0;
                    for (int64_t n = 0; n < N; ++n)
                        acc += Ct[n] * hp[n];
                    yt[p] = acc + Dh * xt[p];
                }
                if (states)
                    memcpy(states + (rt * H + hd) * PN, h, sizeof(double) * (size_t)PN);
            }
            if (final_state)
                memcpy(final_state + (r * H + hd) * PN, h, sizeof(double) * (size_t)PN);
        }
        free(h);
    }
    return 0;
}

int ssd_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
