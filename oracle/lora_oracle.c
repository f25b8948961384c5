/*
 * lora_oracle.c -- plain, slow CPU fp64 oracle for the multi-LoRA adapter
 * execution unit.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no source, header, table or helper
 * with the HIP library; the two meet only through the seeded input
 * generators, which hold none of the method's arithmetic.
 *
 * What it computes (sources, by page title and section):
 *
 *  - The adapter execution unit multiplies the LoRA matrices onto the base
 *    hidden state: the base linear runs and the LoRA product is added as a
 *    residual ("LLM 多 LoRA 推理服务工程 2026", four-layer runtime, the
 *    paragraph on the adapter execution unit).
 *  - A maps hidden size to rank and B maps rank to hidden size (same page,
 *    routing layer, the paragraph on zero-padding lower ranks).
 *  - The scale alpha / rank, with the adapter's own (unpadded) rank, is the
 *    plainest reading of the per-token formula
 *        y = x W^T + (alpha / r) (x A^T) B^T
 *    that the adapter records carry (rank and alpha are stored per adapter:
 *    "Multi-LoRA 在线服务隔离", trusted registry section).
 *  - base_only tokens get the base output only ("xpshop.cn article 492",
 *    section 三, routing default base_only); a token whose adapter mapping is
 *    missing gets an explicit error, never a fallback ("Multi-LoRA 在线服务隔离",
 *    request identity section: default deny).
 *  - Routing groups the tokens of one call by adapter (two-level bucketing,
 *    "LLM 多 LoRA 推理服务工程 2026", routing layer); a bucket above a threshold
 *    is run fused, otherwise separate (same paragraph).
 *
 * Every sum runs in fp64 in ascending index order.  No blocking, no fusion,
 * no reordering.  Inputs arrive already converted to fp64 (the conversion from
 * fp32/fp16/bf16 to fp64 is exact and is done by the caller).
 *
 * Pins (not this file): tests/test_oracle_pins.py checks this oracle against
 * hand-worked examples under tests/golden/, closed forms (selection matrices,
 * one-hot adapters), exact rational arithmetic on tiny inputs, a library
 * matrix product for the base-only special case, a library stable sort for
 * routing, and the padding and linearity invariants.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>

/* Routing keys: an active adapter slot maps to itself, base_only (-1) maps to
 * S, and anything else (out of range, or a slot that is not active) maps to
 * S + 1, the invalid bucket. */
static int token_key(int32_t idx, int S, const int32_t *active)
{
    if (idx == -1)
        return S;
    if (idx >= 0 && idx < S && active[idx] != 0)
        return idx;
    return S + 1;
}

/* Segment modes and policies (same numbering as the library's public enum,
 * restated here; no header is shared). */
enum { MODE_NONE = 0, MODE_FUSED = 1, MODE_SEPARATE = 2 };
enum { POLICY_AUTO = 0, POLICY_FUSED = 1, POLICY_SEPARATE = 2 };

/*
 * oracle_route: counting sort of the tokens of one call by adapter key.
 *
 *   idx[T]          per-token adapter slot, -1 = base_only
 *   active[S]       1 if the slot holds a registered adapter
 *   policy, theta   AUTO: a LoRA bucket with more than theta tokens is FUSED,
 *                   otherwise SEPARATE; FUSED / SEPARATE force every bucket
 *   counts[S+2]     tokens per key
 *   offsets[S+3]    exclusive prefix sum of counts; offsets[S+2] = T
 *   perm[T]         perm[p] = token at sorted position p; ties keep ascending
 *                   token order (stable)
 *   segs[(S+2)*4]   one record {key, start, len, mode} per non-empty key,
 *                   keys ascending
 *   n_seg           number of records written
 *
 * Returns 0, or -1 if scratch memory cannot be had.
 */
int oracle_route(const int32_t *idx, int T, int S, const int32_t *active,
                 int policy, int theta,
                 int32_t *counts, int32_t *offsets, int32_t *perm,
                 int32_t *segs, int32_t *n_seg)
{
    const int nkeys = S + 2;
    int32_t *next = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nkeys > 0 ? nkeys : 1));
    if (next == NULL)
        return -1;

    for (int k = 0; k < nkeys; ++k)
        counts[k] = 0;
    for (int t = 0; t < T; ++t)
        counts[token_key(idx[t], S, active)] += 1;

    offsets[0] = 0;
    for (int k = 0; k < nkeys; ++k)
        offsets[k + 1] = offsets[k] + counts[k];

    for (int k = 0; k < nkeys; ++k)
        next[k] = offsets[k];
    for (int t = 0; t < T; ++t) {
        int k = token_key(idx[t], S, active);
        perm[next[k]] = t;
        next[k] += 1;
    }

    int n = 0;
    for (int k = 0; k < nkeys; ++k) {
        if (counts[k] == 0)
            continue;
        int mode;
        if (k >= S)
            mode = MODE_NONE;
        else if (policy == POLICY_FUSED)
            mode = MODE_FUSED;
        else if (policy == POLICY_SEPARATE)
            mode = MODE_SEPARATE;
        else
            mode = (counts[k] > theta) ? MODE_FUSED : MODE_SEPARATE;
        segs[4 * n + 0] = k;
        segs[4 * n + 1] = offsets[k];
        segs[4 * n + 2] = counts[k];
        segs[4 * n + 3] = mode;
        n += 1;
    }
    *n_seg = n;
    free(next);
    return 0;
}

/*
 * oracle_apply: the per-token formula, one token at a time.
 *
 *   x[T][d_in], W[d_out][d_in]          row-major fp64 (W in nn.Linear layout)
 *   idx[T]                              adapter slot per token, -1 = base_only
 *   active[S], rank[S], alpha[S]        slot table (rank = the adapter's own r)
 *   A_cat, a_off[S]                     slot i's A, [rank[i]][d_in], starts at
 *                                       A_cat + a_off[i]
 *   B_cat, b_off[S]                     slot i's B, [d_out][rank[i]], starts at
 *                                       B_cat + b_off[i]
 *   y[T][d_out]                         output; rows of invalid tokens are NaN
 *   invalid[T]                          1 for a token whose mapping is missing
 *   n_threads                           OpenMP threads over tokens (<= 0: all)
 *
 * Returns the number of invalid tokens, or -1 if scratch memory cannot be had.
 */
long oracle_apply(int T, int d_in, int d_out, int S,
                  const double *x, const double *W, const int32_t *idx,
                  const int32_t *active, const int32_t *rank, const double *alpha,
                  const double *A_cat, const int64_t *a_off,
                  const double *B_cat, const int64_t *b_off,
                  double *y, int32_t *invalid, int n_threads)
{
    long n_invalid = 0;
    int failed = 0;
    const int nt = (n_threads > 0) ? n_threads : omp_get_max_threads();

#pragma omp parallel for schedule(dynamic, 1) reduction(+ : n_invalid) reduction(| : failed) num_threads(nt)
    for (int t = 0; t < T; ++t) {
        const double *xt = x + (size_t)t * d_in;
        double *yt = y + (size_t)t * d_out;
        int32_t i = idx[t];
        int is_base_only = (i == -1);
        int is_valid = (i >= 0 && i < S && active[i] != 0);

        invalid[t] = 0;
        if (!is_base_only && !is_valid) {
            invalid[t] = 1;
            n_invalid += 1;
            for (int n = 0; n < d_out; ++n)
                yt[n] = NAN;
            continue;
        }

        /* base[n] = sum_k x[t][k] * W[n][k] */
        for (int n = 0; n < d_out; ++n) {
            const double *wn = W + (size_t)n * d_in;
            double acc = 0.0;
            for (int k = 0; k < d_in; ++k)
                acc += xt[k] * wn[k];
            yt[n] = acc;
        }
        if (is_base_only)
            continue;

        /* h[j] = sum_k x[t][k] * A_i[j][k],  j < r_i */
        const int r = rank[i];
        const double *Ai = A_cat + a_off[i];
        const double *Bi = B_cat + b_off[i];
        double *h = (double *)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
        if (h == NULL) {
            failed = 1;
            continue;
        }
        for (int j = 0; j < r; ++j) {
            const double *aj = Ai + (size_t)j * d_in;
            double acc = 0.0;
            for (int k = 0; k < d_in; ++k)
                acc += xt[k] * aj[k];
            h[j] = acc;
        }

        /* y[t][n] = base[n] + (alpha_i / r_i) * sum_j h[j] * B_i[n][j] */
        const double s = alpha[i] / (double)r;
        for (int n = 0; n < d_out; ++n) {
            const double *bn = Bi + (size_t)n * r;
            double d = 0.0;
            for (int j = 0; j < r; ++j)
                d += h[j] * bn[j];
            yt[n] = yt[n] + s * d;
        }
        free(h);
    }
    return failed ? -1 : n_invalid;
}
