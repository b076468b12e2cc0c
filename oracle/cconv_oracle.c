/*
 * cconv_oracle.c -- CPU oracle for the depthwise causal short convolution fused with SiLU.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg may load this library. The product path (the HIP library) never links,
 * loads or calls it, and the two share no code.
 *
 * Plain, slow, obviously correct loops written from the definitions, one output element at a
 * time. The same source is compiled twice: ORACLE_REAL=double (the reference values the GPU
 * is compared against) and ORACLE_REAL=float (the fp32 oracle). Every input value is exactly
 * representable in fp32 (bf16 activations and state, bf16 or fp32 taps, fp32 bias), so inputs
 * are passed as float arrays and widened to `real` on use. No FMA contraction (built with
 * -ffp-contract=off), no fast-math.
 *
 * Definitions (sources are the three pages on this op):
 *  - Tap order. [kernel-fun 0.2.0.dev1 wheel, strip.py, `_tap`]: the weight that multiplies
 *    x[t-k] is w[:, W-1-k]. Equivalently z[t] = bias + sum_j w[d, j] * X[t-(W-1)+j].
 *  - Zero history. [strip.py, `_ld_ring` and the backward's note on rows past T]: rows left
 *    of the sequence start read as zero; rows at or past T contribute nothing.
 *  - SiLU and its derivative. [strip.py, `_silu`, `_dsilu`]: y = z*sigma(z);
 *    g = dy * s * (1 + z*(1 - s)) with s = sigma(z). sigma(z) = 1/(1+exp(-z)) is written
 *    from its definition, not from the page's tanh approximation.
 *  - Backward. [strip.py, `_bwd4` docstring]: dx[u] = sum_k w'[k] g[u+k] with
 *    w'[k] = w[:, W-1-k]; dw is the sum over batch and time of g[t] * x[t-k] into column
 *    W-1-k ([strip.py, partial-store comment]); dw and dbias are plain sums over every (b, t)
 *    (the host `cconv_bwd` in strip.py sums the partials deterministically, with no atomics).
 *  - Bias. Present in fla's parameter list ([kernel-fun wheel, _common/compat.py, FLA_KWARGS
 *    row for causal_conv1d]) and in the decode API ([cudnn-frontend PR #797 "Add experimental
 *    causal conv1d decode update", PR description, API]); read as added to z before SiLU, so
 *    dbias = sum g.
 *  - History. [kernel-fun wheel, _common/compat.py: fla's initial_state and
 *    output_final_state]: an optional h0 [B, D, W-1], oldest first (the decode state layout),
 *    replaces the zero history before t = 0; the final state is the last W-1 values of the
 *    extended sequence; the history's gradient is dx at the W-1 virtual rows before t = 0.
 *  - Epilogue. [kernel-fun wheel, _common/compat.py: fla's activation and residual]: without an
 *    activation y = z (and g = dy); a residual is added to the output after the activation.
 *  - Packed batches. [kernel-fun wheel, _common/compat.py: fla's cu_seqlens]: sequences of
 *    different lengths packed along time; offsets cu[0] = 0 <= cu[1] <= ... <= cu[n] = total
 *    mark sequence i as rows cu[i] .. cu[i+1]-1; every sequence has its own zero (or given)
 *    history and nothing crosses a boundary.
 *  - Prefill into the decode pool. [PR #797 discussion: the follow-up's direct
 *    full-sequence-to-decode state handoff]: the history and final state of sequence b live
 *    in slot state_indices[b] of the decode state pool, under the decode slot rule.
 *  - Decode variants. [PR #797 description, API]: conv_state [S, D, L] with L in {3, 4} for
 *    W = 4, i.e. L = W-1 or W; optional cache_seqlens circular-buffer metadata (reserved there,
 *    read here as: entry c mod L takes the new token, entry (c-k) mod L holds the token k
 *    steps back).
 *  - Decode. [PR #797 description, API and semantics]: advance a per-slot state of the last
 *    W-1 inputs by one token; conv_state_indices picks the slot, -1 marks a padding row that
 *    mutates nothing; invalid indices fail closed. Readings: state is stored oldest first
 *    (for the token t being added, state[s, d, j] holds X[t-(W-1)+j]), so w[:, j] pairs
 *    with state[:, j] and w[:, W-1] with the new token; a padding row's output is 0;
 *    NULL indices mean slot n for row n; any index outside [-1, S) or a repeated non-negative
 *    index makes the whole call invalid and nothing is written.
 *
 * Parity pins for every function here live in tests/test_oracle_pins.py (finite
 * differences, a library convolution with autograd, an impulse, closed forms, decode ==
 * forward, W padding). Parity unpinned: nothing beyond the last-ulp behaviour of exp().
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_REAL
#define ORACLE_REAL double
#endif
typedef ORACLE_REAL real;

#define ORACLE_IS_FLOAT (sizeof(real) == sizeof(float))

static real r_exp(real v) { return ORACLE_IS_FLOAT ? (real)expf((float)v) : (real)exp((double)v); }

/* sigma(z) = 1 / (1 + e^-z), written from the definition. */
static real sigmoid(real z) { return (real)1 / ((real)1 + r_exp(-z)); }

/* X[b, t, d]: the input for 0 <= t < T; before t = 0 the history h0[b, d, t + W - 1] (oldest
 * first) when h0 is given, else zero; zero at or past T. */
static real xval(const float* x, const float* h0, int64_t T, int64_t D, int W, int64_t b, int64_t t, int64_t d) {
    if (t >= T) return 0;
    if (t >= 0) return (real)x[(b * T + t) * D + d];
    if (h0 && t >= -(int64_t)(W - 1)) return (real)h0[(b * D + d) * (W - 1) + (t + W - 1)];
    return 0;
}

/* z[b, t, d] = bias[d] + sum_{j=0}^{W-1} w[d, j] * X[b, t-(W-1)+j, d]  (oldest tap first). */
static real z_at(const float* x, const float* h0, int64_t T, int64_t D, const float* w, int W, const float* bias,
                 int64_t b, int64_t t, int64_t d) {
    real z = bias ? (real)bias[d] : (real)0;
    for (int j = 0; j < W; ++j) z = z + (real)w[d * W + j] * xval(x, h0, T, D, W, b, t - (W - 1) + j, d);
    return z;
}

/* g[b, t, d] = dy * dy/dz: with SiLU (act = 1) dy * s * (1 + z*(1-s)), s = sigma(z); without an
 * activation (act = 0, y = z) dy itself; zero outside 0 <= t < T. */
static real g_at(const float* x, const float* h0, const float* dy, int64_t T, int64_t D, const float* w, int W,
                 const float* bias, int64_t b, int64_t t, int64_t d, int act) {
    if (t < 0 || t >= T) return 0;
    real z = z_at(x, h0, T, D, w, W, bias, b, t, d);
    if (!act) return (real)dy[(b * T + t) * D + d];
    real s = sigmoid(z);
    return (real)dy[(b * T + t) * D + d] * s * ((real)1 + z * ((real)1 - s));
}

/* dx[b, u, d] = sum_{j=0}^{W-1} w[d, j] * g[b, u+(W-1)-j, d]; for -(W-1) <= u < 0 this is the
 * gradient of the history value at u (the initial state's gradient). */
static real dx_at(const float* x, const float* h0, const float* dy, int64_t T, int64_t D, const float* w, int W,
                  const float* bias, int64_t b, int64_t u, int64_t d, int act) {
    real acc = 0;
    for (int j = 0; j < W; ++j)
        acc = acc + (real)w[d * W + j] * g_at(x, h0, dy, T, D, w, W, bias, b, u + (W - 1) - j, d, act);
    return acc;
}

/* dw[d, j] = sum_b sum_t g[b, t, d] * X[b, t-(W-1)+j, d]. */
static real dw_at(const float* x, const float* h0, const float* dy, int64_t B, int64_t T, int64_t D,
                  const float* w, int W, const float* bias, int64_t d, int j, int act) {
    real acc = 0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t)
            acc = acc + g_at(x, h0, dy, T, D, w, W, bias, b, t, d, act) * xval(x, h0, T, D, W, b, t - (W - 1) + j, d);
    return acc;
}

/* dbias[d] = sum_b sum_t g[b, t, d]. */
static real dbias_at(const float* x, const float* h0, const float* dy, int64_t B, int64_t T, int64_t D,
                     const float* w, int W, const float* bias, int64_t d, int act) {
    real acc = 0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t) acc = acc + g_at(x, h0, dy, T, D, w, W, bias, b, t, d, act);
    return acc;
}

/* ---------------------------------------------------------------------------------------- */
/* Exported entry points. Arrays are contiguous: x, dy, z, y, dx are [B, T, D]; w is [D, W];  */
/* bias and dbias are [D] (bias may be NULL); dw is [D, W]. Outputs are unrounded `real`.     */
/* OpenMP only spreads independent output elements over threads; every element is computed  */
/* by one thread in the fixed order above, so results do not depend on the thread count.    */
/* ---------------------------------------------------------------------------------------- */

int oracle_real_bytes(void) { return (int)sizeof(real); }

int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (the CPU baseline's one-thread figure); results do not
 * depend on it. */
void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Forward: z (optional) and y = z * sigma(z) for every element. */
void oracle_fwd(const float* x, int64_t B, int64_t T, int64_t D, const float* w, int W,
                const float* bias, real* z_out, real* y_out) {
    int64_t rows = B * T;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / T, t = r % T;
        for (int64_t d = 0; d < D; ++d) {
            real z = z_at(x, NULL, T, D, w, W, bias, b, t, d);
            if (z_out) z_out[r * D + d] = z;
            y_out[r * D + d] = z * sigmoid(z);
        }
    }
}

/* Backward: dx for every element, dw [D, W] and dbias [D] (dbias may be NULL). */
void oracle_bwd(const float* x, const float* dy, int64_t B, int64_t T, int64_t D, const float* w,
                int W, const float* bias, real* dx_out, real* dw_out, real* dbias_out) {
    int64_t rows = B * T;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / T, u = r % T;
        for (int64_t d = 0; d < D; ++d) dx_out[r * D + d] = dx_at(x, NULL, dy, T, D, w, W, bias, b, u, d, 1);
    }
#pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < D; ++d) {
        for (int j = 0; j < W; ++j) dw_out[d * W + j] = dw_at(x, NULL, dy, B, T, D, w, W, bias, d, j, 1);
        if (dbias_out) dbias_out[d] = dbias_at(x, NULL, dy, B, T, D, w, W, bias, d, 1);
    }
}

/* Sampled forward: y at n listed (b, t, d) points of a full-size problem. */
void oracle_fwd_points(const float* x, int64_t B, int64_t T, int64_t D, const float* w, int W,
                       const float* bias, int64_t n, const int64_t* pb, const int64_t* pt,
                       const int64_t* pd, real* y_out) {
    (void)B;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        real z = z_at(x, NULL, T, D, w, W, bias, pb[i], pt[i], pd[i]);
        y_out[i] = z * sigmoid(z);
    }
}

/* Sampled backward: dx at n listed (b, u, d) points. */
void oracle_dx_points(const float* x, const float* dy, int64_t B, int64_t T, int64_t D,
                      const float* w, int W, const float* bias, int64_t n, const int64_t* pb,
                      const int64_t* pu, const int64_t* pd, real* dx_out) {
    (void)B;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) dx_out[i] = dx_at(x, NULL, dy, T, D, w, W, bias, pb[i], pu[i], pd[i], 1);
}

/* Sampled weight gradient: dw[d, :] and dbias[d] for n listed channels (full sums). */
void oracle_dw_channels(const float* x, const float* dy, int64_t B, int64_t T, int64_t D,
                        const float* w, int W, const float* bias, int64_t n, const int64_t* pd,
                        real* dw_out /* [n, W] */, real* dbias_out /* [n] */) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        for (int j = 0; j < W; ++j) dw_out[i * W + j] = dw_at(x, NULL, dy, B, T, D, w, W, bias, pd[i], j, 1);
        dbias_out[i] = dbias_at(x, NULL, dy, B, T, D, w, W, bias, pd[i], 1);
    }
}

/*
 * Forward with a history [kernel-fun wheel, _common/compat.py: fla's initial_state and
 * output_final_state parameters]: h0 [B, D, W-1] (oldest first, NULL = zeros) is the input
 * before t = 0; hT [B, D, W-1] (may be NULL) receives the last W-1 values of the extended
 * sequence (history then x), i.e. the state a decode update continues from.
 */
void oracle_fwd_state(const float* x, const float* h0, int64_t B, int64_t T, int64_t D, const float* w, int W,
                      const float* bias, real* y_out, float* hT_out) {
    int64_t rows = B * T;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / T, t = r % T;
        for (int64_t d = 0; d < D; ++d) {
            real z = z_at(x, h0, T, D, w, W, bias, b, t, d);
            y_out[r * D + d] = z * sigmoid(z);
        }
    }
    if (hT_out)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t d = 0; d < D; ++d)
                for (int j = 0; j < W - 1; ++j)
                    hT_out[(b * D + d) * (W - 1) + j] = (float)xval(x, h0, T, D, W, b, T - (W - 1) + j, d);
}

/* Backward with a history: dx, dw, dbias as oracle_bwd with X extended by h0, and dh0 [B, D,
 * W-1] (may be NULL): the gradient of each history value, dx at u = -(W-1) .. -1. */
void oracle_bwd_state(const float* x, const float* h0, const float* dy, int64_t B, int64_t T, int64_t D,
                      const float* w, int W, const float* bias, real* dx_out, real* dw_out, real* dbias_out,
                      real* dh0_out) {
    int64_t rows = B * T;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / T, u = r % T;
        for (int64_t d = 0; d < D; ++d) dx_out[r * D + d] = dx_at(x, h0, dy, T, D, w, W, bias, b, u, d, 1);
    }
#pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < D; ++d) {
        for (int j = 0; j < W; ++j) dw_out[d * W + j] = dw_at(x, h0, dy, B, T, D, w, W, bias, d, j, 1);
        if (dbias_out) dbias_out[d] = dbias_at(x, h0, dy, B, T, D, w, W, bias, d, 1);
    }
    if (dh0_out)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t d = 0; d < D; ++d)
                for (int j = 0; j < W - 1; ++j)
                    dh0_out[(b * D + d) * (W - 1) + j] = dx_at(x, h0, dy, T, D, w, W, bias, b, -(int64_t)(W - 1) + j, d, 1);
}

/* The epilogue variants of fla's parameter list: act = 0 drops the activation (y = z, so g = dy);
 * a residual r [B, T, D] (NULL: none) is added to the output after the activation (its own
 * gradient is dy, nothing to compute). History h0 as in oracle_fwd_state. */
void oracle_fwd_epi(const float* x, const float* h0, const float* r, int act, int64_t B, int64_t T, int64_t D,
                    const float* w, int W, const float* bias, real* y_out) {
    int64_t rows = B * T;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < rows; ++q) {
        int64_t b = q / T, t = q % T;
        for (int64_t d = 0; d < D; ++d) {
            real z = z_at(x, h0, T, D, w, W, bias, b, t, d);
            real y = act ? z * sigmoid(z) : z;
            if (r) y = y + (real)r[q * D + d];
            y_out[q * D + d] = y;
        }
    }
}

void oracle_bwd_epi(const float* x, const float* h0, const float* dy, int act, int64_t B, int64_t T, int64_t D,
                    const float* w, int W, const float* bias, real* dx_out, real* dw_out, real* dbias_out,
                    real* dh0_out) {
    int64_t rows = B * T;
#pragma omp parallel for schedule(static)
    for (int64_t q = 0; q < rows; ++q) {
        int64_t b = q / T, u = q % T;
        for (int64_t d = 0; d < D; ++d) dx_out[q * D + d] = dx_at(x, h0, dy, T, D, w, W, bias, b, u, d, act);
    }
#pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < D; ++d) {
        for (int j = 0; j < W; ++j) dw_out[d * W + j] = dw_at(x, h0, dy, B, T, D, w, W, bias, d, j, act);
        if (dbias_out) dbias_out[d] = dbias_at(x, h0, dy, B, T, D, w, W, bias, d, act);
    }
    if (dh0_out)
        for (int64_t b = 0; b < B; ++b)
            for (int64_t d = 0; d < D; ++d)
                for (int j = 0; j < W - 1; ++j)
                    dh0_out[(b * D + d) * (W - 1) + j] =
                        dx_at(x, h0, dy, T, D, w, W, bias, b, -(int64_t)(W - 1) + j, d, act);
}

/*
 * Decode update [PR #797 description, API and semantics]. x: [N, D]; state: [S, D, W-1]
 * (in/out, oldest first); idx: [N] or NULL (row n uses slot n, which needs N <= S);
 * y_out: [N, D]. Returns 0 on success, 1 when the indices are invalid (then nothing is
 * written: neither state nor y). For W == 1 the state holds nothing and is not touched.
 */
/* The packed-batch rule: offsets start at 0, never decrease and end at the row count. */
static int offsets_valid(const int32_t* cu, int64_t n, int64_t total) {
    if (cu[0] != 0 || (int64_t)cu[n] != total) return 0;
    for (int64_t i = 0; i < n; ++i)
        if (cu[i] > cu[i + 1]) return 0;
    return 1;
}

/* A packed batch: sequence i is rows cu[i] .. cu[i+1]-1 of x [total, D], with its own history
 * h0[i] (h0 NULL: zeros) and final state hT[i] (NULL: not wanted), both [n, D, W-1]. Each
 * sequence is the forward of a [1, len, D] batch on its own; nothing crosses a boundary. An
 * empty sequence's final state is its history. Offsets that break the rule: returns 1 and
 * writes nothing. */
int oracle_fwd_varlen(const float* x, const int32_t* cu, int64_t n, int64_t total, int64_t D, const float* w,
                      int W, const float* bias, const float* h0, real* y_out, float* hT_out) {
    const int64_t L = W - 1;
    if (!offsets_valid(cu, n, total)) return 1;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t a = cu[i], len = (int64_t)cu[i + 1] - cu[i];
        oracle_fwd_state(x + a * D, h0 ? h0 + i * D * L : NULL, 1, len, D, w, W, bias, y_out + a * D,
                         hT_out ? hT_out + i * D * L : NULL);
    }
    return 0;
}

/* Backward of the packed batch: dx and the history gradient per sequence, dw and dbias summed
 * over the sequences in order. Same offset rule and return value as the forward. */
int oracle_bwd_varlen(const float* x, const float* dy, const int32_t* cu, int64_t n, int64_t total, int64_t D,
                      const float* w, int W, const float* bias, const float* h0, real* dx_out, real* dw_out,
                      real* dbias_out, real* dh0_out) {
    const int64_t L = W - 1;
    if (!offsets_valid(cu, n, total)) return 1;
    real* dwi = (real*)calloc((size_t)(D * W), sizeof(real));
    real* dbi = (real*)calloc((size_t)(D > 0 ? D : 1), sizeof(real));
    if (!dwi || !dbi) {
        free(dwi);
        free(dbi);
        return 2;
    }
    for (int64_t e = 0; e < D * W; ++e) dw_out[e] = 0;
    if (dbias_out)
        for (int64_t d = 0; d < D; ++d) dbias_out[d] = 0;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t a = cu[i], len = (int64_t)cu[i + 1] - cu[i];
        oracle_bwd_state(x + a * D, h0 ? h0 + i * D * L : NULL, dy + a * D, 1, len, D, w, W, bias, dx_out + a * D,
                         dwi, dbi, dh0_out ? dh0_out + i * D * L : NULL);
        for (int64_t e = 0; e < D * W; ++e) dw_out[e] = dw_out[e] + dwi[e];
        if (dbias_out)
            for (int64_t d = 0; d < D; ++d) dbias_out[d] = dbias_out[d] + dbi[d];
    }
    free(dwi);
    free(dbi);
    return 0;
}

/* The decode API's slot rule: every index in [-1, S) and no non-negative slot named twice. */
static int slots_valid(const int32_t* idx, int64_t N, int64_t S) {
    for (int64_t n = 0; n < N; ++n)
        if (idx[n] < -1 || idx[n] >= S) return 0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < n; ++m)
            if (idx[n] >= 0 && idx[n] == idx[m]) return 0;
    return 1;
}

/* Prefill straight into a decode state pool [S, D, W-1]: sequence b reads its history from
 * slot idx[b] when has_init[b] is set (zeros otherwise, and always for idx[b] = -1), and its
 * final state replaces that slot (idx[b] = -1: nothing written). The slot rule is the decode
 * one; a call that breaks it writes nothing (neither y nor state) and returns 1. */
int oracle_fwd_pool(const float* x, int64_t B, int64_t T, int64_t D, const float* w, int W, const float* bias,
                    float* state, int64_t S, const int32_t* idx, const uint8_t* has_init, real* y_out) {
    const int64_t L = W - 1;
    if (!slots_valid(idx, B, S)) return 1;
    float* h0 = (float*)calloc((size_t)(B * D * (L > 0 ? L : 1)), sizeof(float));
    float* hT = (float*)calloc((size_t)(B * D * (L > 0 ? L : 1)), sizeof(float));
    if (!h0 || !hT) {
        free(h0);
        free(hT);
        return 2;
    }
    for (int64_t b = 0; b < B; ++b)
        if (idx[b] >= 0 && has_init && has_init[b])
            memcpy(h0 + b * D * L, state + (int64_t)idx[b] * D * L, (size_t)(D * L) * sizeof(float));
    oracle_fwd_state(x, h0, B, T, D, w, W, bias, y_out, hT);
    for (int64_t b = 0; b < B; ++b)
        if (idx[b] >= 0) memcpy(state + (int64_t)idx[b] * D * L, hT + b * D * L, (size_t)(D * L) * sizeof(float));
    free(h0);
    free(hT);
    return 0;
}

int oracle_update(const float* x, int64_t N, int64_t D, float* state, int64_t S,
                  const int32_t* idx, const float* w, int W, const float* bias, real* y_out) {
    const int64_t L = W - 1;
    /* Validity first, so that an invalid call writes nothing. */
    if (!idx && N > S) return 1;
    if (idx && !slots_valid(idx, N, S)) return 1;
    for (int64_t n = 0; n < N; ++n) {
        int64_t s = idx ? (int64_t)idx[n] : n;
        if (s < 0) {
            for (int64_t d = 0; d < D; ++d) y_out[n * D + d] = 0;
            continue;
        }
        for (int64_t d = 0; d < D; ++d) {
            float* st = state + (s * D + d) * L;
            real z = bias ? (real)bias[d] : (real)0;
            for (int64_t j = 0; j < L; ++j) z = z + (real)w[d * W + j] * (real)st[j];
            z = z + (real)w[d * W + (W - 1)] * (real)x[n * D + d];
            y_out[n * D + d] = z * sigmoid(z);
            /* shift: drop the oldest, append the new token (plain value copies) */
            for (int64_t j = 0; j + 1 < L; ++j) st[j] = st[j + 1];
            if (L > 0) st[L - 1] = x[n * D + d];
        }
    }
    return 0;
}

/*
 * Round to bf16, nearest-even [strip.py, `_st`: downcast with rtne]. Written from the
 * definition: the value is scaled so that bf16's 8 significant bits are the integer part,
 * rounded half-to-even (nearbyint under the default rounding mode), and scaled back.
 * Subnormal bf16 values share fp32's minimum exponent (-126), so their quantum is 2^-133.
 */
/* The decode variants: a state of L entries per channel (L = W-1 or W; with L = W the oldest
 * entry is carried but not used), updated by a shift (drop the oldest, append the token), or,
 * with cache_seqlens, as a circular buffer: for row n with c = cache_seqlens[n], the token k
 * steps back sits in entry (c - k) mod L and the new token is written to entry c mod L, nothing
 * else moves. Validity: the slot rule, every cache_seqlens entry >= 0, L >= 1 in circular mode;
 * an invalid call writes nothing and returns 1. */
int oracle_update_ex(const float* x, int64_t N, int64_t D, float* state, int64_t S, int L, const int32_t* idx,
                     const int32_t* cache_seqlens, const float* w, int W, const float* bias, real* y_out) {
    if (L != W - 1 && L != W) return 1;
    if (cache_seqlens && L < 1) return 1;
    if (!idx && N > S) return 1;
    if (idx && !slots_valid(idx, N, S)) return 1;
    if (cache_seqlens)
        for (int64_t n = 0; n < N; ++n)
            if (cache_seqlens[n] < 0) return 1;
    for (int64_t n = 0; n < N; ++n) {
        const int64_t s = idx ? (int64_t)idx[n] : n;
        if (s < 0) {
            for (int64_t d = 0; d < D; ++d) y_out[n * D + d] = 0;
            continue;
        }
        const int64_t c = cache_seqlens ? (int64_t)cache_seqlens[n] : 0;
        for (int64_t d = 0; d < D; ++d) {
            float* st = state + (s * D + d) * L;
            /* the inputs 1 .. W-1 steps back, in the state's order of entries */
            real z = bias ? (real)bias[d] : (real)0;
            for (int j = 0; j < W - 1; ++j) {
                const int k = W - 1 - j; /* steps back; weight w[d, j] */
                const int64_t e = cache_seqlens ? ((c - k) % L + L) % L : L - k;
                z = z + (real)w[d * W + j] * (real)st[e];
            }
            z = z + (real)w[d * W + (W - 1)] * (real)x[n * D + d];
            y_out[n * D + d] = z * sigmoid(z);
            if (L == 0) continue;
            if (cache_seqlens) {
                st[c % L] = x[n * D + d];
            } else {
                for (int j = 0; j + 1 < L; ++j) st[j] = st[j + 1];
                st[L - 1] = x[n * D + d];
            }
        }
    }
    return 0;
}

static uint16_t bf16_rtne(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(v);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    int e = ilogb(a);
    if (e < -126) e = -126;
    double q = ldexp(1.0, e - 7);
    double r = nearbyint(a / q) * q;
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | (uint16_t)(bits >> 16));
}

void oracle_round_bf16(const real* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_rtne((double)in[i]);
}
