/*
 * CPU oracle for the fused MoE grouped-matmul + finalize-routing operator with
 * MXFP8 inputs.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the GPU library never does, and the two
 * share no code, header or table.
 *
 * Sources (the web pages this operator is defined on):
 *   [P1] "基于 PyPTO 的 MoE 融合算子实践：grouped_matmul_finalize_routing 的
 *        MXFP8 实现与精度验证" (czykbl.com/news/94077)
 *   [P3] CANN API reference "aclnnGroupedMatmulFinalizeRoutingV3"
 *        (hiascend.com, ops-transformer)
 *
 * What is computed, written out as its plain definition ([P1] §2.1, expanded
 * form; [P3] "计算公式" formulas 1 and 2; [P1] §6.3 golden description):
 *
 *   out[row_index[t], n] += w_t * sum_k  dq1(t,k) * dq2(e(t),k,n)
 *   out[off + r, n]      += shared_input_weight * shared_input[r, n]
 *
 * with dq = FP8 (or, in the MXFP4 variant, FP4 E2M1) value * 2^(E8M0 byte - 127),
 * one E8M0 scale per 32 consecutive
 * K elements (the reading of the "[ceil(K/64), ..., 2]" scale layout: sub-block
 * j of 64-block b covers k in [64b+32j, 64b+32j+32)), w_t = logit[t] (1 when
 * logit is absent), and e(t) the expert whose group_list range holds t.
 *
 * Everything is evaluated in double precision.  FP8 x FP8 x 2^k products are
 * exact in double, so the only difference from an exact result is the double
 * summation error (about K * 2^-53 relative), which is negligible against the
 * FP32 tolerance the GPU path is held to.
 *
 * The end of this file adds the A2/A3 W4A8 variant of [P3] (INT8 x INT4 with
 * FP32 per-channel and per-token scales) with the same routing.
 *
 * Output rows are independent and are spread over OpenMP threads; each row
 * is computed whole, in the order written below, by one thread, so the result
 * is the same for any thread count.
 *
 * Alongside out, the oracle returns mag = |out_init| + sum |w_t * term| +
 * |shared term| per element: the sum of the magnitudes of every term that
 * enters that element.  The GPU tolerance is expressed against it.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Error codes returned by oracle_gmm_finalize_routing. */
#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)
#define ORACLE_BAD_GROUP_LIST (-2)
#define ORACLE_BAD_ROW_INDEX (-3)
#define ORACLE_BAD_SHARED_RANGE (-4)
#define ORACLE_NO_MEMORY (-5)

/* ---------------------------------------------------------------------------
 * Bit-level decoders.  The pages name the formats (FP8 E4M3FN / E5M2 data,
 * E8M0FNU scales, bf16 shared input: [P1] §2.1, §3.1) without restating them;
 * these follow the standard definitions of those encodings.
 * ------------------------------------------------------------------------- */

/* FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;
 * exponent 15 with mantissa 7 is NaN; exponent 0 is subnormal. */
double oracle_decode_e4m3fn(uint8_t b)
{
    int s = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* FP8 E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa bits; IEEE-style
 * infinities and NaNs at exponent 31; exponent 0 is subnormal. */
double oracle_decode_e5m2(uint8_t b)
{
    int s = (b >> 7) & 1;
    int e = (b >> 2) & 31;
    int m = b & 3;
    double v;
    if (e == 31)
        v = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)m / 4.0, -14);
    else
        v = ldexp(1.0 + (double)m / 4.0, e - 15);
    return s ? -v : v;
}

/* FP4 E2M1 (the MXFP4 element, [P3] Atlas 350 MX notes): 1 sign, 2 exponent
 * (bias 1), 1 mantissa bit in the low four bits of c; exponent 0 is
 * subnormal; no infinities or NaNs. */
double oracle_decode_e2m1(uint8_t c)
{
    int s = (c >> 3) & 1;
    int e = (c >> 1) & 3;
    int m = c & 1;
    double v;
    if (e == 0)
        v = (double)m / 2.0;
    else
        v = ldexp(1.0 + (double)m / 2.0, e - 1);
    return s ? -v : v;
}

/* E8M0 (unsigned, exponent only, bias 127): 2^(b-127); 0xFF is NaN. */
double oracle_decode_e8m0(uint8_t b)
{
    if (b == 255)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits. */
double oracle_decode_bf16(uint16_t h)
{
    int s = (h >> 15) & 1;
    int e = (h >> 7) & 255;
    int m = h & 127;
    double v;
    if (e == 255)
        v = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        v = ldexp((double)m / 128.0, -126);
    else
        v = ldexp(1.0 + (double)m / 128.0, e - 127);
    return s ? -v : v;
}

/* ---------------------------------------------------------------------------
 * Expert token ranges from group_list ([P1] §4.3, "group_list 的两种格式").
 *   type 0 (prefix sums): expert i owns [group_list[i-1], group_list[i]),
 *                         with group_list[-1] read as 0;
 *   type 1 (counts):      expert i owns [sum(group_list[:i]),
 *                                        sum(group_list[:i]) + group_list[i]).
 * A negative count, a decreasing prefix or a range ending past M is rejected.
 * Rows past the last range belong to no expert and contribute nothing.
 * ------------------------------------------------------------------------- */
int oracle_expert_ranges(const int64_t *group_list, int64_t E, int type,
                         int64_t M, int64_t *start, int64_t *end)
{
    int64_t prev = 0;
    for (int64_t i = 0; i < E; ++i) {
        if (type == 0) {
            start[i] = prev;
            end[i] = group_list[i];
        } else if (type == 1) {
            start[i] = prev;
            end[i] = prev + group_list[i];
        } else {
            return ORACLE_BAD_ARG;
        }
        if (end[i] < start[i] || end[i] > M)
            return ORACLE_BAD_GROUP_LIST;
        prev = end[i];
    }
    return ORACLE_OK;
}

/* Element kinds: 0 FP8 E4M3FN, 1 FP8 E5M2, 2 FP4 E2M1 (two per byte). */
#define ORACLE_E2M1 2

/* Value of every element code of the chosen kind, and of every E8M0 code,
 * built once per call by the decoders above (a cache of them, nothing more). */
static void decode_tables(int fp8_kind, double fp8v[256], double e8m0v[256])
{
    for (int c = 0; c < 256; ++c) {
        if (fp8_kind == ORACLE_E2M1)
            fp8v[c] = c < 16 ? oracle_decode_e2m1((uint8_t)c) : NAN;
        else
            fp8v[c] = fp8_kind == 0 ? oracle_decode_e4m3fn((uint8_t)c)
                                    : oracle_decode_e5m2((uint8_t)c);
        e8m0v[c] = oracle_decode_e8m0((uint8_t)c);
    }
}

/* Bytes of a stored row of `len` elements: one code per byte for FP8, two for
 * E2M1. */
static int64_t row_bytes(int64_t len, int fp8_kind)
{
    return fp8_kind == ORACLE_E2M1 ? len / 2 : len;
}

/* Code of element i of a stored row.  E2M1 rows hold element 2j in the low
 * nibble and element 2j+1 in the high nibble of byte j (the reading of the
 * MXFP4 packing: pairs along the row's contiguous dimension, which is why the
 * pages require an even k, and an even n for a non-transposed x2). */
static uint8_t code_at(const uint8_t *row, int64_t i, int fp8_kind)
{
    if (fp8_kind != ORACLE_E2M1)
        return row[i];
    const uint8_t b = row[i / 2];
    return (i & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
}

/* Arguments every entry point accepts: a known kind, and the even sizes the
 * E2M1 packing needs. */
static int kind_ok(int fp8_kind, int64_t K, int64_t N, int transpose_x2)
{
    if (fp8_kind == 0 || fp8_kind == 1)
        return 1;
    if (fp8_kind != ORACLE_E2M1)
        return 0;
    return K % 2 == 0 && (transpose_x2 || N % 2 == 0);
}

/* ---------------------------------------------------------------------------
 * The operator.
 *
 * Layouts (row-major, contiguous) — [P1] §3.1 input table, [P3] Atlas 350
 * parameter notes:
 *   x1              [M, K]                    FP8 codes
 *   x2              [E, K, N]  (transpose_x2 = 0) or [E, N, K] (= 1), FP8 codes
 *   scale           [KB, N, 2] (transpose_x2 = 0) or [N, KB, 2] (= 1), E8M0,
 *                   KB = ceil(K/64); with scale_per_expert a leading [E] axis
 *   pertoken_scale  [M, KB, 2]                E8M0
 *   group_list      [E] int64, read per group_list_type
 *   logit           [M] float32, or NULL (weight 1)       ([P1] §5.1 has_logit)
 *   row_index       [M] int64, each in [0, batch)          ([P1] §4.2)
 *   shared_input    [R, N] bf16 bits, or NULL             ([P1] §5.1 has_shared_input)
 *   out_init        [batch, N] float32, the initial value of out ([P1] §3.1)
 *
 * The scale of element k of row t of x1 is pertoken_scale[t, k/64, (k/32)%2];
 * the scale of element (k, n) of expert e's weight is scale[k/64, n, (k/32)%2]
 * (or scale[n, k/64, (k/32)%2] when transposed).  The pair axis splits each
 * 64-block of K into its two 32-element halves in K order ([P1] §2.1 says one
 * scale per block, §4.2 says each 64-block holds 2 scales, §6.3 says the golden
 * expands each scale over 32 K elements; this is the reading all three allow).
 *
 * Only the output rows listed in rows[0..n_rows) are computed (all rows when
 * rows is NULL, in which case n_rows must equal batch).  For each listed row b:
 *   res[b] = out_init[b] + sum over tokens t with row_index[t] == b, t in some
 *            expert's range, in ascending t, of w_t * (matmul row t)
 *            + shared term if off <= b < off + R.
 * Results go to res_out[i*N + n] and mag_out[i*N + n] (double).
 * ------------------------------------------------------------------------- */
int oracle_gmm_finalize_routing(
    const uint8_t *x1, const uint8_t *x2, const uint8_t *scale,
    int scale_per_expert, const uint8_t *pertoken_scale,
    const int64_t *group_list, int group_list_type, const float *logit,
    const int64_t *row_index, const uint16_t *shared_input,
    double shared_input_weight, int64_t shared_input_offset,
    int64_t shared_rows, const float *out_init, int transpose_x2,
    int fp8_kind, int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
    const int64_t *rows, int64_t n_rows, double *res_out, double *mag_out)
{
    if (M < 0 || K <= 0 || N < 0 || E <= 0 || batch < 0 || n_rows < 0)
        return ORACLE_BAD_ARG;
    if (!kind_ok(fp8_kind, K, N, transpose_x2))
        return ORACLE_BAD_ARG;
    if (rows == NULL && n_rows != batch)
        return ORACLE_BAD_ARG;
    if (shared_input != NULL &&
        (shared_input_offset < 0 || shared_rows < 0 ||
         shared_input_offset + shared_rows > batch))
        return ORACLE_BAD_SHARED_RANGE;

    const int64_t KB = (K + 63) / 64;
    double fp8v[256], e8m0v[256];
    decode_tables(fp8_kind, fp8v, e8m0v);

    int64_t *start = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    int64_t *end = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    int64_t *expert_of = (int64_t *)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
    int rc = ORACLE_OK;
    int no_memory = 0;
    if (!start || !end || !expert_of) {
        rc = ORACLE_NO_MEMORY;
        goto done;
    }

    rc = oracle_expert_ranges(group_list, E, group_list_type, M, start, end);
    if (rc != ORACLE_OK)
        goto done;

    /* Token -> expert; tokens in no range keep -1 and are never read. */
    for (int64_t t = 0; t < M; ++t)
        expert_of[t] = -1;
    for (int64_t e = 0; e < E; ++e)
        for (int64_t t = start[e]; t < end[e]; ++t)
            expert_of[t] = e;

    /* row_index must lie in [0, batch) for every routed token ([P1] §4.2). */
    for (int64_t t = 0; t < M; ++t)
        if (expert_of[t] >= 0 && (row_index[t] < 0 || row_index[t] >= batch)) {
            rc = ORACLE_BAD_ROW_INDEX;
            goto done;
        }
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t b = rows ? rows[i] : i;
        if (b < 0 || b >= batch) {
            rc = ORACLE_BAD_ARG;
            goto done;
        }
    }

    /* Output rows are independent: each is computed whole by one thread, in
     * the order below, so the result does not depend on the thread count. */
#pragma omp parallel
    {
        double *acc = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *absacc = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!acc || !absacc) {
#pragma omp atomic write
            no_memory = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (!acc || !absacc)
                continue;
            const int64_t b = rows ? rows[i] : i;
            double *res = res_out + i * N;
            double *mag = mag_out + i * N;

            /* out starts from its initial value ([P1] §3.1: out is the initial value). */
            for (int64_t n = 0; n < N; ++n) {
                res[n] = (double)out_init[b * N + n];
                mag[n] = fabs(res[n]);
            }

            /* Routed experts: every token scattered to row b, ascending t
             * ([P1] §2.2 stages 1-3; [P3] formula 2). */
            for (int64_t t = 0; t < M; ++t) {
                const int64_t e = expert_of[t];
                if (e < 0 || row_index[t] != b)
                    continue;
                const double w = logit ? (double)logit[t] : 1.0;

                for (int64_t n = 0; n < N; ++n) {
                    acc[n] = 0.0;
                    absacc[n] = 0.0;
                }

                /* Stage 1: the scaled matmul row, summed over k in ascending
                 * order for each n.  The loop nest is ordered for the memory
                 * layout only; each element's sum is the same sequence either
                 * way. */
                const uint8_t *ps_row = pertoken_scale + t * KB * 2;
                const uint8_t *sc = scale + (scale_per_expert ? e * KB * N * 2 : 0);
                const uint8_t *x1_row = x1 + t * row_bytes(K, fp8_kind);
                if (!transpose_x2) {
                    for (int64_t k = 0; k < K; ++k) {
                        /* row k of expert e's [K, N] weight */
                        const uint8_t *w2 = x2 + (e * K + k) * row_bytes(N, fp8_kind);
                        const double a = fp8v[code_at(x1_row, k, fp8_kind)] *
                                         e8m0v[ps_row[(k / 64) * 2 + (k / 32) % 2]];
                        for (int64_t n = 0; n < N; ++n) {
                            const double bw = fp8v[code_at(w2, n, fp8_kind)] *
                                              e8m0v[sc[((k / 64) * N + n) * 2 + (k / 32) % 2]];
                            const double term = a * bw;
                            acc[n] += term;
                            absacc[n] += fabs(term);
                        }
                    }
                } else {
                    for (int64_t n = 0; n < N; ++n) {
                        /* row n of expert e's [N, K] weight */
                        const uint8_t *w2 = x2 + (e * N + n) * row_bytes(K, fp8_kind);
                        for (int64_t k = 0; k < K; ++k) {
                            const double a = fp8v[code_at(x1_row, k, fp8_kind)] *
                                             e8m0v[ps_row[(k / 64) * 2 + (k / 32) % 2]];
                            const double bw = fp8v[code_at(w2, k, fp8_kind)] *
                                              e8m0v[sc[(n * KB + k / 64) * 2 + (k / 32) % 2]];
                            const double term = a * bw;
                            acc[n] += term;
                            absacc[n] += fabs(term);
                        }
                    }
                }

                /* Stages 2-3: weight by logit, add into row b. */
                for (int64_t n = 0; n < N; ++n) {
                    res[n] += w * acc[n];
                    mag[n] += fabs(w) * absacc[n];
                }
            }

            /* Stage 4: shared expert into rows [off, off + R) ([P1] §2.1,
             * §5.3; [P3] formula 3). */
            if (shared_input && b >= shared_input_offset &&
                b < shared_input_offset + shared_rows) {
                const int64_t r = b - shared_input_offset;
                for (int64_t n = 0; n < N; ++n) {
                    const double v = shared_input_weight *
                                     oracle_decode_bf16(shared_input[r * N + n]);
                    res[n] += v;
                    mag[n] += fabs(v);
                }
            }
        }
        free(acc);
        free(absacc);
    }
    if (no_memory)
        rc = ORACLE_NO_MEMORY;

done:
    free(start);
    free(end);
    free(expert_of);
    return rc;
}

/* Threads the row loops above run on (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------
 * Tolerance support, not part of the operator: a per-element bound on the
 * extra error of a block-scaled dot-product unit that sums each run of 8
 * consecutive K products (k in [8i, 8i + 8)) after aligning them to the
 * largest one's binary exponent E and truncating below 2^(E - 13).  Each
 * product can then lose less than min(|term|, 2^(E - 13)).  Returned, for the
 * selected rows, is
 *   slack[b, n] = sum over tokens t routed to b of |w_t| *
 *                 sum over groups G of sum_{k in G} min(|term_k|, 2^(E_G - 13)).
 * Arguments as for oracle_gmm_finalize_routing.
 * ------------------------------------------------------------------------- */
int oracle_mx_group_slack(
    const uint8_t *x1, const uint8_t *x2, const uint8_t *scale,
    int scale_per_expert, const uint8_t *pertoken_scale,
    const int64_t *group_list, int group_list_type, const float *logit,
    const int64_t *row_index, int transpose_x2, int fp8_kind,
    int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
    const int64_t *rows, int64_t n_rows, double *slack_out)
{
    if (M < 0 || K <= 0 || N < 0 || E <= 0 || batch < 0 || n_rows < 0 ||
        !kind_ok(fp8_kind, K, N, transpose_x2) || (rows == NULL && n_rows != batch))
        return ORACLE_BAD_ARG;
    const int64_t KB = (K + 63) / 64;
    double fp8v[256], e8m0v[256];
    decode_tables(fp8_kind, fp8v, e8m0v);
    int64_t *start = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    int64_t *end = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    int64_t *expert_of = (int64_t *)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
    double term[8];
    int rc = ORACLE_OK;
    if (!start || !end || !expert_of) {
        rc = ORACLE_NO_MEMORY;
        goto done;
    }
    rc = oracle_expert_ranges(group_list, E, group_list_type, M, start, end);
    if (rc != ORACLE_OK)
        goto done;
    for (int64_t t = 0; t < M; ++t)
        expert_of[t] = -1;
    for (int64_t e = 0; e < E; ++e)
        for (int64_t t = start[e]; t < end[e]; ++t)
            expert_of[t] = e;
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t b = rows ? rows[i] : i;
        double *sl = slack_out + i * N;
        for (int64_t n = 0; n < N; ++n)
            sl[n] = 0.0;
        for (int64_t t = 0; t < M; ++t) {
            const int64_t e = expert_of[t];
            if (e < 0 || row_index[t] != b)
                continue;
            const double w = fabs(logit ? (double)logit[t] : 1.0);
            const uint8_t *ps_row = pertoken_scale + t * KB * 2;
            const uint8_t *sc = scale + (scale_per_expert ? e * KB * N * 2 : 0);
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t g0 = 0; g0 < K; g0 += 8) {
                    double mx = 0.0;
                    int cnt = 0;
                    for (int64_t k = g0; k < g0 + 8 && k < K; ++k) {
                        const double a =
                            fp8v[code_at(x1 + t * row_bytes(K, fp8_kind), k, fp8_kind)] *
                            e8m0v[ps_row[(k / 64) * 2 + (k / 32) % 2]];
                        const double bw = transpose_x2
                            ? fp8v[code_at(x2 + (e * N + n) * row_bytes(K, fp8_kind), k,
                                           fp8_kind)] *
                                  e8m0v[sc[(n * KB + k / 64) * 2 + (k / 32) % 2]]
                            : fp8v[code_at(x2 + (e * K + k) * row_bytes(N, fp8_kind), n,
                                           fp8_kind)] *
                                  e8m0v[sc[((k / 64) * N + n) * 2 + (k / 32) % 2]];
                        term[cnt] = fabs(a * bw);
                        if (term[cnt] > mx)
                            mx = term[cnt];
                        ++cnt;
                    }
                    if (mx == 0.0)
                        continue;
                    int ex;
                    frexp(mx, &ex);                      /* mx in [2^(ex-1), 2^ex) */
                    const double q = ldexp(1.0, ex - 1 - 13); /* 2^(E - 13) */
                    for (int c = 0; c < cnt; ++c)
                        acc += term[c] < q ? term[c] : q;
                }
                sl[n] += w * acc;
            }
        }
    }
done:
    free(start);
    free(end);
    free(expert_of);
    return rc;
}

/* ---------------------------------------------------------------------------
 * The A2/A3 W4A8 variant ([P3] A2/A3 parameter notes and pseudo-quant notes):
 * INT8 x1, INT4 weights, a fused per-channel FP32 scale, an FP32 per-token
 * scale, an optional asymmetric offset, then the same routing and shared
 * term as the MX operator.  Formula 1 of [P3] with these operands:
 *
 *   y[t, n] = pertoken_scale[t] * ( scale[e, n] * sum_k x1[t, k] * w[e, k, n]
 *                                   + offset[e, n] * sum_k x1[t, k] )
 *   out[row_index[t], n] += logit[t] * y[t, n]
 *
 * (offset = antiquantOffset * scale, the asymmetric form: dequantised weight
 * (w + antiquantOffset) * scale; absent for the symmetric form.)
 *
 * Layouts: x1 [M, K] int8; x2 [E, K, N/2] bytes, two signed 4-bit values per
 * byte along n, element 2j in the low nibble of byte j (the reading of the
 * "(e, k, n/8) INT32" packing, nibbles in little-endian order); scale and
 * offset [E, 1, N] float32 (one group along K); pertoken_scale [M] float32;
 * the rest as oracle_gmm_finalize_routing.  The integer sums are exact
 * (int64); the rest is double precision.  mag accumulates |init| +
 * |logit * pts| * (|scale| * sum |x w| + |offset| * sum |x|) + |shared|.
 * ------------------------------------------------------------------------- */

/* Signed value of a 4-bit two's complement code. */
static int int4_value(uint8_t c)
{
    return (c & 8) ? (int)(c & 15) - 16 : (int)(c & 15);
}

int oracle_w4a8_finalize_routing(
    const int8_t *x1, const uint8_t *x2, const float *scale, const float *offset,
    const float *pertoken_scale, const int64_t *group_list, int group_list_type,
    const float *logit, const int64_t *row_index, const uint16_t *shared_input,
    double shared_input_weight, int64_t shared_input_offset, int64_t shared_rows,
    const float *out_init, int64_t M, int64_t K, int64_t N, int64_t E, int64_t batch,
    const int64_t *rows, int64_t n_rows, double *res_out, double *mag_out)
{
    if (M < 0 || K <= 0 || N < 0 || N % 2 != 0 || E <= 0 || batch < 0 || n_rows < 0)
        return ORACLE_BAD_ARG;
    if (rows == NULL && n_rows != batch)
        return ORACLE_BAD_ARG;
    if (shared_input != NULL &&
        (shared_input_offset < 0 || shared_rows < 0 ||
         shared_input_offset + shared_rows > batch))
        return ORACLE_BAD_SHARED_RANGE;
    int64_t *start = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    int64_t *end = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
    int64_t *expert_of = (int64_t *)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
    int rc = ORACLE_OK;
    int no_memory = 0;
    if (!start || !end || !expert_of) {
        rc = ORACLE_NO_MEMORY;
        goto done;
    }
    rc = oracle_expert_ranges(group_list, E, group_list_type, M, start, end);
    if (rc != ORACLE_OK)
        goto done;
    for (int64_t t = 0; t < M; ++t)
        expert_of[t] = -1;
    for (int64_t e = 0; e < E; ++e)
        for (int64_t t = start[e]; t < end[e]; ++t)
            expert_of[t] = e;
    for (int64_t t = 0; t < M; ++t)
        if (expert_of[t] >= 0 && (row_index[t] < 0 || row_index[t] >= batch)) {
            rc = ORACLE_BAD_ROW_INDEX;
            goto done;
        }
    for (int64_t i = 0; i < n_rows; ++i) {
        const int64_t b = rows ? rows[i] : i;
        if (b < 0 || b >= batch) {
            rc = ORACLE_BAD_ARG;
            goto done;
        }
    }

    /* One output row per thread at a time, as in oracle_gmm_finalize_routing. */
#pragma omp parallel
    {
        int64_t *dot = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
        int64_t *adot = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N > 0 ? N : 1));
        if (!dot || !adot) {
#pragma omp atomic write
            no_memory = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_rows; ++i) {
            if (!dot || !adot)
                continue;
            const int64_t b = rows ? rows[i] : i;
            double *res = res_out + i * N;
            double *mag = mag_out + i * N;
            for (int64_t n = 0; n < N; ++n) {
                res[n] = (double)out_init[b * N + n];
                mag[n] = fabs(res[n]);
            }
            for (int64_t t = 0; t < M; ++t) {
                const int64_t e = expert_of[t];
                if (e < 0 || row_index[t] != b)
                    continue;
                const double w = (logit ? (double)logit[t] : 1.0) * (double)pertoken_scale[t];
                int64_t xsum = 0, xabs = 0;
                for (int64_t n = 0; n < N; ++n)
                    dot[n] = adot[n] = 0;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t xv = x1[t * K + k];
                    xsum += xv;
                    xabs += xv < 0 ? -xv : xv;
                    const uint8_t *wrow = x2 + (e * K + k) * (N / 2);   /* row k of expert e */
                    for (int64_t n = 0; n < N; ++n) {
                        const uint8_t byte = wrow[n / 2];
                        const int64_t p = xv * int4_value((n & 1) ? (uint8_t)(byte >> 4) : byte);
                        dot[n] += p;
                        adot[n] += p < 0 ? -p : p;
                    }
                }
                for (int64_t n = 0; n < N; ++n) {
                    const double s = (double)scale[e * N + n];
                    const double o = offset ? (double)offset[e * N + n] : 0.0;
                    res[n] += w * (s * (double)dot[n] + o * (double)xsum);
                    mag[n] += fabs(w) * (fabs(s) * (double)adot[n] + fabs(o) * (double)xabs);
                }
            }
            if (shared_input && b >= shared_input_offset &&
                b < shared_input_offset + shared_rows) {
                const int64_t r = b - shared_input_offset;
                for (int64_t n = 0; n < N; ++n) {
                    const double v = shared_input_weight *
                                     oracle_decode_bf16(shared_input[r * N + n]);
                    res[n] += v;
                    mag[n] += fabs(v);
                }
            }
        }
        free(dot);
        free(adot);
    }
    if (no_memory)
        rc = ORACLE_NO_MEMORY;
done:
    free(start);
    free(end);
    free(expert_of);
    return rc;
}
