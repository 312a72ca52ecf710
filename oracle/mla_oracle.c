/*
 * Plain CPU reference ("oracle") for single-token MLA decode.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file; it exists so that tests, the smoke check and the benchmark's CPU
 * baseline can compare the HIP library against an independent, obviously
 * correct computation. It shares no code, header, table or constant with the
 * HIP library.
 *
 * Arithmetic is IEEE binary64 except where a decoder is defined to produce a
 * binary32 value (the dequantised cache element), which is then widened
 * exactly to binary64. Build without -ffast-math.
 *
 * Sources (kernelindex.com pages of the amd-mixed-mla leaderboard):
 *  - Submission 593653, "Slow fallback" `_bmm_reference`: scores are the
 *    query times the transposed cache rows, times SM_SCALE = 1/sqrt(576); a
 *    softmax over the tokens; the weights times the first V_DIM = 512
 *    columns of the same rows.  This file computes exactly that, in fp64.
 *  - Same page, module constants: 16 query heads, 1 KV head, QK_DIM 576
 *    (512 no-RoPE + 64 RoPE), V_DIM 512, page size 1.
 *  - Same page, `_flash_fp8_single` / `_flash_fp8_split_s1`: the split
 *    partial is stored as the normalised output and lse = max + log(sum)
 *    (natural log); `_flash_fp8_split_s2` merges partials by log-sum-exp.
 *  - Submission 754939, `_dq4` (FP4 E2M1 dequantisation) and the V loop of
 *    `mla_s1`: element value = e2m1 magnitude times 2^(e8m0 - 127); in a
 *    packed byte the low nibble is the even element and the high nibble the
 *    odd one; scale column = element index / 32.
 *  - Submission 754939, `quantize_fp8`: one per-tensor fp32 scale, codes in
 *    the fp8 e4m3 format whose finite maximum is 448 (e4m3fn).
 *  - Submission 593653, `_quantize_q_dynamic_into` / `_quantize_q_static_into`
 *    (the fp8-Q path): the query itself quantised to fp8 with one per-tensor
 *    scale; the attention then uses the decoded query (oracle_mla_decode_q8).
 *
 * Readings where the pages leave a step open:
 *  - fp8 decoded value = binary32 product (code value) * kv_scale, one RNE
 *    rounding.
 *  - e8m0 code 255 is NaN; e4m3fn codes 0x7F / 0xFF are NaN.
 *  - An empty sequence gives out = 0 and lse = -inf; an empty split piece is
 *    skipped by the combine.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_HEADS 16
#define OR_DQK 576
#define OR_DV 512
#define OR_MX_BLOCK 32
#define OR_MX_BLOCKS (OR_DQK / OR_MX_BLOCK) /* 18 scale bytes per token */

enum { OR_KV_BF16 = 0, OR_KV_FP8 = 1, OR_KV_MXFP4 = 2 };

/* ------------------------------------------------------------------------ */
/* Decoders                                                                  */
/* ------------------------------------------------------------------------ */

static float bits_to_float(uint32_t u) {
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* bfloat16 is the upper half of an IEEE binary32; widening is exact. */
float oracle_bf16_value(uint16_t bits) { return bits_to_float((uint32_t)bits << 16); }

/*
 * OCP fp8 E4M3 ("fn": no infinities; finite maximum 448 = 0x7E):
 * sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0.
 * Exponent field 0 encodes subnormals m/8 * 2^-6. Exponent 15 with mantissa
 * 7 is NaN; every other code is finite.
 */
float oracle_e4m3fn_value(uint8_t code) {
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return (float)(sign ? -v : v); /* every finite code is exact in binary32 */
}

/*
 * FP4 E2M1 nibble: bit 3 sign, bits 2..1 exponent, bit 0 mantissa.
 * Exponent 0: value = mantissa * 0.5. Otherwise (1 + mantissa/2) * 2^(e-1).
 * (Submission 754939, `_dq4`.)
 */
float oracle_e2m1_value(uint8_t nibble) {
    int n = nibble & 0xF;
    int e = (n >> 1) & 3;
    int m = n & 1;
    double v = (e == 0) ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
    return (float)(((n >> 3) & 1) ? -v : v);
}

/* E8M0 scale: 2^(code - 127); code 255 is NaN (OCP MX). 127 is the neutral
 * scale. (Submission 754939, V loop of `mla_s1`.) */
float oracle_e8m0_value(uint8_t code) {
    if (code == 0xFF) return NAN;
    return (float)ldexp(1.0, (int)code - 127); /* 2^-127 is a binary32 subnormal: exact */
}

/* One dequantised element of an MXFP4 row: binary32 product of the e2m1 value
 * and the block scale (exact unless it overflows to +-inf). */
static float mxfp4_element(const uint8_t* row_codes, const uint8_t* row_scales, int d) {
    uint8_t byte = row_codes[d / 2];
    uint8_t nib = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
    float a = oracle_e2m1_value(nib);
    float s = oracle_e8m0_value(row_scales[d / OR_MX_BLOCK]);
    return a * s;
}

/* Dequantise one physical cache row into 576 binary32 values. */
static void decode_row(int kv_dtype, const void* kv, const void* scales, int64_t row, float* x) {
    int d;
    if (kv_dtype == OR_KV_BF16) {
        const uint16_t* p = (const uint16_t*)kv + row * OR_DQK;
        for (d = 0; d < OR_DQK; ++d) x[d] = oracle_bf16_value(p[d]);
    } else if (kv_dtype == OR_KV_FP8) {
        const uint8_t* p = (const uint8_t*)kv + row * OR_DQK;
        float s = *(const float*)scales;
        for (d = 0; d < OR_DQK; ++d) {
            float c = oracle_e4m3fn_value(p[d]);
            x[d] = c * s; /* one binary32 multiply, round to nearest even */
        }
    } else {
        const uint8_t* p = (const uint8_t*)kv + row * (OR_DQK / 2);
        const uint8_t* sc = (const uint8_t*)scales + row * OR_MX_BLOCKS;
        for (d = 0; d < OR_DQK; ++d) x[d] = mxfp4_element(p, sc, d);
    }
}

/* Public: dequantise `rows` physical rows to binary32 [rows, 576]. */
int oracle_dequant_rows(int kv_dtype, const void* kv, const void* scales, int64_t rows, float* out) {
    int64_t r;
    if (kv_dtype < 0 || kv_dtype > 2 || !kv || !out || rows < 0) return -1;
    if (kv_dtype != OR_KV_BF16 && !scales) return -1;
    for (r = 0; r < rows; ++r) decode_row(kv_dtype, kv, scales, r, out + r * OR_DQK);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

/* Decode the L rows of one sequence, in logical order, widened to binary64. */
static double* gather_sequence(int kv_dtype, const void* kv, const void* scales,
                               const int32_t* kv_indices, int64_t start, int64_t L) {
    double* x = (double*)malloc((size_t)(L > 0 ? L : 1) * OR_DQK * sizeof(double));
    int64_t j;
    if (!x) return NULL;
#pragma omp parallel for schedule(static)
    for (j = 0; j < L; ++j) {
        float row[OR_DQK];
        int d;
        decode_row(kv_dtype, kv, scales, (int64_t)kv_indices[start + j], row);
        for (d = 0; d < OR_DQK; ++d) x[j * OR_DQK + d] = (double)row[d];
    }
    return x;
}

/* Scaled score of query row qh (576 decoded values) against cache row xj. */
static double score(const double* qh, const double* xj, double sm_scale) {
    double acc = 0.0;
    int d;
    for (d = 0; d < OR_DQK; ++d) acc += qh[d] * xj[d];
    return sm_scale * acc;
}

/*
 * Query formats: 0 = bf16 bits [.., 576] (the value itself); 1 = e4m3fn codes
 * with one fp32 scale, decoded like the fp8 cache: the binary32 product
 * (code value) * q_scale, widened to binary64.
 */
static void decode_query(int q_fmt, const void* q, float q_scale, int64_t row, double* qh) {
    int d;
    if (q_fmt == 0) {
        const uint16_t* p = (const uint16_t*)q + row * OR_DQK;
        for (d = 0; d < OR_DQK; ++d) qh[d] = (double)oracle_bf16_value(p[d]);
    } else {
        const uint8_t* p = (const uint8_t*)q + row * OR_DQK;
        for (d = 0; d < OR_DQK; ++d) {
            float v = oracle_e4m3fn_value(p[d]) * q_scale; /* one binary32 multiply */
            qh[d] = (double)v;
        }
    }
}

/*
 * Softmax attention of one head over tokens [j0, j1) of a decoded sequence:
 *   s_j = sm_scale * q . x_j
 *   M = max_j s_j,  Z = sum_j exp(s_j - M)
 *   out = sum_j exp(s_j - M) x_j[0:512] / Z,  lse = M + ln Z.
 * Empty range: out = 0, lse = -inf.
 */
static void attend_head(const double* qh, const double* x, int64_t j0, int64_t j1, double sm_scale,
                        double* out, double* lse) {
    int64_t j;
    int d;
    double M = -INFINITY, Z = 0.0;
    double* s;
    for (d = 0; d < OR_DV; ++d) out[d] = 0.0;
    if (j1 <= j0) {
        *lse = -INFINITY;
        return;
    }
    s = (double*)malloc((size_t)(j1 - j0) * sizeof(double));
    for (j = j0; j < j1; ++j) {
        s[j - j0] = score(qh, x + j * OR_DQK, sm_scale);
        if (s[j - j0] > M) M = s[j - j0];
    }
    for (j = j0; j < j1; ++j) {
        double w = exp(s[j - j0] - M);
        Z += w;
        for (d = 0; d < OR_DV; ++d) out[d] += w * x[j * OR_DQK + d];
    }
    for (d = 0; d < OR_DV; ++d) out[d] /= Z;
    *lse = M + log(Z);
    free(s);
}

/*
 * Naive route for tiny inputs: each probability is formed on its own as
 * exp(s_j) / sum_k exp(s_k) (no max subtraction), then the output is the
 * probability-weighted sum of V rows. Used only to cross-check attend_head.
 */
static void attend_head_brute(const double* qh, const double* x, int64_t L, double sm_scale,
                              double* out, double* lse) {
    int64_t j, k;
    int d;
    double Z = 0.0;
    for (d = 0; d < OR_DV; ++d) out[d] = 0.0;
    if (L <= 0) {
        *lse = -INFINITY;
        return;
    }
    for (k = 0; k < L; ++k) Z += exp(score(qh, x + k * OR_DQK, sm_scale));
    for (j = 0; j < L; ++j) {
        double p = exp(score(qh, x + j * OR_DQK, sm_scale)) / Z;
        for (d = 0; d < OR_DV; ++d) out[d] += p * x[j * OR_DQK + d];
    }
    *lse = log(Z);
}

/*
 * Merge split partials (normalised output O_s, lse_s) into one result.
 * Three algebraically equal forms appear on the pages; `form` selects one:
 *   0: weights w_s = exp(lse_s - max lse) (softmax over the lse values);
 *      out = sum w_s O_s / sum w_s, lse = max + ln sum w_s.
 *      (Submission 703488, `_reduce_splitk_parallel_*`.)
 *   1: pairwise online merge of (lse, O) pairs in split order.
 *      (Submission 593653, `_flash_fp8_split_s2`.)
 *   2: global max M over the per-split maxima m_s, weights exp(m_s - M) l_s
 *      applied to the unnormalised partials O_s l_s.
 *      (Submission 754939, `mla_s2`.)  Here m_s is recovered as the split's
 *      own max score and l_s = exp(lse_s - m_s).
 * Pieces with lse = -inf (empty) are skipped.
 */
static void combine(int S, const double* po, const double* plse, const double* pmax, int form,
                    double* out, double* lse) {
    int s, d;
    for (d = 0; d < OR_DV; ++d) out[d] = 0.0;
    if (form == 0) {
        double M = -INFINITY, W = 0.0;
        for (s = 0; s < S; ++s)
            if (plse[s] > M) M = plse[s];
        if (M == -INFINITY) {
            *lse = -INFINITY;
            return;
        }
        for (s = 0; s < S; ++s) {
            double w;
            if (plse[s] == -INFINITY) continue;
            w = exp(plse[s] - M);
            W += w;
            for (d = 0; d < OR_DV; ++d) out[d] += w * po[s * OR_DV + d];
        }
        for (d = 0; d < OR_DV; ++d) out[d] /= W;
        *lse = M + log(W);
    } else if (form == 1) {
        double cur = -INFINITY;
        for (s = 0; s < S; ++s) {
            double nl, a, b;
            if (plse[s] == -INFINITY) continue;
            if (cur == -INFINITY) {
                for (d = 0; d < OR_DV; ++d) out[d] = po[s * OR_DV + d];
                cur = plse[s];
                continue;
            }
            nl = (cur > plse[s] ? cur : plse[s]);
            nl = nl + log(exp(cur - nl) + exp(plse[s] - nl));
            a = exp(cur - nl);
            b = exp(plse[s] - nl);
            for (d = 0; d < OR_DV; ++d) out[d] = a * out[d] + b * po[s * OR_DV + d];
            cur = nl;
        }
        *lse = cur;
    } else {
        double M = -INFINITY, L = 0.0;
        for (s = 0; s < S; ++s)
            if (plse[s] != -INFINITY && pmax[s] > M) M = pmax[s];
        if (M == -INFINITY) {
            *lse = -INFINITY;
            return;
        }
        for (s = 0; s < S; ++s) {
            double l_s, w;
            if (plse[s] == -INFINITY) continue;
            l_s = exp(plse[s] - pmax[s]);
            w = exp(pmax[s] - M);
            L += w * l_s;
            for (d = 0; d < OR_DV; ++d) out[d] += w * l_s * po[s * OR_DV + d];
        }
        for (d = 0; d < OR_DV; ++d) out[d] /= L;
        *lse = M + log(L);
    }
}

/* Max scaled score of one head over tokens [j0, j1) (-inf when empty). */
static double range_max(const double* qh, const double* x, int64_t j0, int64_t j1, double sm_scale) {
    double M = -INFINITY;
    int64_t j;
    for (j = j0; j < j1; ++j) {
        double s = score(qh, x + j * OR_DQK, sm_scale);
        if (s > M) M = s;
    }
    return M;
}

/*
 * Shared body of the public entries (query format q_fmt as decode_query).
 *   q          bf16 bits [batch, 16, 576] (oracle_mla_decode) or e4m3fn codes
 *              with q_scale (oracle_mla_decode_q8)
 *   kv, scales cache codes and scales (layouts as decode_row)
 *   kv_indptr  [batch + 1], kv_indices [kv_indptr[batch]]
 *   batches    list of n_list batch ids to compute (NULL: all, n_list = batch)
 *   out        [n_list, 16, 512] binary64, lse [n_list, 16] binary64
 *   route      0 = two-pass softmax, 1 = naive brute force,
 *              2 = split into `nsplit` pieces and merge with combine form
 *                  `form` (pieces [floor(k L / n), floor((k+1) L / n)))
 *   nthreads   OpenMP threads (<= 0: library default)
 * Returns 0, or -1 on an invalid argument.
 */
static int decode_any(int q_fmt, const void* q, float q_scale, int kv_dtype, const void* kv, const void* scales,
                      const int32_t* kv_indptr, const int32_t* kv_indices, int batch, double sm_scale,
                      const int32_t* batches, int n_list, int route, int nsplit, int form, int nthreads,
                      double* out, double* lse) {
    int i;
    if (!q || !kv || !kv_indptr || !out || !lse || batch < 0 || n_list < 0) return -1;
    if (kv_dtype < 0 || kv_dtype > 2 || (kv_dtype != OR_KV_BF16 && !scales)) return -1;
    if (route < 0 || route > 2 || (route == 2 && (nsplit < 1 || form < 0 || form > 2))) return -1;
    if (!batches) n_list = batch;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    for (i = 0; i < n_list; ++i) {
        int b = batches ? batches[i] : i;
        int64_t start, L;
        double* x;
        int h;
        if (b < 0 || b >= batch) return -1;
        start = kv_indptr[b];
        L = (int64_t)kv_indptr[b + 1] - start;
        if (L < 0) return -1;
        if (L > 0 && !kv_indices) return -1;
        x = gather_sequence(kv_dtype, kv, scales, kv_indices, start, L);
        if (!x) return -1;
#pragma omp parallel for schedule(dynamic, 1)
        for (h = 0; h < OR_HEADS; ++h) {
            double qh[OR_DQK];
            double* o = out + ((int64_t)i * OR_HEADS + h) * OR_DV;
            double* l = lse + (int64_t)i * OR_HEADS + h;
            decode_query(q_fmt, q, q_scale, (int64_t)b * OR_HEADS + h, qh);
            if (route == 0) {
                attend_head(qh, x, 0, L, sm_scale, o, l);
            } else if (route == 1) {
                attend_head_brute(qh, x, L, sm_scale, o, l);
            } else {
                double* po = (double*)malloc((size_t)nsplit * OR_DV * sizeof(double));
                double* plse = (double*)malloc((size_t)nsplit * sizeof(double));
                double* pmax = (double*)malloc((size_t)nsplit * sizeof(double));
                int s;
                for (s = 0; s < nsplit; ++s) {
                    int64_t j0 = (int64_t)s * L / nsplit, j1 = (int64_t)(s + 1) * L / nsplit;
                    attend_head(qh, x, j0, j1, sm_scale, po + (int64_t)s * OR_DV, plse + s);
                    pmax[s] = range_max(qh, x, j0, j1, sm_scale);
                }
                combine(nsplit, po, plse, pmax, form, o, l);
                free(po);
                free(plse);
                free(pmax);
            }
        }
        free(x);
    }
    return 0;
}

int oracle_mla_decode(const uint16_t* q, int kv_dtype, const void* kv, const void* scales,
                      const int32_t* kv_indptr, const int32_t* kv_indices, int batch, double sm_scale,
                      const int32_t* batches, int n_list, int route, int nsplit, int form, int nthreads,
                      double* out, double* lse) {
    return decode_any(0, q, 1.0f, kv_dtype, kv, scales, kv_indptr, kv_indices, batch, sm_scale, batches, n_list,
                      route, nsplit, form, nthreads, out, lse);
}

/*
 * The same with an fp8 query: q_codes e4m3fn [batch, 16, 576] and one fp32
 * q_scale; query element = binary32 (code value) * q_scale.
 */
int oracle_mla_decode_q8(const uint8_t* q_codes, float q_scale, int kv_dtype, const void* kv, const void* scales,
                         const int32_t* kv_indptr, const int32_t* kv_indices, int batch, double sm_scale,
                         const int32_t* batches, int n_list, int route, int nsplit, int form, int nthreads,
                         double* out, double* lse) {
    return decode_any(1, q_codes, q_scale, kv_dtype, kv, scales, kv_indptr, kv_indices, batch, sm_scale, batches,
                      n_list, route, nsplit, form, nthreads, out, lse);
}

/*
 * Several query tokens per sequence (multi-token decode: MTP / speculative
 * decoding, the pages' `qo_indptr` with q_seq_len tokens per sequence):
 * query row r belongs to the sequence b with qo_indptr[b] <= r <
 * qo_indptr[b+1]; it is token i = r - qo_indptr[b] of that sequence's
 * n = qo_indptr[b+1] - qo_indptr[b] query tokens. It attends
 *   causal = 0: every cache token of sequence b;
 *   causal = 1: the first L - n + 1 + i tokens (the query tokens are the
 *               sequence's last n positions; the last one sees all L tokens,
 *               earlier ones one token fewer each; none when that count <= 0).
 * q is bf16 [total_q, 16, 576]; rows (optional) lists the query rows to
 * compute (n_list of them), else all total_q = qo_indptr[batch]; out and lse
 * get one entry per computed row. route 0: single pass; 1: brute force.
 */
int oracle_mla_decode_mtp(const uint16_t* q, const int32_t* qo_indptr, int causal, int kv_dtype, const void* kv,
                          const void* scales, const int32_t* kv_indptr, const int32_t* kv_indices, int batch,
                          double sm_scale, const int32_t* rows, int n_list, int route, int nthreads, double* out,
                          double* lse) {
    int i, total_q;
    if (!q || !qo_indptr || !kv || !kv_indptr || !out || !lse || batch < 1 || n_list < 0) return -1;
    if (kv_dtype < 0 || kv_dtype > 2 || (kv_dtype != OR_KV_BF16 && !scales)) return -1;
    if (route < 0 || route > 1 || causal < 0 || causal > 1) return -1;
    total_q = qo_indptr[batch];
    if (!rows) n_list = total_q;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    for (i = 0; i < n_list; ++i) {
        int r = rows ? rows[i] : i;
        int b = 0, h;
        int64_t start, L, n, t;
        double* x;
        if (r < 0 || r >= total_q) return -1;
        while (!(qo_indptr[b] <= r && r < qo_indptr[b + 1])) ++b;  /* the sequence holding row r */
        n = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
        t = r - qo_indptr[b];
        start = kv_indptr[b];
        L = (int64_t)kv_indptr[b + 1] - start;
        if (L < 0) return -1;
        if (causal) {
            L = L - n + 1 + t;
            if (L < 0) L = 0;
        }
        if (L > 0 && !kv_indices) return -1;
        x = gather_sequence(kv_dtype, kv, scales, kv_indices, start, L);
        if (!x) return -1;
#pragma omp parallel for schedule(dynamic, 1)
        for (h = 0; h < OR_HEADS; ++h) {
            double qh[OR_DQK];
            double* o = out + ((int64_t)i * OR_HEADS + h) * OR_DV;
            double* l = lse + (int64_t)i * OR_HEADS + h;
            decode_query(0, q, 1.0f, (int64_t)r * OR_HEADS + h, qh);
            if (route == 0)
                attend_head(qh, x, 0, L, sm_scale, o, l);
            else
                attend_head_brute(qh, x, L, sm_scale, o, l);
        }
        free(x);
    }
    return 0;
}

/*
 * Nearest e4m3fn code to a binary32 value, ties to the code with an even
 * mantissa (round to nearest even), by search over the 127 non-negative finite
 * codes. |x| above 448 saturates to 448 (the quantiser clamps before it
 * encodes, so saturation never decides a value there). The sign bit follows
 * the sign of x, so -0 and negative values that round to zero give 0x80.
 * NaN gives 0x7F.
 */
uint8_t oracle_e4m3fn_encode(float x) {
    double a = fabs((double)x), best_err = INFINITY;
    int c, best = 0;
    if (isnan(x)) return 0x7F;
    for (c = 0; c <= 0x7E; ++c) {
        double err = fabs((double)oracle_e4m3fn_value((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best_err = err;
            best = c;
        }
    }
    return (uint8_t)(signbit(x) ? (best | 0x80) : best);
}

/*
 * Per-tensor fp8 quantisation of a bf16 query of n elements (submission
 * 593653, `_quantize_q_static_into` and `_quantize_q_dynamic_into`):
 *   dynamic (mode 1): scale = max(max_i |q_i|, 1e-12) / 448, written to *scale;
 *   static  (mode 0): scale = *scale as given (must be finite and > 0);
 *   code_i = e4m3fn(clamp(q_i / scale, -448, 448)).
 * Every step is one binary32 operation (the bf16 value widened exactly, one
 * division, one comparison-based clamp, one round to nearest even).
 * Returns 0, or -1 for a bad mode or scale.
 */
int oracle_quantize_q_fp8(const uint16_t* q, int64_t n, int mode, float* scale, uint8_t* codes) {
    int64_t i;
    float s;
    if (mode == 1) {
        float amax = 0.0f;
        for (i = 0; i < n; ++i) {
            float a = fabsf(oracle_bf16_value(q[i]));
            if (a > amax) amax = a;
        }
        if (amax < 1e-12f) amax = 1e-12f;
        s = amax / 448.0f;
        *scale = s;
    } else if (mode == 0) {
        s = *scale;
        if (!(s > 0.0f) || isinf(s)) return -1;
    } else {
        return -1;
    }
    for (i = 0; i < n; ++i) {
        float y = oracle_bf16_value(q[i]) / s;
        if (y > 448.0f) y = 448.0f;
        if (y < -448.0f) y = -448.0f;
        codes[i] = oracle_e4m3fn_encode(y);
    }
    return 0;
}

/*
 * Paged cache (more than one row per page). The convention is that of the
 * pages' a16w8 path (submission 616673, `_run_a16w8`: the cache viewed as
 * [pages, page_size, 1, 576], the page table given by kv_indptr / kv_indices
 * counted in pages, and kv_last_page_lens) and of the page tables passed to
 * `mla_decode_fwd` (submission 593653):
 *   - sequence b owns the pages page_ids[page_indptr[b]] ..
 *     page_ids[page_indptr[b+1] - 1], in that order;
 *   - page p holds cache rows p * page_size .. p * page_size + page_size - 1;
 *   - every page of a sequence but its last contributes all page_size rows,
 *     in row order; the last one contributes its first last_page_len[b] rows
 *     (1 .. page_size). With page_size 1 every page is one row and
 *     last_page_len is not read.
 * oracle_expand_pages writes the token-level tables of that convention:
 * tok_indptr [batch + 1] and tok_rows (cache row of every token, in order;
 * room for cap entries). Returns 0, or -1 on an invalid argument.
 */
int oracle_expand_pages(const int32_t* page_indptr, const int32_t* page_ids, const int32_t* last_page_len,
                        int page_size, int batch, int32_t* tok_indptr, int32_t* tok_rows, int64_t cap) {
    int64_t n = 0;
    int b;
    if (!page_indptr || !tok_indptr || batch < 0 || page_size < 1) return -1;
    tok_indptr[0] = 0;
    for (b = 0; b < batch; ++b) {
        int32_t first = page_indptr[b], end = page_indptr[b + 1], k;
        if (end < first) return -1;
        if (end > first && !page_ids) return -1;
        for (k = first; k < end; ++k) {
            int64_t rows_in_page = page_size, i;
            if (k == end - 1 && page_size > 1) {  /* the sequence's last page */
                if (!last_page_len) return -1;
                rows_in_page = last_page_len[b];
                if (rows_in_page < 1 || rows_in_page > page_size) return -1;
            }
            for (i = 0; i < rows_in_page; ++i) {
                int64_t row = (int64_t)page_ids[k] * page_size + i;
                if (n >= cap || row > INT32_MAX) return -1;
                tok_rows[n++] = (int32_t)row;
            }
        }
        if (n > INT32_MAX) return -1;
        tok_indptr[b + 1] = (int32_t)n;
    }
    return 0;
}

/*
 * MLA decode over a paged cache: the pages of each sequence are expanded into
 * its token rows (oracle_expand_pages), then the attention of
 * oracle_mla_decode (route 0) runs over those tokens. Arguments as
 * oracle_mla_decode, with the page table in place of kv_indptr / kv_indices.
 */
int oracle_mla_decode_paged(const uint16_t* q, int kv_dtype, const void* kv, const void* scales,
                            const int32_t* page_indptr, const int32_t* page_ids, const int32_t* last_page_len,
                            int page_size, int batch, double sm_scale, const int32_t* batches, int n_list,
                            int nthreads, double* out, double* lse) {
    int32_t* tok_indptr;
    int32_t* tok_rows;
    int64_t cap;
    int rc;
    if (!page_indptr || batch < 0 || page_size < 1) return -1;
    cap = (int64_t)page_indptr[batch] * page_size;
    if (cap < 0) return -1;
    tok_indptr = (int32_t*)malloc(((size_t)batch + 1) * sizeof(int32_t));
    tok_rows = (int32_t*)malloc((size_t)(cap > 0 ? cap : 1) * sizeof(int32_t));
    rc = (tok_indptr && tok_rows) ? 0 : -1;
    if (rc == 0)
        rc = oracle_expand_pages(page_indptr, page_ids, last_page_len, page_size, batch, tok_indptr, tok_rows, cap);
    if (rc == 0)
        rc = decode_any(0, q, 1.0f, kv_dtype, kv, scales, tok_indptr, tok_rows, batch, sm_scale, batches, n_list, 0, 1,
                        0, nthreads, out, lse);
    free(tok_indptr);
    free(tok_rows);
    return rc;
}

/* Threads the OpenMP runtime will use (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
