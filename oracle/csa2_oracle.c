/*
 * csa2_oracle.c -- plain CPU oracle for CSA2 sparse attention over an FP4 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg use it.  It shares no code, header, table or
 * constant with the GPU library.
 *
 * Sources (pages about DeepSeek-V4.1-Flash; cited by page title and section):
 *   [Brief]  "DeepSeek-V4.1-Flash" course brief (g2c), sections "FP4 cache
 *            entries, and why they're safe", "The global branch: compress,
 *            index, select", "CSA2: most layers don't keep their own cache"
 *            (mode table), "The hierarchical indexer".
 *   [Review] "DeepSeek V4.1 Flash: pushing the limits" talk write-up,
 *            section "The Paper" (Full / Reindex / Reuse walk-through).
 *   [News]   metallab.ai article on the V4.1-Flash KV cache (three modes).
 *   OCP 8-bit floating point (E4M3FN) and OCP MX (E2M1) format definitions.
 *
 * Every function is the plain definition written out, slowly:
 *   - decoders are the format definitions;
 *   - encoders search the whole grid for the nearest value (ties to the
 *     even code), so rounding needs no bit tricks;
 *   - selection sorts every candidate with a library sort;
 *   - attention accumulates in double.
 * Build: gcc -O2 -mfma -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * fp32 operations that define results (amax/6, x/s, the indexer's fmaf
 * chain and head sum) are written as explicit single-precision operations;
 * -ffp-contract=off keeps the compiler from fusing them differently.
 *
 * Parity status: every function here is pinned by tests against format
 * tables, library casts, closed forms, brute force or textbook attention
 * (see tests/test_oracle_*.py).  The pages print no worked numeric example
 * of any code, score or attention output.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_D 512    /* channels of the shared latent ([Brief] "The global branch") */
#define OR_G 16     /* channels per E4M3 scale ([Brief] "FP4 cache entries")       */
#define OR_NG (OR_D / OR_G)

/* ---------------------------------------------------------------- codecs */

/* E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0
 * is subnormal (0 or 0.5).  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (OCP MX). */
double oracle_e2m1_value(uint8_t code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
 * subnormal (m * 2^-9); S.1111.111 is NaN; no infinities; max 448. */
double oracle_e4m3_value(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Nearest non-negative E4M3 value to v >= 0, ties to the even code, values
 * above the largest finite value (448) saturate to it.  The grid is
 * searched exhaustively; differences of two floats are exact in double. */
uint8_t oracle_e4m3_encode(float v) {
    int best = 0, c;
    double bd, d;
    if (!(v > 0.0f)) return 0;
    if (v >= 448.0f) return 0x7E;
    bd = (double)v;
    for (c = 1; c <= 0x7E; ++c) {
        d = fabs((double)v - oracle_e4m3_value((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bd = d;
        }
    }
    return (uint8_t)best;
}

/* Nearest E2M1 value to q, ties to the even code, |q| > 6 saturates to 6.
 * The sign bit is copied from q, so a negative value that rounds to zero
 * encodes as 0x8 (negative zero). */
uint8_t oracle_e2m1_encode(float q) {
    int best = 0, c, neg = signbit(q) ? 1 : 0;
    double a = fabs((double)q), bd = a, d;
    for (c = 1; c < 8; ++c) {
        d = fabs(a - oracle_e2m1_value((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bd = d;
        }
    }
    return (uint8_t)(best | (neg << 3));
}

void oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_e2m1_encode_array(const float* v, int64_t n, uint8_t* out) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) out[i] = oracle_e2m1_encode(v[i]);
}

/* Signed E4M3 of one value: the sign bit of v, then the nearest magnitude
 * as oracle_e4m3_encode picks it (ties to the even code, saturating at 448).
 * A negative value that rounds to zero encodes as 0x80 (negative zero).
 * This is the element format of the local sliding-window cache, which
 * [Brief] "FP4 cache entries, and why they're safe" keeps in FP8. */
uint8_t oracle_e4m3_encode_signed(float v) {
    return (uint8_t)((signbit(v) ? 0x80 : 0) | oracle_e4m3_encode(fabsf(v)));
}

void oracle_e4m3_encode_signed_array(const float* v, int64_t n, uint8_t* out) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) out[i] = oracle_e4m3_encode_signed(v[i]);
}

/* ------------------------------------------------------- quantize on write */

/* One 512-channel row -> 256 code bytes + 32 scale bytes ([Brief] "FP4 cache
 * entries": E2M1 values, one E4M3 scale per 16 channels, no second-level
 * scale; 256 + 32 = 288 bytes per entry).  Per group g of 16 channels:
 *   amax = max |x_c|;  s_f = amax / 6 (fp32);  sb = E4M3(s_f);  s = value(sb)
 *   code_c = E2M1(x_c / s) (fp32 division), or 0 for every channel when s = 0.
 * Byte i of the codes holds channel 2i in its low nibble, 2i+1 in its high. */
static void quantize_row(const float* x, uint8_t* codes, uint8_t* scales) {
    int g, c;
    for (g = 0; g < OR_NG; ++g) {
        float amax = 0.0f, sf, s;
        uint8_t sb;
        for (c = 0; c < OR_G; ++c) {
            float a = fabsf(x[g * OR_G + c]);
            if (a > amax) amax = a;
        }
        sf = amax / 6.0f;
        sb = oracle_e4m3_encode(sf);
        s = (float)oracle_e4m3_value(sb);
        scales[g] = sb;
        for (c = 0; c < OR_G; c += 2) {
            uint8_t lo = 0, hi = 0;
            if (s != 0.0f) {
                lo = oracle_e2m1_encode(x[g * OR_G + c] / s);
                hi = oracle_e2m1_encode(x[g * OR_G + c + 1] / s);
            }
            codes[(g * OR_G + c) / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

void oracle_quantize_rows(const float* x, int64_t n_rows, int64_t row_stride,
                          uint8_t* codes, uint8_t* scales) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n_rows; ++r)
        quantize_row(x + r * row_stride, codes + r * (OR_D / 2), scales + r * OR_NG);
}

/* x_hat_c = E2M1(code_c) * E4M3(scale_g), exact in double. */
void oracle_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t n_rows, double* out) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n_rows; ++r) {
        int c;
        for (c = 0; c < OR_D; ++c) {
            uint8_t byte = codes[r * (OR_D / 2) + c / 2];
            uint8_t code = (c & 1) ? (byte >> 4) : (byte & 15);
            out[r * OR_D + c] = oracle_e2m1_value(code) * oracle_e4m3_value(scales[r * OR_NG + c / OR_G]);
        }
    }
}

/* ---------------------------------------------------------------- indexer */

/* Indexer score of one cached entry for one query row ([Review] "The Paper":
 * indexer Q times indexer K scores each position; [Brief] "The global
 * branch": the indexer has its own multi-head queries and scores every
 * entry).  The pages give no formula; the reading used is the one the tiny
 * decode workload states, sum over heads of ReLU(q_h . k), with one shared
 * key per entry.  The fp32 operation order is fixed so that selection is
 * reproducible bit for bit:
 *   acc_h = +0; for c = 0..D-1: acc_h = fmaf(q[h][c], k[c], acc_h)
 *   rel_h = acc_h > 0 ? acc_h : +0
 *   score = rel_0 + rel_1 + ... + rel_{H-1}   (left to right, fp32). */
static float index_score(const float* q, int H, int Dk, const float* k) {
    float score = 0.0f;
    int h, c;
    for (h = 0; h < H; ++h) {
        float acc = 0.0f, rel;
        for (c = 0; c < Dk; ++c) acc = fmaf(q[h * Dk + c], k[c], acc);
        rel = acc > 0.0f ? acc : 0.0f;
        score = (h == 0) ? rel : score + rel;
    }
    return score;
}

/* scores[j] for entries j = 0..n-1 of one key array (row stride k_stride). */
void oracle_index_scores(const float* q, int32_t H, int32_t Dk, const float* k, int64_t n,
                         int64_t k_stride, float* scores) {
    int64_t j;
#pragma omp parallel for schedule(static)
    for (j = 0; j < n; ++j) scores[j] = index_score(q, H, Dk, k + j * k_stride);
}

/* ---------------------------------------------------------- selection */

typedef struct {
    float s;
    int64_t j;
} or_cand;

/* (score descending, position ascending) */
static int cmp_rank(const void* a, const void* b) {
    const or_cand* x = (const or_cand*)a;
    const or_cand* y = (const or_cand*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->j < y->j) ? -1 : (x->j > y->j);
}

static int cmp_i64(const void* a, const void* b) {
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x < y) ? -1 : (x > y);
}

/* Top-K ([Review] "The Paper": keep the top 512 indices; [Brief] "The global
 * branch": keep the best entries).  Candidate i has score scores[i] and
 * position pos[i] (pos = NULL: position i).  Candidates with a negative
 * position are skipped.  Order all candidates by (score desc, position
 * asc), keep the first min(K, count), write their positions ascending,
 * pad with -1 up to K.  Returns the number kept. */
int64_t oracle_topk(const float* scores, const int64_t* pos, int64_t n, int32_t K, int32_t* out) {
    or_cand* c = (or_cand*)malloc(sizeof(or_cand) * (size_t)(n > 0 ? n : 1));
    int64_t* keep = (int64_t*)malloc(sizeof(int64_t) * (size_t)(K > 0 ? K : 1));
    int64_t i, m = 0, kept;
    for (i = 0; i < n; ++i) {
        int64_t p = pos ? pos[i] : i;
        if (p < 0) continue;
        c[m].s = scores[i];
        c[m].j = p;
        ++m;
    }
    qsort(c, (size_t)m, sizeof(or_cand), cmp_rank);
    kept = m < K ? m : K;
    for (i = 0; i < kept; ++i) keep[i] = c[i].j;
    qsort(keep, (size_t)kept, sizeof(int64_t), cmp_i64);
    for (i = 0; i < K; ++i) out[i] = (i < kept) ? (int32_t)keep[i] : -1;
    free(c);
    free(keep);
    return kept;
}

/* Hierarchical sparse indexer pool ([Brief] "The hierarchical indexer":
 * group positions into blocks of 8, score a block by its best member, keep
 * the top 2,048 blocks = 16,384 candidates).  Block b covers positions
 * [block*b, min(block*b+block, n)).  Keep the top floor(P/block) blocks by
 * (block score desc, block asc), write their member positions ascending,
 * pad with -1 up to P.  Returns the pool length. */
int64_t oracle_hsi_pool(const float* scores, int64_t n, int32_t block, int32_t P, int32_t* pool) {
    int64_t nb = (n + block - 1) / block, b, i, kept, len = 0;
    int32_t nkeep = P / block;
    or_cand* c = (or_cand*)malloc(sizeof(or_cand) * (size_t)(nb > 0 ? nb : 1));
    int64_t* keep = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nkeep > 0 ? nkeep : 1));
    for (b = 0; b < nb; ++b) {
        float best = scores[b * block];
        for (i = b * block + 1; i < n && i < (b + 1) * block; ++i)
            if (scores[i] > best) best = scores[i];
        c[b].s = best;
        c[b].j = b;
    }
    qsort(c, (size_t)nb, sizeof(or_cand), cmp_rank);
    kept = nb < nkeep ? nb : nkeep;
    for (i = 0; i < kept; ++i) keep[i] = c[i].j;
    qsort(keep, (size_t)kept, sizeof(int64_t), cmp_i64);
    for (b = 0; b < kept; ++b)
        for (i = keep[b] * block; i < n && i < (keep[b] + 1) * block; ++i) pool[len++] = (int32_t)i;
    for (i = len; i < P; ++i) pool[i] = -1;
    free(c);
    free(keep);
    return len;
}

/* ------------------------------------------------------ MXFP4 indexer keys */

/* OCP MXFP4 (OCP Microscaling Formats v1.0, the FP4 E2M1 element type):
 * blocks of 32 consecutive values share one E8M0 scale X = 2^(code - 127)
 * ([Brief] "FP4 cache entries, and why they're safe" assumes indexer keys
 * in this format, one 8-bit scale per 32 values).  Conversion as that
 * specification gives it: X = 2^(floor(log2(max |v|)) - 2), 2 being the
 * largest E2M1 exponent; each element = E2M1(v / X), nearest, ties to even,
 * values past 6 clamped to 6, sign kept.  A block of zeros takes code 0.
 * The scale code is clamped to 0..254 (255 is NaN). */
static int mx_scale_code(float amax) {
    int e, c;
    if (!(amax > 0.0f)) return 0;
    (void)frexp((double)amax, &e); /* amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
    c = (e - 1) - 2 + 127;
    return c < 0 ? 0 : (c > 254 ? 254 : c);
}

double oracle_e8m0_value(uint8_t b) { return b == 255 ? NAN : ldexp(1.0, (int)b - 127); }

/* rows of `dim` values (dim a multiple of 32, row stride `stride` floats) ->
 * codes [n][dim/2] (low nibble = even channel) and scales [n][dim/32]. */
void oracle_mxfp4_quantize_rows(const float* x, int64_t n, int64_t stride, int32_t dim, uint8_t* codes,
                                uint8_t* scales) {
    int64_t r;
#pragma omp parallel for schedule(static)
    for (r = 0; r < n; ++r) {
        const float* xr = x + r * stride;
        int b, c;
        for (b = 0; b < dim / 32; ++b) {
            float amax = 0.0f, X;
            int sc;
            for (c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(xr[32 * b + c]));
            sc = mx_scale_code(amax);
            X = (float)oracle_e8m0_value((uint8_t)sc);
            scales[r * (dim / 32) + b] = (uint8_t)sc;
            for (c = 0; c < 32; c += 2) {
                float q0 = xr[32 * b + c] / X, q1 = xr[32 * b + c + 1] / X;
                codes[r * (dim / 2) + 16 * b + c / 2] =
                    (uint8_t)(oracle_e2m1_encode(q0) | (oracle_e2m1_encode(q1) << 4));
            }
        }
    }
}

/* value of channel c = E2M1(code_c) * E8M0(scale of block c/32), as fp32 (exact) */
void oracle_mxfp4_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t n, int32_t dim, float* out) {
    int64_t r;
    int c;
    for (r = 0; r < n; ++r)
        for (c = 0; c < dim; ++c) {
            uint8_t byte = codes[r * (dim / 2) + c / 2];
            uint8_t code = (c & 1) ? (byte >> 4) : (byte & 15);
            out[r * dim + c] = (float)(oracle_e2m1_value(code) * oracle_e8m0_value(scales[r * (dim / 32) + c / 32]));
        }
}

/* ---------------------------------------------------------- attention */

/* Softmax attention of Hq query heads over ns entries given as dequantized
 * 512-channel rows xh[ns][512] (K = V = the entry).  For each head h:
 *   z_i = scale * sum_c q[h][c] * xh_i[c]          (double)
 *   m = max z;  w_i = exp(z_i - m)
 *   o[h] = sum_i w_i xh_i / sum_i w_i;  lse[h] = m + ln(sum_i w_i)
 * ns = 0: o[h] = 0 and lse[h] = -inf. */
static void attend(const float* q, int32_t Hq, const double* xh, int32_t ns, double scale, float* o, float* lse) {
    double* z = (double*)malloc(sizeof(double) * (size_t)(ns > 0 ? ns : 1));
    double* acc = (double*)malloc(sizeof(double) * OR_D);
    int32_t i, h, c;
    for (h = 0; h < Hq; ++h) {
        double m = -INFINITY, l = 0.0;
        if (ns == 0) {
            for (c = 0; c < OR_D; ++c) o[(int64_t)h * OR_D + c] = 0.0f;
            if (lse) lse[h] = -INFINITY;
            continue;
        }
        for (i = 0; i < ns; ++i) {
            double d = 0.0;
            for (c = 0; c < OR_D; ++c) d += (double)q[(int64_t)h * OR_D + c] * xh[(int64_t)i * OR_D + c];
            z[i] = scale * d;
            if (z[i] > m) m = z[i];
        }
        for (c = 0; c < OR_D; ++c) acc[c] = 0.0;
        for (i = 0; i < ns; ++i) {
            double w = exp(z[i] - m);
            l += w;
            for (c = 0; c < OR_D; ++c) acc[c] += w * xh[(int64_t)i * OR_D + c];
        }
        for (c = 0; c < OR_D; ++c) o[(int64_t)h * OR_D + c] = (float)(acc[c] / l);
        if (lse) lse[h] = (float)(m + log(l));
    }
    free(z);
    free(acc);
}

/* The selected FP4 entries of one row, dequantized: positions idx[i] with
 * 0 <= idx[i] < visible, in list order (duplicates kept), entry j at row j
 * of codes/scales.  x_hat[c] = E2M1(code_c) * E4M3(scale of group c/16).
 * Writes up to K rows into xh; returns how many. */
static int32_t gather_fp4(const uint8_t* codes, const uint8_t* scales, const int32_t* idx, int32_t K,
                          int64_t visible, double* xh) {
    int32_t ns = 0, i, c;
    for (i = 0; i < K; ++i) {
        int64_t j = idx[i];
        if (j < 0 || j >= visible) continue;
        for (c = 0; c < OR_D; ++c) {
            uint8_t byte = codes[j * (OR_D / 2) + c / 2];
            uint8_t code = (c & 1) ? (byte >> 4) : (byte & 15);
            xh[(int64_t)ns * OR_D + c] = oracle_e2m1_value(code) * oracle_e4m3_value(scales[j * OR_NG + c / OR_G]);
        }
        ++ns;
    }
    return ns;
}

/* Sparse attention of one query row ([Review] "The Paper": K and V are the
 * same Main KV entry; the selected entries are attended with the normal
 * attention operation; [Brief] "The global branch": one 512-dim latent per
 * entry shared by every query head): attend() over S = the selected
 * positions j with 0 <= j < visible.  codes/scales point at the row's cache
 * segment (entry j at row j). */
void oracle_attention_row(const float* q, int32_t Hq, const uint8_t* codes, const uint8_t* scales,
                          const int32_t* idx, int32_t K, int64_t visible, double scale,
                          float* o, float* lse) {
    double* xh = (double*)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * OR_D);
    int32_t ns = gather_fp4(codes, scales, idx, K, visible, xh);
    attend(q, Hq, xh, ns, scale, o, lse);
    free(xh);
}

/* Several rows at once (rows are independent): row r reads q + r*Hq*512,
 * its cache segment at row_start[r], idx + r*K, visible[r]. */
void oracle_attention_rows(int32_t R, const float* q, int32_t Hq, const uint8_t* codes,
                           const uint8_t* scales, const int64_t* row_start, const int32_t* idx,
                           int32_t K, const int64_t* visible, double scale, float* o, float* lse) {
    int32_t r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < R; ++r)
        oracle_attention_row(q + (int64_t)r * Hq * OR_D, Hq, codes + row_start[r] * (OR_D / 2),
                             scales + row_start[r] * OR_NG, idx + (int64_t)r * K, K, visible[r], scale,
                             o + (int64_t)r * Hq * OR_D, lse ? lse + (int64_t)r * Hq : NULL);
}

/* The local branch joined with the global one ([Review] "The Paper": every
 * layer runs sliding-window attention over the 128 most recent tokens, and
 * the selected Main KV entries are joined to the window's KV for a single
 * attention; [Brief] "Two attention paths in every layer", "The global
 * branch" and the mode table of "CSA2: most layers don't keep their own
 * cache": each layer keeps its own window; "FP4 cache entries, and why
 * they're safe": the local cache stays in FP8).  One softmax over the union of
 *   - the selected FP4 entries, as oracle_attention_row takes them, and
 *   - the row's window entries: rows win_start .. win_start + n - 1 of
 *     win_codes [*][512] (one signed E4M3 byte per channel, no scale),
 *     n = win_len clamped to [0, 128], value E4M3(byte) per channel;
 * window entries are 512-channel latents with K = V, like Main KV entries. */
void oracle_attention_row_swa(const float* q, int32_t Hq, const uint8_t* codes, const uint8_t* scales,
                              const int32_t* idx, int32_t K, int64_t visible, const uint8_t* win_codes,
                              int64_t win_start, int32_t win_len, double scale, float* o, float* lse) {
    int32_t n = win_len < 0 ? 0 : (win_len > 128 ? 128 : win_len);
    double* xh = (double*)malloc(sizeof(double) * (size_t)(K + n > 0 ? K + n : 1) * OR_D);
    int32_t ns = gather_fp4(codes, scales, idx, K, visible, xh), i, c;
    for (i = 0; i < n; ++i) {
        for (c = 0; c < OR_D; ++c)
            xh[(int64_t)(ns + i) * OR_D + c] = oracle_e4m3_value(win_codes[(win_start + i) * OR_D + c]);
    }
    attend(q, Hq, xh, ns + n, scale, o, lse);
    free(xh);
}

void oracle_attention_rows_swa(int32_t R, const float* q, int32_t Hq, const uint8_t* codes,
                               const uint8_t* scales, const int64_t* row_start, const int32_t* idx, int32_t K,
                               const int64_t* visible, const uint8_t* win_codes, const int64_t* win_start,
                               const int32_t* win_len, double scale, float* o, float* lse) {
    int32_t r;
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < R; ++r)
        oracle_attention_row_swa(q + (int64_t)r * Hq * OR_D, Hq, codes + row_start[r] * (OR_D / 2),
                                 scales + row_start[r] * OR_NG, idx + (int64_t)r * K, K, visible[r], win_codes,
                                 win_start[r], win_len[r], scale, o + (int64_t)r * Hq * OR_D,
                                 lse ? lse + (int64_t)r * Hq : NULL);
}

int32_t oracle_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* threads of the parallel loops above (timing only: results do not depend on it) */
void oracle_set_num_threads(int32_t n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
