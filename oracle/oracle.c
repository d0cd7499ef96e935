/*
 * oracle.c -- plain fp64 CPU oracle for one flash-decoding attention step.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may build, load or call this file.  It shares no code,
 * header, table or constant with the HIP library, and it is written to be read against the
 * pages, not to be fast: every score, weight and output element is formed in IEEE double,
 * straight from the definition, in token order.
 *
 * Sources (pages; each function names the passage it follows):
 *   [FA]  "SGLang Prefill 性能优化：用 GPU Trace 剖析 FlashAttention 内核瓶颈", section 2.2:
 *         block score s = q . k^T * scale, softmax over the keys, output = weights . V.
 *   [FD]  "从 SGLang Kernel源码到 GPU Trace：DeepSeek V4.1 Flash-Decode", section 3.1:
 *         ragged batch -- each sequence's keys are located by a start index and its own
 *         seq_len; work follows seq_len[i], never the padded maximum.
 *   [CH15] "第 15 章 · GPU Profiling 与 LLM 推理优化实战", section 15.26 (paged address:
 *         physical page from block_table[b * max_pages + logical_page], then
 *         ((page * page_size + offset) * H + h) * D + d), section 15.11 (quantised KV with
 *         per-token k/v scales, dequantised inside the scan) and section 15.12 (one KV head
 *         serves group = QH / KVH query heads).
 *
 * Readings where the pages are silent:
 *   - q head h reads kv head h / (QH / KVH).
 *   - FP8 means OCP E4M3FN; a dequantised element is decode(byte) * scale, the scale being
 *     one fp32 per tensor or one fp32 per (token, kv head) stored like the cache rows.  INT8 KV
 *     ([CH15] 15.11) is the same with two's-complement int8 codes.
 *   - The empty sequence (seq_len 0) gives out = 0 and lse = -inf.
 *   - lse is the natural log of sum_t exp(s_t).
 *   - A window of nq query tokens per sequence ([FD] 2.2 tiles several query rows per block;
 *     [CH15] 15.21 verifies a window of draft tokens in one pass): the window's tokens are the
 *     last nq tokens already in the cache, so query row m (0-based) sits at position
 *     seq_len - nq + m and attends to tokens [0, seq_len - nq + m]; a row whose range is empty
 *     (seq_len < nq - m) gives out = 0 and lse = -inf.  nq = 1 is the ordinary decode step.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* dtype and scale codes of this file's own interface */
enum { ORC_F16 = 1, ORC_BF16 = 2, ORC_E4M3 = 3, ORC_I8 = 4 };
enum { ORC_SCALE_NONE = 0, ORC_SCALE_TENSOR = 1, ORC_SCALE_TOKEN_HEAD = 2 };

typedef struct {
    const void *q;             /* [batch][hq][d], q_dtype bits                                   */
    const void *k_cache;       /* rows of [hkv][d]: paged rows = block * block_size + slot       */
    const void *v_cache;
    const int32_t *block_table;/* [batch][max_blocks] or NULL (contiguous mode)                  */
    const int32_t *kv_start;   /* [batch] first row (contiguous mode) or NULL                    */
    const int32_t *seq_len;    /* [batch]                                                        */
    const float *k_scale;      /* NULL, [1] or per row [rows][hkv]                              */
    const float *v_scale;
    int32_t batch, hq, hkv, d;
    int32_t block_size, max_blocks;
    int32_t q_dtype, kv_dtype, scale_mode;
    double softmax_scale;
    int32_t nq;                /* query tokens per sequence (0 or 1: one); q is [batch][nq][hq][d] */
} orc_problem;

static int nq_of(const orc_problem *p) { return p->nq > 1 ? p->nq : 1; }

/* --- element decoders (exact conversions to double, written from the format definitions) --- */

/* OCP 8-bit floating point, E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
 * exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity. */
double orc_e4m3_to_double(uint8_t byte) {
    int sign = byte >> 7, e = (byte >> 3) & 0xF, m = byte & 0x7;
    double mag;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
double orc_f16_to_double(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double mag;
    if (e == 0x1F) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)m, -24);
    else mag = ldexp(1.0 + (double)m / 1024.0, e - 15);
    return sign ? -mag : mag;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 mantissa bits. */
double orc_bf16_to_double(uint16_t h) {
    int sign = h >> 15, e = (h >> 7) & 0xFF, m = h & 0x7F;
    double mag;
    if (e == 0xFF) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)m, -133);
    else mag = ldexp(1.0 + (double)m / 128.0, e - 127);
    return sign ? -mag : mag;
}

static double load_elem(const void *base, size_t idx, int dtype) {
    switch (dtype) {
    case ORC_F16: return orc_f16_to_double(((const uint16_t *)base)[idx]);
    case ORC_BF16: return orc_bf16_to_double(((const uint16_t *)base)[idx]);
    case ORC_E4M3: return orc_e4m3_to_double(((const uint8_t *)base)[idx]);
    case ORC_I8: return (double)((const int8_t *)base)[idx];  /* [CH15] 15.11: int8 codes x scale */
    default: return NAN;
    }
}

/* Row of the cache ([rows][hkv][d] view) holding token t of sequence b.
 * Paged: [CH15] 15.26 -- page = block_table[b * max_blocks + t / block_size], slot = t % block_size.
 * Contiguous: [FD] 3.1 -- the sequence starts at kv_start[b]. */
static int64_t token_row(const orc_problem *p, int b, int t) {
    if (p->block_table) {
        int32_t page = p->block_table[(int64_t)b * p->max_blocks + t / p->block_size];
        return (int64_t)page * p->block_size + t % p->block_size;
    }
    return (int64_t)p->kv_start[b] + t;
}

/* Dequantisation scale of (row, kv head g) -- [CH15] 15.11 (per-token scales read with the payload). */
static double row_scale(const float *s, int mode, int64_t row, int hkv, int g) {
    if (mode == ORC_SCALE_TENSOR) return (double)s[0];
    if (mode == ORC_SCALE_TOKEN_HEAD) return (double)s[row * hkv + g];
    return 1.0;
}

/* Unnormalised softmax state of query head h of sequence b over tokens [t0, t1):
 *   m = max_t s_t,  l = sum_t exp(s_t - m),  acc[:] = sum_t exp(s_t - m) * V[t][:]
 * with s_t = softmax_scale * sum_d q[d] * K[t][d]  ([FA] 2.2).  Subtracting m is exact in real
 * arithmetic (it cancels in acc / l); it only keeps exp() finite.  An empty range gives
 * m = -inf, l = 0, acc = 0.  Returns 0, or -1 on a bad argument. */
int orc_attend_range_q(const orc_problem *p, int b, int mq, int h, int t0, int t1,
                       double *m_out, double *l_out, double *acc) {
    const int d = p->d, hkv = p->hkv, group = p->hq / p->hkv, nq = nq_of(p);
    const int g = h / group;                               /* [CH15] 15.12 */
    double *s, *qv, m = -INFINITY, l = 0.0;
    if (b < 0 || b >= p->batch || mq < 0 || mq >= nq || h < 0 || h >= p->hq || t0 < 0 || t1 < t0)
        return -1;
    for (int i = 0; i < d; i++) acc[i] = 0.0;
    if (t1 == t0) { *m_out = -INFINITY; *l_out = 0.0; return 0; }
    s = (double *)malloc(sizeof(double) * (size_t)(t1 - t0));
    qv = (double *)malloc(sizeof(double) * (size_t)d);
    for (int i = 0; i < d; i++)
        qv[i] = load_elem(p->q, (((size_t)b * nq + mq) * p->hq + h) * d + i, p->q_dtype);
    /* scores */
    for (int t = t0; t < t1; t++) {
        int64_t row = token_row(p, b, t);
        double ks = row_scale(p->k_scale, p->scale_mode, row, hkv, g), dot = 0.0;
        size_t base = ((size_t)row * hkv + g) * d;
        for (int i = 0; i < d; i++) dot += qv[i] * (load_elem(p->k_cache, base + i, p->kv_dtype) * ks);
        s[t - t0] = p->softmax_scale * dot;
        if (s[t - t0] > m) m = s[t - t0];
    }
    /* weights and weighted sum of V */
    for (int t = t0; t < t1; t++) {
        int64_t row = token_row(p, b, t);
        double vs = row_scale(p->v_scale, p->scale_mode, row, hkv, g);
        double w = exp(s[t - t0] - m);
        size_t base = ((size_t)row * hkv + g) * d;
        l += w;
        for (int i = 0; i < d; i++) acc[i] += w * (load_elem(p->v_cache, base + i, p->kv_dtype) * vs);
    }
    free(s);
    free(qv);
    *m_out = m;
    *l_out = l;
    return 0;
}

/* The same for query row 0 (the only row of an ordinary decode step). */
int orc_attend_range(const orc_problem *p, int b, int h, int t0, int t1,
                     double *m_out, double *l_out, double *acc) {
    return orc_attend_range_q(p, b, 0, h, t0, t1, m_out, l_out, acc);
}

/* Merge of partial states over disjoint token ranges of one (sequence, head) into the final
 * output.  This is the recurrence of [FA] 2.2 applied to whole partial states: with
 * M = max_i m_i over the non-empty parts, w_i = exp(m_i - M),
 *   out = sum_i w_i acc_i / sum_i w_i l_i,   lse = M + ln(sum_i w_i l_i).
 * Empty parts (l_i = 0) are skipped; all parts empty gives out = 0, lse = -inf. */
void orc_merge(int nparts, const double *m, const double *l, const double *acc, int d,
               double *out, double *lse) {
    double M = -INFINITY, L = 0.0;
    for (int i = 0; i < d; i++) out[i] = 0.0;
    for (int j = 0; j < nparts; j++)
        if (l[j] > 0.0 && m[j] > M) M = m[j];
    if (M == -INFINITY) { *lse = -INFINITY; return; }
    for (int j = 0; j < nparts; j++) {
        double w;
        if (!(l[j] > 0.0)) continue;
        w = exp(m[j] - M);
        L += w * l[j];
        for (int i = 0; i < d; i++) out[i] += w * acc[(size_t)j * d + i];
    }
    for (int i = 0; i < d; i++) out[i] /= L;
    *lse = M + log(L);
}

/* ---------------- full step: softmax(q K^T * scale) V for every (sequence, q head) -------------- */

typedef struct {
    const orc_problem *p;
    const uint8_t *seq_mask;
    double *out, *lse;
    int tid, nthreads, status;
} orc_job;

/* One (b, query row mq, h): out = acc / l over tokens [0, seq_len[b] - nq + mq + 1),
 * lse = m + ln l  ([FA] 2.2; [FD] 3.1; the window reading in the header). */
static int attend_one(const orc_problem *p, int b, int mq, int h, double *out, double *lse) {
    double m, l;
    const int len = p->seq_len[b];
    const int n = len - nq_of(p) + mq + 1;
    if (len < 0) return -1;
    if (n <= 0) {
        for (int i = 0; i < p->d; i++) out[i] = 0.0;
        *lse = -INFINITY;
        return 0;
    }
    if (orc_attend_range_q(p, b, mq, h, 0, n, &m, &l, out)) return -1;
    for (int i = 0; i < p->d; i++) out[i] /= l;
    *lse = m + log(l);
    return 0;
}

static void *worker(void *arg) {
    orc_job *job = (orc_job *)arg;
    const orc_problem *p = job->p;
    const long rows = (long)nq_of(p) * p->hq;  /* (query row, head) pairs per sequence */
    long items = (long)p->batch * rows;
    for (long it = job->tid; it < items; it += job->nthreads) {
        int b = (int)(it / rows), mq = (int)(it % rows / p->hq), h = (int)(it % p->hq);
        if (job->seq_mask && !job->seq_mask[b]) continue;
        if (attend_one(p, b, mq, h, job->out + (size_t)it * p->d, job->lse + it)) job->status = -1;
    }
    return NULL;
}

/* out[batch][nq][hq][d], lse[batch][nq][hq] (both double).  seq_mask (optional) selects the sequences to
 * compute; the others are left untouched.  Work is spread over nthreads POSIX threads by
 * (sequence, head) pairs.  Returns 0, or -1 on a bad argument. */
int orc_decode_attention(const orc_problem *p, const uint8_t *seq_mask, double *out, double *lse,
                         int nthreads) {
    pthread_t *th;
    orc_job *jobs;
    int status = 0;
    if (!p || p->batch <= 0 || p->hq <= 0 || p->hkv <= 0 || p->hq % p->hkv || p->d <= 0) return -1;
    if (p->block_table && p->block_size <= 0) return -1;
    if (!p->block_table && !p->kv_start) return -1;
    if (nthreads < 1) nthreads = 1;
    th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    jobs = (orc_job *)calloc((size_t)nthreads, sizeof(orc_job));
    for (int i = 0; i < nthreads; i++) {
        jobs[i] = (orc_job){p, seq_mask, out, lse, i, nthreads, 0};
        if (i) pthread_create(&th[i], NULL, worker, &jobs[i]);
    }
    worker(&jobs[0]);
    for (int i = 1; i < nthreads; i++) pthread_join(th[i], NULL);
    for (int i = 0; i < nthreads; i++) status |= jobs[i].status;
    free(th);
    free(jobs);
    return status;
}

/* ======================================================================================
 * KV-cache append of the current token: the step that precedes the scan.
 *
 * Sources: [CH15] 15.9 (paged cache writes; its exercise 4 adds a single-token decode append),
 * 15.11 (quantised KV with per-token k/v scales) and 15.18 (row-wise absmax -> scale -> quantise).
 * Readings where the pages are silent: a row is one token's D values of one kv head; its scale is
 * amax|x| / 448 (448 = largest E4M3 value; 1 when the row is all zeros); the quantised value is x /
 * scale, clamped to [-448, 448], rounded to the nearest E4M3 value with ties to an even mantissa.
 * The decision is taken in fp32 -- scale and quotient are fp32 operations -- the precision the
 * kernels quantise in; only the final rounding to E4M3 is done here by exact
 * search.  f16 / bf16 caches store the fp32 value rounded to nearest-even.
 * ====================================================================================== */

/* Nearest finite E4M3 code to x (clamped to +-448), ties to the even code: a plain search over
 * the 127 non-negative finite codes in exact double arithmetic.  NaN gives the NaN code 0x7F;
 * the sign of x (including -0) goes to the sign bit. */
uint8_t orc_e4m3_encode(float x) {
    if (x != x) return 0x7F;
    const int neg = signbit(x) ? 1 : 0;
    double a = fabs((double)x);
    if (a > 448.0) a = 448.0;
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c <= 0x7E; c++) {
        const double d = fabs(orc_e4m3_to_double((uint8_t)c) - a);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)(best | (neg << 7));
}

/* Round a finite double to the nearest value with `mant` explicit significand bits and minimum
 * normal exponent `emin` (IEEE round-to-nearest-even, gradual underflow), by exact scaling:
 * the quantum at x's binade is 2^(e - mant); x / quantum is exact and rint() rounds half to even. */
static double round_to_format(double x, int mant, int emin) {
    if (x == 0.0 || x != x || isinf(x)) return x;
    int e;
    frexp(x, &e);  /* x = f * 2^e, 0.5 <= |f| < 1, so the binade exponent is e - 1 */
    int be = e - 1;
    if (be < emin) be = emin;
    const double quantum = ldexp(1.0, be - mant);
    return rint(x / quantum) * quantum;
}

/* fp32 -> IEEE binary16 bits, round to nearest even (overflow to infinity). */
uint16_t orc_f16_encode(float x) {
    const double r = round_to_format((double)x, 10, -14);
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (r != r) return 0x7E00;
    const double a = fabs(r);
    if (a >= 65536.0) return sign | 0x7C00;  /* 65520 and above round to infinity */
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    const int be = e - 1;
    if (be < -14) return sign | (uint16_t)(a / ldexp(1.0, -24));           /* subnormal */
    return sign | (uint16_t)((be + 15) << 10) | (uint16_t)((a / ldexp(1.0, be) - 1.0) * 1024.0);
}

/* fp32 -> bfloat16 bits, round to nearest even. */
uint16_t orc_bf16_encode(float x) {
    const double r = round_to_format((double)x, 7, -126);
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (r != r) return 0x7FC0;
    const double a = fabs(r);
    if (a >= ldexp(1.0, 128)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int e;
    frexp(a, &e);
    const int be = e - 1;
    if (be < -126) return sign | (uint16_t)(a / ldexp(1.0, -133));         /* subnormal */
    return sign | (uint16_t)((be + 127) << 7) | (uint16_t)((a / ldexp(1.0, be) - 1.0) * 128.0);
}

/* One row, E4M3 ([CH15] 15.18): with scale_in > 0 use it (per-tensor scale), else scale =
 * amax / 448 in fp32 (1 for an all-zero row).  byte[i] = encode(clamp(x[i] / scale, +-448)).
 * Returns the scale used. */
float orc_quantize_row_e4m3(const float *x, int n, float scale_in, uint8_t *out) {
    float scale = scale_in;
    if (!(scale_in > 0.0f)) {
        float amax = 0.0f;
        for (int i = 0; i < n; i++) {
            const float a = fabsf(x[i]);
            if (a > amax) amax = a;
        }
        scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    }
    for (int i = 0; i < n; i++) {
        float q = x[i] / scale;
        if (q > 448.0f) q = 448.0f;
        if (q < -448.0f) q = -448.0f;
        out[i] = orc_e4m3_encode(q);
    }
    return scale;
}

/* One row, INT8 ([CH15] 15.18 row-wise absmax, int8 quant; [CH15] 15.11 per-token scales): with
 * scale_in > 0 use it, else scale = amax / 127 in fp32 (1 for an all-zero row); code[i] = the
 * integer nearest to x[i] / scale (fp32 quotient; ties to even), clamped to [-127, 127].
 * Returns the scale used. */
float orc_quantize_row_i8(const float *x, int n, float scale_in, int8_t *out) {
    float scale = scale_in;
    if (!(scale_in > 0.0f)) {
        float amax = 0.0f;
        for (int i = 0; i < n; i++) {
            const float a = fabsf(x[i]);
            if (a > amax) amax = a;
        }
        scale = amax > 0.0f ? amax / 127.0f : 1.0f;
    }
    for (int i = 0; i < n; i++) {
        double q = rint((double)(x[i] / scale));  /* fp32 quotient, exact in double; half to even */
        if (q > 127.0) q = 127.0;
        if (q < -127.0) q = -127.0;
        out[i] = (int8_t)q;
    }
    return scale;
}

typedef struct {
    const float *k_new;         /* [batch][hkv][d] fp32 (f16 / bf16 inputs converted exactly)    */
    const float *v_new;
    void *k_cache;              /* rows of [hkv][d], kv_dtype                                      */
    void *v_cache;
    float *k_scale;             /* E4M3: [1] (per-tensor, read) or [rows][hkv] (per token, written) */
    float *v_scale;
    const int32_t *block_table; /* [batch][max_blocks] or NULL (contiguous mode)                  */
    const int32_t *kv_start;    /* [batch] or NULL                                                 */
    const int32_t *pos;         /* [batch] token index to write; < 0 skips the sequence           */
    int32_t batch, hkv, d, block_size, max_blocks, kv_dtype, scale_mode;
} orc_append;

/* Write each sequence's new K and V rows into the row of token pos[b] (the [CH15] 15.26 paged
 * address, or kv_start[b] + pos[b]).  Returns 0, or -1 on a bad argument. */
int orc_kv_append(const orc_append *a) {
    if (!a || a->batch <= 0 || a->hkv <= 0 || a->d <= 0) return -1;
    if (!a->block_table && !a->kv_start) return -1;
    if (a->block_table && a->block_size <= 0) return -1;
    for (int b = 0; b < a->batch; b++) {
        const int t = a->pos[b];
        if (t < 0) continue;
        int64_t row;
        if (a->block_table) {
            const int32_t page = a->block_table[(int64_t)b * a->max_blocks + t / a->block_size];
            row = (int64_t)page * a->block_size + t % a->block_size;
        } else {
            row = (int64_t)a->kv_start[b] + t;
        }
        for (int g = 0; g < a->hkv; g++) {
            for (int which = 0; which < 2; which++) {
                const float *x = (which ? a->v_new : a->k_new) + ((size_t)b * a->hkv + g) * a->d;
                void *cache = which ? a->v_cache : a->k_cache;
                float *sc = which ? a->v_scale : a->k_scale;
                const size_t base = ((size_t)row * a->hkv + g) * a->d;
                if (a->kv_dtype == ORC_E4M3) {
                    if (a->scale_mode == ORC_SCALE_TENSOR) {
                        orc_quantize_row_e4m3(x, a->d, sc[0], (uint8_t *)cache + base);
                    } else if (a->scale_mode == ORC_SCALE_TOKEN_HEAD) {
                        sc[row * a->hkv + g] = orc_quantize_row_e4m3(x, a->d, 0.0f, (uint8_t *)cache + base);
                    } else {
                        return -1;
                    }
                } else if (a->kv_dtype == ORC_I8) {
                    if (a->scale_mode == ORC_SCALE_TENSOR) {
                        orc_quantize_row_i8(x, a->d, sc[0], (int8_t *)cache + base);
                    } else if (a->scale_mode == ORC_SCALE_TOKEN_HEAD) {
                        sc[row * a->hkv + g] = orc_quantize_row_i8(x, a->d, 0.0f, (int8_t *)cache + base);
                    } else {
                        return -1;
                    }
                } else if (a->kv_dtype == ORC_F16 || a->kv_dtype == ORC_BF16) {
                    uint16_t *dst = (uint16_t *)cache + base;
                    for (int i = 0; i < a->d; i++)
                        dst[i] = a->kv_dtype == ORC_F16 ? orc_f16_encode(x[i]) : orc_bf16_encode(x[i]);
                } else {
                    return -1;
                }
            }
        }
    }
    return 0;
}
