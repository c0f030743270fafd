/*
 * wqref — CPU oracle for the mixed-precision weight matmul
 *
 *     C[M,N] = A[M,K] · B[N,K]^T        (C is overwritten: beta = 0)
 *
 * A holds f32 activations, row-major [M,K].  B holds weights, row-major
 * [N,K], stored either as IEEE-754 binary16 ("f16"), as Q8_0 blocks (34
 * bytes per 32 consecutive weights of a row: a little-endian f16 scale d
 * followed by 32 two's-complement int8 codes q; the weight is d*q) or as
 * Q4_0 blocks (18 bytes per 32 weights: the f16 scale d, then 16 bytes
 * whose low nibble holds weight 2i and high nibble weight 2i+1 as unsigned
 * codes u; the weight is (u - 8)*d).
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
 * reference the GPU library is checked against.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the GPU library, and neither uses
 * the other.
 *
 * Passages followed (page title; item on the page):
 *  - lattice-inference 0.9.0, forward/metal_qwen35/inner/dispatch.rs;
 *    doc comment of dispatch_matmul_half: C[M,N] = A[M,K] @ B_half[N,K]^T,
 *    A f32, B f16 widened to f32 before accumulation, C f32.
 *  - same page, dispatch_matmul_q8: Q8_0 weights are [N, K/32 * 34] bytes;
 *    dispatch_gemm_q8: m == 0 or n == 0 is a no-op, K must be > 0 and a
 *    multiple of 32.
 *  - lattice-inference 0.1.2, forward/metal_qwen35.rs; kernel matmul_bt:
 *    B is stored [N,K] and read transposed; kernels gemv_q8_decode and
 *    gemm_q8: block = [f16 scale (2 B)][32 x int8 (32 B)], weight = d*q;
 *    QK8_0 = 32, Q8_0_BLOCK_SIZE = 34 and quantize_row_q8_0 (the quantiser);
 *    f32_to_f16 (round to nearest even, with subnormals) and f16_to_f32.
 *  - lattice-inference 0.1.2 page, kernels gemv_q4_decode, gemm_q4 and
 *    gemm_q4_tiled: Q4_0 block = [f16 scale (2 B)][16 bytes of packed 4-bit
 *    codes], weight 2i from the low and 2i+1 from the high nibble of byte i,
 *    value (nibble - 8) * scale; QK4_0 = 32, Q4_0_BLOCK_SIZE = 18.  (One
 *    dispatch comment on the 0.9.0 page says [N, K/32 * 20] bytes; every
 *    kernel reads 18-byte blocks, which is the reading taken.)
 *  - ferrum-kernels 0.7.7, attention/metal/pipelines.rs; MetalPipelines::gemm:
 *    the same product as sgemm(RowMajor, NoTrans, Trans, alpha=1, beta=0).
 *
 * Arithmetic: every decoded weight is an exact binary value and every product
 * a[m,k] * w[n,k] is exact in double (at most 24 + 19 significant bits), so
 * the only rounding is that of the double sum, about K * 2^-53 relative --
 * far below the f32 tolerance the GPU path is held to.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { WQREF_F16 = 0, WQREF_Q8_0 = 1, WQREF_Q4_0 = 2 };
enum { WQREF_QK = 32, WQREF_BLOCK_BYTES = 34, WQREF_Q4_BLOCK_BYTES = 18 };

/* ------------------------------------------------------------------ f16 -- */

/* Exact value of an IEEE-754 binary16 bit pattern (f16_to_f32 on the
 * lattice-inference 0.1.2 page): sign s, 5-bit biased exponent e, 10-bit
 * fraction f.  e == 0: f * 2^-24 (zero or subnormal); e == 31: inf or NaN;
 * otherwise (1024 + f) * 2^(e - 25), i.e. (1 + f/1024) * 2^(e - 15). */
double wqref_f16_value(uint16_t h) {
    const int s = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24);
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + f), e - 25);
    return s ? -mag : mag;
}

/* f32 -> binary16 bits, round to nearest, ties to even (f32_to_f16 on the
 * lattice-inference 0.1.2 page).  Written at the value level: find the
 * spacing 2^q of half values around |x| (q >= -24, the subnormal spacing),
 * round |x| / 2^q to the nearest integer r with ties to even, and encode
 * r * 2^q.  |x| >= 65520 (the midpoint between 65504, the largest finite
 * half, and 65536) rounds to infinity.  NaN stays NaN with the quiet bit
 * set and the top fraction bits kept, as on the page. */
uint16_t wqref_f16_bits(float x) {
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(x)) {
        uint16_t payload = (uint16_t)((u >> 13) & 0x3ffu);
        return (uint16_t)(sign | 0x7c00u | payload | 0x200u);
    }
    const double ax = fabs((double)x);
    if (isinf(x) || ax >= 65520.0) return (uint16_t)(sign | 0x7c00u);
    if (ax == 0.0) return sign;
    int e2;
    frexp(ax, &e2);          /* ax in [2^(e2-1), 2^e2) */
    int q = (e2 - 1) - 10;   /* spacing of 11-bit significands in that binade */
    if (q < -24) q = -24;    /* below 2^-14 the spacing is the subnormal one */
    const double r = nearbyint(ldexp(ax, -q)); /* exact scaling; RNE rounding */
    if (q == -24) {
        /* r * 2^-24 with r in [0, 2048]: the bit pattern is r itself
         * (subnormals f * 2^-24, then (1024 + f) * 2^-24 for exponent 1,
         * and r = 2048 is 2^-13 = exponent 2, fraction 0). */
        return (uint16_t)(sign | (uint16_t)r);
    }
    int E = q + 10;          /* unbiased exponent of the binade */
    double rr = r;           /* in [1024, 2048] */
    if (rr >= 2048.0) {      /* rounding carried into the next binade */
        rr = 1024.0;
        E += 1;
    }
    if (E > 15) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((uint32_t)rr - 1024u));
}

void wqref_f16_bits_array(const float *x, uint16_t *out, int64_t count) {
    for (int64_t i = 0; i < count; ++i) out[i] = wqref_f16_bits(x[i]);
}

void wqref_f16_value_array(const uint16_t *h, double *out, int64_t count) {
    for (int64_t i = 0; i < count; ++i) out[i] = wqref_f16_value(h[i]);
}

/* ----------------------------------------------------------------- Q8_0 -- */

/* Quantise count f32 values (count % 32 == 0) into count/32 Q8_0 blocks,
 * following quantize_row_q8_0 on the lattice-inference 0.1.2 page, in f32:
 *   amax = max |v| over the block (NaN ignored by the max),
 *   d    = amax / 127,
 *   id   = 1 / d, or 0 when d == 0,
 *   bytes 0..1 = f16(d), little-endian,
 *   q_i  = round(v_i * id) -- round half away from zero -- clamped to
 *          [-127, 127] and stored as two's-complement int8.
 * Returns 0, or -1 if count is negative or not a multiple of 32. */
int wqref_q8_0_quantize(const float *x, uint8_t *out, int64_t count) {
    if (count < 0 || count % WQREF_QK) return -1;
    const int64_t nblocks = count / WQREF_QK;
    for (int64_t b = 0; b < nblocks; ++b) {
        const float *v = x + b * WQREF_QK;
        uint8_t *o = out + b * WQREF_BLOCK_BYTES;
        float amax = 0.0f;
        for (int i = 0; i < WQREF_QK; ++i) amax = fmaxf(amax, fabsf(v[i]));
        const float d = amax / 127.0f;
        const float id = (d != 0.0f) ? 1.0f / d : 0.0f;
        const uint16_t h = wqref_f16_bits(d);
        o[0] = (uint8_t)(h & 0xff);
        o[1] = (uint8_t)(h >> 8);
        for (int i = 0; i < WQREF_QK; ++i) {
            float t = roundf(v[i] * id);
            int qi;
            if (isnan(t))
                qi = 0;
            else if (t < -127.0f)
                qi = -127;
            else if (t > 127.0f)
                qi = 127;
            else
                qi = (int)t;
            o[2 + i] = (uint8_t)(int8_t)qi;
        }
    }
    return 0;
}

/* Exact weight w[n,k] of a Q8_0 matrix with K columns (K % 32 == 0):
 * row n starts at byte n*(K/32)*34, block j = k/32 at +34*j, scale d is the
 * little-endian f16 at block bytes 0..1, q = int8 at block byte 2 + k%32. */
static double q8_0_weight(const uint8_t *b, int64_t K, int64_t n, int64_t k) {
    const int64_t nb = K / WQREF_QK;
    const uint8_t *blk = b + (n * nb + k / WQREF_QK) * WQREF_BLOCK_BYTES;
    const uint16_t h = (uint16_t)(blk[0] | (blk[1] << 8));
    const int8_t q = (int8_t)blk[2 + k % WQREF_QK];
    return wqref_f16_value(h) * (double)q;
}

/* Exact weight w[n,k] of a Q4_0 matrix with K columns (K % 32 == 0):
 * row n starts at byte n*(K/32)*18, block j = k/32 at +18*j, scale d is the
 * little-endian f16 at block bytes 0..1; with i = k%32, the code u is the low
 * nibble of block byte 2 + i/2 when i is even and its high nibble when i is
 * odd, and the weight is (u - 8) * d. */
static double q4_0_weight(const uint8_t *b, int64_t K, int64_t n, int64_t k) {
    const int64_t nb = K / WQREF_QK;
    const uint8_t *blk = b + (n * nb + k / WQREF_QK) * WQREF_Q4_BLOCK_BYTES;
    const uint16_t h = (uint16_t)(blk[0] | (blk[1] << 8));
    const int i = (int)(k % WQREF_QK);
    const uint8_t byte = blk[2 + i / 2];
    const int u = (i % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    return (double)(u - 8) * wqref_f16_value(h);
}

static double weight(const void *b, int fmt, int64_t K, int64_t n, int64_t k) {
    if (fmt == WQREF_F16) return wqref_f16_value(((const uint16_t *)b)[n * K + k]);
    if (fmt == WQREF_Q4_0) return q4_0_weight((const uint8_t *)b, K, n, k);
    return q8_0_weight((const uint8_t *)b, K, n, k);
}

static int check_args(const void *b, int fmt, int64_t N, int64_t K) {
    if (N < 0 || K < 0) return -1;
    if (fmt != WQREF_F16 && fmt != WQREF_Q8_0 && fmt != WQREF_Q4_0) return -1;
    if (fmt != WQREF_F16 && (K == 0 || K % WQREF_QK)) return -1;
    if (!b && N > 0 && K > 0) return -1;
    return 0;
}

/* Decode the whole weight matrix into its exact values, w[n*K + k]. */
int wqref_decode(const void *b, int fmt, int64_t N, int64_t K, double *w) {
    if (check_args(b, fmt, N, K)) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) w[n * K + k] = weight(b, fmt, K, n, k);
    return 0;
}

/* --------------------------------------------------------------- matmul -- */

typedef struct {
    const float *a;
    const void *b;
    int fmt;
    int64_t M, N, K;
    double *c, *bound;
    /* full matrix: rows n in [n0, n1); entries: pairs [n0, n1) of the lists */
    int64_t n0, n1;
    const int64_t *em, *en;
} job_t;

/* One output: s = sum_k a[m,k] * w[n,k] and the tolerance scale
 * 1e-5 * sum_k |a[m,k] * w[n,k]| + 1e-6, with w already decoded. */
static void dot(const float *arow, const double *w, int64_t K, double *s_out, double *bnd_out) {
    double s = 0.0, sa = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const double p = (double)arow[k] * w[k];
        s += p;
        sa += fabs(p);
    }
    *s_out = s;
    *bnd_out = 1e-5 * sa + 1e-6;
}

static void *matmul_worker(void *arg) {
    job_t *j = (job_t *)arg;
    double *w = (double *)malloc(sizeof(double) * (size_t)(j->K > 0 ? j->K : 1));
    if (!w) return (void *)1;
    for (int64_t n = j->n0; n < j->n1; ++n) {
        for (int64_t k = 0; k < j->K; ++k) w[k] = weight(j->b, j->fmt, j->K, n, k);
        for (int64_t m = 0; m < j->M; ++m)
            dot(j->a + m * j->K, w, j->K, &j->c[m * j->N + n], &j->bound[m * j->N + n]);
    }
    free(w);
    return NULL;
}

static void *entries_worker(void *arg) {
    job_t *j = (job_t *)arg;
    double *w = (double *)malloc(sizeof(double) * (size_t)(j->K > 0 ? j->K : 1));
    if (!w) return (void *)1;
    for (int64_t i = j->n0; i < j->n1; ++i) {
        const int64_t m = j->em[i], n = j->en[i];
        for (int64_t k = 0; k < j->K; ++k) w[k] = weight(j->b, j->fmt, j->K, n, k);
        dot(j->a + m * j->K, w, j->K, &j->c[i], &j->bound[i]);
    }
    free(w);
    return NULL;
}

static int run_jobs(job_t *base, int64_t total, int nthreads, void *(*fn)(void *)) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 128) nthreads = 128;
    if (total < nthreads) nthreads = total > 0 ? (int)total : 1;
    job_t jobs[128];
    pthread_t tids[128];
    int started[128] = {0};
    int rc = 0;
    const int64_t per = (total + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *base;
        jobs[t].n0 = per * t < total ? per * t : total;
        jobs[t].n1 = per * (t + 1) < total ? per * (t + 1) : total;
        if (t == nthreads - 1 || pthread_create(&tids[t], NULL, fn, &jobs[t]) != 0) {
            if (fn(&jobs[t]) != NULL) rc = -1;
        } else {
            started[t] = 1;
        }
    }
    for (int t = 0; t < nthreads; ++t) {
        void *ret = NULL;
        if (started[t] && (pthread_join(tids[t], &ret) != 0 || ret != NULL)) rc = -1;
    }
    return rc;
}

/* Full product: c[m*N + n] and bound[m*N + n] for every m < M, n < N.
 * K == 0 (f16 only) gives c = 0.  Returns 0, or -1 on bad arguments. */
int wqref_matmul(const float *a, const void *b, int fmt, int64_t M, int64_t N, int64_t K,
                 double *c, double *bound, int nthreads) {
    if (M < 0 || check_args(b, fmt, N, K)) return -1;
    if (M == 0 || N == 0) return 0;
    if (!c || !bound || (!a && K > 0)) return -1;
    job_t base = {a, b, fmt, M, N, K, c, bound, 0, 0, NULL, NULL};
    return run_jobs(&base, N, nthreads, matmul_worker);
}

/* Selected outputs: c[i], bound[i] for the entries (rows[i], cols[i]). */
int wqref_matmul_entries(const float *a, const void *b, int fmt, int64_t M, int64_t N, int64_t K,
                         const int64_t *rows, const int64_t *cols, int64_t count, double *c,
                         double *bound, int nthreads) {
    if (M < 0 || count < 0 || check_args(b, fmt, N, K)) return -1;
    for (int64_t i = 0; i < count; ++i)
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) return -1;
    if (count == 0) return 0;
    job_t base = {a, b, fmt, M, N, K, c, bound, 0, 0, rows, cols};
    return run_jobs(&base, count, nthreads, entries_worker);
}

/* ------------------------------------------------------------ epilogues -- */

/* SiLU of the pages' silu_mul kernel (lattice-inference 0.1.2 page): the gate
 * value divided by one plus e to the minus gate value, here in double. */
double wqref_silu(double x) { return x / (1.0 + exp(-x)); }

void wqref_silu_array(const double *x, double *out, int64_t count) {
    for (int64_t i = 0; i < count; ++i) out[i] = wqref_silu(x[i]);
}

/* Epilogue on finished product sums, element by element.
 *
 * epi 1, residual: out[i,j] = r[i,j] + s[i,j], with acc = s [M, N] and r the
 *   f32 residual the product is added into (gemm_q1_v7_residual in the
 *   oxibonsai-kernels 0.1.4 page's encode_layer_prefill; add_buf on the
 *   lattice-inference 0.1.2 page).  Tolerance: the product's own bound plus
 *   one f32 rounding of the addition, 2^-23 * (|r| + |s|).
 * epi 2, SwiGLU: acc is [M, 2N], columns 0..N-1 the gate sums g and N..2N-1
 *   the up sums u of the same output (gate rows first in the fused gate||up
 *   weight: dispatch_gemm_at on the lattice-inference 0.9.0 page binds gate at
 *   offset 0 and up at the gate's byte size; dispatch_silu_mul_fused computes
 *   silu(first half) * second half); out[i,j] = silu(g) * u.  Tolerance:
 *   silu' lies in (-0.1, 1.1), so a gate error of at most Bg moves silu(g) by
 *   at most 1.1 Bg; with an up error of at most Bu the stored value is within
 *   1.1 Bg (|u| + Bu) + |silu(g)| Bu of the exact one, plus 2^-20 |out| for the
 *   f32 evaluation of silu and of the product.
 * Returns 0, or -1 on bad arguments. */
int wqref_epilogue(int epi, const double *acc, const double *acc_bound, int64_t M, int64_t N,
                   const float *resid, double *out, double *bound) {
    if (M < 0 || N < 0 || !acc || !acc_bound || !out || !bound) return -1;
    if (epi == 1) {
        if (!resid) return -1;
        for (int64_t i = 0; i < M * N; ++i) {
            const double r = (double)resid[i], s = acc[i];
            out[i] = r + s;
            bound[i] = acc_bound[i] + ldexp(fabs(r) + fabs(s), -23);
        }
        return 0;
    }
    if (epi == 2) {
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j) {
                const int64_t gi = i * 2 * N + j, ui = gi + N;
                const double g = acc[gi], u = acc[ui], bg = acc_bound[gi], bu = acc_bound[ui];
                const double sg = wqref_silu(g);
                out[i * N + j] = sg * u;
                bound[i * N + j] = 1.1 * bg * (fabs(u) + bu) + fabs(sg) * bu + ldexp(fabs(sg * u), -20);
            }
        return 0;
    }
    return -1;
}

/* ---------------------------------------------------------------- top-k -- */

/* Ranking of (logit, token id) candidates, from the TopKCandidate /
 * topk_better definitions on the lattice-inference 0.1.2 page: a higher logit
 * ranks first, equal logits rank by the lower id, and a NaN logit never ranks
 * before anything (the first passes there replace a NaN logit by the sentinel
 * (-inf, UINT_MAX), so it is never selected).  Returns <0 when a ranks first. */
typedef struct {
    double v;
    int64_t id;
} wqref_cand;

static int cand_cmp(const void *pa, const void *pb) {
    const wqref_cand *a = (const wqref_cand *)pa, *b = (const wqref_cand *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->id < b->id) ? -1 : (a->id > b->id) ? 1 : 0;
}

/* The topk best of logits[0..n-1] in rank order: vals[r], ids[r].  NaN logits
 * are left out; when fewer than topk remain, the rest is the sentinel
 * (-inf, 4294967295).  A plain sort of every candidate.  Returns 0, or -1 on
 * bad arguments or memory. */
int wqref_topk(const double *logits, int64_t n, int64_t topk, double *vals, int64_t *ids) {
    if (n < 0 || topk < 0 || (n > 0 && !logits) || (topk > 0 && (!vals || !ids))) return -1;
    wqref_cand *c = (wqref_cand *)malloc(sizeof(wqref_cand) * (size_t)(n > 0 ? n : 1));
    if (!c) return -1;
    int64_t cnt = 0;
    for (int64_t i = 0; i < n; ++i)
        if (!isnan(logits[i])) {
            c[cnt].v = logits[i];
            c[cnt].id = i;
            ++cnt;
        }
    qsort(c, (size_t)cnt, sizeof(wqref_cand), cand_cmp);
    for (int64_t r = 0; r < topk; ++r) {
        vals[r] = r < cnt ? c[r].v : -INFINITY;
        ids[r] = r < cnt ? c[r].id : (int64_t)4294967295LL;
    }
    free(c);
    return 0;
}

/* ------------------------------------------------------ decode attention -- */

/* Decode (one query token) grouped-query attention, as the lattice-inference
 * 0.1.2 page's decode_attention / decode_attention_flash_partial +
 * decode_attention_flash_reduce compute it: q is [Hq, D] f32; the K and V
 * caches are [L, Hkv * D] (token-major, head h of token t at t * Hkv * D +
 * h * D), f32 (kvfmt 0) or f16 bit patterns (kvfmt 1, the page's f16-KV
 * variant); query head h reads KV head h / G with G = Hq / Hkv.  For each h:
 * s_t = scale * sum_d q[h, d] k[t, d], p = softmax over t < L of s (written
 * here as exp(s_t - max s) / sum, the same value), out[h, d] = sum_t p_t
 * v[t, d].  L = 0 gives 0 (the reduce pass's l > 0 ? acc / l : 0).
 *
 * Tolerance per output: with B_t = |scale| (1e-5 sum_d |q_d k_td| + 1e-6)
 * the product tolerance of each score, every p_t moves by at most a factor
 * exp(+-2 max_t B_t); so |out - out_ref| <= (expm1(2 max_t B_t) + 1e-5)
 * sum_t p_t |v_td| + 1e-6, the 1e-5 term covering the f32 exponentials and
 * sums.  Returns 0, or -1 on bad arguments or memory. */
static double kv_value(const void *c, int kvfmt, int64_t i) {
    return kvfmt == 1 ? wqref_f16_value(((const uint16_t *)c)[i]) : (double)((const float *)c)[i];
}

int wqref_decode_attention(const float *q, const void *k, const void *v, int kvfmt, int64_t L, int64_t D,
                           int64_t Hq, int64_t Hkv, float scale, double *out, double *bound) {
    if (L < 0 || D <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || (kvfmt != 0 && kvfmt != 1)) return -1;
    if (!q || !out || !bound || (L > 0 && (!k || !v))) return -1;
    const int64_t G = Hq / Hkv, kv_dim = Hkv * D;
    double *s = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double *b = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    if (!s || !b) {
        free(s);
        free(b);
        return -1;
    }
    for (int64_t h = 0; h < Hq; ++h) {
        const int64_t kvh = h / G;
        double smax = -INFINITY, bmax = 0.0;
        for (int64_t t = 0; t < L; ++t) {
            double dot = 0.0, mag = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                const double p = (double)q[h * D + d] * kv_value(k, kvfmt, t * kv_dim + kvh * D + d);
                dot += p;
                mag += fabs(p);
            }
            s[t] = (double)scale * dot;
            b[t] = fabs((double)scale) * (1e-5 * mag + 1e-6);
            if (s[t] > smax) smax = s[t];
            if (b[t] > bmax) bmax = b[t];
        }
        double z = 0.0;
        for (int64_t t = 0; t < L; ++t) {
            s[t] = exp(s[t] - smax); /* unnormalised weight */
            z += s[t];
        }
        for (int64_t d = 0; d < D; ++d) {
            double acc = 0.0, mag = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const double vv = kv_value(v, kvfmt, t * kv_dim + kvh * D + d);
                acc += s[t] * vv;
                mag += s[t] * fabs(vv);
            }
            out[h * D + d] = L > 0 ? acc / z : 0.0;
            bound[h * D + d] = (L > 0 ? (expm1(2.0 * bmax) + 1e-5) * (mag / z) : 0.0) + 1e-6;
        }
    }
    free(s);
    free(b);
    return 0;
}
