/*
 * wqgen — seeded synthetic inputs for the f16 / Q8_0 weight matmul.
 *
 * This module is shared input plumbing: it draws the f32 activations and the
 * f32 weights that both the CPU oracle and the GPU library consume.  It holds
 * none of the matmul's arithmetic (no f16 rounding, no Q8_0 quantisation, no
 * dot products); each side encodes and multiplies with its own code.
 *
 * Generator: counter-based SplitMix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  Output i of a stream with
 * key s is mix64(s + (i + 1) * GAMMA), i.e. the i-th SplitMix64 output
 * started from state s.  Being counter-based, any slice of a stream can be
 * drawn on its own and in parallel, with the same values as a serial draw.
 *
 * Normal variates: Box–Muller (Box & Muller, 1958) in double precision.
 * Element 2p uses r*cos(t) and element 2p+1 uses r*sin(t), where
 * u1 = U(2p), u2 = U(2p+1), r = sqrt(-2 ln u1), t = 2*pi*u2, and
 * U(i) = ((x_i >> 11) + 1) * 2^-53 lies in (0, 1].  The double value
 * mean + std * z is rounded to float (round-to-nearest-even).
 *
 * Stream key for (seed, stream): mix64(mix64(seed) ^ (stream + 1) * GAMMA).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define WQGEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

uint64_t wqgen_stream_key(uint64_t seed, uint64_t stream) {
    return mix64(mix64(seed) ^ ((stream + 1) * WQGEN_GAMMA));
}

/* i-th raw 64-bit output of the stream with the given key. */
uint64_t wqgen_u64(uint64_t key, uint64_t i) {
    return mix64(key + (i + 1) * WQGEN_GAMMA);
}

/* out[i] = output offset + i of stream (seed, stream), for i < count. */
int wqgen_u64_fill(uint64_t *out, uint64_t count, uint64_t seed, uint64_t stream, uint64_t offset) {
    if (count && !out) return -1;
    const uint64_t key = wqgen_stream_key(seed, stream);
    for (uint64_t i = 0; i < count; ++i) out[i] = wqgen_u64(key, offset + i);
    return 0;
}

static inline double unit_open0(uint64_t x) {
    return (double)((x >> 11) + 1) * (1.0 / 9007199254740992.0); /* 2^-53 */
}

/* Standard normal variate number e of the stream (e >= 0). */
double wqgen_normal_at(uint64_t key, uint64_t e) {
    const uint64_t p = e >> 1;
    const double u1 = unit_open0(wqgen_u64(key, 2 * p));
    const double u2 = unit_open0(wqgen_u64(key, 2 * p + 1));
    const double r = sqrt(-2.0 * log(u1));
    const double t = 6.283185307179586476925286766559 * u2;
    return (e & 1) ? r * sin(t) : r * cos(t);
}

typedef struct {
    float *out;
    uint64_t begin, end; /* element range [begin, end) of out */
    uint64_t key, offset;
    double mean, std;
} fill_job;

static void *fill_worker(void *arg) {
    fill_job *j = (fill_job *)arg;
    for (uint64_t i = j->begin; i < j->end; ++i)
        j->out[i] = (float)(j->mean + j->std * wqgen_normal_at(j->key, j->offset + i));
    return NULL;
}

/*
 * Fill out[0..count) with elements offset..offset+count-1 of the normal
 * stream (seed, stream), scaled to N(mean, std^2).  nthreads <= 0 means 1.
 * Returns 0 on success, -1 on bad arguments or thread failure.
 */
int wqgen_normal_f32(float *out, uint64_t count, uint64_t seed, uint64_t stream,
                     uint64_t offset, double mean, double std, int nthreads) {
    if (count == 0) return 0;
    if (!out) return -1;
    if (nthreads <= 0) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((uint64_t)nthreads > count / 4096 + 1) nthreads = (int)(count / 4096 + 1);
    const uint64_t key = wqgen_stream_key(seed, stream);
    fill_job jobs[256];
    pthread_t tids[256];
    int started[256] = {0};
    const uint64_t per = (count + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        uint64_t b = per * (uint64_t)t, e = b + per;
        if (b > count) b = count;
        if (e > count) e = count;
        jobs[t] = (fill_job){out, b, e, key, offset, mean, std};
        if (t == nthreads - 1 || pthread_create(&tids[t], NULL, fill_worker, &jobs[t]) != 0) {
            fill_worker(&jobs[t]); /* last slice (or a failed spawn) runs here */
        } else {
            started[t] = 1;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (started[t] && pthread_join(tids[t], NULL) != 0) rc = -1;
    return rc;
}
