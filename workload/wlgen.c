/*
 * Seeded synthetic-input generator: normal weights and activations.
 *
 * This file holds none of the sparse-FFN method's arithmetic. It only
 * produces the random inputs (bf16 weight bundles and fp32 activation
 * vectors) that both the CPU oracle and the HIP path consume.
 *
 * Generator: value i of a stream with 64-bit key k comes from the pair
 * p = i / 2. The pair's 64 random bits are the SplitMix64 output for
 * state k + (p + 1) * 0x9E3779B97F4A7C15 (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014). The
 * top 24 bits give u1 in (0, 1], the low 24 bits give u2 in [0, 1), and
 * the Box-Muller transform (Box and Muller, 1958) turns (u1, u2) into two
 * standard normals z0 = r cos(2 pi u2), z1 = r sin(2 pi u2) with
 * r = sqrt(-2 ln u1), evaluated in single precision. Because each value
 * depends only on (key, i), any slice can be regenerated on its own, in
 * any thread order, with identical bits.
 *
 * bf16 output: the normal times std is rounded to float32, then to bf16
 * with round-to-nearest-even on the float32 bit pattern (the generator
 * never produces NaN or Inf).
 */
#define _GNU_SOURCE
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

#define WL_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t wl_splitmix64(uint64_t state) {
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* The pair p of standard normals of stream `key` (single-precision Box-Muller). */
static inline void wl_normal_pair(uint64_t key, uint64_t p, float* z0, float* z1) {
    const float two_pi = 6.28318530717958647692f;
    uint64_t h = wl_splitmix64(key + (p + 1ULL) * WL_GAMMA);
    float u1 = (float)((h >> 40) + 1ULL) * (1.0f / 16777216.0f); /* (0, 1], exact */
    float u2 = (float)(h & 0xFFFFFFULL) * (1.0f / 16777216.0f);  /* [0, 1), exact */
    float r = sqrtf(-2.0f * logf(u1));
    float s, c;
    sincosf(two_pi * u2, &s, &c);
    *z0 = r * c;
    *z1 = r * s;
}

/* Standard normal number `i` of stream `key`. */
static inline float wl_normal(uint64_t key, uint64_t i) {
    float z0, z1;
    wl_normal_pair(key, i >> 1, &z0, &z1);
    return (i & 1ULL) ? z1 : z0;
}

static inline uint16_t wl_f32_to_bf16_rne(float f) {
    union { float f; uint32_t u; } v;
    v.f = f;
    uint32_t lsb = (v.u >> 16) & 1u;
    return (uint16_t)((v.u + 0x7FFFu + lsb) >> 16);
}

typedef struct {
    void* out;
    int is_bf16;
    uint64_t key, first, count;
    double scale;
} wl_job;

static void* wl_worker(void* arg) {
    wl_job* j = (wl_job*)arg;
    const float sc = (float)j->scale;
    uint64_t i = j->first, end = j->first + j->count, k = 0;
    uint16_t* ob = (uint16_t*)j->out;
    float* of = (float*)j->out;
#define WL_PUT(v)                                              \
    do {                                                       \
        if (j->is_bf16) ob[k] = wl_f32_to_bf16_rne((v) * sc);  \
        else of[k] = (v) * sc;                                 \
        ++k;                                                   \
    } while (0)
    if (i < end && (i & 1ULL)) { WL_PUT(wl_normal(j->key, i)); ++i; }
    for (; i + 1 < end; i += 2) {
        float z0, z1;
        wl_normal_pair(j->key, i >> 1, &z0, &z1);
        WL_PUT(z0);
        WL_PUT(z1);
    }
    if (i < end) { WL_PUT(wl_normal(j->key, i)); ++i; }
#undef WL_PUT
    return NULL;
}

static int wl_fill(void* out, int is_bf16, uint64_t key, uint64_t first, uint64_t count,
                   double scale, int threads) {
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if ((uint64_t)threads > count / 65536 + 1) threads = (int)(count / 65536 + 1);
    pthread_t tid[256];
    wl_job jobs[256];
    uint64_t per = count / (uint64_t)threads, rem = count % (uint64_t)threads, off = 0;
    size_t esz = is_bf16 ? 2 : 4;
    for (int t = 0; t < threads; ++t) {
        uint64_t c = per + ((uint64_t)t < rem ? 1 : 0);
        jobs[t].out = (char*)out + off * esz;
        jobs[t].is_bf16 = is_bf16;
        jobs[t].key = key;
        jobs[t].first = first + off;
        jobs[t].count = c;
        jobs[t].scale = scale;
        off += c;
    }
    int started = 0;
    for (int t = 1; t < threads; ++t) {
        if (pthread_create(&tid[t], NULL, wl_worker, &jobs[t]) != 0) break;
        started = t;
    }
    wl_worker(&jobs[0]);
    for (int t = 1; t <= started; ++t) pthread_join(tid[t], NULL);
    for (int t = started + 1; t < threads; ++t) wl_worker(&jobs[t]); /* create failed: run inline */
    return 0;
}

/* out[k] = bf16(std * z(key, first + k)), k < count. */
int wl_fill_bf16(uint16_t* out, uint64_t key, uint64_t first, uint64_t count, double std,
                 int threads) {
    return wl_fill(out, 1, key, first, count, std, threads);
}

/* out[k] = float(std * z(key, first + k)), k < count. */
int wl_fill_f32(float* out, uint64_t key, uint64_t first, uint64_t count, double std,
                int threads) {
    return wl_fill(out, 0, key, first, count, std, threads);
}

/*
 * Gather bundles without holding the whole store: bundle b of a layer stream
 * is values [b * bundle_elems, (b + 1) * bundle_elems). out[j] = bundle ids[j].
 */
int wl_fill_bundles_bf16(uint16_t* out, uint64_t key, const int32_t* ids, int64_t n,
                         uint64_t bundle_elems, double std) {
    for (int64_t j = 0; j < n; ++j) {
        uint64_t first = (uint64_t)ids[j] * bundle_elems;
        wl_job job = {out + (uint64_t)j * bundle_elems, 1, key, first, bundle_elems, std};
        wl_worker(&job);
    }
    return 0;
}
