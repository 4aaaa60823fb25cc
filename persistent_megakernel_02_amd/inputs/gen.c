/*
 * Seeded synthetic inputs for the decode step: bf16 weights, prompt tokens and
 * pre-filled KV contexts.  This file holds no arithmetic of the decode method;
 * both the CPU oracle (through its tests) and the HIP path consume what it
 * produces, so they always see identical inputs.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  A stream with seed k yields draw i as
 * mix(k + (i + 1) * 0x9E3779B97F4A7C15), so any element can be produced
 * independently of the others (counter based), and the work splits across
 * threads without changing a single value.
 *
 * Normals: Box-Muller on draws (2j, 2j+1) gives the pair (z_{2j}, z_{2j+1}).
 * Values are formed in double as mean + std * z, rounded to fp32 by the C cast
 * (round to nearest even) and then to bf16 (round to nearest even).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t gen_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t gen_draw(uint64_t key, uint64_t i) {
    return gen_mix(key + (i + 1) * GEN_GAMMA);
}

uint64_t gen_key(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b) {
    uint64_t k = gen_mix(seed + GEN_GAMMA);
    k = gen_mix(k ^ (tag * GEN_GAMMA));
    k = gen_mix(k ^ ((a + 1) * 0xD1B54A32D192ED03ULL));
    k = gen_mix(k ^ ((b + 1) * 0x8CB92BA72F3D8DD7ULL));
    return k;
}

uint64_t gen_u64(uint64_t key, uint64_t i) { return gen_draw(key, i); }

static inline uint16_t gen_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline void gen_pair(uint64_t key, uint64_t j, double* z0, double* z1) {
    const double two53 = 1.0 / 9007199254740992.0;
    double u1 = (double)((gen_draw(key, 2 * j) >> 11) + 1) * two53;  /* (0, 1] */
    double u2 = (double)(gen_draw(key, 2 * j + 1) >> 11) * two53;    /* [0, 1) */
    double r = sqrt(-2.0 * log(u1));
    double t = 6.283185307179586476925 * u2;
    *z0 = r * cos(t);
    *z1 = r * sin(t);
}

double gen_normal_at(uint64_t key, uint64_t i) {
    double z0, z1;
    gen_pair(key, i >> 1, &z0, &z1);
    return (i & 1) ? z1 : z0;
}

typedef struct {
    uint64_t key, begin, end;
    double mean, std;
    uint16_t* out;
} gen_job;

static void* gen_normal_worker(void* p) {
    gen_job* jb = (gen_job*)p;
    for (uint64_t i = jb->begin; i < jb->end; i += 2) {
        double z0, z1;
        gen_pair(jb->key, i >> 1, &z0, &z1);
        jb->out[i] = gen_f32_to_bf16((float)(jb->mean + jb->std * z0));
        if (i + 1 < jb->end) jb->out[i + 1] = gen_f32_to_bf16((float)(jb->mean + jb->std * z1));
    }
    return 0;
}

/* out[i] = bf16(float(mean + std * z_i)) for i in [0, n).  Work is split on
 * even element boundaries, so the values do not depend on nthreads. */
void gen_normal_bf16(uint64_t key, uint64_t n, double mean, double std, uint16_t* out, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (n < (1u << 16)) nthreads = 1;
    pthread_t th[64];
    int created[64];
    gen_job jobs[64];
    uint64_t per = ((n / (uint64_t)nthreads) + 2) & ~1ULL;
    for (int t = 0; t < nthreads; ++t) {
        uint64_t b = per * (uint64_t)t, e = b + per;
        if (b > n) b = n;
        if (e > n || t == nthreads - 1) e = n;
        jobs[t].key = key; jobs[t].begin = b; jobs[t].end = e;
        jobs[t].mean = mean; jobs[t].std = std; jobs[t].out = out;
        created[t] = 0;
        if (b >= e) continue;
        if (nthreads > 1 && pthread_create(&th[t], 0, gen_normal_worker, &jobs[t]) == 0) created[t] = 1;
        else gen_normal_worker(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (created[t]) pthread_join(th[t], 0);
}

/* Uniform integers in [0, m): high 32 bits of the draw scaled by m. */
void gen_uniform_int(uint64_t key, uint64_t n, uint32_t m, int32_t* out) {
    for (uint64_t i = 0; i < n; ++i) {
        uint64_t hi = gen_draw(key, i) >> 32;
        out[i] = (int32_t)((hi * (uint64_t)m) >> 32);
    }
}
