/*
 * gen.c -- bulk seeded draws for the synthetic workloads (SplitMix64 +
 * Box-Muller).  Input generation only: nothing here touches RoPE,
 * quantisation or a contraction.  Same definitions as workloads/__init__.py:
 *   x_i = mix(seed + (i+1) * 0x9E3779B97F4A7C15)            (SplitMix64, Vigna)
 *   u_i = ((x_i >> 11) + 0.5) * 2^-53
 *   n_i = sqrt(-2 ln u_{2i}) * cos(2 pi u_{2i+1})           (Box-Muller, cosine branch)
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static uint64_t wl_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static double wl_uniform(uint64_t seed, uint64_t i) {
    uint64_t x = wl_mix(seed + (i + 1) * 0x9E3779B97F4A7C15ULL);
    return ((double)(x >> 11) + 0.5) * 0x1p-53;
}

static double wl_normal(uint64_t seed, uint64_t i) {
    double u1 = wl_uniform(seed, 2 * i);
    double u2 = wl_uniform(seed, 2 * i + 1);
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

static uint16_t wl_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

struct wl_job {
    uint64_t seed, oseed, i0, i1;
    double std, op, omul;
    int kind; /* 0: f32 normal, 1: bf16 normal (+ outliers) */
    void* out;
};

static void* wl_worker(void* arg) {
    struct wl_job* j = (struct wl_job*)arg;
    for (uint64_t i = j->i0; i < j->i1; ++i) {
        double v = wl_normal(j->seed, i) * j->std;
        if (j->kind == 0) {
            ((float*)j->out)[i] = (float)v;
        } else {
            if (j->op > 0.0 && wl_uniform(j->oseed, i) < j->op) v *= j->omul;
            ((uint16_t*)j->out)[i] = wl_f32_to_bf16((float)v);
        }
    }
    return 0;
}

static void wl_run(struct wl_job base, uint64_t n, int nthreads) {
    pthread_t th[64];
    struct wl_job jobs[64];
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (n < (uint64_t)nthreads * 4096) nthreads = 1;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].i0 = n * (uint64_t)t / (uint64_t)nthreads;
        jobs[t].i1 = n * (uint64_t)(t + 1) / (uint64_t)nthreads;
        pthread_create(&th[t], 0, wl_worker, &jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], 0);
}

/* n fp32 normals N(0, std^2). */
void wl_normal_f32(uint64_t seed, uint64_t n, double std, float* out, int nthreads) {
    struct wl_job b = {seed, 0, 0, 0, std, 0.0, 1.0, 0, out};
    wl_run(b, n, nthreads);
}

/* n bf16 normals N(0, std^2); with probability op (stream oseed) an element is
 * multiplied by omul before rounding. */
void wl_normal_bf16(uint64_t seed, uint64_t n, double std, uint64_t oseed, double op, double omul,
                    uint16_t* out, int nthreads) {
    struct wl_job b = {seed, oseed, 0, 0, std, op, omul, 1, out};
    wl_run(b, n, nthreads);
}
