/*
 * Seeded synthetic inputs, host side.
 *
 * This module holds no arithmetic of the MoE layer. It turns (seed, tensor id,
 * element index) into one value, so that the oracle and the GPU path can be fed
 * identical tensors without either of them producing the other's inputs. The
 * device twin (synth_dev.hip) implements the same definitions; the two are
 * compared element by element in the tests.
 *
 * Generator: Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror
 * and Shaw ("Parallel random numbers: as easy as 1, 2, 3", SC'11): a 128-bit
 * counter and a 64-bit key, ten rounds of two 32x32->64 multiplies with the
 * published multipliers and Weyl key increments.
 *
 * Laws (all arithmetic in IEEE double, no contraction, then one rounding):
 *   normal element i:  pair q = i/2, counter (q_lo, q_hi, tid, 0), key (seed_lo, seed_hi)
 *                      u1 = (top 53 bits of word1:word0 + 0.5) * 2^-53   in (0,1)
 *                      u2 = (top 53 bits of word3:word2) * 2^-53          in [0,1)
 *                      Box & Muller (1958): r = sqrt(-2 ln u1), z = r cos(2 pi u2) for even i,
 *                      r sin(2 pi u2) for odd i;  v = mean + std * z
 *   uniform element i: counter (i_lo, i_hi, tid, 1), u = (top 53 bits of word1:word0) * 2^-53,
 *                      v = lo + (hi - lo) * u
 *   storage:           fp32 = v rounded to nearest float; bf16 = that float rounded to nearest
 *                      even bf16 (upper 16 bits of the float, round-to-nearest-even).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static void philox_round(uint32_t c[4], const uint32_t k[2]) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k[0];
    uint32_t n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; ++r) {
        if (r) { k[0] += PHILOX_W0; k[1] += PHILOX_W1; }
        philox_round(c, k);
    }
    memcpy(out, c, sizeof(c));
}

static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* NaN stays NaN */
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

static double synth_normal_value(uint64_t seed, uint32_t tid, int64_t i, double mean, double std) {
    uint64_t q = (uint64_t)i >> 1;
    uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), tid, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    synth_philox4x32_10(ctr, key, w);
    uint64_t a = (((uint64_t)w[1] << 32) | w[0]) >> 11;
    uint64_t b = (((uint64_t)w[3] << 32) | w[2]) >> 11;
    double u1 = ((double)a + 0.5) * 0x1p-53;
    double u2 = (double)b * 0x1p-53;
    double r = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586 * u2;
    double z = (i & 1) ? r * sin(th) : r * cos(th);
    double s = std * z;
    return mean + s;
}

static double synth_uniform_value(uint64_t seed, uint32_t tid, int64_t i, double lo, double hi) {
    uint32_t ctr[4] = {(uint32_t)(uint64_t)i, (uint32_t)((uint64_t)i >> 32), tid, 1u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    synth_philox4x32_10(ctr, key, w);
    uint64_t a = (((uint64_t)w[1] << 32) | w[0]) >> 11;
    double u = (double)a * 0x1p-53;
    double span = hi - lo;
    double s = span * u;
    return lo + s;
}

typedef struct {
    void* dst; int dtype; int law; int64_t start, n;
    uint64_t seed; uint32_t tid; double p0, p1;
} job_t;

static void run_range(const job_t* j, int64_t b, int64_t e) {
    for (int64_t k = b; k < e; ++k) {
        int64_t i = j->start + k;
        double v = j->law == 0 ? synth_normal_value(j->seed, j->tid, i, j->p0, j->p1)
                               : synth_uniform_value(j->seed, j->tid, i, j->p0, j->p1);
        float f = (float)v;
        if (j->dtype == 0) ((float*)j->dst)[k] = f;
        else ((uint16_t*)j->dst)[k] = f32_to_bf16_rne(f);
    }
}

typedef struct { const job_t* j; int64_t b, e; } slice_t;
static void* run_slice(void* p) { slice_t* s = (slice_t*)p; run_range(s->j, s->b, s->e); return 0; }

static void fill(job_t* j, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 64) nthreads = 64;
    if (j->n < 65536) nthreads = 1;
    if (nthreads == 1) { run_range(j, 0, j->n); return; }
    pthread_t th[64];
    slice_t sl[64];
    for (int t = 0; t < nthreads; ++t) {
        sl[t].j = j;
        sl[t].b = j->n * t / nthreads;
        sl[t].e = j->n * (t + 1) / nthreads;
        pthread_create(&th[t], 0, run_slice, &sl[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], 0);
}

/* dtype: 0 = fp32, 1 = bf16 (stored as uint16). Fills dst[0..n) with elements start..start+n. */
void synth_fill_normal(void* dst, int dtype, int64_t start, int64_t n, uint64_t seed, uint32_t tid,
                       double mean, double std, int nthreads) {
    job_t j = {dst, dtype, 0, start, n, seed, tid, mean, std};
    fill(&j, nthreads);
}

void synth_fill_uniform(void* dst, int dtype, int64_t start, int64_t n, uint64_t seed, uint32_t tid,
                        double lo, double hi, int nthreads) {
    job_t j = {dst, dtype, 1, start, n, seed, tid, lo, hi};
    fill(&j, nthreads);
}

/* Fisher-Yates shuffle of 0..n-1 driven by the same generator (counter (i, 0, tid, 2)). */
void synth_permutation(int32_t* perm, int32_t n, uint64_t seed, uint32_t tid) {
    for (int32_t i = 0; i < n; ++i) perm[i] = i;
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    for (int32_t i = n - 1; i > 0; --i) {
        uint32_t ctr[4] = {(uint32_t)i, 0u, tid, 2u};
        uint32_t w[4];
        synth_philox4x32_10(ctr, key, w);
        uint64_t r = ((uint64_t)w[1] << 32) | w[0];
        int32_t j = (int32_t)(r % (uint64_t)(i + 1));
        int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    }
}
