/*
 * Seeded synthetic inputs for the BLOOM decode workloads: weights, prompt ids,
 * attention scores and left-pad lengths.
 *
 * Input generation only: nothing here computes any part of the model.  Both
 * the CPU oracle (through the tests) and the GPU library receive arrays
 * written by these functions, so the two sides see bit-identical inputs.
 *
 * Every value is a pure function of (seed, tensor id, flat index): one 64-bit
 * counter hash per element, so any slice can be regenerated alone and the
 * result does not depend on the number of threads.
 *
 *   hash      SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
 *             pseudorandom number generators", OOPSLA 2014), applied to
 *             key + index with key = SplitMix64(seed << 32 ^ tensor_id).
 *   normal    Irwin-Hall sum of the four 16-bit fields of one hash, centred:
 *             z = f0+f1+f2+f3 - 131070 (an exact integer, |z| <= 131070),
 *             value = mean + fp32(z) * fp32(sigma / sd4) with
 *             sd4 = sqrt((65536^2 - 1) / 3), each operation one IEEE fp32
 *             round-to-nearest-even step; then rounded to bf16 / fp16 (RNE)
 *             when the storage type asks for it.
 *   int8      hash mod 255 - 127, uniform on {-127..127}.
 *   scale     fp16( s0 * (0.5 + (hash >> 40) * 2^-24) ), fp32 arithmetic.
 *   ids       hash mod n (uniform token ids), lo + hash mod (hi-lo+1).
 *
 * Built with plain gcc -O2 (no fast-math) so fp32 steps are IEEE exact.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t smix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tid) {
  return smix((seed << 32) ^ tid);
}

static inline uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* fp32 -> bf16 bits, round to nearest even; NaN stays NaN. */
static inline uint16_t to_bf16(float f) {
  uint32_t u = f2u(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* fp32 -> IEEE binary16 bits, round to nearest even, with subnormals. */
static inline uint16_t to_f16(float f) {
  uint32_t u = f2u(f);
  uint32_t sign = (u >> 16) & 0x8000u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);      /* NaN */
  if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);     /* >= 65520 rounds to inf */
  if (a < 0x38800000u) {                                       /* below 2^-14: subnormal */
    if (a < 0x33000000u) return (uint16_t)sign;                /* < 2^-25: rounds to 0 */
    uint32_t mant = (a & 0x7fffffu) | 0x800000u;
    int e = (int)(a >> 23);                                    /* 102..112 */
    int shift = 126 - e;                                       /* 14..24 */
    uint32_t half = mant >> shift;
    uint32_t rem = mant & ((1u << shift) - 1u);
    uint32_t mid = 1u << (shift - 1);
    if (rem > mid || (rem == mid && (half & 1u))) half++;
    return (uint16_t)(sign | half);
  }
  uint32_t r = a + 0x0fffu + ((a >> 13) & 1u);
  r -= 0x38000000u;                                            /* rebias 127 -> 15 */
  return (uint16_t)(sign | (r >> 13));
}

enum { KIND_F32 = 0, KIND_BF16 = 1, KIND_F16 = 2 };

typedef struct {
  uint64_t key, begin, end;
  int kind;
  float mean, scale;
  void *out;
  int op;            /* 0 normal, 1 int8, 2 scale, 3 ids */
  uint64_t modulus;
  int64_t lo;
} job_t;

static void run_job(const job_t *j) {
  for (uint64_t i = j->begin; i < j->end; ++i) {
    uint64_t r = smix(j->key + i);
    switch (j->op) {
      case 0: {
        int32_t s = (int32_t)(r & 0xffffu) + (int32_t)((r >> 16) & 0xffffu) +
                    (int32_t)((r >> 32) & 0xffffu) + (int32_t)(r >> 48);
        float v = (float)(s - 131070) * j->scale;
        if (j->mean != 0.0f) v = j->mean + v;
        if (j->kind == KIND_F32) ((float *)j->out)[i] = v;
        else if (j->kind == KIND_BF16) ((uint16_t *)j->out)[i] = to_bf16(v);
        else ((uint16_t *)j->out)[i] = to_f16(v);
        break;
      }
      case 1:
        ((int8_t *)j->out)[i] = (int8_t)((int)(r % 255u) - 127);
        break;
      case 2: {
        float u = (float)(r >> 40) * 5.9604644775390625e-8f; /* 2^-24, exact */
        float v = j->scale * (0.5f + u);
        ((uint16_t *)j->out)[i] = to_f16(v);
        break;
      }
      case 3:
        ((int32_t *)j->out)[i] = (int32_t)(j->lo + (int64_t)(r % j->modulus));
        break;
    }
  }
}

static void *thread_main(void *p) { run_job((const job_t *)p); return NULL; }

#define MAX_THREADS 64

static void run_parallel(job_t base, uint64_t n, int threads) {
  if (threads < 1) threads = 1;
  if (threads > MAX_THREADS) threads = MAX_THREADS;
  if (n < (1u << 20)) threads = 1;
  if (threads == 1) { base.begin = 0; base.end = n; run_job(&base); return; }
  pthread_t tids[MAX_THREADS];
  int live[MAX_THREADS];
  job_t jobs[MAX_THREADS];
  for (int t = 0; t < threads; ++t) {
    jobs[t] = base;
    jobs[t].begin = n * (uint64_t)t / (uint64_t)threads;
    jobs[t].end = n * (uint64_t)(t + 1) / (uint64_t)threads;
    live[t] = pthread_create(&tids[t], NULL, thread_main, &jobs[t]) == 0;
    if (!live[t]) run_job(&jobs[t]);   /* could not start a thread: do it here */
  }
  for (int t = 0; t < threads; ++t)
    if (live[t]) pthread_join(tids[t], NULL);
}

/* Scale that maps the centred Irwin-Hall(4) integer onto standard deviation sigma. */
static float ih4_scale(double sigma) {
  return (float)(sigma / sqrt((65536.0 * 65536.0 - 1.0) / 3.0));
}

void bi_fill_normal(uint64_t seed, uint64_t tid, uint64_t n, double sigma, float mean,
                    int kind, void *out, int threads) {
  job_t j; memset(&j, 0, sizeof j);
  j.key = stream_key(seed, tid); j.kind = kind; j.mean = mean; j.scale = ih4_scale(sigma);
  j.out = out; j.op = 0;
  run_parallel(j, n, threads);
}

void bi_fill_int8(uint64_t seed, uint64_t tid, uint64_t n, int8_t *out, int threads) {
  job_t j; memset(&j, 0, sizeof j);
  j.key = stream_key(seed, tid); j.out = out; j.op = 1;
  run_parallel(j, n, threads);
}

void bi_fill_scale_f16(uint64_t seed, uint64_t tid, uint64_t n, float s0, uint16_t *out,
                       int threads) {
  job_t j; memset(&j, 0, sizeof j);
  j.key = stream_key(seed, tid); j.scale = s0; j.out = out; j.op = 2;
  run_parallel(j, n, threads);
}

void bi_fill_ids(uint64_t seed, uint64_t tid, uint64_t n, int64_t lo, uint64_t modulus,
                 int32_t *out) {
  job_t j; memset(&j, 0, sizeof j);
  j.key = stream_key(seed, tid); j.out = out; j.op = 3; j.lo = lo; j.modulus = modulus ? modulus : 1;
  run_parallel(j, n, 1);
}

/* Raw hash, exposed so tests can check the generator against its definition. */
uint64_t bi_hash(uint64_t seed, uint64_t tid, uint64_t i) {
  return smix(stream_key(seed, tid) + i);
}

uint16_t bi_f32_to_bf16(float f) { return to_bf16(f); }
uint16_t bi_f32_to_f16(float f) { return to_f16(f); }
