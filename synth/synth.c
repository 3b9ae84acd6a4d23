/*
 * Seeded synthetic inputs for the RMSNorm workloads.
 *
 * This file only draws random numbers. It computes nothing of RMSNorm and
 * shares no code with either the CPU oracle or the HIP library; both of those
 * receive the arrays written here as plain inputs.
 *
 * Generator: counter-based SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014). The n-th 64-bit output of
 * stream `key` is mix64(key + (n + 1) * 0x9E3779B97F4A7C15), so any element
 * can be produced independently of the others and of the thread count.
 * Normal deviates: Box-Muller in double (Box and Muller, 1958); element i uses
 * the pair of outputs (2*(i/2), 2*(i/2)+1) and takes the cosine branch for
 * even i, the sine branch for odd i.
 * bf16 values are formed by keeping the top 16 bits of the fp32 sample
 * (round toward zero); the workloads only need bf16 numbers distributed like
 * scale * N(0, 1).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Stream key: distinct (seed, stream) pairs give unrelated sequences. */
uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return mix64(seed * SYNTH_GOLDEN + mix64(stream + 0x632BE59BD9B4E019ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t n) {
  return mix64(key + (n + 1) * SYNTH_GOLDEN);
}

static inline double normal_at(uint64_t key, uint64_t i) {
  const uint64_t p = i >> 1;
  const uint64_t a = draw(key, 2 * p);
  const uint64_t b = draw(key, 2 * p + 1);
  const double u1 = (double)((a >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
  const double u2 = (double)(b >> 11) * 0x1.0p-53;       /* [0, 1) */
  const double rad = sqrt(-2.0 * log(u1));
  const double th = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? rad * sin(th) : rad * cos(th);
}

static inline uint16_t to_bf16_trunc(float v) {
  uint32_t u;
  memcpy(&u, &v, 4);
  return (uint16_t)(u >> 16);
}

/* out[i] = draw i (first <= i < first + n) of stream (seed, stream). */
void synth_u64(uint64_t seed, uint64_t stream, uint64_t first, int64_t n,
               uint64_t* out) {
  const uint64_t key = synth_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = draw(key, first + (uint64_t)i);
}

/* out[i] = mean + std * N(0,1), the product and sum taken in fp32. */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t first, int64_t n,
                      float mean, float std, float* out) {
  const uint64_t key = synth_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) {
    const float z = (float)normal_at(key, first + (uint64_t)i);
    const float s = std * z;
    out[i] = mean + s;
  }
}

typedef struct {
  uint64_t key;
  int64_t row0, r_begin, r_end, D, ld;
  float scale;
  uint16_t* out;
} rows_job;

static void* rows_worker(void* arg) {
  const rows_job* j = (const rows_job*)arg;
  for (int64_t r = j->r_begin; r < j->r_end; ++r) {
    uint16_t* dst = j->out + r * j->ld;
    const uint64_t base = (uint64_t)(j->row0 + r) * (uint64_t)j->D;
    for (int64_t c = 0; c < j->D; ++c) {
      const float z = (float)normal_at(j->key, base + (uint64_t)c);
      dst[c] = to_bf16_trunc(j->scale * z);
    }
  }
  return NULL;
}

/*
 * Rows row0 .. row0+nrows-1 of a [*, D] bf16 matrix whose element (t, c)
 * is scale * N(0,1) drawn at counter t*D + c. Row r of the result is written
 * at out + r*ld (ld >= D elements); columns D..ld-1 are left untouched.
 */
void synth_normal_bf16_rows(uint64_t seed, uint64_t stream, int64_t row0,
                            int64_t nrows, int64_t D, int64_t ld, float scale,
                            uint16_t* out, int nthreads) {
  const uint64_t key = synth_key(seed, stream);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (nrows < 4 * nthreads) nthreads = 1;
  rows_job jobs[64];
  pthread_t tid[64];
  int created[64];
  const int64_t per = (nrows + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].key = key;
    jobs[t].row0 = row0;
    jobs[t].r_begin = t * per < nrows ? t * per : nrows;
    jobs[t].r_end = (t + 1) * per < nrows ? (t + 1) * per : nrows;
    jobs[t].D = D;
    jobs[t].ld = ld;
    jobs[t].scale = scale;
    jobs[t].out = out;
  }
  if (nthreads == 1) {
    rows_worker(&jobs[0]);
    return;
  }
  for (int t = 0; t < nthreads; ++t) {
    created[t] = pthread_create(&tid[t], NULL, rows_worker, &jobs[t]) == 0;
    if (!created[t]) rows_worker(&jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t)
    if (created[t]) pthread_join(tid[t], NULL);
}
