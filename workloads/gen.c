/* Seeded synthetic input generator shared by the GPU path's tests/bench and
 * the CPU oracle.  It holds none of the method's arithmetic: it only draws
 * numbers and rounds them to the storage type.
 *
 * Every sample is a pure function of (seed, stream, global index), so a
 * buffer can be filled in any order, by any number of threads, in pieces,
 * and always comes out with identical bytes.
 *
 *   uniforms : Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 *              numbers: as easy as 1, 2, 3", SC'11), counter = (index lo,
 *              index hi, stream, 0), key = (seed lo, seed hi).
 *   normals  : Box-Muller on two of the four 32-bit words, in double;
 *              even global index takes the cosine branch, odd the sine.
 *   bf16     : round-to-nearest-even of the fp32 value (no NaNs occur).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    k0 += PHILOX_W0; k1 += PHILOX_W1;
  }
}

/* Four raw words for counter `idx` of `stream`. */
void skvgen_philox(uint64_t seed, uint64_t stream, uint64_t idx, uint32_t out[4]) {
  uint32_t c[4] = {(uint32_t)idx, (uint32_t)(idx >> 32), (uint32_t)stream,
                   (uint32_t)(stream >> 32)};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

static inline double u01(uint32_t x) { return ((double)x + 0.5) * (1.0 / 4294967296.0); }

static inline double normal_at(uint64_t seed, uint64_t stream, uint64_t g) {
  uint32_t w[4];
  skvgen_philox(seed, stream, g >> 1, w);
  double r = sqrt(-2.0 * log(u01(w[0])));
  double th = 6.283185307179586476925 * u01(w[1]);
  return (g & 1) ? r * sin(th) : r * cos(th);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t u = v.u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* out[i] = (float)(normal(offset+i)) * scale[(offset+i) % period]  (scale may be NULL => 1) */
void skvgen_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, size_t n,
                       const float* scale, uint64_t period, float* out) {
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)n; ++i) {
    uint64_t g = offset + (uint64_t)i;
    float x = (float)normal_at(seed, stream, g);
    if (scale) x = x * scale[g % period];
    out[i] = x;
  }
}

/* Same values as skvgen_normal_f32, rounded to bf16 (stored as uint16 bits). */
void skvgen_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, size_t n,
                        const float* scale, uint64_t period, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)n; ++i) {
    uint64_t g = offset + (uint64_t)i;
    float x = (float)normal_at(seed, stream, g);
    if (scale) x = x * scale[g % period];
    out[i] = f32_to_bf16_rne(x);
  }
}

/* Keys with a log-normal norm: for key j (global key index key0+j),
 *   g = d normals of stream `s_dir` at indices (key0+j)*d + c,
 *   n = exp(sigma * normal of stream `s_norm` at index key0+j),
 *   key = n * g / |g|   (double), rounded to fp32 then bf16. */
void skvgen_lognormal_keys_bf16(uint64_t seed, uint64_t s_dir, uint64_t s_norm, uint64_t key0,
                                size_t n_keys, int d, double sigma, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (long long j = 0; j < (long long)n_keys; ++j) {
    uint64_t key = key0 + (uint64_t)j;
    double g[1024];
    double ss = 0.0;
    for (int c = 0; c < d; ++c) {
      g[c] = normal_at(seed, s_dir, key * (uint64_t)d + (uint64_t)c);
      ss += g[c] * g[c];
    }
    double nrm = exp(sigma * normal_at(seed, s_norm, key));
    double f = nrm / sqrt(ss);
    for (int c = 0; c < d; ++c) out[(size_t)j * d + c] = f32_to_bf16_rne((float)(g[c] * f));
  }
}

/* Uniform 64-bit words (for permutations and sampling on the host). */
void skvgen_u64(uint64_t seed, uint64_t stream, uint64_t offset, size_t n, uint64_t* out) {
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < (long long)n; ++i) {
    uint32_t w[4];
    skvgen_philox(seed, stream, offset + (uint64_t)i, w);
    out[i] = ((uint64_t)w[0] << 32) | w[1];
  }
}
