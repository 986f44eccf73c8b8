/*
 * Seeded synthetic tensors for the MoE workloads.
 *
 * This file holds no part of the MoE method: it only draws numbers. Both the
 * GPU path's tests/bench and the CPU oracle receive the arrays it writes.
 *
 * Generator: a counter-based stream. A stream is named by three integers
 * (config id, tensor role, index within the role). Element i of the stream is a
 * pure function of (stream key, i), so any sub-range (a prefix of tokens, one
 * expert's weights, a sample of rows) can be drawn without drawing the rest,
 * and the result does not depend on how the range is split over threads.
 *
 *   mix64      : the SplitMix64 output function (Steele, Lea and Flood,
 *                "Fast splittable pseudorandom number generators", OOPSLA 2014).
 *   key        : mix64 chained over the three stream integers.
 *   pair j     : two 64-bit draws h1 = mix64(key + (2j+1)*G), h2 = mix64(key + (2j+2)*G),
 *                G = 0x9E3779B97F4A7C15 (the golden-ratio Weyl increment);
 *                u1 = ((h1 >> 11) + 1) * 2^-53 in (0, 1], u2 = (h2 >> 11) * 2^-53 in [0, 1).
 *   normals    : Box-Muller (Box and Muller, 1958): r = sqrt(-2 ln u1),
 *                element 2j = r cos(2 pi u2), element 2j+1 = r sin(2 pi u2),
 *                computed in double, times the requested standard deviation,
 *                then rounded to fp32 (and, for bf16 output, from fp32 to bf16
 *                by round-to-nearest-even).
 */
#include <math.h>
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static uint64_t stream_key(uint64_t a, uint64_t b, uint64_t c) {
  uint64_t k = mix64(0x6D6F652D73796E74ULL ^ a);
  k = mix64(k + GOLDEN * (b + 1));
  k = mix64(k + GOLDEN * (c + 1));
  return k;
}

static inline double normal_at(uint64_t key, int64_t i) {
  const uint64_t j = (uint64_t)(i >> 1);
  const uint64_t h1 = mix64(key + (2 * j + 1) * GOLDEN);
  const uint64_t h2 = mix64(key + (2 * j + 2) * GOLDEN);
  const double u1 = (double)((h1 >> 11) + 1) * 0x1.0p-53;
  const double u2 = (double)(h2 >> 11) * 0x1.0p-53;
  const double r = sqrt(-2.0 * log(u1));
  const double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v = {f};
  uint32_t u = v.u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* out[n] = fp32(std * normal(stream, start + n)), n in [0, count). */
void wl_normal_f32(uint64_t a, uint64_t b, uint64_t c, int64_t start, int64_t count,
                   double std, float* out) {
  const uint64_t key = stream_key(a, b, c);
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < count; ++n) out[n] = (float)(std * normal_at(key, start + n));
}

/* The same values as wl_normal_f32, rounded to bf16 (bit patterns). */
void wl_normal_bf16(uint64_t a, uint64_t b, uint64_t c, int64_t start, int64_t count,
                    double std, uint16_t* out) {
  const uint64_t key = stream_key(a, b, c);
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < count; ++n)
    out[n] = f32_to_bf16_rne((float)(std * normal_at(key, start + n)));
}

/* Gather rows of a row-major [*, cols] stream: out[r, :] = stream row rows[r]. */
void wl_normal_rows_f32(uint64_t a, uint64_t b, uint64_t c, const int64_t* rows, int64_t nrows,
                        int64_t cols, double std, float* out) {
  const uint64_t key = stream_key(a, b, c);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r)
    for (int64_t h = 0; h < cols; ++h)
      out[r * cols + h] = (float)(std * normal_at(key, rows[r] * cols + h));
}

void wl_normal_rows_bf16(uint64_t a, uint64_t b, uint64_t c, const int64_t* rows, int64_t nrows,
                         int64_t cols, double std, uint16_t* out) {
  const uint64_t key = stream_key(a, b, c);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r)
    for (int64_t h = 0; h < cols; ++h)
      out[r * cols + h] = f32_to_bf16_rne((float)(std * normal_at(key, rows[r] * cols + h)));
}
