/*
 * Seeded synthetic input generator shared by the oracle side and the GPU side.
 *
 * It holds none of the attention method's arithmetic: it only draws numbers.
 *
 * Uniforms come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used counter-style: the k-th
 * 64-bit draw of a stream is mix(key + (k + 1) * GAMMA), so any element can be
 * produced independently of the others and the fill runs in parallel.
 * Normals come from the Box-Muller transform in fp64: draws 2p and 2p+1 of a
 * stream give z[2p] = r cos(t) and z[2p+1] = r sin(t), r = sqrt(-2 ln(1 - u0)),
 * t = 2 pi u1.
 *
 * Output is fp32; the Python side rounds it to fp16 (round to nearest even).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of sub-stream `sid` under `seed`. */
uint64_t gen_stream_key(uint64_t seed, uint64_t sid) {
  return mix64(mix64(seed * GAMMA + 0x632BE59BD9B4E019ULL) ^ (sid * 0xD1B54A32D192ED03ULL));
}

static inline double u01(uint64_t key, uint64_t k) {
  /* 53 random bits -> [0, 1) */
  return (double)(mix64(key + (k + 1) * GAMMA) >> 11) * 0x1.0p-53;
}

/* n uniforms in [0,1) of stream (seed, sid), starting at draw `start`. */
void gen_uniform(uint64_t seed, uint64_t sid, uint64_t start, uint64_t n, double* out) {
  uint64_t key = gen_stream_key(seed, sid);
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = u01(key, start + (uint64_t)i);
}

static inline double normal_at(uint64_t key, uint64_t idx) {
  uint64_t p = idx >> 1;
  double u0 = u01(key, 2 * p), u1 = u01(key, 2 * p + 1);
  double r = sqrt(-2.0 * log(1.0 - u0));
  double t = 6.283185307179586 * u1;
  return (idx & 1) ? r * sin(t) : r * cos(t);
}

/* n standard normals (fp64) of stream (seed, sid), starting at element `start`. */
void gen_normal(uint64_t seed, uint64_t sid, uint64_t start, uint64_t n, double* out) {
  uint64_t key = gen_stream_key(seed, sid);
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = normal_at(key, start + (uint64_t)i);
}

/*
 * Fill a [G, N, d] tensor (G = B*H heads) with fp32 values
 *   x[g, n, c] = (z + shift[g*d + c]) * scale[g*d + c]
 * where z is the element's standard normal of stream (seed, sid) in row-major
 * order.  shift / scale may be NULL (0 and 1).
 */
void gen_tensor(uint64_t seed, uint64_t sid, int64_t G, int64_t N, int64_t d,
                const double* shift, const double* scale, float* out) {
  uint64_t key = gen_stream_key(seed, sid);
  int64_t total = G * N * d;
  #pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < total; ++i) {
    int64_t c = i % d, g = i / (N * d);
    double z = normal_at(key, (uint64_t)i);
    if (shift) z += shift[g * d + c];
    if (scale) z *= scale[g * d + c];
    out[i] = (float)z;
  }
}
