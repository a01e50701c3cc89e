/*
 * Seeded synthetic-input generator shared by the oracle tests and the HIP
 * path's harness.  It holds none of the SwiftKV method's arithmetic: it only
 * turns (seed, stream, element index) into numbers.
 *
 * Generator: Philox4x32-10, the counter-based generator defined by Salmon,
 * Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3"
 * (SC'11).  A 128-bit counter is enciphered under a 64-bit key by ten rounds
 * of two 32x32->64 multiplies with the paper's multipliers, the key being
 * advanced by the Weyl constants between rounds.
 *
 * Normal variates: Box-Muller in double precision (Box & Muller, 1958) on two
 * 53-bit uniforms in (0,1) built from the four 32-bit Philox words of one
 * counter value; counter value i yields elements 2i and 2i+1.
 *
 * Counter layout for element pair i of stream s: (lo32(i), hi32(i), lo32(s),
 * hi32(s)); key = (lo32(seed), hi32(seed)).
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC philox.c -o libskv_inputs.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
  uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
  uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
  uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  uint32_t n0 = hi1 ^ c[1] ^ k[0];
  uint32_t n2 = hi0 ^ c[3] ^ k[1];
  c[0] = n0;
  c[1] = lo1;
  c[2] = n2;
  c[3] = lo0;
}

void skvin_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  philox_round(c, k);
  for (int r = 1; r < 10; ++r) {
    k[0] += PHILOX_W0;
    k[1] += PHILOX_W1;
    philox_round(c, k);
  }
  memcpy(out, c, sizeof(c));
}

static inline void block(uint64_t seed, uint64_t stream, uint64_t i, uint32_t out[4]) {
  uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), (uint32_t)stream, (uint32_t)(stream >> 32)};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  skvin_philox4x32_10(ctr, key, out);
}

/* 53-bit uniform in the open interval (0,1) from two 32-bit words. */
static inline double u53(uint32_t a, uint32_t b) {
  uint64_t m = ((uint64_t)a << 21) ^ (uint64_t)(b >> 11);
  m &= ((uint64_t)1 << 53) - 1;
  return ((double)m + 0.5) * (1.0 / 9007199254740992.0);
}

static inline void normal_pair(uint64_t seed, uint64_t stream, uint64_t i, double* z0, double* z1) {
  uint32_t w[4];
  block(seed, stream, i, w);
  double u1 = u53(w[0], w[1]);
  double u2 = u53(w[2], w[3]);
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(t);
  *z1 = r * sin(t);
}

/* float -> bf16 bits, round to nearest even (NaN kept quiet). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* out[e] = mean + std * N(0,1)_e as fp32 (rounded once from double). */
void skvin_normal_f32(uint64_t seed, uint64_t stream, uint64_t n, double mean, double std, float* out) {
  int64_t npairs = (int64_t)((n + 1) / 2);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < npairs; ++i) {
    double z0, z1;
    normal_pair(seed, stream, (uint64_t)i, &z0, &z1);
    uint64_t e = 2 * (uint64_t)i;
    out[e] = (float)(mean + std * z0);
    if (e + 1 < n) out[e + 1] = (float)(mean + std * z1);
  }
}

/* Same values as skvin_normal_f32, then rounded RNE to bf16 bits. */
void skvin_normal_bf16(uint64_t seed, uint64_t stream, uint64_t n, double mean, double std, uint16_t* out) {
  int64_t npairs = (int64_t)((n + 1) / 2);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < npairs; ++i) {
    double z0, z1;
    normal_pair(seed, stream, (uint64_t)i, &z0, &z1);
    uint64_t e = 2 * (uint64_t)i;
    out[e] = f32_to_bf16_rne((float)(mean + std * z0));
    if (e + 1 < n) out[e + 1] = f32_to_bf16_rne((float)(mean + std * z1));
  }
}

/* out[e] = lo + (hi - lo) * U(0,1)_e as fp32; one counter value per element. */
void skvin_uniform_f32(uint64_t seed, uint64_t stream, uint64_t n, double lo, double hi, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    uint32_t w[4];
    block(seed, stream, (uint64_t)i, w);
    out[i] = (float)(lo + (hi - lo) * u53(w[0], w[1]));
  }
}

/* Same values as skvin_uniform_f32, then rounded RNE to bf16 bits. */
void skvin_uniform_bf16(uint64_t seed, uint64_t stream, uint64_t n, double lo, double hi, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    uint32_t w[4];
    block(seed, stream, (uint64_t)i, w);
    out[i] = f32_to_bf16_rne((float)(lo + (hi - lo) * u53(w[0], w[1])));
  }
}

/* Integers uniform in [0, range): floor(U * range) with a 53-bit U. */
void skvin_randint(uint64_t seed, uint64_t stream, uint64_t n, uint64_t range, int64_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    uint32_t w[4];
    block(seed, stream, (uint64_t)i, w);
    uint64_t v = (uint64_t)(u53(w[0], w[1]) * (double)range);
    if (v >= range) v = range - 1;
    out[i] = (int64_t)v;
  }
}

/* Raw Philox words for element i of a stream (used by the known-answer test). */
void skvin_raw(uint64_t seed, uint64_t stream, uint64_t i, uint32_t out[4]) { block(seed, stream, i, out); }
