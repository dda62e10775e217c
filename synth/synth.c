/*
 * Seeded synthetic inputs for the MoE layer: the only code that both the CPU
 * oracle and the GPU path consume.  It holds none of the layer's arithmetic —
 * only the production of input tensors:
 *
 *   - Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 *     easy as 1, 2, 3", SC 2011): counter-based, so element i of a tensor is a
 *     pure function of (seed, tensor id, i) and does not depend on the thread
 *     count or on the order in which chunks are produced.
 *   - Box–Muller transform for normal variates.
 *   - fp32 -> bf16 round-to-nearest-even, to store bf16 input tensors.
 *   - OCP Microscaling (MX) v1.0 quantisation of fp32 weights to MXFP4
 *     (E2M1 elements, one E8M0 scale per 32 elements along the reduction axis).
 *
 * Element i of a tensor uses Philox block i/4 (counter = {i/4 lo, i/4 hi, 0, 0},
 * key = {seed, tensor}); lanes (0,1) and (2,3) of the block form two
 * Box–Muller pairs.
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

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                         uint32_t out[4]) {
  uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
  uint32_t k[2] = {key_in[0], key_in[1]};
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k[0] += PHILOX_W0;
      k[1] += PHILOX_W1;
    }
    philox_round(c, k);
  }
  memcpy(out, c, sizeof(c));
}

static inline void block_u32(uint32_t seed, uint32_t tensor, uint64_t blk,
                             uint32_t out[4]) {
  uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), 0u, 0u};
  uint32_t key[2] = {seed, tensor};
  synth_philox4x32_10(ctr, key, out);
}

/* Raw 32-bit draws: element i = lane (i % 4) of block i / 4. */
void synth_u32(uint32_t seed, uint32_t tensor, uint64_t offset, uint64_t n,
               uint32_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    uint64_t g = offset + (uint64_t)i;
    uint32_t b[4];
    block_u32(seed, tensor, g >> 2, b);
    out[i] = b[g & 3];
  }
}

static inline double u01(uint32_t v) { /* strictly inside (0,1) */
  return ((double)v + 0.5) * (1.0 / 4294967296.0);
}

/* Normal(mean, std) as double for elements [offset, offset+n). */
static void normal_block(uint32_t seed, uint32_t tensor, uint64_t blk,
                         double out[4]) {
  uint32_t b[4];
  block_u32(seed, tensor, blk, b);
  const double two_pi = 6.283185307179586476925286766559;
  for (int p = 0; p < 2; ++p) {
    double r = sqrt(-2.0 * log(u01(b[2 * p])));
    double a = two_pi * u01(b[2 * p + 1]);
    out[2 * p] = r * cos(a);
    out[2 * p + 1] = r * sin(a);
  }
}

void synth_normal_f64(uint32_t seed, uint32_t tensor, uint64_t offset,
                      uint64_t n, double mean, double std, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    uint64_t g = offset + (uint64_t)i;
    double z[4];
    normal_block(seed, tensor, g >> 2, z);
    out[i] = mean + std * z[g & 3];
  }
}

void synth_normal_f32(uint32_t seed, uint32_t tensor, uint64_t offset,
                      uint64_t n, double mean, double std, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    uint64_t g = offset + (uint64_t)i;
    double z[4];
    normal_block(seed, tensor, g >> 2, z);
    out[i] = (float)(mean + std * z[g & 3]);
  }
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet). */
static inline uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

void synth_normal_bf16(uint32_t seed, uint32_t tensor, uint64_t offset,
                       uint64_t n, double mean, double std, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    uint64_t g = offset + (uint64_t)i;
    double z[4];
    normal_block(seed, tensor, g >> 2, z);
    out[i] = to_bf16((float)(mean + std * z[g & 3]));
  }
}

void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = to_bf16(in[i]);
}

/*
 * OCP MX v1.0 quantisation to MXFP4, blocks of 32 consecutive elements along
 * each row (the reduction axis).  Shared exponent X = floor(log2(amax)) - 2
 * (2 = the largest E2M1 exponent), clamped to the E8M0 range [-127, 127];
 * element = E2M1 value nearest to w / 2^X (ties to even mantissa), saturated to
 * +-6.  An all-zero block gets scale byte 0 (2^-127).  Codes are packed two per
 * byte, element 2i in the low nibble.
 */
static uint8_t e2m1_encode(double v) {
  /* magnitudes of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6 */
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  uint8_t s = (v < 0.0 || (v == 0.0 && signbit(v))) ? 8u : 0u;
  double a = fabs(v);
  if (a >= 6.0) return s | 7u;
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    double dc = fabs(a - mag[c]), db = fabs(a - mag[best]);
    /* ties go to the even code (mantissa bit 0) */
    if (dc < db || (dc == db && (c & 1) == 0)) best = c;
  }
  return s | (uint8_t)best;
}

void synth_mxfp4_quantize(const float* w, int64_t rows, int64_t cols,
                          uint8_t* codes, uint8_t* scales) {
  const int64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* blk = w + r * cols + b * 32;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) {
        double a = fabs((double)blk[i]);
        if (a > amax) amax = a;
      }
      int X;
      if (amax == 0.0) {
        X = -127;
      } else {
        int e;
        frexp(amax, &e); /* amax = f * 2^e, f in [0.5, 1) -> floor(log2) = e-1 */
        X = (e - 1) - 2;
        if (X < -127) X = -127;
        if (X > 127) X = 127;
      }
      scales[r * nb + b] = (uint8_t)(X + 127);
      for (int i = 0; i < 32; i += 2) {
        uint8_t lo = e2m1_encode(ldexp((double)blk[i], -X));
        uint8_t hi = e2m1_encode(ldexp((double)blk[i + 1], -X));
        codes[r * (cols / 2) + b * 16 + i / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}
