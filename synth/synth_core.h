/*
 * synth_core.h -- scalar core of the seeded input generator, shared by the
 * host build (synth.c, gcc) and the device build (synth_gpu.hip, hipcc).
 *
 * Holds input distributions only, no arithmetic of the recurrence.
 *
 * Bit-identical on CPU and GPU by construction: integer Philox, then fp64
 * transforms that use only IEEE-754 basic operations (+, -, *, /), integer
 * conversions and bit manipulation, in a fixed order. No library
 * transcendental, no hardware sqrt, no fused multiply-add (both builds use
 * -ffp-contract=off), so every operation is correctly rounded the same way
 * on both sides.
 *
 *   - Philox-4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel random numbers:
 *     as easy as 1, 2, 3", SC'11;
 *   - normals: Box-Muller transform (Box & Muller, 1958);
 *   - log: mantissa/exponent split, log m = 2 atanh((m-1)/(m+1)) series;
 *   - exp: Cody-Waite reduction by ln 2, Taylor series, exponent assembly;
 *   - log1p(y), 0 <= y <= 1: 2 atanh(y / (2 + y)) series;
 *   - sin/cos of 2*pi*u: exact quadrant split of 4u, octant symmetry, Taylor;
 *   - sqrt: inverse-sqrt Newton from a bit-level seed, one final correction.
 * Accuracy of each is about 1e-16 relative (checked against the C library
 * in the tests); exactness across the two builds is what matters.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#ifdef __HIPCC__
#define SYN_FN __host__ __device__ static inline
#else
#define SYN_FN static inline
#endif

#define SYN_M0 0xD2511F53u
#define SYN_M1 0xCD9E8D57u
#define SYN_W0 0x9E3779B9u
#define SYN_W1 0xBB67AE85u

enum { SYN_NORMAL = 0, SYN_UNIT_ROW = 1, SYN_NEG_SOFTPLUS = 2, SYN_SIGMOID = 3 };
enum { SYN_F64 = 0, SYN_F32 = 1, SYN_BF16 = 2 };

SYN_FN void syn_round(uint32_t* c, uint32_t k0, uint32_t k1) {
  const uint64_t p0 = (uint64_t)SYN_M0 * c[0];
  const uint64_t p1 = (uint64_t)SYN_M1 * c[2];
  const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
  const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
  c[1] = (uint32_t)p1;
  c[3] = (uint32_t)p0;
  c[0] = n0;
  c[2] = n2;
}

/* Philox-4x32 with ten rounds; the key is bumped by the Weyl constants between rounds */
SYN_FN void syn_philox(uint32_t c[4], uint32_t k0, uint32_t k1) {
  syn_round(c, k0, k1);
  for (int r = 1; r < 10; ++r) {
    k0 += SYN_W0;
    k1 += SYN_W1;
    syn_round(c, k0, k1);
  }
}

SYN_FN uint64_t syn_bits(double x) {
  union { double d; uint64_t u; } v;
  v.d = x;
  return v.u;
}
SYN_FN double syn_from_bits(uint64_t u) {
  union { double d; uint64_t u; } v;
  v.u = u;
  return v.d;
}

/* 53-bit uniform in [0, 1) from two words */
SYN_FN double syn_u53(uint32_t hi, uint32_t lo) {
  return ((double)(hi >> 5) * 67108864.0 + (double)(lo >> 6)) * (1.0 / 9007199254740992.0);
}

/* sqrt for finite x >= 0: inverse-sqrt Newton from a bit-level seed, then one
   Newton correction of the square root itself; no division, no hardware sqrt */
SYN_FN double syn_sqrt(double x) {
  if (!(x > 0.0)) return 0.0;
  double y = syn_from_bits(0x5fe6eb50c7b537a9ull - (syn_bits(x) >> 1)); /* ~1/sqrt(x), within 4% */
  for (int i = 0; i < 5; ++i) y = y * (1.5 - 0.5 * x * y * y);
  double r = x * y;
  r = r + 0.5 * y * (x - r * r);
  return r;
}

#define SYN_LN2 0.69314718055994530941723212145818
#define SYN_LN2_HI 6.93147180369123816490e-01 /* upper bits of ln 2, n*HI exact for |n| < 2^11 */
#define SYN_LN2_LO 1.90821492927058770002e-10
#define SYN_SQRT2 1.41421356237309504880168872420970

/* 2 * atanh(s) for |s| <= 1/3: odd series to s^39 (Horner, constant-folded coefficients) */
SYN_FN double syn_2atanh(double s) {
  const double s2 = s * s;
  const double p = 1.0 / 1.0 + s2 * (1.0 / 3.0 + s2 * (1.0 / 5.0 + s2 * (1.0 / 7.0 + s2 * (1.0 / 9.0 + s2 * (1.0 / 11.0 + s2 * (1.0 / 13.0 + s2 * (1.0 / 15.0 + s2 * (1.0 / 17.0 + s2 * (1.0 / 19.0 + s2 * (1.0 / 21.0 + s2 * (1.0 / 23.0 + s2 * (1.0 / 25.0 + s2 * (1.0 / 27.0 + s2 * (1.0 / 29.0 + s2 * (1.0 / 31.0 + s2 * (1.0 / 33.0 + s2 * (1.0 / 35.0 + s2 * (1.0 / 37.0 + s2 * (1.0 / 39.0)))))))))))))))))));
  return 2.0 * s * p;
}

/* natural log for finite x > 0 (normal range) */
SYN_FN double syn_log(double x) {
  const uint64_t b = syn_bits(x);
  int e = (int)((b >> 52) & 0x7ff) - 1023;
  double m = syn_from_bits((b & 0x000fffffffffffffull) | 0x3ff0000000000000ull); /* [1, 2) */
  if (m > SYN_SQRT2) { m = 0.5 * m; e += 1; }
  return (double)e * SYN_LN2 + syn_2atanh((m - 1.0) / (m + 1.0));
}

/* exp for finite x (0 below -700, +inf above 700): Cody-Waite reduction by
   ln 2, Taylor series of e^r to r^18 on |r| <= 0.35, exact scaling by 2^n */
SYN_FN double syn_exp(double x) {
  if (x < -700.0) return 0.0;
  if (x > 700.0) return __builtin_inf();
  const double kd = x * (1.0 / SYN_LN2);
  const int64_t n = (int64_t)(kd + (kd >= 0.0 ? 0.5 : -0.5));
  const double r = (x - (double)n * SYN_LN2_HI) - (double)n * SYN_LN2_LO;
  const double p = 1.0 + r * (1.0 / 1.0 + r * (1.0 / 2.0 + r * (1.0 / 6.0 + r * (1.0 / 24.0 + r * (1.0 / 120.0 + r * (1.0 / 720.0 + r * (1.0 / 5040.0 + r * (1.0 / 40320.0 + r * (1.0 / 362880.0 + r * (1.0 / 3628800.0 + r * (1.0 / 39916800.0 + r * (1.0 / 479001600.0 + r * (1.0 / 6227020800.0 + r * (1.0 / 87178291200.0 + r * (1.0 / 1307674368000.0 + r * (1.0 / 20922789888000.0 + r * (1.0 / 355687428096000.0 + r * (1.0 / 6402373705728000.0))))))))))))))))));
  const int64_t n1 = n / 2, n2 = n - n1; /* two exact power-of-two scalings */
  return p * syn_from_bits((uint64_t)(1023 + n1) << 52) * syn_from_bits((uint64_t)(1023 + n2) << 52);
}

/* log(1 + y) for 0 <= y <= 1 */
SYN_FN double syn_log1p01(double y) { return syn_2atanh(y / (2.0 + y)); }

/* sin and cos of t in [0, pi/4]: Taylor series to t^19 / t^20 */
SYN_FN void syn_sincos_oct(double t, double* s, double* c) {
  const double t2 = t * t;
  *s = t * (1.0 / 1.0 + t2 * (-1.0 / 6.0 + t2 * (1.0 / 120.0 + t2 * (-1.0 / 5040.0 + t2 * (1.0 / 362880.0 + t2 * (-1.0 / 39916800.0 + t2 * (1.0 / 6227020800.0 + t2 * (-1.0 / 1307674368000.0 + t2 * (1.0 / 355687428096000.0 + t2 * (-1.0 / 121645100408832000.0))))))))));
  *c = 1.0 / 1.0 + t2 * (-1.0 / 2.0 + t2 * (1.0 / 24.0 + t2 * (-1.0 / 720.0 + t2 * (1.0 / 40320.0 + t2 * (-1.0 / 3628800.0 + t2 * (1.0 / 479001600.0 + t2 * (-1.0 / 87178291200.0 + t2 * (1.0 / 20922789888000.0 + t2 * (-1.0 / 6402373705728000.0 + t2 * (1.0 / 2432902008176640000.0))))))))));
}

#define SYN_PI_2 1.57079632679489661923132169163975

/* sin(2 pi u), cos(2 pi u) for u in [0, 1) */
SYN_FN void syn_sincos_2pi(double u, double* s, double* c) {
  const double x = 4.0 * u;           /* exact */
  const int q = (int)x;               /* quadrant 0..3 */
  double f = x - (double)q;           /* exact, [0, 1) */
  int flip = 0;
  if (f > 0.5) { f = 1.0 - f; flip = 1; } /* exact */
  double so, co;
  syn_sincos_oct(f * SYN_PI_2, &so, &co);
  double sq = flip ? co : so, cq = flip ? so : co; /* angle inside the quadrant */
  if (q == 0) { *s = sq; *c = cq; }
  else if (q == 1) { *s = cq; *c = -sq; }
  else if (q == 2) { *s = -sq; *c = -cq; }
  else { *s = -cq; *c = sq; }
}

/* standard normal pair for pair index p of (seed, tid, sub) */
SYN_FN void syn_normal_pair(uint64_t seed, uint32_t tid, uint32_t sub, uint64_t p, double* z0, double* z1) {
  uint32_t w[4] = {(uint32_t)p, (uint32_t)(p >> 32), sub, (uint32_t)(seed >> 32)};
  syn_philox(w, (uint32_t)seed, tid);
  const double u1 = 1.0 - syn_u53(w[0], w[1]); /* (0, 1] */
  const double u2 = syn_u53(w[2], w[3]);       /* [0, 1) */
  const double r = syn_sqrt(-2.0 * syn_log(u1));
  double s, c;
  syn_sincos_2pi(u2, &s, &c);
  *z0 = r * c;
  *z1 = r * s;
}

/* uniform in (0, 1] for index i of (seed, tid, sub) */
SYN_FN double syn_uniform(uint64_t seed, uint32_t tid, uint32_t sub, uint64_t i) {
  uint32_t w[4] = {(uint32_t)i, (uint32_t)(i >> 32), sub, (uint32_t)(seed >> 32)};
  syn_philox(w, (uint32_t)seed, tid);
  return 1.0 - syn_u53(w[0], w[1]);
}

SYN_FN double syn_neg_softplus(double z) {
  const double az = z < 0.0 ? -z : z;
  return -((z > 0.0 ? z : 0.0) + syn_log1p01(syn_exp(-az)));
}

SYN_FN double syn_sigmoid(double z) { return 1.0 / (1.0 + syn_exp(-z)); }

/*
 * fp64 -> bf16 bit pattern, round to nearest, ties to even, directly from
 * fp64 (no intermediate fp32 rounding). Normal-range fast path rounds the
 * significand to 7 fraction bits with an integer add; a carry bumps the
 * exponent. Below the bf16 normal range the quantum is fixed at 2^-133.
 */
SYN_FN uint16_t syn_bf16(double x) {
  uint64_t b = syn_bits(x);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000);
  const uint64_t e = (b >> 52) & 0x7ff;
  if (e == 0x7ff) return (uint16_t)(sign | ((b & 0x000fffffffffffffull) ? 0x7fc0 : 0x7f80));
  if (e > 1023 + 127) return (uint16_t)(sign | 0x7f80);
  if (e >= 1023 - 126) {
    const uint64_t lsb = (b >> 45) & 1;
    b += ((uint64_t)1 << 44) - 1 + lsb;
    if (((b >> 52) & 0x7ff) > 1023 + 127) return (uint16_t)(sign | 0x7f80);
    /* re-bias the fp64 exponent to the fp32/bf16 one */
    const uint64_t e2 = ((b >> 52) & 0x7ff) - 1023 + 127;
    return (uint16_t)(sign | (uint16_t)(e2 << 7) | (uint16_t)((b >> 45) & 0x7f));
  }
  /* subnormal bf16: value = n * 2^-133, n = round(|x| * 2^133) */
  const double ax = syn_from_bits(b & 0x7fffffffffffffffull) * 10889035741470030830827987437816582766592.0; /* 2^133 */
  uint32_t n = (uint32_t)ax;                 /* truncation; ax <= 2^7 here */
  const double fr = ax - (double)n;           /* exact */
  if (fr > 0.5 || (fr == 0.5 && (n & 1))) n += 1;
  return (uint16_t)(sign | (uint16_t)n);       /* n == 128 rolls into the smallest normal */
}

/* fp64 -> fp32 round to nearest even: the C conversion on both builds */
SYN_FN float syn_f32(double x) { return (float)x; }

#endif /* SYNTH_CORE_H */
