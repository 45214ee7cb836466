/*
 * synth_math.h - the arithmetic of the seeded synthetic-input generator.
 *
 * This header is included by the CPU generator (synth.c, built with gcc) and
 * by the GPU generator (synth_gpu.hip, built with hipcc).  The includer
 * defines SYN_FN (the function qualifier) before including it.  Every step
 * uses integer operations or single IEEE-754 double/float operations (add,
 * sub, mul, div, sqrt, rint), each correctly rounded, and both translation
 * units are compiled with -ffp-contract=off, so the CPU and the GPU produce
 * identical bits for every generated value.  A test compares them.
 *
 * Nothing here is part of the mixture-of-experts method: it only makes
 * inputs (hidden states, router gates, quantised expert weights).
 *
 * Random numbers: Philox4x32-10, the counter-based generator of Salmon,
 * Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
 * (SC'11).  Normals: the Box-Muller transform, with ln, sin and cos written
 * out as fixed series so that no platform libm decides a bit.
 */
#ifndef SYNTH_MATH_H
#define SYNTH_MATH_H

#include <stdint.h>

#ifndef SYN_FN
#error "define SYN_FN before including synth_math.h"
#endif

/* ---------------------------------------------------------------- Philox */
#define SYN_PHILOX_M0 0xD2511F53u
#define SYN_PHILOX_M1 0xCD9E8D57u
#define SYN_PHILOX_W0 0x9E3779B9u
#define SYN_PHILOX_W1 0xBB67AE85u

SYN_FN void syn_philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                              uint32_t k0, uint32_t k1, uint32_t out[4]) {
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += SYN_PHILOX_W0; k1 += SYN_PHILOX_W1; }
    const uint64_t p0 = (uint64_t)SYN_PHILOX_M0 * (uint64_t)c0;
    const uint64_t p1 = (uint64_t)SYN_PHILOX_M1 * (uint64_t)c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* ------------------------------------------------- ln, sin, cos by series */
/* ln(n * 2^-32) for n in [1, 2^32]: n = m * 2^e with m in [sqrt(1/2), sqrt(2)),
 * ln m = 2 atanh(s), s = (m-1)/(m+1), |s| < 0.1716, series to s^21. */
SYN_FN double syn_ln_u32(uint64_t n) {
  if (n >= 4294967296ull) return 0.0;
  int e = 63 - __builtin_clzll(n);
  double inv_pow2;                                    /* 2^-e, built from its bits */
  {
    const uint64_t bits = (uint64_t)(1023 - e) << 52;
    __builtin_memcpy(&inv_pow2, &bits, 8);
  }
  double m = (double)n * inv_pow2;                    /* exact: power-of-two scaling */
  if (m > 1.4142135623730951) { m = m * 0.5; e += 1; }
  const double s = (m - 1.0) / (m + 1.0);
  const double s2 = s * s;
  double p = 1.0 / 21.0;
  p = p * s2 + 1.0 / 19.0;
  p = p * s2 + 1.0 / 17.0;
  p = p * s2 + 1.0 / 15.0;
  p = p * s2 + 1.0 / 13.0;
  p = p * s2 + 1.0 / 11.0;
  p = p * s2 + 1.0 / 9.0;
  p = p * s2 + 1.0 / 7.0;
  p = p * s2 + 1.0 / 5.0;
  p = p * s2 + 1.0 / 3.0;
  p = p * s2 + 1.0;
  const double lnm = 2.0 * s * p;
  return (double)(e - 32) * 0.6931471805599453 + lnm;
}

/* sin and cos of 2*pi*b/2^32: the quadrant comes from the top two bits (an
 * exact reduction), the remainder phi in [0, pi/2) goes through Taylor series
 * to degree 23. */
SYN_FN void syn_sincos_turn(uint32_t b, double* sn, double* cs) {
  const uint32_t q = b >> 30;
  const double f = (double)(b & 0x3FFFFFFFu) * (1.0 / 1073741824.0);
  const double phi = f * 1.5707963267948966;
  const double p2 = phi * phi;
  double S = -1.0 / 25852016738884976640000.0;           /* -1/23! */
  S = S * p2 + 1.0 / 51090942171709440000.0;             /* 1/21! */
  S = S * p2 - 1.0 / 121645100408832000.0;               /* 1/19! */
  S = S * p2 + 1.0 / 355687428096000.0;                  /* 1/17! */
  S = S * p2 - 1.0 / 1307674368000.0;                    /* 1/15! */
  S = S * p2 + 1.0 / 6227020800.0;                       /* 1/13! */
  S = S * p2 - 1.0 / 39916800.0;                         /* 1/11! */
  S = S * p2 + 1.0 / 362880.0;                           /* 1/9!  */
  S = S * p2 - 1.0 / 5040.0;                             /* 1/7!  */
  S = S * p2 + 1.0 / 120.0;                              /* 1/5!  */
  S = S * p2 - 1.0 / 6.0;                                /* 1/3!  */
  S = S * p2 + 1.0;
  const double sphi = phi * S;
  double C = 1.0 / 1124000727777607680000.0;             /* 1/22! */
  C = C * p2 - 1.0 / 2432902008176640000.0;              /* 1/20! */
  C = C * p2 + 1.0 / 6402373705728000.0;                 /* 1/18! */
  C = C * p2 - 1.0 / 20922789888000.0;                   /* 1/16! */
  C = C * p2 + 1.0 / 87178291200.0;                      /* 1/14! */
  C = C * p2 - 1.0 / 479001600.0;                        /* 1/12! */
  C = C * p2 + 1.0 / 3628800.0;                          /* 1/10! */
  C = C * p2 - 1.0 / 40320.0;                            /* 1/8!  */
  C = C * p2 + 1.0 / 720.0;                              /* 1/6!  */
  C = C * p2 - 1.0 / 24.0;                               /* 1/4!  */
  C = C * p2 + 1.0 / 2.0;                                /* 1/2!  */
  C = 1.0 - C * p2;
  const double cphi = C;
  switch (q) {
    case 0: *cs = cphi;  *sn = sphi;  break;
    case 1: *cs = -sphi; *sn = cphi;  break;
    case 2: *cs = -cphi; *sn = -sphi; break;
    default: *cs = sphi; *sn = -cphi; break;
  }
}

/* Two standard normals from one Philox output pair (a, b): Box-Muller with
 * u1 = (a+1)/2^32 in (0, 1] and angle 2*pi*b/2^32. */
SYN_FN void syn_box_muller(uint32_t a, uint32_t b, double* z0, double* z1) {
  const double r = sqrt(-2.0 * syn_ln_u32((uint64_t)a + 1u));
  double sn, cs;
  syn_sincos_turn(b, &sn, &cs);
  *z0 = r * cs;
  *z1 = r * sn;
}

/* Standard normal number n of the stream (seed, layer, tensor, stream_id).
 * Element n uses Philox counter (n/2 low, n/2 high, stream_id,
 * layer<<8 | tensor) with key (seed low, seed high); even n take the cosine
 * branch of Box-Muller on output words 0,1, odd n the sine branch. */
SYN_FN double syn_normal(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t stream_id,
                         uint64_t n) {
  uint32_t o[4];
  const uint64_t j = n >> 1;
  syn_philox4x32_10((uint32_t)j, (uint32_t)(j >> 32), stream_id, (layer << 8) | (tensor & 0xFFu),
                    (uint32_t)seed, (uint32_t)(seed >> 32), o);
  double z0, z1;
  syn_box_muller(o[0], o[1], &z0, &z1);
  return (n & 1u) ? z1 : z0;
}

/* --------------------------------------------------------- bf16 helpers */
SYN_FN uint32_t syn_f32_bits(float f) { uint32_t u; __builtin_memcpy(&u, &f, 4); return u; }
SYN_FN float syn_bits_f32(uint32_t u) { float f; __builtin_memcpy(&f, &u, 4); return f; }
/* round-to-nearest-even fp32 -> bf16 (finite inputs) */
SYN_FN uint16_t syn_bf16_rne(float f) {
  uint32_t u = syn_f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
SYN_FN float syn_bf16_f32(uint16_t h) { return syn_bits_f32((uint32_t)h << 16); }

/* ------------------------------------------------ 4-bit affine quantiser */
/* One group of 64 consecutive fp32 weights of a row -> 8 packed words
 * (element i at bits 4*(i%8) of word i/8), a bf16 scale s and bias b with
 * w ~= s*q + b.  s = bf16((max-min)/15), b = bf16(min),
 * q = clamp(rint((w-b)/s), 0, 15), and q = 0 when s == 0. */
SYN_FN void syn_quantize_group64(const float* w, uint32_t* words, uint16_t* s_out, uint16_t* b_out) {
  float mn = w[0], mx = w[0];
  for (int i = 1; i < 64; ++i) {
    mn = w[i] < mn ? w[i] : mn;
    mx = w[i] > mx ? w[i] : mx;
  }
  const float range = mx - mn;
  const float sf = range / 15.0f;
  const uint16_t s16 = syn_bf16_rne(sf);
  const uint16_t b16 = syn_bf16_rne(mn);
  const float s = syn_bf16_f32(s16);
  const float b = syn_bf16_f32(b16);
  for (int j = 0; j < 8; ++j) {
    uint32_t word = 0;
    for (int i = 0; i < 8; ++i) {
      uint32_t q = 0;
      if (s > 0.0f) {
        float t = rintf((w[8 * j + i] - b) / s);
        t = t < 0.0f ? 0.0f : (t > 15.0f ? 15.0f : t);
        q = (uint32_t)t;
      }
      word |= q << (4 * i);
    }
    words[j] = word;
  }
  *s_out = s16;
  *b_out = b16;
}

/* One quantised group of the generated matrix (seed, layer, tensor, expert):
 * row r, group g of a [rows, cols] matrix whose element (r, c) is
 * float(sigma * normal(r*cols + c)). */
SYN_FN void syn_gen_group(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t expert,
                          int64_t cols, int64_t r, int64_t g, double sigma,
                          uint32_t* words, uint16_t* s_out, uint16_t* b_out) {
  float w[64];
  const uint64_t n0 = (uint64_t)(r * cols + g * 64);
  for (int i = 0; i < 64; i += 2) {
    uint32_t o[4];
    const uint64_t j = (n0 + (uint64_t)i) >> 1;
    syn_philox4x32_10((uint32_t)j, (uint32_t)(j >> 32), expert, (layer << 8) | (tensor & 0xFFu),
                      (uint32_t)seed, (uint32_t)(seed >> 32), o);
    double z0, z1;
    syn_box_muller(o[0], o[1], &z0, &z1);
    w[i] = (float)(sigma * z0);
    w[i + 1] = (float)(sigma * z1);
  }
  syn_quantize_group64(w, words, s_out, b_out);
}

#endif /* SYNTH_MATH_H */
