/*
 * synth.c - CPU side of the seeded synthetic-input generator.
 *
 * Makes the inputs of one routed mixture-of-experts layer: hidden states
 * (fp32 normals, then RMS-normalised), router gates (fp32 or bf16 normals),
 * and expert projection matrices drawn as fp32 normals and quantised to
 * 4-bit affine codes with group size 64 (packed u32 words, bf16 scales and
 * biases).  The GPU generator (synth_gpu.hip) makes the same bits.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared synth.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define SYN_FN static inline
#include "synth_math.h"

#define SYN_API __attribute__((visibility("default")))

SYN_API void synth_philox(const uint32_t* ctr, const uint32_t* key, uint32_t* out) {
  syn_philox4x32_10(ctr[0], ctr[1], ctr[2], ctr[3], key[0], key[1], out);
}

SYN_API double synth_normal_one(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t stream_id,
                                uint64_t n) {
  return syn_normal(seed, layer, tensor, stream_id, n);
}

SYN_API double synth_ln_u32(uint64_t n) { return syn_ln_u32(n); }

SYN_API void synth_sincos_turn(uint32_t b, double* sn, double* cs) { syn_sincos_turn(b, sn, cs); }

/* out[i] = float(sigma * normal(start + i)), i < n */
SYN_API void synth_normals(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t stream_id,
                           uint64_t start, int64_t n, double sigma, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = (float)(sigma * syn_normal(seed, layer, tensor, stream_id, start + (uint64_t)i));
}

/* Hidden states [B, d]: z = float(normal(t*d + i)), then per row
 * x = float(z / sqrt(mean(z^2) + eps)) with the mean and root in double. */
SYN_API void synth_hidden(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t stream_id,
                          int B, int d, double eps, float* out) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < B; ++t) {
    float* row = out + (int64_t)t * d;
    double ss = 0.0;
    for (int i = 0; i < d; ++i) {
      const float z = (float)syn_normal(seed, layer, tensor, stream_id, (uint64_t)t * d + i);
      row[i] = z;
      ss = ss + (double)z * (double)z;
    }
    const double inv = 1.0 / sqrt(ss / (double)d + eps);
    for (int i = 0; i < d; ++i) row[i] = (float)((double)row[i] * inv);
  }
}

/* Router gate [E, d]: float(sigma * normal(e*d + i)); as bf16 bit patterns
 * (round to nearest even) when as_bf16 != 0, else fp32. */
SYN_API void synth_router(uint64_t seed, uint32_t layer, uint32_t tensor, int E, int d, double sigma,
                          int as_bf16, void* out) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < (int64_t)E * d; ++n) {
    const float w = (float)(sigma * syn_normal(seed, layer, tensor, 0, (uint64_t)n));
    if (as_bf16)
      ((uint16_t*)out)[n] = syn_bf16_rne(w);
    else
      ((float*)out)[n] = w;
  }
}

/* Quantised expert matrices for experts e0 .. e0+nE-1 of one tensor:
 * expert e's [rows, cols] matrix goes to w + (e-e0)*stride_w (u32 words,
 * row-major [rows, cols/8]) and s/b + (e-e0)*stride_sb ([rows, cols/64]). */
SYN_API int synth_quant_experts(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t e0, int nE,
                                int rows, int cols, double sigma, uint32_t* w, uint16_t* s,
                                uint16_t* b, int64_t stride_w, int64_t stride_sb) {
  if (cols % 64 != 0 || rows <= 0 || nE <= 0) return -1;
  const int64_t G = cols / 64;
  const int64_t total = (int64_t)nE * rows * G;
#pragma omp parallel for schedule(static)
  for (int64_t u = 0; u < total; ++u) {
    const int64_t e = u / ((int64_t)rows * G);
    const int64_t rem = u % ((int64_t)rows * G);
    const int64_t r = rem / G, g = rem % G;
    syn_gen_group(seed, layer, tensor, e0 + (uint32_t)e, cols, r, g, sigma,
                  w + e * stride_w + r * (cols / 8) + g * 8,
                  s + e * stride_sb + r * G + g,
                  b + e * stride_sb + r * G + g);
  }
  return 0;
}

/* Quantise a given fp32 matrix [rows, cols] with the same group rule. */
SYN_API int synth_quantize_matrix(const float* W, int rows, int cols, uint32_t* w, uint16_t* s,
                                  uint16_t* b) {
  if (cols % 64 != 0) return -1;
  const int64_t G = cols / 64;
#pragma omp parallel for schedule(static)
  for (int64_t u = 0; u < (int64_t)rows * G; ++u) {
    const int64_t r = u / G, g = u % G;
    syn_quantize_group64(W + r * cols + g * 64, w + r * (cols / 8) + g * 8, s + u, b + u);
  }
  return 0;
}

SYN_API int synth_num_threads(void) { return omp_get_max_threads(); }
