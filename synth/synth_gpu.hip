// synth_gpu.hip - GPU side of the seeded synthetic-input generator.
//
// Same recipe and same bits as synth.c (both include synth_math.h and are
// built with -ffp-contract=off).  It exists only so that multi-gigabyte
// expert stacks can be made in device memory in well under a second; the
// tests compare its output with the CPU generator's bit for bit.
//
// Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off -fPIC -shared
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#define SYN_FN __device__ static inline
#include "synth_math.h"

#define SYN_API extern "C" __attribute__((visibility("default")))

namespace {

__global__ void k_quant_experts(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t e0,
                                int64_t nE, int64_t rows, int64_t cols, double sigma, uint32_t* w,
                                uint16_t* s, uint16_t* b, int64_t stride_w, int64_t stride_sb) {
  const int64_t G = cols / 64;
  const int64_t total = nE * rows * G;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = u / (rows * G);
    const int64_t rem = u - e * rows * G;
    const int64_t r = rem / G, g = rem - r * G;
    uint32_t words[8];
    uint16_t sv, bv;
    syn_gen_group(seed, layer, tensor, e0 + (uint32_t)e, cols, r, g, sigma, words, &sv, &bv);
    uint32_t* dst = w + e * stride_w + r * (cols / 8) + g * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = words[j];
    s[e * stride_sb + r * G + g] = sv;
    b[e * stride_sb + r * G + g] = bv;
  }
}

__global__ void k_normals(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t stream_id,
                          uint64_t start, int64_t n, double sigma, float* out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = (float)(sigma * syn_normal(seed, layer, tensor, stream_id, start + (uint64_t)i));
}

// One thread per row: the row's sum of squares is a sequential fp64 sum, as on the CPU.
// One block per token: the normals in parallel, then the sum of squares in
// index order by one thread (fp64, the same order as the CPU generator, so
// the rows are bit-identical), then the scaling in parallel.
__global__ __launch_bounds__(256) void k_hidden(uint64_t seed, uint32_t layer, uint32_t tensor,
                                                 uint32_t stream_id, int B, int d, double eps,
                                                 float* out) {
  __shared__ double inv_s;
  const int t = blockIdx.x;
  if (t >= B) return;
  float* row = out + (int64_t)t * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x)
    row[i] = (float)syn_normal(seed, layer, tensor, stream_id, (uint64_t)t * d + i);
  __syncthreads();
  if (threadIdx.x == 0) {
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss = ss + (double)row[i] * (double)row[i];
    inv_s = 1.0 / sqrt(ss / (double)d + eps);
  }
  __syncthreads();
  const double inv = inv_s;
  for (int i = threadIdx.x; i < d; i += blockDim.x) row[i] = (float)((double)row[i] * inv);
}

__global__ void k_router(uint64_t seed, uint32_t layer, uint32_t tensor, int64_t n, double sigma,
                         int as_bf16, void* out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float w = (float)(sigma * syn_normal(seed, layer, tensor, 0, (uint64_t)i));
    if (as_bf16)
      ((uint16_t*)out)[i] = syn_bf16_rne(w);
    else
      ((float*)out)[i] = w;
  }
}

int grid_for(int64_t n, int block) {
  int64_t g = (n + block - 1) / block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

SYN_API int synth_gpu_quant_experts(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t e0,
                                    int nE, int rows, int cols, double sigma, uint32_t* w,
                                    uint16_t* s, uint16_t* b, int64_t stride_w, int64_t stride_sb,
                                    void* stream) {
  if (cols % 64 != 0 || rows <= 0 || nE <= 0) return -1;
  const int64_t total = (int64_t)nE * rows * (cols / 64);
  hipLaunchKernelGGL(k_quant_experts, dim3(grid_for(total, 256)), dim3(256), 0,
                     (hipStream_t)stream, seed, layer, tensor, e0, (int64_t)nE, (int64_t)rows,
                     (int64_t)cols, sigma, w, s, b, stride_w, stride_sb);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

SYN_API int synth_gpu_normals(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t stream_id,
                              uint64_t start, int64_t n, double sigma, float* out, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(k_normals, dim3(grid_for(n, 256)), dim3(256), 0, (hipStream_t)stream, seed,
                     layer, tensor, stream_id, start, n, sigma, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

SYN_API int synth_gpu_hidden(uint64_t seed, uint32_t layer, uint32_t tensor, uint32_t stream_id,
                             int B, int d, double eps, float* out, void* stream) {
  if (B <= 0) return 0;
  hipLaunchKernelGGL(k_hidden, dim3(B), dim3(256), 0, (hipStream_t)stream, seed, layer,
                     tensor, stream_id, B, d, eps, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

SYN_API int synth_gpu_router(uint64_t seed, uint32_t layer, uint32_t tensor, int E, int d,
                             double sigma, int as_bf16, void* out, void* stream) {
  const int64_t n = (int64_t)E * d;
  hipLaunchKernelGGL(k_router, dim3(grid_for(n, 256)), dim3(256), 0, (hipStream_t)stream, seed,
                     layer, tensor, n, sigma, as_bf16, out);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
