// norm.hip - the between-layer norm of a stack of routed MoE layers:
// h <- RMSNorm(h + MoE(h)) (the residual add is the layer's combine; this is
// the norm), RMSNorm(v) = v / sqrt(mean(v^2) + eps) with unit gain.  The
// backbone's RMS norms sit before attention and before each FFN ("Surface
// Scout", weight inventory); with attention left out they meet here.
#include "device.hpp"
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kNormThreads = 256;

// One block per row: the factor by block_row_inv (the order the router also
// follows when it normalises a row itself), then the scaling.  out may alias
// v.
__global__ __launch_bounds__(kNormThreads) void k_rmsnorm(const float* v, int d, float eps,
                                                          float* out) {
  static_assert(kNormThreads == 256, "block_row_inv's summation order");
  __shared__ float part[kNormThreads / 64];
  const int t = blockIdx.x;
  const float4* row = reinterpret_cast<const float4*>(v + (int64_t)t * d);
  const int n4 = d / 4;
  const float inv = block_row_inv(v + (int64_t)t * d, d, eps, part);
  float4* dst = reinterpret_cast<float4*>(out + (int64_t)t * d);
  for (int i = threadIdx.x; i < n4; i += kNormThreads) {
    const float4 q = row[i];
    dst[i] = make_float4(q.x * inv, q.y * inv, q.z * inv, q.w * inv);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const float* v, int B, int d, float eps, float* out, hipStream_t s) {
  hipLaunchKernelGGL(k_rmsnorm, dim3(B), dim3(kNormThreads), 0, s, v, d, eps, out);
  return hipGetLastError();
}

}  // namespace smoe
