// diag.hip - smoe_stream_read: a plain streaming read of a device buffer, the
// calibration that measurements of the layer's kernels are set against (the
// read bandwidth this part reaches on a pure stream of 16-byte loads).
#include "device.hpp"
#include "smoe_internal.hpp"

#define SMOE_API extern "C" __attribute__((visibility("default")))

namespace smoe {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;        // 16-byte loads in flight per thread

// Grid-stride read of n16 16-byte words; each block writes the xor of what
// it read to sink[block], so that no load can be dropped.
__global__ __launch_bounds__(kReadThreads) void k_stream_read(const uint4* src, int64_t n16,
                                                              uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = ld_stream4(reinterpret_cast<const uint32_t*>(src + i + u * stride));
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = ld_stream4(reinterpret_cast<const uint32_t*>(src + i));
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[kReadThreads / 64];
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace
}  // namespace smoe

SMOE_API int smoe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                              void* stream) {
  if (src == nullptr || sink == nullptr || (reinterpret_cast<uintptr_t>(src) & 15) != 0 ||
      bytes % 16 != 0 || blocks < 1 || blocks > (1 << 20))
    return SMOE_EINVAL;
  if (bytes == 0) return SMOE_OK;
  hipLaunchKernelGGL(smoe::k_stream_read, dim3(blocks), dim3(smoe::kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                     (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? SMOE_OK : SMOE_EHIP;
}
