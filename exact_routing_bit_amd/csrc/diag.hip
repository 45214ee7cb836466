// diag.hip - calibrations that measurements of the layer's kernels are set
// against:
//   smoe_stream_read: a plain streaming read of a device buffer (the read
//     bandwidth this part reaches on a pure stream of 16-byte loads);
//   smoe_dma_read: the same bytes streamed global -> LDS by the direct copy
//     path the prefill FFN kernels use, in their access pattern (64-byte
//     pieces of 16-row tiles, a three-stage ring per wave, two workgroups of
//     four waves per compute unit) or in plain row-major order: the rate that
//     path reaches with no arithmetic behind it;
//   smoe_empty_launch: a kernel that does nothing (the cost of one more
//     launch in a stream of back-to-back kernels);
//   smoe_gpu_sleep: one wave that waits a given time on the device's clock
//     (queued ahead of a timed region, it lets the host enqueue the region's
//     first launches before the device reaches them);
//   smoe_grid_barrier: one device-wide barrier of a cooperative grid (the
//     cost of the alternative to a launch boundary: every block releases its
//     stores at device scope, counts itself in and waits for all the others).
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

// One 64-row unit of a [rows, row_bytes] matrix per wave, four waves a
// block, streamed into a ring of three 4 KB stages per wave with the direct
// global -> LDS copies; the wave xors one word of every landed stage (so
// that each wait means something) and the block writes the xor to
// sink[block].
//   kMode 0: stage k is bytes 64k .. 64k + 63 of each of the 64 rows, one
//            copy per 16-row tile (lane l: row l % 16, 16-byte piece l / 16),
//            the odd stages (a line's second half) nontemporal when rows start
//            on 128-byte lines: the words of the prefill FFN's stages;
//   kMode 1: stage k is the unit's bytes 4096k .. 4096k + 4095 in memory
//            order, one 1 KB copy per quarter.
constexpr int kDmaRing = 3;
constexpr int kDmaStageBytes = 4096;
template <int kMode>
__device__ __forceinline__ void dma_stage(const char* unit, int64_t row_bytes, int k, char* slot,
                                          int lane, bool nt) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const char* src = kMode == 0
                          ? unit + (int64_t)(16 * i + (lane & 15)) * row_bytes + 64 * k + 16 * (lane >> 4)
                          : unit + (int64_t)k * kDmaStageBytes + 1024 * i + 16 * lane;
    if (nt) dma16_to_lds_nt(src, slot + 1024 * i);
    else dma16_to_lds(src, slot + 1024 * i);
  }
}
template <int kMode>
__global__ __launch_bounds__(256, 2) void k_dma_read(const char* src, int64_t row_bytes, int units,
                                                     uint32_t* sink) {
  __shared__ __align__(16) char ring[kDmaRing][4][kDmaStageBytes];
  __shared__ uint32_t red[4];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + wave;
  uint32_t acc = 0;
  if (unit < units) {                               // uniform in the wave
    const char* base = src + (int64_t)unit * 64 * row_bytes;
    const int nst = (int)(64 * row_bytes / kDmaStageBytes);
    const bool line_aligned = row_bytes % 128 == 0;
    dma_stage<kMode>(base, row_bytes, 0, ring[0][wave], lane, false);
    if (nst > 1) dma_stage<kMode>(base, row_bytes, 1, ring[1][wave], lane, kMode == 0 && line_aligned);
    for (int k = 0; k < nst; ++k) {
      // slot (k + 2) % 3 held stage k - 1, whose word this wave has read
      if (k + 2 < nst)
        dma_stage<kMode>(base, row_bytes, k + 2, ring[(k + 2) % kDmaRing][wave], lane,
                         kMode == 0 && line_aligned && ((k + 2) & 1));
      if (k + 2 < nst) wait_vmcnt<8>();
      else if (k + 1 < nst) wait_vmcnt<4>();
      else wait_vmcnt<0>();
      acc ^= *reinterpret_cast<const uint32_t*>(ring[k % kDmaRing][wave] + 16 * lane);
    }
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ void k_empty() {}

// Waits `ticks` of the 100 MHz s_memrealtime clock, then ends.
__global__ __launch_bounds__(64) void k_sleep(uint64_t ticks) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < ticks) __builtin_amdgcn_s_sleep(16);
}

constexpr int kSpinLimit = 1 << 22;   // bounded wait: about 0.1 s, then give up

// Each block: its barrier, one acquire-release increment of *counter at
// device scope by thread 0, then (thread 0) acquire loads until all blocks
// have arrived or the spin limit is reached.  stamps[3 b ..]: s_memrealtime
// (100 MHz) at the block's start, after its increment, after its wait.
__global__ __launch_bounds__(256) void k_grid_barrier(uint32_t* counter, uint64_t* stamps,
                                                      int32_t* timed_out) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    int it = 0;
    while (__hip_atomic_load(counter, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < gridDim.x &&
           it < kSpinLimit) {
      __builtin_amdgcn_s_sleep(1);
      ++it;
    }
    if (it >= kSpinLimit) __hip_atomic_store(timed_out, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t t2 = __builtin_amdgcn_s_memrealtime();
    stamps[3 * blockIdx.x + 0] = t0;
    stamps[3 * blockIdx.x + 1] = t1;
    stamps[3 * blockIdx.x + 2] = t2;
  }
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

SMOE_API int smoe_dma_read(const void* src, size_t bytes, int32_t row_bytes, int32_t mode,
                           uint32_t* sink, int32_t sink_n, void* stream) {
  if (src == nullptr || sink == nullptr || (reinterpret_cast<uintptr_t>(src) & 15) != 0 ||
      row_bytes < 64 || row_bytes > 65536 || row_bytes % 64 != 0 || (mode != 0 && mode != 1))
    return SMOE_EINVAL;
  const int64_t units = (int64_t)(bytes / ((size_t)row_bytes * 64));
  const int64_t blocks = (units + 3) / 4;
  if (units > (1 << 24) || blocks > sink_n) return SMOE_EINVAL;
  if (units == 0) return SMOE_OK;
  const char* p = static_cast<const char*>(src);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == 0)
    hipLaunchKernelGGL(smoe::k_dma_read<0>, dim3((unsigned)blocks), dim3(256), 0, s, p,
                       (int64_t)row_bytes, (int)units, sink);
  else
    hipLaunchKernelGGL(smoe::k_dma_read<1>, dim3((unsigned)blocks), dim3(256), 0, s, p,
                       (int64_t)row_bytes, (int)units, sink);
  return hipGetLastError() == hipSuccess ? SMOE_OK : SMOE_EHIP;
}

SMOE_API int smoe_empty_launch(int32_t blocks, int32_t count, void* stream) {
  if (blocks < 1 || blocks > (1 << 20) || count < 0 || count > (1 << 20)) return SMOE_EINVAL;
  for (int i = 0; i < count; ++i)
    hipLaunchKernelGGL(smoe::k_empty, dim3(blocks), dim3(64), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? SMOE_OK : SMOE_EHIP;
}

SMOE_API int smoe_gpu_sleep(int32_t us, void* stream) {
  if (us < 0 || us > 100000) return SMOE_EINVAL;
  hipLaunchKernelGGL(smoe::k_sleep, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     (uint64_t)us * 100u);
  return hipGetLastError() == hipSuccess ? SMOE_OK : SMOE_EHIP;
}

SMOE_API int smoe_grid_barrier(int32_t blocks, uint32_t* counter, uint64_t* stamps,
                               int32_t* timed_out, void* stream) {
  if (blocks < 1 || blocks > 4096 || counter == nullptr || stamps == nullptr ||
      timed_out == nullptr)
    return SMOE_EINVAL;
  void* args[] = {&counter, &stamps, &timed_out};
  const hipError_t err = hipLaunchCooperativeKernel(
      reinterpret_cast<const void*>(smoe::k_grid_barrier), dim3(blocks), dim3(256), args, 0,
      static_cast<hipStream_t>(stream));
  return err == hipSuccess ? SMOE_OK : SMOE_EHIP;
}
