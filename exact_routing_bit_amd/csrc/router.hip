// router.hip - exact routing and the layer-major inversion on the device.
//
//  k_logits_prep : logits[t,e] = sum_i Wr[e,i] x[t,i] (fp32), one wave per
//                  (expert, 8-token tile); the same launch converts x to the
//                  prepped fp16 activation layout the expert kernels read.
//  k_topk_union  : one workgroup.  Top-k per token by (logit desc, index asc)
//                  with softmax / norm_topk_prob weights ("Data Flow", serial
//                  step "EXACT ROUTING"; "Surface Scout", model config), then
//                  the union of the batch's experts and the per-expert pair
//                  lists ("Layer-Major Batched Prefill", "The Inversion"),
//                  all from LDS, with no host synchronisation.
#include <float.h>
#include <limits.h>

#include "device.hpp"
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kLogitTokens = 8;   // tokens per logits block
constexpr int kLogitWaves = 4;    // experts per logits block (one per wave)

// Prepped activations of one (token, 64-input group): 8 chunks + group sums.
__device__ void prep_group(const float* x, int d, int t, int g, uint16_t* xp, float2* xs) {
  const float4* src = reinterpret_cast<const float4*>(x + (int64_t)t * d + g * 64);
  uint4* dst = reinterpret_cast<uint4*>(xp + (int64_t)t * d + g * 64);
  float X = 0.f, S = 0.f;
#pragma unroll 2
  for (int c = 0; c < 8; ++c) {
    const float4 lo = src[2 * c], hi = src[2 * c + 1];
    const float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    dst[c] = prep_chunk(v, &X, &S);
  }
  xs[(int64_t)t * (d / 64) + g] = make_float2(X, 1024.0f * S);
}

template <bool kBf16>
__global__ __launch_bounds__(256) void k_logits_prep(RouteArgs a, int do_logits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (do_logits) {
    const int e = blockIdx.x * kLogitWaves + wave;
    const int t0 = blockIdx.y * kLogitTokens;
    const int nt = min(kLogitTokens, a.B - t0);
    if (e < a.E && nt > 0) {
      float acc[kLogitTokens];
#pragma unroll
      for (int j = 0; j < kLogitTokens; ++j) acc[j] = 0.f;
      for (int i = lane * 8; i < a.d; i += 512) {
        float wv[8];
        if (kBf16) {
          const uint4 raw =
              *reinterpret_cast<const uint4*>((const uint16_t*)a.router_w + (int64_t)e * a.d + i);
          const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            wv[2 * q] = __uint_as_float(r4[q] << 16);
            wv[2 * q + 1] = __uint_as_float(r4[q] & 0xFFFF0000u);
          }
        } else {
          const float4* wp = reinterpret_cast<const float4*>((const float*)a.router_w +
                                                             (int64_t)e * a.d + i);
          const float4 lo = wp[0], hi = wp[1];
          wv[0] = lo.x; wv[1] = lo.y; wv[2] = lo.z; wv[3] = lo.w;
          wv[4] = hi.x; wv[5] = hi.y; wv[6] = hi.z; wv[7] = hi.w;
        }
#pragma unroll
        for (int j = 0; j < kLogitTokens; ++j) {
          if (j < nt) {
            const float4* xp4 = reinterpret_cast<const float4*>(a.x + (int64_t)(t0 + j) * a.d + i);
            const float4 lo = xp4[0], hi = xp4[1];
            acc[j] += wv[0] * lo.x + wv[1] * lo.y + wv[2] * lo.z + wv[3] * lo.w + wv[4] * hi.x +
                      wv[5] * hi.y + wv[6] * hi.z + wv[7] * hi.w;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kLogitTokens; ++j) {
        const float tot = wave_sum(acc[j]);
        if (j < nt && lane == 0) a.logits[(int64_t)(t0 + j) * a.E + e] = tot;
      }
    }
  }
  if (a.xp != nullptr) {
    const int G = a.d / 64;
    const int units = a.B * G;
    const int nthreads = gridDim.x * gridDim.y * blockDim.x;
    const int gid = (blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x;
    for (int u = gid; u < units; u += nthreads) prep_group(a.x, a.d, u / G, u % G, a.xp, a.xs);
  }
}

__global__ __launch_bounds__(256) void k_prep(const float* x, int B, int d, uint16_t* xp,
                                              float2* xs) {
  const int G = d / 64;
  const int u = blockIdx.x * blockDim.x + threadIdx.x;
  if (u < B * G) prep_group(x, d, u / G, u % G, xp, xs);
}

// (v, e) ranks above (bv, be): larger logit, or equal logit and lower index.
__device__ __forceinline__ bool ranks_above(float v, int e, float bv, int be) {
  return v > bv || (v == bv && e < be);
}

constexpr int kTopkThreads = 512;

__global__ __launch_bounds__(kTopkThreads) void k_topk_union(RouteArgs a, int do_topk,
                                                             int do_union) {
  __shared__ int32_t s_idx[kMaxPairs];
  __shared__ int32_t s_hist[kMaxExperts];
  __shared__ int32_t s_pos[kMaxExperts];
  __shared__ uint32_t s_mask[kMaxExperts * (kMaxPairs / 32)];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nwaves = kTopkThreads / 64;
  const int E = a.E, K = a.K, B = a.B, P = B * K;

  if (do_topk) {
    for (int t = wave; t < B; t += nwaves) {
      float v[4];
      bool taken[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        v[j] = e < E ? a.logits[(int64_t)t * E + e] : -FLT_MAX;
        taken[j] = e >= E;
      }
      float my_v = 0.f;
      int my_e = 0;
      for (int k = 0; k < K; ++k) {
        float bv = -INFINITY;
        int be = INT_MAX;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = lane + 64 * j;
          if (!taken[j] && ranks_above(v[j], e, bv, be)) { bv = v[j]; be = e; }
        }
        for (int off = 32; off > 0; off >>= 1) {
          const float ov = __shfl_xor(bv, off, 64);
          const int oe = __shfl_xor(be, off, 64);
          if (ranks_above(ov, oe, bv, be)) { bv = ov; be = oe; }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (be == lane + 64 * j) taken[j] = true;
        if (lane == k) { my_v = bv; my_e = be; }
      }
      // weights: p_k = exp(l_k - max); divide by the top-k sum (norm_topk_prob)
      // or by the full softmax denominator.
      const float m = __shfl(my_v, 0, 64);
      const float p = lane < K ? expf(my_v - m) : 0.f;
      float den;
      if (a.norm) {
        den = wave_sum(p);
      } else {
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (lane + 64 * j < E) z += expf(v[j] - m);
        den = wave_sum(z);
      }
      if (lane < K) {
        a.topk_idx[t * K + lane] = my_e;
        a.topk_w[t * K + lane] = p / den;
        s_idx[t * K + lane] = my_e;
      }
    }
  }
  if (!do_union) return;
  __syncthreads();
  if (!do_topk)
    for (int p = threadIdx.x; p < P; p += kTopkThreads) s_idx[p] = a.topk_idx[p];
  const int W = (P + 31) / 32;
  for (int i = threadIdx.x; i < E; i += kTopkThreads) s_hist[i] = 0;
  for (int i = threadIdx.x; i < E * W; i += kTopkThreads) s_mask[i] = 0u;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += kTopkThreads) {
    const int e = s_idx[p];
    if (e >= 0 && e < E) {
      atomicAdd(&s_hist[e], 1);
      atomicOr(&s_mask[e * W + (p >> 5)], 1u << (p & 31));
    } else {
      atomicOr(a.status, (uint32_t)SMOE_STATUS_BAD_EXPERT);
      a.pair_pos[p] = -1;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // exclusive scans of counts and of non-empty experts; lane l owns experts 4l..4l+3
    int c[4], cnt = 0, nz = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      c[j] = e < E ? s_hist[e] : 0;
      cnt += c[j];
      nz += c[j] > 0;
    }
    int inc_c = cnt, inc_nz = nz;
    for (int off = 1; off < 64; off <<= 1) {
      const int oc = __shfl_up(inc_c, off, 64), onz = __shfl_up(inc_nz, off, 64);
      if (lane >= off) { inc_c += oc; inc_nz += onz; }
    }
    int pos = inc_c - cnt, uid = inc_nz - nz;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      if (e < E) s_pos[e] = pos;
      if (c[j] > 0) {
        a.union_experts[uid] = e;
        a.expert_offsets[uid] = pos;
        uid += 1;
      }
      pos += c[j];
    }
    if (lane == 63) {
      *a.n_union = inc_nz;
      a.expert_offsets[inc_nz] = inc_c;
    }
  }
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += kTopkThreads) {
    const int e = s_idx[p];
    if (e < 0 || e >= E) continue;
    const uint32_t* m = s_mask + e * W;
    int rank = __popc(m[p >> 5] & ((1u << (p & 31)) - 1u));
    for (int i = 0; i < (p >> 5); ++i) rank += __popc(m[i]);
    const int q = s_pos[e] + rank;
    a.pair_list[q] = p;
    a.pair_pos[p] = q;
  }
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_router(const RouteArgs& a, bool logits_in, bool do_topk, bool do_union,
                         hipStream_t s) {
  const bool do_logits = !logits_in;
  if (do_logits || a.xp != nullptr) {
    const dim3 grid((a.E + kLogitWaves - 1) / kLogitWaves,
                    (a.B + kLogitTokens - 1) / kLogitTokens);
    if (a.router_bf16)
      hipLaunchKernelGGL(k_logits_prep<true>, grid, dim3(256), 0, s, a, (int)do_logits);
    else
      hipLaunchKernelGGL(k_logits_prep<false>, grid, dim3(256), 0, s, a, (int)do_logits);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (do_topk || do_union) {
    hipLaunchKernelGGL(k_topk_union, dim3(1), dim3(kTopkThreads), 0, s, a, (int)do_topk,
                       (int)do_union);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_prep(const float* x, int B, int d, uint16_t* xp, float2* xs, hipStream_t s) {
  const int units = B * (d / 64);
  hipLaunchKernelGGL(k_prep, dim3((units + 255) / 256), dim3(256), 0, s, x, B, d, xp, xs);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_u32, dim3((n + 255) / 256), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace smoe
