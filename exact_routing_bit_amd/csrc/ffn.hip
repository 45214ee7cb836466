// ffn.hip - dispatch of the expert FFN passes and the combine of large batches.
//
// Small batches (B <= 2: the decode regime) take the matrix-vector kernels of
// ffn_gemv.hip, whose down pass also combines.  Prefill chunks take the MFMA
// kernels of ffn_mfma.hip, which write y per pair, and k_combine below forms
// out[t] = residual[t] + sum_k w[t,k] y[t*K+k] in rank order ("Data Flow":
// "gather GPU outputs x routing weights -> routed_out", "residual += ..."),
// plus the shared expert's output when the layer has one:
// residual + (shared_out + routed_out).
// No float atomics: every output element has exactly one writer.
#include "device.hpp"
#include "smoe_internal.hpp"

namespace smoe {
namespace {

// out[t, r] = residual[t, r] + sum_k w[t, k] * y[t*K + k, r], k ascending;
// with a shared expert, residual + (sy[t, r] + that sum).
__global__ __launch_bounds__(256) void k_combine(FfnArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;   // one float4 of out
  const int per_row = a.d / 4;
  if (i >= a.B * per_row) return;
  const int t = i / per_row, r4 = i - t * per_row;
  // every load first (pair rows are always valid memory; a dropped pair's row
  // is loaded and not used), so that they overlap instead of each waiting on
  // the previous pair's position
  float4 y[kMaxTopK];
  float w[kMaxTopK];
  int pos[kMaxTopK];
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k < a.K) {
      const int p = t * a.K + k;
      pos[k] = a.pair_pos[p];
      w[k] = a.topk_w[p];
      y[k] = reinterpret_cast<const float4*>(a.y + (int64_t)p * a.d)[r4];
    }
  }
  const float4 res = a.residual ? reinterpret_cast<const float4*>(a.residual + (int64_t)t * a.d)[r4]
                                : make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 shv = a.fs > 0 ? reinterpret_cast<const float4*>(a.sy + (int64_t)t * a.d)[r4]
                              : make_float4(0.f, 0.f, 0.f, 0.f);
  // k ascending, fp32, then the residual
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < kMaxTopK; ++k) {
    if (k < a.K && pos[k] >= 0) {
      acc.x += w[k] * y[k].x;
      acc.y += w[k] * y[k].y;
      acc.z += w[k] * y[k].z;
      acc.w += w[k] * y[k].w;
    }
  }
  if (a.fs > 0) {                                 // shared_out + routed_out
    acc.x = shv.x + acc.x;
    acc.y = shv.y + acc.y;
    acc.z = shv.z + acc.z;
    acc.w = shv.w + acc.w;
  }
  if (a.residual) {
    acc.x = res.x + acc.x;
    acc.y = res.y + acc.y;
    acc.z = res.z + acc.z;
    acc.w = res.w + acc.w;
  }
  reinterpret_cast<float4*>(a.out + (int64_t)t * a.d)[r4] = acc;
}

}  // namespace

hipError_t launch_gate_up(const FfnArgs& a, hipStream_t s, const LaunchTiming* t) {
  if (gemv_path_ok(a)) return launch_gemv(a, s, true, t);
  return launch_ffn_mfma(a, s, true, t);
}

// For small batches the down kernel also does the combine.
hipError_t launch_down(const FfnArgs& a, hipStream_t s, const LaunchTiming* t) {
  if (gemv_path_ok(a)) return launch_gemv(a, s, false, t);
  return launch_ffn_mfma(a, s, false, t);
}

hipError_t launch_combine(const FfnArgs& a, hipStream_t s, const LaunchTiming* t) {
  if (gemv_path_ok(a)) return hipSuccess;
  const int n4 = a.B * a.d / 4;
  SMOE_LAUNCH(t, k_combine, dim3((n4 + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s) {
  hipError_t err = launch_gate_up(a, s);
  if (err == hipSuccess) err = launch_down(a, s);
  if (err == hipSuccess) err = launch_combine(a, s);
  return err;
}

}  // namespace smoe
