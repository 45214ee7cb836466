// route_dev.hpp - the router's per-block work for batches of B <= 2 tokens,
// shared by the router kernel and the single-launch decode layer: a token's
// activations into the prepped fp16 layout, and one expert's gate matvec
// ("Data Flow", serial step "EXACT ROUTING": gate matvec on the hidden state).
#pragma once

#include "device.hpp"
#include "smoe_internal.hpp"

namespace smoe {

constexpr int kRouteThreads = 256;              // 4 waves a block
static_assert(kRouteThreads == 256, "block_row_inv needs blocks of 256 threads");

// Prepped activations of one token per 256-thread block: thread j takes the
// 16-input pieces j and j + 256 (d <= 8192), so that the four pieces of a
// group of 64 inputs sit in four neighbouring lanes of one wave.  Every
// thread of the block must call it (it has block barriers).
//   1. the pieces are loaded (with norm_out: scaled by inv, the token's
//      RMSNorm factor, and written to norm_out);
//   2. the row's largest magnitude m gives a_t = 2^-floor(log2 m), clamped
//      to 2^-30 .. 2^30 (1 for a zero row), so that max |a_t x| is in [1, 2);
//   3. a_t * x goes to the prepped fp16 layout; the group sums are each
//      lane's piece sums added over the group's four lanes (the same order in
//      all four), and a_t goes to xa[t].
// All loads of a thread are issued before its first store.
constexpr int kPrepPieces = 2;                  // 16-input pieces a thread: 8192 / 16 / 256
__device__ __forceinline__ float token_scale(float mx) {
  if (!(mx > 0.0f)) return 1.0f;
  const int e = min(max(ilogbf(mx), -30), 30);
  return __builtin_ldexpf(1.0f, -e);
}
__device__ inline void prep_token(const float* x, int d, int t, uint16_t* xp, float2* xs, float* xa,
                           float* norm_out, float inv, float* red) {
  const int tid = threadIdx.x;
  const int np = d / 16;                        // pieces of the row, 4 a group
  const int nr = np > 256 ? 2 : 1;              // uniform
  float4 v4[kPrepPieces][4];
#pragma unroll
  for (int r = 0; r < kPrepPieces; ++r) {
    if (r >= nr) break;
    const int p = tid + 256 * r;
    const bool live = p < np;
    const float4* src = reinterpret_cast<const float4*>(x + (int64_t)t * d + (live ? p : 0) * 16);
#pragma unroll
    for (int c = 0; c < 4; ++c) v4[r][c] = live ? src[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float mx = 0.f;
#pragma unroll
  for (int r = 0; r < kPrepPieces; ++r) {
    if (r >= nr) break;
    const int p = tid + 256 * r;
    if (norm_out != nullptr) {
      float4* hn = reinterpret_cast<float4*>(norm_out + (int64_t)t * d + p * 16);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v4[r][c] = make_float4(v4[r][c].x * inv, v4[r][c].y * inv, v4[r][c].z * inv,
                               v4[r][c].w * inv);
        if (p < np) hn[c] = v4[r][c];
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v4[r][c].x), fabsf(v4[r][c].y)),
                           fmaxf(fabsf(v4[r][c].z), fabsf(v4[r][c].w))));
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  const float a = token_scale(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])));
  __syncthreads();                                // red may be reused after this
  const int G = d / 64;
#pragma unroll
  for (int r = 0; r < kPrepPieces; ++r) {
    if (r >= nr) break;
    const int p = tid + 256 * r;
    float X = 0.f, S = 0.f;
    uint4 out[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float4 lo = v4[r][2 * c], hi = v4[r][2 * c + 1];
      const float v[8] = {lo.x * a, lo.y * a, lo.z * a, lo.w * a, hi.x * a, hi.y * a, hi.z * a,
                          hi.w * a};
      out[c] = prep_chunk(v, &X, &S);
    }
    // every lane takes part (dead pieces add zeros: a group is live or dead as a whole)
    X = segment_sum16(X, 4);
    S = segment_sum16(S, 4);
    if (p < np) {
      uint4* dst = reinterpret_cast<uint4*>(xp + (int64_t)t * d + p * 16);
      dst[0] = out[0];
      dst[1] = out[1];
      if ((p & 3) == 0) xs[(int64_t)t * G + p / 4] = make_float2(X, 1024.0f * S);
    }
  }
  if (tid == 0) xa[t] = a;
}

// Logits of expert e for the NT = B <= 2 tokens, one 256-thread block: the
// row splits into pieces of 512 inputs, wave w taking pieces w, w + 4, ...
// (kM of them; lane l takes inputs 512 P + 8 l .. + 7, zeros past d).  Each
// wave's sums go to part[wave][t], and the block adds the four in wave
// order.  With a.norm_out the inputs are x * inv_t (the tokens' RMSNorm
// factors, from block_row_inv as smoe_rmsnorm forms them), rounded as
// smoe_rmsnorm rounds them.  Every thread of the block must call it (it has
// block barriers).  The gate rows are requested first (HBM), then the
// factors are formed, then the inputs (caches) are read.
template <bool kBf16, int NT, int kM>
__device__ inline void logits_block(const RouteArgs& a, int e, float (*part)[NT]) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = __lane_id();
  const int d = a.d;
  int idx[kM];
  bool ok[kM];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    idx[m] = 512 * (wave + 4 * m) + 8 * lane;
    ok[m] = idx[m] < d;
  }
  float w[kM][8];
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const int64_t at = (int64_t)e * d + (ok[m] ? idx[m] : 0);
    if (kBf16) {
      const uint4 raw = *reinterpret_cast<const uint4*>((const uint16_t*)a.router_w + at);
      const uint32_t r4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        w[m][2 * z] = ok[m] ? __uint_as_float(r4[z] << 16) : 0.f;
        w[m][2 * z + 1] = ok[m] ? __uint_as_float(r4[z] & 0xFFFF0000u) : 0.f;
      }
    } else {
      const float4* wp = reinterpret_cast<const float4*>((const float*)a.router_w + at);
      const float4 lo = wp[0], hi = wp[1];
      const float v8[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int z = 0; z < 8; ++z) w[m][z] = ok[m] ? v8[z] : 0.f;
    }
  }
  float inv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    inv[t] = a.norm_out != nullptr ? block_row_inv(a.x + (int64_t)t * d, d, a.norm_eps, &part[0][0])
                                   : 1.0f;
  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float4 xv[kM][2];
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      const float4* xp4 = reinterpret_cast<const float4*>(a.x + (int64_t)t * d + (ok[m] ? idx[m] : 0));
      xv[m][0] = xp4[0];
      xv[m][1] = xp4[1];
    }
    float sum = 0.f;
#pragma unroll
    for (int m = 0; m < kM; ++m) {
      float v8[8] = {xv[m][0].x, xv[m][0].y, xv[m][0].z, xv[m][0].w,
                     xv[m][1].x, xv[m][1].y, xv[m][1].z, xv[m][1].w};
      if (a.norm_out != nullptr) {
#pragma unroll
        for (int z = 0; z < 8; ++z) v8[z] *= inv[t];
      }
#pragma unroll
      for (int z = 0; z < 8; ++z) sum = fmaf(w[m][z], v8[z], sum);
    }
    acc[t] = wave_sum(sum);
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) part[wave][t] = acc[t];
  }
  __syncthreads();
  if ((int)threadIdx.x < NT) {
    const int t = threadIdx.x;
    a.logits[(int64_t)t * a.E + e] = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
  }
}

// Pieces of 512 inputs a wave for a row of d inputs.
inline int route_pieces(int d) { return d <= 2048 ? 1 : d <= 4096 ? 2 : 4; }

}  // namespace smoe
