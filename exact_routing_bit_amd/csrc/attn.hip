// attn.hip - the attention block around the routed MoE layer ("Data Flow",
// the layer loop: RMS norm -> Q/K/V projections (bf16 matrix-vector
// products) -> per-head QK-RMSNorm -> RoPE -> K/V append into the layer's KV
// ring -> causal GQA attention -> O projection -> residual; "Surface Scout",
// the model config and "KV-Cache").
//
// Five kernels per call of B tokens at positions pos0 .. pos0+B-1:
//  k_attn_in      RMS norm of each token (block_row_inv, unit gain), rounded
//                 to bf16: the projection's input;
//  k_gemv_bf16    out[t, r] (+)= sum_c W[r, c] x[t, c] for bf16 W [R, C] and
//                 bf16 x, fp32 accumulation (v_dot2_f32_bf16): the QKV
//                 projection, and later the O projection with the residual;
//                 one 4-wave block per CU, each wave streaming 16-byte pieces
//                 of its rows through a two-item ring of raw buffer loads
//                 (constant per-lane offsets, the rows' place in scalar
//                 registers), x of the tokens in LDS;
//  k_attn_prep    per (token, head vector): QK-norm and RoPE of q and k (the
//                 angle pos * theta^(-2i/hd) in fp64, the rotate-half pairs
//                 (i, i + 64) in one lane), q kept in fp32, k and v rounded
//                 to bf16 into ring slot pos mod ctx;
//  k_attn_decode  per (256-position split, key/value head, token): the split's
//                 scores for the head's 16 query heads, their max and
//                 exponent sum, and the exponent-weighted sum of V;
//  k_attn_merge   per (query head, token): the splits combined in order,
//                 rounded to bf16 (the O projection's input).
#include <algorithm>

#include "device.hpp"
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kHd = kAttnHeadDim;       // head dimension (128)
constexpr int kAttnThreads = 256;
constexpr int kMaxGroup = kAttnMaxGroup;  // query heads per key/value head
constexpr int kSplit = kAttnSplit;        // cached positions per k_attn_decode block

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ------------------------------------------------------------- k_attn_in
__global__ __launch_bounds__(kAttnThreads) void k_attn_in(const float* x, int d, float eps,
                                                          uint16_t* xb) {
  __shared__ float part[kAttnThreads / 64];
  const int t = blockIdx.x;
  const float* row = x + (int64_t)t * d;
  const float inv = block_row_inv(row, d, eps, part);
  const float4* r4 = reinterpret_cast<const float4*>(row);
  uint2* o2 = reinterpret_cast<uint2*>(xb + (int64_t)t * d);
  for (int i = threadIdx.x; i < d / 4; i += kAttnThreads) {
    const float4 v = r4[i];
    o2[i] = make_uint2(bf16_rne(v.x * inv) | (bf16_rne(v.y * inv) << 16),
                       bf16_rne(v.z * inv) | (bf16_rne(v.w * inv) << 16));
  }
}

// ----------------------------------------------------------- k_gemv_bf16
// Lane l reads the 8 values at columns 512 m + 8 l (m < C/512) of each row.
// An item is 16 such pieces a lane: 16 / (C/512) rows.
template <int kChunks>
struct GemvItem {
  static constexpr int kRows = 16 / kChunks;
  uint4 w[kRows][kChunks];
};

// Per-lane byte offsets of an item's 16 pieces, the same for every item (the
// whole offset is in the vector operand, which the resource's range check
// covers: the pieces of rows past R read zeros and touch no memory).
template <int kChunks>
struct GemvLane {
  uint32_t off[GemvItem<kChunks>::kRows][kChunks];
};
template <int kChunks>
__device__ __forceinline__ GemvLane<kChunks> gemv_lane(int lane) {
  constexpr int C = kChunks * 512;
  GemvLane<kChunks> o;
#pragma unroll
  for (int j = 0; j < GemvItem<kChunks>::kRows; ++j)
#pragma unroll
    for (int m = 0; m < kChunks; ++m) o.off[j][m] = (uint32_t)((j * C + m * 512 + lane * 8) * 2);
  return o;
}

template <int kChunks>
__device__ __forceinline__ void gemv_load(const uint16_t* W, int R, int item, int n_items,
                                          const GemvLane<kChunks>& lo, GemvItem<kChunks>& it) {
  constexpr int C = kChunks * 512, kRows = GemvItem<kChunks>::kRows;
  const bool live = item < n_items;
  const int r0 = (live ? item : 0) * kRows;
  const int rows = live ? min(kRows, R - r0) : 0;
  const auto rs = buffer_rsrc(W + (int64_t)r0 * C, (uint32_t)(rows * C * 2));
#pragma unroll
  for (int j = 0; j < kRows; ++j)
#pragma unroll
    for (int m = 0; m < kChunks; ++m) it.w[j][m] = buf_load4_nt(rs, lo.off[j][m]);
  __builtin_amdgcn_sched_barrier(0);
}

// The item's row sums go to the wave's LDS rows (st[j * NTOK + t]); a global
// store inside the loop would count in vmcnt behind the ring's loads.
template <int NTOK, int kChunks>
__device__ __forceinline__ void gemv_compute(const uint4 (*xs)[kChunks * 64], int lane,
                                             const GemvItem<kChunks>& it, float* st) {
  constexpr int kRows = GemvItem<kChunks>::kRows;
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    uint4 xv[kChunks];
#pragma unroll
    for (int m = 0; m < kChunks; ++m) xv[m] = xs[t][m * 64 + lane];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < kChunks; ++m) {
        acc = dot2_bf16(it.w[j][m].x, xv[m].x, acc);
        acc = dot2_bf16(it.w[j][m].y, xv[m].y, acc);
        acc = dot2_bf16(it.w[j][m].z, xv[m].z, acc);
        acc = dot2_bf16(it.w[j][m].w, xv[m].w, acc);
      }
      const float tot = wave_sum(acc);
      if (lane == 0) st[j * NTOK + t] = tot;
    }
  }
}

constexpr int kGemvMaxItems = 16;     // items per wave (their sums staged in LDS)

// out[t, r] = (residual[t, r] +) sum_c Wm[r, c] x[t, c], t < NTOK, C = 512 kChunks.
template <int NTOK, int kChunks>
__global__ __launch_bounds__(kAttnThreads) void k_gemv_bf16(const uint16_t* Wm, int R,
                                                            const uint16_t* x,
                                                            const float* residual, float* out) {
  constexpr int C = kChunks * 512;
  __shared__ uint4 xs[NTOK][C / 8];
  for (int i = threadIdx.x; i < NTOK * (C / 8); i += kAttnThreads)
    xs[i / (C / 8)][i % (C / 8)] = reinterpret_cast<const uint4*>(x)[i];
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n_items = (R + GemvItem<kChunks>::kRows - 1) / GemvItem<kChunks>::kRows;
  const int NW = gridDim.x * (kAttnThreads / 64);
  const int wid = blockIdx.x * (kAttnThreads / 64) + wave;
  if (wid >= n_items) return;                     // no barrier follows
  constexpr int kRows = GemvItem<kChunks>::kRows;
  __shared__ float st[kAttnThreads / 64][kGemvMaxItems * kRows * NTOK];
  // two items in flight: the next one's loads go out before this one is
  // computed; the grid gives every wave at most kGemvMaxItems items
  const GemvLane<kChunks> lo = gemv_lane<kChunks>(lane);
  GemvItem<kChunks> b0, b1;
  gemv_load<kChunks>(Wm, R, wid, n_items, lo, b0);
  for (int i = wid, loc = 0;; i += 2 * NW, loc += 2) {
    gemv_load<kChunks>(Wm, R, i + NW, n_items, lo, b1);
    gemv_compute<NTOK, kChunks>(xs, lane, b0, &st[wave][loc * kRows * NTOK]);
    if (i + NW >= n_items) break;
    gemv_load<kChunks>(Wm, R, i + 2 * NW, n_items, lo, b0);
    gemv_compute<NTOK, kChunks>(xs, lane, b1, &st[wave][(loc + 1) * kRows * NTOK]);
    if (i + 2 * NW >= n_items) break;
  }
  // the wave's rows out (its own LDS rows: the wave's LDS accesses are ordered)
  const int n_mine = (n_items - wid + NW - 1) / NW;
  for (int q = lane; q < n_mine * kRows * NTOK; q += 64) {
    const int loc = q / (kRows * NTOK), j = (q / NTOK) % kRows, t = q % NTOK;
    const int r = (wid + loc * NW) * kRows + j;
    if (r < R) {
      const int64_t o = (int64_t)t * R + r;
      out[o] = residual ? residual[o] + st[wave][q] : st[wave][q];
    }
  }
}

// ------------------------------------------------------------ k_attn_prep
// One wave per (head vector, token): vectors 0 .. H-1 are q, then Hkv k, then
// Hkv v.  Lane l holds elements l and l + 64, the pair RoPE rotates together.
__global__ __launch_bounds__(kAttnThreads) void k_attn_prep(AttnArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int H = a.H, G = a.Hkv;
  const int vec = blockIdx.x * (kAttnThreads / 64) + wave;
  if (vec >= H + 2 * G) return;
  const int t = blockIdx.y;
  const int64_t pos = a.pos0 + t;
  const float* src = a.qkv + (int64_t)t * a.qkv_rows + (int64_t)vec * kHd;
  float x0 = src[lane], x1 = src[lane + 64];
  const bool is_v = vec >= H + G;
  if (!is_v) {
    // QK-norm (unit gain), then RoPE at the token's absolute position
    const float ss = wave_sum(x0 * x0 + x1 * x1);
    const float inv = 1.0f / sqrtf(ss / (float)kHd + a.eps);
    x0 *= inv;
    x1 *= inv;
    const double ang = (double)pos * pow(a.theta, -2.0 * (double)lane / (double)kHd);
    const float c = (float)cos(ang), s = (float)sin(ang);
    const float r0 = x0 * c - x1 * s, r1 = x1 * c + x0 * s;
    x0 = r0;
    x1 = r1;
  }
  if (vec < H) {
    float* q = a.q + ((int64_t)t * H + vec) * kHd;
    q[lane] = x0;
    q[lane + 64] = x1;
  } else {
    const bool is_k = !is_v;
    const int g = is_k ? vec - H : vec - H - G;
    uint16_t* cache = is_k ? a.k_cache : a.v_cache;
    const int64_t slot = pos % a.ctx;
    uint16_t* dst = cache + ((int64_t)g * a.ctx + slot) * kHd;
    dst[lane] = (uint16_t)bf16_rne(x0);
    dst[lane + 64] = (uint16_t)bf16_rne(x1);
  }
}

// ---------------------------------------------------------- k_attn_decode
// Block (split s, key/value head g, token t): the split's positions are
// start .. start + n - 1 with start = lo + 256 s (lo: the first position the
// ring holds) and n clipped to the token's own position.  Writes, per query
// head of the group, m = the max score, l = sum exp(score - m) and
// o = sum exp(score - m) v (unnormalised); an empty split writes l = 0.
__global__ __launch_bounds__(kAttnThreads) void k_attn_decode(AttnArgs a) {
  __shared__ float qs[kMaxGroup][kHd];
  __shared__ float ps[kMaxGroup][kSplit];
  __shared__ float red[kMaxGroup][kAttnThreads / 64];
  const int s = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.H / a.Hkv;                       // query heads of this group
  const int64_t pos = a.pos0 + t;
  const int64_t p_last = a.pos0 + a.B - 1;
  const int64_t lo = p_last - a.ctx + 1 > 0 ? p_last - a.ctx + 1 : 0;
  const int64_t start = lo + (int64_t)s * kSplit;
  const int64_t avail = pos + 1 - start;
  const int n = avail <= 0 ? 0 : (avail >= kSplit ? kSplit : (int)avail);
  const int64_t base = (((int64_t)t * a.Hkv + g) * a.nsplit + s) * kMaxGroup;
  float* po = a.part_o + base * kHd;
  float2* pml = reinterpret_cast<float2*>(a.part_ml) + base;
  if (n == 0) {                                    // whole block
    if (tid < kMaxGroup) pml[tid] = make_float2(0.f, 0.f);
    return;
  }
  // the group's queries, scaled by 1/sqrt(hd)
  const float scale = 1.0f / sqrtf((float)kHd);
  for (int i = tid; i < G * kHd; i += kAttnThreads)
    qs[i / kHd][i % kHd] = a.q[((int64_t)t * a.H + (int64_t)g * G + i / kHd) * kHd + i % kHd] * scale;
  __syncthreads();
  const int64_t slot0 = start % a.ctx;
  // scores: thread j takes position start + j
  const bool live = tid < n;
  int64_t slot = slot0 + (live ? tid : 0);
  if (slot >= a.ctx) slot -= a.ctx;
  const uint4* krow = reinterpret_cast<const uint4*>(a.k_cache + ((int64_t)g * a.ctx + slot) * kHd);
  float sc[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) sc[h] = 0.f;
#pragma unroll 4
  for (int c = 0; c < kHd / 8; ++c) {
    const uint4 kv = krow[c];
    const float kf[8] = {bf16_lo(kv.x), bf16_hi(kv.x), bf16_lo(kv.y), bf16_hi(kv.y),
                         bf16_lo(kv.z), bf16_hi(kv.z), bf16_lo(kv.w), bf16_hi(kv.w)};
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < G) {
        const float4 qa = *reinterpret_cast<const float4*>(&qs[h][c * 8]);
        const float4 qb = *reinterpret_cast<const float4*>(&qs[h][c * 8 + 4]);
        float acc = sc[h];
        acc = __builtin_fmaf(qa.x, kf[0], acc);
        acc = __builtin_fmaf(qa.y, kf[1], acc);
        acc = __builtin_fmaf(qa.z, kf[2], acc);
        acc = __builtin_fmaf(qa.w, kf[3], acc);
        acc = __builtin_fmaf(qb.x, kf[4], acc);
        acc = __builtin_fmaf(qb.y, kf[5], acc);
        acc = __builtin_fmaf(qb.z, kf[6], acc);
        acc = __builtin_fmaf(qb.w, kf[7], acc);
        sc[h] = acc;
      }
    }
  }
  // per head: the split's max, the exponents and their sum
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h < G) {
      const float m = wave_max(live ? sc[h] : -FLT_MAX);
      if (lane == 0) red[h][wave] = m;
    }
  }
  __syncthreads();
  float mh[kMaxGroup];
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h)
    mh[h] = h < G ? fmaxf(fmaxf(red[h][0], red[h][1]), fmaxf(red[h][2], red[h][3])) : 0.f;
  __syncthreads();                                 // red is reused below
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h < G) {
      const float p = live ? expf(sc[h] - mh[h]) : 0.f;
      ps[h][tid] = p;
      const float ws = wave_sum(p);
      if (lane == 0) red[h][wave] = ws;
    }
  }
  __syncthreads();
  // o[h][d] = sum_j p[h][j] v[j][d]: thread (dims 2 d2, 2 d2 + 1; heads wave, wave + 4, ...)
  const int d2 = lane;
  float o0[kMaxGroup / 4], o1[kMaxGroup / 4];
#pragma unroll
  for (int k = 0; k < kMaxGroup / 4; ++k) o0[k] = o1[k] = 0.f;
  const uint32_t* vbase = reinterpret_cast<const uint32_t*>(a.v_cache + (int64_t)g * a.ctx * kHd);
  int64_t vs = slot0;
  for (int j = 0; j < n; ++j) {
    const uint32_t vv = vbase[vs * (kHd / 2) + d2];
    const float v0 = bf16_lo(vv), v1 = bf16_hi(vv);
#pragma unroll
    for (int k = 0; k < kMaxGroup / 4; ++k) {
      const int h = wave + 4 * k;
      if (h < G) {
        const float p = ps[h][j];
        o0[k] = __builtin_fmaf(p, v0, o0[k]);
        o1[k] = __builtin_fmaf(p, v1, o1[k]);
      }
    }
    vs = vs + 1 == a.ctx ? 0 : vs + 1;
  }
#pragma unroll
  for (int k = 0; k < kMaxGroup / 4; ++k) {
    const int h = wave + 4 * k;
    if (h < G) {
      float* oh = po + (int64_t)h * kHd;
      oh[2 * d2] = o0[k];
      oh[2 * d2 + 1] = o1[k];
    }
  }
  if (tid < G) {
    const int h = tid;
    const float l = ((red[h][0] + red[h][1]) + red[h][2]) + red[h][3];
    pml[h] = make_float2(mh[h], l);
  }
}

// ----------------------------------------------------------- k_attn_merge
// Block (query head h, token t), thread = dimension: the splits in order.
__global__ __launch_bounds__(kHd) void k_attn_merge(AttnArgs a) {
  const int h = blockIdx.x, t = blockIdx.y, d = threadIdx.x;
  const int G = a.H / a.Hkv, g = h / G, hh = h % G;
  const int64_t base = (((int64_t)t * a.Hkv + g) * a.nsplit) * kMaxGroup + hh;
  const float2* pml = reinterpret_cast<const float2*>(a.part_ml);
  float M = -FLT_MAX;
  for (int s = 0; s < a.nsplit; ++s) {
    const float2 ml = pml[base + (int64_t)s * kMaxGroup];
    if (ml.y > 0.f) M = fmaxf(M, ml.x);
  }
  float num = 0.f, den = 0.f;
  for (int s = 0; s < a.nsplit; ++s) {
    const int64_t at = base + (int64_t)s * kMaxGroup;
    const float2 ml = pml[at];
    if (ml.y > 0.f) {
      const float w = expf(ml.x - M);
      num = __builtin_fmaf(w, a.part_o[at * kHd + d], num);
      den = __builtin_fmaf(w, ml.y, den);
    }
  }
  a.ob[(int64_t)t * a.H * kHd + (int64_t)h * kHd + d] = (uint16_t)bf16_rne(num / den);
}

int cu_count_attn() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

template <int NTOK, int kChunks>
hipError_t launch_gemv_c(const uint16_t* Wm, int R, const uint16_t* x, const float* residual,
                         float* out, hipStream_t s, const LaunchTiming* t) {
  const int ncu = cu_count_attn();
  if (ncu <= 0) return hipErrorInvalidDevice;
  const int items = (R + GemvItem<kChunks>::kRows - 1) / GemvItem<kChunks>::kRows;
  // one block per CU, but enough blocks that no wave has more than kGemvMaxItems items
  const int grid = std::max(std::min((items + 3) / 4, ncu),
                            (items + 4 * kGemvMaxItems - 1) / (4 * kGemvMaxItems));
  SMOE_LAUNCH(t, (k_gemv_bf16<NTOK, kChunks>), dim3(grid), dim3(kAttnThreads), 0, s, Wm, R, x,
              residual, out);
  return hipGetLastError();
}

template <int NTOK>
hipError_t launch_gemv_n(const uint16_t* Wm, int R, int C, const uint16_t* x,
                         const float* residual, float* out, hipStream_t s, const LaunchTiming* t) {
  switch (C / 512) {
    case 1: return launch_gemv_c<NTOK, 1>(Wm, R, x, residual, out, s, t);
    case 2: return launch_gemv_c<NTOK, 2>(Wm, R, x, residual, out, s, t);
    case 4: return launch_gemv_c<NTOK, 4>(Wm, R, x, residual, out, s, t);
    case 8: return launch_gemv_c<NTOK, 8>(Wm, R, x, residual, out, s, t);
    case 16: return launch_gemv_c<NTOK, 16>(Wm, R, x, residual, out, s, t);
    default: return hipErrorInvalidValue;
  }
}

// out[t] = (residual[t] +) W x[t] for B tokens, two at a time.
hipError_t launch_gemv_bf16(const uint16_t* Wm, int R, int C, const uint16_t* x, int B,
                            const float* residual, float* out, hipStream_t s,
                            const LaunchTiming* t = nullptr) {
  for (int t0 = 0; t0 < B; t0 += 2) {
    const uint16_t* xt = x + (int64_t)t0 * C;
    const float* rt = residual ? residual + (int64_t)t0 * R : nullptr;
    float* ot = out + (int64_t)t0 * R;
    const hipError_t err = B - t0 >= 2 ? launch_gemv_n<2>(Wm, R, C, xt, rt, ot, s, t)
                                       : launch_gemv_n<1>(Wm, R, C, xt, rt, ot, s, t);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace

bool attn_shape_ok(int d, int H, int Hkv, int hd) {
  if (hd != kHd || H < 1 || Hkv < 1 || H % Hkv != 0 || H / Hkv > kMaxGroup) return false;
  const int q_dim = H * kHd;
  const int c_ok = (d % 512 == 0 && d >= 512 && d <= 8192) && (q_dim % 512 == 0 && q_dim <= 8192);
  return c_ok && (16 % (d / 512) == 0) && (16 % (q_dim / 512) == 0);
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t s, int stage, const LaunchTiming* t) {
  hipError_t err = hipSuccess;
  const int rows = a.qkv_rows;
  if (stage < 0 || stage == 0) {
    hipLaunchKernelGGL(k_attn_in, dim3(a.B), dim3(kAttnThreads), 0, s, a.x, a.d, a.eps, a.xb);
    err = hipGetLastError();
    if (err == hipSuccess)
      err = launch_gemv_bf16(a.wqkv, rows, a.d, a.xb, a.B, nullptr, a.qkv, s, stage == 0 ? t : nullptr);
    if (err != hipSuccess) return err;
  }
  if (stage < 0 || stage == 1) {
    const dim3 gp((a.H + 2 * a.Hkv + 3) / 4, a.B);
    hipLaunchKernelGGL(k_attn_prep, gp, dim3(kAttnThreads), 0, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    SMOE_LAUNCH(stage == 1 ? t : nullptr, k_attn_decode, dim3(a.nsplit, a.Hkv, a.B),
                dim3(kAttnThreads), 0, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_attn_merge, dim3(a.H, a.B), dim3(kHd), 0, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (stage < 0 || stage == 2)
    err = launch_gemv_bf16(a.wo, a.d, a.H * kHd, a.ob, a.B, a.x, a.out, s, stage == 2 ? t : nullptr);
  return err;
}

}  // namespace smoe
