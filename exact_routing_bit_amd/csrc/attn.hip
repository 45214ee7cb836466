// attn.hip - the attention block around the routed MoE layer ("Data Flow",
// the layer loop: RMS norm -> Q/K/V projections (bf16 matrix-vector
// products) -> per-head QK-RMSNorm -> RoPE -> K/V append into the layer's KV
// ring -> causal GQA attention -> O projection -> residual; "Surface Scout",
// the model config and "KV-Cache").
//
// Four launches per call of B tokens at positions pos0 .. pos0+B-1:
//  k_gemv_bf16    QKV projection: out[t, r] = sum_c W[r, c] x[t, c] for bf16
//                 W [R, C] and bf16 x, fp32 accumulation (v_dot2_f32_bf16),
//                 x = bf16(RMSNorm(x)) formed by each block into LDS (unit
//                 gain); one 4-wave block per CU, each wave streaming 16-byte
//                 pieces of its rows through a two-item ring of range-checked
//                 buffer loads (constant per-lane offsets), row sums staged
//                 in LDS and written after the loop;
//  k_attn_decode  per (256-position split, key/value head, token): appends
//                 the call's K/V that fall in the split (QK-norm and RoPE of
//                 k, the angle pos * theta^(-2i/hd) in fp64, the rotate-half
//                 pair (i, i + 64) in one lane; bf16 into ring slot pos mod
//                 ctx), forms its query heads the same way, stages the
//                 split's V in LDS and computes the scores, their max and
//                 exponent sum, and the exponent-weighted sum of V;
//  k_attn_merge   per (query head, token): the splits combined in order,
//                 rounded to bf16 (the O projection's input);
//  k_gemv_bf16    O projection plus the residual.
// Chunks of kAttnProjMinBatch tokens or more run each projection as one pass
// over the weights instead: k_rms_bf16 (the normed input as bf16 rows, QKV
// only), k_proj_mfma (bf16 MFMA tiles over 512-input slices) and
// k_proj_reduce (the slices' sums in order, plus the residual).
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
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi): two bf16 products carry
// x to about 2^-16 relative.  Eight values in, both halves packed.
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], uint4& hi, uint4& lo) {
  uint32_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = bf16_rne(x[e]);
    l[e] = bf16_rne(x[e] - __uint_as_float(h[e] << 16));
  }
  hi = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
  lo = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16));
}
__device__ __forceinline__ floatx4 mfma_bf16(const uint4& a, const uint4& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ float segment_max16(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  return fmaxf(v, dpp<kDppMirror>(v));
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

// out[t, r] = (residual[t, r] +) sum_c Wm[r, c] x[t, c], t < NTOK, C = 512 kChunks,
// with x the bf16 rows given, or (xf set) bf16(RMSNorm(xf[t])) formed by every
// block for itself (block_row_inv, unit gain).
template <int NTOK, int kChunks>
__global__ __launch_bounds__(kAttnThreads) void k_gemv_bf16(const uint16_t* Wm, int R,
                                                            const uint16_t* x, const float* xf,
                                                            float eps, const float* residual,
                                                            float* out) {
  constexpr int C = kChunks * 512;
  __shared__ uint4 xs[NTOK][C / 8];
  __shared__ float part[kAttnThreads / 64];
  if (xf != nullptr) {
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
      const float* row = xf + (int64_t)t * C;
      const float inv = block_row_inv(row, C, eps, part);
      const float4* r4 = reinterpret_cast<const float4*>(row);
      uint2* x2 = reinterpret_cast<uint2*>(xs[t]);
      for (int i = threadIdx.x; i < C / 4; i += kAttnThreads) {
        const float4 v = r4[i];
        x2[i] = make_uint2(bf16_rne(v.x * inv) | (bf16_rne(v.y * inv) << 16),
                           bf16_rne(v.z * inv) | (bf16_rne(v.w * inv) << 16));
      }
    }
  } else {
    for (int i = threadIdx.x; i < NTOK * (C / 8); i += kAttnThreads)
      xs[i / (C / 8)][i % (C / 8)] = reinterpret_cast<const uint4*>(x)[i];
  }
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

// RoPE's cos and sin for this lane's pair (lane, lane + 64) at position pos:
// angle pos * theta^(-2 lane / hd), in fp64 (the same for every head).
__device__ __forceinline__ float2 rope_cs(int64_t pos, double theta) {
  const int lane = threadIdx.x & 63;
  const double ang = (double)pos * pow(theta, -2.0 * (double)lane / (double)kHd);
  return make_float2((float)cos(ang), (float)sin(ang));
}
// ------------------------------------------------------ batched projections
// Chunks of kAttnProjMinBatch .. 64 tokens take one pass over the weights for
// all of their tokens, on the MFMA units, with the inputs split into slices of
// kAttnProjK and the slices' partial sums added in a fixed order afterwards.
constexpr int kProjRows = 64;                 // weight rows per block, 16 per wave
constexpr int kProjK = kAttnProjK;            // inputs per block
constexpr int kProjLdsRow = kProjK / 8 + 1;   // uint4 per staged token row (16 B padding)
constexpr int kProjOutRow = kProjRows + 4;    // floats per token row of the result tile

// xb[t] = bf16(RMSNorm(x[t])), unit gain (the arithmetic of k_gemv_bf16's
// fused norm), and rope[t] = RoPE's (cos, sin) of position pos0 + t for each
// pair, formed as the attention kernel forms them; one block per token.
__global__ __launch_bounds__(kAttnThreads) void k_rms_bf16(const float* x, int C, float eps,
                                                           uint16_t* xb, int64_t pos0,
                                                           double theta, float2* rope) {
  __shared__ float part[kAttnThreads / 64];
  if (threadIdx.x < kHd / 2)
    rope[(int64_t)blockIdx.x * (kHd / 2) + threadIdx.x] = rope_cs(pos0 + blockIdx.x, theta);
  const float* row = x + (int64_t)blockIdx.x * C;
  const float inv = block_row_inv(row, C, eps, part);
  const float4* r4 = reinterpret_cast<const float4*>(row);
  uint2* o2 = reinterpret_cast<uint2*>(xb + (int64_t)blockIdx.x * C);
  for (int i = threadIdx.x; i < C / 4; i += kAttnThreads) {
    const float4 v = r4[i];
    o2[i] = make_uint2(bf16_rne(v.x * inv) | (bf16_rne(v.y * inv) << 16),
                       bf16_rne(v.z * inv) | (bf16_rne(v.w * inv) << 16));
  }
}

// Block (row block rb, input slice ks), NT = ceil(B / 16):
//   part[ks, t, r] = sum_{c in slice ks} W[r, c] xb[t, c],  t < B, r in rb's 64 rows.
// The tokens' slice is staged in LDS (token rows past B read zeros).  Wave w
// streams rows 64 rb + 16 w .. + 15: lane (m = lane % 16, q = lane / 16)
// holds inputs 32 s + 8 q .. + 7 of row m for s = 0..15, the A operand of
// v_mfma_f32_16x16x32_bf16 (m = row, n = token, k = input), all 16 loads
// issued at once.  The 64 x 16 NT result goes through LDS, so that each
// token's 64 partial sums leave as one 256-byte run.  R must be a multiple of
// 64 and C of kProjK.
template <int NT>
__global__ __launch_bounds__(kAttnThreads) void k_proj_mfma(const uint16_t* W, int R, int C,
                                                            const uint16_t* xb, int B,
                                                            float* part) {
  static_assert(NT * 16 * kProjOutRow * 4 <= NT * 16 * kProjLdsRow * 16, "result tile fits");
  __shared__ uint4 xs[NT * 16][kProjLdsRow];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = blockIdx.x, ks = blockIdx.y, k0 = ks * kProjK;
  const auto rw = buffer_rsrc(W, (uint32_t)((size_t)R * C * 2));
  const uint32_t wo =
      (uint32_t)(((size_t)(rb * kProjRows + wave * 16 + (lane & 15)) * C + k0 + 8 * (lane >> 4)) * 2);
  uint4 a[kProjK / 32];
#pragma unroll
  for (int s = 0; s < kProjK / 32; ++s) a[s] = buf_load4_nt(rw, wo + 64 * s);
  // the tokens' slice: thread (row i / 64 of each group of 4, piece tid % 64)
  const auto rx = buffer_rsrc(xb, (uint32_t)((size_t)B * C * 2));
#pragma unroll
  for (int i = 0; i < NT * 4; ++i) {
    const int t = 4 * i + (tid >> 6);
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
        rx, (int)(((size_t)t * C + k0 + 8 * lane) * 2), 0, 0);
    xs[t][lane] = make_uint4(v.x, v.y, v.z, v.w);
  }
  __syncthreads();
  floatx4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15, q = lane >> 4;
#pragma unroll
  for (int s = 0; s < kProjK / 32; ++s)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma_bf16(a[s], xs[nt * 16 + n][4 * s + q], acc[nt]);
  __syncthreads();                                 // xs is reused for the result tile
  float(*ot)[kProjOutRow] = reinterpret_cast<float(*)[kProjOutRow]>(&xs[0][0]);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) ot[nt * 16 + n][wave * 16 + 4 * q + i] = acc[nt][i];
  __syncthreads();
  for (int e = tid; e < B * (kProjRows / 4); e += kAttnThreads) {
    const int t = e / (kProjRows / 4), c4 = e % (kProjRows / 4);
    const float4 v = make_float4(ot[t][4 * c4], ot[t][4 * c4 + 1], ot[t][4 * c4 + 2], ot[t][4 * c4 + 3]);
    reinterpret_cast<float4*>(part + ((int64_t)ks * B + t) * R + rb * kProjRows)[c4] = v;
  }
}

// out[t, r] = (residual[t, r] +) (part[0, t, r] + part[1, t, r] + ...), the
// slices in order; one float4 per thread.
__global__ __launch_bounds__(kAttnThreads) void k_proj_reduce(const float* part, int S, int n4,
                                                              const float* residual, float* out) {
  const int i = blockIdx.x * kAttnThreads + threadIdx.x;
  if (i >= n4) return;
  const float4* p4 = reinterpret_cast<const float4*>(part);
  float4 v = p4[i];
  for (int s = 1; s < S; ++s) {
    const float4 w = p4[(int64_t)s * n4 + i];
    v.x += w.x;
    v.y += w.y;
    v.z += w.z;
    v.w += w.w;
  }
  if (residual != nullptr) {
    const float4 r = reinterpret_cast<const float4*>(residual)[i];
    v = make_float4(r.x + v.x, r.y + v.y, r.z + v.z, r.w + v.w);
  }
  reinterpret_cast<float4*>(out)[i] = v;
}


// ------------------------------------------------------------- attention
// QK-norm (unit gain), then the rotation by cs, of one head vector held as
// (x0, x1) = elements (lane, lane + 64): the rotate-half pair of one lane.
__device__ __forceinline__ void qk_norm_rope(float& x0, float& x1, float2 cs, float eps) {
  const float ss = wave_sum(x0 * x0 + x1 * x1);
  const float inv = 1.0f / sqrtf(ss / (float)kHd + eps);
  x0 *= inv;
  x1 *= inv;
  const float r0 = x0 * cs.x - x1 * cs.y, r1 = x1 * cs.x + x0 * cs.y;
  x0 = r0;
  x1 = r1;
}

// The query operands of one MFMA score tile: lane (head col, dims
// 32 st + 8 lg .. + 7) as bf16 high and low parts.
__device__ __forceinline__ void query_operands(const float (*qs)[kHd], int col, int lg,
                                               uint4 (&qh)[kHd / 32], uint4 (&ql)[kHd / 32]) {
#pragma unroll
  for (int st = 0; st < kHd / 32; ++st) {
    const float4 xa = *reinterpret_cast<const float4*>(&qs[col][32 * st + 8 * lg]);
    const float4 xb = *reinterpret_cast<const float4*>(&qs[col][32 * st + 8 * lg + 4]);
    const float x[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
    split_bf16x8(x, qh[st], ql[st]);
  }
}

// Block (split s, key/value head g, tokens t0 .. t1 - 1: a group of a.tgroup
// tokens of the call).  The split's positions are start .. start + 255 with
// start = lo + 256 s (lo: the first position the ring holds after the call);
// token t reads n_t of them, up to its own.
//  1. The call's K/V that fall in the split are formed (k: QK-norm + RoPE;
//     v as is) and appended, by every group's block of the split alike (the
//     same bits), so that each block reads what it wrote after its barrier.
//  2. The first token's G query heads: QK-norm + RoPE, scaled by 1/sqrt(hd),
//     into LDS.
//  3. K and V of the split into LDS, as many positions as the group's last
//     token reads (every load issued first; the query operands are formed
//     meanwhile).
//  4. Per token, scores as 16 x 16 MFMA tiles (query heads x positions); per
//     head the max m, p = exp(score - m) (0 past n_t) and l = sum p.
//  5. o = sum_j p_j v_j per head, as MFMA tiles.  Writes (m, l) and o; a split
//     that the token does not reach writes l = 0.  Then the next token's
//     queries (2) and again from 4, against the same staged K and V.
// kTable: RoPE's (cos, sin) come from a.rope (chunks) rather than being formed
// here (decode).
template <bool kTable>
__global__ __launch_bounds__(kAttnThreads) void k_attn_decode(AttnArgs a) {
  // LDS: p (rows padded: the A-operand reads of 16 rows hit distinct banks),
  // whose first 8 KB first hold the scaled queries; K row-major and V
  // transposed (padded rows), the MFMA operands' 16-byte pieces
  __shared__ float ps[kMaxGroup][kSplit + 4];
  __shared__ uint4 kl[kSplit][kHd / 8 + 1];
  __shared__ uint16_t vt[kHd][kSplit + 8];
  __shared__ float red[kMaxGroup][kAttnThreads / 64];
  __shared__ float redl[kMaxGroup][kAttnThreads / 64];
  float (*qs)[kHd] = reinterpret_cast<float (*)[kHd]>(&ps[0][0]);
  const int s = blockIdx.x, g = blockIdx.y;
  const int t0 = blockIdx.z * a.tgroup, t1 = min(a.B, t0 + a.tgroup);   // the block's tokens
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.H / a.Hkv;
  const int64_t p_last = a.pos0 + a.B - 1;
  const int64_t lo = p_last - a.ctx + 1 > 0 ? p_last - a.ctx + 1 : 0;
  const int64_t start = lo + (int64_t)s * kSplit;
  // 1. the call's K/V in this split
  const int64_t a_lo = start > a.pos0 ? start : a.pos0;
  const int64_t a_hi = start + kSplit - 1 < p_last ? start + kSplit - 1 : p_last;
  for (int64_t p = a_lo + wave; p <= a_hi; p += kAttnThreads / 64) {
    const float* src = a.qkv + (p - a.pos0) * a.qkv_rows;
    const float* ks = src + (int64_t)(a.H + g) * kHd;
    const float* vsrc = src + (int64_t)(a.H + a.Hkv + g) * kHd;
    float k0 = ks[lane], k1 = ks[lane + 64];
    const float v0 = vsrc[lane], v1 = vsrc[lane + 64];
    const float2 cs = kTable ? a.rope[(p - a.pos0) * (kHd / 2) + lane] : rope_cs(p, a.theta);
    qk_norm_rope(k0, k1, cs, a.eps);
    const int64_t row = ((int64_t)g * a.ctx + p % a.ctx) * kHd;
    a.k_cache[row + lane] = (uint16_t)bf16_rne(k0);
    a.k_cache[row + lane + 64] = (uint16_t)bf16_rne(k1);
    a.v_cache[row + lane] = (uint16_t)bf16_rne(v0);
    a.v_cache[row + lane + 64] = (uint16_t)bf16_rne(v1);
  }
  // 2. the first token's queries (rows G .. 15 zero: the loops below run over
  //    all 16 rows without a branch on G, whose LDS reads would each wait)
  const float scale = 1.0f / sqrtf((float)kHd);
  auto form_queries = [&](int t) {
    for (int i = G * kHd + tid; i < kMaxGroup * kHd; i += kAttnThreads) qs[i / kHd][i % kHd] = 0.f;
    const float2 cs = kTable ? a.rope[(int64_t)t * (kHd / 2) + lane]
                             : rope_cs(a.pos0 + t, a.theta);   // once per token
    for (int h = wave; h < G; h += kAttnThreads / 64) {
      const float* qsrc = a.qkv + (int64_t)t * a.qkv_rows + (int64_t)(g * G + h) * kHd;
      float q0 = qsrc[lane], q1 = qsrc[lane + 64];
      qk_norm_rope(q0, q1, cs, a.eps);
      qs[h][lane] = q0 * scale;
      qs[h][lane + 64] = q1 * scale;
    }
  };
  // positions of the split that token t reads (non-decreasing in t)
  auto n_of = [&](int t) {
    const int64_t avail = a.pos0 + t + 1 - start;
    return avail <= 0 ? 0 : (avail >= kSplit ? kSplit : (int)avail);
  };
  auto part_base = [&](int t) { return (((int64_t)t * a.Hkv + g) * a.nsplit + s) * kMaxGroup; };
  const int n_last = n_of(t1 - 1);
  if (n_last == 0) {                               // whole block; its appends are done
    if (tid < kMaxGroup)
      for (int t = t0; t < t1; ++t)
        reinterpret_cast<float2*>(a.part_ml)[part_base(t) + tid] = make_float2(0.f, 0.f);
    return;
  }
  form_queries(t0);
  __syncthreads();                                 // appends and queries visible to the block
  const int64_t slot0 = start % a.ctx;
  const int col = lane & 15, lg = lane >> 4;
  // 3. K (row-major) and V (transposed) of the split into LDS: thread i copies
  //    16-byte piece i % 16 of row i / 16 (i = tid + 256 k), every load issued
  //    first; the query operands (hi, lo) come out of LDS meanwhile: lane
  //    (head col, dims 32 s + 8 lg .. +7)
  constexpr int kPieces = kSplit * (kHd / 8) / kAttnThreads;
  uint4 qh[kHd / 32], ql[kHd / 32];
  {
    // thread tid: chunk c = tid % 16 of rows tid / 16 + 16 k; one 32-bit byte
    // offset per row serves K and V (ring of this head: ctx * 256 bytes)
    const uint32_t ring_bytes = (uint32_t)(a.ctx * kHd * 2);
    const auto krs = buffer_rsrc(a.k_cache + (int64_t)g * a.ctx * kHd, ring_bytes);
    const auto vrs = buffer_rsrc(a.v_cache + (int64_t)g * a.ctx * kHd, ring_bytes);
    uint4 kr[kPieces], vr[kPieces];
#pragma unroll
    for (int k = 0; k < kPieces; ++k) {
      const int j = (tid >> 4) + 16 * k;
      int64_t sl = slot0 + (j < n_last ? j : 0);
      if (sl >= a.ctx) sl -= a.ctx;
      const uint32_t off = (uint32_t)(sl * (kHd * 2) + (tid & 15) * 16);
      kr[k] = buf_load4_nt(krs, off);
      vr[k] = buf_load4_nt(vrs, off);
    }
    query_operands(qs, col, lg, qh, ql);
#pragma unroll
    for (int k = 0; k < kPieces; ++k) {
      const int i = tid + kAttnThreads * k, j = i >> 4, c = i & 15;
      kl[j][c] = kr[k];
      const uint32_t w[4] = {vr[k].x, vr[k].y, vr[k].z, vr[k].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt[8 * c + 2 * e][j] = (uint16_t)(w[e] & 0xFFFFu);
        vt[8 * c + 2 * e + 1][j] = (uint16_t)(w[e] >> 16);
      }
    }
  }
  __syncthreads();                                 // K, V in LDS; the queries are read
  // 4.-6. per token of the group, against the staged K and V
  for (int t = t0;;) {
    const int n = n_of(t);
    // chunks: the next token's query rows are requested now and used after
    // this token (head wave + 4 i of the group, clamped; a fixed count, so
    // that no load sits behind a branch)
    float nq[kMaxGroup / 4][2];
    if constexpr (kTable) {
      const int tn = t + 1 < t1 ? t + 1 : t;
#pragma unroll
      for (int i = 0; i < kMaxGroup / 4; ++i) {
        const int h = min(wave + 4 * i, G - 1);
        const float* qsrc = a.qkv + (int64_t)tn * a.qkv_rows + (int64_t)(g * G + h) * kHd;
        nq[i][0] = qsrc[lane];
        nq[i][1] = qsrc[lane + 64];
      }
    }
    float* po = a.part_o + part_base(t) * kHd;
    float2* pml = reinterpret_cast<float2*>(a.part_ml) + part_base(t);
    if (n == 0) {                                  // uniform over the block
      if (tid < kMaxGroup) pml[tid] = make_float2(0.f, 0.f);
    } else {
      // 4. scores S[head][position] = q . k (q pre-scaled): wave w, positions
      //    64 w + 16 T + col; D[i] = S[4 lg + i][that position]
      floatx4 sc[4];
    #pragma unroll
      for (int T = 0; T < 4; ++T) {
        sc[T] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int j = 64 * wave + 16 * T + col;
    #pragma unroll
        for (int st = 0; st < kHd / 32; ++st) {
          const uint4 b = kl[j][4 * st + lg];
          sc[T] = mfma_bf16(qh[st], b, sc[T]);
          sc[T] = mfma_bf16(ql[st], b, sc[T]);
        }
      }
      // 5. per head: max over the split, p = exp(score - max) (0 past n), sum of p
      float mx[4];
    #pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = -FLT_MAX;
    #pragma unroll
        for (int T = 0; T < 4; ++T) m = fmaxf(m, 64 * wave + 16 * T + col < n ? sc[T][i] : -FLT_MAX);
        mx[i] = segment_max16(m);
        if (col == 0) red[4 * lg + i][wave] = mx[i];
      }
      __syncthreads();
      float mh[4];
    #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * lg + i;
        mh[i] = fmaxf(fmaxf(red[h][0], red[h][1]), fmaxf(red[h][2], red[h][3]));
        float acc = 0.f;
    #pragma unroll
        for (int T = 0; T < 4; ++T) {
          const int j = 64 * wave + 16 * T + col;
          const float p = j < n ? expf(sc[T][i] - mh[i]) : 0.f;
          ps[h][j] = p;
          acc += p;
        }
        acc = segment_sum16(acc, 16);
        if (col == 0) redl[h][wave] = acc;
      }
      __syncthreads();
      // 6. O[head][dim] = sum_j p[head][j] v[j][dim]: wave w, dims 16 dt + col for
      //    dt = 2 w, 2 w + 1; A = p (hi, lo) of (head col, positions 32 s + 8 lg ..)
      floatx4 oc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    #pragma unroll 2
      for (int st = 0; st < kSplit / 32; ++st) {
        const float4 pa = *reinterpret_cast<const float4*>(&ps[col][32 * st + 8 * lg]);
        const float4 pb = *reinterpret_cast<const float4*>(&ps[col][32 * st + 8 * lg + 4]);
        const float pv[8] = {pa.x, pa.y, pa.z, pa.w, pb.x, pb.y, pb.z, pb.w};
        uint4 ph, pl;
        split_bf16x8(pv, ph, pl);
    #pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int dt = 2 * wave + u;
          const uint4 b = *reinterpret_cast<const uint4*>(&vt[16 * dt + col][32 * st + 8 * lg]);
          oc[u] = mfma_bf16(ph, b, oc[u]);
          oc[u] = mfma_bf16(pl, b, oc[u]);
        }
      }
    #pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int d = 16 * (2 * wave + u) + col;
    #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 4 * lg + i;
          if (h < G) po[(int64_t)h * kHd + d] = oc[u][i];
        }
      }
      if (tid < G) {
        const int h = tid;
        const float m = fmaxf(fmaxf(red[h][0], red[h][1]), fmaxf(red[h][2], red[h][3]));
        const float l = ((redl[h][0] + redl[h][1]) + redl[h][2]) + redl[h][3];
        pml[h] = make_float2(m, l);
      }
    }
    if (++t >= t1) break;
    __syncthreads();                               // p, red, redl read; qs may be rewritten
    if constexpr (kTable) {
      for (int i = G * kHd + tid; i < kMaxGroup * kHd; i += kAttnThreads) qs[i / kHd][i % kHd] = 0.f;
      const float2 cs = a.rope[(int64_t)t * (kHd / 2) + lane];
#pragma unroll
      for (int i = 0; i < kMaxGroup / 4; ++i) {
        const int h = wave + 4 * i;
        if (h < G) {
          float q0 = nq[i][0], q1 = nq[i][1];
          qk_norm_rope(q0, q1, cs, a.eps);
          qs[h][lane] = q0 * scale;
          qs[h][lane + 64] = q1 * scale;
        }
      }
    } else {
      form_queries(t);
    }
    __syncthreads();
    query_operands(qs, col, lg, qh, ql);
  }
}

// ----------------------------------------------------------- k_attn_merge
// Block (query head h, token t), thread = dimension: the splits in order.
__global__ __launch_bounds__(kHd) void k_attn_merge(AttnArgs a) {
  const int h = blockIdx.x, t = blockIdx.y, d = threadIdx.x;
  const int G = a.H / a.Hkv, g = h / G, hh = h % G;
  const int64_t base = (((int64_t)t * a.Hkv + g) * a.nsplit) * kMaxGroup + hh;
  const float2* pml = reinterpret_cast<const float2*>(a.part_ml);
  // one pass, the running max rescaling what came before; no branch, so that
  // the loads of a group of splits go out together (an empty split, l = 0,
  // has an unwritten o, which the selects keep out)
  float M = -FLT_MAX, num = 0.f, den = 0.f;
  for (int s0 = 0; s0 < a.nsplit; s0 += 16) {       // groups of 16, indices clamped
#pragma unroll
   for (int u = 0; u < 16; ++u) {
    const int s = s0 + u;
    const int64_t at = base + (int64_t)(s < a.nsplit ? s : a.nsplit - 1) * kMaxGroup;
    const float2 ml = pml[at];
    const float o = a.part_o[at * kHd + d];
    const bool has = s < a.nsplit && ml.y > 0.f;
    const float Mn = has ? fmaxf(M, ml.x) : M;
    const float r = expf(M - Mn), w = has ? expf(ml.x - Mn) : 0.f;
    num = __builtin_fmaf(w, has ? o : 0.f, num * r);
    den = __builtin_fmaf(w, has ? ml.y : 0.f, den * r);
    M = Mn;
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
hipError_t launch_gemv_c(const uint16_t* Wm, int R, const uint16_t* x, const float* xf, float eps,
                         const float* residual, float* out, hipStream_t s, const LaunchTiming* t) {
  const int ncu = cu_count_attn();
  if (ncu <= 0) return hipErrorInvalidDevice;
  const int items = (R + GemvItem<kChunks>::kRows - 1) / GemvItem<kChunks>::kRows;
  // one block per CU, but enough blocks that no wave has more than kGemvMaxItems items
  const int grid = std::max(std::min((items + 3) / 4, ncu),
                            (items + 4 * kGemvMaxItems - 1) / (4 * kGemvMaxItems));
  SMOE_LAUNCH(t, (k_gemv_bf16<NTOK, kChunks>), dim3(grid), dim3(kAttnThreads), 0, s, Wm, R, x,
              xf, eps, residual, out);
  return hipGetLastError();
}

template <int NTOK>
hipError_t launch_gemv_n(const uint16_t* Wm, int R, int C, const uint16_t* x, const float* xf,
                         float eps, const float* residual, float* out, hipStream_t s,
                         const LaunchTiming* t) {
  switch (C / 512) {
    case 1: return launch_gemv_c<NTOK, 1>(Wm, R, x, xf, eps, residual, out, s, t);
    case 2: return launch_gemv_c<NTOK, 2>(Wm, R, x, xf, eps, residual, out, s, t);
    case 4: return launch_gemv_c<NTOK, 4>(Wm, R, x, xf, eps, residual, out, s, t);
    case 8: return launch_gemv_c<NTOK, 8>(Wm, R, x, xf, eps, residual, out, s, t);
    case 16: return launch_gemv_c<NTOK, 16>(Wm, R, x, xf, eps, residual, out, s, t);
    default: return hipErrorInvalidValue;
  }
}

// out = (residual +) W xb for B >= kAttnProjMinBatch tokens of bf16 rows xb:
// the slices' partial sums, then their ordered sum.
hipError_t launch_proj(const uint16_t* Wm, int R, int C, const uint16_t* xb, int B,
                       const float* residual, float* out, float* part, hipStream_t s,
                       const LaunchTiming* t) {
  if (R % kProjRows != 0 || C % kProjK != 0 || B < 1 || B > 64) return hipErrorInvalidValue;
  const dim3 grid(R / kProjRows, C / kProjK);
  switch ((B + 15) / 16) {
    case 1: SMOE_LAUNCH(t, k_proj_mfma<1>, grid, dim3(kAttnThreads), 0, s, Wm, R, C, xb, B, part); break;
    case 2: SMOE_LAUNCH(t, k_proj_mfma<2>, grid, dim3(kAttnThreads), 0, s, Wm, R, C, xb, B, part); break;
    case 3: SMOE_LAUNCH(t, k_proj_mfma<3>, grid, dim3(kAttnThreads), 0, s, Wm, R, C, xb, B, part); break;
    default: SMOE_LAUNCH(t, k_proj_mfma<4>, grid, dim3(kAttnThreads), 0, s, Wm, R, C, xb, B, part); break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n4 = B * R / 4;
  hipLaunchKernelGGL(k_proj_reduce, dim3((n4 + kAttnThreads - 1) / kAttnThreads),
                     dim3(kAttnThreads), 0, s, part, C / kProjK, n4, residual, out);
  return hipGetLastError();
}

// out[t] = (residual[t] +) W x[t] for B tokens, two at a time; x is either
// bf16 rows or (xf) fp32 rows to normalise first.
hipError_t launch_gemv_bf16(const uint16_t* Wm, int R, int C, const uint16_t* x, const float* xf,
                            float eps, int B, const float* residual, float* out, hipStream_t s,
                            const LaunchTiming* t = nullptr) {
  for (int t0 = 0; t0 < B; t0 += 2) {
    const uint16_t* xt = x ? x + (int64_t)t0 * C : nullptr;
    const float* xft = xf ? xf + (int64_t)t0 * C : nullptr;
    const float* rt = residual ? residual + (int64_t)t0 * R : nullptr;
    float* ot = out + (int64_t)t0 * R;
    const hipError_t err = B - t0 >= 2 ? launch_gemv_n<2>(Wm, R, C, xt, xft, eps, rt, ot, s, t)
                                       : launch_gemv_n<1>(Wm, R, C, xt, xft, eps, rt, ot, s, t);
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
  const bool batched = a.B >= kAttnProjMinBatch;
  if (batched && (a.xb == nullptr || a.ppart == nullptr || a.rope == nullptr))
    return hipErrorInvalidValue;
  if (stage < 0 || stage == 0) {
    if (batched) {
      hipLaunchKernelGGL(k_rms_bf16, dim3(a.B), dim3(kAttnThreads), 0, s, a.x, a.d, a.eps, a.xb,
                         a.pos0, a.theta, a.rope);
      err = hipGetLastError();
      if (err == hipSuccess)
        err = launch_proj(a.wqkv, rows, a.d, a.xb, a.B, nullptr, a.qkv, a.ppart, s,
                          stage == 0 ? t : nullptr);
    } else {
      err = launch_gemv_bf16(a.wqkv, rows, a.d, nullptr, a.x, a.eps, a.B, nullptr, a.qkv, s,
                             stage == 0 ? t : nullptr);
    }
    if (err != hipSuccess) return err;
  }
  if (stage < 0 || stage == 1) {
    // token groups: about one block per CU (each block stages its split's
    // K and V once, which costs more than the CUs' idle tails of larger
    // groups); one token a block for decode
    const int ncu = cu_count_attn();
    if (ncu <= 0) return hipErrorInvalidDevice;
    const int heads_splits = a.nsplit * a.Hkv;
    const int ngroups = std::max(1, std::min(a.B, (ncu + heads_splits - 1) / heads_splits));
    AttnArgs b = a;
    b.tgroup = (a.B + ngroups - 1) / ngroups;
    const dim3 grid(a.nsplit, a.Hkv, (a.B + b.tgroup - 1) / b.tgroup);
    if (batched)
      SMOE_LAUNCH(stage == 1 ? t : nullptr, k_attn_decode<true>, grid, dim3(kAttnThreads), 0, s, b);
    else
      SMOE_LAUNCH(stage == 1 ? t : nullptr, k_attn_decode<false>, grid, dim3(kAttnThreads), 0, s, b);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_attn_merge, dim3(a.H, a.B), dim3(kHd), 0, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (stage < 0 || stage == 2)
    err = batched ? launch_proj(a.wo, a.d, a.H * kHd, a.ob, a.B, a.x, a.out, a.ppart, s,
                                stage == 2 ? t : nullptr)
                  : launch_gemv_bf16(a.wo, a.d, a.H * kHd, a.ob, nullptr, 0.f, a.B, a.x, a.out,
                                     s, stage == 2 ? t : nullptr);
  return err;
}

}  // namespace smoe
