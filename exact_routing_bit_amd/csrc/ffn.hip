// ffn.hip - the token-batch fused expert FFN over 4-bit affine weights.
//
// "Layer-Major Batched Prefill", step 6: each union expert is applied to
// every pair routed to it in one two-pass dispatch (gate_up, then down),
// one dequantisation stream of its weights shared by all of its pairs.
// "SSD Streaming Expert Layers", "Math Contract": h = silu(gate x) * up x,
// y = down h.  "Data Flow": out = residual + sum_k w_k y_k.
//
// Grid of both passes: (row tiles, min(E, B*K)) blocks; block y = u serves
// union expert u and exits when u >= n_union (read on the device), so no
// host synchronisation is needed.  Each block owns four 16-row weight tiles:
//   gate_up: gate rows c0..c0+31 and up rows c0..c0+31 -> h[:, c0..c0+31]
//   down:    rows r0..r0+63                            -> y[:, r0..r0+63]
// Per expert the block takes one of two paths, uniformly:
//   VALU (n_e <= kValuMaxPairs): threads own (row, group) items, five
//     integer ops turn a word into four fp16 pairs and v_dot2_f32_f16
//     accumulates against the prepped activations;
//   MFMA (n_e > kValuMaxPairs): the same dequantised words are the B operand
//     of v_mfma_f32_16x16x32_f16 (16 weight rows), the pairs' activations the
//     A operand (16 pairs per token tile); the 4 waves split K.
// Both apply the group scale and bias in fp32 per 64-input group:
//   sum_i (s q_i + b) x_i = s * (D - C) + b * X,  D = sum (1024 + m q) stored.
// No float atomics anywhere: every output element has one writer.
#include "device.hpp"
#include "smoe_internal.hpp"

namespace smoe {
namespace {

// Threads per weight row in the VALU path: the largest power of two that
// divides the group count, capped at 64 (so each lane's groups are fixed).
__device__ __forceinline__ int threads_per_row(int G) {
  int t = 1;
  while (t < 64 && (G % (2 * t)) == 0) t *= 2;
  return t;
}

template <bool kGateUp>
struct Tile {
  // Weight matrix and first row of 16-row tile T (0..3) of block (x) for expert e.
  __device__ static void locate(const FfnArgs& a, int e, int T, const uint32_t** w,
                                const uint16_t** s, const uint16_t** b, int* row0) {
    const QMat& m = kGateUp ? (T < 2 ? a.gate : a.up) : a.down;
    *w = m.w + e * m.stride_w;
    *s = m.s + e * m.stride_sb;
    *b = m.b + e * m.stride_sb;
    *row0 = kGateUp ? (int)blockIdx.x * kGateUpCols + (T & 1) * 16
                    : (int)blockIdx.x * kDownRows + T * 16;
  }
};

// Prepped activation row (as 16-byte chunks) and group sums of a pair.
template <bool kGateUp>
__device__ __forceinline__ const uint4* act_row(const FfnArgs& a, int pair) {
  return kGateUp ? reinterpret_cast<const uint4*>(a.xp + (int64_t)(pair / a.K) * a.d)
                 : reinterpret_cast<const uint4*>(a.hp + (int64_t)pair * a.f);
}
template <bool kGateUp>
__device__ __forceinline__ float2 act_sums(const FfnArgs& a, int pair, int g) {
  if (kGateUp) return a.xs[(int64_t)(pair / a.K) * (a.d / 64) + g];
  const float2* hs = a.hs + ((int64_t)pair * (a.f / 64) + g) * 2;
  const float2 lo = hs[0], hi = hs[1];
  return make_float2(lo.x + hi.x, lo.y + hi.y);
}

// Epilogue of gate_up: h = silu(g) * u for the block's 32 columns of pair
// `pair`, stored prepped, plus this half-group's sums.  gv/uv: 32 values.
__device__ void store_h(const FfnArgs& a, int pair, const float* gv, const float* uv) {
  const int c0 = blockIdx.x * kGateUpCols;
  uint4* dst = reinterpret_cast<uint4*>(a.hp + (int64_t)pair * a.f + c0);
  float X = 0.f, S = 0.f;
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = silu_mul(gv[ch * 8 + i], uv[ch * 8 + i]);
    dst[ch] = prep_chunk(v, &X, &S);
  }
  a.hs[((int64_t)pair * (a.f / 64) + c0 / 64) * 2 + (c0 % 64) / 32] = make_float2(X, 1024.0f * S);
}

// ---------------------------------------------------------------- VALU path
template <bool kGateUp>
__device__ void ffn_valu(const FfnArgs& a, int e, int pb, int ne, char* smem) {
  const int K = kGateUp ? a.d : a.f;
  const int G = K / 64;
  const int C = K / 8;                                   // 16-byte chunks per row
  uint4* lx = reinterpret_cast<uint4*>(smem);            // [ne][C]
  float2* ls = reinterpret_cast<float2*>(lx + ne * C);   // [ne][G]
  float* lo = reinterpret_cast<float*>(ls + ne * G);     // [64][ne]
  for (int i = threadIdx.x; i < ne * C; i += kFfnThreads) {
    const int j = i / C;
    lx[i] = act_row<kGateUp>(a, a.pair_list[pb + j])[i - j * C];
  }
  for (int i = threadIdx.x; i < ne * G; i += kFfnThreads) {
    const int j = i / G;
    ls[i] = act_sums<kGateUp>(a, a.pair_list[pb + j], i - j * G);
  }
  __syncthreads();
  const int tpr = threads_per_row(G);
  const int rpp = kFfnThreads / tpr;
  const int li = threadIdx.x % tpr, slot = threadIdx.x / tpr;
  for (int rr = slot; rr < 64; rr += rpp) {
    const uint32_t* w;
    const uint16_t *s, *b;
    int row0;
    Tile<kGateUp>::locate(a, e, rr / 16, &w, &s, &b, &row0);
    const int row = row0 + (rr & 15);
    const uint32_t* wrow = w + (int64_t)row * C;
    float part[kValuMaxPairs];
#pragma unroll
    for (int j = 0; j < kValuMaxPairs; ++j) part[j] = 0.f;
    for (int g = li; g < G; g += tpr) {
      const uint4 w0 = ld_stream4(wrow + 8 * g);
      const uint4 w1 = ld_stream4(wrow + 8 * g + 4);
      const float sc = bf16_to_f32(s[(int64_t)row * G + g]);
      const float bi = bf16_to_f32(b[(int64_t)row * G + g]);
#pragma unroll
      for (int j = 0; j < kValuMaxPairs; ++j) {
        if (j < ne) {
          const uint4* xc = lx + j * C + 8 * g;
          float acc = 0.f;
          acc = dot_word(w0.x, xc[0], acc);
          acc = dot_word(w0.y, xc[1], acc);
          acc = dot_word(w0.z, xc[2], acc);
          acc = dot_word(w0.w, xc[3], acc);
          acc = dot_word(w1.x, xc[4], acc);
          acc = dot_word(w1.y, xc[5], acc);
          acc = dot_word(w1.z, xc[6], acc);
          acc = dot_word(w1.w, xc[7], acc);
          const float2 xsum = ls[j * G + g];
          part[j] += sc * (acc - xsum.y) + bi * xsum.x;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kValuMaxPairs; ++j) {
      if (j < ne) {
        const float tot = segment_sum(part[j], tpr);
        if (li == 0) lo[rr * ne + j] = tot;
      }
    }
  }
  __syncthreads();
  if (kGateUp) {
    if (threadIdx.x < ne) {
      const int j = threadIdx.x;
      float gv[32], uv[32];
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        gv[c] = lo[c * ne + j];
        uv[c] = lo[(32 + c) * ne + j];
      }
      store_h(a, a.pair_list[pb + j], gv, uv);
    }
  } else {
    const int r0 = blockIdx.x * kDownRows;
    for (int i = threadIdx.x; i < 64 * ne; i += kFfnThreads) {
      const int j = i / 64, rr = i % 64;
      a.y[(int64_t)a.pair_list[pb + j] * a.d + r0 + rr] = lo[rr * ne + j];
    }
  }
}

// ---------------------------------------------------------------- MFMA path
template <bool kGateUp>
__device__ void ffn_mfma(const FfnArgs& a, int e, int pb, int ne, char* smem) {
  const int K = kGateUp ? a.d : a.f;
  const int G = K / 64;
  const int C = K / 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, lg = lane >> 4;
  float2* ls = reinterpret_cast<float2*>(smem);                      // [16][G]
  float* red = reinterpret_cast<float*>(ls + 16 * G);                // [4 w][4 T][64][4]
  const int g0 = (G * wave) / 4, g1 = (G * (wave + 1)) / 4;

  const uint32_t* tw[4];
  const uint16_t *ts[4], *tb[4];
  int trow[4];
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    Tile<kGateUp>::locate(a, e, T, &tw[T], &ts[T], &tb[T], &trow[T]);
    trow[T] += col;
  }

  for (int tt = 0; tt * 16 < ne; ++tt) {
    const int nt = min(16, ne - tt * 16);
    for (int i = threadIdx.x; i < 16 * G; i += kFfnThreads) {
      const int m = i / G, g = i - m * G;
      ls[i] = m < nt ? act_sums<kGateUp>(a, a.pair_list[pb + tt * 16 + m], g) : make_float2(0.f, 0.f);
    }
    __syncthreads();
    const bool valid = col < nt;
    const uint4* arow = valid ? act_row<kGateUp>(a, a.pair_list[pb + tt * 16 + col]) : nullptr;
    floatx4 acc[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) acc[T] = floatx4{0.f, 0.f, 0.f, 0.f};
    for (int g = g0; g < g1; ++g) {
      uint4 a0 = make_uint4(0, 0, 0, 0), a1 = a0;
      if (valid) {
        a0 = arow[8 * g + 2 * lg];
        a1 = arow[8 * g + 2 * lg + 1];
      }
      const half8_t A0 = __builtin_bit_cast(half8_t, a0);
      const half8_t A1 = __builtin_bit_cast(half8_t, a1);
      float2 xsum[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xsum[i] = ls[(4 * lg + i) * G + g];
#pragma unroll
      for (int T = 0; T < 4; ++T) {
        const uint2 wv = ld_stream2(tw[T] + (int64_t)trow[T] * C + 8 * g + 2 * lg);
        const float sc = bf16_to_f32(ts[T][(int64_t)trow[T] * G + g]);
        const float bi = bf16_to_f32(tb[T][(int64_t)trow[T] * G + g]);
        floatx4 D = floatx4{-xsum[0].y, -xsum[1].y, -xsum[2].y, -xsum[3].y};
        D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, word_operand(wv.x), D, 0, 0, 0);
        D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, word_operand(wv.y), D, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[T][i] += sc * D[i] + bi * xsum[i].x;
      }
    }
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((wave * 4 + T) * 64 + lane) * 4 + i] = acc[T][i];
    __syncthreads();
    // element (pair slot m, weight row n) of tile T sits at lane 16*(m/4)+n, entry m%4
    auto total = [&](int T, int m, int n) {
      const int at = (T * 64 + 16 * (m >> 2) + n) * 4 + (m & 3);
      float v = red[at];
      for (int w = 1; w < 4; ++w) v += red[w * 4 * 64 * 4 + at];
      return v;
    };
    if (kGateUp) {
      if (threadIdx.x < nt) {
        const int m = threadIdx.x;
        float gv[32], uv[32];
#pragma unroll
        for (int c = 0; c < 32; ++c) {
          gv[c] = total(c >> 4, m, c & 15);
          uv[c] = total(2 + (c >> 4), m, c & 15);
        }
        store_h(a, a.pair_list[pb + tt * 16 + m], gv, uv);
      }
    } else {
      const int r0 = blockIdx.x * kDownRows;
      for (int i = threadIdx.x; i < 64 * nt; i += kFfnThreads) {
        const int m = i / 64, rr = i % 64;
        a.y[(int64_t)a.pair_list[pb + tt * 16 + m] * a.d + r0 + rr] = total(rr >> 4, m, rr & 15);
      }
    }
    __syncthreads();
  }
}

template <bool kGateUp>
__global__ __launch_bounds__(kFfnThreads) void k_expert_ffn(FfnArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int u = blockIdx.y;
  if (u >= *a.n_union) return;
  const int e = a.union_experts[u];
  const int pb = a.expert_offsets[u];
  const int ne = a.expert_offsets[u + 1] - pb;
  if (ne <= 0) return;
  if (ne <= kValuMaxPairs)
    ffn_valu<kGateUp>(a, e, pb, ne, smem);
  else
    ffn_mfma<kGateUp>(a, e, pb, ne, smem);
}

// out[t, r] = residual[t, r] + sum_k w[t, k] * y[t*K + k, r], k ascending.
__global__ __launch_bounds__(256) void k_combine(FfnArgs a) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;   // one float4 of out
  const int per_row = a.d / 4;
  if (i >= a.B * per_row) return;
  const int t = i / per_row, r4 = i - t * per_row;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < a.K; ++k) {
    const int p = t * a.K + k;
    if (a.pair_pos[p] < 0) continue;
    const float w = a.topk_w[p];
    const float4 y = reinterpret_cast<const float4*>(a.y + (int64_t)p * a.d)[r4];
    acc.x += w * y.x;
    acc.y += w * y.y;
    acc.z += w * y.z;
    acc.w += w * y.w;
  }
  if (a.residual) {
    const float4 res = reinterpret_cast<const float4*>(a.residual + (int64_t)t * a.d)[r4];
    acc.x = res.x + acc.x;
    acc.y = res.y + acc.y;
    acc.z = res.z + acc.z;
    acc.w = res.w + acc.w;
  }
  reinterpret_cast<float4*>(a.out + (int64_t)t * a.d)[r4] = acc;
}

size_t ffn_smem_bytes(int K) {
  const int G = K / 64, C = K / 8;
  const size_t valu = (size_t)kValuMaxPairs * C * 16 + (size_t)kValuMaxPairs * G * 8 +
                      64 * kValuMaxPairs * 4;
  const size_t mfma = (size_t)16 * G * 8 + 4 * 4 * 64 * 4 * 4;
  return valu > mfma ? valu : mfma;
}

}  // namespace

hipError_t launch_gate_up(const FfnArgs& a, hipStream_t s) {
  const int max_union = a.E < a.B * a.K ? a.E : a.B * a.K;
  hipLaunchKernelGGL(k_expert_ffn<true>, dim3(a.f / kGateUpCols, max_union), dim3(kFfnThreads),
                     ffn_smem_bytes(a.d), s, a);
  return hipGetLastError();
}

hipError_t launch_down(const FfnArgs& a, hipStream_t s) {
  const int max_union = a.E < a.B * a.K ? a.E : a.B * a.K;
  hipLaunchKernelGGL(k_expert_ffn<false>, dim3(a.d / kDownRows, max_union), dim3(kFfnThreads),
                     ffn_smem_bytes(a.f), s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const FfnArgs& a, hipStream_t s) {
  const int n4 = a.B * a.d / 4;
  hipLaunchKernelGGL(k_combine, dim3((n4 + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s) {
  hipError_t err = launch_gate_up(a, s);
  if (err == hipSuccess) err = launch_down(a, s);
  if (err == hipSuccess) err = launch_combine(a, s);
  return err;
}

}  // namespace smoe
