// ffn_mfma.hip - the token-batch expert FFN for prefill chunks (B >= 3).
//
// "Layer-Major Batched Prefill", step 6: every union expert is applied to all
// of its routed pairs in one pass over its weights (gate_up, then down).
// Each wave owns one unit = (union expert, 64 weight rows) and streams the
// unit's rows over the whole input dimension, so the expert's bytes are read
// once per layer for up to 16 pairs (an expert that serves more pairs is
// streamed once per 16-pair tile, which keeps a single small register body).
//
//   gate_up unit: gate rows j0..j0+31 and up rows j0..j0+31 (four 16-row
//     tiles) -> h[pair, j0..j0+31] = silu(g) * u (prepped fp16) and the
//     half-group sums of h that the down pass needs;
//   down unit: down rows r0..r0+63 -> y[pair, r0..r0+63] (fp32).
//
// Per 64-input group g, the dequantised words of each 16-row tile are the B
// operand of two v_mfma_f32_16x16x32_f16 (one per 32-input half), the pairs'
// prepped activations the A operand; the group's scale and bias are applied
// in fp32 right after ("SSD Streaming Expert Layers", "Quantized Layout":
// w = s*q + b):
//     acc += s * (D - C) + b * X,   D = sum_k (1024 + m q_k) stored_k,
// with the accumulator seeded by -C so D - C comes straight out of the MFMA.
// Every union expert of a prefill chunk takes this tile: per weight word the
// VALU work is the 5-op dequantisation plus ~4 ops of epilogue whether the
// expert serves one pair or sixteen, so the kernel stays uniform.
//
// Memory: weights arrive with 8-byte loads per lane (16 rows x 32 contiguous
// bytes per instruction and tile), software-pipelined two stages of
// kGroupsPerStage groups deep, so compute of one stage overlaps the loads of
// the next.  Activations come from L2, group sums from LDS.
#include "device.hpp"
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerUnit = 64;
constexpr int kMaxExpertPairs = 64;                // pairs per expert (B <= 64)

template <int GPS>
struct Stage {
  uint2 w[GPS][4];                                 // 2 words per tile and group
  uint32_t sb[GPS][4];                             // bf16 scale | bf16 bias << 16
  uint4 a[GPS][2];                                 // A operand (this lane's pair)
};

struct UnitPtrs {
  const uint32_t* w[4];
  const uint16_t* s[4];
  const uint16_t* b[4];
};

template <bool kNT>
__device__ __forceinline__ uint2 ld_w2(const uint32_t* p) {
  if (kNT) return ld_stream2(p);
  return *reinterpret_cast<const uint2*>(p);
}

// Loads of groups g0 .. g0 + GPS - 1, clamped to the last group (the compute
// step gives the copies zero weight).
template <int GPS, bool kNT>
__device__ __forceinline__ void load_stage(const UnitPtrs& P, const uint4* arow, bool avalid,
                                           int g0, int G, int lg, Stage<GPS>& st) {
#pragma unroll
  for (int gg = 0; gg < GPS; ++gg) {
    const int g = min(g0 + gg, G - 1);
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      st.w[gg][T] = ld_w2<kNT>(P.w[T] + 8 * g + 2 * lg);
      st.sb[gg][T] = (uint32_t)P.s[T][g] | ((uint32_t)P.b[T][g] << 16);
    }
    const uint4 a0 = arow[8 * g + 2 * lg], a1 = arow[8 * g + 2 * lg + 1];
    const uint4 z = make_uint4(0, 0, 0, 0);
    st.a[gg][0] = avalid ? a0 : z;
    st.a[gg][1] = avalid ? a1 : z;
  }
}

// acc += s (D - C) + b X for the groups of one stage; groups past the end
// (clamped copies) get s = b = 0.
template <int GPS>
__device__ __forceinline__ void compute_stage(const Stage<GPS>& cur, int g0, int G, const float2* ls,
                                              int ne, int m0, int lg, floatx4 (&acc)[4]) {
#pragma unroll
  for (int gg = 0; gg < GPS; ++gg) {
    const int g = g0 + gg;
    const bool live = g < G;
    const int gc = min(g, G - 1);
    const half8_t A0 = __builtin_bit_cast(half8_t, cur.a[gg][0]);
    const half8_t A1 = __builtin_bit_cast(half8_t, cur.a[gg][1]);
    float2 xsum[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 4 * lg + i;
      const float2 v = ls[min(m, ne - 1) * G + gc];
      xsum[i] = m < ne ? v : make_float2(0.f, 0.f);
    }
    const floatx4 seed = floatx4{-xsum[0].y, -xsum[1].y, -xsum[2].y, -xsum[3].y};
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const uint32_t sbv = live ? cur.sb[gg][T] : 0u;
      const float sc = __uint_as_float(sbv << 16);
      const float bi = __uint_as_float(sbv & 0xFFFF0000u);
      floatx4 D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, word_operand(cur.w[gg][T].x), seed, 0,
                                                         0, 0);
      D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, word_operand(cur.w[gg][T].y), D, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[T][i] += sc * D[i] + bi * xsum[i].x;
    }
  }
}

// One 16-pair token tile (the expert's pairs m0 .. m0+15) of this wave's unit.
template <bool kGateUp, int GPS, bool kNT>
__device__ __forceinline__ void unit_tile(const FfnArgs& a, const UnitPtrs& P, const int (&rows0)[4],
                                          const int* lpair, const float2* ls, int ne, int m0,
                                          int unit, int G) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, lg = lane >> 4;
  const int ma = m0 + col;                         // this lane's pair in the A operand
  const bool avalid = ma < ne;
  const int pa = lpair[avalid ? ma : m0];
  const uint4* arow = kGateUp ? reinterpret_cast<const uint4*>(a.xp + (int64_t)(pa / a.K) * a.d)
                              : reinterpret_cast<const uint4*>(a.hp + (int64_t)pa * a.f);

  floatx4 acc[4];
#pragma unroll
  for (int T = 0; T < 4; ++T) acc[T] = floatx4{0.f, 0.f, 0.f, 0.f};

  Stage<GPS> st0, st1;
  load_stage<GPS, kNT>(P, arow, avalid, 0, G, lg, st0);
  load_stage<GPS, kNT>(P, arow, avalid, GPS, G, lg, st1);
  for (int g0 = 0; g0 < G; g0 += 2 * GPS) {
    compute_stage<GPS>(st0, g0, G, ls, ne, m0, lg, acc);
    load_stage<GPS, kNT>(P, arow, avalid, g0 + 2 * GPS, G, lg, st0);
    compute_stage<GPS>(st1, g0 + GPS, G, ls, ne, m0, lg, acc);
    load_stage<GPS, kNT>(P, arow, avalid, g0 + 3 * GPS, G, lg, st1);
  }

  // epilogue: lane holds (pair slot m0 + 4 lg + i, row rows0[T] + col)
  if (kGateUp) {
    // h for columns j = unit*32 + Th*16 + col, from gate tile Th and up tile Th+2
    float X[4] = {0.f, 0.f, 0.f, 0.f}, S[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int Th = 0; Th < 2; ++Th) {
      const int j = unit * 32 + Th * 16 + col;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 4 * lg + i;
        const float h = silu_mul(acc[Th][i], acc[Th + 2][i]);
        const half_t xi = (half_t)h;
        const half_t stv = (j & 1) ? (half_t)((float)xi * 0.0625f) : xi;
        const float stf = (float)stv;
        S[i] += stf;
        X[i] += (j & 1) ? stf * 16.0f : stf;
        if (m < ne) {
          const int n = j & 7;
          a.hp[(int64_t)lpair[m] * a.f + (j & ~7) + 2 * (n & 3) + (n >> 2)] = f16_bits(stv);
        }
      }
    }
    // sums over the unit's 32 columns: the 16 lanes of a row segment
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float Xt = segment_sum16(X[i], 16), St = segment_sum16(S[i], 16);
      const int m = m0 + 4 * lg + i;
      if (col == 0 && m < ne) {
        const int j0 = unit * 32;
        a.hs[((int64_t)lpair[m] * (a.f / 64) + j0 / 64) * 2 + (j0 % 64) / 32] =
            make_float2(Xt, 1024.0f * St);
      }
    }
  } else {
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + 4 * lg + i;
        if (m < ne) a.y[(int64_t)lpair[m] * a.d + rows0[T] + col] = acc[T][i];
      }
  }
}

template <bool kGateUp, int GPS, bool kNT>
__global__ __launch_bounds__(kThreads, 2) void k_ffn_mfma(FfnArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int u = blockIdx.y;
  const int nU = *a.n_union;
  if (u >= nU) return;
  const int e = a.union_experts[u];
  const int pb = a.expert_offsets[u];
  const int ne = a.expert_offsets[u + 1] - pb;     // 1 .. kMaxExpertPairs
  const int K = kGateUp ? a.d : a.f;
  const int G = K / 64, C = K / 8;

  // pairs of this expert and their group sums in LDS: ls[m][g] = (X, C)
  int* lpair = reinterpret_cast<int*>(smem);                                  // [kMaxExpertPairs]
  float2* ls = reinterpret_cast<float2*>(smem + 4 * kMaxExpertPairs);              // [ne][G]
  for (int i = threadIdx.x; i < ne; i += kThreads) lpair[i] = a.pair_list[pb + i];
  __syncthreads();
  for (int i = threadIdx.x; i < ne * G; i += kThreads) {
    const int m = i / G, g = i - m * G;
    const int p = lpair[m];
    float2 v;
    if (kGateUp) {
      v = a.xs[(int64_t)(p / a.K) * G + g];
    } else {
      const float2* hs = a.hs + ((int64_t)p * G + g) * 2;
      const float2 lo = hs[0], hi = hs[1];
      v = make_float2(lo.x + hi.x, lo.y + hi.y);
    }
    ls[i] = v;
  }
  __syncthreads();

  // this wave's unit: four 16-row tiles (waves past the last unit stop here;
  // no block barrier follows)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int unit = blockIdx.x * kWaves + wave;
  const int units = kGateUp ? a.f / 32 : a.d / kRowsPerUnit;
  if (unit >= units) return;
  const int col = threadIdx.x & 15;
  UnitPtrs P;
  int rows0[4];
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    const QMat& m = kGateUp ? (T < 2 ? a.gate : a.up) : a.down;   // T is a constant here
    rows0[T] = kGateUp ? unit * 32 + (T & 1) * 16 : unit * kRowsPerUnit + T * 16;
    const int64_t row = rows0[T] + col;
    P.w[T] = m.w + e * m.stride_w + row * C;
    P.s[T] = m.s + e * m.stride_sb + row * G;
    P.b[T] = m.b + e * m.stride_sb + row * G;
  }
  for (int m0 = 0; m0 < ne; m0 += 16) unit_tile<kGateUp, GPS, kNT>(a, P, rows0, lpair, ls, ne, m0, unit, G);
}

}  // namespace

size_t mfma_smem_bytes(const FfnArgs& a, bool gate_up) {
  const int G = (gate_up ? a.d : a.f) / 64;
  // an expert serves at most one pair per token
  return 4 * kMaxExpertPairs + (size_t)a.B * G * sizeof(float2);
}

hipError_t launch_ffn_mfma(const FfnArgs& a, hipStream_t s, bool gate_up) {
  if (a.B > kMaxExpertPairs) return hipErrorInvalidValue;
  const int max_union = a.E < a.B * a.K ? a.E : a.B * a.K;
  const int units = gate_up ? a.f / 32 : a.d / kRowsPerUnit;
  const dim3 grid((units + kWaves - 1) / kWaves, max_union);
  if (gate_up)
    hipLaunchKernelGGL((k_ffn_mfma<true, 1, false>), grid, dim3(kThreads), mfma_smem_bytes(a, true), s, a);
  else
    hipLaunchKernelGGL((k_ffn_mfma<false, 1, false>), grid, dim3(kThreads), mfma_smem_bytes(a, false), s,
                       a);
  return hipGetLastError();
}

}  // namespace smoe
