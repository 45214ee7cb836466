// ffn_gemv.hip - the expert FFN when every union expert serves one or two
// pairs (B <= 2 tokens, the decode regime of "Data Flow", Regime 2).
//
// Each union expert is a matrix-vector product ("Layer-Major Batched
// Prefill", step 6, with B = 1): the work is a pure stream of the expert
// bytes, so both kernels are built to keep many 16-byte loads in flight:
//
//  k_gate_up_gemv: wave = (union expert, 4 consecutive j); it loads the 4 gate
//    rows and 4 up rows before any arithmetic, holds the pairs' activations
//    for its fixed groups in registers, reduces rows with DPP, and writes
//    h_j = silu(g_j) * u_j ("SSD Streaming Expert Layers", "Math Contract")
//    as prepped fp16.
//  k_down_combine_gemv: block = 8 output rows for ALL union experts; its
//    weight loads are issued first, h and its group sums are staged in LDS
//    meanwhile, and the block finishes with the weighted combine of its rows
//    in rank order ("Data Flow": routed_out, residual += ...), so y never
//    leaves the chip.
//
// Lane layout: a row of G groups (64 inputs each) is spread over TPR lanes
// (the largest power of two dividing G, at most 64), each lane owning GPL =
// G/TPR consecutive groups (32*GPL contiguous bytes of the row), so one wave
// instruction covers 64/TPR rows.
#include "device.hpp"
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kGemvThreads = 256;
constexpr int kJPerWave = 4;          // gate_up: j-rows per wave
constexpr int kDownRowsGemv = 8;      // down: output rows per block
// down: (expert, row step) items per wave per batch of loads
template <int GPL>
constexpr int items_per_wave() { return GPL >= 3 ? 2 : 4; }

// Prepped position (half index within the row) of column c.
__device__ __forceinline__ int prepped_pos(int c) {
  const int n = c & 7;
  return (c & ~7) + 2 * (n & 3) + (n >> 2);
}

// Dot of one lane's GPL groups (8 words each) against prepped activations,
// with the fp32 group epilogue: sum_g s_g (D_g - C_g) + b_g X_g.
template <int GPL>
__device__ __forceinline__ float lane_row_dot(const uint4 (&w)[GPL][2], const float (&sc)[GPL],
                                              const float (&bi)[GPL], const uint4* xc,
                                              const float2* xsum) {
  float part = 0.f;
#pragma unroll
  for (int gi = 0; gi < GPL; ++gi) {
    float acc = 0.f;
    acc = dot_word(w[gi][0].x, xc[gi * 8 + 0], acc);
    acc = dot_word(w[gi][0].y, xc[gi * 8 + 1], acc);
    acc = dot_word(w[gi][0].z, xc[gi * 8 + 2], acc);
    acc = dot_word(w[gi][0].w, xc[gi * 8 + 3], acc);
    acc = dot_word(w[gi][1].x, xc[gi * 8 + 4], acc);
    acc = dot_word(w[gi][1].y, xc[gi * 8 + 5], acc);
    acc = dot_word(w[gi][1].z, xc[gi * 8 + 6], acc);
    acc = dot_word(w[gi][1].w, xc[gi * 8 + 7], acc);
    part += sc[gi] * (acc - xsum[gi].y) + bi[gi] * xsum[gi].x;
  }
  return part;
}

// ----------------------------------------------------------------- gate_up
template <int NTOK>
__global__ __launch_bounds__(kGemvThreads) void k_gate_up_gemv(FfnArgs a) {
  constexpr int kRows = 2 * kJPerWave;            // gate rows then up rows
  __shared__ float red[kGemvThreads / 64][kRows][NTOK];
  const int u = blockIdx.y;                        // < min(E, B*K): index always in range
  const int nU = *a.n_union;
  const int e = a.union_experts[u];
  const int pb = a.expert_offsets[u];
  const int ne = a.expert_offsets[u + 1] - pb;     // 1 .. NTOK
  if (u >= nU) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int d = a.d, G = d / 64, C = d / 8;
  const int tpr = G, rps = 64 / tpr;               // one group per lane
  const int li = lane % tpr, slot = lane / tpr;
  const int j0 = (blockIdx.x * (kGemvThreads / 64) + wave) * kJPerWave;
  // per-expert bases (uniform), selected per lane by pointer, never by struct index
  const uint32_t* gw = a.gate.w + e * a.gate.stride_w;
  const uint16_t* gs = a.gate.s + e * a.gate.stride_sb;
  const uint16_t* gb = a.gate.b + e * a.gate.stride_sb;
  const uint32_t* uw = a.up.w + e * a.up.stride_w;
  const uint16_t* us = a.up.s + e * a.up.stride_sb;
  const uint16_t* ub = a.up.b + e * a.up.stride_sb;

  // 1. every weight load of this wave, raw; steps past the wave's rows are
  //    skipped uniformly, lanes past them load a valid row and get zero scale
  const int nsteps = (kRows + rps - 1) / rps;
  uint4 w[kRows][2];
  uint32_t sraw[kRows], braw[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    if (k < nsteps) {
      const int rs = k * rps + slot;
      const bool live = rs < kRows;
      const int rsc = live ? rs : kRows - 1;
      const bool is_up = rsc >= kJPerWave;
      const int64_t row = j0 + (rsc & (kJPerWave - 1));
      const uint32_t* wr = (is_up ? uw : gw) + row * C + li * 8;
      const int64_t sidx = row * G + li;
      w[k][0] = ld_stream4(wr);
      w[k][1] = ld_stream4(wr + 4);
      const uint32_t sv = (is_up ? us : gs)[sidx], bv = (is_up ? ub : gb)[sidx];
      sraw[k] = live ? sv : 0u;
      braw[k] = live ? bv : 0u;
    }
  }
  // 2. the pairs' activations for this lane's group
  uint4 xr[NTOK][8];
  float2 xs[NTOK];
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    const int tok = NTOK == 1 && a.B == 1 ? 0 : a.pair_list[pb + min(t, ne - 1)] / a.K;
    const uint4* src = reinterpret_cast<const uint4*>(a.xp + (int64_t)tok * d) + li * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) xr[t][q] = src[q];
    xs[t] = a.xs[(int64_t)tok * G + li];
  }
  const int pair0 = a.pair_list[pb];
  const int pair1 = NTOK > 1 ? a.pair_list[pb + min(1, ne - 1)] : pair0;
  // 3. dot products, row sums across the row's lanes
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    if (k < nsteps) {   // uniform: every lane takes part in the reductions
      const int rs = k * rps + slot;
      const float sc[1] = {bf16_to_f32((uint16_t)sraw[k])};
      const float bi[1] = {bf16_to_f32((uint16_t)braw[k])};
      const uint4 wk[1][2] = {{w[k][0], w[k][1]}};
#pragma unroll
      for (int t = 0; t < NTOK; ++t) {
        if (t < ne) {
          float part = lane_row_dot<1>(wk, sc, bi, xr[t], &xs[t]);
          part = segment_sum(part, tpr);
          if (li == 0 && rs < kRows) red[wave][rs][t] = part;
        }
      }
    }
  }
  __syncthreads();
  // 4. h_j = silu(g_j) * u_j, stored prepped
  if (lane < kJPerWave * ne) {
    const int jj = lane % kJPerWave, t = lane / kJPerWave;
    const int j = j0 + jj;
    const float h = silu_mul(red[wave][jj][t], red[wave][kJPerWave + jj][t]);
    const half_t hv = (j & 1) ? (half_t)((float)(half_t)h * 0.0625f) : (half_t)h;
    a.hp[(int64_t)(t == 0 ? pair0 : pair1) * a.f + prepped_pos(j)] = f16_bits(hv);
  }
}

// --------------------------------------------------------- down + combine
// Issue the loads of (up to) IPW items starting at `first`.
template <int GPL, int IPW = items_per_wave<GPL>()>
__device__ __forceinline__ void down_load_items(
    const FfnArgs& a, int first, int items, int steps, int rps, int slot, int li, int r0, int C,
    int G, uint4 (&w)[IPW][GPL][2], uint32_t (&sraw)[IPW][GPL],
    uint32_t (&braw)[IPW][GPL], int (&pbs)[IPW],
    int (&nes)[IPW]) {
#pragma unroll
  for (int q = 0; q < IPW; ++q) {
    // dead items / lanes load a valid duplicate row and get zero scale and bias
    const int it = first + q * 4;
    const bool live_item = it < items;
    const int itc = live_item ? it : items - 1;
    const int uu = itc / steps, st = itc % steps;
    const int e = a.union_experts[uu];
    pbs[q] = live_item ? a.expert_offsets[uu] : 0;
    nes[q] = live_item ? a.expert_offsets[uu + 1] - a.expert_offsets[uu] : 0;
    const int rr = st * rps + slot;
    const bool live = live_item && rr < kDownRowsGemv;
    const int64_t row = r0 + min(rr, kDownRowsGemv - 1);
    const uint32_t* wr = a.down.w + e * a.down.stride_w + row * C + li * GPL * 8;
    const uint16_t* sr = a.down.s + e * a.down.stride_sb + row * G + li * GPL;
    const uint16_t* br = a.down.b + e * a.down.stride_sb + row * G + li * GPL;
#pragma unroll
    for (int gi = 0; gi < GPL; ++gi) {
      w[q][gi][0] = ld_stream4(wr + gi * 8);
      w[q][gi][1] = ld_stream4(wr + gi * 8 + 4);
      const uint32_t sv = sr[gi], bv = br[gi];
      sraw[q][gi] = live ? sv : 0u;
      braw[q][gi] = live ? bv : 0u;
    }
  }
}

template <int GPL>
__global__ __launch_bounds__(kGemvThreads) void k_down_combine_gemv(FfnArgs a) {
  constexpr int IPW = items_per_wave<GPL>();
  extern __shared__ __align__(16) char smem[];
  const int f = a.f, G = f / 64, C = f / 8, K = a.K, B = a.B, P = B * K;
  const int hx_chunks = (P * C + 63) / 64 * 64;                        // padded for the DMA tail
  uint4* hx = reinterpret_cast<uint4*>(smem);                          // [P][C] prepped h
  float2* hsum = reinterpret_cast<float2*>(hx + hx_chunks);            // [P][G] (X, C)
  float* ylds = reinterpret_cast<float*>(hsum + (size_t)P * G);        // [P][kDownRowsGemv]
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nU = *a.n_union;
  const int tpr = G / GPL, rps = 64 / tpr;
  const int li = lane % tpr, slot = lane / tpr;
  const int steps = (kDownRowsGemv + rps - 1) / rps;   // row steps per expert
  const int r0 = blockIdx.x * kDownRowsGemv;
  const int items = nU * steps;

  // this wave's items (expert slot, row step), dealt round-robin over the 4 waves;
  // expert ids are read as scalars and every weight load is issued at once
  uint4 w[IPW][GPL][2];
  uint32_t sraw[IPW][GPL], braw[IPW][GPL];
  int pbs[IPW], nes[IPW];
  down_load_items<GPL>(a, wave, items, steps, rps, slot, li, r0, C, G, w, sraw, braw, pbs, nes);
  // h of every pair (written by gate_up, L2-resident) goes straight to LDS:
  // each wave copies 1 KB per instruction (lane i -> 16 bytes at base + 16 i)
  {
    const int nchunk = P * C;
    const uint4* src = reinterpret_cast<const uint4*>(a.hp);
    for (int cb = wave * 64; cb < nchunk; cb += kGemvThreads) {
      const int i = min(cb + lane, nchunk - 1);
      __builtin_amdgcn_global_load_lds(src + i, (__attribute__((address_space(3))) void*)(hx + cb),
                                       16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < P * G; i += kGemvThreads) {
    const uint16_t* hh = reinterpret_cast<const uint16_t*>(hx + (size_t)(i / G) * C + (i % G) * 8);
    // halves of a chunk: (x0,x4) (x1/16,x5/16) (x2,x6) (x3/16,x7/16)
    float X = 0.f, S = 0.f;
#pragma unroll 8
    for (int z = 0; z < 64; ++z) {
      const float st = (float)bits_f16(hh[z]);
      S += st;
      X += (z & 2) ? 16.0f * st : st;
    }
    hsum[i] = make_float2(X, 1024.0f * S);
  }
  __syncthreads();

  for (int first = wave; first < items; first += 4 * IPW) {
    if (first != wave)
      down_load_items<GPL>(a, first, items, steps, rps, slot, li, r0, C, G, w, sraw, braw, pbs, nes);
#pragma unroll
    for (int q = 0; q < IPW; ++q) {
      const int it = first + q * 4;
      if (it < items) {   // uniform across the wave
        const int st = it % steps;
        const int rr = st * rps + slot;
        float sc[GPL], bi[GPL];
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          sc[gi] = bf16_to_f32((uint16_t)sraw[q][gi]);
          bi[gi] = bf16_to_f32((uint16_t)braw[q][gi]);
        }
        for (int j = 0; j < nes[q]; ++j) {
          const int p = a.pair_list[pbs[q] + j];
          const uint4* xc = hx + (size_t)p * C + li * GPL * 8;
          const float2* xsm = hsum + (size_t)p * G + li * GPL;
          float part = lane_row_dot<GPL>(w[q], sc, bi, xc, xsm);
          part = segment_sum(part, tpr);
          if (li == 0 && rr < kDownRowsGemv) ylds[p * kDownRowsGemv + rr] = part;
        }
      }
    }
  }
  __syncthreads();
  // combine: out[t, r] = residual[t, r] + sum_k w[t, k] * y[t*K + k, r], k ascending
  for (int i = threadIdx.x; i < B * kDownRowsGemv; i += kGemvThreads) {
    const int t = i / kDownRowsGemv, rr = i % kDownRowsGemv;
    float acc = 0.f;
    for (int k = 0; k < K; ++k) {
      const int p = t * K + k;
      if (a.pair_pos[p] < 0) continue;
      acc += a.topk_w[p] * ylds[p * kDownRowsGemv + rr];
    }
    const int64_t o = (int64_t)t * a.d + r0 + rr;
    const float res = a.residual ? a.residual[o] : 0.f;
    a.out[o] = res + acc;
  }
}

size_t down_gemv_smem(const FfnArgs& a) {
  const size_t P = (size_t)a.B * a.K;
  const size_t hx_chunks = (P * (a.f / 8) + 63) / 64 * 64;
  return hx_chunks * 16 + P * (a.f / 64) * 8 + P * kDownRowsGemv * 4;
}

template <int GPL>
hipError_t launch_down_gemv(const FfnArgs& a, hipStream_t s, const LaunchTiming* t) {
  SMOE_LAUNCH(t, k_down_combine_gemv<GPL>, dim3(a.d / kDownRowsGemv), dim3(kGemvThreads),
                     down_gemv_smem(a), s,
                     a);
  return hipGetLastError();
}

int gpl_of(int G) {
  int t = 1;
  while (t < 64 && G % (2 * t) == 0) t *= 2;
  return G / t;
}

}  // namespace

// The small-batch path applies when every expert serves at most two pairs,
// the staged h fits in LDS, and the lanes' group counts are supported
// (gate_up: one group per lane; down: up to three).
bool gemv_path_ok(const FfnArgs& a) {
  if (a.B > 2 || a.B * a.K > 16) return false;
  if (gpl_of(a.d / 64) != 1 || gpl_of(a.f / 64) > 3) return false;
  if (a.f % (kJPerWave * (kGemvThreads / 64)) != 0 || a.d % kDownRowsGemv != 0) return false;
  return down_gemv_smem(a) <= 64 * 1024;
}

hipError_t launch_gemv(const FfnArgs& a, hipStream_t s, bool gate_up, const LaunchTiming* t) {
  if (gate_up) {
    const int max_union = a.E < a.B * a.K ? a.E : a.B * a.K;
    const dim3 grid(a.f / (kJPerWave * (kGemvThreads / 64)), max_union);
    if (a.B == 1)
      SMOE_LAUNCH(t, k_gate_up_gemv<1>, grid, dim3(kGemvThreads), 0, s, a);
    else
      SMOE_LAUNCH(t, k_gate_up_gemv<2>, grid, dim3(kGemvThreads), 0, s, a);
    return hipGetLastError();
  }
  switch (gpl_of(a.f / 64)) {
    case 1: return launch_down_gemv<1>(a, s, t);
    case 2: return launch_down_gemv<2>(a, s, t);
    default: return launch_down_gemv<3>(a, s, t);
  }
}

}  // namespace smoe
