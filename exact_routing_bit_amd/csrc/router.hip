// router.hip - exact routing and the layer-major inversion on the device.
//
// One launch (B <= 2) or two do the whole routing step ("Data Flow", serial step "EXACT
// ROUTING: gate matvec on heavy_normed -> ranked top-k", "norm_topk_prob
// weights"; "Layer-Major Batched Prefill", "The Inversion"):
//   1. blocks compute logits[t,e] = sum_i Wr[e,i] x[t,i] (fp32) for a tile
//      of experts x tokens (B <= 2: one expert and every token a block, its
//      row split over the four waves; B >= 3: 4 tokens x 16 experts x one K
//      slice of at most 1024 inputs a block, x staged in LDS), and further
//      blocks (one a token) convert x into the prepped fp16 activation layout
//      the expert kernels read;
//   2. the last blocks to finish (integer tickets) rank every token's experts
//      by (logit descending, index ascending), form the softmax /
//      norm_topk_prob weights, and build the union of the batch's experts with
//      the sorted per-expert pair lists, all from LDS.  B <= 2 grids finish in
//      one last block; B >= 3 grids hand their K-slice partial sums to a
//      top-k grid (a token a wave), whose last block builds the union.
// No host synchronisation; downstream grids read n_union on the device.
#include <float.h>
#include <limits.h>

#include "device.hpp"
#include "route_dev.hpp"
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kMaxRouteTok = 2;                 // k_route's batches; larger ones are tiled
constexpr int kTailThreads = 1024;              // stand-alone top-k / union block
constexpr int kTopkThreads = 256;               // top-k grid: one token per wave
constexpr int kMaxTicketBlocks = 64;            // larger grids hand the tail to its own kernel

// Top-k of one token's E <= 256 logits by one full wave; writes indices and
// weights (rank order) to global memory and the indices to s_idx.
__device__ __forceinline__ void topk_token(const RouteArgs& a, int t, int32_t* s_idx,
                                           TopkScratch* sc) {
  const int lane = __lane_id();
  const int E = a.E, K = a.K;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? a.logits[(int64_t)t * E + e] : -FLT_MAX;
  }
  float my_v;
  int my_e;
  wave_topk(v, E, K, my_v, my_e, sc);
  const float w = topk_weight(v, E, K, a.norm != 0, my_v);
  if (lane < K) {
    a.topk_idx[t * K + lane] = my_e;
    a.topk_w[t * K + lane] = w;
    s_idx[t * K + lane] = my_e;
  }
}

struct UnionSmem {
  int32_t idx[kMaxPairs];
  int32_t hist[kMaxExperts];
  int32_t pos[kMaxExperts];
  alignas(16) uint32_t mask[kMaxExperts * (kMaxPairs / 32)];   // rows of 16-byte pieces
  alignas(16) uint16_t before[kMaxExperts * (kMaxPairs / 32)];  // the row's bits in earlier words
  TopkScratch topk[16];   // one per wave (blocks of up to 1024 threads)
};

static_assert(sizeof(UnionSmem) <= 64 * 1024, "the router's tail takes it as dynamic LDS");

// Inclusive prefix sum over the wave (lane order), by DPP: shifts of 1, 2,
// 4, 8 within rows of 16, then row 0's total into row 1 and row 2's into row
// 3, then row 1's into rows 2 and 3.  Lanes whose source lies outside the
// row read 0.  Every lane of the wave must be active.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2, 3
  return v;
}

// Union of the batch's experts and the per-expert pair lists, by one block
// (a multiple of 64 threads, at least two waves) from us->idx[0..P).
__device__ __forceinline__ void build_union(const RouteArgs& a, UnionSmem* us) {
  const int nthr = blockDim.x, tid = threadIdx.x;
  const int E = a.E, P = a.B * a.K;
  const int W = ((P + 31) / 32 + 3) & ~3;         // mask words an expert: whole 16-byte pieces
  for (int i = tid; i < E; i += nthr) us->hist[i] = 0;
  for (int i = tid; i < E * W / 4; i += nthr)
    reinterpret_cast<uint4*>(us->mask)[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  for (int p = tid; p < P; p += nthr) {
    const int e = us->idx[p];
    if (e >= 0 && e < E) {
      atomicAdd(&us->hist[e], 1);
      atomicOr(&us->mask[e * W + (p >> 5)], 1u << (p & 31));
    } else {
      atomicOr(a.status, (uint32_t)SMOE_STATUS_BAD_EXPERT);
      a.pair_pos[p] = -1;
    }
  }
  __syncthreads();
  // (blocks of at least two waves) the waves past the first count, for every
  // expert row and mask word, the row's bits in the words before it, while
  // the first wave scans the experts
  for (int e = tid - 64; e >= 0 && e < E; e += nthr - 64) {
    const uint4* m4 = reinterpret_cast<const uint4*>(us->mask + e * W);
    uint16_t* b = us->before + e * W;
    int run = 0;
    for (int i = 0; i < W / 4; ++i) {
      const uint4 v = m4[i];
      b[4 * i] = (uint16_t)run;
      run += __popc(v.x);
      b[4 * i + 1] = (uint16_t)run;
      run += __popc(v.y);
      b[4 * i + 2] = (uint16_t)run;
      run += __popc(v.z);
      b[4 * i + 3] = (uint16_t)run;
      run += __popc(v.w);
    }
  }
  if (tid < 64) {
    // exclusive scans of pair counts and of non-empty experts; lane l owns experts 4l..4l+3
    const int lane = tid;
    int c[4], cnt = 0, nz = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      c[j] = e < E ? us->hist[e] : 0;
      cnt += c[j];
      nz += c[j] > 0;
    }
    const int inc_c = wave_scan_incl(cnt), inc_nz = wave_scan_incl(nz);
    int pos = inc_c - cnt, uid = inc_nz - nz;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * lane + j;
      if (e < E) us->pos[e] = pos;
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
  for (int p = tid; p < P; p += nthr) {
    const int e = us->idx[p];
    if (e < 0 || e >= E) continue;
    // rank = the expert's pairs before p: its bits in the words before p's,
    // then those below p in p's own word
    const int at = e * W + (p >> 5);
    const int rank = us->before[at] + __popc(us->mask[at] & ((1u << (p & 31)) - 1u));
    const int q = us->pos[e] + rank;
    a.pair_list[q] = p;
    a.pair_pos[p] = q;
  }
}

// Top-k of every token, then (optionally) the union, by the calling block.
__device__ __forceinline__ void route_tail(const RouteArgs& a, bool do_topk, bool do_union,
                                           UnionSmem* us) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), nwaves = blockDim.x >> 6;
  if (do_topk)
    for (int t = wave; t < a.B; t += nwaves) topk_token(a, t, us->idx, &us->topk[wave]);
  if (!do_union) return;
  __syncthreads();
  if (!do_topk)
    for (int p = threadIdx.x; p < a.B * a.K; p += blockDim.x) us->idx[p] = a.topk_idx[p];
  build_union(a, us);
}


// B <= 2 tokens (NT = B), one grid row: blocks [0, B) prep a token's
// activations (prep_token), blocks B .. B + E - 1 form the logits of one
// expert each (logits_block).  do_tail: the last block to finish ranks and
// builds the union, in dynamic LDS of sizeof(UnionSmem) bytes that only such
// launches ask for (the decode layer's router needs none).
template <bool kBf16, int NT, int kM>
__global__ __launch_bounds__(kRouteThreads) void k_route(RouteArgs a, int do_tail,
                                                         uint32_t* ticket) {
  extern __shared__ __align__(16) char route_dyn[];
  __shared__ int is_last;
  __shared__ float part[kRouteThreads / 64][NT];
  if ((int)blockIdx.x < NT) {
    if (a.xp != nullptr) {
      const int t = blockIdx.x;
      const float inv = a.norm_out != nullptr
                            ? block_row_inv(a.x + (int64_t)t * a.d, a.d, a.norm_eps, &part[0][0])
                            : 1.0f;
      prep_token(a.x, a.d, t, a.xp, a.xs, a.xa, a.norm_out, inv, &part[0][0]);
    }
  } else {
    logits_block<kBf16, NT, kM>(a, blockIdx.x - NT, part);
  }
  if (!do_tail) return;
  // The last block to finish reads every block's logits.  Each wave releases
  // its own stores at device (agent) scope before the block counts itself in
  // with an acquire-release ticket; the last block acquires at the same scope
  // before it reads.  The XCDs' L2 caches are not coherent with each other,
  // so a release by one thread would not cover the stores of another wave.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t n = gridDim.x * gridDim.y;
    const uint32_t t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (t == n - 1);
    // the next launch is ordered after this one by the kernel boundary
    if (is_last) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  route_tail(a, true, a.n_union != nullptr, reinterpret_cast<UnionSmem*>(route_dyn));
}

// ------------------------------------------------ tiled logits (B >= 3)
// The logits of a batch are a small matrix product, logits = x Wr^T, of
// [B, d] fp32 by [E, d]; a grid that gave every wave one expert and two
// tokens would read x from the caches once per expert.  Here a block owns a
// tile of kTileTok tokens x kTileExp experts x one K slice of 256 kM inputs:
// the tokens' slice of x is staged once in LDS and used by all 16 experts
// (each wave streams four gate rows), and the slices' partial sums go to a
// workspace buffer, which k_topk_grid adds up in slice order.  The slice is
// the narrowest of 256, 512, 1024 inputs that cuts d into at most
// kMaxSlices: short slices make short dependent chains (load, stage, sum)
// spread over more blocks.  No tickets here: a device-scope release costs
// an L2 writeback, and hundreds of them (one per block) cost far more than
// the kernel boundary that publishes the partials.
constexpr int kTileTok = 4;
constexpr int kTileExp = 16;                    // four experts a wave
constexpr int kMaxSlices = 8;
static_assert(kTileExp / 4 * kTileTok == 16, "two eight-row transpose-reduces per wave");

// 4-input pieces a lane takes per slice (slice = 256 kM inputs) for a row of d.
inline int slice_pieces(int d) { return d <= 8 * 256 ? 1 : d <= 8 * 512 ? 2 : 4; }
inline int n_slices(int d) { return (d + 256 * slice_pieces(d) - 1) / (256 * slice_pieces(d)); }

// Gate values of expert e at inputs k0 + 256 m + 4 l .. + 3 (lane l, m < kM),
// zeros past d or for e >= E.
template <bool kBf16, int kM>
__device__ __forceinline__ void gate_slice(const RouteArgs& a, int e, int k0, float4 (&w)[kM]) {
  const int lane = __lane_id();
#pragma unroll
  for (int m = 0; m < kM; ++m) {
    const int i = k0 + 256 * m + 4 * lane;
    const bool ok = e < a.E && i < a.d;
    const int64_t at = ok ? (int64_t)e * a.d + i : 0;
    if (kBf16) {
      const uint2 raw = *reinterpret_cast<const uint2*>((const uint16_t*)a.router_w + at);
      w[m] = ok ? make_float4(__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xFFFF0000u),
                              __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xFFFF0000u))
                : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
      const float4 v = *reinterpret_cast<const float4*>((const float*)a.router_w + at);
      w[m] = ok ? v : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// grid (one-dimensional): the prep blocks (one a token, first, as they have
// the longer chains), then ceil(B/4) tile rows of ceil(E/16) * n_slices logit
// blocks.  Logit block (eb, ks) of tile row ty: experts 16 eb .., inputs
// 256 kM ks .., tokens 4 ty ..; partial sums to lgp[ks][t][e].
template <bool kBf16, int kM>
__global__ __launch_bounds__(kRouteThreads) void k_route_tiled(RouteArgs a) {
  constexpr int kK = 256 * kM;                  // the slice
  __shared__ float xt[kTileTok][kK];
  __shared__ float part[kRouteThreads / 64];
  const int n_ks = (a.d + kK - 1) / kK;
  const int n_logit = ((a.E + kTileExp - 1) / kTileExp) * n_ks;
  const int n_prep = a.xp != nullptr ? a.B : 0;
  if ((int)blockIdx.x < n_prep) {
    prep_token(a.x, a.d, blockIdx.x, a.xp, a.xs, a.xa, nullptr, 1.0f, part);
    return;
  }
  const int lb = blockIdx.x - n_prep;
  const int t0 = (lb / n_logit) * kTileTok, bx = lb % n_logit;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = __lane_id();
  const int ew = (bx / n_ks) * kTileExp + 4 * wave, ks = bx % n_ks;
  const int k0 = ks * kK;
  // the wave's four gate rows first: they come from HBM, x from the caches
  float4 w[4][kM];
#pragma unroll
  for (int j = 0; j < 4; ++j) gate_slice<kBf16, kM>(a, ew + j, k0, w[j]);
  // x[t0 .., k0 ..] -> LDS, zeros past the batch or past d
#pragma unroll
  for (int j = 0; j < kTileTok * kK / 4 / kRouteThreads; ++j) {
    const int f4 = j * kRouteThreads + threadIdx.x;          // float4 index in the tile
    const int t = f4 / (kK / 4), c = (f4 % (kK / 4)) * 4;
    const bool ok = t0 + t < a.B && k0 + c < a.d;
    const float4 v = ok ? *reinterpret_cast<const float4*>(a.x + (int64_t)(t0 + t) * a.d + k0 + c)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(&xt[t][c]) = v;
  }
  __syncthreads();
  // acc[h][4 j + t]: expert ew + 2 h + j, token t0 + t
  float acc[2][8] = {};
#pragma unroll
  for (int m = 0; m < kM; ++m) {
#pragma unroll
    for (int t = 0; t < kTileTok; ++t) {
      const float4 xv = *reinterpret_cast<const float4*>(&xt[t][256 * m + 4 * lane]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j / 2][4 * (j % 2) + t] += w[j][m].x * xv.x + w[j][m].y * xv.y + w[j][m].z * xv.z +
                                       w[j][m].w * xv.w;
    }
  }
  // two transpose-reduces: lanes 8 r .. 8 r + 7 get the totals of row r of each
  const float s0 = rows8_wave_sum(acc[0]);
  const float s1 = rows8_wave_sum(acc[1]);
  const int r = lane >> 3, t = r % kTileTok, jj = r / kTileTok;
  if ((lane & 7) == 0 && t0 + t < a.B) {
    float* dst = a.lgp + ((int64_t)ks * a.B + t0 + t) * a.E;
    if (ew + jj < a.E) dst[ew + jj] = s0;
    if (ew + 2 + jj < a.E) dst[ew + 2 + jj] = s1;
  }
}

// Top-k, one token per wave over a grid, and then (do_union) the union by
// the last block to finish, found with an integer ticket (status[2]) that it
// resets for the next call.  n_ks > 0: the logits are first formed from
// k_route_tiled's K-slice partials (added in slice order) and written out;
// else they are read as given.  The indices reach the last block through
// the memory model at device scope: the block's barrier orders its waves'
// stores before thread 0's acquire-release ticket increment (release is
// cumulative), and the last block acquires before it reads.
__global__ __launch_bounds__(kTopkThreads) void k_topk_grid(RouteArgs a, int n_ks, int do_union,
                                                           uint32_t* ticket) {
  __shared__ UnionSmem us;
  __shared__ int is_last;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kTopkThreads / 64) + wave;
  const int E = a.E, K = a.K;
  if (t < a.B) {
    float v[4];
    if (n_ks > 0) {
      // every slice's partials requested at once, then added in slice order
      // (unrolled and predicated: a loop to n_ks would index the array at
      // run time, which puts it in scratch memory)
      float p[4][kMaxSlices];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
#pragma unroll
        for (int ks = 0; ks < kMaxSlices; ++ks)
          p[j][ks] = (e < E && ks < n_ks) ? a.lgp[((int64_t)ks * a.B + t) * E + e] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        float sum = p[j][0];
#pragma unroll
        for (int ks = 1; ks < kMaxSlices; ++ks)
          if (ks < n_ks) sum += p[j][ks];
        v[j] = e < E ? sum : -FLT_MAX;
        if (e < E) a.logits[(int64_t)t * E + e] = sum;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        v[j] = e < E ? a.logits[(int64_t)t * E + e] : -FLT_MAX;
      }
    }
    float my_v;
    int my_e;
    wave_topk(v, E, K, my_v, my_e, &us.topk[wave]);
    const float w = topk_weight(v, E, K, a.norm != 0, my_v);
    if (lane < K) {
      a.topk_idx[t * K + lane] = my_e;
      a.topk_w[t * K + lane] = w;
    }
  }
  if (!do_union) return;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t n = gridDim.x;
    const uint32_t tk = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_ACQ_REL,
                                               __HIP_MEMORY_SCOPE_AGENT);
    is_last = (tk == n - 1);
    // the next launch is ordered after this one by the kernel boundary
    if (is_last) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int P = a.B * K;
  for (int p = threadIdx.x; p < P; p += blockDim.x) us.idx[p] = a.topk_idx[p];
  __syncthreads();
  build_union(a, &us);
}

// Logits only from k_route_tiled's partials (no top-k): one token per wave.
__global__ __launch_bounds__(kTopkThreads) void k_sum_slices(RouteArgs a, int n_ks) {
  const int t = blockIdx.x * (kTopkThreads / 64) + (int)(threadIdx.x >> 6);
  if (t >= a.B) return;
  for (int e = threadIdx.x & 63; e < a.E; e += 64) {
    float sum = a.lgp[(int64_t)t * a.E + e];
    for (int ks = 1; ks < n_ks; ++ks) sum += a.lgp[((int64_t)ks * a.B + t) * a.E + e];
    a.logits[(int64_t)t * a.E + e] = sum;
  }
}

// Ranked routing ("Data Flow", the routing step: ranked top-(8+spec), the
// ranks past K queued as speculative prefetch; "Surface Scout": the current
// token's lower gate ranks): one token per wave, the top R = K + spec by
// (logit descending, index ascending); lanes k < K also write the top-K
// index and weight.
__global__ __launch_bounds__(kTopkThreads) void k_topk_ranked(RouteArgs a, int R,
                                                             int32_t* ranked) {
  __shared__ TopkScratch sc[kTopkThreads / 64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kTopkThreads / 64) + wave;
  if (t >= a.B) return;                            // whole wave
  const int E = a.E, K = a.K;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? a.logits[(int64_t)t * E + e] : -FLT_MAX;
  }
  float my_v;
  int my_e;
  wave_topk(v, E, R, my_v, my_e, &sc[wave]);
  const float w = topk_weight(v, E, K, a.norm != 0, my_v);   // lanes < K only
  if (lane < K) {
    a.topk_idx[(int64_t)t * K + lane] = my_e;
    a.topk_w[(int64_t)t * K + lane] = w;
  }
  if (lane < R) ranked[(int64_t)t * R + lane] = my_e;
}

// Top-k only (logits given) and/or union only (indices given): one block.
__global__ __launch_bounds__(kTailThreads) void k_topk_union(RouteArgs a, int do_topk,
                                                             int do_union) {
  __shared__ UnionSmem us;
  route_tail(a, do_topk != 0, do_union != 0, &us);
}

// grid: one block per token
__global__ __launch_bounds__(256) void k_prep(const float* x, int d, uint16_t* xp, float2* xs,
                                              float* xa) {
  __shared__ float red[4];
  prep_token(x, d, blockIdx.x, xp, xs, xa, nullptr, 1.0f, red);
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_topk_ranked(const RouteArgs& a, int R, int32_t* ranked, hipStream_t s) {
  const int blocks = (a.B + kTopkThreads / 64 - 1) / (kTopkThreads / 64);
  hipLaunchKernelGGL(k_topk_ranked, dim3(blocks), dim3(kTopkThreads), 0, s, a, R, ranked);
  return hipGetLastError();
}

hipError_t launch_router(const RouteArgs& a, bool logits_in, bool do_topk, bool do_union,
                         hipStream_t s, const LaunchTiming* t) {
  RouteArgs r = a;
  if (!do_union) r.n_union = nullptr;
  bool tail_done = false;
  if (!logits_in && a.B > kMaxRouteTok) {
    // tiles of 4 tokens x 16 experts x one K slice (+ activation prep), then
    // the slices' sums with the top-k and union (or the sums alone)
    if (a.norm_out != nullptr) return hipErrorInvalidValue;   // the norm is fused at B <= 2 only
    const int prep_blocks = a.xp != nullptr ? a.B : 0;         // a token a block
    const int n_ks = n_slices(a.d);
    const int n_logit = ((a.E + kTileExp - 1) / kTileExp) * n_ks;
    const dim3 grid(prep_blocks + n_logit * ((a.B + kTileTok - 1) / kTileTok));
    const int pieces = slice_pieces(a.d);
#define SMOE_TILED(BF, M) SMOE_LAUNCH(t, (k_route_tiled<BF, M>), grid, dim3(kRouteThreads), 0, s, r)
    if (a.router_bf16) {
      if (pieces == 1) SMOE_TILED(true, 1);
      else if (pieces == 2) SMOE_TILED(true, 2);
      else SMOE_TILED(true, 4);
    } else {
      if (pieces == 1) SMOE_TILED(false, 1);
      else if (pieces == 2) SMOE_TILED(false, 2);
      else SMOE_TILED(false, 4);
    }
#undef SMOE_TILED
    const int blocks = (a.B + kTopkThreads / 64 - 1) / (kTopkThreads / 64);
    if (do_topk)
      hipLaunchKernelGGL(k_topk_grid, dim3(blocks), dim3(kTopkThreads), 0, s, r, n_ks,
                         (int)do_union, a.status + 2);
    else
      hipLaunchKernelGGL(k_sum_slices, dim3(blocks), dim3(kTopkThreads), 0, s, r, n_ks);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess || do_topk || !do_union) return err;
    logits_in = true;                               // only a stand-alone union is left
  }
  if (!logits_in) {
    // B <= 2: a block per token's prep (first, as they have the longer
    // chains), then a block per expert's logits; small grids finish
    // top-k/union in their last block
    const dim3 grid(a.B + a.E);
    const bool fused = (do_topk || do_union) && (int)grid.x <= kMaxTicketBlocks;
    uint32_t* ticket = a.status + 1;
    const int pieces = route_pieces(a.d);
    const size_t tail_lds = fused ? sizeof(UnionSmem) : 0;
#define SMOE_ROUTE(BF, NT, M) \
  SMOE_LAUNCH(t, (k_route<BF, NT, M>), grid, dim3(kRouteThreads), tail_lds, s, r, (int)fused, ticket)
#define SMOE_ROUTE_M(BF, NT)                  \
  do {                                        \
    if (pieces == 1) SMOE_ROUTE(BF, NT, 1);   \
    else if (pieces == 2) SMOE_ROUTE(BF, NT, 2); \
    else SMOE_ROUTE(BF, NT, 4);               \
  } while (0)
    if (a.router_bf16) {
      if (a.B == 1) SMOE_ROUTE_M(true, 1);
      else SMOE_ROUTE_M(true, 2);
    } else {
      if (a.B == 1) SMOE_ROUTE_M(false, 1);
      else SMOE_ROUTE_M(false, 2);
    }
#undef SMOE_ROUTE_M
#undef SMOE_ROUTE
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    tail_done = fused;
  }
  if (!tail_done && do_topk) {
    const int blocks = (a.B + kTopkThreads / 64 - 1) / (kTopkThreads / 64);
    hipLaunchKernelGGL(k_topk_grid, dim3(blocks), dim3(kTopkThreads), 0, s, r, 0, (int)do_union,
                       a.status + 2);
    return hipGetLastError();
  }
  if (!tail_done && do_union) {
    hipLaunchKernelGGL(k_topk_union, dim3(1), dim3(kTailThreads), 0, s, r, 0, 1);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_prep(const float* x, int B, int d, uint16_t* xp, float2* xs, float* xa,
                       hipStream_t s) {
  hipLaunchKernelGGL(k_prep, dim3(B), dim3(256), 0, s, x, d, xp, xs, xa);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_u32, dim3((n + 255) / 256), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace smoe
