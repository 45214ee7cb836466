// smoe_internal.hpp - shared declarations of libsmoe's kernels and host code.
//
// Data layouts in device memory (all row-major):
//   quantised weights  u32 [rows, cols/8], element c at bits 4*(c%8) of word
//                      c/8; bf16 scale/bias [rows, cols/64]
//                      ("SSD Streaming Expert Layers", "Quantized Layout").
//   prepped activations fp16 [rows, K]: for every 8 consecutive inputs
//                      x0..x7 (one packed weight word) the 8 halves are
//                      (x0, x4), (x1/16, x5/16), (x2, x6), (x3/16, x7/16),
//                      the pairing that the nibble-to-fp16 conversion of a
//                      word produces (see dequant_word).  Per 64-input group:
//                      X = sum of the fp16 inputs, C = 1024 * sum of the
//                      stored halves (float2 per group).
//   h (gate/up output) is stored in the same prepped layout, with its group
//                      sums as two 32-column partials per group.
//   token scales       xa [B] f32: a power of two a_t per token.  The prepped
//                      activations hold a_t * x (a_t brings the row's largest
//                      magnitude into [1, 2)), and h of a pair of token t is stored as
//                      a_t^2 * h, so that neither leaves the fp16 range when
//                      the hidden states or the weights are far from O(1).
//                      Dot products over them are rescaled by 1/a_t (gate,
//                      up) and 1/a_t^2 (down) in fp32, which is exact.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/smoe.h"

namespace smoe {

// ------------------------------------------------------------ constants
constexpr int kMaxBatch = SMOE_MAX_BATCH;
constexpr int kMaxExperts = SMOE_MAX_EXPERTS;
constexpr int kMaxTopK = SMOE_MAX_TOPK;
constexpr int kMaxPairs = kMaxBatch * kMaxTopK;

// ------------------------------------------------------------ workspace
struct WsLayout {
  size_t status;   // uint32 status word (+ padding)
  size_t logits;   // [B, E] f32
  size_t lgp;      // [<= 8 K slices, B, E] f32 partial logits (B >= 3)
  size_t xp;       // [B, d] f16 prepped activations
  size_t xs;       // [B, d/64] float2 group sums of xp
  size_t xa;       // [B] f32 token scales (powers of two)
  size_t hp;       // [P, f] f16 prepped h
  size_t hs;       // [P, f/64, 2] float2 half-group sums of hp
  size_t y;        // [P, d] f32 per-pair expert outputs
  size_t meta;     // 512 B: the decode kernels' packed routing metadata
  size_t shp;      // [B, fs] f16 prepped h of the shared expert
  size_t shs;      // [B, fs/64, 2] float2 half-group sums of shp
  size_t sy;       // [B, d] f32 shared expert output (prefill path)
  size_t total;
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline WsLayout ws_layout(const smoe_layer_desc& L, int B) {
  WsLayout w{};
  const size_t P = (size_t)B * L.top_k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  w.status = take(256);
  w.logits = take((size_t)B * L.num_experts * 4);
  w.lgp = take((size_t)8 * B * L.num_experts * 4);   // at most 8 K slices
  w.xp = take((size_t)B * L.d_model * 2);
  w.xs = take((size_t)B * (L.d_model / 64) * 8);
  w.xa = take((size_t)B * 4);
  w.hp = take(P * L.ffn_dim * 2);
  w.hs = take(P * (L.ffn_dim / 64) * 2 * 8);
  w.y = take(P * L.d_model * 4);
  w.meta = take(512);
  const size_t fs = L.shared_ffn_dim > 0 ? (size_t)L.shared_ffn_dim : 0;
  w.shp = take((size_t)B * fs * 2);
  w.shs = take((size_t)B * (fs / 64) * 2 * 8);
  w.sy = take(fs ? (size_t)B * L.d_model * 4 : 0);
  w.total = off;
  return w;
}

// ------------------------------------------------------- kernel arguments
struct QMat {
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  int64_t stride_w;
  int64_t stride_sb;
};

struct RouteArgs {
  const void* router_w;
  int router_bf16;
  const float* x;
  int B, d, E, K, norm;
  float* logits;       // read (logits_in) or written
  float* lgp;          // K-slice partial logits (workspace), B >= 3
  int32_t* topk_idx;
  float* topk_w;
  uint32_t* status;
  // prepped activations (written by the router kernel when non-null)
  uint16_t* xp;
  float2* xs;
  float* xa;
  // union outputs (built after top-k when non-null)
  int32_t* n_union;
  int32_t* union_experts;
  int32_t* expert_offsets;
  int32_t* pair_list;
  int32_t* pair_pos;
  // when non-null, x is a previous layer's raw output: the router routes
  // RMSNorm(x) (eps norm_eps) and writes it here (B <= 2, logits + prep only)
  float* norm_out;
  float norm_eps;
};

struct FfnArgs {
  QMat gate, up, down;
  int B, d, f, E, K;
  const int32_t* n_union;
  const int32_t* union_experts;
  const int32_t* expert_offsets;
  const int32_t* pair_list;
  const int32_t* pair_pos;
  const float* topk_w;
  const float* residual;
  float* out;
  const uint16_t* xp;
  const float2* xs;
  const float* xa;     // token scales a_t (see the layouts above)
  uint16_t* hp;
  float2* hs;
  float* y;
  uint32_t* status;  // workspace status area: status bits, tickets, sync counters
  // decode kernels: the call's routing metadata in one packed block (written
  // by the routed gate_up kernel; read by the down kernel when dec_meta_valid)
  int32_t* dec_meta;
  int dec_meta_valid;
  // the shared expert (fs > 0): one matrix each (expert 0, strides unused),
  // applied to every token; its h in shp/shs like hp/hs with token t as the
  // pair, its output in sy (prefill path; the decode path combines in-kernel)
  QMat sgate, sup, sdown;
  int fs;
  uint16_t* shp;
  float2* shs;
  float* sy;
};

// Routing done inside the decode gate_up kernel (smoe_moe_layer with B <= 2):
// every block ranks the logits itself and builds the union in LDS; block 0
// also writes the routing outputs.
struct DecodeRoute {
  const float* logits;     // [B, E] from the router kernel
  int norm;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* n_union;
  int32_t* union_experts;
  int32_t* expert_offsets;
  int32_t* pair_list;
  int32_t* pair_pos;
  int32_t* dec_meta;       // packed copy of the routing metadata (block 0 writes it)
};

// ------------------------------------------------------- attention block
constexpr int kAttnHeadDim = 128;   // head dimension
constexpr int kAttnMaxGroup = 16;   // query heads per key/value head
constexpr int kAttnSplit = 256;     // cached positions per attention block
constexpr int kAttnProjMinBatch = 3;  // chunks of this many tokens or more: batched projections
constexpr int kAttnProjK = 512;       // inputs per block of a batched projection (the K split)

// Workspace of the attention block for up to B tokens ([DF] layer loop).
struct AttnWsLayout {
  size_t qkv;      // [B, (H + 2 Hkv) hd] f32
  size_t part_o;   // [B, Hkv, nsplit, 16, hd] f32
  size_t part_ml;  // [B, Hkv, nsplit, 16] (max, sum) pairs
  size_t ob;       // [B, H hd] bf16: the attention output
  size_t xb;       // [B, d] bf16: the normed input (batched projections only)
  size_t ppart;    // [K splits, B, rows] f32: partial sums (batched projections only)
  size_t rope;     // [B, hd / 2] (cos, sin) of the tokens' positions (batched path only)
  size_t total;
};

inline int attn_nsplit_max(int64_t ctx) { return (int)((ctx + kAttnSplit - 1) / kAttnSplit); }

inline AttnWsLayout attn_ws_layout(const smoe_attn_desc& D, int B) {
  AttnWsLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  const size_t hd = kAttnHeadDim, H = D.num_heads, G = D.num_kv_heads;
  const size_t ns = (size_t)attn_nsplit_max(D.ctx);
  w.qkv = take((size_t)B * (H + 2 * G) * hd * 4);
  w.part_o = take((size_t)B * G * ns * kAttnMaxGroup * hd * 4);
  w.part_ml = take((size_t)B * G * ns * kAttnMaxGroup * 8);
  w.ob = take((size_t)B * H * hd * 2);
  if (B >= kAttnProjMinBatch) {
    const size_t d = (size_t)D.d_model, qkv_rows = (H + 2 * G) * hd;
    w.xb = take((size_t)B * d * 2);
    w.ppart = take((size_t)B * std::max(d / kAttnProjK * qkv_rows, H * hd / kAttnProjK * d) * 4);
    w.rope = take((size_t)B * (hd / 2) * 8);
  }
  w.total = off;
  return w;
}

struct AttnArgs {
  const float* x;          // [B, d] input hidden states (also the residual)
  float* out;              // [B, d]
  const uint16_t* wqkv;    // [(H + 2 Hkv) hd, d] bf16
  const uint16_t* wo;      // [d, H hd] bf16
  uint16_t* k_cache;       // [Hkv, ctx, hd] bf16
  uint16_t* v_cache;
  int B, d, H, Hkv, qkv_rows, nsplit;
  int tgroup;              // tokens per attention block (set by the launcher)
  int64_t pos0, ctx;
  double theta;
  float eps;
  float* qkv;
  float* part_o;
  float* part_ml;
  uint16_t* ob;
  uint16_t* xb;            // batched projections only
  float* ppart;
  float2* rope;            // batched path only: (cos, sin) per token and pair
};

// ------------------------------------------------------------- launchers
// Optional timing events for a stage's main kernel: when `start` is set the
// kernel is launched with hipExtLaunchKernelGGL, which submits the events
// together with the dispatch (no host-side gap between them).
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
#define SMOE_LAUNCH(timing, kernel, grid, block, shmem, stream, ...)                              \
  do {                                                                                           \
    if ((timing) != nullptr && (timing)->start != nullptr)                                       \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, (timing)->start, (timing)->stop, \
                            0, __VA_ARGS__);                                                     \
    else                                                                                         \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                       \
  } while (0)

// Host-side validation and set-up of one layer call (api.cpp): fills r and a
// for workspace ws; SMOE_OK or the SMOE_E* error.  Launches nothing.
int layer_setup(const smoe_layer_desc* desc, const void* router_w, const smoe_experts* experts,
                const float* x, int32_t B, const float* residual, float* out, float* logits,
                int32_t* topk_idx, float* topk_w, const smoe_union* un, void* ws, size_t ws_bytes,
                RouteArgs* r, FfnArgs* a);
// The kernels of one whole layer call set up by layer_setup, in stream order.
hipError_t launch_layer(const RouteArgs& r, const FfnArgs& a, hipStream_t s);

// Compute units of the current device (0 when the query fails).
int cu_count();

// All return hipSuccess or the launch error.
hipError_t launch_router(const RouteArgs& a, bool logits_in, bool do_topk, bool do_union,
                         hipStream_t s, const LaunchTiming* t = nullptr);
// Top R = K + spec of every token from a.logits (one token per wave): the
// top K indices and weights to a.topk_idx / a.topk_w, all R indices in rank
// order to ranked [B, R].
hipError_t launch_topk_ranked(const RouteArgs& a, int R, int32_t* ranked, hipStream_t s);
hipError_t launch_prep(const float* x, int B, int d, uint16_t* xp, float2* xs, float* xa,
                       hipStream_t s);
hipError_t launch_ffn(const FfnArgs& a, hipStream_t s);
hipError_t launch_gate_up(const FfnArgs& a, hipStream_t s, const LaunchTiming* t = nullptr);
hipError_t launch_down(const FfnArgs& a, hipStream_t s, const LaunchTiming* t = nullptr);
hipError_t launch_combine(const FfnArgs& a, hipStream_t s, const LaunchTiming* t = nullptr);
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int n, hipStream_t s);
hipError_t launch_rmsnorm(const float* v, int B, int d, float eps, float* out, hipStream_t s);
// small-batch (B <= 2) matrix-vector kernels
bool gemv_path_ok(const FfnArgs& a);
hipError_t launch_gemv(const FfnArgs& a, hipStream_t s, bool gate_up,
                       const LaunchTiming* t = nullptr);
// The decode layer (B = 1, bf16 router, no shared expert, d of 2048 or 4096)
// in one cooperative launch; single_layer_ok says whether a call qualifies.
bool single_layer_ok(const RouteArgs& ra, const FfnArgs& a);
hipError_t launch_single_layer(const RouteArgs& ra, const FfnArgs& a, const DecodeRoute& r,
                               hipStream_t s);
// gate_up with the routing tail (top-k, weights, union) folded in; the router
// kernel then only computes logits and the prepped activations
hipError_t launch_gate_up_routed(const FfnArgs& a, const DecodeRoute& r, hipStream_t s,
                                 const LaunchTiming* t = nullptr);
// attention block: stage -1 = all, 0 = norm + QKV, 1 = prep + attention +
// merge, 2 = O projection + residual (t times that stage's main kernel)
bool attn_shape_ok(int d, int H, int Hkv, int hd);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s, int stage = -1,
                       const LaunchTiming* t = nullptr);
// prefill-chunk MFMA kernels
hipError_t launch_ffn_mfma(const FfnArgs& a, hipStream_t s, bool gate_up,
                           const LaunchTiming* t = nullptr);

}  // namespace smoe
