// api.cpp - the C-ABI entry points of libsmoe (declared in include/smoe.h).
//
// Every entry point validates all arguments on the host before launching
// anything, then enqueues kernels on the caller's stream and returns without
// synchronising (smoe_read_status excepted).
#include <hip/hip_runtime.h>
#include <algorithm>

#include <cstdint>
#include <cstring>

#include "smoe_internal.hpp"

#define SMOE_API extern "C" __attribute__((visibility("default")))

namespace {

using smoe::WsLayout;

constexpr int kMaxDim = 8192;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_desc(const smoe_layer_desc* L) {
  if (L == nullptr) return SMOE_EINVAL;
  if (L->group_size != SMOE_GROUP) return SMOE_EUNSUPPORTED;
  if (L->d_model < 64 || L->d_model > kMaxDim || L->d_model % 64 != 0) return SMOE_EUNSUPPORTED;
  if (L->ffn_dim < 64 || L->ffn_dim > kMaxDim || L->ffn_dim % 64 != 0) return SMOE_EUNSUPPORTED;
  if (L->num_experts < 1 || L->num_experts > SMOE_MAX_EXPERTS) return SMOE_EUNSUPPORTED;
  if (L->top_k < 1 || L->top_k > SMOE_MAX_TOPK || L->top_k > L->num_experts)
    return SMOE_EUNSUPPORTED;
  if (L->norm_topk_prob != 0 && L->norm_topk_prob != 1) return SMOE_EINVAL;
  if (L->router_dtype != SMOE_F32 && L->router_dtype != SMOE_BF16) return SMOE_EUNSUPPORTED;
  if (L->shared_ffn_dim != 0 &&
      (L->shared_ffn_dim < 64 || L->shared_ffn_dim > kMaxDim || L->shared_ffn_dim % 64 != 0))
    return SMOE_EUNSUPPORTED;
  return SMOE_OK;
}

int check_batch(int32_t B) {
  if (B < 0) return SMOE_EINVAL;
  if (B > SMOE_MAX_BATCH) return SMOE_EUNSUPPORTED;
  return SMOE_OK;
}

int check_ws(const smoe_layer_desc* L, int32_t B, const void* ws, size_t ws_bytes) {
  if (ws == nullptr || !aligned(ws, 256)) return SMOE_EINVAL;
  if (ws_bytes < smoe::ws_layout(*L, B).total) return SMOE_EWORKSPACE;
  return SMOE_OK;
}

int check_union(const smoe_union* un) {
  if (un == nullptr || un->n_union == nullptr || un->union_experts == nullptr ||
      un->expert_offsets == nullptr || un->pair_list == nullptr || un->pair_pos == nullptr)
    return SMOE_EINVAL;
  return SMOE_OK;
}

int check_qmat(const smoe_qmat& m, int rows, int cols) {
  if (m.w == nullptr || m.s == nullptr || m.b == nullptr) return SMOE_EINVAL;
  if (!aligned(m.w, 16) || !aligned(m.s, 2) || !aligned(m.b, 2)) return SMOE_EINVAL;
  // every expert's matrix must start 16-byte aligned and not overlap the next
  if (m.expert_stride_w < (int64_t)rows * cols / 8 || (m.expert_stride_w * 4) % 16 != 0)
    return SMOE_EINVAL;
  if (m.expert_stride_sb < (int64_t)rows * cols / 64) return SMOE_EINVAL;
  return SMOE_OK;
}

int check_experts(const smoe_layer_desc* L, const smoe_experts* ex) {
  if (ex == nullptr) return SMOE_EINVAL;
  int rc = check_qmat(ex->gate, L->ffn_dim, L->d_model);
  if (rc == SMOE_OK) rc = check_qmat(ex->up, L->ffn_dim, L->d_model);
  if (rc == SMOE_OK) rc = check_qmat(ex->down, L->d_model, L->ffn_dim);
  if (rc == SMOE_OK && L->shared_ffn_dim > 0) {
    for (const smoe_qmat* m : {&ex->shared_gate, &ex->shared_up, &ex->shared_down}) {
      if (m->w == nullptr || m->s == nullptr || m->b == nullptr || !aligned(m->w, 16) ||
          !aligned(m->s, 2) || !aligned(m->b, 2))
        return SMOE_EINVAL;
    }
  }
  return rc;
}

template <class T>
T* ws_at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

smoe::QMat to_q(const smoe_qmat& m) {
  return smoe::QMat{m.w, m.s, m.b, m.expert_stride_w, m.expert_stride_sb};
}
// A single matrix (the shared expert): expert 0 only, so the strides are unused.
smoe::QMat to_q1(const smoe_qmat& m) { return smoe::QMat{m.w, m.s, m.b, 0, 0}; }

smoe::FfnArgs ffn_args(const smoe_layer_desc* L, const smoe_experts* ex, const smoe_union* un,
                       const float* topk_w, int32_t B, const float* residual, float* out, void* ws,
                       const WsLayout& lay) {
  smoe::FfnArgs a{};
  a.gate = to_q(ex->gate);
  a.up = to_q(ex->up);
  a.down = to_q(ex->down);
  a.B = B;
  a.d = L->d_model;
  a.f = L->ffn_dim;
  a.E = L->num_experts;
  a.K = L->top_k;
  a.n_union = un->n_union;
  a.union_experts = un->union_experts;
  a.expert_offsets = un->expert_offsets;
  a.pair_list = un->pair_list;
  a.pair_pos = un->pair_pos;
  a.topk_w = topk_w;
  a.residual = residual;
  a.out = out;
  a.xp = ws_at<uint16_t>(ws, lay.xp);
  a.xs = ws_at<float2>(ws, lay.xs);
  a.xa = ws_at<float>(ws, lay.xa);
  a.hp = ws_at<uint16_t>(ws, lay.hp);
  a.hs = ws_at<float2>(ws, lay.hs);
  a.y = ws_at<float>(ws, lay.y);
  a.dec_meta = ws_at<int32_t>(ws, lay.meta);
  a.dec_meta_valid = 0;
  a.status = ws_at<uint32_t>(ws, lay.status);
  a.fs = L->shared_ffn_dim;
  if (a.fs > 0) {
    a.sgate = to_q1(ex->shared_gate);
    a.sup = to_q1(ex->shared_up);
    a.sdown = to_q1(ex->shared_down);
    a.shp = ws_at<uint16_t>(ws, lay.shp);
    a.shs = ws_at<float2>(ws, lay.shs);
    a.sy = ws_at<float>(ws, lay.sy);
  }
  return a;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? SMOE_OK : SMOE_EHIP; }

}  // namespace

SMOE_API size_t smoe_workspace_size(const smoe_layer_desc* desc, int32_t max_batch) {
  if (check_desc(desc) != SMOE_OK || max_batch < 1 || max_batch > SMOE_MAX_BATCH) return 0;
  return smoe::ws_layout(*desc, max_batch).total;
}

SMOE_API int smoe_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < 256) return SMOE_EINVAL;
  return hip_rc(smoe::launch_fill_u32(static_cast<uint32_t*>(ws), 0u, 64,
                                      static_cast<hipStream_t>(stream)));
}

SMOE_API int smoe_route(const smoe_layer_desc* desc, const void* router_w, const float* x,
                        int32_t B, float* logits, int32_t* topk_idx, float* topk_w,
                        uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc == SMOE_OK) rc = check_batch(B);
  if (rc != SMOE_OK) return rc;
  if ((flags & ~SMOE_ROUTE_LOGITS_IN) != 0) return SMOE_EINVAL;
  if (B == 0) return SMOE_OK;
  const bool logits_in = (flags & SMOE_ROUTE_LOGITS_IN) != 0;
  if (topk_idx == nullptr || topk_w == nullptr) return SMOE_EINVAL;
  if (logits_in && logits == nullptr) return SMOE_EINVAL;
  if (!logits_in) {
    if (router_w == nullptr || x == nullptr || !aligned(router_w, 16) || !aligned(x, 16))
      return SMOE_EINVAL;
  }
  rc = check_ws(desc, B, ws, ws_bytes);
  if (rc != SMOE_OK) return rc;
  const WsLayout lay = smoe::ws_layout(*desc, B);
  smoe::RouteArgs a{};
  a.router_w = router_w;
  a.router_bf16 = desc->router_dtype == SMOE_BF16;
  a.x = x;
  a.B = B;
  a.d = desc->d_model;
  a.E = desc->num_experts;
  a.K = desc->top_k;
  a.norm = desc->norm_topk_prob;
  a.logits = logits ? logits : ws_at<float>(ws, lay.logits);
  a.lgp = ws_at<float>(ws, lay.lgp);
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.status = ws_at<uint32_t>(ws, lay.status);
  return hip_rc(smoe::launch_router(a, logits_in, true, false, static_cast<hipStream_t>(stream)));
}

SMOE_API int smoe_route_ranked(const smoe_layer_desc* desc, const void* router_w,
                               const float* x, int32_t B, float* logits, int32_t spec,
                               int32_t* ranked_idx, int32_t* topk_idx, float* topk_w,
                               uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc == SMOE_OK) rc = check_batch(B);
  if (rc != SMOE_OK) return rc;
  if ((flags & ~SMOE_ROUTE_LOGITS_IN) != 0) return SMOE_EINVAL;
  if (spec < 0 || desc->top_k + spec > SMOE_MAX_TOPK || desc->top_k + spec > desc->num_experts)
    return SMOE_EUNSUPPORTED;
  if (B == 0) return SMOE_OK;
  const bool logits_in = (flags & SMOE_ROUTE_LOGITS_IN) != 0;
  if (topk_idx == nullptr || topk_w == nullptr || ranked_idx == nullptr) return SMOE_EINVAL;
  if (logits_in && logits == nullptr) return SMOE_EINVAL;
  if (!logits_in) {
    if (router_w == nullptr || x == nullptr || !aligned(router_w, 16) || !aligned(x, 16))
      return SMOE_EINVAL;
  }
  rc = check_ws(desc, B, ws, ws_bytes);
  if (rc != SMOE_OK) return rc;
  const WsLayout lay = smoe::ws_layout(*desc, B);
  smoe::RouteArgs a{};
  a.router_w = router_w;
  a.router_bf16 = desc->router_dtype == SMOE_BF16;
  a.x = x;
  a.B = B;
  a.d = desc->d_model;
  a.E = desc->num_experts;
  a.K = desc->top_k;
  a.norm = desc->norm_topk_prob;
  a.logits = logits ? logits : ws_at<float>(ws, lay.logits);
  a.lgp = ws_at<float>(ws, lay.lgp);
  a.topk_idx = topk_idx;
  a.topk_w = topk_w;
  a.status = ws_at<uint32_t>(ws, lay.status);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  if (!logits_in) err = smoe::launch_router(a, false, false, false, s);   // logits only
  if (err == hipSuccess) err = smoe::launch_topk_ranked(a, desc->top_k + spec, ranked_idx, s);
  return hip_rc(err);
}

SMOE_API int smoe_build_union(const smoe_layer_desc* desc, const int32_t* topk_idx, int32_t B,
                              const smoe_union* un, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc == SMOE_OK) rc = check_batch(B);
  if (rc == SMOE_OK) rc = check_union(un);
  if (rc != SMOE_OK) return rc;
  if (topk_idx == nullptr && B > 0) return SMOE_EINVAL;
  rc = check_ws(desc, B, ws, ws_bytes);
  if (rc != SMOE_OK) return rc;
  const WsLayout lay = smoe::ws_layout(*desc, B);
  smoe::RouteArgs a{};
  a.B = B;
  a.d = desc->d_model;
  a.E = desc->num_experts;
  a.K = desc->top_k;
  a.topk_idx = const_cast<int32_t*>(topk_idx);  // read-only in union-only mode
  a.status = ws_at<uint32_t>(ws, lay.status);
  a.n_union = un->n_union;
  a.union_experts = un->union_experts;
  a.expert_offsets = un->expert_offsets;
  a.pair_list = un->pair_list;
  a.pair_pos = un->pair_pos;
  // B == 0 still writes n_union = 0 so that a later forward is a no-op
  return hip_rc(smoe::launch_router(a, true, false, true, static_cast<hipStream_t>(stream)));
}

SMOE_API int smoe_moe_forward(const smoe_layer_desc* desc, const smoe_experts* experts,
                              const float* x, const int32_t* topk_idx, const float* topk_w,
                              const smoe_union* un, int32_t B, const float* residual, float* out,
                              void* ws, size_t ws_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc == SMOE_OK) rc = check_batch(B);
  if (rc == SMOE_OK) rc = check_union(un);
  if (rc == SMOE_OK) rc = check_experts(desc, experts);
  if (rc != SMOE_OK) return rc;
  if (B == 0) return SMOE_OK;
  if (x == nullptr || topk_idx == nullptr || topk_w == nullptr || out == nullptr ||
      !aligned(x, 16) || !aligned(out, 16) || (residual != nullptr && !aligned(residual, 16)))
    return SMOE_EINVAL;
  rc = check_ws(desc, B, ws, ws_bytes);
  if (rc != SMOE_OK) return rc;
  const WsLayout lay = smoe::ws_layout(*desc, B);
  hipStream_t s = static_cast<hipStream_t>(stream);
  smoe::FfnArgs a = ffn_args(desc, experts, un, topk_w, B, residual, out, ws, lay);
  hipError_t err = smoe::launch_prep(x, B, desc->d_model, ws_at<uint16_t>(ws, lay.xp),
                                     ws_at<float2>(ws, lay.xs), ws_at<float>(ws, lay.xa), s);
  if (err != hipSuccess) return SMOE_EHIP;
  return hip_rc(smoe::launch_ffn(a, s));
}

namespace smoe {

// Validation and argument set-up shared by smoe_moe_layer, its stages and
// the no-allocation variant.
int layer_setup(const smoe_layer_desc* desc, const void* router_w, const smoe_experts* experts,
                const float* x, int32_t B, const float* residual, float* out, float* logits,
                int32_t* topk_idx, float* topk_w, const smoe_union* un, void* ws, size_t ws_bytes,
                smoe::RouteArgs* r, smoe::FfnArgs* a) {
  int rc = check_desc(desc);
  if (rc == SMOE_OK) rc = check_batch(B);
  if (rc == SMOE_OK) rc = check_union(un);
  if (rc == SMOE_OK) rc = check_experts(desc, experts);
  if (rc != SMOE_OK) return rc;
  if (B == 0) return SMOE_OK;
  if (router_w == nullptr || x == nullptr || out == nullptr || topk_idx == nullptr ||
      topk_w == nullptr || !aligned(router_w, 16) || !aligned(x, 16) || !aligned(out, 16) ||
      (residual != nullptr && !aligned(residual, 16)))
    return SMOE_EINVAL;
  rc = check_ws(desc, B, ws, ws_bytes);
  if (rc != SMOE_OK) return rc;
  const WsLayout lay = smoe::ws_layout(*desc, B);
  *r = smoe::RouteArgs{};
  r->router_w = router_w;
  r->router_bf16 = desc->router_dtype == SMOE_BF16;
  r->x = x;
  r->B = B;
  r->d = desc->d_model;
  r->E = desc->num_experts;
  r->K = desc->top_k;
  r->norm = desc->norm_topk_prob;
  r->logits = logits ? logits : ws_at<float>(ws, lay.logits);
  r->lgp = ws_at<float>(ws, lay.lgp);
  r->topk_idx = topk_idx;
  r->topk_w = topk_w;
  r->status = ws_at<uint32_t>(ws, lay.status);
  r->xp = ws_at<uint16_t>(ws, lay.xp);
  r->xs = ws_at<float2>(ws, lay.xs);
  r->xa = ws_at<float>(ws, lay.xa);
  r->n_union = un->n_union;
  r->union_experts = un->union_experts;
  r->expert_offsets = un->expert_offsets;
  r->pair_list = un->pair_list;
  r->pair_pos = un->pair_pos;
  *a = ffn_args(desc, experts, un, topk_w, B, residual, out, ws, lay);
  return SMOE_OK;
}

}  // namespace smoe

namespace {

// Decode batches (B <= 2) on the matrix-vector path: the router kernel only
// computes logits and preps the activations, the gate_up kernel ranks the
// logits and builds the union itself (see ffn_gemv.hip), then down + combine.
smoe::DecodeRoute decode_route(const smoe::RouteArgs& r) {
  smoe::DecodeRoute d{};
  d.logits = r.logits;
  d.norm = r.norm;
  d.topk_idx = r.topk_idx;
  d.topk_w = r.topk_w;
  d.n_union = r.n_union;
  d.union_experts = r.union_experts;
  d.expert_offsets = r.expert_offsets;
  d.pair_list = r.pair_list;
  d.pair_pos = r.pair_pos;
  d.dec_meta = nullptr;
  return d;
}

hipError_t launch_decode_logits(const smoe::RouteArgs& r, hipStream_t s,
                                const smoe::LaunchTiming* t = nullptr) {
  return smoe::launch_router(r, false, false, false, s, t);   // logits + activation prep
}

}  // namespace

namespace smoe {

// The kernels of one whole layer, in stream order.
hipError_t launch_layer(const smoe::RouteArgs& r, const smoe::FfnArgs& a, hipStream_t s) {
  hipError_t err;
  if (smoe::gemv_path_ok(a)) {
    // the routed gate_up kernel also packs the routing metadata for down
    smoe::DecodeRoute dr = decode_route(r);
    dr.dec_meta = a.dec_meta;
    smoe::FfnArgs ad = a;
    ad.dec_meta_valid = 1;
    err = launch_decode_logits(r, s);
    if (err == hipSuccess) err = smoe::launch_gate_up_routed(a, dr, s);
    if (err == hipSuccess) err = smoe::launch_down(ad, s);
    return err;
  }
  err = smoe::launch_router(r, false, true, true, s);
  if (err == hipSuccess) err = smoe::launch_ffn(a, s);
  return err;
}

}  // namespace smoe

using smoe::launch_layer;
using smoe::layer_setup;

SMOE_API int smoe_moe_layer(const smoe_layer_desc* desc, const void* router_w,
                            const smoe_experts* experts, const float* x, int32_t B,
                            const float* residual, float* out, float* logits, int32_t* topk_idx,
                            float* topk_w, const smoe_union* un, void* ws, size_t ws_bytes,
                            void* stream) {
  smoe::RouteArgs r;
  smoe::FfnArgs a;
  const int rc = layer_setup(desc, router_w, experts, x, B, residual, out, logits, topk_idx,
                             topk_w, un, ws, ws_bytes, &r, &a);
  if (rc != SMOE_OK || B == 0) return rc;
  return hip_rc(launch_layer(r, a, static_cast<hipStream_t>(stream)));
}

SMOE_API int smoe_moe_layer_single(const smoe_layer_desc* desc, const void* router_w,
                                   const smoe_experts* experts, const float* x, int32_t B,
                                   const float* residual, float* out, float* logits,
                                   int32_t* topk_idx, float* topk_w, const smoe_union* un,
                                   void* ws, size_t ws_bytes, void* stream) {
  smoe::RouteArgs r;
  smoe::FfnArgs a;
  const int rc = layer_setup(desc, router_w, experts, x, B, residual, out, logits, topk_idx,
                             topk_w, un, ws, ws_bytes, &r, &a);
  if (rc != SMOE_OK || B == 0) return rc;
  if (!smoe::single_layer_ok(r, a)) return SMOE_EUNSUPPORTED;
  // the same routing handoff as the three launches: block 0 of the gate_up
  // pass packs the metadata that the down pass reads
  smoe::DecodeRoute dr = decode_route(r);
  dr.dec_meta = a.dec_meta;
  a.dec_meta_valid = 1;
  return hip_rc(smoe::launch_single_layer(r, a, dr, static_cast<hipStream_t>(stream)));
}

SMOE_API int smoe_moe_layer_stage(int stage, const smoe_layer_desc* desc, const void* router_w,
                                  const smoe_experts* experts, const float* x, int32_t B,
                                  const float* residual, float* out, float* logits,
                                  int32_t* topk_idx, float* topk_w, const smoe_union* un, void* ws,
                                  size_t ws_bytes, void* stream, void* start_event,
                                  void* stop_event) {
  if (stage < SMOE_STAGE_ROUTE || stage > SMOE_STAGE_COMBINE) return SMOE_EINVAL;
  if ((start_event == nullptr) != (stop_event == nullptr)) return SMOE_EINVAL;
  smoe::RouteArgs r;
  smoe::FfnArgs a;
  const int rc = layer_setup(desc, router_w, experts, x, B, residual, out, logits, topk_idx,
                             topk_w, un, ws, ws_bytes, &r, &a);
  if (rc != SMOE_OK || B == 0) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  smoe::LaunchTiming timing;
  timing.start = static_cast<hipEvent_t>(start_event);
  timing.stop = static_cast<hipEvent_t>(stop_event);
  const smoe::LaunchTiming* t = start_event != nullptr ? &timing : nullptr;
  const bool decode = smoe::gemv_path_ok(a);
  switch (stage) {
    case SMOE_STAGE_ROUTE:
      return hip_rc(decode ? launch_decode_logits(r, s, t)
                           : smoe::launch_router(r, false, true, true, s, t));
    case SMOE_STAGE_GATE_UP:
      return hip_rc(decode ? smoe::launch_gate_up_routed(a, decode_route(r), s, t)
                           : smoe::launch_gate_up(a, s, t));
    case SMOE_STAGE_DOWN: return hip_rc(smoe::launch_down(a, s, t));
    default: return hip_rc(smoe::launch_combine(a, s, t));
  }
}

SMOE_API int smoe_rmsnorm(const float* v, int32_t B, int32_t d, float eps, float* out,
                          void* stream) {
  if (B < 0) return SMOE_EINVAL;
  if (d < 64 || d > kMaxDim || d % 64 != 0) return SMOE_EUNSUPPORTED;
  if (!(eps > 0.0f)) return SMOE_EINVAL;
  if (B == 0) return SMOE_OK;
  if (v == nullptr || out == nullptr || !aligned(v, 16) || !aligned(out, 16)) return SMOE_EINVAL;
  return hip_rc(smoe::launch_rmsnorm(v, B, d, eps, out, static_cast<hipStream_t>(stream)));
}

namespace {

// One batch of tokens through a stack (smoe_stack_forward): its arguments,
// checked once before anything is launched, and the state carried from one
// layer to the next.
struct StackRun {
  const smoe_layer_desc* desc = nullptr;
  int n_layers = 0;
  const void* const* router_w = nullptr;
  const smoe_experts* experts = nullptr;
  float* h = nullptr;
  int B = 0;
  float eps = 0.0f;
  float* tmp = nullptr;
  int32_t* topk_idx = nullptr;
  float* topk_w = nullptr;
  int32_t* n_union = nullptr;
  smoe_union un{};
  void* ws = nullptr;
  size_t ws_bytes = 0;
  // Decode-sized layers (B <= 2) leave the norm of their output to the next
  // layer's router, which forms the same factor as smoe_rmsnorm (the same
  // summation order), routes the normalised rows and writes them to h: one
  // launch fewer per layer, bit-identical results.
  bool norm_pending = false;                      // tmp holds the raw output, h is stale

  int setup(int l, smoe::RouteArgs* r, smoe::FfnArgs* a) const {
    const int64_t per_layer = (int64_t)B * desc->top_k;
    smoe_union u = un;
    if (n_union != nullptr) u.n_union = n_union + l;
    return layer_setup(desc, router_w[l], experts + l, h, B, h, tmp, nullptr,
                       topk_idx ? topk_idx + l * per_layer : nullptr,
                       topk_w ? topk_w + l * per_layer : nullptr, &u, ws, ws_bytes, r, a);
  }

  // every check of smoe_stack_forward; SMOE_OK with nothing to do when
  // n_layers or B is 0 (empty() then holds)
  int check() const {
    if (n_layers < 0 || !(eps > 0.0f)) return SMOE_EINVAL;
    int rc = check_desc(desc);
    if (rc == SMOE_OK) rc = check_batch(B);
    if (rc != SMOE_OK) return rc;
    if (empty()) return SMOE_OK;
    if (router_w == nullptr || experts == nullptr || h == nullptr || tmp == nullptr || h == tmp ||
        !aligned(h, 16) || !aligned(tmp, 16))
      return SMOE_EINVAL;
    // every layer is checked before the first launch, so a bad layer leaves h as it was
    for (int l = 0; l < n_layers; ++l) {
      smoe::RouteArgs r;
      smoe::FfnArgs a;
      rc = setup(l, &r, &a);
      if (rc != SMOE_OK) return rc;
    }
    return SMOE_OK;
  }

  bool empty() const { return n_layers == 0 || B == 0; }

  // layer l and its norm (or the norm left to layer l + 1's router)
  hipError_t launch(int l, hipStream_t s) {
    smoe::RouteArgs r;
    smoe::FfnArgs a;
    setup(l, &r, &a);
    if (norm_pending) {
      r.x = tmp;
      r.norm_out = h;
      r.norm_eps = eps;
    }
    hipError_t err = launch_layer(r, a, s);
    norm_pending = smoe::gemv_path_ok(a) && B <= 2;
    if (err == hipSuccess && !norm_pending)
      err = smoe::launch_rmsnorm(tmp, B, desc->d_model, eps, h, s);
    return err;
  }

  // the last layer's norm, when it was left to a next layer
  hipError_t finish(hipStream_t s) {
    if (!norm_pending) return hipSuccess;
    norm_pending = false;
    return smoe::launch_rmsnorm(tmp, B, desc->d_model, eps, h, s);
  }
};

// The ordering events of smoe_stack_forward_chunks, kept per host thread and
// device (created on first use, never destroyed; no device memory).
hipError_t chunk_event(int slot, hipEvent_t* ev) {
  constexpr int kDevs = 64;
  thread_local hipEvent_t cache[kDevs][SMOE_MAX_STACK_CHUNKS + 1] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kDevs) return hipErrorInvalidDevice;
  if (cache[dev][slot] == nullptr) {
    err = hipEventCreateWithFlags(&cache[dev][slot], hipEventDisableTiming);
    if (err != hipSuccess) {
      cache[dev][slot] = nullptr;
      return err;
    }
  }
  *ev = cache[dev][slot];
  return hipSuccess;
}

}  // namespace

SMOE_API int smoe_stack_forward(const smoe_layer_desc* desc, int32_t n_layers,
                                const void* const* router_w, const smoe_experts* experts,
                                float* h, int32_t B, float eps, float* tmp, int32_t* topk_idx,
                                float* topk_w, int32_t* n_union, const smoe_union* un, void* ws,
                                size_t ws_bytes, void* stream) {
  if (un == nullptr) return SMOE_EINVAL;
  StackRun run;
  run.desc = desc;
  run.n_layers = n_layers;
  run.router_w = router_w;
  run.experts = experts;
  run.h = h;
  run.B = B;
  run.eps = eps;
  run.tmp = tmp;
  run.topk_idx = topk_idx;
  run.topk_w = topk_w;
  run.n_union = n_union;
  run.un = *un;
  run.ws = ws;
  run.ws_bytes = ws_bytes;
  const int rc = run.check();
  if (rc != SMOE_OK || run.empty()) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int l = 0; l < n_layers; ++l)
    if (run.launch(l, s) != hipSuccess) return SMOE_EHIP;
  return hip_rc(run.finish(s));
}

SMOE_API int smoe_stack_forward_chunks(const smoe_layer_desc* desc, int32_t n_layers,
                                       const void* const* router_w, const smoe_experts* experts,
                                       float eps, const smoe_stack_chunk* chunks,
                                       int32_t n_chunks) {
  if (chunks == nullptr || n_chunks < 1 || n_chunks > SMOE_MAX_STACK_CHUNKS) return SMOE_EINVAL;
  StackRun run[SMOE_MAX_STACK_CHUNKS];
  hipStream_t st[SMOE_MAX_STACK_CHUNKS];
  int n = 0;                                       // chunks with work, in order
  for (int i = 0; i < n_chunks; ++i) {
    const smoe_stack_chunk& c = chunks[i];
    StackRun& q = run[n];
    q.desc = desc;
    q.n_layers = n_layers;
    q.router_w = router_w;
    q.experts = experts;
    q.h = c.h;
    q.B = c.B;
    q.eps = eps;
    q.tmp = c.tmp;
    q.topk_idx = c.topk_idx;
    q.topk_w = c.topk_w;
    q.n_union = c.n_union;
    q.un = c.un;
    q.ws = c.ws;
    q.ws_bytes = c.ws_bytes;
    const int rc = q.check();
    if (rc != SMOE_OK) return rc;
    // nothing a chunk writes may be another chunk's
    for (int j = 0; j < n; ++j) {
      const StackRun& o = run[j];
      const void* mine[] = {q.h, q.tmp, q.topk_idx, q.topk_w, q.n_union, q.un.n_union,
                            q.un.union_experts, q.un.expert_offsets, q.un.pair_list,
                            q.un.pair_pos, q.ws};
      const void* theirs[] = {o.h, o.tmp, o.topk_idx, o.topk_w, o.n_union, o.un.n_union,
                              o.un.union_experts, o.un.expert_offsets, o.un.pair_list,
                              o.un.pair_pos, o.ws};
      for (const void* a : mine)
        for (const void* b : theirs)
          if (a != nullptr && a == b) return SMOE_EINVAL;
    }
    if (!q.empty()) st[n++] = static_cast<hipStream_t>(c.stream);
  }
  if (n == 0) return SMOE_OK;
  hipEvent_t ev[SMOE_MAX_STACK_CHUNKS + 1];
  for (int i = 0; i <= n; ++i)
    if (chunk_event(i, &ev[i]) != hipSuccess) return SMOE_EHIP;
  // fork: every stream after the work already queued on the first
  hipError_t err = hipSuccess;
  if (n > 1) err = hipEventRecord(ev[n], st[0]);
  for (int i = 1; i < n && err == hipSuccess; ++i) err = hipStreamWaitEvent(st[i], ev[n], 0);
  // Step t issues layer t - i of chunk i.  Chunks are issued last to first,
  // so that chunk i waits on ev[i - 1] as recorded after chunk i - 1's same
  // layer (one step earlier), before chunk i - 1 records it again.
  for (int t = 0; t < n_layers + n - 1 && err == hipSuccess; ++t) {
    for (int i = n - 1; i >= 0 && err == hipSuccess; --i) {
      const int l = t - i;
      if (l < 0 || l >= n_layers) continue;
      if (i > 0) err = hipStreamWaitEvent(st[i], ev[i - 1], 0);
      if (err == hipSuccess) err = run[i].launch(l, st[i]);
      if (err == hipSuccess && i + 1 < n) err = hipEventRecord(ev[i], st[i]);
    }
  }
  // join: the first stream after every chunk's last launch
  for (int i = 0; i < n && err == hipSuccess; ++i) err = run[i].finish(st[i]);
  for (int i = 1; i < n && err == hipSuccess; ++i) {
    err = hipEventRecord(ev[i], st[i]);
    if (err == hipSuccess) err = hipStreamWaitEvent(st[0], ev[i], 0);
  }
  return hip_rc(err);
}

namespace {

int check_attn(const smoe_attn_desc* D) {
  if (D == nullptr) return SMOE_EINVAL;
  if (!(D->rope_theta > 0.0) || !(D->eps > 0.0f) || D->reserved != 0) return SMOE_EINVAL;
  if (!smoe::attn_shape_ok(D->d_model, D->num_heads, D->num_kv_heads, D->head_dim))
    return SMOE_EUNSUPPORTED;
  if (D->ctx < 1 || D->ctx > (int64_t)1 << 22) return SMOE_EUNSUPPORTED;
  return SMOE_OK;
}

int attn_setup(const smoe_attn_desc* D, const uint16_t* wqkv, const uint16_t* wo, const float* x,
               int32_t B, int64_t pos0, uint16_t* k_cache, uint16_t* v_cache, float* out,
               void* ws, size_t ws_bytes, smoe::AttnArgs* a) {
  int rc = check_attn(D);
  if (rc == SMOE_OK) rc = check_batch(B);
  if (rc != SMOE_OK) return rc;
  if (B > D->ctx) return SMOE_EUNSUPPORTED;
  if (pos0 < 0) return SMOE_EINVAL;
  if (B == 0) return SMOE_OK;
  for (const void* p : {(const void*)wqkv, (const void*)wo, (const void*)x, (const void*)out,
                        (const void*)k_cache, (const void*)v_cache})
    if (p == nullptr || !aligned(p, 16)) return SMOE_EINVAL;
  if (ws == nullptr || !aligned(ws, 256)) return SMOE_EINVAL;
  const smoe::AttnWsLayout lay = smoe::attn_ws_layout(*D, B);
  if (ws_bytes < lay.total) return SMOE_EWORKSPACE;
  *a = smoe::AttnArgs{};
  a->x = x;
  a->out = out;
  a->wqkv = wqkv;
  a->wo = wo;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->B = B;
  a->d = D->d_model;
  a->H = D->num_heads;
  a->Hkv = D->num_kv_heads;
  a->qkv_rows = (D->num_heads + 2 * D->num_kv_heads) * smoe::kAttnHeadDim;
  a->pos0 = pos0;
  a->ctx = D->ctx;
  const int64_t p_last = pos0 + B - 1;
  const int64_t window = p_last + 1 < D->ctx ? p_last + 1 : D->ctx;
  a->nsplit = (int)((window + smoe::kAttnSplit - 1) / smoe::kAttnSplit);
  a->theta = D->rope_theta;
  a->eps = D->eps;
  a->qkv = ws_at<float>(ws, lay.qkv);
  a->part_o = ws_at<float>(ws, lay.part_o);
  a->part_ml = ws_at<float>(ws, lay.part_ml);
  a->ob = ws_at<uint16_t>(ws, lay.ob);
  a->xb = B >= smoe::kAttnProjMinBatch ? ws_at<uint16_t>(ws, lay.xb) : nullptr;
  a->ppart = B >= smoe::kAttnProjMinBatch ? ws_at<float>(ws, lay.ppart) : nullptr;
  a->rope = B >= smoe::kAttnProjMinBatch ? ws_at<float2>(ws, lay.rope) : nullptr;
  return SMOE_OK;
}

}  // namespace

SMOE_API size_t smoe_attn_workspace_size(const smoe_attn_desc* desc, int32_t max_batch) {
  if (check_attn(desc) != SMOE_OK || max_batch < 1 || max_batch > SMOE_MAX_BATCH) return 0;
  return smoe::attn_ws_layout(*desc, max_batch).total;
}

SMOE_API int smoe_attn_forward(const smoe_attn_desc* desc, const uint16_t* wqkv,
                               const uint16_t* wo, const float* x, int32_t B, int64_t pos0,
                               uint16_t* k_cache, uint16_t* v_cache, float* out, void* ws,
                               size_t ws_bytes, void* stream) {
  smoe::AttnArgs a;
  const int rc = attn_setup(desc, wqkv, wo, x, B, pos0, k_cache, v_cache, out, ws, ws_bytes, &a);
  if (rc != SMOE_OK || B == 0) return rc;
  return hip_rc(smoe::launch_attn(a, static_cast<hipStream_t>(stream)));
}

SMOE_API int smoe_attn_forward_stage(int stage, const smoe_attn_desc* desc, const uint16_t* wqkv,
                                     const uint16_t* wo, const float* x, int32_t B, int64_t pos0,
                                     uint16_t* k_cache, uint16_t* v_cache, float* out, void* ws,
                                     size_t ws_bytes, void* stream, void* start_event,
                                     void* stop_event) {
  if (stage < 0 || stage > 2) return SMOE_EINVAL;
  if ((start_event == nullptr) != (stop_event == nullptr)) return SMOE_EINVAL;
  smoe::AttnArgs a;
  const int rc = attn_setup(desc, wqkv, wo, x, B, pos0, k_cache, v_cache, out, ws, ws_bytes, &a);
  if (rc != SMOE_OK || B == 0) return rc;
  smoe::LaunchTiming timing;
  timing.start = static_cast<hipEvent_t>(start_event);
  timing.stop = static_cast<hipEvent_t>(stop_event);
  return hip_rc(smoe::launch_attn(a, static_cast<hipStream_t>(stream), stage,
                                  start_event != nullptr ? &timing : nullptr));
}

SMOE_API int smoe_read_status(const void* ws, size_t ws_bytes, void* stream,
                              uint32_t* status_out) {
  if (ws == nullptr || ws_bytes < 256 || status_out == nullptr) return SMOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(s) != hipSuccess) return SMOE_EHIP;
  uint32_t v = 0;
  if (hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return SMOE_EHIP;
  *status_out = v;
  return SMOE_OK;
}

SMOE_API const char* smoe_strerror(int code) {
  switch (code) {
    case SMOE_OK: return "success";
    case SMOE_EINVAL: return "invalid argument (null or misaligned pointer, bad flag or batch)";
    case SMOE_EUNSUPPORTED: return "unsupported shape or dtype";
    case SMOE_EWORKSPACE: return "workspace too small";
    case SMOE_EHIP: return "HIP runtime or kernel launch error";
    default: return "unknown error code";
  }
}
