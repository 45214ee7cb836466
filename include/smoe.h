/*
 * smoe.h - C-ABI of libsmoe: one routed mixture-of-experts layer on an
 * AMD Instinct MI355X (gfx950), every expert resident in device memory.
 *
 * The layer (the pages it follows are named in brackets):
 *   [LMP] "Layer-Major Batched Prefill" (S-MoE internals docs)
 *   [DF]  "Data Flow" (S-MoE architecture docs)
 *   [SSD] "SSD Streaming Expert Layers" (edge0 streaming.md)
 *   [SC]  "Surface Scout" (S-MoE architecture docs)
 *
 *   1. exact routing: router gate matvec on the true hidden state, softmax,
 *      top-k, norm_topk_prob renormalisation ([DF] serial step "EXACT
 *      ROUTING"; [LMP] "Choreography Per Chunk" step 5; [SC] model config);
 *   2. the layer-major inversion: the batch's experts deduplicated into a
 *      union, each with the list of (token, rank) pairs routed to it
 *      ([LMP] "The Inversion");
 *   3. the token-batch fused SwiGLU expert FFN down(silu(gate x) * up x) over
 *      4-bit affine weights, each union expert's bytes streamed once for all
 *      of its pairs ([LMP] step 6; [SSD] "Math Contract", "Quantized Layout");
 *   4. the weighted combine into the residual, in fixed rank order
 *      ([DF] "gather GPU outputs x routing weights", "residual += ...").
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless a comment says "host".  The
 *     descriptor structs themselves are host memory, read during the call.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise, except smoe_read_status.
 *   - The caller owns every buffer: weights, activations, outputs, union
 *     lists and the workspace.  The library allocates nothing and never
 *     frees caller memory; apart from the device scratch array of
 *     smoe_moe_layer_noalloc (below), it keeps no state between calls.
 *   - Return 0 on success or a negative SMOE_E* code.  Every argument check
 *     happens before anything is launched, so a failed call has no effect.
 *   - Pair p = t*top_k + k is token t's rank-k expert.
 *   - Calls sharing one workspace must be ordered on one stream.
 */
#ifndef SMOE_H
#define SMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ----------------------------------------------------------- error codes */
#define SMOE_OK 0
#define SMOE_EINVAL -1        /* null or misaligned pointer, B < 0, bad flag */
#define SMOE_EUNSUPPORTED -2  /* shape outside the supported range (below) */
#define SMOE_EWORKSPACE -3    /* workspace too small */
#define SMOE_EHIP -4          /* a HIP runtime call or kernel launch failed */

/* ------------------------------------------------------------ constants */
#define SMOE_F32 0            /* router gate element type: fp32 */
#define SMOE_BF16 1           /* router gate element type: bf16 bit patterns */
#define SMOE_MAX_BATCH 64     /* tokens per call (a prefill chunk, [DF] Regime 1) */
#define SMOE_MAX_EXPERTS 256
#define SMOE_MAX_TOPK 16
#define SMOE_GROUP 64         /* quantisation group size along the input axis */

/* smoe_route flags */
#define SMOE_ROUTE_LOGITS_IN 0x1u /* read logits from `logits` instead of computing them */

/* Device status bits, accumulated in the workspace until cleared. */
#define SMOE_STATUS_BAD_EXPERT 0x1u /* an expert id outside [0, E) was given; its pair is skipped */
#define SMOE_STATUS_SYNC_TIMEOUT 0x2u /* smoe_moe_layer_single: a device-wide barrier gave up waiting */

/* ----------------------------------------------------------- descriptors */
/* Supported: d_model and ffn_dim multiples of 64 in [64, 8192];
 * 1 <= num_experts <= 256; 1 <= top_k <= min(num_experts, 16);
 * group_size == 64; router_dtype SMOE_F32 or SMOE_BF16;
 * shared_ffn_dim 0 or a multiple of 64 in [64, 8192]. */
typedef struct smoe_layer_desc {
  int32_t d_model;
  int32_t ffn_dim;
  int32_t num_experts;
  int32_t top_k;
  int32_t group_size;     /* must be 64 */
  int32_t norm_topk_prob; /* 1: top-k weights renormalised to sum 1; 0: raw softmax */
  int32_t router_dtype;   /* SMOE_F32 or SMOE_BF16 */
  /* Width of the layer's shared expert, 0 for none ([DF] layer flow: a
   * shared expert FFN beside the routed ones, giving shared_out; [SC] model
   * config, shared expert width, 0 = none).  With one, every layer call
   * adds it:  out = residual + (shared_out + routed_out). */
  int32_t shared_ffn_dim;
} smoe_layer_desc;

/* One quantised projection of every expert ([SSD] "Quantized Layout"):
 * expert e's matrix [rows, cols] is w + e*expert_stride_w (u32 words,
 * row-major [rows, cols/8]; element c of a row is bits 4*(c%8)..+3 of word
 * c/8) with per-group bf16 scale s and bias b at s/b + e*expert_stride_sb
 * ([rows, cols/64]); the weight is s*q + b.  Strides are in elements.
 * w, s and b must be 16-byte aligned; with 4 KiB alignment or better, rows
 * keep their 16-byte alignment for every supported shape. */
typedef struct smoe_qmat {
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  int64_t expert_stride_w;
  int64_t expert_stride_sb;
} smoe_qmat;

/* gate and up are [ffn_dim, d_model] per expert, down is [d_model, ffn_dim].
 * The fused gate_up layout of [SSD] ("gate rows on top, up rows below",
 * [E, 2*ffn_dim, d_model/8]) is expressed as gate.w = gu,
 * up.w = gu + ffn_dim*d_model/8, both with expert_stride_w = 2*ffn_dim*d_model/8
 * (and likewise for s and b). */
typedef struct smoe_experts {
  smoe_qmat gate;
  smoe_qmat up;
  smoe_qmat down;
  /* The shared expert, read only when desc->shared_ffn_dim = fs > 0 ([SC]
   * weight inventory: the shared expert of architectures that have one):
   * one always-active SwiGLU expert applied to every token, in the same
   * format with a single matrix each (expert strides ignored): gate and up
   * [fs, d_model], down [d_model, fs]; fused as above with ffn_dim -> fs. */
  smoe_qmat shared_gate;
  smoe_qmat shared_up;
  smoe_qmat shared_down;
} smoe_experts;

/* The layer-major inversion ([LMP] "The Inversion"), all int32 device arrays:
 *   n_union[1]                 number of distinct experts routed to;
 *   union_experts[min(E,B*K)]  those experts, ascending;
 *   expert_offsets[min(E,B*K)+1]  union expert u owns
 *                              pair_list[expert_offsets[u] .. expert_offsets[u+1]);
 *   pair_list[B*K]             pairs grouped by union expert, ascending within;
 *   pair_pos[B*K]              position of pair p in pair_list (-1: skipped). */
typedef struct smoe_union {
  int32_t* n_union;
  int32_t* union_experts;
  int32_t* expert_offsets;
  int32_t* pair_list;
  int32_t* pair_pos;
} smoe_union;

/* ------------------------------------------------------------ workspace */
/* Bytes of device workspace needed for calls with up to max_batch tokens
 * (1..64).  0 when the descriptor is unsupported.  Host only. */
size_t smoe_workspace_size(const smoe_layer_desc* desc, int32_t max_batch);

/* Clears the workspace's status word.  Call once after allocating a
 * workspace; afterwards the library keeps it consistent.  Async on stream. */
int smoe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------- routing */
/* Exact routing of B tokens ([DF] "EXACT ROUTING: gate matvec on
 * heavy_normed -> ranked top-k", "norm_topk_prob weights"):
 *   logits[t,e] = sum_i Wr[e,i] * x[t,i]     (fp32 accumulation)
 *   topk_idx[t,:] = the top_k experts by (logit descending, index ascending)
 *   topk_w[t,k]   = softmax weight of topk_idx[t,k], renormalised over the
 *                   top_k when norm_topk_prob.
 * router_w: [E, d] fp32 or bf16 per desc->router_dtype.  x: [B, d] fp32.
 * logits: [B, E] fp32; nullable unless SMOE_ROUTE_LOGITS_IN; when given
 * without the flag it receives the logits.  With SMOE_ROUTE_LOGITS_IN the
 * logits are read from it and router_w/x may be NULL (top-k stage only).
 * topk_idx [B, top_k] int32, topk_w [B, top_k] fp32: outputs, rank order.
 * B == 0 is a no-op. */
int smoe_route(const smoe_layer_desc* desc, const void* router_w, const float* x, int32_t B,
               float* logits, int32_t* topk_idx, float* topk_w, uint32_t flags, void* ws,
               size_t ws_bytes, void* stream);

/* Ranked routing: smoe_route, plus each token's R = top_k + spec
 * highest-ranked experts in rank order ([DF], the routing step: ranked
 * top-(8+spec), ranks 8 and up queued as speculative prefetch for the next
 * token; [SC]: prefetch of the current token's lower gate ranks, --spec N).
 * ranked_idx: [B, R] int32, rank order by (logit descending, index
 * ascending); ranked_idx[t, :top_k] equals topk_idx[t, :].  The weights
 * cover the top_k only.  0 <= spec and R <= min(SMOE_MAX_TOPK, E), else
 * SMOE_EUNSUPPORTED; the other arguments and errors as smoe_route.
 * B == 0 is a no-op. */
int smoe_route_ranked(const smoe_layer_desc* desc, const void* router_w, const float* x,
                      int32_t B, float* logits, int32_t spec, int32_t* ranked_idx,
                      int32_t* topk_idx, float* topk_w, uint32_t flags, void* ws, size_t ws_bytes,
                      void* stream);

/* Builds the union and the pair lists from topk_idx [B, top_k] on the
 * device, with no host synchronisation ([LMP] "dedupe -> expert UNION").
 * Ids outside [0, E) set SMOE_STATUS_BAD_EXPERT and their pairs are left
 * out (pair_pos = -1). */
int smoe_build_union(const smoe_layer_desc* desc, const int32_t* topk_idx, int32_t B,
                     const smoe_union* un, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------- expert FFN */
/* The token-batch fused expert FFN and the combine ([LMP] step 6; [SSD]
 * "Math Contract"; [DF] "residual += shared_out + routed_out"):
 *   for every union expert e and every pair p = (t, k) in its list:
 *     h_p = silu(Wg_e x_t) * (Wu_e x_t),   y_p = Wd_e h_p
 *   out[t] = residual[t] + (w[t,0] y_(t,0) + w[t,1] y_(t,1) + ...), k ascending.
 * Each union expert's weights are read once for all of its pairs.
 * x: [B, d] fp32; topk_idx/topk_w as produced by smoe_route (or injected);
 * un: as produced by smoe_build_union for the same topk_idx;
 * residual: [B, d] fp32 or NULL (zero); out: [B, d] fp32, may alias residual.
 * Activations enter the dot products as fp16 and the gate/up output h is kept
 * as fp16; every sum and the scale/bias arithmetic are fp32. */
int smoe_moe_forward(const smoe_layer_desc* desc, const smoe_experts* experts, const float* x,
                     const int32_t* topk_idx, const float* topk_w, const smoe_union* un,
                     int32_t B, const float* residual, float* out, void* ws, size_t ws_bytes,
                     void* stream);

/* The whole layer in one call: smoe_route + smoe_build_union +
 * smoe_moe_forward with shared launches.  topk_idx, topk_w and un are
 * written as by those calls; logits (nullable) receives the logits. */
int smoe_moe_layer(const smoe_layer_desc* desc, const void* router_w, const smoe_experts* experts,
                   const float* x, int32_t B, const float* residual, float* out, float* logits,
                   int32_t* topk_idx, float* topk_w, const smoe_union* un, void* ws,
                   size_t ws_bytes, void* stream);

/* smoe_moe_layer as ONE cooperative launch ([DF] serial step trace: a
 * step's routing, experts and combine submitted as one unit; [LMP]
 * "Choreography Per Chunk" steps 5-6 at B = 1).  The same work in one grid
 * of one workgroup per compute unit: the token's activation prep and every
 * expert's gate matvec, a device-wide barrier, top-k + union + gate_up, a
 * second barrier, down + the weighted combine.  At each barrier every
 * workgroup releases its waves' stores and acquires with one increment at
 * device scope (after its own barrier); a wait that passes about
 * 2^22 polls sets SMOE_STATUS_SYNC_TIMEOUT in the workspace status and goes
 * on, so the launch always ends.  Results are bit for bit those of
 * smoe_moe_layer on the same inputs.  Supported: B = 1, a bf16 router, no
 * shared expert, d_model 2048 or 4096, the decode path's ffn_dim and top_k
 * (top_k <= 16); else SMOE_EUNSUPPORTED (nothing launched).  The runtime
 * refuses the launch (SMOE_EHIP) when the grid cannot be resident at once.
 * Not for HIP graph capture: use smoe_moe_layer there.  On this part it is
 * slower than smoe_moe_layer's three launches: a device-wide barrier costs
 * several launch boundaries (the calibrations in bench.py measure both).
 * Arguments, outputs and other errors as smoe_moe_layer. */
int smoe_moe_layer_single(const smoe_layer_desc* desc, const void* router_w,
                          const smoe_experts* experts, const float* x, int32_t B,
                          const float* residual, float* out, float* logits, int32_t* topk_idx,
                          float* topk_w, const smoe_union* un, void* ws, size_t ws_bytes,
                          void* stream);

/* smoe_moe_layer without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The
 * arguments and results are those of smoe_moe_layer with ws/ws_bytes left
 * out; the kernels are the same, so the outputs are bit for bit those of
 * smoe_moe_layer on the same inputs.
 * The scratch (status word, logits, prepped activations, h, per-pair
 * outputs) is a device array of the library's own, smoe_noalloc_scratch_bytes()
 * = 16 MiB, which every GPU the library runs on holds until the process
 * ends; its address is taken on a device's first call, which also clears
 * its status area with a kernel on `stream`.  A call needing more scratch
 * than that (smoe_workspace_size(desc, B) > 16 MiB: e.g. d_model 8192 with
 * ffn_dim 8192 at 64 tokens) returns SMOE_EWORKSPACE and launches nothing.
 * Every call on one GPU shares that GPU's array and it keeps the last call's
 * contents: calls that may overlap on one GPU (two streams, or host threads
 * without ordering) race; calls ordered on one stream do not.  Invalid
 * expert ids are skipped as in smoe_moe_layer; their status bit is not
 * reported by this entry point.  Other errors as smoe_moe_layer. */
int smoe_moe_layer_noalloc(const smoe_layer_desc* desc, const void* router_w,
                           const smoe_experts* experts, const float* x, int32_t B,
                           const float* residual, float* out, float* logits, int32_t* topk_idx,
                           float* topk_w, const smoe_union* un, void* stream);

/* Bytes of the device scratch smoe_moe_layer_noalloc uses (host only). */
size_t smoe_noalloc_scratch_bytes(void);

/* Diagnostic: enqueue one stage of smoe_moe_layer, so that a caller can time
 * each one.  Same arguments as smoe_moe_layer, plus two optional hipEvent_t
 * handles (both NULL, or both created with timing enabled): when given, the
 * stage's main kernel (k_route, the gate_up kernel, the down kernel or
 * k_combine) is launched together with start_event and stop_event in one
 * submission (hipExtLaunchKernelGGL), so no host-side gap falls between
 * them; the pair still includes the runtime's own marker overhead of a few
 * microseconds.  Enqueuing
 * SMOE_STAGE_ROUTE, _GATE_UP, _DOWN and _COMBINE in this order on one stream
 * launches exactly the kernels of one smoe_moe_layer call, in the same order.
 * For decode batches (B <= 2 with B * top_k <= 16: the matrix-vector path,
 * at every d_model, ffn_dim and shared_ffn_dim the descriptor allows) the
 * ROUTE stage only
 * computes the logits; the ranking, weights, union and activation prep run
 * at the start of the GATE_UP stage's kernel, and COMBINE is part of DOWN.
 * SMOE_EINVAL when only one event is given. */
#define SMOE_STAGE_ROUTE 0    /* logits + activation prep, top-k + union */
#define SMOE_STAGE_GATE_UP 1  /* gate/up projections and SwiGLU for every union expert */
#define SMOE_STAGE_DOWN 2     /* down projection for every union expert */
#define SMOE_STAGE_COMBINE 3  /* weighted combine into the residual */
int smoe_moe_layer_stage(int stage, const smoe_layer_desc* desc, const void* router_w,
                         const smoe_experts* experts, const float* x, int32_t B,
                         const float* residual, float* out, float* logits, int32_t* topk_idx,
                         float* topk_w, const smoe_union* un, void* ws, size_t ws_bytes,
                         void* stream, void* start_event, void* stop_event);

/* ----------------------------------------------------- attention block */
/* The attention block around the routed layer ([DF] layer loop: RMS norm,
 * Q/K/V projections as bf16 matrix-vector products, per-head QK-RMSNorm,
 * RoPE, K/V append into the layer's KV ring, causal GQA attention, O
 * projection, residual; [LMP] "Choreography Per Chunk" steps 1-4; [SC] the
 * model config and "KV-Cache").  For B tokens at positions pos0 .. pos0+B-1:
 *   xn = bf16(RMSNorm(x))                      unit gain, eps, fp32;
 *   [q; k; v] = Wqkv xn                        fp32 accumulation;
 *   q_h, k_g <- RMSNorm (unit gain, eps) of each head, then RoPE at the
 *     token's position p: pair (i, i + hd/2) rotated by p * rope_theta^(-2i/hd);
 *   K[g, p mod ctx] = bf16(k_g), V[g, p mod ctx] = bf16(v_g)   (all B first);
 *   o_h = softmax_j(q_h . K[g, j] / sqrt(hd)) V[g, j], g = h / (H / Hkv),
 *     over the cached positions j <= p that the ring holds after the call
 *     (p_last - ctx + 1 .. p_last);
 *   out = x + Wo bf16(o).
 * Supported: head_dim 128; H % Hkv == 0 with H / Hkv <= 16; d_model and
 * num_heads * 128 each one of 512, 1024, 2048, 4096, 8192; 1 <= ctx <= 2^22
 * and B <= min(ctx, 64); else SMOE_EUNSUPPORTED. */
typedef struct smoe_attn_desc {
  double rope_theta;      /* e.g. 1e6; > 0 */
  int64_t ctx;            /* KV ring slots per layer */
  int32_t d_model;
  int32_t num_heads;      /* query heads H */
  int32_t num_kv_heads;   /* key/value heads Hkv */
  int32_t head_dim;       /* must be 128 */
  float eps;              /* RMS norm epsilon, > 0 */
  int32_t reserved;       /* 0 */
} smoe_attn_desc;

/* Bytes of device workspace for calls of up to max_batch (1..64) tokens; 0
 * when the descriptor is unsupported.  Host only.  From 3 tokens on it also
 * holds the batched projections' bf16 inputs and fp32 partial sums (one set
 * per 512-input slice: at d_model 4096 with 64 + 2 x 4 heads, about 19 MB for
 * 64 tokens). */
size_t smoe_attn_workspace_size(const smoe_attn_desc* desc, int32_t max_batch);

/* One call of the block (a decode step, B <= 2, which runs matrix-vector
 * projections, or a chunk of B = 3..64 tokens, whose projections read each
 * weight matrix once for all of its tokens):
 *   wqkv  [(H + 2 Hkv) 128, d_model] bf16 bits, rows of q, then k, then v;
 *   wo    [d_model, H 128] bf16 bits;
 *   x     [B, d_model] f32; out [B, d_model] f32 (out may be x);
 *   k_cache, v_cache  [Hkv, ctx, 128] bf16 bits, updated in place; slots not
 *         written by this call must hold the K/V of the positions the ring
 *         covers (pos0 - ctx + B .. pos0 - 1, where >= 0).
 * Pointers are device pointers, 16-byte aligned; pos0 >= 0.  Errors as
 * smoe_route; B == 0 is a no-op. */
int smoe_attn_forward(const smoe_attn_desc* desc, const uint16_t* wqkv, const uint16_t* wo,
                      const float* x, int32_t B, int64_t pos0, uint16_t* k_cache,
                      uint16_t* v_cache, float* out, void* ws, size_t ws_bytes, void* stream);

/* Diagnostic: one stage of smoe_attn_forward (0: norm + QKV projection;
 * 1: QK-norm, RoPE, K/V append, attention; 2: O projection + residual), for
 * per-kernel timing; the event pair (hipEvent_t, both or neither) brackets
 * that stage's main kernel. */
int smoe_attn_forward_stage(int stage, const smoe_attn_desc* desc, const uint16_t* wqkv,
                            const uint16_t* wo, const float* x, int32_t B, int64_t pos0,
                            uint16_t* k_cache, uint16_t* v_cache, float* out, void* ws,
                            size_t ws_bytes, void* stream, void* start_event, void* stop_event);

/* ----------------------------------------------------- between layers */
/* The norm between stacked layers, h <- RMSNorm(h + MoE(h)): run
 * smoe_moe_layer with residual = h, then this on its output.  The backbone
 * keeps an RMS norm before attention and one before the FFN of every layer
 * ([SC] weight inventory, "layer norms"); with attention left out the two
 * meet between the MoE blocks.  Unit gain here:
 *   out[t,:] = v[t,:] / sqrt(mean_i v[t,i]^2 + eps)     (fp32)
 * v, out: [B, d] fp32, 16-byte aligned; out may equal v (in place).
 * d: multiple of 64 in [64, 8192]; eps > 0; B >= 0 (0 is a no-op).
 * Async on stream. */
int smoe_rmsnorm(const float* v, int32_t B, int32_t d, float eps, float* out, void* stream);

/* B tokens through a stack of n_layers routed layers of one shape, each
 * followed by the norm (the per-layer loop of [DF]'s serial step trace with
 * attention left out):
 *   for l = 0 .. n_layers-1:   h <- RMSNorm(h + MoE_l(h))
 * where MoE_l is smoe_moe_layer with router_w[l], experts[l] and
 * residual = h.  h: [B, d] fp32, updated in place; tmp: [B, d] fp32
 * scratch, distinct from h.  router_w, experts: HOST arrays of n_layers
 * entries (device pointers inside, as for smoe_moe_layer).
 * topk_idx [n_layers, B, top_k] int32 and topk_w [n_layers, B, top_k] fp32
 * receive every layer's routing; n_union (nullable) [n_layers] int32
 * receives every layer's union size (else un->n_union holds the last
 * layer's); the other union arrays of un hold the last layer's lists.
 * ws: one workspace sized for (desc, B), shared by the layers.
 * All layers are validated before the first launch: on an error nothing is
 * launched and h is unchanged.  n_layers == 0 or B == 0 is a no-op.
 * The results are bit-identical to that loop of smoe_moe_layer and
 * smoe_rmsnorm calls; for decode-sized batches the norm of a layer's output
 * is formed inside the next layer's router (the same summation order), so
 * the stack launches one kernel fewer per layer.
 * Async on stream; eps > 0. */
int smoe_stack_forward(const smoe_layer_desc* desc, int32_t n_layers, const void* const* router_w,
                       const smoe_experts* experts, float* h, int32_t B, float eps, float* tmp,
                       int32_t* topk_idx, float* topk_w, int32_t* n_union, const smoe_union* un,
                       void* ws, size_t ws_bytes, void* stream);

/* One chunk of a prompt for smoe_stack_forward_chunks: the arguments of
 * smoe_stack_forward that belong to one batch of tokens, with the same
 * meaning and layout.  Every chunk has buffers of its own: h, tmp, the
 * routing outputs, the union arrays and the workspace may not be shared
 * between chunks.  stream: the chunk's own stream (chunks on one stream run
 * one after another, still correctly). */
typedef struct smoe_stack_chunk {
  float* h;            /* [B, d] fp32, updated in place */
  int32_t B;           /* 0 .. 64 tokens; 0 is skipped */
  float* tmp;          /* [B, d] fp32 scratch, distinct from h */
  int32_t* topk_idx;   /* [n_layers, B, top_k] int32 */
  float* topk_w;       /* [n_layers, B, top_k] fp32 */
  int32_t* n_union;    /* [n_layers] int32, or NULL */
  smoe_union un;
  void* ws;            /* workspace sized for (desc, B) */
  size_t ws_bytes;
  void* stream;
} smoe_stack_chunk;

#define SMOE_MAX_STACK_CHUNKS 8

/* The chunks of a prompt through one stack, several in flight at once
 * ([LMP] "Choreography Per Chunk": every chunk of up to 64 tokens goes
 * through the layers in order, each layer's union streamed once for the
 * chunk).  Chunk i runs on chunks[i].stream and starts its layer l when
 * chunk i-1 has finished its own layer l, the order causal attention over
 * the chunks would need; so while one chunk's FFN streams its experts, the
 * next chunk's routing, combine and norm, which wait on latency rather than
 * on HBM, run beside it.  Each chunk's outputs are bit-identical to
 * smoe_stack_forward on that chunk alone.
 * n_chunks: 1 .. SMOE_MAX_STACK_CHUNKS.  The call is ordered on
 * chunks[0].stream like one launch: the other streams first wait for what
 * is queued there, and it waits for all of them at the end.  Every chunk and
 * layer is checked before the first launch (on an error nothing is launched):
 * the errors of smoe_stack_forward, and SMOE_EINVAL when two chunks share h,
 * tmp, a routing output, a union array or the workspace.  The library keeps
 * SMOE_MAX_STACK_CHUNKS + 1 HIP events per host thread and device for the
 * ordering, created on first use (no device memory).  Async. */
int smoe_stack_forward_chunks(const smoe_layer_desc* desc, int32_t n_layers,
                              const void* const* router_w, const smoe_experts* experts, float eps,
                              const smoe_stack_chunk* chunks, int32_t n_chunks);

/* ---------------------------------------------------------- calibration */
/* Diagnostic: a plain streaming read of `bytes` (a multiple of 16) at `src`
 * (16-byte aligned) by `blocks` workgroups of 256 threads with 16-byte
 * nontemporal loads; block b writes the xor of what it read to sink[b]
 * (sink: `blocks` uint32, device).  Measures the read bandwidth the part
 * reaches on a pure stream, against which the layer's kernels are judged.
 * Async on stream; SMOE_EINVAL on bad arguments, 1 <= blocks <= 2^20. */
int smoe_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, void* stream);

/* Diagnostic: the direct global -> LDS copy path that the prefill FFN
 * kernels stream their weights through ([LMP] "Choreography Per Chunk"
 * step 6), with no arithmetic behind it.  `src` (16-byte aligned) is read as
 * a [rows, row_bytes] matrix (row_bytes a multiple of 64 in 64 .. 65536;
 * rows = bytes / row_bytes, whole 64-row units only); each wave streams one
 * 64-row unit through a ring of three 4 KB stages in LDS, four waves a
 * workgroup, two workgroups per compute unit.  mode 0: the FFN's pattern
 * (stage k = bytes 64k .. 64k+63 of every row of the unit, 16-row tiles,
 * the second half of each 128-byte line with the nontemporal hint); mode
 * 1: the unit's bytes in memory order, 4 KB a stage.  Block b writes a xor
 * of what it read to sink[b] (sink: sink_n uint32, device, at least
 * ceil(units / 4)).  Async on stream; SMOE_EINVAL on bad arguments. */
int smoe_dma_read(const void* src, size_t bytes, int32_t row_bytes, int32_t mode, uint32_t* sink,
                  int32_t sink_n, void* stream);

/* Diagnostic: `count` (0 .. 2^20) back-to-back launches, from this one
 * call, of a kernel of `blocks` (1 .. 2^20) workgroups of 64 threads that
 * does nothing; timed on the stream, the mean is the cost of one more
 * kernel boundary on the device (the host enqueues faster than that).
 * Async on stream; SMOE_EINVAL on bad counts, SMOE_EHIP when a launch
 * fails. */
int smoe_empty_launch(int32_t blocks, int32_t count, void* stream);

/* Diagnostic: one wave that waits `us` (0 .. 100000) microseconds of the
 * device's 100 MHz clock and ends.  Queued ahead of a timed region, it keeps
 * the device busy while the host enqueues the region's first launches, so
 * the region's time does not include the host's latency to its first kernel.
 * Async on stream; SMOE_EINVAL on a bad duration, SMOE_EHIP when the launch
 * fails. */
int smoe_gpu_sleep(int32_t us, void* stream);

/* Diagnostic: one device-wide barrier, the in-kernel alternative to a kernel
 * boundary.  A cooperative grid of `blocks` (1 .. 4096) workgroups of 256
 * threads, all resident at once (the runtime refuses the launch otherwise:
 * SMOE_EHIP); each block passes its own barrier, thread 0 increments
 * *counter (acquire-release, device scope: one release of the block's
 * stores) and then polls it with acquire loads until all blocks have arrived
 * or about 2^22 polls have passed, when it sets *timed_out = 1 and goes on,
 * so the kernel always ends.  stamps (device, 3 * blocks uint64) receive per
 * block the s_memrealtime count (100 MHz) at its start, after its increment
 * and after its wait.  *counter must be 0 on entry (the caller clears it);
 * it is left at `blocks`.  Async on stream; SMOE_EINVAL on bad arguments. */
int smoe_grid_barrier(int32_t blocks, uint32_t* counter, uint64_t* stamps, int32_t* timed_out,
                      void* stream);

/* ------------------------------------------------------------ utilities */
/* Synchronises `stream`, then copies the workspace status bits into
 * *status_out (host).  For tests and diagnostics, not for the hot path. */
int smoe_read_status(const void* ws, size_t ws_bytes, void* stream, uint32_t* status_out);

/* A static, human-readable name for an SMOE_* return code. */
const char* smoe_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* SMOE_H */
