/*
 * oracle.h - plain CPU reference for one routed mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this code; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark do.  It shares no code, header, table or constant with
 * the GPU library: it reads the same input bytes and nothing else.
 *
 * Arithmetic: fp32 with sequential accumulation in index order, compiled
 * with -ffp-contract=off (every product and every sum rounded separately).
 * Parallel loops (OpenMP) only split independent outputs; each output is
 * still computed by one thread in the same order, so results do not depend
 * on the thread count.
 *
 * Citations name the web pages the method is described on:
 *  [DF]  "Data Flow" (S-MoE architecture docs)
 *  [LMP] "Layer-Major Batched Prefill" (S-MoE internals docs)
 *  [SSD] "SSD Streaming Expert Layers" (edge0 streaming.md)
 *  [SC]  "Surface Scout" (S-MoE architecture docs)
 */
#ifndef SMOE_ORACLE_H
#define SMOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One quantised projection for all experts: expert e's packed words start at
 * w + e*stride_w ([rows, cols/8] u32, element c of a row at bits 4*(c%8) of
 * word c/8), its bf16 scales and biases at s/b + e*stride_sb ([rows, cols/64]). */
typedef struct {
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
  int64_t stride_w;
  int64_t stride_sb;
} oracle_qmat;

/* Router logits, [LMP] step 5 / [DF] "exact routing":
 * logits[t,e] = sum_i float(Wr[e,i]) * x[t,i], i ascending. */
void oracle_router_logits(const void* Wr, int wr_is_bf16, const float* x, int B, int d, int E,
                          float* logits);

/* Softmax, top-k and norm_topk_prob ([DF] serial step "EXACT ROUTING";
 * [SC] model config): ranks sorted by (logit desc, expert index asc); full
 * softmax p; w[t,k] = p[idx] / sum_k' p[idx_k'] when norm != 0, else p[idx]. */
void oracle_topk_softmax(const float* logits, int B, int E, int K, int norm, int32_t* idx,
                         float* w);
// The R highest-ranked experts per token, rank order (ranked [B, R]).
void oracle_rank(const float* logits, int B, int E, int R, int32_t* ranked);

/* Routing weights of a given K-expert set per token (rank order as given),
 * from the full softmax of the logits: p_e / sum over the set (norm) or p_e.
 * For the top-k set it equals oracle_topk_softmax's weights.  Returns -1 on
 * an id outside [0, E), else 0. */
int oracle_weights_of(const float* logits, int B, int E, int K, int norm, const int32_t* idx,
                      float* w);

/* Expert union and per-expert pair lists ([LMP] "The Inversion": dedupe the
 * chunk's experts, apply each union expert to every routed token).
 * Pair p = t*K + k.  Returns n_union; union_experts ascending;
 * offsets[u]..offsets[u+1] index pair_list; pairs ascending within an
 * expert; pair_pos[p] = position of p in pair_list.  Returns -1 when an
 * expert id is outside [0, E). */
int oracle_build_union(const int32_t* idx, int B, int K, int E, int32_t* union_experts,
                       int32_t* offsets, int32_t* pair_list, int32_t* pair_pos);

/* 4-bit affine dequantisation ([SSD] "Quantized Layout"):
 * W[r,c] = float(s[r,c/64]) * q[r,c] + float(b[r,c/64]). */
void oracle_dequant(const uint32_t* w, const uint16_t* s, const uint16_t* b, int rows, int cols,
                    float* out);

/* SwiGLU expert FFN on dense fp32 weights ([SSD] "Math Contract"):
 * g = Wg x, u = Wu x, h = silu(g) * u, y = Wd h.  Wg, Wu: [f, d]; Wd: [d, f].
 * h (nullable) receives h; g_out/u_out (nullable) receive g and u. */
void oracle_expert_ffn(const float* Wg, const float* Wu, const float* Wd, const float* x, int d,
                       int f, float* g_out, float* u_out, float* h, float* y);

/* Token-major layer: for each token, for each of its K experts, dequantise
 * and apply the expert, then combine.  out[t] = residual[t] + sum_k w[t,k] y[t,k]
 * with the k-ascending sum formed first ([DF] "gather GPU outputs x routing
 * weights -> routed_out", "residual += shared_out + routed_out").
 * residual may be NULL (treated as zero).  y_pairs (nullable) receives
 * y for every pair, [B*K, d]. */
int oracle_moe_token_major(const oracle_qmat* gate, const oracle_qmat* up, const oracle_qmat* down,
                           int d, int f, int E, const float* x, int B, int K, const int32_t* idx,
                           const float* w, const float* residual, float* out, float* y_pairs);

/* Layer-major layer ([LMP] "The Inversion"): build the union, dequantise each
 * union expert once, apply it to every pair in its list, then the same
 * combine.  Must equal the token-major result bit for bit. */
int oracle_moe_layer_major(const oracle_qmat* gate, const oracle_qmat* up, const oracle_qmat* down,
                           int d, int f, int E, const float* x, int B, int K, const int32_t* idx,
                           const float* w, const float* residual, float* out, float* y_pairs);

/* Shared-expert FFN ([DF] layer flow: the shared expert FFN beside the routed
 * experts, giving shared_out; [SC] weight inventory: the shared expert of
 * architectures that have one): one always-active SwiGLU expert of width fs
 * on every token, shared_out[t] = Wd_s (silu(Wg_s x_t) * Wu_s x_t).  gate/up
 * hold one [fs, d] matrix, down one [d, fs] (expert 0 of each qmat). */
void oracle_shared_ffn(const oracle_qmat* gate, const oracle_qmat* up, const oracle_qmat* down,
                       int d, int fs, const float* x, int B, float* shared_out);

/* Combine with a shared expert ([DF] "residual += shared_out + routed_out"):
 * routed_out[t] = sum over k ascending of w[t,k] y[t*K+k] (formed first), then
 * out[t] = residual[t] + (shared_out[t] + routed_out[t]).  residual may be
 * NULL (zero). */
void oracle_combine_shared(const float* y_pairs, const float* w, const float* shared_out,
                           const float* residual, int B, int K, int d, float* out);

/* RMSNorm with unit gain: out = v / sqrt(mean(v^2) + eps), fp32, sum ascending. */
void oracle_rmsnorm(const float* v, int B, int d, float eps, float* out);

/* Threads OpenMP will use. */
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
