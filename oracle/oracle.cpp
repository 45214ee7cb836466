// oracle.cpp - plain CPU reference for one routed mixture-of-experts layer.
//
// TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU
// baseline of the benchmark, never by the product library.  Shares no code
// with the GPU library.  See oracle.h for the contract of every function and
// the page each one follows.
//
// Build: g++ -std=c++17 -O2 -ffp-contract=off -fopenmp -fPIC -shared oracle.cpp
// (no -ffast-math: every fp32 product and sum is rounded on its own).

#include "oracle.h"

#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

namespace {

float bf16_to_float(uint16_t h) {
  uint32_t u = static_cast<uint32_t>(h) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Sequential fp32 dot product, index ascending.
float dot_seq(const float* a, const float* b, int n) {
  float acc = 0.0f;
  for (int i = 0; i < n; ++i) {
    const float prod = a[i] * b[i];
    acc = acc + prod;
  }
  return acc;
}

// y[r] = dot(W[r,:], x) for r < rows.
void matvec(const float* W, const float* x, int rows, int cols, float* y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) y[r] = dot_seq(W + static_cast<int64_t>(r) * cols, x, cols);
}

// silu(g) * u, the SwiGLU gate ([SSD] "Math Contract": silu(gate) * up).
float swiglu(float g, float u) {
  const float sig_den = 1.0f + std::exp(-g);
  const float silu = g / sig_den;
  return silu * u;
}

struct DenseExpert {
  std::vector<float> Wg, Wu, Wd;
};

void dequant_expert(const oracle_qmat* gate, const oracle_qmat* up, const oracle_qmat* down, int d,
                    int f, int e, DenseExpert* out) {
  out->Wg.resize(static_cast<size_t>(f) * d);
  out->Wu.resize(static_cast<size_t>(f) * d);
  out->Wd.resize(static_cast<size_t>(d) * f);
  oracle_dequant(gate->w + e * gate->stride_w, gate->s + e * gate->stride_sb,
                 gate->b + e * gate->stride_sb, f, d, out->Wg.data());
  oracle_dequant(up->w + e * up->stride_w, up->s + e * up->stride_sb, up->b + e * up->stride_sb, f,
                 d, out->Wu.data());
  oracle_dequant(down->w + e * down->stride_w, down->s + e * down->stride_sb,
                 down->b + e * down->stride_sb, d, f, out->Wd.data());
}

// out[t] = residual[t] + (sum over k ascending of w[t,k] * y[t*K+k]).
void combine(const float* y_pairs, const float* w, const float* residual, int B, int K, int d,
             float* out) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < B; ++t) {
    for (int r = 0; r < d; ++r) {
      float acc = 0.0f;
      for (int k = 0; k < K; ++k) {
        const float term = w[t * K + k] * y_pairs[(static_cast<int64_t>(t) * K + k) * d + r];
        acc = acc + term;
      }
      const float res = residual ? residual[static_cast<int64_t>(t) * d + r] : 0.0f;
      out[static_cast<int64_t>(t) * d + r] = res + acc;
    }
  }
}

}  // namespace

extern "C" {

void oracle_router_logits(const void* Wr, int wr_is_bf16, const float* x, int B, int d, int E,
                          float* logits) {
  // The gate is widened to fp32 (bf16 -> fp32 is exact), then each logit is
  // one sequential fp32 dot product.
  std::vector<float> W(static_cast<size_t>(E) * d);
  for (size_t n = 0; n < W.size(); ++n)
    W[n] = wr_is_bf16 ? bf16_to_float(static_cast<const uint16_t*>(Wr)[n])
                      : static_cast<const float*>(Wr)[n];
  for (int t = 0; t < B; ++t)
    for (int e = 0; e < E; ++e)
      logits[static_cast<int64_t>(t) * E + e] =
          dot_seq(W.data() + static_cast<int64_t>(e) * d, x + static_cast<int64_t>(t) * d, d);
}

void oracle_topk_softmax(const float* logits, int B, int E, int K, int norm, int32_t* idx,
                         float* w) {
  std::vector<int> order(E);
  std::vector<float> p(E);
  for (int t = 0; t < B; ++t) {
    const float* l = logits + static_cast<int64_t>(t) * E;
    // Rank every expert: larger logit first; equal logits by lower index.
    for (int e = 0; e < E; ++e) order[e] = e;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return l[a] > l[b]; });
    // Full softmax over all E experts, max-subtracted.
    float m = l[0];
    for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
    float Z = 0.0f;
    for (int e = 0; e < E; ++e) {
      p[e] = std::exp(l[e] - m);
      Z = Z + p[e];
    }
    for (int e = 0; e < E; ++e) p[e] = p[e] / Z;
    // Top-k in rank order, then optional renormalisation to sum 1.
    float S = 0.0f;
    for (int k = 0; k < K; ++k) S = S + p[order[k]];
    for (int k = 0; k < K; ++k) {
      idx[t * K + k] = order[k];
      w[t * K + k] = norm ? p[order[k]] / S : p[order[k]];
    }
  }
}

// Routing weights of a given set of K experts per token (idx, rank order as
// given), from the same full softmax as oracle_topk_softmax: p over all E,
// then p of the set divided by its sum (norm) or p itself.  For the top-k set
// this is exactly oracle_topk_softmax's weights; tests use it where two
// correct routings differ at a near-tie and the weights of the other set are
// needed.  Ids outside [0, E) give -1.
int oracle_weights_of(const float* logits, int B, int E, int K, int norm, const int32_t* idx,
                      float* w) {
  std::vector<float> p(E);
  for (int t = 0; t < B; ++t) {
    const float* l = logits + static_cast<int64_t>(t) * E;
    for (int k = 0; k < K; ++k)
      if (idx[t * K + k] < 0 || idx[t * K + k] >= E) return -1;
    float m = l[0];
    for (int e = 1; e < E; ++e) m = l[e] > m ? l[e] : m;
    float Z = 0.0f;
    for (int e = 0; e < E; ++e) {
      p[e] = std::exp(l[e] - m);
      Z = Z + p[e];
    }
    for (int e = 0; e < E; ++e) p[e] = p[e] / Z;
    float S = 0.0f;
    for (int k = 0; k < K; ++k) S = S + p[idx[t * K + k]];
    for (int k = 0; k < K; ++k) {
      const float pk = p[idx[t * K + k]];
      w[t * K + k] = norm ? pk / S : pk;
    }
  }
  return 0;
}

// The R highest-ranked experts of each token, in rank order: larger logit
// first, equal logits by lower index ("Data Flow", the routing step: ranked
// top-(8+spec), ranks 8 and up queued for speculative prefetch; "Surface
// Scout": the current token's lower gate ranks).  The first K equal
// oracle_topk_softmax's indices.
void oracle_rank(const float* logits, int B, int E, int R, int32_t* ranked) {
  std::vector<int> order(E);
  for (int t = 0; t < B; ++t) {
    const float* l = logits + static_cast<int64_t>(t) * E;
    for (int e = 0; e < E; ++e) order[e] = e;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return l[a] > l[b]; });
    for (int k = 0; k < R; ++k) ranked[static_cast<int64_t>(t) * R + k] = order[k];
  }
}

int oracle_build_union(const int32_t* idx, int B, int K, int E, int32_t* union_experts,
                       int32_t* offsets, int32_t* pair_list, int32_t* pair_pos) {
  const int P = B * K;
  for (int p = 0; p < P; ++p)
    if (idx[p] < 0 || idx[p] >= E) return -1;
  // Distinct experts, ascending.
  std::vector<int> count(E, 0);
  for (int p = 0; p < P; ++p) count[idx[p]] += 1;
  int n_union = 0;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) {
    if (count[e] == 0) continue;
    union_experts[n_union] = e;
    offsets[n_union + 1] = offsets[n_union] + count[e];
    n_union += 1;
  }
  // Each union expert's pairs, ascending p: a plain filter over all pairs.
  for (int u = 0; u < n_union; ++u) {
    int pos = offsets[u];
    for (int p = 0; p < P; ++p) {
      if (idx[p] != union_experts[u]) continue;
      pair_list[pos] = p;
      pair_pos[p] = pos;
      pos += 1;
    }
  }
  return n_union;
}

void oracle_dequant(const uint32_t* w, const uint16_t* s, const uint16_t* b, int rows, int cols,
                    float* out) {
  const int words_per_row = cols / 8, groups_per_row = cols / 64;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    for (int c = 0; c < cols; ++c) {
      const uint32_t word = w[static_cast<int64_t>(r) * words_per_row + c / 8];
      const uint32_t q = (word >> (4 * (c % 8))) & 0xFu;
      const float sc = bf16_to_float(s[static_cast<int64_t>(r) * groups_per_row + c / 64]);
      const float bi = bf16_to_float(b[static_cast<int64_t>(r) * groups_per_row + c / 64]);
      const float sq = sc * static_cast<float>(q);
      out[static_cast<int64_t>(r) * cols + c] = sq + bi;
    }
  }
}

void oracle_expert_ffn(const float* Wg, const float* Wu, const float* Wd, const float* x, int d,
                       int f, float* g_out, float* u_out, float* h, float* y) {
  std::vector<float> g(f), u(f), hh(f);
  matvec(Wg, x, f, d, g.data());
  matvec(Wu, x, f, d, u.data());
  for (int j = 0; j < f; ++j) hh[j] = swiglu(g[j], u[j]);
  matvec(Wd, hh.data(), d, f, y);
  if (g_out) std::memcpy(g_out, g.data(), sizeof(float) * f);
  if (u_out) std::memcpy(u_out, u.data(), sizeof(float) * f);
  if (h) std::memcpy(h, hh.data(), sizeof(float) * f);
}

int oracle_moe_token_major(const oracle_qmat* gate, const oracle_qmat* up, const oracle_qmat* down,
                           int d, int f, int E, const float* x, int B, int K, const int32_t* idx,
                           const float* w, const float* residual, float* out, float* y_pairs) {
  for (int p = 0; p < B * K; ++p)
    if (idx[p] < 0 || idx[p] >= E) return -1;
  std::vector<float> Y(static_cast<size_t>(B) * K * d);
  DenseExpert ex;
  for (int t = 0; t < B; ++t) {
    for (int k = 0; k < K; ++k) {
      const int e = idx[t * K + k];
      dequant_expert(gate, up, down, d, f, e, &ex);  // fetched per (token, rank)
      oracle_expert_ffn(ex.Wg.data(), ex.Wu.data(), ex.Wd.data(), x + static_cast<int64_t>(t) * d,
                        d, f, nullptr, nullptr, nullptr,
                        Y.data() + (static_cast<int64_t>(t) * K + k) * d);
    }
  }
  combine(Y.data(), w, residual, B, K, d, out);
  if (y_pairs) std::memcpy(y_pairs, Y.data(), sizeof(float) * Y.size());
  return 0;
}

int oracle_moe_layer_major(const oracle_qmat* gate, const oracle_qmat* up, const oracle_qmat* down,
                           int d, int f, int E, const float* x, int B, int K, const int32_t* idx,
                           const float* w, const float* residual, float* out, float* y_pairs) {
  const int P = B * K;
  std::vector<int32_t> uexp(std::max(1, std::min(E, P))), off(std::max(1, std::min(E, P)) + 1),
      plist(std::max(1, P)), ppos(std::max(1, P));
  const int n_union = oracle_build_union(idx, B, K, E, uexp.data(), off.data(), plist.data(),
                                         ppos.data());
  if (n_union < 0) return -1;
  std::vector<float> Y(static_cast<size_t>(P) * d);
  DenseExpert ex;
  for (int u = 0; u < n_union; ++u) {
    dequant_expert(gate, up, down, d, f, uexp[u], &ex);  // fetched once per union expert
    for (int i = off[u]; i < off[u + 1]; ++i) {
      const int p = plist[i];
      const int t = p / K;
      oracle_expert_ffn(ex.Wg.data(), ex.Wu.data(), ex.Wd.data(), x + static_cast<int64_t>(t) * d,
                        d, f, nullptr, nullptr, nullptr, Y.data() + static_cast<int64_t>(p) * d);
    }
  }
  combine(Y.data(), w, residual, B, K, d, out);
  if (y_pairs) std::memcpy(y_pairs, Y.data(), sizeof(float) * Y.size());
  return 0;
}

void oracle_shared_ffn(const oracle_qmat* gate, const oracle_qmat* up, const oracle_qmat* down,
                       int d, int fs, const float* x, int B, float* shared_out) {
  DenseExpert ex;
  dequant_expert(gate, up, down, d, fs, 0, &ex);
  for (int t = 0; t < B; ++t)
    oracle_expert_ffn(ex.Wg.data(), ex.Wu.data(), ex.Wd.data(), x + static_cast<int64_t>(t) * d, d,
                      fs, nullptr, nullptr, nullptr, shared_out + static_cast<int64_t>(t) * d);
}

void oracle_combine_shared(const float* y_pairs, const float* w, const float* shared_out,
                           const float* residual, int B, int K, int d, float* out) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < B; ++t) {
    for (int r = 0; r < d; ++r) {
      float routed = 0.0f;
      for (int k = 0; k < K; ++k) {
        const float term = w[t * K + k] * y_pairs[(static_cast<int64_t>(t) * K + k) * d + r];
        routed = routed + term;
      }
      const int64_t o = static_cast<int64_t>(t) * d + r;
      const float both = shared_out[o] + routed;
      const float res = residual ? residual[o] : 0.0f;
      out[o] = res + both;
    }
  }
}

void oracle_rmsnorm(const float* v, int B, int d, float eps, float* out) {
  for (int t = 0; t < B; ++t) {
    const float* row = v + static_cast<int64_t>(t) * d;
    float ss = 0.0f;
    for (int i = 0; i < d; ++i) ss = ss + row[i] * row[i];
    const float mean = ss / static_cast<float>(d);
    // the definition as written: each element divided by the root
    const float root = std::sqrt(mean + eps);
    for (int i = 0; i < d; ++i) out[static_cast<int64_t>(t) * d + i] = row[i] / root;
  }
}

int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { omp_set_num_threads(n); }

}  // extern "C"
