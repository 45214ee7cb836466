// ffn_gemv.hip - the expert FFN when every union expert serves one or two
// pairs (B <= 2 tokens, the decode regime of "Data Flow", Regime 2).
//
// Each union expert is then a matrix-vector product ("Layer-Major Batched
// Prefill", step 6, with B = 1): the work is a pure stream of the expert
// bytes, done by two kernels so that the kernel boundary (one cache
// writeback for the whole device) publishes h, instead of in-kernel
// device-scope fences, which on a multi-XCD part write back an XCD's whole L2
// each time:
//
//  k_gate_up_gemv: one item per wave (union expert, two consecutive j: 2 gate
//    rows + 2 up rows, 8 KB at d = 4096), streamed through a two-item ring;
//    h_j = silu(g_j) * u_j ("SSD Streaming Expert Layers", "Math Contract")
//    is written as prepped fp16.
//  k_down_combine_gemv: a block owns 8 output rows for ALL union experts, one
//    (union expert, 8 rows) item per wave, and finishes with the weighted
//    combine of its rows in rank order ("Data Flow": gather outputs x routing
//    weights, residual += ...), so y never leaves the chip.
//
// Both kernels stage the call's routing metadata (at most 16 pairs) in LDS
// first, so no dependent global load sits inside their loops.
//
// A shared expert ("Data Flow": the shared expert FFN beside the routed ones)
// rides along as more items of the same launches: gate_up items past the
// routed ones cover its rows (every token a pair), and down items past the
// routed ones cover its rows in chunks, whose partial sums the combine adds
// up first: out = residual + (shared_out + routed_out).
//
// Lane layouts.  gate_up: a row's d/64 groups (64 inputs each) over TPR = 32
// or 64 lanes, one or two groups a lane (lanes past the row's end idle), so
// any d that is a multiple of 64 up to 8192.  down: lane L owns NW = 1, 2 or
// 4 consecutive words of every row (of a chunk of at most 64 NW words) and
// the matching slice of h, so that a lane reads its h once per item and uses
// it for all 8 rows; the row sums then come from one transpose-reduce over
// the wave.  Rows longer than 256 words split into equal chunks (one item
// each), whose partial sums the combine adds in chunk order.
#include <algorithm>

#include "device.hpp"
#include "route_dev.hpp"
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
// gate_up item: kJ consecutive j, gate rows then up rows; two j at one
// 64-input group per lane, one j at two groups per lane (d > 4096), so that
// an item is 8 KB of weights at d = 4096 and at d = 8192 alike
template <int GPL>
constexpr int kItemJ = 2 / GPL;
constexpr int kDnRows = 8;            // down: output rows per block item
constexpr int kMaxDecPairs = 16;      // B * K <= 16 on this path
// gate_up: one 4-wave block per compute unit, i.e. one streaming wave per SIMD:
// the arithmetic (about 9 VALU ops per packed word) then hides under the next
// item's loads instead of piling up once all of a burst has landed
constexpr int kGuBlocksPerCU = 1;
constexpr int kGuDepth = 2;           // gate_up: items per wave in the load ring
constexpr int kGuMaxItems = 64;       // gate_up: items per wave (h staged in LDS)
constexpr int kDnBlocksPerCU = 2;     // down: two blocks per CU (one row block each at d = 4096)
constexpr int kDnThreads = 512;       // down: 8 waves a block, one item each at d = 4096
constexpr int kDnWaves = kDnThreads / 64;
constexpr int kMaxDecF = 8192;        // f and fs on this path

// Prepped position (half index within the row) of column c.
__device__ __forceinline__ int prepped_pos(int c) {
  const int n = c & 7;
  return (c & ~7) + 2 * (n & 3) + (n >> 2);
}

// Dot of one lane's GPL groups (8 words each) against prepped activations,
// with the fp32 group epilogue: sum_g s_g (D_g - C_g) + b_g X_g.  Group gi's
// activations are xc[gi * gstride * 8 ...] and its sums xsum[gi * gstride].
template <int GPL>
__device__ __forceinline__ float lane_row_dot(const uint4 (&w)[GPL][2], const float (&sc)[GPL],
                                              const float (&bi)[GPL], const uint4* xc,
                                              const float2* xsum, int gstride = 1) {
  float part = 0.f;
#pragma unroll
  for (int gi = 0; gi < GPL; ++gi) {
    const uint4* xg = xc + gi * gstride * 8;
    float acc = 0.f;
    acc = dot_word(w[gi][0].x, xg[0], acc);
    acc = dot_word(w[gi][0].y, xg[1], acc);
    acc = dot_word(w[gi][0].z, xg[2], acc);
    acc = dot_word(w[gi][0].w, xg[3], acc);
    acc = dot_word(w[gi][1].x, xg[4], acc);
    acc = dot_word(w[gi][1].y, xg[5], acc);
    acc = dot_word(w[gi][1].z, xg[6], acc);
    acc = dot_word(w[gi][1].w, xg[7], acc);
    const float2 xsg = xsum[gi * gstride];
    part += sc[gi] * (acc - xsg.y) + bi[gi] * xsg.x;
  }
  return part;
}

// Routing metadata of the call (at most 16 pairs), staged once in LDS.  The
// routed gate_up kernel also writes it, in this layout, to FfnArgs::dec_meta,
// so that the down kernel reads it with one load per thread instead of
// gathering it from six arrays.
struct DecMeta {
  int n_union;
  int experts[kMaxDecPairs];
  int offsets[kMaxDecPairs + 1];
  int pairs[kMaxDecPairs];    // pair_list
  int pos[kMaxDecPairs];      // pair_pos
  float w[kMaxDecPairs];      // topk_w
};
constexpr int kDecMetaWords = sizeof(DecMeta) / 4;
static_assert(sizeof(DecMeta) == 4 * (5 * kMaxDecPairs + 2) && sizeof(DecMeta) <= 512,
              "DecMeta is the packed layout of FfnArgs::dec_meta");

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------------------ gate_up items
// One item: union slot u, j0 = 2 * (item % (f/2)); rows (gate j0, gate j0+1,
// up j0, up j0+1).  TPR lanes per row, 64/TPR rows per step; lane li of a row
// takes groups li + TPR gi (gi < GPL) of its 64-input groups.  A (lane, gi)
// past the row's last group is dead: its loads read nothing (an offset past
// every buffer) and return zero words, scale and bias, so it adds 0.
template <int TPR, int GPL>
struct GuBuf {
  static constexpr int kSteps = 2 * kItemJ<GPL> / (64 / TPR);
  uint4 w[kSteps][GPL][2];
  uint32_t s[kSteps][GPL], b[kSteps][GPL];
};

// Per-lane byte offsets of a gate_up item's loads, the same for every item:
// step k covers rows rs = k kRps + slot (gate j0 + rs, or up j0 + rs - kJ).
template <int TPR, int GPL>
struct GuLane {
  uint32_t w[GuBuf<TPR, GPL>::kSteps][GPL];   // packed words, first 16 bytes
  uint32_t s[GuBuf<TPR, GPL>::kSteps][GPL];   // scale and bias (bf16)
};
template <int TPR, int GPL>
__device__ __forceinline__ GuLane<TPR, GPL> gu_lane(const FfnArgs& a, int lane) {
  constexpr int kRps = 64 / TPR, kJ = kItemJ<GPL>;
  const int G = a.d / 64, C = a.d / 8;
  const int li = lane % TPR, slot = lane / TPR;
  GuLane<TPR, GPL> o;
#pragma unroll
  for (int k = 0; k < GuBuf<TPR, GPL>::kSteps; ++k) {
    const int r = (k * kRps + slot) % kJ;           // row within the item's kJ
#pragma unroll
    for (int gi = 0; gi < GPL; ++gi) {
      const int grp = li + TPR * gi;
      o.w[k][gi] = grp < G ? (uint32_t)(r * C + grp * 8) * 4 : kBufferDead;
      o.s[k][gi] = grp < G ? (uint32_t)(r * G + grp) * 2 : kBufferDead;
    }
  }
  return o;
}

// Issue the loads of one item.  Everything that changes from item to item
// (expert, rows, past-the-end) lives in the buffer resources, which are
// scalar: the loop writes no vector register before these loads, so the
// compiler has no reason to wait for the previous item's loads first.  An
// item past the end gets empty resources: its loads return zeros and touch
// no memory.
// Expert e's matrix of a projection, or the shared expert's one (sh).
struct QPtr {
  const uint32_t* w;
  const uint16_t* s;
  const uint16_t* b;
};
__device__ __forceinline__ QPtr expert_mat(const QMat& m, const QMat& shared, bool sh, int e) {
  return sh ? QPtr{shared.w, shared.s, shared.b}
            : QPtr{m.w + e * m.stride_w, m.s + e * m.stride_sb, m.b + e * m.stride_sb};
}
// The same as mask arithmetic on both addresses (sh uniform): inside the ring
// loop a branch around the multiplies would need a vector register for its
// condition, and the compiler then waits for the loads in flight first.
template <class T>
__device__ __forceinline__ const T* pick(bool sh, const T* if_sh, const T* if_not) {
  const uint64_t m = 0 - (uint64_t)sh;
  const uint64_t a = reinterpret_cast<uint64_t>(if_sh), b = reinterpret_cast<uint64_t>(if_not);
  return reinterpret_cast<const T*>(b ^ ((a ^ b) & m));
}
__device__ __forceinline__ QPtr expert_mat_nb(const QMat& m, const QMat& shared, bool sh, int e) {
  return QPtr{pick(sh, shared.w, m.w + e * m.stride_w), pick(sh, shared.s, m.s + e * m.stride_sb),
              pick(sh, shared.b, m.b + e * m.stride_sb)};
}

// Items 0 .. nR-1 are routed (union slot, j0); items from nR on cover the
// shared expert's rows, j0 = 2 (item - nR).  kShared: the layer has a shared
// expert (a separate instance: the extra pointers would otherwise crowd the
// scalar registers of the routed-only loop).
template <int TPR, int GPL, bool kShared>
__device__ __forceinline__ void gu_load(const FfnArgs& a, int lane_expert, int item, int n_items,
                                        int nR, const GuLane<TPR, GPL>& lo, GuBuf<TPR, GPL>& buf) {
  constexpr int kRps = 64 / TPR, kJ = kItemJ<GPL>;
  const int per = a.f / kJ;
  const bool live = item < n_items;
  const int itc = live ? item : n_items - 1;
  const bool sh = kShared && itc >= nR;
  // kShared: no branches in here (see pick); a shared item's u is a valid
  // slot whose expert goes unused
  const int u = kShared ? uniform((int)((unsigned)max(min(itc, nR - 1), 0) / (unsigned)per))
                        : uniform(itc / per);
  const int j0 = (sh ? itc - nR : itc - u * per) * kJ;
  // union slot u's expert, from lane u of a register (no LDS read, so no
  // temporary register is written while the ring's loads are in flight)
  const int e = __builtin_amdgcn_readlane(lane_expert, u);
  const int G = a.d / 64, C = a.d / 8;
  const uint32_t wbytes = live ? (uint32_t)(kJ * C * 4) : 0u;
  const uint32_t sbytes = live ? (uint32_t)(kJ * G * 2) : 0u;
  const int64_t wr = (int64_t)j0 * C, sr = (int64_t)j0 * G;
  const QPtr g = expert_mat_nb(a.gate, a.sgate, sh, e), up = expert_mat_nb(a.up, a.sup, sh, e);
  const auto gw = buffer_rsrc(g.w + wr, wbytes);
  const auto gs = buffer_rsrc(g.s + sr, sbytes);
  const auto gb = buffer_rsrc(g.b + sr, sbytes);
  const auto uw = buffer_rsrc(up.w + wr, wbytes);
  const auto us = buffer_rsrc(up.s + sr, sbytes);
  const auto ub = buffer_rsrc(up.b + sr, sbytes);
#pragma unroll
  for (int k = 0; k < GuBuf<TPR, GPL>::kSteps; ++k) {
    const bool is_up = k * kRps >= kJ;             // rows k kRps ..: gate rows, then up rows
#pragma unroll
    for (int gi = 0; gi < GPL; ++gi) {
      buf.w[k][gi][0] = buf_load4_nt(is_up ? uw : gw, lo.w[k][gi]);
      buf.w[k][gi][1] = buf_load4_nt(is_up ? uw : gw, lo.w[k][gi] + 16);
      buf.s[k][gi] = buf_load_u16_nt(is_up ? us : gs, lo.s[k][gi]);
      buf.b[k][gi] = buf_load_u16_nt(is_up ? ub : gb, lo.s[k][gi]);
    }
  }
  // keep every load of the item here: left to itself the scheduler sinks the
  // scale/bias loads to their first use, after the next item's loads, which
  // exposes a full memory latency per item
  __builtin_amdgcn_sched_barrier(0);
}

// Computes one item and stages its h values (fp16 bits, prepped scaling) in
// the wave's LDS row st: st[jj * NTOK + q] = h of row j0 + jj for the union
// expert's q-th pair (q < its pair count).  xr/xs: the lane's group of the
// prepped activations of token t (t < NTOK).
template <int NTOK, int TPR, int GPL, bool kShared>
__device__ __forceinline__ void gu_compute(const FfnArgs& a, const DecMeta& m, int item, int nR,
                                           int lane, const GuBuf<TPR, GPL>& buf,
                                           const uint4 (&xr)[NTOK][GPL * 8],
                                           const float2 (&xs)[NTOK][GPL],
                                           const float (&xa)[NTOK], uint16_t* st) {
  constexpr int kRps = 64 / TPR, kJ = kItemJ<GPL>;
  static_assert(kRps == 1 || kRps == kJ, "a step holds gate rows only or up rows only");
  const int per = a.f / kJ;
  const bool sh = kShared && item >= nR;          // a shared-expert item: pair q = token q
  const int u = sh ? 0 : uniform(item / per);
  const int j0 = (sh ? item - nR : item - u * per) * kJ;
  const int pb = sh ? 0 : uniform(m.offsets[u]);
  const int ne = sh ? a.B : uniform(m.offsets[u + 1]) - pb;   // 1 .. NTOK
  const int li = lane % TPR, slot = lane / TPR;
  // r[k][t]: row (k*kRps + slot) against token t
  float r[GuBuf<TPR, GPL>::kSteps][NTOK];
#pragma unroll
  for (int k = 0; k < GuBuf<TPR, GPL>::kSteps; ++k) {
    float sc[GPL], bi[GPL];
#pragma unroll
    for (int gi = 0; gi < GPL; ++gi) {
      sc[gi] = bf16_to_f32((uint16_t)buf.s[k][gi]);
      bi[gi] = bf16_to_f32((uint16_t)buf.b[k][gi]);
    }
#pragma unroll
    for (int t = 0; t < NTOK; ++t)
      r[k][t] = segment_sum(lane_row_dot<GPL>(buf.w[k], sc, bi, xr[t], xs[t]), TPR);
  }
  // gate row j0 + jj sits in step jj / kRps at slot jj % kRps, its up row in
  // step (kJ + jj) / kRps at the same slot (kRps is 1 or 2 = kJ)
#pragma unroll
  for (int jj = 0; jj < kJ; ++jj) {
    if (kRps == 1 || slot == jj % kRps) {
      const int kg = jj / kRps, ku = (kJ + jj) / kRps;
      const int j = j0 + jj;
#pragma unroll
      for (int q = 0; q < NTOK; ++q) {
        if (q >= ne) break;
        const int t = NTOK == 1 ? 0 : (sh ? q : uniform(m.pairs[pb + q]) / a.K);
        const int ti = (NTOK == 1 || t == 0) ? 0 : NTOK - 1;
        // the sums were taken over a_t x: 1/a_t (exact) gives g and u, and h
        // is stored as a_t^2 h
        const float at = xa[ti], ia = 1.0f / at;
        const float g = r[kg][ti] * ia;
        const float up = r[ku][ti] * ia;
        const float h = silu_mul(g, up) * (at * at);
        const half_t hv = (j & 1) ? (half_t)((float)(half_t)h * 0.0625f) : (half_t)h;
        if (li == 0) st[jj * NTOK + q] = f16_bits(hv);
      }
    }
  }
}

// ------------------------------------------------------------- down items
// Lane layout of the down kernel: a row, or a chunk of it, of at most 64 NW
// words spreads over the wave, lane L owning words NW L .. NW L + NW - 1
// (8 NW inputs, inside group NW L / 8) and the matching NW chunks of h, read
// once per item and kept in registers for all kDnRows rows of the item.  NW
// is the smallest of 1, 2, 4 whose 64 NW words hold a routed row (f <= 2048);
// past that, NW = 4 and the rows split into chunks.  Lanes past a chunk's
// last word repeat the last live lane's addresses with zero scale and bias.
template <int NTOK, int NW>
struct DnItem {
  uint32_t w[kDnRows][NW];
  uint32_t s[kDnRows], b[kDnRows];
  uint4 h[NTOK][NW];
};

// How the down rows split into chunks: routed rows (f/8 words) into nr
// chunks of wr words, the shared expert's (fs/8 words) into ns chunks of ws
// words; equal widths in whole groups (multiples of 8 words), the last chunk
// shorter when the width does not divide, each at most 64 NW words.
struct DnChunks {
  int nr, wr, ns, ws;
};
__host__ __device__ inline void dn_split(int words, int nw, int& n, int& w) {
  n = (words + 64 * nw - 1) / (64 * nw);
  w = n == 0 ? 0 : ((words + n - 1) / n + 7) / 8 * 8;
}
constexpr int kMaxRtChunks = 4;       // routed rows: f <= 8192 at 256 words a chunk
constexpr int kMaxShChunks = 16;      // shared rows: fs <= 8192 at 64 words a chunk
constexpr int kShRow0 = kMaxDecPairs * kMaxRtChunks;   // first shared ylds row

// Issue the loads of item `item` of a row block (rows r0 .. r0+7): items
// below nU nr are routed, slot item / nr, chunk item % nr; the rest are the
// shared expert's chunks (pair q = token q).  h of the slot's pairs first
// (the compute needs it first), then row by row the row's words, scale and
// bias, so that each row's dot and epilogue wait for that row's loads only.
// No branch: dead pair slots repeat the last live pair.  Returns in ne the
// slot's pair count, in ys[q] the ylds row of its q-th pair (pair p, chunk
// c: row p kMaxRtChunks + c; shared chunk c, token t: kShRow0 + 2 c + t) and
// in ysc[q] 1/a_t^2 of that pair's token.
template <int NTOK, int NW, bool kShared>
__device__ __forceinline__ void down_load(const FfnArgs& a, const DecMeta& m, int item, int nU,
                                          const DnChunks& g, int r0, int lane,
                                          const float (&ib)[2], DnItem<NTOK, NW>& it, int& ne,
                                          int (&ys)[NTOK], float (&ysc)[NTOK]) {
  const int nRI = nU * g.nr;
  const bool sh = kShared && item >= nRI;
  const int u = sh ? 0 : uniform(item / g.nr);
  const int c = sh ? item - nRI : item - u * g.nr;
  const int Cr = sh ? a.fs / 8 : a.f / 8, Gr = Cr / 8;    // words and groups of a row
  const int cw = c * (sh ? g.ws : g.wr);                 // the chunk's first word
  const int NL = min(sh ? g.ws : g.wr, Cr - cw) / NW;
  // Buffer loads: the rows' part of an offset is scalar (soffset), the lane's
  // part a vector offset fixed for the item, so that issuing them takes no
  // vector address arithmetic.  Lanes past the chunk's last word load past
  // every resource, which returns zeros: their h sums, dots, scales and
  // biases all vanish.
  const bool lane_live = lane < NL;
  const uint32_t vw = lane_live ? (uint32_t)(cw + lane * NW) * 4u : kBufferDead;
  const uint32_t vs = lane_live ? (uint32_t)(cw / 8 + (lane * NW) / 8) * 2u : kBufferDead;
  const uint32_t vh = lane_live ? (uint32_t)(cw + lane * NW) * 16u : kBufferDead;
  // an empty union (every routed id invalid) has no routed items; an invalid
  // id in a live slot cannot occur, but would read expert 0
  const int e0 = sh ? 0 : uniform(m.experts[u]);
  const int e = (unsigned)e0 < (unsigned)a.E ? e0 : 0;
  const int pb = sh ? 0 : uniform(m.offsets[u]);
  ne = sh ? a.B : uniform(m.offsets[u + 1]) - pb;
  // h of pair p: Cr chunks of 8 prepped halves; chunk i goes with word i of a row
  const uint4* hsrc = reinterpret_cast<const uint4*>(sh ? a.shp : a.hp);
#pragma unroll
  for (int q = 0; q < NTOK; ++q) {
    const int qq = max(min(q, ne - 1), 0);
    const int p = sh ? qq : uniform(m.pairs[pb + qq]);
    ys[q] = sh ? kShRow0 + 2 * c + qq : p * kMaxRtChunks + c;
    // 1/a_t^2 of the pair's token (one token: always ib[0], which also keeps
    // the pick from becoming an indexed private array)
    ysc[q] = (NTOK == 1 || (sh ? qq : p / a.K) == 0) ? ib[0] : ib[1];
    const auto rh = buffer_rsrc(hsrc + (int64_t)p * Cr, (uint32_t)Cr * 16u);
#pragma unroll
    for (int k = 0; k < NW; ++k) it.h[q][k] = buf_load4(rh, vh + 16u * k);
  }
  const QPtr dn = expert_mat(a.down, a.sdown, sh, e);
  const auto rw = buffer_rsrc(dn.w + (int64_t)r0 * Cr, (uint32_t)(kDnRows * Cr) * 4u);
  const auto rs = buffer_rsrc(dn.s + (int64_t)r0 * Gr, (uint32_t)(kDnRows * Gr) * 2u);
  const auto rb = buffer_rsrc(dn.b + (int64_t)r0 * Gr, (uint32_t)(kDnRows * Gr) * 2u);
#pragma unroll
  for (int r = 0; r < kDnRows; ++r) {
    const int sow = r * Cr * 4, sos = r * Gr * 2;
    if constexpr (NW == 4) {
      const uint4 v = buf_load4_nt(rw, vw, sow);
      it.w[r][0] = v.x, it.w[r][1] = v.y, it.w[r][2] = v.z, it.w[r][3] = v.w;
    } else if constexpr (NW == 2) {
      const uint2 v = buf_load2_nt(rw, vw, sow);
      it.w[r][0] = v.x, it.w[r][1] = v.y;
    } else {
      it.w[r][0] = buf_load1_nt(rw, vw, sow);
    }
    it.s[r] = buf_load_u16_nt(rs, vs, sos);
    it.b[r] = buf_load_u16_nt(rb, vs, sos);
    __builtin_amdgcn_sched_barrier(0);             // in row order, each row's three together
  }
  __builtin_amdgcn_sched_barrier(0);               // issue them here (see gu_load)
}

// One item: the group sums of its pairs' h slices, the eight row dots, the
// wave sums, and the rows' outputs into ylds[ys[q]][row] (live pairs only).
template <int NTOK, int NW>
__device__ __forceinline__ void down_compute(int ne, const int (&ys)[NTOK], const float (&ysc)[NTOK],
                                             int lane, const DnItem<NTOK, NW>& it, float* ylds) {
  float sc[kDnRows], bi[kDnRows];
#pragma unroll
  for (int r = 0; r < kDnRows; ++r) {
    sc[r] = bf16_to_f32((uint16_t)it.s[r]);
    bi[r] = bf16_to_f32((uint16_t)it.b[r]);
  }
  const half2_t one = {(half_t)1.0f, (half_t)1.0f};
  const half2_t sixteen = {(half_t)16.0f, (half_t)16.0f};
#pragma unroll
  for (int q = 0; q < NTOK; ++q) {
    // slot z of a chunk holds (x_z, x_{z+4}), odd z pre-divided by 16: S sums
    // the stored halves (the 1024 offsets of the dequantised nibbles), X the
    // true values (the bias term)
    float S = 0.f, X = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const uint32_t hw[4] = {it.h[q][k].x, it.h[q][k].y, it.h[q][k].z, it.h[q][k].w};
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        const half2_t hv = __builtin_bit_cast(half2_t, hw[z]);
        S = __builtin_amdgcn_fdot2(hv, one, S, false);
        X = __builtin_amdgcn_fdot2(hv, (z & 1) ? sixteen : one, X, false);
      }
    }
    const float S1024 = 1024.0f * S;
    float part[kDnRows];
#pragma unroll
    for (int r = 0; r < kDnRows; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < NW; ++k) acc = dot_word(it.w[r][k], it.h[q][k], acc);
      part[r] = sc[r] * (acc - S1024) + bi[r] * X;
    }
    // h held a_t^2 h: 1/a_t^2 (exact) gives the row outputs
    const float y = rows8_wave_sum(part) * ysc[q];
    if (q < ne && (lane & 7) == 0) ylds[ys[q] * kDnRows + (lane >> 3)] = y;
  }
}

// Routing metadata -> LDS (union arrays hold min(E, P) experts).
__device__ __forceinline__ void load_meta(const FfnArgs& a, DecMeta& m) {
  const int P = a.B * a.K, maxU = min(a.E, P);
  if (threadIdx.x == 0) m.n_union = *a.n_union;
  if (threadIdx.x <= kMaxDecPairs) {
    const int i = threadIdx.x;
    if (i < maxU) m.experts[i] = a.union_experts[i];
    if (i <= maxU) m.offsets[i] = a.expert_offsets[i];
    if (i < P) {
      m.pairs[i] = a.pair_list[i];
      m.pos[i] = a.pair_pos[i];
      m.w[i] = a.topk_w[i];
    }
  }
  __syncthreads();
}

// The routing of the call, in LDS, from the logits (B <= 2 tokens, one wave
// per token): top-k and weights exactly as the router's own tail computes
// them ("Data Flow", serial step "EXACT ROUTING"), then the union and pair
// lists ("Layer-Major Batched Prefill", "The Inversion") by wave 0 with
// readlane counts over the P <= 16 pairs: pairs grouped by ascending expert,
// ascending within.  Block 0 writes the same outputs smoe_route and
// smoe_build_union would.
// What wave 0 keeps of a single token's routing until the kernel's end, when
// block 0 writes the routing outputs (the next kernel is the first reader).
struct RouteKeep {
  float v[4];
  TopkSel t;
};

template <int NTOK>
__device__ __forceinline__ void route_meta(const FfnArgs& a, const DecodeRoute& r, DecMeta& m,
                                           RouteKeep& keep, TopkScratch* tks, int blk) {
  __shared__ int s_e[kMaxDecPairs];
  __shared__ float s_w[kMaxDecPairs];
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int E = a.E, K = a.K, P = a.B * a.K;
  if (NTOK == 1) {
    // one token: its K experts are distinct, so the union is the selected set
    // in ascending expert order and union slot q holds the one pair of that
    // expert, the pair of its rank.  The items need only the set, so the
    // ranks (route_rank) are left until the first items' loads are out.
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        keep.v[j] = e < E ? r.logits[e] : -FLT_MAX;
      }
      uint32_t key[4];
      if (E <= 128) {
        topk_keys<2>(keep.v, E, key);
        topk_compact<2>(keep.v, key, topk_threshold<2>(key, K), K, tks, m.experts);
      } else {
        topk_keys<4>(keep.v, E, key);
        topk_compact<4>(keep.v, key, topk_threshold<4>(key, K), K, tks, m.experts);
      }
      if (lane <= K) m.offsets[lane] = lane;
      if (lane == 0) m.n_union = K;
    }
    __syncthreads();
    return;
  }
  if (wave < a.B) {
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < E ? r.logits[(int64_t)wave * E + e] : -FLT_MAX;
    }
    float my_v;
    int my_e;
    wave_topk(v, E, K, my_v, my_e, &tks[wave]);
    const float w = topk_weight(v, E, K, r.norm != 0, my_v);
    if (lane < K) {
      s_e[wave * K + lane] = my_e;
      s_w[wave * K + lane] = w;
    }
  }
  __syncthreads();
  if (wave == 0) {
    // every pair's expert by broadcast LDS reads (no readlane chains)
    const bool in = lane < P;
    const int e = in ? s_e[lane] : 0x7FFFFFFF;
    int eq[kMaxDecPairs];
#pragma unroll
    for (int q = 0; q < kMaxDecPairs; ++q) eq[q] = q < P ? s_e[q] : 0x7FFFFFFF;
    int less = 0, same_before = 0;
#pragma unroll
    for (int q = 0; q < kMaxDecPairs; ++q) {
      less += eq[q] < e ? 1 : 0;
      same_before += (q < lane && eq[q] == e) ? 1 : 0;
    }
    const bool first = in && same_before == 0;
    const uint64_t firsts = __ballot(first);
    int distinct_less = 0;
#pragma unroll
    for (int q = 0; q < kMaxDecPairs; ++q)
      distinct_less += (((firsts >> q) & 1) && eq[q] < e) ? 1 : 0;
    const int nU = __popcll(firsts);
    const int qpos = less + same_before;          // place of this pair in pair_list
    if (in) {
      m.pairs[qpos] = lane;
      m.pos[lane] = qpos;
      m.w[lane] = s_w[lane];
      if (first) {
        m.experts[distinct_less] = e;
        m.offsets[distinct_less] = less;
      }
    }
    if (lane == 0) {
      m.n_union = nU;
      m.offsets[nU] = P;
    }
    if (blk == 0) {
      if (in) {
        r.topk_idx[lane] = e;
        r.topk_w[lane] = s_w[lane];
        r.pair_list[qpos] = lane;
        r.pair_pos[lane] = qpos;
        if (first) {
          r.union_experts[distinct_less] = e;
          r.expert_offsets[distinct_less] = less;
        }
      }
      if (lane == 0) {
        *r.n_union = nU;
        r.expert_offsets[nU] = P;
      }
    }
  }
  __syncthreads();
  // block 0: the packed copy for the down kernel
  if (blk == 0 && r.dec_meta != nullptr && threadIdx.x < kDecMetaWords)
    r.dec_meta[threadIdx.x] = reinterpret_cast<const int*>(&m)[threadIdx.x];
}

// One token's ranks, from the selection route_meta<1> left in the scratch:
// every wave ranks for itself (the pair of each union slot, for its own h
// flush, into its own LDS row), so that no barrier is needed; block 0's wave
// 0 also keeps what it writes at the kernel's end.
__device__ __forceinline__ void route_rank(int K, int* slot_pair, RouteKeep& keep,
                                           TopkScratch* tks) {
  keep.t = topk_rank(K, tks);
  if ((int)__lane_id() < K) slot_pair[__lane_id()] = keep.t.srank;
}

// grid: one 4-wave block per compute unit (at most one wave per item).  Wave
// w takes items w, w + W, w + 2W, ...; the next item's loads go out before
// the current one is computed, so each wave streams its share with one item
// in flight while it computes.
// The gate_up pass of block blk of a grid of nblk 4-wave blocks (the kernel
// below, or a phase of the single-launch layer).
template <int NTOK, int TPR, int GPL, bool kRoute, bool kShared>
__device__ __forceinline__ void gate_up_body(const FfnArgs& a, const DecodeRoute& r, int blk,
                                             int nblk) {
  constexpr int kJ = kItemJ<GPL>;
  __shared__ DecMeta m;
  __shared__ TopkScratch tks[2];
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // one routed token: each wave ranks the selected experts once its first
  // items are in flight (route_rank)
  constexpr bool kLateRank = kRoute && NTOK == 1;
  __shared__ int slot_pair[kDecWaves][kMaxDecPairs];
  RouteKeep keep;
  if (kRoute)
    route_meta<NTOK>(a, r, m, keep, tks, blk);
  else
    load_meta(a, m);
  const int nU = uniform(m.n_union);
  const int nR = nU * (a.f / kJ);                 // routed items; then the shared expert's
  const int n_items = nR + (kShared ? a.fs / kJ : 0);
  const int W = nblk * kDecWaves;
  const int wid = blk * kDecWaves + wave;
  if (wid >= n_items) return;                     // no barrier follows
  // this lane's group of every token's prepped activations, loaded first:
  // they are few and cached, and the weight loads queue behind them
  const int G = a.d / 64, li = lane % TPR;
  uint4 xr[NTOK][GPL * 8];
  float2 xs[NTOK][GPL];
  float xa[NTOK];
#pragma unroll
  for (int t = 0; t < NTOK; ++t) {
    const int tt = min(t, a.B - 1);
#pragma unroll
    for (int gi = 0; gi < GPL; ++gi) {
      // a dead group (past the row) reads the last one: finite, weighted by 0
      const int grp = min(li + TPR * gi, G - 1);
      const uint4* src = reinterpret_cast<const uint4*>(a.xp + (int64_t)tt * a.d) + grp * 8;
#pragma unroll
      for (int q = 0; q < 8; ++q) xr[t][gi * 8 + q] = src[q];
      xs[t][gi] = a.xs[(int64_t)tt * G + grp];
    }
    xa[t] = a.xa[tt];
  }
  // a ring of kGuDepth items: item i computes while the next kGuDepth - 1
  // items of this wave (i + W, i + 2W, ...) are in flight.  Loads past the
  // end go to a dead offset (no memory access), so every item's bytes are
  // read once and the loop body stays straight-line.
  const int lane_expert = m.experts[min(lane, kMaxDecPairs - 1)];
  // h is staged in LDS and written out after the loop: a global store inside
  // the loop would count in vmcnt behind the ring's loads, and the compiler
  // waits for it (and so for every load before it) before reusing its data
  // registers.  The grid gives every wave at most kGuMaxItems items.
  __shared__ uint16_t hst[kDecWaves][kGuMaxItems][kJ * NTOK];
  const GuLane<TPR, GPL> lo = gu_lane<TPR, GPL>(a, lane);
  GuBuf<TPR, GPL> b[kGuDepth];
#pragma unroll
  for (int s = 0; s < kGuDepth - 1; ++s)
    gu_load<TPR, GPL, kShared>(a, lane_expert, wid + s * W, n_items, nR, lo, b[s]);
  for (int i = wid, loc = 0;; i += kGuDepth * W) {
#pragma unroll
    for (int s = 0; s < kGuDepth; ++s, ++loc) {
      const int it = i + s * W;
      if (it >= n_items) goto flush;
      gu_load<TPR, GPL, kShared>(a, lane_expert, it + (kGuDepth - 1) * W, n_items, nR, lo,
                                 b[(s + kGuDepth - 1) % kGuDepth]);
      if (kLateRank && loc == 0) route_rank(a.K, slot_pair[wave], keep, tks);
      gu_compute<NTOK, TPR, GPL, kShared>(a, m, it, nR, lane, b[s], xr, xs, xa, hst[wave][loc]);
    }
  }
flush:
  {
    // the wave's own LDS rows: the wave's LDS accesses are ordered
    const int n_mine = (n_items - wid + W - 1) / W;
    const int per = a.f / kJ;
    for (int q = lane; q < n_mine * kJ * NTOK; q += 64) {
      const int loc = q / (kJ * NTOK), rr = q % (kJ * NTOK);
      const int jj = rr / NTOK, k = rr % NTOK;
      const int item = wid + loc * W;
      if (kShared && item >= nR) {                // shared expert: pair k = token k
        const int j = (item - nR) * kJ + jj;
        if (k < a.B) a.shp[(int64_t)k * a.fs + prepped_pos(j)] = hst[wave][loc][rr];
        continue;
      }
      const int u = item / per;
      const int j = (item - u * per) * kJ + jj;
      const int pb = m.offsets[u];
      if (k < m.offsets[u + 1] - pb) {
        const int p = kLateRank ? slot_pair[wave][u] : m.pairs[pb + k];
        a.hp[(int64_t)p * a.f + prepped_pos(j)] = hst[wave][loc][rr];
      }
    }
  }
  if (kRoute && NTOK == 1 && blk == 0 && wave == 0) {
    // the single token's routing outputs, as smoe_route and smoe_build_union
    // would write them (pair k = rank k; union slot q = the q-th expert)
    const int K = a.K;
    const float w = topk_weight(keep.v, a.E, K, r.norm != 0, keep.t.my_v);
    if (lane < K) {
      r.topk_idx[lane] = keep.t.my_e;
      r.topk_w[lane] = w;
      r.union_experts[lane] = keep.t.se;
      r.expert_offsets[lane] = lane;
      r.pair_list[lane] = keep.t.srank;
      r.pair_pos[keep.t.srank] = lane;
    }
    if (lane == 0) {
      *r.n_union = K;
      r.expert_offsets[K] = K;
    }
    if (r.dec_meta != nullptr) {
      // the same, packed as DecMeta for the down kernel
      DecMeta* pm = reinterpret_cast<DecMeta*>(r.dec_meta);
      if (lane < K) {
        pm->experts[lane] = keep.t.se;
        pm->offsets[lane] = lane;
        pm->pairs[lane] = keep.t.srank;
        pm->pos[keep.t.srank] = lane;
        pm->w[lane] = w;
      }
      if (lane == 0) {
        pm->n_union = K;
        pm->offsets[K] = K;
      }
    }
  }
}

template <int NTOK, int TPR, int GPL, bool kRoute, bool kShared>
__global__ __launch_bounds__(kDecThreads) void k_gate_up_gemv(FfnArgs a, DecodeRoute r) {
  gate_up_body<NTOK, TPR, GPL, kRoute, kShared>(a, r, blockIdx.x, gridDim.x);
}

// grid: two 8-wave blocks per compute unit (at most one per row block);
// block b takes row blocks b, b + grid, ... of 8 output rows x all union
// experts, one (union slot, row block) item per wave, and ends each row block
// with the weighted combine of its rows in rank order.  The down pass of
// block blk of nblk blocks of kWaves waves (the kernel below, or a phase of
// the single-launch layer).
template <int NTOK, int NW, bool kShared, int kWaves>
__device__ __forceinline__ void down_body(const FfnArgs& a, int blk, int nblk) {
  __shared__ DecMeta m;
  __shared__ float ylds[(kShRow0 + 2 * kMaxShChunks) * kDnRows];
  const int wave = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // the first row block's residual, fetched before anything waits
  float res_pref = 0.f;
  if (a.residual != nullptr && (int)threadIdx.x < a.B * kDnRows)
    res_pref = a.residual[(int64_t)(threadIdx.x / kDnRows) * a.d + blk * kDnRows +
                          threadIdx.x % kDnRows];
  if (a.dec_meta_valid) {
    if (threadIdx.x < kDecMetaWords) reinterpret_cast<int*>(&m)[threadIdx.x] = a.dec_meta[threadIdx.x];
    __syncthreads();
  } else {
    load_meta(a, m);
  }
  const int nU = uniform(m.n_union);
  // the rows' chunks (one item each), so that items weigh about as much as
  // each other
  DnChunks g;
  dn_split(a.f / 8, NW, g.nr, g.wr);
  g.ns = 0, g.ws = 0;
  if (kShared) dn_split(a.fs / 8, NW, g.ns, g.ws);
  const int n_items = nU * g.nr + g.ns;
  const int n_rb = a.d / kDnRows;
  const int K = a.K;
  // 1/a_t^2 of the (at most two) tokens
  float ib[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float at = a.xa[min(t, a.B - 1)];
    ib[t] = 1.0f / (at * at);
  }
  for (int rb = blk; rb < n_rb; rb += nblk) {
    const int r0 = rb * kDnRows;
    for (int u = wave; u < n_items; u += kWaves) {
      DnItem<NTOK, NW> it;
      int ne, ys[NTOK];
      float ysc[NTOK];
      down_load<NTOK, NW, kShared>(a, m, u, nU, g, r0, lane, ib, it, ne, ys, ysc);
      down_compute<NTOK, NW>(ne, ys, ysc, lane, it, ylds);
    }
    __syncthreads();
    // combine: out[t, r] = residual[t, r] + sum_k w[t, k] * y[t*K + k, r], k
    // ascending, each y the sum of its chunks in order (with a shared expert:
    // residual + (shared + that sum)); a batch of eight pairs' values is read
    // before it is summed
    if ((int)threadIdx.x < a.B * kDnRows) {
      const int t = threadIdx.x / kDnRows, rr = threadIdx.x % kDnRows;
      float acc = 0.f;
      for (int k0 = 0; k0 < K; k0 += 8) {
        float yv[8], wv[8];
        int pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int p = t * K + min(k0 + j, K - 1);
          pv[j] = m.pos[p];
          wv[j] = m.w[p];
          const float* yp = ylds + p * kMaxRtChunks * kDnRows + rr;
          yv[j] = yp[0];
          for (int c = 1; c < g.nr; ++c) yv[j] += yp[c * kDnRows];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (k0 + j < K && pv[j] >= 0) acc += wv[j] * yv[j];
      }
      if (kShared) {
        // shared_out (its chunks in order) + routed_out
        float shv = 0.f;
        for (int c = 0; c < g.ns; ++c) shv += ylds[(kShRow0 + 2 * c + t) * kDnRows + rr];
        acc = shv + acc;
      }
      const int64_t o = (int64_t)t * a.d + r0 + rr;
      const float res = rb == blk ? res_pref : (a.residual ? a.residual[o] : 0.f);
      a.out[o] = res + acc;
    }
    // ylds is free again for the block's next row block (the barrier would
    // also wait for the stores above, so the last row block goes without)
    if (rb + nblk < n_rb) __syncthreads();
  }
}

template <int NTOK, int NW, bool kShared>
__global__ __launch_bounds__(kDnThreads) void k_down_combine_gemv(FfnArgs a) {
  down_body<NTOK, NW, kShared, kDnWaves>(a, blockIdx.x, gridDim.x);
}


template <int NTOK, int TPR, int GPL, bool kRoute>
hipError_t launch_gate_up_gemv(const FfnArgs& a, const DecodeRoute& r, hipStream_t s,
                               const LaunchTiming* t) {
  constexpr int kJ = kItemJ<GPL>;
  const int max_union = a.E < a.B * a.K ? a.E : a.B * a.K;
  const int items = max_union * (a.f / kJ) + a.fs / kJ;
  const int ncu = cu_count();
  if (ncu <= 0) return hipErrorInvalidDevice;
  // one block per CU, but enough blocks that no wave has more than
  // kGuMaxItems items (its LDS staging rows)
  const int per_block = kDecWaves * kGuMaxItems;
  const int grid = std::max(std::min((items + kDecWaves - 1) / kDecWaves, ncu * kGuBlocksPerCU),
                            (items + per_block - 1) / per_block);
  if (a.fs > 0)
    SMOE_LAUNCH(t, (k_gate_up_gemv<NTOK, TPR, GPL, kRoute, true>), dim3(grid), dim3(kDecThreads),
                0, s, a, r);
  else
    SMOE_LAUNCH(t, (k_gate_up_gemv<NTOK, TPR, GPL, kRoute, false>), dim3(grid), dim3(kDecThreads),
                0, s, a, r);
  return hipGetLastError();
}

// Lanes per row and groups per lane for a row of d inputs (G = d/64 groups):
// 32 lanes up to 32 groups, 64 lanes up to 64, then two groups a lane.
template <int NTOK, bool kRoute>
hipError_t launch_gate_up_ntok(const FfnArgs& a, const DecodeRoute& r, hipStream_t s,
                               const LaunchTiming* t) {
  const int G = a.d / 64;
  if (G <= 32) return launch_gate_up_gemv<NTOK, 32, 1, kRoute>(a, r, s, t);
  if (G <= 64) return launch_gate_up_gemv<NTOK, 64, 1, kRoute>(a, r, s, t);
  return launch_gate_up_gemv<NTOK, 64, 2, kRoute>(a, r, s, t);
}
template <bool kRoute>
hipError_t launch_gate_up_any(const FfnArgs& a, const DecodeRoute& r, hipStream_t s,
                              const LaunchTiming* t) {
  return a.B == 1 ? launch_gate_up_ntok<1, kRoute>(a, r, s, t)
                  : launch_gate_up_ntok<2, kRoute>(a, r, s, t);
}

// Words per lane: the fewest (1, 2, 4) whose 64-lane span holds a routed row.
template <int NTOK, int NW>
hipError_t launch_down_nw(const FfnArgs& a, hipStream_t s, const LaunchTiming* t) {
  const int ncu = cu_count();
  if (ncu <= 0) return hipErrorInvalidDevice;
  const int grid = std::min(a.d / kDnRows, ncu * kDnBlocksPerCU);
  if (a.fs > 0)
    SMOE_LAUNCH(t, (k_down_combine_gemv<NTOK, NW, true>), dim3(grid), dim3(kDnThreads), 0, s, a);
  else
    SMOE_LAUNCH(t, (k_down_combine_gemv<NTOK, NW, false>), dim3(grid), dim3(kDnThreads), 0, s, a);
  return hipGetLastError();
}
template <int NTOK>
hipError_t launch_down_gemv(const FfnArgs& a, hipStream_t s, const LaunchTiming* t) {
  const int words = a.f / 8;
  if (words <= 64) return launch_down_nw<NTOK, 1>(a, s, t);
  if (words <= 128) return launch_down_nw<NTOK, 2>(a, s, t);
  return launch_down_nw<NTOK, 4>(a, s, t);
}

// ------------------------------------------------ the single-launch layer
// The decode layer (B = 1) as one cooperative grid ("Data Flow", serial step
// trace: the routing, the experts and the combine of a step as one unit of
// work): the router's per-block items (the token's activation prep, each
// expert's gate matvec), a device-wide barrier, the gate_up pass (which ranks
// the logits and builds the union first), a second barrier, and the down pass
// with the combine, run by the same workgroups.  The barriers follow the
// memory model at device scope: the block's barrier orders its waves' stores
// before thread 0's acquire-release increment (a release is cumulative over
// what happens before it, so one increment releases the whole block), thread
// 0 waits for all blocks with relaxed loads and then acquires, and the
// block's second barrier orders that acquire before every wave's next reads
// (the caches it invalidates are the ones those waves read through).  One
// release and one acquire a block: a fence in every wave made each barrier
// several times slower.  A wait is bounded: past about
// 2^22 polls it sets SMOE_STATUS_SYNC_TIMEOUT and goes on, so the grid always
// drains.  Counters: status words kSingleBar .. +2 (two barriers, then an exit
// ticket whose last holder clears all three for the next launch).
constexpr int kSingleBar = 4;
constexpr int kSingleSpin = 1 << 22;

__device__ __forceinline__ void grid_sync(uint32_t* count, uint32_t nblk, uint32_t* status) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    int it = 0;
    while (__hip_atomic_load(count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < nblk) {
      if (++it > kSingleSpin) {
        __hip_atomic_fetch_or(status, (uint32_t)SMOE_STATUS_SYNC_TIMEOUT, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

template <int TPR, int NW, int kM>
__global__ __launch_bounds__(kDecThreads) void k_layer_single(RouteArgs ra, FfnArgs a,
                                                             DecodeRoute r) {
  static_assert(kDecThreads == kRouteThreads, "the router's items need 4-wave blocks");
  __shared__ float part[kRouteThreads / 64][1];
  const int blk = blockIdx.x, nblk = gridDim.x;
  uint32_t* bar = a.status + kSingleBar;
  // 1. the token's prep and the E gate matvecs, one item a block at a time
  for (int w = blk; w < 1 + ra.E; w += nblk) {
    if (w == 0)
      prep_token(ra.x, ra.d, 0, ra.xp, ra.xs, ra.xa, nullptr, 1.0f, &part[0][0]);
    else
      logits_block<true, 1, kM>(ra, w - 1, part);
    __syncthreads();                               // part is the next item's
  }
  grid_sync(bar, nblk, a.status);
  // 2. top-k, union and gate_up
  gate_up_body<1, TPR, 1, true, false>(a, r, blk, nblk);
  grid_sync(bar + 1, nblk, a.status);
  // 3. down and the combine
  down_body<1, NW, false, kDecWaves>(a, blk, nblk);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t =
        __hip_atomic_fetch_add(bar + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t == (uint32_t)nblk - 1) {                 // every block is past both barriers
#pragma unroll
      for (int i = 0; i < 3; ++i)
        __hip_atomic_store(bar + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int TPR, int NW, int kM>
hipError_t launch_single_t(const RouteArgs& ra, const FfnArgs& a, const DecodeRoute& r, int grid,
                           hipStream_t s) {
  RouteArgs ra_ = ra;
  FfnArgs a_ = a;
  DecodeRoute r_ = r;
  void* args[] = {&ra_, &a_, &r_};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(k_layer_single<TPR, NW, kM>),
                                    dim3(grid), dim3(kDecThreads), args, 0, s);
}

template <int TPR, int NW, int kM>
hipError_t single_fits(int grid, bool* ok) {
  int per_cu = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
      &per_cu, reinterpret_cast<const void*>(k_layer_single<TPR, NW, kM>), kDecThreads, 0);
  *ok = e == hipSuccess && per_cu * cu_count() >= grid;
  return e;
}

}  // namespace

bool single_layer_ok(const RouteArgs& ra, const FfnArgs& a) {
  return a.B == 1 && a.fs == 0 && ra.router_bf16 && ra.norm_out == nullptr && gemv_path_ok(a) &&
         (a.d == 2048 || a.d == 4096) && a.E + 1 <= 4096;
}

hipError_t launch_single_layer(const RouteArgs& ra, const FfnArgs& a, const DecodeRoute& r,
                               hipStream_t s) {
  // the gate_up pass's grid (launch_gate_up_gemv): one block per CU, or more
  // when a wave would hold more than kGuMaxItems items
  const int max_union = a.E < a.K ? a.E : a.K;
  const int items = max_union * (a.f / kItemJ<1>);
  const int ncu = cu_count();
  if (ncu <= 0) return hipErrorInvalidDevice;
  const int per_block = kDecWaves * kGuMaxItems;
  const int grid = std::max(std::min((items + kDecWaves - 1) / kDecWaves, ncu * kGuBlocksPerCU),
                            (items + per_block - 1) / per_block);
  const int words = a.f / 8;
  const int nw = words <= 64 ? 1 : words <= 128 ? 2 : 4;
  bool fits = false;
#define SMOE_SINGLE(TPR, NW, M)                                        \
  do {                                                                 \
    const hipError_t e = single_fits<TPR, NW, M>(grid, &fits);          \
    if (e != hipSuccess) return e;                                     \
    if (!fits) return hipErrorCooperativeLaunchTooLarge;               \
    return launch_single_t<TPR, NW, M>(ra, a, r, grid, s);             \
  } while (0)
  if (a.d == 2048) {
    if (nw == 1) SMOE_SINGLE(32, 1, 1);
    if (nw == 2) SMOE_SINGLE(32, 2, 1);
    SMOE_SINGLE(32, 4, 1);
  }
  if (nw == 1) SMOE_SINGLE(64, 1, 2);
  if (nw == 2) SMOE_SINGLE(64, 2, 2);
  SMOE_SINGLE(64, 4, 2);
#undef SMOE_SINGLE
}

// Compute units of the current device, cached per device (an attribute
// lookup, not state of any call).
int cu_count() {
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

// The decode path applies to B <= 2 tokens (B*K <= 16), d a multiple of 64
// up to 8192 (a gate_up row over 32 or 64 lanes, one or two groups a lane),
// f and fs multiples of 64 up to 8192 (down rows in at most 4 routed and 16
// shared chunks).
bool gemv_path_ok(const FfnArgs& a) {
  if (a.B < 1 || a.B > 2 || a.B * a.K > kMaxDecPairs) return false;
  if (a.d < 64 || a.d > 8192 || a.d % 64 != 0) return false;
  if (a.fs < 0 || a.fs > kMaxDecF || a.fs % 64 != 0) return false;
  return a.f >= 64 && a.f <= kMaxDecF && a.f % 64 == 0;
}

hipError_t launch_gemv(const FfnArgs& a, hipStream_t s, bool gate_up, const LaunchTiming* t) {
  if (gate_up) return launch_gate_up_any<false>(a, DecodeRoute{}, s, t);
  return a.B == 1 ? launch_down_gemv<1>(a, s, t) : launch_down_gemv<2>(a, s, t);
}

hipError_t launch_gate_up_routed(const FfnArgs& a, const DecodeRoute& r, hipStream_t s,
                                 const LaunchTiming* t) {
  return launch_gate_up_any<true>(a, r, s, t);
}

}  // namespace smoe
