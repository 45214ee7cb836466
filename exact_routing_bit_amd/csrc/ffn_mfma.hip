// ffn_mfma.hip - the token-batch expert FFN for prefill chunks (B >= 3).
//
// "Layer-Major Batched Prefill", step 6: every union expert is applied to all
// of its routed pairs in one pass over its weights (gate_up, then down).
// A workgroup serves one union expert and one 16-pair token tile; each of its
// four waves owns a unit of 64 weight rows and streams them over the whole
// input dimension, so an expert's bytes are read once per layer for up to 16
// pairs (an expert that serves more is streamed once per 16-pair tile).
//
//   gate_up unit: gate rows j0..j0+31 and up rows j0..j0+31 (four 16-row
//     tiles) -> h[pair, j0..j0+31] = silu(g) * u (prepped fp16) and the
//     half-group sums of h that the down pass needs;
//   down unit: down rows r0..r0+63 -> y[pair, r0..r0+63] (fp32).
//
// Arithmetic.  Per 64-input group g and 16-row tile, the dequantised words
// are the B operand of two v_mfma_f32_16x16x32_f16 (one per 32-input half),
// the pairs' prepped activations the A operand, and the group's scale and
// bias are applied in fp32 right after ("SSD Streaming Expert Layers",
// "Quantized Layout": w = s*q + b):
//     acc += s * (D - C) + b * X,   D = sum_k (1024 + m q_k) stored_k,
// with the MFMA accumulator seeded by -C so that D - C comes straight out.
//
// Memory.  Everything a stage of two groups needs - the wave's 64 rows x 64
// bytes of packed words, their scales and biases, the tile's activations and
// group sums - is copied global -> LDS by the DMA path (global_load_lds, 16
// bytes a lane for the words and activations), three stages deep.  The copies
// hold no registers while in flight, so each wave keeps two stages (8 KB of
// weights) in the air while it computes on the third, and the words arrive
// as whole 64-byte row segments however the MFMA wants them laid out.  The
// activations and sums of a stage are shared by the four waves (one copy
// instruction each) behind one workgroup barrier per stage.  Scales and
// biases (kFastSB: up to 64 groups, 16-byte aligned rows) are read once per
// workgroup into registers, four lanes per row reading its run of bytes in
// one piece, and handed to the lanes that use them with ds_bpermute every
// four stages; reading them 16 bytes a row every four stages instead made
// scattered small requests that cost more than the packed words.  Otherwise
// one aligned dword per row and group is copied each stage.
#include "device.hpp"
#include "smoe_internal.hpp"

namespace smoe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTiles = 4;                          // 16-row tiles per wave (64 rows)
constexpr int kPairTile = 16;                      // pairs per token tile (MFMA M)
constexpr int kMaxTiles = kMaxBatch / kPairTile;   // token tiles of the widest pass (64 pairs)
constexpr int kGps = 2;                            // groups per pipeline stage
constexpr int kSuper = 4;                          // stages per scale/bias handout (kFastSB)
static_assert(kMaxTiles == 4, "a wide pass holds every pair of a 64-token chunk");

// A pass streams one unit of weight rows once and applies it to NT token
// tiles (16 NT pairs).  An expert with at most 16 pairs takes the narrow
// pass (NT = 1, a ring of three stages); one with more (at most 64: every
// token of the chunk) the wide pass (NT = 4, two stages), so that every
// expert's bytes are read once per layer.
//
// One ring slot (one stage).  Layouts, 16-byte entries unless noted:
//   W  [wave][tile][chunk 4][row 16]    chunk c = group c/2, words 4(c%2)..+3
//   A  [token tile NT][word 16][pair 16]   prepped activations of one word
//   XS f32, gate_up: [group 2][X|C][token tile NT][pair 16]
//           down:    [group 2][half 2][token tile NT][X|C][pair 16]
//   SB [wave][s|b][group 2][col 16][tile 4]          u32, the aligned dword
//                                        holding that row's bf16 s (or b)
//                                        (only without kFastSB)
// kFastSB keeps scales and biases in registers (see the pass).
constexpr int kWBytes = kWaves * kTiles * 1024;
constexpr int kABytes = 16 * kPairTile * 16;       // per token tile
constexpr int kXSBytes = kGps * 2 * 2 * kPairTile * 4;   // per token tile
constexpr int kSBSlotBytes = kWaves * 2 * kGps * 256;
constexpr int kOffA = kWBytes;
template <int NT>
constexpr int off_xs() { return kOffA + NT * kABytes; }
template <int NT>
constexpr int off_sb() { return off_xs<NT>() + NT * kXSBytes; }
template <bool kFastSB, int NT>
constexpr int slot_bytes() { return off_sb<NT>() + (kFastSB ? 0 : kSBSlotBytes); }
// the narrow pass (fast scale/bias variant, three stages) and the wide pass
// (scales and biases through the slots, two stages) share the LDS buffer
template <bool kFastSB>
constexpr int ring_bytes() {
  return 3 * slot_bytes<kFastSB, 1>() > 2 * slot_bytes<false, kMaxTiles>()
             ? 3 * slot_bytes<kFastSB, 1>()
             : 2 * slot_bytes<false, kMaxTiles>();
}

// Copy instructions per wave and stage: words (one per tile), activations
// (one per token tile), sums (gate_up: one; down: one per two token tiles)
// and, without kFastSB, the scale/bias dwords.
template <bool kGateUp, bool kFastSB, int NT>
constexpr int copies_of_rest() {
  return NT + (kGateUp ? 1 : (NT + 1) / 2) + (kFastSB ? 0 : 2 * kGps);
}
template <bool kGateUp, bool kFastSB, int NT>
constexpr int copies_of_stage() {
  return kTiles + copies_of_rest<kGateUp, kFastSB, NT>();
}

// Per-lane copy sources that stay fixed over the K loop.
template <int NT>
struct Sources {
  const uint32_t* w[kTiles];   // row (tile T, lane%16), chunk half (lane/16)%2
  const uint16_t* s;           // scales of this lane's copy row (group 0)
  const uint16_t* b;           // biases of the same row
  const uint4* act[NT];        // token tile n: activation row of pair lane%16,
                               // word 4(wave%2) + lane/16
  const float* sums[(NT + 1) / 2];   // group sums (see issue_rest)
};

__device__ __forceinline__ const void* align4(const uint16_t* p) {
  return reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(p) & ~(uintptr_t)3);
}

// Copies of stage k (groups gA = 2k and gB = min(2k+1, G-1)) into `slot`:
// the packed words (issue_words, kTiles copies) and the rest (issue_rest:
// activations, sums and, without kFastSB, the scale/bias dwords).
// Stage k copies bytes 64k .. 64k+63 of every row: with rows that start on a
// 128-byte line (line_aligned), an even stage reads the first half of its
// lines and the next (odd) stage the second half, which is then the line's
// last use: that copy carries the nontemporal hint, so that the streamed
// weights leave the L2 first and the activations that every workgroup of an
// expert re-reads stay in it.
// uoff: words from the pass's first unit of rows to the one being streamed.
template <int NT>
__device__ __forceinline__ void issue_words(const Sources<NT>& S, char* slot, int k, int G,
                                            int wave, int lane, bool line_aligned,
                                            int64_t uoff = 0) {
  const int gA = 2 * k, gB = min(2 * k + 1, G - 1);
  // packed words: lanes 0-31 copy group gA, lanes 32-63 group gB
  const int gw = (lane >> 5) ? gB : gA;
  if (line_aligned && (k & 1)) {
#pragma unroll
    for (int T = 0; T < kTiles; ++T)
      dma16_to_lds_nt(S.w[T] + uoff + gw * 8, slot + (wave * kTiles + T) * 1024);
  } else {
#pragma unroll
    for (int T = 0; T < kTiles; ++T)
      dma16_to_lds(S.w[T] + uoff + gw * 8, slot + (wave * kTiles + T) * 1024);
  }
}
template <bool kGateUp, bool kFastSB, int NT>
__device__ __forceinline__ void issue_rest(const Sources<NT>& S, char* slot, int k, int G,
                                           int wave, int lane) {
  const int gA = 2 * k, gB = min(2 * k + 1, G - 1);
  // activations: waves 0,1 (mod 4) copy the words of group gA, waves 2,3
  // those of gB (with more than four waves, the others copy the same bytes
  // again, so that every wave issues the same copies)
  const int wq = wave & 3;
  const int ga = wq < 2 ? gA : gB;
#pragma unroll
  for (int n = 0; n < NT; ++n)
    dma16_to_lds(S.act[n] + ga * 8, slot + kOffA + n * kABytes + wq * 1024);
  // group sums: wq = 2 * group + (gate_up: X|C, down: half); lane L covers
  // token tile L/16 (gate_up) or, per copy c, tile 2c + L/32 with X|C (L/16)%2
  if (kGateUp) {
    if (lane < 16 * NT) dma4_to_lds(S.sums[0] + ga * 2, slot + off_xs<NT>() + wq * NT * 64);
  } else {
#pragma unroll
    for (int c = 0; c < (NT + 1) / 2; ++c)
      if (lane < 32 * min(2, NT - 2 * c))
        dma4_to_lds(S.sums[c] + ga * 4, slot + off_xs<NT>() + wq * NT * 128 + c * 256);
  }
  if (!kFastSB) {
    // one dword a lane, the aligned one that holds the value
    char* sb = slot + off_sb<NT>() + wave * (2 * kGps * 256);
    dma4_to_lds(align4(S.s + gA), sb);
    dma4_to_lds(align4(S.s + gB), sb + 256);
    dma4_to_lds(align4(S.b + gA), sb + 512);
    dma4_to_lds(align4(S.b + gB), sb + 768);
  }
}
// The uint4 that lane src/4 holds in v.
__device__ __forceinline__ uint4 bpermute4(int src, const uint4& v) {
  return make_uint4((uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.x),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.y),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.z),
                    (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.w));
}

// bf16 in the upper (hi) or lower half of a dword, as fp32
__device__ __forceinline__ float bf16_half(uint32_t w, bool hi) {
  return __uint_as_float(hi ? (w & 0xFFFF0000u) : (w << 16));
}

// Scales and biases of this lane's rows, kFastSB: 8 groups of tile T in
// sbw[T] (u16 pairs), biases in bbw[T].
struct SBRegs {
  uint4 s[kTiles], b[kTiles];
};

// acc[T][n] += s (D - C) + b X over the two groups of stage k, token tile n.
//   kFastSB: scales/biases from `regs` (groups 8j.. of the current four stages,
//            kk = k % 4 static);
//   else:    from the slot, with `parity` bit T (scales) and 4 + T (biases) =
//            the u16 address parity of group 0 of this lane's row in tile T.
// Each group's words are dequantised once and used for every token tile.
template <bool kGateUp, bool kFastSB, int NT, int kk>
__device__ __forceinline__ void compute_stage(const char* slot, int k, int G, int wave, int col,
                                              int lg, const SBRegs& regs, uint32_t parity,
                                              floatx4 (&acc)[kTiles][NT]) {
#pragma unroll
  for (int gl = 0; gl < kGps; ++gl) {
    const bool live = kFastSB || 2 * k + gl < G;   // uniform; a clamped copy otherwise
    uint32_t sw[kTiles], bw[kTiles];
    if (kFastSB) {
#pragma unroll
      for (int T = 0; T < kTiles; ++T) {
        const uint32_t sv[4] = {regs.s[T].x, regs.s[T].y, regs.s[T].z, regs.s[T].w};
        const uint32_t bv[4] = {regs.b[T].x, regs.b[T].y, regs.b[T].z, regs.b[T].w};
        sw[T] = sv[kk];                            // groups 2kk, 2kk+1 of the eight
        bw[T] = bv[kk];
      }
    } else {
      const char* sb = slot + off_sb<NT>() + wave * (2 * kGps * 256) + gl * 256 + col * 16;
      const uint4 s4 = *reinterpret_cast<const uint4*>(sb);
      const uint4 b4 = *reinterpret_cast<const uint4*>(sb + 512);
      sw[0] = s4.x; sw[1] = s4.y; sw[2] = s4.z; sw[3] = s4.w;
      bw[0] = b4.x; bw[1] = b4.y; bw[2] = b4.z; bw[3] = b4.w;
    }
    const char* wrow =
        slot + (wave * kTiles) * 1024 + ((2 * gl + (lg >> 1)) * 16 + col) * 16 + (lg & 1) * 8;
    float sc[kTiles], bi[kTiles];
#pragma unroll
    for (int T = 0; T < kTiles; ++T) {
      const bool shi = kFastSB ? gl == 1 : (((parity >> T) & 1) ^ gl) != 0;
      const bool bhi = kFastSB ? gl == 1 : (((parity >> (4 + T)) & 1) ^ gl) != 0;
      sc[T] = live ? bf16_half(sw[T], shi) : 0.f;
      bi[T] = live ? bf16_half(bw[T], bhi) : 0.f;
    }
    // one token tile: each row tile's words dequantised as they are used;
    // several: dequantised once for all of them
    half8_t w0[NT == 1 ? 1 : kTiles], w1[NT == 1 ? 1 : kTiles];
    if (NT > 1) {
#pragma unroll
      for (int T = 0; T < kTiles; ++T) {
        const uint2 w2 = *reinterpret_cast<const uint2*>(wrow + T * 1024);
        w0[NT == 1 ? 0 : T] = word_operand(w2.x);
        w1[NT == 1 ? 0 : T] = word_operand(w2.y);
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const char* an = slot + kOffA + n * kABytes;
      const half8_t A0 = *reinterpret_cast<const half8_t*>(an + ((gl * 8 + 2 * lg) * 16 + col) * 16);
      const half8_t A1 =
          *reinterpret_cast<const half8_t*>(an + ((gl * 8 + 2 * lg + 1) * 16 + col) * 16);
      floatx4 X, Cs;
      if (kGateUp) {
        const char* xs = slot + off_xs<NT>() + (gl * 2 * NT + n) * 64 + 16 * lg;
        X = *reinterpret_cast<const floatx4*>(xs);
        Cs = *reinterpret_cast<const floatx4*>(xs + NT * 64);
      } else {
        const char* xs = slot + off_xs<NT>() + (gl * 2 * NT + n) * 128 + 16 * lg;
        const int hstep = NT * 128;                 // half 0 -> half 1
        X = *reinterpret_cast<const floatx4*>(xs) + *reinterpret_cast<const floatx4*>(xs + hstep);
        Cs = *reinterpret_cast<const floatx4*>(xs + 64) +
             *reinterpret_cast<const floatx4*>(xs + hstep + 64);
      }
      const floatx4 seed = -Cs;
#pragma unroll
      for (int T = 0; T < kTiles; ++T) {
        half8_t o0, o1;
        if (NT == 1) {
          const uint2 w2 = *reinterpret_cast<const uint2*>(wrow + T * 1024);
          o0 = word_operand(w2.x);
          o1 = word_operand(w2.y);
        } else {
          o0 = w0[NT == 1 ? 0 : T];
          o1 = w1[NT == 1 ? 0 : T];
        }
        floatx4 D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, o0, seed, 0, 0, 0);
        D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, o1, D, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[T][n][i] = __builtin_fmaf(sc[T], D[i], acc[T][n][i]);
          acc[T][n][i] = __builtin_fmaf(bi[T], X[i], acc[T][n][i]);
        }
      }
    }
  }
}

// Waits until every copy of this wave for stage k has landed, allowing (some
// of) the copies of the stages issued after it to stay in flight.  Issue
// order: the words of stages 0 .. R-2, then their rest (the prologue), then
// in stage j's iteration the words and rest of stage j + R - 1.  In the
// steady state (k >= R-2, and R-2 later stages issued) exactly R-2 full
// stages follow stage k's copies; before it (R = 3, k = 0) the next stage's
// rest; at the end nothing.  Three cases only: more branches in the
// unrolled stage loop made the compiler spill.
template <int kRest, int kStage, int kRingN>
__device__ __forceinline__ void wait_stage(int k, int nst) {
  if (k >= kRingN - 2 && k + kRingN - 2 < nst)
    wait_vmcnt<(kRingN - 2) * kStage>();
  else if (k < kRingN - 2 && k + 1 < nst)
    wait_vmcnt<kRest>();
  else
    wait_vmcnt<0>();
}

// What a workgroup's pass needs to know about its expert (or the shared one).
struct PassCtx {
  bool sh;                 // the shared expert (pair q = token q)
  int e, pb, ne;           // expert, first pair in pair_list, pair count (>= 1)
  int F, Kt;               // the expert's width; pair q serves token q / Kt
  QMat qg, qu, qd;
  uint16_t* hp;
  float2* hs;
  float* yout;
  int unit;                // this wave's unit of rows
  bool has_unit;           // false: a copy of the last unit, nothing written
  int unit2;               // a second unit streamed right after the first (kU = 2)
  bool has_unit2;
};

// The whole pass of one wave's unit over the expert's K dimension for its
// pairs, in passes of 16 NT pairs (one pass when NT = 4), kRingN stages in
// the ring.  kU = 2 (the narrow down pass over at most 32 groups, a multiple
// of eight): the wave streams a second unit (c.unit2) right behind the first
// through the same ring, so that one fill and one drain serve both; the
// first unit's accumulators are held until the end, and its scales and
// biases take the register half that more than 32 groups would use.
template <bool kGateUp, bool kFastSB, int NT, int kRingN, int kU = 1>
__device__ __forceinline__ void ffn_pass(const FfnArgs& a, const PassCtx& c, char* ring,
                                         int* lpair) {
  constexpr int kSlot = slot_bytes<kFastSB, NT>();
  constexpr int kRest = copies_of_rest<kGateUp, kFastSB, NT>();
  constexpr int kStage = copies_of_stage<kGateUp, kFastSB, NT>();
  static_assert(kRingN == 2 || kRingN == 3, "two or three stages in the ring");
  static_assert(kU == 1 || (kU == 2 && !kGateUp && kFastSB && NT == 1),
                "two units: the narrow down pass with scales in registers");
  const int K = kGateUp ? a.d : c.F;
  const int G = K / 64, C = K / 8;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, lg = lane >> 4;
  const int e = c.e, ne = c.ne, F = c.F, Kt = c.Kt;
  const QMat &qg = c.qg, &qu = c.qu, &qd = c.qd;
  int rows0[kTiles];
#pragma unroll
  for (int T = 0; T < kTiles; ++T)
    rows0[T] = kGateUp ? c.unit * 32 + (T & 1) * 16 : c.unit * 64 + T * 16;

  Sources<NT> S;
#pragma unroll
  for (int T = 0; T < kTiles; ++T) {
    const QMat& m = kGateUp ? (T < 2 ? qg : qu) : qd;   // T is a constant here
    S.w[T] = m.w + e * m.stride_w + (int64_t)(rows0[T] + (lane & 15)) * C + ((lane >> 4) & 1) * 4;
  }
  {
    // scale/bias copy row of this lane: kFastSB (tile lane/16, col lane%16),
    // else (tile lane%4, col lane/4)
    const int T = kFastSB ? lane >> 4 : lane & 3;
    const int r = kFastSB ? lane & 15 : lane >> 2;
    const bool up = kGateUp && T >= 2;
    const uint16_t* s0 = kGateUp ? qg.s : qd.s;
    const uint16_t* b0 = kGateUp ? qg.b : qd.b;
    const int64_t st0 = kGateUp ? qg.stride_sb : qd.stride_sb;
    const uint16_t* sp = up ? qu.s : s0;
    const uint16_t* bp = up ? qu.b : b0;
    const int64_t stride = up ? qu.stride_sb : st0;
    const int row = (kGateUp ? c.unit * 32 + (T & 1) * 16 : c.unit * 64 + T * 16) + r;
    S.s = sp + e * stride + (int64_t)row * G;
    S.b = bp + e * stride + (int64_t)row * G;
  }
  uint32_t parity = 0;                             // see compute_stage
  if (!kFastSB) {
#pragma unroll
    for (int T = 0; T < kTiles; ++T) {
      const QMat& m = kGateUp ? (T < 2 ? qg : qu) : qd;
      const int64_t first = e * m.stride_sb + (int64_t)(rows0[T] + col) * G;
      parity |= (uint32_t)((reinterpret_cast<uintptr_t>(m.s + first) >> 1) & 1) << T;
      parity |= (uint32_t)((reinterpret_cast<uintptr_t>(m.b + first) >> 1) & 1) << (4 + T);
    }
  }
  const int nst = (G + kGps - 1) / kGps;
  const int nstT = kU * nst;                       // stages of the whole pass
  // the second unit: rows and words past the first (kU = 2)
  const int rdu = kU == 2 ? (c.unit2 - c.unit) * 64 : 0;
  const int64_t du = (int64_t)rdu * C;
  // rows of C words start on 128-byte lines when every expert's matrix does
  bool line_aligned = (C * 4) % 128 == 0;
#pragma unroll
  for (int T = 0; T < kTiles; ++T) {
    const QMat& m = kGateUp ? (T < 2 ? qg : qu) : qd;
    line_aligned = line_aligned && (reinterpret_cast<uintptr_t>(m.w + e * m.stride_w) & 127) == 0;
  }
  // One pass: the narrow pass serves at most 16 pairs and the wide one at
  // most 64, every token of a chunk (pass m0 = 0 of 16 NT pair slots).
  constexpr int m0 = 0;
  __syncthreads();                                 // a previous pass is done with the ring
  // The start's three independent reads go out together instead of one after
  // another: the pass's pair ids (copied like the rest, so that no
  // compiler-counted load sits behind the copies; lane L: pair slot L of the
  // 16 NT), the first stages' words (they need only the expert) and, with
  // kFastSB, this wave's scales and biases for the whole K loop.  Those are
  // read once as contiguous runs (lane l: row rows0[T] + l/4, 16-byte piece
  // 4h + l%4 of the row's G/8), not as 16-byte pieces of 64 rows per four
  // stages; each group of four stages hands every lane its rows' piece with
  // ds_bpermute.  They are the last loads issued, so the compiler's wait for
  // them (it counts only its own loads) also covers the copies before them.
  if (lane < kPairTile * NT) {
    if (c.sh)
      lpair[lane] = min(m0 + lane, ne - 1);        // the shared expert's pairs are the tokens
    else
      dma4_to_lds(a.pair_list + c.pb + min(m0 + lane, ne - 1), lpair);
  }
  issue_words<NT>(S, ring, 0, G, wave, lane, line_aligned);
  if (kRingN >= 3 && nstT > 1) issue_words<NT>(S, ring + kSlot, 1, G, wave, lane, line_aligned);
  uint4 sbs[kTiles][2], sbb[kTiles][2];
  if (kFastSB) {
    const int P = G / 8;                           // <= 8 pieces a row (G <= 64)
#pragma unroll
    for (int T = 0; T < kTiles; ++T) {
      const QMat& m = kGateUp ? (T < 2 ? qg : qu) : qd;
      const int64_t row = rows0[T] + (lane >> 2);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // kU = 2 (P <= 4): half h holds unit h's pieces
        const int piece = kU == 2 ? (lane & 3) : 4 * h + (lane & 3);
        const int pc = piece < P ? piece : 0;      // a valid address; the value is unused
        const int64_t at = e * m.stride_sb + (row + (h == 1 ? rdu : 0)) * G + pc * 8;
        sbs[T][h] = *reinterpret_cast<const uint4*>(m.s + at);
        sbb[T][h] = *reinterpret_cast<const uint4*>(m.b + at);
      }
    }
    // wait for them here, while only these copies are in flight
#pragma unroll
    for (int T = 0; T < kTiles; ++T)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        asm volatile("" ::"v"(sbs[T][h].x), "v"(sbs[T][h].y), "v"(sbs[T][h].z), "v"(sbs[T][h].w));
        asm volatile("" ::"v"(sbb[T][h].x), "v"(sbb[T][h].y), "v"(sbb[T][h].z), "v"(sbb[T][h].w));
      }
  }
  {
    // the pair ids landed (the words of the prologue stages behind them)
    if (kRingN >= 3 && nstT > 1) wait_vmcnt<2 * kTiles>();
    else wait_vmcnt<kTiles>();
    // the token scales a_t of the pairs this lane's accumulators hold (pair
    // slots 16 n + 4 lg + i), used in the epilogue only: one token tile reads
    // them here, under the first copies; several read them in the epilogue
    // (held across the K loop, 16 of them cost registers)
    float tsc1[4];
    if (NT == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) tsc1[i] = a.xa[lpair[4 * lg + i] / Kt];
    }
    {
      const int word = 4 * (wave & 1) + (lane >> 4);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int q = lpair[16 * n + (lane & 15)];
        S.act[n] = kGateUp ? reinterpret_cast<const uint4*>(a.xp + (int64_t)(q / Kt) * a.d) + word
                           : reinterpret_cast<const uint4*>(c.hp + (int64_t)q * F) + word;
      }
      if (kGateUp) {
        // lane L: pair slot L (token tile L/16), X or C by wave & 1
        const int q = lpair[min(lane, kPairTile * NT - 1)];
        S.sums[0] = reinterpret_cast<const float*>(a.xs) + (int64_t)(q / Kt) * G * 2 + (wave & 1);
      } else {
        // copy cc, lane L: pair slot 32 cc + L%16 + 16 (L/32), X|C (L/16)%2,
        // half wave & 1
#pragma unroll
        for (int cc = 0; cc < (NT + 1) / 2; ++cc) {
          const int slotp = min(32 * cc + 16 * (lane >> 5) + (lane & 15), kPairTile * NT - 1);
          const int q = lpair[slotp];
          S.sums[cc] = reinterpret_cast<const float*>(c.hs) + (int64_t)q * G * 4 + (wave & 1) * 2 +
                       ((lane >> 4) & 1);
        }
      }
    }
    floatx4 acc[kTiles][NT], acc1[kTiles][NT];     // acc1: the first unit's, when kU = 2
#pragma unroll
    for (int T = 0; T < kTiles; ++T)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[T][n] = floatx4{0.f, 0.f, 0.f, 0.f};
    SBRegs regs;

    issue_rest<kGateUp, kFastSB, NT>(S, ring, 0, G, wave, lane);
    if (kRingN >= 3 && nstT > 1) issue_rest<kGateUp, kFastSB, NT>(S, ring + kSlot, 1, G, wave, lane);
    // stages in fours so that the stage's place in its four is a constant (with
    // two units, nst is a multiple of four: the place is the same in either)
    for (int ks = 0; ks < nstT; ks += kSuper) {
#define SMOE_MFMA_STAGE(kk)                                                                       \
      if (ks + kk < nstT) {                                                                       \
        const int k = ks + kk;                                                                    \
        const int ui = (kU == 2 && k >= nst) ? 1 : 0;  /* unit of stage k, its stage kl */        \
        const int kl = k - ui * nst;                                                              \
        wait_stage<kRest, kStage, kRingN>(k, nstT);  /* this wave's copies of stage k landed */   \
        const int kn = k + kRingN - 1;  /* the stage whose copies go out now */                   \
        const int un = (kU == 2 && kn >= nst) ? 1 : 0;                                            \
        const int knl = kn - un * nst;                                                            \
        /* this wave's words of stage kn go to its own part of slot k-1, which */                \
        /* only it reads (its compute of k-1 is done): no need to wait for the others */         \
        if (kn < nstT)                                                                            \
          issue_words<NT>(S, ring + (kn % kRingN) * kSlot, knl, G, wave, lane, line_aligned,      \
                          un * du);                                                               \
        barrier_no_wait();           /* every wave's copies of k landed; slot k-1 is free */      \
        if (kn < nstT)                                                                            \
          issue_rest<kGateUp, kFastSB, NT>(S, ring + (kn % kRingN) * kSlot, knl, G, wave, lane);  \
        if (kFastSB && kk == 0) {                                                                 \
          const int j = kl / kSuper;                 /* groups 8j .. 8j+7: piece j */             \
          const int src = (col * 4 + (j & 3)) * 4;   /* lane holding this row's piece j */        \
          const int hh = kU == 2 ? ui : (j < 4 ? 0 : 1);                                          \
          _Pragma("unroll") for (int T = 0; T < kTiles; ++T) {                                   \
            regs.s[T] = bpermute4(src, hh == 0 ? sbs[T][0] : sbs[T][1]);                          \
            regs.b[T] = bpermute4(src, hh == 0 ? sbb[T][0] : sbb[T][1]);                          \
          }                                                                                       \
        }                                                                                         \
        if (kU == 2 && k == nst) {   /* the second unit starts: hold the first's sums */          \
          _Pragma("unroll") for (int T = 0; T < kTiles; ++T) {                                   \
            acc1[T][0] = acc[T][0];                                                               \
            acc[T][0] = floatx4{0.f, 0.f, 0.f, 0.f};                                              \
          }                                                                                       \
        }                                                                                         \
        compute_stage<kGateUp, kFastSB, NT, kk>(ring + (k % kRingN) * kSlot, kl, G, wave, col,    \
                                                lg, regs, parity, acc);                           \
      }
      SMOE_MFMA_STAGE(0)
      SMOE_MFMA_STAGE(1)
      SMOE_MFMA_STAGE(2)
      SMOE_MFMA_STAGE(3)
#undef SMOE_MFMA_STAGE
    }
    if (!c.has_unit) return;

    // epilogue: lane holds (pair slot m0 + 16 n + 4 lg + i, row rows0[T] + col)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float tsc[4];                                  // a_t of the lane's pairs
#pragma unroll
      for (int i = 0; i < 4; ++i) tsc[i] = NT == 1 ? tsc1[i] : a.xa[lpair[16 * n + 4 * lg + i] / Kt];
      if (kGateUp) {
        // h for columns j = unit*32 + Th*16 + col, from gate tile Th and up tile Th+2
        float X[4] = {0.f, 0.f, 0.f, 0.f}, Sm[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int Th = 0; Th < 2; ++Th) {
          const int j = c.unit * 32 + Th * 16 + col;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int ms = 16 * n + 4 * lg + i;      // pair slot in the pass
            // the sums were taken over a_t x: 1/a_t (exact) gives g and u, and
            // h is stored as a_t^2 h
            const float at = tsc[i], ia = 1.0f / at;
            const float h = silu_mul(acc[Th][n][i] * ia, acc[Th + 2][n][i] * ia) * (at * at);
            const half_t xi = (half_t)h;
            const half_t stv = (j & 1) ? (half_t)((float)xi * 0.0625f) : xi;
            const float stf = (float)stv;
            Sm[i] += stf;
            X[i] += (j & 1) ? stf * 16.0f : stf;
            if (m0 + ms < ne) {
              const int nn = j & 7;
              c.hp[(int64_t)lpair[ms] * F + (j & ~7) + 2 * (nn & 3) + (nn >> 2)] = f16_bits(stv);
            }
          }
        }
        // sums over the unit's 32 columns: the 16 lanes of a row segment
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float Xt = segment_sum16(X[i], 16), St = segment_sum16(Sm[i], 16);
          const int ms = 16 * n + 4 * lg + i;
          if (col == 0 && m0 + ms < ne) {
            const int j0 = c.unit * 32;
            c.hs[((int64_t)lpair[ms] * (F / 64) + j0 / 64) * 2 + (j0 % 64) / 32] =
                make_float2(Xt, 1024.0f * St);
          }
        }
      } else {
        // h held a_t^2 h: 1/a_t^2 (exact) gives the outputs (kU = 2: the
        // first unit from its held sums, the second one rdu rows further)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ms = 16 * n + 4 * lg + i;
          const float ib = 1.0f / (tsc[i] * tsc[i]);
          if (m0 + ms < ne) {
#pragma unroll
            for (int T = 0; T < kTiles; ++T)
              c.yout[(int64_t)lpair[ms] * a.d + rows0[T] + col] =
                  (kU == 2 ? acc1[T][n][i] : acc[T][n][i]) * ib;
            if (kU == 2 && c.has_unit2) {
#pragma unroll
              for (int T = 0; T < kTiles; ++T)
                c.yout[(int64_t)lpair[ms] * a.d + rows0[T] + rdu + col] = acc[T][n][i] * ib;
            }
          }
        }
      }
    }
  }
}

// kU = 2 (down only): every wave takes two units, four apart, so that a
// block covers 4 kU units.
template <bool kGateUp, bool kFastSB, int kU>
__global__ __launch_bounds__(kThreads, 2) void k_ffn_mfma(FfnArgs a) {
  __shared__ __align__(16) char ring[ring_bytes<kFastSB>()];
  __shared__ int lpair_w[kWaves][kPairTile * kMaxTiles];   // each wave's copy of the pass's pair ids
  // The grid is one row of blocks for the shared expert (if the layer has
  // one: every token is one of its pairs, pair q = token q), then one row per
  // union slot, laid out one after another along x: bx is the block within
  // its row (kWaves units each), u its row.  The shared row goes first, as
  // its blocks serve the most pairs.
  const int units_r = kGateUp ? a.f / 32 : a.d / 64;
  const int units_s = kGateUp ? a.fs / 32 : a.d / 64;
  constexpr int kUB = kWaves * kU;                // units a block
  const int gx_r = (units_r + kUB - 1) / kUB, gx_s = (units_s + kUB - 1) / kUB;
  const int n_sh = a.fs > 0 ? 1 : 0;
  const int b_lin = blockIdx.x;
  const bool sh = b_lin < n_sh * gx_s;
  const int b_r = b_lin - n_sh * gx_s;
  const int u = sh ? -1 : b_r / gx_r;
  const int bx = sh ? b_lin : b_r - u * gx_r;
  const int ul = sh ? 0 : u;
  // the union's size and this slot's expert and offsets in one round trip (slot
  // u < the largest union is always inside the union arrays)
  const int nU = *a.n_union;
  const int e_ld = a.union_experts[ul];
  const int pb_ld = a.expert_offsets[ul];
  const int pe_ld = a.expert_offsets[ul + 1];
  if (!sh && u >= nU) return;
  PassCtx c;
  c.sh = sh;
  c.e = sh ? 0 : e_ld;
  c.pb = sh ? 0 : pb_ld;
  c.ne = sh ? a.B : pe_ld - pb_ld;                 // 1 .. B <= 64
  c.F = sh ? a.fs : a.f;
  c.Kt = sh ? 1 : a.K;
  c.qg = sh ? a.sgate : a.gate;
  c.qu = sh ? a.sup : a.up;
  c.qd = sh ? a.sdown : a.down;
  c.hp = sh ? a.shp : a.hp;
  c.hs = sh ? a.shs : a.hs;
  c.yout = sh ? a.sy : a.y;
  // this wave's unit; waves past the last unit run along on a copy of the
  // last one (they take part in the shared copies and barriers) and write nothing
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int units = sh ? units_s : units_r;
  c.has_unit = bx * kUB + wave < units;
  c.unit = min(bx * kUB + wave, units - 1);
  c.has_unit2 = kU == 2 && bx * kUB + kWaves + wave < units;
  c.unit2 = kU == 2 ? min(bx * kUB + kWaves + wave, units - 1) : c.unit;
  int* lpair = lpair_w[wave];
  if (__builtin_amdgcn_readfirstlane(c.ne) > kPairTile) {
    // the wide pass, unit by unit
    ffn_pass<kGateUp, false, kMaxTiles, 2>(a, c, ring, lpair);
    if (kU == 2) {
      PassCtx c2 = c;
      c2.unit = c.unit2;
      c2.has_unit = c.has_unit2;
      ffn_pass<kGateUp, false, kMaxTiles, 2>(a, c2, ring, lpair);
    }
  } else {
    ffn_pass<kGateUp, kFastSB, 1, 3, kU>(a, c, ring, lpair);
  }
}

// 16-byte scale/bias copies need 8 | G, 8 | stride and 16-byte aligned bases
bool fast_sb_ok(const QMat& m, int G) {
  return G % 8 == 0 && G <= 64 && m.stride_sb % 8 == 0 && (reinterpret_cast<uintptr_t>(m.s) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(m.b) & 15) == 0;
}

}  // namespace

hipError_t launch_ffn_mfma(const FfnArgs& a, hipStream_t s, bool gate_up, const LaunchTiming* t) {
  const int max_union = a.E < a.B * a.K ? a.E : a.B * a.K;
  const bool shared = a.fs > 0;
  // a row of blocks for the shared expert, then one per union slot (see the
  // kernel), along x
  const int n_sh = shared ? 1 : 0;
  const int units_r = gate_up ? a.f / 32 : a.d / 64;
  const int units_s = gate_up ? a.fs / 32 : a.d / 64;
  // down with scales and biases in registers over 8, 16, 24 or 32 groups:
  // two units a wave.  Not with a shared expert on its wide pass (more than
  // 16 tokens): its blocks, which serve every token and take the longest,
  // would run their two units one after the other.
  auto two_units_ok = [](int K) { return K % 512 == 0 && K <= 2048; };
  const bool fast_dn = !gate_up && fast_sb_ok(a.down, a.f / 64) && (!shared || fast_sb_ok(a.sdown, a.fs / 64));
  const int kU =
      fast_dn && two_units_ok(a.f) && (!shared || (two_units_ok(a.fs) && a.B <= kPairTile)) ? 2 : 1;
  const int gx_r = (units_r + kWaves * kU - 1) / (kWaves * kU);
  const int gx_s = (units_s + kWaves * kU - 1) / (kWaves * kU);
  const dim3 grid(n_sh * gx_s + max_union * gx_r);
  if (gate_up) {
    const bool fast = fast_sb_ok(a.gate, a.d / 64) && fast_sb_ok(a.up, a.d / 64) &&
                      (!shared || (fast_sb_ok(a.sgate, a.d / 64) && fast_sb_ok(a.sup, a.d / 64)));
    if (fast)
      SMOE_LAUNCH(t, (k_ffn_mfma<true, true, 1>), grid, dim3(kThreads), 0, s, a);
    else
      SMOE_LAUNCH(t, (k_ffn_mfma<true, false, 1>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (kU == 2)
      SMOE_LAUNCH(t, (k_ffn_mfma<false, true, 2>), grid, dim3(kThreads), 0, s, a);
    else if (fast_dn)
      SMOE_LAUNCH(t, (k_ffn_mfma<false, true, 1>), grid, dim3(kThreads), 0, s, a);
    else
      SMOE_LAUNCH(t, (k_ffn_mfma<false, false, 1>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace smoe
