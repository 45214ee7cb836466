// device.hpp - device-side helpers of libsmoe (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

namespace smoe {

typedef _Float16 half_t;
typedef half_t half2_t __attribute__((ext_vector_type(2)));
typedef half_t half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming loads of weight words: marked nontemporal so that the expert
// bytes, read once, do not evict the activations from the caches.
__device__ __forceinline__ uint4 ld_stream4(const uint32_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream2(const uint32_t* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

// Direct global -> LDS copies (no VGPRs held while in flight).  Each active
// lane copies n bytes from its own source address to lds_base + n * lane;
// lds_base must be wave-uniform (it goes to M0).  The copies count in vmcnt
// and are complete in LDS once the issuing wave's vmcnt has dropped past
// them.  They are written as inline assembly so that the compiler neither
// tracks them nor inserts its own (whole-queue) waits for them: callers wait
// with wait_vmcnt<N>() themselves.  M0 is written here; the kernels that use
// these copies make no other use of M0 (no dynamic register indexing).  The
// s_nop is the one wait state required between an M0 write and an LDS copy.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
__device__ __forceinline__ void dma16_to_lds(const void* src, void* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src),
               "s"(lds_addr(lds_base))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_to_lds(const void* src, void* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src),
               "s"(lds_addr(lds_base))
               : "memory", "m0");
}
#pragma clang diagnostic pop
// Wait until at most N vector-memory operations of this wave are in flight.
// The memory clobber keeps the compiler from moving LDS reads above it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier without the implied wait for all outstanding memory
// operations (the LDS copies of later stages stay in flight).
__device__ __forceinline__ void barrier_no_wait() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

__device__ __forceinline__ uint16_t f16_bits(half_t h) { return __builtin_bit_cast(uint16_t, h); }
__device__ __forceinline__ half_t bits_f16(uint16_t u) { return __builtin_bit_cast(half_t, u); }

// Four fp16 pairs from one packed word of eight 4-bit codes q0..q7
// (q_i at bits 4i..4i+3).  OR-ing a code into the mantissa of 1024.0h
// (0x6400) gives 1024 + code exactly (the magic-number conversion of Kim et
// al., "Who Says Elephants Can't Run", 2022).  Codes at bit offset 4 inside
// a half land at mantissa bits 4..7 and read as 1024 + 16*code, so the
// activation paired with them is pre-divided by 16:
//   p0 = (1024+q0, 1024+q4)        p1 = (1024+16 q1, 1024+16 q5)
//   p2 = (1024+q2, 1024+q6)        p3 = (1024+16 q3, 1024+16 q7)
// Five integer ops per word.
// The masks live in registers: gfx9 VOP3 instructions take no literal
// operands, so with the masks as literals the compiler splits every
// (w & mask) | magic into a v_and and a v_or.  Produced by (pure, hence
// hoisted and shared) inline assembly, they stay opaque and each half pair is
// one v_and_or_b32.
struct NibbleMasks {
  uint32_t lo, hi, magic;
};
__device__ __forceinline__ NibbleMasks nibble_masks() {
  NibbleMasks m;
  asm("v_mov_b32 %0, 0x000f000f" : "=v"(m.lo));
  asm("v_mov_b32 %0, 0x00f000f0" : "=v"(m.hi));
  asm("s_mov_b32 %0, 0x64006400" : "=s"(m.magic));
  return m;
}
__device__ __forceinline__ void dequant_word(uint32_t w, uint32_t p[4]) {
  const NibbleMasks m = nibble_masks();
  p[0] = (w & m.lo) | m.magic;
  p[1] = (w & m.hi) | m.magic;
  const uint32_t w8 = w >> 8;
  p[2] = (w8 & m.lo) | m.magic;
  p[3] = (w8 & m.hi) | m.magic;
}

// acc + sum over the word's 8 inputs of (1024 + m*q) * stored, where the
// prepped activation chunk xc holds the matching stored halves.
__device__ __forceinline__ float dot_word(uint32_t w, const uint4& xc, float acc) {
  uint32_t p[4];
  dequant_word(w, p);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, p[0]), __builtin_bit_cast(half2_t, xc.x),
                               acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, p[1]), __builtin_bit_cast(half2_t, xc.y),
                               acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, p[2]), __builtin_bit_cast(half2_t, xc.z),
                               acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, p[3]), __builtin_bit_cast(half2_t, xc.w),
                               acc, false);
  return acc;
}

// The MFMA operand (8 halves) of one packed word, in the same slot order.
__device__ __forceinline__ half8_t word_operand(uint32_t w) {
  uint32_t p[4];
  dequant_word(w, p);
  uint4 v = make_uint4(p[0], p[1], p[2], p[3]);
  return __builtin_bit_cast(half8_t, v);
}

// ----------------------------------------------------- cross-lane reductions
// DPP lane moves (VALU, a few cycles each) instead of ds_bpermute shuffles.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF,
                                                            0xF, false));
}
template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, kCtrl, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i within 16

__device__ __forceinline__ float readlane(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Sum over aligned segments of `width` lanes (1, 2, 4, 8 or 16); every lane of
// a segment gets the segment total (each lane in a fixed order).
__device__ __forceinline__ float segment_sum16(float v, int width) {
  if (width >= 2) v += dpp<kDppXor1>(v);
  if (width >= 4) v += dpp<kDppXor2>(v);
  if (width >= 8) v += dpp<kDppHalfMirror>(v);
  if (width >= 16) v += dpp<kDppMirror>(v);
  return v;
}

// Wave-wide sum, the same value in every lane: 16-lane DPP sums, then the
// four row totals added in lane order 0, 16, 32, 48.
__device__ __forceinline__ float wave_sum(float v) {
  v = segment_sum16(v, 16);
  return ((readlane(v, 0) + readlane(v, 16)) + readlane(v, 32)) + readlane(v, 48);
}

// Sum over aligned segments of `width` lanes (power of two <= 64).  For width
// <= 16 every lane of a segment gets the total; for 32 and 64 the total is
// returned to every lane of the segment through readlane.
__device__ __forceinline__ float segment_sum(float v, int width) {
  if (width <= 16) return segment_sum16(v, width);
  v = segment_sum16(v, 16);
  if (width == 64) return ((readlane(v, 0) + readlane(v, 16)) + readlane(v, 32)) + readlane(v, 48);
  const float lo = readlane(v, 0) + readlane(v, 16);
  const float hi = readlane(v, 32) + readlane(v, 48);
  return (__lane_id() < 32) ? lo : hi;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  v = fmaxf(v, dpp<kDppMirror>(v));
  return fmaxf(fmaxf(readlane(v, 0), readlane(v, 16)), fmaxf(readlane(v, 32), readlane(v, 48)));
}

__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<kDppXor1>(v));
  v = min(v, dpp_i<kDppXor2>(v));
  v = min(v, dpp_i<kDppHalfMirror>(v));
  v = min(v, dpp_i<kDppMirror>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Top-k of one row of E <= 256 logits by one full wave (v[j] = logit of expert
// lane + 64 j, -FLT_MAX past E): after the call lane k < K holds the rank-k
// logit and expert, ranked by logit descending and, on equal logits, expert
// index ascending.  K rounds of a wave-wide arg-max (DPP max, then the lowest
// index among the maxima).
__device__ __forceinline__ void wave_topk(const float (&v)[4], int E, int K, float& my_v,
                                          int& my_e) {
  const int lane = __lane_id();
  bool live[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) live[j] = lane + 64 * j < E;
  my_v = 0.f;
  my_e = 0;
  for (int k = 0; k < K; ++k) {
    // this lane's best live candidate (ascending j keeps the lower index on ties)
    float bv = -INFINITY;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (live[j] && (v[j] > bv || (v[j] == bv && e < be))) {
        bv = v[j];
        be = e;
      }
    }
    const float m = wave_max(bv);
    const int win = wave_min_i(bv == m ? be : 0x7FFFFFFF);   // lowest index among the maxima
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (win == lane + 64 * j) live[j] = false;
    if (lane == k) {
      my_v = m;
      my_e = win;
    }
  }
}

// Routing weight of the lane's rank (lane < K) from wave_topk's results:
// exp(l - max) over the top-k sum (norm_topk_prob) or over all E experts.
__device__ __forceinline__ float topk_weight(const float (&v)[4], int E, int K, bool norm,
                                             float my_v) {
  const int lane = __lane_id();
  const float top = readlane(my_v, 0);
  const float p = lane < K ? expf(my_v - top) : 0.f;
  float den;
  if (norm) {
    den = wave_sum(p);
  } else {
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j < E) z += expf(v[j] - top);
    den = wave_sum(z);
  }
  return p / den;
}

// The stored halves of 8 consecutive inputs (one packed word's worth) in the
// prepped order, plus their contributions to the group sums X and C/1024.
__device__ __forceinline__ uint4 prep_chunk(const float v[8], float* X, float* S) {
  uint16_t hsv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const half_t xi = (half_t)v[i];                       // round to nearest even
    const half_t st = (i & 1) ? (half_t)((float)xi * 0.0625f) : xi;
    hsv[i] = f16_bits(st);
    const float stf = (float)st;
    *S += stf;
    *X += (i & 1) ? stf * 16.0f : stf;
  }
  // slot order: (x0,x4) (x1,x5) (x2,x6) (x3,x7)
  uint4 c;
  c.x = (uint32_t)hsv[0] | ((uint32_t)hsv[4] << 16);
  c.y = (uint32_t)hsv[1] | ((uint32_t)hsv[5] << 16);
  c.z = (uint32_t)hsv[2] | ((uint32_t)hsv[6] << 16);
  c.w = (uint32_t)hsv[3] | ((uint32_t)hsv[7] << 16);
  return c;
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

}  // namespace smoe
