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
__device__ __forceinline__ uint32_t ld_stream1(const uint32_t* p) {
  return __builtin_nontemporal_load(p);
}
__device__ __forceinline__ uint2 ld_stream2(const uint32_t* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

// Raw buffer loads.  A load at an offset at or past the resource's byte
// count returns zero and makes no memory access, so a pipelined loop can
// prefetch past its end with straight-line code (no branch, whose merge
// would make the compiler's wait counts conservative) and no wasted bytes.
constexpr uint32_t kBufferDead = 0x80000000u;   // an offset past every resource
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  // dword 3 = 0x00020000: raw 32-bit data format, no swizzle (gfx9 family)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// 16, 8 or 4 bytes, nontemporal (streamed once, see ld_stream4); soff is a
// wave-uniform byte offset added in a scalar register
__device__ __forceinline__ uint4 buf_load4_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff = 0) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, soff, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 buf_load2_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff = 0) {
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, soff, 2);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t buf_load1_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, soff, 2);
}
// 16 bytes, cached (data that other workgroups read again)
__device__ __forceinline__ uint4 buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff = 0) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t buf_load_u16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
// 2 bytes, nontemporal (a streamed scale or bias)
__device__ __forceinline__ uint32_t buf_load_u16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                    int soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, soff, 2);
}
__device__ __forceinline__ uint32_t ld_stream_u16(const uint16_t* p) {
  return __builtin_nontemporal_load(p);
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
// The same with the nontemporal hint: for the last read of a line, which may
// then leave the cache first (the line's other half was read before).
__device__ __forceinline__ void dma16_to_lds_nt(const void* src, void* lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src),
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
constexpr int kDppRowRor8 = 0x128;     // lane i <- lane i^8 within 16 (rotate by 8)

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

// v_permlane32_swap / v_permlane16_swap through inline assembly: with the
// compiler's builtins, the second register of the swapped pair was dropped
// (both sums read the first).  The s_nop pairs cover the VALU-write ->
// permlane-read and permlane-write -> VALU-read hazards, which the compiler
// does not see through an asm statement.
__device__ __forceinline__ void permlane32_swap(float& x, float& y) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}
__device__ __forceinline__ void permlane16_swap(float& x, float& y) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
}

// Sum over the wave of eight per-lane row partials v[0..7]: afterwards every
// lane of 8L' .. 8L'+7 holds the total of row L' (= lane / 8).  Bit 5 of the
// lane is folded by permlane32 swaps (lanes 32-63 of the first register
// trade places with lanes 0-31 of the second, so lanes 0-31 keep rows 0-3 and
// lanes 32-63 rows 4-7), bit 4 by permlane16 swaps (odd 16-lane rows of the
// first with even rows of the second), bit 3 by a DPP exchange, and bits 0-2
// by DPP adds: about 20 VALU operations for eight rows.
__device__ __forceinline__ float rows8_wave_sum(const float (&v)[8]) {
  float a4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float x = v[j], y = v[j + 4];
    permlane32_swap(x, y);
    a4[j] = x + y;                                 // row j + 4 bit5
  }
  float c2[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float x = a4[j], y = a4[j + 2];
    permlane16_swap(x, y);
    c2[j] = x + y;                                 // row j + 2 bit4 + 4 bit5
  }
  // lane bit 3 picks which of the two it keeps; the partner lane^8 sends the other
  const bool b3 = (__lane_id() & 8) != 0;
  const float keep = b3 ? c2[1] : c2[0];
  const float send = b3 ? c2[0] : c2[1];
  const float t = keep + dpp<kDppRowRor8>(send);
  return segment_sum16(t, 8);
}

// Root-mean-square normalisation of one row of d floats (d % 4 == 0, d <=
// 8192): inv = 1 / sqrt(mean(row^2) + eps), formed by a block of 256 threads
// in one fixed order: thread i adds the squares of float4s i, i + 256, ...
// as an fma chain (all of its loads issued first; the slots past the row
// add fma(0, 0, s) = s), each wave's threads are summed by wave_sum, and the
// four wave sums are added in order.  Every thread of the block must call
// it; `part` is 4 floats of LDS; the result is the same in every thread.
__device__ __forceinline__ float sumsq4(float ss, const float4& q) {
  ss = __builtin_fmaf(q.x, q.x, ss);
  ss = __builtin_fmaf(q.y, q.y, ss);
  ss = __builtin_fmaf(q.z, q.z, ss);
  return __builtin_fmaf(q.w, q.w, ss);
}
constexpr int kRowInvMaxPerThread = 8;            // 8192 / 4 / 256
__device__ __forceinline__ float block_row_inv(const float* row, int d, float eps, float* part) {
  const float4* r4 = reinterpret_cast<const float4*>(row);
  const int n4 = d / 4, tid = threadIdx.x;
  float4 q[kRowInvMaxPerThread];
#pragma unroll
  for (int j = 0; j < kRowInvMaxPerThread; ++j) {
    const int i = tid + 256 * j;
    q[j] = r4[i < n4 ? i : 0];
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kRowInvMaxPerThread; ++j) {
    const bool in = tid + 256 * j < n4;
    ss = sumsq4(ss, in ? q[j] : make_float4(0.f, 0.f, 0.f, 0.f));
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float tot = ((part[0] + part[1]) + part[2]) + part[3];
  __syncthreads();                                // part may be reused after this
  return 1.0f / sqrtf(tot / (float)d + eps);
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

// Per-wave LDS scratch of wave_topk: the K selected entries in expert order.
constexpr int kTopkMax = 16;
struct alignas(16) TopkScratch {
  uint32_t key[kTopkMax];
  int e[kTopkMax];
  float v[kTopkMax];
};

// Order-preserving map of a float to an unsigned key: x > y (as floats, no
// NaN) exactly when key(x) > key(y).  -0 is first made +0 (x + 0 rounds it to
// +0), so that the two zeros compare equal, as floats do.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Counts of the wave's keys at or above c1, c2 and c3 (NJ = 2 or 4 keys per
// lane).  The compares are VOP3 v_cmp into SGPR pairs of their own, issued
// together in one block: the compiler's ballots all go through VCC (or one
// reused pair), which chains every compare behind the previous mask's count.
// Every lane of the wave must be active (inactive lanes read as 0).
template <int NJ>
__device__ __forceinline__ void count_ge3(const uint32_t (&key)[4], uint32_t c1, uint32_t c2,
                                          uint32_t c3, int& n1, int& n2, int& n3);
template <>
__device__ __forceinline__ void count_ge3<2>(const uint32_t (&key)[4], uint32_t c1, uint32_t c2,
                                             uint32_t c3, int& n1, int& n2, int& n3) {
  uint64_t a0, a1, b0, b1, d0, d1;
  asm("v_cmp_ge_u32_e64 %0, %6, %8\n\t"
      "v_cmp_ge_u32_e64 %1, %7, %8\n\t"
      "v_cmp_ge_u32_e64 %2, %6, %9\n\t"
      "v_cmp_ge_u32_e64 %3, %7, %9\n\t"
      "v_cmp_ge_u32_e64 %4, %6, %10\n\t"
      "v_cmp_ge_u32_e64 %5, %7, %10"
      : "=&s"(a0), "=&s"(a1), "=&s"(b0), "=&s"(b1), "=&s"(d0), "=&s"(d1)
      : "v"(key[0]), "v"(key[1]), "s"(c1), "s"(c2), "s"(c3));
  n1 = __popcll(a0) + __popcll(a1);
  n2 = __popcll(b0) + __popcll(b1);
  n3 = __popcll(d0) + __popcll(d1);
}
template <>
__device__ __forceinline__ void count_ge3<4>(const uint32_t (&key)[4], uint32_t c1, uint32_t c2,
                                             uint32_t c3, int& n1, int& n2, int& n3) {
  int x1, x2, x3, y1, y2, y3;
  const uint32_t lo[4] = {key[0], key[1], 0u, 0u}, hi[4] = {key[2], key[3], 0u, 0u};
  count_ge3<2>(lo, c1, c2, c3, x1, x2, x3);
  count_ge3<2>(hi, c1, c2, c3, y1, y2, y3);
  n1 = x1 + y1;
  n2 = x2 + y2;
  n3 = x3 + y3;
}

// A key threshold t with #{key > t} <= K <= #{key >= t} (so that the top K
// are the keys above t plus the lowest-index keys equal to t): the K-th
// largest key, built two bits per step from the top (the three candidate
// counts of a step are independent), or earlier the first prefix that
// exactly K keys reach.
template <int NJ>
__device__ __forceinline__ uint32_t topk_threshold(const uint32_t (&key)[4], int K) {
  uint32_t t = 0;
#pragma unroll
  for (int sh = 30; sh >= 0; sh -= 2) {
    const uint32_t c1 = t | (1u << sh), c2 = t | (2u << sh), c3 = t | (3u << sh);
    int n1, n2, n3;
    count_ge3<NJ>(key, c1, c2, c3, n1, n2, n3);
    const int n = n3 >= K ? n3 : (n2 >= K ? n2 : n1);
    t = n3 >= K ? c3 : (n2 >= K ? c2 : (n1 >= K ? c1 : t));
    if (n == K) break;                            // exactly K keys at or above t
  }
  return t;
}

// Wave masks of key[j] > t and key[j] == t (j < 2), each in an SGPR pair of
// its own (see count_ge3); the trailing s_nop covers a following VALU read of
// the masks.
__device__ __forceinline__ void masks_gt_eq2(uint32_t k0, uint32_t k1, uint32_t t, uint64_t& gt0,
                                             uint64_t& gt1, uint64_t& eq0, uint64_t& eq1) {
  asm("v_cmp_gt_u32_e64 %0, %4, %6\n\t"
      "v_cmp_gt_u32_e64 %1, %5, %6\n\t"
      "v_cmp_eq_u32_e64 %2, %4, %6\n\t"
      "v_cmp_eq_u32_e64 %3, %5, %6\n\t"
      "s_nop 4"
      : "=&s"(gt0), "=&s"(gt1), "=&s"(eq0), "=&s"(eq1)
      : "v"(k0), "v"(k1), "s"(t));
}
__device__ __forceinline__ void masks_nz2(uint32_t a0, uint32_t a1, uint64_t& m0, uint64_t& m1) {
  asm("v_cmp_ne_u32_e64 %0, 0, %2\n\t"
      "v_cmp_ne_u32_e64 %1, 0, %3\n\t"
      "s_nop 4"
      : "=&s"(m0), "=&s"(m1)
      : "v"(a0), "v"(a1));
}
// Set bits of m below this lane.
__device__ __forceinline__ int bits_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// Result of wave_topk_sel.  Lane q < K: se/sv = the q-th selected expert in
// ascending expert order and its logit, srank = its rank.  Lane k < K:
// my_e/my_v = the rank-k expert and logit.  Lanes >= K: zeros.
struct TopkSel {
  int se;
  float sv;
  int srank;
  int my_e;
  float my_v;
};

// Order keys of the lane's candidates (expert lane + 64 j); 0 past E.
template <int NJ>
__device__ __forceinline__ void topk_keys(const float (&v)[4], int E, uint32_t (&key)[4]) {
  const int lane = __lane_id();
#pragma unroll
  for (int j = 0; j < 4; ++j) key[j] = (j < NJ && lane + 64 * j < E) ? order_key(v[j]) : 0u;
}

// Step 2 of wave_topk_sel for one row, given its threshold t: the keys above
// t, plus the lowest-index keys equal to t up to K in all, are copied in
// expert order to the wave's scratch (and, when `order` is not null, their
// experts to order[0 .. K-1]).
template <int NJ>
__device__ __forceinline__ void topk_compact(const float (&v)[4], const uint32_t (&key)[4],
                                             uint32_t t, int K, TopkScratch* sc, int* order) {
  const int lane = __lane_id();
  uint64_t gt[4], eq[4];
#pragma unroll
  for (int j = 0; j < NJ; j += 2) masks_gt_eq2(key[j], key[j + 1], t, gt[j], gt[j + 1], eq[j], eq[j + 1]);
  int n_gt = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) n_gt += __popcll(gt[j]);
  const int need = K - n_gt;                      // keys equal to t to take (>= 0)
  // selection and place in expert order (expert lane + 64 j: j, then lane)
  uint32_t sel[4];
  int ties = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const bool is_gt = (gt[j] >> lane) & 1, is_eq = (eq[j] >> lane) & 1;
    sel[j] = (is_gt || (is_eq && ties + bits_below(eq[j]) < need)) ? 1u : 0u;
    ties += __popcll(eq[j]);
  }
  uint64_t ms[4];
#pragma unroll
  for (int j = 0; j < NJ; j += 2) masks_nz2(sel[j], sel[j + 1], ms[j], ms[j + 1]);
  int taken = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (sel[j]) {
      const int p = taken + bits_below(ms[j]);
      sc->key[p] = key[j];
      sc->e[p] = lane + 64 * j;
      sc->v[p] = v[j];
      if (order != nullptr) order[p] = lane + 64 * j;
    }
    taken += __popcll(ms[j]);
  }
}

// Step 3 of wave_topk_sel: each of the K selected entries in the wave's
// scratch (written by topk_compact of this wave) ranks itself against the
// other K-1 and is sent to the lane of its rank (ds_permute).
__device__ __forceinline__ TopkSel topk_rank(int K, TopkScratch* sc) {
  const int lane = __lane_id();
  // a wave's LDS accesses execute in order; keep the compiler from moving the
  // reads above the writes
  asm volatile("" ::: "memory");
  const bool mine = lane < K;
  const int ql = mine ? lane : 0;
  const uint32_t qk = sc->key[ql];
  const int qe = sc->e[ql];
  const float qv = sc->v[ql];
  // all K entries by 16-byte broadcast reads issued together (entries past K
  // are stale and masked), then a branch-free count
  uint4 k4[kTopkMax / 4], e4[kTopkMax / 4];
#pragma unroll
  for (int i = 0; i < kTopkMax / 4; ++i) {
    k4[i] = reinterpret_cast<const uint4*>(sc->key)[i];
    e4[i] = reinterpret_cast<const uint4*>(sc->e)[i];
  }
  int rank = 0;
#pragma unroll
  for (int r = 0; r < kTopkMax; ++r) {
    const uint4& kq = k4[r / 4];
    const uint4& eq = e4[r / 4];
    const uint32_t kr = (r % 4 == 0) ? kq.x : (r % 4 == 1) ? kq.y : (r % 4 == 2) ? kq.z : kq.w;
    const int er = (int)((r % 4 == 0) ? eq.x : (r % 4 == 1) ? eq.y : (r % 4 == 2) ? eq.z : eq.w);
    const int before = (int)(kr > qk) | ((int)(kr == qk) & (int)(er < qe));
    rank += (r < K) ? before : 0;
  }
  asm volatile("" ::: "memory");                  // the scratch may be reused after this
  const int dst = mine ? rank : lane;             // a permutation of the lanes
  const float pv = __int_as_float(__builtin_amdgcn_ds_permute(dst << 2, __float_as_int(qv)));
  const int pe = __builtin_amdgcn_ds_permute(dst << 2, qe);
  TopkSel out;
  out.se = mine ? qe : 0;
  out.sv = mine ? qv : 0.f;
  out.srank = mine ? rank : 0;
  out.my_e = mine ? pe : 0;
  out.my_v = mine ? pv : 0.f;
  return out;
}

// Steps 2 and 3 of wave_topk_sel for one row, given its threshold t.
template <int NJ>
__device__ __forceinline__ TopkSel topk_finish(const float (&v)[4], const uint32_t (&key)[4],
                                               uint32_t t, int K, TopkScratch* sc) {
  topk_compact<NJ>(v, key, t, K, sc, nullptr);
  return topk_rank(K, sc);
}

// Top-k of one row of E <= 64 * NJ logits by one full wave (v[j] = logit of
// expert lane + 64 j; entries past E are ignored), K <= 16, ranked by logit
// descending and, on equal logits, expert index ascending:
//   1. a threshold t (topk_threshold: wave mask counts);
//   2. the keys above t, plus the lowest-index keys equal to t up to K in all,
//      are copied in expert order to the wave's scratch;
//   3. each of the K ranks itself against the other K-1 and is sent to the
//      lane of its rank (ds_permute).
// Candidates past E get key 0, below every real key, so no step needs a
// branch on E.  sc: this wave's scratch in LDS (no other wave may use it
// meanwhile).  Every lane of the wave must be active.
template <int NJ>
__device__ __forceinline__ TopkSel wave_topk_sel(const float (&v)[4], int E, int K,
                                                 TopkScratch* sc) {
  uint32_t key[4];
  topk_keys<NJ>(v, E, key);
  return topk_finish<NJ>(v, key, topk_threshold<NJ>(key, K), K, sc);
}

// Top-k of one row of E <= 256 logits (see wave_topk_sel): lane k < K gets
// the rank-k logit and expert.
__device__ __forceinline__ void wave_topk(const float (&v)[4], int E, int K, float& my_v,
                                          int& my_e, TopkScratch* sc) {
  const TopkSel t = E <= 128 ? wave_topk_sel<2>(v, E, K, sc) : wave_topk_sel<4>(v, E, K, sc);
  my_v = t.my_v;
  my_e = t.my_e;
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
