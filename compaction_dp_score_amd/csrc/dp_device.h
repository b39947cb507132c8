// Device-side helpers of libdecoprune (gfx950): vector types, division by an
// invariant integer, bf16 conversion, the RoPE pair rotation and the layout of
// the re-index tables.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decoprune.h"

// Every floating-point step of this library is written so that each product
// and each sum is rounded on its own: no fused multiply-add contraction.
#pragma clang fp contract(off)

namespace dp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 256;          // threads per workgroup (4 wave64s)

// ---------------------------------------------------------------------------
// Division of a 32-bit unsigned n by a divisor fixed for a launch, as a
// multiply-high and shifts (Granlund & Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994, section 4).
// ---------------------------------------------------------------------------
struct FastDiv {
  uint32_t d;   // divisor, >= 1
  uint32_t m;   // magic multiplier
  uint32_t l;   // ceil(log2 d)
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while ((1ull << l) < (uint64_t)d) ++l;
  f.l = l;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << l) - (uint64_t)d)) / d + 1ull);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  if (f.l == 0) return n;                       // d == 1
  uint32_t t = __umulhi(n, f.m);
  return (t + ((n - t) >> 1)) >> (f.l - 1);
}

// ---------------------------------------------------------------------------
// XCD-contiguous work order.  The dispatcher deals workgroups to the chip's 8
// XCDs in turn (workgroup id mod 8), so in plain order neighbouring work items,
// which stream neighbouring memory, land on different XCDs.  This maps the
// workgroup id to a work item so that each XCD takes one contiguous eighth of
// the `live` items (a bijection onto [0, live) when the grid is a multiple of
// 8 and at least `live`); surplus workgroups get UINT32_MAX.  Measured on the
// in-place re-index of split keys: 3 % more bandwidth than plain order.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t xcd_item(uint32_t bid, uint32_t live) {
  const uint32_t per = (live + kXcds - 1) / kXcds;
  const uint32_t k = bid / kXcds;
  if (k >= per) return UINT32_MAX;
  const uint32_t l = (bid % kXcds) * per + k;
  return l < live ? l : UINT32_MAX;
}

inline uint64_t xcd_grid(uint64_t g) { return (g + kXcds - 1) / kXcds * kXcds; }

// A read through the constant address space: a wave-uniform address becomes a
// scalar load.  Only for arrays that the kernel reading them does not write
// (the scalar cache is not kept coherent with the kernel's own stores).
template <class T>
__device__ __forceinline__ T uniform_load(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32.  Widening is exact.  Narrowing rounds to nearest, ties to
// even, and keeps NaN a quiet NaN.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u) return (u >> 16) | 0x0040u;
  uint32_t lsb = (u >> 16) & 1u;
  return (u + 0x7FFFu + lsb) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// One RoPE pair rotation (a, b) -> (a c - b s, a s + b c), every product and
// sum rounded separately.
__device__ __forceinline__ void rotate_pair(float a, float b, float c, float s, float& a2,
                                            float& b2) {
  float ac = a * c;
  float bs = b * s;
  float as = a * s;
  float bc = b * c;
  a2 = ac - bs;
  b2 = as + bc;
}

// Two fp32 values to two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16_hw(float lo, float hi) {
  f32x2 in = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(in, bf16x2));
}

// Rotate the pairs of one 16-byte vector of keys given its {cos, sin} table
// entries t01 = (c0 s0 c1 s1) and t23 = (c2 s2 c3 s3).  dtype 1: bf16, 4 pairs;
// dtype 0: fp32, 2 pairs (t23 unused).  Only the first n_valid pairs change;
// the result is selected per pair, without branches.
__device__ __forceinline__ u32x4 rotate_vec_tab(u32x4 v, int dtype, f32x4 t01, f32x4 t23,
                                                int n_valid) {
  if (dtype == DP_BF16) {
    const float cc[4] = {t01.x, t01.z, t23.x, t23.z};
    const float ss[4] = {t01.y, t01.w, t23.y, t23.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a2, b2;
      rotate_pair(bf16_lo(v[q]), bf16_hi(v[q]), cc[q], ss[q], a2, b2);
      const uint32_t r = pack_bf16_hw(a2, b2);
      v[q] = q < n_valid ? r : v[q];
    }
  } else {
    const float cc[2] = {t01.x, t01.z};
    const float ss[2] = {t01.y, t01.w};
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float a2, b2;
      rotate_pair(__uint_as_float(v[2 * q]), __uint_as_float(v[2 * q + 1]), cc[q], ss[q], a2, b2);
      v[2 * q] = q < n_valid ? __float_as_uint(a2) : v[2 * q];
      v[2 * q + 1] = q < n_valid ? __float_as_uint(b2) : v[2 * q + 1];
    }
  }
  return v;
}

// Same, reading the table at cs (16-byte aligned; the table is padded so that
// the entries of four pairs are readable).
__device__ __forceinline__ u32x4 rotate_vec(u32x4 v, int dtype, const f32x2* cs, int n_valid) {
  const f32x4* t = reinterpret_cast<const f32x4*>(cs);
  const f32x4 t01 = t[0];
  const f32x4 t23 = dtype == DP_BF16 ? t[1] : t01;
  return rotate_vec_tab(v, dtype, t01, t23, n_valid);
}

// Layout of the RoPE workspace: delta[n_frames] (fp32, padded to 16 bytes),
// then {cos, sin}[n_frames][pairs_padded] with pairs_padded a multiple of 4,
// then a 32-byte tail so that four pairs can always be read from any vector's
// first pair.
struct RopeView {
  const float* delta;
  const f32x2* cs;
  int32_t pairs_padded;
  int32_t n_pairs;
  int32_t n_frames;
  int32_t tv_begin;    // first 16-byte vector of the temporal block in a head row
  int32_t tv_count;    // vectors touched by the temporal block
  int32_t ppv;         // pairs per 16-byte vector: 4 (bf16) or 2 (fp32)
  // In-place passes walk, for every head of a token row, vectors
  // [wv_begin, wv_begin + wv_count) of that head's segment, the segments
  // head_stride_v vectors apart; the temporal block starts tv_off vectors into
  // a segment.  Interleaved keys: the segment is the head row and the walk
  // covers the temporal block rounded out to 128-byte boundaries (clamped to
  // the head row; vectors outside the block are written back unchanged: a
  // partly written line costs the memory controller a read-modify-write,
  // which measured slower than the extra bytes).  Split keys: the segment is
  // the head's temporal block in the row's leading plane, walked exactly.
  int32_t wv_begin;
  int32_t wv_count;
  int32_t head_stride_v;
  int32_t tv_off;
  // Whole-row passes (gather, append) locate vector c of a row by
  // h = c / seg and tv = c - h seg - tv_off, with seg = head_stride_v; a
  // vector is in a temporal block iff 0 <= tv < tv_count and c < blk_end
  // (interleaved: every head row; split: the leading plane of n_heads blocks).
  int32_t blk_end;
  int32_t split;
};

}  // namespace dp
