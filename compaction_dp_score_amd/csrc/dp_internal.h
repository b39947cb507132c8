// Internal helpers of libdecoprune (gfx950).  Not part of the public ABI.
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

// Rotate the pairs of one 16-byte vector of keys.  dtype 1: bf16, 4 pairs;
// dtype 0: fp32, 2 pairs.  cs points at {cos, sin} of the vector's first pair;
// only the first n_valid pairs are rotated.
__device__ __forceinline__ u32x4 rotate_vec(u32x4 v, int dtype, const f32x2* cs, int n_valid) {
  if (dtype == DP_BF16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < n_valid) {
        f32x2 t = cs[q];
        float a2, b2;
        rotate_pair(bf16_lo(v[q]), bf16_hi(v[q]), t.x, t.y, a2, b2);
        v[q] = pack_bf16(a2, b2);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (q < n_valid) {
        f32x2 t = cs[q];
        float a2, b2;
        rotate_pair(__uint_as_float(v[2 * q]), __uint_as_float(v[2 * q + 1]), t.x, t.y, a2, b2);
        v[2 * q] = __float_as_uint(a2);
        v[2 * q + 1] = __float_as_uint(b2);
      }
    }
  }
  return v;
}

// Layout of the RoPE workspace: delta[n_frames] (fp32, padded to 16 bytes),
// then {cos, sin}[n_frames][pairs_padded] with pairs_padded a multiple of 4.
struct RopeView {
  const float* delta;
  const f32x2* cs;
  int32_t pairs_padded;
  int32_t n_pairs;
  int32_t n_frames;
  int32_t tv_begin;    // first 16-byte vector of the temporal block in a head row
  int32_t tv_count;    // vectors touched by the temporal block
  int32_t ppv;         // pairs per 16-byte vector: 4 (bf16) or 2 (fp32)
};

// ---------------------------------------------------------------------------
// Host side: error text and launch helpers (api.hip implements them).
// ---------------------------------------------------------------------------
dp_status fail(dp_status s, const char* fmt, ...);
dp_status check_launch(const char* what);

inline int elem_size(int dtype) { return dtype == DP_BF16 ? 2 : 4; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Launchers (one per source file).
dp_status launch_score_mask(const float* x0, const float* xf, int32_t d, int64_t stride,
                            const dp_mask_policy& pol, float* ell, uint8_t* keep,
                            hipStream_t s);
dp_status launch_compact(const uint8_t* keep, int64_t T, int32_t* idx, int64_t* n_kept,
                         const int32_t* rf_src, int32_t* rf_dst, int32_t* ws, hipStream_t s);
dp_status launch_rope_prepare(const dp_rope& r, void* ws, RopeView* view, int dtype,
                              int head_dim, hipStream_t s);
dp_status launch_gather(const dp_kv& kv, const int32_t* idx, const int64_t* n_kept,
                        const int32_t* row_frame, const RopeView* rope, hipStream_t s);
dp_status launch_reindex(void* const* k, int32_t n_layers, int32_t n_heads, int32_t head_dim,
                         int32_t dtype, int64_t rows_cap, const int64_t* n_rows,
                         const int32_t* row_frame, const RopeView& rope, hipStream_t s);
dp_status launch_hs_offsets(const uint8_t* head_class, int32_t L, int32_t H,
                            const int64_t* class_len, int32_t n_classes, int64_t* offsets,
                            hipStream_t s);
dp_status launch_hs_gather(const dp_kv_hs& kv, const uint8_t* head_class, int32_t n_classes,
                           const int32_t* const* class_idx, const int64_t* class_len,
                           const int64_t* class_cap, const int64_t* offsets,
                           const int32_t* const* class_rf, const RopeView* rope,
                           hipStream_t s);
dp_status launch_hs_reindex(void* k, int64_t k_cap, int32_t L, int32_t H, int32_t head_dim, int32_t dtype,
                            const uint8_t* head_class, int32_t n_classes,
                            const int64_t* class_len, const int64_t* class_cap,
                            const int64_t* offsets, const int32_t* const* class_rf,
                            const RopeView& rope, hipStream_t s);

}  // namespace dp
