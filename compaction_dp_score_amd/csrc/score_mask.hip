// dp_score_mask: per-token discrepancy score and keep mask.
//
// The DeCoPrune page (section 어떻게 동작하나) scores each token of a chunk by
// the mean squared gap between the clean prediction recorded at the probe
// step and the final output, and thresholds it with gamma; the mask is shared
// by every layer, the sink chunk and the last w chunks are always kept.
//
// Launch layout: blocks [0, n_score_blocks) score rows; a group of G lanes
// (G = P/4, P the channel count padded to a power of two) owns one row, lane
// k loads channels 4k..4k+3, and the pairwise tree q_c += q_{c+h} runs as
// shuffles for h >= 4 and inside the lane for h = 2, 1.  Blocks after those
// write the keep bytes of every row that is not scored (sink, window, earlier
// history), 16 rows per thread.  The score is HBM-bound: 8d bytes read and
// 1 (+4 with ell) written per scored row.
#include "dp_internal.h"

namespace dp {
namespace {

struct ScoreArgs {
  const float* x0;
  const float* xf;
  float* ell;
  uint8_t* keep;
  int64_t stride;
  int64_t T, sink_end, win_begin, sc_begin, sc_end;
  int32_t d, P, G, vec;
  float gamma;
  int32_t reversed, streaming;
  uint32_t n_score_blocks;
};

__device__ __forceinline__ f32x4 load4(const float* row, int c, int d, bool vec) {
  if (vec) return *reinterpret_cast<const f32x4*>(row + c);   // c < d, d % 4 == 0
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (c + 0 < d) v.x = row[c + 0];
  if (c + 1 < d) v.y = row[c + 1];
  if (c + 2 < d) v.z = row[c + 2];
  if (c + 3 < d) v.w = row[c + 3];
  return v;
}

__device__ __forceinline__ f32x4 shfl_down4(f32x4 v, int delta, int width) {
  f32x4 r;
  r.x = __shfl_down(v.x, delta, width);
  r.y = __shfl_down(v.y, delta, width);
  r.z = __shfl_down(v.z, delta, width);
  r.w = __shfl_down(v.w, delta, width);
  return r;
}

__device__ __forceinline__ uint8_t outside_keep(int64_t t, const ScoreArgs& a) {
  if (t < a.sink_end || t >= a.win_begin) return 1;
  return a.streaming ? 0 : 1;   // scored rows in streaming mode also land here
}

__global__ __launch_bounds__(kBlock) void score_mask_kernel(ScoreArgs a) {
  if (blockIdx.x < a.n_score_blocks) {
    // ---- scoring part ----
    const int G = a.G;
    const int lane_in_group = threadIdx.x % G;
    const int64_t row = (int64_t)blockIdx.x * (kBlock / G) + threadIdx.x / G;
    const bool live = row < a.sc_end - a.sc_begin;
    f32x4 q = {0.f, 0.f, 0.f, 0.f};
    const int c = 4 * lane_in_group;
    if (live && c < a.d) {
      const float* r0 = a.x0 + row * a.stride;
      const float* r1 = a.xf + row * a.stride;
      f32x4 u = load4(r0, c, a.d, a.vec != 0);
      f32x4 w = load4(r1, c, a.d, a.vec != 0);
      f32x4 e = u - w;
      q = e * e;                     // padded channels stay +0 (0 - 0 = +0)
    }
    // pairwise tree, h = P/2 .. 4 across lanes (lane k pairs with k + h/4)
    for (int h = a.P / 2; h >= 4; h /= 2) {
      f32x4 o = shfl_down4(q, h / 4, G);
      q = q + o;
    }
    if (a.P >= 4) {                  // h = 2, then h = 1
      q.x = q.x + q.z;
      q.y = q.y + q.w;
      q.x = q.x + q.y;
    } else if (a.P == 2) {           // h = 1
      q.x = q.x + q.y;
    }
    if (live && lane_in_group == 0) {
      float ell = (float)((double)q.x / (double)a.d);
      bool big = ell >= a.gamma;     // NaN fails
      if (a.ell) a.ell[row] = ell;
      a.keep[a.sc_begin + row] = (uint8_t)(a.reversed ? !big : big);
    }
    return;
  }
  // ---- keep bytes of the rows that are not scored ----
  const int64_t t0 = ((int64_t)(blockIdx.x - a.n_score_blocks) * kBlock + threadIdx.x) * 16;
  if (t0 >= a.T) return;
  const bool scoring = !a.streaming;
  const bool touches_scored = scoring && t0 < a.sc_end && t0 + 16 > a.sc_begin;
  if (!touches_scored && t0 + 16 <= a.T && (((uintptr_t)(a.keep + t0)) & 15u) == 0) {
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) word |= (uint32_t)outside_keep(t0 + 4 * w + b, a) << (8 * b);
      v[w] = word;
    }
    *reinterpret_cast<u32x4*>(a.keep + t0) = v;
    return;
  }
  for (int b = 0; b < 16; ++b) {
    int64_t t = t0 + b;
    if (t >= a.T) break;
    if (scoring && t >= a.sc_begin && t < a.sc_end) continue;   // written by the scoring part
    a.keep[t] = outside_keep(t, a);
  }
}

}  // namespace

dp_status launch_score_mask(const float* x0, const float* xf, int32_t d, int64_t stride,
                            const dp_mask_policy& pol, float* ell, uint8_t* keep,
                            hipStream_t s) {
  ScoreArgs a;
  a.x0 = x0;
  a.xf = xf;
  a.ell = ell;
  a.keep = keep;
  a.stride = stride;
  a.T = pol.seq_len;
  a.sink_end = pol.sink_len;
  a.win_begin = pol.seq_len - pol.window_len;
  a.sc_begin = pol.scored_begin;
  a.sc_end = pol.scored_begin + pol.n_scored;
  a.d = d;
  int P = 1;
  while (P < d) P *= 2;
  a.P = P;
  a.G = P >= 4 ? P / 4 : 1;
  a.vec = (d % 4 == 0) && (stride % 4 == 0) && aligned16(x0) && aligned16(xf);
  a.gamma = pol.gamma;
  a.reversed = pol.reversed;
  a.streaming = pol.mode == DP_MODE_STREAMING;
  const int64_t rows_per_block = kBlock / a.G;
  const int64_t n_sc = a.streaming ? 0 : pol.n_scored;
  const int64_t nsb = (n_sc + rows_per_block - 1) / rows_per_block;
  const int64_t nfb = (pol.seq_len + 16 * kBlock - 1) / (16 * kBlock);
  a.n_score_blocks = (uint32_t)nsb;
  const int64_t grid = nsb + nfb;
  if (grid <= 0) return DP_OK;
  hipLaunchKernelGGL(score_mask_kernel, dim3((uint32_t)grid), dim3(kBlock), 0, s, a);
  return check_launch("score_mask_kernel");
}

}  // namespace dp
