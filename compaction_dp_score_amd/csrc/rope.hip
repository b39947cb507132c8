// RoPE temporal re-index of retained keys (DeCoPrune page, section 무엇과
// 다른가): an old key's temporal coordinate t moves to t~ = q0 - g(q0 - t),
// g leaving recent offsets alone and compressing older ones linearly; only
// the temporal phase of the keys changes.
//
// rope_prepare_kernel: one wavefront per frame computes
//   D = q0 - t, g(D), t~ = q0 - g(D), delta = t~ - p (p: phase the keys
//   carry), and for each temporal pair j the {cos, sin} of theta_j * delta
//   (fp32 angle, fp64 sincos, rounded to fp32); then p <- t~.
// reindex_kernel: in place over the temporal 16-byte vectors of every
//   (row, head) of each layer; rows of frames with delta == 0 are neither read
//   nor written.  HBM-bound: 2 * 2*n_pairs*elem bytes per re-indexed head row.
#include "dp_internal.h"

namespace dp {
namespace {

__global__ __launch_bounds__(64) void rope_prepare_kernel(
    const float* __restrict__ theta, int32_t n_pairs, int32_t pairs_padded,
    const float* __restrict__ frame_t, float* __restrict__ frame_phase, float q0, float knee,
    float inv_factor, float* __restrict__ delta, f32x2* __restrict__ cs) {
  const int f = blockIdx.x;
  const float D = q0 - frame_t[f];
  float gD;
  if (D <= knee) {
    gD = D;
  } else {
    float over = D - knee;
    float squeezed = over * inv_factor;
    gD = knee + squeezed;
  }
  const float t_new = q0 - gD;
  const float dl = t_new - frame_phase[f];
  for (int j = threadIdx.x; j < pairs_padded; j += 64) {
    f32x2 v = {1.0f, 0.0f};
    if (j < n_pairs) {
      float ang = theta[j] * dl;
      double sd, cd;
      sincos((double)ang, &sd, &cd);
      v.x = (float)cd;
      v.y = (float)sd;
    }
    cs[(int64_t)f * pairs_padded + j] = v;
  }
  __syncthreads();   // every lane has read frame_phase[f] before it changes
  if (threadIdx.x == 0) {
    delta[f] = dl;
    frame_phase[f] = t_new;
  }
}

struct ReindexArgs {
  void* const* layers;
  const int32_t* row_frame;
  const int64_t* n_rows;
  int64_t rows_cap;
  FastDiv div_row;    // vectors per row  = H * tv_count
  FastDiv div_head;   // vectors per head = tv_count
  uint32_t vph;       // 16-byte vectors per head row
  uint32_t n_heads;
  uint32_t total_cap; // rows_cap * H * tv_count
  int32_t dtype;
  RopeView rope;
};

template <int U>
__global__ __launch_bounds__(kBlock) void reindex_kernel(ReindexArgs a) {
  const uint32_t first = blockIdx.x * (kBlock * U);
  int64_t n = a.rows_cap;
  if (a.n_rows) n = min(n, *a.n_rows);
  const uint32_t total = (uint32_t)min((int64_t)a.total_cap, n * (int64_t)a.div_row.d);
  if (first >= total) return;
  u32x4* base = reinterpret_cast<u32x4*>(a.layers[blockIdx.y]);
  u32x4 v[U];
  int64_t addr[U];
  int frame[U];
  uint32_t tv_of[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    uint32_t i = first + u * kBlock + threadIdx.x;
    addr[u] = -1;
    if (i < total) {
      uint32_t j = fdiv(i, a.div_row);
      uint32_t rem = i - j * a.div_row.d;
      uint32_t h = fdiv(rem, a.div_head);
      uint32_t tv = rem - h * a.div_head.d;
      int f = a.row_frame[j];
      // a frame outside the table is skipped rather than read out of bounds
      if ((uint32_t)f < (uint32_t)a.rope.n_frames && a.rope.delta[f] != 0.0f) {
        frame[u] = f;
        tv_of[u] = tv;
        addr[u] = ((int64_t)j * a.n_heads + h) * a.vph + a.rope.tv_begin + tv;
        v[u] = __builtin_nontemporal_load(base + addr[u]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (addr[u] >= 0) {
      int p0 = (int)tv_of[u] * a.rope.ppv;
      int nv = min(a.rope.ppv, a.rope.n_pairs - p0);
      const f32x2* cs = a.rope.cs + (int64_t)frame[u] * a.rope.pairs_padded + p0;
      __builtin_nontemporal_store(rotate_vec(v[u], a.dtype, cs, nv), base + addr[u]);
    }
  }
}

}  // namespace

size_t rope_ws_bytes(int32_t n_frames, int32_t n_pairs) {
  size_t pp = (size_t)((n_pairs + 3) / 4) * 4;
  size_t dbytes = ((size_t)n_frames * 4 + 15) / 16 * 16;
  return dbytes + (size_t)n_frames * pp * sizeof(f32x2) + 32;   // 32-byte tail: see gather
}

dp_status launch_rope_prepare(const dp_rope& r, void* ws, RopeView* view, int dtype,
                              int head_dim, hipStream_t s) {
  const int32_t pp = (r.n_pairs + 3) / 4 * 4;
  const size_t dbytes = ((size_t)r.n_frames * 4 + 15) / 16 * 16;
  float* delta = reinterpret_cast<float*>(ws);
  f32x2* cs = reinterpret_cast<f32x2*>(reinterpret_cast<char*>(ws) + dbytes);
  hipLaunchKernelGGL(rope_prepare_kernel, dim3(r.n_frames), dim3(64), 0, s, r.theta, r.n_pairs,
                     pp, r.frame_t, r.frame_phase, r.q0, r.knee, r.inv_factor, delta, cs);
  dp_status st = check_launch("rope_prepare_kernel");
  if (st != DP_OK) return st;
  const int esz = elem_size(dtype);
  view->delta = delta;
  view->cs = cs;
  view->pairs_padded = pp;
  view->n_pairs = r.n_pairs;
  view->n_frames = r.n_frames;
  view->ppv = 16 / (2 * esz);
  view->tv_begin = (2 * r.pair_begin * esz) / 16;
  const int end_bytes = 2 * (r.pair_begin + r.n_pairs) * esz;
  view->tv_count = (end_bytes + 15) / 16 - view->tv_begin;
  (void)head_dim;
  return DP_OK;
}

dp_status launch_reindex(void* const* k, int32_t n_layers, int32_t n_heads, int32_t head_dim,
                         int32_t dtype, int64_t rows_cap, const int64_t* n_rows,
                         const int32_t* row_frame, const RopeView& rope, hipStream_t s) {
  ReindexArgs a;
  a.layers = k;
  a.row_frame = row_frame;
  a.n_rows = n_rows;
  a.rows_cap = rows_cap;
  a.div_row = make_fastdiv((uint32_t)(n_heads * rope.tv_count));
  a.div_head = make_fastdiv((uint32_t)rope.tv_count);
  a.vph = (uint32_t)(head_dim * elem_size(dtype) / 16);
  a.n_heads = (uint32_t)n_heads;
  a.total_cap = (uint32_t)(rows_cap * n_heads * rope.tv_count);
  a.dtype = dtype;
  a.rope = rope;
  if (a.total_cap == 0) return DP_OK;
  constexpr int U = 4;
  const uint32_t gx = (uint32_t)(((uint64_t)a.total_cap + kBlock * U - 1) / (kBlock * U));
  hipLaunchKernelGGL(reindex_kernel<U>, dim3(gx, n_layers), dim3(kBlock), 0, s, a);
  return check_launch("reindex_kernel");
}

}  // namespace dp
