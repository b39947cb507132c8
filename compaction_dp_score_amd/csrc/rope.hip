// RoPE temporal re-index of retained keys (DeCoPrune page, section 무엇과
// 다른가): an old key's temporal coordinate t moves to t~ = q0 - g(q0 - t),
// g leaving recent offsets alone and compressing older ones linearly; only
// the temporal phase of the keys changes.
//
// rope_prepare_kernel: one wavefront per frame computes
//   D = q0 - t, g(D), t~ = q0 - g(D) (or, on the compressed axis, t/c past
//   the knee), delta = t~ - p (p: phase the keys carry), and for each temporal
//   pair j the {cos, sin} of theta_j * delta (fp32 angle, fp64 sincos, rounded
//   to fp32); then p <- t~.
// reindex_kernel: in place over every (row, head) of each layer, touching the
//   128-byte lines that hold the temporal pairs; rows of frames with delta == 0
//   are neither read nor written.  HBM-bound: the method needs
//   2 * 2*n_pairs*elem bytes per re-indexed head row.  With interleaved keys
//   the temporal block of a head row straddles lines and whole-line rewriting
//   moves 2 * (lines * 128) bytes (512 of 352 for 44 bf16 pairs); with split
//   keys the blocks of all heads are the row's leading lines and exactly the
//   method's bytes move.
// shift_table_kernel + shift_kernel: the steady-state form.  Once a frame is
//   past the knee before and after a step, its phase step is the same for every
//   such frame (q0 advances F frames: F (1 - 1/c)), so a row range holding only
//   such frames is rotated by one uniform step: one {cos, sin} table (written
//   by a one-workgroup launch) and no row frames; the rotation pass has the
//   layout of reindex_kernel.
#include "dp_internal.h"

namespace dp {
namespace {

__global__ __launch_bounds__(64) void rope_prepare_kernel(
    const float* __restrict__ theta, int32_t n_pairs, int32_t pairs_padded,
    const float* __restrict__ frame_t, float* __restrict__ frame_phase, float q0, float knee,
    float inv_factor, int axis, float* __restrict__ delta, f32x2* __restrict__ cs) {
  const int f = blockIdx.x;
  const float D = q0 - frame_t[f];
  float t_new;
  if (D > knee && axis == DP_AXIS_COMPRESSED) {
    t_new = frame_t[f] * inv_factor;    // t/c: the part of t~ that is the key's own
  } else {
    float gD = D;
    if (D > knee) {
      float over = D - knee;
      float squeezed = over * inv_factor;
      gD = knee + squeezed;
    }
    t_new = q0 - gD;
  }
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
  int64_t row_begin;
  int64_t rows_cap;
  FastDiv div_row;    // vectors per row  = H * wv_count
  FastDiv div_head;   // vectors per head = wv_count
  uint32_t row_vec;   // 16-byte vectors per token row (H * vph)
  uint32_t n_layers;
  int32_t dtype;
  RopeView rope;
};

// Two 16-byte vectors per lane: a wavefront takes 128 consecutive vectors of a
// layer's walked span (every (row, head) segment, row-major), a workgroup 512.
// Workgroups map to (layer, tile) in XCD-contiguous order over the live tiles,
// counted from the device-side row count, so surplus workgroups leave at once.
// With rows of >= 128 walked vectors (WAVE_ROWS) a wavefront spans at most two
// rows: their frames and phase steps are scalar loads, and a wavefront whose
// rows both have delta == 0 (the recent window) leaves before touching the
// keys; otherwise each lane looks its rows up.  The {cos, sin} entries of a
// wavefront's rows are then staged (STAGE, when a head row has at most kTabTv
// temporal vectors): the wavefront's two frames need only 2 tv_count distinct
// 32-byte entries, so lanes e < 2 tv_count load one each before the data loads
// go out and write it to the wavefront's slot in LDS after them, and every
// lane reads its vectors' entries from there (measured on the one-minute cache:
// 1.3-1.5 % faster with split keys, 2 % with interleaved keys, than every lane
// loading its own entries; outputs unchanged).  Otherwise each lane loads its
// entries before the data.  Both vectors' data loads are in flight together;
// vectors outside the temporal block are written back unchanged so that whole
// 128-byte lines are rewritten.  Measured on the one-minute cache with split
// keys: two vectors per lane 4 % and the XCD order 3 % faster than one vector
// per lane in plain order; three or four vectors per lane, 512-lane
// workgroups and temporal (cached) loads or stores no better.
constexpr int kWaveSpan = 128;              // walked vectors per wavefront
constexpr int kSpan = kBlock / 64 * kWaveSpan;
constexpr int kTabTv = 32;                  // staged table: temporal vectors per head row

template <bool WAVE_ROWS, bool STAGE>
__global__ __launch_bounds__(kBlock) void reindex_kernel(ReindexArgs a) {
  __shared__ f32x4 tab_s[STAGE ? kBlock / 64 : 1][2][STAGE ? kTabTv : 1][2];
  int64_t end = a.rows_cap;
  if (a.n_rows) end = min(end, *a.n_rows);
  const int64_t n = end - a.row_begin;               // rows [row_begin, end)
  if (n <= 0) return;
  const uint32_t per_row = a.div_row.d;
  const uint32_t per_layer = (uint32_t)(n * (int64_t)per_row);
  const uint32_t tiles = (per_layer + kSpan - 1) / kSpan;
  const uint32_t item = xcd_item(blockIdx.x, tiles * a.n_layers);
  if (item == UINT32_MAX) return;
  const uint32_t layer = item / tiles;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t w0 = (item - layer * tiles) * kSpan + wave * kWaveSpan;
  if (w0 >= per_layer) return;
  const uint32_t lane = threadIdx.x & 63;
  const int32_t* __restrict__ rframe = a.row_frame + a.row_begin;
  const uint32_t nf = (uint32_t)a.rope.n_frames;
  uint32_t ja = 0;
  int fa = 0, fb = 0;
  float da = 0.0f, db = 0.0f;
  if (WAVE_ROWS) {
    ja = fdiv(w0, a.div_row);
    const uint32_t jb = (int64_t)ja + 1 < n ? ja + 1 : ja;
    fa = uniform_load(rframe + ja);
    fb = uniform_load(rframe + jb);
    // a frame outside the table is skipped rather than read out of bounds
    da = (uint32_t)fa < nf ? uniform_load(a.rope.delta + fa) : 0.0f;
    db = (uint32_t)fb < nf ? uniform_load(a.rope.delta + fb) : 0.0f;
    if (da == 0.0f && db == 0.0f) return;
  }
  // STAGE: lane e < 2 tv_count loads entry (frame a if e < tv_count else b,
  // vector e mod tv_count) of the {cos, sin} table (entry 0 for a frame that
  // does not move)
  f32x4 st0 = {}, st1 = {};
  int st_f = 0, st_v = 0;
  const bool st_ld = STAGE && (int)lane < 2 * a.rope.tv_count;
  if (STAGE && st_ld) {
    st_f = (int)lane >= a.rope.tv_count;
    st_v = (int)lane - st_f * a.rope.tv_count;
    const int fx = st_f ? fb : fa;
    const float dx = st_f ? db : da;
    const f32x4* t = reinterpret_cast<const f32x4*>(
        a.rope.cs + (int64_t)(dx != 0.0f ? fx : 0) * a.rope.pairs_padded + st_v * a.rope.ppv);
    st0 = t[0];
    st1 = t[1];
  }
  u32x4* __restrict__ lay = reinterpret_cast<u32x4*>(a.layers[layer]);
  u32x4* p[2];
  f32x4 t01[2], t23[2];
  bool go[2], in_block[2];
  int nv[2];
  int sel[2] = {0, 0}, tvs[2] = {0, 0};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t i = w0 + u * 64 + lane;
    const bool live = i < per_layer;
    const uint32_t j = fdiv(live ? i : w0, a.div_row);
    int f;
    float dl;
    if (WAVE_ROWS) {
      f = j != ja ? fb : fa;
      dl = j != ja ? db : da;
    } else {
      f = rframe[j];
      dl = (uint32_t)f < nf ? a.rope.delta[f] : 0.0f;
    }
    go[u] = live && dl != 0.0f;
    const uint32_t rem = (live ? i : w0) - j * per_row;
    const uint32_t h = fdiv(rem, a.div_head);
    const int wq = a.rope.wv_begin + (int)(rem - h * a.div_head.d);   // vector in the segment
    const int tv = wq - a.rope.tv_off;
    in_block[u] = tv >= 0 && tv < a.rope.tv_count;
    const int p0 = in_block[u] ? tv * a.rope.ppv : 0;
    nv[u] = min(a.rope.ppv, a.rope.n_pairs - p0);
    if (!STAGE) {
      const f32x4* t = reinterpret_cast<const f32x4*>(
          a.rope.cs + (int64_t)(go[u] ? f : 0) * a.rope.pairs_padded + p0);
      t01[u] = t[0];     // the table has a 32-byte tail, so t[1] is readable
      t23[u] = t[1];
    } else {
      sel[u] = j != ja;
      tvs[u] = in_block[u] ? tv : 0;
    }
    p[u] = lay + (a.row_begin + (int64_t)j) * a.row_vec + h * a.rope.head_stride_v + wq;
  }
  u32x4 v[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (go[u]) v[u] = __builtin_nontemporal_load(p[u]);
  if (STAGE) {
    if (st_ld) {
      tab_s[wave][st_f][st_v][0] = st0;
      tab_s[wave][st_f][st_v][1] = st1;
    }
    __builtin_amdgcn_wave_barrier();     // LDS accesses of one wavefront stay in order
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      t01[u] = tab_s[wave][sel[u]][tvs[u]][0];
      t23[u] = tab_s[wave][sel[u]][tvs[u]][1];
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!go[u]) continue;
    if (in_block[u]) v[u] = rotate_vec_tab(v[u], a.dtype, t01[u], t23[u], nv[u]);
    __builtin_nontemporal_store(v[u], p[u]);
  }
}

// The {cos, sin} table of one uniform step, for every pair (fp32 angle, fp64
// sincos, as rope_prepare_kernel), padded with the identity so that four pairs
// can be read from any vector's first pair.
__global__ __launch_bounds__(64) void shift_table_kernel(const float* __restrict__ theta,
                                                         int32_t n_pairs, int32_t entries,
                                                         float delta, f32x2* __restrict__ cs) {
  for (int j = threadIdx.x; j < entries; j += 64) {
    f32x2 v = {1.0f, 0.0f};
    if (j < n_pairs) {
      float ang = theta[j] * delta;
      double sd, cd;
      sincos((double)ang, &sd, &cd);
      v.x = (float)cd;
      v.y = (float)sd;
    }
    cs[j] = v;
  }
}

struct ShiftArgs {
  void* const* layers;
  const int64_t* n_rows;
  int64_t row_begin;
  int64_t rows_cap;
  const f32x2* cs;    // the step's table
  int32_t n_pairs;
  FastDiv div_row;    // walked vectors per row = H * wv_count
  FastDiv div_head;   // walked vectors per head = wv_count
  uint32_t row_vec;   // 16-byte vectors per token row (H * vph)
  uint32_t n_layers;
  int32_t dtype;
  int32_t tv_off, tv_count, ppv, wv_begin, head_stride_v;
};

// The walk of reindex_kernel (two vectors per lane, XCD-contiguous order) with
// the same table for every row: no row frames.  STAGE: lanes e < tv_count load
// the table entry of vector e once and share it through the wavefront's LDS
// slot, as reindex_kernel does.
template <bool STAGE>
__global__ __launch_bounds__(kBlock) void shift_kernel(ShiftArgs a) {
  __shared__ f32x4 tab_s[STAGE ? kBlock / 64 : 1][STAGE ? kTabTv : 1][2];
  int64_t end = a.rows_cap;
  if (a.n_rows) end = min(end, *a.n_rows);
  const int64_t n = end - a.row_begin;                 // rows [row_begin, end)
  if (n <= 0) return;
  const uint32_t per_row = a.div_row.d;
  const uint32_t per_layer = (uint32_t)(n * (int64_t)per_row);
  const uint32_t tiles = (per_layer + kSpan - 1) / kSpan;
  const uint32_t item = xcd_item(blockIdx.x, tiles * a.n_layers);
  if (item == UINT32_MAX) return;
  const uint32_t layer = item / tiles;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t w0 = (item - layer * tiles) * kSpan + wave * kWaveSpan;
  if (w0 >= per_layer) return;
  const uint32_t lane = threadIdx.x & 63;
  f32x4 st0 = {}, st1 = {};
  const bool st_ld = STAGE && (int)lane < a.tv_count;
  if (STAGE && st_ld) {
    const f32x4* t = reinterpret_cast<const f32x4*>(a.cs + (int)lane * a.ppv);
    st0 = t[0];
    st1 = t[1];
  }
  u32x4* __restrict__ lay = reinterpret_cast<u32x4*>(a.layers[layer]);
  u32x4* p[2];
  f32x4 t01[2], t23[2];
  bool live[2], in_block[2];
  int nv[2];
  int tvs[2] = {0, 0};
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t i = w0 + u * 64 + lane;
    live[u] = i < per_layer;
    const uint32_t ii = live[u] ? i : w0;
    const uint32_t j = fdiv(ii, a.div_row);
    const uint32_t rem = ii - j * per_row;
    const uint32_t h = fdiv(rem, a.div_head);
    const int wq = a.wv_begin + (int)(rem - h * a.div_head.d);   // vector in the segment
    const int tv = wq - a.tv_off;
    in_block[u] = tv >= 0 && tv < a.tv_count;
    const int p0 = in_block[u] ? tv * a.ppv : 0;
    nv[u] = min(a.ppv, a.n_pairs - p0);
    if (!STAGE) {
      const f32x4* t = reinterpret_cast<const f32x4*>(a.cs + p0);
      t01[u] = t[0];     // the table is padded, so t[1] is readable
      t23[u] = t[1];
    } else {
      tvs[u] = in_block[u] ? tv : 0;
    }
    p[u] = lay + (a.row_begin + (int64_t)j) * a.row_vec + h * a.head_stride_v + wq;
  }
  u32x4 v[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (live[u]) v[u] = __builtin_nontemporal_load(p[u]);
  if (STAGE) {
    if (st_ld) {
      tab_s[wave][lane][0] = st0;
      tab_s[wave][lane][1] = st1;
    }
    __builtin_amdgcn_wave_barrier();     // LDS accesses of one wavefront stay in order
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      t01[u] = tab_s[wave][tvs[u]][0];
      t23[u] = tab_s[wave][tvs[u]][1];
    }
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (!live[u]) continue;
    if (in_block[u]) v[u] = rotate_vec_tab(v[u], a.dtype, t01[u], t23[u], nv[u]);
    __builtin_nontemporal_store(v[u], p[u]);
  }
}

}  // namespace

size_t rope_ws_bytes(int32_t n_frames, int32_t n_pairs) {
  size_t pp = (size_t)((n_pairs + 3) / 4) * 4;
  size_t dbytes = ((size_t)n_frames * 4 + 15) / 16 * 16;
  return dbytes + (size_t)n_frames * pp * sizeof(f32x2) + 32;   // 32-byte tail: see gather
}

void rope_view(const dp_rope& r, const void* ws, RopeView* view, int dtype, int head_dim,
               int n_heads) {
  const int32_t pp = (r.n_pairs + 3) / 4 * 4;
  const size_t dbytes = ((size_t)r.n_frames * 4 + 15) / 16 * 16;
  const float* delta = reinterpret_cast<const float*>(ws);
  const f32x2* cs =
      ws ? reinterpret_cast<const f32x2*>(reinterpret_cast<const char*>(ws) + dbytes) : nullptr;
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
  const int vph = head_dim * esz / 16;
  view->split = r.key_layout == DP_KEY_SPLIT;
  if (view->split) {
    // the head's temporal block, exactly (whole vectors, checked by the caller)
    view->wv_begin = 0;
    view->wv_count = view->tv_count;
    view->head_stride_v = view->tv_count;
    view->tv_off = 0;
    view->blk_end = n_heads * view->tv_count;
  } else {
    const int wb = view->tv_begin / 8 * 8;
    int we = (view->tv_begin + view->tv_count + 7) / 8 * 8;
    if (we > vph) we = vph;
    view->wv_begin = wb;
    view->wv_count = we - wb;
    view->head_stride_v = vph;
    view->tv_off = view->tv_begin;
    view->blk_end = 0x7FFFFFFF;
  }
}

dp_status launch_rope_prepare(const dp_rope& r, void* ws, RopeView* view, int dtype,
                              int head_dim, int n_heads, hipStream_t s) {
  const int32_t pp = (r.n_pairs + 3) / 4 * 4;
  const size_t dbytes = ((size_t)r.n_frames * 4 + 15) / 16 * 16;
  float* delta = reinterpret_cast<float*>(ws);
  f32x2* cs = reinterpret_cast<f32x2*>(reinterpret_cast<char*>(ws) + dbytes);
  hipLaunchKernelGGL(rope_prepare_kernel, dim3(r.n_frames), dim3(64), 0, s, r.theta, r.n_pairs,
                     pp, r.frame_t, r.frame_phase, r.q0, r.knee, r.inv_factor, r.axis, delta, cs);
  dp_status st = check_launch("rope_prepare_kernel");
  if (st != DP_OK) return st;
  rope_view(r, ws, view, dtype, head_dim, n_heads);
  return DP_OK;
}

dp_status launch_reindex(void* const* k, int32_t n_layers, int32_t n_heads, int32_t head_dim,
                         int32_t dtype, int64_t row_begin, int64_t rows_cap,
                         const int64_t* n_rows, const int32_t* row_frame, const RopeView& rope,
                         hipStream_t s) {
  ReindexArgs a;
  a.layers = k;
  a.row_frame = row_frame;
  a.n_rows = n_rows;
  a.row_begin = row_begin;
  a.rows_cap = rows_cap;
  a.div_row = make_fastdiv((uint32_t)(n_heads * rope.wv_count));
  a.div_head = make_fastdiv((uint32_t)rope.wv_count);
  a.row_vec = (uint32_t)(n_heads * (head_dim * elem_size(dtype) / 16));
  a.n_layers = (uint32_t)n_layers;
  a.dtype = dtype;
  a.rope = rope;
  const uint64_t span = rows_cap > row_begin ? (uint64_t)(rows_cap - row_begin) : 0;
  const uint64_t gx = xcd_grid((span * a.div_row.d + kSpan - 1) / kSpan * (uint64_t)n_layers);
  if (gx == 0) return DP_OK;
  if (a.div_row.d >= (uint32_t)kWaveSpan && rope.tv_count <= kTabTv)
    hipLaunchKernelGGL((reindex_kernel<true, true>), dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  else if (a.div_row.d >= (uint32_t)kWaveSpan)
    hipLaunchKernelGGL((reindex_kernel<true, false>), dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((reindex_kernel<false, false>), dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  return check_launch("reindex_kernel");
}

size_t rope_shift_ws_bytes(int32_t n_pairs) {
  return (size_t)((n_pairs + 3) / 4 * 4 + 4) * sizeof(f32x2);
}

dp_status launch_rope_shift(void* const* k, int32_t n_layers, int32_t n_heads, int32_t head_dim,
                            int32_t dtype, int64_t row_begin, int64_t rows_cap,
                            const int64_t* n_rows, const float* theta, int32_t pair_begin,
                            int32_t n_pairs, int32_t key_layout, float delta, void* ws,
                            hipStream_t s) {
  if (delta == 0.0f || rows_cap <= row_begin) return DP_OK;   // nothing moves
  dp_rope r{};
  r.pair_begin = pair_begin;
  r.n_pairs = n_pairs;
  r.n_frames = 1;
  r.key_layout = key_layout;
  RopeView view{};
  rope_view(r, nullptr, &view, dtype, head_dim, n_heads);      // pair layout only
  f32x2* cs = reinterpret_cast<f32x2*>(ws);
  hipLaunchKernelGGL(shift_table_kernel, dim3(1), dim3(64), 0, s, theta, n_pairs,
                     view.pairs_padded + 4, delta, cs);
  dp_status st = check_launch("shift_table_kernel");
  if (st != DP_OK) return st;
  ShiftArgs a;
  a.layers = k;
  a.n_rows = n_rows;
  a.row_begin = row_begin;
  a.rows_cap = rows_cap;
  a.cs = cs;
  a.n_pairs = n_pairs;
  a.div_row = make_fastdiv((uint32_t)(n_heads * view.wv_count));
  a.div_head = make_fastdiv((uint32_t)view.wv_count);
  a.row_vec = (uint32_t)(n_heads * (head_dim * elem_size(dtype) / 16));
  a.n_layers = (uint32_t)n_layers;
  a.dtype = dtype;
  a.tv_off = view.tv_off;
  a.tv_count = view.tv_count;
  a.ppv = view.ppv;
  a.wv_begin = view.wv_begin;
  a.head_stride_v = view.head_stride_v;
  const uint64_t gx = xcd_grid(((uint64_t)(rows_cap - row_begin) * a.div_row.d + kSpan - 1) /
                               kSpan * (uint64_t)n_layers);
  if (a.tv_count <= kTabTv)
    hipLaunchKernelGGL(shift_kernel<true>, dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL(shift_kernel<false>, dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  return check_launch("shift_kernel");
}

}  // namespace dp
