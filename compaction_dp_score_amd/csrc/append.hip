// dp_append_kept: segment-append compaction in place.
//
// The DeCoPrune page (section 어떻게 동작하나) compacts a chunk when it leaves
// the dense window.  With the cache kept as [sink | window ring | history] in
// one buffer per layer, only the kept rows of the slot that holds the leaving
// chunk move: they are appended at the history tail.  append_kernel copies them
// for all layers, K and V, in one launch (grid y = layer and K|V; a fixed
// number of workgroups per slab stride over the live tiles; one 16-byte vector
// per lane, non-temporal); append_finish_kernel then retires the slot's row frames
// (-1) and advances the tail.  Both launches re-derive the appended span from
// the same device values, and the finish launch runs after the copy on the
// stream, so the tail is never read after it changes.  Optionally the K rows
// are re-rotated on the way by their frames' phase steps (the first re-index of
// a chunk that has just left the window), as the gather does: the lookups go
// out before the data load and the rotation costs no extra HBM bytes.
#include "dp_internal.h"

namespace dp {
namespace {

constexpr uint32_t kAppendBlocksPerSlab = 1024;

struct AppendArgs {
  void* const* k_layers;
  void* const* v_layers;
  const int32_t* idx;
  const int64_t* n_kept;
  int64_t* tail;
  int32_t* row_frame;
  int32_t* dev_error;
  int64_t capacity;
  int64_t slot_begin;
  int64_t slot_rows;
  FastDiv div_row;     // 16-byte vectors per row
  FastDiv div_head;    // 16-byte vectors per head row
  uint32_t n_slabs;    // n_layers * n_kv
  int32_t n_kv;
  int32_t dtype;
  int32_t has_rope;
  RopeView rope;
};

// The appended span [t0, t0 + n); false (with the status) when it would pass
// the capacity or overlap the slot.
__device__ __forceinline__ bool append_span(const AppendArgs& a, int64_t& t0, int64_t& n,
                                            int& err) {
  const int64_t nk = *a.n_kept;
  t0 = *a.tail;
  n = nk < 0 ? 0 : (nk > a.slot_rows ? a.slot_rows : nk);
  err = DP_OK;
  if (t0 < 0 || t0 + n > a.capacity) err = DP_ECAPACITY;
  else if (n > 0 && t0 < a.slot_begin + a.slot_rows && t0 + n > a.slot_begin) err = DP_ERANGE;
  return err == DP_OK;
}

__global__ __launch_bounds__(kBlock) void append_kernel(AppendArgs a) {
  int64_t t0, n;
  int err;
  if (!append_span(a, t0, n, err)) return;            // reported by append_finish_kernel
  const uint32_t per_slab = (uint32_t)(n * (int64_t)a.div_row.d);
  const uint32_t tiles = (per_slab + kBlock - 1) / kBlock;
  const int layer = (int)(blockIdx.y / a.n_kv);
  const bool is_v = (blockIdx.y % a.n_kv) == 1;
  u32x4* __restrict__ base = reinterpret_cast<u32x4*>(is_v ? a.v_layers[layer] : a.k_layers[layer]);
  // A chunk keeps a small share of its rows, so the grid is a fixed number of
  // workgroups per slab that stride over the live tiles (no idle workgroups).
  const bool rope = a.has_rope && !is_v;
  for (uint32_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const uint32_t i = t * kBlock + threadIdx.x;
    if (i >= per_slab) break;
    const uint32_t j = fdiv(i, a.div_row);
    const uint32_t c = i - j * a.div_row.d;
    // When the wavefront's vectors lie in one row (always, when a row is a
    // multiple of 64 vectors), the row's index entry, frame and phase step are
    // scalar loads: the index list, the slot's frames and the steps are not
    // written by this kernel (the frames it writes are at the tail, outside the
    // slot).
    const uint32_t j0 = __builtin_amdgcn_readfirstlane(j);
    const bool one_row = __builtin_amdgcn_ballot_w64(j != j0) == 0;
    const int32_t s = one_row ? uniform_load(a.idx + j0) : a.idx[j];
    const bool sv = (uint64_t)(uint32_t)s < (uint64_t)a.slot_rows;  // out-of-range entries skipped
    const int64_t src = (a.slot_begin + (sv ? s : 0)) * (int64_t)a.div_row.d + c;
    if (rope) {
      // the row's frame, its phase step and {cos, sin} are requested before the
      // data (vector loads retire in order); lanes outside the temporal block
      // read entry 0 and keep their data
      const uint32_t h = fdiv(c, a.div_head);
      const int tv = (int)(c - h * a.div_head.d) - a.rope.tv_off;
      const bool in_block = tv >= 0 && tv < a.rope.tv_count && (int)c < a.rope.blk_end;
      const int32_t* frow = a.row_frame + a.slot_begin + (sv ? s : 0);
      const int f = one_row ? uniform_load(frow) : *frow;
      const bool fv = (uint32_t)f < (uint32_t)a.rope.n_frames;
      const int fc = fv ? f : 0;
      const int p0 = in_block ? tv * a.rope.ppv : 0;
      const f32x4* tb =
          reinterpret_cast<const f32x4*>(a.rope.cs + (int64_t)fc * a.rope.pairs_padded + p0);
      const float dl = one_row ? uniform_load(a.rope.delta + fc) : a.rope.delta[fc];
      const f32x4 t01 = tb[0];     // the table has a 32-byte tail, so tb[1] is readable
      const f32x4 t23 = tb[1];
      u32x4 v = __builtin_nontemporal_load(base + src);
      __builtin_amdgcn_sched_barrier(0);
      const int nv = min(a.rope.ppv, a.rope.n_pairs - p0);
      const u32x4 r = rotate_vec_tab(v, a.dtype, t01, t23, nv);
      if (in_block && fv && dl != 0.0f) v = r;
      if (sv) __builtin_nontemporal_store(v, base + (t0 + j) * (int64_t)a.div_row.d + c);
    } else if (sv) {
      const u32x4 v = __builtin_nontemporal_load(base + src);
      __builtin_nontemporal_store(v, base + (t0 + j) * (int64_t)a.div_row.d + c);
    }
    if (sv && a.row_frame && blockIdx.y == 0 && c == 0)
      a.row_frame[t0 + j] = a.row_frame[a.slot_begin + s];
  }
}

__global__ __launch_bounds__(kBlock) void append_finish_kernel(AppendArgs a) {
  int64_t t0, n;
  int err;
  const bool ok = append_span(a, t0, n, err);
  __syncthreads();                                     // every lane has read *tail
  if (!ok) {
    if (threadIdx.x == 0 && a.dev_error) *a.dev_error = err;
    return;
  }
  if (a.row_frame)
    for (int64_t r = threadIdx.x; r < a.slot_rows; r += kBlock) a.row_frame[a.slot_begin + r] = -1;
  if (threadIdx.x == 0) *a.tail = t0 + n;
}

}  // namespace

dp_status launch_append(const dp_kv_inplace& kv, int64_t slot_begin, int64_t slot_rows,
                        const int32_t* idx, const int64_t* n_kept, int64_t* tail,
                        int32_t* row_frame, const RopeView* rope, hipStream_t s) {
  AppendArgs a;
  a.k_layers = kv.k_layers;
  a.v_layers = kv.v_layers;
  a.idx = idx;
  a.n_kept = n_kept;
  a.tail = tail;
  a.row_frame = row_frame;
  a.dev_error = kv.dev_error;
  a.capacity = kv.capacity;
  a.slot_begin = slot_begin;
  a.slot_rows = slot_rows;
  a.div_row = make_fastdiv((uint32_t)((int64_t)kv.n_heads * kv.head_dim * elem_size(kv.dtype) / 16));
  // segment of the fused rotation's walk: the head row (interleaved keys) or
  // the head's temporal block in the row's leading plane (split keys)
  a.div_head = make_fastdiv(rope ? (uint32_t)rope->head_stride_v
                                 : (uint32_t)(kv.head_dim * elem_size(kv.dtype) / 16));
  a.dtype = kv.dtype;
  a.has_rope = rope != nullptr;
  a.rope = rope ? *rope : RopeView{};
  a.n_kv = kv.v_layers ? 2 : 1;
  a.n_slabs = (uint32_t)(kv.n_layers * a.n_kv);
  const uint64_t tiles_cap = ((uint64_t)slot_rows * a.div_row.d + kBlock - 1) / kBlock;
  const uint32_t gx = (uint32_t)(tiles_cap < kAppendBlocksPerSlab ? tiles_cap : kAppendBlocksPerSlab);
  if (gx > 0) {
    hipLaunchKernelGGL(append_kernel, dim3(gx, a.n_slabs), dim3(kBlock), 0, s, a);
    dp_status st = check_launch("append_kernel");
    if (st != DP_OK) return st;
  }
  hipLaunchKernelGGL(append_finish_kernel, dim3(1), dim3(kBlock), 0, s, a);
  return check_launch("append_finish_kernel");
}

}  // namespace dp
