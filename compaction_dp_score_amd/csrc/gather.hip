// dp_gather_kv: physical gather of the kept rows of every layer.
//
// The DeCoPrune page (section 어떻게 동작하나) updates the cache physically:
// when a non-sink chunk leaves the window, each layer keeps only the selected
// entries K[m], V[m], so the KV sequence length really shrinks.
//
// One launch covers all layers and both K and V.  The destination of each
// (layer, K|V) slab is a flat array of 16-byte vectors; vector i is column
// c = i mod RV of destination row j = i div RV (RV = row bytes / 16, division
// by multiply-high), read from source row idx[j].  The grid is 1-D and sized
// by the destination capacity; every workgroup reads the kept count first and
// derives (slab, tile) from its id with the number of live tiles per slab, in
// XCD-contiguous order over the live tiles (each XCD streams one contiguous
// eighth; measured 1.6 % faster than plain order at the two-minute eviction),
// so surplus workgroups exit at once.  Consecutive lanes
// read and write consecutive 16-byte vectors of one row (a row is 10 KiB for
// 40 heads x 128 bf16), with non-temporal loads and stores: the data is used
// once.  Optionally the K vectors of the temporal RoPE block are re-rotated
// in registers on the way (no extra HBM bytes).  HBM-bound: 2 x row bytes per
// kept row per layer and tensor.
#include "dp_internal.h"

namespace dp {
namespace {


struct GatherArgs {
  const void* const* k_src;
  const void* const* v_src;
  void* const* k_dst;
  void* const* v_dst;
  const int32_t* idx;
  const int64_t* n_kept;
  int64_t dst_cap;
  int64_t src_rows;
  int32_t* dev_error;
  FastDiv div_row;     // RV: 16-byte vectors per row
  FastDiv div_head;    // segment of the fused rotation's walk (see RopeView)
  uint32_t total_cap;  // dst_cap * RV
  uint32_t n_slabs;    // n_layers * n_kv
  int32_t n_kv;        // 1 (K only) or 2
  int32_t dtype;
  int32_t has_rope;
  const int32_t* row_frame;
  RopeView rope;
};

template <bool ROPE>
__global__ __launch_bounds__(kBlock) void gather_kernel(GatherArgs a) {
  const int64_t nk = *a.n_kept;
  const int64_t n = nk < a.dst_cap ? nk : a.dst_cap;
  if (nk > a.dst_cap && a.dev_error && blockIdx.x == 0 && threadIdx.x == 0)
    *a.dev_error = DP_ECAPACITY;
  const uint32_t per_slab = (uint32_t)(n * (int64_t)a.div_row.d);
  const uint32_t tiles = (per_slab + kBlock - 1) / kBlock;
  if (tiles == 0) return;
  const uint32_t item = xcd_item(blockIdx.x, tiles * a.n_slabs);
  if (item == UINT32_MAX) return;
  const uint32_t slab = item / tiles;
  const uint32_t i = (item - slab * tiles) * kBlock + threadIdx.x;
  const int layer = (int)(slab / a.n_kv);
  const bool is_v = (slab % a.n_kv) == 1;
  const u32x4* __restrict__ src =
      reinterpret_cast<const u32x4*>(is_v ? a.v_src[layer] : a.k_src[layer]);
  u32x4* __restrict__ dst = reinterpret_cast<u32x4*>(is_v ? a.v_dst[layer] : a.k_dst[layer]);
  if (i >= per_slab) return;
  const uint32_t j = fdiv(i, a.div_row);
  const uint32_t c = i - j * a.div_row.d;
  if (ROPE && !is_v) {
    // K with the fused re-index.  All lookups the rotation needs are requested
    // before the HBM load of the data (vector loads retire in issue order):
    // the source row and the frame (scalar loads when the wavefront lies in
    // one row, as it does for rows of a multiple of 64 vectors), then the
    // frame's phase step and {cos, sin} (L2 hits that return while the data is
    // in flight).  Lanes outside the temporal block read entry 0 and keep
    // their data.
    const uint32_t h = fdiv(c, a.div_head);
    const int tv = (int)(c - h * a.div_head.d) - a.rope.tv_off;
    const bool in_block = tv >= 0 && tv < a.rope.tv_count && (int)c < a.rope.blk_end;
    const uint32_t j0 = __builtin_amdgcn_readfirstlane(j);
    const bool one_row = __builtin_amdgcn_ballot_w64(j != j0) == 0;
    int32_t s;
    int f;
    if (one_row) {
      s = uniform_load(a.idx + j0);
      f = uniform_load(a.row_frame + j0);
    } else {
      s = a.idx[j];
      f = a.row_frame[j];
    }
    const bool sv = (uint32_t)s < (uint64_t)a.src_rows;   // out-of-range entries are skipped
    const bool fv = (uint32_t)f < (uint32_t)a.rope.n_frames;
    const int fc = fv ? f : 0;
    const int p0 = in_block ? tv * a.rope.ppv : 0;
    const f32x4* t = reinterpret_cast<const f32x4*>(a.rope.cs + (int64_t)fc * a.rope.pairs_padded + p0);
    const float dl = a.rope.delta[fc];
    const f32x4 t01 = t[0];       // the table has a 32-byte tail, so t[1] is readable
    const f32x4 t23 = t[1];
    u32x4 v = __builtin_nontemporal_load(src + (int64_t)(sv ? s : 0) * a.div_row.d + c);
    __builtin_amdgcn_sched_barrier(0);   // the phase-step test stays after the data load
    const int nv = min(a.rope.ppv, a.rope.n_pairs - p0);
    const u32x4 r = rotate_vec_tab(v, a.dtype, t01, t23, nv);
    if (in_block && fv && dl != 0.0f) v = r;
    if (sv) __builtin_nontemporal_store(v, dst + i);
    return;
  }
  const int32_t s = a.idx[j];
  if ((uint32_t)s >= (uint64_t)a.src_rows) return;        // out-of-range entries are skipped
  const u32x4 v = __builtin_nontemporal_load(src + (int64_t)s * a.div_row.d + c);
  __builtin_nontemporal_store(v, dst + i);
}

}  // namespace

dp_status launch_gather(const dp_kv& kv, const int32_t* idx, const int64_t* n_kept,
                        const int32_t* row_frame, const RopeView* rope, hipStream_t s) {
  GatherArgs a;
  a.k_src = kv.k_src;
  a.v_src = kv.v_src;
  a.k_dst = kv.k_dst;
  a.v_dst = kv.v_dst;
  a.idx = idx;
  a.n_kept = n_kept;
  a.dst_cap = kv.dst_capacity;
  a.src_rows = kv.src_rows;
  a.dev_error = kv.dev_error;
  const uint32_t rv = (uint32_t)((int64_t)kv.n_heads * kv.head_dim * elem_size(kv.dtype) / 16);
  a.div_row = make_fastdiv(rv);
  // segment of the fused rotation's walk: the head row (interleaved keys) or
  // the head's temporal block in the row's leading plane (split keys)
  a.div_head = make_fastdiv(rope ? (uint32_t)rope->head_stride_v
                                 : (uint32_t)(kv.head_dim * elem_size(kv.dtype) / 16));
  a.total_cap = (uint32_t)(kv.dst_capacity * rv);
  a.n_kv = kv.v_src ? 2 : 1;
  a.dtype = kv.dtype;
  a.has_rope = rope != nullptr;
  a.row_frame = row_frame;
  if (rope) a.rope = *rope;
  else a.rope = RopeView{};
  a.n_slabs = (uint32_t)(kv.n_layers * a.n_kv);
  if (a.total_cap == 0) return DP_OK;
  const uint64_t gx = xcd_grid((uint64_t)a.n_slabs * (((uint64_t)a.total_cap + kBlock - 1) / kBlock));
  if (rope)
    hipLaunchKernelGGL(gather_kernel<true>, dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL(gather_kernel<false>, dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  return check_launch("gather_kernel");
}

}  // namespace dp
