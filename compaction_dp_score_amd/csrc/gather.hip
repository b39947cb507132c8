// dp_gather_kv: physical gather of the kept rows of every layer.
//
// The DeCoPrune page (section 어떻게 동작하나) updates the cache physically:
// when a non-sink chunk leaves the window, each layer keeps only the selected
// entries K[m], V[m], so the KV sequence length really shrinks.
//
// One launch covers all layers and both K and V: blockIdx.y = (layer, K|V),
// blockIdx.x walks the destination slab of that layer as a flat array of
// 16-byte vectors.  Vector i of the slab is column c = i mod RV of destination
// row j = i div RV (RV = row bytes / 16, division by multiply-high), read from
// source row idx[j].  Consecutive lanes read and write consecutive 16-byte
// vectors of the same row, so every wavefront moves 1 KiB contiguous on both
// sides; a row is 10 KiB for 40 heads x 128 bf16.  Optionally the K vectors of
// the temporal RoPE block are re-rotated in registers on the way (no extra
// HBM bytes).  HBM-bound: 2 x row bytes per kept row per layer and tensor.
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
  FastDiv div_head;    // vectors per head row
  uint32_t total_cap;  // dst_cap * RV
  int32_t n_kv;        // 1 (K only) or 2
  int32_t dtype;
  int32_t has_rope;
  const int32_t* row_frame;
  RopeView rope;
};

template <int U>
__global__ __launch_bounds__(kBlock) void gather_kernel(GatherArgs a) {
  const int64_t nk = *a.n_kept;
  const int64_t n = nk < a.dst_cap ? nk : a.dst_cap;
  if (nk > a.dst_cap && a.dev_error && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
    *a.dev_error = DP_ECAPACITY;
  const uint32_t total = (uint32_t)(n * (int64_t)a.div_row.d);
  const uint32_t first = blockIdx.x * (kBlock * U);
  if (first >= total) return;
  const int layer = blockIdx.y / a.n_kv;
  const bool is_v = (blockIdx.y % a.n_kv) == 1;
  const u32x4* __restrict__ src =
      reinterpret_cast<const u32x4*>(is_v ? a.v_src[layer] : a.k_src[layer]);
  u32x4* __restrict__ dst = reinterpret_cast<u32x4*>(is_v ? a.v_dst[layer] : a.k_dst[layer]);
  const bool rope = a.has_rope && !is_v;

  u32x4 v[U];
  uint32_t jrow[U], col[U];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t i = first + u * kBlock + threadIdx.x;
    ok[u] = false;
    if (i < total) {
      const uint32_t j = fdiv(i, a.div_row);
      const uint32_t c = i - j * a.div_row.d;
      const int32_t s = a.idx[j];
      jrow[u] = j;
      col[u] = c;
      if ((uint32_t)s < (uint64_t)a.src_rows) {   // out-of-range entries are skipped
        v[u] = src[(int64_t)s * a.div_row.d + c];
        ok[u] = true;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!ok[u]) continue;
    u32x4 w = v[u];
    if (rope) {
      const uint32_t h = fdiv(col[u], a.div_head);
      const int tv = (int)(col[u] - h * a.div_head.d) - a.rope.tv_begin;
      if (tv >= 0 && tv < a.rope.tv_count) {
        const int f = a.row_frame[jrow[u]];
        if ((uint32_t)f < (uint32_t)a.rope.n_frames && a.rope.delta[f] != 0.0f) {
          const int p0 = tv * a.rope.ppv;
          const int nv = min(a.rope.ppv, a.rope.n_pairs - p0);
          w = rotate_vec(w, a.dtype, a.rope.cs + (int64_t)f * a.rope.pairs_padded + p0, nv);
        }
      }
    }
    __builtin_nontemporal_store(w, dst + first + u * kBlock + threadIdx.x);
  }
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
  a.div_head = make_fastdiv((uint32_t)(kv.head_dim * elem_size(kv.dtype) / 16));
  a.total_cap = (uint32_t)(kv.dst_capacity * rv);
  a.n_kv = kv.v_src ? 2 : 1;
  a.dtype = kv.dtype;
  a.has_rope = rope != nullptr;
  a.row_frame = row_frame;
  if (rope) a.rope = *rope;
  else a.rope = RopeView{};
  if (a.total_cap == 0) return DP_OK;
  constexpr int U = 1;
  const uint32_t gx = (uint32_t)(((uint64_t)a.total_cap + kBlock * U - 1) / (kBlock * U));
  hipLaunchKernelGGL(gather_kernel<U>, dim3(gx, kv.n_layers * a.n_kv), dim3(kBlock), 0, s, a);
  return check_launch("gather_kernel");
}

}  // namespace dp
