// DeCoPrune-HS: head-specialised ragged cache (DeCoPrune page, section 무엇과
// 다른가).  Dynamic heads keep the DeCoPrune mask, static heads follow the
// Streaming policy (sink + recent window), so heads of one layer keep
// different row sets and the cache becomes ragged per head.
//
// hs_offsets_kernel: one workgroup scans the per-(layer, head) lengths into
//   int64 offsets (row-major over layer, head).
// hs_gather_kernel: blockIdx.y = (layer, K|V); blockIdx.x = one tile of kRT
//   consecutive entries of one class's index list.  The workgroup lists the
//   heads of that class in its layer (LDS) and copies, for each such head, the
//   kRT head rows (head_dim elements each) to that head's contiguous run in the
//   packed output, so every head's writes are kRT * head-row bytes contiguous.
//   Optionally re-rotates the temporal K vectors on the way.
// hs_reindex_kernel: the same walk over a packed ragged K cache, touching only
//   the temporal vectors, in place.
#include "dp_internal.h"

namespace dp {
namespace {

constexpr int kRT = 16;          // class-list entries per workgroup tile
constexpr int kLogRT = 4;
constexpr int kMaxHeads = 1024;

__global__ __launch_bounds__(kBlock) void hs_offsets_kernel(const uint8_t* __restrict__ head_class,
                                                            int64_t n, const int64_t* __restrict__ class_len,
                                                            int32_t n_classes,
                                                            int64_t* __restrict__ offsets) {
  __shared__ int64_t wave_tot[kBlock / 64];
  __shared__ int64_t carry_s;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x / 64;
  for (int64_t start = 0; start < n; start += kBlock) {
    const int64_t i = start + threadIdx.x;
    int64_t v = 0;
    if (i < n) {
      const int c = head_class[i];
      v = c < n_classes ? class_len[c] : 0;
    }
    int64_t x = v;
    for (int o = 1; o < 64; o *= 2) {
      int64_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    int64_t before = carry_s;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    if (i < n) offsets[i + 1] = before + x;
    int64_t chunk = 0;
    for (int w = 0; w < kBlock / 64; ++w) chunk += wave_tot[w];
    __syncthreads();
    if (threadIdx.x == 0) carry_s += chunk;
    __syncthreads();
  }
  if (threadIdx.x == 0) offsets[0] = 0;
}

struct HsArgs {
  const void* const* k_src;       // gather: token-major layers
  const void* const* v_src;
  void* k_out;                    // packed per-head rows
  void* v_out;
  const uint8_t* head_class;
  const int32_t* const* class_idx;
  const int32_t* const* class_rf;
  const int64_t* class_len;
  const int64_t* offsets;
  int32_t* dev_error;
  int64_t src_rows;
  int64_t out_cap;
  int64_t class_cap[DP_HS_MAX_CLASSES];
  uint32_t tile_base[DP_HS_MAX_CLASSES + 1];
  int32_t n_classes;
  int32_t n_heads;
  int32_t n_kv;
  int32_t dtype;
  int32_t has_rope;
  uint32_t vph;                   // 16-byte vectors per head row
  FastDiv div_inner;              // vectors walked per head row: vph (gather) or tv_count
  RopeView rope;
};

// Common prologue: class, first entry, live rows, head list of the class in
// this layer.  Returns the number of heads (0: nothing to do).
__device__ int hs_setup(const HsArgs& a, int layer, int& cls, int64_t& j0, int& rows,
                        int* heads, int64_t* head_off) {
  cls = 0;
  while (cls + 1 < a.n_classes && blockIdx.x >= a.tile_base[cls + 1]) ++cls;
  j0 = (int64_t)(blockIdx.x - a.tile_base[cls]) * kRT;
  int64_t len = a.class_len[cls];
  if (len > a.class_cap[cls]) {
    if (a.dev_error && blockIdx.x == a.tile_base[cls] && threadIdx.x == 0) *a.dev_error = DP_ECAPACITY;
    len = a.class_cap[cls];
  }
  if (j0 >= len) return 0;
  rows = (int)min((int64_t)kRT, len - j0);
  __shared__ int nh_s;
  if (threadIdx.x == 0) {
    int nh = 0;
    const uint8_t* hc = a.head_class + (int64_t)layer * a.n_heads;
    for (int h = 0; h < a.n_heads; ++h)
      if (hc[h] == cls) {
        heads[nh] = h;
        head_off[nh] = a.offsets[(int64_t)layer * a.n_heads + h];
        ++nh;
      }
    nh_s = nh;
  }
  __syncthreads();
  return nh_s;
}

template <int U>
__global__ __launch_bounds__(kBlock) void hs_gather_kernel(HsArgs a) {
  __shared__ int heads[kMaxHeads];
  __shared__ int64_t head_off[kMaxHeads];
  const int layer = blockIdx.y / a.n_kv;
  const bool is_v = (blockIdx.y % a.n_kv) == 1;
  int cls, rows;
  int64_t j0;
  const int nh = hs_setup(a, layer, cls, j0, rows, heads, head_off);
  if (nh == 0) return;
  const u32x4* __restrict__ src =
      reinterpret_cast<const u32x4*>(is_v ? a.v_src[layer] : a.k_src[layer]);
  u32x4* __restrict__ out = reinterpret_cast<u32x4*>(is_v ? a.v_out : a.k_out);
  const int32_t* __restrict__ list = a.class_idx[cls];
  const int32_t* __restrict__ rf = a.has_rope ? a.class_rf[cls] : nullptr;
  const bool rope = a.has_rope && !is_v;
  const uint32_t per_head = (uint32_t)kRT * a.vph;
  const uint32_t total = (uint32_t)nh * per_head;
  bool overflow = false;
  for (uint32_t base = 0; base < total; base += kBlock * U) {
    u32x4 v[U];
    int64_t dst_i[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = base + u * kBlock + threadIdx.x;
      dst_i[u] = -1;
      if (i < total) {
        const uint32_t t = fdiv(i, a.div_inner);           // (head, row)
        const uint32_t q = i - t * a.div_inner.d;           // vector in the head row
        const int r = (int)(t & (kRT - 1));
        const int k = (int)(t >> kLogRT);
        if (r < rows) {
          const int64_t j = j0 + r;
          const int32_t s = list[j];
          const int64_t o = head_off[k] + j;
          if (o >= a.out_cap) {
            overflow = true;
          } else if ((uint32_t)s < (uint64_t)a.src_rows) {
            v[u] = src[((int64_t)s * a.n_heads + heads[k]) * a.vph + q];
            if (rope) {
              const int tv = (int)q - a.rope.tv_begin;
              const int f = rf[j];
              if (tv >= 0 && tv < a.rope.tv_count && (uint32_t)f < (uint32_t)a.rope.n_frames &&
                  a.rope.delta[f] != 0.0f) {
                const int p0 = tv * a.rope.ppv;
                const int nv = min(a.rope.ppv, a.rope.n_pairs - p0);
                v[u] = rotate_vec(v[u], a.dtype, a.rope.cs + (int64_t)f * a.rope.pairs_padded + p0, nv);
              }
            }
            dst_i[u] = o * a.vph + q;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (dst_i[u] >= 0) __builtin_nontemporal_store(v[u], out + dst_i[u]);
  }
  if (overflow && a.dev_error) *a.dev_error = DP_ECAPACITY;
}

template <int U>
__global__ __launch_bounds__(kBlock) void hs_reindex_kernel(HsArgs a) {
  __shared__ int heads[kMaxHeads];
  __shared__ int64_t head_off[kMaxHeads];
  const int layer = blockIdx.y;
  int cls, rows;
  int64_t j0;
  const int nh = hs_setup(a, layer, cls, j0, rows, heads, head_off);
  if (nh == 0) return;
  u32x4* __restrict__ kbuf = reinterpret_cast<u32x4*>(a.k_out);
  const int32_t* __restrict__ rf = a.class_rf[cls];
  const uint32_t total = (uint32_t)nh * kRT * a.div_inner.d;
  for (uint32_t base = 0; base < total; base += kBlock * U) {
    u32x4 v[U];
    int64_t at[U];
    int fr[U], tvs[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = base + u * kBlock + threadIdx.x;
      at[u] = -1;
      if (i < total) {
        const uint32_t t = fdiv(i, a.div_inner);
        const int tv = (int)(i - t * a.div_inner.d);
        const int r = (int)(t & (kRT - 1));
        const int k = (int)(t >> kLogRT);
        if (r < rows) {
          const int64_t j = j0 + r;
          const int f = rf[j];
          const int64_t o = head_off[k] + j;
          if (o < a.out_cap && (uint32_t)f < (uint32_t)a.rope.n_frames && a.rope.delta[f] != 0.0f) {
            at[u] = o * a.vph + a.rope.tv_begin + tv;
            fr[u] = f;
            tvs[u] = tv;
            v[u] = __builtin_nontemporal_load(kbuf + at[u]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (at[u] >= 0) {
        const int p0 = tvs[u] * a.rope.ppv;
        const int nv = min(a.rope.ppv, a.rope.n_pairs - p0);
        __builtin_nontemporal_store(
            rotate_vec(v[u], a.dtype, a.rope.cs + (int64_t)fr[u] * a.rope.pairs_padded + p0, nv),
            kbuf + at[u]);
      }
    }
  }
}

void fill_tiles(HsArgs& a, const int64_t* class_cap, int32_t n_classes) {
  a.n_classes = n_classes;
  uint32_t acc = 0;
  for (int c = 0; c < DP_HS_MAX_CLASSES; ++c) {
    a.tile_base[c] = acc;
    a.class_cap[c] = c < n_classes ? class_cap[c] : 0;
    if (c < n_classes) acc += (uint32_t)((class_cap[c] + kRT - 1) / kRT);
  }
  a.tile_base[DP_HS_MAX_CLASSES] = acc;
}

}  // namespace

uint64_t hs_tiles(const int64_t* class_cap, int32_t n_classes) {
  uint64_t acc = 0;
  for (int c = 0; c < n_classes; ++c) acc += (uint64_t)((class_cap[c] + kRT - 1) / kRT);
  return acc;
}

int hs_max_heads() { return kMaxHeads; }

dp_status launch_hs_offsets(const uint8_t* head_class, int32_t L, int32_t H,
                            const int64_t* class_len, int32_t n_classes, int64_t* offsets,
                            hipStream_t s) {
  hipLaunchKernelGGL(hs_offsets_kernel, dim3(1), dim3(kBlock), 0, s, head_class,
                     (int64_t)L * H, class_len, n_classes, offsets);
  return check_launch("hs_offsets_kernel");
}

dp_status launch_hs_gather(const dp_kv_hs& kv, const uint8_t* head_class, int32_t n_classes,
                           const int32_t* const* class_idx, const int64_t* class_len,
                           const int64_t* class_cap, const int64_t* offsets,
                           const int32_t* const* class_rf, const RopeView* rope,
                           hipStream_t s) {
  HsArgs a{};
  a.k_src = kv.k_src;
  a.v_src = kv.v_src;
  a.k_out = kv.k_out;
  a.v_out = kv.v_out;
  a.head_class = head_class;
  a.class_idx = class_idx;
  a.class_rf = class_rf;
  a.class_len = class_len;
  a.offsets = offsets;
  a.dev_error = kv.dev_error;
  a.src_rows = kv.src_rows;
  a.out_cap = kv.out_capacity;
  a.n_heads = kv.n_heads;
  a.n_kv = kv.v_src ? 2 : 1;
  a.dtype = kv.dtype;
  a.has_rope = rope != nullptr;
  if (rope) a.rope = *rope;
  a.vph = (uint32_t)(kv.head_dim * elem_size(kv.dtype) / 16);
  a.div_inner = make_fastdiv(a.vph);
  fill_tiles(a, class_cap, n_classes);
  const uint32_t gx = a.tile_base[DP_HS_MAX_CLASSES];
  if (gx == 0) return DP_OK;
  hipLaunchKernelGGL(hs_gather_kernel<4>, dim3(gx, kv.n_layers * a.n_kv), dim3(kBlock), 0, s, a);
  return check_launch("hs_gather_kernel");
}

dp_status launch_hs_reindex(void* k, int64_t k_cap, int32_t L, int32_t H, int32_t head_dim, int32_t dtype,
                            const uint8_t* head_class, int32_t n_classes,
                            const int64_t* class_len, const int64_t* class_cap,
                            const int64_t* offsets, const int32_t* const* class_rf,
                            const RopeView& rope, hipStream_t s) {
  HsArgs a{};
  a.k_out = k;
  a.head_class = head_class;
  a.class_rf = class_rf;
  a.class_len = class_len;
  a.offsets = offsets;
  a.out_cap = k_cap;
  a.n_heads = H;
  a.n_kv = 1;
  a.dtype = dtype;
  a.has_rope = 1;
  a.rope = rope;
  a.vph = (uint32_t)(head_dim * elem_size(dtype) / 16);
  a.div_inner = make_fastdiv((uint32_t)rope.tv_count);
  fill_tiles(a, class_cap, n_classes);
  const uint32_t gx = a.tile_base[DP_HS_MAX_CLASSES];
  if (gx == 0) return DP_OK;
  hipLaunchKernelGGL(hs_reindex_kernel<4>, dim3(gx, L), dim3(kBlock), 0, s, a);
  return check_launch("hs_reindex_kernel");
}

}  // namespace dp
