// DeCoPrune-HS: head-specialised ragged cache (DeCoPrune page, section 무엇과
// 다른가).  Dynamic heads keep the DeCoPrune mask, static heads follow the
// Streaming policy (sink + recent window), so heads of one layer keep
// different row sets and the cache becomes ragged per head.
//
// hs_offsets_kernel: one workgroup scans the per-(layer, head) lengths into
//   int64 offsets (row-major over layer, head).
// hs_gather_kernel: one workgroup per (layer, K|V, tile of kRT consecutive
//   entries of one class's index list).  The workgroup lists the heads of that
//   class in its layer (LDS) and copies, for each such head, the kRT head rows
//   (head_dim elements each) to that head's contiguous run in the packed
//   output, so every head's writes are kRT * head-row bytes contiguous.  Tiles
//   of 128 entries amortise the prologue (measured: 16-entry tiles 4.9 TB/s,
//   64-128 entries 5.3 TB/s).  Optionally re-rotates the temporal K vectors on
//   the way.
// hs_reindex_kernel: the same walk over a packed ragged K cache, in place,
//   rewriting the whole 128-byte lines that hold the temporal pairs.
// Split keys: a split output run of n head rows holds its n temporal blocks,
// then its n remaining parts, so the re-index of a run is one contiguous span
// of whole lines; split source rows hold the temporal blocks of all heads
// first.  The two are independent: interleaved source rows keep each head row
// on whole lines of its own, so the two classes of a layer share no source
// line (with split sources a line holds blocks of both classes and is read
// twice: measured 0.51 of HBM peak against 0.69 on the HS workload).
#include "dp_internal.h"

namespace dp {
namespace {

constexpr int kRT = 128;         // class-list entries per workgroup tile
constexpr int kLogRT = 7;
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
  int32_t n_classes;
  int32_t n_heads;
  int32_t n_layers;
  int32_t n_kv;
  int32_t dtype;
  int32_t has_rope;
  uint32_t vph;                   // 16-byte vectors per head row
  FastDiv div_inner;              // vectors walked per head row: vph (gather) or wv_count
  RopeView rope;
  // split keys: temporal vectors [tvb, tvb + tvc) of a head row, svc = vph - tvc;
  // split: the packed runs, split_src: the source token rows
  int32_t split, split_src;
  uint32_t tvb, tvc, svc;
};

// Per-workgroup state shared by the gather and the re-index.
struct HsTile {
  int cls;          // class of this tile
  int64_t j0;       // first entry of the class list
  int64_t n_run;    // entries of the class list: the length of each of its heads' runs
  int rows;         // live entries in the tile (<= kRT)
  int nh;           // heads of the class in this layer
  int slab;         // (layer, K|V) index
};

// Maps the 1-D workgroup id to (slab, class, tile) using the device-side class
// lengths, so surplus workgroups leave at once; the gather takes the live
// tiles in XCD-contiguous order (on the HS workload, paired runs in
// alternating processes: 0.04 of peak more on average than plain order, 5 of 6
// pairs ahead), the re-index in plain order (3-4 % slower in XCD order); then lists the class's heads of this layer (a wavefront ballot, in head
// order) with their output offsets, and each tile row's source index, frame and
// phase step, all into LDS.  Returns false when the workgroup has no work.
__device__ bool hs_setup(const HsArgs& a, int n_slab_per_layer, bool xcd_order, HsTile& tl,
                         int* heads, int64_t* head_off, int32_t* s_src, int* s_f, float* s_dl) {
  uint32_t pre[DP_HS_MAX_CLASSES + 1];
  int64_t lens[DP_HS_MAX_CLASSES];
  pre[0] = 0;
  bool overflow = false;
#pragma unroll
  for (int c = 0; c < DP_HS_MAX_CLASSES; ++c) {
    int64_t len = 0;
    if (c < a.n_classes) {
      len = a.class_len[c];
      if (len > a.class_cap[c]) {
        overflow = true;
        len = a.class_cap[c];
      }
      if (len < 0) len = 0;
    }
    lens[c] = len;
    pre[c + 1] = pre[c] + (uint32_t)((len + kRT - 1) / kRT);
  }
  if (overflow && a.dev_error && blockIdx.x == 0 && threadIdx.x == 0) *a.dev_error = DP_ECAPACITY;
  const uint32_t live = pre[a.n_classes];
  if (live == 0) return false;
  const uint32_t n_items = live * (uint32_t)(a.n_layers * n_slab_per_layer);
  const uint32_t item = xcd_order ? xcd_item(blockIdx.x, n_items) : blockIdx.x;
  if (item >= n_items) return false;
  const uint32_t slab = item / live;
  const uint32_t r = item - slab * live;
  int cls = 0;
#pragma unroll
  for (int c = 1; c < DP_HS_MAX_CLASSES; ++c)
    if (c < a.n_classes && r >= pre[c]) cls = c;
  tl.cls = cls;
  tl.slab = (int)slab;
  tl.j0 = (int64_t)(r - pre[cls]) * kRT;
  tl.n_run = lens[cls];
  tl.rows = (int)min((int64_t)kRT, lens[cls] - tl.j0);
  const int layer = (int)slab / n_slab_per_layer;

  __shared__ int nh_s;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {                      // wave 0: the class's heads, in order
    const uint8_t* hc = a.head_class + (int64_t)layer * a.n_heads;
    int base = 0;
    for (int h0 = 0; h0 < a.n_heads; h0 += 64) {
      const int h = h0 + lane;
      const bool m = h < a.n_heads && hc[h] == cls;
      const uint64_t mask = __ballot(m);
      if (m) {
        const int rank = base + __popcll(mask & (lane == 0 ? 0ull : (~0ull >> (64 - lane))));
        heads[rank] = h;
        head_off[rank] = a.offsets[(int64_t)layer * a.n_heads + h];
      }
      base += __popcll(mask);
    }
    if (lane == 0) nh_s = base;
  } else if (threadIdx.x < 64 + kRT) {         // wave 1: the tile rows
    const int rr = threadIdx.x - 64;
    int32_t src = -1;
    int f = 0;
    float dl = 0.0f;
    if (rr < tl.rows) {
      const int64_t j = tl.j0 + rr;
      if (a.class_idx) src = a.class_idx[cls][j];
      if (a.has_rope) {
        f = a.class_rf[cls][j];
        if ((uint32_t)f < (uint32_t)a.rope.n_frames) dl = a.rope.delta[f];
        else f = 0;
      }
    }
    s_src[rr] = src;
    s_f[rr] = f;
    s_dl[rr] = dl;
  }
  __syncthreads();
  tl.nh = nh_s;
  return tl.nh > 0;
}

// SD / SS: split output runs / split source rows (compile-time, so that each
// instance carries only its own address arithmetic: with both layouts in one
// body the interleaved gather needed 66 registers instead of 50, one wavefront
// per SIMD fewer)
template <int U, bool SD, bool SS>
__global__ __launch_bounds__(kBlock) void hs_gather_kernel(HsArgs a) {
  __shared__ int heads[kMaxHeads];
  __shared__ int64_t head_off[kMaxHeads];
  __shared__ int32_t s_src[kRT];
  __shared__ int s_f[kRT];
  __shared__ float s_dl[kRT];
  HsTile tl;
  if (!hs_setup(a, a.n_kv, true, tl, heads, head_off, s_src, s_f, s_dl)) return;
  const int layer = tl.slab / a.n_kv;
  const bool is_v = (tl.slab % a.n_kv) == 1;
  const u32x4* __restrict__ src =
      reinterpret_cast<const u32x4*>(is_v ? a.v_src[layer] : a.k_src[layer]);
  u32x4* __restrict__ out = reinterpret_cast<u32x4*>(is_v ? a.v_out : a.k_out);
  const bool rope = a.has_rope && !is_v;
  const uint32_t total = (uint32_t)tl.nh * kRT * a.vph;
  bool overflow = false;
  for (uint32_t b0 = 0; b0 < total; b0 += kBlock * U) {
    u32x4 v[U];
    int64_t dst_i[U];
    f32x4 t01[U], t23[U];
    int nv[U];
    bool rot[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = b0 + u * kBlock + threadIdx.x;
      dst_i[u] = -1;
      rot[u] = false;
      if (i < total) {
        const uint32_t t = fdiv(i, a.div_inner);           // (head, row)
        const uint32_t q = i - t * a.div_inner.d;           // vector in the head row
        const int r = (int)(t & (kRT - 1));
        const int k = (int)(t >> kLogRT);
        const int32_t s = s_src[r];
        if (r < tl.rows && (uint32_t)s < (uint64_t)a.src_rows) {
          const int64_t o = head_off[k] + tl.j0 + r;
          const bool split_k = SD && !is_v;               // split output run
          const bool split_s = SS && !is_v;               // split source row
          // a split run is placed whole, so all of it must fit
          if (head_off[k] < 0 || (split_k ? head_off[k] + tl.n_run : o + 1) > a.out_cap) {
            overflow = true;
          } else {
            // natural vector q of head row (s, h): its place in the source row
            // and in the output run
            const int h = heads[k];
            const bool tq = q >= a.tvb && q < a.tvb + a.tvc;
            const uint32_t sq = q < a.tvb ? q : q - a.tvc;   // index among the other vectors
            int64_t src_i = ((int64_t)s * a.n_heads + h) * a.vph + q;
            dst_i[u] = o * a.vph + q;
            if (split_s)
              src_i = (int64_t)s * a.n_heads * a.vph +
                      (tq ? (int64_t)h * a.tvc + (q - a.tvb)
                          : (int64_t)a.n_heads * a.tvc + (int64_t)h * a.svc + sq);
            if (split_k) {
              const int64_t jr = tl.j0 + r;                  // row within the run
              dst_i[u] = head_off[k] * a.vph +
                         (tq ? jr * a.tvc + (q - a.tvb) : tl.n_run * a.tvc + jr * a.svc + sq);
            }
            if (rope) {
              const int tv = (int)q - a.rope.tv_begin;
              if (tv >= 0 && tv < a.rope.tv_count && s_dl[r] != 0.0f) {
                const int p0 = tv * a.rope.ppv;
                nv[u] = min(a.rope.ppv, a.rope.n_pairs - p0);
                const f32x4* tp = reinterpret_cast<const f32x4*>(
                    a.rope.cs + (int64_t)s_f[r] * a.rope.pairs_padded + p0);
                t01[u] = tp[0];
                t23[u] = tp[1];
                rot[u] = true;
              }
            }
            v[u] = __builtin_nontemporal_load(src + src_i);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (dst_i[u] >= 0) {
        u32x4 w = v[u];
        if (rot[u]) w = rotate_vec_tab(w, a.dtype, t01[u], t23[u], nv[u]);
        __builtin_nontemporal_store(w, out + dst_i[u]);
      }
    }
  }
  if (overflow && a.dev_error) *a.dev_error = DP_ECAPACITY;
}

template <int U, bool SPLIT>
__global__ __launch_bounds__(kBlock) void hs_reindex_kernel(HsArgs a) {
  __shared__ int heads[kMaxHeads];
  __shared__ int64_t head_off[kMaxHeads];
  __shared__ int32_t s_src[kRT];
  __shared__ int s_f[kRT];
  __shared__ float s_dl[kRT];
  HsTile tl;
  if (!hs_setup(a, 1, false, tl, heads, head_off, s_src, s_f, s_dl)) return;
  bool any = false;
  for (int r = 0; r < tl.rows; ++r) any = any || s_dl[r] != 0.0f;
  if (!any) return;
  u32x4* __restrict__ kbuf = reinterpret_cast<u32x4*>(a.k_out);
  const uint32_t total = (uint32_t)tl.nh * kRT * a.div_inner.d;
  for (uint32_t b0 = 0; b0 < total; b0 += kBlock * U) {
    u32x4 v[U];
    int64_t at[U];
    f32x4 t01[U], t23[U];
    int nv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t i = b0 + u * kBlock + threadIdx.x;
      at[u] = -1;
      if (i < total) {
        const uint32_t t = fdiv(i, a.div_inner);
        const int wq = a.rope.wv_begin + (int)(i - t * a.div_inner.d);   // vector in the segment
        const int r = (int)(t & (kRT - 1));
        const int k = (int)(t >> kLogRT);
        if (r < tl.rows && s_dl[r] != 0.0f) {
          const int64_t o = head_off[k] + tl.j0 + r;
          // interleaved: the row's lines holding the block; split: the row's
          // temporal block in the run's leading plane (the whole run must fit)
          if (head_off[k] >= 0 && (SPLIT ? head_off[k] + tl.n_run <= a.out_cap : o < a.out_cap)) {
            at[u] = SPLIT ? head_off[k] * a.vph + (tl.j0 + r) * a.tvc + wq : o * a.vph + wq;
            const int tv = wq - a.rope.tv_off;
            const bool in_block = tv >= 0 && tv < a.rope.tv_count;
            const int p0 = in_block ? tv * a.rope.ppv : 0;
            nv[u] = in_block ? min(a.rope.ppv, a.rope.n_pairs - p0) : 0;
            const f32x4* tp = reinterpret_cast<const f32x4*>(
                a.rope.cs + (int64_t)s_f[r] * a.rope.pairs_padded + p0);
            t01[u] = tp[0];
            t23[u] = tp[1];
            v[u] = __builtin_nontemporal_load(kbuf + at[u]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (at[u] >= 0)
        __builtin_nontemporal_store(rotate_vec_tab(v[u], a.dtype, t01[u], t23[u], nv[u]),
                                    kbuf + at[u]);
  }
}

void fill_caps(HsArgs& a, const int64_t* class_cap, int32_t n_classes) {
  a.n_classes = n_classes;
  for (int c = 0; c < DP_HS_MAX_CLASSES; ++c) a.class_cap[c] = c < n_classes ? class_cap[c] : 0;
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
  a.n_layers = kv.n_layers;
  a.n_kv = kv.v_src ? 2 : 1;
  a.dtype = kv.dtype;
  a.has_rope = rope != nullptr;
  if (rope) a.rope = *rope;
  a.vph = (uint32_t)(kv.head_dim * elem_size(kv.dtype) / 16);
  a.div_inner = make_fastdiv(a.vph);
  a.split = kv.key_layout == DP_KEY_SPLIT;
  a.split_src = kv.src_key_layout == DP_KEY_SPLIT;
  if (a.split || a.split_src) {
    const int esz = elem_size(kv.dtype);
    a.tvb = (uint32_t)(2 * kv.pair_begin * esz / 16);
    a.tvc = (uint32_t)(2 * kv.n_pairs * esz / 16);
    a.svc = a.vph - a.tvc;
  }
  fill_caps(a, class_cap, n_classes);
  const uint64_t gx = xcd_grid(hs_tiles(class_cap, n_classes) * (uint64_t)(kv.n_layers * a.n_kv));
  if (gx == 0) return DP_OK;
  // two vectors in flight per lane and pass: measured 2-4 % faster than four
  // on the HS workload, eight 21 % slower, one no better
  if (a.split && a.split_src)
    hipLaunchKernelGGL((hs_gather_kernel<2, true, true>), dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  else if (a.split)
    hipLaunchKernelGGL((hs_gather_kernel<2, true, false>), dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  else if (a.split_src)
    hipLaunchKernelGGL((hs_gather_kernel<2, false, true>), dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((hs_gather_kernel<2, false, false>), dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  return check_launch("hs_gather_kernel");
}

dp_status launch_hs_reindex(void* k, int64_t k_cap, int32_t L, int32_t H, int32_t head_dim,
                            int32_t dtype, const uint8_t* head_class, int32_t n_classes,
                            const int64_t* class_len, const int64_t* class_cap,
                            const int64_t* offsets, const int32_t* const* class_rf,
                            const RopeView& rope, hipStream_t s) {
  HsArgs a{};
  a.k_out = k;
  a.head_class = head_class;
  a.class_idx = nullptr;
  a.class_rf = class_rf;
  a.class_len = class_len;
  a.offsets = offsets;
  a.out_cap = k_cap;
  a.n_heads = H;
  a.n_layers = L;
  a.n_kv = 1;
  a.dtype = dtype;
  a.has_rope = 1;
  a.rope = rope;
  a.vph = (uint32_t)(head_dim * elem_size(dtype) / 16);
  a.div_inner = make_fastdiv((uint32_t)rope.wv_count);
  a.split = rope.split;
  a.tvb = (uint32_t)rope.tv_begin;
  a.tvc = (uint32_t)rope.tv_count;
  a.svc = a.vph - a.tvc;
  fill_caps(a, class_cap, n_classes);
  const uint64_t gx = hs_tiles(class_cap, n_classes) * (uint64_t)L;
  if (gx == 0) return DP_OK;
  // two vectors in flight per lane and pass, as for the gather (1.8 % faster than four)
  if (a.split)
    hipLaunchKernelGGL((hs_reindex_kernel<2, true>), dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL((hs_reindex_kernel<2, false>), dim3((uint32_t)gx), dim3(kBlock), 0, s, a);
  return check_launch("hs_reindex_kernel");
}

}  // namespace dp
