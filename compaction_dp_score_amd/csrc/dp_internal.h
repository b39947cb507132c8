// Internal host-side declarations of libdecoprune: error text, launch helpers
// and one launcher per source file.  Not part of the public ABI.
#pragma once

#include "dp_device.h"

namespace dp {

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
size_t score_index_ws_bytes(int64_t T);
dp_status launch_score_index(const float* x0, const float* xf, int32_t d, int64_t stride,
                             const dp_mask_policy& pol, float* ell, uint8_t* keep, int32_t* idx,
                             int64_t* n_kept, const int32_t* rf_src, int32_t* rf_dst, void* ws,
                             int32_t* dev_error, uint32_t spin_limit, hipStream_t s);
size_t compact_ws_bytes(int64_t T);
size_t compact_scratch_bytes();
dp_status compact_scratch(hipStream_t s, int32_t** out);
dp_status launch_compact(const uint8_t* keep, int64_t T, int32_t* idx, int64_t* n_kept,
                         const int32_t* rf_src, int32_t* rf_dst, int32_t* ws, hipStream_t s);
dp_status launch_rope_prepare(const dp_rope& r, void* ws, RopeView* view, int dtype,
                              int head_dim, int n_heads, hipStream_t s);
dp_status launch_gather(const dp_kv& kv, const int32_t* idx, const int64_t* n_kept,
                        const int32_t* row_frame, const RopeView* rope, hipStream_t s);
void rope_view(const dp_rope& r, const void* ws, RopeView* view, int dtype, int head_dim,
               int n_heads);
size_t rope_shift_ws_bytes(int32_t n_pairs);
dp_status launch_rope_shift(void* const* k, int32_t n_layers, int32_t n_heads, int32_t head_dim,
                            int32_t dtype, int64_t row_begin, int64_t rows_cap,
                            const int64_t* n_rows, const float* theta, int32_t pair_begin,
                            int32_t n_pairs, int32_t key_layout, float delta, void* ws,
                            hipStream_t s);
dp_status launch_reindex(void* const* k, int32_t n_layers, int32_t n_heads, int32_t head_dim,
                         int32_t dtype, int64_t row_begin, int64_t rows_cap,
                         const int64_t* n_rows, const int32_t* row_frame, const RopeView& rope,
                         hipStream_t s);
dp_status launch_append(const dp_kv_inplace& kv, int64_t slot_begin, int64_t slot_rows,
                        const int32_t* idx, const int64_t* n_kept, int64_t* tail,
                        int32_t* row_frame, const RopeView* rope, hipStream_t s);
dp_status launch_attention(const void* q, const void* k, const void* v, void* o, int64_t n_q,
                           int64_t kv_cap, const int64_t* n_kv, int32_t n_heads, float scale,
                           int32_t key_layout, int32_t pair_begin, int32_t n_pairs,
                           hipStream_t s);
dp_status launch_attention_lag(const void* q, const void* k, const void* v, void* o,
                               int64_t n_q, int64_t kv_cap, const int64_t* n_kv,
                               int64_t plain_begin, int64_t plain_end, const float* theta,
                               int32_t pair_begin, int32_t n_pairs, float lag, int32_t n_heads,
                               float scale, int32_t key_layout, hipStream_t s);
// Lagged ragged attention: the last plain_tail rows of each head's run (and
// the chunk block) plain, the rest against the query rotated by -lag.
struct HsLag {
  int64_t plain_tail;
  const float* theta;
  int32_t pair_begin;
  int32_t n_pairs;
  float lag;
};
dp_status launch_hs_attention(const void* q, const void* k_ragged, const void* v_ragged,
                              int64_t ragged_capacity, const int64_t* head_offsets,
                              const void* k_chunk, const void* v_chunk, int64_t n_chunk, void* o,
                              int64_t n_q, int32_t n_heads, float scale, int32_t key_layout,
                              int32_t pair_begin, int32_t n_pairs, hipStream_t s,
                              const HsLag* lag = nullptr);
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
