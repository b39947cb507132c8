// C ABI of libdecoprune: argument checks on the host, then stream-ordered
// launches.  See include/decoprune.h for the contract of every entry point.
#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "dp_internal.h"

namespace dp {

size_t rope_ws_bytes(int32_t n_frames, int32_t n_pairs);
uint64_t hs_tiles(const int64_t* class_cap, int32_t n_classes);
int hs_max_heads();

namespace {
thread_local char g_err[512] = "";
constexpr int64_t kMaxRows = (int64_t)1 << 31;      // int32 row indices
constexpr int64_t kMaxVec = (int64_t)1 << 31;       // 16-byte vectors per launch slab
constexpr uint32_t kScoreIndexSpinLimit = 1u << 20;   // polls before DP_ESTALL
constexpr int32_t kMaxAttnHeads = 65536;           // 64 key rows of a tile addressed in 32 bits
}  // namespace

dp_status fail(dp_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

dp_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DP_EHIP, "%s: %s", what, hipGetErrorString(e));
  return DP_OK;
}

namespace {

void ok() { g_err[0] = '\0'; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

dp_status check_shape(int32_t n_layers, int32_t n_heads, int32_t head_dim, int32_t dtype,
                      const char* who) {
  if (n_layers < 1 || n_heads < 1 || head_dim < 2 || (head_dim & 1))
    return fail(DP_EINVAL, "%s: need n_layers >= 1, n_heads >= 1, even head_dim >= 2", who);
  if (dtype != DP_F32 && dtype != DP_BF16) return fail(DP_EINVAL, "%s: unknown dtype %d", who, dtype);
  if (((int64_t)head_dim * elem_size(dtype)) % 16 != 0)
    return fail(DP_EALIGN, "%s: head_dim * element size must be a multiple of 16 bytes", who);
  return DP_OK;
}

// Layout of the keys: DP_KEY_INTERLEAVED (the pairs are not read) or
// DP_KEY_SPLIT with a temporal block of whole 16-byte vectors.
dp_status check_key_layout(int32_t key_layout, int32_t pair_begin, int32_t n_pairs,
                           int32_t head_dim, int32_t dtype, const char* who) {
  if (key_layout == DP_KEY_INTERLEAVED) return DP_OK;
  if (key_layout != DP_KEY_SPLIT) return fail(DP_EINVAL, "%s: unknown key_layout %d", who, key_layout);
  if (n_pairs < 1 || pair_begin < 0 || 2 * ((int64_t)pair_begin + n_pairs) > head_dim)
    return fail(DP_ERANGE, "%s: split keys need temporal pairs [%d, %d + %d) within head_dim/2",
                who, pair_begin, pair_begin, n_pairs);
  if ((2 * (int64_t)pair_begin * elem_size(dtype)) % 16 != 0 ||
      (2 * (int64_t)n_pairs * elem_size(dtype)) % 16 != 0)
    return fail(DP_EALIGN, "%s: split keys need the temporal block to start and end on 16-byte "
                           "boundaries", who);
  return DP_OK;
}

dp_status check_rope(const dp_rope* r, int32_t head_dim, int32_t dtype, const void* ws,
                     size_t ws_bytes, const char* who) {
  if (r->n_pairs < 1 || r->pair_begin < 0 || r->n_frames < 1 ||
      (r->axis != DP_AXIS_PAGE && r->axis != DP_AXIS_COMPRESSED))
    return fail(DP_EINVAL, "%s: rope needs n_pairs >= 1, pair_begin >= 0, n_frames >= 1 and a "
                           "known axis", who);
  if (2 * ((int64_t)r->pair_begin + r->n_pairs) > head_dim)
    return fail(DP_ERANGE, "%s: temporal pairs [%d, %d) exceed head_dim/2 = %d", who,
                r->pair_begin, r->pair_begin + r->n_pairs, head_dim / 2);
  if ((2 * (int64_t)r->pair_begin * elem_size(dtype)) % 16 != 0)
    return fail(DP_EALIGN, "%s: the temporal block must start on a 16-byte boundary", who);
  if (!r->theta || !r->frame_t || !r->frame_phase)
    return fail(DP_EINVAL, "%s: rope theta, frame_t and frame_phase are required", who);
  if (!ws || !aligned(ws, 16))
    return fail(ws ? DP_EALIGN : DP_EINVAL, "%s: rope workspace must be a 16-byte aligned pointer", who);
  if (ws_bytes < rope_ws_bytes(r->n_frames, r->n_pairs))
    return fail(DP_EINVAL, "%s: workspace of %zu bytes < %zu needed", who, ws_bytes,
                rope_ws_bytes(r->n_frames, r->n_pairs));
  return check_key_layout(r->key_layout, r->pair_begin, r->n_pairs, head_dim, dtype, who);
}


}  // namespace
}  // namespace dp

using namespace dp;

extern "C" {

int dp_abi_version(void) { return DP_ABI_VERSION; }

const char* dp_status_str(int s) {
  switch (s) {
    case DP_OK: return "DP_OK";
    case DP_EINVAL: return "DP_EINVAL";
    case DP_EALIGN: return "DP_EALIGN";
    case DP_ERANGE: return "DP_ERANGE";
    case DP_ECAPACITY: return "DP_ECAPACITY";
    case DP_EHIP: return "DP_EHIP";
    case DP_EUNSUPPORTED: return "DP_EUNSUPPORTED";
    case DP_ESTALL: return "DP_ESTALL";
    default: return "DP_UNKNOWN";
  }
}

const char* dp_last_error(void) { return g_err; }

// Checks shared by dp_score_mask and dp_score_index; *scoring tells whether
// rows are scored (score mode with n_scored > 0).
static dp_status check_score(const float* x0_hat, const float* x_final, int32_t d,
                             int64_t row_stride, const dp_mask_policy* p, const float* ell_out,
                             const char* fn, bool* scoring) {
  if (p->seq_len < 1 || p->seq_len >= kMaxRows)
    return fail(DP_ERANGE, "%s: seq_len %lld outside [1, 2^31)", fn, (long long)p->seq_len);
  if (p->sink_len < 0 || p->window_len < 0 || p->n_scored < 0 || p->scored_begin < p->sink_len ||
      p->scored_begin + p->n_scored > p->seq_len - p->window_len)
    return fail(DP_EINVAL,
                "%s: need 0 <= sink_len <= scored_begin and scored_begin + n_scored <= "
                "seq_len - window_len", fn);
  if ((p->mode != DP_MODE_SCORE && p->mode != DP_MODE_STREAMING) ||
      (p->reversed != 0 && p->reversed != 1) || p->reserved != 0)
    return fail(DP_EINVAL, "%s: mode, reversed or reserved out of range", fn);
  *scoring = p->mode == DP_MODE_SCORE && p->n_scored > 0;
  if (*scoring) {
    if (!x0_hat || !x_final) return fail(DP_EINVAL, "%s: x0_hat and x_final are required", fn);
    if (d < 1 || d > 256) return fail(DP_ERANGE, "%s: d = %d outside [1, 256]", fn, d);
    if (row_stride < d) return fail(DP_EINVAL, "%s: row_stride < d", fn);
    if (!aligned(x0_hat, 4) || !aligned(x_final, 4) || (ell_out && !aligned(ell_out, 4)))
      return fail(DP_EALIGN, "%s: float arrays must be 4-byte aligned", fn);
    if (row_stride > ((int64_t)1 << 40) / p->n_scored)
      return fail(DP_ERANGE, "%s: input too large", fn);
  }
  return DP_OK;
}

dp_status dp_score_mask(const float* x0_hat, const float* x_final, int32_t d,
                        int64_t row_stride, const dp_mask_policy* p, float* ell_out,
                        uint8_t* keep_out, void* stream) {
  if (!p || !keep_out) return fail(DP_EINVAL, "dp_score_mask: policy and keep_out are required");
  bool scoring = false;
  dp_status st = check_score(x0_hat, x_final, d, row_stride, p, ell_out, "dp_score_mask", &scoring);
  if (st != DP_OK) return st;
  (void)hipGetLastError();
  st = launch_score_mask(x0_hat, x_final, d, row_stride, *p, scoring ? ell_out : nullptr,
                         keep_out, (hipStream_t)stream);
  if (st == DP_OK) ok();
  return st;
}

size_t dp_score_index_workspace_bytes(int64_t seq_len) {
  return score_index_ws_bytes(seq_len < 0 ? 0 : seq_len);
}

dp_status dp_score_index(const float* x0_hat, const float* x_final, int32_t d,
                         int64_t row_stride, const dp_mask_policy* p, float* ell_out,
                         uint8_t* keep_out, int32_t* idx_out, int64_t* n_kept,
                         const int32_t* row_frame_src, int32_t* row_frame_dst, void* ws,
                         size_t ws_bytes, int32_t* dev_error, void* stream) {
  if (!p || !idx_out || !n_kept || !ws)
    return fail(DP_EINVAL, "dp_score_index: policy, idx_out, n_kept and workspace are required");
  if ((row_frame_src == nullptr) != (row_frame_dst == nullptr))
    return fail(DP_EINVAL, "dp_score_index: row_frame_src and row_frame_dst go together");
  bool scoring = false;
  dp_status st = check_score(x0_hat, x_final, d, row_stride, p, ell_out, "dp_score_index", &scoring);
  if (st != DP_OK) return st;
  if (!aligned(n_kept, 8) || !aligned(ws, 8) || !aligned(idx_out, 4) ||
      (row_frame_src && (!aligned(row_frame_src, 4) || !aligned(row_frame_dst, 4))) ||
      (dev_error && !aligned(dev_error, 4)))
    return fail(DP_EALIGN, "dp_score_index: n_kept and workspace must be 8-byte, index arrays "
                           "4-byte aligned");
  if (ws_bytes < score_index_ws_bytes(p->seq_len))
    return fail(DP_EINVAL, "dp_score_index: workspace of %zu bytes < %zu needed", ws_bytes,
                score_index_ws_bytes(p->seq_len));
  (void)hipGetLastError();
  st = launch_score_index(x0_hat, x_final, d, row_stride, *p, scoring ? ell_out : nullptr,
                          keep_out, idx_out, n_kept, row_frame_src, row_frame_dst, ws, dev_error,
                          kScoreIndexSpinLimit, (hipStream_t)stream);
  if (st == DP_OK) ok();
  return st;
}

size_t dp_compact_workspace_bytes(int64_t seq_len) {
  return compact_ws_bytes(seq_len < 0 ? 0 : seq_len);
}

dp_status dp_compact_index(const uint8_t* keep, int64_t seq_len, int32_t* idx_out,
                           int64_t* n_kept, const int32_t* row_frame_src,
                           int32_t* row_frame_dst, void* ws, size_t ws_bytes, void* stream) {
  if (seq_len < 0 || seq_len >= kMaxRows)
    return fail(DP_ERANGE, "dp_compact_index: seq_len %lld outside [0, 2^31)", (long long)seq_len);
  if ((seq_len > 0 && (!keep || !idx_out)) || !n_kept || !ws)
    return fail(DP_EINVAL, "dp_compact_index: keep, idx_out, n_kept and workspace are required");
  if ((row_frame_src == nullptr) != (row_frame_dst == nullptr))
    return fail(DP_EINVAL, "dp_compact_index: row_frame_src and row_frame_dst go together");
  if (!aligned(n_kept, 8) || !aligned(ws, 4) || (idx_out && !aligned(idx_out, 4)))
    return fail(DP_EALIGN, "dp_compact_index: n_kept must be 8-byte, idx and workspace 4-byte aligned");
  if (ws_bytes < compact_ws_bytes(seq_len))
    return fail(DP_EINVAL, "dp_compact_index: workspace of %zu bytes < %zu needed", ws_bytes,
                compact_ws_bytes(seq_len));
  (void)hipGetLastError();
  dp_status st = launch_compact(keep, seq_len, idx_out, n_kept, row_frame_src, row_frame_dst,
                                (int32_t*)ws, (hipStream_t)stream);
  if (st == DP_OK) ok();
  return st;
}

dp_status dp_compact_index_noalloc(const uint8_t* keep, int64_t seq_len, int32_t* idx_out,
                                   int64_t* n_kept, const int32_t* row_frame_src,
                                   int32_t* row_frame_dst, void* stream) {
  const char* who = "dp_compact_index_noalloc";
  if (seq_len < 0 || seq_len >= kMaxRows)
    return fail(DP_ERANGE, "%s: seq_len %lld outside [0, 2^31)", who, (long long)seq_len);
  if ((seq_len > 0 && (!keep || !idx_out)) || !n_kept)
    return fail(DP_EINVAL, "%s: keep, idx_out and n_kept are required", who);
  if ((row_frame_src == nullptr) != (row_frame_dst == nullptr))
    return fail(DP_EINVAL, "%s: row_frame_src and row_frame_dst go together", who);
  if (!aligned(n_kept, 8) || (idx_out && !aligned(idx_out, 4)))
    return fail(DP_EALIGN, "%s: n_kept must be 8-byte, idx 4-byte aligned", who);
  if (compact_ws_bytes(seq_len) > compact_scratch_bytes())
    return fail(DP_ERANGE, "%s: %lld rows need %zu bytes of scratch, more than the %zu held",
                who, (long long)seq_len, compact_ws_bytes(seq_len), compact_scratch_bytes());
  (void)hipGetLastError();
  int32_t* scratch_ptr = nullptr;
  dp_status st = compact_scratch((hipStream_t)stream, &scratch_ptr);
  if (st != DP_OK) return st;
  st = launch_compact(keep, seq_len, idx_out, n_kept, row_frame_src, row_frame_dst, scratch_ptr,
                      (hipStream_t)stream);
  if (st == DP_OK) ok();
  return st;
}

size_t dp_rope_workspace_bytes(int32_t n_frames, int32_t n_pairs) {
  if (n_frames < 0 || n_pairs < 0) return 0;
  return rope_ws_bytes(n_frames, n_pairs);
}

dp_status dp_gather_kv(const dp_kv* kv, const int32_t* idx, const int64_t* n_kept,
                       const int32_t* row_frame, const dp_rope* rope, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!kv || !idx || !n_kept) return fail(DP_EINVAL, "dp_gather_kv: kv, idx and n_kept are required");
  dp_status st = check_shape(kv->n_layers, kv->n_heads, kv->head_dim, kv->dtype, "dp_gather_kv");
  if (st != DP_OK) return st;
  if (!kv->k_src || !kv->k_dst || ((kv->v_src == nullptr) != (kv->v_dst == nullptr)))
    return fail(DP_EINVAL, "dp_gather_kv: k_src/k_dst required, v_src/v_dst go together");
  if (kv->src_rows < 0 || kv->src_rows >= kMaxRows || kv->dst_capacity < 0)
    return fail(DP_ERANGE, "dp_gather_kv: src_rows outside [0, 2^31) or negative capacity");
  const int64_t rv = (int64_t)kv->n_heads * kv->head_dim * elem_size(kv->dtype) / 16;
  if (kv->dst_capacity > kMaxVec / rv)
    return fail(DP_ERANGE, "dp_gather_kv: a destination layer over 32 GiB is not supported");
  const int n_kv = kv->v_src ? 2 : 1;
  if ((int64_t)kv->n_layers * n_kv * ((kv->dst_capacity * rv + 255) / 256) >= kMaxVec)
    return fail(DP_ERANGE, "dp_gather_kv: layers x capacity too large for one launch");
  if (!aligned(n_kept, 8) || (kv->dev_error && !aligned(kv->dev_error, 4)))
    return fail(DP_EALIGN, "dp_gather_kv: n_kept must be 8-byte aligned");
  if (rope) {
    st = check_rope(rope, kv->head_dim, kv->dtype, ws, ws_bytes, "dp_gather_kv");
    if (st != DP_OK) return st;
    if (!row_frame) return fail(DP_EINVAL, "dp_gather_kv: fused re-index needs row_frame");
  }
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  RopeView view{};
  if (rope) {
    st = launch_rope_prepare(*rope, ws, &view, kv->dtype, kv->head_dim, kv->n_heads, s);
    if (st != DP_OK) return st;
  }
  st = launch_gather(*kv, idx, n_kept, row_frame, rope ? &view : nullptr, s);
  if (st == DP_OK) ok();
  return st;
}

static dp_status check_reindex(void* const* k_layers, int32_t n_layers, int32_t n_heads,
                               int32_t head_dim, int32_t dtype, int64_t row_begin,
                               int64_t rows_capacity, const int64_t* n_rows,
                               const int32_t* row_frame, const dp_rope* rope, const void* ws,
                               size_t ws_bytes, const char* who) {
  if (!k_layers || !row_frame || !rope)
    return fail(DP_EINVAL, "%s: k_layers, row_frame and rope are required", who);
  dp_status st = check_shape(n_layers, n_heads, head_dim, dtype, who);
  if (st != DP_OK) return st;
  st = check_rope(rope, head_dim, dtype, ws, ws_bytes, who);
  if (st != DP_OK) return st;
  const int64_t per_row = (int64_t)n_heads * (head_dim * elem_size(dtype) / 16);
  const int64_t span = rows_capacity - row_begin;
  if (row_begin < 0 || rows_capacity < 0 || rows_capacity >= kMaxRows || span * per_row >= kMaxVec ||
      (span > 0 && (span * per_row + 255) / 256 * n_layers >= kMaxVec))
    return fail(DP_ERANGE, "%s: rows x layers out of range", who);
  if (n_rows && !aligned(n_rows, 8)) return fail(DP_EALIGN, "%s: n_rows alignment", who);
  return DP_OK;
}

dp_status dp_rope_reindex(void* const* k_layers, int32_t n_layers, int32_t n_heads,
                          int32_t head_dim, int32_t dtype, int64_t rows_capacity,
                          const int64_t* n_rows, const int32_t* row_frame, const dp_rope* rope,
                          void* ws, size_t ws_bytes, void* stream) {
  dp_status st = check_reindex(k_layers, n_layers, n_heads, head_dim, dtype, 0, rows_capacity,
                               n_rows, row_frame, rope, ws, ws_bytes, "dp_rope_reindex");
  if (st != DP_OK) return st;
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  RopeView view{};
  st = launch_rope_prepare(*rope, ws, &view, dtype, head_dim, n_heads, s);
  if (st != DP_OK) return st;
  st = launch_reindex(k_layers, n_layers, n_heads, head_dim, dtype, 0, rows_capacity, n_rows,
                      row_frame, view, s);
  if (st == DP_OK) ok();
  return st;
}

dp_status dp_rope_prepare(const dp_rope* rope, int32_t head_dim, int32_t dtype, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!rope) return fail(DP_EINVAL, "dp_rope_prepare: rope is required");
  dp_status st = check_shape(1, 1, head_dim, dtype, "dp_rope_prepare");
  if (st != DP_OK) return st;
  st = check_rope(rope, head_dim, dtype, ws, ws_bytes, "dp_rope_prepare");
  if (st != DP_OK) return st;
  (void)hipGetLastError();
  RopeView view{};
  st = launch_rope_prepare(*rope, ws, &view, dtype, head_dim, 1, (hipStream_t)stream);
  if (st == DP_OK) ok();
  return st;
}

dp_status dp_rope_apply(void* const* k_layers, int32_t n_layers, int32_t n_heads, int32_t head_dim,
                        int32_t dtype, int64_t row_begin, int64_t rows_capacity,
                        const int64_t* n_rows, const int32_t* row_frame, const dp_rope* rope,
                        const void* ws, size_t ws_bytes, void* stream) {
  dp_status st = check_reindex(k_layers, n_layers, n_heads, head_dim, dtype, row_begin,
                               rows_capacity, n_rows, row_frame, rope, ws, ws_bytes,
                               "dp_rope_apply");
  if (st != DP_OK) return st;
  if (rows_capacity <= row_begin) {
    ok();
    return DP_OK;
  }
  (void)hipGetLastError();
  RopeView view{};
  rope_view(*rope, ws, &view, dtype, head_dim, n_heads);
  st = launch_reindex(k_layers, n_layers, n_heads, head_dim, dtype, row_begin, rows_capacity,
                      n_rows, row_frame, view, (hipStream_t)stream);
  if (st == DP_OK) ok();
  return st;
}

size_t dp_rope_shift_workspace_bytes(int32_t n_pairs) {
  return rope_shift_ws_bytes(n_pairs < 1 ? 1 : n_pairs);
}

dp_status dp_rope_shift(void* const* k_layers, int32_t n_layers, int32_t n_heads,
                        int32_t head_dim, int32_t dtype, int64_t row_begin,
                        int64_t rows_capacity, const int64_t* n_rows, const float* theta,
                        int32_t pair_begin, int32_t n_pairs, int32_t key_layout, float delta,
                        void* ws, size_t ws_bytes, void* stream) {
  const char* who = "dp_rope_shift";
  if (!k_layers || !theta || !ws)
    return fail(DP_EINVAL, "%s: k_layers, theta and workspace are required", who);
  dp_status st = check_shape(n_layers, n_heads, head_dim, dtype, who);
  if (st != DP_OK) return st;
  if (n_pairs < 1 || pair_begin < 0 || n_pairs > 4096)
    return fail(DP_EINVAL, "%s: need 1 <= n_pairs <= 4096 and pair_begin >= 0", who);
  if (2 * ((int64_t)pair_begin + n_pairs) > head_dim)
    return fail(DP_ERANGE, "%s: temporal pairs [%d, %d) exceed head_dim/2 = %d", who, pair_begin,
                pair_begin + n_pairs, head_dim / 2);
  if ((2 * (int64_t)pair_begin * elem_size(dtype)) % 16 != 0)
    return fail(DP_EALIGN, "%s: the temporal block must start on a 16-byte boundary", who);
  st = check_key_layout(key_layout, pair_begin, n_pairs, head_dim, dtype, who);
  if (st != DP_OK) return st;
  if (!(delta - delta == 0.0f)) return fail(DP_EINVAL, "%s: delta must be finite", who);
  const int64_t per_row = (int64_t)n_heads * (head_dim * elem_size(dtype) / 16);
  const int64_t span = rows_capacity - row_begin;
  if (row_begin < 0 || rows_capacity < 0 || rows_capacity >= kMaxRows || span * per_row >= kMaxVec)
    return fail(DP_ERANGE, "%s: rows x layers out of range", who);
  if (n_rows && !aligned(n_rows, 8)) return fail(DP_EALIGN, "%s: n_rows alignment", who);
  if (!aligned(theta, 4) || !aligned(ws, 16)) return fail(DP_EALIGN, "%s: theta or workspace alignment", who);
  if (ws_bytes < rope_shift_ws_bytes(n_pairs))
    return fail(DP_EINVAL, "%s: workspace of %zu bytes < %zu needed", who, ws_bytes,
                rope_shift_ws_bytes(n_pairs));
  if (span > 0 && (span * per_row + 255) / 256 * n_layers >= kMaxVec)
    return fail(DP_ERANGE, "%s: rows x layers out of range", who);
  (void)hipGetLastError();
  st = launch_rope_shift(k_layers, n_layers, n_heads, head_dim, dtype, row_begin, rows_capacity,
                         n_rows, theta, pair_begin, n_pairs, key_layout, delta, ws,
                         (hipStream_t)stream);
  if (st == DP_OK) ok();
  return st;
}

dp_status dp_append_kept(const dp_kv_inplace* kv, int64_t slot_begin, int64_t slot_rows,
                         const int32_t* idx, const int64_t* n_kept, int64_t* tail,
                         int32_t* row_frame, const dp_rope* fused_rope, const void* ws,
                         size_t ws_bytes, void* stream) {
  if (!kv || !n_kept || !tail || (slot_rows > 0 && !idx))
    return fail(DP_EINVAL, "dp_append_kept: kv, idx, n_kept and tail are required");
  dp_status st = check_shape(kv->n_layers, kv->n_heads, kv->head_dim, kv->dtype, "dp_append_kept");
  if (st != DP_OK) return st;
  if (!kv->k_layers) return fail(DP_EINVAL, "dp_append_kept: k_layers is required");
  if (kv->capacity < 0 || kv->capacity >= kMaxRows || slot_begin < 0 || slot_rows < 0 ||
      slot_begin + slot_rows > kv->capacity)
    return fail(DP_ERANGE, "dp_append_kept: need 0 <= slot_begin, slot_begin + slot_rows <= "
                "capacity < 2^31");
  const int64_t rv = (int64_t)kv->n_heads * kv->head_dim * elem_size(kv->dtype) / 16;
  const int n_kv = kv->v_layers ? 2 : 1;
  if (slot_rows * rv >= kMaxVec || (int64_t)kv->n_layers * n_kv > 65535)
    return fail(DP_ERANGE, "dp_append_kept: slot or layer count too large for one launch");
  if (!aligned(n_kept, 8) || !aligned(tail, 8) || (idx && !aligned(idx, 4)) ||
      (row_frame && !aligned(row_frame, 4)) || (kv->dev_error && !aligned(kv->dev_error, 4)))
    return fail(DP_EALIGN, "dp_append_kept: misaligned count, tail, index or frame array");
  RopeView view{};
  if (fused_rope) {
    if (!row_frame) return fail(DP_EINVAL, "dp_append_kept: a fused re-index needs row_frame");
    st = check_rope(fused_rope, kv->head_dim, kv->dtype, ws, ws_bytes, "dp_append_kept");
    if (st != DP_OK) return st;
    rope_view(*fused_rope, ws, &view, kv->dtype, kv->head_dim, kv->n_heads);
  }
  (void)hipGetLastError();
  st = launch_append(*kv, slot_begin, slot_rows, idx, n_kept, tail, row_frame,
                     fused_rope ? &view : nullptr, (hipStream_t)stream);
  if (st == DP_OK) ok();
  return st;
}

dp_status dp_hs_offsets(const uint8_t* head_class, int32_t n_layers, int32_t n_heads,
                        const int64_t* class_len, int32_t n_classes, int64_t* offsets,
                        void* stream) {
  if (!head_class || !class_len || !offsets)
    return fail(DP_EINVAL, "dp_hs_offsets: head_class, class_len and offsets are required");
  if (n_layers < 1 || n_heads < 1 || n_classes < 1 || n_classes > DP_HS_MAX_CLASSES)
    return fail(DP_EINVAL, "dp_hs_offsets: need n_layers, n_heads >= 1 and 1 <= n_classes <= %d",
                DP_HS_MAX_CLASSES);
  if ((int64_t)n_layers * n_heads >= kMaxRows) return fail(DP_ERANGE, "dp_hs_offsets: too many heads");
  if (!aligned(class_len, 8) || !aligned(offsets, 8))
    return fail(DP_EALIGN, "dp_hs_offsets: int64 arrays must be 8-byte aligned");
  (void)hipGetLastError();
  dp_status st = launch_hs_offsets(head_class, n_layers, n_heads, class_len, n_classes, offsets,
                                   (hipStream_t)stream);
  if (st == DP_OK) ok();
  return st;
}

static dp_status check_hs_common(int32_t n_layers, int32_t n_heads, int32_t head_dim,
                                 int32_t dtype, const uint8_t* head_class, int32_t n_classes,
                                 const int64_t* class_len, const int64_t* class_cap,
                                 const int64_t* offsets, const char* who) {
  dp_status st = check_shape(n_layers, n_heads, head_dim, dtype, who);
  if (st != DP_OK) return st;
  if (n_heads > hs_max_heads()) return fail(DP_ERANGE, "%s: n_heads > %d", who, hs_max_heads());
  if (!head_class || !class_len || !class_cap || !offsets)
    return fail(DP_EINVAL, "%s: head_class, class_len, class_capacity and offsets are required", who);
  if (n_classes < 1 || n_classes > DP_HS_MAX_CLASSES)
    return fail(DP_EINVAL, "%s: n_classes outside [1, %d]", who, DP_HS_MAX_CLASSES);
  for (int c = 0; c < n_classes; ++c)
    if (class_cap[c] < 0 || class_cap[c] >= kMaxRows)
      return fail(DP_ERANGE, "%s: class_capacity[%d] outside [0, 2^31)", who, c);
  if (hs_tiles(class_cap, n_classes) * (uint64_t)n_layers * 2 >= ((uint64_t)1 << 31))
    return fail(DP_ERANGE, "%s: class capacities x layers too large for one launch", who);
  return DP_OK;
}

dp_status dp_hs_gather_kv(const dp_kv_hs* kv, const uint8_t* head_class, int32_t n_classes,
                          const int32_t* const* class_idx, const int64_t* class_len,
                          const int64_t* class_cap, const int64_t* offsets,
                          const int32_t* const* class_rf, const dp_rope* rope, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!kv || !class_idx) return fail(DP_EINVAL, "dp_hs_gather_kv: kv and class_idx are required");
  dp_status st = check_hs_common(kv->n_layers, kv->n_heads, kv->head_dim, kv->dtype, head_class,
                                 n_classes, class_len, class_cap, offsets, "dp_hs_gather_kv");
  if (st != DP_OK) return st;
  if (!kv->k_src || !kv->k_out || ((kv->v_src == nullptr) != (kv->v_out == nullptr)))
    return fail(DP_EINVAL, "dp_hs_gather_kv: k_src/k_out required, v_src/v_out go together");
  if (!aligned(kv->k_out, 16) || (kv->v_out && !aligned(kv->v_out, 16)))
    return fail(DP_EALIGN, "dp_hs_gather_kv: outputs must be 16-byte aligned");
  if (kv->src_rows < 0 || kv->src_rows >= kMaxRows || kv->out_capacity < 0)
    return fail(DP_ERANGE, "dp_hs_gather_kv: src_rows or out_capacity out of range");
  st = check_key_layout(kv->key_layout, kv->pair_begin, kv->n_pairs, kv->head_dim, kv->dtype,
                        "dp_hs_gather_kv");
  if (st != DP_OK) return st;
  st = check_key_layout(kv->src_key_layout, kv->pair_begin, kv->n_pairs, kv->head_dim, kv->dtype,
                        "dp_hs_gather_kv (source rows)");
  if (st != DP_OK) return st;
  if (rope) {
    st = check_rope(rope, kv->head_dim, kv->dtype, ws, ws_bytes, "dp_hs_gather_kv");
    if (st != DP_OK) return st;
    if (!class_rf) return fail(DP_EINVAL, "dp_hs_gather_kv: fused re-index needs class_row_frame");
    if (rope->key_layout != kv->key_layout ||
        (kv->key_layout == DP_KEY_SPLIT &&
         (rope->pair_begin != kv->pair_begin || rope->n_pairs != kv->n_pairs)))
      return fail(DP_EINVAL, "dp_hs_gather_kv: the rope and the cache name different key layouts");
  }
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  RopeView view{};
  if (rope) {
    st = launch_rope_prepare(*rope, ws, &view, kv->dtype, kv->head_dim, kv->n_heads, s);
    if (st != DP_OK) return st;
  }
  st = launch_hs_gather(*kv, head_class, n_classes, class_idx, class_len, class_cap, offsets,
                        class_rf, rope ? &view : nullptr, s);
  if (st == DP_OK) ok();
  return st;
}

dp_status dp_hs_rope_reindex(void* k_ragged, int64_t k_capacity, int32_t n_layers,
                             int32_t n_heads, int32_t head_dim, int32_t dtype, const uint8_t* head_class, int32_t n_classes,
                             const int64_t* class_len, const int64_t* class_cap,
                             const int64_t* offsets, const int32_t* const* class_rf,
                             const dp_rope* rope, void* ws, size_t ws_bytes, void* stream) {
  if (!k_ragged || !class_rf || !rope)
    return fail(DP_EINVAL, "dp_hs_rope_reindex: k_ragged, class_row_frame and rope are required");
  dp_status st = check_hs_common(n_layers, n_heads, head_dim, dtype, head_class, n_classes,
                                 class_len, class_cap, offsets, "dp_hs_rope_reindex");
  if (st != DP_OK) return st;
  if (!aligned(k_ragged, 16)) return fail(DP_EALIGN, "dp_hs_rope_reindex: k_ragged alignment");
  if (k_capacity < 0) return fail(DP_ERANGE, "dp_hs_rope_reindex: negative k_capacity");
  st = check_rope(rope, head_dim, dtype, ws, ws_bytes, "dp_hs_rope_reindex");
  if (st != DP_OK) return st;
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  RopeView view{};
  st = launch_rope_prepare(*rope, ws, &view, dtype, head_dim, n_heads, s);
  if (st != DP_OK) return st;
  st = launch_hs_reindex(k_ragged, k_capacity, n_layers, n_heads, head_dim, dtype, head_class, n_classes,
                         class_len, class_cap, offsets, class_rf, view, s);
  if (st == DP_OK) ok();
  return st;
}

dp_status dp_attention(const void* q, const void* k, const void* v, void* o, int64_t n_q,
                       int64_t kv_capacity, const int64_t* n_kv, int32_t n_heads,
                       int32_t head_dim, int32_t dtype, float scale, int32_t key_layout,
                       int32_t pair_begin, int32_t n_pairs, void* stream) {
  if (!q || !k || !v || !o) return fail(DP_EINVAL, "dp_attention: q, k, v and o are required");
  if (dtype != DP_BF16 || head_dim != 128)
    return fail(DP_EUNSUPPORTED, "dp_attention: only bf16 with head_dim 128 is implemented");
  if (n_heads < 1 || n_heads > kMaxAttnHeads || n_q < 0 || kv_capacity < 0 || n_q >= kMaxRows ||
      kv_capacity >= kMaxRows)
    return fail(DP_ERANGE, "dp_attention: need 1 <= n_heads <= 65536 and 0 <= n_q, kv_capacity < 2^31");
  if ((n_q + 127) / 128 * (int64_t)n_heads >= kMaxVec)
    return fail(DP_ERANGE, "dp_attention: too many query tiles for one launch");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (n_kv && !aligned(n_kv, 8)))
    return fail(DP_EALIGN, "dp_attention: tensors must be 16-byte aligned");
  if (!(scale > 0.0f && scale <= 3.0e38f))
    return fail(DP_EINVAL, "dp_attention: scale must be positive and finite");
  dp_status st = check_key_layout(key_layout, pair_begin, n_pairs, head_dim, dtype, "dp_attention");
  if (st != DP_OK) return st;
  (void)hipGetLastError();
  st = launch_attention(q, k, v, o, n_q, kv_capacity, n_kv, n_heads, scale, key_layout,
                        pair_begin, n_pairs, (hipStream_t)stream);
  if (st == DP_OK) ok();
  return st;
}

dp_status dp_attention_lag(const void* q, const void* k, const void* v, void* o, int64_t n_q,
                           int64_t kv_capacity, const int64_t* n_kv, int64_t plain_begin,
                           int64_t plain_end, const float* theta, int32_t pair_begin,
                           int32_t n_pairs, float lag, int32_t n_heads, int32_t head_dim,
                           int32_t dtype, float scale, int32_t key_layout, void* stream) {
  if (!q || !k || !v || !o || !theta)
    return fail(DP_EINVAL, "dp_attention_lag: q, k, v, o and theta are required");
  if (dtype != DP_BF16 || head_dim != 128)
    return fail(DP_EUNSUPPORTED, "dp_attention_lag: only bf16 with head_dim 128 is implemented");
  if (n_heads < 1 || n_heads > kMaxAttnHeads || n_q < 0 || kv_capacity < 0 || n_q >= kMaxRows ||
      kv_capacity >= kMaxRows)
    return fail(DP_ERANGE, "dp_attention_lag: need 1 <= n_heads <= 65536 and 0 <= n_q, "
                           "kv_capacity < 2^31");
  if ((n_q + 127) / 128 * (int64_t)n_heads >= kMaxVec)
    return fail(DP_ERANGE, "dp_attention_lag: too many query tiles for one launch");
  if (plain_begin < 0 || plain_end < plain_begin)
    return fail(DP_ERANGE, "dp_attention_lag: need 0 <= plain_begin <= plain_end");
  if (n_pairs < 1 || pair_begin < 0 || 2 * ((int64_t)pair_begin + n_pairs) > head_dim)
    return fail(DP_ERANGE, "dp_attention_lag: temporal pairs [%d, %d + %d) outside head_dim/2",
                pair_begin, pair_begin, n_pairs);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (n_kv && !aligned(n_kv, 8)) || !aligned(theta, 4))
    return fail(DP_EALIGN, "dp_attention_lag: tensors must be 16-byte aligned");
  if (!(scale > 0.0f && scale <= 3.0e38f))
    return fail(DP_EINVAL, "dp_attention_lag: scale must be positive and finite");
  if (!(lag >= -3.0e38f && lag <= 3.0e38f))
    return fail(DP_EINVAL, "dp_attention_lag: lag must be finite");
  dp_status st = check_key_layout(key_layout, pair_begin, n_pairs, head_dim, dtype,
                                  "dp_attention_lag");
  if (st != DP_OK) return st;
  (void)hipGetLastError();
  st = launch_attention_lag(q, k, v, o, n_q, kv_capacity, n_kv, plain_begin, plain_end, theta,
                            pair_begin, n_pairs, lag, n_heads, scale, key_layout,
                            (hipStream_t)stream);
  if (st == DP_OK) ok();
  return st;
}

static dp_status hs_attention_impl(const char* who, const void* q, const void* k_ragged,
                            const void* v_ragged, int64_t ragged_capacity, const int64_t* offsets,
                            int32_t layer, const void* k_chunk, const void* v_chunk,
                            int64_t n_chunk, void* o, int64_t n_q, int32_t n_heads,
                            int32_t head_dim, int32_t dtype, float scale, int32_t key_layout,
                            int32_t pair_begin, int32_t n_pairs, const dp::HsLag* lag,
                            void* stream) {
  if (!q || !k_ragged || !v_ragged || !offsets || !o)
    return fail(DP_EINVAL, "%s: q, k_ragged, v_ragged, offsets and o are required", who);
  if (!k_chunk != !v_chunk)
    return fail(DP_EINVAL, "%s: k_chunk and v_chunk are both given or both NULL", who);
  if (dtype != DP_BF16 || head_dim != 128)
    return fail(DP_EUNSUPPORTED, "%s: only bf16 with head_dim 128 is implemented", who);
  if (n_heads < 1 || n_heads > kMaxAttnHeads || layer < 0 || n_q < 0 || n_q >= kMaxRows ||
      ragged_capacity < 0 ||
      ragged_capacity >= ((int64_t)1 << 40) || (k_chunk && (n_chunk < 0 || n_chunk >= kMaxRows)))
    return fail(DP_ERANGE, "%s: need 1 <= n_heads <= 65536, layer >= 0, 0 <= n_q, n_chunk "
                           "< 2^31 and 0 <= ragged_capacity < 2^40", who);
  if ((int64_t)layer * n_heads >= kMaxRows)
    return fail(DP_ERANGE, "%s: layer * n_heads beyond the offsets range", who);
  if ((n_q + 127) / 128 * (int64_t)n_heads >= kMaxVec)
    return fail(DP_ERANGE, "%s: too many query tiles for one launch", who);
  if (!aligned(q, 16) || !aligned(k_ragged, 16) || !aligned(v_ragged, 16) || !aligned(o, 16) ||
      !aligned(offsets, 8) || (k_chunk && (!aligned(k_chunk, 16) || !aligned(v_chunk, 16))))
    return fail(DP_EALIGN, "%s: tensors must be 16-byte aligned (offsets 8)", who);
  if (!(scale > 0.0f && scale <= 3.0e38f))
    return fail(DP_EINVAL, "%s: scale must be positive and finite", who);
  dp_status st = check_key_layout(key_layout, pair_begin, n_pairs, head_dim, dtype, who);
  if (st != DP_OK) return st;
  (void)hipGetLastError();
  st = launch_hs_attention(q, k_ragged, v_ragged, ragged_capacity,
                           offsets + (int64_t)layer * n_heads, k_chunk, v_chunk, n_chunk, o, n_q,
                           n_heads, scale, key_layout, pair_begin, n_pairs, (hipStream_t)stream,
                           lag);
  if (st == DP_OK) ok();
  return st;
}

dp_status dp_hs_attention_lag(const void* q, const void* k_ragged, const void* v_ragged,
                              int64_t ragged_capacity, const int64_t* offsets, int32_t layer,
                              const void* k_chunk, const void* v_chunk, int64_t n_chunk, void* o,
                              int64_t n_q, int32_t n_heads, int32_t head_dim, int32_t dtype,
                              float scale, int64_t plain_tail, const float* theta,
                              int32_t pair_begin, int32_t n_pairs, float lag, int32_t key_layout,
                              void* stream) {
  if (!theta) return fail(DP_EINVAL, "dp_hs_attention_lag: theta is required");
  if (dtype != DP_BF16 || head_dim != 128)
    return fail(DP_EUNSUPPORTED, "dp_hs_attention_lag: only bf16 with head_dim 128 is implemented");
  if (plain_tail < 0) return fail(DP_ERANGE, "dp_hs_attention_lag: need plain_tail >= 0");
  if (n_pairs < 1 || pair_begin < 0 || 2 * ((int64_t)pair_begin + n_pairs) > head_dim)
    return fail(DP_ERANGE, "dp_hs_attention_lag: temporal pairs [%d, %d + %d) outside head_dim/2",
                pair_begin, pair_begin, n_pairs);
  if (!aligned(theta, 4)) return fail(DP_EALIGN, "dp_hs_attention_lag: theta must be 4-byte aligned");
  if (!(lag >= -3.0e38f && lag <= 3.0e38f))
    return fail(DP_EINVAL, "dp_hs_attention_lag: lag must be finite");
  const dp::HsLag hl{plain_tail, theta, pair_begin, n_pairs, lag};
  return hs_attention_impl("dp_hs_attention_lag", q, k_ragged, v_ragged, ragged_capacity, offsets,
                           layer, k_chunk, v_chunk, n_chunk, o, n_q, n_heads, head_dim, dtype,
                           scale, key_layout, pair_begin, n_pairs, &hl, stream);
}

dp_status dp_hs_attention(const void* q, const void* k_ragged, const void* v_ragged,
                          int64_t ragged_capacity, const int64_t* offsets, int32_t layer,
                          const void* k_chunk, const void* v_chunk, int64_t n_chunk, void* o,
                          int64_t n_q, int32_t n_heads, int32_t head_dim, int32_t dtype,
                          float scale, int32_t key_layout, int32_t pair_begin, int32_t n_pairs,
                          void* stream) {
  return hs_attention_impl("dp_hs_attention", q, k_ragged, v_ragged, ragged_capacity, offsets,
                           layer, k_chunk, v_chunk, n_chunk, o, n_q, n_heads, head_dim, dtype,
                           scale, key_layout, pair_begin, n_pairs, nullptr, stream);
}

dp_status dp_pr_add(dp_pr_counter* acc, int64_t visible, int64_t full) {
  if (!acc) return fail(DP_EINVAL, "dp_pr_add: counter is required");
  if (visible < 0 || full < 0 || visible > full)
    return fail(DP_EINVAL, "dp_pr_add: need 0 <= visible <= full");
  acc->visible += visible;
  acc->full += full;
  ok();
  return DP_OK;
}

double dp_pr_value(const dp_pr_counter* acc) {
  if (!acc || acc->full == 0) return 0.0;
  return 1.0 - (double)acc->visible / (double)acc->full;
}

}  // extern "C"
