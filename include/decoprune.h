/*
 * decoprune.h — C ABI of libdecoprune, the history-KV compaction path of
 * DeCoPrune for autoregressive chunked video diffusion, on one AMD Instinct
 * MI355X (gfx950).
 *
 * Source of the method.  Citations name the web page
 *   "DeCoPrune이 디노이징 불일치로 비디오 KV 캐시를 85% 줄인다"
 *   (onedev.kr/papers/726), called "the DeCoPrune page" below,
 * and one of its sections:
 *   무엇인가 (what it is), 어떻게 동작하나 (how it works),
 *   무엇과 다른가 (how it differs), 어떻게 쓰나 (how to use it),
 *   전제와 한계 (premises and limits).
 *
 * The path, one prune step:
 *   1. dp_score_mask    per-token discrepancy l = (1/d)||x0_hat(tau*) - x_final||^2
 *                       and the threshold mask with sink/window protection;
 *   2. dp_compact_index ascending list of kept token rows;
 *   3. dp_gather_kv     physical gather K[m], V[m] of every layer into a shorter
 *                       dense cache (optionally re-rotating K while copying);
 *   4. dp_rope_reindex  in-place RoPE temporal re-indexing of retained keys,
 *                       t~ = q0 - g(q0 - t).
 * plus the head-specialised ragged variant (DeCoPrune-HS, dp_hs_*) and the
 * pruning-ratio counter (dp_pr_*).
 *
 * Conventions shared by every entry point
 *   - Pointers documented "device" are HIP device pointers on the current
 *     device; "host" pointers are read before the call returns.
 *   - stream is a hipStream_t passed as void*; NULL is the null stream.  Every
 *     compute call only enqueues work on that stream and returns; results are
 *     visible to later work on the same stream.  No call synchronises the
 *     device, allocates memory, or keeps state between calls, except the
 *     thread-local error text of dp_last_error() and the library's static
 *     device array that dp_compact_index_noalloc uses instead of a workspace
 *     (described at its declaration).
 *   - The caller owns every buffer.  Scratch memory comes from a caller
 *     workspace sized by the matching *_workspace_bytes() function.  Every
 *     buffer a call reaches, the layer buffers named by device arrays of
 *     pointers included, must stay allocated until the work enqueued on the
 *     stream has finished (the library holds no references; with a caching
 *     allocator, memory freed early may still read back intact until the
 *     allocator returns it to the driver, after which the kernel faults).
 *   - All argument checks run on the host before the first HIP call.  A failed
 *     check returns DP_EINVAL / DP_EALIGN / DP_ERANGE / DP_EUNSUPPORTED and
 *     enqueues nothing.  A failed launch returns DP_EHIP.  dp_last_error()
 *     then describes the failure.  No C++ exception crosses this boundary.
 *   - Conditions only the device can see (a kept count above a destination
 *     capacity) are clamped on the device and reported by writing
 *     DP_ECAPACITY to the optional device word dev_error.
 *   - Token rows are indexed with int32 (seq_len < 2^31); element offsets and
 *     ragged offsets are 64-bit.
 */
#ifndef DECOPRUNE_H
#define DECOPRUNE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DP_ABI_VERSION 3

typedef enum {
  DP_OK = 0,
  DP_EINVAL = 1,        /* null pointer, bad size or inconsistent ranges       */
  DP_EALIGN = 2,        /* pointer or row size not aligned as required          */
  DP_ERANGE = 3,        /* size beyond a documented limit                       */
  DP_ECAPACITY = 4,     /* device-side only: more kept rows than capacity       */
  DP_EHIP = 5,          /* a HIP launch or runtime call failed                  */
  DP_EUNSUPPORTED = 6,  /* valid request outside what the library implements   */
  DP_ESTALL = 7         /* device-side only: a bounded wait between workgroups
                           ran out (results of that call are not valid)        */
} dp_status;

typedef enum { DP_F32 = 0, DP_BF16 = 1 } dp_dtype;

/* DP_MODE_SCORE: scored rows keep by the threshold test; rows that are neither
 *   sink, window nor scored (history compacted by earlier steps) are kept.
 * DP_MODE_STREAMING: only sink and window rows are kept (the Streaming policy
 *   the HS variant gives its static heads) [DeCoPrune page, 무엇과 다른가]. */
typedef enum { DP_MODE_SCORE = 0, DP_MODE_STREAMING = 1 } dp_mode;

int         dp_abi_version(void);
const char* dp_status_str(int status);
/* Text of the last non-OK return on the calling thread ("" if none). */
const char* dp_last_error(void);

/* ------------------------------------------------------------------------- *
 * 1. Score and mask            [DeCoPrune page, 어떻게 동작하나]
 *
 * The page scores each token of a freshly generated chunk by the mean squared
 * gap between the clean prediction recorded at the probe step tau* and the
 * final denoised output, thresholds it with gamma into a binary mask that
 * every layer shares, keeps the high-discrepancy tokens, always keeps the sink
 * chunk and keeps the w most recent chunks dense.
 *
 * Rows of the cache, t in [0, seq_len):
 *   [0, sink_len)                         sink: keep = 1
 *   [scored_begin, scored_begin+n_scored) scored: keep = (l >= gamma),
 *                                         or !(l >= gamma) when reversed
 *                                         (the reversed-criterion ablation of
 *                                         [DeCoPrune page, 전제와 한계]);
 *                                         keep = 0 in DP_MODE_STREAMING
 *   [seq_len-window_len, seq_len)         window: keep = 1
 *   any other row                         keep = 1 (SCORE) / 0 (STREAMING)
 * Requires sink_len <= scored_begin and
 * scored_begin + n_scored <= seq_len - window_len.
 * A NaN score fails "l >= gamma", so the reversed mask is the exact complement.
 * ------------------------------------------------------------------------- */
typedef struct {
  int64_t seq_len;       /* T rows in the cache, 1 <= T < 2^31            */
  int64_t sink_len;      /* rows [0, sink_len) always kept                */
  int64_t window_len;    /* rows [T - window_len, T) always kept          */
  int64_t scored_begin;  /* first scored row                              */
  int64_t n_scored;      /* number of scored rows (may be 0)              */
  float   gamma;         /* threshold, keep iff l >= gamma                */
  int32_t reversed;      /* 0 or 1                                        */
  int32_t mode;          /* dp_mode                                       */
  int32_t reserved;      /* must be 0                                     */
} dp_mask_policy;

/* x0_hat, x_final: device fp32 [n_scored][row_stride]; row i is cache row
 *   scored_begin + i, channels [0, d) are used.  May be NULL when n_scored is
 *   0 or mode is DP_MODE_STREAMING (then not read).  4-byte aligned.
 * d: 1..256.  row_stride >= d (in floats).
 * ell_out: device fp32 [n_scored] or NULL; receives l of every scored row.
 * keep_out: device uint8 [seq_len], receives 0/1 for every row.
 * l is evaluated in fp32: e_c = x0_hat - x_final, q_c = e_c*e_c (no fused
 * multiply-add), q padded with +0 to the next power of two P >= d and summed
 * by the pairwise tree q_c += q_{c+h} for h = P/2, P/4, ..., 1; then
 * l = (float)((double)q_0 / d). */
dp_status dp_score_mask(const float* x0_hat, const float* x_final, int32_t d,
                        int64_t row_stride, const dp_mask_policy* policy,
                        float* ell_out, uint8_t* keep_out, void* stream);

/* ------------------------------------------------------------------------- *
 * 2. Kept-index list           [DeCoPrune page, 어떻게 동작하나]
 *
 * idx_out[j] is the j-th row t (ascending) with keep[t] != 0, so that the
 * gathered cache K[m], V[m] keeps the original token order.  *n_kept (device
 * int64) receives the count.  When row_frame_src/row_frame_dst are both
 * non-NULL, row_frame_dst[j] = row_frame_src[idx_out[j]] (the latent frame of
 * each kept row, used by the RoPE re-index).
 * keep: device uint8 [seq_len]; idx_out: device int32, capacity seq_len;
 * workspace: device, >= dp_compact_workspace_bytes(seq_len) bytes, 4-aligned.
 * Two launches, no host synchronisation.
 * ------------------------------------------------------------------------- */
size_t    dp_compact_workspace_bytes(int64_t seq_len);
dp_status dp_compact_index(const uint8_t* keep, int64_t seq_len, int32_t* idx_out,
                           int64_t* n_kept, const int32_t* row_frame_src,
                           int32_t* row_frame_dst, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * 2'. Kept-index list without a workspace, for callers that cannot allocate
 *     device memory (work under HIP graph capture, serving loops and
 *     harnesses that forbid hipMalloc).
 *
 * Arguments, results and errors as dp_compact_index, without the workspace:
 * the per-tile counts live in a static device array of the library, 2 MiB
 * (one count per 4,096 rows, enough for every seq_len < 2^31), that every GPU
 * the library runs on holds until the process ends.  The array of the current
 * device (hipGetDevice) is used, and stream must belong to that device
 * (DP_EINVAL otherwise); its address is looked up on the first call on each
 * device.  Nothing is allocated.  Every call on one GPU uses the same array,
 * so calls that overlap in time on one GPU (other streams, other threads)
 * race and give wrong lists: order them on one stream.  Nothing in the array
 * needs clearing between calls (each call writes every count it reads).
 * ------------------------------------------------------------------------- */
dp_status dp_compact_index_noalloc(const uint8_t* keep, int64_t seq_len, int32_t* idx_out,
                                   int64_t* n_kept, const int32_t* row_frame_src,
                                   int32_t* row_frame_dst, void* stream);

/* ------------------------------------------------------------------------- *
 * 1+2. Score, mask and kept-index list in one launch
 *                              [DeCoPrune page, 어떻게 동작하나]
 *
 * The same results as dp_score_mask followed by dp_compact_index (bit for
 * bit: ell_out, keep_out, idx_out, *n_kept and row_frame_dst) from one call.
 * When at most 1024 tiles cover the rows (scored rows in tiles of four rows
 * per lane group, e.g. 64 rows at d = 64; other rows in tiles of 256 to 2048
 * rows), it is a single launch: workgroups score and mask their tile and find
 * the output offset of its kept rows by a decoupled look-back over the tiles
 * before them.  Longer scored ranges run as the separate score and compaction
 * kernels, which are faster there (the one-launch form serialises on its tile
 * ticket).  ell_out and keep_out may be NULL (not written).  idx_out: device
 * int32, capacity seq_len; n_kept: device int64.
 * workspace: device, >= dp_score_index_workspace_bytes(seq_len) bytes,
 * 8-byte aligned, zero-filled before its first use; every call leaves it ready
 * for the next call, so it is cleared once, not per call (calls that share a
 * workspace must be ordered on one stream).  dev_error (device int32 or NULL)
 * receives DP_ESTALL if a workgroup's bounded wait for its predecessors ran
 * out, or if the workspace was not zero-filled; the outputs of that call are
 * then not valid and the workspace must be zero-filled again.
 * Policy and score arguments are checked as for dp_score_mask.
 * ------------------------------------------------------------------------- */
size_t    dp_score_index_workspace_bytes(int64_t seq_len);
dp_status dp_score_index(const float* x0_hat, const float* x_final, int32_t d,
                         int64_t row_stride, const dp_mask_policy* policy, float* ell_out,
                         uint8_t* keep_out, int32_t* idx_out, int64_t* n_kept,
                         const int32_t* row_frame_src, int32_t* row_frame_dst,
                         void* workspace, size_t workspace_bytes, int32_t* dev_error,
                         void* stream);

/* ------------------------------------------------------------------------- *
 * RoPE temporal re-index parameters   [DeCoPrune page, 무엇과 다른가]
 *
 * The page moves the temporal coordinate of old context keys to
 * t~ = q0 - g(q0 - t), where g leaves recent offsets unchanged and compresses
 * older ones linearly; only the temporal phase of the keys changes.  Readings
 * used here: positions are latent-frame indices; q0 is the first frame of the
 * chunk about to be generated; g(D) = D for D <= knee and
 * knee + (D - knee) * inv_factor otherwise (continuous at the knee).
 * A key row carries the phase p of its frame; it is rotated by
 * theta_j * (t~ - p) on every temporal pair j, and p becomes t~.
 *
 * Temporal pairs are dims (2j, 2j+1) of each head row for
 * j in [pair_begin, pair_begin + n_pairs); the standard RoPE rotation
 * (a, b) -> (a cos - b sin, a sin + b cos) is applied in fp32 with
 * cos/sin the fp32 roundings of the fp64 cos/sin of the fp32 angle
 * theta_j * delta, products and sums rounded separately (no fused
 * multiply-add), and the result stored back rounded to nearest even.
 * Rows whose frame has delta == 0 are not written.
 *
 * Phase axis.  DP_AXIS_PAGE: the phase a key gets is t~ itself.
 * DP_AXIS_COMPRESSED: past the knee t~ = t/c + A with A = (1 - 1/c)(q0 - knee)
 * the same for every such key, so a key past the knee gets phase
 * t * inv_factor (= t/c) once, when it first passes the knee, and keeps it;
 * attention then rotates the query back by A for those keys
 * (dp_attention_lag), which gives the scores of the page's t~ without
 * rewriting old keys at every step.  Keys within the knee keep phase t.
 * ------------------------------------------------------------------------- */
typedef enum { DP_AXIS_PAGE = 0, DP_AXIS_COMPRESSED = 1 } dp_axis;

/* Key layout (where a key row keeps its temporal pairs).  Keys are token-major,
 * one row per token holding all n_heads heads; V is never permuted.
 *   DP_KEY_INTERLEAVED: the row is [n_heads][head_dim], each head's dims in
 *     order.
 *   DP_KEY_SPLIT: the row holds first the temporal block of every head
 *     (head h: dims [2 pair_begin, 2 (pair_begin + n_pairs)) at elements
 *     [h * 2 n_pairs, (h + 1) * 2 n_pairs)), then the remaining dims of every
 *     head (head h: dims [0, 2 pair_begin) and [2 (pair_begin + n_pairs),
 *     head_dim), in order, at elements n_heads * 2 n_pairs +
 *     h * (head_dim - 2 n_pairs) ...).  A fixed permutation of a key row's
 *     elements, which a model absorbs into its key projection; attention
 *     reads it back per head.  Only the key temporal phase changes in a
 *     re-index [DeCoPrune page, 무엇과 다른가], so in this layout a re-index
 *     reads and writes the rows' leading n_heads * 2 n_pairs elements, whole
 *     128-byte lines, and nothing else.  Requires 2 n_pairs * elem_size to be
 *     a multiple of 16 bytes (DP_EALIGN otherwise).
 *   A packed per-head (HS) run of n head rows in this layout holds the n
 *   temporal blocks, then the n remaining parts.
 */
typedef enum { DP_KEY_INTERLEAVED = 0, DP_KEY_SPLIT = 1 } dp_key_layout;

typedef struct {
  int32_t      pair_begin;   /* first temporal pair                              */
  int32_t      n_pairs;      /* pairs in the temporal block, >= 1               */
  const float* theta;        /* device fp32 [n_pairs] angular frequencies       */
  int32_t      n_frames;     /* frames described by frame_t/frame_phase, >= 1   */
  int32_t      axis;         /* dp_axis                                          */
  const float* frame_t;      /* device fp32 [n_frames] original index t        */
  float*       frame_phase;  /* device fp32 [n_frames] phase p; set to t~      */
  float        q0;           /* query origin (frames)                            */
  float        knee;         /* offsets <= knee are left unchanged               */
  float        inv_factor;   /* 1/c, the linear compression of older offsets     */
  int32_t      key_layout;   /* dp_key_layout of the keys the re-index rotates   */
} dp_rope;

/* Workspace of a re-index (per-frame delta and cos/sin table). */
size_t dp_rope_workspace_bytes(int32_t n_frames, int32_t n_pairs);

/* ------------------------------------------------------------------------- *
 * 3. Physical gather           [DeCoPrune page, 어떻게 동작하나]
 *
 * When a non-sink chunk leaves the dense window, every layer keeps only the
 * selected entries, so the KV sequence really gets shorter.  For every layer
 * l < n_layers and j < min(*n_kept, dst_capacity):
 *   k_dst[l][j][:][:] = k_src[l][idx[j]][:][:]   (bit copy)
 *   v_dst[l][j][:][:] = v_src[l][idx[j]][:][:]   (if v_src != NULL)
 * All layers, K and V in one launch.  Caches are token-major
 * [rows][n_heads][head_dim] of dtype, one device allocation per layer, given
 * as device arrays of n_layers device pointers.  Each layer base is 16-byte
 * aligned and n_heads*head_dim*elem_size is a multiple of 16.
 * If *n_kept > dst_capacity the copy is clamped and *dev_error = DP_ECAPACITY.
 * idx entries must lie in [0, src_rows) (as dp_compact_index produces).
 * With fused_rope != NULL, K rows are re-rotated while copied (section 4);
 * row_frame (device int32 [dst_capacity]) then gives the frame of gathered row
 * j and workspace must hold dp_rope_workspace_bytes(); V is never rotated.
 * Source and destination must not overlap.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void* const* k_src;  /* device array [n_layers] of device layer bases  */
  const void* const* v_src;  /* same, or NULL for a K-only gather               */
  void* const*       k_dst;  /* device array [n_layers] of device layer bases  */
  void* const*       v_dst;  /* NULL iff v_src is NULL                          */
  int32_t n_layers;          /* >= 1                                            */
  int32_t n_heads;           /* >= 1                                            */
  int32_t head_dim;          /* >= 2, even                                      */
  int32_t dtype;             /* dp_dtype                                        */
  int64_t src_rows;          /* rows of each source layer                       */
  int64_t dst_capacity;      /* rows of each destination layer                  */
  int32_t* dev_error;        /* device int32 or NULL                            */
} dp_kv;

dp_status dp_gather_kv(const dp_kv* kv, const int32_t* idx, const int64_t* n_kept,
                       const int32_t* row_frame, const dp_rope* fused_rope,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * 4. In-place RoPE re-index    [DeCoPrune page, 무엇과 다른가]
 *
 * Re-rotates, in place, the temporal pairs of every head of rows
 * [0, min(rows_capacity, *n_rows)) of each layer k_layers[l]
 * (token-major [rows][n_heads][head_dim]) as described above.  n_rows is a
 * device int64 or NULL (then rows_capacity rows).  row_frame: device int32
 * [rows_capacity], frame of each row, in [0, n_frames).  Each frame's
 * phase is advanced once per call, so every retained row of a listed frame
 * must be in the range re-indexed by this call.
 * ------------------------------------------------------------------------- */
dp_status dp_rope_reindex(void* const* k_layers, int32_t n_layers, int32_t n_heads,
                          int32_t head_dim, int32_t dtype, int64_t rows_capacity,
                          const int64_t* n_rows, const int32_t* row_frame,
                          const dp_rope* rope, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Two-phase form of the same re-index, for caches whose re-indexed rows are
 * not one range (the [sink | window ring | history] layout of dp_append_kept):
 * dp_rope_prepare computes the per-frame phase steps and {cos, sin} table into
 * the workspace and advances frame_phase, once per step; dp_rope_apply then
 * re-rotates rows [row_begin, min(rows_capacity, *n_rows)) (n_rows device or
 * NULL) of every layer from that table, and may be called for several row
 * ranges.  The dp_rope passed to both must describe the same tables; apply
 * reads only its pair layout and frame count.  head_dim and dtype are those
 * of the keys apply will rotate. */
dp_status dp_rope_prepare(const dp_rope* rope, int32_t head_dim, int32_t dtype, void* workspace,
                          size_t workspace_bytes, void* stream);
dp_status dp_rope_apply(void* const* k_layers, int32_t n_layers, int32_t n_heads,
                        int32_t head_dim, int32_t dtype, int64_t row_begin,
                        int64_t rows_capacity, const int64_t* n_rows, const int32_t* row_frame,
                        const dp_rope* rope, const void* workspace, size_t workspace_bytes,
                        void* stream);

/* dp_rope_shift: the steady-state re-index [DeCoPrune page, 무엇과 다른가].
 * A frame past the knee before and after a step moves by the same amount as
 * every other such frame: q0 advances F frames per step, so t~ advances by
 * F * (1 - 1/c) (3.5 frames for 4-frame chunks and c = 8).  A row range that
 * holds only such rows (in the ring layout: the sink and the history appended
 * before this step) is therefore rotated by one uniform step delta, with no
 * row frames and no per-frame table: every temporal pair j of rows
 * [row_begin, min(rows_capacity, *n_rows)) of every layer is rotated by
 * theta_j * delta, with cos/sin, rounding and storage as in section 4 (the
 * result equals dp_rope_apply on those rows bit for bit when each of their
 * frames has step delta).  theta: device fp32 [n_pairs]; delta finite
 * (0 writes nothing).  workspace: device, 16-byte aligned, at least
 * dp_rope_shift_workspace_bytes(n_pairs) bytes (the step's {cos, sin} table;
 * calls that share it must be ordered on one stream).  Frame phases are not
 * touched: the caller's dp_rope_prepare of the step advances every frame.
 * key_layout: dp_key_layout of the keys.  Two launches (the table, then the
 * rotation).
 * ------------------------------------------------------------------------- */
size_t    dp_rope_shift_workspace_bytes(int32_t n_pairs);
dp_status dp_rope_shift(void* const* k_layers, int32_t n_layers, int32_t n_heads,
                        int32_t head_dim, int32_t dtype, int64_t row_begin,
                        int64_t rows_capacity, const int64_t* n_rows, const float* theta,
                        int32_t pair_begin, int32_t n_pairs, int32_t key_layout, float delta,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * 4b. Segment-append compaction in place     [DeCoPrune page, 어떻게 동작하나]
 *
 * The page compacts a chunk when it leaves the dense window; only that chunk's
 * rows change state.  With the cache laid out per layer as
 *   [sink | window ring of chunk slots | history]        (rows [0, *tail))
 * in one buffer of `capacity` rows, the kept rows of the slot holding the
 * leaving chunk are appended at the history tail, so the sink, the other
 * window slots and earlier history never move and the visible cache stays
 * one contiguous row range.  For every layer l and j < n = *n_kept:
 *   K[l][*tail + j] = K[l][slot_begin + idx[j]]     (bit copy; V likewise)
 *   row_frame[*tail + j] = row_frame[slot_begin + idx[j]]   (if row_frame)
 * then row_frame[slot_begin .. slot_begin + slot_rows) = -1 (the slot's rows are
 * retired: the re-index skips them until the next chunk is written into the
 * slot together with its frames) and *tail += n.  idx holds slot-relative rows
 * (dp_compact_index over the slot's keep mask), ascending, in [0, slot_rows).
 * Device-side checks: if the appended rows would pass `capacity` or overlap
 * the slot, nothing is copied or advanced and *dev_error = DP_ECAPACITY or
 * DP_ERANGE.  Two launches on `stream`.  The old keys are then re-indexed in
 * place: dp_rope_prepare once, then dp_rope_apply over the sink rows and over
 * the history rows [history_begin, *tail) (n_rows = tail); the window slots
 * need no re-index while they are in the window.
 * fused_rope (or NULL): the K rows are re-rotated while copied, each by its
 * frame's phase step, from the tables a dp_rope_prepare of this step wrote
 * into workspace (fused_rope is read for its pair layout and frame count, as by
 * dp_rope_apply; row_frame is then required).  This is the first re-index of a
 * chunk that has just left the window.  In the steady state the other old
 * keys all move by one uniform step, so a step is: dp_rope_shift over the sink
 * and over [history_begin, *tail) (before this call, so the tail is the old
 * one), dp_rope_prepare, then this call with the fused re-index.
 * ------------------------------------------------------------------------- */
typedef struct {
  void* const* k_layers;     /* device array [n_layers]: [capacity][n_heads][head_dim] */
  void* const* v_layers;     /* same, or NULL                                          */
  int32_t n_layers, n_heads, head_dim, dtype;
  int64_t capacity;          /* rows of each layer buffer, < 2^31                      */
  int32_t* dev_error;        /* device int32 or NULL                                   */
} dp_kv_inplace;

dp_status dp_append_kept(const dp_kv_inplace* kv, int64_t slot_begin, int64_t slot_rows,
                         const int32_t* idx, const int64_t* n_kept, int64_t* tail,
                         int32_t* row_frame, const dp_rope* fused_rope,
                         const void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * 5. DeCoPrune-HS: head-specialised ragged cache   [DeCoPrune page, 무엇과 다른가]
 *
 * The page splits heads into dynamic heads, which follow the DeCoPrune mask,
 * and static heads, which follow the Streaming policy (sink + recent window).
 * Here every (layer, head) names a class c = head_class[l*n_heads + h] in
 * [0, n_classes); class c keeps the rows of its own kept-index list
 * class_idx[c] (length *class_len[c], produced by dp_compact_index from the
 * class's mask).  Head (l, h) gets n_{l,h} = class_len[head_class[l,h]] rows.
 *
 * dp_hs_offsets: offsets[0] = 0, offsets[i+1] = offsets[i] + n_i over
 *   i = l*n_heads + h in row-major order; offsets is device int64
 *   [n_layers*n_heads + 1].  One launch.
 * dp_hs_gather_kv: for each (l, h) and j < n_{l,h}:
 *   k_out[offsets[l,h] + j][:] = k_src[l][class_idx[c][j]][h][:]
 *   (and V).  Output is packed per head, [offsets[L*H]][head_dim].  Rows
 *   beyond out_capacity are dropped and *dev_error = DP_ECAPACITY.
 *   class_capacity (host int64 [n_classes]) bounds each class's list length
 *   (sizes the grid; lists longer than it are clamped and flagged).
 *   With fused_rope, K is re-rotated while copied; class_row_frame (device
 *   array [n_classes] of device int32 lists) gives the frame of each listed row.
 * dp_hs_rope_reindex: in-place re-index of a ragged K cache laid out as above;
 *   k_capacity is the number of head rows in k_ragged (rows beyond it are
 *   skipped).
 * Key layouts (dp_kv_hs.src_key_layout for the source token rows,
 *   dp_kv_hs.key_layout for the packed runs, one pair range for both; for the
 *   re-index the rope's): with DP_KEY_SPLIT runs each output run holds its
 *   temporal blocks, then the remaining parts (a run's head rows are then not
 *   head_dim apart), so the re-index of a run rewrites only whole lines; with
 *   DP_KEY_SPLIT sources the token rows are split rows.  Any pairing is
 *   allowed: interleaved sources with split runs read whole head rows and
 *   write split runs (the two classes of a layer then share no source line).
 *   A fused_rope must name the runs' layout and pairs (DP_EINVAL).  V is
 *   packed as plain head rows in every case.
 * class_idx / class_row_frame are device arrays of n_classes device pointers;
 * class_len is device int64 [n_classes].  n_classes <= DP_HS_MAX_CLASSES.
 *
 * Ring layout for a rollout (no entry point of its own): the split is fixed
 * per layer, so a model may order each layer's heads class by class (a
 * permutation of its projection weights) and keep one token-major cache per
 * class: static [sink | window ring], dynamic [sink | window ring | history].
 * All dynamic heads keep the same rows, so an eviction is dp_append_kept over
 * the dynamic buffers of all layers (n_heads = heads of the class), the static
 * class only retires the slot, the old keys are re-indexed by dp_rope_apply
 * (both sinks, the dynamic history), and attention runs per class buffer with
 * dp_attention (queries of the class's heads, keys [0, *tail) or the static
 * buffer's rows).
 * ------------------------------------------------------------------------- */
#define DP_HS_MAX_CLASSES 8

typedef struct {
  const void* const* k_src;  /* device array [n_layers], token-major layers     */
  const void* const* v_src;  /* same, or NULL                                   */
  void*   k_out;             /* device [out_capacity][head_dim]                 */
  void*   v_out;             /* NULL iff v_src is NULL                          */
  int32_t n_layers, n_heads, head_dim, dtype;
  int64_t src_rows;          /* rows of each source layer                       */
  int64_t out_capacity;      /* head-rows available in k_out / v_out            */
  int32_t* dev_error;        /* device int32 or NULL                            */
  int32_t key_layout;        /* dp_key_layout of the packed runs in k_out       */
  int32_t pair_begin;        /* temporal pairs of the split layout              */
  int32_t n_pairs;           /*   (ignored when neither layout is split)        */
  int32_t src_key_layout;    /* dp_key_layout of the k_src token rows           */
} dp_kv_hs;

dp_status dp_hs_offsets(const uint8_t* head_class, int32_t n_layers, int32_t n_heads,
                        const int64_t* class_len, int32_t n_classes, int64_t* offsets,
                        void* stream);

dp_status dp_hs_gather_kv(const dp_kv_hs* kv, const uint8_t* head_class,
                          int32_t n_classes, const int32_t* const* class_idx,
                          const int64_t* class_len, const int64_t* class_capacity,
                          const int64_t* offsets, const int32_t* const* class_row_frame,
                          const dp_rope* fused_rope, void* workspace,
                          size_t workspace_bytes, void* stream);

dp_status dp_hs_rope_reindex(void* k_ragged, int64_t k_capacity, int32_t n_layers,
                             int32_t n_heads, int32_t head_dim, int32_t dtype,
                             const uint8_t* head_class,
                             int32_t n_classes, const int64_t* class_len,
                             const int64_t* class_capacity, const int64_t* offsets,
                             const int32_t* const* class_row_frame, const dp_rope* rope,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------- *
 * 7. Attention over the compacted cache   [DeCoPrune page, 무엇인가 and 전제와 한계]
 *
 * The page's motivation: every new chunk attends to the KV cache of the whole
 * history, so its cost grows with the rollout; the continuation speed-up it
 * reports comes from this attention running over the compacted cache.  For
 * each head h and query i < n_q:
 *   o[i][h][:] = sum_{j < n} softmax_j(scale * <q[i][h], k[j][h]>) v[j][h][:]
 * with n = min(kv_capacity, *n_kv) (n_kv device int64, or NULL for
 * kv_capacity); n = 0 gives zeros.  q, o: [n_q][n_heads][head_dim];
 * k, v: [kv_capacity][n_heads][head_dim] (one layer of the cache, e.g. the
 * ring layout's rows [0, tail) including the chunk itself); all bf16, 16-byte
 * aligned, o not overlapping the inputs; 1 <= n_heads <= 65536 (DP_ERANGE);
 * scale > 0 and finite (DP_EINVAL otherwise).  fp32 accumulation and softmax;
 * head_dim 128 and bf16 only (DP_EUNSUPPORTED otherwise).  No mask: every
 * query sees every cached row.  key_layout: dp_key_layout of k, with the
 * temporal pairs [pair_begin, pair_begin + n_pairs) of DP_KEY_SPLIT (ignored
 * for DP_KEY_INTERLEAVED; checked as for dp_rope_shift); q, v and o are
 * never permuted.  One launch.
 * ------------------------------------------------------------------------- */
dp_status dp_attention(const void* q, const void* k, const void* v, void* o, int64_t n_q,
                       int64_t kv_capacity, const int64_t* n_kv, int32_t n_heads,
                       int32_t head_dim, int32_t dtype, float scale, int32_t key_layout,
                       int32_t pair_begin, int32_t n_pairs, void* stream);

/* dp_attention_lag: the same attention over a cache whose keys past the knee
 *   are kept on the compressed time axis (dp_rope.axis = DP_AXIS_COMPRESSED)
 *   [DeCoPrune page, 어떻게 쓰나 (the temporal re-index t~ = q0 - g(q0 - t))].
 *   Past the knee t~ = t/c + A with A = (1 - 1/c)(q0 - knee) common to all such
 *   keys; a key stored at phase t/c scores against the query turned back by A
 *   exactly as the key at phase t~ scores against the query (RoPE scores depend
 *   on the phase difference only), so the old keys need no rewrite when q0
 *   advances.  Rows j in [plain_begin, plain_end) (the window and the chunk,
 *   within the knee) see q as given; every other row j < n sees q with the
 *   temporal pairs [pair_begin, pair_begin + n_pairs) rotated by -lag (lag = A
 *   in frames; the angle fp32 theta[p] * -lag, fp64 sincos rounded to fp32,
 *   products and sums rounded separately, bf16 round-to-nearest-even: the
 *   rotation dp_rope_apply makes for a phase change of -lag).  theta: device
 *   fp32 [n_pairs].  Other arguments, layout, n, limits and errors as for
 *   dp_attention; plain_begin >= 0 and plain_end >= plain_begin (DP_ERANGE;
 *   both clamped to n); n_pairs >= 1, pair_begin >= 0 and
 *   2 (pair_begin + n_pairs) <= head_dim (DP_ERANGE); lag finite (DP_EINVAL).
 *   With plain_begin = 0 and plain_end >= n this is dp_attention, bit for bit.
 *   key_layout: as for dp_attention, with the same temporal pairs.  One launch.
 * ------------------------------------------------------------------------- */
dp_status dp_attention_lag(const void* q, const void* k, const void* v, void* o, int64_t n_q,
                           int64_t kv_capacity, const int64_t* n_kv, int64_t plain_begin,
                           int64_t plain_end, const float* theta, int32_t pair_begin,
                           int32_t n_pairs, float lag, int32_t n_heads, int32_t head_dim,
                           int32_t dtype, float scale, int32_t key_layout, void* stream);

/* dp_hs_attention: the same attention over the ragged DeCoPrune-HS cache
 *   [DeCoPrune page, 무엇인가 (DeCoPrune-HS: static heads see only the sink
 *   and the recent window, dynamic heads the pruned history)].  Head h of
 *   layer `layer` sees its own run of the packed per-head cache,
 *     k_ragged[offsets[layer*n_heads + h] + j][:],  j < n_{layer,h}
 *   (offsets as written by dp_hs_offsets, device int64, at least
 *   (layer+1)*n_heads + 1 entries; runs are clamped to [0, ragged_capacity)
 *   head rows, so no row outside k_ragged is read), followed by the n_chunk
 *   rows of an optional dense block k_chunk, v_chunk [n_chunk][n_heads][head_dim]
 *   (the chunk's own keys; both NULL for none).  q, o: [n_q][n_heads][head_dim].
 *   bf16, head_dim 128 (DP_EUNSUPPORTED otherwise); scale as for dp_attention;
 *   fp32 accumulation and softmax; a head with no rows gives zeros.
 *   key_layout, pair_begin, n_pairs: as for dp_attention; with DP_KEY_SPLIT
 *   each run of k_ragged holds its temporal blocks, then its remaining parts
 *   (as dp_hs_gather_kv writes it), and k_chunk is split token rows.
 *   One launch.
 * ------------------------------------------------------------------------- */
dp_status dp_hs_attention(const void* q, const void* k_ragged, const void* v_ragged,
                          int64_t ragged_capacity, const int64_t* offsets, int32_t layer,
                          const void* k_chunk, const void* v_chunk, int64_t n_chunk, void* o,
                          int64_t n_q, int32_t n_heads, int32_t head_dim, int32_t dtype,
                          float scale, int32_t key_layout, int32_t pair_begin, int32_t n_pairs,
                          void* stream);

/* dp_hs_attention_lag: dp_hs_attention over a ragged cache whose keys past the
 *   knee are on the compressed time axis (see dp_attention_lag)
 *   [DeCoPrune page, 무엇인가 (DeCoPrune-HS) and 어떻게 쓰나 (the temporal
 *   re-index)].  In each head's run the last plain_tail rows (the window, kept
 *   by every head and within the knee; the whole run when it is shorter) and
 *   the chunk block see q as given; every other row of the run sees q with the
 *   temporal pairs rotated by -lag (rounding as dp_attention_lag).  Other
 *   arguments, layout, limits and errors as for dp_hs_attention; plain_tail >= 0
 *   (DP_ERANGE); theta, pair_begin, n_pairs, lag as for dp_attention_lag.  With
 *   plain_tail >= every run's length this is dp_hs_attention, bit for bit.
 *   key_layout: as for dp_hs_attention, with the same temporal pairs.
 *   One launch.
 * ------------------------------------------------------------------------- */
dp_status dp_hs_attention_lag(const void* q, const void* k_ragged, const void* v_ragged,
                              int64_t ragged_capacity, const int64_t* offsets, int32_t layer,
                              const void* k_chunk, const void* v_chunk, int64_t n_chunk, void* o,
                              int64_t n_q, int32_t n_heads, int32_t head_dim, int32_t dtype,
                              float scale, int64_t plain_tail, const float* theta,
                              int32_t pair_begin, int32_t n_pairs, float lag, int32_t key_layout,
                              void* stream);

/* ------------------------------------------------------------------------- *
 * 6. Pruning ratio             [DeCoPrune page, 어떻게 쓰나 and 전제와 한계]
 *
 * The page measures efficiency as the cumulative reduction, against FullKV,
 * of the history KV positions attention can see, counted per chunk, layer and
 * head; it is not a peak-memory or total-compute saving.  A counter adds, per
 * step, the visible positions (sum over layers and heads of kept rows) and the
 * FullKV positions (layers * heads * full history rows).
 * PR = 1 - visible / full (0 when full is 0).  Host-only, no HIP call.
 * ------------------------------------------------------------------------- */
typedef struct {
  int64_t visible;
  int64_t full;
} dp_pr_counter;

dp_status dp_pr_add(dp_pr_counter* acc, int64_t visible_positions, int64_t full_positions);
double    dp_pr_value(const dp_pr_counter* acc);

#ifdef __cplusplus
}
#endif
#endif /* DECOPRUNE_H */
