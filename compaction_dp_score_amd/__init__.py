"""Python binding of libdecoprune (argument marshalling only).

Every function has the name of the C entry point it calls and takes torch
tensors on the GPU; all work runs in the library's HIP kernels on the
caller's current stream.  Importing this package loads the in-tree
``libdecoprune.so`` and fails loudly if it is not built.  Errors of the C
ABI raise ``DPError`` with the library's own message.

Method source: the page "DeCoPrune이 디노이징 불일치로 비디오 KV 캐시를 85%
줄인다" (onedev.kr/papers/726); the C header include/decoprune.h cites the
section behind every entry point.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdecoprune.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libdecoprune.so is not built (run __graft_entry__.build() or "
                      "python compaction_dp_score_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)
ABI_VERSION = 3                # DP_ABI_VERSION of the include/decoprune.h this binding follows
_lib.dp_abi_version.restype = ctypes.c_int
if _lib.dp_abi_version() != ABI_VERSION:
    raise ImportError("libdecoprune.so reports ABI %d, this binding follows ABI %d: rebuild it"
                      % (_lib.dp_abi_version(), ABI_VERSION))

DP_OK, DP_EINVAL, DP_EALIGN, DP_ERANGE, DP_ECAPACITY, DP_EHIP, DP_EUNSUPPORTED, DP_ESTALL = range(8)
DP_F32, DP_BF16 = 0, 1
DP_MODE_SCORE, DP_MODE_STREAMING = 0, 1
DP_HS_MAX_CLASSES = 8
DP_AXIS_PAGE, DP_AXIS_COMPRESSED = 0, 1
DP_KEY_INTERLEAVED, DP_KEY_SPLIT = 0, 1

_P = ctypes.c_void_p
_i32, _i64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float


class DPError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (dp_status_str(status), message))
        self.status = status


class dp_mask_policy(ctypes.Structure):
    _fields_ = [("seq_len", _i64), ("sink_len", _i64), ("window_len", _i64),
                ("scored_begin", _i64), ("n_scored", _i64), ("gamma", _f32),
                ("reversed", _i32), ("mode", _i32), ("reserved", _i32)]


class dp_rope(ctypes.Structure):
    _fields_ = [("pair_begin", _i32), ("n_pairs", _i32), ("theta", _P), ("n_frames", _i32),
                ("axis", _i32), ("frame_t", _P), ("frame_phase", _P), ("q0", _f32),
                ("knee", _f32), ("inv_factor", _f32), ("key_layout", _i32)]


class dp_kv(ctypes.Structure):
    _fields_ = [("k_src", _P), ("v_src", _P), ("k_dst", _P), ("v_dst", _P),
                ("n_layers", _i32), ("n_heads", _i32), ("head_dim", _i32), ("dtype", _i32),
                ("src_rows", _i64), ("dst_capacity", _i64), ("dev_error", _P)]


class dp_kv_hs(ctypes.Structure):
    _fields_ = [("k_src", _P), ("v_src", _P), ("k_out", _P), ("v_out", _P),
                ("n_layers", _i32), ("n_heads", _i32), ("head_dim", _i32), ("dtype", _i32),
                ("src_rows", _i64), ("out_capacity", _i64), ("dev_error", _P),
                ("key_layout", _i32), ("pair_begin", _i32), ("n_pairs", _i32),
                ("src_key_layout", _i32)]


class dp_kv_inplace(ctypes.Structure):
    _fields_ = [("k_layers", _P), ("v_layers", _P), ("n_layers", _i32), ("n_heads", _i32),
                ("head_dim", _i32), ("dtype", _i32), ("capacity", _i64), ("dev_error", _P)]


class dp_pr_counter(ctypes.Structure):
    _fields_ = [("visible", _i64), ("full", _i64)]


def _sig(name, args, res=ctypes.c_int):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_lib_abi = _sig("dp_abi_version", [])
_lib_status_str = _sig("dp_status_str", [ctypes.c_int], ctypes.c_char_p)
_lib_last_error = _sig("dp_last_error", [], ctypes.c_char_p)
_lib_score_mask = _sig("dp_score_mask", [_P, _P, _i32, _i64, ctypes.POINTER(dp_mask_policy), _P, _P, _P])
_lib_compact_ws = _sig("dp_compact_workspace_bytes", [_i64], ctypes.c_size_t)
_lib_compact = _sig("dp_compact_index", [_P, _i64, _P, _P, _P, _P, _P, ctypes.c_size_t, _P])
_lib_compact_noalloc = _sig("dp_compact_index_noalloc", [_P, _i64, _P, _P, _P, _P, _P])
_lib_rope_ws = _sig("dp_rope_workspace_bytes", [_i32, _i32], ctypes.c_size_t)
_lib_gather = _sig("dp_gather_kv", [ctypes.POINTER(dp_kv), _P, _P, _P, ctypes.POINTER(dp_rope), _P,
                                    ctypes.c_size_t, _P])
_lib_reindex = _sig("dp_rope_reindex", [_P, _i32, _i32, _i32, _i32, _i64, _P, _P,
                                        ctypes.POINTER(dp_rope), _P, ctypes.c_size_t, _P])
_lib_rope_prepare = _sig("dp_rope_prepare", [ctypes.POINTER(dp_rope), _i32, _i32, _P, ctypes.c_size_t, _P])
_lib_rope_apply = _sig("dp_rope_apply", [_P, _i32, _i32, _i32, _i32, _i64, _i64, _P, _P,
                                         ctypes.POINTER(dp_rope), _P, ctypes.c_size_t, _P])
_lib_rope_shift_ws = _sig("dp_rope_shift_workspace_bytes", [_i32], ctypes.c_size_t)
_lib_rope_shift = _sig("dp_rope_shift", [_P, _i32, _i32, _i32, _i32, _i64, _i64, _P, _P, _i32, _i32,
                                         _i32, _f32, _P, ctypes.c_size_t, _P])
_lib_append = _sig("dp_append_kept", [ctypes.POINTER(dp_kv_inplace), _i64, _i64, _P, _P, _P, _P,
                                        ctypes.POINTER(dp_rope), _P, ctypes.c_size_t, _P])
_lib_hs_offsets = _sig("dp_hs_offsets", [_P, _i32, _i32, _P, _i32, _P, _P])
_lib_hs_gather = _sig("dp_hs_gather_kv", [ctypes.POINTER(dp_kv_hs), _P, _i32, _P, _P,
                                          ctypes.POINTER(_i64), _P, _P, ctypes.POINTER(dp_rope),
                                          _P, ctypes.c_size_t, _P])
_lib_hs_reindex = _sig("dp_hs_rope_reindex", [_P, _i64, _i32, _i32, _i32, _i32, _P, _i32, _P,
                                              ctypes.POINTER(_i64), _P, _P, ctypes.POINTER(dp_rope),
                                              _P, ctypes.c_size_t, _P])
_lib_si_ws = _sig("dp_score_index_workspace_bytes", [_i64], ctypes.c_size_t)
_lib_score_index = _sig("dp_score_index", [_P, _P, _i32, _i64, ctypes.POINTER(dp_mask_policy), _P,
                                           _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P])
_lib_attention = _sig("dp_attention", [_P, _P, _P, _P, _i64, _i64, _P, _i32, _i32, _i32, _f32,
                                      _i32, _i32, _i32, _P])
_lib_attention_lag = _sig("dp_attention_lag", [_P, _P, _P, _P, _i64, _i64, _P, _i64, _i64, _P,
                                                _i32, _i32, _f32, _i32, _i32, _i32, _f32, _i32, _P])
_lib_hs_attention = _sig("dp_hs_attention", [_P, _P, _P, _i64, _P, _i32, _P, _P, _i64, _P, _i64,
                                              _i32, _i32, _i32, _f32, _i32, _i32, _i32, _P])
_lib_hs_attention_lag = _sig("dp_hs_attention_lag", [_P, _P, _P, _i64, _P, _i32, _P, _P, _i64, _P,
                                                      _i64, _i32, _i32, _i32, _f32, _i64, _P, _i32,
                                                      _i32, _f32, _i32, _P])
_lib_pr_add = _sig("dp_pr_add", [ctypes.POINTER(dp_pr_counter), _i64, _i64])
_lib_pr_value = _sig("dp_pr_value", [ctypes.POINTER(dp_pr_counter)], ctypes.c_double)

EXPORTED = ["dp_abi_version", "dp_status_str", "dp_last_error", "dp_score_mask",
            "dp_compact_workspace_bytes", "dp_compact_index", "dp_compact_index_noalloc",
            "dp_rope_workspace_bytes",
            "dp_gather_kv", "dp_rope_reindex", "dp_rope_prepare", "dp_rope_apply", "dp_rope_shift_workspace_bytes",
            "dp_rope_shift", "dp_append_kept",
            "dp_hs_offsets", "dp_hs_gather_kv",
            "dp_hs_rope_reindex", "dp_attention", "dp_attention_lag", "dp_hs_attention",
            "dp_hs_attention_lag", "dp_score_index_workspace_bytes",
            "dp_score_index", "dp_pr_add", "dp_pr_value"]


def dp_abi_version():
    return _lib_abi()


def dp_status_str(status):
    return _lib_status_str(status).decode()


def dp_last_error():
    return _lib_last_error().decode()


def _check(status):
    if status != DP_OK:
        raise DPError(status, dp_last_error())


def _ptr(t):
    """Device (or host) address of a tensor, None for None."""
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dtype_code(t):
    if t.dtype == torch.float32:
        return DP_F32
    if t.dtype == torch.bfloat16:
        return DP_BF16
    raise TypeError("K/V caches must be float32 or bfloat16, got %s" % t.dtype)


def ptr_array(tensors, device):
    """Device array of the data pointers of ``tensors`` (int64), or None.

    The array holds references to the tensors, so that memory it points at
    lives as long as the array does: a tensor reachable only through a pointer
    array would otherwise be freed into the caching allocator at once (its
    memory still mapped, so kernels reading it seem to work) and released to
    the driver by the next torch.cuda.empty_cache() (which entering
    torch.cuda.graph calls), after which a kernel reaching it through the array
    faults."""
    if tensors is None:
        return None
    tensors = list(tensors)
    arr = torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=device)
    arr._dp_targets = tensors
    return arr


def make_rope(theta, frame_t, frame_phase, q0, knee, inv_factor, pair_begin=0, axis=0,
              key_layout=DP_KEY_INTERLEAVED):
    """A dp_rope over device tensors theta [n_pairs], frame_t/frame_phase [n_frames].

    axis: DP_AXIS_PAGE (0) or DP_AXIS_COMPRESSED (1); key_layout: DP_KEY_INTERLEAVED
    (0) or DP_KEY_SPLIT (1), the layout of the keys the re-index rotates."""
    r = dp_rope()
    r.pair_begin = pair_begin
    r.n_pairs = theta.numel()
    r.theta = theta.data_ptr()
    r.n_frames = frame_t.numel()
    r.axis = int(axis)
    r.frame_t = frame_t.data_ptr()
    r.frame_phase = frame_phase.data_ptr()
    r.q0, r.knee, r.inv_factor = float(q0), float(knee), float(inv_factor)
    r.key_layout = int(key_layout)
    r._tensors = (theta, frame_t, frame_phase)   # the struct holds raw pointers: keep them alive
    return r


def make_policy(seq_len, sink_len, window_len, scored_begin, n_scored, gamma,
                reversed=False, mode=DP_MODE_SCORE):
    p = dp_mask_policy()
    p.seq_len, p.sink_len, p.window_len = seq_len, sink_len, window_len
    p.scored_begin, p.n_scored, p.gamma = scored_begin, n_scored, float(gamma)
    p.reversed, p.mode, p.reserved = int(bool(reversed)), int(mode), 0
    return p


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------
def dp_score_mask(x0_hat, x_final, d, row_stride, policy, ell_out, keep_out, stream=None):
    _check(_lib_score_mask(_ptr(x0_hat), _ptr(x_final), d, row_stride, ctypes.byref(policy),
                           _ptr(ell_out), _ptr(keep_out), _stream(stream)))


def dp_compact_workspace_bytes(seq_len):
    return _lib_compact_ws(seq_len)


def dp_score_index_workspace_bytes(seq_len):
    return _lib_si_ws(int(seq_len))


def dp_score_index(x0_hat, x_final, d, row_stride, policy, ell_out, keep_out, idx_out, n_kept,
                   row_frame_src, row_frame_dst, workspace, dev_error=None, stream=None):
    """Score, mask and kept-index list in one launch; the workspace must be
    zero-filled before its first use (torch.zeros) and is reused as is."""
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib_score_index(_ptr(x0_hat), _ptr(x_final), d, int(row_stride), ctypes.byref(policy),
                            _ptr(ell_out), _ptr(keep_out), _ptr(idx_out), _ptr(n_kept),
                            _ptr(row_frame_src), _ptr(row_frame_dst), _ptr(workspace), ws_bytes,
                            _ptr(dev_error), _stream(stream)))


def dp_compact_index(keep, seq_len, idx_out, n_kept, row_frame_src, row_frame_dst, workspace,
                     stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib_compact(_ptr(keep), seq_len, _ptr(idx_out), _ptr(n_kept), _ptr(row_frame_src),
                        _ptr(row_frame_dst), _ptr(workspace), ws_bytes, _stream(stream)))


def dp_compact_index_noalloc(keep, seq_len, idx_out, n_kept, row_frame_src, row_frame_dst,
                             stream=None):
    """dp_compact_index with the library's static scratch of the current device
    (no workspace, nothing allocated)."""
    _check(_lib_compact_noalloc(_ptr(keep), int(seq_len), _ptr(idx_out), _ptr(n_kept),
                                _ptr(row_frame_src), _ptr(row_frame_dst), _stream(stream)))


def dp_rope_workspace_bytes(n_frames, n_pairs):
    return _lib_rope_ws(n_frames, n_pairs)


def dp_gather_kv(kv, idx, n_kept, row_frame=None, fused_rope=None, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib_gather(ctypes.byref(kv), _ptr(idx), _ptr(n_kept), _ptr(row_frame),
                       ctypes.byref(fused_rope) if fused_rope is not None else None,
                       _ptr(workspace), ws_bytes, _stream(stream)))


def dp_rope_reindex(k_layers, n_layers, n_heads, head_dim, dtype, rows_capacity, n_rows,
                    row_frame, rope, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib_reindex(_ptr(k_layers), n_layers, n_heads, head_dim, dtype, rows_capacity,
                        _ptr(n_rows), _ptr(row_frame), ctypes.byref(rope), _ptr(workspace),
                        ws_bytes, _stream(stream)))


def dp_rope_prepare(rope, head_dim, dtype, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib_rope_prepare(ctypes.byref(rope), head_dim, dtype, _ptr(workspace), ws_bytes,
                             _stream(stream)))


def dp_rope_apply(k_layers, n_layers, n_heads, head_dim, dtype, row_begin, rows_capacity, n_rows,
                  row_frame, rope, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib_rope_apply(_ptr(k_layers), n_layers, n_heads, head_dim, dtype, int(row_begin),
                           int(rows_capacity), _ptr(n_rows), _ptr(row_frame), ctypes.byref(rope),
                           _ptr(workspace), ws_bytes, _stream(stream)))


def dp_rope_shift_workspace_bytes(n_pairs):
    return _lib_rope_shift_ws(int(n_pairs))


def dp_rope_shift(k_layers, n_layers, n_heads, head_dim, dtype, row_begin, rows_capacity, n_rows,
                  theta, pair_begin, n_pairs, delta, workspace, stream=None,
                  key_layout=DP_KEY_INTERLEAVED):
    """k_layers: device int64 tensor of layer base pointers (ptr_array)."""
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib_rope_shift(_ptr(k_layers), n_layers, n_heads, head_dim, dtype, int(row_begin),
                           int(rows_capacity), _ptr(n_rows), _ptr(theta), pair_begin, n_pairs,
                           int(key_layout), float(delta), _ptr(workspace), ws_bytes,
                           _stream(stream)))


def dp_append_kept(kv, slot_begin, slot_rows, idx, n_kept, tail, row_frame=None, fused_rope=None,
                   workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib_append(ctypes.byref(kv), int(slot_begin), int(slot_rows), _ptr(idx), _ptr(n_kept),
                       _ptr(tail), _ptr(row_frame),
                       ctypes.byref(fused_rope) if fused_rope is not None else None,
                       _ptr(workspace), ws_bytes, _stream(stream)))


def dp_hs_offsets(head_class, n_layers, n_heads, class_len, n_classes, offsets, stream=None):
    _check(_lib_hs_offsets(_ptr(head_class), n_layers, n_heads, _ptr(class_len), n_classes,
                           _ptr(offsets), _stream(stream)))


def _cap_array(class_capacity):
    arr = (_i64 * len(class_capacity))(*[int(c) for c in class_capacity])
    return arr


def dp_hs_gather_kv(kv, head_class, n_classes, class_idx, class_len, class_capacity, offsets,
                    class_row_frame=None, fused_rope=None, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib_hs_gather(ctypes.byref(kv), _ptr(head_class), n_classes, _ptr(class_idx),
                          _ptr(class_len), _cap_array(class_capacity), _ptr(offsets),
                          _ptr(class_row_frame),
                          ctypes.byref(fused_rope) if fused_rope is not None else None,
                          _ptr(workspace), ws_bytes, _stream(stream)))


def dp_hs_rope_reindex(k_ragged, k_capacity, n_layers, n_heads, head_dim, dtype, head_class,
                       n_classes, class_len, class_capacity, offsets, class_row_frame, rope,
                       workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib_hs_reindex(_ptr(k_ragged), int(k_capacity), n_layers, n_heads, head_dim, dtype, _ptr(head_class),
                           n_classes, _ptr(class_len), _cap_array(class_capacity), _ptr(offsets),
                           _ptr(class_row_frame), ctypes.byref(rope), _ptr(workspace), ws_bytes,
                           _stream(stream)))


def dp_attention(q, k, v, o, n_q, kv_capacity, n_kv, n_heads, head_dim, dtype, scale,
                 stream=None, key_layout=DP_KEY_INTERLEAVED, pair_begin=0, n_pairs=0):
    _check(_lib_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(o), int(n_q), int(kv_capacity),
                          _ptr(n_kv), n_heads, head_dim, dtype, float(scale), int(key_layout),
                          int(pair_begin), int(n_pairs), _stream(stream)))


def dp_attention_lag(q, k, v, o, n_q, kv_capacity, n_kv, plain_begin, plain_end, theta,
                     pair_begin, n_pairs, lag, n_heads, head_dim, dtype, scale, stream=None,
                     key_layout=DP_KEY_INTERLEAVED):
    _check(_lib_attention_lag(_ptr(q), _ptr(k), _ptr(v), _ptr(o), int(n_q), int(kv_capacity),
                              _ptr(n_kv), int(plain_begin), int(plain_end), _ptr(theta),
                              int(pair_begin), int(n_pairs), float(lag), n_heads, head_dim, dtype,
                              float(scale), int(key_layout), _stream(stream)))


def dp_hs_attention(q, k_ragged, v_ragged, ragged_capacity, offsets, layer, k_chunk, v_chunk,
                    n_chunk, o, n_q, n_heads, head_dim, dtype, scale, stream=None,
                    key_layout=DP_KEY_INTERLEAVED, pair_begin=0, n_pairs=0):
    _check(_lib_hs_attention(_ptr(q), _ptr(k_ragged), _ptr(v_ragged), int(ragged_capacity),
                             _ptr(offsets), int(layer), _ptr(k_chunk), _ptr(v_chunk), int(n_chunk),
                             _ptr(o), int(n_q), n_heads, head_dim, dtype, float(scale),
                             int(key_layout), int(pair_begin), int(n_pairs), _stream(stream)))


def dp_hs_attention_lag(q, k_ragged, v_ragged, ragged_capacity, offsets, layer, k_chunk, v_chunk,
                        n_chunk, o, n_q, n_heads, head_dim, dtype, scale, plain_tail, theta,
                        pair_begin, n_pairs, lag, stream=None, key_layout=DP_KEY_INTERLEAVED):
    _check(_lib_hs_attention_lag(_ptr(q), _ptr(k_ragged), _ptr(v_ragged), int(ragged_capacity),
                                 _ptr(offsets), int(layer), _ptr(k_chunk), _ptr(v_chunk),
                                 int(n_chunk), _ptr(o), int(n_q), n_heads, head_dim, dtype,
                                 float(scale), int(plain_tail), _ptr(theta), int(pair_begin),
                                 int(n_pairs), float(lag), int(key_layout), _stream(stream)))


def dp_pr_add(counter, visible_positions, full_positions):
    _check(_lib_pr_add(ctypes.byref(counter), int(visible_positions), int(full_positions)))


def dp_pr_value(counter):
    return _lib_pr_value(ctypes.byref(counter))
