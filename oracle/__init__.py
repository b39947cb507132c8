"""CPU oracle of the DeCoPrune history-KV compaction path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It wraps the plain C
implementation in ``dp_oracle.c`` (numpy in, numpy out) and shares no code
with the HIP library.

Method source: the page "DeCoPrune이 디노이징 불일치로 비디오 KV 캐시를 85%
줄인다" (onedev.kr/papers/726), "the DeCoPrune page".  Each function names the
section it follows.  Every function here is pinned by a CPU test against a
closed form, an invariant, a library routine or brute force.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build(force=True)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.oracle_abi.restype = ctypes.c_int
        L.oracle_score_f32.argtypes = [P, P, i64, i32, i64, P]
        L.oracle_score_f64.argtypes = [P, P, i64, i32, i64, P]
        L.oracle_mask.argtypes = [P, i64, i64, i64, i64, i64, f32, i32, i32, P]
        L.oracle_compact.argtypes = [P, i64, P]
        L.oracle_compact.restype = i64
        L.oracle_gather.argtypes = [P, i64, i64, i64, P, i64, P, i64]
        L.oracle_gather_i32.argtypes = [P, P, i64, P]
        L.oracle_append_kept.argtypes = [P, i64, i64, i64, i64, i64, P, i64, i64, P]
        L.oracle_append_kept.restype = i64
        L.oracle_rope_frames.argtypes = [i32, P, P, f32, f32, f32, i32, P, P, P, P]
        L.oracle_rope_frames_compressed.argtypes = [i32, P, P, f32, f32, f32, i32, P, P, P, P]
        L.oracle_rope_rows.argtypes = [P, i32, i64, i32, i32, i32, i32, P, P, P, P]
        L.oracle_rope_uniform.argtypes = [i32, P, f32, P, P]
        L.oracle_rope_headrows.argtypes = [P, i32, i64, i32, i32, i32, P, P, P, P]
        L.oracle_hs_offsets.argtypes = [P, i32, i32, P, P]
        L.oracle_hs_gather_layer.argtypes = [P, i32, i32, i32, i32, P, P, P, P, P, P]
        L.oracle_attention.argtypes = [P, P, P, P, i64, i64, i32, i32, ctypes.c_double, P]
        L.oracle_attention_f64.argtypes = [P, P, P, P, i64, i64, i32, i32, ctypes.c_double, P]
        L.oracle_rope_rows_f64.argtypes = [P, i64, i32, i32, i32, i32, P, P, P]
        L.oracle_pr.argtypes = [i64, i64]
        L.oracle_pr.restype = ctypes.c_double
        _lib = L
    return _lib


def _p(a):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# Score [DeCoPrune page, 어떻게 동작하나]
# --------------------------------------------------------------------------
def score_f32(x0_hat, x_final, d=None):
    """l_i = (1/d)||x0_hat_i - x_final_i||^2 in fp32, fixed pairwise order."""
    a = _c(x0_hat, np.float32)
    b = _c(x_final, np.float32)
    assert a.shape == b.shape and a.ndim == 2
    n, stride = a.shape
    d = stride if d is None else d
    assert 1 <= d <= min(stride, 1024)
    out = np.empty(n, np.float32)
    lib().oracle_score_f32(_p(a), _p(b), n, d, stride, _p(out))
    return out


def score_f64(x0_hat, x_final, d=None):
    """Same quantity, fp64, left-to-right sum."""
    a = _c(x0_hat, np.float32)
    b = _c(x_final, np.float32)
    n, stride = a.shape
    d = stride if d is None else d
    out = np.empty(n, np.float64)
    lib().oracle_score_f64(_p(a), _p(b), n, d, stride, _p(out))
    return out


# --------------------------------------------------------------------------
# Mask [DeCoPrune page, 어떻게 동작하나; reversed: 전제와 한계]
# --------------------------------------------------------------------------
def mask(ell, seq_len, sink_len, window_len, scored_begin, n_scored, gamma,
         reversed=False, streaming=False):
    assert 0 <= sink_len <= scored_begin
    assert scored_begin + n_scored <= seq_len - window_len
    e = _c(ell if ell is not None else np.zeros(0, np.float32), np.float32)
    assert e.shape[0] >= (0 if streaming else n_scored)
    if e.shape[0] == 0:
        e = np.zeros(1, np.float32)
    keep = np.empty(seq_len, np.uint8)
    lib().oracle_mask(_p(e), seq_len, sink_len, window_len, scored_begin, n_scored,
                      np.float32(gamma), int(bool(reversed)), int(bool(streaming)), _p(keep))
    return keep


def compact(keep):
    k = _c(keep, np.uint8)
    idx = np.empty(max(1, k.shape[0]), np.int32)
    n = lib().oracle_compact(_p(k), k.shape[0], _p(idx))
    return idx[:n].copy()


# --------------------------------------------------------------------------
# Gather [DeCoPrune page, 어떻게 동작하나]
# --------------------------------------------------------------------------
def gather(src, idx):
    """src: [L, rows, ...] any dtype -> [L, len(idx), ...] bit copy of rows idx."""
    s = np.ascontiguousarray(src)
    idx = _c(idx, np.int32)
    L, rows = s.shape[0], s.shape[1]
    row_bytes = int(np.prod(s.shape[2:], dtype=np.int64)) * s.itemsize
    assert idx.size == 0 or (idx.min() >= 0 and idx.max() < rows)
    out = np.empty((L, idx.shape[0]) + s.shape[2:], s.dtype)
    if idx.shape[0]:
        lib().oracle_gather(_p(s), L, rows, row_bytes, _p(idx), idx.shape[0], _p(out),
                            idx.shape[0])
    return out


def gather_i32(src, idx):
    s = _c(src, np.int32)
    idx = _c(idx, np.int32)
    out = np.empty(idx.shape[0], np.int32)
    if idx.shape[0]:
        lib().oracle_gather_i32(_p(s), _p(idx), idx.shape[0], _p(out))
    return out


def append_kept(buf, slot_begin, slot_rows, idx, tail, row_frame=None):
    """In place on buf [L, capacity, ...]: append the kept rows idx (slot-relative)
    of the slot at the tail; returns the new tail (-1: refused, unchanged)."""
    assert buf.flags.c_contiguous
    idx = _c(idx, np.int32)
    assert idx.size == 0 or (idx.min() >= 0 and idx.max() < slot_rows)
    L, cap = buf.shape[0], buf.shape[1]
    row_bytes = int(np.prod(buf.shape[2:], dtype=np.int64)) * buf.itemsize
    if row_frame is not None:
        assert row_frame.dtype == np.int32 and row_frame.flags.c_contiguous
    rf = _p(row_frame) if row_frame is not None else None
    return lib().oracle_append_kept(_p(buf), L, cap, row_bytes, slot_begin, slot_rows,
                                    _p(idx) if idx.size else None, idx.shape[0], tail, rf)


# --------------------------------------------------------------------------
# RoPE re-index [DeCoPrune page, 무엇과 다른가]
# --------------------------------------------------------------------------
def rope_frames(frame_t, frame_phase, q0, knee, inv_factor, theta, compressed=False):
    """Per-frame delta and cos/sin tables; returns (delta, cos, sin, new_phase).
    compressed: the phase a key past the knee takes is t/c (the compressed
    time axis) instead of t~."""
    ft = _c(frame_t, np.float32)
    ph = _c(frame_phase, np.float32).copy()
    th = _c(theta, np.float32)
    nf, npairs = ft.shape[0], th.shape[0]
    delta = np.empty(nf, np.float32)
    c = np.empty((nf, npairs), np.float32)
    s = np.empty((nf, npairs), np.float32)
    fn = lib().oracle_rope_frames_compressed if compressed else lib().oracle_rope_frames
    fn(nf, _p(ft), _p(ph), np.float32(q0), np.float32(knee), np.float32(inv_factor), npairs,
       _p(th), _p(delta), _p(c), _p(s))
    return delta, c, s, ph


def rope_uniform(theta, delta):
    """Tables of one uniform phase step delta for every row (frame 0 of a
    one-frame table); use with rope_rows and row_frame all 0."""
    th = _c(theta, np.float32)
    n = th.shape[0]
    c = np.empty((1, n), np.float32)
    s = np.empty((1, n), np.float32)
    lib().oracle_rope_uniform(n, _p(th), np.float32(delta), _p(c), _p(s))
    return np.array([delta], np.float32), c, s, None


def _dtype_code(a):
    if a.dtype == np.float32:
        return 0
    if a.dtype == np.uint16:  # bf16 bit patterns
        return 1
    raise TypeError("keys must be float32 or uint16 (bf16 bits)")


def rope_rows(k, row_frame, pair_begin, tables):
    """In-place re-index of k: [rows, H, D] float32 or uint16 (bf16 bits)."""
    assert k.flags.c_contiguous and k.ndim == 3
    delta, c, s, _ = tables
    rf = _c(row_frame, np.int32)
    assert rf.shape[0] >= k.shape[0]
    npairs = c.shape[1]
    assert 2 * (pair_begin + npairs) <= k.shape[2]
    lib().oracle_rope_rows(_p(k), _dtype_code(k), k.shape[0], k.shape[1], k.shape[2],
                           pair_begin, npairs, _p(rf), _p(delta), _p(c), _p(s))
    return k


def rope_headrows(k, row_frame, pair_begin, tables):
    """In-place re-index of per-head rows k: [rows, D]."""
    assert k.flags.c_contiguous and k.ndim == 2
    delta, c, s, _ = tables
    rf = _c(row_frame, np.int32)
    npairs = c.shape[1]
    lib().oracle_rope_headrows(_p(k), _dtype_code(k), k.shape[0], k.shape[1], pair_begin,
                               npairs, _p(rf), _p(delta), _p(c), _p(s))
    return k


# --------------------------------------------------------------------------
# DeCoPrune-HS [DeCoPrune page, 무엇과 다른가]
# --------------------------------------------------------------------------
def hs_offsets(head_class, class_len):
    hc = _c(head_class, np.uint8)
    L, H = hc.shape
    cl = _c(class_len, np.int64)
    off = np.empty(L * H + 1, np.int64)
    lib().oracle_hs_offsets(_p(hc), L, H, _p(cl), _p(off))
    return off


def hs_gather_layer(src_layer, layer, head_class, class_lists, offsets, out):
    """Gather one layer's heads into the packed per-head buffer ``out``
    ([total head rows, D]); src_layer: [rows, H, D]."""
    s = np.ascontiguousarray(src_layer)
    hc = _c(head_class, np.uint8)
    L, H = hc.shape
    lens = np.array([len(x) for x in class_lists], np.int64)
    base = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    cat = _c(np.concatenate([np.asarray(x, np.int32) for x in class_lists] + [np.zeros(1, np.int32)]),
             np.int32)
    off = _c(offsets, np.int64)
    assert out.flags.c_contiguous and out.dtype == s.dtype
    lib().oracle_hs_gather_layer(_p(s), layer, H, s.shape[2], s.itemsize, _p(hc), _p(cat),
                                 _p(base), _p(lens), _p(off), _p(out))
    return out


def attention(q, k, v, rows, n_kv=None, scale=None):
    """Attention of the listed query rows over keys [0, n_kv) (float64 result
    [len(rows), H, D]); q, k, v: [rows, H, D] bf16 bit patterns (uint16)."""
    q, k, v = (np.ascontiguousarray(x) for x in (q, k, v))
    if q.dtype == np.float64 or k.dtype == np.float64 or v.dtype == np.float64:
        return _attention_f64(q, k, v, rows, n_kv, scale)
    assert q.dtype == k.dtype == v.dtype == np.uint16
    H, D = q.shape[1], q.shape[2]
    n_kv = k.shape[0] if n_kv is None else n_kv
    assert 1 <= n_kv <= k.shape[0] and v.shape[0] >= n_kv
    rows = _c(rows, np.int64)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < q.shape[0])
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.empty((rows.shape[0], H, D), np.float64)
    lib().oracle_attention(_p(q), _p(k), _p(v), _p(rows), rows.shape[0], n_kv, H, D, scale, _p(out))
    return out


def _f64(a):
    """float64 values of bf16 bit patterns (uint16) or of a float array."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _attention_f64(q, k, v, rows, n_kv, scale):
    """attention() over float64 values (bf16 inputs are widened exactly)."""
    q, k, v = (np.ascontiguousarray(_f64(x)) for x in (q, k, v))
    H, D = q.shape[1], q.shape[2]
    n_kv = k.shape[0] if n_kv is None else n_kv
    assert 1 <= n_kv <= k.shape[0] and v.shape[0] >= n_kv
    rows = _c(rows, np.int64)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.empty((rows.shape[0], H, D), np.float64)
    lib().oracle_attention_f64(_p(q), _p(k), _p(v), _p(rows), rows.shape[0], n_kv, H, D, scale,
                               _p(out))
    return out


def rope_rows_f64(k, row_frame, pair_begin, step, theta):
    """Exact float64 re-index of k [rows, H, D] (float64, in place): pair j of
    row r rotated by theta_j * step[row_frame[r]]."""
    assert k.dtype == np.float64 and k.flags.c_contiguous and k.ndim == 3
    rf = _c(row_frame, np.int32)
    st = _c(step, np.float64)
    th = _c(theta, np.float64)
    assert 2 * (pair_begin + th.shape[0]) <= k.shape[2]
    lib().oracle_rope_rows_f64(_p(k), k.shape[0], k.shape[1], k.shape[2], pair_begin,
                               th.shape[0], _p(rf), _p(st), _p(th))
    return k


def hs_attention(q, k_ragged, v_ragged, offsets, layer, rows, k_chunk=None, v_chunk=None,
                 scale=None):
    """Attention over the ragged DeCoPrune-HS cache [DeCoPrune page, 무엇인가
    (DeCoPrune-HS)]: head h of ``layer`` attends to its own run
    k_ragged[offsets[layer*H + h] : offsets[layer*H + h + 1]] ([head rows, D])
    followed by the dense chunk rows k_chunk[:, h] ([n_chunk, H, D], optional).
    Evaluated head by head with ``attention``; a head with no rows gives zeros.
    Returns float64 [len(rows), H, D]."""
    q = np.ascontiguousarray(q)
    H, D = q.shape[1], q.shape[2]
    off = np.asarray(offsets, np.int64)
    rows = np.asarray(rows, np.int64)
    out = np.zeros((rows.shape[0], H, D), np.float64)
    for h in range(H):
        lo, hi = int(off[layer * H + h]), int(off[layer * H + h + 1])
        kh, vh = k_ragged[lo:hi], v_ragged[lo:hi]
        if k_chunk is not None:
            kh = np.concatenate([kh, k_chunk[:, h]])
            vh = np.concatenate([vh, v_chunk[:, h]])
        if kh.shape[0] == 0:
            continue
        out[:, h] = attention(np.ascontiguousarray(q[:, h:h + 1]), kh[:, None], vh[:, None],
                              rows, scale=scale)[:, 0]
    return out


def pr(visible, full):
    """Pruning ratio 1 - visible/full [DeCoPrune page, 어떻게 쓰나]."""
    return lib().oracle_pr(int(visible), int(full))


# --------------------------------------------------------------------------
# One whole prune step, step by step in the page's order
# --------------------------------------------------------------------------
def prune_step(x0_hat, x_final, d, policy, k, v, row_frame=None, rope=None,
               pair_begin=0):
    """k, v: [L, T, H, D] (float32 or uint16 bf16 bits); policy: dict with
    seq_len, sink_len, window_len, scored_begin, n_scored, gamma, reversed,
    streaming.  rope: None or dict theta, frame_t, frame_phase, q0, knee,
    inv_factor.  Returns dict ell, keep, idx, k, v, row_frame, tables."""
    streaming = bool(policy.get("streaming", False))
    ell = None
    if not streaming and policy["n_scored"] > 0:
        ell = score_f32(np.asarray(x0_hat)[:, :d], np.asarray(x_final)[:, :d], d)
    keep = mask(ell, policy["seq_len"], policy["sink_len"], policy["window_len"],
                policy["scored_begin"], policy["n_scored"], policy["gamma"],
                policy.get("reversed", False), streaming)
    idx = compact(keep)
    k2 = gather(k, idx)
    v2 = gather(v, idx) if v is not None else None
    rf2 = gather_i32(row_frame, idx) if row_frame is not None else None
    tables = None
    if rope is not None:
        tables = rope_frames(rope["frame_t"], rope["frame_phase"], rope["q0"], rope["knee"],
                             rope["inv_factor"], rope["theta"])
        for l in range(k2.shape[0]):
            rope_rows(k2[l], rf2, pair_begin, tables)
    return dict(ell=ell, keep=keep, idx=idx, k=k2, v=v2, row_frame=rf2, tables=tables)
