"""Seeded synthetic inputs for the DeCoPrune compaction path.

This module generates inputs only: workload shapes, score inputs, key/value
caches, RoPE frequency tables, frame tables and head splits.  It holds none of
the method's arithmetic (no score, mask, index, gather or rotation), so both
the HIP library's tests and the CPU oracle may draw from it.

Workloads (their sizes follow the setup the DeCoPrune page reports: 832x480
video, 4 latent frames per chunk, 1560 = 52x30 tokens per latent frame,
gamma = 0.10 [DeCoPrune page, 전제와 한계]):

  tiny      1 layer, 2 heads, head_dim 64, fp32; 8 chunks of 64 tokens
            (one latent frame per chunk); d = 16; sink chunk 0, window 2
            chunks, chunks 1..5 scored.
  eviction  40 layers x 40 heads x 128, bf16; sink + the chunk leaving the
            window + a 3-chunk window (5 x 6240 tokens); d = 64.
  reindex   keys only, 40 x 40 x 128 bf16; retained cache of a 60-chunk
            (240-frame) history: sink, 15% of the 56 prunable chunks, window.
  prefix    58-chunk observed prefix (361,920 tokens), all 57 non-sink chunks
            scored, no window; per-chunk mean noise level varies.
  hs        30-chunk history (187,200 tokens); per layer a seeded half of the
            heads are static (sink + 3-chunk window), the rest use the mask.

Key/value elements are drawn from a counter-based generator so that any
element can be recomputed on the host: element ``key`` of stream ``s`` takes
entry ``z >> 48`` of a 65,536-entry table of standard-normal quantiles
Phi^-1((j + 1/2) / 65536), where ``z`` is the SplitMix64 output function
(Steele, Lea and Flood, 2014) applied to a seeded Weyl sequence.
"""
import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
MIX1 = np.uint64(0xBF58476D1CE4E5B9)
MIX2 = np.uint64(0x94D049BB133111EB)
STREAM_MUL = np.uint64(0xD1B54A32D192ED03)

STREAM_K = 1
STREAM_V = 2

TOKENS_PER_FRAME = 1560          # 52 x 30 latent tokens at 832x480
FRAMES_PER_CHUNK = 4
CHUNK_TOKENS = TOKENS_PER_FRAME * FRAMES_PER_CHUNK   # 6240


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    n_heads: int
    head_dim: int
    dtype: str                 # "f32" or "bf16"
    n_chunks: int
    tokens_per_frame: int
    frames_per_chunk: int
    sink_chunks: int
    window_chunks: int
    scored_chunks: Tuple[int, int]   # [first, last] chunk indices scored (inclusive); (0,-1) = none
    d: int = 64
    gamma: float = 0.10
    sigma: Tuple[float, float] = (0.05, 0.44)   # log-uniform range of the per-token noise level
    sigma_per_chunk: bool = False              # prefix: per-chunk mean level, per-token jitter
    rope_pairs: int = 44
    rope_base: float = 10000.0
    rope_knee: float = 12.0
    rope_factor: float = 8.0
    rope_q0: Optional[float] = None            # None: first frame of the next chunk
    seed: int = 0

    @property
    def chunk_tokens(self):
        return self.tokens_per_frame * self.frames_per_chunk

    @property
    def seq_len(self):
        return self.n_chunks * self.chunk_tokens

    @property
    def sink_len(self):
        return self.sink_chunks * self.chunk_tokens

    @property
    def window_len(self):
        return self.window_chunks * self.chunk_tokens

    @property
    def scored_begin(self):
        a, b = self.scored_chunks
        return a * self.chunk_tokens if b >= a else self.sink_len

    @property
    def n_scored(self):
        a, b = self.scored_chunks
        return (b - a + 1) * self.chunk_tokens if b >= a else 0

    @property
    def n_frames(self):
        return self.n_chunks * self.frames_per_chunk

    @property
    def q0(self):
        return float(self.n_frames) if self.rope_q0 is None else float(self.rope_q0)

    @property
    def row_elems(self):
        return self.n_heads * self.head_dim

    @property
    def elem_size(self):
        return 4 if self.dtype == "f32" else 2


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, "f32", 8, 64, 1, 1, 2, (1, 5), d=16,
                     sigma=(0.05, 1.0), rope_pairs=8, rope_knee=2.0, rope_factor=4.0),
    "eviction": Workload("eviction", 40, 40, 128, "bf16", 5, TOKENS_PER_FRAME,
                         FRAMES_PER_CHUNK, 1, 3, (1, 1)),
    "reindex": Workload("reindex", 40, 40, 128, "bf16", 60, TOKENS_PER_FRAME,
                        FRAMES_PER_CHUNK, 1, 3, (1, 56)),
    "prefix": Workload("prefix", 40, 40, 128, "bf16", 58, TOKENS_PER_FRAME,
                       FRAMES_PER_CHUNK, 1, 0, (1, 57), sigma=(0.05, 0.42),
                       sigma_per_chunk=True),
    "hs": Workload("hs", 40, 40, 128, "bf16", 30, TOKENS_PER_FRAME, FRAMES_PER_CHUNK,
                   1, 3, (1, 26)),
}


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(w, **changes)


# --------------------------------------------------------------------------
# Score inputs: x_final ~ N(0,1), x0_hat = x_final + sigma_i * N(0,1)
# --------------------------------------------------------------------------
def score_inputs(w: Workload, seed: Optional[int] = None):
    """Returns (x0_hat, x_final) fp32 [n_scored, d] for the scored rows."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    n, d = w.n_scored, w.d
    x_final = rng.standard_normal((n, d))
    lo, hi = np.log(w.sigma[0]), np.log(w.sigma[1])
    if w.sigma_per_chunk:
        n_ch = n // w.chunk_tokens
        chunk_sigma = np.exp(rng.uniform(lo, hi, size=n_ch))
        sig = np.repeat(chunk_sigma, w.chunk_tokens) * np.exp(0.35 * rng.standard_normal(n))
    else:
        sig = np.exp(rng.uniform(lo, hi, size=n))
    x0_hat = x_final + sig[:, None] * rng.standard_normal((n, d))
    return x0_hat.astype(np.float32), x_final.astype(np.float32)


# --------------------------------------------------------------------------
# RoPE inputs: frequencies of the temporal block, frame tables
# --------------------------------------------------------------------------
def rope_theta(n_pairs: int, base: float = 10000.0) -> np.ndarray:
    """theta_j = base^(-j/n_pairs), j < n_pairs, rounded to fp32 (the model's
    own temporal-axis frequencies; an input of the re-index)."""
    j = np.arange(n_pairs, dtype=np.float64)
    return (base ** (-j / n_pairs)).astype(np.float32)


def frame_tables(w: Workload):
    """(frame_t, frame_phase): original frame index t of each frame and the
    phase the stored keys carry (freshly written keys carry p = t)."""
    t = np.arange(w.n_frames, dtype=np.float32)
    return t, t.copy()


def row_frame(w: Workload) -> np.ndarray:
    return (np.arange(w.seq_len, dtype=np.int64) // w.tokens_per_frame).astype(np.int32)


def retained_keep(w: Workload, rate: float = 0.15, seed: Optional[int] = None) -> np.ndarray:
    """Keep flags of a retained cache: sink and window kept, every prunable row
    kept with probability ``rate`` (Bernoulli, seeded)."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 7)
    keep = (rng.random(w.seq_len) < rate).astype(np.uint8)
    keep[: w.sink_len] = 1
    if w.window_len:
        keep[w.seq_len - w.window_len:] = 1
    return keep


def ring_layout(w: Workload, rate: float = 0.15):
    """Rows of one layer of the ring-layout cache at q0, when the next chunk
    (index n_chunks) attends: [sink | slots: the window chunks and the next
    chunk | history: the retained rows of the prunable chunks], the retained
    rows as retained_keep() draws them.  Returns (row_frame int32 [rows],
    slot_begin, slot_end); a row's frame is its token index // tokens_per_frame."""
    C = w.chunk_tokens
    keep = retained_keep(w, rate)
    first, last = w.scored_chunks
    hist = np.flatnonzero(keep[first * C:(last + 1) * C]) + first * C
    slots = np.arange((last + 1) * C, (w.n_chunks + 1) * C)
    rows = np.concatenate([np.arange(w.sink_len), slots, hist])
    return (rows // w.tokens_per_frame).astype(np.int32), w.sink_len, w.sink_len + slots.size


def hs_head_class(w: Workload, static_fraction: float = 0.5, seed: Optional[int] = None):
    """[L, H] uint8: 0 = static head, 1 = dynamic head; per layer a seeded
    permutation, the first H*static_fraction heads are static."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 11)
    n_static = int(round(w.n_heads * static_fraction))
    cls = np.ones((w.n_layers, w.n_heads), np.uint8)
    for l in range(w.n_layers):
        perm = rng.permutation(w.n_heads)
        cls[l, perm[:n_static]] = 0
    return cls


# --------------------------------------------------------------------------
# Key/value caches
# --------------------------------------------------------------------------
_tables = {}


def kv_table(dtype: str) -> np.ndarray:
    """65,536 standard-normal quantiles as fp32 (uint32 bits) or bf16 (uint16 bits)."""
    if dtype not in _tables:
        from scipy.special import ndtri
        q = ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0).astype(np.float32)
        if dtype == "f32":
            _tables[dtype] = q.view(np.uint32).copy()
        else:
            import torch
            _tables[dtype] = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy() \
                .view(np.uint16).copy()
    return _tables[dtype]


def stream_key(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        return np.uint64(seed) * GOLDEN ^ np.uint64(stream + 1) * STREAM_MUL


def _splitmix(keys: np.ndarray, skey: np.uint64) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = skey + (keys + np.uint64(1)) * GOLDEN
        z = (z ^ (z >> np.uint64(30))) * MIX1
        z = (z ^ (z >> np.uint64(27))) * MIX2
        z = z ^ (z >> np.uint64(31))
    return z


def kv_rows_host(dtype: str, seed: int, stream: int, layer: int, rows, src_rows: int,
                 row_elems: int, cols=None) -> np.ndarray:
    """Host twin of the device fill: the elements of ``rows`` of one layer,
    [len(rows), row_elems] as uint16 (bf16 bits) or float32; with ``cols``
    only those element columns, [len(rows), len(cols)]."""
    rows = np.asarray(rows, np.uint64)
    cols = np.arange(row_elems, dtype=np.uint64) if cols is None else np.asarray(cols, np.uint64)
    keys = ((np.uint64(layer) * np.uint64(src_rows) + rows[:, None]) * np.uint64(row_elems)
            + cols[None, :])
    z = _splitmix(keys, stream_key(seed, stream))
    out = kv_table(dtype)[(z >> np.uint64(48)).astype(np.int64)]
    return out.view(np.float32) if dtype == "f32" else out


def kv_layer_host(dtype, seed, stream, layer, src_rows, row_elems):
    return kv_rows_host(dtype, seed, stream, layer, np.arange(src_rows), src_rows, row_elems)


_fill_lib = None
_dev_tables = {}


def _fill():
    global _fill_lib
    if _fill_lib is None:
        from . import build as _b
        path = _b.LIB
        if not os.path.exists(path):
            raise RuntimeError("libdpsynth.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        L.dpsynth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                   ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_void_p]
        L.dpsynth_fill.restype = ctypes.c_int
        L.dpsynth_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.dpsynth_copy.restype = ctypes.c_int
        _fill_lib = L
    return _fill_lib


def kv_fill_device(tensor, dtype: str, seed: int, stream: int, layer: int, src_rows: int,
                   row_elems: int):
    """Fill a device tensor holding one layer [src_rows, row_elems] with the
    same elements kv_rows_host() gives."""
    import torch
    assert tensor.is_cuda and tensor.is_contiguous()
    assert tensor.numel() == src_rows * row_elems
    assert tensor.element_size() == (4 if dtype == "f32" else 2)
    dev = tensor.device
    key = (dtype, dev.index)
    if key not in _dev_tables:
        t = kv_table(dtype)
        _dev_tables[key] = torch.from_numpy(t.view(np.int32) if dtype == "f32" else t.view(np.int16)).to(dev)
    tab = _dev_tables[key]
    key_base = int(layer) * int(src_rows) * int(row_elems)
    st = torch.cuda.current_stream(dev).cuda_stream
    rc = _fill().dpsynth_fill(ctypes.c_void_p(tensor.data_ptr()), 0 if dtype == "f32" else 1,
                              ctypes.c_uint64(int(stream_key(seed, stream))),
                              ctypes.c_uint64(key_base), tensor.numel(),
                              ctypes.c_void_p(tab.data_ptr()), ctypes.c_void_p(st))
    if rc != 0:
        raise RuntimeError("dpsynth_fill failed (%d)" % rc)
    return tensor


def device_copy(dst, src):
    """Plain 16-byte-vector copy of a contiguous device tensor (bandwidth and
    counter reference; not part of the method)."""
    import torch
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == nbytes and nbytes % 16 == 0
    st = torch.cuda.current_stream(src.device).cuda_stream
    rc = _fill().dpsynth_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()),
                              nbytes // 16, ctypes.c_void_p(st))
    if rc != 0:
        raise RuntimeError("dpsynth_copy failed (%d)" % rc)
