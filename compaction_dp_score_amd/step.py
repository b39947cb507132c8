"""One DeCoPrune prune step over the C ABI, with its buffers held on the GPU.

``PruneStep`` owns the device buffers a step needs (keep mask, kept-index
list, kept count, gathered row frames, workspaces) and enqueues, on the
current stream:

  dp_score_index -> dp_gather_kv (K re-rotated in the same pass when a RoPE
  re-index is configured)

which is the chunk-eviction update of the DeCoPrune page (section 어떻게
동작하나: score, threshold mask shared by all layers, physical gather) with
the temporal re-index of section 무엇과 다른가.  With fused=False the first
call is split into dp_score_mask -> dp_compact_index (the same results in
more launches).  Nothing here computes; it allocates once and marshals
arguments.
"""
import torch

from . import (DP_AXIS_COMPRESSED, DP_MODE_SCORE, dp_append_kept, dp_kv_inplace, dp_compact_index,
               dp_compact_workspace_bytes, dp_gather_kv, dp_kv, dp_rope_apply, dp_rope_prepare,
               dp_rope_workspace_bytes, dp_score_index, dp_score_index_workspace_bytes,
               dp_score_mask, dtype_code, make_policy, make_rope, ptr_array)


class PruneStep:
    def __init__(self, *, k_src, v_src, k_dst, v_dst, seq_len, sink_len, window_len,
                 scored_begin, n_scored, gamma, d, row_frame=None, rope=None,
                 reversed=False, mode=DP_MODE_SCORE, keep_ell=False, fused=True):
        """k_src/v_src/k_dst/v_dst: lists of per-layer device tensors
        [rows, heads, head_dim]; v_* may be None.  rope: None or a dict with
        theta, frame_t, frame_phase (device tensors), q0, knee, inv_factor,
        and optionally pair_begin and key_layout (dp_key_layout of the keys)."""
        dev = k_src[0].device
        self.device = dev
        self.seq_len = seq_len
        self.d = d
        self.n_layers = len(k_src)
        rows, heads, hd = k_src[0].shape
        self._keep_alive = []
        self.policy = make_policy(seq_len, sink_len, window_len, scored_begin, n_scored, gamma,
                                  reversed, mode)
        self.keep = torch.empty(seq_len, dtype=torch.uint8, device=dev)
        self.ell = torch.empty(max(1, n_scored), dtype=torch.float32, device=dev) if keep_ell else None
        self.idx = torch.empty(max(1, seq_len), dtype=torch.int32, device=dev)
        self.n_kept = torch.zeros(1, dtype=torch.int64, device=dev)
        self.dev_error = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ws_compact = torch.empty(dp_compact_workspace_bytes(seq_len) // 4 + 1,
                                      dtype=torch.int32, device=dev)
        self.fused = fused
        # zero-filled once; every dp_score_index call leaves it ready for the next
        self.ws_index = torch.zeros(dp_score_index_workspace_bytes(seq_len) // 8 + 1,
                                    dtype=torch.int64, device=dev)
        self.row_frame_src = row_frame
        self.row_frame_dst = (torch.empty(max(1, seq_len), dtype=torch.int32, device=dev)
                              if row_frame is not None else None)
        kv = dp_kv()
        arrs = [ptr_array(k_src, dev), ptr_array(v_src, dev), ptr_array(k_dst, dev),
                ptr_array(v_dst, dev)]
        self._keep_alive += arrs
        kv.k_src, kv.v_src, kv.k_dst, kv.v_dst = [a.data_ptr() if a is not None else None
                                                  for a in arrs]
        kv.n_layers, kv.n_heads, kv.head_dim = self.n_layers, heads, hd
        kv.dtype = dtype_code(k_src[0])
        kv.src_rows = rows
        kv.dst_capacity = k_dst[0].shape[0]
        kv.dev_error = self.dev_error.data_ptr()
        self.kv = kv
        self.rope = None
        self.ws_rope = None
        if rope is not None:
            self._keep_alive += [rope["theta"], rope["frame_t"], rope["frame_phase"]]
            self.rope = make_rope(rope["theta"], rope["frame_t"], rope["frame_phase"],
                                  rope["q0"], rope["knee"], rope["inv_factor"],
                                  rope.get("pair_begin", 0),
                                  key_layout=rope.get("key_layout", 0))
            nb = dp_rope_workspace_bytes(self.rope.n_frames, self.rope.n_pairs)
            self.ws_rope = torch.empty((nb + 15) // 16 * 4, dtype=torch.float32, device=dev)

    def run(self, x0_hat, x_final, row_stride=None, stream=None):
        """Enqueue score -> index -> gather (+ re-index) on the current stream."""
        stride = self.d if row_stride is None else row_stride
        if not self.fused:
            dp_score_mask(x0_hat, x_final, self.d, stride, self.policy, self.ell, self.keep, stream)
            self.run_from_keep(stream)
            return
        dp_score_index(x0_hat, x_final, self.d, stride, self.policy, self.ell, self.keep, self.idx,
                       self.n_kept, self.row_frame_src, self.row_frame_dst, self.ws_index,
                       self.dev_error, stream)
        self.gather(stream)

    def run_from_keep(self, stream=None):
        """Index and gather from a keep mask already in self.keep."""
        dp_compact_index(self.keep, self.seq_len, self.idx, self.n_kept, self.row_frame_src,
                         self.row_frame_dst, self.ws_compact, stream)
        self.gather(stream)

    def gather(self, stream=None):
        dp_gather_kv(self.kv, self.idx, self.n_kept,
                     self.row_frame_dst if self.rope is not None else None,
                     self.rope, self.ws_rope, stream)


class RingStep:
    """The eviction step in the ring layout, in place (segment append).

    Per layer one buffer ``[sink | ring of R chunk slots | history]`` of
    ``capacity`` rows (``k_layers``/``v_layers``: lists of per-layer device
    tensors [capacity, heads, head_dim]), one device int32 row-frame table
    shared by the layers (-1 marks a row with no key), and a device tail (the
    end of the history).  ``evict(slot, x0_hat, x_final, q0)`` enqueues, on the
    current stream, the DeCoPrune page's update when the chunk in ring slot
    ``slot`` leaves the window (section 어떻게 동작하나): its score, mask and
    kept-index list in one launch (dp_score_index), the append of its kept rows
    at the history tail for every layer (dp_append_kept, which retires the
    slot), and the re-index of section 무엇과 다른가 for the new query origin
    ``q0``:

      page axis        dp_rope_prepare, then dp_rope_apply over the sink and
                       over the history [history_begin, tail) (the appended
                       rows included);
      compressed axis  dp_rope_prepare, dp_rope_apply over the sink (its
                       frames move from t to t/c once, when they pass the
                       knee; rows whose frame does not move are neither read
                       nor written), and the leaving chunk's one re-index
                       fused into the append; no history key is rewritten
                       (the attention turns its query back by the common lag,
                       dp_attention_lag).

    The window slots are never re-indexed, which is right only while every
    frame of the window lies within the knee: with F frames per chunk and
    n_slots - 1 window chunks after an eviction, the knee must be at least
    (n_slots - 1) F.  On the compressed axis the leaving chunk must also be
    wholly past the knee when it is appended (knee < (n_slots - 1) F + 1),
    since no history key is visited afterwards.  The constructor checks both.

    The model then writes the next chunk's K and V into the freed slot and
    calls ``write_chunk(slot, frames)`` with the rows' frames.  Nothing here
    computes; it allocates once and marshals arguments, so ``evict`` can be
    captured into a HIP graph and replayed (the model restores or advances
    the tail, the slot's frames and the phase table between replays).
    """

    def __init__(self, *, k_layers, v_layers, sink_len, chunk_rows, n_slots, frames_per_chunk,
                 row_frame, tail, d, gamma, rope, axis=0):
        """row_frame: device int32 [capacity]; tail: device int64 [1] (the end
        of the visible rows); frames_per_chunk: latent frames of one chunk;
        rope: dict with theta, frame_t, frame_phase (device tensors), knee,
        inv_factor and optionally pair_begin and key_layout (q0 is given per
        eviction); axis: DP_AXIS_PAGE or DP_AXIS_COMPRESSED."""
        span = (n_slots - 1) * frames_per_chunk          # frames of the window after an eviction
        knee = float(rope["knee"])
        if knee < span:
            raise ValueError("RingStep: knee %g < window span %d frames: window keys would keep "
                             "their phase past the knee" % (knee, span))
        if axis == DP_AXIS_COMPRESSED and knee >= span + 1:
            raise ValueError("RingStep: on the compressed axis the knee (%g) must lie below %d "
                             "frames, so that the leaving chunk is past it when appended"
                             % (knee, span + 1))
        dev = k_layers[0].device
        cap, heads, hd = k_layers[0].shape
        self.capacity, self.heads, self.head_dim = cap, heads, hd
        self.n_layers = len(k_layers)
        self.dtype = dtype_code(k_layers[0])
        self.sink_len, self.chunk_rows, self.n_slots = sink_len, chunk_rows, n_slots
        self.history_begin = sink_len + n_slots * chunk_rows
        self.row_frame, self.tail, self.d, self.axis = row_frame, tail, d, axis
        self.rope_args = dict(rope)
        self.policy = make_policy(chunk_rows, 0, 0, 0, chunk_rows, gamma)
        self.keep = torch.empty(chunk_rows, dtype=torch.uint8, device=dev)
        self.idx = torch.empty(chunk_rows, dtype=torch.int32, device=dev)
        self.n_kept = torch.zeros(1, dtype=torch.int64, device=dev)
        self.dev_error = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ws_index = torch.zeros(dp_score_index_workspace_bytes(chunk_rows) // 8 + 1,
                                    dtype=torch.int64, device=dev)
        n_frames = rope["frame_t"].shape[0]
        n_pairs = rope["theta"].shape[0]
        nb = dp_rope_workspace_bytes(n_frames, n_pairs)
        self.ws_rope = torch.empty((nb + 15) // 16 * 4, dtype=torch.float32, device=dev)
        self.arr_k = ptr_array(k_layers, dev)
        self.arr_v = ptr_array(v_layers, dev) if v_layers is not None else None
        kv = dp_kv_inplace()
        kv.k_layers = self.arr_k.data_ptr()
        kv.v_layers = self.arr_v.data_ptr() if self.arr_v is not None else None
        kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = self.n_layers, heads, hd, self.dtype
        kv.capacity = cap
        kv.dev_error = self.dev_error.data_ptr()
        self.kv = kv
        self._keep_alive = [k_layers, v_layers, rope["theta"], rope["frame_t"],
                            rope["frame_phase"]]

    def _rope(self, q0):
        r = self.rope_args
        return make_rope(r["theta"], r["frame_t"], r["frame_phase"], q0, r["knee"],
                         r["inv_factor"], r.get("pair_begin", 0), axis=self.axis,
                         key_layout=r.get("key_layout", 0))

    def evict(self, slot, x0_hat, x_final, q0, row_stride=None, stream=None):
        """Enqueue the eviction of ring slot ``slot`` for query origin q0."""
        stride = self.d if row_stride is None else row_stride
        begin = self.sink_len + slot * self.chunk_rows
        dp_score_index(x0_hat, x_final, self.d, stride, self.policy, None, self.keep, self.idx,
                       self.n_kept, None, None, self.ws_index, self.dev_error, stream)
        rope = self._rope(q0)
        dp_rope_prepare(rope, self.head_dim, self.dtype, self.ws_rope, stream)
        if self.axis == DP_AXIS_COMPRESSED:
            dp_rope_apply(self.arr_k, self.n_layers, self.heads, self.head_dim, self.dtype, 0,
                          self.sink_len, None, self.row_frame, rope, self.ws_rope, stream)
            dp_append_kept(self.kv, begin, self.chunk_rows, self.idx, self.n_kept, self.tail,
                           self.row_frame, rope, self.ws_rope, stream)
            return
        dp_append_kept(self.kv, begin, self.chunk_rows, self.idx, self.n_kept, self.tail,
                       self.row_frame, None, None, stream)
        dp_rope_apply(self.arr_k, self.n_layers, self.heads, self.head_dim, self.dtype, 0,
                      self.sink_len, None, self.row_frame, rope, self.ws_rope, stream)
        dp_rope_apply(self.arr_k, self.n_layers, self.heads, self.head_dim, self.dtype,
                      self.history_begin, self.capacity, self.tail, self.row_frame, rope,
                      self.ws_rope, stream)

    def write_chunk(self, slot, frames):
        """Set the row frames of the chunk the model wrote into ring slot
        ``slot`` (device int32 [chunk_rows])."""
        begin = self.sink_len + slot * self.chunk_rows
        self.row_frame[begin:begin + self.chunk_rows].copy_(frames)
