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

from . import (DP_MODE_SCORE, dp_compact_index, dp_compact_workspace_bytes, dp_gather_kv,
               dp_kv, dp_rope_workspace_bytes, dp_score_index, dp_score_index_workspace_bytes,
               dp_score_mask, dtype_code, make_policy, make_rope, ptr_array)


class PruneStep:
    def __init__(self, *, k_src, v_src, k_dst, v_dst, seq_len, sink_len, window_len,
                 scored_begin, n_scored, gamma, d, row_frame=None, rope=None,
                 reversed=False, mode=DP_MODE_SCORE, keep_ell=False, fused=True):
        """k_src/v_src/k_dst/v_dst: lists of per-layer device tensors
        [rows, heads, head_dim]; v_* may be None.  rope: None or a dict with
        theta, frame_t, frame_phase (device tensors), q0, knee, inv_factor,
        pair_begin."""
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
                                  rope.get("pair_begin", 0))
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
