"""GPU parity at the full sizes of the five workloads, in the launch
configuration bench.py times (one gather launch over all layers, K and V).

Mask, kept-index list, counts, offsets and frame phases are compared with the
oracle on every row; gathered / re-indexed K and V on sampled rows, whose
expected values the oracle computes one by one from inputs regenerated on the
host (the key/value generator is counter-based).  Bars: bit-exact for masks,
indices and V; keys within max-abs 2e-2 (bf16) / 1e-5 (fp32).
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import dpsynth
import oracle
from compaction_dp_score_amd.step import PruneStep
from gpu_helpers import bits, device, keys_close

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _sample_rows(n, boundaries, k=48, seed=0):
    rng = np.random.default_rng(seed)
    pts = {0, 1, n - 2, n - 1}
    for b in boundaries:
        for d in (-2, -1, 0, 1):
            if 0 <= b + d < n:
                pts.add(int(b + d))
    pts.update(int(x) for x in rng.integers(0, n, k))
    return np.array(sorted(p for p in pts if 0 <= p < n), np.int64)


def _fill(dev, w, rows, layers, stream_id):
    out = []
    for l in layers:
        t = torch.empty((rows, w.n_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
        dpsynth.kv_fill_device(t, "bf16", w.seed, stream_id, l, rows, w.n_heads * w.head_dim)
        out.append(t)
    return out


def _expected_rows(w, layer, stream_id, src_rows, total_rows):
    r = dpsynth.kv_rows_host("bf16", w.seed, stream_id, layer, src_rows, total_rows,
                             w.n_heads * w.head_dim)
    return np.ascontiguousarray(r.reshape(len(src_rows), w.n_heads, w.head_dim))


def _rope_host(w, q0=None):
    theta = dpsynth.rope_theta(w.rope_pairs, w.rope_base)
    ft, fp = dpsynth.frame_tables(w)
    return dict(theta=theta, frame_t=ft, frame_phase=fp, q0=w.q0 if q0 is None else q0,
                knee=w.rope_knee, inv_factor=np.float32(1.0 / w.rope_factor))


def _rope_dev(host, dev):
    return dict(theta=torch.from_numpy(host["theta"]).to(dev),
                frame_t=torch.from_numpy(host["frame_t"]).to(dev),
                frame_phase=torch.from_numpy(host["frame_phase"].copy()).to(dev),
                q0=host["q0"], knee=host["knee"], inv_factor=float(host["inv_factor"]))


def _tables(host):
    return oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"], host["knee"],
                              host["inv_factor"], host["theta"])


def test_eviction_step_full_size():
    """40 layers x 40 heads x 128 bf16, K and V, 31,200 tokens; score, mask,
    index and gather with the fused re-index in one step."""
    dev = device()
    w = dpsynth.WORKLOADS["eviction"]
    T, L = w.seq_len, w.n_layers
    x0, xf = dpsynth.score_inputs(w)
    k_src = _fill(dev, w, T, range(L), dpsynth.STREAM_K)
    v_src = _fill(dev, w, T, range(L), dpsynth.STREAM_V)
    k_dst = [torch.empty_like(t) for t in k_src]
    v_dst = [torch.empty_like(t) for t in v_src]
    host = _rope_host(w)
    rope = _rope_dev(host, dev)
    rf = dpsynth.row_frame(w)
    step = PruneStep(k_src=k_src, v_src=v_src, k_dst=k_dst, v_dst=v_dst, seq_len=T,
                     sink_len=w.sink_len, window_len=w.window_len, scored_begin=w.scored_begin,
                     n_scored=w.n_scored, gamma=w.gamma, d=w.d,
                     row_frame=torch.from_numpy(rf).to(dev), rope=rope, keep_ell=True)
    step.run(torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev))
    torch.cuda.synchronize()

    ell = oracle.score_f32(x0, xf, w.d)
    keep = oracle.mask(ell, T, w.sink_len, w.window_len, w.scored_begin, w.n_scored, w.gamma)
    idx = oracle.compact(keep)
    n = idx.shape[0]
    assert np.array_equal(step.ell.cpu().numpy().view(np.uint32), ell.view(np.uint32))
    assert np.array_equal(step.keep.cpu().numpy(), keep)
    assert int(step.n_kept.item()) == n and int(step.dev_error.item()) == 0
    assert np.array_equal(step.idx[:n].cpu().numpy(), idx)
    tables = _tables(host)
    assert np.array_equal(rope["frame_phase"].cpu().numpy(), tables[3])
    rf2 = oracle.gather_i32(rf, idx)
    assert np.array_equal(step.row_frame_dst[:n].cpu().numpy(), rf2)
    # PR of this step (pruning ratio against FullKV)
    c = dp.dp_pr_counter()
    dp.dp_pr_add(c, L * w.n_heads * n, L * w.n_heads * T)
    assert abs(dp.dp_pr_value(c) - oracle.pr(n, T)) < 1e-15

    js = _sample_rows(n, [w.sink_len, int(np.searchsorted(idx, T - w.window_len))])
    inexact = 0
    for l in (0, 13, 27, L - 1):
        got_k = bits(k_dst[l][torch.from_numpy(js).to(dev)])
        got_v = bits(v_dst[l][torch.from_numpy(js).to(dev)])
        want_v = _expected_rows(w, l, dpsynth.STREAM_V, idx[js], T)
        want_k = _expected_rows(w, l, dpsynth.STREAM_K, idx[js], T)
        oracle.rope_rows(want_k, rf2[js], 0, tables)
        assert np.array_equal(got_v, want_v), l
        ok, worst, ne = keys_close(got_k, want_k, TOL_BF16)
        assert ok, (l, worst)
        inexact += ne
    print("eviction: %d kept, %d non-identical sampled key elements" % (n, inexact))
    del step, k_src, v_src, k_dst, v_dst
    _free()


def test_reindex_full_size():
    """Re-index of the retained cache of a one-minute history: 40 x 40 x 128
    bf16 keys, 240 frames, q0 = 240, knee 12, factor 8."""
    dev = device()
    w = dpsynth.WORKLOADS["reindex"]
    L, H, D = w.n_layers, w.n_heads, w.head_dim
    kept = np.flatnonzero(dpsynth.retained_keep(w))
    rows = kept.shape[0]
    rf = dpsynth.row_frame(w)[kept].astype(np.int32)
    ks = _fill(dev, w, rows, range(L), dpsynth.STREAM_K)
    host = _rope_host(w)
    rd = _rope_dev(host, dev)
    rope = dp.make_rope(rd["theta"], rd["frame_t"], rd["frame_phase"], host["q0"], host["knee"],
                        host["inv_factor"])
    ws = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                     dtype=torch.float32, device=dev)
    arr = dp.ptr_array(ks, dev)
    dp.dp_rope_reindex(arr, L, H, D, dp.DP_BF16, rows, None, torch.from_numpy(rf).to(dev), rope, ws)
    torch.cuda.synchronize()
    tables = _tables(host)
    assert np.array_equal(rd["frame_phase"].cpu().numpy(), tables[3])
    js = _sample_rows(rows, [w.sink_len, int(np.searchsorted(kept, w.seq_len - w.window_len))],
                      seed=1)
    inexact = 0
    for l in (0, 19, L - 1):
        got = bits(ks[l][torch.from_numpy(js).to(dev)])
        want = _expected_rows(w, l, dpsynth.STREAM_K, js, rows)
        oracle.rope_rows(want, rf[js], 0, tables)
        ok, worst, ne = keys_close(got, want, TOL_BF16)
        assert ok, (l, worst)
        inexact += ne
    print("reindex: %d retained rows, %d non-identical sampled key elements" % (rows, inexact))
    del ks
    _free()


def test_prefix_full_size_slab():
    """Prefix pruning: 361,920 tokens, 57 scored chunks, one 20-layer slab of
    K and V (the 40-layer cache exceeds one GPU's memory)."""
    dev = device()
    w = dpsynth.WORKLOADS["prefix"]
    T, H, D = w.seq_len, w.n_heads, w.head_dim
    slab = list(range(20, 40))                 # the second slab
    x0, xf = dpsynth.score_inputs(w)
    ell = oracle.score_f32(x0, xf, w.d)
    keep = oracle.mask(ell, T, w.sink_len, w.window_len, w.scored_begin, w.n_scored, w.gamma)
    idx = oracle.compact(keep)
    n = idx.shape[0]
    k_src = _fill(dev, w, T, slab, dpsynth.STREAM_K)
    v_src = _fill(dev, w, T, slab, dpsynth.STREAM_V)
    k_dst = [torch.empty((n, H, D), dtype=torch.bfloat16, device=dev) for _ in slab]
    v_dst = [torch.empty((n, H, D), dtype=torch.bfloat16, device=dev) for _ in slab]
    step = PruneStep(k_src=k_src, v_src=v_src, k_dst=k_dst, v_dst=v_dst, seq_len=T,
                     sink_len=w.sink_len, window_len=w.window_len, scored_begin=w.scored_begin,
                     n_scored=w.n_scored, gamma=w.gamma, d=w.d, keep_ell=True)
    step.run(torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev))
    torch.cuda.synchronize()
    assert np.array_equal(step.ell.cpu().numpy().view(np.uint32), ell.view(np.uint32))
    assert np.array_equal(step.keep.cpu().numpy(), keep)
    assert int(step.n_kept.item()) == n and int(step.dev_error.item()) == 0
    assert np.array_equal(step.idx[:n].cpu().numpy(), idx)
    # per-chunk keep rates vary widely by construction
    rates = keep[w.sink_len:].reshape(-1, w.chunk_tokens).mean(axis=1)
    assert rates.min() < 0.05 and rates.max() > 0.4
    js = _sample_rows(n, [w.sink_len, n // 2], seed=2)
    for i, l in ((0, slab[0]), (len(slab) - 1, slab[-1])):
        sel = torch.from_numpy(js).to(dev)
        assert np.array_equal(bits(k_dst[i][sel]), _expected_rows(w, l, dpsynth.STREAM_K, idx[js], T))
        assert np.array_equal(bits(v_dst[i][sel]), _expected_rows(w, l, dpsynth.STREAM_V, idx[js], T))
    del step, k_src, v_src, k_dst, v_dst
    _free()


def test_hs_full_size():
    """DeCoPrune-HS: 40 x 40 x 128 bf16, 187,200 tokens, seeded half of the
    heads static per layer; ragged per-head output with the fused re-index."""
    dev = device()
    w = dpsynth.WORKLOADS["hs"]
    T, H, D, L = w.seq_len, w.n_heads, w.head_dim, w.n_layers
    x0, xf = dpsynth.score_inputs(w)
    cls = dpsynth.hs_head_class(w)
    rf = dpsynth.row_frame(w)
    # oracle: class lists and offsets
    ell = oracle.score_f32(x0, xf, w.d)
    lst_s = oracle.compact(oracle.mask(None, T, w.sink_len, w.window_len, w.scored_begin,
                                       w.n_scored, w.gamma, streaming=True))
    lst_d = oracle.compact(oracle.mask(ell, T, w.sink_len, w.window_len, w.scored_begin,
                                       w.n_scored, w.gamma))
    lens = np.array([len(lst_s), len(lst_d)], np.int64)
    off = oracle.hs_offsets(cls, lens)
    # GPU
    head_class = torch.from_numpy(cls.ravel().copy()).to(dev)
    k_src = _fill(dev, w, T, range(L), dpsynth.STREAM_K)
    v_src = _fill(dev, w, T, range(L), dpsynth.STREAM_V)
    x0d, xfd = torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev)
    keeps = [torch.empty(T, dtype=torch.uint8, device=dev) for _ in range(2)]
    dp.dp_score_mask(None, None, w.d, w.d, dp.make_policy(T, w.sink_len, w.window_len,
                     w.scored_begin, w.n_scored, w.gamma, mode=dp.DP_MODE_STREAMING), None, keeps[0])
    dp.dp_score_mask(x0d, xfd, w.d, w.d, dp.make_policy(T, w.sink_len, w.window_len,
                     w.scored_begin, w.n_scored, w.gamma), None, keeps[1])
    lists = [torch.empty(T, dtype=torch.int32, device=dev) for _ in range(2)]
    rfs = [torch.empty(T, dtype=torch.int32, device=dev) for _ in range(2)]
    glens = torch.zeros(2, dtype=torch.int64, device=dev)
    ws_c = torch.empty(dp.dp_compact_workspace_bytes(T) // 4 + 1, dtype=torch.int32, device=dev)
    rf_d = torch.from_numpy(rf).to(dev)
    for c in range(2):
        dp.dp_compact_index(keeps[c], T, lists[c], glens[c:c + 1], rf_d, rfs[c], ws_c)
    offsets = torch.empty(L * H + 1, dtype=torch.int64, device=dev)
    dp.dp_hs_offsets(head_class, L, H, glens, 2, offsets)
    torch.cuda.synchronize()
    assert np.array_equal(glens.cpu().numpy(), lens)
    assert np.array_equal(offsets.cpu().numpy(), off)
    total = int(off[-1])
    k_out = torch.empty((total, D), dtype=torch.bfloat16, device=dev)
    v_out = torch.empty((total, D), dtype=torch.bfloat16, device=dev)
    kv = dp.dp_kv_hs()
    arrs = [dp.ptr_array(k_src, dev), dp.ptr_array(v_src, dev)]
    kv.k_src, kv.v_src = arrs[0].data_ptr(), arrs[1].data_ptr()
    kv.k_out, kv.v_out = k_out.data_ptr(), v_out.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dp.DP_BF16
    kv.src_rows, kv.out_capacity = T, total
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv.dev_error = err.data_ptr()
    host = _rope_host(w)
    rd = _rope_dev(host, dev)
    rope = dp.make_rope(rd["theta"], rd["frame_t"], rd["frame_phase"], host["q0"], host["knee"],
                        host["inv_factor"])
    ws = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                     dtype=torch.float32, device=dev)
    dp.dp_hs_gather_kv(kv, head_class, 2, dp.ptr_array(lists, dev), glens, [T, T], offsets,
                       dp.ptr_array(rfs, dev), rope, ws)
    torch.cuda.synchronize()
    assert err.item() == 0
    tables = _tables(host)
    assert np.array_equal(rd["frame_phase"].cpu().numpy(), tables[3])
    rng = np.random.default_rng(3)
    inexact = 0
    for l, h in [(0, 0), (7, 13), (21, 39), (L - 1, H - 1)] + [
            (int(a), int(b)) for a, b in zip(rng.integers(0, L, 6), rng.integers(0, H, 6))]:
        i = l * H + h
        lst = lst_s if cls[l, h] == 0 else lst_d
        js = _sample_rows(len(lst), [w.sink_len], k=24, seed=i)
        src_rows = lst[js]
        want_k = _expected_rows(w, l, dpsynth.STREAM_K, src_rows, T)[:, h, :].copy()
        want_v = _expected_rows(w, l, dpsynth.STREAM_V, src_rows, T)[:, h, :].copy()
        oracle.rope_headrows(want_k, rf[src_rows], 0, tables)
        sel = torch.from_numpy(off[i] + js).to(dev)
        assert np.array_equal(bits(v_out[sel]), want_v), (l, h)
        ok, worst, ne = keys_close(bits(k_out[sel]), want_k, TOL_BF16)
        assert ok, (l, h, worst)
        inexact += ne
    print("hs: %d head rows, PR %.4f, %d non-identical sampled key elements"
          % (total, 1 - total / (L * H * T), inexact))
    del k_src, v_src, k_out, v_out
    _free()


@pytest.mark.parametrize("reversed_", [False, True])
def test_tiny_workload_every_row(reversed_):
    """The tiny workload (1 layer, 2 heads, head_dim 64, fp32, 8 chunks of 64
    tokens, d = 16): every output row against the oracle, for the criterion and
    for the reversed one (its complement on the scored rows)."""
    dev = device()
    w = dpsynth.WORKLOADS["tiny"]
    T, H, D, L = w.seq_len, w.n_heads, w.head_dim, w.n_layers
    x0, xf = dpsynth.score_inputs(w)
    kh = np.stack([dpsynth.kv_layer_host("f32", w.seed, dpsynth.STREAM_K, l, T, H * D)
                   for l in range(L)]).reshape(L, T, H, D)
    vh = np.stack([dpsynth.kv_layer_host("f32", w.seed, dpsynth.STREAM_V, l, T, H * D)
                   for l in range(L)]).reshape(L, T, H, D)
    rf = dpsynth.row_frame(w)
    host = _rope_host(w)
    rope = _rope_dev(host, dev)
    k_src = [torch.from_numpy(kh[l]).to(dev) for l in range(L)]
    v_src = [torch.from_numpy(vh[l]).to(dev) for l in range(L)]
    k_dst = [torch.zeros_like(t) for t in k_src]
    v_dst = [torch.zeros_like(t) for t in v_src]
    step = PruneStep(k_src=k_src, v_src=v_src, k_dst=k_dst, v_dst=v_dst, seq_len=T,
                     sink_len=w.sink_len, window_len=w.window_len, scored_begin=w.scored_begin,
                     n_scored=w.n_scored, gamma=w.gamma, d=w.d, reversed=reversed_,
                     row_frame=torch.from_numpy(rf).to(dev), rope=rope, keep_ell=True)
    step.run(torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev))
    torch.cuda.synchronize()
    pol = dict(seq_len=T, sink_len=w.sink_len, window_len=w.window_len,
               scored_begin=w.scored_begin, n_scored=w.n_scored, gamma=w.gamma,
               reversed=reversed_)
    want = oracle.prune_step(x0, xf, w.d, pol, kh, vh, rf, host)
    n = want["idx"].shape[0]
    assert np.array_equal(step.keep.cpu().numpy(), want["keep"])
    assert int(step.n_kept.item()) == n
    assert np.array_equal(step.idx[:n].cpu().numpy(), want["idx"])
    for l in range(L):
        assert np.array_equal(bits(v_dst[l][:n]), want["v"][l].view(np.uint32))
        ok, worst, ne = keys_close(bits(k_dst[l][:n]), want["k"][l].view(np.uint32), 1e-5)
        assert ok, worst
        assert np.all(bits(k_dst[l][n:]) == 0)
    # the sink chunk and the window are kept, whatever the criterion
    assert np.all(want["keep"][:w.sink_len] == 1) and np.all(want["keep"][T - w.window_len:] == 1)
    print("tiny (reversed=%s): %d of %d kept, PR %.4f" % (reversed_, n, T, oracle.pr(n, T)))


def test_steady_step_full_size():
    """The steady-state step of the one-minute rollout in the ring layout, as
    bench.py times it: 40 x 40 x 128 bf16, [sink | 4 ring slots | history of
    the retained rows of chunks 1-55 | room]; chunk 56 leaves the window for
    q0 = 240.  The sink and history move by the uniform step 3.5 frames
    (dp_rope_shift), the leaving chunk's kept rows are appended with their
    first re-index fused.  Sampled rows of three layers against the oracle."""
    dev = device()
    w = dpsynth.WORKLOADS["reindex"]
    L, H, D, C, tpf = w.n_layers, w.n_heads, w.head_dim, w.chunk_tokens, w.tokens_per_frame
    hist_rows = np.flatnonzero(dpsynth.retained_keep(w)[C:56 * C]) + C
    n_hist = hist_rows.shape[0]
    hb = 5 * C
    cap = hb + n_hist + C
    slot_begin = C
    rf = np.full(cap, -1, np.int32)
    rf[:C] = np.arange(C) // tpf
    rf[C:hb] = (56 * C + np.arange(4 * C)) // tpf
    rf[hb:hb + n_hist] = hist_rows // tpf
    ks = _fill(dev, w, cap, range(L), dpsynth.STREAM_K)
    vs = _fill(dev, w, cap, range(L), dpsynth.STREAM_V)
    we = dpsynth.WORKLOADS["eviction"]
    x0, xf = dpsynth.score_inputs(we)
    widx = oracle.compact(oracle.mask(oracle.score_f32(x0, xf, we.d), C, 0, 0, 0, C, w.gamma))
    n = widx.shape[0]
    host = _rope_host(w, q0=w.q0 - 4)                 # phases after the previous step (q0 = 236)
    phase0 = _tables(host)[3]
    host = dict(host, q0=w.q0, frame_phase=phase0)
    rd = _rope_dev(host, dev)
    # device step
    kv = dp.dp_kv_inplace()
    ak, av = dp.ptr_array(ks, dev), dp.ptr_array(vs, dev)
    kv.k_layers, kv.v_layers = ak.data_ptr(), av.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dp.DP_BF16
    kv.capacity = cap
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv.dev_error = err.data_ptr()
    keep = torch.empty(C, dtype=torch.uint8, device=dev)
    idx = torch.empty(C, dtype=torch.int32, device=dev)
    nk = torch.zeros(1, dtype=torch.int64, device=dev)
    ws_si = torch.zeros(dp.dp_score_index_workspace_bytes(C) // 8 + 1, dtype=torch.int64,
                        device=dev)
    dp.dp_score_index(torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev), we.d, we.d,
                      dp.make_policy(C, 0, 0, 0, C, w.gamma), None, keep, idx, nk, None, None,
                      ws_si, err)
    tail = torch.tensor([hb + n_hist], dtype=torch.int64, device=dev)
    rf_d = torch.from_numpy(rf).to(dev)
    ws_s = torch.empty(dp.dp_rope_shift_workspace_bytes(w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    step = 4 * (1 - 1 / w.rope_factor)
    dp.dp_rope_shift(ak, L, H, D, dp.DP_BF16, 0, C, None, rd["theta"], 0, w.rope_pairs, step, ws_s)
    dp.dp_rope_shift(ak, L, H, D, dp.DP_BF16, hb, cap, tail, rd["theta"], 0, w.rope_pairs, step,
                     ws_s)
    rope = dp.make_rope(rd["theta"], rd["frame_t"], rd["frame_phase"], host["q0"], host["knee"],
                        host["inv_factor"])
    ws_r = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
    dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf_d, rope, ws_r)
    torch.cuda.synchronize()
    assert err.item() == 0 and nk.item() == n and tail.item() == hb + n_hist + n
    tables = _tables(host)
    assert np.array_equal(rd["frame_phase"].cpu().numpy(), tables[3])
    uniform = oracle.rope_uniform(host["theta"], step)
    old_rows = np.concatenate([_sample_rows(C, [], k=16, seed=2),
                               hb + _sample_rows(n_hist, [], k=32, seed=3)])
    ring_rows = C + _sample_rows(4 * C, [C, 2 * C, 3 * C], k=8, seed=4)
    app = _sample_rows(n, [], k=24, seed=5)
    src = slot_begin + widx[app]
    assert np.array_equal(rf_d.cpu().numpy()[hb + n_hist + app], rf[src])
    inexact = 0
    for l in (0, 19, L - 1):
        got = bits(ks[l][torch.from_numpy(old_rows).to(dev)])
        want = _expected_rows(w, l, dpsynth.STREAM_K, old_rows, cap)
        oracle.rope_rows(want, np.zeros(len(old_rows), np.int32), 0, uniform)
        ok, worst, ne = keys_close(got, want, TOL_BF16)
        assert ok, ("old keys", l, worst)
        inexact += ne
        got = bits(ks[l][torch.from_numpy(ring_rows).to(dev)])
        assert np.array_equal(got, _expected_rows(w, l, dpsynth.STREAM_K, ring_rows, cap)), l
        got = bits(ks[l][torch.from_numpy(hb + n_hist + app).to(dev)])
        want = _expected_rows(w, l, dpsynth.STREAM_K, src, cap)
        oracle.rope_rows(want, rf[src], 0, tables)
        ok, worst, ne = keys_close(got, want, TOL_BF16)
        assert ok, ("appended keys", l, worst)
        inexact += ne
        got = bits(vs[l][torch.from_numpy(hb + n_hist + app).to(dev)])
        assert np.array_equal(got, _expected_rows(w, l, dpsynth.STREAM_V, src, cap)), l
    print("steady step: %d history rows, %d appended, %d non-identical sampled key elements"
          % (n_hist, n, inexact))
    del ks, vs
    _free()


def _tables_compressed(host):
    return oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"], host["knee"],
                              host["inv_factor"], host["theta"], compressed=True)


def test_steady_lazy_step_full_size():
    """The steady-state step on the compressed time axis, as bench.py times it
    (workload steady_lazy): 40 x 40 x 128 bf16, [sink | 4 ring slots | history
    of the retained rows of chunks 1-55 | room]; chunk 56 leaves the window for
    q0 = 240.  No old key is written; the leaving chunk's kept rows are
    appended with its frames moved from phase t to t/c (fused).  Sampled rows
    of three layers against the oracle's compressed-axis tables."""
    dev = device()
    w = dpsynth.WORKLOADS["reindex"]
    L, H, D, C, tpf = w.n_layers, w.n_heads, w.head_dim, w.chunk_tokens, w.tokens_per_frame
    hist_rows = np.flatnonzero(dpsynth.retained_keep(w)[C:56 * C]) + C
    n_hist = hist_rows.shape[0]
    hb = 5 * C
    cap = hb + n_hist + C
    slot_begin = C
    rf = np.full(cap, -1, np.int32)
    rf[:C] = np.arange(C) // tpf
    rf[C:hb] = (56 * C + np.arange(4 * C)) // tpf
    rf[hb:hb + n_hist] = hist_rows // tpf
    ks = _fill(dev, w, cap, range(L), dpsynth.STREAM_K)
    vs = _fill(dev, w, cap, range(L), dpsynth.STREAM_V)
    we = dpsynth.WORKLOADS["eviction"]
    x0, xf = dpsynth.score_inputs(we)
    widx = oracle.compact(oracle.mask(oracle.score_f32(x0, xf, we.d), C, 0, 0, 0, C, w.gamma))
    n = widx.shape[0]
    host = _rope_host(w, q0=w.q0 - 4)                 # phases after the previous step (q0 = 236)
    phase0 = _tables_compressed(host)[3]
    host = dict(host, q0=w.q0, frame_phase=phase0)
    rd = _rope_dev(host, dev)
    kv = dp.dp_kv_inplace()
    ak, av = dp.ptr_array(ks, dev), dp.ptr_array(vs, dev)
    kv.k_layers, kv.v_layers = ak.data_ptr(), av.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dp.DP_BF16
    kv.capacity = cap
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv.dev_error = err.data_ptr()
    keep = torch.empty(C, dtype=torch.uint8, device=dev)
    idx = torch.empty(C, dtype=torch.int32, device=dev)
    nk = torch.zeros(1, dtype=torch.int64, device=dev)
    ws_si = torch.zeros(dp.dp_score_index_workspace_bytes(C) // 8 + 1, dtype=torch.int64,
                        device=dev)
    dp.dp_score_index(torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev), we.d, we.d,
                      dp.make_policy(C, 0, 0, 0, C, w.gamma), None, keep, idx, nk, None, None,
                      ws_si, err)
    tail = torch.tensor([hb + n_hist], dtype=torch.int64, device=dev)
    rf_d = torch.from_numpy(rf).to(dev)
    rope = dp.make_rope(rd["theta"], rd["frame_t"], rd["frame_phase"], host["q0"], host["knee"],
                        host["inv_factor"], axis=dp.DP_AXIS_COMPRESSED)
    ws_r = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
    dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf_d, rope, ws_r)
    torch.cuda.synchronize()
    assert err.item() == 0 and nk.item() == n and tail.item() == hb + n_hist + n
    tables = _tables_compressed(host)
    assert np.array_equal(rd["frame_phase"].cpu().numpy(), tables[3])
    moved = np.flatnonzero(tables[0] != 0)                   # frames whose phase changes
    assert np.array_equal(moved, np.arange(224, 228))       # chunk 56 only: t -> t/c
    old_rows = np.concatenate([_sample_rows(C, [], k=16, seed=2),
                               hb + _sample_rows(n_hist, [], k=32, seed=3)])
    ring_rows = C + _sample_rows(4 * C, [C, 2 * C, 3 * C], k=8, seed=4)
    app = _sample_rows(n, [], k=24, seed=5)
    src = slot_begin + widx[app]
    assert np.array_equal(rf_d.cpu().numpy()[hb + n_hist + app], rf[src])
    inexact = 0
    for l in (0, 19, L - 1):
        for rows in (old_rows, ring_rows):                   # never written
            got = bits(ks[l][torch.from_numpy(rows).to(dev)])
            assert np.array_equal(got, _expected_rows(w, l, dpsynth.STREAM_K, rows, cap)), l
        got = bits(ks[l][torch.from_numpy(hb + n_hist + app).to(dev)])
        want = _expected_rows(w, l, dpsynth.STREAM_K, src, cap)
        oracle.rope_rows(want, rf[src], 0, tables)
        ok, worst, ne = keys_close(got, want, TOL_BF16)
        assert ok, ("appended keys", l, worst)
        inexact += ne
        got = bits(vs[l][torch.from_numpy(hb + n_hist + app).to(dev)])
        assert np.array_equal(got, _expected_rows(w, l, dpsynth.STREAM_V, src, cap)), l
    print("compressed-axis steady step: %d history rows, %d appended, %d non-identical sampled "
          "key elements" % (n_hist, n, inexact))
    del ks, vs
    _free()


def test_hs_ring_step_full_size():
    """The HS eviction step in the ring layout, as bench.py times it (workload
    hs_ring): per layer the 20 dynamic heads of the HS workload keep one
    token-major cache [sink | 4 ring slots | history of the retained rows of
    chunks 1-25 | room] (20 x 128 bf16 per row, 40 layers); chunk 26 leaves the
    window for q0 = 120 and its kept rows are appended to every layer's dynamic
    cache with the re-index fused on the compressed axis.  Sampled rows of three
    layers against the oracle; the static class's cache is not touched by the
    call."""
    dev = device()
    w = dpsynth.WORKLOADS["hs"]
    L, D, C, tpf = w.n_layers, w.head_dim, w.chunk_tokens, w.tokens_per_frame
    HC = w.n_heads // 2
    hist_rows = np.flatnonzero(dpsynth.retained_keep(w)[C:26 * C]) + C
    n_hist = hist_rows.shape[0]
    hb = 5 * C
    cap = hb + n_hist + C
    slot_begin = C
    rf = np.full(cap, -1, np.int32)
    rf[:C] = np.arange(C) // tpf
    rf[C:hb] = (26 * C + np.arange(4 * C)) // tpf
    rf[hb:hb + n_hist] = hist_rows // tpf

    def fill(stream_id):
        out = []
        for l in range(L):
            t = torch.empty((cap, HC, D), dtype=torch.bfloat16, device=dev)
            dpsynth.kv_fill_device(t, "bf16", w.seed, stream_id, l, cap, HC * D)
            out.append(t)
        return out

    def expected(layer, stream_id, rows):
        r = dpsynth.kv_rows_host("bf16", w.seed, stream_id, layer, rows, cap, HC * D)
        return np.ascontiguousarray(r.reshape(len(rows), HC, D))

    ks, vs = fill(dpsynth.STREAM_K), fill(dpsynth.STREAM_V)
    we = dpsynth.WORKLOADS["eviction"]
    x0, xf = dpsynth.score_inputs(we)
    widx = oracle.compact(oracle.mask(oracle.score_f32(x0, xf, we.d), C, 0, 0, 0, C, w.gamma))
    n = widx.shape[0]
    host = _rope_host(w, q0=w.q0 - 4)                 # phases after the previous step (q0 = 116)
    phase0 = _tables_compressed(host)[3]
    host = dict(host, q0=w.q0, frame_phase=phase0)
    rd = _rope_dev(host, dev)
    kv = dp.dp_kv_inplace()
    ak, av = dp.ptr_array(ks, dev), dp.ptr_array(vs, dev)
    kv.k_layers, kv.v_layers = ak.data_ptr(), av.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, HC, D, dp.DP_BF16
    kv.capacity = cap
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv.dev_error = err.data_ptr()
    keep = torch.empty(C, dtype=torch.uint8, device=dev)
    idx = torch.empty(C, dtype=torch.int32, device=dev)
    nk = torch.zeros(1, dtype=torch.int64, device=dev)
    ws_si = torch.zeros(dp.dp_score_index_workspace_bytes(C) // 8 + 1, dtype=torch.int64,
                        device=dev)
    dp.dp_score_index(torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev), we.d, we.d,
                      dp.make_policy(C, 0, 0, 0, C, w.gamma), None, keep, idx, nk, None, None,
                      ws_si, err)
    tail = torch.tensor([hb + n_hist], dtype=torch.int64, device=dev)
    rf_d = torch.from_numpy(rf).to(dev)
    rope = dp.make_rope(rd["theta"], rd["frame_t"], rd["frame_phase"], host["q0"], host["knee"],
                        host["inv_factor"], axis=dp.DP_AXIS_COMPRESSED)
    ws_r = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
    dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf_d, rope, ws_r)
    torch.cuda.synchronize()
    assert err.item() == 0 and nk.item() == n and tail.item() == hb + n_hist + n
    tables = _tables_compressed(host)
    assert np.array_equal(rd["frame_phase"].cpu().numpy(), tables[3])
    assert np.array_equal(np.flatnonzero(tables[0] != 0), np.arange(104, 108))   # chunk 26 only
    rf_after = rf_d.cpu().numpy()
    assert np.all(rf_after[slot_begin:slot_begin + C] == -1)                  # the slot is retired
    old_rows = np.concatenate([_sample_rows(C, [], k=16, seed=12),
                               hb + _sample_rows(n_hist, [], k=32, seed=13)])
    ring_rows = C + _sample_rows(4 * C, [C, 2 * C, 3 * C], k=8, seed=14)
    app = _sample_rows(n, [], k=24, seed=15)
    src = slot_begin + widx[app]
    assert np.array_equal(rf_after[hb + n_hist + app], rf[src])
    inexact = 0
    for l in (0, 19, L - 1):
        for rows in (old_rows, ring_rows):                   # never written
            got = bits(ks[l][torch.from_numpy(rows).to(dev)])
            assert np.array_equal(got, expected(l, dpsynth.STREAM_K, rows)), l
        got = bits(ks[l][torch.from_numpy(hb + n_hist + app).to(dev)])
        want = expected(l, dpsynth.STREAM_K, src)
        oracle.rope_rows(want, rf[src], 0, tables)
        ok, worst, ne = keys_close(got, want, TOL_BF16)
        assert ok, ("appended keys", l, worst)
        inexact += ne
        got = bits(vs[l][torch.from_numpy(hb + n_hist + app).to(dev)])
        assert np.array_equal(got, expected(l, dpsynth.STREAM_V, src)), l
    print("HS ring step: %d history rows, %d appended, %d non-identical sampled key elements"
          % (n_hist, n, inexact))
    del ks, vs
    _free()
