"""GPU parity at the full sizes of the five workloads, in the launch
configuration bench.py times (one gather launch over all layers, K and V).

Mask, kept-index list, counts, offsets and frame phases are compared with the
oracle on every row.  Gathered / re-indexed K and V are compared on every
element of every layer: on the device against the source rows at the oracle's
index list (V and the dims outside the temporal block bit for bit, rows whose
frame does not move bit for bit, temporal pairs within the bar of the float64
rotation by the oracle's own cos/sin tables), and, for whole layers, on the
host against the C oracle's gather and re-index of the source copied back.
The sources are the seeded generator's fill (tied to its host twin on sampled
rows); the in-place passes regenerate their source into a scratch buffer.
Bars: bit-exact for masks, indices and V; keys within max-abs 2e-2 (bf16) /
1e-5 (fp32).  The re-index workloads run on both key layouts (split keys are
what bench.py times for them): split caches are permuted from the fill before
the call and back after it (data movement only), then checked as above.
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import dpsynth
import oracle
from compaction_dp_score_amd.step import PruneStep
from gpu_helpers import bits, device, from_split, keys_close, to_split

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
BLOCK_ELEMS = 1 << 24          # elements of one device comparison block


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _fill(dev, w, rows, layers, stream_id, heads=None):
    heads = w.n_heads if heads is None else heads
    out = []
    for l in layers:
        t = torch.empty((rows, heads, w.head_dim), dtype=torch.bfloat16, device=dev)
        dpsynth.kv_fill_device(t, "bf16", w.seed, stream_id, l, rows, heads * w.head_dim)
        out.append(t)
    return out


def _tie_to_host(t, w, layer, stream_id, rows_total, heads=None):
    """The device fill of one layer equals the generator's host twin on
    sampled rows (so the fill is the documented input)."""
    heads = w.n_heads if heads is None else heads
    n = t.shape[0]
    rows = np.unique(np.array([0, 1, n // 3, n // 2, n - 2, n - 1], np.int64))
    host = dpsynth.kv_rows_host("bf16", w.seed, stream_id, layer, rows, rows_total,
                                heads * w.head_dim)
    assert np.array_equal(bits(t[torch.from_numpy(rows).to(t.device)]).reshape(len(rows), -1),
                          host), layer


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


def _tables(host, compressed=False):
    return oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"], host["knee"],
                              host["inv_factor"], host["theta"], compressed=compressed)


def _tables_dev(tables, dev):
    return tuple(torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in tables[:3])


def _i64(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(dev)


LAYOUTS = [dp.DP_KEY_INTERLEAVED, dp.DP_KEY_SPLIT]


def _to_layout(layers, layout, n_pairs):
    """Permute natural key layers in place into `layout` (split: the temporal
    blocks of all heads first)."""
    if layout == dp.DP_KEY_SPLIT:
        for t in layers:
            t.copy_(to_split(t, 0, n_pairs))


class _Natural:
    """Key layers read back in the natural layout (one layer converted at a
    time, the last one cached)."""

    def __init__(self, layers, layout, n_pairs):
        self.layers, self.layout, self.n_pairs = layers, layout, n_pairs
        self.last = (None, None)

    def __getitem__(self, l):
        if self.layout != dp.DP_KEY_SPLIT:
            return self.layers[l]
        if self.last[0] != l:
            self.last = (l, from_split(self.layers[l], 0, self.n_pairs))
        return self.last[1]


def _same(a, b):
    """Bit-for-bit equality of two bf16 device tensors."""
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _check_rotated(got, src, frames, tabd, n_pairs, pair_begin=0, tol=TOL_BF16):
    """Every element of got [n, H, D] (bf16, device) against src [n, H, D]
    re-indexed for the frames ``frames`` (device int64 [n]) with the oracle's
    tables tabd = (delta, cos, sin) on the device: dims outside the temporal
    block and rows whose frame has delta 0 bit for bit; temporal pairs within
    tol of the float64 rotation (a c - b s, a s + b c) by the oracle's cos/sin
    entries.  Returns (max |error|, count of elements that differ from that
    rotation rounded to bf16)."""
    delta, ct, st = tabd
    lo, hi = 2 * pair_begin, 2 * (pair_begin + n_pairs)
    worst, inexact = 0.0, 0
    rb = max(1, BLOCK_ELEMS // max(1, got[0].numel()))
    for b in range(0, got.shape[0], rb):
        g, x, f = got[b:b + rb], src[b:b + rb], frames[b:b + rb]
        assert _same(g[..., :lo], x[..., :lo]) and _same(g[..., hi:], x[..., hi:])
        still = delta[f] == 0
        assert _same(g[still], x[still])
        xd = x[..., lo:hi].double()
        a, bb = xd[..., 0::2], xd[..., 1::2]
        c, sn = ct[f][:, None, :].double(), st[f][:, None, :].double()
        want = torch.empty_like(xd)
        want[..., 0::2] = a * c - bb * sn
        want[..., 1::2] = a * sn + bb * c
        gd = g[..., lo:hi].double()
        worst = max(worst, float((gd - want).abs().max().item()) if gd.numel() else 0.0)
        inexact += int((gd != want.to(torch.bfloat16).double()).sum().item())
    assert worst <= tol, worst
    return worst, inexact


def _oracle_layer(src_k, src_v, idx, got_k, got_v, rf2=None, tables=None, tol=TOL_BF16):
    """One whole layer through the C oracle: gather of the source copied back
    (K and V), the K re-index, every element compared."""
    want_k = oracle.gather(bits(src_k)[None], idx)[0]
    if tables is not None:
        oracle.rope_rows(want_k, rf2, 0, tables)
    ok, worst, ne = keys_close(bits(got_k), want_k, tol)
    assert ok, worst
    if src_v is not None:
        assert np.array_equal(bits(got_v), oracle.gather(bits(src_v)[None], idx)[0])
    return ne


def test_eviction_step_full_size():
    """40 layers x 40 heads x 128 bf16, K and V, 31,200 tokens; score, mask,
    index and gather with the fused re-index in one step.  K and V of all 40
    layers element by element; layers 0, 19 and 39 also through the C oracle."""
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

    idx_d, rf2_d, tabd = _i64(idx, dev), _i64(rf2, dev), _tables_dev(tables, dev)
    worst, inexact = 0.0, 0
    for l in range(L):
        _tie_to_host(k_src[l], w, l, dpsynth.STREAM_K, T)
        _tie_to_host(v_src[l], w, l, dpsynth.STREAM_V, T)
        assert _same(v_dst[l][:n], v_src[l].index_select(0, idx_d)), l
        e, ne = _check_rotated(k_dst[l][:n], k_src[l].index_select(0, idx_d), rf2_d, tabd,
                               w.rope_pairs)
        worst, inexact = max(worst, e), inexact + ne
    for l in (0, 19, L - 1):
        _oracle_layer(k_src[l], v_src[l], idx, k_dst[l][:n], v_dst[l][:n], rf2, tables)
    print("eviction: %d kept x %d layers, max |key error| %.3g, %d key elements off the "
          "float64 rotation's bf16" % (n, L, worst, inexact))
    del step, k_src, v_src, k_dst, v_dst
    _free()


@pytest.mark.parametrize("layout", LAYOUTS)
def test_reindex_full_size(layout):
    """Re-index of the retained cache of a one-minute history: 40 x 40 x 128
    bf16 keys, 240 frames, q0 = 240, knee 12, factor 8, on either key layout.
    Every key of all 40 layers against its regenerated source; layers 0, 19
    and 39 also through the C oracle."""
    dev = device()
    w = dpsynth.WORKLOADS["reindex"]
    L, H, D = w.n_layers, w.n_heads, w.head_dim
    kept = np.flatnonzero(dpsynth.retained_keep(w))
    rows = kept.shape[0]
    rf = dpsynth.row_frame(w)[kept].astype(np.int32)
    ks = _fill(dev, w, rows, range(L), dpsynth.STREAM_K)
    _to_layout(ks, layout, w.rope_pairs)
    host = _rope_host(w)
    rd = _rope_dev(host, dev)
    rope = dp.make_rope(rd["theta"], rd["frame_t"], rd["frame_phase"], host["q0"], host["knee"],
                        host["inv_factor"], key_layout=layout)
    ws = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                     dtype=torch.float32, device=dev)
    arr = dp.ptr_array(ks, dev)
    dp.dp_rope_reindex(arr, L, H, D, dp.DP_BF16, rows, None, torch.from_numpy(rf).to(dev), rope, ws)
    torch.cuda.synchronize()
    tables = _tables(host)
    assert np.array_equal(rd["frame_phase"].cpu().numpy(), tables[3])
    rf_d, tabd = _i64(rf, dev), _tables_dev(tables, dev)
    src = torch.empty_like(ks[0])
    nat = _Natural(ks, layout, w.rope_pairs)
    worst, inexact = 0.0, 0
    for l in range(L):
        dpsynth.kv_fill_device(src, "bf16", w.seed, dpsynth.STREAM_K, l, rows, H * D)
        _tie_to_host(src, w, l, dpsynth.STREAM_K, rows)
        e, ne = _check_rotated(nat[l], src, rf_d, tabd, w.rope_pairs)
        worst, inexact = max(worst, e), inexact + ne
        if l in (0, 19, L - 1):
            _oracle_layer(src, None, np.arange(rows, dtype=np.int32), nat[l], None, rf, tables)
    print("reindex (layout %d): %d retained rows x %d layers, max |key error| %.3g, %d key "
          "elements off the float64 rotation's bf16" % (layout, rows, L, worst, inexact))
    del ks, src
    _free()


@pytest.mark.parametrize("slab", [0, 1])
def test_prefix_full_size_slab(slab):
    """Prefix pruning: 361,920 tokens, 57 scored chunks, one 20-layer slab of
    K and V per call (the 40-layer cache exceeds one GPU's memory); both slabs
    run.  Every kept row of every layer of the slab element by element; one
    layer of the slab also through the C oracle."""
    dev = device()
    w = dpsynth.WORKLOADS["prefix"]
    T, H, D = w.seq_len, w.n_heads, w.head_dim
    layers = list(range(20 * slab, 20 * slab + 20))
    x0, xf = dpsynth.score_inputs(w)
    ell = oracle.score_f32(x0, xf, w.d)
    keep = oracle.mask(ell, T, w.sink_len, w.window_len, w.scored_begin, w.n_scored, w.gamma)
    idx = oracle.compact(keep)
    n = idx.shape[0]
    k_src = _fill(dev, w, T, layers, dpsynth.STREAM_K)
    v_src = _fill(dev, w, T, layers, dpsynth.STREAM_V)
    k_dst = [torch.empty((n, H, D), dtype=torch.bfloat16, device=dev) for _ in layers]
    v_dst = [torch.empty((n, H, D), dtype=torch.bfloat16, device=dev) for _ in layers]
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
    idx_d = _i64(idx, dev)
    for i, l in enumerate(layers):
        _tie_to_host(k_src[i], w, l, dpsynth.STREAM_K, T)
        _tie_to_host(v_src[i], w, l, dpsynth.STREAM_V, T)
        assert _same(k_dst[i], k_src[i].index_select(0, idx_d)), l
        assert _same(v_dst[i], v_src[i].index_select(0, idx_d)), l
    i = 0 if slab == 0 else len(layers) - 1
    _oracle_layer(k_src[i], v_src[i], idx, k_dst[i], v_dst[i], tol=0.0)
    print("prefix slab %d (layers %d-%d): %d of %d rows kept, every element checked"
          % (slab, layers[0], layers[-1], n, T))
    del step, k_src, v_src, k_dst, v_dst
    _free()


def test_hs_full_size():
    """DeCoPrune-HS: 40 x 40 x 128 bf16, 187,200 tokens, seeded half of the
    heads static per layer; ragged per-head output with the fused re-index.
    Every (layer, head) run element by element; layers 0 and 39 also through
    the C oracle's per-head gather and re-index."""
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
    for c, lst in enumerate((lst_s, lst_d)):
        assert np.array_equal(lists[c][:len(lst)].cpu().numpy(), lst)
        assert np.array_equal(rfs[c][:len(lst)].cpu().numpy(), rf[lst])
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
    tabd = _tables_dev(tables, dev)
    lst_dev = [_i64(lst_s, dev), _i64(lst_d, dev)]
    worst, inexact = 0.0, 0
    for l in range(L):
        _tie_to_host(k_src[l], w, l, dpsynth.STREAM_K, T)
        _tie_to_host(v_src[l], w, l, dpsynth.STREAM_V, T)
        for c in range(2):
            heads = np.flatnonzero(cls[l] == c)
            if heads.size == 0:
                continue
            nc = int(lens[c])
            # every run of this class, head-major: [heads, nc, D] -> [heads * nc, 1, D]
            hsel = _i64(heads, dev)
            src_k = k_src[l].index_select(0, lst_dev[c]).index_select(1, hsel)
            src_v = v_src[l].index_select(0, lst_dev[c]).index_select(1, hsel)
            src_k = src_k.permute(1, 0, 2).reshape(-1, 1, D)
            src_v = src_v.permute(1, 0, 2).reshape(-1, 1, D)
            out_rows = (off[l * H + heads][:, None] + np.arange(nc)[None, :]).ravel()
            osel = _i64(out_rows, dev)
            assert _same(v_out.index_select(0, osel).view(-1, 1, D), src_v), (l, c)
            frames = lst_dev[c].new_tensor(np.tile(rf[(lst_s, lst_d)[c]], heads.size))
            e, ne = _check_rotated(k_out.index_select(0, osel).view(-1, 1, D), src_k, frames, tabd,
                                   w.rope_pairs)
            worst, inexact = max(worst, e), inexact + ne
    # whole layers through the C oracle's per-head gather and re-index
    for l in (0, L - 1):
        sk, sv = bits(k_src[l]), bits(v_src[l])
        lo, hi = int(off[l * H]), int(off[(l + 1) * H])
        wk = np.zeros((hi - lo, D), np.uint16)       # this layer's runs: offsets shifted to 0
        wv = np.zeros((hi - lo, D), np.uint16)
        oracle.hs_gather_layer(sk, l, cls, [lst_s, lst_d], off - lo, wk)
        oracle.hs_gather_layer(sv, l, cls, [lst_s, lst_d], off - lo, wv)
        frames = np.concatenate([rf[(lst_s, lst_d)[cls[l, h]]] for h in range(H)]).astype(np.int32)
        oracle.rope_headrows(wk, frames, 0, tables)
        assert np.array_equal(bits(v_out[lo:hi]), wv), l
        ok, e, _ = keys_close(bits(k_out[lo:hi]), wk, TOL_BF16)
        assert ok, (l, e)
    print("hs: %d head rows, PR %.4f, every (layer, head) run checked, max |key error| %.3g, "
          "%d key elements off the float64 rotation's bf16"
          % (total, 1 - total / (L * H * T), worst, inexact))
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


def _ring_setup(w, last_hist_chunk):
    """Row frames of the one-step ring layout [sink | 4 slots | history of the
    retained rows of chunks 1..last_hist_chunk | room for one chunk]."""
    C, tpf = w.chunk_tokens, w.tokens_per_frame
    hist_rows = np.flatnonzero(dpsynth.retained_keep(w)[C:(last_hist_chunk + 1) * C]) + C
    n_hist = hist_rows.shape[0]
    hb = 5 * C
    cap = hb + n_hist + C
    rf = np.full(cap, -1, np.int32)
    rf[:C] = np.arange(C) // tpf
    rf[C:hb] = ((last_hist_chunk + 1) * C + np.arange(4 * C)) // tpf
    rf[hb:hb + n_hist] = hist_rows // tpf
    return rf, n_hist, hb, cap


def _check_ring_layer(w, l, heads, cap, ks, vs, hb, n_hist, slot_begin, widx, rf, old_tabd,
                      tabd, dev, scratch):
    """Every row of one layer of a ring-layout cache after one eviction step
    against the regenerated fill: the old rows (sink, history) re-indexed by
    old_tabd (None: untouched), the ring slots untouched, the appended rows =
    the leaving slot's kept rows re-indexed by tabd, the rows past the new tail
    untouched; V untouched except the appended rows, which are copies."""
    C, D = w.chunk_tokens, w.head_dim
    n = widx.shape[0]
    tail = hb + n_hist + n
    sk, sv = scratch
    dpsynth.kv_fill_device(sk, "bf16", w.seed, dpsynth.STREAM_K, l, cap, heads * D)
    dpsynth.kv_fill_device(sv, "bf16", w.seed, dpsynth.STREAM_V, l, cap, heads * D)
    _tie_to_host(sk, w, l, dpsynth.STREAM_K, cap, heads)
    _tie_to_host(sv, w, l, dpsynth.STREAM_V, cap, heads)
    worst, inexact = 0.0, 0
    for lo, hi in ((0, C), (hb, hb + n_hist)):
        if old_tabd is None:
            assert _same(ks[l][lo:hi], sk[lo:hi]), l
        else:
            zero = torch.zeros(hi - lo, dtype=torch.int64, device=dev)
            e, ne = _check_rotated(ks[l][lo:hi], sk[lo:hi], zero, old_tabd, w.rope_pairs)
            worst, inexact = max(worst, e), inexact + ne
    assert _same(ks[l][C:hb], sk[C:hb]) and _same(ks[l][tail:], sk[tail:]), l
    src = _i64(slot_begin + widx, dev)
    e, ne = _check_rotated(ks[l][hb + n_hist:tail], sk.index_select(0, src),
                           _i64(rf[slot_begin + widx], dev), tabd, w.rope_pairs)
    worst, inexact = max(worst, e), inexact + ne
    assert _same(vs[l][:hb + n_hist], sv[:hb + n_hist]) and _same(vs[l][tail:], sv[tail:]), l
    assert _same(vs[l][hb + n_hist:tail], sv.index_select(0, src)), l
    return worst, inexact


def _append_step(w, dev, heads, cap, ks, vs, rf, tail0, x0, xf, d):
    """The device buffers of one ring-layout eviction and the leaving chunk's
    kept-index list (dp_score_index)."""
    C, D, L = w.chunk_tokens, w.head_dim, w.n_layers
    kv = dp.dp_kv_inplace()
    ak, av = dp.ptr_array(ks, dev), dp.ptr_array(vs, dev)
    kv.k_layers, kv.v_layers = ak.data_ptr(), av.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, heads, D, dp.DP_BF16
    kv.capacity = cap
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv.dev_error = err.data_ptr()
    keep = torch.empty(C, dtype=torch.uint8, device=dev)
    idx = torch.empty(C, dtype=torch.int32, device=dev)
    nk = torch.zeros(1, dtype=torch.int64, device=dev)
    ws_si = torch.zeros(dp.dp_score_index_workspace_bytes(C) // 8 + 1, dtype=torch.int64,
                        device=dev)
    dp.dp_score_index(torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev), d, d,
                      dp.make_policy(C, 0, 0, 0, C, w.gamma), None, keep, idx, nk, None, None,
                      ws_si, err)
    tail = torch.tensor([tail0], dtype=torch.int64, device=dev)
    rf_d = torch.from_numpy(rf).to(dev)
    return dict(kv=kv, ak=ak, av=av, err=err, idx=idx, nk=nk, tail=tail, rf_d=rf_d)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_steady_step_full_size(layout):
    """The steady-state step of the one-minute rollout in the ring layout, as
    bench.py times it: 40 x 40 x 128 bf16, [sink | 4 ring slots | history of
    the retained rows of chunks 1-55 | room]; chunk 56 leaves the window for
    q0 = 240.  The sink and history move by the uniform step 3.5 frames
    (dp_rope_shift), the leaving chunk's kept rows are appended with their
    first re-index fused; either key layout.  Every row of all 40 layers
    against the oracle's tables applied to the regenerated fill."""
    dev = device()
    w = dpsynth.WORKLOADS["reindex"]
    L, H, D, C = w.n_layers, w.n_heads, w.head_dim, w.chunk_tokens
    rf, n_hist, hb, cap = _ring_setup(w, 55)
    slot_begin = C
    ks = _fill(dev, w, cap, range(L), dpsynth.STREAM_K)
    _to_layout(ks, layout, w.rope_pairs)
    vs = _fill(dev, w, cap, range(L), dpsynth.STREAM_V)
    we = dpsynth.WORKLOADS["eviction"]
    x0, xf = dpsynth.score_inputs(we)
    widx = oracle.compact(oracle.mask(oracle.score_f32(x0, xf, we.d), C, 0, 0, 0, C, w.gamma))
    n = widx.shape[0]
    host = _rope_host(w, q0=w.q0 - 4)                 # phases after the previous step (q0 = 236)
    phase0 = _tables(host)[3]
    host = dict(host, q0=w.q0, frame_phase=phase0)
    rd = _rope_dev(host, dev)
    rope = dp.make_rope(rd["theta"], rd["frame_t"], rd["frame_phase"], host["q0"], host["knee"],
                        host["inv_factor"], key_layout=layout)
    ws_r = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    st = _append_step(w, dev, H, cap, ks, vs, rf, hb + n_hist, x0, xf, we.d)
    ws_s = torch.empty(dp.dp_rope_shift_workspace_bytes(w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    step = 4 * (1 - 1 / w.rope_factor)
    ak = st["ak"]
    dp.dp_rope_shift(ak, L, H, D, dp.DP_BF16, 0, C, None, rd["theta"], 0, w.rope_pairs, step, ws_s,
                     key_layout=layout)
    dp.dp_rope_shift(ak, L, H, D, dp.DP_BF16, hb, cap, st["tail"], rd["theta"], 0, w.rope_pairs,
                     step, ws_s, key_layout=layout)
    dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
    dp.dp_append_kept(st["kv"], slot_begin, C, st["idx"], st["nk"], st["tail"], st["rf_d"], rope,
                      ws_r)
    torch.cuda.synchronize()
    assert st["err"].item() == 0 and st["nk"].item() == n and st["tail"].item() == hb + n_hist + n
    tables = _tables(host)
    assert np.array_equal(rd["frame_phase"].cpu().numpy(), tables[3])
    rf_after = st["rf_d"].cpu().numpy()
    assert np.all(rf_after[slot_begin:slot_begin + C] == -1)
    assert np.array_equal(rf_after[hb + n_hist:hb + n_hist + n], rf[slot_begin + widx])
    uniform = _tables_dev(oracle.rope_uniform(host["theta"], step), dev)
    tabd = _tables_dev(tables, dev)
    scratch = (torch.empty_like(ks[0]), torch.empty_like(vs[0]))
    nat = _Natural(ks, layout, w.rope_pairs)
    worst, inexact = 0.0, 0
    for l in range(L):
        e, ne = _check_ring_layer(w, l, H, cap, nat, vs, hb, n_hist, slot_begin, widx, rf, uniform,
                                  tabd, dev, scratch)
        worst, inexact = max(worst, e), inexact + ne
    print("steady step (layout %d): %d history rows, %d appended, every row of %d layers, max "
          "|key error| %.3g, %d key elements off the float64 rotation's bf16"
          % (layout, n_hist, n, L, worst, inexact))
    del ks, vs, scratch
    _free()


@pytest.mark.parametrize("layout", LAYOUTS)
def test_append_step_full_size(layout):
    """The eviction step in the ring layout as bench.py times it (the append
    workload): 40 x 40 x 128 bf16 at the two-minute shape, one buffer per
    layer [sink | 4 ring slots | room for one chunk of history]; the chunk in
    ring slot 0 leaves the window: its kept rows are appended at the tail (K
    and V, all layers), then dp_rope_prepare and dp_rope_apply over the sink
    and over the history [T, tail) re-index the old keys for q0 = 20; either
    key layout.  Every row of all 40 layers against the regenerated fill."""
    dev = device()
    w = dpsynth.WORKLOADS["eviction"]
    T, H, D, L, C = w.seq_len, w.n_heads, w.head_dim, w.n_layers, w.chunk_tokens
    cap, slot_begin = T + C, C
    ks = _fill(dev, w, cap, range(L), dpsynth.STREAM_K)
    _to_layout(ks, layout, w.rope_pairs)
    vs = _fill(dev, w, cap, range(L), dpsynth.STREAM_V)
    x0, xf = dpsynth.score_inputs(w)
    widx = oracle.compact(oracle.mask(oracle.score_f32(x0, xf, w.d), C, 0, 0, 0, C, w.gamma))
    n = widx.shape[0]
    rf = np.full(cap, -1, np.int32)
    rf[:T] = dpsynth.row_frame(w)
    host = _rope_host(w)
    rd = _rope_dev(host, dev)
    rope = dp.make_rope(rd["theta"], rd["frame_t"], rd["frame_phase"], host["q0"], host["knee"],
                        host["inv_factor"], key_layout=layout)
    ws_r = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    st = _append_step(w, dev, H, cap, ks, vs, rf, T, x0, xf, w.d)
    dp.dp_append_kept(st["kv"], slot_begin, C, st["idx"], st["nk"], st["tail"], st["rf_d"])
    dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
    dp.dp_rope_apply(st["ak"], L, H, D, dp.DP_BF16, 0, w.sink_len, None, st["rf_d"], rope, ws_r)
    dp.dp_rope_apply(st["ak"], L, H, D, dp.DP_BF16, T, cap, st["tail"], st["rf_d"], rope, ws_r)
    torch.cuda.synchronize()
    assert st["err"].item() == 0 and st["nk"].item() == n and st["tail"].item() == T + n
    tables = _tables(host)
    assert np.array_equal(rd["frame_phase"].cpu().numpy(), tables[3])
    rf_after = st["rf_d"].cpu().numpy()
    assert np.all(rf_after[slot_begin:slot_begin + C] == -1)
    assert np.array_equal(rf_after[T:T + n], rf[slot_begin + widx])
    tabd = _tables_dev(tables, dev)
    sk, sv = torch.empty_like(ks[0]), torch.empty_like(vs[0])
    nat = _Natural(ks, layout, w.rope_pairs)
    sink = w.sink_len
    src = _i64(slot_begin + widx, dev)
    rf_sink, rf_app = _i64(rf[:sink], dev), _i64(rf[slot_begin + widx], dev)
    worst, inexact = 0.0, 0
    for l in range(L):
        dpsynth.kv_fill_device(sk, "bf16", w.seed, dpsynth.STREAM_K, l, cap, H * D)
        dpsynth.kv_fill_device(sv, "bf16", w.seed, dpsynth.STREAM_V, l, cap, H * D)
        _tie_to_host(sk, w, l, dpsynth.STREAM_K, cap)
        _tie_to_host(sv, w, l, dpsynth.STREAM_V, cap)
        g = nat[l]
        e, ne = _check_rotated(g[:sink], sk[:sink], rf_sink, tabd, w.rope_pairs)
        worst, inexact = max(worst, e), inexact + ne
        assert _same(g[sink:T], sk[sink:T]) and _same(g[T + n:], sk[T + n:]), l
        e, ne = _check_rotated(g[T:T + n], sk.index_select(0, src), rf_app, tabd, w.rope_pairs)
        worst, inexact = max(worst, e), inexact + ne
        assert _same(vs[l][:T], sv[:T]) and _same(vs[l][T + n:], sv[T + n:]), l
        assert _same(vs[l][T:T + n], sv.index_select(0, src)), l
    print("append step (layout %d): %d rows appended, every row of %d layers, max |key error| "
          "%.3g, %d key elements off the float64 rotation's bf16" % (layout, n, L, worst, inexact))
    del ks, vs, sk, sv
    _free()


def test_steady_lazy_step_full_size():
    """The steady-state step on the compressed time axis, as bench.py times it
    (workload steady_lazy): 40 x 40 x 128 bf16, [sink | 4 ring slots | history
    of the retained rows of chunks 1-55 | room]; chunk 56 leaves the window for
    q0 = 240.  No old key is written; the leaving chunk's kept rows are
    appended with its frames moved from phase t to t/c (fused).  Every row of
    all 40 layers against the oracle's compressed-axis tables applied to the
    regenerated fill."""
    dev = device()
    w = dpsynth.WORKLOADS["reindex"]
    L, H, D, C = w.n_layers, w.n_heads, w.head_dim, w.chunk_tokens
    rf, n_hist, hb, cap = _ring_setup(w, 55)
    slot_begin = C
    ks = _fill(dev, w, cap, range(L), dpsynth.STREAM_K)
    vs = _fill(dev, w, cap, range(L), dpsynth.STREAM_V)
    we = dpsynth.WORKLOADS["eviction"]
    x0, xf = dpsynth.score_inputs(we)
    widx = oracle.compact(oracle.mask(oracle.score_f32(x0, xf, we.d), C, 0, 0, 0, C, w.gamma))
    n = widx.shape[0]
    host = _rope_host(w, q0=w.q0 - 4)                 # phases after the previous step (q0 = 236)
    phase0 = _tables(host, compressed=True)[3]
    host = dict(host, q0=w.q0, frame_phase=phase0)
    rd = _rope_dev(host, dev)
    rope = dp.make_rope(rd["theta"], rd["frame_t"], rd["frame_phase"], host["q0"], host["knee"],
                        host["inv_factor"], axis=dp.DP_AXIS_COMPRESSED)
    ws_r = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    st = _append_step(w, dev, H, cap, ks, vs, rf, hb + n_hist, x0, xf, we.d)
    dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
    dp.dp_append_kept(st["kv"], slot_begin, C, st["idx"], st["nk"], st["tail"], st["rf_d"], rope,
                      ws_r)
    torch.cuda.synchronize()
    assert st["err"].item() == 0 and st["nk"].item() == n and st["tail"].item() == hb + n_hist + n
    tables = _tables(host, compressed=True)
    assert np.array_equal(rd["frame_phase"].cpu().numpy(), tables[3])
    moved = np.flatnonzero(tables[0] != 0)                   # frames whose phase changes
    assert np.array_equal(moved, np.arange(224, 228))       # chunk 56 only: t -> t/c
    rf_after = st["rf_d"].cpu().numpy()
    assert np.all(rf_after[slot_begin:slot_begin + C] == -1)
    assert np.array_equal(rf_after[hb + n_hist:hb + n_hist + n], rf[slot_begin + widx])
    tabd = _tables_dev(tables, dev)
    scratch = (torch.empty_like(ks[0]), torch.empty_like(vs[0]))
    worst, inexact = 0.0, 0
    for l in range(L):
        e, ne = _check_ring_layer(w, l, H, cap, ks, vs, hb, n_hist, slot_begin, widx, rf, None,
                                  tabd, dev, scratch)
        worst, inexact = max(worst, e), inexact + ne
    print("compressed-axis steady step: %d history rows, %d appended, every row of %d layers, "
          "max |key error| %.3g, %d key elements off the float64 rotation's bf16"
          % (n_hist, n, L, worst, inexact))
    del ks, vs, scratch
    _free()


def test_hs_ring_step_full_size():
    """The HS eviction step in the ring layout, as bench.py times it (workload
    hs_ring): per layer the 20 dynamic heads of the HS workload keep one
    token-major cache [sink | 4 ring slots | history of the retained rows of
    chunks 1-25 | room] (20 x 128 bf16 per row, 40 layers); chunk 26 leaves the
    window for q0 = 120 and its kept rows are appended to every layer's dynamic
    cache with the re-index fused on the compressed axis.  Every row of all 40
    layers against the oracle; the static class's cache is not touched by the
    call."""
    dev = device()
    w = dpsynth.WORKLOADS["hs"]
    L, D, C = w.n_layers, w.head_dim, w.chunk_tokens
    HC = w.n_heads // 2
    rf, n_hist, hb, cap = _ring_setup(w, 25)
    slot_begin = C
    ks = _fill(dev, w, cap, range(L), dpsynth.STREAM_K, heads=HC)
    vs = _fill(dev, w, cap, range(L), dpsynth.STREAM_V, heads=HC)
    we = dpsynth.WORKLOADS["eviction"]
    x0, xf = dpsynth.score_inputs(we)
    widx = oracle.compact(oracle.mask(oracle.score_f32(x0, xf, we.d), C, 0, 0, 0, C, w.gamma))
    n = widx.shape[0]
    host = _rope_host(w, q0=w.q0 - 4)                 # phases after the previous step (q0 = 116)
    phase0 = _tables(host, compressed=True)[3]
    host = dict(host, q0=w.q0, frame_phase=phase0)
    rd = _rope_dev(host, dev)
    rope = dp.make_rope(rd["theta"], rd["frame_t"], rd["frame_phase"], host["q0"], host["knee"],
                        host["inv_factor"], axis=dp.DP_AXIS_COMPRESSED)
    ws_r = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    st = _append_step(w, dev, HC, cap, ks, vs, rf, hb + n_hist, x0, xf, we.d)
    dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
    dp.dp_append_kept(st["kv"], slot_begin, C, st["idx"], st["nk"], st["tail"], st["rf_d"], rope,
                      ws_r)
    torch.cuda.synchronize()
    assert st["err"].item() == 0 and st["nk"].item() == n and st["tail"].item() == hb + n_hist + n
    tables = _tables(host, compressed=True)
    assert np.array_equal(rd["frame_phase"].cpu().numpy(), tables[3])
    assert np.array_equal(np.flatnonzero(tables[0] != 0), np.arange(104, 108))   # chunk 26 only
    rf_after = st["rf_d"].cpu().numpy()
    assert np.all(rf_after[slot_begin:slot_begin + C] == -1)                  # the slot is retired
    assert np.array_equal(rf_after[hb + n_hist:hb + n_hist + n], rf[slot_begin + widx])
    tabd = _tables_dev(tables, dev)
    scratch = (torch.empty_like(ks[0]), torch.empty_like(vs[0]))
    worst, inexact = 0.0, 0
    for l in range(L):
        e, ne = _check_ring_layer(w, l, HC, cap, ks, vs, hb, n_hist, slot_begin, widx, rf, None,
                                  tabd, dev, scratch)
        worst, inexact = max(worst, e), inexact + ne
    print("HS ring step: %d history rows, %d appended, every row of %d layers, max |key error| "
          "%.3g, %d key elements off the float64 rotation's bf16" % (n_hist, n, L, worst, inexact))
    del ks, vs, scratch
    _free()
