"""Seeded sweeps over shapes inside the ABI's contract.

Each case draws a shape (layers, rows, heads, head_dim, dtype), a keep mask of
a random rate with a sink and a window, a tokens-per-frame count and a
temporal pair range, and checks one entry point against the oracle: the kept
index list and the physical gather of K[m], V[m] (DeCoPrune page, section
어떻게 동작하나), with or without the fused re-index of the key temporal
phase (section 무엇과 다른가), the in-place re-index over a row range whose
end is a device count, the ring-layout append, attention, the one-launch
index phase and the DeCoPrune-HS gather and re-index.  Bars as
elsewhere: index lists, V and untouched keys bit for bit, re-indexed keys
within 2e-2 (bf16) or 1e-5 (fp32), attention within the derived bound.
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import oracle
from gpu_helpers import bits, device, keys_close, to_dev
from test_gpu_parity import TOL, _dev_layers, _gpu_idx, _kv_struct, _layers, _rope_inputs

pytestmark = pytest.mark.gpu


def _draw(rng):
    dtype = dp.DP_BF16 if rng.random() < 0.7 else dp.DP_F32
    per16 = 8 if dtype == dp.DP_BF16 else 4            # elements per 16 bytes
    D = per16 * int(rng.integers(1, 17))               # 16 .. 256 bytes per head row
    H = int(rng.integers(1, 25))
    T = int(rng.integers(1, 2500))
    L = int(rng.integers(1, 4))
    tpf = int(rng.integers(1, 150))
    step = per16 // 2                                  # pairs per 16 bytes
    pb = step * int(rng.integers(0, D // 2 // step))
    npairs = int(rng.integers(1, D // 2 - pb + 1))
    return L, T, H, D, dtype, tpf, pb, npairs


CASES = list(range(24))


@pytest.mark.parametrize("case", CASES)
def test_gather_sweep(case):
    dev = device()
    rng = np.random.default_rng(1000 + case)
    L, T, H, D, dtype, tpf, pb, npairs = _draw(rng)
    fused = case % 3 != 0
    axis = dp.DP_AXIS_COMPRESSED if case % 4 == 1 else dp.DP_AXIS_PAGE
    with_v = case % 5 != 0
    sink, window = int(rng.integers(0, T + 1)), 0
    window = int(rng.integers(0, T - sink + 1))
    keep = (rng.random(T) < rng.random()).astype(np.uint8)
    keep[:sink] = 1
    keep[T - window:] = 1
    kb = _layers(rng, L, T, H, D, dtype, scale=3.0)
    vb = _layers(rng, L, T, H, D, dtype)
    rf = (np.arange(T) // tpf).astype(np.int32)
    n_frames = (T + tpf - 1) // tpf
    cap = T if case % 2 == 0 else int(keep.sum())        # a destination of exactly the kept rows
    k_src, v_src = _dev_layers(kb, dtype, dev), _dev_layers(vb, dtype, dev)
    tdt = torch.bfloat16 if dtype == dp.DP_BF16 else torch.float32
    k_dst = [torch.zeros((cap + 4, H, D), dtype=tdt, device=dev) for _ in range(L)]
    v_dst = [torch.zeros((cap + 4, H, D), dtype=tdt, device=dev) for _ in range(L)] if with_v else None
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive = []
    kv = _kv_struct(k_src, v_src if with_v else None, k_dst, v_dst, cap, err, alive)
    idx, n, rf_out = _gpu_idx(keep, dev, rf)
    host, devt = _rope_inputs(rng, n_frames, npairs, float(n_frames) + float(rng.random()),
                              float(rng.integers(0, 8)), float(rng.integers(1, 9)), dev,
                              bool(case % 2))
    if fused:
        rope = dp.make_rope(devt["theta"], devt["frame_t"], devt["frame_phase"], host["q0"],
                            host["knee"], host["inv_factor"], pb, axis=axis)
        ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, npairs) // 4 + 4,
                         dtype=torch.float32, device=dev)
        dp.dp_gather_kv(kv, idx, n, rf_out, rope, ws)
    else:
        dp.dp_gather_kv(kv, idx, n)
    torch.cuda.synchronize()
    widx = oracle.compact(keep)
    m = widx.shape[0]
    assert int(n.item()) == m and err.item() == 0, (case, m)
    assert np.array_equal(idx[:m].cpu().numpy(), widx)
    kk = kb.view(np.float32) if dtype == dp.DP_F32 else kb
    wk = oracle.gather(kk, widx)
    if fused:
        tables = oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"],
                                    host["knee"], host["inv_factor"], host["theta"],
                                    compressed=axis == dp.DP_AXIS_COMPRESSED)
        wrf = oracle.gather_i32(rf, widx)
        for l in range(L):
            oracle.rope_rows(wk[l], wrf, pb, tables)
        assert np.array_equal(devt["frame_phase"].cpu().numpy(), tables[3])
    wk_bits = wk.view(np.uint32) if dtype == dp.DP_F32 else wk
    for l in range(L):
        if fused:
            ok, worst, _ = keys_close(bits(k_dst[l][:m]), wk_bits[l], TOL[dtype])
            assert ok, (case, l, worst)
        else:
            assert np.array_equal(bits(k_dst[l][:m]), wk_bits[l]), (case, l)
        assert np.all(bits(k_dst[l][m:]) == 0), (case, l)
    if with_v:
        wv = oracle.gather(vb, widx)
        for l in range(L):
            assert np.array_equal(bits(v_dst[l][:m]), wv[l]), (case, l)
            assert np.all(bits(v_dst[l][m:]) == 0), (case, l)


@pytest.mark.parametrize("case", CASES)
def test_reindex_sweep(case):
    dev = device()
    rng = np.random.default_rng(2000 + case)
    L, T, H, D, dtype, tpf, pb, npairs = _draw(rng)
    kb = _layers(rng, L, T, H, D, dtype, scale=3.0)
    rf = (np.arange(T) // tpf).astype(np.int32)
    if case % 3 == 0:
        rf[rng.random(T) < 0.05] = -1                  # rows with no key: left alone
    n_frames = (T + tpf - 1) // tpf
    n_rows = int(rng.integers(0, T + 1))               # device-side end of the visible rows
    k = _dev_layers(kb, dtype, dev)
    host, devt = _rope_inputs(rng, n_frames, npairs, float(n_frames) + float(rng.random()),
                              float(rng.integers(0, 8)), float(rng.integers(1, 9)), dev,
                              bool(case % 2))
    axis = dp.DP_AXIS_COMPRESSED if case % 4 == 1 else dp.DP_AXIS_PAGE
    rope = dp.make_rope(devt["theta"], devt["frame_t"], devt["frame_phase"], host["q0"],
                        host["knee"], host["inv_factor"], pb, axis=axis)
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, npairs) // 4 + 4, dtype=torch.float32,
                     device=dev)
    arr = dp.ptr_array(k, dev)
    nr = torch.tensor([n_rows], dtype=torch.int64, device=dev)
    dp.dp_rope_reindex(arr, L, H, D, dtype, T, nr, to_dev(rf, dev), rope, ws)
    torch.cuda.synchronize()
    kk = (kb.view(np.float32) if dtype == dp.DP_F32 else kb).copy()
    tables = oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"], host["knee"],
                                host["inv_factor"], host["theta"],
                                compressed=axis == dp.DP_AXIS_COMPRESSED)
    no_key = rf < 0                                    # the oracle takes frames in range only:
    rf_in = np.where(no_key, 0, rf).astype(np.int32)   # such rows are restored afterwards
    orig = kk.copy()
    for l in range(L):
        oracle.rope_rows(kk[l, :n_rows], rf_in[:n_rows], pb, tables)
    kk[:, no_key] = orig[:, no_key]
    want = kk.view(np.uint32) if dtype == dp.DP_F32 else kk
    for l in range(L):
        got = bits(k[l])
        ok, worst, _ = keys_close(got[:n_rows], want[l, :n_rows], TOL[dtype])
        assert ok, (case, l, worst)
        assert np.array_equal(got[n_rows:], want[l, n_rows:]), (case, l)   # rows past the end
    assert np.array_equal(devt["frame_phase"].cpu().numpy(), tables[3])


@pytest.mark.parametrize("case", list(range(16)))
def test_append_sweep(case):
    """dp_append_kept at random ring shapes: the slot's kept rows land at the
    tail (all layers, K and V), the slot's frames are retired and the tail
    advances (section 어떻게 동작하나); with the fused re-index the appended
    keys also take their frames' phase step (section 무엇과 다른가)."""
    from test_gpu_append import _buf, _dev, _inplace, _slot_index
    dev = device()
    rng = np.random.default_rng(3000 + case)
    L, _, H, D, dtype, tpf, pb, npairs = _draw(rng)
    C = int(rng.integers(1, 400))
    R = int(rng.integers(1, 5))
    sink = int(rng.integers(0, 100))
    hist = int(rng.integers(C, 3 * C + 1))
    cap = sink + R * C + hist
    slot = int(rng.integers(0, R))
    slot_begin = sink + slot * C
    tail0 = int(rng.integers(sink + R * C, cap - C + 1))
    fused = case % 2 == 1
    with_v = case % 3 != 0
    keep = (rng.random(C) < rng.random()).astype(np.uint8)
    kb, vb = _buf(rng, L, cap, H, D, dtype), _buf(rng, L, cap, H, D, dtype)
    n_frames = (cap + tpf - 1) // tpf
    rf = (np.arange(cap) // tpf).astype(np.int32)
    k, v = _dev(kb, dtype, dev), (_dev(vb, dtype, dev) if with_v else None)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive = []
    kv = _inplace(k, v, dtype, cap, err, alive)
    idx, n = _slot_index(keep, dev)
    tail = torch.tensor([tail0], dtype=torch.int64, device=dev)
    rf_d = to_dev(rf, dev)
    host, devt = _rope_inputs(rng, n_frames, npairs, float(n_frames) + float(rng.random()),
                              float(rng.integers(0, 8)), float(rng.integers(1, 9)), dev,
                              bool(case % 4 == 0))
    if fused:
        rope = dp.make_rope(devt["theta"], devt["frame_t"], devt["frame_phase"], host["q0"],
                            host["knee"], host["inv_factor"], pb)
        ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, npairs) // 4 + 4,
                         dtype=torch.float32, device=dev)
        dp.dp_rope_prepare(rope, D, dtype, ws)
        dp.dp_append_kept(kv, slot_begin, C, idx, n, tail, rf_d, rope, ws)
    else:
        dp.dp_append_kept(kv, slot_begin, C, idx, n, tail, rf_d)
    torch.cuda.synchronize()
    widx = oracle.compact(keep)
    m = widx.shape[0]
    assert err.item() == 0 and tail.item() == tail0 + m, case
    kk = (kb.view(np.float32) if dtype == dp.DP_F32 else kb).copy()
    rfo = rf.copy()
    t1 = oracle.append_kept(kk, slot_begin, C, widx, tail0, rfo)
    assert t1 == tail0 + m
    assert np.array_equal(rf_d.cpu().numpy(), rfo), case
    if fused:
        tables = oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"],
                                    host["knee"], host["inv_factor"], host["theta"])
        for l in range(L):
            sub = np.ascontiguousarray(kk[l, tail0:tail0 + m])
            oracle.rope_rows(sub, rfo[tail0:tail0 + m], pb, tables)
            kk[l, tail0:tail0 + m] = sub
        assert np.array_equal(devt["frame_phase"].cpu().numpy(), tables[3])
    want = kk.view(np.uint32) if dtype == dp.DP_F32 else kk
    for l in range(L):
        got = bits(k[l])
        ok, worst, _ = keys_close(got[tail0:tail0 + m], want[l, tail0:tail0 + m], TOL[dtype])
        assert ok, (case, l, worst)
        rest = np.ones(cap, bool)
        rest[tail0:tail0 + m] = False
        assert np.array_equal(got[rest], want[l][rest]), (case, l)     # nothing else moves
    if with_v:
        vv = vb.copy()
        oracle.append_kept(vv, slot_begin, C, widx, tail0, None)
        for l in range(L):
            assert np.array_equal(bits(v[l]), vv[l]), (case, l)


@pytest.mark.parametrize("case", list(range(10)))
def test_attention_sweep(case):
    """dp_attention (the next chunk's queries over the compacted cache, the
    step the page's continuation speed-up comes from, section 무엇인가) at
    random query and key counts, head counts and scales, the key count on the
    device or the host, every output against the float64 oracle under the
    derived bound."""
    from gpu_helpers import bf16_abs, bf16_from_bits, bf16_norms, check_attention, random_bf16_bits
    dev = device()
    rng = np.random.default_rng(4000 + case)
    D = 128
    n_q = int(rng.integers(1, 600))
    n_kv = int(rng.integers(1, 1500))
    H = int(rng.integers(1, 10))
    scale = float(np.exp(rng.uniform(np.log(0.02), np.log(0.5))))
    q = random_bf16_bits(rng, (n_q, H, D))
    extra = int(rng.integers(0, 70))
    k = random_bf16_bits(rng, (n_kv + extra, H, D))
    v = random_bf16_bits(rng, (n_kv + extra, H, D))
    k[n_kv:] = 0x7FC0                                 # rows past the count are never read
    v[n_kv:] = 0x7FC0
    qd, kd, vd = bf16_from_bits(q, dev), bf16_from_bits(k, dev), bf16_from_bits(v, dev)
    od = torch.zeros((n_q, H, D), dtype=torch.bfloat16, device=dev)
    if case % 2:
        dp.dp_attention(qd, kd, vd, od, n_q, n_kv + extra,
                        torch.tensor([n_kv], dtype=torch.int64, device=dev), H, D, dp.DP_BF16,
                        scale)
    else:
        dp.dp_attention(qd, kd, vd, od, n_q, n_kv, None, H, D, dp.DP_BF16, scale)
    torch.cuda.synchronize()
    rows = np.arange(n_q)
    want = oracle.attention(q, k, v, rows, n_kv=n_kv, scale=scale)
    want_abs = oracle.attention(q, k, bf16_abs(v), rows, n_kv=n_kv, scale=scale)
    kmax = bf16_norms(k[:n_kv]).max(axis=0)
    check_attention(bits(od), want, want_abs, bf16_norms(q), kmax, scale, n_kv, ("sweep", case))


@pytest.mark.parametrize("case", list(range(16)))
def test_score_index_sweep(case):
    """dp_score_index (score, threshold mask, kept-index list in one launch;
    section 어떻게 동작하나) at random sequence lengths, policies (sink,
    window, scored range, threshold, reversed criterion, Streaming) and score
    widths, one zero-filled workspace for all cases of a size: scores, mask,
    list, count and gathered row frames bit for bit."""
    from test_gpu_score_index import Fused, _score_case as score_case
    dev = device()
    rng = np.random.default_rng(5000 + case)
    T = int(rng.integers(1, 40000))
    sink = int(rng.integers(0, T + 1))
    window = int(rng.integers(0, T - sink + 1))
    sb = int(rng.integers(sink, T - window + 1))
    ns = int(rng.integers(0, T - window - sb + 1))
    d = int(rng.integers(1, 257))
    stride = d + int(rng.integers(0, 9))
    reversed_ = bool(case % 3 == 1)
    streaming = bool(case % 5 == 4)
    x0, xf = score_case(rng, max(ns, 1), d, stride)
    x0, xf = x0[:ns], xf[:ns]
    ell = oracle.score_f32(x0, xf, d) if ns else np.zeros(0, np.float32)
    gamma = float(np.nanmedian(ell)) if ns and rng.random() < 0.5 else float(rng.random() * 2)
    pol = dp.make_policy(T, sink, window, sb, ns, gamma, reversed_,
                         dp.DP_MODE_STREAMING if streaming else dp.DP_MODE_SCORE)
    want = oracle.mask(ell if ns else None, T, sink, window, sb, ns, gamma, reversed_, streaming)
    rf = rng.integers(0, 1 << 30, T).astype(np.int32)
    f = Fused(dev, T)
    ell_d = torch.full((max(ns, 1),), -1.0, dtype=torch.float32, device=dev)
    dummy = np.zeros((1, stride), np.float32)
    x0d = to_dev(np.ascontiguousarray(x0) if ns else dummy, dev)
    xfd = to_dev(np.ascontiguousarray(xf) if ns else dummy, dev)
    for rep in range(2):                               # the workspace is left ready for the next call
        f.run(x0d, xfd, d, stride, pol, ell_d, to_dev(rf, dev))
        f.check(T, want, rf)
    if ns and not streaming:
        got = ell_d[:ns].cpu().numpy()
        both_nan = np.isnan(got) & np.isnan(ell)
        assert np.array_equal(got.view(np.uint32)[~both_nan], ell.view(np.uint32)[~both_nan]), case


@pytest.mark.parametrize("case", list(range(12)))
def test_hs_sweep(case):
    """DeCoPrune-HS at random shapes (section 무엇과 다른가): 1 to 8 head
    classes with their own kept-row lists, a random class per (layer, head),
    list capacities with or without slack, the gather with or without the
    fused re-index, or followed by the re-index of the packed cache."""
    dev = device()
    rng = np.random.default_rng(6000 + case)
    L, T, H, D, dtype, tpf, pb, npairs = _draw(rng)
    T = min(T, 1500)
    nc = int(rng.integers(1, dp.DP_HS_MAX_CLASSES + 1))
    mode = case % 3                                     # 0 plain, 1 fused, 2 separate re-index
    lists_h = [np.flatnonzero(rng.random(T) < rng.random()).astype(np.int32) for _ in range(nc)]
    cls = rng.integers(0, nc, (L, H)).astype(np.uint8)
    wlens = np.array([len(x) for x in lists_h], np.int64)
    woff = oracle.hs_offsets(cls, wlens)
    total = int(woff[-1])
    caps = [int(wlens[c]) + (int(rng.integers(0, 50)) if rng.random() < 0.5 else 0) for c in range(nc)]
    rf = (np.arange(T) // tpf).astype(np.int32)
    n_frames = (T + tpf - 1) // tpf
    kb, vb = _layers(rng, L, T, H, D, dtype, scale=3.0), _layers(rng, L, T, H, D, dtype)
    lists = [torch.zeros(max(1, caps[c]), dtype=torch.int32, device=dev) for c in range(nc)]
    rfs = [torch.zeros(max(1, caps[c]), dtype=torch.int32, device=dev) for c in range(nc)]
    for c in range(nc):
        if wlens[c]:
            lists[c][:wlens[c]] = to_dev(lists_h[c], dev)
            rfs[c][:wlens[c]] = to_dev(rf[lists_h[c]], dev)
    lens = to_dev(wlens, dev)
    head_class = to_dev(cls.ravel(), dev)
    offsets = torch.empty(L * H + 1, dtype=torch.int64, device=dev)
    dp.dp_hs_offsets(head_class, L, H, lens, nc, offsets)
    tdt = torch.bfloat16 if dtype == dp.DP_BF16 else torch.float32
    k_out = torch.zeros((total + 8, D), dtype=tdt, device=dev)
    v_out = torch.zeros((total + 8, D), dtype=tdt, device=dev)
    k_src, v_src = _dev_layers(kb, dtype, dev), _dev_layers(vb, dtype, dev)
    kv = dp.dp_kv_hs()
    arrs = [dp.ptr_array(k_src, dev), dp.ptr_array(v_src, dev)]
    kv.k_src, kv.v_src = arrs[0].data_ptr(), arrs[1].data_ptr()
    kv.k_out, kv.v_out = k_out.data_ptr(), v_out.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dtype
    kv.src_rows, kv.out_capacity = T, total
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv.dev_error = err.data_ptr()
    cidx, crf = dp.ptr_array(lists, dev), dp.ptr_array(rfs, dev)
    host, devt = _rope_inputs(rng, n_frames, npairs, float(n_frames) + float(rng.random()),
                              float(rng.integers(0, 8)), float(rng.integers(1, 9)), dev,
                              bool(case % 2))
    rope = dp.make_rope(devt["theta"], devt["frame_t"], devt["frame_phase"], host["q0"],
                        host["knee"], host["inv_factor"], pb)
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, npairs) // 4 + 4, dtype=torch.float32,
                     device=dev)
    if mode == 1:
        dp.dp_hs_gather_kv(kv, head_class, nc, cidx, lens, caps, offsets, crf, rope, ws)
    else:
        dp.dp_hs_gather_kv(kv, head_class, nc, cidx, lens, caps, offsets)
        if mode == 2:
            dp.dp_hs_rope_reindex(k_out, total, L, H, D, dtype, head_class, nc, lens, caps,
                                  offsets, crf, rope, ws)
    torch.cuda.synchronize()
    assert err.item() == 0, case
    assert np.array_equal(offsets.cpu().numpy(), woff)
    kk = kb.view(np.float32) if dtype == dp.DP_F32 else kb
    w_k = np.zeros((total, D), kk.dtype)
    w_v = np.zeros((total, D), vb.dtype)
    for l in range(L):
        oracle.hs_gather_layer(kk[l], l, cls, lists_h, woff, w_k)
        oracle.hs_gather_layer(vb[l], l, cls, lists_h, woff, w_v)
    assert np.array_equal(bits(v_out[:total]), w_v), case
    if mode:
        tables = oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"],
                                    host["knee"], host["inv_factor"], host["theta"])
        w_rf = np.zeros(total, np.int32)
        for i in range(L * H):
            w_rf[woff[i]:woff[i + 1]] = rf[lists_h[cls.ravel()[i]]]
        oracle.rope_headrows(w_k, w_rf, pb, tables)
        assert np.array_equal(devt["frame_phase"].cpu().numpy(), tables[3])
    want = w_k.view(np.uint32) if dtype == dp.DP_F32 else w_k
    if mode:
        ok, worst, _ = keys_close(bits(k_out[:total]), want, TOL[dtype])
        assert ok, (case, worst)
    else:
        assert np.array_equal(bits(k_out[:total]), want), case
    assert np.all(bits(k_out[total:]) == 0) and np.all(bits(v_out[total:]) == 0)
