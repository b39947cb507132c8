"""GPU parity of the split key layout (DP_KEY_SPLIT) against the interleaved
layout and the oracle.

Only the key temporal phase changes in a re-index (DeCoPrune page, section
무엇과 다른가), so a cache may keep each token row's temporal blocks (all
heads) ahead of the other dims; the re-index then touches whole 128-byte lines
only.  The layout is a fixed permutation of a key row, so every entry point
must give, in the split layout, exactly the interleaved layout's results on the
same keys, permuted: re-index, uniform shift, gather and append with the fused
re-index, the DeCoPrune-HS gather and re-index (runs hold their temporal blocks
first), and attention over dense, lagged, ragged and ragged-lagged caches.
Every comparison is bit for bit after converting back; the interleaved results
are compared with the oracle as well (re-indexed keys within max-abs 2e-2 bf16 /
1e-5 fp32).  The conversions only move data.
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import dpsynth
import oracle
from gpu_helpers import (bf16_from_bits, bits, device, from_split, keys_close, random_bf16_bits,
                         random_f32, run_from_split, run_to_split, to_dev, to_split)

pytestmark = pytest.mark.gpu

TOL = {dp.DP_BF16: 2e-2, dp.DP_F32: 1e-5}
SPLIT = dp.DP_KEY_SPLIT

CASES = [  # L, T, H, D, dtype, tokens_per_frame, pair_begin, n_pairs
    (2, 4000, 6, 128, dp.DP_BF16, 100, 0, 44),
    (1, 3000, 3, 64, dp.DP_BF16, 64, 4, 12),       # the block starts at dim 8
    (2, 2048, 2, 64, dp.DP_F32, 64, 2, 8),
    (1, 1500, 5, 32, dp.DP_F32, 50, 0, 16),        # every dim is temporal
    (1, 1300, 24, 128, dp.DP_BF16, 100, 0, 44),    # rows of 384 vectors
    (2, 999, 16, 128, dp.DP_BF16, 37, 0, 44),      # rows of exactly 256 vectors, ragged frames
]


def _layers(rng, L, T, H, D, dtype, scale=2.0):
    if dtype == dp.DP_BF16:
        return random_bf16_bits(rng, (L, T, H, D), scale)
    return random_f32(rng, (L, T, H, D), scale).view(np.uint32)


def _dev(b, dtype, dev):
    if dtype == dp.DP_BF16:
        return [bf16_from_bits(b[l], dev) for l in range(b.shape[0])]
    return [to_dev(b[l].view(np.float32), dev) for l in range(b.shape[0])]


def _rope_pair(rng, n_frames, npairs, q0, knee, factor, dev, pb, axis=dp.DP_AXIS_PAGE,
               layouts=(dp.DP_KEY_INTERLEAVED, SPLIT)):
    """Host tables and device ropes (by default one interleaved, one split)
    with their own phase tables and workspaces, so each call advances its own
    phases."""
    theta = dpsynth.rope_theta(npairs)
    ft = np.arange(n_frames, dtype=np.float32)
    fp = ft.copy()
    fp[: n_frames // 3] += np.float32(0.5)          # some keys carry an earlier re-index
    host = dict(theta=theta, frame_t=ft, frame_phase=fp, q0=q0, knee=knee,
                inv_factor=np.float32(1.0 / factor))
    out = []
    for layout in layouts:
        th, ftd, fpd = to_dev(theta, dev), to_dev(ft, dev), to_dev(fp.copy(), dev)
        r = dp.make_rope(th, ftd, fpd, q0, knee, 1.0 / factor, pb, axis=axis, key_layout=layout)
        ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, npairs) // 4 + 4,
                         dtype=torch.float32, device=dev)
        out.append((r, fpd, ws))
    return host, out


def _tables(host, axis=dp.DP_AXIS_PAGE):
    return oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"], host["knee"],
                              host["inv_factor"], host["theta"],
                              compressed=axis == dp.DP_AXIS_COMPRESSED)


def _same_after(split_layers, inter_layers, pb, npairs):
    for l, (a, b) in enumerate(zip(split_layers, inter_layers)):
        assert np.array_equal(bits(from_split(a, pb, npairs)), bits(b)), l


@pytest.mark.parametrize("L,T,H,D,dtype,tpf,pb,npairs", CASES)
@pytest.mark.parametrize("device_rows", [False, True])
def test_split_rope_reindex(L, T, H, D, dtype, tpf, pb, npairs, device_rows):
    dev = device()
    rng = np.random.default_rng(T + H + npairs)
    kb = _layers(rng, L, T, H, D, dtype)
    rf = (np.arange(T) // tpf).astype(np.int32)
    n_frames = (T + tpf - 1) // tpf
    host, ((ri, fpi, wsi), (rs, fps, wss)) = _rope_pair(rng, n_frames, npairs, float(n_frames),
                                                        7.0, 3.0, dev, pb)
    ki = _dev(kb, dtype, dev)
    ks = [to_split(t, pb, npairs).contiguous() for t in _dev(kb, dtype, dev)]
    n_rows = T - 37 if device_rows else T
    nr = torch.tensor([n_rows], dtype=torch.int64, device=dev) if device_rows else None
    rf_d = to_dev(rf, dev)
    dp.dp_rope_reindex(dp.ptr_array(ki, dev), L, H, D, dtype, T, nr, rf_d, ri, wsi)
    dp.dp_rope_reindex(dp.ptr_array(ks, dev), L, H, D, dtype, T, nr, rf_d, rs, wss)
    torch.cuda.synchronize()
    _same_after(ks, ki, pb, npairs)
    tables = _tables(host)
    assert np.array_equal(fps.cpu().numpy(), tables[3]) and np.array_equal(fpi.cpu().numpy(),
                                                                          tables[3])
    kk = kb.view(np.float32) if dtype == dp.DP_F32 else kb
    for l in range(L):
        want = kk[l].copy()
        oracle.rope_rows(want[:n_rows], rf[:n_rows], pb, tables)
        w = want.view(np.uint32) if dtype == dp.DP_F32 else want
        ok, worst, _ = keys_close(bits(ki[l]), w, TOL[dtype])
        assert ok, (l, worst)


@pytest.mark.parametrize("L,T,H,D,dtype,tpf,pb,npairs", CASES[:3])
def test_split_rope_prepare_then_apply_and_shift(L, T, H, D, dtype, tpf, pb, npairs):
    """dp_rope_apply on two row ranges (the second bounded by a device count)
    and dp_rope_shift over a range, in both layouts."""
    dev = device()
    rng = np.random.default_rng(T + 3)
    kb = _layers(rng, L, T, H, D, dtype)
    rf = (np.arange(T) // tpf).astype(np.int32)
    n_frames = (T + tpf - 1) // tpf
    host, ((ri, fpi, wsi), (rs, fps, wss)) = _rope_pair(rng, n_frames, npairs, float(n_frames),
                                                        5.0, 2.0, dev, pb)
    ki = _dev(kb, dtype, dev)
    ks = [to_split(t, pb, npairs).contiguous() for t in _dev(kb, dtype, dev)]
    rf_d = to_dev(rf, dev)
    a0, a1, b0, b1 = 0, T // 3, T // 2, T
    nr = torch.tensor([T - 11], dtype=torch.int64, device=dev)
    for k, r, ws, kl in ((ki, ri, wsi, dp.DP_KEY_INTERLEAVED), (ks, rs, wss, SPLIT)):
        arr = dp.ptr_array(k, dev)
        dp.dp_rope_prepare(r, D, dtype, ws)
        dp.dp_rope_apply(arr, L, H, D, dtype, a0, a1, None, rf_d, r, ws)
        dp.dp_rope_apply(arr, L, H, D, dtype, b0, b1, nr, rf_d, r, ws)
        sws = torch.empty(dp.dp_rope_shift_workspace_bytes(npairs) // 4 + 4, dtype=torch.float32,
                          device=dev)
        dp.dp_rope_shift(arr, L, H, D, dtype, a1, b0, None, r._tensors[0], pb, npairs, 3.5, sws,
                         key_layout=kl)
    torch.cuda.synchronize()
    _same_after(ks, ki, pb, npairs)
    tables = _tables(host)
    uni = oracle.rope_uniform(host["theta"], 3.5)
    kk = kb.view(np.float32) if dtype == dp.DP_F32 else kb
    for l in range(L):
        want = kk[l].copy()
        for lo, hi in ((a0, a1), (b0, T - 11)):
            sub = np.ascontiguousarray(want[lo:hi])
            oracle.rope_rows(sub, rf[lo:hi], pb, tables)
            want[lo:hi] = sub
        sub = np.ascontiguousarray(want[a1:b0])
        oracle.rope_rows(sub, np.zeros(b0 - a1, np.int32), pb, uni)
        want[a1:b0] = sub
        w = want.view(np.uint32) if dtype == dp.DP_F32 else want
        ok, worst, _ = keys_close(bits(ki[l]), w, TOL[dtype])
        assert ok, (l, worst)


def _kv(k_src, v_src, k_dst, v_dst, cap, err, alive):
    kv = dp.dp_kv()
    arrs = [dp.ptr_array(x, k_src[0].device) for x in (k_src, v_src, k_dst, v_dst)]
    alive += arrs
    kv.k_src, kv.v_src, kv.k_dst, kv.v_dst = [a.data_ptr() for a in arrs]
    T, H, D = k_src[0].shape
    kv.n_layers, kv.n_heads, kv.head_dim = len(k_src), H, D
    kv.dtype = dp.dtype_code(k_src[0])
    kv.src_rows, kv.dst_capacity = T, cap
    kv.dev_error = err.data_ptr()
    return kv


@pytest.mark.parametrize("L,T,H,D,dtype,tpf,pb,npairs", CASES)
@pytest.mark.parametrize("axis", [dp.DP_AXIS_PAGE, dp.DP_AXIS_COMPRESSED])
def test_split_gather_with_fused_reindex(L, T, H, D, dtype, tpf, pb, npairs, axis):
    dev = device()
    rng = np.random.default_rng(T * 3 + axis)
    kb, vb = _layers(rng, L, T, H, D, dtype), _layers(rng, L, T, H, D, dtype)
    keep = (rng.random(T) < 0.3).astype(np.uint8)
    keep[: T // 10] = 1
    rf = (np.arange(T) // tpf).astype(np.int32)
    n_frames = (T + tpf - 1) // tpf
    host, ((ri, _, wsi), (rs, _, wss)) = _rope_pair(rng, n_frames, npairs, float(n_frames), 6.0,
                                                    4.0, dev, pb, axis)
    idx_h = oracle.compact(keep)
    n = idx_h.shape[0]
    idx = to_dev(idx_h, dev)
    nk = torch.tensor([n], dtype=torch.int64, device=dev)
    rf2 = to_dev(rf[idx_h], dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive, outs = [], []
    for layout, r, ws in ((dp.DP_KEY_INTERLEAVED, ri, wsi), (SPLIT, rs, wss)):
        ksrc = _dev(kb, dtype, dev)
        if layout == SPLIT:
            ksrc = [to_split(t, pb, npairs).contiguous() for t in ksrc]
        vsrc = _dev(vb, dtype, dev)
        kdst = [torch.zeros_like(t) for t in ksrc]
        vdst = [torch.zeros_like(t) for t in vsrc]
        kv = _kv(ksrc, vsrc, kdst, vdst, T, err, alive)
        dp.dp_gather_kv(kv, idx, nk, rf2, r, ws)
        outs.append((kdst, vdst))
    torch.cuda.synchronize()
    assert err.item() == 0
    (ki, vi), (ks, vs) = outs
    _same_after(ks, ki, pb, npairs)
    for l in range(L):
        assert torch.equal(vs[l].view(torch.int16 if dtype == dp.DP_BF16 else torch.int32),
                           vi[l].view(torch.int16 if dtype == dp.DP_BF16 else torch.int32))
    tables = _tables(host, axis)
    kk = kb.view(np.float32) if dtype == dp.DP_F32 else kb
    want = oracle.gather(kk, idx_h)
    for l in range(L):
        oracle.rope_rows(want[l], rf[idx_h], pb, tables)
        w = want[l].view(np.uint32) if dtype == dp.DP_F32 else want[l]
        ok, worst, _ = keys_close(bits(ki[l][:n]), w, TOL[dtype])
        assert ok, (l, worst)
        assert np.array_equal(bits(vi[l][:n]), oracle.gather(vb, idx_h)[l])


@pytest.mark.parametrize("L,T,H,D,dtype,tpf,pb,npairs", CASES[:4])
def test_split_append_with_fused_reindex(L, T, H, D, dtype, tpf, pb, npairs):
    """The ring layout's append of a leaving slot's kept rows, re-indexed on the
    way, in both layouts."""
    dev = device()
    rng = np.random.default_rng(T + 17)
    C = T // 5
    cap = 7 * C
    kb = np.zeros((L, cap, H, D), np.uint16 if dtype == dp.DP_BF16 else np.uint32)
    vb = np.zeros_like(kb)
    kb[:, :5 * C] = _layers(rng, L, 5 * C, H, D, dtype)
    vb[:, :5 * C] = _layers(rng, L, 5 * C, H, D, dtype)
    rf = np.full(cap, -1, np.int32)
    rf[:5 * C] = np.arange(5 * C) // tpf
    n_frames = (5 * C + tpf - 1) // tpf
    host, ((ri, _, wsi), (rs, _, wss)) = _rope_pair(rng, n_frames, npairs, float(n_frames),
                                                    3.0 * C / tpf, 4.0, dev, pb)
    keep = (rng.random(C) < 0.4).astype(np.uint8)
    widx = oracle.compact(keep)
    idx, nk = to_dev(widx, dev), torch.tensor([widx.shape[0]], dtype=torch.int64, device=dev)
    outs, alive = [], []
    for layout, r, ws in ((dp.DP_KEY_INTERLEAVED, ri, wsi), (SPLIT, rs, wss)):
        k = _dev(kb, dtype, dev)
        if layout == SPLIT:
            k = [to_split(t, pb, npairs).contiguous() for t in k]
        v = _dev(vb, dtype, dev)
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        kv = dp.dp_kv_inplace()
        arrs = [dp.ptr_array(k, dev), dp.ptr_array(v, dev)]
        alive += arrs
        kv.k_layers, kv.v_layers = arrs[0].data_ptr(), arrs[1].data_ptr()
        kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dtype
        kv.capacity, kv.dev_error = cap, err.data_ptr()
        tail = torch.tensor([5 * C], dtype=torch.int64, device=dev)
        rf_d = to_dev(rf, dev)
        dp.dp_rope_prepare(r, D, dtype, ws)
        dp.dp_append_kept(kv, C, C, idx, nk, tail, rf_d, r, ws)
        outs.append((k, v, tail, rf_d, err))
    torch.cuda.synchronize()
    (ki, vi, ti, rfi, ei), (ks, vs, ts, rfs, es) = outs
    assert ei.item() == 0 and es.item() == 0 and ti.item() == ts.item() == 5 * C + widx.shape[0]
    assert torch.equal(rfi, rfs)
    _same_after(ks, ki, pb, npairs)
    for l in range(L):
        assert np.array_equal(bits(vs[l]), bits(vi[l]))
    tables = _tables(host)
    kk = (kb.view(np.float32) if dtype == dp.DP_F32 else kb).copy()
    orf = rf.copy()
    t1 = oracle.append_kept(kk, C, C, widx, 5 * C, orf)
    for l in range(L):
        sub = np.ascontiguousarray(kk[l][5 * C:t1])
        oracle.rope_rows(sub, orf[5 * C:t1], pb, tables)
        kk[l][5 * C:t1] = sub
        w = kk[l].view(np.uint32) if dtype == dp.DP_F32 else kk[l]
        ok, worst, _ = keys_close(bits(ki[l]), w, TOL[dtype])
        assert ok, (l, worst)


@pytest.mark.parametrize("dtype,D,pb,npairs", [(dp.DP_BF16, 128, 0, 44), (dp.DP_BF16, 64, 4, 8),
                                               (dp.DP_F32, 32, 2, 6)])
@pytest.mark.parametrize("fused", [False, True])
def test_split_hs_gather_and_reindex(dtype, D, pb, npairs, fused):
    """The DeCoPrune-HS packed cache in the split layout: every run holds its
    temporal blocks, then its other parts; gathered from split token rows or
    from interleaved ones, with the re-index fused or as a pass of its own, it
    is the interleaved packed cache run by run (V: plain head rows in all)."""
    dev = device()
    rng = np.random.default_rng(D + npairs + fused)
    L, H, T, tpf, sink, window = 3, 6, 3000, 50, 150, 450
    kb, vb = _layers(rng, L, T, H, D, dtype), _layers(rng, L, T, H, D, dtype)
    cls = rng.integers(0, 2, (L, H)).astype(np.uint8)
    cls[0, :] = 0
    keep_d = (rng.random(T) < 0.3).astype(np.uint8)
    keep_d[:sink] = 1
    keep_d[T - window:] = 1
    keep_s = np.zeros(T, np.uint8)
    keep_s[:sink] = 1
    keep_s[T - window:] = 1
    lists_h = [oracle.compact(keep_s), oracle.compact(keep_d)]
    lens_h = np.array([len(x) for x in lists_h], np.int64)
    off_h = oracle.hs_offsets(cls, lens_h)
    total = int(off_h[-1])
    rf = (np.arange(T) // tpf).astype(np.int32)
    n_frames = T // tpf
    host, ((ri, _, wsi), (rs, _, wss), (rm, _, wsm)) = _rope_pair(
        rng, n_frames, npairs, float(n_frames), 9.0, 4.0, dev, pb,
        layouts=(dp.DP_KEY_INTERLEAVED, SPLIT, SPLIT))
    lists = [to_dev(x, dev) for x in lists_h]
    rfs = [to_dev(rf[x], dev) for x in lists_h]
    lens = to_dev(lens_h, dev)
    offsets = to_dev(off_h, dev)
    head_class = to_dev(cls.ravel(), dev)
    tdt = torch.bfloat16 if dtype == dp.DP_BF16 else torch.float32
    outs, alive = [], []
    for src_layout, layout, r, ws in ((dp.DP_KEY_INTERLEAVED, dp.DP_KEY_INTERLEAVED, ri, wsi),
                                      (SPLIT, SPLIT, rs, wss),
                                      (dp.DP_KEY_INTERLEAVED, SPLIT, rm, wsm)):
        ksrc = _dev(kb, dtype, dev)
        if src_layout == SPLIT:
            ksrc = [to_split(t, pb, npairs).contiguous() for t in ksrc]
        vsrc = _dev(vb, dtype, dev)
        k_out = torch.zeros((total + 8, D), dtype=tdt, device=dev)
        v_out = torch.zeros((total + 8, D), dtype=tdt, device=dev)
        kv = dp.dp_kv_hs()
        arrs = [dp.ptr_array(ksrc, dev), dp.ptr_array(vsrc, dev)]
        alive += arrs + [ksrc, vsrc]
        kv.k_src, kv.v_src = arrs[0].data_ptr(), arrs[1].data_ptr()
        kv.k_out, kv.v_out = k_out.data_ptr(), v_out.data_ptr()
        kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dtype
        kv.src_rows, kv.out_capacity = T, total
        kv.key_layout, kv.pair_begin, kv.n_pairs = layout, pb, npairs
        kv.src_key_layout = src_layout
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        kv.dev_error = err.data_ptr()
        cidx, crf = dp.ptr_array(lists, dev), dp.ptr_array(rfs, dev)
        alive += [cidx, crf]
        if fused:
            dp.dp_hs_gather_kv(kv, head_class, 2, cidx, lens, [T, T], offsets, crf, r, ws)
        else:
            dp.dp_hs_gather_kv(kv, head_class, 2, cidx, lens, [T, T], offsets)
            dp.dp_hs_rope_reindex(k_out, total, L, H, D, dtype, head_class, 2, lens, [T, T],
                                  offsets, crf, r, ws)
        outs.append((k_out, v_out, err))
    torch.cuda.synchronize()
    (ki, vi, ei) = outs[0]
    ki_h = bits(ki)
    iv = torch.int16 if dtype == dp.DP_BF16 else torch.int32
    for ks, vs, es in outs[1:]:
        assert ei.item() == 0 and es.item() == 0
        assert torch.equal(vs.view(iv), vi.view(iv))
        ks_h = bits(ks)
        for i in range(L * H):
            lo, hi = int(off_h[i]), int(off_h[i + 1])
            assert np.array_equal(run_from_split(ks_h[lo:hi], pb, npairs), ki_h[lo:hi]), i
        assert np.all(ks_h[total:] == 0)
    # the interleaved packed cache against the oracle
    tables = _tables(host)
    kk = kb.view(np.float32) if dtype == dp.DP_F32 else kb
    w_k = np.zeros((total, D), kk.dtype)
    for l in range(L):
        oracle.hs_gather_layer(kk[l], l, cls, lists_h, off_h, w_k)
    w_rf = np.concatenate([rf[lists_h[c]] for c in cls.ravel()]).astype(np.int32)
    oracle.rope_headrows(w_k, w_rf, pb, tables)
    w = w_k.view(np.uint32) if dtype == dp.DP_F32 else w_k
    ok, worst, _ = keys_close(ki_h[:total], w, TOL[dtype])
    assert ok, worst


# --------------------------------------------------------------------------
# attention over split keys: the tiles land in LDS as for interleaved keys, so
# the outputs are bit for bit those of the interleaved layout
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n_q,n_kv,H,pb,npairs", [(300, 1000, 8, 0, 44), (129, 577, 3, 4, 12),
                                                  (64, 65, 8, 16, 48)])
def test_split_attention_dense_and_lagged(n_q, n_kv, H, pb, npairs):
    dev = device()
    rng = np.random.default_rng(n_q + n_kv)
    D = 128
    q = bf16_from_bits(random_bf16_bits(rng, (n_q, H, D)), dev)
    kb = random_bf16_bits(rng, (n_kv + 5, H, D))
    k = bf16_from_bits(kb, dev)
    ksp = to_split(k, pb, npairs).contiguous()
    v = bf16_from_bits(random_bf16_bits(rng, (n_kv + 5, H, D)), dev)
    nk = torch.tensor([n_kv], dtype=torch.int64, device=dev)
    theta = to_dev(dpsynth.rope_theta(npairs), dev)
    scale = 1.0 / np.sqrt(D)
    oi, osp = torch.empty_like(q), torch.empty_like(q)
    dp.dp_attention(q, k, v, oi, n_q, n_kv + 5, nk, H, D, dp.DP_BF16, scale)
    dp.dp_attention(q, ksp, v, osp, n_q, n_kv + 5, nk, H, D, dp.DP_BF16, scale, key_layout=SPLIT,
                    pair_begin=pb, n_pairs=npairs)
    torch.cuda.synchronize()
    assert torch.equal(oi.view(torch.int16), osp.view(torch.int16))
    want = oracle.attention(bits(q), kb, bits(v), np.arange(0, n_q, 7), n_kv=n_kv, scale=scale)
    got = bits(oi)[np.arange(0, n_q, 7)]
    gf = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.max(np.abs(gf - want)) < 4e-3 + 1e-2 * np.max(np.abs(want))
    pa, pe = n_kv // 3, n_kv // 3 + 100
    for kk, oo, kl in ((k, oi, dp.DP_KEY_INTERLEAVED), (ksp, osp, SPLIT)):
        dp.dp_attention_lag(q, kk, v, oo, n_q, n_kv + 5, nk, pa, pe, theta, pb, npairs, 7.25, H, D,
                            dp.DP_BF16, scale, key_layout=kl)
    torch.cuda.synchronize()
    assert torch.equal(oi.view(torch.int16), osp.view(torch.int16))


@pytest.mark.parametrize("lag", [False, True])
def test_split_hs_attention(lag):
    """Ragged runs of unequal length (one empty) with the chunk block after
    them, split keys against interleaved keys, bit for bit."""
    dev = device()
    rng = np.random.default_rng(7 + lag)
    L, H, D, n_q, nc, pb, npairs = 2, 8, 128, 200, 70, 0, 44
    lens = rng.integers(0, 400, (L, H))
    lens[1, 3] = 0
    lens[1, 5] = 1
    off_h = np.concatenate([[0], np.cumsum(lens.ravel())]).astype(np.int64)
    total = int(off_h[-1])
    kr = random_bf16_bits(rng, (total, D))
    vr = bf16_from_bits(random_bf16_bits(rng, (total, D)), dev)
    kr_sp = kr.copy()
    for i in range(L * H):
        lo, hi = int(off_h[i]), int(off_h[i + 1])
        kr_sp[lo:hi] = run_to_split(kr[lo:hi], pb, npairs)
    kc = random_bf16_bits(rng, (nc, H, D))
    vc = bf16_from_bits(random_bf16_bits(rng, (nc, H, D)), dev)
    q = bf16_from_bits(random_bf16_bits(rng, (n_q, H, D)), dev)
    offsets = to_dev(off_h, dev)
    theta = to_dev(dpsynth.rope_theta(npairs), dev)
    outs = []
    for layout, kk, kch in ((dp.DP_KEY_INTERLEAVED, kr, kc), (SPLIT, kr_sp, to_split(kc, pb, npairs))):
        o = torch.empty_like(q)
        kd, kcd = bf16_from_bits(kk, dev), bf16_from_bits(kch, dev)
        for layer in range(L):
            if lag:
                dp.dp_hs_attention_lag(q, kd, vr, total, offsets, layer, kcd, vc, nc, o, n_q, H, D,
                                       dp.DP_BF16, 0.09, 60, theta, pb, npairs, 5.5,
                                       key_layout=layout)
            else:
                dp.dp_hs_attention(q, kd, vr, total, offsets, layer, kcd, vc, nc, o, n_q, H, D,
                                   dp.DP_BF16, 0.09, key_layout=layout, pair_begin=pb,
                                   n_pairs=npairs)
            torch.cuda.synchronize()
            outs.append(bits(o).copy())
    half = len(outs) // 2
    for a, b in zip(outs[:half], outs[half:]):
        assert np.array_equal(a, b)
