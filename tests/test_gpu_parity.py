"""GPU parity of every libdecoprune entry point against the CPU oracle.

Sizes span several workgroup tiles with ragged tails; edge cases cover empty
and full masks, ties at gamma, NaN/Inf scores, partial RoPE vectors,
capacity overflow and device-side row counts.  Bar: mask, index list,
gathered K/V and offsets bit-exact; re-indexed keys within max-abs 2e-2
(bf16) / 1e-5 (fp32), and the number of non-identical elements is reported.
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import dpsynth
import oracle
from gpu_helpers import (bf16_from_bits, bits, device, keys_close, random_bf16_bits, random_f32,
                         to_dev)

pytestmark = pytest.mark.gpu

TOL = {dp.DP_BF16: 2e-2, dp.DP_F32: 1e-5}


# --------------------------------------------------------------------------
# score + mask
# --------------------------------------------------------------------------
def _score_case(rng, n, d, stride):
    xf = rng.standard_normal((n, stride)).astype(np.float32)
    sig = np.exp(rng.uniform(np.log(0.05), np.log(1.0), n))[:, None]
    x0 = (xf + sig * rng.standard_normal((n, stride))).astype(np.float32)
    # specials: equal rows, NaN, Inf, denormal differences
    x0[3] = xf[3]
    x0[5, 0] = np.nan
    x0[7, d - 1] = np.inf
    x0[9, :d] = xf[9, :d] + np.float32(1e-40)
    return x0, xf


@pytest.mark.parametrize("d,stride", [(1, 1), (2, 2), (3, 5), (4, 4), (5, 8), (16, 16), (48, 52),
                                      (64, 64), (100, 100), (256, 256)])
def test_score_mask_matches_oracle(d, stride):
    dev = device()
    rng = np.random.default_rng(d * 1000 + stride)
    T, sink, window, sb = 9000 + d, 128, 700, 300
    ns = T - window - sb - 37
    x0, xf = _score_case(rng, ns, d, stride)
    ell_o = oracle.score_f32(x0, xf, d)
    gamma = float(np.nanmedian(ell_o))            # a tie: this value is in ell
    for reversed_ in (False, True):
        pol = dp.make_policy(T, sink, window, sb, ns, gamma, reversed_)
        keep = torch.full((T,), 7, dtype=torch.uint8, device=dev)
        ell = torch.empty(ns, dtype=torch.float32, device=dev)
        dp.dp_score_mask(to_dev(x0, dev), to_dev(xf, dev), d, stride, pol, ell, keep)
        torch.cuda.synchronize()
        g = ell.cpu().numpy()
        both_nan = np.isnan(g) & np.isnan(ell_o)
        assert np.array_equal(g.view(np.uint32)[~both_nan], ell_o.view(np.uint32)[~both_nan])
        want = oracle.mask(ell_o, T, sink, window, sb, ns, gamma, reversed_)
        assert np.array_equal(keep.cpu().numpy(), want)


def test_score_mask_streaming_gamma_zero_and_no_scored_rows():
    dev = device()
    rng = np.random.default_rng(3)
    T, sink, window, sb, ns, d = 20000, 6240 // 4, 4680, 2000, 9000, 64
    x0, xf = _score_case(rng, ns, d, d)
    x0d, xfd = to_dev(x0, dev), to_dev(xf, dev)
    keep = torch.empty(T, dtype=torch.uint8, device=dev)
    # streaming: only sink + window kept, scores not read
    pol = dp.make_policy(T, sink, window, sb, ns, 0.1, mode=dp.DP_MODE_STREAMING)
    dp.dp_score_mask(None, None, d, d, pol, None, keep)
    assert np.array_equal(keep.cpu().numpy(), oracle.mask(None, T, sink, window, sb, ns, 0.1,
                                                          streaming=True))
    # gamma = 0 keeps every non-NaN row
    pol = dp.make_policy(T, sink, window, sb, ns, 0.0)
    dp.dp_score_mask(x0d, xfd, d, d, pol, None, keep)
    want = oracle.mask(oracle.score_f32(x0, xf), T, sink, window, sb, ns, 0.0)
    assert np.array_equal(keep.cpu().numpy(), want)
    assert want.sum() == T - 1                    # only the NaN row drops
    # no scored rows, T not a multiple of 16, unaligned keep pointer
    big = torch.empty(T + 1, dtype=torch.uint8, device=dev)
    pol = dp.make_policy(T - 3, 7, 5, 7, 0, 0.1)
    dp.dp_score_mask(None, None, d, d, pol, None, big[1:])
    assert np.all(big[1:T - 2].cpu().numpy() == 1)
    pol = dp.make_policy(1, 0, 1, 0, 0, 0.1)
    dp.dp_score_mask(None, None, d, d, pol, None, keep)
    assert keep[0].item() == 1


# --------------------------------------------------------------------------
# compaction
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T", [1, 255, 4095, 4096, 4097, 12289, 100003, 361920])
@pytest.mark.parametrize("rate", [0.0, 0.15, 0.5, 1.0])
def test_compact_index_matches_oracle(T, rate):
    dev = device()
    rng = np.random.default_rng(T + int(rate * 100))
    keep = (rng.random(T) < rate).astype(np.uint8)
    keep[rng.random(T) < 0.01] = 3                 # any nonzero byte counts as kept
    rf = rng.integers(0, 1 << 30, T).astype(np.int32)
    idx = torch.full((T,), -1, dtype=torch.int32, device=dev)
    rf_out = torch.full((T,), -1, dtype=torch.int32, device=dev)
    n_kept = torch.full((1,), -5, dtype=torch.int64, device=dev)
    ws = torch.empty(dp.dp_compact_workspace_bytes(T) // 4, dtype=torch.int32, device=dev)
    dp.dp_compact_index(to_dev(keep, dev), T, idx, n_kept, to_dev(rf, dev), rf_out, ws)
    torch.cuda.synchronize()
    want = oracle.compact(keep)
    n = int(n_kept.item())
    assert n == want.shape[0]
    assert np.array_equal(idx[:n].cpu().numpy(), want)
    assert np.all(idx[n:].cpu().numpy() == -1)
    assert np.array_equal(rf_out[:n].cpu().numpy(), oracle.gather_i32(rf, want))


@pytest.mark.parametrize("T,offset", [(3 * 4096 + 77, 16), (3 * 4096 + 77, 5), (4096, 0),
                                      (2048 * 4096, 0), (2050 * 4096 - 3, 7)])
def test_compact_index_byte_values_and_alignment(T, offset):
    """Kept bytes of every kind (1, 3, 127, 128, 255) at a keep address that is
    16-byte aligned or not; tile counts on both sides of the count at which the
    tile offsets are summed by the write launch itself (2,048 tiles of 4,096
    rows) instead of a separate scan launch."""
    dev = device()
    rng = np.random.default_rng(T + offset)
    keep = np.zeros(T, np.uint8)
    pick = rng.random(T) < 0.3
    keep[pick] = rng.choice(np.array([1, 3, 127, 128, 255], np.uint8), int(pick.sum()))
    buf = torch.zeros(T + 32, dtype=torch.uint8, device=dev)
    buf[offset:offset + T] = to_dev(keep, dev)
    idx = torch.full((T,), -1, dtype=torch.int32, device=dev)
    n_kept = torch.full((1,), -5, dtype=torch.int64, device=dev)
    ws = torch.empty(dp.dp_compact_workspace_bytes(T) // 4, dtype=torch.int32, device=dev)
    dp.dp_compact_index(buf[offset:], T, idx, n_kept, None, None, ws)
    torch.cuda.synchronize()
    want = oracle.compact(keep)
    n = int(n_kept.item())
    assert n == want.shape[0]
    assert np.array_equal(idx[:n].cpu().numpy(), want)
    assert np.all(idx[n:].cpu().numpy() == -1)


def test_compact_index_empty_sequence():
    dev = device()
    n_kept = torch.full((1,), -5, dtype=torch.int64, device=dev)
    ws = torch.empty(1, dtype=torch.int32, device=dev)
    dp.dp_compact_index(None, 0, None, n_kept, None, None, ws)
    assert n_kept.item() == 0


# --------------------------------------------------------------------------
# gather (+ fused re-index)
# --------------------------------------------------------------------------
def _layers(rng, L, T, H, D, dtype, scale=1.0):
    if dtype == dp.DP_BF16:
        b = random_bf16_bits(rng, (L, T, H, D), scale)
        b[0, 0, 0, :2] = [0x7FC1, 0xFF80]            # a NaN payload and -Inf travel as bits
    else:
        b = random_f32(rng, (L, T, H, D), scale).view(np.uint32)
        b[0, 0, 0, :2] = [0x7FC00001, 0xFF800000]
    return b


def _dev_layers(b, dtype, dev):
    if dtype == dp.DP_BF16:
        return [bf16_from_bits(b[l], dev) for l in range(b.shape[0])]
    return [to_dev(b[l].view(np.float32), dev) for l in range(b.shape[0])]


def _kv_struct(k_src, v_src, k_dst, v_dst, cap, dev_error, keep_alive):
    kv = dp.dp_kv()
    arrs = [dp.ptr_array(x, k_src[0].device) for x in (k_src, v_src, k_dst, v_dst)]
    keep_alive += arrs
    kv.k_src, kv.v_src, kv.k_dst, kv.v_dst = [a.data_ptr() if a is not None else None for a in arrs]
    T, H, D = k_src[0].shape
    kv.n_layers, kv.n_heads, kv.head_dim = len(k_src), H, D
    kv.dtype = dp.dtype_code(k_src[0])
    kv.src_rows, kv.dst_capacity = T, cap
    kv.dev_error = dev_error.data_ptr() if dev_error is not None else None
    return kv


def _keep_mask(rng, T, rate, sink, window):
    keep = (rng.random(T) < rate).astype(np.uint8)
    keep[:sink] = 1
    keep[T - window:] = 1
    return keep


def _gpu_idx(keep, dev, rf=None):
    T = keep.shape[0]
    idx = torch.empty(max(1, T), dtype=torch.int32, device=dev)
    n = torch.zeros(1, dtype=torch.int64, device=dev)
    ws = torch.empty(dp.dp_compact_workspace_bytes(T) // 4, dtype=torch.int32, device=dev)
    rf_out = torch.empty(max(1, T), dtype=torch.int32, device=dev) if rf is not None else None
    dp.dp_compact_index(to_dev(keep, dev), T, idx, n, to_dev(rf, dev) if rf is not None else None,
                        rf_out, ws)
    return idx, n, rf_out


GATHER_SHAPES = [  # L, T, H, D, dtype
    (3, 5000, 5, 32, dp.DP_BF16),
    (2, 3001, 2, 64, dp.DP_F32),
    (1, 777, 1, 8, dp.DP_BF16),
    (2, 2500, 40, 128, dp.DP_BF16),
]


@pytest.mark.parametrize("L,T,H,D,dtype", GATHER_SHAPES)
@pytest.mark.parametrize("with_v", [True, False])
def test_gather_kv_bit_exact(L, T, H, D, dtype, with_v):
    dev = device()
    rng = np.random.default_rng(L * T + H)
    kb, vb = _layers(rng, L, T, H, D, dtype), _layers(rng, L, T, H, D, dtype)
    keep = _keep_mask(rng, T, 0.3, 17, 33)
    k_src, v_src = _dev_layers(kb, dtype, dev), _dev_layers(vb, dtype, dev)
    if not with_v:
        v_src = None
    k_dst = [torch.empty_like(t) for t in k_src]
    v_dst = [torch.empty_like(t) for t in v_src] if with_v else None
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive = []
    kv = _kv_struct(k_src, v_src, k_dst, v_dst, T, err, alive)
    idx, n, _ = _gpu_idx(keep, dev)
    dp.dp_gather_kv(kv, idx, n)
    torch.cuda.synchronize()
    want_idx = oracle.compact(keep)
    m = want_idx.shape[0]
    assert int(n.item()) == m and err.item() == 0
    wk = oracle.gather(kb, want_idx)
    for l in range(L):
        assert np.array_equal(bits(k_dst[l][:m]), wk[l])
    if with_v:
        wv = oracle.gather(vb, want_idx)
        for l in range(L):
            assert np.array_equal(bits(v_dst[l][:m]), wv[l])


def test_gather_kv_capacity_overflow_is_clamped_and_flagged():
    dev = device()
    rng = np.random.default_rng(9)
    L, T, H, D, dtype = 2, 3000, 4, 64, dp.DP_BF16
    kb = _layers(rng, L, T, H, D, dtype)
    keep = _keep_mask(rng, T, 0.5, 10, 10)
    k_src = _dev_layers(kb, dtype, dev)
    cap = 1000
    guard = 64
    k_dst = [torch.zeros((cap + guard, H, D), dtype=torch.bfloat16, device=dev) for _ in range(L)]
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive = []
    kv = _kv_struct(k_src, None, k_dst, None, cap, err, alive)
    idx, n, _ = _gpu_idx(keep, dev)
    dp.dp_gather_kv(kv, idx, n)
    torch.cuda.synchronize()
    assert err.item() == dp.DP_ECAPACITY
    want = oracle.gather(kb, oracle.compact(keep)[:cap])
    for l in range(L):
        assert np.array_equal(bits(k_dst[l][:cap]), want[l])
        assert np.all(bits(k_dst[l][cap:]) == 0)          # guard rows untouched


def test_gather_kv_nothing_kept_and_zero_capacity():
    dev = device()
    rng = np.random.default_rng(10)
    L, T, H, D, dtype = 1, 500, 2, 64, dp.DP_F32
    kb = _layers(rng, L, T, H, D, dtype)
    k_src = _dev_layers(kb, dtype, dev)
    k_dst = [torch.zeros_like(k_src[0])]
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive = []
    keep = np.zeros(T, np.uint8)
    idx, n, _ = _gpu_idx(keep, dev)
    dp.dp_gather_kv(_kv_struct(k_src, None, k_dst, None, T, err, alive), idx, n)
    dp.dp_gather_kv(_kv_struct(k_src, None, k_dst, None, 0, err, alive), idx, n)
    torch.cuda.synchronize()
    assert n.item() == 0 and err.item() == 0
    assert np.all(bits(k_dst[0]) == 0)


def _rope_inputs(rng, n_frames, n_pairs, q0, knee, factor, dev, phase_jitter=False):
    theta = dpsynth.rope_theta(n_pairs)
    ft = np.arange(n_frames, dtype=np.float32)
    fp = ft.copy()
    if phase_jitter:      # keys that already carry an earlier re-index
        fp[: n_frames // 2] += np.float32(0.5)
    host = dict(theta=theta, frame_t=ft, frame_phase=fp, q0=q0, knee=knee,
                inv_factor=np.float32(1.0 / factor))
    devt = dict(theta=to_dev(theta, dev), frame_t=to_dev(ft, dev), frame_phase=to_dev(fp, dev))
    return host, devt


ROPE_CASES = [  # L, T, H, D, dtype, tokens_per_frame, pair_begin, n_pairs
    (2, 4000, 6, 128, dp.DP_BF16, 100, 0, 44),
    (1, 3000, 3, 64, dp.DP_BF16, 64, 4, 6),        # block ends inside a 16-byte vector
    (2, 2048, 2, 64, dp.DP_F32, 64, 2, 8),
    (1, 1500, 5, 32, dp.DP_F32, 50, 0, 16),        # every dim is temporal
    (1, 1300, 24, 128, dp.DP_BF16, 100, 0, 44),    # rows of 384 vectors: a workgroup spans <= 2 rows
    (2, 999, 16, 128, dp.DP_BF16, 37, 0, 44),      # rows of exactly 256 vectors, ragged frames
]


@pytest.mark.parametrize("L,T,H,D,dtype,tpf,pb,npairs", ROPE_CASES)
@pytest.mark.parametrize("axis", [dp.DP_AXIS_PAGE, dp.DP_AXIS_COMPRESSED])
def test_gather_with_fused_reindex(L, T, H, D, dtype, tpf, pb, npairs, axis):
    dev = device()
    rng = np.random.default_rng(T + D)
    kb = _layers(rng, L, T, H, D, dtype, scale=3.0)
    vb = _layers(rng, L, T, H, D, dtype)
    n_frames = (T + tpf - 1) // tpf
    rf = (np.arange(T) // tpf).astype(np.int32)
    keep = _keep_mask(rng, T, 0.25, tpf, 3 * tpf)
    host, devt = _rope_inputs(rng, n_frames, npairs, float(n_frames), 3.0 * 1, 4.0, dev, True)
    k_src, v_src = _dev_layers(kb, dtype, dev), _dev_layers(vb, dtype, dev)
    k_dst = [torch.empty_like(t) for t in k_src]
    v_dst = [torch.empty_like(t) for t in v_src]
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive = []
    kv = _kv_struct(k_src, v_src, k_dst, v_dst, T, err, alive)
    idx, n, rf_out = _gpu_idx(keep, dev, rf)
    rope = dp.make_rope(devt["theta"], devt["frame_t"], devt["frame_phase"], host["q0"],
                        host["knee"], host["inv_factor"], pb, axis=axis)
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, npairs) // 4, dtype=torch.float32,
                     device=dev)
    dp.dp_gather_kv(kv, idx, n, rf_out, rope, ws)
    torch.cuda.synchronize()
    kk = kb.view(np.float32) if dtype == dp.DP_F32 else kb
    widx = oracle.compact(keep)
    m = widx.shape[0]
    assert int(n.item()) == m and err.item() == 0
    wk = oracle.gather(kk, widx)
    tables = oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"], host["knee"],
                                host["inv_factor"], host["theta"],
                                compressed=axis == dp.DP_AXIS_COMPRESSED)
    wrf = oracle.gather_i32(rf, widx)
    for l in range(L):
        oracle.rope_rows(wk[l], wrf, pb, tables)
    wk_bits = wk.view(np.uint32) if dtype == dp.DP_F32 else wk
    wv = oracle.gather(vb, widx)
    inexact = 0
    for l in range(L):
        ok, worst, ne = keys_close(bits(k_dst[l][:m]), wk_bits[l], TOL[dtype])
        assert ok, (l, worst)
        inexact += ne
        assert np.array_equal(bits(v_dst[l][:m]), wv[l])
    print("fused re-index: %d non-identical key elements" % inexact)
    assert np.array_equal(devt["frame_phase"].cpu().numpy(), tables[3])
    assert np.array_equal(rf_out[:m].cpu().numpy(), wrf)


# --------------------------------------------------------------------------
# standalone re-index
# --------------------------------------------------------------------------
@pytest.mark.parametrize("L,T,H,D,dtype,tpf,pb,npairs", ROPE_CASES)
@pytest.mark.parametrize("device_rows", [False, True])
def test_rope_reindex_in_place(L, T, H, D, dtype, tpf, pb, npairs, device_rows):
    dev = device()
    rng = np.random.default_rng(T * 3 + D)
    kb = _layers(rng, L, T, H, D, dtype, scale=3.0)
    n_frames = (T + tpf - 1) // tpf
    rf = (np.arange(T) // tpf).astype(np.int32)
    host, devt = _rope_inputs(rng, n_frames, npairs, float(n_frames), 5.0, 8.0, dev, True)
    k = _dev_layers(kb, dtype, dev)
    arr = dp.ptr_array(k, dev)
    rows = T - 123 if device_rows else T
    n_rows = torch.tensor([rows], dtype=torch.int64, device=dev) if device_rows else None
    rope = dp.make_rope(devt["theta"], devt["frame_t"], devt["frame_phase"], host["q0"],
                        host["knee"], host["inv_factor"], pb)
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, npairs) // 4, dtype=torch.float32,
                     device=dev)
    dp.dp_rope_reindex(arr, L, H, D, dtype, T, n_rows, to_dev(rf, dev), rope, ws)
    torch.cuda.synchronize()
    kk = (kb.view(np.float32) if dtype == dp.DP_F32 else kb).copy()
    tables = oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"], host["knee"],
                                host["inv_factor"], host["theta"])
    inexact = 0
    for l in range(L):
        sub = np.ascontiguousarray(kk[l][:rows])
        oracle.rope_rows(sub, rf, pb, tables)
        kk[l][:rows] = sub
        want = kk[l].view(np.uint32) if dtype == dp.DP_F32 else kk[l]
        ok, worst, ne = keys_close(bits(k[l]), want, TOL[dtype])
        assert ok, (l, worst)
        inexact += ne
        assert np.array_equal(bits(k[l])[rows:], (kb[l].view(np.uint32) if dtype == dp.DP_F32 else kb[l])[rows:])
    print("re-index: %d non-identical key elements" % inexact)
    assert np.array_equal(devt["frame_phase"].cpu().numpy(), tables[3])


@pytest.mark.parametrize("L,T,H,D,dtype,tpf,pb,npairs", ROPE_CASES[:1] + ROPE_CASES[2:3] + ROPE_CASES[4:5])
def test_rope_prepare_then_apply_on_two_ranges(L, T, H, D, dtype, tpf, pb, npairs):
    """One prepare, then apply on [a, b) and on [c, *n_rows): the same rotation as
    the one-call re-index on those rows; every other row is untouched."""
    dev = device()
    rng = np.random.default_rng(T * 5 + D)
    kb = _layers(rng, L, T, H, D, dtype, scale=3.0)
    n_frames = (T + tpf - 1) // tpf
    rf = (np.arange(T) // tpf).astype(np.int32)
    host, devt = _rope_inputs(rng, n_frames, npairs, float(n_frames), 5.0, 8.0, dev, True)
    k = _dev_layers(kb, dtype, dev)
    arr = dp.ptr_array(k, dev)
    a, b, c, e = 3, T // 3, T // 2 + 7, T - 11
    rope = dp.make_rope(devt["theta"], devt["frame_t"], devt["frame_phase"], host["q0"],
                        host["knee"], host["inv_factor"], pb)
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, npairs) // 4, dtype=torch.float32,
                     device=dev)
    rfd = to_dev(rf, dev)
    dp.dp_rope_prepare(rope, D, dtype, ws)
    dp.dp_rope_apply(arr, L, H, D, dtype, a, b, None, rfd, rope, ws)
    dp.dp_rope_apply(arr, L, H, D, dtype, c, T, torch.tensor([e], dtype=torch.int64, device=dev),
                     rfd, rope, ws)
    dp.dp_rope_apply(arr, L, H, D, dtype, b, b, None, rfd, rope, ws)      # empty range
    torch.cuda.synchronize()
    kk = (kb.view(np.float32) if dtype == dp.DP_F32 else kb).copy()
    tables = oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"], host["knee"],
                                host["inv_factor"], host["theta"])
    assert np.array_equal(devt["frame_phase"].cpu().numpy(), tables[3])
    for l in range(L):
        for lo, hi in ((a, b), (c, e)):
            sub = np.ascontiguousarray(kk[l][lo:hi])
            oracle.rope_rows(sub, rf[lo:hi], pb, tables)
            kk[l][lo:hi] = sub
        want = kk[l].view(np.uint32) if dtype == dp.DP_F32 else kk[l]
        ok, worst, ne = keys_close(bits(k[l]), want, TOL[dtype])
        assert ok, (l, worst)
        assert ne == 0, ne


def test_rope_reindex_factor_one_is_identity():
    dev = device()
    rng = np.random.default_rng(21)
    L, T, H, D = 1, 2000, 4, 128
    kb = _layers(rng, L, T, H, D, dp.DP_BF16, 3.0)
    k = _dev_layers(kb, dp.DP_BF16, dev)
    rf = (np.arange(T) // 100).astype(np.int32)
    host, devt = _rope_inputs(rng, 20, 44, 20.0, 3.0, 1.0, dev, False)
    rope = dp.make_rope(devt["theta"], devt["frame_t"], devt["frame_phase"], 20.0, 3.0, 1.0, 0)
    ws = torch.empty(dp.dp_rope_workspace_bytes(20, 44) // 4, dtype=torch.float32, device=dev)
    dp.dp_rope_reindex(dp.ptr_array(k, dev), L, H, D, dp.DP_BF16, T, None, to_dev(rf, dev), rope, ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(k[0]), kb[0])


# --------------------------------------------------------------------------
# DeCoPrune-HS
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,D", [(dp.DP_BF16, 64), (dp.DP_F32, 32), (dp.DP_BF16, 128)])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("axis", [dp.DP_AXIS_PAGE, dp.DP_AXIS_COMPRESSED])
def test_hs_ragged_gather_and_reindex(dtype, D, fused, axis):
    dev = device()
    rng = np.random.default_rng(D + fused)
    L, H, T, tpf = 3, 6, 3000, 50
    sink, window = 150, 450
    kb = _layers(rng, L, T, H, D, dtype, scale=3.0)
    vb = _layers(rng, L, T, H, D, dtype)
    cls = rng.integers(0, 2, (L, H)).astype(np.uint8)
    cls[0, :] = 0                     # a layer with only static heads
    ns = T - sink - window
    x0, xf = _score_case(rng, ns, 16, 16)
    rf = (np.arange(T) // tpf).astype(np.int32)
    n_frames = T // tpf
    npairs = 8 if dtype == dp.DP_F32 else 12
    host, devt = _rope_inputs(rng, n_frames, npairs, float(n_frames), 9.0, 4.0, dev, False)

    # class lists on the GPU: 0 = static (streaming), 1 = dynamic (score mask)
    keep_s = torch.empty(T, dtype=torch.uint8, device=dev)
    keep_d = torch.empty(T, dtype=torch.uint8, device=dev)
    dp.dp_score_mask(None, None, 16, 16, dp.make_policy(T, sink, window, sink, ns, 0.1,
                                                        mode=dp.DP_MODE_STREAMING), None, keep_s)
    dp.dp_score_mask(to_dev(x0, dev), to_dev(xf, dev), 16, 16,
                     dp.make_policy(T, sink, window, sink, ns, 0.1), None, keep_d)
    lists, lens, rfs, alive = [], torch.zeros(2, dtype=torch.int64, device=dev), [], []
    ws_c = torch.empty(dp.dp_compact_workspace_bytes(T) // 4, dtype=torch.int32, device=dev)
    rf_d = to_dev(rf, dev)
    for c, kp in enumerate((keep_s, keep_d)):
        idx = torch.empty(T, dtype=torch.int32, device=dev)
        rfo = torch.empty(T, dtype=torch.int32, device=dev)
        dp.dp_compact_index(kp, T, idx, lens[c:c + 1], rf_d, rfo, ws_c)
        lists.append(idx)
        rfs.append(rfo)
    head_class = to_dev(cls.ravel(), dev)
    offsets = torch.empty(L * H + 1, dtype=torch.int64, device=dev)
    dp.dp_hs_offsets(head_class, L, H, lens, 2, offsets)
    torch.cuda.synchronize()

    # oracle
    ell = oracle.score_f32(x0, xf)
    ws_list = oracle.compact(oracle.mask(None, T, sink, window, sink, ns, 0.1, streaming=True))
    wd_list = oracle.compact(oracle.mask(ell, T, sink, window, sink, ns, 0.1))
    wlens = np.array([len(ws_list), len(wd_list)], np.int64)
    assert np.array_equal(lens.cpu().numpy(), wlens)
    woff = oracle.hs_offsets(cls, wlens)
    assert np.array_equal(offsets.cpu().numpy(), woff)

    total = int(woff[-1])
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
    cidx = dp.ptr_array(lists, dev)
    crf = dp.ptr_array(rfs, dev)
    caps = [T, T]
    rope = dp.make_rope(devt["theta"], devt["frame_t"], devt["frame_phase"], host["q0"],
                        host["knee"], host["inv_factor"], 0, axis=axis)
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, npairs) // 4, dtype=torch.float32,
                     device=dev)
    if fused:
        dp.dp_hs_gather_kv(kv, head_class, 2, cidx, lens, caps, offsets, crf, rope, ws)
    else:
        dp.dp_hs_gather_kv(kv, head_class, 2, cidx, lens, caps, offsets)
        dp.dp_hs_rope_reindex(k_out, total, L, H, D, dtype, head_class, 2, lens, caps, offsets,
                              crf, rope, ws)
    torch.cuda.synchronize()
    assert err.item() == 0

    kk = kb.view(np.float32) if dtype == dp.DP_F32 else kb
    w_k = np.zeros((total, D), kk.dtype)
    w_v = np.zeros((total, D), vb.dtype)
    for l in range(L):
        oracle.hs_gather_layer(kk[l], l, cls, [ws_list, wd_list], woff, w_k)
        oracle.hs_gather_layer(vb[l], l, cls, [ws_list, wd_list], woff, w_v)
    assert np.array_equal(bits(v_out[:total]), w_v)
    tables = oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"], host["knee"],
                                host["inv_factor"], host["theta"],
                                compressed=axis == dp.DP_AXIS_COMPRESSED)
    w_rf = np.zeros(total, np.int32)
    for i in range(L * H):
        lst = ws_list if cls.ravel()[i] == 0 else wd_list
        w_rf[woff[i]:woff[i + 1]] = rf[lst]
    oracle.rope_headrows(w_k, w_rf, 0, tables)
    want = w_k.view(np.uint32) if dtype == dp.DP_F32 else w_k
    ok, worst, ne = keys_close(bits(k_out[:total]), want, TOL[dtype])
    assert ok, worst
    print("HS re-index: %d non-identical key elements" % ne)
    assert np.all(bits(k_out[total:]) == 0) and np.all(bits(v_out[total:]) == 0)


@pytest.mark.parametrize("static_cap", [0, 500])
@pytest.mark.parametrize("fused", [False, True])
def test_hs_gather_with_an_empty_class(static_cap, fused):
    """One head class keeps no row (its heads' runs are empty; its list
    capacity zero or not): the other class's runs are gathered and re-indexed
    as usual, nothing is written past the total."""
    dev = device()
    rng = np.random.default_rng(40 + static_cap + fused)
    L, H, T, D, tpf, dtype = 2, 5, 900, 128, 30, dp.DP_BF16
    kb, vb = _layers(rng, L, T, H, D, dtype, scale=3.0), _layers(rng, L, T, H, D, dtype)
    cls = np.array([[0, 1, 0, 1, 1], [1, 0, 0, 1, 0]], np.uint8)
    lists_h = [np.zeros(0, np.int32), np.sort(rng.choice(T, 333, replace=False)).astype(np.int32)]
    wlens = np.array([0, 333], np.int64)
    woff = oracle.hs_offsets(cls, wlens)
    total = int(woff[-1])
    rf = (np.arange(T) // tpf).astype(np.int32)
    n_frames = T // tpf
    host, devt = _rope_inputs(rng, n_frames, 44, float(n_frames), 9.0, 4.0, dev, False)
    lists = [torch.zeros(max(1, T), dtype=torch.int32, device=dev) for _ in range(2)]
    rfs = [torch.zeros(max(1, T), dtype=torch.int32, device=dev) for _ in range(2)]
    lists[1][:333] = to_dev(lists_h[1], dev)
    rfs[1][:333] = to_dev(rf[lists_h[1]], dev)
    lens = to_dev(wlens, dev)
    head_class = to_dev(cls.ravel(), dev)
    offsets = torch.empty(L * H + 1, dtype=torch.int64, device=dev)
    dp.dp_hs_offsets(head_class, L, H, lens, 2, offsets)
    k_out = torch.zeros((total + 8, D), dtype=torch.bfloat16, device=dev)
    v_out = torch.zeros((total + 8, D), dtype=torch.bfloat16, device=dev)
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
    caps = [static_cap, T]
    rope = dp.make_rope(devt["theta"], devt["frame_t"], devt["frame_phase"], host["q0"],
                        host["knee"], host["inv_factor"])
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, 44) // 4, dtype=torch.float32,
                     device=dev)
    if fused:
        dp.dp_hs_gather_kv(kv, head_class, 2, cidx, lens, caps, offsets, crf, rope, ws)
    else:
        dp.dp_hs_gather_kv(kv, head_class, 2, cidx, lens, caps, offsets)
        dp.dp_hs_rope_reindex(k_out, total, L, H, D, dtype, head_class, 2, lens, caps, offsets,
                              crf, rope, ws)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert np.array_equal(offsets.cpu().numpy(), woff)
    w_k = np.zeros((total, D), kb.dtype)
    w_v = np.zeros((total, D), vb.dtype)
    for l in range(L):
        oracle.hs_gather_layer(kb[l], l, cls, lists_h, woff, w_k)
        oracle.hs_gather_layer(vb[l], l, cls, lists_h, woff, w_v)
    assert np.array_equal(bits(v_out[:total]), w_v)
    tables = oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"], host["knee"],
                                host["inv_factor"], host["theta"])
    w_rf = np.zeros(total, np.int32)
    for i in range(L * H):
        w_rf[woff[i]:woff[i + 1]] = rf[lists_h[cls.ravel()[i]]]
    oracle.rope_headrows(w_k, w_rf, 0, tables)
    ok, worst, _ = keys_close(bits(k_out[:total]), w_k, TOL[dtype])
    assert ok, worst
    assert np.all(bits(k_out[total:]) == 0) and np.all(bits(v_out[total:]) == 0)


@pytest.mark.parametrize("fused", [False, True])
def test_hs_gather_with_many_classes(fused):
    """More head classes than the page's two, each with its own policy (the
    Streaming class, score masks at three thresholds, the reversed criterion
    and a random mask), up to the ABI's limit of DP_HS_MAX_CLASSES: a class
    with a single head in a layer, classes absent from a layer, a list filled
    to its capacity exactly, and a class with no rows.  Every run is gathered
    and re-indexed as the oracle does it class by class."""
    dev = device()
    rng = np.random.default_rng(77 + fused)
    L, H, T, D, tpf, dtype = 3, 9, 1500, 128, 25, dp.DP_BF16
    sink, window = 75, 300
    ns = T - sink - window
    nc = dp.DP_HS_MAX_CLASSES
    kb, vb = _layers(rng, L, T, H, D, dtype, scale=3.0), _layers(rng, L, T, H, D, dtype)
    x0, xf = _score_case(rng, ns, 32, 32)
    ell = oracle.score_f32(x0, xf)
    rand_keep = (rng.random(T) < 0.2).astype(np.uint8)
    # class lists from the oracle (the index path is checked elsewhere)
    lists_h = [oracle.compact(oracle.mask(None, T, sink, window, sink, ns, 0.1, streaming=True)),
               oracle.compact(oracle.mask(ell, T, sink, window, sink, ns, 0.05)),
               oracle.compact(oracle.mask(ell, T, sink, window, sink, ns, 0.1)),
               oracle.compact(oracle.mask(ell, T, sink, window, sink, ns, 0.3)),
               oracle.compact(oracle.mask(ell, T, sink, window, sink, ns, 0.1, reversed=True)),
               oracle.compact(rand_keep),
               np.zeros(0, np.int32),
               oracle.compact(oracle.mask(ell, T, sink, window, sink, ns, 0.2))]
    lists_h = [np.asarray(x, np.int32) for x in lists_h]
    assert len(lists_h) == nc
    cls = np.array([[0, 1, 2, 3, 4, 5, 6, 7, 2],      # every class, one head each but class 2
                    [7, 7, 7, 1, 1, 1, 1, 7, 7],      # two classes only
                    [3, 0, 5, 3, 0, 5, 3, 0, 4]],     # one head of class 4
                   np.uint8)
    wlens = np.array([len(x) for x in lists_h], np.int64)
    woff = oracle.hs_offsets(cls, wlens)
    total = int(woff[-1])
    rf = (np.arange(T) // tpf).astype(np.int32)
    n_frames = T // tpf
    host, devt = _rope_inputs(rng, n_frames, 44, float(n_frames), 9.0, 4.0, dev, True)
    caps = [T] * nc
    caps[3] = int(wlens[3])                           # filled to its capacity exactly
    caps[6] = 0
    lists = [torch.zeros(max(1, caps[c]), dtype=torch.int32, device=dev) for c in range(nc)]
    rfs = [torch.zeros(max(1, caps[c]), dtype=torch.int32, device=dev) for c in range(nc)]
    for c in range(nc):
        n = int(wlens[c])
        if n:
            lists[c][:n] = to_dev(lists_h[c], dev)
            rfs[c][:n] = to_dev(rf[lists_h[c]], dev)
    lens = to_dev(wlens, dev)
    head_class = to_dev(cls.ravel(), dev)
    offsets = torch.empty(L * H + 1, dtype=torch.int64, device=dev)
    dp.dp_hs_offsets(head_class, L, H, lens, nc, offsets)
    k_out = torch.zeros((total + 8, D), dtype=torch.bfloat16, device=dev)
    v_out = torch.zeros((total + 8, D), dtype=torch.bfloat16, device=dev)
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
    rope = dp.make_rope(devt["theta"], devt["frame_t"], devt["frame_phase"], host["q0"],
                        host["knee"], host["inv_factor"])
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, 44) // 4, dtype=torch.float32,
                     device=dev)
    if fused:
        dp.dp_hs_gather_kv(kv, head_class, nc, cidx, lens, caps, offsets, crf, rope, ws)
    else:
        dp.dp_hs_gather_kv(kv, head_class, nc, cidx, lens, caps, offsets)
        dp.dp_hs_rope_reindex(k_out, total, L, H, D, dtype, head_class, nc, lens, caps, offsets,
                              crf, rope, ws)
    torch.cuda.synchronize()
    assert err.item() == 0
    assert np.array_equal(offsets.cpu().numpy(), woff)
    w_k = np.zeros((total, D), kb.dtype)
    w_v = np.zeros((total, D), vb.dtype)
    for l in range(L):
        oracle.hs_gather_layer(kb[l], l, cls, lists_h, woff, w_k)
        oracle.hs_gather_layer(vb[l], l, cls, lists_h, woff, w_v)
    assert np.array_equal(bits(v_out[:total]), w_v)
    tables = oracle.rope_frames(host["frame_t"], host["frame_phase"], host["q0"], host["knee"],
                                host["inv_factor"], host["theta"])
    w_rf = np.zeros(total, np.int32)
    for i in range(L * H):
        w_rf[woff[i]:woff[i + 1]] = rf[lists_h[cls.ravel()[i]]]
    oracle.rope_headrows(w_k, w_rf, 0, tables)
    ok, worst, _ = keys_close(bits(k_out[:total]), w_k, TOL[dtype])
    assert ok, worst
    assert np.all(bits(k_out[total:]) == 0) and np.all(bits(v_out[total:]) == 0)


# --------------------------------------------------------------------------
# whole tiny workload (1 layer, 2 heads, head_dim 64, fp32, 8 chunks of 64)
# --------------------------------------------------------------------------
def test_tiny_workload_end_to_end():
    import __graft_entry__
    device()
    __graft_entry__.smoke()


def test_compact_and_gather_at_the_int32_row_limit():
    """Maximum size: 2^31 - 1 rows, the most an int32 row index addresses (the
    API's limit).  A random keep mask (rows 0 and T - 1 kept) is compacted and
    K and V rows of 16 bytes (one head of 8 bf16) are gathered; the index list
    is checked to be ascending and to list exactly the kept rows, and every
    gathered row against its source, in chunks, on the device."""
    dev = device()
    if torch.cuda.get_device_properties(0).total_memory < (200 << 30):
        pytest.skip("needs about 140 GiB of device memory")
    T = (1 << 31) - 1
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    keep = (torch.rand(T, device=dev, generator=g) < 0.3).to(torch.uint8)
    keep[0] = 1
    keep[T - 1] = 1
    idx = torch.empty(T, dtype=torch.int32, device=dev)
    n_dev = torch.zeros(1, dtype=torch.int64, device=dev)
    ws = torch.empty(dp.dp_compact_workspace_bytes(T) // 4 + 1, dtype=torch.int32, device=dev)
    dp.dp_compact_index(keep, T, idx, n_dev, None, None, ws)
    torch.cuda.synchronize()
    n = int(n_dev.item())
    assert n == int(keep.sum(dtype=torch.int64).item())
    assert int(idx[0].item()) == 0 and int(idx[n - 1].item()) == T - 1
    step = 1 << 28
    for a in range(0, n, step):
        b = min(n, a + step)
        seg = idx[a:b].long()
        assert bool((keep[seg] == 1).all().item())
        if b - a > 1:
            assert bool((seg[1:] > seg[:-1]).all().item())
        if a > 0:
            assert int(idx[a].item()) > int(idx[a - 1].item())
        del seg
    del ws
    torch.cuda.empty_cache()

    srcs = [torch.randint(-32768, 32767, (T, 1, 8), dtype=torch.int16, device=dev,
                          generator=g).view(torch.bfloat16) for _ in range(2)]
    dsts = [torch.empty((n, 1, 8), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive = []
    kv = _kv_struct([srcs[0]], [srcs[1]], [dsts[0]], [dsts[1]], n, err, alive)
    dp.dp_gather_kv(kv, idx, n_dev)
    torch.cuda.synchronize()
    assert err.item() == 0
    # checked in chunks through the source window each chunk's (ascending)
    # indices span, so no single torch launch sees a 2^31-row operand
    step = 1 << 24
    for s_, d_ in zip(srcs, dsts):
        s16, d16 = s_.view(torch.int16), d_.view(torch.int16)
        for a in range(0, n, step):
            b = min(n, a + step)
            lo, hi = int(idx[a].item()), int(idx[b - 1].item()) + 1
            loc = idx[a:b].long() - lo
            assert torch.equal(d16[a:b], s16[lo:hi].index_select(0, loc)), a
    print("int32 row limit: %d rows, %d kept, gathered bit for bit" % (T, n))
    del srcs, dsts, keep, idx
    torch.cuda.empty_cache()


def test_score_mask_and_score_index_at_the_int32_row_limit():
    """Maximum size for the mask and the one-call index: a 2^31 - 1 row
    sequence with a sink, a window, one scored chunk (the eviction step's
    6,240 scores) and history in between (kept in score mode).  dp_score_index
    takes its separate-kernel path at this size; both calls must give the same
    mask, and the index list the kept rows."""
    dev = device()
    if torch.cuda.get_device_properties(0).total_memory < (64 << 30):
        pytest.skip("needs about 20 GiB of device memory")
    T = (1 << 31) - 1
    w = dpsynth.WORKLOADS["eviction"]
    C, d = w.chunk_tokens, w.d
    sink, window = C, 3 * C
    x0, xf = dpsynth.score_inputs(w)
    x0d, xfd = to_dev(x0, dev), to_dev(xf, dev)
    pol = dp.make_policy(T, sink, window, sink, C, w.gamma)
    keep = torch.empty(T, dtype=torch.uint8, device=dev)
    dp.dp_score_mask(x0d, xfd, d, d, pol, None, keep)
    want_sc = oracle.mask(oracle.score_f32(x0, xf, d), C, 0, 0, 0, C, w.gamma)
    torch.cuda.synchronize()
    assert np.array_equal(keep[sink:sink + C].cpu().numpy(), want_sc)
    assert bool((keep[:sink] == 1).all().item()) and bool((keep[T - window:] == 1).all().item())
    n_want = T - (C - int(want_sc.sum()))
    assert int(keep.sum(dtype=torch.int64).item()) == n_want      # history rows all kept

    keep2 = torch.empty(T, dtype=torch.uint8, device=dev)
    idx = torch.empty(T, dtype=torch.int32, device=dev)
    n_dev = torch.zeros(1, dtype=torch.int64, device=dev)
    ws = torch.zeros(dp.dp_score_index_workspace_bytes(T) // 8 + 1, dtype=torch.int64, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dp.dp_score_index(x0d, xfd, d, d, pol, None, keep2, idx, n_dev, None, None, ws, err)
    torch.cuda.synchronize()
    assert err.item() == 0 and int(n_dev.item()) == n_want
    assert torch.equal(keep2, keep)
    n = n_want
    assert int(idx[0].item()) == 0 and int(idx[n - 1].item()) == T - 1
    dropped = torch.from_numpy(np.flatnonzero(want_sc == 0) + sink).to(dev)
    step = 1 << 24
    for a in range(0, n, step):
        b = min(n, a + step)
        seg = idx[a:b].long()
        assert bool((keep[seg] == 1).all().item())
        if b - a > 1:
            assert bool((seg[1:] > seg[:-1]).all().item())
        if a > 0:
            assert int(idx[a].item()) > int(idx[a - 1].item())
    assert not bool(torch.isin(dropped, idx[:sink + C].long()).any().item())
    print("int32 row limit: mask and index over %d rows, %d kept" % (T, n))
    del keep, keep2, idx, ws
    torch.cuda.empty_cache()


def test_rope_reindex_at_the_int32_row_limit():
    """Maximum size for the in-place re-index: 2^31 - 1 rows of one 8-dim bf16
    head (4 temporal pairs, one 16-byte vector per row), 2,048 frames of 2^20
    rows; the last frames lie within the knee and stay untouched.  Sampled rows
    against the oracle."""
    dev = device()
    if torch.cuda.get_device_properties(0).total_memory < (64 << 30):
        pytest.skip("needs about 40 GiB of device memory")
    T, tpf, n_frames = (1 << 31) - 1, 1 << 20, 2048
    g = torch.Generator(device=dev)
    g.manual_seed(9)
    k = torch.randn((T, 1, 8), device=dev, generator=g, dtype=torch.bfloat16).mul_(2.0)
    rf = torch.arange(T, device=dev, dtype=torch.int32) >> 20
    theta = dpsynth.rope_theta(4)
    ft = np.arange(n_frames, dtype=np.float32)
    host = dict(theta=theta, frame_t=ft, frame_phase=ft.copy(), q0=float(n_frames), knee=6.0,
                inv_factor=np.float32(0.125))
    rows = np.unique(np.concatenate([[0, 1, tpf - 1, tpf, T // 2, T - tpf - 1, T - 2, T - 1],
                                     np.random.default_rng(3).integers(0, T, 4000)]))
    def sampled():                    # row views stacked: no launch sees a 2^31-row index
        return bits(torch.stack([k[int(r)] for r in rows]))

    before = sampled()
    rope = dp.make_rope(to_dev(theta, dev), to_dev(ft, dev), to_dev(ft.copy(), dev), host["q0"],
                        host["knee"], host["inv_factor"])
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, 4) // 4 + 4, dtype=torch.float32,
                     device=dev)
    arr = dp.ptr_array([k], dev)
    dp.dp_rope_reindex(arr, 1, 1, 8, dp.DP_BF16, T, None, rf, rope, ws)
    torch.cuda.synchronize()
    got = sampled()
    tables = oracle.rope_frames(ft, ft.copy(), host["q0"], host["knee"], host["inv_factor"], theta)
    want = before.copy()
    oracle.rope_rows(want, (rows >> 20).astype(np.int32), 0, tables)
    ok, worst, _ = keys_close(got, want, TOL[dp.DP_BF16])
    assert ok, worst
    recent = (n_frames - (rows >> 20)) <= host["knee"]
    assert recent.any() and np.array_equal(got[recent], before[recent])
    print("int32 row limit: re-index over %d rows, %d sampled" % (T, rows.shape[0]))
    del k, rf, arr
    torch.cuda.empty_cache()
