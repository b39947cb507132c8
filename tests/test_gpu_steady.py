"""GPU parity of the steady-state re-index: dp_rope_shift (one uniform phase
step over a row range, no row frames) and the re-index fused into
dp_append_kept, against the oracle, and a ring-layout rollout that uses them
from the second step on, bit for bit against the general path
(dp_rope_prepare + dp_rope_apply over every old key) and the oracle.

In a rollout q0 advances F frames per step, so every frame that was past the
knee before the step and still is after it moves by F (1 - 1/c) (pinned in
the oracle tests); only the chunk that has just left the window needs its
per-frame step, and it is re-rotated while the append copies it.
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import dpsynth
import oracle
from gpu_helpers import bf16_from_bits, bits, device, random_bf16_bits, to_dev

pytestmark = pytest.mark.gpu


def _layers(rng, L, T, H, D, dtype, dev):
    if dtype == dp.DP_BF16:
        b = random_bf16_bits(rng, (L, T, H, D), 2.0)
        return b, [bf16_from_bits(b[l], dev) for l in range(L)]
    b = rng.standard_normal((L, T, H, D)).astype(np.float32)
    return b.view(np.uint32), [to_dev(b[l], dev) for l in range(L)]


def _sws(npairs, dev):
    return torch.empty(dp.dp_rope_shift_workspace_bytes(npairs) // 4 + 4, dtype=torch.float32,
                       device=dev)


def _host(b, dtype):
    return b if dtype == dp.DP_BF16 else b.view(np.float32)


@pytest.mark.parametrize("L,T,H,D,dtype,pb,npairs,rb,cap,dev_rows", [
    (2, 300, 8, 128, dp.DP_BF16, 0, 44, 0, 300, False),
    (3, 257, 5, 64, dp.DP_BF16, 4, 13, 10, 250, True),
    (2, 130, 4, 64, dp.DP_F32, 2, 12, 7, 130, False),
    (1, 100, 40, 128, dp.DP_BF16, 8, 44, 31, 100, True),
    (2, 64, 3, 32, dp.DP_F32, 0, 16, 0, 64, True),
])
def test_rope_shift_matches_oracle(L, T, H, D, dtype, pb, npairs, rb, cap, dev_rows):
    dev = device()
    rng = np.random.default_rng(T + H + npairs)
    kb, k = _layers(rng, L, T, H, D, dtype, dev)
    theta = dpsynth.rope_theta(npairs)
    n_rows = cap - 3 if dev_rows else cap                    # a device count below the capacity
    nd = torch.tensor([n_rows], dtype=torch.int64, device=dev) if dev_rows else None
    arr = dp.ptr_array(k, dev)
    dp.dp_rope_shift(arr, L, H, D, dtype, rb, cap, nd, to_dev(theta, dev), pb, npairs, 3.5,
                     _sws(npairs, dev))
    torch.cuda.synchronize()
    tab = oracle.rope_uniform(theta, 3.5)
    for l in range(L):
        want = _host(kb[l].copy(), dtype)
        sub = np.ascontiguousarray(want[rb:n_rows])
        oracle.rope_rows(sub, np.zeros(sub.shape[0], np.int32), pb, tab)
        want[rb:n_rows] = sub
        assert np.array_equal(bits(k[l]), want.view(kb.dtype)), l   # rows outside untouched


def test_rope_shift_zero_step_writes_nothing():
    dev = device()
    rng = np.random.default_rng(3)
    kb, k = _layers(rng, 1, 50, 2, 64, dp.DP_BF16, dev)
    dp.dp_rope_shift(dp.ptr_array(k, dev), 1, 2, 64, dp.DP_BF16, 0, 50, None,
                     to_dev(dpsynth.rope_theta(8), dev), 0, 8, 0.0, _sws(8, dev))
    torch.cuda.synchronize()
    assert np.array_equal(bits(k[0]), kb[0])


def test_rope_shift_equals_apply_when_every_frame_steps_uniformly():
    """Frames that were past the knee at the previous q0 and still are: the
    per-frame tables hold the uniform step for each, and both paths agree
    bit for bit."""
    dev = device()
    rng = np.random.default_rng(4)
    L, H, D, npairs, tpf = 2, 6, 128, 44, 5
    F, knee, c = 4, 12.0, 8.0
    q0_prev, q0 = 40.0, 44.0
    frames = np.arange(0, 20, dtype=np.float32)             # all past the knee at both q0
    T = frames.shape[0] * tpf
    theta = dpsynth.rope_theta(npairs)
    _, _, _, ph = oracle.rope_frames(frames, frames, q0_prev, knee, np.float32(1 / c), theta)
    kb, k1 = _layers(rng, L, T, H, D, dp.DP_BF16, dev)
    k2 = [t.clone() for t in k1]
    rf = to_dev((np.arange(T) // tpf).astype(np.int32), dev)
    th = to_dev(theta, dev)
    rope = dp.make_rope(th, to_dev(frames, dev), to_dev(ph, dev), q0, knee, 1 / c)
    ws = torch.empty(dp.dp_rope_workspace_bytes(frames.shape[0], npairs) // 4 + 4,
                     dtype=torch.float32, device=dev)
    dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws)
    dp.dp_rope_apply(dp.ptr_array(k1, dev), L, H, D, dp.DP_BF16, 0, T, None, rf, rope, ws)
    dp.dp_rope_shift(dp.ptr_array(k2, dev), L, H, D, dp.DP_BF16, 0, T, None, th, 0, npairs,
                     F * (1 - 1 / c), _sws(npairs, dev))
    torch.cuda.synchronize()
    for l in range(L):
        assert np.array_equal(bits(k1[l]), bits(k2[l])), l
        assert not np.array_equal(bits(k1[l]), kb[l])


def test_append_with_fused_reindex_matches_oracle():
    dev = device()
    rng = np.random.default_rng(6)
    L, H, D, C, npairs, tpf = 2, 5, 64, 300, 12, 50
    cap = C * 4
    kb, k = _layers(rng, L, cap, H, D, dp.DP_BF16, dev)
    vb, v = _layers(rng, L, cap, H, D, dp.DP_BF16, dev)
    n_frames = cap // tpf
    rf = (np.arange(cap) // tpf).astype(np.int32)
    frames = np.arange(n_frames, dtype=np.float32)
    theta = dpsynth.rope_theta(npairs)
    q0, knee, c = float(n_frames), 6.0, 4.0
    slot_begin, tail0 = C, 2 * C
    keep = (rng.random(C) < 0.3).astype(np.uint8)
    idx = torch.empty(C, dtype=torch.int32, device=dev)
    nk = torch.zeros(1, dtype=torch.int64, device=dev)
    wsc = torch.empty(dp.dp_compact_workspace_bytes(C) // 4 + 1, dtype=torch.int32, device=dev)
    dp.dp_compact_index(to_dev(keep, dev), C, idx, nk, None, None, wsc)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv = dp.dp_kv_inplace()
    arr_k, arr_v = dp.ptr_array(k, dev), dp.ptr_array(v, dev)
    kv.k_layers, kv.v_layers = arr_k.data_ptr(), arr_v.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dp.DP_BF16
    kv.capacity, kv.dev_error = cap, err.data_ptr()
    phase = to_dev(frames.copy(), dev)
    rope = dp.make_rope(to_dev(theta, dev), to_dev(frames, dev), phase, q0, knee, 1 / c)
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, npairs) // 4 + 4, dtype=torch.float32,
                     device=dev)
    tail = torch.tensor([tail0], dtype=torch.int64, device=dev)
    rf_d = to_dev(rf, dev)
    dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws)
    dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf_d, rope, ws)
    torch.cuda.synchronize()
    assert err.item() == 0
    widx = oracle.compact(keep)
    n = widx.shape[0]
    tables = oracle.rope_frames(frames, frames, q0, knee, np.float32(1 / c), theta)
    for l in range(L):
        want_k = kb[l].copy()
        orf = rf.copy()
        oracle.append_kept(want_k[None], slot_begin, C, widx, tail0, orf)   # [1, cap, H, D]
        sub = np.ascontiguousarray(want_k[tail0:tail0 + n])
        oracle.rope_rows(sub, orf[tail0:tail0 + n], 0, tables)
        want_k[tail0:tail0 + n] = sub
        assert np.array_equal(bits(k[l]), want_k), l
        want_v = vb[l].copy()
        oracle.append_kept(want_v[None], slot_begin, C, widx, tail0, None)
        assert np.array_equal(bits(v[l]), want_v), l              # V is never rotated
    assert tail.item() == tail0 + n
    assert np.array_equal(phase.cpu().numpy(), tables[3])


# ring-layout rollout (as in the append tests): 2 frames per chunk, window 2
L, H, D = 2, 3, 64
TPF, F = 16, 2
C = TPF * F
W = 2
R = W + 1
STEPS = 6
NPAIRS = 12
KNEE = float(W * F)
FACTOR = 4.0
STEP = F * (1 - 1 / FACTOR)            # the uniform phase step: 1.5 frames


def test_steady_ring_rollout_equals_general_path_and_oracle():
    dev = device()
    rng = np.random.default_rng(8)
    n_frames = (R + 2 + STEPS) * F
    theta = dpsynth.rope_theta(NPAIRS)
    frame_t = np.arange(n_frames, dtype=np.float32)
    cap = C + R * C + STEPS * C
    hist = C + R * C
    kb = np.zeros((L, cap, H, D), np.uint16)
    vb = np.zeros((L, cap, H, D), np.uint16)
    kb[:, :hist] = random_bf16_bits(rng, (L, hist, H, D), 2.0)
    vb[:, :hist] = random_bf16_bits(rng, (L, hist, H, D))
    rf = np.full(cap, -1, np.int32)
    rf[:hist] = np.arange(hist) // TPF
    th_d, ft_d = to_dev(theta, dev), to_dev(frame_t, dev)
    sws = _sws(NPAIRS, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    paths = {}
    for name in ("general", "steady"):
        k = [bf16_from_bits(kb[l], dev) for l in range(L)]
        v = [bf16_from_bits(vb[l], dev) for l in range(L)]
        kv = dp.dp_kv_inplace()
        ak, av = dp.ptr_array(k, dev), dp.ptr_array(v, dev)
        kv.k_layers, kv.v_layers = ak.data_ptr(), av.data_ptr()
        kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dp.DP_BF16
        kv.capacity, kv.dev_error = cap, err.data_ptr()
        paths[name] = dict(k=k, v=v, kv=kv, ak=ak, av=av, rf=to_dev(rf, dev),
                           tail=torch.tensor([hist], dtype=torch.int64, device=dev),
                           phase=to_dev(frame_t.copy(), dev),
                           ws=torch.empty(dp.dp_rope_workspace_bytes(n_frames, NPAIRS) // 4 + 4,
                                          dtype=torch.float32, device=dev))
    ok_, orf, otail, ophase = kb.copy(), rf.copy(), hist, frame_t.copy()
    for s in range(STEPS):
        slot = s % R
        sb = C + slot * C
        q0 = float((R + 1 + s) * F)
        keep = (rng.random(C) < 0.25).astype(np.uint8)
        idx = torch.empty(C, dtype=torch.int32, device=dev)
        nk = torch.zeros(1, dtype=torch.int64, device=dev)
        wsc = torch.empty(dp.dp_compact_workspace_bytes(C) // 4 + 1, dtype=torch.int32, device=dev)
        dp.dp_compact_index(to_dev(keep, dev), C, idx, nk, None, None, wsc)
        k_new = random_bf16_bits(rng, (L, C, H, D), 2.0)
        for name, p in paths.items():
            rope = dp.make_rope(th_d, ft_d, p["phase"], q0, KNEE, 1.0 / FACTOR)
            if name == "general":
                dp.dp_append_kept(p["kv"], sb, C, idx, nk, p["tail"], p["rf"])
                dp.dp_rope_prepare(rope, D, dp.DP_BF16, p["ws"])
                dp.dp_rope_apply(p["ak"], L, H, D, dp.DP_BF16, 0, C, None, p["rf"], rope, p["ws"])
                dp.dp_rope_apply(p["ak"], L, H, D, dp.DP_BF16, hist, cap, p["tail"], p["rf"], rope,
                                 p["ws"])
            else:
                if s == 0:                       # the sink's first re-index: per frame
                    dp.dp_rope_prepare(rope, D, dp.DP_BF16, p["ws"])
                    dp.dp_rope_apply(p["ak"], L, H, D, dp.DP_BF16, 0, C, None, p["rf"], rope,
                                     p["ws"])
                else:                            # every old key moves by the uniform step
                    dp.dp_rope_shift(p["ak"], L, H, D, dp.DP_BF16, 0, C, None, th_d, 0, NPAIRS,
                                     STEP, sws)
                    dp.dp_rope_shift(p["ak"], L, H, D, dp.DP_BF16, hist, cap, p["tail"], th_d, 0,
                                     NPAIRS, STEP, sws)
                    dp.dp_rope_prepare(rope, D, dp.DP_BF16, p["ws"])
                dp.dp_append_kept(p["kv"], sb, C, idx, nk, p["tail"], p["rf"], rope, p["ws"])
            for l in range(L):                   # the model writes the next chunk into the slot
                p["k"][l][sb:sb + C] = bf16_from_bits(k_new[l], dev)
            p["rf"][sb:sb + C] = torch.from_numpy(((R + 1 + s) * F + np.arange(C) // TPF)
                                                  .astype(np.int32)).to(dev)
        torch.cuda.synchronize()
        assert err.item() == 0, s
        # oracle: append, then re-index every old key by its frame's step
        widx = oracle.compact(keep)
        otail = oracle.append_kept(ok_, sb, C, widx, otail, orf)
        tables = oracle.rope_frames(frame_t, ophase, q0, KNEE, np.float32(1.0 / FACTOR), theta)
        ophase = tables[3]
        for l in range(L):
            for lo, hi in ((0, C), (hist, otail)):
                rows = np.arange(lo, hi)
                rows = rows[orf[rows] >= 0]
                sub = np.ascontiguousarray(ok_[l][rows])
                oracle.rope_rows(sub, orf[rows], 0, tables)
                ok_[l][rows] = sub
        ok_[:, sb:sb + C] = k_new
        orf[sb:sb + C] = (R + 1 + s) * F + np.arange(C) // TPF
        for name, p in paths.items():
            assert p["tail"].item() == otail, (s, name)
            assert np.array_equal(p["phase"].cpu().numpy(), ophase), (s, name)
            assert np.array_equal(p["rf"].cpu().numpy(), orf), (s, name)
            for l in range(L):
                assert np.array_equal(bits(p["k"][l]), ok_[l]), (s, name, l)
    print("steady rollout: %d steps, tail %d" % (STEPS, otail))
