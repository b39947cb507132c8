"""GPU parity of the segment-append compaction in place (dp_append_kept) and of
a rollout in the [sink | window ring | history] layout.

The DeCoPrune page (section 어떻게 동작하나) compacts a chunk when it leaves
the window.  Appending only the kept rows of that chunk at the history tail
must give, step after step, the same set of cached rows (contents and
frames) as the out-of-place gather of the whole cache; only the row order
differs, which attention does not see.
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import dpsynth
import oracle
from gpu_helpers import bf16_from_bits, bits, device, keys_close, random_bf16_bits, to_dev

pytestmark = pytest.mark.gpu


def _buf(rng, L, cap, H, D, dtype):
    if dtype == dp.DP_BF16:
        return random_bf16_bits(rng, (L, cap, H, D))
    return rng.standard_normal((L, cap, H, D)).astype(np.float32).view(np.uint32)


def _dev(b, dtype, dev):
    if dtype == dp.DP_BF16:
        return [bf16_from_bits(b[l], dev) for l in range(b.shape[0])]
    return [to_dev(b[l].view(np.float32), dev) for l in range(b.shape[0])]


def _inplace(k, v, dtype, cap, err, alive):
    kv = dp.dp_kv_inplace()
    arrs = [dp.ptr_array(k, k[0].device), dp.ptr_array(v, k[0].device) if v is not None else None]
    alive += arrs
    kv.k_layers = arrs[0].data_ptr()
    kv.v_layers = arrs[1].data_ptr() if arrs[1] is not None else None
    _, H, D = k[0].shape
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = len(k), H, D, dtype
    kv.capacity = cap
    kv.dev_error = err.data_ptr()
    return kv


def _slot_index(keep_slot, dev):
    C = keep_slot.shape[0]
    idx = torch.empty(C, dtype=torch.int32, device=dev)
    n = torch.zeros(1, dtype=torch.int64, device=dev)
    ws = torch.empty(dp.dp_compact_workspace_bytes(C) // 4, dtype=torch.int32, device=dev)
    dp.dp_compact_index(to_dev(keep_slot, dev), C, idx, n, None, None, ws)
    return idx, n


@pytest.mark.parametrize("L,H,D,dtype,C", [(3, 5, 32, dp.DP_BF16, 700), (2, 2, 64, dp.DP_F32, 333),
                                         (2, 40, 128, dp.DP_BF16, 1560)])
@pytest.mark.parametrize("with_v", [True, False])
def test_append_kept_matches_oracle(L, H, D, dtype, C, with_v):
    dev = device()
    rng = np.random.default_rng(C + H)
    R = 3
    cap = C + R * C + 2 * C
    kb, vb = _buf(rng, L, cap, H, D, dtype), _buf(rng, L, cap, H, D, dtype)
    rf = rng.integers(0, 90, cap).astype(np.int32)
    tail0 = C + R * C + C // 3                       # some history already there
    slot = 1
    slot_begin = C + slot * C
    keep = (rng.random(C) < 0.3).astype(np.uint8)
    k, v = _dev(kb, dtype, dev), (_dev(vb, dtype, dev) if with_v else None)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive = []
    kv = _inplace(k, v, dtype, cap, err, alive)
    idx, n = _slot_index(keep, dev)
    tail = torch.tensor([tail0], dtype=torch.int64, device=dev)
    rf_d = to_dev(rf, dev)
    dp.dp_append_kept(kv, slot_begin, C, idx, n, tail, rf_d)
    torch.cuda.synchronize()
    widx = oracle.compact(keep)
    kk = kb.copy()
    rfo = rf.copy()
    t1 = oracle.append_kept(kk, slot_begin, C, widx, tail0, rfo)
    assert err.item() == 0 and tail.item() == t1
    assert np.array_equal(rf_d.cpu().numpy(), rfo)
    for l in range(L):
        assert np.array_equal(bits(k[l]), kk[l]), l
    if with_v:
        vv = vb.copy()
        oracle.append_kept(vv, slot_begin, C, widx, tail0, None)
        for l in range(L):
            assert np.array_equal(bits(v[l]), vv[l]), l


@pytest.mark.parametrize("rate", [0.0, 1.0])
def test_append_kept_nothing_or_everything(rate):
    """The leaving chunk keeps none of its rows (the tail stays, the slot's
    frames are still retired) or all of them (the whole slot is appended)."""
    dev = device()
    rng = np.random.default_rng(int(rate * 10) + 5)
    L, H, D, dtype, C, R = 2, 40, 128, dp.DP_BF16, 1560, 3
    cap = C + R * C + 2 * C
    kb, vb = _buf(rng, L, cap, H, D, dtype), _buf(rng, L, cap, H, D, dtype)
    rf = rng.integers(0, 90, cap).astype(np.int32)
    tail0 = C + R * C + 17
    slot_begin = C + 2 * C
    keep = np.full(C, 1 if rate else 0, np.uint8)
    k, v = _dev(kb, dtype, dev), _dev(vb, dtype, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive = []
    kv = _inplace(k, v, dtype, cap, err, alive)
    idx, n = _slot_index(keep, dev)
    tail = torch.tensor([tail0], dtype=torch.int64, device=dev)
    rf_d = to_dev(rf, dev)
    dp.dp_append_kept(kv, slot_begin, C, idx, n, tail, rf_d)
    torch.cuda.synchronize()
    widx = oracle.compact(keep)
    assert widx.shape[0] == (C if rate else 0)
    kk, vv, rfo = kb.copy(), vb.copy(), rf.copy()
    t1 = oracle.append_kept(kk, slot_begin, C, widx, tail0, rfo)
    oracle.append_kept(vv, slot_begin, C, widx, tail0, None)
    assert err.item() == 0 and tail.item() == t1 == tail0 + widx.shape[0]
    assert np.array_equal(rf_d.cpu().numpy(), rfo)
    assert np.all(rfo[slot_begin:slot_begin + C] == -1)
    for l in range(L):
        assert np.array_equal(bits(k[l]), kk[l]), l
        assert np.array_equal(bits(v[l]), vv[l]), l


@pytest.mark.parametrize("case", ["capacity", "overlap"])
def test_append_kept_refuses_on_device(case):
    dev = device()
    rng = np.random.default_rng(7)
    L, H, D, C = 2, 4, 64, 256
    cap = 6 * C
    kb = _buf(rng, L, cap, H, D, dp.DP_BF16)
    keep = np.ones(C, np.uint8)
    k = _dev(kb, dp.DP_BF16, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive = []
    kv = _inplace(k, None, dp.DP_BF16, cap, err, alive)
    idx, n = _slot_index(keep, dev)
    slot_begin = C
    tail0 = cap - C // 2 if case == "capacity" else slot_begin + 10
    tail = torch.tensor([tail0], dtype=torch.int64, device=dev)
    rf = to_dev(np.arange(cap, dtype=np.int32), dev)
    dp.dp_append_kept(kv, slot_begin, C, idx, n, tail, rf)
    torch.cuda.synchronize()
    assert err.item() == (dp.DP_ECAPACITY if case == "capacity" else dp.DP_ERANGE)
    assert tail.item() == tail0
    assert np.array_equal(rf.cpu().numpy(), np.arange(cap))
    for l in range(L):
        assert np.array_equal(bits(k[l]), kb[l])


# --------------------------------------------------------------------------
# rollout in the ring layout vs the out-of-place rollout of the same inputs
# --------------------------------------------------------------------------
L, H, D = 2, 3, 64
TPF, F = 16, 2
C = TPF * F
W = 2                     # window chunks after the eviction; the ring holds W + 1 slots
R = W + 1
STEPS = 6
NPAIRS = 12
KNEE = float(W * F)
FACTOR = 4.0


def _scores(rng):
    xf = rng.standard_normal((C, 16)).astype(np.float32)
    sig = np.exp(rng.uniform(np.log(0.05), np.log(0.6), C))[:, None]
    return (xf + sig * rng.standard_normal((C, 16))).astype(np.float32), xf


def _rope_rows_valid(k, rf, tables):
    """Oracle re-index of the rows whose frame is valid (retired rows skipped)."""
    rows = np.flatnonzero(rf >= 0)
    sub = np.ascontiguousarray(k[rows])
    oracle.rope_rows(sub, rf[rows], 0, tables)
    k[rows] = sub


def test_ring_rollout_matches_oracle_and_out_of_place():
    dev = device()
    rng = np.random.default_rng(5)
    n_frames = (R + 2 + STEPS) * F
    theta = dpsynth.rope_theta(NPAIRS)
    frame_t = np.arange(n_frames, dtype=np.float32)
    cap = C + R * C + STEPS * C
    # initial chunks: sink (chunk 0) and chunks 1..R in ring slots 0..R-1
    init_k = random_bf16_bits(rng, (L, (R + 1) * C, H, D), 2.0)
    init_v = random_bf16_bits(rng, (L, (R + 1) * C, H, D))
    init_rf = (np.arange((R + 1) * C) // TPF).astype(np.int32)
    draws = []
    for s in range(STEPS):
        x0, xf = _scores(rng)
        draws.append((x0, xf, random_bf16_bits(rng, (L, C, H, D), 2.0),
                      random_bf16_bits(rng, (L, C, H, D))))

    # ---- GPU, ring layout ----
    kb = np.zeros((L, cap, H, D), np.uint16)
    vb = np.zeros((L, cap, H, D), np.uint16)
    kb[:, :(R + 1) * C], vb[:, :(R + 1) * C] = init_k, init_v
    rf = np.full(cap, -1, np.int32)
    rf[:(R + 1) * C] = init_rf
    k, v = _dev(kb, dp.DP_BF16, dev), _dev(vb, dp.DP_BF16, dev)
    rf_d = to_dev(rf, dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive = []
    kv = _inplace(k, v, dp.DP_BF16, cap, err, alive)
    tail = torch.tensor([(R + 1) * C], dtype=torch.int64, device=dev)
    phase_d = to_dev(frame_t.copy(), dev)
    th_d, ft_d = to_dev(theta, dev), to_dev(frame_t, dev)
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, NPAIRS) // 4 + 4, dtype=torch.float32,
                     device=dev)
    arr_k = dp.ptr_array(k, dev)
    # ---- oracle, ring layout ----
    ok_, ov_, orf, otail, ophase = kb.copy(), vb.copy(), rf.copy(), (R + 1) * C, frame_t.copy()
    # ---- oracle, out-of-place layout ----
    pk, pv, prf = init_k.copy(), init_v.copy(), init_rf.copy()
    pphase = frame_t.copy()
    for s in range(STEPS):
        x0, xf, k_new, v_new = draws[s]
        slot = s % R
        sb = C + slot * C
        q0 = float((R + 1 + s) * F)                 # first frame of the next chunk
        # GPU
        keep = torch.empty(C, dtype=torch.uint8, device=dev)
        dp.dp_score_mask(to_dev(x0, dev), to_dev(xf, dev), 16, 16,
                         dp.make_policy(C, 0, 0, 0, C, 0.1), None, keep)
        idx = torch.empty(C, dtype=torch.int32, device=dev)
        nk = torch.zeros(1, dtype=torch.int64, device=dev)
        wsc = torch.empty(dp.dp_compact_workspace_bytes(C) // 4, dtype=torch.int32, device=dev)
        dp.dp_compact_index(keep, C, idx, nk, None, None, wsc)
        dp.dp_append_kept(kv, sb, C, idx, nk, tail, rf_d)
        rope = dp.make_rope(th_d, ft_d, phase_d, q0, KNEE, 1.0 / FACTOR)
        dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws)                  # old keys only:
        dp.dp_rope_apply(arr_k, L, H, D, dp.DP_BF16, 0, C, None, rf_d, rope, ws)        # sink
        dp.dp_rope_apply(arr_k, L, H, D, dp.DP_BF16, C + R * C, cap, tail, rf_d, rope, ws)  # history
        c_new = R + 1 + s
        for l in range(L):                          # the model writes the new chunk into the slot
            k[l][sb:sb + C] = bf16_from_bits(k_new[l], dev)
            v[l][sb:sb + C] = bf16_from_bits(v_new[l], dev)
        rf_d[sb:sb + C] = torch.from_numpy((c_new * F + np.arange(C) // TPF).astype(np.int32)).to(dev)
        torch.cuda.synchronize()
        assert err.item() == 0, s
        # oracle, ring layout
        ell = oracle.score_f32(x0, xf)
        widx = oracle.compact(oracle.mask(ell, C, 0, 0, 0, C, 0.1))
        otail = oracle.append_kept(ok_, sb, C, widx, otail, orf)
        oracle.append_kept(ov_, sb, C, widx, otail - widx.shape[0], None)
        tables = oracle.rope_frames(frame_t, ophase, q0, KNEE, np.float32(1.0 / FACTOR), theta)
        ophase = tables[3]
        for l in range(L):
            view = ok_[l][:otail]
            _rope_rows_valid(view, orf[:otail], tables)
        ok_[:, sb:sb + C], ov_[:, sb:sb + C] = k_new, v_new
        orf[sb:sb + C] = c_new * F + np.arange(C) // TPF
        assert tail.item() == otail, s
        assert np.array_equal(rf_d.cpu().numpy(), orf), s
        assert np.array_equal(phase_d.cpu().numpy(), ophase), s
        for l in range(L):
            assert np.array_equal(bits(v[l]), ov_[l]), (s, l)
            good, worst, _ = keys_close(bits(k[l]), ok_[l], 2e-2)
            assert good, (s, l, worst)
        # oracle, out-of-place: gather the whole cache, then append the new chunk
        T = pk.shape[1]
        keep_p = oracle.mask(ell, T, C, W * C, T - (W + 1) * C, C, 0.1)
        pidx = oracle.compact(keep_p)
        pk, pv, prf = oracle.gather(pk, pidx), oracle.gather(pv, pidx), oracle.gather_i32(prf, pidx)
        tables_p = oracle.rope_frames(frame_t, pphase, q0, KNEE, np.float32(1.0 / FACTOR), theta)
        pphase = tables_p[3]
        for l in range(L):
            oracle.rope_rows(pk[l], prf, 0, tables_p)
        pk = np.concatenate([pk, k_new], axis=1)
        pv = np.concatenate([pv, v_new], axis=1)
        prf = np.concatenate([prf, (c_new * F + np.arange(C) // TPF).astype(np.int32)])
    # the ring cache holds the same rows as the out-of-place cache, in another order
    live = np.flatnonzero(orf[:otail] >= 0)
    assert live.shape[0] == pk.shape[1]

    def canon(kc, vc, rfc):
        keyv = np.concatenate([rfc[:, None].astype(np.int64),
                               kc.transpose(1, 0, 2, 3).reshape(rfc.shape[0], -1).astype(np.int64),
                               vc.transpose(1, 0, 2, 3).reshape(rfc.shape[0], -1).astype(np.int64)],
                              axis=1)
        return keyv[np.lexsort(keyv.T[::-1])]

    ring = canon(ok_[:, live], ov_[:, live], orf[live])
    flat = canon(pk, pv, prf)
    assert np.array_equal(ring, flat)
    print("ring rollout: %d steps, %d live rows of %d slots+history" % (STEPS, live.shape[0], otail))


@pytest.mark.parametrize("axis", [dp.DP_AXIS_PAGE, dp.DP_AXIS_COMPRESSED])
def test_ring_step_helper_against_oracle(axis):
    """compaction_dp_score_amd.step.RingStep rolled six evictions forward,
    against the oracle's own rollout of the ring layout on the same inputs:
    the leaving chunk's score, mask and index list, its append at the tail
    (K, V and frames), then the page's re-index of every live key for the new
    q0 (on the compressed axis the frames past the knee take the phase t/c),
    the window rows included, with no assumption about which rows move.
    After every step: tail, row frames and phase table exact, V bit for bit,
    K within the re-index tolerance (DeCoPrune page, 어떻게 동작하나 and
    무엇과 다른가).  On the compressed axis the sink crosses the knee at the
    first step, so a helper that left it out fails here."""
    from compaction_dp_score_amd.step import RingStep
    dev = device()
    rng = np.random.default_rng(23)
    n_frames = (R + 2 + STEPS) * F
    theta = dpsynth.rope_theta(NPAIRS)
    frame_t = np.arange(n_frames, dtype=np.float32)
    cap = C + R * C + STEPS * C
    kb = np.zeros((L, cap, H, D), np.uint16)
    vb = np.zeros((L, cap, H, D), np.uint16)
    kb[:, :(R + 1) * C] = random_bf16_bits(rng, (L, (R + 1) * C, H, D), 2.0)
    vb[:, :(R + 1) * C] = random_bf16_bits(rng, (L, (R + 1) * C, H, D))
    rf0 = np.full(cap, -1, np.int32)
    rf0[:(R + 1) * C] = np.arange((R + 1) * C) // TPF
    th_d, ft_d = to_dev(theta, dev), to_dev(frame_t, dev)
    hk, hv = _dev(kb, dp.DP_BF16, dev), _dev(vb, dp.DP_BF16, dev)
    hrf = to_dev(rf0, dev)
    htail = torch.tensor([(R + 1) * C], dtype=torch.int64, device=dev)
    hphase = to_dev(frame_t.copy(), dev)
    step = RingStep(k_layers=hk, v_layers=hv, sink_len=C, chunk_rows=C, n_slots=R,
                    frames_per_chunk=F, row_frame=hrf, tail=htail, d=16, gamma=0.1,
                    rope=dict(theta=th_d, frame_t=ft_d, frame_phase=hphase, knee=KNEE,
                              inv_factor=1.0 / FACTOR), axis=axis)
    compressed = axis == dp.DP_AXIS_COMPRESSED
    ok_, ov_, orf, otail, ophase = kb.copy(), vb.copy(), rf0.copy(), (R + 1) * C, frame_t.copy()
    for s in range(STEPS):
        x0, xf = _scores(rng)
        k_new = random_bf16_bits(rng, (L, C, H, D), 2.0)
        v_new = random_bf16_bits(rng, (L, C, H, D))
        slot = s % R
        sb = C + slot * C
        q0 = float((R + 1 + s) * F)                 # first frame of the next chunk
        new_frames = ((R + 1 + s) * F + np.arange(C) // TPF).astype(np.int32)
        step.evict(slot, to_dev(x0, dev), to_dev(xf, dev), q0)
        for l in range(L):                          # the model writes the next chunk
            hk[l][sb:sb + C] = bf16_from_bits(k_new[l], dev)
            hv[l][sb:sb + C] = bf16_from_bits(v_new[l], dev)
        step.write_chunk(slot, to_dev(new_frames, dev))
        # oracle
        widx = oracle.compact(oracle.mask(oracle.score_f32(x0, xf), C, 0, 0, 0, C, 0.1))
        t_before = otail
        otail = oracle.append_kept(ok_, sb, C, widx, otail, orf)
        oracle.append_kept(ov_, sb, C, widx, t_before, None)
        tables = oracle.rope_frames(frame_t, ophase, q0, KNEE, np.float32(1.0 / FACTOR), theta,
                                    compressed=compressed)
        ophase = tables[3]
        for l in range(L):
            view = ok_[l][:otail]
            _rope_rows_valid(view, orf[:otail], tables)
        ok_[:, sb:sb + C], ov_[:, sb:sb + C] = k_new, v_new
        orf[sb:sb + C] = new_frames
        torch.cuda.synchronize()
        assert step.dev_error.item() == 0, s
        assert htail.item() == otail, s
        assert np.array_equal(hrf.cpu().numpy(), orf), s
        assert np.array_equal(hphase.cpu().numpy(), ophase), s
        for l in range(L):
            assert np.array_equal(bits(hv[l]), ov_[l]), (s, l)
            good, worst, _ = keys_close(bits(hk[l]), ok_[l], 2e-2)
            assert good, (s, l, worst)
    if compressed:                                  # every live key past the knee is at t/c
        live = np.flatnonzero(orf[:otail] >= 0)
        past = q0 - frame_t[orf[live]] > KNEE
        assert np.array_equal(ophase[orf[live][past]], frame_t[orf[live][past]] / FACTOR)


def test_ring_step_knee_must_cover_the_window():
    """A knee below the window span would leave window keys at their written
    phase past the knee; on the compressed axis a knee a frame or more above it
    would append rows that cross it later in the history, where no key is
    visited again: the helper refuses both."""
    from compaction_dp_score_amd.step import RingStep
    dev = device()
    k = [torch.zeros((8 * C, H, D), dtype=torch.bfloat16, device=dev)]
    args = dict(k_layers=k, v_layers=None, sink_len=C, chunk_rows=C, n_slots=R,
                frames_per_chunk=F, row_frame=torch.full((8 * C,), -1, dtype=torch.int32,
                                                         device=dev),
                tail=torch.zeros(1, dtype=torch.int64, device=dev), d=16, gamma=0.1)
    rope = dict(theta=torch.ones(NPAIRS, device=dev), frame_t=torch.zeros(4, device=dev),
                frame_phase=torch.zeros(4, device=dev), inv_factor=0.25)
    for axis in (dp.DP_AXIS_PAGE, dp.DP_AXIS_COMPRESSED):
        with pytest.raises(ValueError):
            RingStep(rope=dict(rope, knee=KNEE - 0.5), axis=axis, **args)
        RingStep(rope=dict(rope, knee=KNEE), axis=axis, **args)
    with pytest.raises(ValueError):
        RingStep(rope=dict(rope, knee=KNEE + 1), axis=dp.DP_AXIS_COMPRESSED, **args)
    RingStep(rope=dict(rope, knee=KNEE + 1), axis=dp.DP_AXIS_PAGE, **args)
