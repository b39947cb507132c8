"""GPU parity of the compressed time axis: keys past the RoPE knee re-indexed
once to phase t/c (dp_rope_prepare / dp_rope_apply / dp_append_kept with
axis DP_AXIS_COMPRESSED) and attended with dp_attention_lag, against the
float64 oracle of the page's own semantics: every key at t~ = q0 - g(q0 - t),
rotated exactly from the phase it was written at, then plain attention.

Tolerance: 6e-3 + 1e-2 |o|.  Against the page-axis reference this path has,
besides the dense kernel's roundings (bf16 probabilities and output), two
more: the rotated query and the once-rotated keys are bf16 (relative 2^-9 per
element, independent), which perturbs a score by about 2^-9 scale |q o k|_2
~ 2e-3 and an output, a probability-weighted mean of those perturbations
times (v - o), by about 1e-3 at these sizes.  The bar checks the rotation
semantics: a query turned the wrong way (lag of the wrong sign) misses by
~0.3.  That every 64-key tile of every lagged and plain range is read once is
checked separately under the derived bound of the dense kernel
(tests/test_gpu_attention_tiles.py), on keys that are zero on the temporal
pairs, where the lag changes nothing.
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import dpsynth
import oracle
from gpu_helpers import bf16_from_bits, bits, device, random_bf16_bits, to_dev

pytestmark = pytest.mark.gpu

ATOL, RTOL = 6e-3, 1e-2


def _check(got_bits, want, tag):
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(got - want)
    bound = ATOL + RTOL * np.abs(want)
    assert np.all(err <= bound), (tag, float((err - bound).max()), float(err.max()))
    return float(err.max())


def _page_phase(t, q0, knee, c):
    """t~ = q0 - g(q0 - t) in float64 (exact: every value is a multiple of 1/c)."""
    d = q0 - np.asarray(t, np.float64)
    return q0 - np.where(d <= knee, d, knee + (d - knee) / c)


def _page_reference(q, k, v, frame_of_row, frame_t, q0, knee, c, pair_begin, theta, rows,
                    n_kv=None):
    """Attention with every key at its page phase t~: the keys as written (phase
    t) rotated exactly in float64 by theta_j (t~ - t)."""
    n = k.shape[0] if n_kv is None else n_kv
    k64 = oracle._f64(k[:n]).copy()
    step = _page_phase(frame_t, q0, knee, c) - np.asarray(frame_t, np.float64)
    oracle.rope_rows_f64(k64, frame_of_row[:n], pair_begin, step, np.asarray(theta, np.float64))
    return oracle.attention(oracle._f64(q), k64, oracle._f64(v[:n]), rows)


def _compress(kd_list, H, D, n_rows, ranges, rf_d, theta_d, frame_t, q0, knee, c, pair_begin,
              dev):
    """Keys of the listed row ranges move to the compressed axis (phase t/c past
    the knee) through dp_rope_prepare + dp_rope_apply; returns the phases."""
    n_frames = frame_t.shape[0]
    npairs = theta_d.shape[0]
    phase = to_dev(frame_t.astype(np.float32), dev)
    rope = dp.make_rope(theta_d, to_dev(frame_t.astype(np.float32), dev), phase, q0, knee,
                        1.0 / c, pair_begin=pair_begin, axis=dp.DP_AXIS_COMPRESSED)
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, npairs) // 4 + 4, dtype=torch.float32,
                     device=dev)
    arr = dp.ptr_array(kd_list, dev)
    dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws)
    for lo, hi in ranges:
        dp.dp_rope_apply(arr, len(kd_list), H, D, dp.DP_BF16, lo, hi, None, rf_d, rope, ws)
    torch.cuda.synchronize()
    return phase.cpu().numpy(), arr


@pytest.mark.parametrize("n_q,n_kv,H", [(130, 700, 8), (1, 65, 5), (257, 64, 3)])
@pytest.mark.parametrize("device_count", [False, True])
def test_lag_reduces_to_dense_attention(n_q, n_kv, H, device_count):
    """One plain range over every row, or every row lagged by 0: the tile order
    is that of dp_attention and the result is bit for bit the same."""
    dev = device()
    rng = np.random.default_rng(n_q + n_kv + H)
    D, extra = 128, 21
    q = random_bf16_bits(rng, (n_q, H, D))
    k = random_bf16_bits(rng, (n_kv + extra, H, D))
    v = random_bf16_bits(rng, (n_kv + extra, H, D))
    k[n_kv:] = 0x7FC0                                 # NaN beyond the count: never read
    v[n_kv:] = 0x7FC0
    qd, kd, vd = bf16_from_bits(q, dev), bf16_from_bits(k, dev), bf16_from_bits(v, dev)
    theta = to_dev(dpsynth.rope_theta(44), dev)
    cap, cnt = (n_kv + extra, torch.tensor([n_kv], dtype=torch.int64, device=dev)) \
        if device_count else (n_kv, None)
    scale = 1.0 / np.sqrt(D)
    ref = torch.zeros((n_q, H, D), dtype=torch.bfloat16, device=dev)
    dp.dp_attention(qd, kd, vd, ref, n_q, cap, cnt, H, D, dp.DP_BF16, scale)
    for pb, pe, lag in ((0, cap + 5, 37.5), (0, n_kv, -3.0), (0, 0, 0.0), (n_kv, n_kv + 9, 0.0)):
        od = torch.full((n_q, H, D), 7.0, dtype=torch.bfloat16, device=dev)
        dp.dp_attention_lag(qd, kd, vd, od, n_q, cap, cnt, pb, pe, theta, 0, 44, lag, H, D,
                            dp.DP_BF16, scale)
        torch.cuda.synchronize()
        assert np.array_equal(bits(od), bits(ref)), (pb, pe, lag)


@pytest.mark.parametrize("H,pair_begin,npairs", [(8, 0, 44), (5, 4, 20), (3, 0, 64)])
@pytest.mark.parametrize("layout", ["ring", "time", "empty_plain"])
def test_lag_matches_page_axis_oracle(H, pair_begin, npairs, layout):
    """A cache whose sink and history are past the knee and whose window and
    chunk are not.  ring: [sink | window + chunk | history], the plain range in
    the middle; time: [sink | history | window + chunk], the plain range at the
    end (plain_end past the count); empty_plain: every row past the knee.
    Segment lengths are not multiples of the 64-key tile."""
    dev = device()
    rng = np.random.default_rng(H * 100 + npairs + len(layout))
    D, tpf, c, knee = 128, 16, 8.0, 12.0
    n_sink, n_win, n_hist, n_q = 70, 130 if layout != "empty_plain" else 0, 333, 150
    q0 = 240.0
    # frames: sink 0..4, history spread over 5..227 (past the knee), window and
    # chunk within the knee of q0 (228..243)
    t_sink = np.arange(n_sink) // tpf
    t_hist = 5 + (np.arange(n_hist) * (q0 - knee - 5)) // n_hist
    t_win = q0 - knee + (np.arange(n_win) * 16) // max(n_win, 1)
    if layout == "ring":
        t_rows = np.concatenate([t_sink, t_win, t_hist])
        plain = (n_sink, n_sink + n_win)
    else:
        t_rows = np.concatenate([t_sink, t_hist, t_win])
        plain = (n_sink + n_hist, 10 ** 6) if layout == "time" else (37, 37)
    n = t_rows.shape[0]
    frame_t = np.arange(int(q0) + 4, dtype=np.float64)
    rf = t_rows.astype(np.int32)
    assert np.all((q0 - frame_t[rf] > knee) == ((np.arange(n) < plain[0]) | (np.arange(n) >= plain[1])))
    q = random_bf16_bits(rng, (n_q, H, D))
    k = random_bf16_bits(rng, (n + 9, H, D))
    v = random_bf16_bits(rng, (n + 9, H, D))
    theta = dpsynth.rope_theta(npairs)
    kd = bf16_from_bits(k, dev)
    rf_d = to_dev(np.concatenate([rf, np.full(9, -1, np.int32)]), dev)
    _compress([kd], H, D, n, [(0, n)], rf_d, to_dev(theta, dev), frame_t, q0, knee, c,
              pair_begin, dev)
    lag = (1.0 - 1.0 / c) * (q0 - knee)
    od = torch.zeros((n_q, H, D), dtype=torch.bfloat16, device=dev)
    cnt = torch.tensor([n], dtype=torch.int64, device=dev)
    dp.dp_attention_lag(bf16_from_bits(q, dev), kd, bf16_from_bits(v, dev), od, n_q, n + 9, cnt,
                        plain[0], plain[1], to_dev(theta, dev), pair_begin, npairs, lag, H, D,
                        dp.DP_BF16, 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    want = _page_reference(q, k, v, rf, frame_t, q0, knee, c, pair_begin, theta,
                           np.arange(n_q), n_kv=n)
    err = _check(bits(od), want, (layout, H, npairs))
    print("lag attention %s H=%d pairs=%d: max |err| %.2e" % (layout, H, npairs, err))


def test_lag_zero_rows_gives_zeros():
    dev = device()
    H, D, n_q = 8, 128, 40
    q = torch.ones((n_q, H, D), dtype=torch.bfloat16, device=dev)
    k = torch.ones((64, H, D), dtype=torch.bfloat16, device=dev)
    od = torch.full((n_q, H, D), 3.0, dtype=torch.bfloat16, device=dev)
    zero = torch.zeros(1, dtype=torch.int64, device=dev)
    theta = to_dev(dpsynth.rope_theta(8), dev)
    dp.dp_attention_lag(q, k, k, od, n_q, 64, zero, 10, 20, theta, 0, 8, 5.0, H, D, dp.DP_BF16, 0.1)
    torch.cuda.synchronize()
    assert np.all(bits(od) == 0)


# ring-layout rollout on the compressed axis: 2 frames per chunk, a window of
# 2 chunks whose span equals the knee, so the chunk that leaves the window is
# the only one that crosses the knee; the append re-indexes it on the way and
# no other key is ever rewritten
H_R, D_R, TPF, F, W = 3, 128, 16, 2, 2
C = TPF * F
R = W + 1
STEPS = 6
NPAIRS = 12
KNEE = float(W * F)
FACTOR = 4.0


def test_lag_ring_rollout_matches_page_axis_oracle():
    dev = device()
    rng = np.random.default_rng(12)
    L = 2
    n_frames = (R + 2 + STEPS) * F
    theta = dpsynth.rope_theta(NPAIRS)
    frame_t = np.arange(n_frames, dtype=np.float32)
    cap = C + R * C + STEPS * C
    hist = C + R * C
    orig = np.zeros((L, cap, H_R, D_R), np.uint16)          # keys as written (phase t)
    vb = np.zeros((L, cap, H_R, D_R), np.uint16)
    orig[:, :hist] = random_bf16_bits(rng, (L, hist, H_R, D_R), 2.0)
    vb[:, :hist] = random_bf16_bits(rng, (L, hist, H_R, D_R))
    rf = np.full(cap, -1, np.int32)
    rf[:hist] = np.arange(hist) // TPF
    k = [bf16_from_bits(orig[l], dev) for l in range(L)]
    v = [bf16_from_bits(vb[l], dev) for l in range(L)]
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv = dp.dp_kv_inplace()
    ak, av = dp.ptr_array(k, dev), dp.ptr_array(v, dev)
    kv.k_layers, kv.v_layers = ak.data_ptr(), av.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H_R, D_R, dp.DP_BF16
    kv.capacity, kv.dev_error = cap, err.data_ptr()
    rf_d, th_d, ft_d = to_dev(rf, dev), to_dev(theta, dev), to_dev(frame_t, dev)
    tail = torch.tensor([hist], dtype=torch.int64, device=dev)
    phase = to_dev(frame_t.copy(), dev)
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, NPAIRS) // 4 + 4, dtype=torch.float32,
                     device=dev)
    orf, otail = rf.copy(), hist
    ok_, ophase = orig.copy(), frame_t.copy()            # the keys as the device should hold them
    n_q = 70
    for s in range(STEPS):
        slot = s % R
        sb = C + slot * C
        q0 = float((R + 1 + s) * F)
        keep = (rng.random(C) < 0.3).astype(np.uint8)
        idx = torch.empty(C, dtype=torch.int32, device=dev)
        nk = torch.zeros(1, dtype=torch.int64, device=dev)
        wsc = torch.empty(dp.dp_compact_workspace_bytes(C) // 4 + 1, dtype=torch.int32, device=dev)
        dp.dp_compact_index(to_dev(keep, dev), C, idx, nk, None, None, wsc)
        rope = dp.make_rope(th_d, ft_d, phase, q0, KNEE, 1.0 / FACTOR, axis=dp.DP_AXIS_COMPRESSED)
        dp.dp_rope_prepare(rope, D_R, dp.DP_BF16, ws)
        if s == 0:                                   # the sink crosses the knee once
            dp.dp_rope_apply(ak, L, H_R, D_R, dp.DP_BF16, 0, C, None, rf_d, rope, ws)
        dp.dp_append_kept(kv, sb, C, idx, nk, tail, rf_d, rope, ws)
        k_new = random_bf16_bits(rng, (L, C, H_R, D_R), 2.0)
        v_new = random_bf16_bits(rng, (L, C, H_R, D_R))
        new_frames = ((R + 1 + s) * F + np.arange(C) // TPF).astype(np.int32)
        for l in range(L):                           # the model writes the next chunk
            k[l][sb:sb + C] = bf16_from_bits(k_new[l], dev)
            v[l][sb:sb + C] = bf16_from_bits(v_new[l], dev)
        rf_d[sb:sb + C] = torch.from_numpy(new_frames).to(dev)
        # host twins: the keys as written (for the page-axis reference) and the
        # keys re-indexed on the compressed axis by the oracle (bit for bit)
        widx = oracle.compact(keep)
        tables = oracle.rope_frames(frame_t, ophase, q0, KNEE, np.float32(1.0 / FACTOR), theta,
                                    compressed=True)
        ophase = tables[3]
        t_before = otail
        orf_twin = orf.copy()
        otail = oracle.append_kept(orig, sb, C, widx, otail, orf)
        oracle.append_kept(ok_, sb, C, widx, t_before, orf_twin)
        oracle.append_kept(vb, sb, C, widx, t_before, None)
        for l in range(L):
            for lo, hi in (((0, C), (t_before, otail)) if s == 0 else ((t_before, otail),)):
                sub = np.ascontiguousarray(ok_[l][lo:hi])
                oracle.rope_rows(sub, orf[lo:hi], 0, tables)
                ok_[l][lo:hi] = sub
        orig[:, sb:sb + C] = k_new
        ok_[:, sb:sb + C] = k_new
        vb[:, sb:sb + C] = v_new
        orf[sb:sb + C] = new_frames
        torch.cuda.synchronize()
        assert err.item() == 0 and tail.item() == otail, s
        assert np.array_equal(phase.cpu().numpy(), ophase), s
        for l in range(L):
            assert np.array_equal(bits(k[l]), ok_[l]), (s, l)
            assert np.array_equal(bits(v[l]), vb[l]), (s, l)
        # every visible key past the knee is on the compressed axis, the rest at t
        d = q0 - frame_t[orf[:otail]]
        assert np.all((d > KNEE) == ((np.arange(otail) < C) | (np.arange(otail) >= hist))), s
        q = random_bf16_bits(rng, (n_q, H_R, D_R))
        lag = (1.0 - 1.0 / FACTOR) * (q0 - KNEE)
        for l in range(L):
            od = torch.zeros((n_q, H_R, D_R), dtype=torch.bfloat16, device=dev)
            dp.dp_attention_lag(bf16_from_bits(q, dev), k[l], v[l], od, n_q, cap, tail, C, hist,
                                th_d, 0, NPAIRS, lag, H_R, D_R, dp.DP_BF16, 1.0 / np.sqrt(D_R))
            torch.cuda.synchronize()
            want = _page_reference(q, orig[l], vb[l], orf, frame_t, q0, KNEE, FACTOR, 0, theta,
                                   np.arange(n_q), n_kv=otail)
            _check(bits(od), want, (s, l))
    print("lag ring rollout: %d steps, tail %d" % (STEPS, otail))


def test_lag_one_minute_ring_shape_sampled():
    """The launch the attention_lag benchmark times: 6,240 queries over the
    83,412-row one-minute cache in the ring layout (sink | window chunks and
    the chunk | retained history), 40 heads x 128, 44 temporal pairs, the old
    keys re-indexed to the compressed axis first; seven queries of three heads
    are checked against the page-axis oracle over all 83,412 keys."""
    dev = device()
    w = dpsynth.WORKLOADS["reindex"]
    H, D, C = w.n_heads, w.head_dim, w.chunk_tokens
    rf, plain_begin, plain_end = dpsynth.ring_layout(w)
    n = rf.shape[0]
    seed = 4
    q = torch.empty((C, H, D), dtype=torch.bfloat16, device=dev)
    k = torch.empty((n, H, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty((n, H, D), dtype=torch.bfloat16, device=dev)
    dpsynth.kv_fill_device(q, "bf16", seed, 3, 0, C, H * D)
    dpsynth.kv_fill_device(k, "bf16", seed, dpsynth.STREAM_K, 0, n, H * D)
    dpsynth.kv_fill_device(v, "bf16", seed, dpsynth.STREAM_V, 0, n, H * D)
    rows = np.array([0, 1, 127, 128, 3000, 6111, 6239])
    heads = np.array([0, 17, 39])
    cols = (heads[:, None] * D + np.arange(D)[None, :]).ravel()
    hd = len(heads)
    # the generator's fill of the checked heads, read back before anything runs
    # on it (the host twin of the whole columns is too slow to draw here), and
    # tied to the host twin on sampled rows
    hd_idx = torch.from_numpy(heads).to(dev)
    kh = bits(k.index_select(1, hd_idx))
    vh = bits(v.index_select(1, hd_idx))
    probe = np.array([0, 1, 6239, 6240, 31199, 31200, n // 2, n - 1])
    for t_, stream in ((kh, dpsynth.STREAM_K), (vh, dpsynth.STREAM_V)):
        host = dpsynth.kv_rows_host("bf16", seed, stream, 0, probe, n, H * D, cols)
        assert np.array_equal(t_[probe].reshape(len(probe), -1), host)
    theta = dpsynth.rope_theta(w.rope_pairs, w.rope_base)
    frame_t = np.arange(w.n_frames + w.frames_per_chunk, dtype=np.float64)
    c, knee, q0 = w.rope_factor, w.rope_knee, w.q0
    _compress([k], H, D, n, [(0, n)], to_dev(rf, dev), to_dev(theta, dev), frame_t, q0, knee, c,
              0, dev)
    lag = (1.0 - 1.0 / c) * (q0 - knee)
    o = torch.empty_like(q)
    dp.dp_attention_lag(q, k, v, o, C, n, None, plain_begin, plain_end, to_dev(theta, dev), 0,
                        w.rope_pairs, lag, H, D, dp.DP_BF16, 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    qh = np.zeros((C, hd, D), np.uint16)
    qh[rows] = dpsynth.kv_rows_host("bf16", seed, 3, 0, rows, C, H * D, cols).reshape(-1, hd, D)
    want = _page_reference(qh, kh, vh, rf, frame_t, q0, knee, c, 0, theta, rows)
    got = bits(o[torch.from_numpy(rows).to(dev)])[:, heads]
    err = _check(got, want, "one-minute ring shape")
    print("one-minute ring lag attention: %d rows, max |err| %.2e over %d queries x %d heads"
          % (n, err, len(rows), hd))


def _ragged_layout(rng, H, n_sink, n_win, hist_lens, q0, knee, tpf):
    """Per-head runs [sink | retained history | window] in time order, the
    frame of every ragged row, and the head offsets."""
    frames, off = [], [0]
    for h in range(H):
        t_sink = np.arange(n_sink) // tpf
        n_hist = hist_lens[h]
        t_hist = np.sort(rng.integers(n_sink // tpf + 1, int(q0 - knee), n_hist)) if n_hist else \
            np.zeros(0, np.int64)
        t_win = q0 - knee + (np.arange(n_win) * 16) // max(n_win, 1)
        fr = np.concatenate([t_sink, t_hist, t_win]).astype(np.int32)
        frames.append(fr)
        off.append(off[-1] + fr.shape[0])
    return np.concatenate(frames), np.asarray(off, np.int64)


@pytest.mark.parametrize("H,n_chunk,tail_mode", [(8, 70, "window"), (5, 0, "window"),
                                                 (3, 33, "zero"), (8, 0, "longer")])
def test_hs_lag_matches_page_axis_oracle(H, n_chunk, tail_mode):
    """DeCoPrune-HS runs of unequal length (static heads: sink + window; dynamic
    heads: sink + retained history + window), keys past the knee moved to the
    compressed axis, then dp_hs_attention_lag with the window as each run's
    plain tail, against the page-axis oracle per head.  tail_mode: the window
    length; zero (every row, the window's too, given frames past the knee);
    longer than every run (every row within the knee)."""
    dev = device()
    rng = np.random.default_rng(H * 10 + n_chunk + len(tail_mode))
    D, tpf, c, knee, q0, n_q = 128, 16, 8.0, 12.0, 240.0, 140
    n_sink, n_win = 50, 90
    hist_lens = [0 if h % 2 == 0 or tail_mode == "longer" else int(rng.integers(60, 260))
                 for h in range(H)]
    frames, off = _ragged_layout(rng, H, n_sink, n_win, hist_lens, q0, knee, tpf)
    if tail_mode == "zero":                      # every row past the knee: no plain tail
        frames = np.minimum(frames, int(q0 - knee) - 1).astype(np.int32)
    tail = {"window": n_win, "zero": 0, "longer": n_sink + n_win + 100}[tail_mode]
    if tail_mode == "longer":                    # a tail longer than every run: all plain
        frames = np.maximum(frames, int(q0 - knee)).astype(np.int32)
    total = int(off[-1])
    frame_t = np.arange(int(q0) + 4, dtype=np.float64)
    kr = random_bf16_bits(rng, (total + 7, D))
    vr = random_bf16_bits(rng, (total + 7, D))
    q = random_bf16_bits(rng, (n_q, H, D))
    kc = random_bf16_bits(rng, (max(n_chunk, 1), H, D))
    vc = random_bf16_bits(rng, (max(n_chunk, 1), H, D))
    theta = dpsynth.rope_theta(44)
    krd = bf16_from_bits(kr, dev)
    rf_d = to_dev(np.concatenate([frames, np.full(7, -1, np.int32)]), dev)
    # the packed cache as one [rows, 1 head, D] layer for the re-index
    _compress([krd.view(total + 7, 1, D)], 1, D, total, [(0, total)], rf_d, to_dev(theta, dev),
              frame_t, q0, knee, c, 0, dev)
    lag = (1.0 - 1.0 / c) * (q0 - knee)
    od = torch.zeros((n_q, H, D), dtype=torch.bfloat16, device=dev)
    kcd = bf16_from_bits(kc, dev) if n_chunk else None
    vcd = bf16_from_bits(vc, dev) if n_chunk else None
    dp.dp_hs_attention_lag(bf16_from_bits(q, dev), krd, bf16_from_bits(vr, dev), total,
                           to_dev(off, dev), 0, kcd, vcd, n_chunk, od, n_q, H, D, dp.DP_BF16,
                           1.0 / np.sqrt(D), tail, to_dev(theta, dev), 0, 44, lag)
    torch.cuda.synchronize()
    # the lagged rows must be exactly those past the knee
    past = q0 - frame_t[frames] > knee
    for h in range(H):
        lo, hi = int(off[h]), int(off[h + 1])
        t = min(tail, hi - lo)
        assert np.all(past[lo:hi - t]) and not np.any(past[hi - t:hi]), h
    want = np.zeros((n_q, H, D))
    for h in range(H):
        lo, hi = int(off[h]), int(off[h + 1])
        kh = kr[lo:hi][:, None]
        vh = vr[lo:hi][:, None]
        fh = frames[lo:hi]
        if n_chunk:                               # chunk rows: frames within the knee
            kh = np.concatenate([kh, kc[:n_chunk, h:h + 1]])
            vh = np.concatenate([vh, vc[:n_chunk, h:h + 1]])
            fh = np.concatenate([fh, np.full(n_chunk, int(q0), np.int32)])
        want[:, h] = _page_reference(np.ascontiguousarray(q[:, h:h + 1]), np.ascontiguousarray(kh),
                                     np.ascontiguousarray(vh), fh, frame_t, q0, knee, c, 0,
                                     theta, np.arange(n_q))[:, 0]
    err = _check(bits(od), want, ("hs lag", H, n_chunk, tail_mode))
    print("hs lag attention H=%d chunk=%d tail=%s: max |err| %.2e" % (H, n_chunk, tail_mode, err))


def test_hs_lag_reduces_to_hs_attention():
    """A plain tail as long as every run, or no plain tail and a zero lag:
    the same tiles in the same order as dp_hs_attention, bit for bit (a tail
    that splits a run changes the tile boundaries, hence the summation order)."""
    dev = device()
    rng = np.random.default_rng(77)
    H, D, n_q, n_chunk = 8, 128, 130, 40
    lens = np.array([0, 1, 63, 64, 65, 200, 7, 129], np.int64)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    total = int(off[-1])
    kr = bf16_from_bits(random_bf16_bits(rng, (total, D)), dev)
    vr = bf16_from_bits(random_bf16_bits(rng, (total, D)), dev)
    q = bf16_from_bits(random_bf16_bits(rng, (n_q, H, D)), dev)
    kc = bf16_from_bits(random_bf16_bits(rng, (n_chunk, H, D)), dev)
    vc = bf16_from_bits(random_bf16_bits(rng, (n_chunk, H, D)), dev)
    offd, theta = to_dev(off, dev), to_dev(dpsynth.rope_theta(44), dev)
    ref = torch.zeros((n_q, H, D), dtype=torch.bfloat16, device=dev)
    dp.dp_hs_attention(q, kr, vr, total, offd, 0, kc, vc, n_chunk, ref, n_q, H, D, dp.DP_BF16, 0.09)
    for tail, lag in ((1000, 123.5), (200, -7.0), (0, 0.0)):
        od = torch.full((n_q, H, D), 5.0, dtype=torch.bfloat16, device=dev)
        dp.dp_hs_attention_lag(q, kr, vr, total, offd, 0, kc, vc, n_chunk, od, n_q, H, D,
                               dp.DP_BF16, 0.09, tail, theta, 0, 44, lag)
        torch.cuda.synchronize()
        assert np.array_equal(bits(od), bits(ref)), (tail, lag)
