"""Tile coverage of the attention kernels at the benchmark's full shapes.

The kernels stream a head's keys as passes over contiguous row ranges in tiles
of 64 rows (dense cache: one range; compressed-axis ring layout: the lagged
rows before the plain range, those after it, then the plain range; ragged HS
cache: the head's run, split into its lagged part and plain tail, then the
chunk's own block).  These cases make every tile of every pass visible in the
output: keys are zero except one spike row per tile (dim 127 = 48, outside the
temporal pairs, so the lagged query's rotation does not touch it), every
query has dim 127 = 1, and values are zero except 32 in one tile-specific
column of the spike row.  All scores are then 0 or 48 / sqrt(128) whatever the
query, every query has the same output, and output column c is
32 n_c / l with n_c the spike tiles mapped to c (about ten) and l the softmax
sum.  A tile skipped, read twice, taken from another head or paired with the
wrong value row changes a column by about a tenth or more.

Bound: the derived bound of the attention kernels (gpu_helpers.attention_bound;
here A = |o| since every value is >= 0), about 1 % of |o|, far below a tile's
share.  Every query of every head is compared with the float64 oracle, which
is evaluated on sampled queries (its output does not depend on the query
here, which the samples confirm).
"""
import numpy as np
import torch

import compaction_dp_score_amd as dp
import dpsynth
import oracle
from gpu_helpers import attention_bound, bf16_norms, bits, device, random_bf16_bits

import pytest

pytestmark = pytest.mark.gpu

D = 128
SPIKE_K = 0x4240      # bf16 48.0
SPIKE_V = 0x4200      # bf16 32.0
ONE = 0x3F80          # bf16 1.0


def _spikes(passes, H, tile_base=0):
    """Spike rows of each head: one per 64-row tile of every pass (a pass is
    (first row, rows)); returns per head a list of (row, column)."""
    out = []
    for h in range(H):
        spikes, t_all = [], tile_base
        for pi, (r0, n) in enumerate(passes):
            for t in range((n + 63) // 64):
                rows_here = min(64, n - 64 * t)
                pos = (37 * t + 11 * h + 5 * pi) % rows_here
                spikes.append((r0 + 64 * t + pos, (t_all + 7 * h) % D))
                t_all += 1
        out.append(spikes)
    return out


KMAX = 48.0                    # the spike key's norm


def _bound(want, n_kv, q):
    qmax = float(bf16_norms(q).max())
    return attention_bound(want, np.abs(want), qmax, KMAX, 1.0 / np.sqrt(D), n_kv)


def _bound_check(got_bits, want, n_kv, q, tag):
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(got - want)
    bound = _bound(want, n_kv, q)
    assert np.all(err <= bound), (tag, float((err - bound).max()), float(err.max()))
    return float(err.max())


def _queries(rng, n_q, H):
    q = random_bf16_bits(rng, (n_q, H, D))
    q[..., 127] = ONE
    return q


def _dense_case(n, H, spikes_by_head):
    k = np.zeros((n, H, D), np.uint16)
    v = np.zeros((n, H, D), np.uint16)
    for h, spikes in enumerate(spikes_by_head):
        rows = np.array([r for r, _ in spikes])
        cols = np.array([c for _, c in spikes])
        k[rows, h, 127] = SPIKE_K
        v[rows, h, cols] = SPIKE_V
    return k, v


def _expected(q, k, v, H, sample):
    want = oracle.attention(q, k, v, sample)
    assert np.all(want == want[:1]), "query-independent by construction"
    return want[0]


def test_dense_attention_every_tile_at_the_one_minute_shape():
    """6,240 queries over the 83,412-row compacted one-minute cache (1,303
    full tiles and a last tile of 20 rows), 40 heads: every query of every
    head."""
    dev = device()
    w = dpsynth.WORKLOADS["reindex"]
    H, C = w.n_heads, w.chunk_tokens
    n = int(dpsynth.retained_keep(w).sum()) + C
    assert n % 64 != 0
    rng = np.random.default_rng(71)
    k, v = _dense_case(n, H, _spikes([(0, n)], H))
    q = _queries(rng, C, H)
    qd = torch.from_numpy(q.view(np.int16)).to(dev).view(torch.bfloat16)
    kd = torch.from_numpy(k.view(np.int16)).to(dev).view(torch.bfloat16)
    vd = torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)
    o = torch.empty_like(qd)
    dp.dp_attention(qd, kd, vd, o, C, n, None, H, D, dp.DP_BF16, 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    want = _expected(q, k, v, H, np.array([0, 2979, C - 1]))
    err = _bound_check(bits(o), np.broadcast_to(want, (C, H, D)), n, q, "dense")
    print("dense tiles: %d keys, %d tiles per head, max |err| %.2e" % (n, (n + 63) // 64, err))


def test_lagged_attention_every_tile_of_every_range():
    """The compressed-axis ring layout of the one-minute cache: rows before
    the plain range and after it are lagged, the plain range (window and the
    chunk) is not; each range is its own pass with its own last partial tile.
    Every query of every head.  (The plain range, window and chunk, is 390
    whole tiles; the two lagged ranges end in partial tiles.)"""
    dev = device()
    w = dpsynth.WORKLOADS["reindex"]
    H, C = w.n_heads, w.chunk_tokens
    rf, pa, pb = dpsynth.ring_layout(w)
    n = rf.shape[0]
    passes = [(0, pa), (pb, n - pb), (pa, pb - pa)]
    assert pa % 64 != 0 and (n - pb) % 64 != 0
    rng = np.random.default_rng(72)
    k, v = _dense_case(n, H, _spikes(passes, H))
    q = _queries(rng, C, H)
    qd = torch.from_numpy(q.view(np.int16)).to(dev).view(torch.bfloat16)
    kd = torch.from_numpy(k.view(np.int16)).to(dev).view(torch.bfloat16)
    vd = torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)
    theta = torch.from_numpy(dpsynth.rope_theta(w.rope_pairs, w.rope_base)).to(dev)
    o = torch.empty_like(qd)
    lag = (1.0 - 1.0 / w.rope_factor) * (w.q0 - w.rope_knee)
    dp.dp_attention_lag(qd, kd, vd, o, C, n, None, pa, pb, theta, 0, w.rope_pairs, lag, H, D,
                        dp.DP_BF16, 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    # the lag turns the query's temporal pairs only; keys are zero there, so
    # the scores, and the oracle, are those of plain attention
    want = _expected(q, k, v, H, np.array([0, 4001, C - 1]))
    err = _bound_check(bits(o), np.broadcast_to(want, (C, H, D)), n, q, "lag")
    print("lagged tiles: ranges %s, max |err| %.2e" % ([m for _, m in passes], err))


@pytest.mark.parametrize("lagged", [False, True])
def test_hs_attention_every_tile_of_every_run(lagged):
    """The ragged DeCoPrune-HS cache at the HS workload's shape (one layer, 40
    heads: static runs of 24,960 rows, dynamic runs of the gamma mask's
    length), followed by the chunk's 6,240 rows; with the lag, each run's last
    18,720 rows (the window) are a plain pass of their own.  Every query of
    every head."""
    dev = device()
    w = dpsynth.WORKLOADS["hs"]
    T, H, C = w.seq_len, w.n_heads, w.chunk_tokens
    x0, xf = dpsynth.score_inputs(w)
    ell = oracle.score_f32(x0, xf, w.d)
    n_s = int(oracle.mask(None, T, w.sink_len, w.window_len, w.scored_begin, w.n_scored,
                          w.gamma, streaming=True).sum())
    n_d = int(oracle.mask(ell, T, w.sink_len, w.window_len, w.scored_begin, w.n_scored,
                          w.gamma).sum())
    cls = dpsynth.hs_head_class(w)[:1]
    off = oracle.hs_offsets(cls, np.array([n_s, n_d], np.int64))
    total = int(off[-1])
    tail = w.window_len if lagged else 0
    rng = np.random.default_rng(73 + lagged)
    kr = np.zeros((total, D), np.uint16)
    vr = np.zeros((total, D), np.uint16)
    kc = np.zeros((C, H, D), np.uint16)
    vc = np.zeros((C, H, D), np.uint16)
    n_tiles = []
    for h in range(H):
        lo, hi = int(off[h]), int(off[h + 1])
        n0 = hi - lo
        passes = [(0, n0 - tail), (n0 - tail, tail)] if tail else [(0, n0)]
        run = _spikes(passes, H)[h]
        rows = np.array([r for r, _ in run]) + lo
        cols = np.array([c for _, c in run])
        kr[rows, 127] = SPIKE_K
        vr[rows, cols] = SPIKE_V
        chunk = _spikes([(0, C)], H, tile_base=len(run))[h]
        crow = np.array([r for r, _ in chunk])
        ccol = np.array([c for _, c in chunk])
        kc[crow, h, 127] = SPIKE_K
        vc[crow, h, ccol] = SPIKE_V
        n_tiles.append(len(run) + len(chunk))
    q = _queries(rng, C, H)
    to = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    qd = to(q)
    o = torch.empty_like(qd)
    offd = torch.from_numpy(off).to(dev)
    scale = 1.0 / np.sqrt(D)
    if lagged:
        theta = torch.from_numpy(dpsynth.rope_theta(w.rope_pairs, w.rope_base)).to(dev)
        lag = (1.0 - 1.0 / w.rope_factor) * (w.q0 - w.rope_knee)
        dp.dp_hs_attention_lag(qd, to(kr), to(vr), total, offd, 0, to(kc), to(vc), C, o, C, H, D,
                               dp.DP_BF16, scale, tail, theta, 0, w.rope_pairs, lag)
    else:
        dp.dp_hs_attention(qd, to(kr), to(vr), total, offd, 0, to(kc), to(vc), C, o, C, H, D,
                           dp.DP_BF16, scale)
    torch.cuda.synchronize()
    sample = np.array([0, 3333, C - 1])
    want = oracle.hs_attention(q, kr, vr, off, 0, sample, kc, vc, scale=scale)
    assert np.all(want == want[:1])
    err = _bound_check(bits(o), np.broadcast_to(want[0], (C, H, D)), max(n_s, n_d) + C, q,
                       ("hs", lagged))
    print("hs tiles (lag %s): runs %d / %d rows, %d-%d tiles per head, max |err| %.2e"
          % (lagged, n_s, n_d, min(n_tiles), max(n_tiles), err))


def test_a_skipped_tile_would_fail_the_bound():
    """The bound above is far below one tile's share: dropping any one spike
    from the oracle's inputs moves some output column beyond it (checked on
    the dense one-minute case for a sample of tiles, the last partial one
    included)."""
    w = dpsynth.WORKLOADS["reindex"]
    H, C = 4, w.chunk_tokens
    n = int(dpsynth.retained_keep(w).sum()) + C
    rng = np.random.default_rng(74)
    spikes = _spikes([(0, n)], H)
    k, v = _dense_case(n, H, spikes)
    q = _queries(rng, 2, H)
    full = oracle.attention(q, k, v, [0])[0]
    bound = _bound(full, n, q)
    for t in (0, 1, 700, len(spikes[0]) - 1):
        for h in (0, H - 1):
            r, c = spikes[h][t]
            k2, v2 = k.copy(), v.copy()
            k2[r, h, 127] = 0
            v2[r, h, c] = 0
            drop = oracle.attention(q, k2, v2, [0])[0]
            assert np.any(np.abs(drop - full) > 4 * bound), (t, h)
