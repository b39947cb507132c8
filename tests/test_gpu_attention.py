"""GPU parity of dp_attention (a chunk's queries over the compacted cache)
against the float64 oracle.

Bound: gpu_helpers.attention_bound, derived from the kernel's roundings (bf16
probabilities into P.V, bf16 output, fp32 scores, sums and exp2):
|o - o_ref| <= (2^-8 + delta_scores + gamma_n) (A + |o_ref|) + 1e-6, with
A = sum_j p_j |v_j| / l the oracle's attention over |V|.  Every query of
every head is compared at the small sizes, and every query of one head at
the one-minute shape; the full-shape tile-coverage tests make a dropped or
doubled 64-key tile visible far above this bound.
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import dpsynth
import oracle
from gpu_helpers import (bf16_abs, bf16_from_bits, bf16_norms, bits, check_attention, device,
                         random_bf16_bits)

pytestmark = pytest.mark.gpu


def _check(got_bits, q, k, v, rows, n_kv, scale, tag):
    """Kernel output for query `rows` against the oracle under the derived
    bound; k, v: [rows >= n_kv, H, D] bit patterns (rows past n_kv unread)."""
    rows = np.asarray(rows)
    want = oracle.attention(q, k, v, rows, n_kv=n_kv, scale=scale)
    want_abs = oracle.attention(q, k, bf16_abs(v), rows, n_kv=n_kv, scale=scale)
    kmax = bf16_norms(k[:n_kv]).max(axis=0)                   # per head
    err, ratio = check_attention(got_bits, want, want_abs, bf16_norms(q[rows]), kmax, scale,
                                 n_kv, tag)
    return err, ratio


@pytest.mark.parametrize("n_q,n_kv,H", [(1, 1, 8), (100, 63, 8), (128, 64, 8), (300, 65, 3),
                                        (257, 1000, 8), (129, 777, 5)])
@pytest.mark.parametrize("device_count", [False, True])
def test_attention_matches_oracle(n_q, n_kv, H, device_count):
    dev = device()
    rng = np.random.default_rng(n_q * 7 + n_kv + H)
    D = 128
    q = random_bf16_bits(rng, (n_q, H, D))
    extra = 37                                        # rows beyond the count are never read
    k = random_bf16_bits(rng, (n_kv + extra, H, D))
    v = random_bf16_bits(rng, (n_kv + extra, H, D))
    k[n_kv:] = 0x7FC0                                 # NaN beyond the count
    v[n_kv:] = 0x7FC0
    qd, kd, vd = bf16_from_bits(q, dev), bf16_from_bits(k, dev), bf16_from_bits(v, dev)
    od = torch.zeros((n_q, H, D), dtype=torch.bfloat16, device=dev)
    scale = 1.0 / np.sqrt(D)
    if device_count:
        dp.dp_attention(qd, kd, vd, od, n_q, n_kv + extra,
                        torch.tensor([n_kv], dtype=torch.int64, device=dev), H, D, dp.DP_BF16, scale)
    else:
        dp.dp_attention(qd, kd, vd, od, n_q, n_kv, None, H, D, dp.DP_BF16, scale)
    torch.cuda.synchronize()
    err, ratio = _check(bits(od), q, k, v, np.arange(n_q), n_kv, scale, (n_q, n_kv, H))
    print("attention %dx%d H=%d: max |err| %.2e, %.2f of the bound" % (n_q, n_kv, H, err, ratio))


def test_attention_peaked_and_zero_keys():
    dev = device()
    rng = np.random.default_rng(99)
    n_q, n_kv, H, D = 64, 200, 8, 128
    k = random_bf16_bits(rng, (n_kv, H, D))
    v = random_bf16_bits(rng, (n_kv, H, D), 2.0)
    q = k[:n_q].copy()                                # each query aligned with one key
    qd, kd, vd = bf16_from_bits(q, dev), bf16_from_bits(k, dev), bf16_from_bits(v, dev)
    od = torch.zeros((n_q, H, D), dtype=torch.bfloat16, device=dev)
    dp.dp_attention(qd, kd, vd, od, n_q, n_kv, None, H, D, dp.DP_BF16, 2.0)
    torch.cuda.synchronize()
    _check(bits(od), q, k, v, np.arange(n_q), n_kv, 2.0, "peaked")
    zero = torch.zeros(1, dtype=torch.int64, device=dev)
    od.fill_(1.0)
    dp.dp_attention(qd, kd, vd, od, n_q, n_kv, zero, H, D, dp.DP_BF16, 2.0)
    torch.cuda.synchronize()
    assert np.all(bits(od) == 0)


def test_attention_eviction_shape_sampled():
    """Queries of one 6,240-token chunk over the 32,147 rows the eviction step
    leaves visible (25,907 retained + the chunk itself), 40 heads x 128."""
    dev = device()
    w = dpsynth.WORKLOADS["eviction"]
    H, D = w.n_heads, w.head_dim
    n_q, n_kv = w.chunk_tokens, 25907 + w.chunk_tokens
    q = torch.empty((n_q, H, D), dtype=torch.bfloat16, device=dev)
    k = torch.empty((n_kv, H, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty((n_kv, H, D), dtype=torch.bfloat16, device=dev)
    dpsynth.kv_fill_device(q, "bf16", 1, 3, 0, n_q, H * D)
    dpsynth.kv_fill_device(k, "bf16", 1, dpsynth.STREAM_K, 0, n_kv, H * D)
    dpsynth.kv_fill_device(v, "bf16", 1, dpsynth.STREAM_V, 0, n_kv, H * D)
    o = torch.empty_like(q)
    dp.dp_attention(q, k, v, o, n_q, n_kv, None, H, D, dp.DP_BF16, 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 3000, 6111, 6239])
    qh = dpsynth.kv_rows_host("bf16", 1, 3, 0, rows, n_q, H * D).reshape(len(rows), H, D)
    kh = dpsynth.kv_layer_host("bf16", 1, dpsynth.STREAM_K, 0, n_kv, H * D).reshape(n_kv, H, D)
    vh = dpsynth.kv_layer_host("bf16", 1, dpsynth.STREAM_V, 0, n_kv, H * D).reshape(n_kv, H, D)
    qfull = np.zeros((n_q, H, D), np.uint16)
    qfull[rows] = qh
    got = bits(o[torch.from_numpy(rows).to(dev)])
    err, ratio = _check(got, qfull, kh, vh, rows, n_kv, 1.0 / np.sqrt(D), "eviction shape")
    print("eviction-shape attention: max |err| %.2e (%.2f of the bound) over %d sampled "
          "queries x %d heads" % (err, ratio, len(rows), H))


def test_attention_one_minute_shape_sampled():
    """The launch the attention benchmark times: 6,240 queries over the
    83,412 rows a one-minute history leaves after compaction (sink + retained
    history + window + the chunk), 40 heads x 128, the bench's own inputs.
    Seven queries of three heads against the float64 oracle over all keys; the
    checked heads' keys and values are read back from the generator's device
    fill and tied to its host twin on probe rows."""
    dev = device()
    w = dpsynth.WORKLOADS["reindex"]
    H, D, C = w.n_heads, w.head_dim, w.chunk_tokens
    n = int(dpsynth.retained_keep(w).sum()) + C
    q = torch.empty((C, H, D), dtype=torch.bfloat16, device=dev)
    k = torch.empty((n, H, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty((n, H, D), dtype=torch.bfloat16, device=dev)
    dpsynth.kv_fill_device(q, "bf16", w.seed, 3, 0, C, H * D)
    dpsynth.kv_fill_device(k, "bf16", w.seed, dpsynth.STREAM_K, 0, n, H * D)
    dpsynth.kv_fill_device(v, "bf16", w.seed, dpsynth.STREAM_V, 0, n, H * D)
    o = torch.empty_like(q)
    dp.dp_attention(q, k, v, o, C, n, None, H, D, dp.DP_BF16, 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 3000, 6111, 6239])
    heads = np.array([0, 21, 39])
    cols = (heads[:, None] * D + np.arange(D)[None, :]).ravel()
    hd_idx = torch.from_numpy(heads).to(dev)
    kh = bits(k.index_select(1, hd_idx))
    vh = bits(v.index_select(1, hd_idx))
    probe = np.array([0, 1, 255, 256, n // 3, n // 2, n - 2, n - 1])
    for t_, stream in ((kh, dpsynth.STREAM_K), (vh, dpsynth.STREAM_V)):
        host = dpsynth.kv_rows_host("bf16", w.seed, stream, 0, probe, n, H * D, cols)
        assert np.array_equal(t_[probe].reshape(len(probe), -1), host)
    qh = np.zeros((C, len(heads), D), np.uint16)
    qh[rows] = dpsynth.kv_rows_host("bf16", w.seed, 3, 0, rows, C, H * D, cols).reshape(
        len(rows), len(heads), D)
    got = bits(o[torch.from_numpy(rows).to(dev)])[:, heads]
    err, ratio = _check(got, qh, np.ascontiguousarray(kh), np.ascontiguousarray(vh), rows, n,
                        1.0 / np.sqrt(D), "one-minute shape")
    print("one-minute attention: %d keys, max |err| %.2e (%.2f of the bound) over %d queries "
          "x %d heads" % (n, err, ratio, len(rows), len(heads)))


def test_attention_one_minute_shape_every_query_of_one_head():
    """The same launch (6,240 queries over 83,412 compacted rows, 40 heads):
    every query of head 17 against the float64 oracle over all keys."""
    dev = device()
    w = dpsynth.WORKLOADS["reindex"]
    H, D, C = w.n_heads, w.head_dim, w.chunk_tokens
    n = int(dpsynth.retained_keep(w).sum()) + C
    q = torch.empty((C, H, D), dtype=torch.bfloat16, device=dev)
    k = torch.empty((n, H, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty((n, H, D), dtype=torch.bfloat16, device=dev)
    dpsynth.kv_fill_device(q, "bf16", w.seed, 3, 0, C, H * D)
    dpsynth.kv_fill_device(k, "bf16", w.seed, dpsynth.STREAM_K, 0, n, H * D)
    dpsynth.kv_fill_device(v, "bf16", w.seed, dpsynth.STREAM_V, 0, n, H * D)
    o = torch.empty_like(q)
    dp.dp_attention(q, k, v, o, C, n, None, H, D, dp.DP_BF16, 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    h = 17
    cols = h * D + np.arange(D)
    qh, kh, vh = (np.ascontiguousarray(bits(t[:, h:h + 1])) for t in (q, k, v))
    probe = np.array([0, 1, 4095, 4096, n // 2, n - 1])
    for t_, stream, rows_ in ((kh, dpsynth.STREAM_K, n), (vh, dpsynth.STREAM_V, n), (qh, 3, C)):
        pr = probe[probe < rows_]
        host = dpsynth.kv_rows_host("bf16", w.seed, stream, 0, pr, rows_, H * D, cols)
        assert np.array_equal(t_[pr].reshape(len(pr), -1), host)
    got = bits(o[:, h:h + 1])
    err, ratio = _check(got, qh, kh, vh, np.arange(C), n, 1.0 / np.sqrt(D), "one head, all queries")
    print("one-minute attention, head %d: %d queries x %d keys, max |err| %.2e (%.2f of the "
          "bound)" % (h, C, n, err, ratio))


def _check_hs(got_bits, q, kr, vr, off, layer, rows, kc, vc, scale, tag):
    """dp_hs_attention output against oracle.hs_attention under the derived
    bound (run rows [off[layer*H], off[(layer+1)*H]) and the chunk rows)."""
    H = q.shape[1]
    rows = np.asarray(rows)
    want = oracle.hs_attention(q, kr, vr, off, layer, rows, kc, vc, scale=scale)
    want_abs = oracle.hs_attention(q, kr, bf16_abs(vr), off, layer, rows, kc,
                                   None if vc is None else bf16_abs(vc), scale=scale)
    lo, hi = int(off[layer * H]), int(off[(layer + 1) * H])
    keys = [kr[lo:hi]] + ([] if kc is None else [kc.reshape(-1, kc.shape[-1])])
    kmax = max([float(bf16_norms(x).max()) for x in keys if x.shape[0]] + [0.0])
    n_kv = int(np.diff(off[layer * H:(layer + 1) * H + 1]).max()) + (0 if kc is None else kc.shape[0])
    return check_attention(got_bits, want, want_abs, bf16_norms(q[rows]), kmax, scale, n_kv, tag)


def _ragged_case(rng, lens, H, D, pad):
    off = np.concatenate([[0], np.cumsum(np.asarray(lens, np.int64).ravel())]).astype(np.int64)
    kr = random_bf16_bits(rng, (int(off[-1]) + pad, D))
    vr = random_bf16_bits(rng, (int(off[-1]) + pad, D))
    return off, kr, vr


@pytest.mark.parametrize("H", [5, 8])
@pytest.mark.parametrize("n_chunk", [0, 1, 70])
@pytest.mark.parametrize("layer", [0, 1])
def test_hs_attention_matches_oracle(H, n_chunk, layer):
    """Ragged per-head runs of awkward lengths (empty, one row, around a tile),
    optionally followed by the chunk's dense rows; rows beyond the capacity
    hold NaN and are never read."""
    dev = device()
    rng = np.random.default_rng(100 * H + 10 * n_chunk + layer)
    D, n_q = 128, 133
    base = [0, 1, 63, 64, 65, 200, 7, 129]
    lens = np.array([[base[(h + l) % 8] for h in range(H)] for l in range(2)], np.int64)
    pad = 40
    off, kr, vr = _ragged_case(rng, lens, H, D, pad)
    cap = int(off[-1])
    kr[cap:] = 0x7FC0
    vr[cap:] = 0x7FC0
    q = random_bf16_bits(rng, (n_q, H, D))
    kc = random_bf16_bits(rng, (max(n_chunk, 1), H, D))
    vc = random_bf16_bits(rng, (max(n_chunk, 1), H, D))
    od = torch.zeros((n_q, H, D), dtype=torch.bfloat16, device=dev)
    scale = 1.0 / np.sqrt(D)
    kcd = bf16_from_bits(kc, dev) if n_chunk else None
    vcd = bf16_from_bits(vc, dev) if n_chunk else None
    dp.dp_hs_attention(bf16_from_bits(q, dev), bf16_from_bits(kr, dev), bf16_from_bits(vr, dev),
                       cap, torch.from_numpy(off).to(dev), layer, kcd, vcd, n_chunk, od, n_q, H, D,
                       dp.DP_BF16, scale)
    torch.cuda.synchronize()
    err, ratio = _check_hs(bits(od), q, kr, vr, off, layer, np.arange(n_q),
                           kc[:n_chunk] if n_chunk else None, vc[:n_chunk] if n_chunk else None,
                           scale, ("hs", H, n_chunk, layer))
    print("hs attention H=%d chunk=%d layer=%d: max |err| %.2e (%.2f of the bound)"
          % (H, n_chunk, layer, err, ratio))


@pytest.mark.parametrize("H,n_q", [(8, 64), (8, 300), (16, 545), (24, 257), (16, 1100),
                                   (256, 200), (264, 130)])
def test_hs_attention_every_tile_once(H, n_q):
    """With a head count divisible by the 8 XCDs, each head's query tiles are
    cut in two halves dealt by run length; counts of 1, 3, 5 and 9 tiles leave
    the second half one tile short; 256 heads is the most the workgroup ranks,
    264 takes whole heads in head order.  Bimodal run lengths (short and long heads
    in a seeded order, one empty) with the chunk's rows after them; every
    query of every head is checked, so a tile computed twice into the wrong
    place or never computed fails."""
    dev = device()
    rng = np.random.default_rng(31 * H + n_q)
    D, n_chunk = 128, 50
    lens = np.where(rng.permutation(H) < H // 2, 70, 333).astype(np.int64)[None, :]
    lens[0, int(rng.integers(0, H))] = 0
    off, kr, vr = _ragged_case(rng, lens, H, D, 8)
    cap = int(off[-1])
    kr[cap:] = 0x7FC0
    vr[cap:] = 0x7FC0
    q = random_bf16_bits(rng, (n_q, H, D))
    kc = random_bf16_bits(rng, (n_chunk, H, D))
    vc = random_bf16_bits(rng, (n_chunk, H, D))
    od = torch.full((n_q, H, D), float("nan"), dtype=torch.bfloat16, device=dev)
    scale = 1.0 / np.sqrt(D)
    dp.dp_hs_attention(bf16_from_bits(q, dev), bf16_from_bits(kr, dev), bf16_from_bits(vr, dev),
                       cap, torch.from_numpy(off).to(dev), 0, bf16_from_bits(kc, dev),
                       bf16_from_bits(vc, dev), n_chunk, od, n_q, H, D, dp.DP_BF16, scale)
    torch.cuda.synchronize()
    _check_hs(bits(od), q, kr, vr, off, 0, np.arange(n_q), kc, vc, scale, ("tiles", H, n_q))


def test_hs_attention_clamps_runs_to_capacity():
    """Offsets past the capacity are clamped: the last heads see fewer rows."""
    dev = device()
    rng = np.random.default_rng(7)
    H, D, n_q = 8, 128, 40
    lens = np.array([[30, 10, 50, 20, 64, 1, 0, 90]], np.int64)
    off, kr, vr = _ragged_case(rng, lens, H, D, 0)
    cap = int(off[-1]) - 100                                 # cuts the last run and part of the one before
    q = random_bf16_bits(rng, (n_q, H, D))
    od = torch.zeros((n_q, H, D), dtype=torch.bfloat16, device=dev)
    dp.dp_hs_attention(bf16_from_bits(q, dev), bf16_from_bits(kr, dev), bf16_from_bits(vr, dev),
                       cap, torch.from_numpy(off).to(dev), 0, None, None, 0, od, n_q, H, D,
                       dp.DP_BF16, 0.1)
    torch.cuda.synchronize()
    _check_hs(bits(od), q, kr, vr, np.minimum(off, cap), 0, np.arange(n_q), None, None, 0.1,
              "clamp")


def test_hs_attention_hs_shape_sampled():
    """DeCoPrune-HS shape: 40 heads x 128, per-head runs with the class
    lengths of the 30-chunk HS workload (static heads: sink + window,
    dynamic heads: the gamma mask), layer 1 of a two-layer packed cache,
    followed by the 6,240 chunk rows.  Every head runs; seven queries of six
    heads (static and dynamic) are checked."""
    dev = device()
    w = dpsynth.WORKLOADS["hs"]
    T, H, D = w.seq_len, w.n_heads, w.head_dim
    x0, xf = dpsynth.score_inputs(w)
    ell = oracle.score_f32(x0, xf, w.d)
    n_s = int(oracle.mask(None, T, w.sink_len, w.window_len, w.scored_begin, w.n_scored,
                          w.gamma, streaming=True).sum())
    n_d = int(oracle.mask(ell, T, w.sink_len, w.window_len, w.scored_begin, w.n_scored,
                          w.gamma).sum())
    cls = dpsynth.hs_head_class(w)[:2]
    off = oracle.hs_offsets(cls, np.array([n_s, n_d], np.int64))
    total, n_q = int(off[-1]), w.chunk_tokens
    kr = torch.empty((total, D), dtype=torch.bfloat16, device=dev)
    vr = torch.empty((total, D), dtype=torch.bfloat16, device=dev)
    dpsynth.kv_fill_device(kr, "bf16", 5, dpsynth.STREAM_K, 0, total, D)
    dpsynth.kv_fill_device(vr, "bf16", 5, dpsynth.STREAM_V, 0, total, D)
    q = torch.empty((n_q, H, D), dtype=torch.bfloat16, device=dev)
    kc = torch.empty((n_q, H, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty((n_q, H, D), dtype=torch.bfloat16, device=dev)
    dpsynth.kv_fill_device(q, "bf16", 6, 3, 0, n_q, H * D)
    dpsynth.kv_fill_device(kc, "bf16", 6, dpsynth.STREAM_K, 0, n_q, H * D)
    dpsynth.kv_fill_device(vc, "bf16", 6, dpsynth.STREAM_V, 0, n_q, H * D)
    o = torch.empty_like(q)
    dp.dp_hs_attention(q, kr, vr, total, torch.from_numpy(off).to(dev), 1, kc, vc, n_q, o, n_q,
                       H, D, dp.DP_BF16, 1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 3000, 6111, 6239])
    static = np.flatnonzero(cls[1] == 0)[:3]
    dynamic = np.flatnonzero(cls[1] == 1)[:3]
    heads = np.concatenate([static, dynamic])
    # the checked heads' runs, re-packed on the host, and their chunk columns
    runs = [np.arange(off[H + h], off[H + h + 1]) for h in heads]
    sub_off = np.concatenate([[0], np.cumsum([r.shape[0] for r in runs])]).astype(np.int64)
    all_rows = np.concatenate(runs)
    krh = dpsynth.kv_rows_host("bf16", 5, dpsynth.STREAM_K, 0, all_rows, total, D)
    vrh = dpsynth.kv_rows_host("bf16", 5, dpsynth.STREAM_V, 0, all_rows, total, D)
    kch = dpsynth.kv_layer_host("bf16", 6, dpsynth.STREAM_K, 0, n_q, H * D).reshape(n_q, H, D)
    vch = dpsynth.kv_layer_host("bf16", 6, dpsynth.STREAM_V, 0, n_q, H * D).reshape(n_q, H, D)
    qh = np.zeros((n_q, len(heads), D), np.uint16)
    qh[rows] = dpsynth.kv_rows_host("bf16", 6, 3, 0, rows, n_q, H * D).reshape(len(rows), H, D)[:, heads]
    got = bits(o[torch.from_numpy(rows).to(dev)])[:, heads]
    err, ratio = _check_hs(got, qh, krh, vrh, sub_off, 0, rows, np.ascontiguousarray(kch[:, heads]),
                           np.ascontiguousarray(vch[:, heads]), 1.0 / np.sqrt(D), "hs shape")
    print("hs-shape attention: runs %d / %d rows, max |err| %.2e (%.2f of the bound)"
          % (n_s, n_d, err, ratio))
