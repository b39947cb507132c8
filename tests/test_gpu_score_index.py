"""GPU parity of dp_score_index (score, mask and kept-index list in one
launch with a decoupled look-back) against the oracle's score, mask and
compaction; bit-exact for the scores, the mask, the index list, the count and
the gathered row frames.

One zero-filled workspace serves every call of a test, so the calls also
check that each call leaves it ready for the next (the generation-tagged
tile states), across changing sizes and inside a replayed HIP graph.
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import oracle
from gpu_helpers import device, to_dev

pytestmark = pytest.mark.gpu


def _score_case(rng, n, d, stride, lo=0.05, hi=1.0):
    xf = rng.standard_normal((n, stride)).astype(np.float32)
    sig = np.exp(rng.uniform(np.log(lo), np.log(hi), n))[:, None]
    x0 = (xf + sig * rng.standard_normal((n, stride))).astype(np.float32)
    if n > 9:
        x0[3] = xf[3]                                 # equal rows
        x0[5, 0] = np.nan
        x0[7, d - 1] = np.inf
        x0[9, :d] = xf[9, :d] + np.float32(1e-40)     # denormal differences
    return x0, xf


class Fused:
    """Buffers of one dp_score_index call site; the workspace is zeroed once."""

    def __init__(self, dev, T_max):
        self.dev = dev
        self.ws = torch.zeros(dp.dp_score_index_workspace_bytes(T_max) // 8 + 1, dtype=torch.int64,
                              device=dev)
        self.idx = torch.empty(T_max, dtype=torch.int32, device=dev)
        self.n = torch.empty(1, dtype=torch.int64, device=dev)
        self.keep = torch.empty(T_max, dtype=torch.uint8, device=dev)
        self.rf_dst = torch.empty(T_max, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)

    def run(self, x0d, xfd, d, stride, pol, ell=None, rf_src=None, keep=True):
        T = pol.seq_len
        self.idx.fill_(-7)
        self.keep.fill_(9)
        dp.dp_score_index(x0d, xfd, d, stride, pol, ell, self.keep if keep else None, self.idx,
                          self.n, rf_src, self.rf_dst if rf_src is not None else None, self.ws,
                          self.err)

    def check(self, T, want_keep, rf_src_host=None, keep=True):
        torch.cuda.synchronize()
        assert int(self.err.item()) == 0
        want_idx = oracle.compact(want_keep)
        n = int(self.n.item())
        assert n == want_idx.shape[0]
        assert np.array_equal(self.idx[:n].cpu().numpy(), want_idx)
        assert np.all(self.idx[n:T].cpu().numpy() == -7)           # nothing beyond the count
        if keep:
            assert np.array_equal(self.keep[:T].cpu().numpy(), want_keep)
        if rf_src_host is not None:
            assert np.array_equal(self.rf_dst[:n].cpu().numpy(), rf_src_host[want_idx])
        return n


@pytest.mark.parametrize("d,stride", [(1, 1), (3, 5), (4, 4), (16, 16), (48, 52), (64, 64),
                                      (100, 100), (256, 256)])
def test_score_index_matches_oracle(d, stride):
    dev = device()
    rng = np.random.default_rng(d * 1000 + stride + 5)
    T, sink, window, sb = 9000 + d, 128, 700, 300
    ns = T - window - sb - 37
    x0, xf = _score_case(rng, ns, d, stride)
    ell_o = oracle.score_f32(x0, xf, d)
    gamma = float(np.nanmedian(ell_o))                # a tie: this value is in ell
    rf = rng.integers(0, 1 << 30, T).astype(np.int32)
    f = Fused(dev, T)
    x0d, xfd, rfd = to_dev(x0, dev), to_dev(xf, dev), to_dev(rf, dev)
    for reversed_ in (False, True):
        pol = dp.make_policy(T, sink, window, sb, ns, gamma, reversed_)
        ell = torch.empty(ns, dtype=torch.float32, device=dev)
        f.run(x0d, xfd, d, stride, pol, ell, rfd)
        want = oracle.mask(ell_o, T, sink, window, sb, ns, gamma, reversed_)
        f.check(T, want, rf)
        g = ell.cpu().numpy()
        both_nan = np.isnan(g) & np.isnan(ell_o)
        assert np.array_equal(g.view(np.uint32)[~both_nan], ell_o.view(np.uint32)[~both_nan])


def test_score_index_many_tiles_and_changing_sizes():
    """Sizes that run as one launch with hundreds of tiles (look-backs cross
    windows of 256 tiles; every plain tile size from 256 to 2,048 rows) and
    sizes that run as separate launches (the prefix-pruning shape, 361,920
    rows with 355,680 scored), plus small ragged sizes, all on one workspace."""
    dev = device()
    rng = np.random.default_rng(11)
    d = 64
    T_max, sink = 2000000, 6240
    n_max = 361920 - sink
    x0, xf = _score_case(rng, n_max, d, d, 0.05, 0.42)
    ell_o = oracle.score_f32(x0, xf, d)
    x0d, xfd = to_dev(x0, dev), to_dev(xf, dev)
    f = Fused(dev, T_max)
    S = dp.DP_MODE_STREAMING
    # (T, sink, n_scored, window, gamma, mode)
    cases = [(361920, sink, n_max, 0, 0.10, 0), (361920, sink, n_max, 0, 0.0, 0),
             (1, 1, 0, 0, 0.1, 0), (255, 0, 255, 0, 0.1, 0), (256, 0, 256, 0, 0.1, 0),
             (257, 1, 200, 56, 0.1, 0), (513, 100, 300, 13, 0.1, 0),
             (33000, sink, 33000 - sink, 0, 0.1, 0),           # 444 tiles, 256-row plain tiles
             (200000, sink, 30000, 0, 0.1, 0),                 # 802 tiles, 512-row plain tiles
             (1000000, sink, 0, 18720, 0.1, S),                # 977 tiles of 1,024 rows
             (T_max, sink, 0, 18720, 0.1, S),                  # 977 tiles of 2,048 rows
             (T_max, sink, 0, 0, 0.1, 0),                      # nothing scored: all kept
             (361920, sink, n_max, 0, float("inf"), 0), (361920, sink, n_max, 0, 0.10, 0)]
    for T, s, ns, win, gamma, mode in cases:
        pol = dp.make_policy(T, s, win, s, ns, gamma, mode=mode)
        f.run(x0d if ns else None, xfd if ns else None, d, d, pol)
        want = oracle.mask(ell_o[:ns] if ns else None, T, s, win, s, ns, gamma,
                           streaming=mode == S)
        n = f.check(T, want)
        if T == 361920 and gamma == 0.10:
            assert 0.1 < n / T < 0.2                  # about 15 % kept
    # the separate-launch path with the mask held in the workspace (keep_out
    # NULL) and the row frames gathered, on the same workspace
    T, ns = 361920, n_max
    pol = dp.make_policy(T, sink, 0, sink, ns, 0.10)
    rf = (np.arange(T) // 1560).astype(np.int32)
    f.run(x0d, xfd, d, d, pol, rf_src=to_dev(rf, dev), keep=False)
    f.check(T, oracle.mask(ell_o[:ns], T, sink, 0, sink, ns, 0.10), rf_src_host=rf, keep=False)


def test_score_index_streaming_no_scores_and_optional_outputs():
    dev = device()
    rng = np.random.default_rng(12)
    T, sink, window, sb, ns, d = 20000, 1560, 4680, 2000, 9000, 64
    x0, xf = _score_case(rng, ns, d, d)
    x0d, xfd = to_dev(x0, dev), to_dev(xf, dev)
    f = Fused(dev, T)
    pol = dp.make_policy(T, sink, window, sb, ns, 0.1, mode=dp.DP_MODE_STREAMING)
    f.run(None, None, d, d, pol)
    f.check(T, oracle.mask(None, T, sink, window, sb, ns, 0.1, streaming=True))
    pol = dp.make_policy(T, sink, window, sb, ns, 0.0)              # gamma 0: only NaN drops
    f.run(x0d, xfd, d, d, pol, keep=False)
    want = oracle.mask(oracle.score_f32(x0, xf), T, sink, window, sb, ns, 0.0)
    assert f.check(T, want, keep=False) == T - 1
    pol = dp.make_policy(T - 3, 7, 5, 7, 0, 0.1)                    # no scored rows
    f.run(None, None, d, d, pol)
    f.check(T - 3, np.ones(T - 3, np.uint8))


def test_score_index_graph_replays():
    """Captured once, replayed with new inputs and eager work in between;
    the workspace state carries from replay to replay."""
    dev = device()
    rng = np.random.default_rng(13)
    T, sink, window, d = 31200, 6240, 18720, 64
    sb, ns = sink, 6240
    x0_s = torch.empty((ns, d), dtype=torch.float32, device=dev)
    xf_s = torch.empty((ns, d), dtype=torch.float32, device=dev)
    f = Fused(dev, T)
    pol = dp.make_policy(T, sink, window, sb, ns, 0.1)
    x0, xf = _score_case(rng, ns, d, d, 0.05, 0.44)
    x0_s.copy_(to_dev(x0, dev))
    xf_s.copy_(to_dev(xf, dev))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dp.dp_score_index(x0_s, xf_s, d, d, pol, None, f.keep, f.idx, f.n, None, None, f.ws, f.err)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dp.dp_score_index(x0_s, xf_s, d, d, pol, None, f.keep, f.idx, f.n, None, None, f.ws, f.err)
    torch.cuda.synchronize()
    for rep in range(4):
        x0, xf = _score_case(rng, ns, d, d, 0.05, 0.44)
        x0_s.copy_(to_dev(x0, dev))
        xf_s.copy_(to_dev(xf, dev))
        f.idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle.mask(oracle.score_f32(x0, xf), T, sink, window, sb, ns, 0.1)
        f.check(T, want)


def test_score_index_reports_a_workspace_not_zero_filled():
    """A workspace whose ticket word was never cleared hands every workgroup a
    tile number past the launch's last tile: each one records DP_ESTALL and
    returns at once, writing no mask, index or count (no wait is entered).
    Zero-filling the workspace again makes the next call correct."""
    dev = device()
    rng = np.random.default_rng(41)
    T, sink, window, d = 31200, 6240, 18720, 64
    sb, ns = sink, 6240
    x0, xf = _score_case(rng, ns, d, d, 0.05, 0.44)
    x0d, xfd = to_dev(x0, dev), to_dev(xf, dev)
    pol = dp.make_policy(T, sink, window, sb, ns, 0.1)
    f = Fused(dev, T)
    f.ws.view(torch.int32)[0] = 0x7FFF0000          # ticket word: far past any tile count
    f.n.fill_(-5)
    f.run(x0d, xfd, d, d, pol)
    torch.cuda.synchronize()
    assert int(f.err.item()) == dp.DP_ESTALL
    assert int(f.n.item()) == -5
    assert np.all(f.idx.cpu().numpy() == -7) and np.all(f.keep.cpu().numpy() == 9)
    f.ws.zero_()
    f.err.zero_()
    f.run(x0d, xfd, d, d, pol)
    f.check(T, oracle.mask(oracle.score_f32(x0, xf), T, sink, window, sb, ns, 0.1))
