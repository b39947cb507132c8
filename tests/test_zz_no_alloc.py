"""dp_compact_index_noalloc (the kept-index list with the library's static
scratch, for callers that cannot allocate) against dp_compact_index with a
workspace, called through the C ABI: bit-exact index list, count and gathered
row frames, on consecutive calls whose sizes shrink (the static scratch keeps
the previous call's counts), and on an empty input."""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import oracle
from gpu_helpers import device, to_dev

pytestmark = pytest.mark.gpu


def _with_workspace(keep_d, T, rf_d, dev):
    idx = torch.full((max(1, T),), -7, dtype=torch.int32, device=dev)
    n = torch.full((1,), -5, dtype=torch.int64, device=dev)
    rf2 = torch.full((max(1, T),), -9, dtype=torch.int32, device=dev)
    ws = torch.empty(dp.dp_compact_workspace_bytes(T) // 4 + 1, dtype=torch.int32, device=dev)
    dp.dp_compact_index(keep_d, T, idx, n, rf_d, rf2, ws)
    return idx, n, rf2


def _without(keep_d, T, rf_d, dev):
    idx = torch.full((max(1, T),), -7, dtype=torch.int32, device=dev)
    n = torch.full((1,), -5, dtype=torch.int64, device=dev)
    rf2 = torch.full((max(1, T),), -9, dtype=torch.int32, device=dev)
    dp.dp_compact_index_noalloc(keep_d, T, idx, n, rf_d, rf2)
    return idx, n, rf2


def test_noalloc_index_matches_the_workspace_form():
    dev = device()
    rng = np.random.default_rng(61)
    for T, rate in ((3_000_001, 0.15), (70_001, 0.6), (4_095, 0.5), (1, 1.0), (0, 0.5)):
        keep = (rng.random(T) < rate).astype(np.uint8)
        rf = rng.integers(0, 1 << 30, max(1, T)).astype(np.int32)
        keep_d = to_dev(keep if T else np.zeros(1, np.uint8), dev)
        rf_d = to_dev(rf, dev)
        a = _with_workspace(keep_d, T, rf_d, dev)
        b = _without(keep_d, T, rf_d, dev)
        torch.cuda.synchronize()
        want = oracle.compact(keep)
        n = want.shape[0]
        assert int(a[1].item()) == n and int(b[1].item()) == n, T
        for x, y in zip(a, b):
            assert torch.equal(x, y), T
        assert np.array_equal(b[0][:n].cpu().numpy(), want), T
        assert np.array_equal(b[2][:n].cpu().numpy(), rf[want]), T
        assert np.all(b[0][n:].cpu().numpy() == -7) and np.all(b[2][n:].cpu().numpy() == -9), T


def test_noalloc_index_on_another_stream():
    """Calls on a stream of the current device; the scratch is the device's."""
    dev = device()
    rng = np.random.default_rng(62)
    T = 200_000
    keep = (rng.random(T) < 0.3).astype(np.uint8)
    keep_d = to_dev(keep, dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        idx = torch.empty(T, dtype=torch.int32, device=dev)
        n = torch.empty(1, dtype=torch.int64, device=dev)
        dp.dp_compact_index_noalloc(keep_d, T, idx, n, None, None)
    torch.cuda.synchronize()
    want = oracle.compact(keep)
    assert int(n.item()) == want.shape[0]
    assert np.array_equal(idx[:want.shape[0]].cpu().numpy(), want)
