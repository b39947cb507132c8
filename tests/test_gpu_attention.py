"""GPU parity of dp_attention (a chunk's queries over the compacted cache)
against the float64 oracle.

Tolerance: the kernel rounds the softmax probabilities to bf16 before the
P.V product (relative 2^-9 each) and rounds the output to bf16 (half an ulp,
relative 2^-9); accumulation is fp32.  With |v| below ~5 for N(0,1) data the
probability rounding moves an output by at most ~2^-9 * 5 ~ 0.01 in the worst
case and far less on average, so the bar is |o - o_ref| <= 4e-3 + 1e-2 |o_ref|.
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import dpsynth
import oracle
from gpu_helpers import bf16_from_bits, bits, device, random_bf16_bits

pytestmark = pytest.mark.gpu

ATOL, RTOL = 4e-3, 1e-2


def _check(got_bits, want, tag):
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(got - want)
    bound = ATOL + RTOL * np.abs(want)
    worst = float((err - bound).max())
    assert np.all(err <= bound), (tag, worst, float(err.max()))
    return float(err.max())


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
    want = oracle.attention(q, k, v, np.arange(n_q), n_kv=n_kv, scale=scale)
    err = _check(bits(od), want, (n_q, n_kv, H))
    print("attention %dx%d H=%d: max |err| %.2e" % (n_q, n_kv, H, err))


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
    want = oracle.attention(q, k, v, np.arange(n_q), scale=2.0)
    _check(bits(od), want, "peaked")
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
    want = oracle.attention(qfull, kh, vh, rows)
    got = bits(o[torch.from_numpy(rows).to(dev)])
    err = _check(got, want, "eviction shape")
    print("eviction-shape attention: max |err| %.2e over %d sampled queries x %d heads"
          % (err, len(rows), H))
