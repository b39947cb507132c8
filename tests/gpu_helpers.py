"""Helpers shared by the GPU parity tests (device buffers and bit views)."""
import numpy as np
import pytest
import torch


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def bf16_from_bits(bits_u16, dev):
    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16)).to(dev).view(torch.bfloat16)


def bits(t):
    """Host numpy bit pattern of a device tensor (uint16 for bf16, uint32 for fp32)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.numpy()


def as_float(b):
    """fp32 values of bf16 (uint16) or fp32 (uint32) bit patterns."""
    if b.dtype == np.uint16:
        return (b.astype(np.uint32) << 16).view(np.float32)
    return b.view(np.float32)


def random_bf16_bits(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def random_f32(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def keys_close(got_bits, want_bits, tol):
    """Max-abs difference of two key tensors given as bit patterns; NaNs must match."""
    g, w = as_float(got_bits), as_float(want_bits)
    gn, wn = np.isnan(g), np.isnan(w)
    assert np.array_equal(gn, wn)
    g64, w64 = g[~gn].astype(np.float64), w[~wn].astype(np.float64)
    same = g64 == w64                     # also equal infinities
    with np.errstate(invalid="ignore"):
        d = np.where(same, 0.0, np.abs(g64 - w64))
    worst = float(d.max()) if d.size else 0.0
    exact = int(np.count_nonzero(got_bits != want_bits))
    return worst <= tol, worst, exact
