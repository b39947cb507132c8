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


# ---------------------------------------------------------------------------
# Split key layout (DP_KEY_SPLIT): a fixed permutation of a key row's elements,
# the temporal blocks of all heads first, then every head's other dims.  These
# helpers only move data; tests compare the library in either layout with the
# oracle, which works in the natural layout.
# ---------------------------------------------------------------------------
def split_perm(H, D, pair_begin, n_pairs):
    """Index p with split_row = natural_row[p] for a token row of H heads x D."""
    t = np.arange(2 * pair_begin, 2 * (pair_begin + n_pairs))
    other = np.concatenate([np.arange(0, 2 * pair_begin), np.arange(2 * (pair_begin + n_pairs), D)])
    heads = np.arange(H)[:, None] * D
    return np.concatenate([(heads + t[None, :]).ravel(), (heads + other[None, :]).ravel()])


def to_split(k, pair_begin, n_pairs):
    """[..., H, D] natural -> the same shape holding split rows (numpy or torch)."""
    H, D = k.shape[-2], k.shape[-1]
    p = split_perm(H, D, pair_begin, n_pairs)
    if isinstance(k, torch.Tensor):
        flat = k.reshape(k.shape[:-2] + (H * D,))
        return flat.index_select(-1, torch.from_numpy(p).to(k.device)).reshape(k.shape)
    return np.ascontiguousarray(k.reshape(k.shape[:-2] + (H * D,))[..., p].reshape(k.shape))


def from_split(k, pair_begin, n_pairs):
    """Inverse of to_split."""
    H, D = k.shape[-2], k.shape[-1]
    inv = np.argsort(split_perm(H, D, pair_begin, n_pairs))
    if isinstance(k, torch.Tensor):
        flat = k.reshape(k.shape[:-2] + (H * D,))
        return flat.index_select(-1, torch.from_numpy(inv).to(k.device)).reshape(k.shape)
    return np.ascontiguousarray(k.reshape(k.shape[:-2] + (H * D,))[..., inv].reshape(k.shape))


def run_to_split(run, pair_begin, n_pairs):
    """A packed per-head run [n, D] (natural head rows) -> its split form, the
    same [n, D] buffer holding the n temporal blocks, then the n other parts."""
    n, D = run.shape
    t = slice(2 * pair_begin, 2 * (pair_begin + n_pairs))
    other = np.concatenate([np.arange(0, 2 * pair_begin), np.arange(2 * (pair_begin + n_pairs), D)])
    if isinstance(run, torch.Tensor):
        o = torch.from_numpy(other).to(run.device)
        return torch.cat([run[:, t].reshape(-1), run.index_select(1, o).reshape(-1)]).reshape(n, D)
    return np.concatenate([run[:, t].reshape(-1), run[:, other].reshape(-1)]).reshape(n, D)


def run_from_split(run, pair_begin, n_pairs):
    """Inverse of run_to_split."""
    n, D = run.shape
    tw = 2 * n_pairs
    flat = run.reshape(-1)
    tpart = flat[:n * tw].reshape(n, tw)
    opart = flat[n * tw:].reshape(n, D - tw)
    lo = 2 * pair_begin
    if isinstance(run, torch.Tensor):
        return torch.cat([opart[:, :lo], tpart, opart[:, lo:]], dim=1)
    return np.concatenate([opart[:, :lo], tpart, opart[:, lo:]], axis=1)


# ---------------------------------------------------------------------------
# Error bound of the bf16 attention kernels against the float64 oracle.
#
# The kernel computes scores in fp32 from exact bf16 products, probabilities
# p = exp2(s c - m) in fp32, their sum l in fp32 from the unrounded p, the
# product P V from p rounded to bf16 (relative error <= u = 2^-8), and the
# output O / l rounded to bf16 (<= u |o|).  With A = sum_j p_j |v_j| / l
# (the oracle's attention over |V|):
#   * probability rounding moves the output by at most u A;
#   * the output rounding by at most u |o|;
#   * a score error delta_j moves the output by at most
#     max_j |delta_j| (A + |o|) (first order, o = sum p v / sum p); fp32 sums
#     of D exact products err by at most D 2^-24 sum_i |q_i k_i|, which
#     Cauchy-Schwarz bounds by D 2^-24 |q| max_j |k_j|, times the scale;
#     exp2 and the fused scale add a few fp32 ulps (2^-21 covers them);
#   * fp32 accumulation of O and l over n keys (16 keys per MFMA step, one
#     rescale per 64-key tile at most) errs by at most (n/16 + 64) 2^-23
#     relative to A + |o|.
# bound = (u + delta + gamma_n) (A + |o|) + 1e-6.  A tile dropped, doubled
# or paired with the wrong values moves an output by about its share of the
# probability mass times |v - o|; the full-shape tile-coverage tests make that
# share large on purpose.
# ---------------------------------------------------------------------------
def attention_bound(want, want_abs, q_norm, k_norm_max, scale, n_kv):
    """Per-element bound for outputs `want` [rows, H, D] (float64 oracle)
    given the oracle's attention over |V| `want_abs`, the query norms
    q_norm [rows, H] and the largest key norm k_norm_max (scalar or [H])."""
    D = want.shape[-1]
    delta = D * 2.0 ** -24 * abs(scale) * np.asarray(q_norm)[..., None] * \
        np.asarray(k_norm_max)[..., None] + 2.0 ** -21
    gamma = (n_kv / 16.0 + 64.0) * 2.0 ** -23
    return (2.0 ** -8 + delta + gamma) * (want_abs + np.abs(want)) + 1e-6


def check_attention(got_bits, want, want_abs, q_norm, k_norm_max, scale, n_kv, tag):
    """Assert |got - want| <= attention_bound elementwise; returns the
    largest error and the largest error / bound ratio."""
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(got - want)
    bound = attention_bound(want, want_abs, q_norm, k_norm_max, scale, n_kv)
    assert np.all(err <= bound), (tag, float((err - bound).max()), float(err.max()))
    return float(err.max()), float((err / bound).max())


def bf16_abs(b):
    """|x| of bf16 bit patterns (sign cleared; NaN stays NaN)."""
    return np.asarray(b, np.uint16) & np.uint16(0x7FFF)


def bf16_norms(b):
    """Euclidean norms over the last axis of bf16 bit patterns (float64)."""
    x = (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.sqrt((x * x).sum(-1))
