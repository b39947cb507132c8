"""The attention error bound used by the GPU parity tests, checked on the CPU
against an emulation of the kernel's roundings (numpy float32: fp32 scores,
exp2 with the running max, fp32 sum of the unrounded probabilities, bf16
probabilities into P.V, bf16 output), on random inputs.  The emulation must
stay inside the bound, and the bound must not be vacuous: the emulation's
worst error is within a factor of ten of it."""
import numpy as np
import torch

import oracle
from gpu_helpers import attention_bound, bf16_abs, bf16_norms, random_bf16_bits


def _bf16_round(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _emulate(q, k, v, scale, tile=64):
    """Kernel-order attention of every query over all keys: per 64-key tile
    fp32 scores, running max (raised only when it grows by more than 8 in
    log2 units), p = exp2(s c - m) in fp32, l += sum p, O = O corr + bf16(p) V."""
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    n_q, H, D = qf.shape
    c = np.float32(scale * np.log2(np.e))
    out = np.zeros((n_q, H, D), np.float32)
    for h in range(H):
        s_all = (qf[:, h] @ kf[:, h].T).astype(np.float32)
        m = np.full(n_q, -np.inf, np.float32)
        l = np.zeros(n_q, np.float32)
        o = np.zeros((n_q, D), np.float32)
        for t0 in range(0, kf.shape[0], tile):
            s = s_all[:, t0:t0 + tile]
            mt = (s.max(axis=1) * c).astype(np.float32)
            grow = mt > m + 8
            mn = np.where(grow, np.maximum(m, mt), m)
            corr = np.exp2(np.where(grow, m - mn, 0)).astype(np.float32)
            l, o, m = l * corr, o * corr[:, None], mn
            p = np.exp2(s * c - m[:, None]).astype(np.float32)
            l = (l + p.sum(axis=1, dtype=np.float32)).astype(np.float32)
            o = (o + _bf16_round(p) @ vf[t0:t0 + tile, h]).astype(np.float32)
        out[:, h] = _bf16_round(o / l[:, None])
    return out.astype(np.float64)


def _ratio(q, k, v, scale):
    n = k.shape[0]
    rows = np.arange(q.shape[0])
    want = oracle.attention(q, k, v, rows, scale=scale)
    want_abs = oracle.attention(q, k, bf16_abs(v), rows, scale=scale)
    bound = attention_bound(want, want_abs, bf16_norms(q), bf16_norms(k).max(axis=0), scale, n)
    err = np.abs(_emulate(q, k, v, scale) - want)
    return float((err / bound).max())


def test_emulated_kernel_stays_inside_the_bound_and_near_it():
    """Inside the bound on every element, and within a factor of ten of it on
    each case (the bound is not vacuous: the bf16 output and probability
    roundings it prices do occur at that size)."""
    rng = np.random.default_rng(5)
    for n_q, n_kv, H, scale in ((64, 1000, 2, 1 / np.sqrt(128)), (16, 300, 3, 2.0),
                                (32, 4096, 1, 1 / np.sqrt(128))):
        q = random_bf16_bits(rng, (n_q, H, 128))
        k = random_bf16_bits(rng, (n_kv, H, 128))
        v = random_bf16_bits(rng, (n_kv, H, 128), 2.0)
        r = _ratio(q, k, v, scale)
        assert 0.1 <= r <= 1.0, (n_q, n_kv, H, r)
