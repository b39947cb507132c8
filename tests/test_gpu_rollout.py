"""A rollout of several chunk-eviction steps, GPU against the oracle in
lockstep (DeCoPrune page, sections 어떻게 동작하나 and 무엇과 다른가).

Each step: the chunk leaving the w-chunk window is scored and masked (rows
compacted by earlier steps are kept, the sink is kept), every layer's K and V
are gathered into a new cache with the keys re-indexed for the next query
origin, then a freshly generated chunk is appended.  Frame phases carry over
from step to step, so the incremental re-index is exercised; the cumulative
pruning ratio is checked against the oracle's counts.
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import dpsynth
import oracle
from gpu_helpers import bf16_from_bits, bits, device, keys_close, random_bf16_bits

pytestmark = pytest.mark.gpu

L, H, D = 2, 3, 64
TPF, F = 16, 2            # tokens per frame, frames per chunk
C = TPF * F               # tokens per chunk
W = 2                     # window chunks
STEPS = 7
NPAIRS = 12
KNEE = float(W * F)
FACTOR = 4.0


def _chunk_scores(rng, d=16):
    xf = rng.standard_normal((C, d)).astype(np.float32)
    sig = np.exp(rng.uniform(np.log(0.05), np.log(0.6), C))[:, None]
    x0 = (xf + sig * rng.standard_normal((C, d))).astype(np.float32)
    return x0, xf


def test_rollout_steps_match_oracle():
    dev = device()
    rng = np.random.default_rng(42)
    n_frames_max = (W + 2 + STEPS) * F
    theta = dpsynth.rope_theta(NPAIRS)
    frame_t = np.arange(n_frames_max, dtype=np.float32)
    phase_host = frame_t.copy()                          # oracle's phase table
    phase_dev = torch.from_numpy(phase_host.copy()).to(dev)
    theta_d, ft_d = torch.from_numpy(theta).to(dev), torch.from_numpy(frame_t).to(dev)
    ws_rope = torch.empty(dp.dp_rope_workspace_bytes(n_frames_max, NPAIRS) // 4 + 4,
                          dtype=torch.float32, device=dev)

    # initial cache: sink chunk + W + 1 chunks (the first of them leaves at step 0)
    n0 = (W + 2) * C
    kh = random_bf16_bits(rng, (L, n0, H, D), 2.0)
    vh = random_bf16_bits(rng, (L, n0, H, D))
    rfh = (np.arange(n0) // TPF).astype(np.int32)
    kd = [bf16_from_bits(kh[l], dev) for l in range(L)]
    vd = [bf16_from_bits(vh[l], dev) for l in range(L)]
    rfd = torch.from_numpy(rfh).to(dev)
    pr = dp.dp_pr_counter()
    vis_total, full_total, generated = 0, 0, n0
    for s in range(STEPS):
        T = kh.shape[1]
        sc_begin = T - (W + 1) * C                     # the chunk leaving the window
        x0, xf = _chunk_scores(rng)
        q0 = float((W + 2 + s) * F)                    # first frame of the next chunk
        # ---- GPU step ----
        keep = torch.empty(T, dtype=torch.uint8, device=dev)
        pol = dp.make_policy(T, C, W * C, sc_begin, C, 0.1)
        dp.dp_score_mask(torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev), 16, 16, pol,
                         None, keep)
        idx = torch.empty(T, dtype=torch.int32, device=dev)
        nk = torch.zeros(1, dtype=torch.int64, device=dev)
        rf_new = torch.empty(T, dtype=torch.int32, device=dev)
        ws = torch.empty(dp.dp_compact_workspace_bytes(T) // 4, dtype=torch.int32, device=dev)
        dp.dp_compact_index(keep, T, idx, nk, rfd, rf_new, ws)
        kd2 = [torch.empty_like(t) for t in kd]
        vd2 = [torch.empty_like(t) for t in vd]
        kv = dp.dp_kv()
        arrs = [dp.ptr_array(x, dev) for x in (kd, vd, kd2, vd2)]
        kv.k_src, kv.v_src, kv.k_dst, kv.v_dst = [a.data_ptr() for a in arrs]
        kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dp.DP_BF16
        kv.src_rows, kv.dst_capacity = T, T
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        kv.dev_error = err.data_ptr()
        rope = dp.make_rope(theta_d, ft_d, phase_dev, q0, KNEE, 1.0 / FACTOR)
        dp.dp_gather_kv(kv, idx, nk, rf_new, rope, ws_rope)
        torch.cuda.synchronize()
        n = int(nk.item())
        # ---- oracle step ----
        ell = oracle.score_f32(x0, xf)
        keep_o = oracle.mask(ell, T, C, W * C, sc_begin, C, 0.1)
        idx_o = oracle.compact(keep_o)
        assert np.array_equal(keep.cpu().numpy(), keep_o), s
        assert n == idx_o.shape[0] and err.item() == 0, s
        kh = oracle.gather(kh, idx_o)
        vh = oracle.gather(vh, idx_o)
        rfh = oracle.gather_i32(rfh, idx_o)
        tables = oracle.rope_frames(frame_t, phase_host, q0, KNEE, np.float32(1.0 / FACTOR), theta)
        phase_host = tables[3]
        for l in range(L):
            oracle.rope_rows(kh[l], rfh, 0, tables)
        assert np.array_equal(phase_dev.cpu().numpy(), phase_host), s
        for l in range(L):
            assert np.array_equal(bits(vd2[l][:n]), vh[l]), (s, l)
            ok, worst, _ = keys_close(bits(kd2[l][:n]), kh[l], 2e-2)
            assert ok, (s, l, worst)
            assert np.array_equal(bits(kd2[l][:n]), kh[l]), (s, l)      # in practice bit-exact
        # pruning ratio: visible history positions vs FullKV, cumulative over steps
        dp.dp_pr_add(pr, L * H * n, L * H * generated)
        vis_total += L * H * n
        full_total += L * H * generated
        assert dp.dp_pr_value(pr) == oracle.pr(vis_total, full_total)
        # ---- append a freshly generated chunk (fresh keys carry phase = t) ----
        c_new = W + 2 + s
        k_new = random_bf16_bits(rng, (L, C, H, D), 2.0)
        v_new = random_bf16_bits(rng, (L, C, H, D))
        rf_c = (c_new * F + np.arange(C) // TPF).astype(np.int32)
        kh = np.concatenate([kh, k_new], axis=1)
        vh = np.concatenate([vh, v_new], axis=1)
        rfh = np.concatenate([rfh, rf_c])
        kd = [torch.cat([kd2[l][:n], bf16_from_bits(k_new[l], dev)]) for l in range(L)]
        vd = [torch.cat([vd2[l][:n], bf16_from_bits(v_new[l], dev)]) for l in range(L)]
        rfd = torch.cat([rf_new[:n], torch.from_numpy(rf_c).to(dev)])
        generated += C
    # the sink keys have been re-indexed at every step; the cache keeps the sink rows
    assert np.all(rfh[:C] == np.arange(C) // TPF)
    print("rollout: %d steps, cache %d rows of %d generated, cumulative PR %.4f"
          % (STEPS, kh.shape[1], generated, dp.dp_pr_value(pr)))
