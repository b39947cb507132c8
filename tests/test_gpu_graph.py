"""A whole prune step captured into a HIP graph and replayed.

Every entry point only enqueues work on the caller's stream, allocates
nothing and never synchronises, so score -> index -> gather (with the fused
re-index), and the ring-layout eviction (score and index, table, sink
re-index, append with the fused re-index), can be captured once and
replayed.  The inputs change between replays (new scores, restored phase
table and cache), with eager work and synchronisations in between, and
every replay is compared with the oracle.  Entering torch.cuda.graph empties
torch's allocator cache, so these tests also check that every buffer the
captured kernels reach is still held (the pointer arrays hold their tensors).
"""
import numpy as np
import pytest
import torch

import dpsynth
import oracle
from compaction_dp_score_amd.step import PruneStep
from gpu_helpers import bf16_from_bits, bits, device, keys_close, random_bf16_bits

pytestmark = pytest.mark.gpu


def test_prune_step_graph_replays_match_oracle():
    dev = device()
    rng = np.random.default_rng(31)
    L, H, D, tpf, F = 3, 8, 128, 100, 4
    C = tpf * F
    T = 5 * C                                    # sink + leaving chunk + 3-chunk window
    d = 64
    kb = random_bf16_bits(rng, (L, T, H, D), 2.0)
    vb = random_bf16_bits(rng, (L, T, H, D))
    rf = (np.arange(T) // tpf).astype(np.int32)
    n_frames = T // tpf
    theta = dpsynth.rope_theta(44)
    ft = np.arange(n_frames, dtype=np.float32)
    k_src = [bf16_from_bits(kb[l], dev) for l in range(L)]
    v_src = [bf16_from_bits(vb[l], dev) for l in range(L)]
    k_dst = [torch.zeros_like(t) for t in k_src]
    v_dst = [torch.zeros_like(t) for t in v_src]
    rope = dict(theta=torch.from_numpy(theta).to(dev), frame_t=torch.from_numpy(ft).to(dev),
                frame_phase=torch.from_numpy(ft.copy()).to(dev), q0=float(n_frames), knee=12.0,
                inv_factor=0.125)
    step = PruneStep(k_src=k_src, v_src=v_src, k_dst=k_dst, v_dst=v_dst, seq_len=T, sink_len=C,
                     window_len=3 * C, scored_begin=C, n_scored=C, gamma=0.1, d=d,
                     row_frame=torch.from_numpy(rf).to(dev), rope=rope)
    x0_s = torch.empty((C, d), dtype=torch.float32, device=dev)     # static graph inputs
    xf_s = torch.empty((C, d), dtype=torch.float32, device=dev)
    phase0 = rope["frame_phase"].clone()

    def draw():
        xf = rng.standard_normal((C, d)).astype(np.float32)
        sig = np.exp(rng.uniform(np.log(0.05), np.log(0.44), C))[:, None]
        return (xf + sig * rng.standard_normal((C, d))).astype(np.float32), xf

    # warm up on a side stream, then capture
    x0, xf = draw()
    x0_s.copy_(torch.from_numpy(x0))
    xf_s.copy_(torch.from_numpy(xf))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.run(x0_s, xf_s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    rope["frame_phase"].copy_(phase0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run(x0_s, xf_s)
    torch.cuda.synchronize()

    host_rope = dict(theta=theta, frame_t=ft, frame_phase=ft.copy(), q0=float(n_frames), knee=12.0,
                     inv_factor=np.float32(0.125))
    for rep in range(4):
        x0, xf = draw()
        x0_s.copy_(torch.from_numpy(x0))            # eager work between replays
        xf_s.copy_(torch.from_numpy(xf))
        rope["frame_phase"].copy_(phase0)
        for t in k_dst + v_dst:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle.prune_step(x0, xf, d, dict(seq_len=T, sink_len=C, window_len=3 * C,
                                                 scored_begin=C, n_scored=C, gamma=0.1),
                                 kb, vb, rf, host_rope)
        n = want["idx"].shape[0]
        assert int(step.n_kept.item()) == n, rep
        assert np.array_equal(step.keep.cpu().numpy(), want["keep"]), rep
        assert np.array_equal(step.idx[:n].cpu().numpy(), want["idx"]), rep
        assert np.array_equal(rope["frame_phase"].cpu().numpy(), want["tables"][3]), rep
        for l in range(L):
            assert np.array_equal(bits(v_dst[l][:n]), want["v"][l]), (rep, l)
            ok, worst, _ = keys_close(bits(k_dst[l][:n]), want["k"][l], 2e-2)
            assert ok, (rep, l, worst)
            assert np.all(bits(k_dst[l][n:]) == 0), (rep, l)


def test_random_mask_through_the_same_gather():
    """The page's random-selection ablation keeps rows at random at the same
    ratio; any keep array goes through the same index and gather."""
    dev = device()
    rng = np.random.default_rng(32)
    L, T, H, D = 2, 3000, 4, 64
    kb = random_bf16_bits(rng, (L, T, H, D))
    keep = (rng.random(T) < 0.1457).astype(np.uint8)        # ~85.43 % pruned
    k_src = [bf16_from_bits(kb[l], dev) for l in range(L)]
    k_dst = [torch.zeros_like(t) for t in k_src]
    step = PruneStep(k_src=k_src, v_src=None, k_dst=k_dst, v_dst=None, seq_len=T, sink_len=0,
                     window_len=0, scored_begin=0, n_scored=0, gamma=0.1, d=16)
    step.keep.copy_(torch.from_numpy(keep))
    step.run_from_keep()
    torch.cuda.synchronize()
    idx = oracle.compact(keep)
    n = idx.shape[0]
    assert int(step.n_kept.item()) == n
    want = oracle.gather(kb, idx)
    for l in range(L):
        assert np.array_equal(bits(k_dst[l][:n]), want[l])
    assert abs(oracle.pr(n, T) - 0.8543) < 0.02


def test_ring_step_graph_replays_match_oracle():
    """RingStep.evict on the compressed axis captured once into a graph and
    replayed from the same starting cache (tail, row frames and phase table
    restored eagerly between replays), every replay checked against the
    oracle's ring-layout step: tail, frames and phases exact, V bit for bit,
    keys within the re-index bar."""
    import compaction_dp_score_amd as dp
    from compaction_dp_score_amd.step import RingStep
    from gpu_helpers import to_dev
    dev = device()
    rng = np.random.default_rng(37)
    L, H, D, tpf, F, W = 2, 3, 128, 16, 2, 2
    C, R = tpf * F, W + 1
    knee, factor, npairs = float(W * F), 4.0, 12
    n_frames = (R + 3) * F
    cap = C + R * C + 2 * C
    theta = dpsynth.rope_theta(npairs)
    frame_t = np.arange(n_frames, dtype=np.float32)
    kb = np.zeros((L, cap, H, D), np.uint16)
    vb = np.zeros((L, cap, H, D), np.uint16)
    kb[:, :(R + 1) * C] = random_bf16_bits(rng, (L, (R + 1) * C, H, D), 2.0)
    vb[:, :(R + 1) * C] = random_bf16_bits(rng, (L, (R + 1) * C, H, D))
    rf0 = np.full(cap, -1, np.int32)
    rf0[:(R + 1) * C] = np.arange((R + 1) * C) // tpf
    k = [bf16_from_bits(kb[l], dev) for l in range(L)]
    v = [bf16_from_bits(vb[l], dev) for l in range(L)]
    rf_d, phase = to_dev(rf0, dev), to_dev(frame_t.copy(), dev)
    tail = torch.tensor([(R + 1) * C], dtype=torch.int64, device=dev)
    step = RingStep(k_layers=k, v_layers=v, sink_len=C, chunk_rows=C, n_slots=R,
                    frames_per_chunk=F, row_frame=rf_d, tail=tail, d=16, gamma=0.1,
                    rope=dict(theta=to_dev(theta, dev), frame_t=to_dev(frame_t, dev),
                              frame_phase=phase, knee=knee, inv_factor=1.0 / factor),
                    axis=dp.DP_AXIS_COMPRESSED)
    x0_s = torch.empty((C, 16), dtype=torch.float32, device=dev)
    xf_s = torch.empty((C, 16), dtype=torch.float32, device=dev)
    q0 = float((R + 1) * F)

    def restore():
        for l in range(L):
            k[l].copy_(bf16_from_bits(kb[l], dev))
            v[l].copy_(bf16_from_bits(vb[l], dev))
        rf_d.copy_(to_dev(rf0, dev))
        phase.copy_(to_dev(frame_t, dev))
        tail.fill_((R + 1) * C)
        torch.cuda.synchronize()

    restore()
    step.evict(0, x0_s, xf_s, q0)                   # eager first call
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    restore()
    with torch.cuda.graph(g):
        step.evict(0, x0_s, xf_s, q0)
    for rep in range(3):
        xf = rng.standard_normal((C, 16)).astype(np.float32)
        x0 = (xf + np.exp(rng.uniform(np.log(0.05), np.log(0.6), C))[:, None]
              * rng.standard_normal((C, 16))).astype(np.float32)
        restore()
        x0_s.copy_(to_dev(x0, dev))
        xf_s.copy_(to_dev(xf, dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        widx = oracle.compact(oracle.mask(oracle.score_f32(x0, xf), C, 0, 0, 0, C, 0.1))
        ok_, ov_, orf = kb.copy(), vb.copy(), rf0.copy()
        otail = oracle.append_kept(ok_, C, C, widx, (R + 1) * C, orf)
        oracle.append_kept(ov_, C, C, widx, (R + 1) * C, None)
        tables = oracle.rope_frames(frame_t, frame_t, q0, knee, np.float32(1.0 / factor), theta,
                                    compressed=True)
        live = np.flatnonzero(orf[:otail] >= 0)
        for l in range(L):
            sub = np.ascontiguousarray(ok_[l][live])
            oracle.rope_rows(sub, orf[live], 0, tables)
            ok_[l][live] = sub
        assert step.dev_error.item() == 0 and tail.item() == otail, rep
        assert np.array_equal(rf_d.cpu().numpy(), orf), rep
        assert np.array_equal(phase.cpu().numpy(), tables[3]), rep
        for l in range(L):
            assert np.array_equal(bits(v[l]), ov_[l]), (rep, l)
            good, worst, _ = keys_close(bits(k[l]), ok_[l], 2e-2)
            assert good, (rep, l, worst)
