"""Two prune steps in flight at once on two streams.

Every entry point enqueues its work on the stream it is given and keeps no
state between calls (the workspaces are the caller's), so two steps over
separate buffers can run concurrently: each is enqueued on its own stream,
three times over with new inputs, without a synchronisation in between, and
each stream's last result is compared with the oracle's step (the DeCoPrune
page, section 어떻게 동작하나: score, shared mask, physical gather; section
무엇과 다른가: the key re-index).
"""
import numpy as np
import pytest
import torch

import dpsynth
import oracle
from compaction_dp_score_amd.step import PruneStep
from gpu_helpers import bf16_from_bits, bits, device, keys_close, random_bf16_bits

pytestmark = pytest.mark.gpu


class _Case:
    """One prune step's buffers and its host inputs (sink + leaving chunk +
    3-chunk window; the chunk is scored)."""

    def __init__(self, rng, dev, L, H, D, tpf, F, d):
        C = tpf * F
        T = 5 * C
        self.C, self.T, self.d, self.L = C, T, d, L
        self.rng = rng
        self.kb = random_bf16_bits(rng, (L, T, H, D), 2.0)
        self.vb = random_bf16_bits(rng, (L, T, H, D))
        self.rf = (np.arange(T) // tpf).astype(np.int32)
        n_frames = T // tpf
        theta = dpsynth.rope_theta(44)
        ft = np.arange(n_frames, dtype=np.float32)
        self.host_rope = dict(theta=theta, frame_t=ft, frame_phase=ft.copy(), q0=float(n_frames),
                              knee=12.0, inv_factor=np.float32(0.125))
        k_src = [bf16_from_bits(self.kb[l], dev) for l in range(L)]
        v_src = [bf16_from_bits(self.vb[l], dev) for l in range(L)]
        self.k_dst = [torch.zeros_like(t) for t in k_src]
        self.v_dst = [torch.zeros_like(t) for t in v_src]
        self.rope = dict(theta=torch.from_numpy(theta).to(dev), frame_t=torch.from_numpy(ft).to(dev),
                         frame_phase=torch.from_numpy(ft.copy()).to(dev), q0=float(n_frames),
                         knee=12.0, inv_factor=0.125)
        self.phase0 = self.rope["frame_phase"].clone()
        self.step = PruneStep(k_src=k_src, v_src=v_src, k_dst=self.k_dst, v_dst=self.v_dst,
                              seq_len=T, sink_len=C, window_len=3 * C, scored_begin=C,
                              n_scored=C, gamma=0.1, d=d,
                              row_frame=torch.from_numpy(self.rf).to(dev), rope=self.rope)
        self.keep_alive = [k_src, v_src]

    def draw(self):
        xf = self.rng.standard_normal((self.C, self.d)).astype(np.float32)
        sig = np.exp(self.rng.uniform(np.log(0.05), np.log(0.44), self.C))[:, None]
        x0 = (xf + sig * self.rng.standard_normal((self.C, self.d))).astype(np.float32)
        return x0, xf

    def check(self, x0, xf):
        C, T = self.C, self.T
        want = oracle.prune_step(x0, xf, self.d, dict(seq_len=T, sink_len=C, window_len=3 * C,
                                                      scored_begin=C, n_scored=C, gamma=0.1),
                                 self.kb, self.vb, self.rf, self.host_rope)
        n = want["idx"].shape[0]
        s = self.step
        assert int(s.n_kept.item()) == n
        assert np.array_equal(s.keep.cpu().numpy(), want["keep"])
        assert np.array_equal(s.idx[:n].cpu().numpy(), want["idx"])
        assert np.array_equal(s.row_frame_dst[:n].cpu().numpy(), want["row_frame"])
        for l in range(self.L):
            assert np.array_equal(bits(self.v_dst[l][:n]), want["v"][l]), l
            ok, worst, _ = keys_close(bits(self.k_dst[l][:n]), want["k"][l], 2e-2)
            assert ok, (l, worst)


def test_two_prune_steps_on_two_streams():
    dev = device()
    cases = [_Case(np.random.default_rng(61), dev, 3, 8, 128, 100, 4, 64),
             _Case(np.random.default_rng(62), dev, 2, 6, 128, 60, 4, 32)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]      # default priority
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    last = [None, None]
    keep_alive = []
    for rep in range(3):
        for i, (case, s) in enumerate(zip(cases, streams)):
            x0, xf = case.draw()
            with torch.cuda.stream(s):
                # inputs, the restored phase table and the cleared outputs are
                # all enqueued on this step's own stream, behind its last step
                x0_d = torch.from_numpy(x0).to(dev, non_blocking=False)
                xf_d = torch.from_numpy(xf).to(dev, non_blocking=False)
                case.rope["frame_phase"].copy_(case.phase0)
                for t in case.k_dst + case.v_dst:
                    t.zero_()
                case.step.run(x0_d, xf_d)
            keep_alive.append((x0_d, xf_d))
            last[i] = (x0, xf)
    for s in streams:
        s.synchronize()
    torch.cuda.synchronize()
    for case, (x0, xf) in zip(cases, last):
        case.check(x0, xf)
