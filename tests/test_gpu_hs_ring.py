"""DeCoPrune-HS in the ring layout, through the existing entry points.

The DeCoPrune page (section 무엇과 다른가) splits each layer's heads into a
static class (Streaming: sink + recent window) and a dynamic class (the
DeCoPrune mask); the split is fixed per layer, so a model can order each
layer's heads class by class (a permutation of its projection weights) and
keep one token-major cache per class:
  static  [sink | window ring]                 (never grows)
  dynamic [sink | window ring | history]       (the shared-mask ring layout)
Every dynamic head keeps the same rows (the mask is shared), so a leaving
chunk is compacted by one dp_append_kept over the dynamic buffers of all
layers, the old keys are re-indexed by dp_rope_apply, and attention runs per
class buffer with dp_attention.  This test rolls the layout forward step by
step against the oracle, ties its first step to the HS gather oracle head by
head, and checks that it ends up holding, head by head, the rows of the
out-of-place rollout (a different order) and the same attention outputs.
"""
import numpy as np
import pytest
import torch

import compaction_dp_score_amd as dp
import dpsynth
import oracle
from gpu_helpers import bf16_from_bits, bits, device, keys_close, random_bf16_bits, to_dev

pytestmark = pytest.mark.gpu

L, H, D = 2, 6, 128
HC = H // 2                 # heads per class in every layer
TPF, F = 16, 2
C = TPF * F
W = 2                       # window chunks after an eviction; the ring holds W + 1 slots
R = W + 1
STEPS = 5
NPAIRS = 12
KNEE = float(W * F)
FACTOR = 4.0
ATOL, RTOL = 6e-3, 1e-2


def _scores(rng):
    xf = rng.standard_normal((C, 16)).astype(np.float32)
    sig = np.exp(rng.uniform(np.log(0.05), np.log(0.6), C))[:, None]
    return (xf + sig * rng.standard_normal((C, 16))).astype(np.float32), xf


def _inplace(k, v, cap, err, alive):
    kv = dp.dp_kv_inplace()
    arrs = [dp.ptr_array(k, k[0].device), dp.ptr_array(v, k[0].device)]
    alive += arrs
    kv.k_layers, kv.v_layers = arrs[0].data_ptr(), arrs[1].data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = len(k), k[0].shape[1], D, dp.DP_BF16
    kv.capacity = cap
    kv.dev_error = err.data_ptr()
    return kv, arrs[0]


def _rope_valid(k, rf, tables):
    rows = np.flatnonzero(rf >= 0)
    sub = np.ascontiguousarray(k[rows])
    oracle.rope_rows(sub, rf[rows], 0, tables)
    k[rows] = sub


def _canon(kc, vc, rfc):
    """Rows as a sorted table (frame, K bits, V bits): the row set, order-free."""
    keyv = np.concatenate([rfc[:, None].astype(np.int64),
                           kc.reshape(rfc.shape[0], -1).astype(np.int64),
                           vc.reshape(rfc.shape[0], -1).astype(np.int64)], axis=1)
    return keyv[np.lexsort(keyv.T[::-1])]


def test_hs_ring_rollout_matches_oracle_and_out_of_place():
    dev = device()
    rng = np.random.default_rng(17)
    head_class = np.zeros((L, H), np.uint8)              # 0 static, 1 dynamic
    for l in range(L):
        head_class[l, rng.permutation(H)[:HC]] = 1
    heads = [[np.flatnonzero(head_class[l] == c) for l in range(L)] for c in (0, 1)]
    n_frames = (R + 2 + STEPS) * F
    theta = dpsynth.rope_theta(NPAIRS)
    frame_t = np.arange(n_frames, dtype=np.float32)
    init_k = random_bf16_bits(rng, (L, (R + 1) * C, H, D), 2.0)
    init_v = random_bf16_bits(rng, (L, (R + 1) * C, H, D))
    init_rf = (np.arange((R + 1) * C) // TPF).astype(np.int32)
    draws = []
    for s in range(STEPS):
        x0, xf = _scores(rng)
        draws.append((x0, xf, random_bf16_bits(rng, (L, C, H, D), 2.0),
                      random_bf16_bits(rng, (L, C, H, D))))
    caps = [(R + 1) * C, (R + 1) * C + STEPS * C]        # static, dynamic

    def by_class(a, c):                                  # [L, rows, H, D] -> the class's heads
        return np.ascontiguousarray(np.stack([a[l][:, heads[c][l]] for l in range(L)]))

    # ---- GPU: one token-major ring buffer per class and layer ----
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    alive, gk, gv, grf, kvs, arr_k = [], [], [], [], [], []
    for c in (0, 1):
        kb = np.zeros((L, caps[c], HC, D), np.uint16)
        vb = np.zeros((L, caps[c], HC, D), np.uint16)
        kb[:, :(R + 1) * C], vb[:, :(R + 1) * C] = by_class(init_k, c), by_class(init_v, c)
        rf = np.full(caps[c], -1, np.int32)
        rf[:(R + 1) * C] = init_rf
        gk.append([bf16_from_bits(kb[l], dev) for l in range(L)])
        gv.append([bf16_from_bits(vb[l], dev) for l in range(L)])
        grf.append(to_dev(rf, dev))
        kv, ak = _inplace(gk[c], gv[c], caps[c], err, alive)
        kvs.append(kv)
        arr_k.append(ak)
    tail = torch.tensor([(R + 1) * C], dtype=torch.int64, device=dev)
    phase_d = to_dev(frame_t.copy(), dev)
    th_d, ft_d = to_dev(theta, dev), to_dev(frame_t, dev)
    ws = torch.empty(dp.dp_rope_workspace_bytes(n_frames, NPAIRS) // 4 + 4, dtype=torch.float32,
                     device=dev)

    # ---- oracle: the same ring layout, and the out-of-place rollout per class ----
    ok_ = [np.zeros((L, caps[c], HC, D), np.uint16) for c in (0, 1)]
    ov_ = [np.zeros((L, caps[c], HC, D), np.uint16) for c in (0, 1)]
    orf = [np.full(caps[c], -1, np.int32) for c in (0, 1)]
    for c in (0, 1):
        ok_[c][:, :(R + 1) * C], ov_[c][:, :(R + 1) * C] = by_class(init_k, c), by_class(init_v, c)
        orf[c][:(R + 1) * C] = init_rf
    otail, ophase = (R + 1) * C, frame_t.copy()
    pk = [by_class(init_k, c) for c in (0, 1)]
    pv = [by_class(init_v, c) for c in (0, 1)]
    prf = [init_rf.copy(), init_rf.copy()]
    pphase = frame_t.copy()

    for s in range(STEPS):
        x0, xf, k_new, v_new = draws[s]
        slot = s % R
        sb = C + slot * C
        q0 = float((R + 1 + s) * F)
        c_new = R + 1 + s
        new_rf = (c_new * F + np.arange(C) // TPF).astype(np.int32)
        # GPU: the leaving chunk's shared mask, appended to the dynamic buffers only
        keep = torch.empty(C, dtype=torch.uint8, device=dev)
        dp.dp_score_mask(to_dev(x0, dev), to_dev(xf, dev), 16, 16,
                         dp.make_policy(C, 0, 0, 0, C, 0.1), None, keep)
        idx = torch.empty(C, dtype=torch.int32, device=dev)
        nk = torch.zeros(1, dtype=torch.int64, device=dev)
        wsc = torch.empty(dp.dp_compact_workspace_bytes(C) // 4, dtype=torch.int32, device=dev)
        dp.dp_compact_index(keep, C, idx, nk, None, None, wsc)
        dp.dp_append_kept(kvs[1], sb, C, idx, nk, tail, grf[1])
        grf[0][sb:sb + C] = -1                            # the static class drops the chunk
        rope = dp.make_rope(th_d, ft_d, phase_d, q0, KNEE, 1.0 / FACTOR)
        dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws)
        for c in (0, 1):                                  # sinks of both classes
            dp.dp_rope_apply(arr_k[c], L, HC, D, dp.DP_BF16, 0, C, None, grf[c], rope, ws)
        dp.dp_rope_apply(arr_k[1], L, HC, D, dp.DP_BF16, C + R * C, caps[1], tail, grf[1],
                         rope, ws)                        # dynamic history
        for c in (0, 1):                                  # the new chunk into the freed slot
            kc, vc = by_class(k_new, c), by_class(v_new, c)
            for l in range(L):
                gk[c][l][sb:sb + C] = bf16_from_bits(kc[l], dev)
                gv[c][l][sb:sb + C] = bf16_from_bits(vc[l], dev)
            grf[c][sb:sb + C] = torch.from_numpy(new_rf).to(dev)
        torch.cuda.synchronize()
        assert err.item() == 0, s

        # oracle ring layout
        ell = oracle.score_f32(x0, xf)
        widx = oracle.compact(oracle.mask(ell, C, 0, 0, 0, C, 0.1))
        otail_new = oracle.append_kept(ok_[1], sb, C, widx, otail, orf[1])
        oracle.append_kept(ov_[1], sb, C, widx, otail, None)
        otail = otail_new
        orf[0][sb:sb + C] = -1
        tables = oracle.rope_frames(frame_t, ophase, q0, KNEE, np.float32(1.0 / FACTOR), theta)
        ophase = tables[3]
        for c in (0, 1):
            n_vis = otail if c == 1 else caps[0]
            for l in range(L):
                _rope_valid(ok_[c][l][:n_vis], orf[c][:n_vis], tables)
            ok_[c][:, sb:sb + C] = by_class(k_new, c)
            ov_[c][:, sb:sb + C] = by_class(v_new, c)
            orf[c][sb:sb + C] = new_rf
        assert tail.item() == otail, s
        assert np.array_equal(phase_d.cpu().numpy(), ophase), s
        for c in (0, 1):
            assert np.array_equal(grf[c].cpu().numpy(), orf[c]), (s, c)
            for l in range(L):
                assert np.array_equal(bits(gv[c][l]), ov_[c][l]), (s, c, l)
                good, worst, _ = keys_close(bits(gk[c][l]), ok_[c][l], 2e-2)
                assert good, (s, c, l, worst)

        # oracle out-of-place rollout per class: static heads Streaming, dynamic
        # heads the shared mask, over the class's whole cache
        T = pk[1].shape[1]
        scored = T - (W + 1) * C
        keeps = [oracle.mask(None, pk[0].shape[1], C, W * C, C, 0, 0.1, streaming=True),
                 oracle.mask(ell, T, C, W * C, scored, C, 0.1)]
        tables_p = oracle.rope_frames(frame_t, pphase, q0, KNEE, np.float32(1.0 / FACTOR), theta)
        pphase = tables_p[3]
        for c in (0, 1):
            pidx = oracle.compact(keeps[c])
            if s == 0:
                # the first eviction is the HS gather of the token-major cache
                lists = [oracle.compact(keeps[0]), oracle.compact(keeps[1])]
                off = oracle.hs_offsets(head_class, np.array([len(x) for x in lists]))
                packed = np.zeros((int(off[-1]), D), np.uint16)
                ph = np.zeros((int(off[-1]), D), np.uint16)
                for l in range(L):
                    oracle.hs_gather_layer(init_k[l], l, head_class, lists, off, packed)
                    oracle.hs_gather_layer(init_v[l], l, head_class, lists, off, ph)
                hrf = np.concatenate([init_rf[lists[head_class[l, h]]] for l in range(L)
                                      for h in range(H)]).astype(np.int32)
                oracle.rope_headrows(packed, hrf, 0, tables_p)
            pk[c] = oracle.gather(pk[c], pidx)
            pv[c] = oracle.gather(pv[c], pidx)
            prf[c] = oracle.gather_i32(prf[c], pidx)
            for l in range(L):
                oracle.rope_rows(pk[c][l], prf[c], 0, tables_p)
            if s == 0:
                for l in range(L):
                    for r, h in enumerate(heads[c][l]):
                        a, b = off[l * H + h], off[l * H + h + 1]
                        assert np.array_equal(packed[a:b], pk[c][l][:, r]), (c, l, h)
                        assert np.array_equal(ph[a:b], pv[c][l][:, r]), (c, l, h)
            pk[c] = np.concatenate([pk[c], by_class(k_new, c)], axis=1)
            pv[c] = np.concatenate([pv[c], by_class(v_new, c)], axis=1)
            prf[c] = np.concatenate([prf[c], new_rf])

    # head by head, each class's ring rows are the out-of-place rows (another order)
    for c in (0, 1):
        n_vis = otail if c == 1 else caps[0]
        live = np.flatnonzero(orf[c][:n_vis] >= 0)
        assert live.shape[0] == pk[c].shape[1], c
        for l in range(L):
            for r in range(HC):
                ring = _canon(ok_[c][l][live, r], ov_[c][l][live, r], orf[c][live])
                flat = _canon(pk[c][l][:, r], pv[c][l][:, r], prf[c])
                assert np.array_equal(ring, flat), (c, l, r)

    # attention of a new chunk's queries: per class buffer on the GPU, against
    # the oracle over the out-of-place rows
    q_all = random_bf16_bits(rng, (C, H, D))
    rows = np.arange(C)
    for c in (0, 1):
        n_kv = int(tail.item()) if c == 1 else caps[0]
        for l in range(L):
            qc = np.ascontiguousarray(q_all[:, heads[c][l]])
            o = torch.empty((C, HC, D), dtype=torch.bfloat16, device=dev)
            n_dev = torch.tensor([n_kv], dtype=torch.int64, device=dev)
            dp.dp_attention(bf16_from_bits(qc, dev), gk[c][l], gv[c][l], o, C, caps[c], n_dev, HC,
                            D, dp.DP_BF16, 1.0 / np.sqrt(D))
            torch.cuda.synchronize()
            want = oracle.attention(qc, np.ascontiguousarray(pk[c][l]),
                                    np.ascontiguousarray(pv[c][l]), rows)
            got = o.float().cpu().numpy().astype(np.float64)
            assert np.allclose(got, want, atol=ATOL, rtol=RTOL), \
                (c, l, float(np.max(np.abs(got - want))))
    print("HS ring rollout: %d steps, dynamic tail %d, static %d rows" % (STEPS, otail, caps[0]))
