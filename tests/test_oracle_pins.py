"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks one oracle step against a closed form, an invariant the
DeCoPrune page states, a library routine, or brute force, chosen so that a
plausible slip (a dropped term, a wrong sign, an off-by-one, a transposed
index) fails at least one of them.  Page sections cited:
[DeCoPrune page, 어떻게 동작하나] score, mask, gather;
[DeCoPrune page, 무엇과 다른가] RoPE re-index, HS;
[DeCoPrune page, 어떻게 쓰나] pruning ratio.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import dpsynth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# --------------------------------------------------------------------------
# Score: l = (1/d) ||x0_hat - x_final||^2
# --------------------------------------------------------------------------
@pytest.mark.parametrize("d", [1, 2, 3, 5, 12, 16, 48, 64, 100, 256])
def test_score_equal_inputs_is_positive_zero(d):
    x = np.random.default_rng(d).standard_normal((7, d)).astype(np.float32)
    ell = oracle.score_f32(x, x.copy())
    assert np.all(ell == 0) and not np.any(np.signbit(ell))


@pytest.mark.parametrize("d", [1, 3, 16, 48, 64, 200])
def test_score_single_channel_closed_form(d):
    # one nonzero channel at every position c: l = RN32(e*e) / d
    rng = np.random.default_rng(1)
    for c in range(d):
        e = np.float32(rng.uniform(0.1, 3.0))
        a = np.zeros((1, d), np.float32)
        a[0, c] = e
        b = np.zeros((1, d), np.float32)
        want = np.float32(float(np.float32(e * e)) / d)
        assert oracle.score_f32(a, b)[0] == want, c


@pytest.mark.parametrize("d", [4, 5, 12, 16, 48, 64, 100, 256])
def test_score_integer_inputs_exact(d):
    # small integers: every square and partial sum is exact in fp32, so the
    # result is the exact rational sum/d rounded once to fp32
    rng = np.random.default_rng(d + 100)
    a = rng.integers(-20, 21, size=(50, d)).astype(np.float32)
    b = rng.integers(-20, 21, size=(50, d)).astype(np.float32)
    ell = oracle.score_f32(a, b)
    for i in range(50):
        s = sum(int(x) ** 2 for x in (a[i].astype(np.int64) - b[i].astype(np.int64)))
        assert ell[i] == np.float32(Fraction(s, d).numerator / Fraction(s, d).denominator), i


def test_score_row_stride_reads_only_d_channels():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((9, 40)).astype(np.float32)
    b = rng.standard_normal((9, 40)).astype(np.float32)
    full = oracle.score_f32(a[:, :24].copy(), b[:, :24].copy())
    strided = oracle.score_f32(a, b, d=24)
    assert np.array_equal(full, strided)


@pytest.mark.parametrize("d", [16, 48, 64, 256])
def test_score_f32_within_pairwise_error_bound_of_f64(d):
    rng = np.random.default_rng(d)
    x0 = rng.standard_normal((4000, d)).astype(np.float32)
    xf = (x0 + rng.uniform(0.01, 2.0, (4000, 1)) * rng.standard_normal((4000, d))).astype(np.float32)
    l32 = oracle.score_f32(x0, xf).astype(np.float64)
    e = x0.astype(np.float64) - xf.astype(np.float64)
    l64 = (e * e).sum(axis=1) / d           # brute force, float64 (numpy)
    # pairwise summation: |err| <= (log2 P + 3) u * sum|q|, u = 2^-24
    P = 1 << (d - 1).bit_length()
    bound = (np.log2(P) + 3) * 2.0 ** -24 * l64
    assert np.all(np.abs(l32 - l64) <= bound + 1e-45)
    assert np.allclose(oracle.score_f64(x0, xf), l64, rtol=1e-14, atol=0)


def test_score_mean_is_sigma_squared_for_non_power_of_two_d():
    # E[l] = sigma^2 when x0_hat = x_final + sigma N(0,1): dividing by the
    # padded width instead of d, or dropping channels, would miss by >20%.
    d, n, sigma = 48, 40000, 0.5
    rng = np.random.default_rng(7)
    xf = rng.standard_normal((n, d)).astype(np.float32)
    x0 = (xf + sigma * rng.standard_normal((n, d))).astype(np.float32)
    m = oracle.score_f32(x0, xf).astype(np.float64).mean()
    assert abs(m - sigma ** 2) < 0.01 * sigma ** 2


# --------------------------------------------------------------------------
# Mask
# --------------------------------------------------------------------------
def _policy_rows(T=600, sink=64, window=128, sb=64, ns=300):
    return dict(seq_len=T, sink_len=sink, window_len=window, scored_begin=sb, n_scored=ns)


def test_mask_gamma_zero_keeps_everything():
    rng = np.random.default_rng(0)
    ell = np.abs(rng.standard_normal(300)).astype(np.float32)
    ell[::7] = 0.0
    keep = oracle.mask(ell, gamma=0.0, **_policy_rows())
    assert keep.dtype == np.uint8 and np.all(keep == 1)


def test_mask_reversed_is_complement_on_scored_rows():
    rng = np.random.default_rng(1)
    ell = np.abs(rng.standard_normal(300)).astype(np.float32) * 0.2
    ell[5] = np.nan
    p = _policy_rows()
    a = oracle.mask(ell, gamma=0.1, **p)
    b = oracle.mask(ell, gamma=0.1, reversed=True, **p)
    s = slice(64, 364)
    assert np.array_equal(a[s] ^ b[s], np.ones(300, np.uint8))
    outside = np.r_[0:64, 364:600]
    assert np.array_equal(a[outside], b[outside])
    assert a[64 + 5] == 0 and b[64 + 5] == 1        # NaN: dropped, reversed keeps it


def test_mask_threshold_tie_and_count():
    g = np.float32(0.1)
    ell = np.array([g, np.nextafter(g, np.float32(0)), np.nextafter(g, np.float32(1)), 0, np.inf],
                   np.float32)
    keep = oracle.mask(ell, seq_len=5, sink_len=0, window_len=0, scored_begin=0, n_scored=5,
                       gamma=g)
    assert keep.tolist() == [1, 0, 1, 0, 1]
    rng = np.random.default_rng(3)
    ell = (rng.random(300) * 0.2).astype(np.float32)
    keep = oracle.mask(ell, gamma=0.1, **_policy_rows())
    assert keep[64:364].sum() == np.count_nonzero(ell >= np.float32(0.1))


def test_mask_sink_window_and_history_rows():
    rng = np.random.default_rng(2)
    ell = np.zeros(200, np.float32)          # nothing passes gamma
    p = dict(seq_len=1000, sink_len=100, window_len=300, scored_begin=400, n_scored=200)
    keep = oracle.mask(ell, gamma=0.1, **p)
    assert np.all(keep[:100] == 1) and np.all(keep[700:] == 1)
    assert np.all(keep[400:600] == 0)
    assert np.all(keep[100:400] == 1) and np.all(keep[600:700] == 1)   # earlier history kept
    st = oracle.mask(None, gamma=0.1, streaming=True, **p)
    assert np.array_equal(st, np.r_[np.ones(100), np.zeros(600), np.ones(300)].astype(np.uint8))
    # gamma = +inf with the whole middle scored is the streaming mask
    q = dict(seq_len=1000, sink_len=100, window_len=300, scored_begin=100, n_scored=600)
    ell = rng.random(600).astype(np.float32)
    assert np.array_equal(oracle.mask(ell, gamma=np.inf, **q),
                          oracle.mask(None, gamma=0.1, streaming=True, **q))


# --------------------------------------------------------------------------
# Compaction and gather
# --------------------------------------------------------------------------
@pytest.mark.parametrize("T,rate", [(0, 0.5), (1, 1.0), (1, 0.0), (1000, 0.0), (1000, 1.0),
                                    (4097, 0.15), (70001, 0.5)])
def test_compact_is_flatnonzero(T, rate):
    keep = (np.random.default_rng(T).random(T) < rate).astype(np.uint8)
    idx = oracle.compact(keep)
    assert idx.dtype == np.int32
    assert np.array_equal(idx, np.flatnonzero(keep))
    assert idx.shape[0] == int(keep.sum())


@pytest.mark.parametrize("dtype", [np.float32, np.uint16, np.int8])
def test_gather_is_numpy_take(dtype):
    rng = np.random.default_rng(4)
    src = rng.integers(0, 2 ** 8 if dtype == np.int8 else 2 ** 15, size=(3, 50, 2, 8)).astype(dtype)
    keep = (rng.random(50) < 0.4).astype(np.uint8)
    keep[:5] = 1
    idx = np.flatnonzero(keep)
    out = oracle.gather(src, idx)
    assert np.array_equal(out.view(np.uint8), src[:, idx].view(np.uint8))
    assert np.array_equal(out[:, :5], src[:, :5])       # sink rows bit-identical
    rf = rng.integers(0, 9, 50).astype(np.int32)
    assert np.array_equal(oracle.gather_i32(rf, idx), rf[idx])


def test_append_kept_is_numpy_indexing():
    rng = np.random.default_rng(15)
    L, cap, H, D = 2, 200, 3, 8
    buf = rng.integers(0, 2 ** 15, size=(L, cap, H, D)).astype(np.uint16)
    rf = rng.integers(0, 50, cap).astype(np.int32)
    before, rf0 = buf.copy(), rf.copy()
    slot_begin, slot_rows, tail = 10, 40, 120
    idx = np.flatnonzero(rng.random(slot_rows) < 0.4).astype(np.int32)
    t2 = oracle.append_kept(buf, slot_begin, slot_rows, idx, tail, rf)
    n = idx.shape[0]
    assert t2 == tail + n
    assert np.array_equal(buf[:, tail:tail + n], before[:, slot_begin + idx])
    untouched = np.ones(cap, bool)
    untouched[tail:tail + n] = False
    assert np.array_equal(buf[:, untouched], before[:, untouched])
    assert np.array_equal(rf[tail:tail + n], rf0[slot_begin + idx])
    assert np.all(rf[slot_begin:slot_begin + slot_rows] == -1)
    # refused: past the capacity, or overlapping the slot -- nothing changes
    b2, r2 = buf.copy(), rf.copy()
    assert oracle.append_kept(buf, slot_begin, slot_rows, idx, cap - n + 1, rf) == -1
    assert oracle.append_kept(buf, slot_begin, slot_rows, idx, slot_begin + 5, rf) == -1
    assert np.array_equal(buf, b2) and np.array_equal(rf, r2)


# --------------------------------------------------------------------------
# RoPE re-index
# --------------------------------------------------------------------------
def _t_new_exact(q0, knee, c, t):
    D = Fraction(q0) - Fraction(t)
    g = D if D <= knee else Fraction(knee) + (D - Fraction(knee)) / c
    return Fraction(q0) - g


def test_reindex_positions_tiny_closed_form():
    # q0 = 8, knee 2, factor 4, frames 0..7: t~ = q0 - (knee + (D - knee)/4)
    t = np.arange(8, dtype=np.float32)
    delta, _, _, ph = oracle.rope_frames(t, t, 8.0, 2.0, 0.25, dpsynth.rope_theta(8))
    assert ph.tolist() == [4.5, 4.75, 5.0, 5.25, 5.5, 5.75, 6.0, 7.0]
    assert delta.tolist() == [4.5, 3.75, 3.0, 2.25, 1.5, 0.75, 0.0, 0.0]


def test_reindex_positions_minute_history_closed_form():
    # 240 frames, q0 = 240, knee 12 (the 3-chunk window), factor 8
    t = np.arange(240, dtype=np.float32)
    _, _, _, ph = oracle.rope_frames(t, t, 240.0, 12.0, 0.125, dpsynth.rope_theta(44))
    want = [float(_t_new_exact(240, 12, 8, i)) for i in range(240)]
    assert ph.tolist() == want
    assert ph[0] == 199.5 and ph[227] == 227.875 and np.array_equal(ph[228:], t[228:])
    assert np.all(np.diff(ph) > 0)        # order of keys is preserved


def test_reindex_factor_one_is_identity():
    rng = np.random.default_rng(8)
    k = rng.standard_normal((30, 2, 64)).astype(np.float32)
    rf = (np.arange(30) // 4).astype(np.int32)
    t = np.arange(8, dtype=np.float32)
    tab = oracle.rope_frames(t, t, 8.0, 2.0, 1.0, dpsynth.rope_theta(8))
    assert np.all(tab[0] == 0)
    k2 = oracle.rope_rows(k.copy(), rf, 0, tab)
    assert np.array_equal(k2.view(np.uint32), k.view(np.uint32))


def _rot_f64(k, rf, pair_begin, theta, delta):
    """Independent float64 complex-multiplication form of the rotation."""
    out = k.astype(np.float64).copy()
    npairs = theta.shape[0]
    lo, hi = 2 * pair_begin, 2 * (pair_begin + npairs)
    z = out[..., lo:hi:2] + 1j * out[..., lo + 1:hi:2]
    ang = delta[rf][:, None, None] * theta.astype(np.float64)[None, None, :]
    z = z * np.exp(1j * ang)
    out[..., lo:hi:2] = z.real
    out[..., lo + 1:hi:2] = z.imag
    return out


@pytest.mark.parametrize("pair_begin,npairs", [(0, 8), (4, 12), (0, 32)])
def test_reindex_rotation_matches_complex_multiplication(pair_begin, npairs):
    rng = np.random.default_rng(npairs)
    k = rng.standard_normal((64, 2, 64)).astype(np.float32)
    rf = (np.arange(64) // 8).astype(np.int32)
    theta = dpsynth.rope_theta(npairs)
    t = np.arange(8, dtype=np.float32)
    tab = oracle.rope_frames(t, t, 8.0, 2.0, 0.25, theta)
    got = oracle.rope_rows(k.copy(), rf, pair_begin, tab).astype(np.float64)
    want = _rot_f64(k, rf, pair_begin, theta, tab[0].astype(np.float64))
    assert np.max(np.abs(got - want)) < 2e-6
    # dims outside the temporal block are untouched bit for bit
    mask = np.ones(64, bool)
    mask[2 * pair_begin: 2 * (pair_begin + npairs)] = False
    assert np.array_equal(got[..., mask], k.astype(np.float64)[..., mask])
    # window frames (delta 0) are untouched bit for bit
    assert np.array_equal(got[48:], k[48:].astype(np.float64))


def test_reindex_relative_position_identity():
    # After the re-index, a key of frame t scores against a query at q0 as if
    # it sat at offset g(q0 - t): <R(q0) u, k'> = <R(g) u, v>, with k = R(t) v.
    rng = np.random.default_rng(11)
    npairs, q0, knee, c = 16, 20.0, 4.0, 3.0
    theta = dpsynth.rope_theta(npairs)
    th = theta.astype(np.float64)
    frames = np.arange(20, dtype=np.float32)
    v = rng.standard_normal((20, 2 * npairs))
    vz = v[:, 0::2] + 1j * v[:, 1::2]
    kz = vz * np.exp(1j * np.outer(frames.astype(np.float64), th))
    k = np.empty((20, 1, 2 * npairs), np.float32)
    k[:, 0, 0::2], k[:, 0, 1::2] = kz.real, kz.imag
    tab = oracle.rope_frames(frames, frames, q0, knee, np.float32(1.0 / c), theta)
    k2 = oracle.rope_rows(k.copy(), np.arange(20, dtype=np.int32), 0, tab).astype(np.float64)
    k2z = k2[:, 0, 0::2] + 1j * k2[:, 0, 1::2]
    u = rng.standard_normal(npairs) + 1j * rng.standard_normal(npairs)
    for f in range(20):
        g = float(Fraction(q0) - _t_new_exact(q0, knee, Fraction(c), f))
        lhs = np.real(np.vdot(u * np.exp(1j * th * q0), k2z[f]))
        rhs = np.real(np.vdot(u * np.exp(1j * th * g), vz[f]))
        assert abs(lhs - rhs) < 1e-4 * (1 + abs(rhs)), f


def test_steady_state_phase_step_is_uniform():
    """Rollout of the one-minute setup (4 frames per chunk, knee 12, factor 8):
    once a frame is past the knee before and after a step, its phase step is
    F (1 - 1/c) = 3.5 frames exactly, whatever its frame; frames crossing the
    knee step by less, window frames not at all (exact rationals)."""
    F, knee, c = 4, 12, 8
    theta = dpsynth.rope_theta(44)
    t = np.arange(240, dtype=np.float32)
    ph = t.copy()
    for step in range(1, 20):
        q0 = 4 * F + F * step                       # the chunk about to be generated
        prev_q0 = q0 - F
        visible = t < q0
        delta, cos_t, sin_t, ph_new = oracle.rope_frames(t, ph, float(q0), float(knee),
                                                         np.float32(1.0 / c), theta)
        for f in np.flatnonzero(visible):
            before = prev_q0 - f > knee and step > 1
            after = q0 - f > knee
            d = Fraction(float(delta[f]))
            assert d == _t_new_exact(q0, knee, c, int(f)) - Fraction(float(ph[f])), (step, f)
            if before and after:
                assert d == Fraction(F) * (1 - Fraction(1, c)), (step, f)
            elif not after:
                assert d == 0, (step, f)
            else:                                   # first step past the knee
                assert d > 0, (step, f)
        # the uniform tables equal the per-frame tables of every such frame
        steady = [f for f in np.flatnonzero(visible)
                  if step > 1 and prev_q0 - f > knee and q0 - f > knee]
        if steady:
            _, cu, su, _ = oracle.rope_uniform(theta, 3.5)
            for f in steady:
                assert np.array_equal(cos_t[f].view(np.uint32), cu[0].view(np.uint32))
                assert np.array_equal(sin_t[f].view(np.uint32), su[0].view(np.uint32))
        ph = ph_new


def test_compressed_axis_decomposition():
    """Past the knee, t~ = q0 - knee - (q0 - t - knee)/c splits into a part of
    the key alone, t/c, and a part the same for every such key,
    A = (1 - 1/c)(q0 - knee) (exact rationals), so keys can be kept at phase t/c
    and the query rotated back by A; within the knee t~ = t."""
    for q0, knee, c in ((240, 12, 8), (20, 12, 8), (8, 2, 4), (41, 5, 3)):
        A = (1 - Fraction(1, c)) * (q0 - knee)
        for t in range(q0):
            tn = _t_new_exact(q0, knee, Fraction(c), t)
            if q0 - t > knee:
                assert tn == Fraction(t, c) + A, (q0, t)
            else:
                assert tn == t, (q0, t)


def test_compressed_axis_tables():
    """The compressed-axis frame tables: within the knee they are the page's
    tables bit for bit; past the knee the phase is t/c and adding the common
    term A gives the page's t~ exactly (multiples of 1/c are exact in fp32);
    a frame already at t/c stays (delta 0); the rotation the table encodes
    is that of the fp64 angle theta_j (t/c - t)."""
    theta = dpsynth.rope_theta(44)
    for q0, knee, c in ((240.0, 12.0, 8.0), (20.0, 12.0, 8.0), (8.0, 4.0, 4.0)):
        t = np.arange(int(q0) + 4, dtype=np.float32)
        page = oracle.rope_frames(t, t, q0, knee, np.float32(1 / c), theta)
        comp = oracle.rope_frames(t, t, q0, knee, np.float32(1 / c), theta, compressed=True)
        inside = q0 - t <= knee
        for a, b in zip(page[:3], comp[:3]):
            assert np.array_equal(a[inside], b[inside])
        A = (1 - 1 / c) * (q0 - knee)
        past = ~inside
        assert np.array_equal(comp[3][past].astype(np.float64), t[past] / c)
        assert np.array_equal(comp[3][past].astype(np.float64) + A, page[3][past].astype(np.float64))
        assert np.array_equal(comp[0][past].astype(np.float64), t[past] / c - t[past])
        ang = np.float32(theta[None, :]) * comp[0][:, None]
        assert np.array_equal(comp[1], np.cos(ang.astype(np.float64)).astype(np.float32))
        assert np.array_equal(comp[2], np.sin(ang.astype(np.float64)).astype(np.float32))
        again = oracle.rope_frames(t, comp[3], q0 + 4, knee, np.float32(1 / c), theta,
                                   compressed=True)
        still = q0 - t > knee                       # past the knee before and after
        assert np.all(again[0][still] == 0) and np.all(again[1][still] == 1)
        assert np.all(again[2][still] == 0)


def test_rope_rows_f64_invariants():
    """The float64 re-index: rotations compose, pair norms are kept, and it
    agrees with the fp32-storage re-index within fp32 rounding."""
    rng = np.random.default_rng(22)
    theta = dpsynth.rope_theta(12)
    k = rng.standard_normal((30, 2, 32))
    rf = (np.arange(30) // 3).astype(np.int32)
    d1 = rng.uniform(-20, 20, 10)
    d2 = rng.uniform(-20, 20, 10)
    a = oracle.rope_rows_f64(oracle.rope_rows_f64(k.copy(), rf, 2, d1, theta), rf, 2, d2, theta)
    b = oracle.rope_rows_f64(k.copy(), rf, 2, d1 + d2, theta)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    norm = lambda x: x[..., 4:28:2] ** 2 + x[..., 5:28:2] ** 2
    assert np.allclose(norm(a), norm(k), rtol=1e-12, atol=1e-12)
    assert np.array_equal(a[..., :4], k[..., :4]) and np.array_equal(a[..., 28:], k[..., 28:])
    tab = oracle.rope_uniform(theta, np.float32(3.5))
    k32 = k.astype(np.float32)
    g = oracle.rope_rows(k32.copy(), np.zeros(30, np.int32), 2, tab).astype(np.float64)
    e = oracle.rope_rows_f64(k32.astype(np.float64), np.zeros(30, np.int32), 2,
                             np.array([3.5]), theta.astype(np.float32).astype(np.float64))
    assert np.max(np.abs(g - e)) < 1e-5


def test_uniform_shift_matches_per_frame_rows():
    """A uniform step over rows of many frames is the per-frame re-index with
    every frame's step equal to it (bitwise), and the float64 rotation."""
    rng = np.random.default_rng(13)
    theta = dpsynth.rope_theta(12)
    k = rng.standard_normal((40, 3, 64)).astype(np.float32)
    tab = oracle.rope_uniform(theta, 3.5)
    got = oracle.rope_rows(k.copy(), np.zeros(40, np.int32), 2, tab)
    want = _rot_f64(k, np.zeros(40, np.int64), 2, theta, np.array([3.5]))
    assert np.max(np.abs(got - want)) < 2e-6
    per = (np.full(10, 3.5, np.float32),) + tuple(
        np.repeat(x, 10, axis=0) for x in oracle.rope_uniform(theta, 3.5)[1:3]) + (None,)
    got2 = oracle.rope_rows(k.copy(), (np.arange(40) // 4).astype(np.int32), 2, per)
    assert np.array_equal(got.view(np.uint32), got2.view(np.uint32))


def test_reindex_rotations_compose():
    # two re-index passes (q0 then q0') equal one pass to q0' from the start
    rng = np.random.default_rng(12)
    theta = dpsynth.rope_theta(44)
    t = np.arange(24, dtype=np.float32)
    k = rng.standard_normal((24, 3, 128)).astype(np.float32)
    rf = np.arange(24, dtype=np.int32)
    tab1 = oracle.rope_frames(t, t, 16.0, 12.0, 0.125, theta)
    k1 = oracle.rope_rows(k.copy(), rf, 0, tab1)
    tab2 = oracle.rope_frames(t, tab1[3], 24.0, 12.0, 0.125, theta)
    k12 = oracle.rope_rows(k1, rf, 0, tab2)
    tab3 = oracle.rope_frames(t, t, 24.0, 12.0, 0.125, theta)
    k3 = oracle.rope_rows(k.copy(), rf, 0, tab3)
    assert np.array_equal(tab2[3], tab3[3])
    assert np.max(np.abs(k12 - k3)) < 1e-5


def test_reindex_bf16_storage_rounds_to_nearest_even():
    # torch's fp32 -> bf16 conversion (round to nearest, ties to even) is the
    # reference; the sample is large enough to contain exact ties
    import torch
    rng = np.random.default_rng(13)
    kb = torch.from_numpy(rng.standard_normal((6000, 2, 64)).astype(np.float32) * 3).to(torch.bfloat16)
    k16 = kb.view(torch.int16).numpy().view(np.uint16).copy()
    k32 = kb.to(torch.float32).numpy().copy()
    rf = (np.arange(6000) // 1000).astype(np.int32)
    t = np.arange(8, dtype=np.float32)
    tab = oracle.rope_frames(t, t, 8.0, 2.0, 0.25, dpsynth.rope_theta(32))
    r32 = oracle.rope_rows(k32, rf, 0, tab)
    r16 = oracle.rope_rows(k16, rf, 0, tab)
    ties = np.count_nonzero((r32.view(np.uint32) & 0xFFFF) == 0x8000)
    assert ties > 0
    want = torch.from_numpy(r32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(r16, want)


# --------------------------------------------------------------------------
# DeCoPrune-HS
# --------------------------------------------------------------------------
def test_hs_offsets_and_heads():
    rng = np.random.default_rng(14)
    L, H, T, D = 3, 6, 200, 8
    src = rng.integers(0, 2 ** 15, size=(L, T, H, D)).astype(np.uint16)
    cls = rng.integers(0, 2, size=(L, H)).astype(np.uint8)
    ell = rng.random(120).astype(np.float32) * 0.2
    p = dict(seq_len=T, sink_len=20, window_len=60, scored_begin=20, n_scored=120)
    stat = oracle.compact(oracle.mask(None, gamma=0.1, streaming=True, **p))
    dyn = oracle.compact(oracle.mask(ell, gamma=0.1, **p))
    lens = np.array([len(stat), len(dyn)], np.int64)
    off = oracle.hs_offsets(cls, lens)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(lens[cls.ravel()])]))
    out = np.zeros((off[-1], D), np.uint16)
    for l in range(L):
        oracle.hs_gather_layer(src[l], l, cls, [stat, dyn], off, out)
    for l in range(L):
        for h in range(H):
            i = l * H + h
            rows = stat if cls[l, h] == 0 else dyn
            assert np.array_equal(out[off[i]:off[i + 1]], src[l][rows, h]), (l, h)


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_rope_headrows_equals_rope_rows_and_complex_rotation(dtype):
    """The re-index of a per-head packed cache (DeCoPrune-HS, section 무엇과
    다른가: the ragged per-head runs are re-indexed like the token-major
    cache): on the [rows * H, D] view of a token-major cache, with every head
    row carrying its token's frame, it equals rope_rows bit for bit; with a
    frame of its own per head row (as the packed HS runs have) each head row
    is its frame's float64 complex rotation (fp32 keys), dims outside the
    temporal block and rows of frames with delta 0 stay bit for bit."""
    rng = np.random.default_rng(31)
    rows, H, D, npairs, pb = 48, 3, 64, 12, 2
    theta = dpsynth.rope_theta(npairs)
    t = np.arange(10, dtype=np.float32)
    tab = oracle.rope_frames(t, t, 10.0, 2.0, 0.25, theta)     # frames 8, 9: delta 0
    assert np.unique(tab[0]).shape[0] == 9
    if dtype == np.float32:
        k = rng.standard_normal((rows, H, D)).astype(np.float32)
    else:
        k = _bf16(rng, (rows, H, D), 2.0)
    rf = rng.permutation(np.arange(rows) % 10).astype(np.int32)
    tok = oracle.rope_rows(k.copy(), rf, pb, tab)
    flat = oracle.rope_headrows(k.reshape(rows * H, D).copy(), np.repeat(rf, H), pb, tab)
    assert np.array_equal(flat.reshape(rows, H, D), tok)
    # a frame per head row
    rfh = rng.integers(0, 10, rows * H).astype(np.int32)
    got = oracle.rope_headrows(k.reshape(rows * H, D).copy(), rfh, pb, tab)
    src = k.reshape(rows * H, D)
    keep_dims = np.ones(D, bool)
    keep_dims[2 * pb:2 * (pb + npairs)] = False
    assert np.array_equal(got[:, keep_dims], src[:, keep_dims])
    still = tab[0][rfh] == 0
    assert np.array_equal(got[still], src[still])
    if dtype == np.float32:
        want = _rot_f64(src[:, None, :], rfh, pb, theta, tab[0].astype(np.float64))[:, 0]
        assert np.max(np.abs(got.astype(np.float64) - want)) < 2e-6
    else:
        want = _rot_f64(_f(src)[:, None, :], rfh, pb, theta, tab[0].astype(np.float64))[:, 0]
        # one bf16 rounding of each rotated element (half an ulp: at most 2^-8
        # relative) on top of the fp32 products and sums (a few 2^-24 of the pair)
        err = np.abs(_f(got) - want)
        assert np.all(err <= np.abs(want) * 2.0 ** -8 + 4 * 2.0 ** -24 * np.abs(_f(src)).max())


# --------------------------------------------------------------------------
# Attention over the retained cache
# --------------------------------------------------------------------------
def _bf16(rng, shape, scale=1.0):
    import torch
    x = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16).copy()


def _f(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_attention_matches_numpy_softmax():
    rng = np.random.default_rng(16)
    nq, nk, H, D = 7, 300, 3, 32
    q, k, v = _bf16(rng, (nq, H, D)), _bf16(rng, (nk, H, D)), _bf16(rng, (nk, H, D))
    rows = np.array([0, 3, 6])
    got = oracle.attention(q, k, v, rows, n_kv=250)
    qf, kf, vf = _f(q), _f(k), _f(v)
    for a, i in enumerate(rows):
        for h in range(H):
            s = kf[:250, h] @ qf[i, h] / np.sqrt(D)          # numpy float64 reference
            p = np.exp(s - s.max())
            want = (p / p.sum()) @ vf[:250, h]
            assert np.allclose(got[a, h], want, rtol=1e-12, atol=1e-13)


def test_attention_closed_forms():
    rng = np.random.default_rng(17)
    nk, H, D = 64, 2, 16
    k, v = _bf16(rng, (nk, H, D)), _bf16(rng, (nk, H, D))
    zero_q = np.zeros((1, H, D), np.uint16)
    # a zero query weights every key equally: the output is the mean of V
    got = oracle.attention(zero_q, k, v, [0])
    assert np.allclose(got[0], _f(v).mean(axis=0), rtol=1e-12, atol=1e-14)
    # a single key gives that key's value exactly
    got = oracle.attention(_bf16(rng, (1, H, D)), k, v, [0], n_kv=1)
    assert np.array_equal(got[0], _f(v)[0])
    # a query strongly aligned with one key selects its value
    q = k[5:6].copy()
    got = oracle.attention(q, k, v, [0], scale=1e4)
    assert np.allclose(got[0], _f(v)[5], atol=1e-9)


def test_attention_invariants_and_two_key_closed_form():
    """Properties that fix softmax attention without restating it: the order of
    keys does not matter; adding a vector c to every value row adds c to the
    output (the weights sum to 1); a key listed twice weighs twice; with two
    keys the weight of the first is the logistic function of the score gap."""
    rng = np.random.default_rng(21)
    nq, nk, H, D = 4, 37, 2, 16
    q, k, v = _bf16(rng, (nq, H, D)), _bf16(rng, (nk, H, D)), _bf16(rng, (nk, H, D))
    rows = np.arange(nq)
    base = oracle.attention(q, k, v, rows, scale=0.25)
    perm = rng.permutation(nk)
    assert np.allclose(oracle.attention(q, k[perm], v[perm], rows, scale=0.25), base,
                       rtol=1e-12, atol=1e-14)
    # values on a grid of eighths, so that v and v + 1/2 are both exact in bf16
    import torch
    grid = rng.integers(-32, 33, (nk, H, D)) / 8.0

    def as_bf16(x):
        t = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
        assert np.array_equal(t.float().numpy().astype(np.float64), x)
        return t.view(torch.int16).numpy().view(np.uint16)

    vg = oracle.attention(q, k, as_bf16(grid), rows, scale=0.25)
    vs = oracle.attention(q, k, as_bf16(grid + 0.5), rows, scale=0.25)
    assert np.allclose(vs, vg + 0.5, rtol=1e-12, atol=1e-12)
    # two keys: the logistic weight; listing key 0 twice adds log 2 to its score gap
    k2, v2 = k[:2].copy(), v[:2].copy()
    got = oracle.attention(q, k2, v2, rows, scale=0.25)
    qf, kf, vf2 = _f(q), _f(k2), _f(v2)
    for i in range(nq):
        for h in range(H):
            gap = 0.25 * (qf[i, h] @ kf[0, h] - qf[i, h] @ kf[1, h])
            w0 = 1.0 / (1.0 + np.exp(-gap))                  # logistic weight of key 0
            assert np.allclose(got[i, h], w0 * vf2[0, h] + (1 - w0) * vf2[1, h],
                               rtol=1e-12, atol=1e-13)
    k3 = np.concatenate([k2, k2[:1]])
    v3 = np.concatenate([v2, v2[:1]])
    got3 = oracle.attention(q, k3, v3, rows, scale=0.25)
    for i in range(nq):
        for h in range(H):
            gap = 0.25 * (qf[i, h] @ kf[0, h] - qf[i, h] @ kf[1, h]) + np.log(2.0)
            w0 = 1.0 / (1.0 + np.exp(-gap))
            assert np.allclose(got3[i, h], w0 * vf2[0, h] + (1 - w0) * vf2[1, h],
                               rtol=1e-12, atol=1e-13)


def test_attention_f64_equals_bf16_form_and_closed_forms():
    """The float64-input attention (the reference for keys that are not rounded
    to a storage type): on the exact float64 widening of bf16 inputs it is the
    bf16-input attention bit for bit (the same sums in the same order); on
    float64 inputs that no bf16 holds it satisfies the closed forms: a zero
    query gives the mean of V, one key gives its value, two keys weigh by the
    logistic function of their scaled score gap, adding c to every value row
    adds c, and the order of keys does not matter."""
    rng = np.random.default_rng(32)
    nq, nk, H, D = 5, 41, 2, 16
    q, k, v = _bf16(rng, (nq, H, D)), _bf16(rng, (nk, H, D)), _bf16(rng, (nk, H, D))
    rows = np.array([0, 2, 4])
    for scale in (None, 0.37):
        a = oracle.attention(q, k, v, rows, n_kv=33, scale=scale)
        b = oracle.attention(_f(q), _f(k), _f(v), rows, n_kv=33, scale=scale)
        assert np.array_equal(a.view(np.uint64), b.view(np.uint64))
    qd = rng.standard_normal((nq, H, D)) * 0.7
    kd = rng.standard_normal((nk, H, D)) * 0.7
    vd = rng.standard_normal((nk, H, D))
    got = oracle.attention(np.zeros((1, H, D)), kd, vd, [0])
    assert np.allclose(got[0], vd.mean(axis=0), rtol=1e-12, atol=1e-14)
    got = oracle.attention(qd, kd, vd, [1], n_kv=1)
    assert np.array_equal(got[0], vd[0])
    sc = 0.37
    got = oracle.attention(qd, kd[:2], vd[:2], np.arange(nq), scale=sc)
    for i in range(nq):
        for h in range(H):
            gap = sc * (qd[i, h] @ kd[0, h] - qd[i, h] @ kd[1, h])
            w0 = 1.0 / (1.0 + np.exp(-gap))
            assert np.allclose(got[i, h], w0 * vd[0, h] + (1 - w0) * vd[1, h],
                               rtol=1e-12, atol=1e-13)
    base = oracle.attention(qd, kd, vd, np.arange(nq), scale=sc)
    shift = rng.standard_normal(D)
    assert np.allclose(oracle.attention(qd, kd, vd + shift, np.arange(nq), scale=sc),
                       base + shift, rtol=1e-12, atol=1e-12)
    perm = rng.permutation(nk)
    assert np.allclose(oracle.attention(qd, kd[perm], vd[perm], np.arange(nq), scale=sc), base,
                       rtol=1e-12, atol=1e-14)


def test_hs_attention_per_head_runs_against_numpy():
    """Each head of the chosen layer sees exactly its own run followed by the
    chunk rows; a head with no rows gives zeros (numpy float64 softmax)."""
    rng = np.random.default_rng(18)
    L, H, D, nq, nc = 2, 4, 16, 5, 9
    lens = np.array([[3, 0, 7, 1], [0, 12, 5, 64]], np.int64)        # per (layer, head)
    off = np.concatenate([[0], np.cumsum(lens.ravel())]).astype(np.int64)
    kr, vr = _bf16(rng, (off[-1], D)), _bf16(rng, (off[-1], D))
    kc, vc = _bf16(rng, (nc, H, D)), _bf16(rng, (nc, H, D))
    q = _bf16(rng, (nq, H, D))
    rows = np.array([0, 2, 4])
    for layer in range(L):
        for chunk in (False, True):
            got = oracle.hs_attention(q, kr, vr, off, layer, rows, kc if chunk else None,
                                      vc if chunk else None, scale=0.3)
            for h in range(H):
                lo, hi = off[layer * H + h], off[layer * H + h + 1]
                kh, vh = _f(kr[lo:hi]), _f(vr[lo:hi])
                if chunk:
                    kh, vh = np.concatenate([kh, _f(kc[:, h])]), np.concatenate([vh, _f(vc[:, h])])
                for a, i in enumerate(rows):
                    if kh.shape[0] == 0:
                        assert np.all(got[a, h] == 0)
                        continue
                    sc = kh @ _f(q[i, h]) * 0.3
                    p = np.exp(sc - sc.max())
                    assert np.allclose(got[a, h], (p / p.sum()) @ vh, rtol=1e-12, atol=1e-13)


def test_hs_attention_with_shared_runs_equals_dense_attention():
    """When every head's run lists the same cache rows, the ragged attention
    is the dense attention over those rows followed by the chunk."""
    rng = np.random.default_rng(19)
    T, H, D, nq = 40, 3, 16, 6
    k, v = _bf16(rng, (T, H, D)), _bf16(rng, (T, H, D))
    q = _bf16(rng, (nq, H, D))
    keep = np.flatnonzero(rng.random(T) < 0.5)
    n = keep.shape[0]
    kr = np.concatenate([k[keep, h] for h in range(H)])             # head-major runs
    vr = np.concatenate([v[keep, h] for h in range(H)])
    off = np.arange(H + 1, dtype=np.int64) * n
    kc, vc = k[-4:], v[-4:]
    got = oracle.hs_attention(q, kr, vr, off, 0, np.arange(nq), kc, vc)
    want = oracle.attention(q, np.concatenate([k[keep], kc]), np.concatenate([v[keep], vc]),
                            np.arange(nq))
    assert np.allclose(got, want, rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# One whole prune step
# --------------------------------------------------------------------------
@pytest.mark.parametrize("reversed_", [False, True])
def test_prune_step_on_the_tiny_workload(reversed_):
    """The composition the smoke check compares against, on the tiny workload
    (1 layer, 2 heads x 64, fp32, 8 chunks of 64 rows, gamma 0.1, sink chunk 0,
    chunks 1-5 scored, window of 2 chunks; 8 temporal pairs, q0 = 8, knee 2,
    factor 4), against facts from outside the oracle: the mask from a float64
    numpy score (no row lies within rounding of gamma), the index list from
    numpy.flatnonzero, K and V rows by numpy advanced indexing (V and the
    non-temporal dims of K bit for bit), the row frames likewise, the new
    phases from exact rationals and the re-indexed key pairs from float64
    complex rotation by theta_j (t~ - t) (DeCoPrune page, 어떻게 동작하나 and
    무엇과 다른가)."""
    w = dpsynth.WORKLOADS["tiny"]
    T, H, D, L = w.seq_len, w.n_heads, w.head_dim, w.n_layers
    x0, xf = dpsynth.score_inputs(w)
    k = np.stack([dpsynth.kv_layer_host("f32", w.seed, dpsynth.STREAM_K, l, T, H * D)
                  for l in range(L)]).reshape(L, T, H, D)
    v = np.stack([dpsynth.kv_layer_host("f32", w.seed, dpsynth.STREAM_V, l, T, H * D)
                  for l in range(L)]).reshape(L, T, H, D)
    rf = dpsynth.row_frame(w)
    theta = dpsynth.rope_theta(w.rope_pairs, w.rope_base)
    ft, fp = dpsynth.frame_tables(w)
    got = oracle.prune_step(
        x0, xf, w.d, dict(seq_len=T, sink_len=w.sink_len, window_len=w.window_len,
                          scored_begin=w.scored_begin, n_scored=w.n_scored, gamma=w.gamma,
                          reversed=reversed_),
        k, v, rf, dict(theta=theta, frame_t=ft, frame_phase=fp, q0=w.q0, knee=w.rope_knee,
                       inv_factor=np.float32(1.0 / w.rope_factor)))
    ell = ((x0.astype(np.float64) - xf.astype(np.float64)) ** 2).mean(axis=1)
    assert np.min(np.abs(ell - w.gamma)) > 1e-5 * w.gamma
    big = ell >= w.gamma
    keep = np.ones(T, np.uint8)
    keep[w.scored_begin:w.scored_begin + w.n_scored] = (~big if reversed_ else big)
    assert np.array_equal(got["keep"], keep)
    idx = np.flatnonzero(keep)
    assert np.array_equal(got["idx"], idx)
    assert np.array_equal(got["v"].view(np.uint32), v[:, idx].view(np.uint32))
    assert np.array_equal(got["row_frame"], rf[idx])
    lo, hi = 0, 2 * w.rope_pairs
    assert np.array_equal(got["k"][..., hi:].view(np.uint32), k[:, idx][..., hi:].view(np.uint32))
    t_new = np.array([float(_t_new_exact(w.q0, w.rope_knee, Fraction(w.rope_factor), f))
                      for f in range(w.n_frames)])
    assert np.array_equal(got["tables"][3].astype(np.float64), t_new)
    step = t_new - ft.astype(np.float64)
    for l in range(L):
        want = _rot_f64(k[l][idx], rf[idx], 0, theta, step)
        assert np.max(np.abs(got["k"][l].astype(np.float64) - want)) < 2e-6
    assert np.array_equal(got["k"][..., lo:hi][:, idx >= T - w.window_len],
                          k[:, idx[idx >= T - w.window_len]][..., lo:hi])


# --------------------------------------------------------------------------
# Pruning ratio
# --------------------------------------------------------------------------
def test_pruning_ratio_integer_identity():
    assert oracle.pr(0, 10) == 1.0 and oracle.pr(10, 10) == 0.0 and oracle.pr(0, 0) == 0.0
    L, H, T, n = 40, 40, 31200, 25896
    assert oracle.pr(L * H * n, L * H * T) == 1 - n / T


# --------------------------------------------------------------------------
# Input generator sanity (not method arithmetic)
# --------------------------------------------------------------------------
def test_kv_table_is_standard_normal_quantiles():
    t = dpsynth.kv_table("f32").view(np.float32)
    assert np.array_equal(t, -t[::-1])
    assert abs(t.mean()) < 1e-6 and abs(t.std() - 1) < 2e-3
    b = dpsynth.kv_table("bf16")
    assert b.dtype == np.uint16 and b.shape == (65536,)


def test_kv_host_twin_is_deterministic_and_row_addressable():
    a = dpsynth.kv_layer_host("bf16", 0, 1, 2, 50, 16)
    b = dpsynth.kv_rows_host("bf16", 0, 1, 2, [7, 3], 50, 16)
    assert np.array_equal(a[[7, 3]], b)
    c = dpsynth.kv_rows_host("bf16", 0, 2, 2, [7, 3], 50, 16)
    assert not np.array_equal(b, c)


def test_reindex_trig_table_is_rounded_fp64_trig_of_fp32_angle():
    # cos/sin entries are the fp32 roundings of the float64 cos/sin of the
    # fp32 angle theta_j * delta_f (Python's math module as the reference)
    import math
    theta = dpsynth.rope_theta(44)
    t = np.arange(240, dtype=np.float32)
    delta, c, s, _ = oracle.rope_frames(t, t, 240.0, 12.0, 0.125, theta)
    for f in range(0, 240, 7):
        for j in range(44):
            ang = float(np.float32(theta[j]) * np.float32(delta[f]))
            assert c[f, j] == np.float32(math.cos(ang)) and s[f, j] == np.float32(math.sin(ang))


@pytest.mark.parametrize("name", ["tiny", "eviction", "prefix", "hs"])
def test_workload_masks_are_order_insensitive(name):
    """Reading of the score's precision: a fixed fp32 summation order matters
    only where a score sits at the threshold.  On every workload the fp32 mask
    equals the float64 mask bit for bit, and every token whose float64 score
    lies within 1e-6 * gamma of gamma (one of the prefix workload's 355,680)
    is still farther from gamma than the rounding error of any pairwise fp32
    evaluation (difference, square, a tree of ceil(log2 d) additions, the exact
    division: at most (ceil(log2 d) + 3) u l with u = 2^-24), so its keep bit
    does not depend on the pairing either (DeCoPrune page, section 어떻게
    동작하나: keep tokens whose score reaches gamma)."""
    w = dpsynth.WORKLOADS[name]
    x0, xf = dpsynth.score_inputs(w)
    e64 = oracle.score_f64(x0, xf, w.d)
    e32 = oracle.score_f32(x0, xf, w.d)
    assert np.array_equal(e32 >= np.float32(w.gamma), e64 >= w.gamma)
    near = np.flatnonzero(np.abs(e64 - w.gamma) < 1e-6 * w.gamma)
    assert near.shape[0] <= e64.shape[0] // 100000
    bound = (np.ceil(np.log2(w.d)) + 3) * 2.0 ** -24 * e64[near]
    assert np.all(np.abs(e64[near] - w.gamma) > bound)
    print("%s: %d scored tokens, %d within 1e-6 gamma of gamma, nearest at %.3g gamma"
          % (name, e64.shape[0], near.shape[0], float(np.min(np.abs(e64 - w.gamma)) / w.gamma)))
