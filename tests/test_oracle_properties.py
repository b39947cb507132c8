"""Property tests of the oracle on random tiny shapes (hypothesis).

Invariants the DeCoPrune page's rules imply (section 어떻게 동작하나 for the
score, mask, index and gather, 무엇과 다른가 for the re-index, 어떻게 쓰나 for
PR), checked over random policies and inputs rather than fixed cases: the
protected rows are always kept, the reversed criterion is the complement on
the scored rows, raising the threshold never keeps more rows, the index list
is the ascending list of kept rows, the gather copies exactly those rows, the
score is a non-negative quadratic form, the re-index keeps the order of keys
and the length of every rotated pair, and PR lies in [0, 1].
"""
import math

import numpy as np
from hypothesis import given, settings, strategies as st

import dpsynth
import oracle

SETTINGS = settings(max_examples=60, deadline=None)


@st.composite
def policies(draw):
    T = draw(st.integers(1, 300))
    sink = draw(st.integers(0, T))
    window = draw(st.integers(0, T - sink))
    scored_begin = draw(st.integers(sink, T - window))
    n_scored = draw(st.integers(0, T - window - scored_begin))
    seed = draw(st.integers(0, 2**31))
    return T, sink, window, scored_begin, n_scored, seed


def _ell(seed, n, nan_rate=0.05):
    rng = np.random.default_rng(seed)
    e = (rng.exponential(0.1, n)).astype(np.float32)
    e[rng.random(n) < nan_rate] = np.nan
    return e


@SETTINGS
@given(policies(), st.sampled_from([0.0, 0.05, 0.1, 0.3, math.inf]))
def test_mask_protects_sink_and_window_and_reversed_is_complement(pol, gamma):
    T, sink, window, sb, ns, seed = pol
    ell = _ell(seed, ns)
    keep = oracle.mask(ell, T, sink, window, sb, ns, gamma)
    rev = oracle.mask(ell, T, sink, window, sb, ns, gamma, reversed=True)
    stream = oracle.mask(None, T, sink, window, sb, ns, gamma, streaming=True)
    assert keep.dtype == np.uint8 and set(np.unique(keep)) <= {0, 1}
    assert np.all(keep[:sink] == 1) and np.all(keep[T - window:] == 1)
    assert np.all(stream[:sink] == 1) and np.all(stream[T - window:] == 1)
    assert np.all(stream[sink:T - window] == 0)
    scored = np.zeros(T, bool)
    scored[sb:sb + ns] = True
    assert np.array_equal(rev[scored], 1 - keep[scored])        # exact complement, NaN included
    assert np.array_equal(rev[~scored], keep[~scored])
    assert np.all(keep[~scored] == 1)                            # score mode keeps the rest
    finite = np.isfinite(ell)
    if gamma == 0.0:
        assert np.all(keep[sb:sb + ns][finite] == 1)             # gamma = 0 keeps every score
    assert np.all(keep[sb:sb + ns][~finite] == 0)                # NaN fails the test


@SETTINGS
@given(policies(), st.floats(0, 0.5), st.floats(0, 0.5))
def test_raising_gamma_never_keeps_more_rows(pol, g1, g2):
    T, sink, window, sb, ns, seed = pol
    lo, hi = min(g1, g2), max(g1, g2)
    ell = _ell(seed, ns)
    k_lo = oracle.mask(ell, T, sink, window, sb, ns, np.float32(lo))
    k_hi = oracle.mask(ell, T, sink, window, sb, ns, np.float32(hi))
    assert np.all(k_hi <= k_lo)


@SETTINGS
@given(st.integers(0, 400), st.floats(0, 1), st.integers(0, 2**31))
def test_index_is_the_ascending_list_of_kept_rows(T, rate, seed):
    rng = np.random.default_rng(seed)
    keep = (rng.random(T) < rate).astype(np.uint8)
    idx = oracle.compact(keep)
    assert idx.dtype == np.int32 and idx.shape[0] == int(keep.sum())
    assert np.all(np.diff(idx) > 0)
    assert np.all(keep[idx] == 1)


@SETTINGS
@given(st.integers(1, 3), st.integers(1, 120), st.integers(1, 4), st.sampled_from([8, 16, 32]),
       st.integers(0, 2**31))
def test_gather_copies_exactly_the_listed_rows(L, T, H, D, seed):
    rng = np.random.default_rng(seed)
    src = rng.integers(0, 2**16, (L, T, H, D), dtype=np.uint16)
    keep = (rng.random(T) < 0.5).astype(np.uint8)
    idx = oracle.compact(keep)
    out = oracle.gather(src, idx)
    assert out.shape == (L, idx.shape[0], H, D)
    for j, t in enumerate(idx):
        assert np.array_equal(out[:, j], src[:, t])


@SETTINGS
@given(st.integers(1, 50), st.integers(1, 80), st.integers(0, 2**31), st.integers(-3, 3))
def test_score_is_a_nonnegative_quadratic_form(n, d, seed, k):
    rng = np.random.default_rng(seed)
    xf = rng.standard_normal((n, d)).astype(np.float32)
    x0 = (xf + rng.standard_normal((n, d)) * 0.3).astype(np.float32)
    x0[0] = xf[0]                                                # one row with no discrepancy
    ell = oracle.score_f32(x0, xf)
    assert np.all(ell >= 0) and ell[0] == 0.0 and not np.signbit(ell[0])
    # scaling the discrepancy by 2^k scales every fp32 step exactly: by 4^k
    s = np.float32(2.0 ** k)
    ell2 = oracle.score_f32(x0 * s, xf * s)
    assert np.array_equal(ell2, ell * np.float32(4.0 ** k))


@SETTINGS
@given(st.integers(2, 120), st.integers(0, 24), st.sampled_from([1.0, 2.0, 4.0, 8.0]),
       st.integers(1, 12))
def test_reindex_keeps_key_order_and_identity_inside_the_knee(n_frames, knee, factor, npairs):
    t = np.arange(n_frames, dtype=np.float32)
    q0 = float(n_frames)
    delta, c, s, ph = oracle.rope_frames(t, t, q0, float(knee), np.float32(1.0 / factor),
                                         dpsynth.rope_theta(npairs))
    assert np.all(np.diff(ph) > 0)                               # order of keys preserved
    recent = q0 - t <= knee
    assert np.array_equal(ph[recent], t[recent]) and np.all(delta[recent] == 0)
    if factor == 1.0:
        assert np.all(delta == 0)
    assert np.all(ph >= t) and np.all(ph <= q0)                  # old keys move towards q0
    assert np.all(np.abs(c * c + s * s - 1.0) < 1e-6)


@SETTINGS
@given(st.integers(1, 30), st.integers(1, 3), st.integers(1, 12), st.integers(0, 2**31))
def test_rotation_keeps_pair_lengths(rows, H, npairs, seed):
    rng = np.random.default_rng(seed)
    D = 2 * npairs + 2 * int(rng.integers(0, 4))
    k = rng.standard_normal((rows, H, D)).astype(np.float32)
    before = k.copy()
    n_frames = 40
    t = np.arange(n_frames, dtype=np.float32)
    tables = oracle.rope_frames(t, t, float(n_frames), 4.0, np.float32(0.25),
                                dpsynth.rope_theta(npairs))
    rf = rng.integers(0, n_frames, rows).astype(np.int32)
    oracle.rope_rows(k, rf, 0, tables)
    a = before[..., :2 * npairs].reshape(rows, H, npairs, 2).astype(np.float64)
    b = k[..., :2 * npairs].reshape(rows, H, npairs, 2).astype(np.float64)
    na, nb = np.hypot(a[..., 0], a[..., 1]), np.hypot(b[..., 0], b[..., 1])
    assert np.all(np.abs(na - nb) <= 1e-5 * (1 + na))
    assert np.array_equal(k[..., 2 * npairs:], before[..., 2 * npairs:])   # other dims untouched


@SETTINGS
@given(st.integers(0, 10**9), st.integers(1, 10**9))
def test_pr_is_a_ratio_in_the_unit_interval(visible, full):
    visible = min(visible, full)
    p = oracle.pr(visible, full)
    assert 0.0 <= p <= 1.0
    assert oracle.pr(full, full) == 0.0 and oracle.pr(0, full) == 1.0
    assert abs(p - (full - visible) / full) <= 1e-15
