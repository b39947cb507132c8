"""libdecoprune loads, exports every symbol of include/decoprune.h, and rejects
bad arguments on the host before any HIP call (these tests never reach a
launch, so they run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import compaction_dp_score_amd as dp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decoprune.h")

FAKE = 0x10000          # a 64 KiB-aligned non-null address; never dereferenced here


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dp_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = header_functions()
    assert len(names) == 26, names
    lib = ctypes.CDLL(dp.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(dp.EXPORTED) == names


def test_version_and_status_strings():
    assert dp.dp_abi_version() == 3
    assert dp.dp_status_str(dp.DP_OK) == "DP_OK"
    assert dp.dp_status_str(dp.DP_ECAPACITY) == "DP_ECAPACITY"
    assert dp.dp_status_str(dp.DP_ESTALL) == "DP_ESTALL"
    assert dp.dp_status_str(99) == "DP_UNKNOWN"


def test_struct_layouts_match_header(tmp_path):
    # the ctypes mirrors have the size and field offsets gcc gives the header
    structs = {"dp_mask_policy": dp.dp_mask_policy, "dp_rope": dp.dp_rope, "dp_kv": dp.dp_kv,
               "dp_kv_hs": dp.dp_kv_hs, "dp_pr_counter": dp.dp_pr_counter,
               "dp_kv_inplace": dp.dp_kv_inplace}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "decoprune.h"', 'int main(void){']
    for name, cls in structs.items():
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (name, name))
        for f, _ in cls._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (name, f, name, f))
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)],
                   check=True)
    out = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                 check=True).stdout.splitlines())
    for name, cls in structs.items():
        assert int(out[name]) == ctypes.sizeof(cls), name
        for f, _ in cls._fields_:
            assert int(out["%s.%s" % (name, f)]) == getattr(cls, f).offset, (name, f)


def _status(fn, *args):
    return getattr(dp, "_lib_" + fn)(*args)


def _policy(**kw):
    p = dict(seq_len=1000, sink_len=100, window_len=200, scored_begin=100, n_scored=300,
             gamma=0.1)
    p.update(kw)
    return dp.make_policy(**p)


@pytest.mark.parametrize("kw,d,stride,want", [
    (dict(seq_len=0), 16, 16, dp.DP_ERANGE),
    (dict(seq_len=1 << 31), 16, 16, dp.DP_ERANGE),
    (dict(scored_begin=50), 16, 16, dp.DP_EINVAL),          # scored overlaps the sink
    (dict(n_scored=800), 16, 16, dp.DP_EINVAL),             # scored overlaps the window
    (dict(window_len=-1), 16, 16, dp.DP_EINVAL),
    (dict(), 0, 16, dp.DP_ERANGE),
    (dict(), 257, 300, dp.DP_ERANGE),
    (dict(), 16, 8, dp.DP_EINVAL),
])
def test_score_mask_rejects(kw, d, stride, want):
    p = _policy(**kw)
    st = _status("score_mask", FAKE, FAKE, d, stride, ctypes.byref(p), None, FAKE, None)
    assert st == want, dp.dp_last_error()
    assert dp.dp_last_error()


def test_score_mask_rejects_bad_mode_and_pointers():
    p = _policy()
    p.mode = 2
    assert _status("score_mask", FAKE, FAKE, 16, 16, ctypes.byref(p), None, FAKE, None) == dp.DP_EINVAL
    p = _policy()
    assert _status("score_mask", None, FAKE, 16, 16, ctypes.byref(p), None, FAKE, None) == dp.DP_EINVAL
    assert _status("score_mask", FAKE + 2, FAKE, 16, 16, ctypes.byref(p), None, FAKE, None) == dp.DP_EALIGN
    assert _status("score_mask", FAKE, FAKE, 16, 16, None, None, FAKE, None) == dp.DP_EINVAL
    with pytest.raises(dp.DPError) as e:
        dp.dp_score_mask(None, None, 16, 16, _policy(scored_begin=0), None, None, stream=0)
    assert e.value.status == dp.DP_EINVAL


def test_compact_rejects():
    need = dp.dp_compact_workspace_bytes(10000)
    assert need >= 4 * 3
    assert _status("compact", FAKE, 10000, FAKE, FAKE, None, None, FAKE, need - 1, None) == dp.DP_EINVAL
    assert _status("compact", FAKE, -1, FAKE, FAKE, None, None, FAKE, need, None) == dp.DP_ERANGE
    assert _status("compact", FAKE, 10000, FAKE, FAKE + 4, None, None, FAKE, need, None) == dp.DP_EALIGN
    assert _status("compact", FAKE, 10000, FAKE, FAKE, FAKE, None, FAKE, need, None) == dp.DP_EINVAL
    assert _status("compact", None, 10000, FAKE, FAKE, None, None, FAKE, need, None) == dp.DP_EINVAL


def test_compact_noalloc_rejects():
    # host-side checks of the entry point without a workspace, before any HIP call
    assert _status("compact_noalloc", FAKE, -1, FAKE, FAKE, None, None, None) == dp.DP_ERANGE
    assert _status("compact_noalloc", FAKE, 1 << 31, FAKE, FAKE, None, None, None) == dp.DP_ERANGE
    assert _status("compact_noalloc", FAKE, 10000, FAKE, FAKE + 4, None, None, None) == dp.DP_EALIGN
    assert _status("compact_noalloc", FAKE, 10000, FAKE + 2, FAKE, None, None, None) == dp.DP_EALIGN
    assert _status("compact_noalloc", FAKE, 10000, FAKE, FAKE, FAKE, None, None) == dp.DP_EINVAL
    assert _status("compact_noalloc", None, 10000, FAKE, FAKE, None, None, None) == dp.DP_EINVAL
    assert _status("compact_noalloc", FAKE, 10000, FAKE, None, None, None, None) == dp.DP_EINVAL


def _kv(**kw):
    kv = dp.dp_kv()
    f = dict(k_src=FAKE, v_src=FAKE, k_dst=FAKE, v_dst=FAKE, n_layers=2, n_heads=4, head_dim=64,
             dtype=dp.DP_BF16, src_rows=1000, dst_capacity=1000, dev_error=None)
    f.update(kw)
    for k, v in f.items():
        setattr(kv, k, v)
    return kv


def _rope(**kw):
    r = dp.dp_rope()
    f = dict(pair_begin=0, n_pairs=8, theta=FAKE, n_frames=10, axis=0, frame_t=FAKE,
             frame_phase=FAKE, q0=10.0, knee=2.0, inv_factor=0.25)
    f.update(kw)
    for k, v in f.items():
        setattr(r, k, v)
    return r


@pytest.mark.parametrize("kw,want", [
    (dict(head_dim=63), dp.DP_EINVAL),
    (dict(head_dim=4), dp.DP_EALIGN),                    # 8-byte bf16 head rows
    (dict(dtype=7), dp.DP_EINVAL),
    (dict(v_dst=None), dp.DP_EINVAL),
    (dict(k_src=None), dp.DP_EINVAL),
    (dict(n_layers=0), dp.DP_EINVAL),
    (dict(src_rows=1 << 31), dp.DP_ERANGE),
    (dict(dst_capacity=1 << 40), dp.DP_ERANGE),
    (dict(n_layers=40000, dst_capacity=1000000), dp.DP_ERANGE),
])
def test_gather_rejects(kw, want):
    kv = _kv(**kw)
    assert _status("gather", ctypes.byref(kv), FAKE, FAKE, None, None, None, 0, None) == want


@pytest.mark.parametrize("kw,ws,want", [
    (dict(n_pairs=40), None, dp.DP_ERANGE),              # 2*40 > head_dim 64
    (dict(pair_begin=2), None, dp.DP_EALIGN),            # bf16 block must start on 16 bytes
    (dict(n_pairs=0), None, dp.DP_EINVAL),
    (dict(theta=None), None, dp.DP_EINVAL),
    (dict(), 8, dp.DP_EINVAL),                           # workspace too small
    (dict(axis=2), None, dp.DP_EINVAL),
    (dict(axis=-1), None, dp.DP_EINVAL),
])
def test_fused_rope_rejects(kw, ws, want):
    kv = _kv()
    r = _rope(**kw)
    ws_bytes = dp.dp_rope_workspace_bytes(r.n_frames, max(r.n_pairs, 1)) if ws is None else ws
    st = _status("gather", ctypes.byref(kv), FAKE, FAKE, FAKE, ctypes.byref(r), FAKE, ws_bytes, None)
    assert st == want, dp.dp_last_error()


def test_fused_rope_needs_row_frame_and_aligned_workspace():
    kv, r = _kv(), _rope()
    nb = dp.dp_rope_workspace_bytes(10, 8)
    assert _status("gather", ctypes.byref(kv), FAKE, FAKE, None, ctypes.byref(r), FAKE, nb, None) == dp.DP_EINVAL
    assert _status("gather", ctypes.byref(kv), FAKE, FAKE, FAKE, ctypes.byref(r), FAKE + 8, nb, None) == dp.DP_EALIGN


def test_reindex_rejects():
    r = _rope()
    nb = dp.dp_rope_workspace_bytes(10, 8)
    f = lambda *a: _status("reindex", *a)
    assert f(None, 1, 4, 64, 1, 100, None, FAKE, ctypes.byref(r), FAKE, nb, None) == dp.DP_EINVAL
    assert f(FAKE, 1, 4, 64, 1, -1, None, FAKE, ctypes.byref(r), FAKE, nb, None) == dp.DP_ERANGE
    assert f(FAKE, 1, 4, 64, 1, 100, FAKE + 4, FAKE, ctypes.byref(r), FAKE, nb, None) == dp.DP_EALIGN
    r2 = _rope(pair_begin=1)
    assert f(FAKE, 1, 4, 64, 0, 100, None, FAKE, ctypes.byref(r2), FAKE, nb, None) == dp.DP_EALIGN


def test_hs_rejects():
    caps = (ctypes.c_int64 * 2)(10, 10)
    assert _status("hs_offsets", FAKE, 2, 4, FAKE, 9, FAKE, None) == dp.DP_EINVAL
    assert _status("hs_offsets", FAKE, 2, 4, FAKE + 4, 2, FAKE, None) == dp.DP_EALIGN
    kv = dp.dp_kv_hs()
    kv.k_src, kv.v_src, kv.k_out, kv.v_out = FAKE, FAKE, FAKE, FAKE
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = 2, 2000, 64, dp.DP_BF16
    kv.src_rows, kv.out_capacity = 100, 100
    assert _status("hs_gather", ctypes.byref(kv), FAKE, 2, FAKE, FAKE, caps, FAKE, None, None,
                   None, 0, None) == dp.DP_ERANGE
    kv.n_heads = 4
    bad = (ctypes.c_int64 * 2)(10, -1)
    assert _status("hs_gather", ctypes.byref(kv), FAKE, 2, FAKE, FAKE, bad, FAKE, None, None,
                   None, 0, None) == dp.DP_ERANGE
    kv.k_out = FAKE + 8
    assert _status("hs_gather", ctypes.byref(kv), FAKE, 2, FAKE, FAKE, caps, FAKE, None, None,
                   None, 0, None) == dp.DP_EALIGN
    r = _rope()
    assert _status("hs_reindex", FAKE, 100, 2, 4, 64, 1, FAKE, 2, FAKE, caps, FAKE, None,
                   ctypes.byref(r), FAKE, 4096, None) == dp.DP_EINVAL
    # split keys: the cache's pairs must make whole 16-byte vectors, and a fused
    # re-index must name the cache's layout and pairs
    kv.k_out = FAKE
    kv.key_layout, kv.pair_begin, kv.n_pairs = dp.DP_KEY_SPLIT, 0, 6
    assert _status("hs_gather", ctypes.byref(kv), FAKE, 2, FAKE, FAKE, caps, FAKE, None, None,
                   None, 0, None) == dp.DP_EALIGN
    kv.n_pairs = 8
    nb = dp.dp_rope_workspace_bytes(10, 8)
    for rk in (_rope(), _rope(key_layout=dp.DP_KEY_SPLIT, n_pairs=4)):
        assert _status("hs_gather", ctypes.byref(kv), FAKE, 2, FAKE, FAKE, caps, FAKE, FAKE,
                       ctypes.byref(rk), FAKE, nb, None) == dp.DP_EINVAL
    kv.key_layout = 5
    assert _status("hs_gather", ctypes.byref(kv), FAKE, 2, FAKE, FAKE, caps, FAKE, None, None,
                   None, 0, None) == dp.DP_EINVAL
    # the source rows' layout is checked on its own: unknown, or split with
    # pairs that do not make whole vectors
    kv.key_layout, kv.src_key_layout = dp.DP_KEY_INTERLEAVED, 7
    assert _status("hs_gather", ctypes.byref(kv), FAKE, 2, FAKE, FAKE, caps, FAKE, None, None,
                   None, 0, None) == dp.DP_EINVAL
    kv.src_key_layout, kv.n_pairs = dp.DP_KEY_SPLIT, 6
    assert _status("hs_gather", ctypes.byref(kv), FAKE, 2, FAKE, FAKE, caps, FAKE, None, None,
                   None, 0, None) == dp.DP_EALIGN


def test_pruning_ratio_counter():
    c = dp.dp_pr_counter()
    assert dp.dp_pr_value(c) == 0.0
    L, H, T, n = 40, 40, 31200, 25896
    dp.dp_pr_add(c, L * H * n, L * H * T)
    assert dp.dp_pr_value(c) == 1 - n / T
    dp.dp_pr_add(c, 0, L * H * 6240)                 # a step that drops a whole chunk
    assert dp.dp_pr_value(c) == 1 - (L * H * n) / (L * H * (T + 6240))
    with pytest.raises(dp.DPError):
        dp.dp_pr_add(c, 5, 4)



def _inplace(**kw):
    kv = dp.dp_kv_inplace()
    f = dict(k_layers=FAKE, v_layers=FAKE, n_layers=2, n_heads=4, head_dim=64, dtype=dp.DP_BF16,
             capacity=1000, dev_error=None)
    f.update(kw)
    for k, v in f.items():
        setattr(kv, k, v)
    return kv


@pytest.mark.parametrize("kw,slot,want", [
    (dict(), (900, 200), dp.DP_ERANGE),              # slot passes the capacity
    (dict(), (-1, 10), dp.DP_ERANGE),
    (dict(capacity=1 << 31), (0, 10), dp.DP_ERANGE),
    (dict(k_layers=None), (0, 10), dp.DP_EINVAL),
    (dict(head_dim=7), (0, 10), dp.DP_EINVAL),
    (dict(head_dim=6), (0, 10), dp.DP_EALIGN),
])
def test_append_kept_rejects(kw, slot, want):
    kv = _inplace(**kw)
    st = _status("append", ctypes.byref(kv), slot[0], slot[1], FAKE, FAKE, FAKE, None, None, None,
                 0, None)
    assert st == want, dp.dp_last_error()


def test_append_kept_rejects_missing_and_misaligned():
    kv = _inplace()
    assert _status("append", ctypes.byref(kv), 0, 10, None, FAKE, FAKE, None, None, None, 0,
                   None) == dp.DP_EINVAL
    assert _status("append", ctypes.byref(kv), 0, 10, FAKE, FAKE, None, None, None, None, 0,
                   None) == dp.DP_EINVAL
    assert _status("append", ctypes.byref(kv), 0, 10, FAKE, FAKE + 4, FAKE, None, None, None, 0,
                   None) == dp.DP_EALIGN
    assert _status("append", ctypes.byref(kv), 0, 10, FAKE, FAKE, FAKE, FAKE + 2, None, None, 0,
                   None) == dp.DP_EALIGN


def test_append_kept_fused_rope_and_shift_reject():
    kv = dp.dp_kv_inplace()
    kv.k_layers, kv.v_layers = FAKE, FAKE
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = 2, 4, 64, dp.DP_BF16
    kv.capacity = 1000
    r = _rope()
    # a fused re-index needs the row frames and a large enough workspace
    assert _status("append", ctypes.byref(kv), 0, 10, FAKE, FAKE, FAKE, None, ctypes.byref(r),
                   FAKE, 1 << 20, None) == dp.DP_EINVAL
    assert _status("append", ctypes.byref(kv), 0, 10, FAKE, FAKE, FAKE, FAKE, ctypes.byref(r),
                   FAKE, 8, None) == dp.DP_EINVAL
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("k", FAKE), ("L", 2), ("H", 4), ("D", 64), ("dt", dp.DP_BF16), ("rb", 0), ("cap", 1000),
        ("n", None), ("theta", FAKE), ("pb", 0), ("np", 12), ("kl", 0), ("delta", 3.5),
        ("ws", FAKE), ("wsb", 4096), ("s", None))]
    assert _status("rope_shift", *args(theta=None)) == dp.DP_EINVAL
    assert _status("rope_shift", *args(np=0)) == dp.DP_EINVAL
    assert _status("rope_shift", *args(np=40)) == dp.DP_ERANGE            # past head_dim/2
    assert _status("rope_shift", *args(pb=2)) == dp.DP_EALIGN             # block start not 16 B
    assert _status("rope_shift", *args(delta=float("inf"))) == dp.DP_EINVAL
    assert _status("rope_shift", *args(delta=float("nan"))) == dp.DP_EINVAL
    assert _status("rope_shift", *args(rb=-1)) == dp.DP_ERANGE
    assert _status("rope_shift", *args(n=FAKE + 4)) == dp.DP_EALIGN
    assert _status("rope_shift", *args(D=7)) == dp.DP_EINVAL
    assert _status("rope_shift", *args(ws=None)) == dp.DP_EINVAL
    assert _status("rope_shift", *args(wsb=8)) == dp.DP_EINVAL
    assert _status("rope_shift", *args(ws=FAKE + 8)) == dp.DP_EALIGN
    assert dp.dp_rope_shift_workspace_bytes(44) == (44 + 4) * 8
    assert _status("rope_shift", *args(cap=0)) == dp.DP_OK                 # empty range: nothing
    # split keys: the temporal block must be whole 16-byte vectors (bf16: pairs in fours)
    assert _status("rope_shift", *args(kl=dp.DP_KEY_SPLIT, np=10)) == dp.DP_EALIGN
    assert _status("rope_shift", *args(kl=dp.DP_KEY_SPLIT, np=12, cap=0)) == dp.DP_OK
    assert _status("rope_shift", *args(kl=2)) == dp.DP_EINVAL


def test_rope_prepare_and_apply_reject():
    r = _rope()
    nb = dp.dp_rope_workspace_bytes(10, 8)
    assert _status("rope_prepare", None, 64, 1, FAKE, nb, None) == dp.DP_EINVAL
    assert _status("rope_prepare", ctypes.byref(r), 64, 1, FAKE, nb - 1, None) == dp.DP_EINVAL
    assert _status("rope_prepare", ctypes.byref(r), 63, 1, FAKE, nb, None) == dp.DP_EINVAL
    f = lambda *a: _status("rope_apply", *a)
    assert f(FAKE, 1, 4, 64, 1, -1, 100, None, FAKE, ctypes.byref(r), FAKE, nb, None) == dp.DP_ERANGE
    assert f(FAKE, 1, 4, 64, 1, 0, 1 << 31, None, FAKE, ctypes.byref(r), FAKE, nb, None) == dp.DP_ERANGE
    assert f(FAKE, 1, 4, 64, 1, 0, 100, None, None, ctypes.byref(r), FAKE, nb, None) == dp.DP_EINVAL
    assert f(FAKE, 1, 4, 64, 1, 0, 100, FAKE + 4, FAKE, ctypes.byref(r), FAKE, nb, None) == dp.DP_EALIGN
    # an empty range is accepted without any launch
    assert f(FAKE, 1, 4, 64, 1, 50, 50, None, FAKE, ctypes.byref(r), FAKE, nb, None) == dp.DP_OK


def test_attention_rejects():
    B = dp.DP_BF16
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("q", FAKE), ("k", FAKE), ("v", FAKE), ("o", FAKE), ("n_q", 100), ("cap", 100),
        ("n_kv", None), ("H", 8), ("D", 128), ("dtype", B), ("scale", 0.1), ("kl", 0), ("p0", 0),
        ("np", 0), ("s", None))]
    assert _status("attention", *args(q=None)) == dp.DP_EINVAL
    assert _status("attention", *args(D=64)) == dp.DP_EUNSUPPORTED
    assert _status("attention", *args(dtype=dp.DP_F32)) == dp.DP_EUNSUPPORTED
    assert _status("attention", *args(H=0)) == dp.DP_ERANGE
    assert _status("attention", *args(H=65537)) == dp.DP_ERANGE
    assert _status("attention", *args(cap=-1)) == dp.DP_ERANGE
    assert _status("attention", *args(n_q=1 << 31)) == dp.DP_ERANGE
    assert _status("attention", *args(k=FAKE + 8)) == dp.DP_EALIGN
    assert _status("attention", *args(n_kv=FAKE + 4)) == dp.DP_EALIGN
    for bad in (float("nan"), 0.0, -0.5, float("inf")):
        assert _status("attention", *args(scale=bad)) == dp.DP_EINVAL
    # split keys: a temporal block of whole 16-byte vectors within the head
    assert _status("attention", *args(kl=dp.DP_KEY_SPLIT, np=0)) == dp.DP_ERANGE
    assert _status("attention", *args(kl=dp.DP_KEY_SPLIT, np=44, p0=24)) == dp.DP_ERANGE
    assert _status("attention", *args(kl=dp.DP_KEY_SPLIT, np=42)) == dp.DP_EALIGN
    assert _status("attention", *args(kl=dp.DP_KEY_SPLIT, np=44, p0=2)) == dp.DP_EALIGN
    assert _status("attention", *args(kl=7)) == dp.DP_EINVAL


def test_attention_lag_rejects():
    B = dp.DP_BF16
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("q", FAKE), ("k", FAKE), ("v", FAKE), ("o", FAKE), ("n_q", 100), ("cap", 100),
        ("n_kv", None), ("pb", 10), ("pe", 40), ("theta", FAKE), ("p0", 0), ("np", 44),
        ("lag", 12.5), ("H", 8), ("D", 128), ("dtype", B), ("scale", 0.1), ("kl", 0), ("s", None))]
    f = lambda **kw: _status("attention_lag", *args(**kw))
    assert f(theta=None) == dp.DP_EINVAL
    assert f(o=None) == dp.DP_EINVAL
    assert f(D=64) == dp.DP_EUNSUPPORTED
    assert f(dtype=dp.DP_F32) == dp.DP_EUNSUPPORTED
    assert f(H=0) == dp.DP_ERANGE
    assert f(H=65537) == dp.DP_ERANGE
    assert f(cap=1 << 31) == dp.DP_ERANGE
    assert f(pb=-1) == dp.DP_ERANGE
    assert f(pb=50, pe=49) == dp.DP_ERANGE
    assert f(np=0) == dp.DP_ERANGE
    assert f(p0=-1) == dp.DP_ERANGE
    assert f(p0=20, np=45) == dp.DP_ERANGE          # pairs past head_dim / 2
    assert f(theta=FAKE + 2) == dp.DP_EALIGN
    assert f(v=FAKE + 8) == dp.DP_EALIGN
    for bad in (float("nan"), 0.0, float("inf")):
        assert f(scale=bad) == dp.DP_EINVAL
    for bad in (float("nan"), float("inf"), -float("inf")):
        assert f(lag=bad) == dp.DP_EINVAL
    assert f(kl=dp.DP_KEY_SPLIT, np=42) == dp.DP_EALIGN


def test_hs_attention_rejects():
    B = dp.DP_BF16
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("q", FAKE), ("kr", FAKE), ("vr", FAKE), ("cap", 1000), ("off", FAKE), ("layer", 3),
        ("kc", FAKE), ("vc", FAKE), ("nc", 50), ("o", FAKE), ("n_q", 100), ("H", 8), ("D", 128),
        ("dtype", B), ("scale", 0.1), ("kl", 0), ("p0", 0), ("np", 0), ("s", None))]
    assert _status("hs_attention", *args(off=None)) == dp.DP_EINVAL
    assert _status("hs_attention", *args(vc=None)) == dp.DP_EINVAL       # chunk K without V
    assert _status("hs_attention", *args(D=96)) == dp.DP_EUNSUPPORTED
    assert _status("hs_attention", *args(layer=-1)) == dp.DP_ERANGE
    assert _status("hs_attention", *args(H=65537)) == dp.DP_ERANGE
    assert _status("hs_attention", *args(cap=1 << 40)) == dp.DP_ERANGE
    assert _status("hs_attention", *args(nc=-1)) == dp.DP_ERANGE
    assert _status("hs_attention", *args(layer=1 << 30)) == dp.DP_ERANGE
    assert _status("hs_attention", *args(off=FAKE + 4)) == dp.DP_EALIGN
    assert _status("hs_attention", *args(kc=FAKE + 2)) == dp.DP_EALIGN
    for bad in (float("nan"), 0.0, -0.5, float("inf")):
        assert _status("hs_attention", *args(scale=bad)) == dp.DP_EINVAL
    assert _status("hs_attention", *args(kl=dp.DP_KEY_SPLIT, np=6)) == dp.DP_EALIGN


def test_hs_attention_lag_rejects():
    B = dp.DP_BF16
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("q", FAKE), ("kr", FAKE), ("vr", FAKE), ("cap", 1000), ("off", FAKE), ("layer", 3),
        ("kc", FAKE), ("vc", FAKE), ("nc", 50), ("o", FAKE), ("n_q", 100), ("H", 8), ("D", 128),
        ("dtype", B), ("scale", 0.1), ("tail", 30), ("theta", FAKE), ("p0", 0), ("np", 44),
        ("lag", 2.5), ("kl", 0), ("s", None))]
    f = lambda **kw: _status("hs_attention_lag", *args(**kw))
    assert f(theta=None) == dp.DP_EINVAL
    assert f(off=None) == dp.DP_EINVAL
    assert f(vc=None) == dp.DP_EINVAL
    assert f(D=64) == dp.DP_EUNSUPPORTED
    assert f(tail=-1) == dp.DP_ERANGE
    assert f(np=0) == dp.DP_ERANGE
    assert f(p0=30, np=40) == dp.DP_ERANGE
    assert f(H=65537) == dp.DP_ERANGE
    assert f(theta=FAKE + 2) == dp.DP_EALIGN
    assert f(off=FAKE + 4) == dp.DP_EALIGN
    for bad in (float("nan"), float("inf")):
        assert f(lag=bad) == dp.DP_EINVAL
    assert f(scale=0.0) == dp.DP_EINVAL
    assert f(kl=dp.DP_KEY_SPLIT, p0=2) == dp.DP_EALIGN


def test_score_index_rejects():
    pol = _policy()
    ws_need = dp.dp_score_index_workspace_bytes(1000)
    assert ws_need == 16 + 8 * 1024 + 16 + 1000             # control, states, scratch, mask
    args = lambda **kw: [kw.get(n, d) for n, d in (
        ("x0", FAKE), ("xf", FAKE), ("d", 16), ("stride", 16), ("pol", ctypes.byref(pol)),
        ("ell", None), ("keep", None), ("idx", FAKE), ("n", FAKE), ("rfs", None), ("rfd", None),
        ("ws", FAKE), ("wsb", ws_need), ("err", None), ("s", None))]
    assert _status("score_index", *args(idx=None)) == dp.DP_EINVAL
    assert _status("score_index", *args(ws=None)) == dp.DP_EINVAL
    assert _status("score_index", *args(rfs=FAKE)) == dp.DP_EINVAL     # src without dst
    assert _status("score_index", *args(wsb=ws_need - 1)) == dp.DP_EINVAL
    assert _status("score_index", *args(ws=FAKE + 4)) == dp.DP_EALIGN
    assert _status("score_index", *args(n=FAKE + 4)) == dp.DP_EALIGN
    assert _status("score_index", *args(d=300)) == dp.DP_ERANGE
    assert _status("score_index", *args(x0=None)) == dp.DP_EINVAL
    bad = _policy(scored_begin=50)                           # before the end of the sink
    assert _status("score_index", *args(pol=ctypes.byref(bad))) == dp.DP_EINVAL


def test_pointer_array_keeps_its_tensors():
    """A tensor reached only through a pointer array lives as long as the
    array: otherwise it would be freed into torch's caching allocator and
    released to the driver by the next empty_cache() (torch.cuda.graph runs
    one on entry) while a kernel still holds its address."""
    import gc
    import weakref
    import torch
    ts = [torch.empty(16) for _ in range(3)]
    ref = weakref.ref(ts[1])
    arr = dp.ptr_array(ts, torch.device("cpu"))
    assert arr.tolist() == [t.data_ptr() for t in ts]
    del ts
    gc.collect()
    assert ref() is not None
    del arr
    gc.collect()
    assert ref() is None
