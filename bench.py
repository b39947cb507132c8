"""Benchmark of one DeCoPrune prune step on one MI355X.

Default workload ("eviction"): a single chunk-eviction step at the shape of
the DeCoPrune page's setup (section 전제와 한계: 832x480 video, 4 latent
frames per chunk, gamma = 0.10): 40 layers x 40 heads x head_dim 128 bf16
K and V, 5 chunks of 6,240 tokens (sink + the chunk leaving the window + a
3-chunk window), d = 64 score channels.  One step enqueues

  dp_score_index (score, mask and kept-index list in one launch)
    -> dp_gather_kv (fused RoPE re-index)

over all 40 layers, K and V, with every input resident in HBM.  The frame
phase table is restored before each step so every step re-indexes from the
same state (a 20-float device copy).

Printed: one JSON line with the step's algorithmic HBM bytes per second, the
tokens scored per second, a roofline record of the dominant kernel (the
gather) timed with HIP events on its stream, the index phase timed both as
one launch and as dp_score_mask + dp_compact_index, and the CPU oracle timed
on a bounded layer sample of the same workload on the host cores.

Other workloads (--workload reindex | prefix | hs | append | steady |
steady_lazy | hs_ring | attention | hs_attention | attention_lag) time the
other shapes;
"append" is the same eviction step in the ring layout, where only the leaving
chunk's kept rows move and the old keys are re-indexed in place; "steady" is a
later step of the one-minute rollout in that layout (old keys moved by one
uniform phase step), "steady_lazy" the same step with the old keys on the
compressed time axis (none rewritten), "hs_ring" that step for the HS cache
kept as one ring-layout cache per head class; the attention workloads time the next
chunk's attention over the compacted (ragged HS, or compressed-axis) cache in
TFLOP/s.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s (10^9 B/s)
KEY_LAYOUT = 1                 # of the workload being set up (layout_for)


def make_rope(*args, **kw):
    """dp.make_rope for keys in this run's layout (--key-layout)."""
    import compaction_dp_score_amd as dp
    return dp.make_rope(*args, key_layout=KEY_LAYOUT, **kw)


def attn_layout(w):
    """Key-layout arguments of the attention calls (the workload's temporal pairs)."""
    return dict(key_layout=KEY_LAYOUT, pair_begin=0, n_pairs=w.rope_pairs)
PROFILES = os.path.join(ROOT, "profiles")
CALIB_BYTES = 8 << 30          # size of the calibration copy run in every bench process

# dominant kernel of each workload: (rocprof name prefix, sources it is built from)
KERNELS = {
    "eviction": ("gather_kernel", ("gather.hip", "dp_device.h")),
    "tiny": ("gather_kernel", ("gather.hip", "dp_device.h")),
    "prefix": ("gather_kernel", ("gather.hip", "dp_device.h")),
    "reindex": ("reindex_kernel", ("rope.hip", "dp_device.h")),
    "hs": ("hs_gather_kernel", ("hs.hip", "dp_device.h")),
    "append": ("reindex_kernel", ("rope.hip", "dp_device.h")),
    "attention": ("attn_fwd_kernel", ("attention.hip", "dp_device.h")),
    "hs_attention": ("attn_fwd_kernel", ("attention.hip", "dp_device.h")),
    "steady": ("shift_kernel", ("rope.hip", "dp_device.h")),
    "steady_lazy": ("append_kernel", ("append.hip", "dp_device.h")),
    "attention_lag": ("attn_fwd_kernel", ("attention.hip", "dp_device.h")),
    "hs_ring": ("append_kernel", ("append.hip", "dp_device.h")),
}


def traffic_path(workload):
    return os.path.join(PROFILES, "%s_%s_traffic.txt" % (KERNELS[workload][0], workload))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    help="one workload; without it the eviction step is the headline record and "
                         "the tiny, one-minute re-index, both prefix slabs and HS workloads follow "
                         "under configs",
                    choices=["eviction", "tiny", "reindex", "prefix", "hs", "append", "attention",
                             "hs_attention", "steady", "steady_lazy", "attention_lag", "hs_ring"])
    ap.add_argument("--key-layout", default=None, choices=["split", "interleaved"],
                    help="layout of the key rows: split (the temporal blocks of all heads first; "
                         "the re-index writes whole lines) or interleaved ([heads][head_dim]); "
                         "by default split for the re-index workloads (reindex, steady, append) "
                         "and interleaved for the others (each record names its layout)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fullkv", action="store_true",
                    help="skip the context timings that launch the dominant kernel outside the "
                         "timed steps (attention over the uncompacted cache, the page-axis "
                         "steady step, the other key layout, the HS split runs): profiling "
                         "runs, so that every dispatch is a timed one")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--summarize-stats", metavar="STATS_DIR",
                    help="write the kernel-statistics summary of --workload from a rocprofv3 "
                         "--kernel-trace --stats output directory and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic summary of --workload from two rocprofv3 --pmc "
                         "output directories (FETCH_SIZE, WRITE_SIZE) and exit")
    return ap.parse_args()


def kernel_sources_sha(workload):
    """Hash of the code of the workload's kernel sources, comments and layout
    whitespace removed (a comment edit does not change the kernel)."""
    import hashlib
    import re
    token = re.compile(r'"(?:\\.|[^"\\])*"|//[^\n]*|/\*.*?\*/', re.S)
    h = hashlib.sha256()
    for f in KERNELS[workload][1]:
        with open(os.path.join(ROOT, "compaction_dp_score_amd", "csrc", f)) as fh:
            text = fh.read()
        code = token.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", text)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def profile_flags(workload):
    """bench.py flags of the profiling runs of a workload (no context timings,
    so that every dispatch of the dominant kernel is one of the steps')."""
    return "--no-cpu-baseline --no-fullkv"


def read_traffic(workload):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed rocprofv3 counter summary, if it was taken on the current kernel
    source; else None."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha") != kernel_sources_sha(workload):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """HIP events on the current stream (the stream every launch goes to)."""

    def __init__(self):
        self.pairs = []

    def start(self):
        # both events exist before the start is recorded, so nothing but the
        # record calls sits between them and the launch they bracket (creating
        # the stop event after a short kernel's launch could delay its record
        # past the kernel's end)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(torch.cuda.current_stream())
        self.pairs.append([a, b])

    def stop(self):
        self.pairs[-1][1].record(torch.cuda.current_stream())

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(1, len(self.pairs))


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
def step_ms_eager_and_graph(step, restore, reps=20):
    """Median time of one step enqueued call by call, and of the same step
    captured once into a HIP graph and replayed (restore() runs eagerly before
    each, outside the events).  Every buffer the step reaches must be held by
    the caller: entering torch.cuda.graph empties torch's allocator cache."""
    def timed(fn):
        ms = []
        for _ in range(reps + 1):
            restore()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        return float(np.median(ms[1:]))
    eager = timed(step)
    g = torch.cuda.CUDAGraph()
    restore()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    graph = timed(g.replay)
    restore()
    torch.cuda.synchronize()
    del g
    return {"step_ms_eager": round(eager, 4), "step_ms_graph": round(graph, 4)}


def order_sensitive(x0, xf, d, gamma):
    """Scored tokens whose float64 score lies within 1e-6 of the threshold
    (relative): the only ones whose keep bit could depend on the order in which
    the fp32 score sums its channels.  A property of the inputs, reported with
    each scoring record."""
    e = x0[:, :d].astype(np.float64) - xf[:, :d].astype(np.float64)
    ell = (e * e).sum(axis=1) / d
    g = float(np.float32(gamma))
    return int(np.count_nonzero(np.abs(ell - g) < 1e-6 * g))


def index_compare(step, x0d, xfd, d, reps=20):
    """Time the index phase both ways on the step's buffers (outside the timed
    steps): dp_score_index (one launch) and dp_score_mask + dp_compact_index
    (four launches).  Returns mean microseconds per call of each."""
    import compaction_dp_score_amd as dp

    def fused():
        dp.dp_score_index(x0d, xfd, d, d, step.policy, None, step.keep, step.idx, step.n_kept,
                          step.row_frame_src, step.row_frame_dst, step.ws_index, step.dev_error)

    def separate():
        dp.dp_score_mask(x0d, xfd, d, d, step.policy, None, step.keep)
        dp.dp_compact_index(step.keep, step.seq_len, step.idx, step.n_kept, step.row_frame_src,
                            step.row_frame_dst, step.ws_compact)

    out = {}
    for name, fn in (("fused_us", fused), ("separate_us", separate)):
        fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        out[name] = round(a.elapsed_time(b) * 1e3 / reps, 2)
    return out


def setup_eviction(dev, name="eviction"):
    """The eviction step (or, name "tiny", the tiny workload's step: 1 layer, 2
    heads x 64 fp32, 8 chunks of 64 rows, chunks 1-5 scored)."""
    import compaction_dp_score_amd as dp
    import dpsynth
    from compaction_dp_score_amd.step import PruneStep
    w = dpsynth.WORKLOADS[name]
    T, H, D, L = w.seq_len, w.n_heads, w.head_dim, w.n_layers
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    esz = w.elem_size
    k_src, v_src, k_dst, v_dst = [], [], [], []
    for l in range(L):
        k = torch.empty((T, H, D), dtype=tdt, device=dev)
        v = torch.empty((T, H, D), dtype=tdt, device=dev)
        dpsynth.kv_fill_device(k, w.dtype, w.seed, dpsynth.STREAM_K, l, T, H * D)
        dpsynth.kv_fill_device(v, w.dtype, w.seed, dpsynth.STREAM_V, l, T, H * D)
        k_src.append(k)
        v_src.append(v)
        k_dst.append(torch.empty_like(k))
        v_dst.append(torch.empty_like(v))
    x0, xf = dpsynth.score_inputs(w)
    theta = dpsynth.rope_theta(w.rope_pairs, w.rope_base)
    ft, fp = dpsynth.frame_tables(w)
    rope = dict(theta=torch.from_numpy(theta).to(dev), frame_t=torch.from_numpy(ft).to(dev),
                frame_phase=torch.from_numpy(fp).to(dev), q0=w.q0, knee=w.rope_knee,
                inv_factor=1.0 / w.rope_factor, key_layout=KEY_LAYOUT)
    phase0 = rope["frame_phase"].clone()
    step = PruneStep(k_src=k_src, v_src=v_src, k_dst=k_dst, v_dst=v_dst, seq_len=T,
                     sink_len=w.sink_len, window_len=w.window_len, scored_begin=w.scored_begin,
                     n_scored=w.n_scored, gamma=w.gamma, d=w.d,
                     row_frame=torch.from_numpy(dpsynth.row_frame(w)).to(dev), rope=rope)
    x0d, xfd = torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev)
    gt = Timer()
    st = Timer()

    def run(timed):
        rope["frame_phase"].copy_(phase0)
        if timed:
            st.start()
        dp.dp_score_index(x0d, xfd, w.d, w.d, step.policy, step.ell, step.keep, step.idx,
                          step.n_kept, step.row_frame_src, step.row_frame_dst, step.ws_index,
                          step.dev_error)
        if timed:
            st.stop()
            gt.start()
        dp.dp_gather_kv(step.kv, step.idx, step.n_kept, step.row_frame_dst, step.rope,
                        step.ws_rope)
        if timed:
            gt.stop()

    def accounting():
        n = int(step.n_kept.item())
        assert int(step.dev_error.item()) == 0
        row = H * D * esz
        gather = n * row * 2 * 2 * L
        index = w.n_scored * (8 * w.d) + T + 12 * n        # scores in, keep out, idx + frames
        return dict(n_kept=n, gather_bytes=gather, score_timer=st, index_bytes=index,
                    index_compare=index_compare(step, x0d, xfd, w.d),
                    order_sensitive=order_sensitive(x0, xf, w.d, w.gamma),
                    step_bytes=gather + index, n_scored=w.n_scored,
                    config={"workload": name, "layers": L, "heads": H, "head_dim": D,
                            "kv_dtype": w.dtype, "tokens": T, "chunk_tokens": w.chunk_tokens,
                            "sink_chunks": w.sink_chunks, "window_chunks": w.window_chunks,
                            "scored_tokens": w.n_scored, "d": w.d, "gamma": w.gamma,
                            "rope_pairs": w.rope_pairs, "rope_knee_frames": w.rope_knee,
                            "rope_factor": w.rope_factor, "kept_tokens": n,
                            "pr_step": 1 - n / T})

    def cpu_baseline(seconds):
        if name == "tiny":
            return cpu_baseline_tiny(w, seconds)
        return cpu_baseline_eviction(w, x0, xf, theta, ft, fp, seconds)

    return run, gt, accounting, cpu_baseline


def host_info():
    """The host the CPU legs run on: CPU model, available memory, the cores
    this process may run on, and the OpenMP threads the oracle gets."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next(l.split(":", 1)[1].strip() for l in f if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    mem = None
    try:
        with open("/proc/meminfo") as f:
            mem = next(int(l.split()[1]) for l in f if l.startswith("MemAvailable")) / 1e6
    except (OSError, StopIteration):
        pass
    cores = len(os.sched_getaffinity(0))
    omp = int(os.environ.get("OMP_NUM_THREADS") or cores)
    return {"cpu_model": model, "mem_available_gb": None if mem is None else round(mem, 1),
            "affinity_cores": cores, "omp_threads": omp}


def _timed(fn):
    t0 = time.perf_counter()
    out = fn()
    return out, time.perf_counter() - t0


def _tiled_layers(n_layers, rows, row_elems, seed, tile_rows=512):
    """Host key/value stand-ins: one random bf16 tile repeated over the rows
    (the oracle's work does not depend on the values)."""
    rng = np.random.default_rng(seed)
    tile = rng.integers(0, 1 << 16, (tile_rows, row_elems), dtype=np.uint16) & np.uint16(0xBFFF)
    out = np.empty((n_layers, rows, row_elems), np.uint16)
    for l in range(n_layers):
        for r0 in range(0, rows, tile_rows):
            n = min(tile_rows, rows - r0)
            out[l, r0:r0 + n] = tile[:n]
    return out


def _cpu_record(step_bytes, total_s, threads, sample, steps, extra=None):
    rec = {"value": step_bytes / total_s / 1e9, "unit": "GB/s", "cores": threads,
           "kind": "oracle", "sample": sample, "step_seconds": total_s,
           "step_seconds_by_step": {k: round(v, 6) for k, v in steps.items()}}
    rec.update(host_info())
    if extra:
        rec.update(extra)
    return rec


def cpu_baseline_eviction(w, x0, xf, theta, ft, fp, seconds):
    """Oracle (as it is) on a layer sample of the eviction step: score, mask
    and index once, then gather of K and V and the K re-index on as many
    layers as fit the time budget (the gather's parallel loop is over layers,
    so as many layers at a time as the oracle has threads); scaled to 40
    layers."""
    import dpsynth
    import oracle
    T, H, D, L = w.seq_len, w.n_heads, w.head_dim, w.n_layers
    omp = host_info()["omp_threads"]
    rf = dpsynth.row_frame(w)
    ell, t_score = _timed(lambda: oracle.score_f32(x0, xf, w.d))
    keep, t_mask = _timed(lambda: oracle.mask(ell, T, w.sink_len, w.window_len, w.scored_begin,
                                              w.n_scored, w.gamma))
    (idx, rf2), t_index = _timed(lambda: (lambda i: (i, oracle.gather_i32(rf, i)))(
        oracle.compact(keep)))
    tables, t_tab = _timed(lambda: oracle.rope_frames(ft, fp, w.q0, w.rope_knee,
                                                      np.float32(1.0 / w.rope_factor), theta))
    n_layers = max(1, min(L, omp))
    src = _tiled_layers(n_layers, T, H * D, 1).reshape(n_layers, T, H, D)
    g_times, r_times = [], []
    done = 0
    t_start = time.perf_counter()
    while done < L:
        (kd, vd), tg = _timed(lambda: (oracle.gather(src, idx), oracle.gather(src, idx)))
        _, tr = _timed(lambda: [oracle.rope_rows(kd[l], rf2, 0, tables) for l in range(n_layers)])
        g_times.append(tg / n_layers)
        r_times.append(tr / n_layers)
        done += n_layers
        del kd, vd
        if time.perf_counter() - t_start > seconds:
            break
    steps = {"score": t_score, "mask": t_mask, "index": t_index,
             "gather": L * float(np.median(g_times)),
             "reindex": t_tab + L * float(np.median(r_times))}
    total = sum(steps.values())
    n = idx.shape[0]
    step_bytes = n * H * D * 2 * 2 * 2 * L + w.n_scored * 8 * w.d + T + 2 * T + 12 * n
    return _cpu_record(step_bytes, total, omp,
                       "score, mask and index of the full step once; gather of K and V and the "
                       "K re-index on %d layers at a time (%d layer passes timed, median), scaled "
                       "to 40 layers" % (n_layers, done), steps,
                       {"tokens_scored_per_s": w.n_scored / total})


def cpu_baseline_reindex(w, rows, rf_kept, moved_rows, seconds):
    """Oracle re-index (per-frame tables, then every retained row of a layer)
    on single layers of the one-minute cache until the time budget, scaled to
    40 layers (the row loop is the parallel one)."""
    import oracle
    H, D, L = w.n_heads, w.head_dim, w.n_layers
    omp = host_info()["omp_threads"]
    theta = __import__("dpsynth").rope_theta(w.rope_pairs, w.rope_base)
    ft = np.arange(w.n_frames, dtype=np.float32)
    tables, t_tab = _timed(lambda: oracle.rope_frames(ft, ft, w.q0, w.rope_knee,
                                                      np.float32(1.0 / w.rope_factor), theta))
    src = _tiled_layers(1, rows, H * D, 2).reshape(rows, H, D)
    times = []
    t_start = time.perf_counter()
    while len(times) < L:
        k = src.copy()
        _, tr = _timed(lambda: oracle.rope_rows(k, rf_kept, 0, tables))
        times.append(tr)
        if time.perf_counter() - t_start > seconds:
            break
    steps = {"reindex": t_tab + L * float(np.median(times))}
    total = steps["reindex"]
    b = moved_rows * H * (2 * w.rope_pairs * 2) * 2 * L
    return _cpu_record(b, total, omp, "the K re-index of %d of 40 layers (%d retained rows each), "
                       "median per layer, scaled to 40 layers" % (len(times), rows), steps)


def cpu_baseline_prefix(w, x0, xf, slab_layers, seconds):
    """Oracle prefix pruning: score, mask and index of all 355,680 scored
    rows once; the K and V gather timed on a row sample (the first 1/16 of the
    rows and their kept rows, as many layers at a time as the oracle has
    threads), scaled by kept rows to the slab's 20 layers."""
    import oracle
    T, H, D = w.seq_len, w.n_heads, w.head_dim
    omp = host_info()["omp_threads"]
    ell, t_score = _timed(lambda: oracle.score_f32(x0, xf, w.d))
    keep, t_mask = _timed(lambda: oracle.mask(ell, T, w.sink_len, w.window_len, w.scored_begin,
                                              w.n_scored, w.gamma))
    idx, t_index = _timed(lambda: oracle.compact(keep))
    ts = T // 16
    sub = idx[idx < ts]
    n_layers = max(1, min(slab_layers, omp))
    src = _tiled_layers(n_layers, ts, H * D, 3).reshape(n_layers, ts, H, D)
    times = []
    t_start = time.perf_counter()
    while True:
        _, tg = _timed(lambda: (oracle.gather(src, sub), oracle.gather(src, sub)))
        times.append(tg / n_layers / sub.shape[0])            # seconds per kept row and layer
        if time.perf_counter() - t_start > seconds or len(times) >= 8:
            break
    n = idx.shape[0]
    steps = {"score": t_score, "mask": t_mask, "index": t_index,
             "gather": float(np.median(times)) * n * slab_layers}
    total = sum(steps.values())
    step_bytes = n * H * D * 2 * 2 * 2 * slab_layers + w.n_scored * 8 * w.d + T + 4 * n
    return _cpu_record(step_bytes, total, omp,
                       "score, mask and index of the full prefix once; the K and V gather of the "
                       "%d kept rows among the first %d rows, %d layers at a time (%d passes, "
                       "median per kept row), scaled to %d kept rows x %d layers"
                       % (sub.shape[0], ts, n_layers, len(times), n, slab_layers), steps,
                       {"tokens_scored_per_s": w.n_scored / total})


def cpu_baseline_hs(w, x0, xf, cls, seconds):
    """Oracle DeCoPrune-HS step: score, both class masks and index lists and
    the per-head offsets of the full workload once; the per-head gather of K
    and V and the per-head K re-index timed on one layer restricted to the
    first 1/8 of the rows, scaled by head rows to 40 layers."""
    import dpsynth
    import oracle
    T, H, D, L = w.seq_len, w.n_heads, w.head_dim, w.n_layers
    omp = host_info()["omp_threads"]
    ell, t_score = _timed(lambda: oracle.score_f32(x0, xf, w.d))

    def masks():
        return (oracle.mask(None, T, w.sink_len, w.window_len, w.scored_begin, w.n_scored,
                            w.gamma, streaming=True),
                oracle.mask(ell, T, w.sink_len, w.window_len, w.scored_begin, w.n_scored, w.gamma))
    (ks, kd), t_mask = _timed(masks)
    (lists, off), t_index = _timed(lambda: (lambda ls: (ls, oracle.hs_offsets(
        cls, np.array([len(x) for x in ls], np.int64))))([oracle.compact(ks), oracle.compact(kd)]))
    rf = dpsynth.row_frame(w)
    theta = dpsynth.rope_theta(w.rope_pairs, w.rope_base)
    ft = np.arange(w.n_frames, dtype=np.float32)
    tables = oracle.rope_frames(ft, ft, w.q0, w.rope_knee, np.float32(1.0 / w.rope_factor), theta)
    ts = T // 8
    sub_lists = [x[x < ts] for x in lists]
    sub_lens = np.array([len(x) for x in sub_lists], np.int64)
    sub_off = oracle.hs_offsets(cls[:1], sub_lens)
    src = _tiled_layers(1, ts, H * D, 4).reshape(ts, H, D)
    frames = np.concatenate([rf[sub_lists[c]] for c in cls[0]]).astype(np.int32)
    g_times, r_times = [], []
    t_start = time.perf_counter()
    while True:
        out_k = np.empty((int(sub_off[-1]), D), np.uint16)
        out_v = np.empty_like(out_k)
        _, tg = _timed(lambda: (oracle.hs_gather_layer(src, 0, cls[:1], sub_lists, sub_off, out_k),
                                oracle.hs_gather_layer(src, 0, cls[:1], sub_lists, sub_off, out_v)))
        _, tr = _timed(lambda: oracle.rope_headrows(out_k, frames, 0, tables))
        g_times.append(tg / sub_off[-1])
        r_times.append(tr / sub_off[-1])
        if time.perf_counter() - t_start > seconds or len(g_times) >= 8:
            break
    total_rows = int(off[-1])
    steps = {"score": t_score, "mask": t_mask, "index": t_index,
             "gather": float(np.median(g_times)) * total_rows,
             "reindex": float(np.median(r_times)) * total_rows}
    total = sum(steps.values())
    step_bytes = total_rows * D * 2 * 2 * 2 + w.n_scored * 8 * w.d + 2 * T
    return _cpu_record(step_bytes, total, omp,
                       "score, masks, index lists and offsets of the full step once; the per-head "
                       "gather of K and V and the K re-index of layer 0 over the first %d rows "
                       "(%d head rows; %d passes, median per head row), scaled to %d head rows"
                       % (ts, int(sub_off[-1]), len(g_times), total_rows), steps,
                       {"tokens_scored_per_s": w.n_scored / total})


def cpu_baseline_tiny(w, seconds):
    """The whole tiny step through the oracle (prune_step), repeated for about
    a second; median step time."""
    import dpsynth
    import oracle
    T, H, D = w.seq_len, w.n_heads, w.head_dim
    x0, xf = dpsynth.score_inputs(w)
    kh = dpsynth.kv_layer_host("f32", w.seed, dpsynth.STREAM_K, 0, T, H * D).reshape(1, T, H, D)
    vh = dpsynth.kv_layer_host("f32", w.seed, dpsynth.STREAM_V, 0, T, H * D).reshape(1, T, H, D)
    rf = dpsynth.row_frame(w)
    theta = dpsynth.rope_theta(w.rope_pairs, w.rope_base)
    ft, fp = dpsynth.frame_tables(w)
    pol = dict(seq_len=T, sink_len=w.sink_len, window_len=w.window_len,
               scored_begin=w.scored_begin, n_scored=w.n_scored, gamma=w.gamma)
    rope = dict(theta=theta, frame_t=ft, frame_phase=fp, q0=w.q0, knee=w.rope_knee,
                inv_factor=np.float32(1.0 / w.rope_factor))
    times = []
    t_start = time.perf_counter()
    while time.perf_counter() - t_start < min(seconds, 1.0) or len(times) < 3:
        out, t = _timed(lambda: oracle.prune_step(x0, xf, w.d, pol, kh, vh, rf, rope))
        times.append(t)
    n = out["idx"].shape[0]
    total = float(np.median(times))
    step_bytes = n * H * D * 4 * 2 * 2 + w.n_scored * 8 * w.d + T + 12 * n
    return _cpu_record(step_bytes, total, host_info()["omp_threads"],
                       "the whole step (score, mask, index, gather of K "
                       "and V, K re-index) on the tiny workload, %d repetitions, median"
                       % len(times), {"step": total},
                       {"tokens_scored_per_s": w.n_scored / total})


def setup_reindex(dev):
    import compaction_dp_score_amd as dp
    import dpsynth
    w = dpsynth.WORKLOADS["reindex"]
    T, H, D, L = w.seq_len, w.n_heads, w.head_dim, w.n_layers
    keep = dpsynth.retained_keep(w)
    kept = np.flatnonzero(keep)
    rows = kept.shape[0]
    rf_full = dpsynth.row_frame(w)
    rf = torch.from_numpy(rf_full[kept].astype(np.int32)).to(dev)
    ks = []
    for l in range(L):
        k = torch.empty((rows, H, D), dtype=torch.bfloat16, device=dev)
        dpsynth.kv_fill_device(k, "bf16", w.seed, dpsynth.STREAM_K, l, rows, H * D)
        ks.append(k)
    arr = dp.ptr_array(ks, dev)
    theta = torch.from_numpy(dpsynth.rope_theta(w.rope_pairs, w.rope_base)).to(dev)
    ft, fp = dpsynth.frame_tables(w)
    ftd, fpd = torch.from_numpy(ft).to(dev), torch.from_numpy(fp).to(dev)
    phase0 = fpd.clone()
    rope = make_rope(theta, ftd, fpd, w.q0, w.rope_knee, 1.0 / w.rope_factor)
    ws = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                     dtype=torch.float32, device=dev)
    gt = Timer()
    moved_rows = int(np.count_nonzero(rf_full[kept] < (w.n_frames - w.window_chunks * w.frames_per_chunk)))

    def run(timed):
        fpd.copy_(phase0)
        if timed:
            gt.start()
        dp.dp_rope_reindex(arr, L, H, D, dp.DP_BF16, rows, None, rf, rope, ws)
        if timed:
            gt.stop()

    def accounting():
        b = moved_rows * H * (2 * w.rope_pairs * 2) * 2 * L
        return dict(n_kept=rows, gather_bytes=b, step_bytes=b, n_scored=0,
                    config={"workload": "reindex", "layers": L, "heads": H, "head_dim": D,
                            "kv_dtype": "bf16", "retained_rows": rows, "reindexed_rows": moved_rows,
                            "rope_pairs": w.rope_pairs, "q0": w.q0,
                            "key_layout": "split" if KEY_LAYOUT else "interleaved"},
                    context=None if ARGS.no_fullkv else other_layout_ms())

    def other_layout_ms(reps=3):
        # the same pass on the other key layout (the same bytes of keys, read as
        # that layout), phase table restored before each call
        other = 1 - KEY_LAYOUT
        rope_o = dp.make_rope(theta, ftd, fpd, w.q0, w.rope_knee, 1.0 / w.rope_factor,
                              key_layout=other)
        ms = []
        for _ in range(reps + 1):
            fpd.copy_(phase0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            dp.dp_rope_reindex(arr, L, H, D, dp.DP_BF16, rows, None, rf, rope_o, ws)
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        fpd.copy_(phase0)
        t = float(np.median(ms[1:]))
        b = moved_rows * H * (2 * w.rope_pairs * 2) * 2 * L
        return {"other_layout": "split" if other else "interleaved", "ms": round(t, 4),
                "gbs": round(b / t / 1e6, 1)}

    def cpu_baseline(seconds):
        return cpu_baseline_reindex(w, rows, rf_full[kept].astype(np.int32), moved_rows, seconds)

    return run, gt, accounting, cpu_baseline


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16


def flops_record(args, acc, ms, k_ms):
    """JSON record of a contraction workload (attention): TFLOP/s against the
    dense bf16 MFMA peak."""
    k_ms = k_ms / acc.get("timer_launches", 1)
    tf = acc["step_flops"] / (ms * 1e-3) / 1e12
    ktf = acc["flops_per_launch"] / (k_ms * 1e-3) / 1e12
    rec = {"metric": acc.get("metric", "attention TFLOP/s over the compacted cache"),
           "value": round(tf, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": acc["config"],
           "roofline": {"bound": "mfma", "kernel": KERNELS[args.workload][0],
                        "achieved": round(ktf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(ktf / MFMA_BF16_PEAK_TFLOPS, 4),
                        "traffic": read_traffic(args.workload),
                        "flops_per_launch": acc["flops_per_launch"],
                        "launch_ms": round(k_ms, 4)}}
    rec["copy_ceiling_gbs"] = round(copy_ceiling(torch.device("cuda:0"), CALIB_BYTES), 2)
    if acc.get("context"):
        rec["context"] = acc["context"]
    if acc.get("full_ms"):
        rec["fullkv"] = {"ms": round(acc["full_ms"], 4),
                         "tflops": round(acc["full_flops"] / (acc["full_ms"] * 1e-3) / 1e12, 2),
                         "speedup_of_compaction": round(acc["full_ms"] / k_ms, 3)}
    return rec


def copy_ceiling(dev, nbytes, reps=5):
    """Read+write GB/s of a plain 16-byte-vector device copy of nbytes, in
    the same run (the practical HBM ceiling a gather can approach)."""
    import dpsynth
    src = torch.empty(nbytes // 2, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    dpsynth.device_copy(dst, src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dpsynth.device_copy(dst, src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2.0 * nbytes / (ms * 1e-3) / 1e9


def summarize_pmc(workload, fetch_dir, write_dir):
    """Per-launch HBM bytes of the workload's dominant kernel from rocprofv3
    counter CSVs, each counter scaled by what it reads for the calibration
    copy (CALIB_BYTES read and written by calib_copy_kernel in the same run)."""
    import csv
    import glob
    kname = KERNELS[workload][0]

    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        assert files, "no counter_collection.csv under %s" % d
        vals = {"kernel": [], "calib": []}
        for fn in files:
            for r in csv.DictReader(open(fn)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                if ("::" + kname + "<") in name or ("::" + kname + "(") in name:
                    vals["kernel"].append(float(r["Counter_Value"]))
                elif "calib_copy_kernel" in name:
                    vals["calib"].append(float(r["Counter_Value"]))
        assert vals["kernel"] and vals["calib"], (d, counter, {k: len(v) for k, v in vals.items()})
        return (sum(vals["kernel"]) / len(vals["kernel"]), len(vals["kernel"]),
                sum(vals["calib"]) / len(vals["calib"]))

    fk, fn_, fc = per_kernel(fetch_dir, "FETCH_SIZE")
    wk, wn, wc = per_kernel(write_dir, "WRITE_SIZE")
    fscale = CALIB_BYTES / (fc * 1024.0)
    wscale = CALIB_BYTES / (wc * 1024.0)
    rd = fk * 1024.0 * fscale
    wr = wk * 1024.0 * wscale
    path = traffic_path(workload)
    with open(path, "w") as out:
        out.write("# HBM traffic of %s on the %s workload, per dispatch, from rocprofv3 counters\n"
                  % (kname, workload))
        out.write("# commands (from the repository root; %s as the dominant kernel):\n" % kname)
        out.write("#   rocprofv3 --pmc FETCH_SIZE -d %s -o run -f csv -- python bench.py "
                  "--workload %s %s --steps 2 --warmup 0\n" % (fetch_dir, workload,
                                                             profile_flags(workload)))
        out.write("#   rocprofv3 --pmc WRITE_SIZE -d %s -o run -f csv -- python bench.py "
                  "--workload %s %s --steps 2 --warmup 0\n" % (write_dir, workload,
                                                             profile_flags(workload)))
        out.write("#   python bench.py --workload %s --summarize-pmc %s %s\n"
                  % (workload, fetch_dir, write_dir))
        out.write("# scale: each counter divided by what it reads for calib_copy_kernel, which\n"
                  "# reads and writes %d bytes (a plain 16-byte-vector copy)\n" % CALIB_BYTES)
        out.write("kernel: %s\n" % kname)
        out.write("source_sha: %s\n" % kernel_sources_sha(workload))
        out.write("dispatches_fetch: %d\n" % fn_)
        out.write("dispatches_write: %d\n" % wn)
        out.write("fetch_kib_per_dispatch: %.1f\n" % fk)
        out.write("write_kib_per_dispatch: %.1f\n" % wk)
        out.write("calib_fetch_kib: %.1f\n" % fc)
        out.write("calib_write_kib: %.1f\n" % wc)
        out.write("fetch_scale: %.4f\n" % fscale)
        out.write("write_scale: %.4f\n" % wscale)
        out.write("hbm_read_bytes_per_launch: %.0f\n" % rd)
        out.write("hbm_write_bytes_per_launch: %.0f\n" % wr)
        out.write("hbm_bytes_per_launch: %.0f\n" % (rd + wr))
    print(open(path).read())


def _fill_layers(dev, w, rows, layers, stream_id):
    import dpsynth
    out = []
    for l in layers:
        t = torch.empty((rows, w.n_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
        dpsynth.kv_fill_device(t, "bf16", w.seed, stream_id, l, rows, w.n_heads * w.head_dim)
        out.append(t)
    return out


def setup_append(dev):
    """The eviction step in the ring layout: per layer one buffer
    [sink | ring of 4 chunk slots | history]; the chunk in ring slot 0 leaves
    the window: it is scored (6,240 tokens), its kept rows are appended at the
    history tail (K and V, 40 layers), and the old keys (the sink and the
    history, here the appended rows) are re-indexed in place for q0 = 20 by
    one dp_rope_prepare and two dp_rope_apply calls.  The tail, the slot's row frames
    and the phase table are restored before each step (small device copies)."""
    import compaction_dp_score_amd as dp
    import dpsynth
    w = dpsynth.WORKLOADS["eviction"]
    T, H, D, L, C = w.seq_len, w.n_heads, w.head_dim, w.n_layers, w.chunk_tokens
    cap = T + C                                     # room for one chunk of history
    slot_begin = C                                  # ring slot 0 holds the leaving chunk
    ks = _fill_layers(dev, w, cap, range(L), dpsynth.STREAM_K)
    vs = _fill_layers(dev, w, cap, range(L), dpsynth.STREAM_V)
    x0, xf = dpsynth.score_inputs(w)
    x0d, xfd = torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev)
    rf_full = np.full(cap, -1, np.int32)
    rf_full[:T] = dpsynth.row_frame(w)
    rf0 = torch.from_numpy(rf_full).to(dev)
    rf = rf0.clone()
    kv = dp.dp_kv_inplace()
    arr_k, arr_v = dp.ptr_array(ks, dev), dp.ptr_array(vs, dev)
    kv.k_layers, kv.v_layers = arr_k.data_ptr(), arr_v.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dp.DP_BF16
    kv.capacity = cap
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv.dev_error = err.data_ptr()
    tail0 = torch.tensor([T], dtype=torch.int64, device=dev)
    tail = tail0.clone()
    pol = dp.make_policy(C, 0, 0, 0, C, w.gamma)
    keep = torch.empty(C, dtype=torch.uint8, device=dev)
    idx = torch.empty(C, dtype=torch.int32, device=dev)
    nk = torch.zeros(1, dtype=torch.int64, device=dev)
    ws_c = torch.empty(dp.dp_compact_workspace_bytes(C) // 4 + 1, dtype=torch.int32, device=dev)
    theta = torch.from_numpy(dpsynth.rope_theta(w.rope_pairs, w.rope_base)).to(dev)
    ft, fp = dpsynth.frame_tables(w)
    ftd, fpd = torch.from_numpy(ft).to(dev), torch.from_numpy(fp).to(dev)
    phase0 = fpd.clone()
    rope = make_rope(theta, ftd, fpd, w.q0, w.rope_knee, 1.0 / w.rope_factor)
    ws_r = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    gt = Timer()
    at = Timer()
    keep_alive = [arr_k, arr_v]

    def run(timed):
        tail.copy_(tail0)
        rf.copy_(rf0)
        fpd.copy_(phase0)
        dp.dp_score_mask(x0d, xfd, w.d, w.d, pol, None, keep)
        dp.dp_compact_index(keep, C, idx, nk, None, None, ws_c)
        if timed:
            at.start()
        dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf)
        if timed:
            at.stop()
        dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
        if timed:
            gt.start()
        # old keys only: the sink, and the history [T, tail); the window ring is skipped
        dp.dp_rope_apply(arr_k, L, H, D, dp.DP_BF16, 0, w.sink_len, None, rf, rope, ws_r)
        dp.dp_rope_apply(arr_k, L, H, D, dp.DP_BF16, T, cap, tail, rf, rope, ws_r)
        if timed:
            gt.stop()

    def accounting():
        assert keep_alive and err.item() == 0
        n = int(nk.item())
        append = n * H * D * 2 * 2 * 2 * L
        rotated = (w.sink_len + n) * H * L            # head rows whose frame moves
        reindex = rotated * 2 * w.rope_pairs * 2 * 2
        score = C * (8 * w.d + 1)
        return dict(n_kept=n, gather_bytes=reindex, step_bytes=append + reindex + score,
                    n_scored=C, append_timer=at, append_bytes=append, timer_launches=2,
                    config={"workload": "append", "layout": "sink | ring of 4 chunk slots | history",
                            "layers": L, "heads": H, "head_dim": D, "kv_dtype": "bf16",
                            "tokens": T, "scored_tokens": C, "kept_tokens": n,
                            "appended_bytes": append, "reindexed_head_rows": rotated,
                            "rope_pairs": w.rope_pairs, "q0": w.q0})

    return run, gt, accounting, None


def setup_steady(dev):
    """A steady-state step of the one-minute rollout in the ring layout: per
    layer [sink | ring of 4 chunk slots (chunks 56-59) | history (the retained
    rows of chunks 1-55) | room for one chunk].  Chunk 56 leaves the window for
    q0 = 240: it is scored and indexed in one launch; every old key (sink and
    history, all past the knee at q0 = 236 and 240) moves by the uniform step
    F (1 - 1/c) = 3.5 frames (two dp_rope_shift launches); dp_rope_prepare
    writes the per-frame tables and dp_append_kept appends the chunk's kept
    rows with their first re-index fused.  The tail, the slot's row frames and
    the phase table are restored before each step.  For context the general
    path (append, then dp_rope_apply over the sink and the whole history) is
    timed on the same buffers."""
    import compaction_dp_score_amd as dp
    import dpsynth
    w = dpsynth.WORKLOADS["reindex"]
    H, D, L, C, tpf = w.n_heads, w.head_dim, w.n_layers, w.chunk_tokens, w.tokens_per_frame
    keep_full = dpsynth.retained_keep(w)
    hist_rows = np.flatnonzero(keep_full[C:56 * C]) + C          # retained rows of chunks 1..55
    n_hist = hist_rows.shape[0]
    hb = 5 * C                                                    # sink + 4 ring slots
    cap = hb + n_hist + C
    slot_begin = C                                                # ring slot 0: chunk 56
    rf_host = np.full(cap, -1, np.int32)
    rf_host[:C] = np.arange(C) // tpf
    rf_host[C:hb] = (56 * C + np.arange(4 * C)) // tpf
    rf_host[hb:hb + n_hist] = hist_rows // tpf
    ks = _fill_layers(dev, w, cap, range(L), dpsynth.STREAM_K)
    vs = _fill_layers(dev, w, cap, range(L), dpsynth.STREAM_V)
    x0, xf = dpsynth.score_inputs(dpsynth.WORKLOADS["eviction"])  # one chunk of scores
    x0d, xfd = torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev)
    rf0 = torch.from_numpy(rf_host).to(dev)
    rf = rf0.clone()
    kv = dp.dp_kv_inplace()
    arr_k, arr_v = dp.ptr_array(ks, dev), dp.ptr_array(vs, dev)
    kv.k_layers, kv.v_layers = arr_k.data_ptr(), arr_v.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dp.DP_BF16
    kv.capacity = cap
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv.dev_error = err.data_ptr()
    tail0 = torch.tensor([hb + n_hist], dtype=torch.int64, device=dev)
    tail = tail0.clone()
    pol = dp.make_policy(C, 0, 0, 0, C, w.gamma)
    keep = torch.empty(C, dtype=torch.uint8, device=dev)
    idx = torch.empty(C, dtype=torch.int32, device=dev)
    nk = torch.zeros(1, dtype=torch.int64, device=dev)
    ws_si = torch.zeros(dp.dp_score_index_workspace_bytes(C) // 8 + 1, dtype=torch.int64, device=dev)
    theta = torch.from_numpy(dpsynth.rope_theta(w.rope_pairs, w.rope_base)).to(dev)
    ft, fp = dpsynth.frame_tables(w)
    ftd, fpd = torch.from_numpy(ft).to(dev), torch.from_numpy(fp).to(dev)
    ws_r = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    # the phases the old keys carry after the previous step (q0 = 236)
    dp.dp_rope_prepare(make_rope(theta, ftd, fpd, w.q0 - 4, w.rope_knee, 1.0 / w.rope_factor),
                       D, dp.DP_BF16, ws_r)
    phase0 = fpd.clone()
    rope = make_rope(theta, ftd, fpd, w.q0, w.rope_knee, 1.0 / w.rope_factor)
    step_frames = 4 * (1.0 - 1.0 / w.rope_factor)                 # 3.5
    ws_s = torch.empty(dp.dp_rope_shift_workspace_bytes(w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    gt = Timer()
    keep_alive = [arr_k, arr_v]

    def restore():
        tail.copy_(tail0)
        rf.copy_(rf0)
        fpd.copy_(phase0)

    def run(timed):
        restore()
        dp.dp_score_index(x0d, xfd, w.d, w.d, pol, None, keep, idx, nk, None, None, ws_si, err)
        if timed:
            gt.start()
        dp.dp_rope_shift(arr_k, L, H, D, dp.DP_BF16, 0, C, None, theta, 0, w.rope_pairs,
                         step_frames, ws_s, key_layout=KEY_LAYOUT)
        dp.dp_rope_shift(arr_k, L, H, D, dp.DP_BF16, hb, cap, tail, theta, 0, w.rope_pairs,
                         step_frames, ws_s, key_layout=KEY_LAYOUT)
        if timed:
            gt.stop()
        dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
        dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf, rope, ws_r)

    def general_ms(reps=5):
        def once():
            restore()
            dp.dp_score_index(x0d, xfd, w.d, w.d, pol, None, keep, idx, nk, None, None, ws_si,
                              err)
            dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf)
            dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
            dp.dp_rope_apply(arr_k, L, H, D, dp.DP_BF16, 0, C, None, rf, rope, ws_r)
            dp.dp_rope_apply(arr_k, L, H, D, dp.DP_BF16, hb, cap, tail, rf, rope, ws_r)
        once()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            once()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def accounting():
        assert keep_alive and err.item() == 0
        n = int(nk.item())
        shifted = (C + n_hist) * H * L                  # head rows moved by the uniform step
        shift_bytes = shifted * 2 * w.rope_pairs * 2 * 2
        append = n * H * D * 2 * 2 * 2 * L
        score = C * (8 * w.d + 1)
        return dict(n_kept=n, gather_bytes=shift_bytes, timer_launches=2,
                    step_bytes=shift_bytes + append + score, n_scored=C,
                    context={"general_path_ms_per_step": round(general_ms(), 4)},
                    config={"workload": "steady", "layout": "sink | ring of 4 chunk slots | history",
                            "layers": L, "heads": H, "head_dim": D, "kv_dtype": "bf16",
                            "history_rows": int(n_hist), "scored_tokens": C, "kept_tokens": n,
                            "shifted_head_rows": shifted, "uniform_step_frames": step_frames,
                            "rope_pairs": w.rope_pairs, "q0": w.q0})

    return run, gt, accounting, None


def setup_steady_lazy(dev):
    """The steady-state step of setup_steady on the compressed time axis: the
    old keys (sink and history) carry the phase t/c since they passed the
    knee, so no old key is rewritten when q0 advances; attention turns the
    query back by the common term instead (dp_attention_lag).  Per step: the
    leaving chunk 56 is scored and indexed in one launch, dp_rope_prepare
    writes the per-frame tables (axis DP_AXIS_COMPRESSED: chunk 56's frames
    move from t to t/c, every other frame stays) and dp_append_kept appends
    its kept rows with that re-index fused.  The tail, the slot's row frames
    and the phase table are restored before each step.  For context the same
    step on the page's axis (two uniform shifts over the 32.4 GB of old keys,
    then the same append) is timed on the same buffers."""
    import compaction_dp_score_amd as dp
    import dpsynth
    w = dpsynth.WORKLOADS["reindex"]
    H, D, L, C, tpf = w.n_heads, w.head_dim, w.n_layers, w.chunk_tokens, w.tokens_per_frame
    keep_full = dpsynth.retained_keep(w)
    hist_rows = np.flatnonzero(keep_full[C:56 * C]) + C          # retained rows of chunks 1..55
    n_hist = hist_rows.shape[0]
    hb = 5 * C                                                    # sink + 4 ring slots
    cap = hb + n_hist + C
    slot_begin = C                                                # ring slot 0: chunk 56
    rf_host = np.full(cap, -1, np.int32)
    rf_host[:C] = np.arange(C) // tpf
    rf_host[C:hb] = (56 * C + np.arange(4 * C)) // tpf
    rf_host[hb:hb + n_hist] = hist_rows // tpf
    ks = _fill_layers(dev, w, cap, range(L), dpsynth.STREAM_K)
    vs = _fill_layers(dev, w, cap, range(L), dpsynth.STREAM_V)
    x0, xf = dpsynth.score_inputs(dpsynth.WORKLOADS["eviction"])  # one chunk of scores
    x0d, xfd = torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev)
    rf0 = torch.from_numpy(rf_host).to(dev)
    rf = rf0.clone()
    kv = dp.dp_kv_inplace()
    arr_k, arr_v = dp.ptr_array(ks, dev), dp.ptr_array(vs, dev)
    kv.k_layers, kv.v_layers = arr_k.data_ptr(), arr_v.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dp.DP_BF16
    kv.capacity = cap
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv.dev_error = err.data_ptr()
    tail0 = torch.tensor([hb + n_hist], dtype=torch.int64, device=dev)
    tail = tail0.clone()
    pol = dp.make_policy(C, 0, 0, 0, C, w.gamma)
    keep = torch.empty(C, dtype=torch.uint8, device=dev)
    idx = torch.empty(C, dtype=torch.int32, device=dev)
    nk = torch.zeros(1, dtype=torch.int64, device=dev)
    ws_si = torch.zeros(dp.dp_score_index_workspace_bytes(C) // 8 + 1, dtype=torch.int64, device=dev)
    theta = torch.from_numpy(dpsynth.rope_theta(w.rope_pairs, w.rope_base)).to(dev)
    ft, fp = dpsynth.frame_tables(w)
    ftd, fpd = torch.from_numpy(ft).to(dev), torch.from_numpy(fp).to(dev)
    ws_r = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    # the phases after the previous step (q0 = 236) on the compressed axis
    dp.dp_rope_prepare(make_rope(theta, ftd, fpd, w.q0 - 4, w.rope_knee, 1.0 / w.rope_factor,
                                    axis=dp.DP_AXIS_COMPRESSED), D, dp.DP_BF16, ws_r)
    phase0 = fpd.clone()
    rope = make_rope(theta, ftd, fpd, w.q0, w.rope_knee, 1.0 / w.rope_factor,
                        axis=dp.DP_AXIS_COMPRESSED)
    page_rope = make_rope(theta, ftd, fpd, w.q0, w.rope_knee, 1.0 / w.rope_factor)
    step_frames = 4 * (1.0 - 1.0 / w.rope_factor)                 # 3.5
    ws_s = torch.empty(dp.dp_rope_shift_workspace_bytes(w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    gt = Timer()
    keep_alive = [arr_k, arr_v]

    def restore():
        tail.copy_(tail0)
        rf.copy_(rf0)
        fpd.copy_(phase0)

    def run(timed):
        restore()
        dp.dp_score_index(x0d, xfd, w.d, w.d, pol, None, keep, idx, nk, None, None, ws_si, err)
        dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
        if timed:
            gt.start()
        dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf, rope, ws_r)
        if timed:
            gt.stop()

    def step():
        dp.dp_score_index(x0d, xfd, w.d, w.d, pol, None, keep, idx, nk, None, None, ws_si, err)
        dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
        dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf, rope, ws_r)

    def page_axis_ms(reps=5):
        def once():
            restore()
            dp.dp_score_index(x0d, xfd, w.d, w.d, pol, None, keep, idx, nk, None, None, ws_si,
                              err)
            dp.dp_rope_shift(arr_k, L, H, D, dp.DP_BF16, 0, C, None, theta, 0, w.rope_pairs,
                             step_frames, ws_s, key_layout=KEY_LAYOUT)
            dp.dp_rope_shift(arr_k, L, H, D, dp.DP_BF16, hb, cap, tail, theta, 0, w.rope_pairs,
                             step_frames, ws_s, key_layout=KEY_LAYOUT)
            dp.dp_rope_prepare(page_rope, D, dp.DP_BF16, ws_r)
            dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf, page_rope, ws_r)
        once()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            once()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def accounting():
        assert keep_alive and err.item() == 0
        n = int(nk.item())
        append = n * H * D * 2 * 2 * 2 * L
        score = C * (8 * w.d + 1)
        return dict(n_kept=n, gather_bytes=append, step_bytes=append + score, n_scored=C,
                    context=None if ARGS.no_fullkv else {
                        "page_axis_step_ms": round(page_axis_ms(), 4),
                        **step_ms_eager_and_graph(step, restore)},
                    config={"workload": "steady_lazy",
                            "layout": "sink | ring of 4 chunk slots | history",
                            "time_axis": "compressed (old keys at phase t/c)",
                            "layers": L, "heads": H, "head_dim": D, "kv_dtype": "bf16",
                            "history_rows": int(n_hist), "scored_tokens": C, "kept_tokens": n,
                            "appended_bytes": append, "rope_pairs": w.rope_pairs, "q0": w.q0})

    return run, gt, accounting, None


def setup_hs_ring(dev):
    """DeCoPrune-HS in the ring layout, at the HS workload's shape (40 layers,
    20 static and 20 dynamic heads per layer, 128 dims, bf16): each layer's
    heads are ordered class by class and each class keeps a token-major cache
    of its own; static [sink | 4 chunk slots], dynamic [sink | 4 chunk slots |
    history].  The history is a Bernoulli(0.15) sample of chunks 1-25 (the rate
    the gamma mask keeps), chunk 26 in slot 0 leaves the window at q0 = 120.
    Per step, on the compressed time axis: the leaving chunk is scored and
    indexed in one launch, dp_rope_prepare writes the frame tables, and
    dp_append_kept appends its kept rows to the dynamic caches of all layers
    with the re-index fused; the static class only retires the slot.  The
    tail, the row frames and the phase table are restored before each step.
    For context the same step on the page's axis (the uniform shift of every
    old key of both classes, then the same append) is timed on the same
    buffers."""
    import compaction_dp_score_amd as dp
    import dpsynth
    w = dpsynth.WORKLOADS["hs"]
    H, D, L, C, tpf = w.n_heads, w.head_dim, w.n_layers, w.chunk_tokens, w.tokens_per_frame
    HC = H // 2
    keep_full = dpsynth.retained_keep(w)
    hist_rows = np.flatnonzero(keep_full[C:26 * C]) + C          # retained rows of chunks 1..25
    n_hist = hist_rows.shape[0]
    hb = 5 * C                                                    # sink + 4 ring slots
    cap = hb + n_hist + C
    slot_begin = C                                                # ring slot 0: chunk 26
    rf_host = np.full(cap, -1, np.int32)
    rf_host[:C] = np.arange(C) // tpf
    rf_host[C:hb] = (26 * C + np.arange(4 * C)) // tpf
    rf_host[hb:hb + n_hist] = hist_rows // tpf

    def fill(rows, stream_id):
        out = []
        for l in range(L):
            t = torch.empty((rows, HC, D), dtype=torch.bfloat16, device=dev)
            dpsynth.kv_fill_device(t, "bf16", w.seed, stream_id, l, rows, HC * D)
            out.append(t)
        return out

    kd, vd = fill(cap, dpsynth.STREAM_K), fill(cap, dpsynth.STREAM_V)     # dynamic class
    ks = fill(hb, dpsynth.STREAM_K + 16)                                  # static class, K
    x0, xf = dpsynth.score_inputs(dpsynth.WORKLOADS["eviction"])          # one chunk of scores
    x0d, xfd = torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev)
    rf0 = torch.from_numpy(rf_host).to(dev)
    rf = rf0.clone()
    rf_s0 = torch.from_numpy(rf_host[:hb].copy()).to(dev)
    rf_s = rf_s0.clone()
    kv = dp.dp_kv_inplace()
    arr_k, arr_v, arr_ks = dp.ptr_array(kd, dev), dp.ptr_array(vd, dev), dp.ptr_array(ks, dev)
    kv.k_layers, kv.v_layers = arr_k.data_ptr(), arr_v.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, HC, D, dp.DP_BF16
    kv.capacity = cap
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv.dev_error = err.data_ptr()
    tail0 = torch.tensor([hb + n_hist], dtype=torch.int64, device=dev)
    tail = tail0.clone()
    pol = dp.make_policy(C, 0, 0, 0, C, w.gamma)
    keep = torch.empty(C, dtype=torch.uint8, device=dev)
    idx = torch.empty(C, dtype=torch.int32, device=dev)
    nk = torch.zeros(1, dtype=torch.int64, device=dev)
    ws_si = torch.zeros(dp.dp_score_index_workspace_bytes(C) // 8 + 1, dtype=torch.int64, device=dev)
    theta = torch.from_numpy(dpsynth.rope_theta(w.rope_pairs, w.rope_base)).to(dev)
    ft, fp = dpsynth.frame_tables(w)
    ftd, fpd = torch.from_numpy(ft).to(dev), torch.from_numpy(fp).to(dev)
    ws_r = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    # the phases after the previous step (q0 = 116) on the compressed axis
    dp.dp_rope_prepare(make_rope(theta, ftd, fpd, w.q0 - 4, w.rope_knee, 1.0 / w.rope_factor,
                                    axis=dp.DP_AXIS_COMPRESSED), D, dp.DP_BF16, ws_r)
    phase0 = fpd.clone()
    rope = make_rope(theta, ftd, fpd, w.q0, w.rope_knee, 1.0 / w.rope_factor,
                        axis=dp.DP_AXIS_COMPRESSED)
    page_rope = make_rope(theta, ftd, fpd, w.q0, w.rope_knee, 1.0 / w.rope_factor)
    step_frames = 4 * (1.0 - 1.0 / w.rope_factor)                 # 3.5
    ws_s = torch.empty(dp.dp_rope_shift_workspace_bytes(w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    gt = Timer()
    keep_alive = [arr_k, arr_v, arr_ks]

    def restore():
        tail.copy_(tail0)
        rf.copy_(rf0)
        rf_s.copy_(rf_s0)
        fpd.copy_(phase0)

    def run(timed):
        restore()
        dp.dp_score_index(x0d, xfd, w.d, w.d, pol, None, keep, idx, nk, None, None, ws_si, err)
        dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
        if timed:
            gt.start()
        dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf, rope, ws_r)
        if timed:
            gt.stop()
        rf_s[slot_begin:slot_begin + C].fill_(-1)                 # the static class drops it

    def step():
        dp.dp_score_index(x0d, xfd, w.d, w.d, pol, None, keep, idx, nk, None, None, ws_si, err)
        dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
        dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf, rope, ws_r)
        rf_s[slot_begin:slot_begin + C].fill_(-1)

    def page_axis_ms(reps=5):
        def once():
            restore()
            dp.dp_score_index(x0d, xfd, w.d, w.d, pol, None, keep, idx, nk, None, None, ws_si,
                              err)
            for arr in (arr_ks, arr_k):                            # both sinks
                dp.dp_rope_shift(arr, L, HC, D, dp.DP_BF16, 0, C, None, theta, 0, w.rope_pairs,
                                 step_frames, ws_s, key_layout=KEY_LAYOUT)
            dp.dp_rope_shift(arr_k, L, HC, D, dp.DP_BF16, hb, cap, tail, theta, 0, w.rope_pairs,
                             step_frames, ws_s, key_layout=KEY_LAYOUT)                    # dynamic history
            dp.dp_rope_prepare(page_rope, D, dp.DP_BF16, ws_r)
            dp.dp_append_kept(kv, slot_begin, C, idx, nk, tail, rf, page_rope, ws_r)
            rf_s[slot_begin:slot_begin + C].fill_(-1)
        once()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            once()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def accounting():
        assert keep_alive and err.item() == 0
        n = int(nk.item())
        append = n * HC * D * 2 * 2 * 2 * L
        score = C * (8 * w.d + 1)
        return dict(n_kept=n, gather_bytes=append, step_bytes=append + score, n_scored=C,
                    context=None if ARGS.no_fullkv else {
                        "page_axis_step_ms": round(page_axis_ms(), 4),
                        **step_ms_eager_and_graph(step, restore)},
                    config={"workload": "hs_ring",
                            "layout": "per head class: static sink | 4 chunk slots; "
                                      "dynamic sink | 4 chunk slots | history",
                            "time_axis": "compressed (old keys at phase t/c)",
                            "layers": L, "heads_per_class": HC, "head_dim": D,
                            "kv_dtype": "bf16", "history_rows": int(n_hist), "scored_tokens": C,
                            "kept_tokens": n, "appended_bytes": append,
                            "rope_pairs": w.rope_pairs, "q0": w.q0})

    return run, gt, accounting, None


def setup_attention_lag(dev, layers=4):
    """Attention of the next chunk (6,240 queries, 40 heads x 128, bf16) over
    the same 83,412-row cache as the attention workload, in the ring layout
    [sink | window chunks 57-59 + the chunk | history: retained rows of chunks
    1-56] with the old keys on the compressed time axis (re-indexed once to
    phase t/c, here in the setup): one dp_attention_lag launch per layer, the
    query turned back by (1 - 1/c)(q0 - knee) = 199.5 frames for the sink and
    the history.  For context dp_attention over the same buffers is timed
    once per layer (the cost of the lag)."""
    import compaction_dp_score_amd as dp
    import dpsynth
    w = dpsynth.WORKLOADS["reindex"]
    H, D, C = w.n_heads, w.head_dim, w.chunk_tokens
    rf_host, plain_begin, plain_end = dpsynth.ring_layout(w)
    n = rf_host.shape[0]
    q = torch.empty((C, H, D), dtype=torch.bfloat16, device=dev)
    dpsynth.kv_fill_device(q, "bf16", w.seed, 3, 0, C, H * D)
    ks = _fill_layers(dev, w, n, range(layers), dpsynth.STREAM_K)
    vs = _fill_layers(dev, w, n, range(layers), dpsynth.STREAM_V)
    theta = torch.from_numpy(dpsynth.rope_theta(w.rope_pairs, w.rope_base)).to(dev)
    n_frames = w.n_frames + w.frames_per_chunk           # through the chunk's own frames
    ft = np.arange(n_frames, dtype=np.float32)
    ftd, fpd = torch.from_numpy(ft).to(dev), torch.from_numpy(ft.copy()).to(dev)
    rope = make_rope(theta, ftd, fpd, w.q0, w.rope_knee, 1.0 / w.rope_factor,
                        axis=dp.DP_AXIS_COMPRESSED)
    ws_r = torch.empty(dp.dp_rope_workspace_bytes(n_frames, w.rope_pairs) // 4 + 4,
                       dtype=torch.float32, device=dev)
    rf = torch.from_numpy(rf_host).to(dev)
    arr_k = dp.ptr_array(ks, dev)
    dp.dp_rope_prepare(rope, D, dp.DP_BF16, ws_r)
    dp.dp_rope_apply(arr_k, layers, H, D, dp.DP_BF16, 0, n, None, rf, rope, ws_r)
    lag = (1.0 - 1.0 / w.rope_factor) * (w.q0 - w.rope_knee)
    o = torch.empty_like(q)
    scale = 1.0 / float(np.sqrt(D))
    gt = Timer()

    def launch(l):
        dp.dp_attention_lag(q, ks[l], vs[l], o, C, n, None, plain_begin, plain_end, theta, 0,
                            w.rope_pairs, lag, H, D, dp.DP_BF16, scale, key_layout=KEY_LAYOUT)

    def run(timed):
        for l in range(layers):
            if timed and l == 0:
                gt.start()
            launch(l)
            if timed and l == 0:
                gt.stop()

    def dense_ms(reps=3):
        dp.dp_attention(q, ks[0], vs[0], o, C, n, None, H, D, dp.DP_BF16, scale, **attn_layout(w))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            dp.dp_attention(q, ks[0], vs[0], o, C, n, None, H, D, dp.DP_BF16, scale, **attn_layout(w))
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def accounting():
        flops = 4.0 * C * n * D * H
        rec = dict(n_kept=n, gather_bytes=None, flops_per_launch=flops,
                   step_flops=flops * layers, n_scored=0,
                   metric="attention TFLOP/s over the compacted cache, old keys on the "
                          "compressed time axis",
                   config={"workload": "attention_lag", "layers": layers, "heads": H,
                           "head_dim": D, "dtype": "bf16", "queries": C, "kv_rows": n,
                           "plain_rows": [plain_begin, plain_end], "lag_frames": lag,
                           "rope_pairs": w.rope_pairs})
        if not ARGS.no_fullkv:
            rec["context"] = {"dense_attention_ms": round(dense_ms(), 4)}
        return rec

    return run, gt, accounting, None


def setup_attention(dev, layers=4):
    """Attention of a new chunk (6,240 queries, 40 heads x 128, bf16) over the
    cache a one-minute history leaves after compaction: sink + 15 % of the 56
    prunable chunks + the 3-chunk window + the chunk itself (83,412 rows).  A
    step is one dp_attention launch per layer over `layers` layers (each its own
    cache).  For context the same launch over the FullKV cache (all 60 chunks
    + the chunk, 380,640 rows) is timed once per layer, which gives the
    attention-side speed-up of the compaction."""
    import compaction_dp_score_amd as dp
    import dpsynth
    w = dpsynth.WORKLOADS["reindex"]
    H, D, C = w.n_heads, w.head_dim, w.chunk_tokens
    n_ret = int(dpsynth.retained_keep(w).sum()) + C
    n_full = w.seq_len + C
    q = torch.empty((C, H, D), dtype=torch.bfloat16, device=dev)
    dpsynth.kv_fill_device(q, "bf16", w.seed, 3, 0, C, H * D)
    ks = _fill_layers(dev, w, n_ret, range(layers), dpsynth.STREAM_K)
    vs = _fill_layers(dev, w, n_ret, range(layers), dpsynth.STREAM_V)
    o = torch.empty_like(q)
    scale = 1.0 / float(np.sqrt(D))
    gt = Timer()

    def run(timed):
        for l in range(layers):
            if timed and l == 0:
                gt.start()
            dp.dp_attention(q, ks[l], vs[l], o, C, n_ret, None, H, D, dp.DP_BF16, scale, **attn_layout(w))
            if timed and l == 0:
                gt.stop()

    def full_ms(reps=3):
        kf = torch.empty((n_full, H, D), dtype=torch.bfloat16, device=dev)
        vf = torch.empty((n_full, H, D), dtype=torch.bfloat16, device=dev)
        dpsynth.kv_fill_device(kf, "bf16", w.seed, dpsynth.STREAM_K, 0, n_full, H * D)
        dpsynth.kv_fill_device(vf, "bf16", w.seed, dpsynth.STREAM_V, 0, n_full, H * D)
        dp.dp_attention(q, kf, vf, o, C, n_full, None, H, D, dp.DP_BF16, scale, **attn_layout(w))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            dp.dp_attention(q, kf, vf, o, C, n_full, None, H, D, dp.DP_BF16, scale, **attn_layout(w))
        b.record()
        torch.cuda.synchronize()
        del kf, vf
        return a.elapsed_time(b) / reps

    def accounting():
        flops = 4.0 * C * n_ret * D * H
        return dict(n_kept=n_ret, gather_bytes=None, flops_per_launch=flops,
                    step_flops=flops * layers, n_scored=0,
                    full_ms=None if ARGS.no_fullkv else full_ms(),
                    full_flops=4.0 * C * n_full * D * H,
                    config={"workload": "attention", "layers": layers, "heads": H, "head_dim": D,
                            "dtype": "bf16", "queries": C, "kv_rows": n_ret,
                            "fullkv_rows": n_full})

    return run, gt, accounting, None


def setup_hs_attention(dev, layers=4):
    """Attention of a new chunk (6,240 queries, 40 heads x 128, bf16) over the
    ragged DeCoPrune-HS cache of the 30-chunk HS workload: per layer a seeded
    half of the heads static (sink + 3-chunk window, 24,960 rows), the others
    the shared gamma mask (49,134 rows), each followed by the chunk's own 6,240
    rows.  The per-head lengths and offsets are computed on the device
    (score, mask, index, offsets); the cache contents are synthetic.  A step is
    one dp_hs_attention launch per layer over `layers` layers of one packed
    cache.  For context the dense launch over the FullKV cache (30 chunks + the
    chunk, 193,440 rows) is timed once per layer."""
    import compaction_dp_score_amd as dp
    import dpsynth
    w = dpsynth.WORKLOADS["hs"]
    T, H, D, C = w.seq_len, w.n_heads, w.head_dim, w.chunk_tokens
    x0, xf = dpsynth.score_inputs(w)
    x0d, xfd = torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev)
    cls = dpsynth.hs_head_class(w)[:layers]
    head_class = torch.from_numpy(cls.ravel().copy()).to(dev)
    keeps = [torch.empty(T, dtype=torch.uint8, device=dev) for _ in range(2)]
    lists = [torch.empty(T, dtype=torch.int32, device=dev) for _ in range(2)]
    lens = torch.zeros(2, dtype=torch.int64, device=dev)
    ws_c = torch.empty(dp.dp_compact_workspace_bytes(T) // 4 + 1, dtype=torch.int32, device=dev)
    dp.dp_score_mask(None, None, w.d, w.d, dp.make_policy(T, w.sink_len, w.window_len,
                     w.scored_begin, w.n_scored, w.gamma, mode=dp.DP_MODE_STREAMING), None, keeps[0])
    dp.dp_score_mask(x0d, xfd, w.d, w.d, dp.make_policy(T, w.sink_len, w.window_len,
                     w.scored_begin, w.n_scored, w.gamma), None, keeps[1])
    for c in range(2):
        dp.dp_compact_index(keeps[c], T, lists[c], lens[c:c + 1], None, None, ws_c)
    offsets = torch.empty(layers * H + 1, dtype=torch.int64, device=dev)
    dp.dp_hs_offsets(head_class, layers, H, lens, 2, offsets)
    off = offsets.cpu().numpy()
    total = int(off[-1])
    kr = torch.empty((total, D), dtype=torch.bfloat16, device=dev)
    vr = torch.empty((total, D), dtype=torch.bfloat16, device=dev)
    dpsynth.kv_fill_device(kr, "bf16", w.seed, dpsynth.STREAM_K, 0, total, D)
    dpsynth.kv_fill_device(vr, "bf16", w.seed, dpsynth.STREAM_V, 0, total, D)
    q = torch.empty((C, H, D), dtype=torch.bfloat16, device=dev)
    dpsynth.kv_fill_device(q, "bf16", w.seed, 3, 0, C, H * D)
    kc = _fill_layers(dev, w, C, range(layers), dpsynth.STREAM_K)
    vc = _fill_layers(dev, w, C, range(layers), dpsynth.STREAM_V)
    o = torch.empty_like(q)
    scale = 1.0 / float(np.sqrt(D))
    gt = Timer()
    n_full = T + C

    def run(timed):
        if timed:
            gt.start()
        for l in range(layers):
            dp.dp_hs_attention(q, kr, vr, total, offsets, l, kc[l], vc[l], C, o, C, H, D,
                               dp.DP_BF16, scale, **attn_layout(w))
        if timed:
            gt.stop()

    def full_ms(reps=3):
        kf = torch.empty((n_full, H, D), dtype=torch.bfloat16, device=dev)
        vf = torch.empty((n_full, H, D), dtype=torch.bfloat16, device=dev)
        dpsynth.kv_fill_device(kf, "bf16", w.seed, dpsynth.STREAM_K, 0, n_full, H * D)
        dpsynth.kv_fill_device(vf, "bf16", w.seed, dpsynth.STREAM_V, 0, n_full, H * D)
        dp.dp_attention(q, kf, vf, o, C, n_full, None, H, D, dp.DP_BF16, scale, **attn_layout(w))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            dp.dp_attention(q, kf, vf, o, C, n_full, None, H, D, dp.DP_BF16, scale, **attn_layout(w))
        b.record()
        torch.cuda.synchronize()
        del kf, vf
        return a.elapsed_time(b) / reps

    def lag_ms(reps=3):
        # the same launches on the compressed time axis: each run's window tail
        # (w.window_len rows, within the knee) plain, the rest lagged
        theta = torch.from_numpy(dpsynth.rope_theta(w.rope_pairs, w.rope_base)).to(dev)
        lag = (1.0 - 1.0 / w.rope_factor) * (w.q0 - w.rope_knee)

        def once():
            for l in range(layers):
                dp.dp_hs_attention_lag(q, kr, vr, total, offsets, l, kc[l], vc[l], C, o, C, H, D,
                                       dp.DP_BF16, scale, w.window_len, theta, 0, w.rope_pairs,
                                       lag, key_layout=KEY_LAYOUT)
        once()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            once()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps / layers

    def accounting():
        # the timer spans the `layers` launches (their head runs differ), so the
        # per-launch figure is the mean over them
        step_flops = 4.0 * C * D * float(total + layers * H * C)
        return dict(n_kept=total, gather_bytes=None, flops_per_launch=step_flops / layers,
                    timer_launches=layers, step_flops=step_flops, n_scored=0,
                    full_ms=None if ARGS.no_fullkv else full_ms(),
                    context=None if ARGS.no_fullkv else
                    {"compressed_axis_ms_per_launch": round(lag_ms(), 4)},
                    full_flops=4.0 * C * n_full * D * H,
                    metric="attention TFLOP/s over the ragged DeCoPrune-HS cache",
                    config={"workload": "hs_attention", "layers": layers, "heads": H,
                            "head_dim": D, "dtype": "bf16", "queries": C,
                            "head_rows_static": int(lens[0].item()),
                            "head_rows_dynamic": int(lens[1].item()), "chunk_rows": C,
                            "fullkv_rows": n_full})

    return run, gt, accounting, None


def setup_prefix(dev, slab=0, slab_layers=20):
    """Prefix pruning of a 58-chunk observed context: all 57 non-sink chunks
    scored (d = 64) and compacted.  40 layers of K+V are 296.5 GB, more than
    one GPU's 288 GB, so a step runs on one 20-layer slab at a time (slab 0:
    layers 0-19, slab 1: layers 20-39, each one batched launch)."""
    import compaction_dp_score_amd as dp
    import dpsynth
    from compaction_dp_score_amd.step import PruneStep
    w = dpsynth.WORKLOADS["prefix"]
    T, H, D = w.seq_len, w.n_heads, w.head_dim
    x0, xf = dpsynth.score_inputs(w)
    x0d, xfd = torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev)
    layers = range(slab * slab_layers, (slab + 1) * slab_layers)
    k_src = _fill_layers(dev, w, T, layers, dpsynth.STREAM_K)
    v_src = _fill_layers(dev, w, T, layers, dpsynth.STREAM_V)
    # the kept count sizes the destination (one host read, outside the timing)
    probe = PruneStep(k_src=k_src[:1], v_src=None, k_dst=[k_src[0][:1]], v_dst=None, seq_len=T,
                      sink_len=w.sink_len, window_len=w.window_len, scored_begin=w.scored_begin,
                      n_scored=w.n_scored, gamma=w.gamma, d=w.d)
    dp.dp_score_mask(x0d, xfd, w.d, w.d, probe.policy, None, probe.keep)
    dp.dp_compact_index(probe.keep, T, probe.idx, probe.n_kept, None, None, probe.ws_compact)
    cap = int(probe.n_kept.item())
    del probe
    k_dst = [torch.empty((cap, H, D), dtype=torch.bfloat16, device=dev) for _ in range(slab_layers)]
    v_dst = [torch.empty((cap, H, D), dtype=torch.bfloat16, device=dev) for _ in range(slab_layers)]
    step = PruneStep(k_src=k_src, v_src=v_src, k_dst=k_dst, v_dst=v_dst, seq_len=T,
                     sink_len=w.sink_len, window_len=w.window_len, scored_begin=w.scored_begin,
                     n_scored=w.n_scored, gamma=w.gamma, d=w.d)
    gt = Timer()
    st = Timer()

    def run(timed):
        if timed:
            st.start()
        dp.dp_score_index(x0d, xfd, w.d, w.d, step.policy, None, step.keep, step.idx,
                          step.n_kept, None, None, step.ws_index, step.dev_error)
        if timed:
            st.stop()
            gt.start()
        dp.dp_gather_kv(step.kv, step.idx, step.n_kept)
        if timed:
            gt.stop()

    def accounting():
        n = int(step.n_kept.item())
        assert int(step.dev_error.item()) == 0
        gather = n * H * D * 2 * 2 * 2 * slab_layers
        index = w.n_scored * 8 * w.d + T + 4 * n            # scores in, keep out, idx out
        return dict(n_kept=n, gather_bytes=gather, step_bytes=gather + index,
                    n_scored=w.n_scored, score_timer=st, index_bytes=index,
                    index_compare=index_compare(step, x0d, xfd, w.d),
                    order_sensitive=order_sensitive(x0, xf, w.d, w.gamma),
                    config={"workload": "prefix", "slab": slab, "layers_in_slab": slab_layers,
                            "slab_layers": [layers[0], layers[-1]], "layers": 40,
                            "heads": H, "head_dim": D, "kv_dtype": "bf16", "tokens": T,
                            "scored_tokens": w.n_scored, "d": w.d, "gamma": w.gamma,
                            "kept_tokens": n, "pr_step": 1 - n / T})

    def cpu_baseline(seconds):
        return cpu_baseline_prefix(w, x0, xf, slab_layers, seconds)

    return run, gt, accounting, cpu_baseline


def setup_hs(dev):
    """DeCoPrune-HS: 30-chunk history (187,200 tokens), per layer a seeded
    half of the heads static (sink + 3-chunk window), the rest dynamic (the
    shared gamma mask); ragged per-head output plus the RoPE re-index fused
    into the gather (44 pairs, knee 12 frames, factor 8, q0 = 120)."""
    import compaction_dp_score_amd as dp
    import dpsynth
    w = dpsynth.WORKLOADS["hs"]
    T, H, D, L = w.seq_len, w.n_heads, w.head_dim, w.n_layers
    x0, xf = dpsynth.score_inputs(w)
    x0d, xfd = torch.from_numpy(x0).to(dev), torch.from_numpy(xf).to(dev)
    cls = dpsynth.hs_head_class(w)
    head_class = torch.from_numpy(cls.ravel().copy()).to(dev)
    k_src = _fill_layers(dev, w, T, range(L), dpsynth.STREAM_K)
    v_src = _fill_layers(dev, w, T, range(L), dpsynth.STREAM_V)
    rf = torch.from_numpy(dpsynth.row_frame(w)).to(dev)
    pol_static = dp.make_policy(T, w.sink_len, w.window_len, w.scored_begin, w.n_scored, w.gamma,
                                mode=dp.DP_MODE_STREAMING)
    pol_dyn = dp.make_policy(T, w.sink_len, w.window_len, w.scored_begin, w.n_scored, w.gamma)
    keeps = [torch.empty(T, dtype=torch.uint8, device=dev) for _ in range(2)]
    lists = [torch.empty(T, dtype=torch.int32, device=dev) for _ in range(2)]
    rfs = [torch.empty(T, dtype=torch.int32, device=dev) for _ in range(2)]
    lens = torch.zeros(2, dtype=torch.int64, device=dev)
    ws_c = torch.empty(dp.dp_compact_workspace_bytes(T) // 4 + 1, dtype=torch.int32, device=dev)
    offsets = torch.empty(L * H + 1, dtype=torch.int64, device=dev)
    cidx, crf = dp.ptr_array(lists, dev), dp.ptr_array(rfs, dev)
    caps = [T, T]

    def index_part():
        dp.dp_score_mask(None, None, w.d, w.d, pol_static, None, keeps[0])
        dp.dp_score_mask(x0d, xfd, w.d, w.d, pol_dyn, None, keeps[1])
        for c in range(2):
            dp.dp_compact_index(keeps[c], T, lists[c], lens[c:c + 1], rf, rfs[c], ws_c)
        dp.dp_hs_offsets(head_class, L, H, lens, 2, offsets)

    index_part()
    total = int(offsets[-1].item())
    k_out = torch.empty((total, D), dtype=torch.bfloat16, device=dev)
    v_out = torch.empty((total, D), dtype=torch.bfloat16, device=dev)
    kv = dp.dp_kv_hs()
    arrs = [dp.ptr_array(k_src, dev), dp.ptr_array(v_src, dev)]
    kv.k_src, kv.v_src = arrs[0].data_ptr(), arrs[1].data_ptr()
    kv.k_out, kv.v_out = k_out.data_ptr(), v_out.data_ptr()
    kv.n_layers, kv.n_heads, kv.head_dim, kv.dtype = L, H, D, dp.DP_BF16
    kv.src_rows, kv.out_capacity = T, total
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    kv.dev_error = err.data_ptr()
    # the packed runs in this run's key layout; the source token rows stay
    # interleaved (head rows on whole lines of their own, so the two classes of
    # a layer share no source line)
    kv.key_layout, kv.pair_begin, kv.n_pairs = KEY_LAYOUT, 0, w.rope_pairs
    kv.src_key_layout = dp.DP_KEY_INTERLEAVED
    theta = torch.from_numpy(dpsynth.rope_theta(w.rope_pairs, w.rope_base)).to(dev)
    ft, fp = dpsynth.frame_tables(w)
    ftd, fpd = torch.from_numpy(ft).to(dev), torch.from_numpy(fp).to(dev)
    phase0 = fpd.clone()
    rope = make_rope(theta, ftd, fpd, w.q0, w.rope_knee, 1.0 / w.rope_factor)
    ws = torch.empty(dp.dp_rope_workspace_bytes(w.n_frames, w.rope_pairs) // 4 + 4,
                     dtype=torch.float32, device=dev)
    gt = Timer()
    keep_alive = [arrs, k_out, v_out, cidx, crf, err]   # the kernels hold raw pointers to these

    def run(timed):
        fpd.copy_(phase0)
        index_part()
        if timed:
            gt.start()
        dp.dp_hs_gather_kv(kv, head_class, 2, cidx, lens, caps, offsets, crf, rope, ws)
        if timed:
            gt.stop()

    def _median_ms(fn, reps):
        ms = []
        for _ in range(reps + 1):
            fpd.copy_(phase0)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ms.append(a.elapsed_time(b))
        fpd.copy_(phase0)
        return float(np.median(ms[1:]))

    def unfused_reindex(kvx, ropex, reps=3):
        # the re-index as a pass of its own over the packed cache (the gather
        # without the fused rotation leaves the keys at their old phases):
        # dp_hs_rope_reindex, phase table restored before each call
        dp.dp_hs_gather_kv(kvx, head_class, 2, cidx, lens, caps, offsets)
        t = _median_ms(lambda: dp.dp_hs_rope_reindex(k_out, total, L, H, D, dp.DP_BF16,
                                                     head_class, 2, lens, caps, offsets, crf,
                                                     ropex, ws), reps)
        ln = lens.cpu().numpy()
        per_class = [(cls == c).sum() for c in range(2)]         # heads of each class
        rows = sum(int(per_class[c]) * int(ln[c] - w.window_len) for c in range(2))
        b = rows * 2 * w.rope_pairs * 2 * 2
        return {"unfused_reindex_ms": round(t, 4), "unfused_reindex_bytes": b,
                "unfused_reindex_gbs": round(b / t / 1e6, 1)}

    def context():
        ctx = unfused_reindex(kv, rope)
        if KEY_LAYOUT == dp.DP_KEY_INTERLEAVED:
            # the same step writing split runs (each run's temporal blocks
            # first): the fused gather, and the re-index of such runs as a pass
            # of its own, which then rewrites whole lines only
            kv_s = dp.dp_kv_hs.from_buffer_copy(kv)
            kv_s.key_layout = dp.DP_KEY_SPLIT
            rope_s = dp.make_rope(theta, ftd, fpd, w.q0, w.rope_knee, 1.0 / w.rope_factor,
                                  key_layout=dp.DP_KEY_SPLIT)
            t = _median_ms(lambda: dp.dp_hs_gather_kv(kv_s, head_class, 2, cidx, lens, caps,
                                                      offsets, crf, rope_s, ws), 3)
            gb = int(offsets[-1].item()) * D * 2 * 2 * 2
            ctx["split_runs"] = dict(gather_ms=round(t, 4), gather_gbs=round(gb / t / 1e6, 1),
                                     **unfused_reindex(kv_s, rope_s))
        return ctx

    def accounting():
        assert keep_alive
        tot = int(offsets[-1].item())
        ln = lens.cpu().numpy()
        gather = tot * D * 2 * 2 * 2
        score = w.n_scored * 8 * w.d + 2 * T
        index = 4 * T + 8 * int(ln.sum()) + 8 * (L * H + 1)
        return dict(n_kept=tot, gather_bytes=gather, step_bytes=gather + score + index,
                    n_scored=w.n_scored, order_sensitive=order_sensitive(x0, xf, w.d, w.gamma),
                    context=None if ARGS.no_fullkv else context(),
                    config={"workload": "hs", "layers": L, "heads": H, "head_dim": D,
                            "kv_dtype": "bf16", "tokens": T, "static_heads_per_layer": int(
                                (cls == 0).sum(axis=1)[0]), "static_rows": int(ln[0]),
                            "dynamic_rows": int(ln[1]), "head_rows": tot,
                            "pr_step": 1 - tot / (L * H * T), "rope_pairs": w.rope_pairs,
                            "q0": w.q0, "key_layout": "split" if KEY_LAYOUT else "interleaved",
                            "src_key_layout": "interleaved"})

    def cpu_baseline(seconds):
        return cpu_baseline_hs(w, x0, xf, cls, seconds)

    return run, gt, accounting, cpu_baseline


def summarize_stats(workload, stats_dir, warmup):
    """Short text summary of rocprofv3's kernel statistics CSV; the dominant
    kernel's line is recomputed from the kernel trace without its first
    `warmup` dispatches (the untimed warm-up steps), so its average is that of
    the timed steps."""
    import csv
    import glob
    import re
    files = glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)
    assert files, "no kernel_stats.csv under %s" % stats_dir
    kname = KERNELS[workload][0]
    flags = profile_flags(workload)
    lines = ["# rocprofv3 kernel statistics, %s workload (bench.py --workload %s)" % (workload, workload),
             "# commands (from the repository root):",
             "#   rocprofv3 --kernel-trace --stats -d %s -o run -f csv -- python bench.py "
             "--workload %s %s --warmup %d --steps 10" % (stats_dir, workload, flags, warmup),
             "#   python bench.py --workload %s --warmup %d --summarize-stats %s"
             % (workload, warmup, stats_dir),
             "# dominant kernel: %s; times in ns; fill_kernel and calib_copy_kernel are input" % kname,
             "# generation and the copy-ceiling reference, not part of the step"]
    traces = glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True)
    if traces:
        durs = []
        for r in csv.DictReader(open(traces[0])):
            name = r["Kernel_Name"]
            if ("::" + kname + "<") in name or ("::" + kname + "(") in name:
                durs.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) -
                             int(r["Start_Timestamp"])))
        durs.sort()
        timed = [d for _, d in durs[warmup:]]
        if timed:
            lines.append("# %s, timed steps only (first %d of %d dispatches are warm-up): "
                         "calls %d | avg_ns %.0f | min_ns %d | max_ns %d"
                         % (kname, warmup, len(durs), len(timed), sum(timed) / len(timed),
                            min(timed), max(timed)))
    lines.append("kernel | calls | avg_ns | min_ns | max_ns | total_ns | pct")
    for r in csv.DictReader(open(files[0])):
        name = r["Name"].replace("(anonymous namespace)", "anon")
        m = re.search(r"(\w+)(<[^>()]*>)?\(", name)
        short = m.group(1) + (m.group(2) or "") if m else name[:60]
        lines.append("%s | %s | %.0f | %s | %s | %s | %.2f" % (
            short, r["Calls"], float(r["AverageNs"]), r["MinNs"], r["MaxNs"],
            r["TotalDurationNs"], float(r["Percentage"])))
    path = os.path.join(PROFILES, "%s_%s_kernel_stats.txt" % (kname, workload))
    with open(path, "w") as out:
        out.write("\n".join(lines) + "\n")
    print(open(path).read())


ARGS = None   # parsed command line (the attention setups read --no-fullkv)


# Workloads whose dominant kernel is an in-place re-index of old keys: split
# keys let it rewrite whole lines only (the one-minute re-index: 6.0 against
# 3.9 TB/s).  Elsewhere the layout is the model's natural one: attention over
# split keys is 2.5 % slower (a head row is two pieces on lines it shares with
# its neighbours), the HS gather from split rows reads shared lines twice, and
# the gathers and appends move whole rows either way.
SPLIT_WORKLOADS = ("reindex", "steady", "append")


def layout_for(workload, args):
    """Key layout of a workload's records: --key-layout if given, else split
    for the re-index workloads and interleaved for the others."""
    if args.key_layout is not None:
        return 1 if args.key_layout == "split" else 0
    return 1 if workload in SPLIT_WORKLOADS else 0


def main():
    global ARGS, KEY_LAYOUT
    args = ARGS = parse()
    if args.summarize_stats:
        summarize_stats(args.workload, args.summarize_stats, args.warmup)
        return
    if args.summarize_pmc:
        summarize_pmc(args.workload, *args.summarize_pmc)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the compaction path runs on a single MI355X "
              "(pass --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import compaction_dp_score_amd  # noqa: F401  (fails loudly if the library is missing)
    dev = torch.device("cuda:0")
    setups = {"eviction": setup_eviction, "tiny": lambda d: setup_eviction(d, "tiny"),
              "reindex": setup_reindex, "prefix": setup_prefix,
              "hs": setup_hs, "append": setup_append, "attention": setup_attention,
              "hs_attention": setup_hs_attention, "steady": setup_steady,
              "steady_lazy": setup_steady_lazy, "attention_lag": setup_attention_lag,
              "hs_ring": setup_hs_ring}
    if args.workload is not None:
        rec = measure(args.workload, lambda: setups[args.workload](dev), dev, args)
        print(json.dumps(rec), flush=True)
        return
    # default run: the eviction step is the headline record; the other four
    # workloads (tiny, one-minute re-index, both prefix slabs, HS) follow under
    # "configs", each measured after the previous one's buffers are freed
    rec = measure("eviction", lambda: setup_eviction(dev), dev, args)
    rec["configs"] = {}
    for label, name, make in (
            ("tiny", "tiny", lambda: setup_eviction(dev, "tiny")),
            ("reindex", "reindex", lambda: setup_reindex(dev)),
            ("prefix_slab0", "prefix", lambda: setup_prefix(dev, 0)),
            ("prefix_slab1", "prefix", lambda: setup_prefix(dev, 1)),
            ("hs", "hs", lambda: setup_hs(dev))):
        r = measure(name, make, dev, args, copy_ceiling_too=False)
        for k in ("metric", "n_gpus", "steps", "warmup", "higher_is_better", "scaling",
                  "vs_baseline", "data"):
            r.pop(k, None)
        rec["configs"][label] = r
    print(json.dumps(rec), flush=True)


def measure(workload, make, dev, args, copy_ceiling_too=True):
    """Set up one workload, run args.warmup untimed and args.steps timed steps
    (HIP events on the current stream around the steps), then build its JSON
    record (and its CPU leg); the workload's buffers are freed on return."""
    import gc
    global KEY_LAYOUT
    KEY_LAYOUT = layout_for(workload, args)
    run, gt, accounting, cpu = make()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        run(False)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        run(True)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    acc = accounting()
    acc["config"].setdefault("key_layout", "split" if KEY_LAYOUT else "interleaved")
    if acc.get("flops_per_launch"):
        return flops_record(args, acc, ms, gt.mean_ms())
    gbs = acc["step_bytes"] / (ms * 1e-3) / 1e9
    g_ms = gt.mean_ms()
    g_gbs = acc["gather_bytes"] / (g_ms * 1e-3) / 1e9
    traffic = read_traffic(workload)                  # per dispatch
    if traffic is not None:
        traffic *= acc.get("timer_launches", 1)         # over the timed region
    kernel = KERNELS[workload][0]
    rec = {
        "metric": "compacted KV GB/s (read+write) per prune step, % of HBM peak; tokens scored/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if acc["config"].get("kv_dtype", "bf16") == "bf16" else "f32",
        "data": "synthetic",
        "config": acc["config"],
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tokens_scored_per_s": None,
        "step_bytes": acc["step_bytes"],
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(g_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(g_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": acc["gather_bytes"],
                     "launch_ms": round(g_ms, 4)},
    }
    if acc.get("score_timer") is not None:
        s_ms = acc["score_timer"].mean_ms()
        tps = acc["n_scored"] / (s_ms * 1e-3)
        rec["tokens_scored_per_s"] = round(tps, 1)
        ibytes = acc["index_bytes"]
        rec["score_index_kernel"] = {
            "ms": round(s_ms, 5), "tokens_scored": acc["n_scored"], "bytes": ibytes,
            "gbs": round(ibytes / (s_ms * 1e-3) / 1e9, 2),
            "frac": round(ibytes / (s_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            **acc.get("index_compare", {})}
    if acc.get("append_timer") is not None:
        a_ms = acc["append_timer"].mean_ms()
        rec["append_kernel"] = {"ms": round(a_ms, 5), "bytes": acc["append_bytes"],
                                "gbs": round(acc["append_bytes"] / (a_ms * 1e-3) / 1e9, 2)}
    if acc.get("order_sensitive") is not None:
        rec["order_sensitive_tokens"] = acc["order_sensitive"]
    if acc.get("context"):
        rec["context"] = acc["context"]
    if copy_ceiling_too:
        rec["copy_ceiling_gbs"] = round(copy_ceiling(dev, CALIB_BYTES), 2)
    del run, gt, accounting, acc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if cpu is not None and not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu(args.cpu_seconds)
    del cpu
    gc.collect()
    torch.cuda.empty_cache()
    return rec


if __name__ == "__main__":
    main()
