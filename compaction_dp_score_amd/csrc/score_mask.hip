// dp_score_mask: per-token discrepancy score and keep mask.
//
// The DeCoPrune page (section 어떻게 동작하나) scores each token of a chunk by
// the mean squared gap between the clean prediction recorded at the probe
// step and the final output, and thresholds it with gamma; the mask is shared
// by every layer, the sink chunk and the last w chunks are always kept.
//
// Launch layout: blocks [0, n_score_blocks) score rows; a group of G lanes
// (G = P/4, P the channel count padded to a power of two) owns one row, lane
// k loads channels 4k..4k+3, and the pairwise tree q_c += q_{c+h} runs as
// shuffles for h >= 4 and inside the lane for h = 2, 1.  Blocks after those
// write the keep bytes of every row that is not scored (sink, window, earlier
// history), 16 rows per thread.  The score is HBM-bound: 8d bytes read and
// 1 (+4 with ell) written per scored row.
//
// dp_score_index: the same scores and mask and the ascending kept-index list
// (what dp_compact_index derives from the mask) from one call.  Workgroups
// take tiles in the order of an atomic ticket: scored rows in tiles of
// kSiPasses rows per lane group (64 rows at d = 64), so that scoring keeps as
// many wavefronts busy as dp_score_mask does, other rows in tiles of 2048
// rows.  A workgroup scores and masks its tile into LDS and finds its
// output offset by a decoupled look-back over the tiles before it: each tile
// publishes its kept count, then its inclusive prefix, in a 64-bit status word
// tagged with the call's generation; one wavefront reads 256 predecessors per
// round trip and stops at the nearest inclusive prefix.  A tile only ever
// waits for tiles with lower tickets, which belong to workgroups already
// running, so every wait ends; the wait is also bounded (DP_ESTALL through
// dev_error).  The last workgroup to finish resets the ticket and advances the
// generation, so the workspace is reused by the next call on the stream
// without clearing.  Ranges that need more than kSiMaxTiles tiles run as
// dp_score_mask's kernel followed by the three compaction kernels instead: the
// ticket and the look-back serialise there and lose to separate launches.
#include "dp_internal.h"

namespace dp {
namespace {

struct ScoreArgs {
  const float* x0;
  const float* xf;
  float* ell;
  uint8_t* keep;
  int64_t stride;
  int64_t T, sink_end, win_begin, sc_begin, sc_end;
  int32_t d, P, G, vec;
  float gamma;
  int32_t reversed, streaming;
  uint32_t n_score_blocks;
};

__device__ __forceinline__ f32x4 load4(const float* row, int c, int d, bool vec) {
  if (vec) return *reinterpret_cast<const f32x4*>(row + c);   // c < d, d % 4 == 0
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (c + 0 < d) v.x = row[c + 0];
  if (c + 1 < d) v.y = row[c + 1];
  if (c + 2 < d) v.z = row[c + 2];
  if (c + 3 < d) v.w = row[c + 3];
  return v;
}

__device__ __forceinline__ f32x4 shfl_down4(f32x4 v, int delta, int width) {
  f32x4 r;
  r.x = __shfl_down(v.x, delta, width);
  r.y = __shfl_down(v.y, delta, width);
  r.z = __shfl_down(v.z, delta, width);
  r.w = __shfl_down(v.w, delta, width);
  return r;
}

__device__ __forceinline__ uint8_t outside_keep(int64_t t, const ScoreArgs& a) {
  if (t < a.sink_end || t >= a.win_begin) return 1;
  return a.streaming ? 0 : 1;   // scored rows in streaming mode also land here
}

// The pairwise tree over the squared gaps a group of G lanes holds (lane k has
// channels 4k..4k+3), then l = (float)((double)q_0 / d), valid in the group's
// lane 0.  Every lane of the wavefront must call it (the tree runs as shuffles).
__device__ __forceinline__ float tree_score(const ScoreArgs& a, f32x4 q) {
  // h = P/2 .. 4 across lanes (lane k pairs with k + h/4)
  for (int h = a.P / 2; h >= 4; h /= 2) {
    f32x4 o = shfl_down4(q, h / 4, a.G);
    q = q + o;
  }
  if (a.P >= 4) {                  // h = 2, then h = 1
    q.x = q.x + q.z;
    q.y = q.y + q.w;
    q.x = q.x + q.y;
  } else if (a.P == 2) {           // h = 1
    q.x = q.x + q.y;
  }
  return (float)((double)q.x / (double)a.d);
}

// Score of scored row `row` (relative to the first scored row) by a group of G
// lanes; every lane of the wavefront must call it (the tree runs as shuffles).
// Returns l = (float)((double)q_0 / d) in the group's lane 0 (other lanes:
// partial sums).
__device__ __forceinline__ float group_score(const ScoreArgs& a, int64_t row, bool live,
                                             int lane_in_group) {
  f32x4 q = {0.f, 0.f, 0.f, 0.f};
  const int c = 4 * lane_in_group;
  if (live && c < a.d) {
    const float* r0 = a.x0 + row * a.stride;
    const float* r1 = a.xf + row * a.stride;
    f32x4 u = load4(r0, c, a.d, a.vec != 0);
    f32x4 w = load4(r1, c, a.d, a.vec != 0);
    f32x4 e = u - w;
    q = e * e;                     // padded channels stay +0 (0 - 0 = +0)
  }
  return tree_score(a, q);
}

__device__ __forceinline__ uint8_t scored_keep(const ScoreArgs& a, float ell) {
  const bool big = ell >= a.gamma;   // NaN fails
  return (uint8_t)(a.reversed ? !big : big);
}

__global__ __launch_bounds__(kBlock) void score_mask_kernel(ScoreArgs a) {
  if (blockIdx.x < a.n_score_blocks) {
    // ---- scoring part ----
    const int lane_in_group = threadIdx.x % a.G;
    const int64_t row = (int64_t)blockIdx.x * (kBlock / a.G) + threadIdx.x / a.G;
    const bool live = row < a.sc_end - a.sc_begin;
    const float ell = group_score(a, row, live, lane_in_group);
    if (live && lane_in_group == 0) {
      if (a.ell) a.ell[row] = ell;
      a.keep[a.sc_begin + row] = scored_keep(a, ell);
    }
    return;
  }
  // ---- keep bytes of the rows that are not scored ----
  const int64_t t0 = ((int64_t)(blockIdx.x - a.n_score_blocks) * kBlock + threadIdx.x) * 16;
  if (t0 >= a.T) return;
  const bool scoring = !a.streaming;
  const bool touches_scored = scoring && t0 < a.sc_end && t0 + 16 > a.sc_begin;
  if (!touches_scored && t0 + 16 <= a.T && (((uintptr_t)(a.keep + t0)) & 15u) == 0) {
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) word |= (uint32_t)outside_keep(t0 + 4 * w + b, a) << (8 * b);
      v[w] = word;
    }
    *reinterpret_cast<u32x4*>(a.keep + t0) = v;
    return;
  }
  for (int b = 0; b < 16; ++b) {
    int64_t t = t0 + b;
    if (t >= a.T) break;
    if (scoring && t >= a.sc_begin && t < a.sc_end) continue;   // written by the scoring part
    a.keep[t] = outside_keep(t, a);
  }
}


// ---------------------------------------------------------------------------
// Single launch: score, mask and kept-index list with a decoupled look-back.
// ---------------------------------------------------------------------------
constexpr int kSiMaxTiles = 1024;                 // tiles of one launch (status words)
constexpr int kSiPasses = 4;                      // a scored tile: 4 rows per lane group
constexpr int kSiPlainRounds = 8;                 // a plain tile: 8 x 256 rows
constexpr int kSiWaves = kBlock / 64;
constexpr uint64_t kFlagAgg = 1, kFlagInc = 2;    // status flags
constexpr uint32_t kGenMask = (1u << 30) - 1;

struct IndexArgs {
  int32_t* idx;
  int64_t* n_kept;
  const int32_t* rf_src;
  int32_t* rf_dst;
  uint32_t* ctl;        // [0] ticket, [1] finished workgroups, [2] generation
  uint64_t* status;     // [n_tiles] (generation << 34) | (flag << 32) | value
  int32_t* dev_error;
  uint32_t n_tiles;
  uint32_t spin_limit;
  // tiles [0, n_pre) cover [0, pre_end) and tiles after n_pre + n_sc cover
  // [sc_end, T), plain_rows rows each; tiles [n_pre, n_pre + n_sc) cover the
  // scored rows, scored_rows (kSiPasses rows per lane group) each
  uint32_t n_pre, n_sc;
  int32_t plain_rows, scored_rows;
  int64_t pre_end;
};

__device__ __forceinline__ uint64_t pack_status(uint32_t gen, uint64_t flag, uint32_t v) {
  return ((uint64_t)gen << 34) | (flag << 32) | v;
}

template <int kSiRounds>
__global__ __launch_bounds__(kBlock) void score_index_kernel(ScoreArgs a, IndexArgs x) {
  constexpr int kSiTile = kBlock * kSiRounds;     // rows per tile
  __shared__ uint8_t keep_s[kSiTile];
  __shared__ int cnt[kSiRounds * kSiWaves];
  __shared__ int pre[kSiRounds * kSiWaves];
  __shared__ uint32_t tile_s, gen_s;
  __shared__ int64_t excl_s;
  __shared__ int stalled_s;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) {
    tile_s = atomicAdd(&x.ctl[0], 1u);
    gen_s = __hip_atomic_load(&x.ctl[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kGenMask;
    stalled_s = 0;
  }
  __syncthreads();
  const uint32_t tile = tile_s, gen = gen_s;
  if (tile >= x.n_tiles) {          // the workspace was not zero-filled before first use
    if (threadIdx.x == 0 && x.dev_error) *x.dev_error = DP_ESTALL;
    return;
  }
  int64_t t_begin, t_end;
  bool scored_tile = false;
  if (tile < x.n_pre) {
    t_begin = (int64_t)tile * x.plain_rows;
    t_end = min(t_begin + x.plain_rows, x.pre_end);
  } else if (tile < x.n_pre + x.n_sc) {
    t_begin = a.sc_begin + (int64_t)(tile - x.n_pre) * x.scored_rows;
    t_end = min(t_begin + x.scored_rows, a.sc_end);
    scored_tile = true;
  } else {
    t_begin = a.sc_end + (int64_t)(tile - x.n_pre - x.n_sc) * x.plain_rows;
    t_end = min(t_begin + x.plain_rows, a.T);
  }

  if (scored_tile) {
    // ---- every row is scored: groups of G lanes per row with the arithmetic of
    // dp_score_mask; each group loads its kSiPasses rows before reducing any ----
    const int per_pass = kBlock / a.G;
    const int lane_in_group = threadIdx.x % a.G, grp = threadIdx.x / a.G;
    const int c = 4 * lane_in_group;
    f32x4 q[kSiPasses];
#pragma unroll
    for (int u = 0; u < kSiPasses; ++u) {
      const int64_t t = t_begin + (int64_t)u * per_pass + grp;
      q[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < t_end && c < a.d) {
        const int64_t row = t - a.sc_begin;
        const f32x4 x0v = load4(a.x0 + row * a.stride, c, a.d, a.vec != 0);
        const f32x4 xfv = load4(a.xf + row * a.stride, c, a.d, a.vec != 0);
        const f32x4 e = x0v - xfv;
        q[u] = e * e;                // padded channels stay +0
      }
    }
#pragma unroll
    for (int u = 0; u < kSiPasses; ++u) {
      const int64_t t = t_begin + (int64_t)u * per_pass + grp;
      const float ell = tree_score(a, q[u]);
      if (t < t_end && lane_in_group == 0) {
        if (a.ell) a.ell[t - a.sc_begin] = ell;
        keep_s[t - t_begin] = scored_keep(a, ell);
      }
    }
  } else {
    // ---- sink, window, earlier history (or every row in Streaming mode) ----
#pragma unroll
    for (int r = 0; r < kSiRounds; ++r) {
      const int64_t t = t_begin + r * kBlock + threadIdx.x;
      if (t < t_end) keep_s[t - t_begin] = outside_keep(t, a);
    }
  }
  __syncthreads();

  // ---- tile-local positions: ballot per (round, wavefront), prefix over the 8 counts ----
  bool mine[kSiRounds];
  uint64_t ballots[kSiRounds];
#pragma unroll
  for (int r = 0; r < kSiRounds; ++r) {
    const int64_t t = t_begin + r * kBlock + threadIdx.x;
    const bool in = t < t_end;
    const uint8_t k = in ? keep_s[t - t_begin] : 0;
    if (in && a.keep) a.keep[t] = k;
    mine[r] = k != 0;
    ballots[r] = __ballot(mine[r]);
    if (lane == 0) cnt[r * kSiWaves + wave] = __popcll(ballots[r]);
  }
  __syncthreads();

  if (wave == 0) {
    // exclusive prefix of the (round, wavefront) counts, round-major
    const int v = lane < kSiRounds * kSiWaves ? cnt[lane] : 0;
    int incl = v;
    for (int o = 1; o < kSiRounds * kSiWaves; o *= 2) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane < kSiRounds * kSiWaves) pre[lane] = incl - v;
    const uint32_t count = (uint32_t)__shfl(incl, kSiRounds * kSiWaves - 1, 64);

    // ---- decoupled look-back ----
    // Status words are read and written as relaxed agent-scope atomics: each
    // word carries its flag and value together and nothing else a predecessor
    // writes is read here, so no ordering (and no cache write-back or
    // invalidation) is needed, only coherence of the words themselves.
    int64_t excl = 0;
    if (tile == 0) {
      if (lane == 0)
        __hip_atomic_store(&x.status[0], pack_status(gen, kFlagInc, count), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (lane == 0)
        __hip_atomic_store(&x.status[tile], pack_status(gen, kFlagAgg, count), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      int64_t j = (int64_t)tile - 1;         // newest predecessor not yet summed
      uint32_t polls = 0;
      bool stalled = false;
      // each lane reads 4 consecutive predecessors, so one round trip covers 256 tiles
      while (true) {
        uint64_t w[4];
        bool ready = true;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t k = j - 4 * lane - i;
          w[i] = pack_status(gen, kFlagInc, 0);           // before tile 0: an empty prefix
          if (k >= 0)
            w[i] = __hip_atomic_load(&x.status[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ready = ready && (uint32_t)(w[i] >> 34) == gen && ((w[i] >> 32) & 3u) != 0;
        if (__ballot(!ready) != 0) {                      // some predecessor not published yet
          if (++polls > x.spin_limit) { stalled = true; break; }
          __builtin_amdgcn_s_sleep(2);
          continue;
        }
        // nearest inclusive prefix: in this lane (first of its 4) and across lanes
        int f = 4;
#pragma unroll
        for (int i = 3; i >= 0; --i)
          if (((w[i] >> 32) & 3u) == kFlagInc) f = i;
        const uint64_t inc = __ballot(f < 4);
        const int first = inc ? (int)__builtin_ctzll(inc) : 64;
        int64_t part = 0;
        if (lane <= first) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (lane < first || i <= f) part += (int64_t)(uint32_t)w[i];
        }
        for (int o = 32; o >= 1; o /= 2) part += __shfl_xor(part, o, 64);
        excl += part;
        if (inc) break;
        j -= 256;
      }
      if (stalled && lane == 0) stalled_s = 1;
      if (lane == 0)
        __hip_atomic_store(&x.status[tile], pack_status(gen, kFlagInc, (uint32_t)(excl + count)),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0) {
      excl_s = excl;
      if (tile == x.n_tiles - 1) *x.n_kept = excl + count;
    }
  }
  __syncthreads();

  // ---- write the kept rows at their final positions ----
  const int64_t base = excl_s;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int r = 0; r < kSiRounds; ++r) {
    if (mine[r]) {
      const int64_t t = t_begin + r * kBlock + threadIdx.x;
      const int64_t pos = base + pre[r * kSiWaves + wave] + __popcll(ballots[r] & below);
      if (pos < a.T) {               // always true unless a stall left the prefix invalid
        x.idx[pos] = (int32_t)t;
        if (x.rf_dst) x.rf_dst[pos] = x.rf_src[t];
      }
    }
  }

  // ---- the last workgroup to finish resets the ticket and advances the generation ----
  __syncthreads();
  if (threadIdx.x == 0) {
    if (stalled_s && x.dev_error) *x.dev_error = DP_ESTALL;
    const uint32_t done = atomicAdd(&x.ctl[1], 1u);
    if (done == x.n_tiles - 1) {
      __hip_atomic_store(&x.ctl[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&x.ctl[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&x.ctl[2], (gen + 1u) & kGenMask, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

namespace {

ScoreArgs score_args(const float* x0, const float* xf, int32_t d, int64_t stride,
                     const dp_mask_policy& pol, float* ell, uint8_t* keep) {
  ScoreArgs a;
  a.x0 = x0;
  a.xf = xf;
  a.ell = ell;
  a.keep = keep;
  a.stride = stride;
  a.T = pol.seq_len;
  a.sink_end = pol.sink_len;
  a.win_begin = pol.seq_len - pol.window_len;
  a.sc_begin = pol.scored_begin;
  a.sc_end = pol.scored_begin + pol.n_scored;
  a.d = d;
  int P = 1;
  while (P < d) P *= 2;
  a.P = P;
  a.G = P >= 4 ? P / 4 : 1;
  a.vec = (d % 4 == 0) && (stride % 4 == 0) && aligned16(x0) && aligned16(xf);
  a.gamma = pol.gamma;
  a.reversed = pol.reversed;
  a.streaming = pol.mode == DP_MODE_STREAMING;
  a.n_score_blocks = 0;
  return a;
}

}  // namespace

dp_status launch_score_mask(const float* x0, const float* xf, int32_t d, int64_t stride,
                            const dp_mask_policy& pol, float* ell, uint8_t* keep,
                            hipStream_t s) {
  ScoreArgs a = score_args(x0, xf, d, stride, pol, ell, keep);
  const int64_t rows_per_block = kBlock / a.G;
  const int64_t n_sc = a.streaming ? 0 : pol.n_scored;
  const int64_t nsb = (n_sc + rows_per_block - 1) / rows_per_block;
  const int64_t nfb = (pol.seq_len + 16 * kBlock - 1) / (16 * kBlock);
  a.n_score_blocks = (uint32_t)nsb;
  const int64_t grid = nsb + nfb;
  if (grid <= 0) return DP_OK;
  hipLaunchKernelGGL(score_mask_kernel, dim3((uint32_t)grid), dim3(kBlock), 0, s, a);
  return check_launch("score_mask_kernel");
}

// Workspace: control words, the status words of one launch, then (for calls
// that run as separate launches) the compaction scratch and a keep mask.
size_t score_index_ws_bytes(int64_t T) {
  const size_t comp = (compact_ws_bytes(T) + 15) / 16 * 16;
  return 16 + (size_t)kSiMaxTiles * sizeof(uint64_t) + comp + (size_t)(T > 0 ? T : 1);
}

dp_status launch_score_index(const float* x0, const float* xf, int32_t d, int64_t stride,
                             const dp_mask_policy& pol, float* ell, uint8_t* keep, int32_t* idx,
                             int64_t* n_kept, const int32_t* rf_src, int32_t* rf_dst, void* ws,
                             int32_t* dev_error, uint32_t spin_limit, hipStream_t s) {
  ScoreArgs a = score_args(x0, xf, d, stride, pol, ell, keep);
  const int64_t T = pol.seq_len;
  const bool scoring = !a.streaming && pol.n_scored > 0;
  const int32_t scored_rows = kSiPasses * (kBlock / a.G);
  // plain tiles of 256 x 8 rows: the fewest tiles, and the fastest (eviction step:
  // 12.1-12.8 us against 15.0-15.3 us with 256-row tiles, which take a ticket
  // and a look-back each)
  constexpr int rounds = kSiPlainRounds;
  const int64_t tn = (int64_t)kBlock * rounds;
  int64_t n_pre = 0, n_sc = 0, n_tiles = 0;
  if (scoring) {
    n_pre = (a.sc_begin + tn - 1) / tn;
    n_sc = (pol.n_scored + scored_rows - 1) / scored_rows;
    n_tiles = n_pre + n_sc + (T - a.sc_end + tn - 1) / tn;
  } else {
    n_pre = (T + tn - 1) / tn;
    n_sc = 0;
    n_tiles = n_pre;
  }
  char* w = reinterpret_cast<char*>(ws);
  if (n_tiles > kSiMaxTiles) {
    // Too many tiles for one launch to win (the ticket and the look-back
    // serialise): score and mask, then the three-kernel compaction.
    int32_t* comp = reinterpret_cast<int32_t*>(w + 16 + (size_t)kSiMaxTiles * sizeof(uint64_t));
    uint8_t* mask = keep ? keep
                         : reinterpret_cast<uint8_t*>(comp) + (compact_ws_bytes(T) + 15) / 16 * 16;
    dp_status st = launch_score_mask(x0, xf, d, stride, pol, ell, mask, s);
    if (st != DP_OK) return st;
    return launch_compact(mask, T, idx, n_kept, rf_src, rf_dst, comp, s);
  }
  IndexArgs x;
  x.idx = idx;
  x.n_kept = n_kept;
  x.rf_src = rf_src;
  x.rf_dst = rf_dst;
  x.ctl = reinterpret_cast<uint32_t*>(w);
  x.status = reinterpret_cast<uint64_t*>(w + 16);
  x.dev_error = dev_error;
  x.n_tiles = (uint32_t)n_tiles;
  x.spin_limit = spin_limit;
  x.n_pre = (uint32_t)n_pre;
  x.n_sc = (uint32_t)n_sc;
  x.plain_rows = kBlock * rounds;
  x.scored_rows = scored_rows;
  x.pre_end = scoring ? a.sc_begin : T;
  // (a scored tile, at most 4 x 256 rows, fits the plain tile's LDS rounds)
  static_assert(kSiPasses * kBlock <= kBlock * kSiPlainRounds, "scored tile exceeds the LDS tile");
  const dim3 grid((uint32_t)n_tiles), block(kBlock);
  hipLaunchKernelGGL(score_index_kernel<kSiPlainRounds>, grid, block, 0, s, a, x);
  return check_launch("score_index_kernel");
}

}  // namespace dp
