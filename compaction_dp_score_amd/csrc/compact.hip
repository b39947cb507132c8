// dp_compact_index: ascending list of the kept rows (stream compaction).
//
// The gathered cache K[m], V[m] of the DeCoPrune page (section 어떻게
// 동작하나) keeps the selected rows in token order, so the index list is the
// ascending positions with keep != 0.
//
// Three stream-ordered launches, no host synchronisation and no spinning:
//   1. count:  one workgroup per tile of 4096 rows counts its kept rows
//              (a whole tile at a 16-byte aligned address: one 16-byte load per
//              thread);
//   2. scan:   one workgroup turns the tile counts into exclusive offsets and
//              writes the total to *n_kept;
//   3. write:  each tile is re-read (into LDS, as the count reads it) and
//              taken in 16 rounds of 256 rows; within a round
//              every wavefront takes a ballot of its keep bits and a lane's
//              slot is the popcount of the ballot below it (mbcnt); the 64
//              (round, wavefront) counts of the tile get an exclusive prefix in
//              LDS, so every kept row lands at its final position.
// Up to kFusedScanTiles tiles (8 M rows) the scan launch is left out: each
// write workgroup sums the counts of the tiles before it itself (at most 8 per
// thread) and the last one writes *n_kept.
#include <mutex>

#include "dp_internal.h"

namespace dp {
namespace {

constexpr int kRounds = 16;
constexpr int kTile = kBlock * kRounds;   // 4096 rows per tile
constexpr int kWaves = kBlock / 64;
constexpr int64_t kFusedScanTiles = 2048;

__device__ __forceinline__ int block_sum(int v, int* lds) {
  // wave reduction, then across the 4 waves through LDS
  for (int o = 32; o >= 1; o /= 2) v += __shfl_xor(v, o, 64);
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) lds[wave] = v;
  __syncthreads();
  int total = 0;
  for (int w = 0; w < kWaves; ++w) total += lds[w];
  __syncthreads();
  return total;
}

// Nonzero bytes of a 32-bit word: a byte's top bit is set in
// (b & 0x7f) + 0x7f when its low seven bits are not all zero, or in b itself.
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  return __popc((((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u);
}

__global__ __launch_bounds__(kBlock) void compact_count_kernel(const uint8_t* __restrict__ keep,
                                                               int64_t T,
                                                               int32_t* __restrict__ counts) {
  __shared__ int lds[kWaves];
  const int64_t base = (int64_t)blockIdx.x * kTile;
  int c = 0;
  if (base + kTile <= T && (((uintptr_t)(keep + base)) & 15u) == 0) {
    // a whole, aligned tile: 16 consecutive bytes per thread in one load
    const u32x4 v = reinterpret_cast<const u32x4*>(keep + base)[threadIdx.x];
    c = nonzero_bytes(v[0]) + nonzero_bytes(v[1]) + nonzero_bytes(v[2]) + nonzero_bytes(v[3]);
  } else {
    for (int r = 0; r < kRounds; ++r) {
      int64_t t = base + r * kBlock + threadIdx.x;
      if (t < T && keep[t] != 0) ++c;
    }
  }
  int total = block_sum(c, lds);
  if (threadIdx.x == 0) counts[blockIdx.x] = total;
}

// Exclusive scan of counts[0, n_tiles) in place; *n_kept = total.
__global__ __launch_bounds__(kBlock) void compact_scan_kernel(int32_t* __restrict__ counts,
                                                              int64_t n_tiles,
                                                              int64_t* __restrict__ n_kept) {
  __shared__ int64_t wave_tot[kWaves];
  __shared__ int64_t carry_s;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x / 64;
  for (int64_t start = 0; start < n_tiles; start += kBlock) {
    int64_t i = start + threadIdx.x;
    int64_t v = i < n_tiles ? counts[i] : 0;
    // inclusive scan inside the wavefront
    int64_t x = v;
    for (int o = 1; o < 64; o *= 2) {
      int64_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wave_tot[wave] = x;
    __syncthreads();
    int64_t before = carry_s;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    if (i < n_tiles) counts[i] = (int32_t)(before + x - v);
    int64_t chunk = 0;
    for (int w = 0; w < kWaves; ++w) chunk += wave_tot[w];
    __syncthreads();
    if (threadIdx.x == 0) carry_s += chunk;
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_kept = carry_s;
}

// FUSED_SCAN: `offsets` holds the tile counts; the tile's offset is their sum
// over the tiles before it, and the last tile writes the total to *n_kept.
template <bool FUSED_SCAN>
__global__ __launch_bounds__(kBlock) void compact_write_kernel(
    const uint8_t* __restrict__ keep, int64_t T, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ idx, const int32_t* __restrict__ rf_src, int32_t* __restrict__ rf_dst,
    int64_t* __restrict__ n_kept) {
  __shared__ int cnt[kRounds * kWaves];
  __shared__ int pre[kRounds * kWaves];
  __shared__ int red[kWaves];
  const int64_t base = (int64_t)blockIdx.x * kTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x / 64;
  // the tile's keep bytes go through LDS: one 16-byte load per thread for a
  // whole, aligned tile (byte loads otherwise), issued before the offset sum
  __shared__ __attribute__((aligned(16))) uint8_t keep_s[kTile];
  const bool whole = base + kTile <= T && (((uintptr_t)(keep + base)) & 15u) == 0;
  u32x4 kv = {0u, 0u, 0u, 0u};
  if (whole) kv = reinterpret_cast<const u32x4*>(keep + base)[threadIdx.x];
  int tile_before = 0;
  if (FUSED_SCAN) {
    int part = 0;
    for (uint32_t i = threadIdx.x; i < blockIdx.x; i += kBlock) part += offsets[i];
    tile_before = block_sum(part, red);
    if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0)
      *n_kept = (int64_t)tile_before + offsets[blockIdx.x];
  }
  if (whole) {
    reinterpret_cast<u32x4*>(keep_s)[threadIdx.x] = kv;
  } else {
    for (int r = 0; r < kRounds; ++r) {
      const int64_t t = base + r * kBlock + threadIdx.x;
      keep_s[r * kBlock + threadIdx.x] = t < T ? keep[t] : 0;
    }
  }
  __syncthreads();
  uint64_t ballots[kRounds];
  bool mine[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    mine[r] = keep_s[r * kBlock + threadIdx.x] != 0;
    ballots[r] = __ballot(mine[r]);
    if (lane == 0) cnt[r * kWaves + wave] = __popcll(ballots[r]);
  }
  __syncthreads();
  if (wave == 0) {   // exclusive prefix of the 64 (round, wave) counts, round-major
    int v = cnt[lane];
    int x = v;
    for (int o = 1; o < 64; o *= 2) {
      int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    pre[lane] = x - v;
  }
  __syncthreads();
  const int64_t tile_off = FUSED_SCAN ? (int64_t)tile_before : (int64_t)offsets[blockIdx.x];
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    if (mine[r]) {
      int64_t t = base + r * kBlock + threadIdx.x;
      int64_t pos = tile_off + pre[r * kWaves + wave] + __popcll(ballots[r] & below);
      idx[pos] = (int32_t)t;
      if (rf_dst) rf_dst[pos] = rf_src[t];
    }
  }
}

}  // namespace

dp_status launch_compact(const uint8_t* keep, int64_t T, int32_t* idx, int64_t* n_kept,
                         const int32_t* rf_src, int32_t* rf_dst, int32_t* ws, hipStream_t s) {
  const int64_t n_tiles = (T + kTile - 1) / kTile;
  if (n_tiles > 0) {
    hipLaunchKernelGGL(compact_count_kernel, dim3((uint32_t)n_tiles), dim3(kBlock), 0, s, keep,
                       T, ws);
    dp_status st = check_launch("compact_count_kernel");
    if (st != DP_OK) return st;
  }
  if (n_tiles > 0 && n_tiles <= kFusedScanTiles) {
    hipLaunchKernelGGL(compact_write_kernel<true>, dim3((uint32_t)n_tiles), dim3(kBlock), 0, s,
                       keep, T, ws, idx, rf_src, rf_dst, n_kept);
    return check_launch("compact_write_kernel");
  }
  hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(kBlock), 0, s, ws, n_tiles, n_kept);
  dp_status st = check_launch("compact_scan_kernel");
  if (st != DP_OK || n_tiles == 0) return st;
  hipLaunchKernelGGL(compact_write_kernel<false>, dim3((uint32_t)n_tiles), dim3(kBlock), 0, s,
                     keep, T, ws, idx, rf_src, rf_dst, n_kept);
  return check_launch("compact_write_kernel");
}

size_t compact_ws_bytes(int64_t T) {
  int64_t n_tiles = (T + kTile - 1) / kTile;
  return (size_t)(n_tiles > 0 ? n_tiles : 1) * sizeof(int32_t);
}

// ---------------------------------------------------------------------------
// Scratch of dp_compact_index_noalloc: the per-tile counts (then offsets) of
// one call, for up to 2^31 rows (524,288 tiles, 2 MiB).  Each device holds its
// own copy until the process ends; every call on a device uses that copy.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): each device's address is looked up once,
// with that device current, and kept.
// ---------------------------------------------------------------------------
namespace {
constexpr int64_t kScratchTiles = (((int64_t)1 << 31) + kTile - 1) / kTile;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) int32_t scratch[kScratchTiles];
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t compact_scratch_bytes() { return sizeof(int32_t) * (size_t)kScratchTiles; }

dp_status compact_scratch(hipStream_t s, int32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DP_EHIP, "dp_compact_index_noalloc: hipGetDevice: %s",
                                   hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DP_EUNSUPPORTED, "dp_compact_index_noalloc: device %d beyond %d", dev, kMaxDevices);
  if (s) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return fail(DP_EHIP, "dp_compact_index_noalloc: hipStreamGetDevice: %s",
                                     hipGetErrorString(e));
    if (sdev != dev)
      return fail(DP_EINVAL, "dp_compact_index_noalloc: the stream belongs to device %d, the "
                             "current device is %d", (int)sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DP_EHIP, "dp_compact_index_noalloc: hipGetSymbolAddress: %s",
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return DP_OK;
}

}  // namespace dp
