// dp_compact_index: ascending list of the kept rows (stream compaction).
//
// The gathered cache K[m], V[m] of the DeCoPrune page (section 어떻게
// 동작하나) keeps the selected rows in token order, so the index list is the
// ascending positions with keep != 0.
//
// Three stream-ordered launches, no host synchronisation and no spinning:
//   1. count:  one workgroup per tile of 4096 rows counts its kept rows;
//   2. scan:   one workgroup turns the tile counts into exclusive offsets and
//              writes the total to *n_kept;
//   3. write:  each tile is re-read in 16 rounds of 256 rows; within a round
//              every wavefront takes a ballot of its keep bits and a lane's
//              slot is the popcount of the ballot below it (mbcnt); the 64
//              (round, wavefront) counts of the tile get an exclusive prefix in
//              LDS, so every kept row lands at its final position.
#include <mutex>

#include "dp_internal.h"

namespace dp {
namespace {

constexpr int kRounds = 16;
constexpr int kTile = kBlock * kRounds;   // 4096 rows per tile
constexpr int kWaves = kBlock / 64;

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

__global__ __launch_bounds__(kBlock) void compact_count_kernel(const uint8_t* __restrict__ keep,
                                                               int64_t T,
                                                               int32_t* __restrict__ counts) {
  __shared__ int lds[kWaves];
  const int64_t base = (int64_t)blockIdx.x * kTile;
  int c = 0;
  for (int r = 0; r < kRounds; ++r) {
    int64_t t = base + r * kBlock + threadIdx.x;
    if (t < T && keep[t] != 0) ++c;
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

__global__ __launch_bounds__(kBlock) void compact_write_kernel(
    const uint8_t* __restrict__ keep, int64_t T, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ idx, const int32_t* __restrict__ rf_src, int32_t* __restrict__ rf_dst) {
  __shared__ int cnt[kRounds * kWaves];
  __shared__ int pre[kRounds * kWaves];
  const int64_t base = (int64_t)blockIdx.x * kTile;
  const int lane = threadIdx.x & 63, wave = threadIdx.x / 64;
  uint64_t ballots[kRounds];
  bool mine[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    int64_t t = base + r * kBlock + threadIdx.x;
    mine[r] = t < T && keep[t] != 0;
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
  const int64_t tile_off = offsets[blockIdx.x];
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
  hipLaunchKernelGGL(compact_scan_kernel, dim3(1), dim3(kBlock), 0, s, ws, n_tiles, n_kept);
  dp_status st = check_launch("compact_scan_kernel");
  if (st != DP_OK || n_tiles == 0) return st;
  hipLaunchKernelGGL(compact_write_kernel, dim3((uint32_t)n_tiles), dim3(kBlock), 0, s, keep, T,
                     ws, idx, rf_src, rf_dst);
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
