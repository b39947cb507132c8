// Device twin of dpsynth.kv_rows_host(): fills a buffer with table entries
// picked by the SplitMix64 output function (Steele, Lea and Flood, 2014) of a
// seeded Weyl sequence.  Input generation only; no part of the compaction
// method lives here.
//
// Also a plain 16-byte-vector copy of a known size, the reference the
// benchmark uses for the device-to-device bandwidth ceiling and to scale
// hardware byte counters.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix(uint64_t skey, uint64_t key) {
  uint64_t z = skey + (key + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

template <typename T>
__global__ __launch_bounds__(256) void fill_kernel(T* __restrict__ dst, uint64_t skey,
                                                   uint64_t key_base, int64_t n,
                                                   const T* __restrict__ table) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = table[mix(skey, key_base + (uint64_t)i) >> 48];
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void calib_copy_kernel(const u32x4* __restrict__ src,
                                                         u32x4* __restrict__ dst, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace

extern "C" int dpsynth_copy(void* dst, const void* src, int64_t n16, void* stream) {
  if (n16 <= 0) return 0;
  if (!dst || !src || (((uintptr_t)dst | (uintptr_t)src) & 15u)) return 1;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks >= ((int64_t)1 << 31)) return 1;
  hipLaunchKernelGGL(calib_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int dpsynth_fill(void* dst, int dtype, uint64_t skey, uint64_t key_base,
                            int64_t n, const void* table, void* stream) {
  if (n <= 0) return 0;
  if (!dst || !table) return 1;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == 0)
    hipLaunchKernelGGL(fill_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                       (uint32_t*)dst, skey, key_base, n, (const uint32_t*)table);
  else
    hipLaunchKernelGGL(fill_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                       (uint16_t*)dst, skey, key_base, n, (const uint16_t*)table);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
