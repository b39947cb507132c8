// dp_attention: attention of a chunk's queries over the compacted KV cache.
//
// The DeCoPrune page (sections 무엇인가 and 전제와 한계) motivates the
// compaction by the cost of each new chunk attending to the whole history KV
// cache; the continuation speed-up it reports comes from this step running
// over the shorter cache.  For every head h and query i < n_q:
//   O[i][h] = sum_{j < n_kv} softmax_j(scale * <Q[i][h], K[j][h]>) V[j][h]
// with bf16 inputs and outputs, fp32 accumulation and an online softmax.
//
// Workgroup = 128 queries of one head, 4 wavefronts of 32 queries.  Per tile of
// 64 keys (staged in LDS: K row-major, V transposed):
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16, Q held in registers as the B
//                  operand, so a lane owns one query and 16 of its scores and
//                  the softmax statistics stay in the lane (plus its partner
//                  lane 32 apart, which owns the other 16 keys of the tile);
//   O^T += V^T P^T the probabilities are fed back from the S^T accumulators as
//                  the B operand without moving between lanes: the order of the
//                  contraction over keys is permuted to match, and the V^T
//                  operand reads the same permutation from LDS.
// Query tiles of one head are placed on one XCD (workgroup i runs on XCD
// i mod 8), so the key/value tiles they all stream are shared in that XCD's L2.
//
// A head's keys come in up to two segments, streamed one after the other:
// segment 0 is either the dense token-major cache [rows][heads][head_dim] or,
// for DeCoPrune-HS, the head's own run of rows in the packed per-head cache
// (offsets from dp_hs_offsets, consecutive rows head_dim apart); segment 1 is
// an optional dense block (the chunk's own keys next to a ragged history).
#include "dp_internal.h"

namespace dp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;          // head_dim
constexpr int kBM = 128;         // queries per workgroup
constexpr int kBN = 64;          // keys per tile
constexpr int kKP = kD + 8;      // K tile row pitch (bf16 elements)
constexpr int kVP = kBN + 4;     // V^T tile row pitch (bf16 elements): 34 dwords, so the
                                 // 32 rows one 8-byte read spans fall in distinct banks
constexpr int kXcds = 8;
constexpr int kBufferWord3 = 0x00020000;   // gfx9 raw buffer descriptor, dword 3

struct AttnArgs {
  const uint16_t* q;
  uint16_t* o;
  const uint16_t* k0;  // segment 0
  const uint16_t* v0;
  const int64_t* n_kv; // dense segment 0: device count, or NULL
  const int64_t* off;  // ragged segment 0: device head-row offsets of this layer's heads, or NULL
  int64_t cap0;        // rows (dense) or head rows (ragged) of segment 0
  const uint16_t* k1;  // segment 1: dense [n1][heads][head_dim], or NULL
  const uint16_t* v1;
  int64_t n1;
  int64_t n_q;
  int64_t row;        // elements per token row: n_heads * head_dim
  int32_t n_heads;
  int32_t n_qt;       // query tiles per head
  int32_t xcd_map;    // 1: group the query tiles of a head on one XCD
  float c;            // scale * log2(e)
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool RAGGED>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBN * kKP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kD * kVP];

  int head, qt;
  if (a.xcd_map) {
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int j = slot / a.n_qt;                 // j-th head placed on this XCD
    qt = slot % a.n_qt;
    head = j * kXcds + xcd;
    if (RAGGED && a.n_heads <= kBlock) {
      // Ragged runs differ in length, so heads are ranked by length (longest
      // first, ties by index) and dealt to the XCDs in snake order: every XCD
      // gets the same number of heads and nearly the same number of keys, and
      // the longest heads start first.
      __shared__ int64_t len_s[kBlock];
      __shared__ int head_of_rank[kBlock];
      const int t = threadIdx.x;
      if (t < a.n_heads) {
        const int64_t lo = min(max(a.off[t], (int64_t)0), a.cap0);
        const int64_t hi = min(max(a.off[t + 1], lo), a.cap0);
        len_s[t] = hi - lo;
      }
      __syncthreads();
      if (t < a.n_heads) {
        const int64_t mine = len_s[t];
        int rank = 0;
        for (int u = 0; u < a.n_heads; ++u) {
          const int64_t other = len_s[u];
          rank += (other > mine) | ((other == mine) & (u < t));
        }
        head_of_rank[rank] = t;
      }
      __syncthreads();
      head = head_of_rank[j * kXcds + ((j & 1) ? kXcds - 1 - xcd : xcd)];
    }
  } else {
    head = blockIdx.x / a.n_qt;
    qt = blockIdx.x % a.n_qt;
  }
  if (head >= a.n_heads) return;
  // segment 0 of this head: base element, key stride, count (device values clamped
  // to the capacity, so no key outside [0, cap0) is read)
  int64_t base0, stride0, n0;
  if (RAGGED) {
    const int64_t lo = min(max(a.off[head], (int64_t)0), a.cap0);
    const int64_t hi = min(max(a.off[head + 1], lo), a.cap0);
    base0 = lo * kD;
    stride0 = kD;
    n0 = hi - lo;
  } else {
    base0 = (int64_t)head * kD;
    stride0 = a.row;
    n0 = a.cap0;
    if (a.n_kv) n0 = max(min(n0, *a.n_kv), (int64_t)0);
  }
  const int64_t n1 = RAGGED && a.k1 ? a.n1 : 0;
  const int64_t t0 = (n0 + kBN - 1) / kBN;
  const int64_t n_tiles = t0 + (n1 + kBN - 1) / kBN;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hf = lane >> 5, l32 = lane & 31;
  const int64_t qi = (int64_t)qt * kBM + wave * 32 + l32;
  const bool qvalid = qi < a.n_q;

  // Q as the B operand of S^T = K Q^T: lane holds Q[qi][d] for d = 16 ds + 8 hf + e.
  bf16x8 qb[kD / 16];
  {
    const uint16_t* qrow = a.q + (qvalid ? qi : 0) * a.row + (int64_t)head * kD;
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      u32x4 r = {0u, 0u, 0u, 0u};
      if (qvalid) r = *reinterpret_cast<const u32x4*>(qrow + ds * 16 + hf * 8);
      qb[ds] = __builtin_bit_cast(bf16x8, r);
    }
  }

  f32x16 o[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  // Each thread moves 4 consecutive keys of one 8-element chunk of K and of V.
  // K rows go to LDS as 16-byte writes (the 16 lanes of a key cover its row);
  // V is transposed in registers and written as four keys per 8-byte write,
  // with the keys varying fastest across lanes so that the lanes of a write
  // fall in distinct banks.  The next tile's loads are issued before the
  // current tile's MFMAs so that their latency is hidden.
  const int key4 = (threadIdx.x >> 4) * 4, ch = threadIdx.x & 15;        // K
  const int vkey4 = (threadIdx.x & 15) * 4, vch = threadIdx.x >> 4;      // V
  u32x4 kr[4], vr[4];
  // Tile loads go through buffer descriptors whose base is the tile's first
  // row and whose size ends at the segment's last valid row, so rows past it
  // read as zeros without a per-lane branch (gfx9 buffer range check; the lane
  // offsets stay below 64 rows of the segment's stride, validated on the host).
  auto load_tile = [&](int64_t t) {
    const bool s1 = RAGGED && t >= t0;             // uniform per workgroup
    const uint16_t* kp = s1 ? a.k1 : a.k0;
    const uint16_t* vp = s1 ? a.v1 : a.v0;
    const int64_t stride = s1 ? a.row : stride0;
    const int64_t base = s1 ? (int64_t)head * kD : base0;
    const int64_t n = s1 ? n1 : n0;
    const int64_t kv0 = (s1 ? t - t0 : t) * kBN;
    const int64_t off = base + kv0 * stride;
    const uint32_t bytes = (uint32_t)(min(n - kv0, (int64_t)kBN) * stride * 2);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(kp + off), 0, (int)bytes, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(vp + off), 0, (int)bytes, kBufferWord3);
    const uint32_t st2 = (uint32_t)stride * 2u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      kr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rk, (int)((key4 + u) * st2 + ch * 16), 0, 0));
      vr[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            rv, (int)((vkey4 + u) * st2 + vch * 16), 0, 0));
    }
  };
  if (n_tiles > 0) load_tile(0);
  for (int64_t t = 0; t < n_tiles; ++t) {
    const bool in1 = RAGGED && t >= t0;
    const int64_t kv0 = (in1 ? t - t0 : t) * kBN;   // first key of the tile in its segment
    const int64_t nkv = in1 ? n1 : n0;
    // ---- stage K (row-major) and V (transposed) of 64 keys in LDS ----
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(Ks + (key4 + u) * kKP + ch * 8) = kr[u];
#pragma unroll
    for (int e = 0; e < 8; ++e) {            // element e of the chunk for the 4 keys
      // byte permutes: the low (even e) or high (odd e) halves of two keys' words
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x2 w;
      w[0] = __builtin_amdgcn_perm(vr[1][e >> 1], vr[0][e >> 1], sel);
      w[1] = __builtin_amdgcn_perm(vr[3][e >> 1], vr[2][e >> 1], sel);
      *reinterpret_cast<u32x2*>(Vt + (vch * 8 + e) * kVP + vkey4) = w;
    }
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(t + 1);

    // ---- S^T = K Q^T for two 32-key tiles: the two accumulation chains are
    // interleaved so that consecutive MFMAs do not wait on each other ----
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kt][i] = 0.0f;
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      const bf16x8 ka0 = *reinterpret_cast<const bf16x8*>(Ks + l32 * kKP + ds * 16 + hf * 8);
      const bf16x8 ka1 = *reinterpret_cast<const bf16x8*>(Ks + (32 + l32) * kKP + ds * 16 + hf * 8);
      s[0] = mfma(ka0, qb[ds], s[0]);
      s[1] = mfma(ka1, qb[ds], s[1]);
    }

    // ---- online softmax (base 2), lane-local per query plus partner lane ----
    // Scores are kept unscaled; with c > 0 the scaled maximum is c * max.  Keys
    // past the segment's end exist only in its last tile.
    const int64_t lim = nkv - kv0;                     // valid keys in this tile (> 0)
    if (lim < kBN) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * 32 + 8 * (i >> 2) + 4 * hf + (i & 3) >= lim) s[kt][i] = -INFINITY;
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kt][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * a.c;
    // The reference m is raised only when a score exceeds it by more than 2^8
    // (decided for the whole wavefront, so the rescale is skipped together);
    // below that the probabilities exp2(c s - m) stay under 256, which fp32
    // sums and the bf16 probabilities carry without loss of relative precision.
    if (__builtin_amdgcn_ballot_w64(mt > m + 8.0f)) {
      const float mn = fmaxf(m, mt);
      const float corr = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      l *= corr;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= corr;
    }
    float ls = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], a.c, -m));
        s[kt][i] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 32, 64);
    l += ls;

    // ---- P^T as B operands: key step ks takes accumulator entries 8 (ks & 1) .. +8 of
    // tile ks >> 1, i.e. keys 32 (ks>>1) + 16 (ks&1) + 8 (e>>2) + 4 hf + (e&3) ----
    bf16x8 pb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pack_bf16_hw(s[ks >> 1][8 * (ks & 1) + 2 * e], s[ks >> 1][8 * (ks & 1) + 2 * e + 1]);
      pb[ks] = __builtin_bit_cast(bf16x8, w);
    }

    // ---- O^T += V^T P^T, V^T read in the same key order; per key step the four
    // dim tiles' fragments are read together and feed independent accumulators ----
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int base = (ks >> 1) * 32 + 16 * (ks & 1) + 4 * hf;
      bf16x8 va[kD / 32];
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) {
        const uint16_t* vrow = Vt + (dt * 32 + l32) * kVP + base;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
        va[dt] = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
      }
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) o[dt] = mfma(va[dt], pb[ks], o[dt]);
    }
    __syncthreads();
  }

  // ---- O[qi][head][d], d = 32 dt + 8 g + 4 hf + (0..3) ----
  if (qvalid) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* orow = a.o + qi * a.row + (int64_t)head * kD;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16_hw(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv);
        w[1] = pack_bf16_hw(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + dt * 32 + 8 * g + 4 * hf) = w;
      }
  }
}

}  // namespace

namespace {

dp_status launch(AttnArgs& a, const void* q, void* o, int64_t n_q, int32_t n_heads, float scale,
                 hipStream_t s) {
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.o = reinterpret_cast<uint16_t*>(o);
  a.n_q = n_q;
  a.row = (int64_t)n_heads * kD;
  a.n_heads = n_heads;
  a.n_qt = (int32_t)((n_q + kBM - 1) / kBM);
  a.xcd_map = n_heads % kXcds == 0;
  a.c = scale * 1.4426950408889634f;
  const uint64_t blocks = (uint64_t)a.n_qt * n_heads;
  if (blocks == 0) return DP_OK;
  if (a.off)
    hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3((uint32_t)blocks), dim3(kBlock), 0, s, a);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3((uint32_t)blocks), dim3(kBlock), 0, s, a);
  return check_launch("attn_fwd_kernel");
}

}  // namespace

dp_status launch_attention(const void* q, const void* k, const void* v, void* o, int64_t n_q,
                           int64_t kv_cap, const int64_t* n_kv, int32_t n_heads, float scale,
                           hipStream_t s) {
  AttnArgs a{};
  a.k0 = reinterpret_cast<const uint16_t*>(k);
  a.v0 = reinterpret_cast<const uint16_t*>(v);
  a.n_kv = n_kv;
  a.cap0 = kv_cap;
  return launch(a, q, o, n_q, n_heads, scale, s);
}

dp_status launch_hs_attention(const void* q, const void* k_ragged, const void* v_ragged,
                              int64_t ragged_capacity, const int64_t* head_offsets,
                              const void* k_chunk, const void* v_chunk, int64_t n_chunk, void* o,
                              int64_t n_q, int32_t n_heads, float scale, hipStream_t s) {
  AttnArgs a{};
  a.k0 = reinterpret_cast<const uint16_t*>(k_ragged);
  a.v0 = reinterpret_cast<const uint16_t*>(v_ragged);
  a.off = head_offsets;
  a.cap0 = ragged_capacity;
  a.k1 = reinterpret_cast<const uint16_t*>(k_chunk);
  a.v1 = reinterpret_cast<const uint16_t*>(v_chunk);
  a.n1 = k_chunk ? n_chunk : 0;
  return launch(a, q, o, n_q, n_heads, scale, s);
}

}  // namespace dp
