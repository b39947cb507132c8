// dp_attention: attention of a chunk's queries over the compacted KV cache.
//
// The DeCoPrune page (sections 무엇인가 and 전제와 한계) motivates the
// compaction by the cost of each new chunk attending to the whole history KV
// cache; the continuation speed-up it reports comes from this step running
// over the shorter cache.  For every head h and query i < n_q:
//   O[i][h] = sum_{j < n_kv} softmax_j(scale * <Q[i][h], K[j][h]>) V[j][h]
// with bf16 inputs and outputs, fp32 accumulation and an online softmax.
//
// Workgroup = 256 queries of one head, 8 wavefronts of 32 queries (one
// workgroup per CU: two wavefronts per SIMD).  Per tile of 64 keys (K and V
// row-major in LDS, brought in by the load unit itself, double-buffered):
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16, Q held in registers as the B
//                  operand, so a lane owns one query and 16 of its scores and
//                  the softmax statistics stay in the lane (plus its partner
//                  lane 32 apart, which owns the other 16 keys of the tile);
//   O^T += V^T P^T the probabilities are fed back from the S^T accumulators as
//                  the B operand without moving between lanes: the order of the
//                  contraction over keys is permuted to match, and the V^T
//                  operand is read in the same order by transposing LDS reads.
// The MFMAs of the next tile's S^T and of the previous tile's O^T update are
// issued while the current tile's probabilities are formed.
// Query tiles of one head are placed on one XCD (workgroup i runs on XCD
// i mod 8), so the key/value tiles they all stream are shared in that XCD's L2;
// over a ragged cache each half of a head's tiles is placed on one XCD.
//
// A head's keys come in up to two segments, streamed one after the other:
// segment 0 is either the dense token-major cache [rows][heads][head_dim] or,
// for DeCoPrune-HS, the head's own run of rows in the packed per-head cache
// (offsets from dp_hs_offsets, consecutive rows head_dim apart); segment 1 is
// an optional dense block (the chunk's own keys next to a ragged history).
//
// Compressed time axis (dp_attention_lag): keys past the RoPE knee carry the
// phase t/c instead of t~ = t/c + A, A the same for all of them, so their
// scores need the query turned back by A on the temporal pairs.  The dense
// cache is then streamed as three segments: the lagged rows before the plain
// range, the lagged rows after it (both against the rotated query) and the
// plain range (against the query as given); the query fragment is rebuilt
// once, when the stream reaches the plain range.  On the ragged HS cache
// (dp_hs_attention_lag) each head's run is lagged except its last plain_tail
// rows, which are streamed after it together with the chunk's own block, both
// plain.
//
// Split keys (DP_KEY_SPLIT): a key row keeps the temporal blocks of all heads
// first, so a head's key row is two pieces, its temporal block and its other
// dims; in a ragged run the run's temporal blocks come first.  Only the
// addresses the tile loads read from change: each lane fetches the 16-byte
// chunk that belongs at its LDS position from the piece that holds it, and the
// tile lands in LDS exactly as for interleaved keys.
#include <type_traits>

#include "dp_internal.h"

namespace dp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;          // LDS pointers
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kD = 128;          // head_dim
// Wavefronts per workgroup (32 queries each) by mode: dense and lagged caches
// use 8 (one workgroup per CU, every key/value tile feeds 256 queries); the
// ragged cache uses 4 (two workgroups per CU: twice as many, smaller units of
// work balance per-head runs of unequal length better).
enum { kDense = 0, kRagged = 1, kLag = 2, kRaggedLag = 3 };
constexpr int kSplit = 4;        // mode bit: split keys

template <int MODE> struct Shape {
  static constexpr int kWaves = ((MODE & 3) == kRagged || (MODE & 3) == kRaggedLag) ? 4 : 8;
  static constexpr int kBlock = 64 * kWaves;
  static constexpr int kBM = 32 * kWaves;          // queries per workgroup
  static constexpr int kDmaPerWave = 16 / kWaves;  // 1 KiB tile blocks per operand and wavefront
};
constexpr int kBN = 64;          // keys per tile
constexpr int kXcds = 8;
constexpr int kBufferWord3 = 0x00020000;   // gfx9 raw buffer descriptor, dword 3

// Placement of one pipeline step's instructions: N groups of one MFMA, one LDS
// read and three VALU instructions (after eight LDS reads issued first).  The
// compiler's own order issued the softmax VALU work beside the first half of
// the MFMAs and left the rest of them without any; this spreads it over all
// 32 (measured, outputs bit-identical: +1.6 % dense, +2 % on the ragged cache;
// four or five VALU per MFMA, or 4 or 12 reads first, were slower).  SALU: one
// scalar instruction per group as well, which the ragged kernel (4 wavefronts)
// gained 0-2 % from in two comparisons and the dense one lost 0.4 %.
template <int N, bool SALU> __device__ __forceinline__ void step_schedule() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // VALU
    if constexpr (SALU) __builtin_amdgcn_sched_group_barrier(0x004, 1, 0);   // SALU
    step_schedule<N - 1, SALU>();
  }
}


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
  // kLag: rows outside [plain_begin, plain_end) see the query rotated by
  // -lag on pairs [pair_begin, pair_begin + n_pairs); kRaggedLag: all rows of a
  // head's run but its last plain_tail do (the chunk block is plain)
  int64_t plain_begin;
  int64_t plain_end;
  int64_t plain_tail;
  const float* theta;
  int32_t pair_begin;
  int32_t n_pairs;
  float lag;
  // split keys: 16-byte chunks [tvb, tvb + tvc) of a head's key row are its
  // temporal block (in the leading plane), the other 16 - tvc chunks follow
  int32_t tvb;
  int32_t tvc;
};

// The two values a lane and its partner 32 lanes away hold, in lane order
// (v_permlane32_swap: a VALU exchange, no LDS round trip).
__device__ __forceinline__ f32x2 with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return f32x2{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// Workgroup barrier without a memory fence (a fence would also wait for every
// vector-memory load still in flight).  Callers first wait for the tile loads
// the barrier publishes; every LDS read before it has been consumed; the memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int MODE>
__global__ __launch_bounds__(Shape<MODE>::kBlock) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(AttnArgs a) {
  constexpr bool RAGGED = (MODE & 3) == kRagged || (MODE & 3) == kRaggedLag;
  constexpr bool LAG = (MODE & 3) == kLag || (MODE & 3) == kRaggedLag;
  constexpr bool SPLIT = (MODE & kSplit) != 0;
  constexpr int kAttnBlock = Shape<MODE>::kBlock, kBM = Shape<MODE>::kBM;
  constexpr int kDmaPerWave = Shape<MODE>::kDmaPerWave;
  __shared__ __attribute__((aligned(1024))) uint8_t Kb0[kBN * 256], Kb1[kBN * 256];
  __shared__ __attribute__((aligned(1024))) uint8_t Vb0[kBN * 256], Vb1[kBN * 256];
  lds_u8* const kb0 = (lds_u8*)Kb0;
  lds_u8* const kb1 = (lds_u8*)Kb1;
  lds_u8* const vb0 = (lds_u8*)Vb0;
  lds_u8* const vb1 = (lds_u8*)Vb1;
  __shared__ f32x2 lag_cs[LAG ? kD / 2 : 1];
  if constexpr (LAG) {
    // {cos, sin} of the fp32 angle theta_j * (-lag), from fp64 sincos rounded to
    // fp32: the table the in-place re-index builds for a phase change of -lag
    for (int j = threadIdx.x; j < a.n_pairs; j += kAttnBlock) {
      const float ang = a.theta[j] * -a.lag;
      double sd, cd;
      sincos((double)ang, &sd, &cd);
      lag_cs[j] = f32x2{(float)cd, (float)sd};
    }
    __syncthreads();
  }

  int head, qt;
  if (a.xcd_map) {
    const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    if (RAGGED && a.n_heads <= kAttnBlock) {
      // Ragged runs differ in length.  Each head's query tiles are cut into two
      // halves, the 2H halves ranked by run length (longest first, ties by
      // head, so a head's halves are adjacent) and dealt to the XCDs in snake
      // order: every XCD gets the same number of halves and nearly the same
      // number of keys, a head's keys are read by at most two XCDs, and on
      // each XCD the longest halves start first.  Whole heads dealt the same
      // way leave the XCDs unequal when the heads per XCD are odd and the
      // lengths bimodal (5 per XCD, static and dynamic heads: half the XCDs
      // get three long heads); the halves were 5 % faster there and the same
      // at equal lengths.  The grid holds 2H halves of ceil(tiles / 2) slots.
      __shared__ int64_t len_s[kAttnBlock];
      __shared__ int head_of_rank[kAttnBlock];
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
      const int half_tiles = (a.n_qt + 1) >> 1;
      const int j = slot / half_tiles, u = slot - j * half_tiles;
      const int r = j * kXcds + ((j & 1) ? kXcds - 1 - xcd : xcd);   // rank of the half
      if (r >= 2 * a.n_heads) return;
      head = head_of_rank[r >> 1];
      qt = (r & 1) * half_tiles + u;
      if (qt >= a.n_qt) return;
    } else {
      const int j = slot / a.n_qt;               // j-th head placed on this XCD
      qt = slot % a.n_qt;
      head = j * kXcds + xcd;
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
  // K pieces of split keys: elements of a temporal block and of the other dims
  // of one head row; the K base of a dense segment is the token row (the head's
  // pieces are found by the lanes' chunk offsets), of a ragged run its start,
  // with its other dims n0 temporal blocks further
  const int64_t kte = SPLIT ? (int64_t)a.tvc * 8 : 0, kse = SPLIT ? kD - kte : 0;
  const int64_t kbase0 = SPLIT && !RAGGED ? 0 : base0;
  // kLag: rows [0, pa) and [pb, n) lagged, [pa, pb) plain
  const int64_t pa = LAG ? min(a.plain_begin, n0) : 0;
  const int64_t pb = LAG ? min(max(a.plain_end, a.plain_begin), n0) : 0;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  const int64_t qi = (int64_t)qt * kBM + wave * 32 + l32;
  const bool qvalid = qi < a.n_q;

  // Q as the B operand of S^T = K Q^T: lane holds Q[qi][d] for d = 16 ds + 8 hf + e,
  // i.e. pairs 8 ds + 4 hf + (0..3); with `lagged` the temporal pairs are rotated
  // by -lag (fp32 products and sums rounded separately, then bf16 RNE).
  bf16x8 qb[kD / 16];
  // The wavefront's 32 query rows are read through one buffer descriptor that
  // ends at the last valid query, so rows past n_q read as zeros; the lane
  // offsets are recomputed at each call and hold no registers in between.
  auto load_q = [&](bool lagged) {
    const int64_t q_first = (int64_t)qt * kBM + wave * 32;
    const int64_t q_rows = max(min(a.n_q - q_first, (int64_t)32), (int64_t)0);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.q + q_first * a.row + (int64_t)head * kD), 0, (int)(q_rows * a.row * 2),
        kBufferWord3);
    const int q_off = (int)(l32 * (a.row * 2) + hf * 16);
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      u32x4 r = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, q_off + ds * 32,
                                                                                0, 0));
      if (LAG && lagged) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = ds * 8 + hf * 4 + u - a.pair_begin;
          if (j >= 0 && j < a.n_pairs) {
            const f32x2 cs = lag_cs[j];
            float a2, b2;
            rotate_pair(bf16_lo(r[u]), bf16_hi(r[u]), cs.x, cs.y, a2, b2);
            r[u] = pack_bf16_hw(a2, b2);
          }
        }
      }
      qb[ds] = __builtin_bit_cast(bf16x8, r);
    }
  };

  // ---- key/value tiles: straight from HBM into LDS, double-buffered ----
  // The head's keys are streamed as passes over contiguous row ranges (one per
  // segment; a lagged cache has up to three), each a software pipeline of its
  // own.  A tile is 64 rows of 256 bytes for K and for V, unpadded; each
  // wavefront moves kDmaPerWave KiB of each with 16-byte-per-lane loads whose
  // LDS target is the next 1 KiB (lane L writes bytes 16 L of it), so row
  // r = 4 (kDmaPerWave wave + u) + L / 16 lands in position L % 16.  The lane
  // loads the global chunk that belongs there under an XOR swizzle of the
  // row's 16-byte chunks: K chunk c sits at position c ^ (r & 15) (the 16
  // rows one 16-byte fragment read serves per pass hit all 64 banks once), V
  // chunk c at c ^ 4 (r & 3) (a transposing read serves 32 lanes per pass:
  // 4 rows x 4 chunks of one dim tile, which this places on all 64 banks once;
  // measured: the former c ^ 2 (r & 7) put them on 32 banks, and bank
  // conflicts took a third of the LDS cycles).  Descriptors end at the range's
  // last row, so rows past it arrive as zeros.
  const int dma_row = wave * 4 * kDmaPerWave + (lane >> 4), dma_pos = lane & 15;
  // Split keys: the chunk c = dma_pos ^ (r & 15) a lane loads is found in a
  // dense token row at head h's temporal chunk h tvc + (c - tvb) or, for the
  // other chunks, after all heads' temporal blocks at n_heads tvc +
  // h (16 - tvc) + s (16-byte units; s counts the non-temporal chunks before
  // c); in a ragged run, at c - tvb of the row's temporal piece or s of its
  // other-dims piece.  (Recomputed per tile: a few integer operations.)
  // (which operands to load is a flag, not a null LDS pointer: LDS offset 0 is
  // a valid buffer address)
  // planar: K is a ragged run of split keys (two pieces, kp and kp2)
  auto load_tile = [&](const uint16_t* kp, const uint16_t* kp2, const uint16_t* vp, uint32_t st2,
                       int64_t rows_left, lds_u8* kdst, lds_u8* vdst, bool do_k, bool do_v,
                       bool planar) {
    const uint32_t rows = (uint32_t)min(rows_left, (int64_t)kBN);
    const uint32_t bytes = rows * st2;
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) {
      const int r = dma_row + 4 * u;
      const uint32_t row_off = (uint32_t)r * st2;
      if (do_k) {
        lds_u8* const kl = kdst + (wave * kDmaPerWave + u) * 1024;
        const int c = dma_pos ^ (r & 15);
        const bool tq = c >= a.tvb && c < a.tvb + a.tvc;
        const int sidx = c < a.tvb ? c : c - a.tvc;
        if (SPLIT && RAGGED && planar) {
          // two pieces, each through a descriptor that ends at the tile's last
          // row (rows past it read as zeros); a lane loads from the one holding
          // its chunk
          const uint32_t tb = (uint32_t)kte * 2, sb = (uint32_t)kse * 2;
          if (tq) {
            const __amdgpu_buffer_rsrc_t rt =
                __builtin_amdgcn_make_buffer_rsrc((void*)kp, 0, (int)(rows * tb), kBufferWord3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rt, kl, 16,
                                                     (uint32_t)r * tb + ((uint32_t)(c - a.tvb) << 4),
                                                     0, 0, 0);
          } else {
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc((void*)kp2, 0, (int)(rows * sb), kBufferWord3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, kl, 16,
                                                     (uint32_t)r * sb + ((uint32_t)sidx << 4), 0,
                                                     0, 0);
          }
        } else {
          const uint32_t koff =
              SPLIT ? (uint32_t)(tq ? head * a.tvc + (c - a.tvb)
                                    : a.n_heads * a.tvc + head * (16 - a.tvc) + sidx) << 4
                    : (uint32_t)c << 4;
          const __amdgpu_buffer_rsrc_t rk =
              __builtin_amdgcn_make_buffer_rsrc((void*)kp, 0, (int)bytes, kBufferWord3);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, kl, 16, row_off + koff, 0, 0, 0);
        }
      }
      if (do_v) {
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)vp, 0, (int)bytes, kBufferWord3);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, vdst + (wave * kDmaPerWave + u) * 1024, 16,
            row_off + ((dma_pos ^ ((r & 3) << 2)) << 4), 0, 0, 0);
      }
    }
  };

  // ---- fragment addresses (bytes within a tile) ----
  // K for S^T = K Q^T: lane (l32, hf) reads row kt 32 + l32, chunk 2 ds + hf.
  uint32_t k_off[kD / 16];
#pragma unroll
  for (int ds = 0; ds < kD / 16; ++ds)
    k_off[ds] = l32 * 256 + (((2 * ds + hf) ^ (l32 & 15)) << 4);
  // V^T for O^T += V^T P^T, through ds_read_b64_tr_b16: within each 16 lanes,
  // lane i returns element i % 4 of the 8 bytes lanes 4 k + i / 4 (k = 0..3)
  // point at.  Lane L (sub = L & 15, group (hf, half) = L >> 4) points at key
  // row 16 ks + 8 w + 4 hf + sub / 4, dims 32 dt + 16 half + 4 (sub % 4) .. +3,
  // so it receives V[16 ks + 8 w + 4 hf + k][32 dt + l32], k = 0..3: the keys
  // the P^T operand lists for contraction slots 4 w .. 4 w + 3.
  uint32_t v_off[kD / 32];
  {
    const int sub = lane & 15, half = (lane >> 4) & 1;
    const int vrow = 4 * hf + (sub >> 2);                  // row within 8, = row & 7
    const int lo = 2 * half + ((sub & 3) >> 1);            // chunk bits 0..1 (not swizzled)
    const uint32_t v_a = vrow * 256 + (lo << 4) + 8 * (sub & 1);
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) v_off[dt] = v_a + ((dt ^ (vrow & 3)) << 6);
  }

  f32x16 o[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
  float m = -INFINITY, l = 0.0f;

  // S^T of one tile: two 32-key halves, interleaved accumulation chains
  auto s_tile = [&](const lds_u8* kb, f32x16 (&s)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kt][i] = 0.0f;
#pragma unroll
    for (int ds = 0; ds < kD / 16; ++ds) {
      const bf16x8 ka0 = *reinterpret_cast<const lds_bf16x8*>(kb + k_off[ds]);
      const bf16x8 ka1 = *reinterpret_cast<const lds_bf16x8*>(kb + k_off[ds] + 32 * 256);
      s[0] = mfma(ka0, qb[ds], s[0]);
      s[1] = mfma(ka1, qb[ds], s[1]);
    }
  };
  // mask the keys past the segment's end (last tile only), then the running
  // maximum: raised only when a score exceeds it by more than 2^8 (decided for
  // the whole wavefront, so the rescale is skipped together); below that the
  // probabilities exp2(c s - m) stay under 256, which fp32 sums and the bf16
  // probabilities carry without loss of relative precision.  Scores are kept
  // unscaled; with c > 0 the scaled maximum is c * max.
  // (split in three so that the maximum of a full tile, the common case, is
  // plain VALU work the scheduler can place among the MFMAs of the same block)
  auto s_mask = [&](f32x16 (&s)[2], int64_t lim) {   // lim: valid keys in the tile (> 0)
    if (lim < kBN) {
      // key kt 32 + 8 (i >> 2) + 4 hf + (i & 3) is past the end: compare the
      // constant part against one per-lane bound (32-bit, nothing hoisted)
      const int rem = (int)lim - 4 * hf;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kt * 32 + 8 * (i >> 2) + (i & 3) >= rem) s[kt][i] = -INFINITY;
    }
  };
  auto tile_max = [&](const f32x16 (&s)[2]) {          // scaled maximum of the tile
    float mt = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kt][i]);
    const f32x2 mp = with_partner(mt);
    return fmaxf(mp.x, mp.y) * a.c;
  };
  auto update_m = [&](float mt) {
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
  };
  auto s_max = [&](f32x16 (&s)[2], int64_t lim) {
    s_mask(s, lim);
    update_m(tile_max(s));
  };
  // probabilities, their sum, and P^T as B operands: key step ks takes
  // accumulator entries 8 (ks & 1) .. +8 of tile ks >> 1, i.e. keys
  // 32 (ks >> 1) + 16 (ks & 1) + 8 (e >> 2) + 4 hf + (e & 3)
  auto s_exp = [&](f32x16 (&s)[2], bf16x8 (&pt)[4]) {
    float ls = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], a.c, -m));
        s[kt][i] = pr;
        ls += pr;
      }
    const f32x2 lp = with_partner(ls);
    l += lp.x + lp.y;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pack_bf16_hw(s[ks >> 1][8 * (ks & 1) + 2 * e], s[ks >> 1][8 * (ks & 1) + 2 * e + 1]);
      pt[ks] = __builtin_bit_cast(bf16x8, w);
    }
  };
  // O^T += V^T P^T; per key step the four dim tiles' fragments are read
  // together and feed independent accumulators
  auto o_tile = [&](const lds_u8* vb, const bf16x8 (&pt)[4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 va[kD / 32];
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) {
        const lds_u8* src = vb + v_off[dt] + ks * 4096;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)src);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(src + 2048));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        va[dt] = __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
      }
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) o[dt] = mfma(va[dt], pt[ks], o[dt]);
    }
  };

  // ---- one pass: a software pipeline over rows [0, n_rows) of a range whose
  // first K and V rows are at kp and vp, `stride` elements apart.  Step t forms
  // the probabilities P(t) of tile t while the MFMAs of S(t + 1) and of
  // O += V(t - 1) P(t - 1) run: the three are independent, so every step holds
  // 32 MFMAs beside the whole softmax.  Tile t + 2's K and tile t's V are in
  // flight.  A rescale decided in step t (by the maximum of tile t + 1)
  // multiplies l at once and O in step t + 1, after tile t's product is added,
  // so O and l see the operations, and the order, of a loop that adds each
  // tile's product in its own step.  Buffers alternate with the parity of t
  // (Kb[(t + 1) & 1] holds K(t + 1), Vb[t & 1] holds V(t), P(t) is p0 or p1);
  // the first step (no product yet) is peeled and the loop is unrolled twice so
  // that every buffer and array is named statically. ----
  f32x16 sa[2], sb[2];
  bf16x8 p0[4], p1[4];
  int q_state = -1;                            // query fragments held: -1 none, 0 plain, 1 lagged
  bool pend = false;                           // O owes a rescale (wave-uniform)
  float pend_corr = 1.0f;
  auto update_m_late = [&](float mt) {         // update_m with O's factor deferred
    if (__builtin_amdgcn_ballot_w64(mt > m + 8.0f)) {
      const float mn = fmaxf(m, mt);
      const float corr = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      l *= corr;
      pend = true;
      pend_corr = corr;
    }
  };
  auto apply_pend = [&]() {
    if (pend) {
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= pend_corr;
      pend = false;
    }
  };
  // (planar: K is a ragged run of split keys, kp its temporal piece and kp2 its
  // other-dims piece at the pass's first row; otherwise kp2 is unused)
  auto run_pass = [&](const uint16_t* kp, const uint16_t* kp2, const uint16_t* vp,
                      int64_t stride, int64_t n_rows, int q_want, bool planar) {
    const int64_t n_tiles = (n_rows + kBN - 1) / kBN;
    if (n_tiles <= 0) return;
    const uint32_t st2 = (uint32_t)stride * 2u;
    const int64_t tile_elems = (int64_t)kBN * stride;
    auto tk = [&](int64_t t) { return kp + t * (planar ? kBN * kte : tile_elems); };
    auto tk2 = [&](int64_t t) { return kp2 + t * (planar ? kBN * kse : tile_elems); };
    auto tv = [&](int64_t t) { return vp + t * tile_elems; };
    auto step = [&](auto with_o, int64_t t, f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
                    const lds_u8* k_next, lds_u8* k_free, const lds_u8* v_prev, lds_u8* v_free,
                    const bf16x8 (&p_prev)[4], bf16x8 (&p_cur)[4]) {
      __builtin_amdgcn_s_waitcnt(0);           // this wavefront's K(t + 1), V(t - 1) have landed
      lds_barrier();                           // ... everyone's; K(t), V(t - 2) are free
      if (t + 2 < n_tiles)
        load_tile(tk(t + 2), tk2(t + 2), tv(t + 2), st2, n_rows - (t + 2) * kBN, k_free, v_free,
                  true, false, planar);
      load_tile(tk(t), tk2(t), tv(t), st2, n_rows - t * kBN, k_free, v_free, false, true, planar);
      s_tile(k_next, s_nxt);     // past the last tile: stale LDS, result unused (keeps
                                 // the MFMAs in the same block as the softmax work)
      if constexpr (decltype(with_o)::value) o_tile(v_prev, p_prev);
      s_exp(s_cur, p_cur);
      float mt = tile_max(s_nxt);  // S(t + 1) as computed; corrected below for a last,
                                   // partial tile
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      step_schedule<32, RAGGED>();
      apply_pend();
      if (t + 1 < n_tiles) {
        const int64_t lim = n_rows - (t + 1) * kBN;
        if (lim < kBN) {
          s_mask(s_nxt, lim);
          mt = tile_max(s_nxt);
        }
        update_m_late(mt);
      }
    };
    if (q_state != q_want) {
      load_q(LAG && q_want == 1);
      q_state = q_want;
    }
    load_tile(tk(0), tk2(0), tv(0), st2, n_rows, kb0, vb0, true, false, planar);
    if (n_tiles > 1)
      load_tile(tk(1), tk2(1), tv(1), st2, n_rows - kBN, kb1, vb1, true, false, planar);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    s_tile(kb0, sa);
    s_max(sa, n_rows);
    using no_o = std::integral_constant<bool, false>;
    using with_o = std::integral_constant<bool, true>;
    step(no_o{}, 0, sa, sb, kb1, kb0, vb1, vb0, p1, p0);
    for (int64_t t = 1; t < n_tiles; t += 2) {
      step(with_o{}, t, sb, sa, kb0, kb1, vb0, vb1, p0, p1);
      if (t + 1 < n_tiles) step(with_o{}, t + 1, sa, sb, kb1, kb0, vb1, vb0, p1, p0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();                             // V(n - 1) has landed everywhere
    if ((n_tiles - 1) & 1) o_tile(vb1, p1);    // the last tile's product
    else o_tile(vb0, p0);
    apply_pend();
    lds_barrier();                             // the next pass reuses the buffers
  };
  if (RAGGED) {
    // K of the run: interleaved, head rows kD apart; split, n0 temporal blocks
    // (kte elements each) then n0 other-dims pieces (kse each)
    const uint16_t* kr = a.k0 + base0;
    const uint16_t* kr2 = kr + n0 * kte;
    const int64_t krs = SPLIT ? kte : stride0;
    if (LAG) {                                 // run: lagged rows, then the plain tail
      const int64_t tail = min(max(a.plain_tail, (int64_t)0), n0);
      run_pass(kr, kr2, a.v0 + base0, stride0, n0 - tail, 1, SPLIT);
      run_pass(kr + (n0 - tail) * krs, kr2 + (n0 - tail) * kse,
               a.v0 + base0 + (n0 - tail) * stride0, stride0, tail, 0, SPLIT);
    } else {
      run_pass(kr, kr2, a.v0 + base0, stride0, n0, 0, SPLIT);
    }
    // the chunk block is dense token rows (split keys: the head's pieces are
    // found by the lanes' row offsets from the token row)
    if (a.k1)
      run_pass(a.k1 + (SPLIT ? 0 : (int64_t)head * kD), a.k1, a.v1 + (int64_t)head * kD, a.row,
               a.n1, 0, false);
  } else if (LAG) {
    run_pass(a.k0 + kbase0, a.k0, a.v0 + base0, a.row, pa, 1, false);          // lagged, before
    run_pass(a.k0 + kbase0 + pb * a.row, a.k0, a.v0 + base0 + pb * a.row, a.row, n0 - pb, 1,
             false);                                                          // lagged, after
    run_pass(a.k0 + kbase0 + pa * a.row, a.k0, a.v0 + base0 + pa * a.row, a.row, pb - pa, 0,
             false);                                                          // plain
  } else {
    run_pass(a.k0 + kbase0, a.k0, a.v0 + base0, stride0, n0, 0, false);
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

// Split keys: the head row's temporal 16-byte chunks [tvb, tvb + tvc) (bf16,
// head_dim 128; pair_begin and n_pairs multiples of 4, checked by the caller).
void set_split(AttnArgs& a, int32_t key_layout, int32_t pair_begin, int32_t n_pairs) {
  a.tvb = key_layout == DP_KEY_SPLIT ? pair_begin / 4 : 0;
  a.tvc = key_layout == DP_KEY_SPLIT ? n_pairs / 4 : 0;
}

dp_status launch(AttnArgs& a, const void* q, void* o, int64_t n_q, int32_t n_heads, float scale,
                 hipStream_t s) {
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.o = reinterpret_cast<uint16_t*>(o);
  a.n_q = n_q;
  a.row = (int64_t)n_heads * kD;
  a.n_heads = n_heads;
  const int mode = a.off ? (a.theta ? kRaggedLag : kRagged) : (a.theta ? kLag : kDense);
  const int bm = mode == kLag ? Shape<kLag>::kBM : mode == kRagged ? Shape<kRagged>::kBM
               : mode == kRaggedLag ? Shape<kRaggedLag>::kBM : Shape<kDense>::kBM;
  a.n_qt = (int32_t)((n_q + bm - 1) / bm);
  a.xcd_map = n_heads % kXcds == 0;
  a.c = scale * 1.4426950408889634f;
  // ragged caches on the XCD map: 2H halves of ceil(tiles / 2) slots each
  const bool halves = (mode == kRagged || mode == kRaggedLag) && a.xcd_map &&
                      n_heads <= Shape<kRagged>::kBlock;
  const uint64_t blocks = halves ? (uint64_t)2 * n_heads * ((a.n_qt + 1) / 2)
                                 : (uint64_t)a.n_qt * n_heads;
  if (blocks == 0) return DP_OK;
  const dim3 grid((uint32_t)blocks);
  if (a.tvc > 0) {
    if (mode == kLag)
      hipLaunchKernelGGL(attn_fwd_kernel<kLag | kSplit>, grid, dim3(Shape<kLag>::kBlock), 0, s, a);
    else if (mode == kRagged)
      hipLaunchKernelGGL(attn_fwd_kernel<kRagged | kSplit>, grid, dim3(Shape<kRagged>::kBlock), 0,
                         s, a);
    else if (mode == kRaggedLag)
      hipLaunchKernelGGL(attn_fwd_kernel<kRaggedLag | kSplit>, grid,
                         dim3(Shape<kRaggedLag>::kBlock), 0, s, a);
    else
      hipLaunchKernelGGL(attn_fwd_kernel<kDense | kSplit>, grid, dim3(Shape<kDense>::kBlock), 0, s,
                         a);
  } else {
    if (mode == kLag)
      hipLaunchKernelGGL(attn_fwd_kernel<kLag>, grid, dim3(Shape<kLag>::kBlock), 0, s, a);
    else if (mode == kRagged)
      hipLaunchKernelGGL(attn_fwd_kernel<kRagged>, grid, dim3(Shape<kRagged>::kBlock), 0, s, a);
    else if (mode == kRaggedLag)
      hipLaunchKernelGGL(attn_fwd_kernel<kRaggedLag>, grid, dim3(Shape<kRaggedLag>::kBlock), 0, s,
                         a);
    else
      hipLaunchKernelGGL(attn_fwd_kernel<kDense>, grid, dim3(Shape<kDense>::kBlock), 0, s, a);
  }
  return check_launch("attn_fwd_kernel");
}

}  // namespace

dp_status launch_attention(const void* q, const void* k, const void* v, void* o, int64_t n_q,
                           int64_t kv_cap, const int64_t* n_kv, int32_t n_heads, float scale,
                           int32_t key_layout, int32_t pair_begin, int32_t n_pairs,
                           hipStream_t s) {
  AttnArgs a{};
  set_split(a, key_layout, pair_begin, n_pairs);
  a.k0 = reinterpret_cast<const uint16_t*>(k);
  a.v0 = reinterpret_cast<const uint16_t*>(v);
  a.n_kv = n_kv;
  a.cap0 = kv_cap;
  return launch(a, q, o, n_q, n_heads, scale, s);
}

dp_status launch_attention_lag(const void* q, const void* k, const void* v, void* o,
                               int64_t n_q, int64_t kv_cap, const int64_t* n_kv,
                               int64_t plain_begin, int64_t plain_end, const float* theta,
                               int32_t pair_begin, int32_t n_pairs, float lag, int32_t n_heads,
                               float scale, int32_t key_layout, hipStream_t s) {
  AttnArgs a{};
  set_split(a, key_layout, pair_begin, n_pairs);
  a.k0 = reinterpret_cast<const uint16_t*>(k);
  a.v0 = reinterpret_cast<const uint16_t*>(v);
  a.n_kv = n_kv;
  a.cap0 = kv_cap;
  a.plain_begin = plain_begin;
  a.plain_end = plain_end;
  a.theta = theta;
  a.pair_begin = pair_begin;
  a.n_pairs = n_pairs;
  a.lag = lag;
  return launch(a, q, o, n_q, n_heads, scale, s);
}

dp_status launch_hs_attention(const void* q, const void* k_ragged, const void* v_ragged,
                              int64_t ragged_capacity, const int64_t* head_offsets,
                              const void* k_chunk, const void* v_chunk, int64_t n_chunk, void* o,
                              int64_t n_q, int32_t n_heads, float scale, int32_t key_layout,
                              int32_t pair_begin, int32_t n_pairs, hipStream_t s,
                              const HsLag* lag) {
  AttnArgs a{};
  set_split(a, key_layout, pair_begin, n_pairs);
  if (lag) {
    a.plain_tail = lag->plain_tail;
    a.theta = lag->theta;
    a.pair_begin = lag->pair_begin;
    a.n_pairs = lag->n_pairs;
    a.lag = lag->lag;
  }
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
