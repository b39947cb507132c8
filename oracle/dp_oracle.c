/*
 * dp_oracle.c — plain, slow CPU oracle of the DeCoPrune history-KV compaction
 * path.  TEST INFRASTRUCTURE ONLY: it exists so that tests, the smoke check and
 * the benchmark's CPU-baseline leg can compare the HIP library against an
 * obviously correct evaluation.  No product code may call it, and it shares no
 * code, header or table with the HIP library.
 *
 * Source of the method: the web page
 *   "DeCoPrune이 디노이징 불일치로 비디오 KV 캐시를 85% 줄인다"
 *   (onedev.kr/papers/726), "the DeCoPrune page", sections
 *   어떻게 동작하나 (how it works), 무엇과 다른가 (how it differs),
 *   어떻게 쓰나 (how to use it).
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC.
 * Floating point: fp32 steps are written as separate C float operations, so
 * with -ffp-contract=off every product and sum is rounded on its own (SSE2
 * single precision on x86-64, IEEE round-to-nearest-even).
 *
 * Readings of points the page leaves open (each is listed in the design notes):
 *  - score precision and order: fp32, pairwise tree over channels padded with
 *    +0 to a power of two, division by d in fp64 then rounded to fp32;
 *  - tie: keep iff l >= gamma; NaN is dropped (reversed mode keeps it);
 *  - positions are latent-frame indices; g is continuous piecewise-linear
 *    with a knee; keys carry a per-frame phase p and are rotated by t~ - p;
 *  - temporal pairs are adjacent dims (2j, 2j+1) of a contiguous block.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float bf16_to_f32(uint16_t h);

#define ORACLE_ABI 1
int oracle_abi(void) { return ORACLE_ABI; }

/* ---------------------------------------------------------------------- *
 * Discrepancy score [DeCoPrune page, 어떻게 동작하나]: for each token the
 * mean over the d latent channels of the squared difference between the
 * clean prediction at the probe step and the final output.
 * ---------------------------------------------------------------------- */

/* fp32 evaluation in the fixed pairwise order (the order is a reading: the
 * page gives only the formula).  x0, xf: [n][stride] floats, channels [0,d). */
void oracle_score_f32(const float* x0, const float* xf, int64_t n, int32_t d,
                      int64_t stride, float* ell) {
  int32_t P = 1;
  while (P < d) P *= 2;
  float q[1024];
  for (int64_t i = 0; i < n; ++i) {
    const float* a = x0 + i * stride;
    const float* b = xf + i * stride;
    for (int32_t c = 0; c < P; ++c) {
      if (c < d) {
        float e = a[c] - b[c];
        q[c] = e * e;
      } else {
        q[c] = 0.0f;
      }
    }
    for (int32_t h = P / 2; h >= 1; h /= 2)
      for (int32_t c = 0; c < h; ++c) q[c] = q[c] + q[c + h];
    ell[i] = (float)((double)q[0] / (double)d);
  }
}

/* fp64 evaluation, plain left-to-right sum; used to check the fp32 one and to
 * count tokens whose mask bit depends on rounding. */
void oracle_score_f64(const float* x0, const float* xf, int64_t n, int32_t d,
                      int64_t stride, double* ell) {
  for (int64_t i = 0; i < n; ++i) {
    double s = 0.0;
    for (int32_t c = 0; c < d; ++c) {
      double e = (double)x0[i * stride + c] - (double)xf[i * stride + c];
      s += e * e;
    }
    ell[i] = s / (double)d;
  }
}

/* ---------------------------------------------------------------------- *
 * Mask [DeCoPrune page, 어떻게 동작하나]: threshold gamma, keep the tokens
 * with large discrepancy; the sink chunk and the last w chunks are always
 * kept; one mask serves every layer.  reversed = the ablation that keeps the
 * small-discrepancy tokens [DeCoPrune page, 전제와 한계].  streaming = keep
 * only sink + window (Streaming policy of the HS static heads).
 * ell[i] is the score of row scored_begin + i.
 * ---------------------------------------------------------------------- */
void oracle_mask(const float* ell, int64_t T, int64_t sink_len, int64_t window_len,
                 int64_t scored_begin, int64_t n_scored, float gamma, int32_t reversed,
                 int32_t streaming, uint8_t* keep) {
  for (int64_t t = 0; t < T; ++t) {
    uint8_t k;
    if (t < sink_len || t >= T - window_len) {
      k = 1;
    } else if (t >= scored_begin && t < scored_begin + n_scored) {
      if (streaming) {
        k = 0;
      } else {
        int big = ell[t - scored_begin] >= gamma;
        k = (uint8_t)(reversed ? !big : big);
      }
    } else {
      k = streaming ? 0 : 1;
    }
    keep[t] = k;
  }
}

/* ---------------------------------------------------------------------- *
 * Kept-index list: the ascending positions m with keep = 1, so K[m], V[m]
 * keeps token order.  Returns the count.
 * ---------------------------------------------------------------------- */
int64_t oracle_compact(const uint8_t* keep, int64_t T, int32_t* idx) {
  int64_t n = 0;
  for (int64_t t = 0; t < T; ++t)
    if (keep[t]) idx[n++] = (int32_t)t;
  return n;
}

/* ---------------------------------------------------------------------- *
 * Physical gather [DeCoPrune page, 어떻게 동작하나]: each layer keeps only the
 * selected rows, copied bit for bit into a shorter dense cache.
 * src: n_layers slabs of src_rows rows of row_bytes; dst: n_layers slabs of
 * dst_rows rows.
 * ---------------------------------------------------------------------- */
void oracle_gather(const uint8_t* src, int64_t n_layers, int64_t src_rows,
                   int64_t row_bytes, const int32_t* idx, int64_t n, uint8_t* dst,
                   int64_t dst_rows) {
#pragma omp parallel for schedule(static)
  for (int64_t l = 0; l < n_layers; ++l)
    for (int64_t j = 0; j < n; ++j)
      memcpy(dst + (l * dst_rows + j) * row_bytes,
             src + (l * src_rows + (int64_t)idx[j]) * row_bytes, (size_t)row_bytes);
}

void oracle_gather_i32(const int32_t* src, const int32_t* idx, int64_t n, int32_t* dst) {
  for (int64_t j = 0; j < n; ++j) dst[j] = src[idx[j]];
}

/* ---------------------------------------------------------------------- *
 * Segment-append compaction in place [DeCoPrune page, 어떻게 동작하나]: when a
 * chunk leaves the window, only its kept rows change place: they are copied
 * from the chunk's slot to the history tail of the same buffer (every layer),
 * their frames with them; the slot's frames become -1 (retired).  buf holds
 * n_layers slabs of capacity rows of row_bytes.  Returns the new tail, or -1
 * (nothing changed) if the rows would pass the capacity or overlap the slot.
 * ---------------------------------------------------------------------- */
int64_t oracle_append_kept(uint8_t* buf, int64_t n_layers, int64_t capacity, int64_t row_bytes,
                           int64_t slot_begin, int64_t slot_rows, const int32_t* idx, int64_t n,
                           int64_t tail, int32_t* row_frame) {
  if (tail < 0 || tail + n > capacity) return -1;
  if (n > 0 && tail < slot_begin + slot_rows && tail + n > slot_begin) return -1;
  for (int64_t l = 0; l < n_layers; ++l)
    for (int64_t j = 0; j < n; ++j)
      memcpy(buf + (l * capacity + tail + j) * row_bytes,
             buf + (l * capacity + slot_begin + (int64_t)idx[j]) * row_bytes, (size_t)row_bytes);
  if (row_frame) {
    for (int64_t j = 0; j < n; ++j) row_frame[tail + j] = row_frame[slot_begin + idx[j]];
    for (int64_t r = 0; r < slot_rows; ++r) row_frame[slot_begin + r] = -1;
  }
  return tail + n;
}

/* ---------------------------------------------------------------------- *
 * RoPE temporal re-index [DeCoPrune page, 무엇과 다른가]: old keys move to
 * t~ = q0 - g(q0 - t), g keeps recent offsets and compresses older ones
 * linearly; only the key's temporal phase changes.
 *
 * oracle_rope_frames: per frame f
 *   D = q0 - t_f;  gD = D if D <= knee else knee + (D - knee) * inv_factor;
 *   t~ = q0 - gD;  delta_f = t~ - p_f;  p_f <- t~;
 *   per pair j: angle = theta_j * delta_f (fp32);
 *               cos_fj, sin_fj = fp32 roundings of the fp64 cos, sin.
 * ---------------------------------------------------------------------- */
void oracle_rope_frames(int32_t n_frames, const float* frame_t, float* frame_phase,
                        float q0, float knee, float inv_factor, int32_t n_pairs,
                        const float* theta, float* delta, float* cos_tab, float* sin_tab) {
  for (int32_t f = 0; f < n_frames; ++f) {
    float D = q0 - frame_t[f];
    float gD;
    if (D <= knee) {
      gD = D;
    } else {
      float over = D - knee;
      float squeezed = over * inv_factor;
      gD = knee + squeezed;
    }
    float t_new = q0 - gD;
    float dl = t_new - frame_phase[f];
    delta[f] = dl;
    frame_phase[f] = t_new;
    for (int32_t j = 0; j < n_pairs; ++j) {
      float angle = theta[j] * dl;
      cos_tab[(int64_t)f * n_pairs + j] = (float)cos((double)angle);
      sin_tab[(int64_t)f * n_pairs + j] = (float)sin((double)angle);
    }
  }
}

/* ---------------------------------------------------------------------- *
 * Compressed time axis (a re-parametrisation of the re-index above, not a
 * step the page names): past the knee t~ = q0 - knee - (q0 - t - knee)/c
 * = t/c + (1 - 1/c)(q0 - knee), and the second term is the same for every
 * such key, so a key may carry the phase t/c and leave the common term to
 * the query.  oracle_rope_frames_compressed: per frame f
 *   D = q0 - t_f;  t' = t_f * inv_factor if D > knee, else q0 - D (as above);
 *   delta_f = t' - p_f;  p_f <- t';  cos/sin tables as oracle_rope_frames.
 * ---------------------------------------------------------------------- */
void oracle_rope_frames_compressed(int32_t n_frames, const float* frame_t, float* frame_phase,
                                   float q0, float knee, float inv_factor, int32_t n_pairs,
                                   const float* theta, float* delta, float* cos_tab,
                                   float* sin_tab) {
  for (int32_t f = 0; f < n_frames; ++f) {
    float D = q0 - frame_t[f];
    float t_new = D > knee ? frame_t[f] * inv_factor : q0 - D;
    float dl = t_new - frame_phase[f];
    delta[f] = dl;
    frame_phase[f] = t_new;
    for (int32_t j = 0; j < n_pairs; ++j) {
      float angle = theta[j] * dl;
      cos_tab[(int64_t)f * n_pairs + j] = (float)cos((double)angle);
      sin_tab[(int64_t)f * n_pairs + j] = (float)sin((double)angle);
    }
  }
}

/* ---------------------------------------------------------------------- *
 * Uniform phase step [DeCoPrune page, 무엇과 다른가]: once a frame is past the
 * knee before and after a step, t~ moves by the same amount for every such
 * frame (q0 advances F frames: F (1 - 1/c)), so the keys of all of them are
 * rotated by one table: per pair j, angle = theta_j * delta (fp32), cos and
 * sin the fp32 roundings of the fp64 values (as oracle_rope_frames).
 * ---------------------------------------------------------------------- */
void oracle_rope_uniform(int32_t n_pairs, const float* theta, float delta, float* cos_tab,
                         float* sin_tab) {
  for (int32_t j = 0; j < n_pairs; ++j) {
    float angle = theta[j] * delta;
    cos_tab[j] = (float)cos((double)angle);
    sin_tab[j] = (float)sin((double)angle);
  }
}

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round to nearest, ties to even, keeping NaN a (quiet) NaN. */
static uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t hi = u >> 16, lo = u & 0xFFFFu;
  if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u))) hi += 1u;
  return (uint16_t)hi;
}

/* Rotate the temporal pairs of one (row, head) vector of head_dim elements. */
static void rotate_head(void* head, int32_t dtype, int32_t pair_begin, int32_t n_pairs,
                        const float* c, const float* s) {
  for (int32_t j = 0; j < n_pairs; ++j) {
    int32_t e0 = 2 * (pair_begin + j), e1 = e0 + 1;
    float a, b;
    if (dtype == 0) {
      a = ((float*)head)[e0];
      b = ((float*)head)[e1];
    } else {
      a = bf16_to_f32(((uint16_t*)head)[e0]);
      b = bf16_to_f32(((uint16_t*)head)[e1]);
    }
    float ac = a * c[j], bs = b * s[j], as = a * s[j], bc = b * c[j];
    float a2 = ac - bs;
    float b2 = as + bc;
    if (dtype == 0) {
      ((float*)head)[e0] = a2;
      ((float*)head)[e1] = b2;
    } else {
      ((uint16_t*)head)[e0] = f32_to_bf16(a2);
      ((uint16_t*)head)[e1] = f32_to_bf16(b2);
    }
  }
}

/* Re-index rows [0, n_rows) of a token-major [rows][n_heads][head_dim] cache
 * in place; dtype 0 = fp32, 1 = bf16.  Rows of frames with delta 0 are left
 * untouched. */
void oracle_rope_rows(void* k, int32_t dtype, int64_t n_rows, int32_t n_heads,
                      int32_t head_dim, int32_t pair_begin, int32_t n_pairs,
                      const int32_t* row_frame, const float* delta, const float* cos_tab,
                      const float* sin_tab) {
  int64_t esz = dtype == 0 ? 4 : 2;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    int32_t f = row_frame[r];
    if (delta[f] == 0.0f) continue;
    for (int32_t h = 0; h < n_heads; ++h) {
      uint8_t* head = (uint8_t*)k + ((r * n_heads + h) * (int64_t)head_dim) * esz;
      rotate_head(head, dtype, pair_begin, n_pairs, cos_tab + (int64_t)f * n_pairs,
                  sin_tab + (int64_t)f * n_pairs);
    }
  }
}

/* Same for a per-head packed cache: n_rows head rows of head_dim elements,
 * row_frame per head row. */
void oracle_rope_headrows(void* k, int32_t dtype, int64_t n_rows, int32_t head_dim,
                          int32_t pair_begin, int32_t n_pairs, const int32_t* row_frame,
                          const float* delta, const float* cos_tab, const float* sin_tab) {
  int64_t esz = dtype == 0 ? 4 : 2;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    int32_t f = row_frame[r];
    if (delta[f] == 0.0f) continue;
    rotate_head((uint8_t*)k + r * (int64_t)head_dim * esz, dtype, pair_begin, n_pairs,
                cos_tab + (int64_t)f * n_pairs, sin_tab + (int64_t)f * n_pairs);
  }
}

/* ---------------------------------------------------------------------- *
 * DeCoPrune-HS [DeCoPrune page, 무엇과 다른가]: per (layer, head) a class;
 * the head keeps the rows of its class's index list; output packed per head
 * in (layer, head) row-major order.
 * offsets: [n_layers*n_heads + 1] exclusive scan of the per-head lengths.
 * ---------------------------------------------------------------------- */
void oracle_hs_offsets(const uint8_t* head_class, int32_t n_layers, int32_t n_heads,
                       const int64_t* class_len, int64_t* offsets) {
  offsets[0] = 0;
  for (int64_t i = 0; i < (int64_t)n_layers * n_heads; ++i)
    offsets[i + 1] = offsets[i] + class_len[head_class[i]];
}

/* One layer: src [src_rows][n_heads][head_dim] elements of esz bytes; class
 * lists concatenated in class_idx_cat with class_base[c] as the start of list
 * c; out receives the layer's heads at out + offsets[l*H+h] head rows. */
void oracle_hs_gather_layer(const uint8_t* src, int32_t layer, int32_t n_heads,
                            int32_t head_dim, int32_t esz, const uint8_t* head_class,
                            const int32_t* class_idx_cat, const int64_t* class_base,
                            const int64_t* class_len, const int64_t* offsets, uint8_t* out) {
  int64_t hb = (int64_t)head_dim * esz;
#pragma omp parallel for schedule(static)
  for (int32_t h = 0; h < n_heads; ++h) {
    int64_t i = (int64_t)layer * n_heads + h;
    int32_t c = head_class[i];
    const int32_t* list = class_idx_cat + class_base[c];
    for (int64_t j = 0; j < class_len[c]; ++j)
      memcpy(out + (offsets[i] + j) * hb, src + ((int64_t)list[j] * n_heads + h) * hb,
             (size_t)hb);
  }
}

/* ---------------------------------------------------------------------- *
 * Attention of a chunk over the retained cache [DeCoPrune page, 무엇인가:
 * each chunk attends to the KV cache of the history; 전제와 한계: the
 * continuation speed-up comes from the shorter cache].  For the queries
 * listed in rows (n_rows of them) and every head h:
 *   O[i][h][:] = sum_j softmax_j(scale * <Q[i][h], K[j][h]>) V[j][h][:],  j < n_kv,
 * evaluated in float64 from bf16 inputs; out is [n_rows][H][D] float64.
 * Q, K, V: token-major [rows][H][D] bf16 bit patterns.
 * ---------------------------------------------------------------------- */
void oracle_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int64_t* rows, int64_t n_rows, int64_t n_kv, int32_t H, int32_t D,
                      double scale, double* out) {
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < n_rows * H; ++r) {
    const int64_t qi = rows[r / H];
    const int32_t h = (int32_t)(r % H);
    const uint16_t* qv = q + (qi * H + h) * (int64_t)D;
    double m = -INFINITY;
    double* o = out + r * (int64_t)D;
    for (int32_t c = 0; c < D; ++c) o[c] = 0.0;
    double l = 0.0;
    for (int64_t j = 0; j < n_kv; ++j) {          /* running max and sum, float64 */
      const uint16_t* kv = k + (j * H + h) * (int64_t)D;
      double s = 0.0;
      for (int32_t c = 0; c < D; ++c) s += (double)bf16_to_f32(qv[c]) * (double)bf16_to_f32(kv[c]);
      s *= scale;
      const uint16_t* vv = v + (j * H + h) * (int64_t)D;
      if (s > m) {
        double corr = exp(m - s);
        l *= corr;
        for (int32_t c = 0; c < D; ++c) o[c] *= corr;
        m = s;
      }
      double p = exp(s - m);
      l += p;
      for (int32_t c = 0; c < D; ++c) o[c] += p * (double)bf16_to_f32(vv[c]);
    }
    for (int32_t c = 0; c < D; ++c) o[c] /= l;
  }
}

/* Same attention over float64 inputs (q, k, v: [rows][H][D] doubles), for
 * references that must not round the re-indexed keys to a storage type. */
void oracle_attention_f64(const double* q, const double* k, const double* v,
                          const int64_t* rows, int64_t n_rows, int64_t n_kv, int32_t H,
                          int32_t D, double scale, double* out) {
#pragma omp parallel for schedule(dynamic)
  for (int64_t r = 0; r < n_rows * H; ++r) {
    const int64_t qi = rows[r / H];
    const int32_t h = (int32_t)(r % H);
    const double* qv = q + (qi * H + h) * (int64_t)D;
    double m = -INFINITY;
    double* o = out + r * (int64_t)D;
    for (int32_t c = 0; c < D; ++c) o[c] = 0.0;
    double l = 0.0;
    for (int64_t j = 0; j < n_kv; ++j) {
      const double* kv = k + (j * H + h) * (int64_t)D;
      double s = 0.0;
      for (int32_t c = 0; c < D; ++c) s += qv[c] * kv[c];
      s *= scale;
      const double* vv = v + (j * H + h) * (int64_t)D;
      if (s > m) {
        double corr = exp(m - s);
        l *= corr;
        for (int32_t c = 0; c < D; ++c) o[c] *= corr;
        m = s;
      }
      double p = exp(s - m);
      l += p;
      for (int32_t c = 0; c < D; ++c) o[c] += p * vv[c];
    }
    for (int32_t c = 0; c < D; ++c) o[c] /= l;
  }
}

/* Exact re-index in float64 [DeCoPrune page, 무엇과 다른가]: pair j of every
 * head of row r rotated by theta_j * step[row_frame[r]], with no rounding to a
 * storage type (reference for paths that rotate keys and queries differently). */
void oracle_rope_rows_f64(double* k, int64_t n_rows, int32_t n_heads, int32_t head_dim,
                          int32_t pair_begin, int32_t n_pairs, const int32_t* row_frame,
                          const double* step, const double* theta) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n_rows; ++r) {
    const double d = step[row_frame[r]];
    if (d == 0.0) continue;
    for (int32_t h = 0; h < n_heads; ++h) {
      double* x = k + (r * n_heads + h) * (int64_t)head_dim;
      for (int32_t j = 0; j < n_pairs; ++j) {
        const double c = cos(theta[j] * d), sn = sin(theta[j] * d);
        const double a = x[2 * (pair_begin + j)], b = x[2 * (pair_begin + j) + 1];
        x[2 * (pair_begin + j)] = a * c - b * sn;
        x[2 * (pair_begin + j) + 1] = a * sn + b * c;
      }
    }
  }
}

/* ---------------------------------------------------------------------- *
 * Pruning ratio [DeCoPrune page, 어떻게 쓰나]: 1 - visible / FullKV positions.
 * ---------------------------------------------------------------------- */
double oracle_pr(int64_t visible, int64_t full) {
  return full == 0 ? 0.0 : 1.0 - (double)visible / (double)full;
}
