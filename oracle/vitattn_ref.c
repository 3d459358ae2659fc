/*
 * vitattn_ref.c -- the float64 CPU oracle for bidirectional multi-head
 * scaled-dot-product attention over packed variable-length sequences.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker that the GPU path is
 * compared against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load it; the product library never links, loads or calls it,
 * and it shares no code, header, table or constant with the GPU path.
 *
 * What it computes (the plain definition, not the GPU algorithm):
 *   For every sequence s with rows [a, b) = [cu[s], cu[s+1]), every head h and
 *   every query row i in [a, b):
 *     l_j   = scale * sum_{d<D} Q[i,h,d] * K[j,h,d]          for j in [a, b)
 *     m     = max_j l_j
 *     w_j   = exp(l_j - m)
 *     Z     = sum_j w_j
 *     O[i,h,e] = (sum_j w_j * V[j,h,e]) / Z                  for e < D
 *   Keys never cross a sequence boundary (block-diagonal attention) and there
 *   is no other mask (the attention is bidirectional).
 *
 * Sources (pages as titled in the reference collection):
 *  - "inferencelayer 0.2.1 src/vision_gpu.rs", doc of vis_attn_coop_src,
 *    section "The obstacle, and the way round it": the online update
 *    O <- O*e^(m_old - m_new) + P*V, whose fixed point is the softmax-weighted
 *    average written above; and the closing division of the running output by
 *    the running row sum.
 *  - same page, VisionGpu::forward_one, the segment tables: one image is one
 *    ragged segment and tokens attend within their image, never across it;
 *    several images are several segments (here: the cu_seqlens prefix array).
 *  - "hf2q src/inference/vision/vit_gpu.rs", doc of vit_attention_gpu: full
 *    scaled-dot-product attention with no mask because the ViT is
 *    bidirectional; tensors are seq-major [tokens, heads, head_dim]; and doc of
 *    vit_attention_scores_gpu: the scale is the caller's value (1/sqrt(hd) for
 *    a standard ViT, 1.0 for Gemma 4V), with no implicit scaling.
 *
 * Masks (the *_masked_* entry points; causal = 0 and window = 0 is the
 * definition above).  Within a sequence of length L, query position qi = i - a
 * and key position kj = j - a, key j takes part in row i only if
 *   - causal: kj <= qi + (Lk - Lq), the aligned causal rule of "hanzo-ml
 *     0.11.4 src/vulkan_backend.rs", doc of flash_attn_gpu; here Lk = Lq = L
 *     (self-attention inside one image), so kj <= qi;
 *   - window > 0: |qi - kj| < window.  The pages name the window parameter of
 *     the encoder attention ("inferencelayer 0.2.1 src/vision_gpu.rs",
 *     VisionGpu::forward_one, the attention meta: window 0 means unrestricted)
 *     without defining it; the reading taken here is a symmetric band of
 *     half-width window - 1, which with causal = 1 is the last `window` keys up
 *     to and including the query itself.
 * Every row keeps at least itself (kj = qi passes both rules), so Z > 0.
 *
 * Readings taken where the pages are silent: the max is subtracted before the
 * exponential (a two-pass softmax; mathematically the same result); the scale
 * multiplies the dot product before the max; inputs arrive as float32 values
 * (exact for float32 and for bfloat16 data) and every operation is float64 with
 * libm exp; a zero-length sequence has no rows and writes nothing.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC vitattn_ref.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Whether key j takes part in query row i of the sequence [a, b) (the mask
 * rules in the header; causal = 0 and window = 0 keep every key). */
static int ref_visible(int64_t a, int64_t b, int64_t i, int64_t j, int32_t causal, int32_t window) {
  const int64_t qi = i - a, kj = j - a;
  const int64_t lq = b - a, lk = b - a; /* self-attention: as many keys as queries */
  if (causal && kj > qi + (lk - lq)) return 0;
  if (window > 0 && (qi - kj >= window || kj - qi >= window)) return 0;
  return 1;
}

/* One query row of one head: writes D outputs to out[0..D).  `w` is caller
 * scratch of at least (b - a) doubles.  K and V have n_kv_heads heads (a
 * divisor of n_heads); query head h reads K/V head h / (n_heads / n_kv_heads),
 * the grouping of "hf2q src/inference/vision/vit_gpu.rs", doc of
 * vit_repeat_kv_gpu (each K/V head serves num_kv_groups consecutive query
 * heads).  n_kv_heads == n_heads is plain multi-head attention.  Keys that the
 * mask rules exclude get weight exactly 0: they enter neither the max nor Z. */
static void ref_one_row(const float* q, const float* k, const float* v,
                        int64_t a, int64_t b, int64_t i, int32_t h,
                        int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, double scale,
                        int32_t causal, int32_t window, double* w, double* out) {
  const int64_t row_stride = (int64_t)n_heads * head_dim;
  const int64_t kv_stride = (int64_t)n_kv_heads * head_dim;
  const int32_t hk = h / (n_heads / n_kv_heads);
  const float* qi = q + i * row_stride + (int64_t)h * head_dim;
  /* pass 1: logits of the visible keys and their maximum */
  double m = -INFINITY;
  for (int64_t j = a; j < b; ++j) {
    if (!ref_visible(a, b, i, j, causal, window)) continue;
    const float* kj = k + j * kv_stride + (int64_t)hk * head_dim;
    double dot = 0.0;
    for (int32_t d = 0; d < head_dim; ++d) dot += (double)qi[d] * (double)kj[d];
    double logit = scale * dot;
    w[j - a] = logit;
    if (logit > m) m = logit;
  }
  /* pass 2: weights, their sum, and the weighted average of V */
  double z = 0.0;
  for (int64_t j = a; j < b; ++j) {
    double wj = ref_visible(a, b, i, j, causal, window) ? exp(w[j - a] - m) : 0.0;
    w[j - a] = wj;
    z += wj;
  }
  for (int32_t e = 0; e < head_dim; ++e) out[e] = 0.0;
  for (int64_t j = a; j < b; ++j) {
    if (w[j - a] == 0.0) continue;
    const float* vj = v + j * kv_stride + (int64_t)hk * head_dim;
    for (int32_t e = 0; e < head_dim; ++e) out[e] += w[j - a] * (double)vj[e];
  }
  for (int32_t e = 0; e < head_dim; ++e) out[e] /= z;
}

/* Number of threads an OpenMP region here will use (1 without OpenMP). */
int vitattn_ref_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of threads later OpenMP regions here use (n >= 1; no effect without OpenMP).
   Only the speed of the oracle changes: every output is computed by one thread in a fixed order. */
void vitattn_ref_set_threads(int n) {
#ifdef _OPENMP
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Full output o[T, H, D] (float64) for q [T, H, D] and k, v [T, Hkv, D]
 * (float32 values), Hkv a divisor of H, under the mask rules (causal 0 or 1,
 * window >= 0).  Returns 0, or -1 on a bad argument or an allocation failure. */
int vitattn_ref_fwd_masked_f64(const float* q, const float* k, const float* v, double* o,
                               const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim, double scale,
                               int32_t causal, int32_t window) {
  if (n_seqs < 0 || n_heads <= 0 || head_dim <= 0) return -1;
  if ((causal != 0 && causal != 1) || window < 0) return -1;
  if (n_kv_heads <= 0 || n_heads % n_kv_heads != 0) return -1;
  if (n_seqs == 0) return 0;
  if (!q || !k || !v || !o || !cu_seqlens) return -1;
  int64_t max_len = 0;
  for (int32_t s = 0; s < n_seqs; ++s) {
    int64_t len = (int64_t)cu_seqlens[s + 1] - cu_seqlens[s];
    if (len < 0) return -1;
    if (len > max_len) max_len = len;
  }
  const int64_t n_pairs = (int64_t)n_seqs * n_heads;
  int failed = 0;
#pragma omp parallel
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    if (!w) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t p = 0; p < n_pairs; ++p) {
        int32_t s = (int32_t)(p / n_heads), h = (int32_t)(p % n_heads);
        int64_t a = cu_seqlens[s], b = cu_seqlens[s + 1];
        for (int64_t i = a; i < b; ++i)
          ref_one_row(q, k, v, a, b, i, h, n_heads, n_kv_heads, head_dim, scale, causal, window, w,
                      o + (i * n_heads + h) * (int64_t)head_dim);
      }
      free(w);
    }
  }
  return failed ? -1 : 0;
}

/* No mask: every key of the sequence. */
int vitattn_ref_fwd_gqa_f64(const float* q, const float* k, const float* v, double* o,
                            const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_heads,
                            int32_t n_kv_heads, int32_t head_dim, double scale) {
  return vitattn_ref_fwd_masked_f64(q, k, v, o, cu_seqlens, n_seqs, n_heads, n_kv_heads, head_dim, scale, 0, 0);
}

/* Multi-head attention (as many K/V heads as query heads). */
int vitattn_ref_fwd_f64(const float* q, const float* k, const float* v, double* o,
                        const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_heads,
                        int32_t head_dim, double scale) {
  return vitattn_ref_fwd_gqa_f64(q, k, v, o, cu_seqlens, n_seqs, n_heads, n_heads, head_dim, scale);
}

/* Output for a chosen set of token rows only: o_rows[n_rows, H, D] (float64),
 * rows[r] a global token index in [0, T).  Used where the full output would
 * take too long, under the mask rules.  Returns 0, or -1 on a bad argument. */
int vitattn_ref_rows_masked_f64(const float* q, const float* k, const float* v, double* o_rows,
                                const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_heads,
                                int32_t n_kv_heads, int32_t head_dim, double scale,
                                int32_t causal, int32_t window, const int64_t* rows, int64_t n_rows) {
  if (n_seqs <= 0 || n_heads <= 0 || head_dim <= 0 || n_rows < 0) return -1;
  if ((causal != 0 && causal != 1) || window < 0) return -1;
  if (n_kv_heads <= 0 || n_heads % n_kv_heads != 0) return -1;
  if (!q || !k || !v || !o_rows || !cu_seqlens || (n_rows > 0 && !rows)) return -1;
  const int64_t total = cu_seqlens[n_seqs];
  int64_t max_len = 0;
  for (int32_t s = 0; s < n_seqs; ++s) {
    int64_t len = (int64_t)cu_seqlens[s + 1] - cu_seqlens[s];
    if (len < 0) return -1;
    if (len > max_len) max_len = len;
  }
  for (int64_t r = 0; r < n_rows; ++r)
    if (rows[r] < 0 || rows[r] >= total) return -1;
  int failed = 0;
#pragma omp parallel
  {
    double* w = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    if (!w) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t p = 0; p < n_rows * n_heads; ++p) {
        int64_t r = p / n_heads;
        int32_t h = (int32_t)(p % n_heads);
        int64_t i = rows[r];
        /* the sequence that holds row i: the last s with cu[s] <= i < cu[s+1] */
        int32_t s = 0;
        while (!(cu_seqlens[s] <= i && i < cu_seqlens[s + 1])) ++s;
        ref_one_row(q, k, v, cu_seqlens[s], cu_seqlens[s + 1], i, h, n_heads, n_kv_heads,
                    head_dim, scale, causal, window, w, o_rows + (r * n_heads + h) * (int64_t)head_dim);
      }
      free(w);
    }
  }
  return failed ? -1 : 0;
}

int vitattn_ref_rows_gqa_f64(const float* q, const float* k, const float* v, double* o_rows,
                             const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_heads,
                             int32_t n_kv_heads, int32_t head_dim, double scale,
                             const int64_t* rows, int64_t n_rows) {
  return vitattn_ref_rows_masked_f64(q, k, v, o_rows, cu_seqlens, n_seqs, n_heads, n_kv_heads, head_dim,
                                     scale, 0, 0, rows, n_rows);
}

int vitattn_ref_rows_f64(const float* q, const float* k, const float* v, double* o_rows,
                         const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_heads,
                         int32_t head_dim, double scale, const int64_t* rows, int64_t n_rows) {
  return vitattn_ref_rows_gqa_f64(q, k, v, o_rows, cu_seqlens, n_seqs, n_heads, n_heads, head_dim,
                                  scale, rows, n_rows);
}

/* The attention weights of one (token row, head): p_out[j - a] for the keys j
 * of the row's sequence [a, b).  Returns b - a, or -1 on a bad argument. */
int64_t vitattn_ref_row_probs_f64(const float* q, const float* k, const int32_t* cu_seqlens,
                                  int32_t n_seqs, int32_t n_heads, int32_t head_dim,
                                  double scale, int64_t row, int32_t head, double* p_out) {
  if (n_seqs <= 0 || n_heads <= 0 || head_dim <= 0 || head < 0 || head >= n_heads) return -1;
  if (row < 0 || row >= cu_seqlens[n_seqs]) return -1;
  int32_t s = 0;
  while (!(cu_seqlens[s] <= row && row < cu_seqlens[s + 1])) ++s;
  const int64_t a = cu_seqlens[s], b = cu_seqlens[s + 1];
  const int64_t row_stride = (int64_t)n_heads * head_dim;
  const float* qi = q + row * row_stride + (int64_t)head * head_dim;
  double m = -INFINITY;
  for (int64_t j = a; j < b; ++j) {
    const float* kj = k + j * row_stride + (int64_t)head * head_dim;
    double dot = 0.0;
    for (int32_t d = 0; d < head_dim; ++d) dot += (double)qi[d] * (double)kj[d];
    p_out[j - a] = scale * dot;
    if (p_out[j - a] > m) m = p_out[j - a];
  }
  double z = 0.0;
  for (int64_t j = a; j < b; ++j) {
    p_out[j - a] = exp(p_out[j - a] - m);
    z += p_out[j - a];
  }
  for (int64_t j = a; j < b; ++j) p_out[j - a] /= z;
  return b - a;
}

/* ------------------------------------------------------------------------
 * The input side of the path: split the packed projection output into Q, K
 * and V, optionally normalise Q and K per head (RMS), and apply the rope.
 *
 * Sources (pages as titled in the reference collection):
 *  - "inferencelayer 0.2.1 src/vision_gpu.rs", VIS_QKV_ROPE and its doc: a
 *    packed row holds the query heads, then the key heads, then the value
 *    heads, each head_dim wide; Q and K are rotated with per-token cos/sin
 *    tables [tokens, head_dim] computed by the caller, V is copied; the
 *    rotation is out[d] = x[d] cos[d] + rotate_half(x)[d] sin[d] with
 *    rotate_half(x)[d] = -x[d + D/2] for d < D/2 and x[d - D/2] otherwise.
 *  - same page, GLM_QKV_QKNORM_ROPE: a per-head RMS norm of Q and of K over
 *    head_dim, before the rope, with a [head_dim] gain for each.
 *  - "hf2q src/inference/vision/vit_gpu.rs", doc of vit_rms_norm_gpu and
 *    vit_per_head_rms_norm_gpu: y = x / sqrt(mean(x^2) + eps) * gain, eps
 *    inside the square root, the gain shared by all heads.
 * Readings: with n_kv_heads < n_heads the packed row is Q heads, then
 * n_kv_heads K heads, then n_kv_heads V heads (the grouped-query layout the
 * attention reads); null tables mean no rope, null gains mean no norm.
 *
 * qkv : [T, (H + 2 Hkv) * D] values (float32; exact for 16-bit data).
 * cosv, sinv : [T, D] or both NULL.  qw, kw : [D] or both NULL.
 * q : [T, H, D], k and v : [T, Hkv, D], float64.
 * Returns 0, or -1 on a bad argument.
 * ------------------------------------------------------------------------ */
static void ref_norm_rope(const float* x, const float* cosr, const float* sinr, const float* w,
                          double eps, int32_t D, double* out) {
  double y[1024];
  for (int32_t d = 0; d < D; ++d) y[d] = (double)x[d];
  if (w) {
    double ms = 0.0;
    for (int32_t d = 0; d < D; ++d) ms += y[d] * y[d];
    ms /= (double)D;
    const double r = 1.0 / sqrt(ms + eps);
    for (int32_t d = 0; d < D; ++d) y[d] = y[d] * r * (double)w[d];
  }
  if (cosr) {
    const int32_t h = D / 2;
    for (int32_t d = 0; d < D; ++d) {
      const double rot = d < h ? -y[d + h] : y[d - h];
      out[d] = y[d] * (double)cosr[d] + rot * (double)sinr[d];
    }
  } else {
    for (int32_t d = 0; d < D; ++d) out[d] = y[d];
  }
}

int vitattn_ref_qkv_prologue_f64(const float* qkv, const float* cosv, const float* sinv,
                                 const float* qw, const float* kw, double eps,
                                 double* q, double* k, double* v, int32_t n_tokens,
                                 int32_t n_heads, int32_t n_kv_heads, int32_t head_dim) {
  if (n_tokens < 0 || n_heads <= 0 || n_kv_heads <= 0 || n_heads % n_kv_heads != 0) return -1;
  if (head_dim <= 0 || head_dim % 2 != 0 || head_dim > 1024) return -1;
  if ((cosv == NULL) != (sinv == NULL) || (qw == NULL) != (kw == NULL)) return -1;
  if (qw && !(eps >= 0.0)) return -1;
  if (n_tokens == 0) return 0;
  if (!qkv || !q || !k || !v) return -1;
  const int64_t D = head_dim, H = n_heads, G = n_kv_heads;
  const int64_t row_len = (H + 2 * G) * D;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < n_tokens; ++t) {
    const float* row = qkv + t * row_len;
    const float* c = cosv ? cosv + t * D : NULL;
    const float* s = sinv ? sinv + t * D : NULL;
    for (int64_t h = 0; h < H; ++h) ref_norm_rope(row + h * D, c, s, qw, eps, head_dim, q + (t * H + h) * D);
    for (int64_t h = 0; h < G; ++h) {
      ref_norm_rope(row + (H + h) * D, c, s, kw, eps, head_dim, k + (t * G + h) * D);
      for (int64_t d = 0; d < D; ++d) v[(t * G + h) * D + d] = (double)row[(H + G + h) * D + d];
    }
  }
  return 0;
}
