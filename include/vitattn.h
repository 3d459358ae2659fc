/*
 * vitattn.h -- C ABI of libvitattn, bidirectional multi-head attention for
 * vision-transformer encoders on AMD Instinct MI355X (gfx950).
 *
 * The operation (by page title in the reference collection):
 *  - "hf2q src/inference/vision/vit_gpu.rs", doc of vit_attention_gpu: full
 *    scaled-dot-product attention with no mask, because a ViT encoder is
 *    bidirectional; Q, K, V and the output are seq-major
 *    [tokens, heads, head_dim].  Doc of vit_attention_scores_gpu: the scale
 *    multiplying Q.K^T is the caller's value (1/sqrt(head_dim) for a standard
 *    ViT, 1.0 for Gemma 4V); nothing is scaled implicitly.
 *  - "inferencelayer 0.2.1 src/vision_gpu.rs", VisionGpu::forward_one, the
 *    segment tables: a token attends within its own image and never across;
 *    batching several images is several segments.  Here the segments are the
 *    prefix array cu_seqlens.
 *  - same page, doc of vis_attn_coop_src ("The obstacle, and the way round
 *    it"): the online-softmax recurrence O <- O*e^(m_old-m_new) + P.V over key
 *    tiles, finished by dividing by the running row sum -- the algorithm the
 *    kernels use to reach the result without materialising the scores.
 *
 * For every sequence s in [0, n_seqs), every head h and every token row
 * i in [cu_seqlens[s], cu_seqlens[s+1]):
 *     o[i,h,:] = sum_j softmax_j(scale * q[i,h,:] . k[j,g,:]) * v[j,g,:]
 * with j over the same range [cu_seqlens[s], cu_seqlens[s+1]) (and, for
 * vitattn_fwd_masked, only the keys its mask keeps), and g = h (vitattn_fwd)
 * or g = h / (n_heads / n_kv_heads) (vitattn_fwd_gqa, vitattn_fwd_masked).
 */
#ifndef VITATTN_H
#define VITATTN_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Element types of q, k, v and o.  The 16-bit kinds multiply in their own
 * precision with float32 accumulation: the softmax weights are rounded to the
 * input kind (nearest even) before the P.V product, and a 16-bit output is
 * rounded to nearest even.  F16 and the float32 outputs follow "hf2q
 * src/inference/vision/vit_gpu.rs", vit_attention_gpu (the peer-precision
 * attention: K and V staged in F16 with float32 accumulation, F32 outputs).
 */
typedef enum {
  VITATTN_DTYPE_F32 = 0,          /* q, k, v, o float32; computed in float32 (float32 MFMA) */
  VITATTN_DTYPE_BF16 = 1,         /* q, k, v, o bfloat16 */
  VITATTN_DTYPE_F16 = 2,          /* q, k, v, o IEEE half */
  VITATTN_DTYPE_BF16_OUT_F32 = 3, /* q, k, v bfloat16; o float32 (not rounded to 16 bits) */
  VITATTN_DTYPE_F16_OUT_F32 = 4   /* q, k, v IEEE half; o float32 */
} vitattn_dtype_t;

/* Status codes.  Every entry point returns one of these. */
typedef enum {
  VITATTN_OK = 0,
  VITATTN_ERR_INVALID_ARG = -1,           /* null/misaligned pointer, bad count, non-finite scale */
  VITATTN_ERR_UNSUPPORTED_HEAD_DIM = -2,  /* head_dim not in {64, 72, 80, 128} */
  VITATTN_ERR_UNSUPPORTED_DTYPE = -3,     /* dtype not a vitattn_dtype_t value (0 .. 4) */
  VITATTN_ERR_NO_DEVICE = -4,             /* no HIP device, or the current one is not gfx950 */
  VITATTN_ERR_OOM = -5,                   /* reserved: the forward pass allocates nothing */
  VITATTN_ERR_HIP = -6                    /* a HIP runtime call or kernel launch failed */
} vitattn_status_t;

/*
 * vitattn_fwd -- enqueue one attention forward pass on `stream`.
 *
 * q, k, v : DEVICE pointers, contiguous [T, n_heads, head_dim] of the input
 *           element type of `dtype`, T = cu_seqlens[n_seqs].  16-byte aligned.
 *           Read only.
 * o       : DEVICE pointer, contiguous [T, n_heads, head_dim] of the output
 *           element type of `dtype`, 16-byte aligned, must not overlap q, k or
 *           v.  Every row that lies in some sequence is written; nothing else
 *           is.
 * cu_seqlens : DEVICE pointer to int32[n_seqs + 1]: cu_seqlens[0] is the
 *           first token row, the array is non-decreasing and sequence s owns
 *           rows [cu_seqlens[s], cu_seqlens[s+1]).  Zero-length sequences are
 *           allowed and produce nothing.  This is a precondition the library
 *           does not check (it never reads device memory on the host); the
 *           Python binding checks it when the array is on the host or when
 *           asked to.
 * n_seqs  : number of sequences (images), >= 0.  0 enqueues nothing.
 * n_heads : > 0.  head_dim : 64, 72, 80 or 128.
 * scale   : finite; multiplies q.k before the softmax (1/sqrt(head_dim) for a
 *           standard ViT; 1.0 is valid).
 * Inputs  : q, k and v hold finite values (no NaN, no infinity).  This is a
 *           precondition the library does not check (it never reads device
 *           memory on the host): the kernels are built without NaN handling
 *           in their max and min operations, so a non-finite input gives
 *           unspecified (but in-bounds) output rows for the sequences and
 *           heads that read it.
 * dtype   : a vitattn_dtype_t.
 * stream  : HIP stream to enqueue on (0 = the legacy default stream).
 *
 * Arguments are validated before any HIP call.  The call does not
 * synchronise the host, allocates no device memory and is safe to call from
 * several host threads on different streams.  After a first call on a
 * device (which sets up that device's kernel table), a call enqueues kernel
 * launches (one per 512 sequences) and nothing else, so it may be captured
 * into a HIP graph; each replay reads the buffers' contents at that time.
 * The library never prints, aborts or computes anything on the CPU: a
 * failure is a status code plus a message in vitattn_last_error().  Results
 * are bitwise reproducible for the same inputs and device.
 */
int vitattn_fwd(const void* q, const void* k, const void* v, void* o,
                const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_heads,
                int32_t head_dim, float scale, int32_t dtype, hipStream_t stream);

/*
 * vitattn_fwd_gqa -- the same forward pass with grouped-query attention: k and
 * v carry n_kv_heads heads, a divisor of n_heads, and query head h attends
 * with K/V head h / (n_heads / n_kv_heads).  This is the grouping of "hf2q
 * src/inference/vision/vit_gpu.rs", doc of vit_repeat_kv_gpu, used by
 * gemma4v_block_forward_gpu to widen K and V to the query heads before
 * attention; here the K/V heads are read in place and never copied.
 *
 * q, o    : as for vitattn_fwd, [T, n_heads, head_dim].
 * k, v    : DEVICE pointers, contiguous [T, n_kv_heads, head_dim] of `dtype`,
 *           16-byte aligned.  Read only.
 * n_kv_heads : > 0 and a divisor of n_heads (else VITATTN_ERR_INVALID_ARG,
 *           before any HIP call).  n_kv_heads == n_heads is vitattn_fwd;
 *           n_kv_heads == 1 is multi-query attention.
 * Every other argument, the validation order, the asynchrony and the error
 * behaviour are those of vitattn_fwd.  For each (sequence, query head) the
 * result is bitwise that of vitattn_fwd on K/V whose head h holds K/V head
 * h / (n_heads / n_kv_heads).
 */
int vitattn_fwd_gqa(const void* q, const void* k, const void* v, void* o,
                    const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_heads,
                    int32_t n_kv_heads, int32_t head_dim, float scale, int32_t dtype,
                    hipStream_t stream);

/*
 * vitattn_fwd_masked -- the grouped-query forward pass with a mask inside each
 * sequence.  With the query at position qi and the key at position kj of the
 * same sequence, the key takes part only if
 *   causal == 1 : kj <= qi -- the aligned causal rule kj <= qi + (Lk - Lq) of
 *                 "hanzo-ml 0.11.4 src/vulkan_backend.rs", doc of
 *                 flash_attn_gpu, with as many keys as queries (Lk = Lq);
 *   window > 0  : |qi - kj| < window -- the key window of the encoder
 *                 attention meta in "inferencelayer 0.2.1 src/vision_gpu.rs",
 *                 VisionGpu::forward_one, where 0 means unrestricted (the page
 *                 gives no further definition; this band is the reading taken
 *                 here).  With causal == 1 it keeps the query and the
 *                 window - 1 keys before it.
 * Both rules hold together when both are set.  Every query keeps at least
 * itself, so every output row is defined.  The softmax runs over the kept
 * keys only; the others get weight exactly 0.
 *
 * causal  : 0 or 1 (else VITATTN_ERR_INVALID_ARG, before any HIP call).
 * window  : >= 0 (else VITATTN_ERR_INVALID_ARG).
 * causal == 0 && window == 0 is vitattn_fwd_gqa, bit for bit (the same
 * kernels run).  Every other argument, the validation order, the asynchrony
 * and the error behaviour are those of vitattn_fwd_gqa.
 */
int vitattn_fwd_masked(const void* q, const void* k, const void* v, void* o,
                       const int32_t* cu_seqlens, int32_t n_seqs, int32_t n_heads,
                       int32_t n_kv_heads, int32_t head_dim, float scale, int32_t causal,
                       int32_t window, int32_t dtype, hipStream_t stream);

/*
 * vitattn_qkv_prologue -- enqueue the input side of the attention: split the
 * packed projection output into Q, K and V in the layout vitattn_fwd_gqa
 * reads, normalise Q and K per head (optional) and apply the rope (optional).
 * Sources: "inferencelayer 0.2.1 src/vision_gpu.rs", VIS_QKV_ROPE (the
 * split, rope tables from the caller, V not rotated) and GLM_QKV_QKNORM_ROPE
 * (the per-head RMS norm of Q and K before the rope); "hf2q
 * src/inference/vision/vit_gpu.rs", vit_rms_norm_gpu (eps inside the square
 * root, a [head_dim] gain shared by all heads).
 *
 * For every token t, with x a head vector of D = head_dim elements:
 *   norm (q_weight, k_weight given): x[d] <- x[d] / sqrt(mean(x^2) + eps) * w[d]
 *   rope (cos_table, sin_table given):
 *     out[d] = x[d] cos[t,d] + r[d] sin[t,d],  r[d] = -x[d + D/2] (d < D/2),
 *                                              r[d] =  x[d - D/2] (d >= D/2)
 * applied to the query heads (gain q_weight) and the key heads (k_weight);
 * the value heads are copied.  All arithmetic is float32; 16-bit outputs are
 * rounded to nearest even.
 *
 * qkv     : DEVICE, [n_tokens, (n_heads + 2*n_kv_heads) * head_dim] of dtype:
 *           per token the query heads, then the key heads, then the value
 *           heads.  16-byte aligned.  Read only.
 * cos_table, sin_table : DEVICE float32 [n_tokens, head_dim], 16-byte
 *           aligned, or both NULL (no rope).
 * q_weight, k_weight : DEVICE float32 [head_dim], 16-byte aligned, or both
 *           NULL (no norm).  eps : finite, >= 0 (used only with the gains).
 * q       : DEVICE [n_tokens, n_heads, head_dim] of dtype (written), 16-byte
 *           aligned.
 * k, v    : DEVICE [n_tokens, n_kv_heads, head_dim] of dtype (written),
 *           16-byte aligned.
 *           The outputs must not overlap qkv or each other.
 * n_kv_heads : > 0, a divisor of n_heads.  head_dim : 64, 72, 80 or 128.
 * dtype   : VITATTN_DTYPE_F32, _BF16 or _F16 (inputs and outputs alike;
 *           others give VITATTN_ERR_UNSUPPORTED_DTYPE).
 * n_tokens == 0 enqueues nothing.  Validation, asynchrony and error behaviour
 * are those of vitattn_fwd; no device memory is allocated.
 */
int vitattn_qkv_prologue(const void* qkv, const float* cos_table, const float* sin_table,
                         const float* q_weight, const float* k_weight, float eps, void* q,
                         void* k, void* v, int32_t n_tokens, int32_t n_heads, int32_t n_kv_heads,
                         int32_t head_dim, int32_t dtype, hipStream_t stream);

/* Static, never-NULL description of a status code. */
const char* vitattn_status_string(int status);

/* Thread-local detail of the last failure on this host thread ("" if none). */
const char* vitattn_last_error(void);

/*
 * vitattn_kernel_config -- describe the launch that vitattn_fwd makes for a
 * (head_dim, dtype) pair on the current device, without launching anything.
 * Writes the queries per work item (*block_m), the keys per LDS tile
 * (*block_n), the wavefronts per workgroup (*waves) and the persistent grid
 * size (*grid, workgroups).  Any output pointer may be NULL.  Returns a
 * status code (the same argument errors as vitattn_fwd; NO_DEVICE or HIP if
 * the device cannot be queried).
 */
int vitattn_kernel_config(int32_t head_dim, int32_t dtype, int32_t* block_m,
                          int32_t* block_n, int32_t* waves, int32_t* grid);

#ifdef __cplusplus
}
#endif

#endif /* VITATTN_H */
