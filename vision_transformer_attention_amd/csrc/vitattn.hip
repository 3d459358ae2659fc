// vitattn.hip -- bidirectional multi-head attention over packed variable-length
// sequences for gfx950 (MI355X), behind the C ABI declared in include/vitattn.h.
//
// What is computed (by page title in the reference collection):
//  * "hf2q src/inference/vision/vit_gpu.rs", vit_attention_gpu doc: softmax
//    attention with no mask (the ViT encoder is bidirectional), seq-major
//    [tokens, heads, head_dim] tensors, and (vit_attention_scores_gpu doc) a
//    caller-supplied scale on Q.K^T.
//  * "inferencelayer 0.2.1 src/vision_gpu.rs", VisionGpu::forward_one segment
//    tables: attention stays within one image; several images are several
//    segments, here given by the cu_seqlens prefix array.
//  * same page, vis_attn_coop_src doc ("The obstacle, and the way round it"):
//    the online-softmax update O <- O*e^(m_old - m_new) + P.V over key tiles,
//    finished by a division by the running row sum.  That page keeps the running
//    output in shared memory because its matrix type cannot be scaled; on gfx950
//    MFMA accumulators are ordinary registers, so the rescale happens in place.
//    The same doc names K/V re-reads per query block as the real bound and
//    widening the query block as the lever: here one workgroup stages each K/V
//    tile in LDS once for BLOCK_M queries (several wavefronts), and every K/V
//    byte read from LDS feeds 16*QB queries of one wavefront.
//
// Design (gfx950 specific, wave64):
//  * One persistent launch.  Every workgroup builds the work plan itself from
//    cu_seqlens (sequences ordered longest first, items = (sequence, head,
//    query tile)), then walks the item list with a stride of the grid size.
//    Slots are assigned so that the workgroups of one XCD (blockIdx % 8) take
//    consecutive items, which share a (sequence, head) and so its K/V in that
//    XCD's L2.  When the large query tiles would leave most of the grid idle (one
//    short image), the launch re-plans with small ones, and an unmasked launch whose
//    small items are still too few splits each item's keys between two wavefronts
//    whose partial results are merged through LDS.
//  * Scores are computed transposed, S^T = K.Q^T, with v_mfma_f32_16x16x32_bf16
//    (float32: v_mfma_f32_16x16x4_f32).  In that accumulator layout a lane holds
//    4 keys of one query, so a row max is in-lane plus two cross-lane steps, and
//    the same registers (converted to bf16) are directly the B operand of
//    O^T += V^T.P^T: no data movement between the two products, and the running
//    output of a query sits in the lane that owns its softmax state, so a rescale
//    is a per-lane multiply.
//  * bf16: K/V tiles go HBM -> LDS by buffer_load_dwordx4 ... lds (no VGPRs, no LDS
//    write instructions; scalar addressing through a buffer resource per tile that
//    is bounded by the sequence), double-buffered, K as [key][d] and V as [key][d] read
//    transposed by ds_read_b64_tr_b16, rows padded against bank conflicts.  The
//    exponent offset of each query row is fixed by the first 32 keys and kept
//    while no weight reaches 2 (an in-lane max decides, no cross-lane reduction);
//    the rare rise past that is handled by a rescale.  Row sums come from one more
//    MFMA against a block of ones.  The last tile of a sequence ends at its last
//    key, so only the first step of a work item is partial.
//  * float32: K/V staged through registers (V transposed while staging), running
//    max raised lazily (only past kLazyTau) with a wave-uniform rescale.
//  * head_dim 72 and 80 use a 16-deep tail step in Q.K^T (dims past D are zero in
//    Q) and are padded to 80 for the P.V output rows (blocks of 16).
#include "vitattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <type_traits>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kMaxSeqs = 512;     // sequences planned by one launch (more: several launches)
constexpr int kSortMax = 256;     // sequences ordered longest-first up to this count
constexpr float kLazyTau = 8.0f;  // float32 kernel: headroom (log2) before the running max is raised
constexpr float kHeadroom = 16.0f;  // bf16 kernel: log2 gap between the reference max and the exponent offset
constexpr float kLog2e = 1.4426950408889634f;

// ----------------------------------------------------------------------------
// Work plan, built by every workgroup in LDS.
// ----------------------------------------------------------------------------
struct PlanLds {
  int cu[kMaxSeqs + 1];
  int order[kMaxSeqs];
  int prefix[kMaxSeqs + 1];  // items before sorted position r
  int wave_tot[16];
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// P.prefix[r] = count(0) + ... + count(r - 1) for r = 0 .. n (n >= 1); returns P.prefix[n].
// Thread tid owns positions [tid*per, tid*per + per).
template <int NT, class F>
__device__ int scan_to_prefix(PlanLds& P, int n, F count) {
  const int tid = threadIdx.x;
  const int per = ceil_div(n, NT);
  const int beg = tid * per;
  const int end = min(beg + per, n);
  int local = 0;
  for (int r = beg; r < end; ++r) local += count(r);
  const int lane = tid & 63, wave = tid >> 6;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) P.wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += P.wave_tot[w];
  int run = base + incl - local;
  if (tid == 0) P.prefix[0] = 0;
  for (int r = beg; r < end; ++r) {
    run += count(r);
    P.prefix[r + 1] = run;
  }
  __syncthreads();
  return P.prefix[n];
}

// Loads the sequence bounds of `cu` (n >= 1 sequences) into P and orders the sequences
// longest first (when n <= kSortMax; else in index order).
template <int NT>
__device__ void plan_load(PlanLds& P, const int32_t* __restrict__ cu, int n) {
  const int tid = threadIdx.x;
  for (int i = tid; i <= n; i += NT) P.cu[i] = cu[i];
  __syncthreads();
  if (n <= kSortMax) {
    for (int i = tid; i < n; i += NT) {
      const int li = P.cu[i + 1] - P.cu[i];
      int rank = 0;
      for (int j = 0; j < n; ++j) {
        const int lj = P.cu[j + 1] - P.cu[j];
        rank += (lj > li) || (lj == li && j < i);
      }
      P.order[rank] = i;
    }
  } else {
    for (int i = tid; i < n; i += NT) P.order[i] = i;
  }
  __syncthreads();
}

// Fills P.prefix with the items (sequence, head, bm-query block) of the sequences in P's
// order, after plan_load.  Returns the item count.
template <int NT>
__device__ int plan_items(PlanLds& P, int n, int n_heads, int bm) {
  return scan_to_prefix<NT>(P, n, [&](int r) {
    const int s = P.order[r];
    return ceil_div(P.cu[s + 1] - P.cu[s], bm) * n_heads;
  });
}

// Causal launches: an item's cost grows with its query block's index k inside the image
// (it reads the keys of blocks 0 .. k), so the items are listed by decreasing cost
// instead.  The items of block index k (one per image longer than k*bm and head) form a
// level; levels run from the largest k down, and within a level the images go longest
// first with the heads fastest.  Dealt out in alternating rounds, the list then pairs
// costly items with cheap ones.  P.prefix[p] becomes the items before level p (block index
// K-1-p), p = 0 .. K.  Needs the length-sorted order (n <= kSortMax) and K <= kMaxSeqs
// levels, and runs after plan_items; returns K, or 0 (the sequence plan stays).
template <int NT>
__device__ int build_levels(PlanLds& P, int n, int n_heads, int bm) {
  if (n > kSortMax) return 0;
  const int maxl = P.cu[P.order[0] + 1] - P.cu[P.order[0]];
  const int K = ceil_div(maxl, bm);
  if (K < 1 || K > kMaxSeqs) return 0;
  __syncthreads();  // every thread has read the sequence plan's prefix (the item count)
  scan_to_prefix<NT>(P, K, [&](int p) {
    // images longer than k*bm, k = K-1-p: a prefix of the longest-first order
    const int thr = (K - 1 - p) * bm;
    int lo = 0, hi = n;  // first sorted position whose image is not longer than thr
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      const int s = P.order[mid];
      if (P.cu[s + 1] - P.cu[s] > thr) lo = mid + 1; else hi = mid;
    }
    return lo * n_heads;
  });
  return K;
}

struct Item {
  int a, b;   // key rows [a, b) of the sequence
  int head;
  int q0;     // first query row of the item
};

__device__ __forceinline__ Item map_item(const PlanLds& P, int n, int it, int bm) {
  int lo = 0, hi = n;  // P.prefix[lo] <= it < P.prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (P.prefix[mid] <= it) lo = mid; else hi = mid;
  }
  const int s = P.order[lo];
  Item r;
  r.a = P.cu[s];
  r.b = P.cu[s + 1];
  const int tiles = ceil_div(r.b - r.a, bm);
  const int local = it - P.prefix[lo];
  r.head = local / tiles;
  r.q0 = r.a + (local % tiles) * bm;
  return r;
}

// Masks ("hanzo-ml 0.11.4 src/vulkan_backend.rs", flash_attn_gpu doc: aligned causal, key
// kj <= query qi + (Lk - Lq), which inside one image (Lk = Lq) is kj <= qi; and the encoder
// attention's key window of "inferencelayer 0.2.1 src/vision_gpu.rs", read as
// |qi - kj| < window with 0 = no window).  Positions are global token rows here: both rules
// compare differences of rows of the same image, so the image's start cancels.
__device__ __forceinline__ bool key_visible(int i, int j, int causal, int window) {
  return (!causal | (j <= i)) & ((window <= 0) | ((j - i < window) & (i - j < window)));
}

// Narrows the keys [ka, kb) of an item (queries [q0, qend)) to those some query sees.  The
// result is never empty: query q0 sees itself.
// (Token rows are below 2^31 - 64, so differences of rows and keys never overflow; the
// window is only ever compared with such differences, never added to a row.)
__device__ __forceinline__ void mask_key_range(int& ka, int& kb, int q0, int qend, int causal, int window) {
  if (window > 0) {
    ka = max(ka, q0 - window + 1);              // q0 >= 0: no overflow
    if (window <= kb - qend) kb = qend - 1 + window;  // kb = min(kb, qend - 1 + window)
  }
  if (causal) kb = min(kb, qend);
}

// Item `it` of a level plan of K levels (build_levels).
__device__ __forceinline__ Item map_item_levels(const PlanLds& P, int K, int it, int bm, int n_heads) {
  int lo = 0, hi = K;  // P.prefix[lo] <= it < P.prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (P.prefix[mid] <= it) lo = mid; else hi = mid;
  }
  const int local = it - P.prefix[lo];
  const int s = P.order[local / n_heads];
  Item r;
  r.a = P.cu[s];
  r.b = P.cu[s + 1];
  r.head = local % n_heads;
  r.q0 = r.a + (K - 1 - lo) * bm;
  return r;
}

// ----------------------------------------------------------------------------
// Element-type specific parts.
// ----------------------------------------------------------------------------
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// float32 inputs: v_mfma_f32_16x16x4_f32 for both products (no bf16 rounding).
template <int D_, int QB_, int NW_, int BN_>
struct F32Traits {
  using elem_t = float;
  static constexpr int D = D_, QB = QB_, NW = NW_, BN = BN_;
  static constexpr int NT = NW * 64;
  static constexpr int NQ = QB * 16;
  static constexpr int BM = NW * NQ;
  static constexpr int DK = (D + 15) / 16 * 16;  // contraction in groups of 16 (4 steps of 4)
  static constexpr int NKT = DK / 16;
  static constexpr int DV = (D + 15) / 16 * 16;
  static constexpr int NDB = DV / 16;
  static constexpr int NKB = BN / 16;
  static constexpr int KSTR = DK + 4;
  static constexpr int VSTR = BN + 4;
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int STAGE_ELEMS = K_ELEMS + DV * VSTR;
  static constexpr int CH = D / 4;                // 16-byte chunks per row
  static constexpr int K_UNITS = BN * CH;
  static constexpr int V_UNITS = (BN / 4) * CH;   // 4 keys x 4 dims each
  static constexpr int K_IT = (K_UNITS + NT - 1) / NT;
  static constexpr int V_IT = (V_UNITS + NT - 1) / NT;
  static_assert(D % 4 == 0 && BN % 16 == 0, "tile shape");

  struct QOp { f32x4_t x[QB][NKT]; };
  struct Pre { f32x4_t k[K_IT]; f32x4_t v[V_IT][4]; };

  static __device__ __forceinline__ void load_q(QOp& Q, const elem_t* __restrict__ q, int row0, int qend,
                                                int head, int n_heads, bool negate, int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = row0 + qb * 16 + c;
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
        const int d0 = t * 16 + 4 * g;
        f32x4_t w = {0.f, 0.f, 0.f, 0.f};
        if (row < qend && d0 < D) w = *reinterpret_cast<const f32x4_t*>(q + ((size_t)row * n_heads + head) * D + d0);
        Q.x[qb][t] = negate ? -w : w;
      }
    }
  }

  static __device__ __forceinline__ void zero_pad(elem_t* stage) {
    if constexpr (DK > D) {
      constexpr int PADW = DK - D;
      for (int i = threadIdx.x; i < 2 * BN * PADW; i += NT) {
        const int buf = i / (BN * PADW), rem = i % (BN * PADW);
        stage[buf * STAGE_ELEMS + (rem / PADW) * KSTR + D + rem % PADW] = 0.0f;
      }
    }
  }

  static __device__ __forceinline__ void fetch(Pre& R, const elem_t* __restrict__ k, const elem_t* __restrict__ v,
                                               int key0, int b, int head, int n_heads) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < K_IT; ++i) {
      const int u = tid + i * NT;
      R.k[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (u < K_UNITS) {
        const int key = key0 + u / CH;
        if (key < b) R.k[i] = *reinterpret_cast<const f32x4_t*>(k + ((size_t)key * n_heads + head) * D + (u % CH) * 4);
      }
    }
#pragma unroll
    for (int i = 0; i < V_IT; ++i) {
      const int u = tid + i * NT;
#pragma unroll
      for (int j = 0; j < 4; ++j) R.v[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (u < V_UNITS) {
        const int kbase = key0 + (u / CH) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (kbase + j < b)
            R.v[i][j] = *reinterpret_cast<const f32x4_t*>(v + ((size_t)(kbase + j) * n_heads + head) * D + (u % CH) * 4);
      }
    }
  }

  static __device__ __forceinline__ void store(const Pre& R, elem_t* stage) {
    const int tid = threadIdx.x;
    elem_t* Ks = stage;
    elem_t* Vt = stage + K_ELEMS;
#pragma unroll
    for (int i = 0; i < K_IT; ++i) {
      const int u = tid + i * NT;
      if (u < K_UNITS) *reinterpret_cast<f32x4_t*>(Ks + (u / CH) * KSTR + (u % CH) * 4) = R.k[i];
    }
#pragma unroll
    for (int i = 0; i < V_IT; ++i) {
      const int u = tid + i * NT;
      if (u < V_UNITS) {
        const int kap = (u / CH) * 4;
        const int d0 = (u % CH) * 4;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *reinterpret_cast<f32x4_t*>(Vt + (d0 + e) * VSTR + kap) =
              f32x4_t{R.v[i][0][e], R.v[i][1][e], R.v[i][2][e], R.v[i][3][e]};
      }
    }
  }

  static __device__ __forceinline__ void qk(f32x4_t (&S)[NKB][QB], const QOp& Q, const elem_t* stage, int lane) {
    const int g = lane >> 4, c = lane & 15;
    const elem_t* Ks = stage;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) S[kb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(Ks + (kb * 16 + c) * KSTR + t * 16 + 4 * g);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], Q.x[qb][t][i], S[kb][qb], 0, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ void pv(f32x4_t (&O)[NDB][QB], const f32x4_t (&S)[NKB][QB],
                                            const elem_t* stage, int lane) {
    const int g = lane >> 4, c = lane & 15;
    const elem_t* Vt = stage + K_ELEMS;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(Vt + (db * 16 + c) * VSTR + kb * 16 + 4 * g);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            O[db][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], S[kb][qb][r], O[db][qb], 0, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ void store_out(elem_t* __restrict__ o, size_t off, const f32x4_t& x, float inv) {
    *reinterpret_cast<f32x4_t*>(o + off) = x * inv;
  }
};

// ----------------------------------------------------------------------------
// The attention kernel (persistent).
// ----------------------------------------------------------------------------
template <class T, bool MASK>
__global__ __launch_bounds__(T::NT) void attn_fwd_f32_kernel(
    const typename T::elem_t* __restrict__ q, const typename T::elem_t* __restrict__ k,
    const typename T::elem_t* __restrict__ v, typename T::elem_t* __restrict__ o,
    const int32_t* __restrict__ cu, int n_seqs, int n_heads, int n_kv_heads, float c2, int negate, int causal,
    int window) {
  using elem_t = typename T::elem_t;
  const int kv_group = n_heads / n_kv_heads;  // query heads per K/V head
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  PlanLds& plan = *reinterpret_cast<PlanLds*>(smem);
  elem_t* stage = reinterpret_cast<elem_t*>(smem + ((sizeof(PlanLds) + 15) / 16) * 16);

  plan_load<T::NT>(plan, cu, n_seqs);
  const int n_items = plan_items<T::NT>(plan, n_seqs, n_heads, T::BM);
  T::zero_pad(stage);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int G = gridDim.x;
  const int slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  for (int it = slot; it < n_items; it += G) {
    const Item item = map_item(plan, n_seqs, it, T::BM);
    const int qend = min(item.q0 + T::BM, item.b);
    const int row0 = item.q0 + wave * T::NQ;
    int klo = item.a, khi = item.b;  // the keys that some row of the item sees
    if constexpr (MASK) mask_key_range(klo, khi, item.q0, qend, causal, window);

    typename T::QOp Q;
    T::load_q(Q, q, row0, qend, item.head, n_heads, negate != 0, lane);

    f32x4_t O[T::NDB][T::QB];
#pragma unroll
    for (int db = 0; db < T::NDB; ++db)
#pragma unroll
      for (int qb = 0; qb < T::QB; ++qb) O[db][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m[T::QB], lsum[T::QB];
#pragma unroll
    for (int qb = 0; qb < T::QB; ++qb) { m[qb] = -INFINITY; lsum[qb] = 0.f; }

    const int ntiles = ceil_div(khi - klo, T::BN);
    typename T::Pre pre;
    __syncthreads();  // the previous item is done with both stage buffers
    const int kv_head = item.head / kv_group;
    T::fetch(pre, k, v, klo, khi, kv_head, n_kv_heads);
    T::store(pre, stage);

    for (int t = 0; t < ntiles; ++t) {
      __syncthreads();  // tile t is in LDS; buffer (t+1)&1 is free
      const elem_t* cur = stage + (t & 1) * T::STAGE_ELEMS;
      const int key0 = klo + t * T::BN;
      if (t + 1 < ntiles) T::fetch(pre, k, v, key0 + T::BN, khi, kv_head, n_kv_heads);

      f32x4_t S[T::NKB][T::QB];
      T::qk(S, Q, cur, lane);

      // Keys past the range, and with a mask the keys a row does not see, take no part in
      // the max and get weight exactly 0 below.
      const bool ragged = key0 + T::BN > khi;  // last tile runs past the range
      bool vis[T::NKB][T::QB][4];
      bool partial = ragged;
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < T::QB; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = key0 + kb * 16 + 4 * g + r;
            bool ok = j < khi;
            if constexpr (MASK) ok = ok && key_visible(min(row0 + qb * 16 + c, qend - 1), j, causal, window);
            vis[kb][qb][r] = ok;
          }
      if constexpr (MASK) partial = true;
      if (partial) {
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int qb = 0; qb < T::QB; ++qb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (!vis[kb][qb][r]) S[kb][qb][r] = -INFINITY;
      }

      float alpha[T::QB];
      bool raise = false;
#pragma unroll
      for (int qb = 0; qb < T::QB; ++qb) {
        float mx = S[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[kb][qb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mc = mx * c2;
        alpha[qb] = 1.f;
        if (mx != -INFINITY && mc > m[qb] + kLazyTau) {  // (a masked row may see no key here)
          alpha[qb] = exp2f(m[qb] - mc);
          m[qb] = mc;
          raise = true;
        }
      }
      if (__any(raise)) {
#pragma unroll
        for (int qb = 0; qb < T::QB; ++qb) {
          lsum[qb] *= alpha[qb];
#pragma unroll
          for (int db = 0; db < T::NDB; ++db) O[db][qb] *= alpha[qb];
        }
      }
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < T::QB; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            S[kb][qb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][qb][r], c2, -m[qb]));
      if (partial) {  // weight exactly 0 (also when the scale is 0 or the row is not set yet)
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int qb = 0; qb < T::QB; ++qb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (!vis[kb][qb][r]) S[kb][qb][r] = 0.f;
      }
#pragma unroll
      for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < T::QB; ++qb)
#pragma unroll
          for (int r = 0; r < 4; ++r) lsum[qb] += S[kb][qb][r];

      T::pv(O, S, cur, lane);

      if (t + 1 < ntiles) T::store(pre, stage + ((t + 1) & 1) * T::STAGE_ELEMS);
    }

    // epilogue: O / l for the rows of this wavefront that lie in the sequence
#pragma unroll
    for (int qb = 0; qb < T::QB; ++qb) {
      float l = lsum[qb];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      const float inv = 1.0f / l;
      const int row = row0 + qb * 16 + c;
      if (row < qend) {
#pragma unroll
        for (int db = 0; db < T::NDB; ++db) {
          const int d0 = db * 16 + 4 * g;
          if (d0 < T::D) T::store_out(o, ((size_t)row * n_heads + item.head) * T::D + d0, O[db][qb], inv);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 inputs: direct HBM->LDS staging, v_mfma_f32_16x16x32_bf16 for both products.
//
// LDS layout of one stage (one BN-key tile):
//   K: [BN][KCH chunks of 16 B]  -- LDS has 64 banks of 4 bytes and serves a 16-byte read
//      in passes of 32 lanes; the 32 lanes of one A-operand read cover 8 consecutive rows
//      at 4 column chunks, so the row stride must put those 8 rows on distinct 16-byte bank
//      groups that are also 32-byte aligned.  KCH = 2 (mod 4) does both (10 chunks for
//      head_dim 64..80, 18 for 128); an odd stride costs about 4 extra cycles per read.  The
//      8-byte reads of the 16-deep tail step (head_dim 72, 80: chunks TCH and TCH + 1) take 16
//      rows x one chunk per pass, which a stride of 10 chunks puts 2-way on rows c and c + 8;
//      rows with bit 3 set therefore hold those two chunks swapped (the tail swizzle).  Chunks
//      past the head_dim hold a copy of real data (finite) and meet zero Q columns.
//   V: [BN][VCH chunks of 16 B]  -- natural [key][d] order; read with the transposing
//      ds_read_b64_tr_b16, whose 4-row x 32-byte footprint per 16 lanes is bank-conflict
//      free with a row stride of 8 (mod 32) words.
// Both are filled by buffer_load_dwordx4 with the lds bit: lane l of a wave-wide load
// lands at base + 16*l, so each wave-wide load fills 64 consecutive chunk slots.
// ---------------------------------------------------------------------------
// E_: element kind of q, k, v (kBF16 or kF16); OF32_: the output is float32 instead of the
// input element type.
constexpr int kBF16 = 0, kF16 = 1;
template <int D_, int QB_, int NW_, int BN_, int E_ = kBF16, bool OF32_ = false>
struct Bf16Cfg {
  using elem_t = __bf16;  // 16-bit storage; the bits are bf16 or f16 by E
  static constexpr int D = D_, QB = QB_, NW = NW_, BN = BN_, E = E_;
  static constexpr bool OF32 = OF32_;
  static constexpr int NT = NW * 64;
  static constexpr int NQ = QB * 16;            // queries per wavefront
  static constexpr int BM = NW * NQ;            // queries per work item
  static constexpr int KSUB = 32;               // keys per compute step
  static constexpr int NSUB = BN / KSUB;
  static constexpr int NK32 = D / 32;           // Q.K^T contraction: 32-deep MFMA steps ...
  static constexpr int TAIL = D % 32 ? 1 : 0;   // ... plus one 16-deep step (d past D zero)
  static constexpr int DK = NK32 * 32 + 16 * TAIL;
  static constexpr int DV = (D + 15) / 16 * 16; // O^T rows, padded
  static constexpr int NDB = DV / 16;
  static constexpr int NACC = NDB + 1;         // plus one block for the row sums
  static constexpr int CH = D / 8;              // 16-byte chunks of a row in HBM
  static constexpr int KCH = (DK / 8 + 1) / 4 * 4 + 2;  // smallest >= DK / 8 with KCH % 4 == 2
  static constexpr int TCH = NK32 * 4;                   // first chunk of the 16-deep tail
  static constexpr int VCH = D <= 80 ? 10 : 18;
  static constexpr int KSTR = KCH * 8, VSTR = VCH * 8;  // elements
  static constexpr int K_BYTES = BN * KCH * 16, V_BYTES = BN * VCH * 16;
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
  static constexpr int K_LOADS = BN * KCH / 64, V_LOADS = BN * VCH / 64;
  static constexpr int LOADS = K_LOADS + V_LOADS;
  static_assert(D % 8 == 0 && BN % 64 == 0 && D - NK32 * 32 <= 16, "tile shape");
  static_assert(VCH * 8 >= DV && (VCH * 4) % 32 == 8, "V stride");
  static_assert(KCH * 8 >= DK && KCH % 4 == 2 && KCH - 4 < DK / 8, "K stride");
  static_assert(!TAIL || TCH + 2 == KCH, "the tail swizzle swaps the last two chunks of a K row");
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) unsigned char lds_u8_t;

__device__ __forceinline__ float fbits(unsigned x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ unsigned ubits(float x) { return __builtin_bit_cast(unsigned, x); }

// max over the four lanes l, l^16, l^32, l^48 (permlane swaps: VALU only, no LDS)
__device__ __forceinline__ float max_4groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(ubits(x), ubits(x), false, false);
  x = fmaxf(fbits(a[0]), fbits(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(ubits(x), ubits(x), false, false);
  return fmaxf(fbits(b[0]), fbits(b[1]));
}


// Wave-wide DMA loads of one K/V tile.  The K area takes K_LOADS loads and the V area V_LOADS,
// each load filling 64 consecutive 16-byte chunk slots (lane l of load slot s fills chunk slot
// s*64 + l: key row (s*64 + l) / per-row chunks, chunk (s*64 + l) % per-row chunks; chunks past
// head_dim repeat the last real chunk, so every byte copied is finite data of that row).  Wave
// w issues K slots w, w + NW, ... and then V slots w, w + NW, ...: KPW + VPW loads for every
// wave, so the issue has no branch.  A slot number past the last load stands for the wave's
// previous slot, which is loaded twice (the same bytes to the same place, before the same
// barrier), instead of a branch that skips it.
template <class C>
struct Dma {
  static constexpr int KPW = (C::K_LOADS + C::NW - 1) / C::NW;  // K loads per wave
  static constexpr int VPW = (C::V_LOADS + C::NW - 1) / C::NW;  // V loads per wave
  static constexpr int PER_WAVE = KPW + VPW;
  static_assert(C::K_LOADS > C::NW && C::V_LOADS > C::NW, "each wave has a previous slot to repeat");

  // wave w's i-th slot of an area of n loads
  static __device__ __forceinline__ int slot(int wave, int i, int n) {
    const int s = wave + i * C::NW;
    return s < n ? s : s - C::NW;
  }

  // Byte offset of lane `lane` of slot s (in the K area when IS_K) relative to the tile's row
  // `lead`; rows of the tile before `lead` are filled with copies of row `lead`.
  template <bool IS_K>
  static __device__ __forceinline__ unsigned lane_offset(int s, int lane, int lead, unsigned row_bytes) {
    constexpr int per = IS_K ? C::KCH : C::VCH;
    const unsigned z = (unsigned)(s * 64 + lane);
    const int row = max((int)(z / per), lead) - lead;  // division by a constant
    int ch = (int)(z % per);
    if constexpr (IS_K && C::TAIL) ch ^= (int)(ch >= C::TCH && ((z / per) & 8u) != 0u);  // tail swizzle
    ch = min(ch, C::CH - 1);
    return (unsigned)row * row_bytes + (unsigned)ch * 16u;
  }

  // byte offsets (relative to the tile's first key row) for full tiles.  Computed at the start
  // of every work item from an opaque copy of the lane index, so that the compiler cannot hoist
  // them out of the item loop: held for the whole launch they would be live across every
  // kind of item and push the kernel into spilling.
  static __device__ __forceinline__ void init(unsigned (&off)[PER_WAVE], int wave, int lane, unsigned row_bytes) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < KPW; ++i) off[i] = lane_offset<true>(slot(wave, i, C::K_LOADS), ln, 0, row_bytes);
#pragma unroll
    for (int i = 0; i < VPW; ++i) off[KPW + i] = lane_offset<false>(slot(wave, i, C::V_LOADS), ln, 0, row_bytes);
  }

  // Where a tile's rows come from (wave-uniform): the byte addresses of its first key row in K
  // and V (this K/V head) and the bytes from there to the end of the sequence's last key row.
  // advance() steps to the next tile.
  struct Src {
    const unsigned char* kp;
    const unsigned char* vp;
    long long extent;
    __device__ __forceinline__ void advance(unsigned row_bytes) {
      const unsigned step = (unsigned)C::BN * row_bytes;
      kp += step;
      vp += step;
      extent -= step;
    }
  };
  static __device__ __forceinline__ Src src(const __bf16* __restrict__ k, const __bf16* __restrict__ v, int key0,
                                            int key_end, int head, int n_heads, unsigned row_bytes) {
    const size_t base = ((size_t)key0 * n_heads + head) * C::D;
    return Src{reinterpret_cast<const unsigned char*>(k + base), reinterpret_cast<const unsigned char*>(v + base),
               (long long)(key_end - key0 - 1) * row_bytes + C::D * 2};
  }

  // Enqueue the tile whose rows are keys [key0 - lead, key0 - lead + BN) of `sr` (based at
  // key0): rows before key0 (LEAD, the first tile of a sequence whose length is not a
  // multiple of BN) repeat key0.  The loads go through buffer resources based at key0 and
  // bounded by the last key row of the sequence, so a lane reads at most that far (an offset
  // past it would read zeros, never memory outside the sequence).
  // PARTS: which loads of the wave to issue (1: the K area's, 2: the V area's, 3: both).
  template <bool LEAD, int PARTS = 3>
  static __device__ __forceinline__ void issue(const Src& sr, lds_u8_t* buf, int lead, unsigned row_bytes,
                                               const unsigned (&off)[PER_WAVE], int wave, int lane) {
    const int n_rec = (int)(sr.extent < 0x7fffffffll ? sr.extent : 0x7fffffffll);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)sr.kp, (short)0, n_rec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)sr.vp, (short)0, n_rec, 0x00020000);
    // The first tile's offsets are recomputed here each time: an opaque copy of the lane
    // index keeps the compiler from hoisting their per-lane parts out of the item loop, where
    // they would take 12 registers for the whole launch (and be spilled).
    int ln = lane;
    if constexpr (LEAD) asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < ((PARTS & 1) ? KPW : 0); ++i) {
      const int s = slot(wave, i, C::K_LOADS);
      const unsigned o = LEAD ? lane_offset<true>(s, ln, lead, row_bytes) : off[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(buf + s * 1024), 16, o, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < ((PARTS & 2) ? VPW : 0); ++i) {
      const int s = slot(wave, i, C::V_LOADS);
      const unsigned o = LEAD ? lane_offset<false>(s, ln, lead, row_bytes) : off[KPW + i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(buf + C::K_BYTES + s * 1024), 16, o, 0, 0, 0);
    }
  }

  // The same for a tile given by its first key: the tile [key0 - lead, key0 - lead + BN).
  template <bool LEAD>
  static __device__ __forceinline__ void issue(const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                                               lds_u8_t* buf, int key0, int key_end, int lead, int head,
                                               int n_heads, unsigned row_bytes, const unsigned (&off)[PER_WAVE],
                                               int wave, int lane) {
    issue<LEAD>(src(k, v, key0, key_end, head, n_heads, row_bytes), buf, lead, row_bytes, off, wave, lane);
  }
};

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ unsigned cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// The two 16-bit element kinds.  Operands travel as raw 16-bit lanes (bf16x8_t, s16x4_t)
// and are reinterpreted for the f16 instructions.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// D += A.B, 16x16x32 (A, B: 8 elements per lane)
template <int E>
__device__ __forceinline__ f32x4_t mma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  if constexpr (E == kBF16) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}
// D = A.B, 16x16x16 on a zero accumulator (A, B: 4 elements per lane)
template <int E>
__device__ __forceinline__ f32x4_t mma16_zero(s16x4_t a, s16x4_t b) {
  if constexpr (E == kBF16) return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b),
                                                 f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}
// two floats rounded to nearest even, packed
template <int E>
__device__ __forceinline__ unsigned cvt_pk(float a, float b) {
  if constexpr (E == kBF16) return cvt_pk_bf16(a, b);
  else return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}
// 1.0 twice, in the element kind
template <int E>
constexpr unsigned kOnes2 = E == kBF16 ? 0x3f803f80u : 0x3c003c00u;
// The exponent window of the weights.  bf16 has float32's exponent range: the offset sits
// kHeadroom (16) above the reference max and is raised once a weight would reach 2.  f16
// has 5 exponent bits (normal numbers 2^-14 .. 65504): the offset is the reference max
// itself and is raised once a weight would reach 2^15, so weights stay normal-range
// (the largest at least 1) and never overflow.
template <int E>
constexpr float kHead = E == kBF16 ? kHeadroom : 0.0f;
template <int E>
constexpr float kRaise = E == kBF16 ? 1.0f : 15.0f;

// Operand fragments of one 32-key compute step, read from the LDS tile.
//   K (A operand of S^T = K.Q^T): lane (c, g) holds key kb0+kb*16+c, dims ks*32+8g..+8,
//     and for the 16-deep tail dims NK32*32+4g..+4.
//   V^T (A operand of O^T += V^T.P^T): two transposing reads of [key][d] give lane (c, g)
//     keys kb0+4g+0..3 and kb0+16+4g+0..3 of dim db*16+c, matching the P^T slots.
template <class C>
struct KFrag {
  bf16x8_t a[2][C::NK32];
  s16x4_t t[2];
};
template <class C>
struct VFrag {
  bf16x8_t a[C::NDB];
};

template <class C>
__device__ __forceinline__ void load_k(KFrag<C>& f, const __bf16* Ks, int kb0, int lane) {
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const __bf16* row = Ks + (kb0 + kb * 16 + c) * C::KSTR;
#pragma unroll
    for (int ks = 0; ks < C::NK32; ++ks) f.a[kb][ks] = *reinterpret_cast<const bf16x8_t*>(row + ks * 32 + 8 * g);
    if constexpr (C::TAIL) {
      // tail swizzle: rows with bit 3 set hold the two tail chunks swapped
      int t_off = (4 * g) ^ (c & 8);
      if (kb) asm volatile("" : "+v"(t_off));  // two separate 8-byte reads, not one paired read
      f.t[kb] = *reinterpret_cast<const s16x4_t*>(row + C::NK32 * 32 + t_off);
    }
  }
}

template <class C>
__device__ __forceinline__ void load_v(VFrag<C>& f, const __bf16* Vs, int kb0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const __bf16* v1 = Vs + (kb0 + 4 * g + (i >> 2)) * C::VSTR + 4 * (i & 3);
  const __bf16* v2 = v1 + 16 * C::VSTR;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(v1 + db * 16));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(v2 + db * 16));
    f.a[db] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

// S^T = K.Q^T for 32 keys: S[kb][qb][r] is key kb0+kb*16+4g+r of query row0+qb*16+c.
//
// head_dim 72 and 80 end the contraction with a 16-deep v_mfma_f32_16x16x16_bf16 (on
// gfx950 it costs about as much as a 32-deep step, but keeps K rows, Q operands and the
// DMA at 80 dims instead of 96).  Two hazards of mixing the shapes are kept out by
// construction: all the 16-deep steps are issued first, on zero accumulators (a 16x16x16
// waiting for an accumulator input can have it overwritten by a later transposing LDS
// read), and the 32-deep chains that take their results start only after a scheduling
// fence and 8 wait states (which the compiler does not insert between MFMAs of different
// shapes chained through the accumulator).
template <class C>
__device__ __forceinline__ void qk_32(f32x4_t (&S)[2][C::QB], const KFrag<C>& K, const bf16x8_t (&Q)[C::QB][C::NK32],
                                      const s16x4_t (&QT)[C::QB]) {
  if constexpr (C::TAIL) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
        S[kb][qb] = mma16_zero<C::E>(K.t[kb], QT[qb]);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7");
    __builtin_amdgcn_sched_barrier(0);
  } else {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) S[kb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ks = 0; ks < C::NK32; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
        S[kb][qb] = mma32<C::E>(K.a[kb][ks], Q[qb][ks], S[kb][qb]);
}

// Softmax weights and O^T += V^T.P^T for one 32-key step.
//
// The exponent offset of query row i is M_i = (reference max of c2*s over the keys seen)
// + kHeadroom, and the weights are p = exp2(c2*s - M_i), so the largest weight at the
// time M_i was set is 2^-kHeadroom.  FIRST (the first step of a work item) sets M from
// this step's exact row maxima.  Later steps keep M while every offset c2*s - M stays
// below 1 (weights below 2), which one in-lane max decides for the whole wavefront
// without any cross-lane reduction; otherwise (a row max rose by more than kHeadroom + 1)
// the rows concerned move M up to their new maximum and rescale their running output
// and sum before the weights are taken.  The final division by the row sum removes M from the
// result, so the choice of M only has to keep the weights in range.
//
// Only the FIRST step of an item can hold keys outside the sequence: its first `kinv`
// keys, which take no part in the max and get weight exactly 0 (also when c2 is 0).
template <class C, bool PREFETCH, bool ZERO = false>
__device__ __forceinline__ void weights_pv_32(const f32x4_t (&S)[2][C::QB], const __bf16* Vs, int kb0,
                                              f32x4_t (&O)[C::NACC][C::QB], int lane, KFrag<C>* knext,
                                              const __bf16* Ks, int kb_next);

// The offsets part: S becomes t = c2*s - M in place (FIRST sets M), with the rare raise.
template <class C, bool FIRST>
__device__ __forceinline__ void offsets_32(f32x4_t (&S)[2][C::QB], f32x4_t (&O)[C::NACC][C::QB],
                                           float (&negM)[C::QB], float c2, int kinv, int lane) {
  int g = lane >> 4;
  // (opaque in the first step: otherwise the key positions 16kb + 4g + r it compares are
  // hoisted out of the item loop as eight registers held for the whole launch)
  if constexpr (FIRST) asm volatile("" : "+v"(g));
  if constexpr (FIRST) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (kb * 16 + 4 * g + r < kinv)
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb) S[kb][qb][r] = -INFINITY;
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      float mx = fmaxf(fmaxf(fmaxf(S[0][qb][0], S[0][qb][1]), fmaxf(S[0][qb][2], S[0][qb][3])),
                       fmaxf(fmaxf(S[1][qb][0], S[1][qb][1]), fmaxf(S[1][qb][2], S[1][qb][3])));
      mx = max_4groups(mx);  // finite: at least one key of the step is in the sequence
      negM[qb] = -__builtin_fmaf(mx, c2, kHead<C::E>);
    }
  }
  // t = c2*s - M, in place
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float t = __builtin_fmaf(S[kb][qb][r], c2, negM[qb]);
        if constexpr (FIRST) t = (kb * 16 + 4 * g + r >= kinv) ? t : -INFINITY;
        S[kb][qb][r] = t;
      }
  if constexpr (!FIRST) {
    // one in-lane max over all of the lane's offsets decides for the whole wavefront
    float hi = S[0][0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
        for (int r = 0; r < 4; ++r) hi = fmaxf(hi, S[kb][qb][r]);
    if (__builtin_expect(__any(hi >= kRaise<C::E>), 0)) {  // rare: some row max rose past the window
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        float tm = fmaxf(fmaxf(fmaxf(S[0][qb][0], S[0][qb][1]), fmaxf(S[0][qb][2], S[0][qb][3])),
                         fmaxf(fmaxf(S[1][qb][0], S[1][qb][1]), fmaxf(S[1][qb][2], S[1][qb][3])));
        tm = max_4groups(tm);
        if (tm >= kRaise<C::E>) {  // the same decision in all four lanes of the row
          const float delta = tm + kHead<C::E>;
          negM[qb] -= delta;
          const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
          for (int db = 0; db < C::NACC; ++db) O[db][qb] *= alpha;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) S[kb][qb][r] -= delta;
        }
      }
    }
  }
}

template <class C, bool FIRST, bool PREFETCH = false, bool ZERO = false>
__device__ __forceinline__ void softmax_pv_32(f32x4_t (&S)[2][C::QB], const __bf16* Vs, int kb0,
                                              f32x4_t (&O)[C::NACC][C::QB], float (&negM)[C::QB], float c2, int kinv,
                                              int lane, KFrag<C>* knext = nullptr, const __bf16* Ks = nullptr,
                                              int kb_next = 0) {
  offsets_32<C, FIRST>(S, O, negM, c2, kinv, lane);
  weights_pv_32<C, PREFETCH, ZERO>(S, Vs, kb0, O, lane, knext, Ks, kb_next);
}

// The weights exp2(t) of one 32-key step (t = c2*s - M per element, -inf for no weight),
// rounded to the element kind.
template <class C>
__device__ __forceinline__ void weights_32(const f32x4_t (&S)[2][C::QB], u32x4_t (&W)[C::QB]) {
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      W[qb][j] = cvt_pk<C::E>(__builtin_amdgcn_exp2f(S[j >> 1][qb][(j & 1) * 2]),
                             __builtin_amdgcn_exp2f(S[j >> 1][qb][(j & 1) * 2 + 1]));
}

// O^T += V^T.P^T for one 32-key step, with the row sums alongside (an MFMA of the rounded
// weights against a block of ones), as one matrix burst at raised issue priority.
// ZERO: the first products of an item, on zero accumulators (O need not be initialised).
template <class C, bool ZERO = false>
__device__ __forceinline__ void pv_32(const VFrag<C>& V, const u32x4_t (&W)[C::QB], f32x4_t (&O)[C::NACC][C::QB]) {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
      O[db][qb] = mma32<C::E>(V.a[db], __builtin_bit_cast(bf16x8_t, W[qb]), ZERO ? zero : O[db][qb]);
  const u32x4_t ones = {kOnes2<C::E>, kOnes2<C::E>, kOnes2<C::E>, kOnes2<C::E>};
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
    O[C::NDB][qb] = mma32<C::E>(__builtin_bit_cast(bf16x8_t, ones), __builtin_bit_cast(bf16x8_t, W[qb]),
                                ZERO ? zero : O[C::NDB][qb]);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

// The weights of one 32-key step and O^T += V^T.P^T with the row sums alongside.
template <class C, bool PREFETCH, bool ZERO>
__device__ __forceinline__ void weights_pv_32(const f32x4_t (&S)[2][C::QB], const __bf16* Vs, int kb0,
                                              f32x4_t (&O)[C::NACC][C::QB], int lane, KFrag<C>* knext,
                                              const __bf16* Ks, int kb_next) {
  // The V^T reads are issued only now, after every score MFMA of the step has been
  // consumed: an LDS read may then reuse those MFMAs' operand registers safely, and its
  // latency still hides behind the exponentials.  (step_32_ev and step_32k_ev read them
  // before the score products instead; there the V^T registers stay live across those
  // products, so they are no in-flight MFMA's accumulators either.)
  VFrag<C> V;
  load_v<C>(V, Vs, kb0, lane);
  if constexpr (PREFETCH) load_k<C>(*knext, Ks, kb_next, lane);  // the next step's K, same tile
  u32x4_t W[C::QB];
  weights_32<C>(S, W);
  pv_32<C, ZERO>(V, W, O);
}

// One 32-key step [kb0, kb0 + 32) of the LDS tile: operand reads, both products, softmax.
// FIRST also means the first value products of the item (O is set, not accumulated).
template <class C, bool FIRST>
__device__ __forceinline__ void step_32(const __bf16* Ks, const __bf16* Vs, int kb0, int kinv,
                                        const bf16x8_t (&Q)[C::QB][C::NK32], const s16x4_t (&QT)[C::QB],
                                        f32x4_t (&O)[C::NACC][C::QB], float (&negM)[C::QB], float c2, int lane) {
  f32x4_t S[2][C::QB];
  {
    KFrag<C> kf;
    load_k<C>(kf, Ks, kb0, lane);
    // Matrix bursts run at raised issue priority: while this wavefront feeds the matrix
    // pipe, the other wavefront on the SIMD fills the vector slots, instead of both
    // contending for the pipe in the same phase.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    qk_32<C>(S, kf, Q, QT);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  }
  softmax_pv_32<C, FIRST, false, FIRST>(S, Vs, kb0, O, negM, c2, kinv, lane);
}

// One 32-key step whose V^T operands are read together with its K operands, before the
// score products (for items with one 16-query block per wavefront, whose registers leave
// room for both): the V^T read latency then hides behind the products and the offsets.
template <class C, bool FIRST>
__device__ __forceinline__ void step_32_ev(const __bf16* Ks, const __bf16* Vs, int kb0, int kinv,
                                           const bf16x8_t (&Q)[C::QB][C::NK32], const s16x4_t (&QT)[C::QB],
                                           f32x4_t (&O)[C::NACC][C::QB], float (&negM)[C::QB], float c2, int lane) {
  f32x4_t S[2][C::QB];
  KFrag<C> kf;
  load_k<C>(kf, Ks, kb0, lane);
  VFrag<C> V;
  load_v<C>(V, Vs, kb0, lane);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
  qk_32<C>(S, kf, Q, QT);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  offsets_32<C, FIRST>(S, O, negM, c2, kinv, lane);
  u32x4_t W[C::QB];
  weights_32<C>(S, W);
  pv_32<C>(V, W, O);
}

// A full step whose K fragments were loaded earlier; PREFETCH also loads the next step's
// (in the same tile) while the exponentials run.
template <class C, bool PREFETCH>
__device__ __forceinline__ void step_32k(const KFrag<C>& kf, KFrag<C>& knext, const __bf16* Ks, const __bf16* Vs,
                                         int kb0, const bf16x8_t (&Q)[C::QB][C::NK32], const s16x4_t (&QT)[C::QB],
                                         f32x4_t (&O)[C::NACC][C::QB], float (&negM)[C::QB], float c2, int lane) {
  f32x4_t S[2][C::QB];
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
  qk_32<C>(S, kf, Q, QT);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  softmax_pv_32<C, false, PREFETCH>(S, Vs, kb0, O, negM, c2, 0, lane, &knext, Ks, kb0 + C::KSUB);
}

// step_32k with the V^T operands read at the start of the step, as in step_32_ev, for up to
// kEarlyVMaxQB 16-query blocks per wavefront (with four, the V^T fragments held across the
// score products no longer fit the registers); the next step's K is read once the scores
// are consumed.
constexpr int kEarlyVMaxQB = 2;
template <class C, bool PREFETCH>
__device__ __forceinline__ void step_32k_ev(const KFrag<C>& kf, KFrag<C>& knext, const __bf16* Ks, const __bf16* Vs,
                                            int kb0, const bf16x8_t (&Q)[C::QB][C::NK32], const s16x4_t (&QT)[C::QB],
                                            f32x4_t (&O)[C::NACC][C::QB], float (&negM)[C::QB], float c2, int lane) {
  VFrag<C> V;
  load_v<C>(V, Vs, kb0, lane);
  f32x4_t S[2][C::QB];
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
  qk_32<C>(S, kf, Q, QT);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  offsets_32<C, false>(S, O, negM, c2, 0, lane);
  if constexpr (PREFETCH) load_k<C>(knext, Ks, kb0 + C::KSUB, lane);
  u32x4_t W[C::QB];
  weights_32<C>(S, W);
  pv_32<C>(V, W, O);
}

// Q^T operands: lane (c, g) holds row row0+qb*16+c (rows past qend repeat row qend-1),
// dims ks*32+8g..+8, and for the 16-deep tail dims NK32*32+4g..+4 (zero past D).  A
// negative scale is folded into Q by flipping its sign bits.
template <class C>
__device__ __forceinline__ void load_q16(bf16x8_t (&Q)[C::QB][C::NK32], s16x4_t (&QT)[C::QB],
                                         const __bf16* __restrict__ q, int row0, int qend, int head, int n_heads,
                                         int negate, int lane) {
  const int g = lane >> 4, c = lane & 15;
  const unsigned nmask = negate ? 0x80008000u : 0u;  // wave-uniform: one xor per register, no select
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int row = min(row0 + qb * 16 + c, qend - 1);
    const __bf16* qrow = q + ((size_t)row * n_heads + head) * C::D;
#pragma unroll
    for (int ks = 0; ks < C::NK32; ++ks) {
      u32x4_t w = ld16(qrow + ks * 32 + 8 * g);
      w ^= nmask;
      Q[qb][ks] = __builtin_bit_cast(bf16x8_t, w);
    }
    u32x2_t t = {0u, 0u};
    if (C::TAIL && C::NK32 * 32 + 4 * g < C::D) t = *reinterpret_cast<const u32x2_t*>(qrow + C::NK32 * 32 + 4 * g);
    t ^= nmask;
    QT[qb] = __builtin_bit_cast(s16x4_t, t);
  }
}

// Epilogue: O / l for the rows of this wavefront that lie in the sequence, rounded to the
// output kind.
template <class C>
__device__ __forceinline__ void store_o16(void* __restrict__ o, const f32x4_t (&O)[C::NACC][C::QB], int row0,
                                          int qend, int head, int n_heads, int lane) {
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const float inv = 1.0f / O[C::NDB][qb][0];
    const int row = row0 + qb * 16 + c;
    if (row < qend) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int d0 = db * 16 + 4 * g;
        if (d0 < C::D) {
          const f32x4_t x = O[db][qb];
          const size_t at = ((size_t)row * n_heads + head) * C::D + d0;
          if constexpr (C::OF32)
            *reinterpret_cast<f32x4_t*>(static_cast<float*>(o) + at) = x * inv;
          else
            *reinterpret_cast<u32x2_t*>(static_cast<__bf16*>(o) + at) =
                u32x2_t{cvt_pk<C::E>(x[0] * inv, x[1] * inv), cvt_pk<C::E>(x[2] * inv, x[3] * inv)};
        }
      }
    }
  }
}

// One work item (sequence, head, BM queries from q0) for the whole workgroup.  The K/V
// stage buffers and the DMA offsets depend only on head_dim and the tile shape, so work
// items of different query-block sizes (C::QB) share them.
//
// The keys [a, b) are covered by ntiles tiles of BN keys that END at b: tile 0 starts
// `pad` = ntiles*BN - (b - a) keys before a, its first pad rows repeat key a in LDS and
// are masked in the first step, and every later step is a full one.
template <class C>
__device__ __forceinline__ void run_item(const Item& item, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                         const __bf16* __restrict__ v, void* __restrict__ o, int n_heads,
                                         int n_kv_heads, int kv_group, float c2, int negate, lds_u8_t* stage,
                                         unsigned row_bytes, int wave, int lane) {
  unsigned dma_off[Dma<C>::PER_WAVE];  // computed per item (see Dma::init), not held across items
  Dma<C>::init(dma_off, wave, lane, row_bytes);
  const int kv_head = item.head / kv_group;  // K/V rows are [T, n_kv_heads, D]
  const int qend = min(item.q0 + C::BM, item.b);
  const int row0 = item.q0 + wave * C::NQ;
  const int ntiles = ceil_div(item.b - item.a, C::BN);
  const int pad = ntiles * C::BN - (item.b - item.a);  // 0 <= pad < BN
  const int kstart = item.a - pad;                      // key of tile 0's row 0 (may precede a)

  __syncthreads();  // the previous item is done with both stage buffers
  if (pad > 0)
    Dma<C>::template issue<true>(k, v, stage, item.a, item.b, pad, kv_head, n_kv_heads, row_bytes, dma_off, wave, lane);
  else
    Dma<C>::template issue<false>(k, v, stage, item.a, item.b, 0, kv_head, n_kv_heads, row_bytes, dma_off, wave, lane);
  // tile t >= 1 starts at key kstart + t*BN; sr follows the next tile to issue
  typename Dma<C>::Src sr = Dma<C>::src(k, v, kstart + C::BN, item.b, kv_head, n_kv_heads, row_bytes);
  auto issue_next = [&](int t) {  // tile t (>= 1) into buffer t & 1
    Dma<C>::template issue<false>(sr, stage + (t & 1) * C::STAGE_BYTES, 0, row_bytes, dma_off, wave, lane);
    sr.advance(row_bytes);
  };

  if (row0 >= qend) {
    // No row of this wavefront lies in the sequence (the last, partial item of an image): it
    // keeps only its share of the DMA and the barriers, so that the SIMD time goes to the
    // other workgroup on the CU.  The same barriers as below, one per tile.
    for (int t = 0; t < ntiles; ++t) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (t + 1 < ntiles) issue_next(t + 1);
    }
    return;
  }

  bf16x8_t Q[C::QB][C::NK32];
  s16x4_t QT[C::QB];
  load_q16<C>(Q, QT, q, row0, qend, item.head, n_heads, negate, lane);

  f32x4_t O[C::NACC][C::QB];  // set by the first step's value products
  float negM[C::QB];

  // tile 0: the first step with a key in the sequence sets the exponent offsets
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA of tile 0 has landed
  __syncthreads();                                   // every wave's has
  if (ntiles > 1) issue_next(1);
  const int s0 = pad / C::KSUB;
  {
    const __bf16* Ks = (const __bf16*)(stage);
    const __bf16* Vs = (const __bf16*)(stage + C::K_BYTES);
    step_32<C, true>(Ks, Vs, s0 * C::KSUB, pad - s0 * C::KSUB, Q, QT, O, negM, c2, lane);
  }
  static_assert(C::NSUB == 2, "tile loop below runs two 32-key steps per tile");
  if (s0 == 0) {  // tile 0's second step
    const __bf16* Ks = (const __bf16*)(stage);
    const __bf16* Vs = (const __bf16*)(stage + C::K_BYTES);
    step_32<C, false>(Ks, Vs, C::KSUB, 0, Q, QT, O, negM, c2, lane);
  }
  // every later tile: two full steps; the second step's K operands are read while the first
  // step's exponentials run
  // The next tile's loads go out in two halves, the K area's after the barrier and the V
  // area's between the two steps, so that the workgroups of a CU do not all queue their whole
  // tile at the vector-memory unit at once.
  for (int t = 1; t < ntiles; ++t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA of tile t has landed
    __syncthreads();  // every wave's has; buffer (t+1)&1 is no longer read
    const bool more = t + 1 < ntiles;
    lds_u8_t* nbuf = stage + ((t + 1) & 1) * C::STAGE_BYTES;
    if (more) Dma<C>::template issue<false, 1>(sr, nbuf, 0, row_bytes, dma_off, wave, lane);
    const lds_u8_t* buf = stage + (t & 1) * C::STAGE_BYTES;
    const __bf16* Ks = (const __bf16*)(buf);
    const __bf16* Vs = (const __bf16*)(buf + C::K_BYTES);
    KFrag<C> k0, k1;
    load_k<C>(k0, Ks, 0, lane);
    if constexpr (C::QB <= kEarlyVMaxQB) {
      step_32k_ev<C, true>(k0, k1, Ks, Vs, 0, Q, QT, O, negM, c2, lane);
      if (more) Dma<C>::template issue<false, 2>(sr, nbuf, 0, row_bytes, dma_off, wave, lane);
      step_32k_ev<C, false>(k1, k0, Ks, Vs, C::KSUB, Q, QT, O, negM, c2, lane);
    } else {
      step_32k<C, true>(k0, k1, Ks, Vs, 0, Q, QT, O, negM, c2, lane);
      if (more) Dma<C>::template issue<false, 2>(sr, nbuf, 0, row_bytes, dma_off, wave, lane);
      step_32k<C, false>(k1, k0, Ks, Vs, C::KSUB, Q, QT, O, negM, c2, lane);
    }
    if (more) sr.advance(row_bytes);
  }

  store_o16<C>(o, O, row0, qend, item.head, n_heads, lane);
}

typedef __attribute__((address_space(3))) float lds_f32_t;

// A work item of the short-image plan with the keys split inside the workgroup: the item is
// C::NW/2 query blocks of C::NQ rows, and wavefronts 2p and 2p+1 both hold block p, each
// taking one of the two 32-key steps of every 64-key tile (wavefront 2p+1 the second).  The
// K/V tiles are staged once for all four wavefronts, double-buffered, as in run_item.  Each
// wavefront keeps its own exponent offset, output and row sum over its half of the keys; at
// the end the odd wavefront of a pair leaves them in LDS and the even one merges them in a
// fixed order, scaling each half by 2^(its offset - the larger offset) ("inferencelayer 0.2.1
// src/vision_gpu.rs", vis_attn_coop_src doc, "The obstacle, and the way round it": the same
// rescale as the online update), and stores the rows.  Half the serial steps per item and
// twice the items of run_item<C>: for a short image whose items would otherwise fill at most
// half of the grid, where each item's chain of dependent steps sets the time.
template <class C>
__device__ __forceinline__ void run_item_split(const Item& item, const __bf16* __restrict__ q,
                                               const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                                               void* __restrict__ o, int n_heads, int n_kv_heads, int kv_group,
                                               float c2, int negate, lds_u8_t* stage, unsigned row_bytes,
                                               int wave, int lane_in) {
  // an opaque lane index: the per-lane LDS addresses of this kind of item are computed in it,
  // not hoisted out of the item loop beside those of the large items
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  unsigned dma_off[Dma<C>::PER_WAVE];  // computed per item (see Dma::init), not held across items
  Dma<C>::init(dma_off, wave, lane, row_bytes);
  static_assert(C::NSUB == 2 && C::NW % 2 == 0, "two 32-key steps per tile, wavefronts in pairs");
  static_assert(C::QB == 1, "the merge below hands over one 16-query block per wavefront");
  constexpr int BM = C::NW / 2 * C::NQ;  // queries per item
  constexpr int NV = C::NACC * 4 + 1;    // floats per lane handed over: output, row sum, offset
  static_assert(C::NW / 2 * NV * 64 * 4 <= 2 * C::STAGE_BYTES, "merge area fits the stage buffers");
  const int kv_head = item.head / kv_group;
  const int qend = min(item.q0 + BM, item.b);
  const int half = wave & 1;                        // which 32 keys of each tile
  const int row0 = item.q0 + (wave >> 1) * C::NQ;   // this pair's query block
  const int ntiles = ceil_div(item.b - item.a, C::BN);
  const int pad = ntiles * C::BN - (item.b - item.a);  // 0 <= pad < BN
  const int kstart = item.a - pad;
  // tiles t >= 1 are issued in order; sr follows the next one
  typename Dma<C>::Src sr = Dma<C>::src(k, v, kstart + C::BN, item.b, kv_head, n_kv_heads, row_bytes);
  auto issue_tile = [&](int t) {  // tile t >= 1 into buffer t & 1
    Dma<C>::template issue<false>(sr, stage + (t & 1) * C::STAGE_BYTES, 0, row_bytes, dma_off, wave, lane);
    sr.advance(row_bytes);
  };

  __syncthreads();  // the previous item is done with the stage buffers (and the merge area)
  if (pad > 0)
    Dma<C>::template issue<true>(k, v, stage, item.a, item.b, pad, kv_head, n_kv_heads, row_bytes, dma_off, wave, lane);
  else
    Dma<C>::template issue<false>(k, v, stage, item.a, item.b, 0, kv_head, n_kv_heads, row_bytes, dma_off, wave, lane);

  bf16x8_t Q[C::QB][C::NK32];
  s16x4_t QT[C::QB];
  load_q16<C>(Q, QT, q, row0, qend, item.head, n_heads, negate, lane);

  f32x4_t O[C::NACC][C::QB];
  float negM[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    negM[qb] = INFINITY;  // no key seen yet (the merge weighs such a half by 0)
#pragma unroll
    for (int db = 0; db < C::NACC; ++db) O[db][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int kb0 = half * C::KSUB;  // this wavefront's step inside every tile
  const int kinv = pad - kb0;      // leading keys of that step in tile 0 that precede the image
  bool started = false;            // uniform: the wavefront's first step with a key has run

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA of tile 0 has landed
  __syncthreads();                                   // every wave's has
  if (ntiles > 1) issue_tile(1);
  if (kinv < C::KSUB) {  // tile 0's step holds at least one key of the image
    step_32_ev<C, true>((const __bf16*)stage, (const __bf16*)(stage + C::K_BYTES), kb0, max(kinv, 0), Q, QT, O, negM,
                     c2, lane);
    started = true;
  }
  for (int t = 1; t < ntiles; ++t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA of tile t has landed
    __syncthreads();  // every wave's has; buffer (t+1)&1 is no longer read
    if (t + 1 < ntiles) issue_tile(t + 1);
    const lds_u8_t* buf = stage + (t & 1) * C::STAGE_BYTES;
    if (started) {
      step_32_ev<C, false>((const __bf16*)buf, (const __bf16*)(buf + C::K_BYTES), kb0, 0, Q, QT, O, negM, c2, lane);
    } else {
      step_32_ev<C, true>((const __bf16*)buf, (const __bf16*)(buf + C::K_BYTES), kb0, 0, Q, QT, O, negM, c2, lane);
      started = true;
    }
  }

  // merge the pair's halves: lane-major so that the LDS accesses are conflict free
  __syncthreads();  // every wavefront is done reading the last tile
  lds_f32_t* area = (lds_f32_t*)stage + (wave >> 1) * (NV * 64) + lane;
  if (half) {
#pragma unroll
    for (int db = 0; db < C::NACC; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) area[(db * 4 + r) * 64] = O[db][0][r];
    area[(NV - 1) * 64] = negM[0];
  }
  __syncthreads();
  if (!half) {
    const float other = area[(NV - 1) * 64];
    const float nm = fminf(negM[0], other);  // the larger of the two offsets, negated
    const float f0 = __builtin_amdgcn_exp2f(nm - negM[0]), f1 = __builtin_amdgcn_exp2f(nm - other);
#pragma unroll
    for (int db = 0; db < C::NACC; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) O[db][0][r] = O[db][0][r] * f0 + area[(db * 4 + r) * 64] * f1;
    store_o16<C>(o, O, row0, qend, item.head, n_heads, lane);
  }
}

// ----------------------------------------------------------------------------
// Masked attention (aligned causal and/or a key window; mask rules at key_visible).
//
// An item's keys narrow to [klo, khi), the keys some of its queries see
// (mask_key_range), covered as in run_item by tiles that end at khi.  For its own query
// rows each wavefront finds the run of tiles whose every key all of its rows see; that
// run takes the unmasked tile body, and the tiles before and after it go 32 keys at a
// time: a step that no row sees is skipped, any other goes through step_32_masked, which
// applies per row a lower and an upper key bound.  A row may have no offset yet (negM =
// +inf: none of its keys so far was visible); such a row takes its offset from the first
// step in which it sees a key, exactly as the first step of an unmasked item does.
// ----------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ void step_32_masked(const __bf16* Ks, const __bf16* Vs, int kb0, int key_s,
                                               const bf16x8_t (&Q)[C::QB][C::NK32], const s16x4_t (&QT)[C::QB],
                                               f32x4_t (&O)[C::NACC][C::QB], float (&negM)[C::QB], float c2,
                                               int lane, int row0, int qend, int a, int causal, int window,
                                               bool use_lo, bool use_hi) {
  const int g = lane >> 4, c = lane & 15;
  f32x4_t S[2][C::QB];
  {
    KFrag<C> kf;
    load_k<C>(kf, Ks, kb0, lane);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    qk_32<C>(S, kf, Q, QT);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Element (kb, r) of the lane holds key j = key_s + 4g + u with u = kb*16 + r, and every
  // rule bounds u for the row: j >= a iff u >= a - key_s - 4g; with d = i - key_s - 4g,
  // j <= i iff u <= d, and |i - j| < window iff d - (window - 1) <= u <= d + (window - 1)
  // (saturated: the window may exceed any row difference).  So each element costs a
  // comparison with a constant against the row's bound, made opaque so that it is computed
  // here once per row, not rewritten per element.  use_lo / use_hi (uniform) say whether a
  // lower / upper bound can cut any key of the step for any row of the wavefront.
  float tm[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int d = min(row0 + qb * 16 + c, qend - 1) - key_s - 4 * g;  // rows past the item act as its last row
    if (use_lo) {
      int lo = a - key_s - 4 * g, t;
      if (window > 0) lo = max(lo, __builtin_sub_overflow(d, window - 1, &t) ? (int)0x80000000 : t);
      asm volatile("" : "+v"(lo));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kb * 16 + r < lo) S[kb][qb][r] = -INFINITY;
    }
    if (use_hi) {
      int hi = causal ? d : 0x7fffffff, t;
      if (window > 0) hi = min(hi, __builtin_add_overflow(d, window - 1, &t) ? 0x7fffffff : t);
      asm volatile("" : "+v"(hi));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kb * 16 + r > hi) S[kb][qb][r] = -INFINITY;
    }
    float x = S[0][qb][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) x = fmaxf(x, S[kb][qb][r]);
    tm[qb] = max_4groups(x);  // the same in the four lanes of the row
  }
  // A row that sees a key here and whose max leaves the exponent window (always the case
  // for a row without an offset, negM = +inf) moves its offset to this max and rescales its
  // running output and row sum (by 0 for a row without an offset, whose are 0).  Rare after
  // the first visible step, so one vote skips it for the whole wavefront.
  bool need[C::QB], any = false;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    need[qb] = tm[qb] != -INFINITY && __builtin_fmaf(tm[qb], c2, negM[qb]) >= kRaise<C::E>;
    any = any || need[qb];
  }
  if (__any(any)) {
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      if (need[qb]) {
        const float nm = -__builtin_fmaf(tm[qb], c2, kHead<C::E>);
        const float alpha = __builtin_amdgcn_exp2f(nm - negM[qb]);
#pragma unroll
        for (int db = 0; db < C::NACC; ++db) O[db][qb] *= alpha;
        negM[qb] = nm;
      }
    }
  }
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = S[kb][qb][r];
        S[kb][qb][r] = x == -INFINITY ? -INFINITY : __builtin_fmaf(x, c2, negM[qb]);
      }
  weights_pv_32<C, false>(S, Vs, kb0, O, lane, nullptr, nullptr, 0);
}

template <class C>
__device__ __forceinline__ void run_item_masked(const Item& item, const __bf16* __restrict__ q,
                                                const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                                                void* __restrict__ o, int n_heads, int n_kv_heads, int kv_group,
                                                float c2, int negate, int causal, int window, lds_u8_t* stage,
                                                unsigned row_bytes, int wave, int lane) {
  unsigned dma_off[Dma<C>::PER_WAVE];  // computed per item (see Dma::init), not held across items
  Dma<C>::init(dma_off, wave, lane, row_bytes);
  const int kv_head = item.head / kv_group;
  const int qend = min(item.q0 + C::BM, item.b);
  const int row0 = item.q0 + wave * C::NQ;
  int klo = item.a, khi = item.b;
  mask_key_range(klo, khi, item.q0, qend, causal, window);
  const int ntiles = ceil_div(khi - klo, C::BN);
  const int pad = ntiles * C::BN - (khi - klo);  // 0 <= pad < BN
  const int kstart = klo - pad;                   // key of tile 0's row 0
  // this wavefront's query rows, clamped into the item like the Q rows
  const int wlo = min(row0, qend - 1), whi = min(row0 + C::NQ - 1, qend - 1);
  const bool idle = row0 >= qend;  // no row of the wavefront lies in the sequence

  __syncthreads();  // the previous item is done with both stage buffers
  if (pad > 0)
    Dma<C>::template issue<true>(k, v, stage, klo, khi, pad, kv_head, n_kv_heads, row_bytes, dma_off, wave, lane);
  else
    Dma<C>::template issue<false>(k, v, stage, klo, khi, 0, kv_head, n_kv_heads, row_bytes, dma_off, wave, lane);

  bf16x8_t Q[C::QB][C::NK32];
  s16x4_t QT[C::QB];
  load_q16<C>(Q, QT, q, row0, qend, item.head, n_heads, negate, lane);

  f32x4_t O[C::NACC][C::QB];
  float negM[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    negM[qb] = INFINITY;  // no offset yet
#pragma unroll
    for (int db = 0; db < C::NACC; ++db) O[db][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  bool ready = false;  // every row of the wavefront has an offset

  // The tiles whose 64 keys every row of this wavefront sees form one run [f0, f1): the
  // keys visible to all of the rows [wlo, whi] are [ka, kz] below.  Before and after the
  // run, each 32-key step is skipped when no row sees a key of it and otherwise masked
  // element by element; the run itself takes the unmasked tile body (after one masked
  // tile if some row still has no offset).  The three phases are separate loops, each
  // with one barrier per tile like every other wavefront's, so that the register
  // allocation of the unmasked body is not shared with the masked steps.
  int ka = item.a, kz = item.b - 1;
  if (causal) kz = min(kz, wlo);
  if (window > 0) {
    ka = max(ka, whi - window + 1);
    if (window - 1 <= kz - wlo) kz = wlo + window - 1;  // kz = min(kz, wlo + window - 1)
  }
  int f0 = ceil_div(ka - kstart, C::BN);       // ka >= klo >= kstart
  int f1 = min(ntiles, (kz - kstart + 1) / C::BN);  // kz >= wlo >= kstart
  if (idle || f1 <= f0) f0 = f1 = ntiles;      // no run: every tile is masked (or skipped)

  // one tile: wait for its DMA, let every wave pass the barrier, start the next tile's DMA
  auto begin_tile = [&](int t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA of tile t has landed
    __syncthreads();  // every wave's has; buffer (t+1)&1 is no longer read
    if (t + 1 < ntiles)
      Dma<C>::template issue<false>(k, v, stage + ((t + 1) & 1) * C::STAGE_BYTES, kstart + (t + 1) * C::BN, khi, 0,
                                    kv_head, n_kv_heads, row_bytes, dma_off, wave, lane);
  };
  // the masked steps of tile t
  auto masked_tile = [&](int t) {
    if (idle) return;
    const lds_u8_t* buf = stage + (t & 1) * C::STAGE_BYTES;
    const __bf16* Ks = (const __bf16*)(buf);
    const __bf16* Vs = (const __bf16*)(buf + C::K_BYTES);
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) {
      const int s = kstart + t * C::BN + sub * C::KSUB, e = s + C::KSUB - 1;  // the step's keys [s, e]
      const bool none = e < item.a || (causal && s > whi) || (window > 0 && (wlo - e >= window || s - whi >= window));
      if (none) continue;
      step_32_masked<C>(Ks, Vs, sub * C::KSUB, s, Q, QT, O, negM, c2, lane, row0, qend, item.a, causal, window,
                        s < ka, e > kz);
    }
    bool set = true;
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) set = set && negM[qb] != INFINITY;
    ready = __all(set);
  };

  int t = 0;
  for (; t < f0; ++t) {
    begin_tile(t);
    masked_tile(t);
  }
  if (t < f1 && !ready) {  // the run's first tile sets the offsets of the rows still without one
    begin_tile(t);
    masked_tile(t);
    ++t;
  }
  for (; t < f1; ++t) {  // every row has an offset and sees every key of the tile
    begin_tile(t);
    const lds_u8_t* buf = stage + (t & 1) * C::STAGE_BYTES;
    const __bf16* Ks = (const __bf16*)(buf);
    const __bf16* Vs = (const __bf16*)(buf + C::K_BYTES);
    KFrag<C> k0, k1;
    load_k<C>(k0, Ks, 0, lane);
    if constexpr (C::QB <= kEarlyVMaxQB) {
      step_32k_ev<C, true>(k0, k1, Ks, Vs, 0, Q, QT, O, negM, c2, lane);
      step_32k_ev<C, false>(k1, k0, Ks, Vs, C::KSUB, Q, QT, O, negM, c2, lane);
    } else {
      step_32k<C, true>(k0, k1, Ks, Vs, 0, Q, QT, O, negM, c2, lane);
      step_32k<C, false>(k1, k0, Ks, Vs, C::KSUB, Q, QT, O, negM, c2, lane);
    }
  }
  for (; t < ntiles; ++t) {
    begin_tile(t);
    masked_tile(t);
  }
  store_o16<C>(o, O, row0, qend, item.head, n_heads, lane);
}

// The bf16 kernel.  CA and CB differ only in the queries per wavefront (CA::QB >= CB::QB).
// The launch works with CA's large query blocks unless they would leave most of the grid
// idle (a short single image), in which case it re-plans with CB's small blocks: more
// items, so more of the machine works, each item over the same keys.
template <class CA, class CB, bool MASK>
__global__ __launch_bounds__(CA::NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    void* __restrict__ o, const int32_t* __restrict__ cu, int n_seqs, int n_heads, int n_kv_heads, float c2,
    int negate, int causal, int window) {
  static_assert(CA::D == CB::D && CA::NW == CB::NW && CA::BN == CB::BN && CA::STAGE_BYTES == CB::STAGE_BYTES &&
                    CA::E == CB::E && CA::OF32 == CB::OF32,
                "the two query-block sizes share the staging layout and the element kinds");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  PlanLds& plan = *reinterpret_cast<PlanLds*>(smem);
  lds_u8_t* stage = (lds_u8_t*)smem + ((sizeof(PlanLds) + 15) / 16) * 16;

  const int G = gridDim.x;
  // Every decision below depends only on cu_seqlens, so every workgroup takes the same.
  // Short images, whose large items would fill less than half of the grid, take CB's small
  // query blocks; unmasked, when even twice as many of those items fit in one round of the
  // grid, each is split further between wavefront pairs by keys (run_item_split).
  int n_items;
  bool small, split = false;
  if (n_seqs == 1) {
    // One image: the same plan in closed form, without the ordering and the scans.
    const int a = cu[0], b = cu[1];
    auto count = [&](int bm_) { return ceil_div(b - a, bm_) * n_heads; };
    n_items = count(CA::BM);
    small = 2 * n_items < G;
    if (small) {
      n_items = count(CB::BM);
      if constexpr (!MASK) {
        split = 2 * n_items <= G;
        if (split) n_items = count(CB::BM / 2);
      }
    }
    if (threadIdx.x == 0) {
      plan.cu[0] = a;
      plan.cu[1] = b;
      plan.order[0] = 0;
      plan.prefix[0] = 0;
      plan.prefix[1] = n_items;
    }
    __syncthreads();
  } else {
    plan_load<CA::NT>(plan, cu, n_seqs);
    n_items = plan_items<CA::NT>(plan, n_seqs, n_heads, CA::BM);
    small = 2 * n_items < G;
    if (small) {
      __syncthreads();  // everyone has read the item count
      n_items = plan_items<CA::NT>(plan, n_seqs, n_heads, CB::BM);
      if constexpr (!MASK) {
        split = 2 * n_items <= G;
        if (split) {
          __syncthreads();
          n_items = plan_items<CA::NT>(plan, n_seqs, n_heads, CB::BM / 2);
        }
      }
    }
  }
  const int bm = split ? CB::BM / 2 : (small ? CB::BM : CA::BM);
  int levels = 0;  // a causal launch lists its items by decreasing cost when it can
  if constexpr (MASK) {
    if (causal) levels = build_levels<CA::NT>(plan, n_seqs, n_heads, bm);
  }
  // the wave index and every item field are uniform across a wavefront: keep them in scalar
  // registers, so that the per-tile DMA issue is scalar address arithmetic
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int xcd = blockIdx.x & 7, xj = blockIdx.x >> 3;  // workgroups go to the 8 XCDs round-robin
  const unsigned row_bytes = (unsigned)n_kv_heads * CA::D * 2u;  // one K/V row
  const int kv_group = n_heads / n_kv_heads;                       // query heads per K/V head

  // Items in longest-first order are dealt out in rounds ("tiers") of R = G/2 items, one per
  // CU.  The hardware places workgroups b and b + G/2 on one CU, and the older of the two
  // (b < G/2) issues first: paired, it runs about 1.45 times as fast as the younger one.  So
  // even tiers go to the older halves of the CU pairs and odd tiers to the younger halves, with
  // the direction reversed every second tier (tier 2 pairs the largest items of the older
  // halves' first tier with the smallest of their second): the older halves get the larger
  // items, and the CU totals stay even.  Within a tier of m items, XCD x takes the contiguous
  // run [x*m/8, (x+1)*m/8) (items of one sequence and head share K/V in that XCD's L2), so a
  // last, partial tier still spreads over all XCDs.  Items that fit in one round of the
  // grid (short images), and a grid that is not a multiple of 16, are dealt in rounds of the
  // whole grid instead, alternating direction.
  const bool tiered = (G & 15) == 0 && n_items > G;
  const int R = tiered ? G >> 1 : G;                      // items per tier
  const int half = tiered ? (blockIdx.x >= R ? 1 : 0) : 0;  // the younger half of a CU pair
  const int xk = tiered ? (blockIdx.x - half * R) >> 3 : xj;  // position inside the XCD's run
  for (int tier = half;; tier += tiered ? 2 : 1) {
    const int base = tier * R;
    if (base >= n_items) break;
    const int m = min(R, n_items - base);
    const int lo = (xcd * m) >> 3, cnt = (((xcd + 1) * m) >> 3) - lo;
    if (xk >= cnt) break;  // only the last tier can leave a workgroup without an item
    const int kk = lo + xk;
    const bool rev = tiered ? ((tier >> 1) & 1) : (tier & 1);
    const int it = base + (rev ? m - 1 - kk : kk);
    Item item = levels ? map_item_levels(plan, levels, it, bm, n_heads) : map_item(plan, n_seqs, it, bm);
    item.a = __builtin_amdgcn_readfirstlane(item.a);
    item.b = __builtin_amdgcn_readfirstlane(item.b);
    item.head = __builtin_amdgcn_readfirstlane(item.head);
    item.q0 = __builtin_amdgcn_readfirstlane(item.q0);
    if constexpr (MASK) {
      if (small)
        run_item_masked<CB>(item, q, k, v, o, n_heads, n_kv_heads, kv_group, c2, negate, causal, window, stage,
                            row_bytes, wave, lane);
      else
        run_item_masked<CA>(item, q, k, v, o, n_heads, n_kv_heads, kv_group, c2, negate, causal, window, stage,
                            row_bytes, wave, lane);
    } else {
      if (split)
        run_item_split<CB>(item, q, k, v, o, n_heads, n_kv_heads, kv_group, c2, negate, stage, row_bytes, wave,
                           lane);
      else if (small)
        run_item<CB>(item, q, k, v, o, n_heads, n_kv_heads, kv_group, c2, negate, stage, row_bytes, wave, lane);
      else
        run_item<CA>(item, q, k, v, o, n_heads, n_kv_heads, kv_group, c2, negate, stage, row_bytes, wave, lane);
    }
  }
}

// ----------------------------------------------------------------------------
// The input side of the path: the packed projection output split into Q, K and V in the
// layout the attention kernels read, with an optional per-head RMS norm of Q and K and the
// rope ("inferencelayer 0.2.1 src/vision_gpu.rs", VIS_QKV_ROPE and GLM_QKV_QKNORM_ROPE;
// "hf2q src/inference/vision/vit_gpu.rs", vit_rms_norm_gpu: y = x / sqrt(mean(x^2) + eps)
// * gain).  A packed row is [H query heads | Hkv key heads | Hkv value heads] of D elements.
// HBM-bound: every element is read once and written once, and the cos/sin tables
// ([tokens, D] float32) are read once per token row.
//
// One wavefront per token row: it loads the cos/sin values and the gains of its elements
// once and reuses them for every head of the row, and walks the row's head vectors (one
// contiguous run of (H + 2 Hkv) * D elements) a few at a time.  A head vector sits in a group
// of GS lanes (a power of two), EL elements per lane; EL is 8 (16-byte loads of 16-bit data)
// where half a head is a whole number of 8-element lanes (D = 64, 80, 128) and 4 otherwise
// (D = 72).  The rotate_half partner of a lane's elements (element d pairs with d +- D/2) is
// then the whole EL of the lane D/(2 EL) away, one shuffle per element, and the RMS sum is an
// xor butterfly inside the group.
// ----------------------------------------------------------------------------
constexpr int kF32Elem = 2;  // element kind of float32 data (the 16-bit kinds are kBF16, kF16)

// N (4 or 8) consecutive elements <-> float.  Eight 16-bit elements move as one 16-byte
// access, marked non-temporal: every byte is touched once, so it need not stay in the caches.
template <int E, int N>
struct ElemN {
  static __device__ __forceinline__ void load(const unsigned char* p, float (&x)[N]) {
    if constexpr (E != kF32Elem && N == 8) {
      const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
      if constexpr (E == kBF16) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          x[2 * h] = __uint_as_float(w[h] << 16);
          x[2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
        }
      } else {  // (the whole vector reinterpreted at once: a per-word bit_cast of w[h] was
                // compiled as the first word's, repeated)
        const f16x8_t hv = __builtin_bit_cast(f16x8_t, w);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (float)hv[i];
      }
      return;
    }
#pragma unroll
    for (int h = 0; h < N / 4; ++h) {
      const unsigned char* ph = p + h * 4 * (E == kF32Elem ? 4 : 2);
      if constexpr (E == kF32Elem) {
        const f32x4_t w = *reinterpret_cast<const f32x4_t*>(ph);
        for (int i = 0; i < 4; ++i) x[4 * h + i] = w[i];
      } else if constexpr (E == kBF16) {
        const u32x2_t w = *reinterpret_cast<const u32x2_t*>(ph);
        x[4 * h + 0] = __uint_as_float(w[0] << 16);
        x[4 * h + 1] = __uint_as_float(w[0] & 0xffff0000u);
        x[4 * h + 2] = __uint_as_float(w[1] << 16);
        x[4 * h + 3] = __uint_as_float(w[1] & 0xffff0000u);
      } else {
        const f16x4_t w = *reinterpret_cast<const f16x4_t*>(ph);
        for (int i = 0; i < 4; ++i) x[4 * h + i] = (float)w[i];
      }
    }
  }
  static __device__ __forceinline__ void store(unsigned char* p, const float (&x)[N]) {
    if constexpr (E != kF32Elem && N == 8) {
      const u32x4_t w = {cvt_pk<E>(x[0], x[1]), cvt_pk<E>(x[2], x[3]), cvt_pk<E>(x[4], x[5]), cvt_pk<E>(x[6], x[7])};
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
      return;
    }
#pragma unroll
    for (int h = 0; h < N / 4; ++h) {
      unsigned char* ph = p + h * 4 * (E == kF32Elem ? 4 : 2);
      if constexpr (E == kF32Elem)
        *reinterpret_cast<f32x4_t*>(ph) = f32x4_t{x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]};
      else
        *reinterpret_cast<u32x2_t*>(ph) =
            u32x2_t{cvt_pk<E>(x[4 * h], x[4 * h + 1]), cvt_pk<E>(x[4 * h + 2], x[4 * h + 3])};
    }
  }
};

__device__ __forceinline__ void load_f32n(const float* p, float* x, int n) {
  for (int h = 0; h < n / 4; ++h) {
    const f32x4_t w = *reinterpret_cast<const f32x4_t*>(p + 4 * h);
    for (int i = 0; i < 4; ++i) x[4 * h + i] = w[i];
  }
}

constexpr int kPrologueThreads = 256;  // four token rows per workgroup

template <int E, int D>
__global__ __launch_bounds__(kPrologueThreads) void qkv_prologue_kernel(
    const unsigned char* __restrict__ qkv, const float* __restrict__ cosv, const float* __restrict__ sinv,
    const float* __restrict__ qw, const float* __restrict__ kw, float eps, unsigned char* __restrict__ q,
    unsigned char* __restrict__ k, unsigned char* __restrict__ v, int n_tokens, int n_heads, int n_kv_heads) {
  constexpr int EL = (D / 2) % 8 == 0 ? 8 : 4;  // elements per lane
  constexpr int LH = D / EL;                      // lanes holding a head vector
  constexpr int GS = LH <= 8 ? 8 : (LH <= 16 ? 16 : 32);
  constexpr int HPI = 64 / GS;  // head vectors per pass of the wavefront
  constexpr int ES = E == kF32Elem ? 4 : 2;
  static_assert(D % 8 == 0 && LH <= 32 && (LH % 2) == 0, "halves of a head vector are whole lanes");
  const int lane = threadIdx.x & 63;
  const int hg = lane / GS, j = lane % GS;
  const bool on = j < LH;
  const int row = blockIdx.x * (kPrologueThreads / 64) + (threadIdx.x >> 6);
  if (row >= n_tokens) return;  // the whole wavefront; no barrier follows
  const int nh3 = n_heads + 2 * n_kv_heads;
  const bool low = j < LH / 2;
  const int src = (lane & ~(GS - 1)) + (low ? j + LH / 2 : j - LH / 2);  // rope partner lane

  float c[EL], sn[EL], wq[EL], wk[EL];
  if (cosv && on) {
    load_f32n(cosv + (size_t)row * D + j * EL, c, EL);
    load_f32n(sinv + (size_t)row * D + j * EL, sn, EL);
  }
  if (qw && on) {
    load_f32n(qw + j * EL, wq, EL);
    load_f32n(kw + j * EL, wk, EL);
  }
  const unsigned char* in = qkv + (size_t)row * nh3 * D * ES;
  for (int base = 0; base < nh3; base += HPI) {
    const int slot = base + hg;
    const bool live = on && slot < nh3;
    const bool is_q = slot < n_heads, is_v = slot >= n_heads + n_kv_heads;
    float x[EL];
#pragma unroll
    for (int i = 0; i < EL; ++i) x[i] = 0.f;
    if (live) ElemN<E, EL>::load(in + ((size_t)slot * D + j * EL) * ES, x);
    if (qw) {  // per-head RMS norm of Q and K
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < EL; ++i) ss += x[i] * x[i];
#pragma unroll
      for (int m = 1; m < GS; m <<= 1) ss += __shfl_xor(ss, m);
      if (!is_v) {
        const float r = 1.0f / sqrtf(ss * (1.0f / D) + eps);
#pragma unroll
        for (int i = 0; i < EL; ++i) x[i] = x[i] * r * (is_q ? wq[i] : wk[i]);
      }
    }
    if (cosv) {  // rope: x[d] cos[d] + rotate_half(x)[d] sin[d]
      float pr[EL];
#pragma unroll
      for (int i = 0; i < EL; ++i) pr[i] = __shfl(x[i], src);
      if (!is_v) {
#pragma unroll
        for (int i = 0; i < EL; ++i) x[i] = x[i] * c[i] + (low ? -pr[i] : pr[i]) * sn[i];
      }
    }
    if (live) {
      unsigned char* dst;
      if (is_q)
        dst = q + (((size_t)row * n_heads + slot) * D + j * EL) * ES;
      else if (!is_v)
        dst = k + (((size_t)row * n_kv_heads + (slot - n_heads)) * D + j * EL) * ES;
      else
        dst = v + (((size_t)row * n_kv_heads + (slot - n_heads - n_kv_heads)) * D + j * EL) * ES;
      ElemN<E, EL>::store(dst, x);
    }
  }
}

// ----------------------------------------------------------------------------
// Host side.
// ----------------------------------------------------------------------------
thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

struct KernelDesc {
  const void* func;
  int bm, bn, waves, nt;
  size_t lds;
};

template <class T, bool MASK>
KernelDesc describe_f32() {
  KernelDesc d;
  d.func = reinterpret_cast<const void*>(&attn_fwd_f32_kernel<T, MASK>);
  d.bm = T::BM;
  d.bn = T::BN;
  d.waves = T::NW;
  d.nt = T::NT;
  d.lds = ((sizeof(PlanLds) + 15) / 16) * 16 + 2 * (size_t)T::STAGE_ELEMS * sizeof(typename T::elem_t);
  return d;
}

template <class C, class CB, bool MASK>
KernelDesc describe_bf16() {
  KernelDesc d;
  d.func = reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<C, CB, MASK>);
  d.bm = C::BM;
  d.bn = C::BN;
  d.waves = C::NW;
  d.nt = C::NT;
  d.lds = ((sizeof(PlanLds) + 15) / 16) * 16 + 2 * (size_t)C::STAGE_BYTES;
  return d;
}

// Tile choices per (dtype, head_dim).
#ifndef VITATTN_BF16_QB
#define VITATTN_BF16_QB 4
#endif
#ifndef VITATTN_BF16_NW
#define VITATTN_BF16_NW 4
#endif
#ifndef VITATTN_BF16_QB_128
#define VITATTN_BF16_QB_128 2
#endif
#ifndef VITATTN_BF16_QB_SMALL
#define VITATTN_BF16_QB_SMALL 1
#endif
// 16-bit kernels: the large and the small query blocks for each element and output kind
template <int D, int E, bool OF32>
using KCfg = Bf16Cfg<D, D == 128 ? VITATTN_BF16_QB_128 : VITATTN_BF16_QB, VITATTN_BF16_NW, 64, E, OF32>;
template <int D, int E, bool OF32>
using SCfg = Bf16Cfg<D, VITATTN_BF16_QB_SMALL, VITATTN_BF16_NW, 64, E, OF32>;
// masked kernels: the large query blocks of the unmasked kernel for a causal mask or a wide
// window, and 2 blocks per wavefront (1 at head_dim 128) for a narrow window, whose items
// see fewer keys beyond their own rows when they are shorter
#ifndef VITATTN_BF16_QB_NARROW
#define VITATTN_BF16_QB_NARROW 2
#endif
#ifndef VITATTN_BF16_QB_NARROW_128
#define VITATTN_BF16_QB_NARROW_128 1
#endif
template <int D, int E, bool OF32>
using NCfg = Bf16Cfg<D, D == 128 ? VITATTN_BF16_QB_NARROW_128 : VITATTN_BF16_QB_NARROW, VITATTN_BF16_NW, 64, E, OF32>;
// a window is narrow when a query sees fewer keys than this (2*window - 1, or window with
// the causal rule): there the shorter items waste less than the larger ones gain
constexpr long long kNarrowKeys = 1024;
using K_f32_64 = F32Traits<64, 1, 4, 32>;
using K_f32_72 = F32Traits<72, 1, 4, 32>;
using K_f32_80 = F32Traits<80, 1, 4, 32>;
using K_f32_128 = F32Traits<128, 1, 4, 32>;

// Kernel table index: (mask kind * 5 + dtype) * 4 + head_dim slot, with dtype codes as in
// vitattn_dtype_t and mask kind 0 (none), 1 (causal or a wide window: the masked kernel with
// the large query blocks) or 2 (a narrow window: the masked kernel with small ones).
int kernel_index(int32_t head_dim, int32_t dtype, int mask_kind = 0) {
  int hd;
  switch (head_dim) {
    case 64: hd = 0; break;
    case 72: hd = 1; break;
    case 80: hd = 2; break;
    case 128: hd = 3; break;
    default: return -1;
  }
  return (mask_kind * 5 + dtype) * 4 + hd;
}

int mask_kind_of(int32_t causal, int32_t window) {
  if (!causal && window <= 0) return 0;
  if (window <= 0) return 1;
  const long long seen = causal ? (long long)window : 2LL * window - 1;
  return seen < kNarrowKeys ? 2 : 1;
}

template <int E, bool OF32, int MK>
KernelDesc describe16(int hd) {
  if constexpr (MK == 2) {
    switch (hd) {
      case 0: return describe_bf16<NCfg<64, E, OF32>, SCfg<64, E, OF32>, true>();
      case 1: return describe_bf16<NCfg<72, E, OF32>, SCfg<72, E, OF32>, true>();
      case 2: return describe_bf16<NCfg<80, E, OF32>, SCfg<80, E, OF32>, true>();
      default: return describe_bf16<NCfg<128, E, OF32>, SCfg<128, E, OF32>, true>();
    }
  } else {
    switch (hd) {
      case 0: return describe_bf16<KCfg<64, E, OF32>, SCfg<64, E, OF32>, MK == 1>();
      case 1: return describe_bf16<KCfg<72, E, OF32>, SCfg<72, E, OF32>, MK == 1>();
      case 2: return describe_bf16<KCfg<80, E, OF32>, SCfg<80, E, OF32>, MK == 1>();
      default: return describe_bf16<KCfg<128, E, OF32>, SCfg<128, E, OF32>, MK == 1>();
    }
  }
}

template <int MK>
KernelDesc kernel_desc_of(int dtype, int hd) {
  switch (dtype) {
    case VITATTN_DTYPE_F32:  // one masked float32 kernel serves both mask kinds
      switch (hd) {
        case 0: return describe_f32<K_f32_64, MK != 0>();
        case 1: return describe_f32<K_f32_72, MK != 0>();
        case 2: return describe_f32<K_f32_80, MK != 0>();
        default: return describe_f32<K_f32_128, MK != 0>();
      }
    case VITATTN_DTYPE_BF16: return describe16<kBF16, false, MK>(hd);
    case VITATTN_DTYPE_F16: return describe16<kF16, false, MK>(hd);
    case VITATTN_DTYPE_BF16_OUT_F32: return describe16<kBF16, true, MK>(hd);
    default: return describe16<kF16, true, MK>(hd);
  }
}

KernelDesc kernel_desc(int idx) {
  const int hd = idx % 4, dtype = (idx / 4) % 5, mk = idx / 20;
  if (mk == 2) return kernel_desc_of<2>(dtype, hd);
  return mk == 1 ? kernel_desc_of<1>(dtype, hd) : kernel_desc_of<0>(dtype, hd);
}

constexpr int kNumKernels = 60;  // 3 mask kinds x 5 dtype codes x 4 head dims
constexpr int kMaxDevices = 64;

struct DeviceState {
  std::once_flag once;
  int status = VITATTN_OK;
  char err[256] = "";
  int n_cus = 0;
  int grid[kNumKernels] = {};
};
DeviceState g_dev[kMaxDevices];

void init_device(DeviceState& st, int dev) {
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    st.status = VITATTN_ERR_HIP;
    snprintf(st.err, sizeof(st.err), "hipGetDeviceProperties: %s", hipGetErrorString(e));
    return;
  }
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    st.status = VITATTN_ERR_NO_DEVICE;
    snprintf(st.err, sizeof(st.err), "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
    return;
  }
  st.n_cus = prop.multiProcessorCount;
  for (int i = 0; i < kNumKernels; ++i) {
    const KernelDesc d = kernel_desc(i);
    e = hipFuncSetAttribute(d.func, hipFuncAttributeMaxDynamicSharedMemorySize, (int)d.lds);
    if (e != hipSuccess) {
      st.status = VITATTN_ERR_HIP;
      snprintf(st.err, sizeof(st.err), "hipFuncSetAttribute: %s", hipGetErrorString(e));
      return;
    }
    int per_cu = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, d.func, d.nt, d.lds);
    if (e != hipSuccess || per_cu < 1) {
      st.status = VITATTN_ERR_HIP;
      snprintf(st.err, sizeof(st.err), "occupancy query failed for kernel %d: %s", i, hipGetErrorString(e));
      return;
    }
    int grid = st.n_cus * per_cu;
    grid = grid < 8 ? 8 : grid / 8 * 8;  // slots are assigned per XCD (8 per device)
    st.grid[i] = grid;
  }
}

int get_device_state(DeviceState** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(VITATTN_ERR_NO_DEVICE, "no HIP device: %s", hipGetErrorString(e));
  if (dev >= kMaxDevices) return fail(VITATTN_ERR_NO_DEVICE, "device index %d out of range", dev);
  DeviceState& st = g_dev[dev];
  std::call_once(st.once, init_device, std::ref(st), dev);
  if (st.status != VITATTN_OK) return fail(st.status, "%s", st.err);
  *out = &st;
  return VITATTN_OK;
}

int validate(int32_t head_dim, int32_t dtype) {
  if (dtype < VITATTN_DTYPE_F32 || dtype > VITATTN_DTYPE_F16_OUT_F32)
    return fail(VITATTN_ERR_UNSUPPORTED_DTYPE, "dtype %d is not a vitattn_dtype_t code (0 .. 4)", dtype);
  if (kernel_index(head_dim, dtype) < 0)
    return fail(VITATTN_ERR_UNSUPPORTED_HEAD_DIM, "head_dim %d not in {64, 72, 80, 128}", head_dim);
  return VITATTN_OK;
}

// The prologue launch: kernel by (element kind, head_dim).
const void* prologue_kernel(int32_t dtype, int32_t head_dim) {
  auto pick = [&](auto e) -> const void* {
    constexpr int E = decltype(e)::value;
    switch (head_dim) {
      case 64: return reinterpret_cast<const void*>(&qkv_prologue_kernel<E, 64>);
      case 72: return reinterpret_cast<const void*>(&qkv_prologue_kernel<E, 72>);
      case 80: return reinterpret_cast<const void*>(&qkv_prologue_kernel<E, 80>);
      case 128: return reinterpret_cast<const void*>(&qkv_prologue_kernel<E, 128>);
      default: return nullptr;
    }
  };
  switch (dtype) {
    case VITATTN_DTYPE_F32: return pick(std::integral_constant<int, kF32Elem>{});
    case VITATTN_DTYPE_BF16: return pick(std::integral_constant<int, kBF16>{});
    case VITATTN_DTYPE_F16: return pick(std::integral_constant<int, kF16>{});
    default: return nullptr;
  }
}

}  // namespace

extern "C" {

const char* vitattn_status_string(int status) {
  switch (status) {
    case VITATTN_OK: return "ok";
    case VITATTN_ERR_INVALID_ARG: return "invalid argument";
    case VITATTN_ERR_UNSUPPORTED_HEAD_DIM: return "unsupported head_dim";
    case VITATTN_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case VITATTN_ERR_NO_DEVICE: return "no usable gfx950 device";
    case VITATTN_ERR_OOM: return "out of device memory";
    case VITATTN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* vitattn_last_error(void) { return g_last_error; }

int vitattn_kernel_config(int32_t head_dim, int32_t dtype, int32_t* block_m, int32_t* block_n, int32_t* waves,
                          int32_t* grid) {
  g_last_error[0] = '\0';
  int rc = validate(head_dim, dtype);
  if (rc != VITATTN_OK) return rc;
  DeviceState* st = nullptr;
  rc = get_device_state(&st);
  if (rc != VITATTN_OK) return rc;
  const int idx = kernel_index(head_dim, dtype);
  const KernelDesc d = kernel_desc(idx);
  if (block_m) *block_m = d.bm;
  if (block_n) *block_n = d.bn;
  if (waves) *waves = d.waves;
  if (grid) *grid = st->grid[idx];
  return VITATTN_OK;
}

int vitattn_fwd_masked(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens,
                       int32_t n_seqs, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                       int32_t causal, int32_t window, int32_t dtype, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (n_seqs < 0) return fail(VITATTN_ERR_INVALID_ARG, "n_seqs must be >= 0 (got %d)", n_seqs);
  if (n_heads <= 0) return fail(VITATTN_ERR_INVALID_ARG, "n_heads must be > 0 (got %d)", n_heads);
  if (n_kv_heads <= 0 || n_heads % n_kv_heads != 0)
    return fail(VITATTN_ERR_INVALID_ARG, "n_kv_heads must be a positive divisor of n_heads (got %d for %d heads)",
                n_kv_heads, n_heads);
  int rc = validate(head_dim, dtype);
  if (rc != VITATTN_OK) return rc;
  if (!std::isfinite(scale)) return fail(VITATTN_ERR_INVALID_ARG, "scale must be finite");
  if (causal != 0 && causal != 1) return fail(VITATTN_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (window < 0) return fail(VITATTN_ERR_INVALID_ARG, "window must be >= 0 (got %d)", window);
  if (n_seqs == 0) return VITATTN_OK;
  if (!q || !k || !v || !o || !cu_seqlens) return fail(VITATTN_ERR_INVALID_ARG, "null pointer argument");
  const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u;
  if (mis) return fail(VITATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if ((uintptr_t)cu_seqlens & 3u) return fail(VITATTN_ERR_INVALID_ARG, "cu_seqlens must be 4-byte aligned");
  if ((int64_t)n_heads * head_dim > (1 << 24)) return fail(VITATTN_ERR_INVALID_ARG, "n_heads * head_dim too large");

  DeviceState* st = nullptr;
  rc = get_device_state(&st);
  if (rc != VITATTN_OK) return rc;
  const int idx = kernel_index(head_dim, dtype, mask_kind_of(causal, window));
  const KernelDesc d = kernel_desc(idx);
  const float c2 = std::fabs(scale) * kLog2e;
  const int negate = scale < 0.0f ? 1 : 0;

  (void)hipGetLastError();  // clear a stale error so the check below is ours
  for (int32_t s0 = 0; s0 < n_seqs; s0 += kMaxSeqs) {
    const int n = n_seqs - s0 < kMaxSeqs ? n_seqs - s0 : kMaxSeqs;
    if (dtype != VITATTN_DTYPE_F32) {  // 16-bit inputs (bf16 or f16 bits); o by the output kind
      const __bf16* qq = static_cast<const __bf16*>(q);
      const __bf16* kk = static_cast<const __bf16*>(k);
      const __bf16* vv = static_cast<const __bf16*>(v);
      void* oo = o;
      const int32_t* cc = cu_seqlens + s0;
      void* args[] = {&qq, &kk, &vv, &oo, (void*)&cc, (void*)&n, (void*)&n_heads, (void*)&n_kv_heads,
                      (void*)&c2, (void*)&negate, (void*)&causal, (void*)&window};
      hipError_t e = hipLaunchKernel(d.func, dim3(st->grid[idx]), dim3(d.nt), args, d.lds, stream);
      if (e != hipSuccess) return fail(VITATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    } else {
      const float* qq = static_cast<const float*>(q);
      const float* kk = static_cast<const float*>(k);
      const float* vv = static_cast<const float*>(v);
      float* oo = static_cast<float*>(o);
      const int32_t* cc = cu_seqlens + s0;
      void* args[] = {&qq, &kk, &vv, &oo, (void*)&cc, (void*)&n, (void*)&n_heads, (void*)&n_kv_heads,
                      (void*)&c2, (void*)&negate, (void*)&causal, (void*)&window};
      hipError_t e = hipLaunchKernel(d.func, dim3(st->grid[idx]), dim3(d.nt), args, d.lds, stream);
      if (e != hipSuccess) return fail(VITATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(VITATTN_ERR_HIP, "after launch: %s", hipGetErrorString(e));
  return VITATTN_OK;
}

int vitattn_fwd_gqa(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens,
                    int32_t n_seqs, int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, float scale,
                    int32_t dtype, hipStream_t stream) {
  return vitattn_fwd_masked(q, k, v, o, cu_seqlens, n_seqs, n_heads, n_kv_heads, head_dim, scale, 0, 0, dtype,
                            stream);
}

int vitattn_fwd(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens, int32_t n_seqs,
                int32_t n_heads, int32_t head_dim, float scale, int32_t dtype, hipStream_t stream) {
  return vitattn_fwd_gqa(q, k, v, o, cu_seqlens, n_seqs, n_heads, n_heads, head_dim, scale, dtype, stream);
}

int vitattn_qkv_prologue(const void* qkv, const float* cos_table, const float* sin_table, const float* q_weight,
                         const float* k_weight, float eps, void* q, void* k, void* v, int32_t n_tokens,
                         int32_t n_heads, int32_t n_kv_heads, int32_t head_dim, int32_t dtype, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (n_tokens < 0) return fail(VITATTN_ERR_INVALID_ARG, "n_tokens must be >= 0 (got %d)", n_tokens);
  if (n_heads <= 0) return fail(VITATTN_ERR_INVALID_ARG, "n_heads must be > 0 (got %d)", n_heads);
  if (n_kv_heads <= 0 || n_heads % n_kv_heads != 0)
    return fail(VITATTN_ERR_INVALID_ARG, "n_kv_heads must be a positive divisor of n_heads (got %d for %d heads)",
                n_kv_heads, n_heads);
  if (dtype != VITATTN_DTYPE_F32 && dtype != VITATTN_DTYPE_BF16 && dtype != VITATTN_DTYPE_F16)
    return fail(VITATTN_ERR_UNSUPPORTED_DTYPE, "the prologue takes dtype F32, BF16 or F16 (got %d)", dtype);
  const void* func = prologue_kernel(dtype, head_dim);
  if (!func) return fail(VITATTN_ERR_UNSUPPORTED_HEAD_DIM, "head_dim %d not in {64, 72, 80, 128}", head_dim);
  if ((cos_table == nullptr) != (sin_table == nullptr))
    return fail(VITATTN_ERR_INVALID_ARG, "give both rope tables or neither");
  if ((q_weight == nullptr) != (k_weight == nullptr))
    return fail(VITATTN_ERR_INVALID_ARG, "give both norm gains or neither");
  if (q_weight && !(std::isfinite(eps) && eps >= 0.0f)) return fail(VITATTN_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (n_tokens == 0) return VITATTN_OK;
  if (!qkv || !q || !k || !v) return fail(VITATTN_ERR_INVALID_ARG, "null pointer argument");
  if (((uintptr_t)qkv | (uintptr_t)q | (uintptr_t)k | (uintptr_t)v) & 15u)
    return fail(VITATTN_ERR_INVALID_ARG, "qkv, q, k and v must be 16-byte aligned");
  if (((uintptr_t)cos_table | (uintptr_t)sin_table | (uintptr_t)q_weight | (uintptr_t)k_weight) & 15u)
    return fail(VITATTN_ERR_INVALID_ARG, "the rope tables and norm gains must be 16-byte aligned");
  DeviceState* st = nullptr;
  int rc = get_device_state(&st);
  if (rc != VITATTN_OK) return rc;
  if ((long long)n_tokens * (n_heads + 2LL * n_kv_heads) * head_dim >= (1LL << 40))
    return fail(VITATTN_ERR_INVALID_ARG, "qkv too large");
  const long long blocks = ((long long)n_tokens + kPrologueThreads / 64 - 1) / (kPrologueThreads / 64);
  const unsigned char* a0 = static_cast<const unsigned char*>(qkv);
  unsigned char *a1 = static_cast<unsigned char*>(q), *a2 = static_cast<unsigned char*>(k),
                *a3 = static_cast<unsigned char*>(v);
  int nh = n_heads, nkv = n_kv_heads;
  int nt = n_tokens;
  void* args[] = {&a0, (void*)&cos_table, (void*)&sin_table, (void*)&q_weight, (void*)&k_weight, &eps,
                  &a1, &a2, &a3, &nt, &nh, &nkv};
  (void)hipGetLastError();
  hipError_t e = hipLaunchKernel(func, dim3((unsigned)blocks), dim3(kPrologueThreads), args, 0, stream);
  if (e != hipSuccess) return fail(VITATTN_ERR_HIP, "prologue launch: %s", hipGetErrorString(e));
  e = hipGetLastError();
  if (e != hipSuccess) return fail(VITATTN_ERR_HIP, "after prologue launch: %s", hipGetErrorString(e));
  return VITATTN_OK;
}

}  // extern "C"
