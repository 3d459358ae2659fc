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
//    XCD's L2.
//  * Scores are computed transposed, S^T = K.Q^T, with v_mfma_f32_16x16x32_bf16
//    (float32: v_mfma_f32_16x16x4_f32).  In that accumulator layout a lane holds
//    4 keys of one query, so the row max is in-lane plus two cross-lane steps,
//    and the same registers (converted to bf16) are directly the B operand of
//    O^T += V^T.P^T: no data movement between the two products, and the running
//    output of a query sits in the lane that owns its softmax state, so the
//    rescale is a per-lane multiply.
//  * The running max is raised lazily: only when a tile's max exceeds it by more
//    than kLazyTau (log2 units).  Exponentials are then at most 2^kLazyTau, which
//    float32 sums and bf16 weights carry without loss, and the accumulator rescale
//    is skipped (wave-uniform branch) on almost every tile.  The final division by
//    the row sum makes the result independent of which max was used.
//  * K tiles sit in LDS as [key][d] and V tiles as V^T [d][key] (transposed while
//    staging, with the keys permuted to match the P^T register layout), both with
//    16-byte row padding against bank conflicts and double-buffered: tile t+1 is
//    fetched into registers while tile t is computed.
//  * head_dim 72 and 80 are zero-padded to 96 for the Q.K^T contraction (K steps of
//    32) and to 80 for the P.V output rows (blocks of 16); padded K columns are
//    zeroed in LDS once, padded Q columns are zero in registers.
#include "vitattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kMaxSeqs = 512;     // sequences planned by one launch (more: several launches)
constexpr int kSortMax = 256;     // sequences ordered longest-first up to this count
constexpr float kLazyTau = 8.0f;  // headroom (log2) before the running max is raised
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

// Fills P for sequences [0, n) of `cu` (n >= 1).  Returns the item count.
template <int NT>
__device__ int build_plan(PlanLds& P, const int32_t* __restrict__ cu, int n, int n_heads, int bm) {
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
  // Exclusive scan of items per sorted position: thread tid owns positions
  // [tid*per, tid*per + per).
  const int per = ceil_div(n, NT);
  const int beg = tid * per;
  const int end = min(beg + per, n);
  int local = 0;
  for (int r = beg; r < end; ++r) {
    const int s = P.order[r];
    local += ceil_div(P.cu[s + 1] - P.cu[s], bm) * n_heads;
  }
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
    const int s = P.order[r];
    run += ceil_div(P.cu[s + 1] - P.cu[s], bm) * n_heads;
    P.prefix[r + 1] = run;
  }
  __syncthreads();
  return P.prefix[n];
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

// ----------------------------------------------------------------------------
// Element-type specific parts.
// ----------------------------------------------------------------------------
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// bf16 inputs: v_mfma_f32_16x16x32_bf16 for both products.
template <int D_, int QB_, int NW_, int BN_>
struct Bf16Traits {
  using elem_t = __bf16;
  static constexpr int D = D_, QB = QB_, NW = NW_, BN = BN_;
  static constexpr int NT = NW * 64;
  static constexpr int NQ = QB * 16;            // queries per wavefront
  static constexpr int BM = NW * NQ;            // queries per item
  static constexpr int DK = (D + 31) / 32 * 32; // Q.K^T contraction, padded
  static constexpr int NKS = DK / 32;
  static constexpr int DV = (D + 15) / 16 * 16; // output rows of O^T, padded
  static constexpr int NDB = DV / 16;
  static constexpr int NKB = BN / 16;
  static constexpr int NKC = BN / 32;
  static constexpr int KSTR = DK + 8;           // LDS row stride of K (elements)
  static constexpr int VSTR = BN + 8;           // LDS row stride of V^T (elements)
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int STAGE_ELEMS = K_ELEMS + DV * VSTR;
  static constexpr int CH = D / 8;              // 16-byte chunks per row
  static constexpr int K_UNITS = BN * CH;
  static constexpr int V_UNITS = (BN / 4) * CH; // 4 keys x 8 dims each
  static constexpr int K_IT = (K_UNITS + NT - 1) / NT;
  static constexpr int V_IT = (V_UNITS + NT - 1) / NT;
  static_assert(D % 8 == 0 && BN % 32 == 0, "tile shape");

  struct QOp { bf16x8_t x[QB][NKS]; };
  struct Pre { u32x4_t k[K_IT]; u32x4_t v[V_IT][4]; };

  static __device__ __forceinline__ void load_q(QOp& Q, const elem_t* __restrict__ q, int row0, int qend,
                                                int head, int n_heads, bool negate, int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int row = row0 + qb * 16 + c;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int d0 = ks * 32 + 8 * g;
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (row < qend && d0 < D) w = ld16(q + ((size_t)row * n_heads + head) * D + d0);
        if (negate) w ^= 0x80008000u;
        Q.x[qb][ks] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
  }

  static __device__ __forceinline__ void zero_pad(elem_t* stage) {
    // K columns D..DK-1 of every row, both buffers; never written afterwards.
    if constexpr (DK > D) {
      constexpr int PADW = DK - D;
      for (int i = threadIdx.x; i < 2 * BN * PADW; i += NT) {
        const int buf = i / (BN * PADW), rem = i % (BN * PADW);
        stage[buf * STAGE_ELEMS + (rem / PADW) * KSTR + D + rem % PADW] = (elem_t)0.0f;
      }
    }
  }

  static __device__ __forceinline__ void fetch(Pre& R, const elem_t* __restrict__ k, const elem_t* __restrict__ v,
                                               int key0, int b, int head, int n_heads) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < K_IT; ++i) {
      const int u = tid + i * NT;
      R.k[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (u < K_UNITS) {
        const int key = key0 + u / CH;
        if (key < b) R.k[i] = ld16(k + ((size_t)key * n_heads + head) * D + (u % CH) * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < V_IT; ++i) {
      const int u = tid + i * NT;
#pragma unroll
      for (int j = 0; j < 4; ++j) R.v[i][j] = u32x4_t{0u, 0u, 0u, 0u};
      if (u < V_UNITS) {
        const int kbase = key0 + (u / CH) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (kbase + j < b) R.v[i][j] = ld16(v + ((size_t)(kbase + j) * n_heads + head) * D + (u % CH) * 8);
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
      if (u < K_UNITS) *reinterpret_cast<u32x4_t*>(Ks + (u / CH) * KSTR + (u % CH) * 8) = R.k[i];
    }
#pragma unroll
    for (int i = 0; i < V_IT; ++i) {
      const int u = tid + i * NT;
      if (u < V_UNITS) {
        const int kap = (u / CH) * 4;          // first key of the group, within the tile
        const int kc = kap >> 5, kl = kap & 31;
        const int pos = kc * 32 + 8 * ((kl & 15) >> 2) + 4 * (kl >> 4);
        const int d0 = (u % CH) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          unsigned lo, hi;
          if (e & 1) {
            lo = (R.v[i][0][w] >> 16) | (R.v[i][1][w] & 0xffff0000u);
            hi = (R.v[i][2][w] >> 16) | (R.v[i][3][w] & 0xffff0000u);
          } else {
            lo = (R.v[i][0][w] & 0xffffu) | (R.v[i][1][w] << 16);
            hi = (R.v[i][2][w] & 0xffffu) | (R.v[i][3][w] << 16);
          }
          *reinterpret_cast<u32x2_t*>(Vt + (d0 + e) * VSTR + pos) = u32x2_t{lo, hi};
        }
      }
    }
  }

  // S^T[kb][qb] = K_tile . Q^T
  static __device__ __forceinline__ void qk(f32x4_t (&S)[NKB][QB], const QOp& Q, const elem_t* stage, int lane) {
    const int g = lane >> 4, c = lane & 15;
    const elem_t* Ks = stage;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) S[kb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Ks + (kb * 16 + c) * KSTR + ks * 32 + 8 * g);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Q.x[qb][ks], S[kb][qb], 0, 0, 0);
      }
    }
  }

  // O^T[db][qb] += V^T_tile . P^T, P held in S (float32, already exponentiated)
  static __device__ __forceinline__ void pv(f32x4_t (&O)[NDB][QB], const f32x4_t (&S)[NKB][QB],
                                            const elem_t* stage, int lane) {
    const int g = lane >> 4, c = lane & 15;
    const elem_t* Vt = stage + K_ELEMS;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      bf16x8_t pb[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pb[qb][j] = (__bf16)S[2 * kc][qb][j];
          pb[qb][4 + j] = (__bf16)S[2 * kc + 1][qb][j];
        }
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Vt + (db * 16 + c) * VSTR + kc * 32 + 8 * g);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          O[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[qb], O[db][qb], 0, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ void store_out(elem_t* __restrict__ o, size_t off, const f32x4_t& x, float inv) {
    __bf16 t0 = (__bf16)(x[0] * inv), t1 = (__bf16)(x[1] * inv), t2 = (__bf16)(x[2] * inv), t3 = (__bf16)(x[3] * inv);
    const unsigned lo = (unsigned)__builtin_bit_cast(unsigned short, t0) | ((unsigned)__builtin_bit_cast(unsigned short, t1) << 16);
    const unsigned hi = (unsigned)__builtin_bit_cast(unsigned short, t2) | ((unsigned)__builtin_bit_cast(unsigned short, t3) << 16);
    *reinterpret_cast<u32x2_t*>(o + off) = u32x2_t{lo, hi};
  }
};

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
template <class T>
__global__ __launch_bounds__(T::NT) void attn_fwd_kernel(
    const typename T::elem_t* __restrict__ q, const typename T::elem_t* __restrict__ k,
    const typename T::elem_t* __restrict__ v, typename T::elem_t* __restrict__ o,
    const int32_t* __restrict__ cu, int n_seqs, int n_heads, float c2, int negate) {
  using elem_t = typename T::elem_t;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  PlanLds& plan = *reinterpret_cast<PlanLds*>(smem);
  elem_t* stage = reinterpret_cast<elem_t*>(smem + ((sizeof(PlanLds) + 15) / 16) * 16);

  const int n_items = build_plan<T::NT>(plan, cu, n_seqs, n_heads, T::BM);
  T::zero_pad(stage);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int G = gridDim.x;
  const int slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);

  for (int it = slot; it < n_items; it += G) {
    const Item item = map_item(plan, n_seqs, it, T::BM);
    const int qend = min(item.q0 + T::BM, item.b);
    const int row0 = item.q0 + wave * T::NQ;

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

    const int ntiles = ceil_div(item.b - item.a, T::BN);
    typename T::Pre pre;
    __syncthreads();  // the previous item is done with both stage buffers
    T::fetch(pre, k, v, item.a, item.b, item.head, n_heads);
    T::store(pre, stage);

    for (int t = 0; t < ntiles; ++t) {
      __syncthreads();  // tile t is in LDS; buffer (t+1)&1 is free
      const elem_t* cur = stage + (t & 1) * T::STAGE_ELEMS;
      const int key0 = item.a + t * T::BN;
      if (t + 1 < ntiles) T::fetch(pre, k, v, key0 + T::BN, item.b, item.head, n_heads);

      f32x4_t S[T::NKB][T::QB];
      T::qk(S, Q, cur, lane);

      const bool ragged = key0 + T::BN > item.b;  // last tile runs past the sequence
      if (ragged) {  // keys past the sequence take no part in the max ...
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key0 + kb * 16 + 4 * g + r >= item.b)
#pragma unroll
              for (int qb = 0; qb < T::QB; ++qb) S[kb][qb][r] = -INFINITY;
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
        if (mc > m[qb] + kLazyTau) {
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
      if (ragged) {  // ... and get weight exactly 0 (also when the scale is 0)
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (key0 + kb * 16 + 4 * g + r >= item.b)
#pragma unroll
              for (int qb = 0; qb < T::QB; ++qb) S[kb][qb][r] = 0.f;
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

template <class T>
KernelDesc describe() {
  KernelDesc d;
  d.func = reinterpret_cast<const void*>(&attn_fwd_kernel<T>);
  d.bm = T::BM;
  d.bn = T::BN;
  d.waves = T::NW;
  d.nt = T::NT;
  d.lds = ((sizeof(PlanLds) + 15) / 16) * 16 + 2 * (size_t)T::STAGE_ELEMS * sizeof(typename T::elem_t);
  return d;
}

// Tile choices per (dtype, head_dim).
using K_bf16_64 = Bf16Traits<64, 2, 4, 64>;
using K_bf16_72 = Bf16Traits<72, 2, 4, 64>;
using K_bf16_80 = Bf16Traits<80, 2, 4, 64>;
using K_bf16_128 = Bf16Traits<128, 2, 4, 64>;
using K_f32_64 = F32Traits<64, 1, 4, 32>;
using K_f32_72 = F32Traits<72, 1, 4, 32>;
using K_f32_80 = F32Traits<80, 1, 4, 32>;
using K_f32_128 = F32Traits<128, 1, 4, 32>;

int kernel_index(int32_t head_dim, int32_t dtype) {
  int hd;
  switch (head_dim) {
    case 64: hd = 0; break;
    case 72: hd = 1; break;
    case 80: hd = 2; break;
    case 128: hd = 3; break;
    default: return -1;
  }
  return dtype * 4 + hd;
}

KernelDesc kernel_desc(int idx) {
  switch (idx) {
    case 0: return describe<K_f32_64>();
    case 1: return describe<K_f32_72>();
    case 2: return describe<K_f32_80>();
    case 3: return describe<K_f32_128>();
    case 4: return describe<K_bf16_64>();
    case 5: return describe<K_bf16_72>();
    case 6: return describe<K_bf16_80>();
    default: return describe<K_bf16_128>();
  }
}

constexpr int kNumKernels = 8;
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
  if (dtype != VITATTN_DTYPE_F32 && dtype != VITATTN_DTYPE_BF16)
    return fail(VITATTN_ERR_UNSUPPORTED_DTYPE, "dtype %d is not VITATTN_DTYPE_F32 (0) or VITATTN_DTYPE_BF16 (1)", dtype);
  if (kernel_index(head_dim, dtype) < 0)
    return fail(VITATTN_ERR_UNSUPPORTED_HEAD_DIM, "head_dim %d not in {64, 72, 80, 128}", head_dim);
  return VITATTN_OK;
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

int vitattn_fwd(const void* q, const void* k, const void* v, void* o, const int32_t* cu_seqlens, int32_t n_seqs,
                int32_t n_heads, int32_t head_dim, float scale, int32_t dtype, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (n_seqs < 0) return fail(VITATTN_ERR_INVALID_ARG, "n_seqs must be >= 0 (got %d)", n_seqs);
  if (n_heads <= 0) return fail(VITATTN_ERR_INVALID_ARG, "n_heads must be > 0 (got %d)", n_heads);
  int rc = validate(head_dim, dtype);
  if (rc != VITATTN_OK) return rc;
  if (!std::isfinite(scale)) return fail(VITATTN_ERR_INVALID_ARG, "scale must be finite");
  if (n_seqs == 0) return VITATTN_OK;
  if (!q || !k || !v || !o || !cu_seqlens) return fail(VITATTN_ERR_INVALID_ARG, "null pointer argument");
  const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u;
  if (mis) return fail(VITATTN_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
  if ((uintptr_t)cu_seqlens & 3u) return fail(VITATTN_ERR_INVALID_ARG, "cu_seqlens must be 4-byte aligned");
  if ((int64_t)n_heads * head_dim > (1 << 24)) return fail(VITATTN_ERR_INVALID_ARG, "n_heads * head_dim too large");

  DeviceState* st = nullptr;
  rc = get_device_state(&st);
  if (rc != VITATTN_OK) return rc;
  const int idx = kernel_index(head_dim, dtype);
  const KernelDesc d = kernel_desc(idx);
  const float c2 = std::fabs(scale) * kLog2e;
  const int negate = scale < 0.0f ? 1 : 0;

  (void)hipGetLastError();  // clear a stale error so the check below is ours
  for (int32_t s0 = 0; s0 < n_seqs; s0 += kMaxSeqs) {
    const int n = n_seqs - s0 < kMaxSeqs ? n_seqs - s0 : kMaxSeqs;
    if (dtype == VITATTN_DTYPE_BF16) {
      const __bf16* qq = static_cast<const __bf16*>(q);
      const __bf16* kk = static_cast<const __bf16*>(k);
      const __bf16* vv = static_cast<const __bf16*>(v);
      __bf16* oo = static_cast<__bf16*>(o);
      const int32_t* cc = cu_seqlens + s0;
      void* args[] = {&qq, &kk, &vv, &oo, (void*)&cc, (void*)&n, (void*)&n_heads, (void*)&c2, (void*)&negate};
      hipError_t e = hipLaunchKernel(d.func, dim3(st->grid[idx]), dim3(d.nt), args, d.lds, stream);
      if (e != hipSuccess) return fail(VITATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    } else {
      const float* qq = static_cast<const float*>(q);
      const float* kk = static_cast<const float*>(k);
      const float* vv = static_cast<const float*>(v);
      float* oo = static_cast<float*>(o);
      const int32_t* cc = cu_seqlens + s0;
      void* args[] = {&qq, &kk, &vv, &oo, (void*)&cc, (void*)&n, (void*)&n_heads, (void*)&c2, (void*)&negate};
      hipError_t e = hipLaunchKernel(d.func, dim3(st->grid[idx]), dim3(d.nt), args, d.lds, stream);
      if (e != hipSuccess) return fail(VITATTN_ERR_HIP, "kernel launch: %s", hipGetErrorString(e));
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(VITATTN_ERR_HIP, "after launch: %s", hipGetErrorString(e));
  return VITATTN_OK;
}

}  // extern "C"
