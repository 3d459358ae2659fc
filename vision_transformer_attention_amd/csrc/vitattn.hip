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
__global__ __launch_bounds__(T::NT) void attn_fwd_f32_kernel(
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

// ---------------------------------------------------------------------------
// bf16 inputs: direct HBM->LDS staging, v_mfma_f32_16x16x32_bf16 for both products.
//
// LDS layout of one stage (one BN-key tile):
//   K: [BN][KCH chunks of 16 B]  -- row stride KCH*4 words = 4*odd, so the 16-byte
//      A-operand reads of 8 consecutive rows hit distinct banks.  Chunks past the
//      head_dim hold a copy of real data (finite) and meet zero Q columns.
//   V: [BN][VCH chunks of 16 B]  -- natural [key][d] order; read with the transposing
//      ds_read_b64_tr_b16, whose 4-row x 32-byte footprint per 16 lanes is bank-conflict
//      free with a row stride of 8 (mod 32) words.
// Both are filled by global_load_lds_dwordx4: lane l of a wave-wide load lands at
// base + 16*l, so each wave-wide load fills 64 consecutive chunk slots.
// ---------------------------------------------------------------------------
template <int D_, int QB_, int NW_, int BN_, bool SUM_MFMA_>
struct Bf16Cfg {
  using elem_t = __bf16;
  static constexpr int D = D_, QB = QB_, NW = NW_, BN = BN_;
  static constexpr bool SUM_MFMA = SUM_MFMA_;   // row sums by an MFMA against a block of ones
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
  static constexpr int NACC = NDB + (SUM_MFMA ? 1 : 0);
  static constexpr int CH = D / 8;              // 16-byte chunks of a row in HBM
  static constexpr int KCH = DK / 8 + 1;
  static constexpr int VCH = D <= 80 ? 10 : 18;
  static constexpr int KSTR = KCH * 8, VSTR = VCH * 8;  // elements
  static constexpr int K_BYTES = BN * KCH * 16, V_BYTES = BN * VCH * 16;
  static constexpr int STAGE_BYTES = K_BYTES + V_BYTES;
  static constexpr int K_LOADS = BN * KCH / 64, V_LOADS = BN * VCH / 64;
  static constexpr int LOADS = K_LOADS + V_LOADS;
  static_assert(D % 8 == 0 && BN % 64 == 0 && D - NK32 * 32 <= 16, "tile shape");
  static_assert(VCH * 8 >= DV && (VCH * 4) % 32 == 8, "V stride");
  static_assert(((KCH * 4) / 4) % 2 == 1, "K stride");
};

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ float fbits(unsigned x) { return __builtin_bit_cast(float, x); }
__device__ __forceinline__ unsigned ubits(float x) { return __builtin_bit_cast(unsigned, x); }

// max over the four lanes l, l^16, l^32, l^48 (permlane swaps: VALU only, no LDS)
__device__ __forceinline__ float max_4groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(ubits(x), ubits(x), false, false);
  x = fmaxf(fbits(a[0]), fbits(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(ubits(x), ubits(x), false, false);
  return fmaxf(fbits(b[0]), fbits(b[1]));
}
__device__ __forceinline__ float sum_4groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(ubits(x), ubits(x), false, false);
  x = fbits(a[0]) + fbits(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(ubits(x), ubits(x), false, false);
  return fbits(b[0]) + fbits(b[1]);
}


// Wave-wide DMA loads of one K/V tile.  Load i of wave w is the tile's load number
// wl = w + i*NW; lane l of it fills chunk slot z = (wl or wl - K_LOADS)*64 + l of the
// K or V area, i.e. key row z / per and chunk z % per (chunks past head_dim repeat
// the last real chunk, so every byte copied is finite data of that row).
template <class C>
struct Dma {
  static constexpr int PER_WAVE = (C::LOADS + C::NW - 1) / C::NW;

  static __device__ __forceinline__ unsigned lane_offset(int wl, int lane, int key_limit, unsigned row_bytes) {
    const bool is_k = wl < C::K_LOADS;
    const int z = (is_k ? wl : wl - C::K_LOADS) * 64 + lane;
    const int per = is_k ? C::KCH : C::VCH;
    const int row = min(z / per, key_limit);
    const int ch = min(z % per, C::CH - 1);
    return (unsigned)row * row_bytes + (unsigned)ch * 16u;
  }

  // byte offsets (relative to the tile's first key row) for full tiles
  static __device__ __forceinline__ void init(unsigned (&off)[PER_WAVE], int wave, int lane, unsigned row_bytes) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int wl = wave + i * C::NW;
      off[i] = wl < C::LOADS ? lane_offset(wl, lane, C::BN - 1, row_bytes) : 0u;
    }
  }

  // Enqueue the tile with keys [key0, key0 + BN); a RAGGED tile clamps rows to b - 1.
  template <bool RAGGED>
  static __device__ __forceinline__ void issue(const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                                               unsigned char* buf, int key0, int b, int head, int n_heads,
                                               unsigned row_bytes, const unsigned (&off)[PER_WAVE], int wave,
                                               int lane) {
    const size_t base = ((size_t)key0 * n_heads + head) * C::D;
    const unsigned char* kb = reinterpret_cast<const unsigned char*>(k + base);
    const unsigned char* vb = reinterpret_cast<const unsigned char*>(v + base);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int wl = wave + i * C::NW;
      if (wl < C::LOADS) {
        const bool is_k = wl < C::K_LOADS;
        const unsigned o = RAGGED ? lane_offset(wl, lane, b - 1 - key0, row_bytes) : off[i];
        const unsigned char* src = (is_k ? kb : vb) + o;
        unsigned char* dst = buf + (is_k ? wl * 1024 : C::K_BYTES + (wl - C::K_LOADS) * 1024);
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)dst, 16, 0, 0);
      }
    }
  }
};

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ unsigned cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// One compute step over 32 keys [kb0, kb0 + 32) of the LDS tile.  RAGGED: only the
// first `kvalid` of them belong to the sequence.
template <class C, bool RAGGED>
__device__ __forceinline__ void attend_32(const __bf16* Ks, const __bf16* Vs, int kb0, int kvalid,
                                         const bf16x8_t (&Q)[C::QB][C::NK32], const s16x4_t (&QT)[C::QB],
                                         f32x4_t (&O)[C::NACC][C::QB],
                                         float (&m)[C::QB], float (&lsum)[C::QB], float c2, int lane) {
  const int g = lane >> 4, c = lane & 15;
  // ---- S^T = K.Q^T: lane holds keys kb0+kb*16+4g+r of query c of each block qb
  f32x4_t S[2][C::QB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) S[kb][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < C::NK32; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(Ks + (kb0 + kb * 16 + c) * C::KSTR + ks * 32 + 8 * g);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
        S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Q[qb][ks], S[kb][qb], 0, 0, 0);
    }
  if constexpr (C::TAIL) {  // dims NK32*32 + 4g..+4 in a 16-deep step
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const s16x4_t a = *reinterpret_cast<const s16x4_t*>(Ks + (kb0 + kb * 16 + c) * C::KSTR + C::NK32 * 32 + 4 * g);
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
        S[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, QT[qb], S[kb][qb], 0, 0, 0);
    }
  }
  if constexpr (RAGGED) {  // keys past the sequence take no part in the max ...
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (kb * 16 + 4 * g + r >= kvalid)
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb) S[kb][qb][r] = -INFINITY;
  }
  // ---- row max over the 32 keys; the running max is raised only past kLazyTau
  float alpha[C::QB];
  bool raise = false;
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    float mx = fmaxf(fmaxf(fmaxf(S[0][qb][0], S[0][qb][1]), fmaxf(S[0][qb][2], S[0][qb][3])),
                     fmaxf(fmaxf(S[1][qb][0], S[1][qb][1]), fmaxf(S[1][qb][2], S[1][qb][3])));
    mx = max_4groups(mx);
    const float mc = mx * c2;
    alpha[qb] = 1.f;
    if (mc > m[qb] + kLazyTau) {
      alpha[qb] = __builtin_amdgcn_exp2f(m[qb] - mc);
      m[qb] = mc;
      raise = true;
    }
  }
  if (__any(raise)) {
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      lsum[qb] *= alpha[qb];
#pragma unroll
      for (int db = 0; db < C::NACC; ++db) O[db][qb] *= alpha[qb];
    }
  }
  // ---- P = exp2(S*c - m) as the bf16 B operand of O^T += V^T.P^T
  bf16x8_t P[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    float p[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) p[kb * 4 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][qb][r], c2, -m[qb]));
    if constexpr (RAGGED) {  // ... and weigh exactly 0 (also when the scale is 0)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kb * 16 + 4 * g + r >= kvalid) p[kb * 4 + r] = 0.f;
    }
    if constexpr (!C::SUM_MFMA) {
#pragma unroll
      for (int j = 0; j < 8; ++j) lsum[qb] += p[j];
    }
    const u32x4_t w = {cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3]), cvt_pk_bf16(p[4], p[5]),
                       cvt_pk_bf16(p[6], p[7])};
    P[qb] = __builtin_bit_cast(bf16x8_t, w);
  }
  // ---- V^T fragments: two transposing reads of [key][d] give lane (c, g) the keys
  //      kb0+4g+0..3 and kb0+16+4g+0..3 of dim db*16+c, matching the P^T slots
  const int i = lane & 15;
  const __bf16* v1 = Vs + (kb0 + 4 * g + (i >> 2)) * C::VSTR + 4 * (i & 3);
  const __bf16* v2 = v1 + 16 * C::VSTR;
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(v1 + db * 16));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(v2 + db * 16));
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) O[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, P[qb], O[db][qb], 0, 0, 0);
  }
  if constexpr (C::SUM_MFMA) {  // row sums of the rounded weights, by MFMA against ones
    const u32x4_t ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb)
      O[C::NDB][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ones), P[qb],
                                                               O[C::NDB][qb], 0, 0, 0);
  }
}

// One work item (sequence, head, BM queries from q0) for the whole workgroup.  The K/V
// stage buffers and the DMA offsets depend only on head_dim and the tile shape, so work
// items of different query-block sizes (C::QB) share them.
template <class C>
__device__ __forceinline__ void run_item(const Item& item, const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                         const __bf16* __restrict__ v, __bf16* __restrict__ o, int n_heads, float c2,
                                         int negate, unsigned char* stage, unsigned row_bytes,
                                         const unsigned (&dma_off)[Dma<C>::PER_WAVE], int wave, int lane) {
  const int g = lane >> 4, c = lane & 15;
  const int qend = min(item.q0 + C::BM, item.b);
  const int row0 = item.q0 + wave * C::NQ;
  const int ntiles = ceil_div(item.b - item.a, C::BN);
  const bool last_ragged = (item.b - item.a) % C::BN != 0;

  __syncthreads();  // the previous item is done with both stage buffers
  if (ntiles == 1 && last_ragged)
    Dma<C>::template issue<true>(k, v, stage, item.a, item.b, item.head, n_heads, row_bytes, dma_off, wave, lane);
  else
    Dma<C>::template issue<false>(k, v, stage, item.a, item.b, item.head, n_heads, row_bytes, dma_off, wave, lane);

  // Q^T operands: lane (c, g) holds row row0+qb*16+c, dims ks*32+8g..+8, and for the
  // 16-deep tail dims NK32*32+4g..+4 (zero past D)
  bf16x8_t Q[C::QB][C::NK32];
  s16x4_t QT[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int row = min(row0 + qb * 16 + c, qend - 1);
    const __bf16* qrow = q + ((size_t)row * n_heads + item.head) * C::D;
#pragma unroll
    for (int ks = 0; ks < C::NK32; ++ks) {
      u32x4_t w = ld16(qrow + ks * 32 + 8 * g);
      if (negate) w ^= 0x80008000u;
      Q[qb][ks] = __builtin_bit_cast(bf16x8_t, w);
    }
    u32x2_t t = {0u, 0u};
    if (C::TAIL && C::NK32 * 32 + 4 * g < C::D) t = *reinterpret_cast<const u32x2_t*>(qrow + C::NK32 * 32 + 4 * g);
    if (negate) t ^= 0x80008000u;
    QT[qb] = __builtin_bit_cast(s16x4_t, t);
  }

  f32x4_t O[C::NACC][C::QB];
#pragma unroll
  for (int db = 0; db < C::NACC; ++db)
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) O[db][qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m[C::QB], lsum[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) { m[qb] = -INFINITY; lsum[qb] = 0.f; }

  for (int t = 0; t < ntiles; ++t) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA of tile t has landed
    __syncthreads();  // every wave's has; buffer (t+1)&1 is no longer read
    const int key0 = item.a + t * C::BN;
    if (t + 1 < ntiles) {
      unsigned char* nb = stage + ((t + 1) & 1) * C::STAGE_BYTES;
      if (t + 2 == ntiles && last_ragged)
        Dma<C>::template issue<true>(k, v, nb, key0 + C::BN, item.b, item.head, n_heads, row_bytes, dma_off, wave,
                                     lane);
      else
        Dma<C>::template issue<false>(k, v, nb, key0 + C::BN, item.b, item.head, n_heads, row_bytes, dma_off, wave,
                                      lane);
    }
    const unsigned char* buf = stage + (t & 1) * C::STAGE_BYTES;
    const __bf16* Ks = reinterpret_cast<const __bf16*>(buf);
    const __bf16* Vs = reinterpret_cast<const __bf16*>(buf + C::K_BYTES);
#pragma unroll
    for (int sub = 0; sub < C::NSUB; ++sub) {
      const int kvalid = item.b - (key0 + sub * C::KSUB);
      if (kvalid >= C::KSUB)
        attend_32<C, false>(Ks, Vs, sub * C::KSUB, C::KSUB, Q, QT, O, m, lsum, c2, lane);
      else if (kvalid > 0)
        attend_32<C, true>(Ks, Vs, sub * C::KSUB, kvalid, Q, QT, O, m, lsum, c2, lane);
    }
  }

  // ---- epilogue: O / l for the rows of this wavefront that lie in the sequence
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const float l = C::SUM_MFMA ? O[C::NDB][qb][0] : sum_4groups(lsum[qb]);
    const float inv = 1.0f / l;
    const int row = row0 + qb * 16 + c;
    if (row < qend) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int d0 = db * 16 + 4 * g;
        if (d0 < C::D) {
          const f32x4_t x = O[db][qb];
          *reinterpret_cast<u32x2_t*>(o + ((size_t)row * n_heads + item.head) * C::D + d0) =
              u32x2_t{cvt_pk_bf16(x[0] * inv, x[1] * inv), cvt_pk_bf16(x[2] * inv, x[3] * inv)};
        }
      }
    }
  }
}

// The bf16 kernel.  CA and CB differ only in the queries per wavefront (CA::QB > CB::QB).
// The launch works with CA's large query blocks unless they would leave most of the grid
// idle (a short single image), in which case it re-plans with CB's small blocks: more
// items, so more of the machine works, each item over the same keys.
template <class CA, class CB>
__global__ __launch_bounds__(CA::NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, const int32_t* __restrict__ cu, int n_seqs, int n_heads, float c2, int negate) {
  static_assert(CA::D == CB::D && CA::NW == CB::NW && CA::BN == CB::BN && CA::STAGE_BYTES == CB::STAGE_BYTES,
                "the two query-block sizes share the staging layout");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  PlanLds& plan = *reinterpret_cast<PlanLds*>(smem);
  unsigned char* stage = smem + ((sizeof(PlanLds) + 15) / 16) * 16;

  const int G = gridDim.x;
  int n_items = build_plan<CA::NT>(plan, cu, n_seqs, n_heads, CA::BM);
  const bool small = 2 * n_items < G;  // the same decision in every workgroup
  if (small) {
    __syncthreads();  // everyone has read the first plan's item count
    n_items = build_plan<CA::NT>(plan, cu, n_seqs, n_heads, CB::BM);
  }
  const int bm = small ? CB::BM : CA::BM;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int slot = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const unsigned row_bytes = (unsigned)n_heads * CA::D * 2u;
  unsigned dma_off[Dma<CA>::PER_WAVE];
  Dma<CA>::init(dma_off, wave, lane, row_bytes);

  // Items in longest-first order are dealt out in rounds of G, alternating direction
  // (round r, slot s -> item r*G + s, or r*G + G-1-s on odd rounds) to even out the load.
  for (int round = 0;; ++round) {
    const int it = round * G + ((round & 1) ? G - 1 - slot : slot);
    if (it >= n_items) break;
    const Item item = map_item(plan, n_seqs, it, bm);
    if (small)
      run_item<CB>(item, q, k, v, o, n_heads, c2, negate, stage, row_bytes, dma_off, wave, lane);
    else
      run_item<CA>(item, q, k, v, o, n_heads, c2, negate, stage, row_bytes, dma_off, wave, lane);
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
KernelDesc describe_f32() {
  KernelDesc d;
  d.func = reinterpret_cast<const void*>(&attn_fwd_f32_kernel<T>);
  d.bm = T::BM;
  d.bn = T::BN;
  d.waves = T::NW;
  d.nt = T::NT;
  d.lds = ((sizeof(PlanLds) + 15) / 16) * 16 + 2 * (size_t)T::STAGE_ELEMS * sizeof(typename T::elem_t);
  return d;
}

template <class C, class CB>
KernelDesc describe_bf16() {
  KernelDesc d;
  d.func = reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<C, CB>);
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
#ifndef VITATTN_BF16_SUM_MFMA
#define VITATTN_BF16_SUM_MFMA true
#endif
#ifndef VITATTN_BF16_QB_SMALL
#define VITATTN_BF16_QB_SMALL 1
#endif
using K_bf16_64 = Bf16Cfg<64, VITATTN_BF16_QB, VITATTN_BF16_NW, 64, VITATTN_BF16_SUM_MFMA>;
using K_bf16_72 = Bf16Cfg<72, VITATTN_BF16_QB, VITATTN_BF16_NW, 64, VITATTN_BF16_SUM_MFMA>;
using K_bf16_80 = Bf16Cfg<80, VITATTN_BF16_QB, VITATTN_BF16_NW, 64, VITATTN_BF16_SUM_MFMA>;
using K_bf16_128 = Bf16Cfg<128, VITATTN_BF16_QB_128, VITATTN_BF16_NW, 64, VITATTN_BF16_SUM_MFMA>;
using S_bf16_64 = Bf16Cfg<64, VITATTN_BF16_QB_SMALL, VITATTN_BF16_NW, 64, VITATTN_BF16_SUM_MFMA>;
using S_bf16_72 = Bf16Cfg<72, VITATTN_BF16_QB_SMALL, VITATTN_BF16_NW, 64, VITATTN_BF16_SUM_MFMA>;
using S_bf16_80 = Bf16Cfg<80, VITATTN_BF16_QB_SMALL, VITATTN_BF16_NW, 64, VITATTN_BF16_SUM_MFMA>;
using S_bf16_128 = Bf16Cfg<128, VITATTN_BF16_QB_SMALL, VITATTN_BF16_NW, 64, VITATTN_BF16_SUM_MFMA>;
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
    case 0: return describe_f32<K_f32_64>();
    case 1: return describe_f32<K_f32_72>();
    case 2: return describe_f32<K_f32_80>();
    case 3: return describe_f32<K_f32_128>();
    case 4: return describe_bf16<K_bf16_64, S_bf16_64>();
    case 5: return describe_bf16<K_bf16_72, S_bf16_72>();
    case 6: return describe_bf16<K_bf16_80, S_bf16_80>();
    default: return describe_bf16<K_bf16_128, S_bf16_128>();
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
