// Block-importance estimator for dynamic block-sparse attention (gfx950).
//
// Stage one of the two-stage estimate-then-attend scheme (DSV page, Abstract):
// pooled block scores pick, per query block, the key blocks worth visiting.
// Selection is Top-p over a row softmax of the pooled scores (GSRS page,
// Abstract), optionally restricted to an earlier step's blocks ("reduced
// search", GSRS page, Abstract and Figure 4 caption).
//
// Kernels, in launch order:
//   pool_kernel     HBM-streaming mean of Q and K over every token block (K
//                   also per sub-block for hierarchical block scoring)
//   logits_kernel   pooled logits scale * Qbar Kbar^T per head, an fp32 GEMM
//                   on the matrix cores in 64 x 64 tiles; with sub-blocks, a
//                   block's logit is the log-sum-exp of its sub-blocks' (the
//                   reading of the DFSAttn page's hierarchical block scoring,
//                   Abstract)
//   select_full_kernel  (every block a candidate) one wavefront per row:
//                   softmax over the row, Top-p cut found by bisection on the
//                   ordered logit bits (no sort; it stops once a single block
//                   is left in the cut's range), ties at the cut broken by
//                   lower block id, forced prefix blocks; the selection of
//                   64 blocks is one ballot -> selection bitmask
//   select_kernel   the same rule over each row's candidate blocks (reduced
//                   search); the whole CSR row is streamed through a
//                   per-wavefront bitmask indexed by block id, so repeats
//                   count once -> selection bitmask
//   csr_kernel      per workgroup of 8 rows: sum of the earlier rows' counts,
//                   scan of its own -> CSR row_ptr; bitmasks -> ascending
//                   col_idx (one wavefront per 2 rows, 64 blocks per store)
//
// Mask narrowing (GSRS page, Abstract and Figure 4 caption: exact attention
// weights, later searches restricted to an earlier step's blocks) reuses
// select_kernel in its FROM_MASS form -- the weights are a CSR row's block
// masses instead of exp(logit - max) -- followed by the same csr_kernel.
//
// Structured head masks (SVG page, Abstract: spatial and temporal heads;
// Sparse-vDiT page, Abstract: diagonal, multi-diagonal and vertical-stripe
// patterns): pattern_kernel evaluates the block relation of each row's head
// with interval arithmetic on frames and spatial positions, one key block per
// lane, into the same bitmask, then the same csr_kernel.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kThreads = 256;
constexpr int kSortMax = 4096;   // largest candidate row (nb <= 4096)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <class T>
struct Load8;
template <>
struct Load8<__bf16> {
  // 8 consecutive bf16 -> 8 floats (one 16-byte load).  Non-temporal: each
  // element is read once, so the load does not allocate in the caches
  // (measured 5-10 % faster pooling, the following forward unchanged).
  __device__ static void get(const __bf16* p, float* out) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Load8<float> {
  __device__ static void get(const float* p, float* out) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
};

// Mean over the valid tokens of one block, for Q and K at once; K also per
// sub-block when GS > 1 (GS sub-blocks of BS / GS tokens, for hierarchical
// block scoring).  grid.x = rows from r0 (one workgroup per (b, h, block));
// 256 threads.  Thread t reads the 8-element chunk (t % (D/8)) of G = 256 /
// (D/8) row groups; row group g serves sub-block m = g % GS, rows
// m * BS/GS + g / GS + it * G/GS, so each thread's K rows stay in one
// sub-block (GS = 1: rows g, g + G, ...).  A full block (the common case)
// issues all of a thread's loads before summing any.
template <class T, int D, int BS, int GS>
__global__ __launch_bounds__(kThreads) void pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                        float* __restrict__ qbar, float* __restrict__ kbar,
                                                        int N, int nb, int r0) {
  constexpr int CPR = D / 8;            // chunks per row
  constexpr int G = kThreads / CPR;     // row groups
  constexpr int GG = G / GS;            // row groups per sub-block
  constexpr int W = BS / GS;            // rows per sub-block
  constexpr int ITER = W / GG;          // rows per thread in a full block (= BS / G)
  static_assert(GS <= G && W % GG == 0, "sub-blocks must split over the row groups");
  __shared__ float part[2][G][D];
  const int r = r0 + blockIdx.x;        // = bh * nb + i
  const int bh = r / nb, i = r - bh * nb;
  const int lo = i * BS;
  const int nv = min(BS, N - lo);
  const int c = threadIdx.x % CPR, g = threadIdx.x / CPR;
  const int m = g % GS, gg = g / GS;
  const int t0 = m * W + gg;            // first row of this thread; then + GG per step
  float sq[8] = {}, sk[8] = {};
  const size_t base = ((size_t)bh * N + lo) * D + c * 8;
  if (nv == BS) {
    float a[ITER][8], b[ITER][8];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      Load8<T>::get(q + base + (size_t)(t0 + it * GG) * D, a[it]);
      Load8<T>::get(k + base + (size_t)(t0 + it * GG) * D, b[it]);
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it)
#pragma unroll
      for (int e = 0; e < 8; ++e) { sq[e] += a[it][e]; sk[e] += b[it][e]; }
  } else {
    for (int it = 0; it < ITER; ++it) {
      const int t = t0 + it * GG;
      if (t >= nv) break;               // rows of a sub-block ascend with it
      float a[8], b[8];
      Load8<T>::get(q + base + (size_t)t * D, a);
      Load8<T>::get(k + base + (size_t)t * D, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) { sq[e] += a[e]; sk[e] += b[e]; }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) { part[0][g][c * 8 + e] = sq[e]; part[1][g][c * 8 + e] = sk[e]; }
  __syncthreads();
  for (int x = threadIdx.x; x < D + GS * D; x += kThreads) {
    if (x < D) {
      float s = 0.f;
      for (int g2 = 0; g2 < G; ++g2) s += part[0][g2][x];
      qbar[(size_t)r * D + x] = s / (float)nv;
    } else {
      const int ms = (x - D) / D, d = (x - D) % D;
      const int cnt = max(0, min(W, nv - ms * W));
      float s = 0.f;
      for (int g2 = 0; g2 < GG; ++g2) s += part[1][g2 * GS + ms][d];
      kbar[((size_t)r * GS + ms) * D + d] = cnt > 0 ? s / (float)cnt : 0.f;
    }
  }
}

__device__ __forceinline__ uint32_t ordered_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Lane exchange through DPP (a VALU move from another lane of the same row).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
// Max and sum over aligned groups of GS consecutive lanes (GS = 2, 4, 8):
// DPP quad permutes for lanes ^ 1 and ^ 2, ds_bpermute for ^ 4.
template <int GS>
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, __uint_as_float(dpp<0xB1>(__float_as_uint(x))));       // quad_perm [1,0,3,2]
  if constexpr (GS >= 4) x = fmaxf(x, __uint_as_float(dpp<0x4E>(__float_as_uint(x))));   // [2,3,0,1]
  if constexpr (GS >= 8) x = fmaxf(x, __shfl_xor(x, 4));
  return x;
}
template <int GS>
__device__ __forceinline__ float group_sum(float x) {
  x += __uint_as_float(dpp<0xB1>(__float_as_uint(x)));
  if constexpr (GS >= 4) x += __uint_as_float(dpp<0x4E>(__float_as_uint(x)));
  if constexpr (GS >= 8) x += __shfl_xor(x, 4);
  return x;
}

// Pooled logits L[bh, i, j] = scale * <Qbar_i, Kbar_j> for one 64 x 64 tile
// of one head on the fp32 matrix cores (v_mfma_f32_32x32x2_f32: fp32
// products, fp32 accumulation, twice the rate of the vector FMA path).  256
// threads; wave w computes the 32 x 32 sub-tile (w / 2, w % 2), d summed in
// ascending pairs.  With GS > 1 the 64 columns are key sub-blocks (GS per
// block) and the epilogue writes each block's logit as the natural
// log-sum-exp of its non-empty sub-blocks' logits (GS consecutive lanes;
// max and sum by lane exchanges, exp2 / log2 on the transcendental unit).
// grid (ceil(nb * GS / 64), ceil(nb / 64), heads from bh0).
typedef float floatx16 __attribute__((ext_vector_type(16)));
template <int D, int GS>
__global__ __launch_bounds__(kThreads) void logits_kernel(const float* __restrict__ qbar,
                                                          const float* __restrict__ kbar,
                                                          float* __restrict__ logits, int nb, float scale,
                                                          int bh0, int N, int bs) {
  // 64 x DC slices of Qbar and Kbar go to LDS transposed to [d][row] (row
  // padded to 68), every 16-byte load of a slice in flight before its
  // stores; lanes cover 64 rows of one 4-wide d slice, so the transposed LDS
  // writes are conflict free.  Then DC / 2 MFMAs per slice.
  constexpr int DC = 32;   // 32: best of 32 / 64 / D measured (more resident workgroups)
  __shared__ __attribute__((aligned(16))) float qs[DC][68];
  __shared__ __attribute__((aligned(16))) float ks[DC][68];
  const int nk = nb * GS;                 // key columns (blocks or sub-blocks)
  const int j0 = blockIdx.x * 64, i0 = blockIdx.y * 64, bh = bh0 + blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = (wave >> 1) * 32, wj = (wave & 1) * 32;
  const int l32 = lane & 31, hi = lane >> 5;
  const float* qh = qbar + (size_t)bh * nb * D;
  const float* kh = kbar + (size_t)bh * nk * D;
  constexpr int LOADS = 64 * DC / 4 / kThreads;  // float4 loads per thread, matrix and slice
  floatx16 acc = {};
  for (int d0 = 0; d0 < D; d0 += DC) {
    float4 qa[LOADS], ka[LOADS];
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int x = tid + it * kThreads, row = x & 63, c4 = x >> 6;
      qa[it] = i0 + row < nb ? *reinterpret_cast<const float4*>(qh + (size_t)(i0 + row) * D + d0 + 4 * c4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
      ka[it] = j0 + row < nk ? *reinterpret_cast<const float4*>(kh + (size_t)(j0 + row) * D + d0 + 4 * c4)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int x = tid + it * kThreads, row = x & 63, c4 = x >> 6;
      qs[4 * c4][row] = qa[it].x; qs[4 * c4 + 1][row] = qa[it].y;
      qs[4 * c4 + 2][row] = qa[it].z; qs[4 * c4 + 3][row] = qa[it].w;
      ks[4 * c4][row] = ka[it].x; ks[4 * c4 + 1][row] = ka[it].y;
      ks[4 * c4 + 2][row] = ka[it].z; ks[4 * c4 + 3][row] = ka[it].w;
    }
    __syncthreads();
    // A[m][k] = Qbar[wi + m][d0 + kk + k] from lane m + 32k; B[k][n] = Kbar[wj + n][d0 + kk + k]
#pragma unroll 8
    for (int kk = 0; kk < DC; kk += 2)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(qs[kk + hi][wi + l32], ks[kk + hi][wj + l32], acc, 0, 0, 0);
    __syncthreads();
  }
  // accumulator element v of lane l: row 8(v/4) + 4(l/32) + v%4, column l%32
  const int jc = j0 + wj + l32;
  if constexpr (GS == 1) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = i0 + wi + 8 * (v >> 2) + 4 * hi + (v & 3);
      if (i < nb && jc < nb) logits[((size_t)bh * nb + i) * nb + jc] = acc[v] * scale;
    }
  } else {
    const int jb = jc / GS, ms = jc % GS;
    const bool live = jc < nk && jb * bs + ms * (bs / GS) < N;   // sub-block holds a token
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float x = live ? acc[v] * scale : -INFINITY;
      // a written block (jb < nb) has a token in sub-block 0: mx finite, e >= 1
      const float mx = group_max<GS>(x);
      const float e = group_sum<GS>(live ? __builtin_amdgcn_exp2f((x - mx) * kLog2e) : 0.f);
      const int i = i0 + wi + 8 * (v >> 2) + 4 * hi + (v & 3);
      if (ms == 0 && i < nb && jb < nb)
        logits[((size_t)bh * nb + i) * nb + jb] = mx + __builtin_amdgcn_logf(e) * kLn2;
    }
  }
}

// Wave-wide reductions as a butterfly of VALU lane exchanges: DPP quad
// permutes (lane ^ 1, lane ^ 2), DPP row mirrors (within 8, within 16 lanes),
// then v_permlane16_swap (rows 0<->1, 2<->3) and v_permlane32_swap (halves).
// Each step combines a lane's value with its partner's; partners hold the
// same two operands, so with a commutative op every lane ends with the
// bitwise-same result (no LDS traffic, unlike ds_bpermute shuffles).
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t x, Op op) {
  x = op(x, dpp<0xB1>(x));    // quad_perm [1,0,3,2]
  x = op(x, dpp<0x4E>(x));    // quad_perm [2,3,0,1]
  x = op(x, dpp<0x141>(x));   // row_half_mirror
  x = op(x, dpp<0x140>(x));   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(b[0], b[1]);
}
__device__ __forceinline__ float wave_sum(float x) {
  return __uint_as_float(wave_reduce(__float_as_uint(x), [](uint32_t u, uint32_t v) {
    return __float_as_uint(__uint_as_float(u) + __uint_as_float(v));
  }));
}
__device__ __forceinline__ int wave_sum_i(int x) {
  return (int)wave_reduce((uint32_t)x, [](uint32_t u, uint32_t v) { return u + v; });
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  return wave_reduce(x, [](uint32_t u, uint32_t v) { return u > v ? u : v; });
}
__device__ __forceinline__ float wave_fmax(float x) {
  return __uint_as_float(wave_reduce(__float_as_uint(x), [](uint32_t u, uint32_t v) {
    return __float_as_uint(fmaxf(__uint_as_float(u), __uint_as_float(v)));
  }));
}
// Uniform copy of a value that every lane already holds.
__device__ __forceinline__ float uniform(float x) {
  return __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(x)));
}

// Early end of the bisection for the cut key.  Once bit b is decided the cut
// lies in [T, T + 2^b) (T's lower bits are zero), with M(T) >= p Z and
// M(T + 2^b) < p Z.  If exactly one present block's key x falls in that
// range, M is constant on [T, x] and on (x, T + 2^b], so the cut is x.
// Ballots count the blocks in range; the result is wave-uniform.  Tied keys
// in range keep the bisection going.
template <int EPL>
__device__ __forceinline__ bool isolated_cut(const uint32_t (&key)[EPL], uint32_t T, int b, uint32_t& cut) {
  int n = 0;
  uint32_t kin = 0u;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const bool in = key[e] != 0u && (key[e] ^ T) < (1u << b);
    n += __popcll(__ballot(in));
    kin = in ? key[e] : kin;
  }
  if (n != 1) return false;
  cut = __builtin_amdgcn_readfirstlane(wave_umax(kin));
  return true;
}
// Bits after which the bisection tests for an isolated cut (steps 12, 16,
// 20 and 24 of 32): on the video workloads' pooled logits the cut key is
// alone in its range after 15-17 steps on average.
__device__ __forceinline__ constexpr bool isolation_check(int bit) {
  return bit == 20 || bit == 16 || bit == 12 || bit == 8;
}

// Top-p over one mask row held in registers, one row per wavefront: lane l
// holds blocks j = 64e + l, e < EPL.  key[e] is the order-preserving bit
// pattern of the block's sort value (its logit, or its mass when narrowing),
// 0 for a block that is not a candidate; ev[e] is its weight, exp(s - max)
// or the mass (0 when absent).  With M(T) = sum of the weights of blocks whose
// key is >= T and Z = M(1), the cut key L* is the largest T with
// M(T) >= p Z, found bit by bit from the top; every block above L* is kept,
// and blocks exactly at L* are added in ascending id until the mass reaches
// p Z.  That is the shortest prefix of the (value desc, id asc) ranking whose
// cumulative share reaches p, summed in another order.  Forced blocks
// (j < n_forced) join after the cut.  The selection of element e is one
// ballot, whose halves are bitmask words 2e and 2e + 1.
template <int EPL>
__device__ __forceinline__ void select_row(const uint32_t (&key)[EPL], const float (&ev)[EPL], float top_p,
                                           int nb, int n_forced, int r, int32_t* __restrict__ counts,
                                           uint32_t* __restrict__ bits, int words, int lane) {
  float zl = 0.f;
  bool any = false;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    zl += ev[e];
    any = any || key[e] != 0u;
  }
  const float Z = uniform(wave_sum(zl));
  uint32_t cut = 1u;                         // keep every present block by default
  int k_tie = -1;                            // >= 0: tied blocks at the cut to add
  if (top_p < 1.0f && Z > 0.f && __any(any)) {
    const float thr = top_p * Z;
    uint32_t T = 0u;
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t c = T | (1u << bit);
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) m += key[e] >= c ? ev[e] : 0.f;
      if (uniform(wave_sum(m)) >= thr) T = c;
      if (isolation_check(bit) && isolated_cut<EPL>(key, T, bit, T)) break;
    }
    cut = T;                                 // L*: M(L*) >= p Z > M(L* + 1)
    int nt = 0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) nt += key[e] == T ? 1 : 0;
    const int n_tie = __builtin_amdgcn_readfirstlane(wave_sum_i(nt));
    if (n_tie > 1) {
      float mg = 0.f, et = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        mg += key[e] > T ? ev[e] : 0.f;
        if (key[e] == T) et = ev[e];
      }
      const float m_gt = uniform(wave_sum(mg));
      const float etie = uniform(wave_fmax(et));   // tied blocks share one weight
      // add tied blocks one at a time, as a walk in ascending id would
      float acc = m_gt;
      k_tie = 0;
      while (k_tie < n_tie) {
        acc += etie;
        ++k_tie;
        if (acc >= thr) break;
      }
    }
  }
  const int forced = min(n_forced, nb);
  int cnt = 0, tied_before = 0;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const bool present = key[e] != 0u;
    bool take = present && (k_tie >= 0 ? key[e] > cut : key[e] >= cut);
    if (k_tie >= 0) {
      const bool tied = present && key[e] == cut;
      const uint64_t tb = __ballot(tied);
      const int rank = tied_before + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(tb >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)tb, 0u));
      take = take || (tied && rank < k_tie);
      tied_before += __popcll(tb);
    }
    uint64_t sel = __ballot(take);
    const int nf = forced - e * 64;          // forced blocks j < n_forced in this element
    if (nf > 0) sel |= nf >= 64 ? ~0ull : ((1ull << nf) - 1ull);
    cnt += __popcll(sel);
    const int w = 2 * e + (lane & 1);
    if (lane < 2 && w < words) bits[(size_t)r * words + w] = (uint32_t)(sel >> (32 * (lane & 1)));
  }
  if (lane == 0) counts[r] = cnt;
}

// Weights exp(s - max) of a row of logits held as (key, value) pairs; absent
// blocks (key 0) get weight 0.
template <int EPL>
__device__ __forceinline__ void softmax_weights(const uint32_t (&key)[EPL], float (&ev)[EPL]) {
  uint32_t kmax = 0u;
#pragma unroll
  for (int e = 0; e < EPL; ++e) kmax = max(kmax, key[e]);
  kmax = wave_umax(kmax);
  const float smax = kmax ? unordered_bits(kmax) : 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) ev[e] = key[e] ? __builtin_amdgcn_exp2f((ev[e] - smax) * kLog2e) : 0.f;
}

// Full search (every block a candidate): one mask row per wavefront, 4 per
// workgroup, the row's pooled logits read from `logits` [R, nb].
template <int EPL>
__global__ __launch_bounds__(kThreads) void select_full_kernel(const float* __restrict__ logits, int nb, int R,
                                                               float top_p, int n_forced,
                                                               int32_t* __restrict__ counts,
                                                               uint32_t* __restrict__ bits, int words) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (r >= R) return;                        // whole wavefront leaves together
  const float* lrow = logits + (size_t)r * nb;
  uint32_t key[EPL];                         // ordered logit bits; 0 = no block
  float ev[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int t = e * 64 + lane;
    const bool ok = t < nb;
    const float sv = lrow[ok ? t : 0];
    key[e] = ok ? ordered_bits(sv) : 0u;
    ev[e] = sv;
  }
  softmax_weights<EPL>(key, ev);
  select_row<EPL>(key, ev, top_p, nb, n_forced, r, counts, bits, words, lane);
}

// Rows read from a CSR over the same R rows (one row per wavefront, 4 per
// workgroup), every entry of a row, in chunks of 64: reduced search scores
// only the blocks a row lists (the softmax is over them alone); narrowing
// (FROM_MASS) ranks them by the block masses aligned with the CSR entries.
// A block id marks its slot (lane j % 64, element j / 64) in a per-wavefront
// LDS bitmask, so repeats count once whatever their order; FROM_MASS keeps
// the first listing's position with an LDS atomicMin and reads that entry's
// mass (a negative or NaN mass counts as 0).  Ids outside [0, nb) and entries
// at or past cand_cap are ignored; a row is read up to 2^31 - 1 entries.
template <int EPL, bool FROM_MASS>
__global__ __launch_bounds__(kThreads) void select_kernel(
    const float* __restrict__ logits, int nb, int R, float top_p, const int32_t* __restrict__ cand_ptr,
    const int32_t* __restrict__ cand_idx, int64_t cand_cap, int n_forced, int32_t* __restrict__ counts,
    uint32_t* __restrict__ bits, int words) {
  constexpr int L = EPL * 64;                // block slots of a row
  constexpr int NF = FROM_MASS ? L : 1;
  __shared__ uint32_t seen[kThreads / 64][L / 32];
  __shared__ int32_t first[kThreads / 64][NF];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r = blockIdx.x * (kThreads / 64) + wid;
  if (r >= R) return;                        // whole wavefront leaves together
  uint32_t* my_seen = seen[wid];
  int32_t* my_first = first[wid];
  for (int w = lane; w < L / 32; w += 64) my_seen[w] = 0u;
  if constexpr (FROM_MASS)
    for (int t = lane; t < L; t += 64) my_first[t] = 0x7fffffff;
  __builtin_amdgcn_wave_barrier();

  int64_t a = cand_ptr[r], b = cand_ptr[r + 1];
  if (b > cand_cap) b = cand_cap;
  if (a < 0) a = 0;
  if (a > b) a = b;
  const int n = (int)min<int64_t>(b - a, 0x7fffffff);
  for (int t0 = 0; t0 < n; t0 += 64) {
    const int t = t0 + lane;
    const int j = t < n ? cand_idx[a + t] : -1;
    if (j >= 0 && j < nb) {
      atomicOr(&my_seen[j >> 5], 1u << (j & 31));
      if constexpr (FROM_MASS) atomicMin(&my_first[j], t);
    }
  }
  __builtin_amdgcn_wave_barrier();

  uint32_t key[EPL];
  float ev[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const int j = e * 64 + lane;
    const bool present = j < nb && ((my_seen[j >> 5] >> (j & 31)) & 1u);
    float sv = 0.f;
    if (present) {
      if constexpr (FROM_MASS) {
        const float m = logits[a + my_first[j]];
        sv = m > 0.f ? m : 0.f;              // NaN compares false
      } else {
        sv = logits[(size_t)r * nb + j];
      }
    }
    key[e] = present ? ordered_bits(sv) : 0u;  // finite values order above 0
    ev[e] = sv;
  }
  if constexpr (!FROM_MASS) softmax_weights<EPL>(key, ev);
  select_row<EPL>(key, ev, top_p, nb, n_forced, r, counts, bits, words, lane);
}

// CSR assembly in one launch.  Workgroup b takes rows [8b, 8b + 8): it sums
// the counts of every earlier row (16-byte loads, wave and workgroup sums;
// at most R counts, read from L2), scans its own 8 counts across lanes and
// writes their row_ptr (and row_ptr[R]).  Then each wavefront writes 2 rows'
// ids: for every 64 blocks of a row's bitmask (two words, uniform), lane l
// stores block 64c + l at the row offset plus the number of set bits below
// its own (mbcnt), so a row takes one masked store per 64 blocks.  Ids at
// positions >= cap are dropped; row_ptr keeps the exact offsets.
constexpr int kCsrRowsPerWave = 2;   // 2 of 2 / 4 / 8 measured best (more workgroups)
constexpr int kCsrRows = 4 * kCsrRowsPerWave;     // rows per workgroup (<= 64)

// Blocks j0 .. j0 + 63 of one row, selected by the 64-bit mask (hi:lo),
// written from position pos on in ascending order.
__device__ __forceinline__ void emit64(uint32_t lo, uint32_t hi, int j0, int64_t pos, int32_t* __restrict__ col_idx,
                                       int64_t cap, int lane) {
  const uint32_t word = lane < 32 ? lo : hi;
  const bool set = (word >> (lane & 31)) & 1u;
  const int rank = (int)__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
  const int64_t at = pos + rank;
  if (set && at < cap) col_idx[at] = j0 + lane;
}

__global__ __launch_bounds__(kThreads) void csr_kernel(const int32_t* __restrict__ counts,
                                                       const uint32_t* __restrict__ bits,
                                                       int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
                                                       int64_t cap, int R, int words) {
  constexpr int RW = kCsrRowsPerWave;
  __shared__ int wsum[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r0 = blockIdx.x * kCsrRows;            // a multiple of 4
  int s = 0;
  const int4* c4 = reinterpret_cast<const int4*>(counts);
  const int n4 = r0 / 4;
  int x = tid;
  for (; x + 7 * kThreads < n4; x += 8 * kThreads) {   // eight 16-byte loads in flight per thread
    int4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = c4[x + u * kThreads];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u].x + v[u].y + v[u].z + v[u].w;
  }
  for (; x < n4; x += kThreads) {
    const int4 v = c4[x];
    s += v.x + v.y + v.z + v.w;
  }
  s = wave_sum_i(s);
  if (lane == 0) wsum[wid] = s;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) base += wsum[w];
  const int cx = (lane < kCsrRows && r0 + lane < R) ? counts[r0 + lane] : 0;
  int inc = cx;                                    // inclusive scan over lanes
#pragma unroll
  for (int off = 1; off < kCsrRows; off <<= 1) {
    const int y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  const int exc = inc - cx;                        // offset of row r0 + lane within the workgroup
  if (wid == 0 && lane < kCsrRows && r0 + lane < R) {
    row_ptr[r0 + lane] = base + exc;
    if (r0 + lane == R - 1) row_ptr[R] = base + inc;
  }
  const int x0 = wid * RW;
  if (words <= 64) {                               // a row's words in one load (lane w: word w), 8 rows at once
    uint32_t bw[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      const int r = r0 + x0 + j;
      bw[j] = (r < R && lane < words) ? bits[(size_t)r * words + lane] : 0u;
    }
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      int64_t pos = (int64_t)base + __builtin_amdgcn_readlane(exc, x0 + j);
      for (int c = 0; c < words; c += 2) {
        const uint32_t lo = __builtin_amdgcn_readlane(bw[j], c);
        const uint32_t hi = c + 1 < words ? __builtin_amdgcn_readlane(bw[j], c + 1) : 0u;
        emit64(lo, hi, c * 32, pos, col_idx, cap, lane);
        pos += __popc(lo) + __popc(hi);
      }
    }
  } else {
    for (int j = 0; j < RW; ++j) {
      const int r = r0 + x0 + j;
      if (r >= R) break;
      int64_t pos = (int64_t)base + __builtin_amdgcn_readlane(exc, x0 + j);
      const uint32_t* row = bits + (size_t)r * words;
      for (int c = 0; c < words; c += 2) {
        const uint32_t lo = row[c];
        const uint32_t hi = c + 1 < words ? row[c + 1] : 0u;
        emit64(lo, hi, c * 32, pos, col_idx, cap, lane);
        pos += __popc(lo) + __popc(hi);
      }
    }
  }
}

// Token range of block i and its video part, in the frame geometry of the
// structured patterns (tokens [0, prefix) are text; video token n is at frame
// (n - prefix) / F, spatial index (n - prefix) % F).
struct BlockGeo {
  int vlo, hi;     // video tokens [vlo, hi); empty when vlo >= hi
  bool text;       // the block holds a text token
};
__device__ __forceinline__ BlockGeo block_geo(int i, int bs, int N, int prefix) {
  const int lo = i * bs, hi = min(lo + bs, N);
  return {max(lo, prefix), hi, lo < prefix};
}
// Spatial positions of a block's video tokens as up to two intervals.
__device__ __forceinline__ int spot_intervals(const BlockGeo& g, int prefix, int F, int (&a)[2], int (&b)[2]) {
  const int len = g.hi - g.vlo;
  if (len >= F) { a[0] = 0; b[0] = F - 1; return 1; }
  const int s0 = (g.vlo - prefix) % F, s1 = (g.hi - 1 - prefix) % F;
  if (s0 <= s1) { a[0] = s0; b[0] = s1; return 1; }
  a[0] = s0; b[0] = F - 1; a[1] = 0; b[1] = s1;
  return 2;
}

// One wavefront per mask row: the row's key blocks under its head's pattern
// -> selection bitmask and count, one block per lane and one ballot (two
// bitmask words) per 64 blocks.  Unknown kinds give dense rows.
__global__ __launch_bounds__(kThreads) void pattern_kernel(const int32_t* __restrict__ head_kind, int nb, int R,
                                                           int N, int bs, int prefix, int F, int band, int period,
                                                           const int32_t* __restrict__ stripes, int n_stripes,
                                                           int32_t* __restrict__ counts, uint32_t* __restrict__ bits,
                                                           int words) {
  __shared__ uint32_t stripe_bits[kSortMax / 32];
  for (int w = threadIdx.x; w < words; w += kThreads) stripe_bits[w] = 0u;
  __syncthreads();
  for (int t = threadIdx.x; t < n_stripes; t += kThreads) {
    const int j = stripes[t];
    if (j >= 0 && j < nb) atomicOr(&stripe_bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r = blockIdx.x * (kThreads / 64) + wid;
  if (r >= R) return;
  const int i = r % nb;
  const int kind = head_kind[r / nb];
  const BlockGeo gi = block_geo(i, bs, N, prefix);
  const bool vi = gi.vlo < gi.hi;
  int ai[2], bi[2], ni = 0;
  if (kind == BSA_PATTERN_TEMPORAL && vi) ni = spot_intervals(gi, prefix, F, ai, bi);
  const int fi0 = vi ? (gi.vlo - prefix) / F : 0, fi1 = vi ? (gi.hi - 1 - prefix) / F : -1;
  int cnt = 0;
  for (int j0 = 0; j0 < nb; j0 += 64) {      // lane l decides block j0 + l; one ballot per 64 blocks
    const int j = j0 + lane;
    bool keep = false;
    if (j < nb) {
      const BlockGeo gj = block_geo(j, bs, N, prefix);
      const bool vj = gj.vlo < gj.hi;
      const int d = i - j;
      if (gi.text || gj.text) {
        keep = true;
      } else if (kind == BSA_PATTERN_SPATIAL) {
        const int fj0 = (gj.vlo - prefix) / F, fj1 = (gj.hi - 1 - prefix) / F;
        keep = vi && vj && fi0 <= fj1 && fj0 <= fi1;
      } else if (kind == BSA_PATTERN_TEMPORAL) {
        if (vi && vj) {
          int aj[2], bj[2];
          const int nj = spot_intervals(gj, prefix, F, aj, bj);
          for (int x = 0; x < ni; ++x)
            for (int y = 0; y < nj; ++y) keep = keep || (ai[x] <= bj[y] && aj[y] <= bi[x]);
        }
      } else if (kind == BSA_PATTERN_DIAGONAL) {
        keep = abs(d) <= band;
      } else if (kind == BSA_PATTERN_MULTI_DIAGONAL) {
        const int m = ((d % period) + period) % period;
        keep = min(m, period - m) <= band;
      } else if (kind == BSA_PATTERN_STRIPES) {
        keep = ((stripe_bits[j >> 5] >> (j & 31)) & 1u) || abs(d) <= band;
      } else {
        keep = true;                         // BSA_PATTERN_DENSE and unknown kinds
      }
    }
    const uint64_t sel = __ballot(keep);
    const int w = j0 / 32 + (lane & 1);      // bitmask words 2c and 2c + 1
    if (lane < 2 && w < words) bits[(size_t)r * words + w] = (uint32_t)(sel >> (32 * (lane & 1)));
    cnt += __popcll(sel);
  }
  if (lane == 0) counts[r] = cnt;
}

}  // namespace

EstimateWs carve_estimate(const Problem& p, int sub_blocks, void* ws, size_t* bytes) {
  Carver c(ws);
  EstimateWs w;
  w.words = (p.nb + 31) / 32;
  w.qbar = c.take<float>((size_t)p.R * p.D);
  w.kbar = c.take<float>((size_t)p.R * sub_blocks * p.D);
  w.counts = c.take<int32_t>((size_t)p.R);
  w.bits = c.take<uint32_t>((size_t)p.R * w.words);
  w.logits = c.take<float>((size_t)p.R * p.nb);
  *bytes = align_up(c.off, 256);
  return w;
}

template <class T, int D, int GS>
static void launch_pool_logits(const Problem& p, const void* q, const void* k, float scale, const EstimateWs& w,
                               hipStream_t s) {
  if (p.bs == 128)
    pool_kernel<T, D, 128, GS><<<p.R, kThreads, 0, s>>>(static_cast<const T*>(q), static_cast<const T*>(k), w.qbar,
                                                        w.kbar, p.N, p.nb, 0);
  else
    pool_kernel<T, D, 64, GS><<<p.R, kThreads, 0, s>>>(static_cast<const T*>(q), static_cast<const T*>(k), w.qbar,
                                                       w.kbar, p.N, p.nb, 0);
  const dim3 g((p.nb * GS + 63) / 64, (p.nb + 63) / 64, p.B * p.H);
  logits_kernel<D, GS><<<g, kThreads, 0, s>>>(w.qbar, w.kbar, w.logits, p.nb, scale, 0, p.N, p.bs);
}

template <class T, int D>
static void launch_pool_logits_gs(const Problem& p, const void* q, const void* k, float scale, int sub_blocks,
                                  const EstimateWs& w, hipStream_t s) {
  switch (sub_blocks) {
    case 1: launch_pool_logits<T, D, 1>(p, q, k, scale, w, s); break;
    case 2: launch_pool_logits<T, D, 2>(p, q, k, scale, w, s); break;
    case 4: launch_pool_logits<T, D, 4>(p, q, k, scale, w, s); break;
    default: launch_pool_logits<T, D, 8>(p, q, k, scale, w, s); break;
  }
}

template <int EPL, bool FROM_MASS>
static void launch_select(const Problem& p, const float* vals, float top_p, const bsa_csr* cand, int n_forced,
                          int32_t* counts, uint32_t* bits, int words, hipStream_t s) {
  select_kernel<EPL, FROM_MASS><<<(p.R + 3) / 4, kThreads, 0, s>>>(
      vals, p.nb, p.R, top_p, cand ? cand->row_ptr : nullptr, cand ? cand->col_idx : nullptr,
      cand ? cand->capacity : 0, n_forced, counts, bits, words);
}

template <bool FROM_MASS>
static void launch_select_any(const Problem& p, const float* vals, float top_p, const bsa_csr* cand, int n_forced,
                              int32_t* counts, uint32_t* bits, int words, hipStream_t s) {
  if (p.nb <= 64) launch_select<1, FROM_MASS>(p, vals, top_p, cand, n_forced, counts, bits, words, s);
  else if (p.nb <= 256) launch_select<4, FROM_MASS>(p, vals, top_p, cand, n_forced, counts, bits, words, s);
  else if (p.nb <= 1024) launch_select<16, FROM_MASS>(p, vals, top_p, cand, n_forced, counts, bits, words, s);
  else launch_select<64, FROM_MASS>(p, vals, top_p, cand, n_forced, counts, bits, words, s);
}

static void launch_csr(const Problem& p, const int32_t* counts, const uint32_t* bits, int words, const bsa_csr* out,
                       hipStream_t s) {
  csr_kernel<<<(p.R + kCsrRows - 1) / kCsrRows, kThreads, 0, s>>>(counts, bits, out->row_ptr, out->col_idx,
                                                                  out->capacity, p.R, words);
}

hipError_t launch_estimate(const Problem& p, const void* q, const void* k, float top_p, float scale,
                           const bsa_csr* cand, int keep_prefix_tokens, int sub_blocks, const bsa_csr* out,
                           const EstimateWs& w, hipStream_t s) {
  const int n_forced = min(p.nb, (keep_prefix_tokens + p.bs - 1) / p.bs);
  const bool bf = p.dtype == BSA_BF16;
  if (p.D == 64) {
    if (bf) launch_pool_logits_gs<__bf16, 64>(p, q, k, scale, sub_blocks, w, s);
    else launch_pool_logits_gs<float, 64>(p, q, k, scale, sub_blocks, w, s);
  } else {
    if (bf) launch_pool_logits_gs<__bf16, 128>(p, q, k, scale, sub_blocks, w, s);
    else launch_pool_logits_gs<float, 128>(p, q, k, scale, sub_blocks, w, s);
  }
  if (cand) {
    launch_select_any<false>(p, w.logits, top_p, cand, n_forced, w.counts, w.bits, w.words, s);
  } else {
    const unsigned g = (unsigned)((p.R + 3) / 4);
    if (p.nb <= 64)
      select_full_kernel<1><<<g, kThreads, 0, s>>>(w.logits, p.nb, p.R, top_p, n_forced, w.counts, w.bits, w.words);
    else if (p.nb <= 256)
      select_full_kernel<4><<<g, kThreads, 0, s>>>(w.logits, p.nb, p.R, top_p, n_forced, w.counts, w.bits, w.words);
    else if (p.nb <= 1024)
      select_full_kernel<16><<<g, kThreads, 0, s>>>(w.logits, p.nb, p.R, top_p, n_forced, w.counts, w.bits,
                                                   w.words);
    else
      select_full_kernel<64><<<g, kThreads, 0, s>>>(w.logits, p.nb, p.R, top_p, n_forced, w.counts, w.bits,
                                                   w.words);
  }
  launch_csr(p, w.counts, w.bits, w.words, out, s);
  return hipGetLastError();
}

SelectWs carve_select(const Problem& p, void* ws, size_t* bytes) {
  Carver c(ws);
  SelectWs w;
  w.words = (p.nb + 31) / 32;
  w.counts = c.take<int32_t>((size_t)p.R);
  w.bits = c.take<uint32_t>((size_t)p.R * w.words);
  *bytes = align_up(c.off, 256);
  return w;
}

hipError_t launch_select_from_mass(const Problem& p, const bsa_csr* mask, const float* mass, float top_p,
                                   int keep_prefix_tokens, const bsa_csr* out, const SelectWs& w, hipStream_t s) {
  const int n_forced = min(p.nb, (keep_prefix_tokens + p.bs - 1) / p.bs);
  launch_select_any<true>(p, mass, top_p, mask, n_forced, w.counts, w.bits, w.words, s);
  launch_csr(p, w.counts, w.bits, w.words, out, s);
  return hipGetLastError();
}

hipError_t launch_structured_mask(const Problem& p, const int32_t* head_kind, const bsa_pattern_params& prm,
                                  const bsa_csr* out, const SelectWs& w, hipStream_t s) {
  pattern_kernel<<<(p.R + 3) / 4, kThreads, 0, s>>>(head_kind, p.nb, p.R, p.N, p.bs, prm.prefix_tokens,
                                                    prm.frame_tokens, prm.band, prm.period, prm.stripes,
                                                    prm.n_stripes, w.counts, w.bits, w.words);
  launch_csr(p, w.counts, w.bits, w.words, out, s);
  return hipGetLastError();
}

}  // namespace bsa
