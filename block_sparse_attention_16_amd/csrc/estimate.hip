// Block-importance estimator for dynamic block-sparse attention (gfx950).
//
// Stage one of the two-stage estimate-then-attend scheme (DSV page, Abstract):
// pooled block scores pick, per query block, the key blocks worth visiting.
// Selection is Top-p over a row softmax of the pooled scores (GSRS page,
// Abstract), optionally restricted to an earlier step's blocks ("reduced
// search", GSRS page, Abstract and Figure 4 caption).
//
// Kernels, in launch order:
//   pool_kernel     HBM-streaming mean of Q and K over every token block
//   select_kernel   one row per workgroup: pooled logits over the candidates,
//                   LDS bitonic sort by (logit desc, id asc), fp32 softmax,
//                   prefix sum, Top-p cut, forced prefix blocks -> bitmask
//   scan_kernel     exclusive scan of the per-row counts -> CSR row_ptr
//   compact_kernel  one wavefront per row: bitmask -> ascending col_idx
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kThreads = 256;
constexpr int kSortMax = 4096;   // largest candidate row (nb <= 4096)

template <class T>
struct Load8;
template <>
struct Load8<__bf16> {
  // 8 consecutive bf16 -> 8 floats (one 16-byte load)
  __device__ static void get(const __bf16* p, float* out) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
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

// Mean over the valid tokens of one block, for Q and K at once.
// grid.x = R (one workgroup per (b, h, block)); 256 threads.
// Thread t reads the 8-element chunk (t % (D/8)) of rows t/(D/8), +G, ...
template <class T, int D>
__global__ __launch_bounds__(kThreads) void pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                        float* __restrict__ qbar, float* __restrict__ kbar,
                                                        int N, int bs, int nb) {
  constexpr int CPR = D / 8;            // chunks per row
  constexpr int G = kThreads / CPR;     // row groups
  __shared__ float part[2][G][D];
  const int r = blockIdx.x;             // = bh * nb + i
  const int bh = r / nb, i = r - bh * nb;
  const int lo = i * bs;
  const int nv = min(bs, N - lo);
  const int c = threadIdx.x % CPR, g = threadIdx.x / CPR;
  float sq[8] = {}, sk[8] = {};
  const size_t base = ((size_t)bh * N + lo) * D + c * 8;
  for (int t = g; t < nv; t += G) {
    float a[8], b[8];
    Load8<T>::get(q + base + (size_t)t * D, a);
    Load8<T>::get(k + base + (size_t)t * D, b);
#pragma unroll
    for (int e = 0; e < 8; ++e) { sq[e] += a[e]; sk[e] += b[e]; }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) { part[0][g][c * 8 + e] = sq[e]; part[1][g][c * 8 + e] = sk[e]; }
  __syncthreads();
  if (threadIdx.x < 2 * D) {
    const int which = threadIdx.x / D, d = threadIdx.x % D;
    float s = 0.f;
    for (int gg = 0; gg < G; ++gg) s += part[which][gg][d];
    float* dst = which ? kbar : qbar;
    dst[(size_t)r * D + d] = s / (float)nv;
  }
}

__device__ __forceinline__ uint32_t ordered_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// One mask row per workgroup.  Produces counts[r] and the selection bitmask.
template <int D>
__global__ __launch_bounds__(kThreads) void select_kernel(
    const float* __restrict__ qbar, const float* __restrict__ kbar, int nb, float top_p, float scale,
    const int32_t* __restrict__ cand_ptr, const int32_t* __restrict__ cand_idx, int64_t cand_cap,
    int n_forced, int32_t* __restrict__ counts, uint32_t* __restrict__ bits, int words) {
  __shared__ unsigned long long key[kSortMax];
  __shared__ float pre[kSortMax];
  __shared__ float qrow[D];
  __shared__ float wsum[kThreads / 64];
  __shared__ float tsum[kThreads];
  __shared__ uint32_t sel[kSortMax / 32];
  __shared__ int first_hit;
  __shared__ int nvalid_s;

  const int r = blockIdx.x;
  const int bh = r / nb;
  const int tid = threadIdx.x;

  // candidate range
  int n_c;
  int64_t lo = 0;
  if (cand_ptr) {
    int64_t a = cand_ptr[r], b = cand_ptr[r + 1];
    if (b > cand_cap) b = cand_cap;
    if (a < 0) a = 0;
    if (a > b) a = b;
    lo = a;
    n_c = (int)min<int64_t>(b - a, kSortMax);
  } else {
    n_c = nb;
  }
  int n_pow2 = 1;
  while (n_pow2 < n_c) n_pow2 <<= 1;

  if (tid < D) qrow[tid] = qbar[(size_t)r * D + tid];
  if (tid == 0) { first_hit = 0x7fffffff; nvalid_s = 0; }
  for (int w = tid; w < words; w += kThreads) sel[w] = 0u;
  __syncthreads();

  // pooled logits -> 64-bit sort keys (ordered logit bits << 32 | ~id); 0 = absent
  for (int t = tid; t < n_pow2; t += kThreads) {
    unsigned long long kk = 0ull;
    if (t < n_c) {
      int j = cand_ptr ? cand_idx[lo + t] : t;
      if (j >= 0 && j < nb) {
        const float4* kr = reinterpret_cast<const float4*>(kbar + ((size_t)bh * nb + j) * D);
        float acc = 0.f;
#pragma unroll 8
        for (int d4 = 0; d4 < D / 4; ++d4) {
          float4 v = kr[d4];
          acc = fmaf(qrow[4 * d4 + 0], v.x, acc);
          acc = fmaf(qrow[4 * d4 + 1], v.y, acc);
          acc = fmaf(qrow[4 * d4 + 2], v.z, acc);
          acc = fmaf(qrow[4 * d4 + 3], v.w, acc);
        }
        const float s = acc * scale;
        kk = ((unsigned long long)ordered_bits(s) << 32) | (unsigned long long)(~(uint32_t)j);
      }
    }
    key[t] = kk;
  }
  __syncthreads();

  // bitonic sort, descending
  for (int kk = 2; kk <= n_pow2; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int t = tid; t < (n_pow2 >> 1); t += kThreads) {
        const int a = (t / j) * 2 * j + (t % j);
        const int b = a + j;
        const unsigned long long x = key[a], y = key[b];
        const bool desc = (a & kk) == 0;
        if (desc ? (x < y) : (x > y)) { key[a] = y; key[b] = x; }
      }
      __syncthreads();
    }
  }

  // exp of (logit - max) for valid, non-duplicate entries; per-thread chunk prefix sums
  const float smax = unordered_bits((uint32_t)(key[0] >> 32));
  const int chunk = n_pow2 >= kThreads ? n_pow2 / kThreads : 1;
  const int c0 = tid * chunk;
  float run = 0.f;
  int nv_local = 0;
  for (int t = c0; t < c0 + chunk && t < n_pow2; ++t) {
    const unsigned long long kv = key[t];
    float e = 0.f;
    if (kv != 0ull) {
      ++nv_local;
      const bool dup = t > 0 && key[t - 1] == kv;
      if (!dup) e = expf(unordered_bits((uint32_t)(kv >> 32)) - smax);
    }
    run += e;
    pre[t] = run;
  }
  tsum[tid] = run;
  if (nv_local) atomicAdd(&nvalid_s, nv_local);
  __syncthreads();
  // inclusive scan of the per-thread totals (Hillis-Steele)
  for (int off = 1; off < kThreads; off <<= 1) {
    float v = tid >= off ? tsum[tid - off] : 0.f;
    __syncthreads();
    tsum[tid] += v;
    __syncthreads();
  }
  const float offset = tid > 0 ? tsum[tid - 1] : 0.f;
  const float total = tsum[kThreads - 1];
  const int nvalid = nvalid_s;
  const bool take_all = !(top_p < 1.0f);
  const float thr = top_p * total;
  for (int t = c0; t < c0 + chunk && t < nvalid; ++t) {
    pre[t] += offset;
    if (!take_all && pre[t] >= thr) { atomicMin(&first_hit, t); break; }
  }
  __syncthreads();
  const int last = take_all ? nvalid - 1 : min(first_hit, nvalid - 1);
  for (int t = tid; t <= last; t += kThreads) {
    const unsigned long long kv = key[t];
    const bool dup = t > 0 && key[t - 1] == kv;
    if (!dup) {
      const int j = (int)(~(uint32_t)(kv & 0xffffffffull));
      atomicOr(&sel[j >> 5], 1u << (j & 31));
    }
  }
  for (int j = tid; j < n_forced; j += kThreads) atomicOr(&sel[j >> 5], 1u << (j & 31));
  __syncthreads();

  int cnt = 0;
  for (int w = tid; w < words; w += kThreads) {
    const uint32_t b = sel[w];
    bits[(size_t)r * words + w] = b;
    cnt += __popc(b);
  }
  // block reduction of the count
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = __int_as_float(cnt);
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
    for (int w = 0; w < kThreads / 64; ++w) tot += __float_as_int(wsum[w]);
    counts[r] = tot;
  }
}

// Exclusive scan of counts[R] into row_ptr[R+1]; a single workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts, int32_t* __restrict__ row_ptr,
                                                    int R) {
  __shared__ int wtot[16];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < R; base += 1024) {
    const int idx = base + tid;
    const int v = idx < R ? counts[idx] : 0;
    int x = v;
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wtot[wid] = x;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wid; ++w) wbase += wtot[w];
    const int carry = carry_s;
    if (idx < R) row_ptr[idx] = carry + wbase + x - v;
    __syncthreads();
    if (tid == 1023) carry_s = carry + wbase + x;
    __syncthreads();
  }
  if (tid == 0) row_ptr[R] = carry_s;
}

// One wavefront per row: set bits -> ascending block ids at row_ptr[r].
__global__ __launch_bounds__(kThreads) void compact_kernel(const uint32_t* __restrict__ bits,
                                                           const int32_t* __restrict__ row_ptr,
                                                           int32_t* __restrict__ col_idx, int64_t cap, int R,
                                                           int words) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (r >= R) return;
  int64_t pos_base = row_ptr[r];
  for (int w0 = 0; w0 < words; w0 += 64) {
    const int w = w0 + lane;
    const uint32_t b = w < words ? bits[(size_t)r * words + w] : 0u;
    const int pc = __popc(b);
    int x = pc;
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    int64_t pos = pos_base + x - pc;
    uint32_t m = b;
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      if (pos >= 0 && pos < cap) col_idx[pos] = w * 32 + bit;
      ++pos;
    }
    pos_base += __shfl(x, 63);
  }
}

}  // namespace

EstimateWs carve_estimate(const Problem& p, void* ws, size_t* bytes) {
  Carver c(ws);
  EstimateWs w;
  w.words = (p.nb + 31) / 32;
  w.qbar = c.take<float>((size_t)p.R * p.D);
  w.kbar = c.take<float>((size_t)p.R * p.D);
  w.counts = c.take<int32_t>((size_t)p.R);
  w.bits = c.take<uint32_t>((size_t)p.R * w.words);
  *bytes = align_up(c.off, 256);
  return w;
}

template <class T, int D>
static void launch_pool_select(const Problem& p, const void* q, const void* k, float top_p, float scale,
                               const bsa_csr* cand, int n_forced, const EstimateWs& w, hipStream_t s) {
  pool_kernel<T, D><<<p.R, kThreads, 0, s>>>(static_cast<const T*>(q), static_cast<const T*>(k), w.qbar, w.kbar,
                                             p.N, p.bs, p.nb);
  select_kernel<D><<<p.R, kThreads, 0, s>>>(w.qbar, w.kbar, p.nb, top_p, scale, cand ? cand->row_ptr : nullptr,
                                            cand ? cand->col_idx : nullptr, cand ? cand->capacity : 0, n_forced,
                                            w.counts, w.bits, w.words);
}

hipError_t launch_estimate(const Problem& p, const void* q, const void* k, float top_p, float scale,
                           const bsa_csr* cand, int keep_prefix_tokens, const bsa_csr* out, const EstimateWs& w,
                           hipStream_t s) {
  const int n_forced = min(p.nb, (keep_prefix_tokens + p.bs - 1) / p.bs);
  const bool bf = p.dtype == BSA_BF16;
  if (p.D == 64) {
    if (bf) launch_pool_select<__bf16, 64>(p, q, k, top_p, scale, cand, n_forced, w, s);
    else launch_pool_select<float, 64>(p, q, k, top_p, scale, cand, n_forced, w, s);
  } else {
    if (bf) launch_pool_select<__bf16, 128>(p, q, k, top_p, scale, cand, n_forced, w, s);
    else launch_pool_select<float, 128>(p, q, k, top_p, scale, cand, n_forced, w, s);
  }
  scan_kernel<<<1, 1024, 0, s>>>(w.counts, out->row_ptr, p.R);
  compact_kernel<<<(p.R + 3) / 4, kThreads, 0, s>>>(w.bits, out->row_ptr, out->col_idx, out->capacity, p.R,
                                                    w.words);
  return hipGetLastError();
}

}  // namespace bsa
