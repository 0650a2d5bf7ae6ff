// fp32 debug path of the sparse attention forward (same contract as the bf16
// MFMA kernel: O, natural-log LSE and exact per-block attention mass over the
// CSR block mask; GSRS page, Abstract and Figure 3 caption).
//
// Plain fp32 FMA arithmetic with precise expf/logf, for checking against the
// float64 oracle at 1e-5.  One workgroup per mask row; TPQ = D/32 threads
// share a query (32 dimensions each); key blocks stream through LDS in
// 32-key chunks and every key is folded into the online softmax one by one.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kChunk = 32;

template <int D>
__global__ void fwd32_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                             const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t cap,
                             float* __restrict__ o, float* __restrict__ lse, float* __restrict__ mass,
                             float* __restrict__ part, int N, int bs, int nb, float scale) {
  constexpr int TPQ = D / 32;
  __shared__ float ks[kChunk][D + 1];
  __shared__ float vs[kChunk][D + 1];
  __shared__ float lse_s[128];
  __shared__ float red[16];
  const int r = blockIdx.x;
  const int bh = r / nb, i = r - bh * nb;
  const int tid = threadIdx.x;
  const int ql = tid / TPQ, sl = tid % TPQ;     // query in block, 32-dim slice
  const int q0 = i * bs, nq = min(bs, N - q0);
  const int qq = q0 + ql;
  const bool qvalid = ql < nq;
  int64_t e0 = row_ptr[r], e1 = row_ptr[r + 1];
  if (e1 > cap) e1 = cap;
  if (e0 < 0) e0 = 0;
  if (e0 > e1) e0 = e1;

  float qv[32], acc[32];
  for (int d = 0; d < 32; ++d) {
    qv[d] = qvalid ? q[((size_t)bh * N + qq) * D + sl * 32 + d] : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const size_t head = (size_t)bh * N * D;

  for (int64_t e = e0; e < e1; ++e) {
    const int j = col_idx[e];
    const bool valid = j >= 0 && j < nb;
    float lb = 0.f;   // this block's sum of exp(s - m)
    for (int c0 = 0; valid && c0 < bs; c0 += kChunk) {
      __syncthreads();
      for (int x = tid; x < kChunk * D; x += blockDim.x) {
        const int kr = x / D, d = x % D;
        const int key = j * bs + c0 + kr;
        const bool in = c0 + kr < bs && key < N;
        ks[kr][d] = in ? k[head + (size_t)key * D + d] : 0.f;
        vs[kr][d] = in ? v[head + (size_t)key * D + d] : 0.f;
      }
      __syncthreads();
      for (int kr = 0; kr < kChunk; ++kr) {
        const int key = j * bs + c0 + kr;
        float s = 0.f;
        for (int d = 0; d < 32; ++d) s = fmaf(qv[d], ks[kr][sl * 32 + d], s);
        for (int off = 1; off < TPQ; off <<= 1) s += __shfl_xor(s, off);
        if (c0 + kr >= bs || key >= N) continue;
        s *= scale;
        const float m_new = fmaxf(m, s);
        const float alpha = expf(m - m_new);
        const float p = expf(s - m_new);
        for (int d = 0; d < 32; ++d) acc[d] = fmaf(acc[d], alpha, p * vs[kr][sl * 32 + d]);
        l = l * alpha + p;
        lb = lb * alpha + p;
        m = m_new;
      }
    }
    if (part != nullptr && sl == 0) part[(size_t)e * bs + ql] = lb > 0.f ? m + logf(lb) : -INFINITY;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lsev = l > 0.f ? m + logf(l) : -INFINITY;
  if (qvalid) {
    for (int d = 0; d < 32; ++d) o[((size_t)bh * N + qq) * D + sl * 32 + d] = acc[d] * inv;
    if (sl == 0) lse[(size_t)bh * N + qq] = lsev;
  }
  if (sl == 0) lse_s[ql] = lsev;
  if (mass == nullptr) return;
  __syncthreads();
  const int nthreads = blockDim.x;
  for (int64_t e = e0; e < e1; ++e) {
    const int j = col_idx[e];
    float x = 0.f;
    if (j >= 0 && j < nb)
      for (int t = tid; t < nq; t += nthreads) x += expf(part[(size_t)e * bs + t] - lse_s[t]);
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
    if ((tid & 63) == 0) red[tid >> 6] = x;
    __syncthreads();
    if (tid == 0) {
      float s = 0.f;
      for (int w = 0; w < nthreads / 64; ++w) s += red[w];
      mass[e] = s / (float)nq;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_forward_fp32(const Problem& p, const void* q, const void* k, const void* v, float scale,
                               const bsa_csr* mask, void* o, float* lse, float* mass, const ForwardWs& w,
                               hipStream_t s) {
  const int threads = p.bs * (p.D / 32);
  if (p.D == 64)
    fwd32_kernel<64><<<p.R, threads, 0, s>>>(static_cast<const float*>(q), static_cast<const float*>(k),
                                             static_cast<const float*>(v), mask->row_ptr, mask->col_idx,
                                             mask->capacity, static_cast<float*>(o), lse, mass,
                                             mass ? w.part : nullptr, p.N, p.bs, p.nb, scale);
  else
    fwd32_kernel<128><<<p.R, threads, 0, s>>>(static_cast<const float*>(q), static_cast<const float*>(k),
                                              static_cast<const float*>(v), mask->row_ptr, mask->col_idx,
                                              mask->capacity, static_cast<float*>(o), lse, mass,
                                              mass ? w.part : nullptr, p.N, p.bs, p.nb, scale);
  return hipGetLastError();
}

}  // namespace bsa
