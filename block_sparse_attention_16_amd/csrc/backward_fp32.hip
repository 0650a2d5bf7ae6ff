// fp32 debug path of the sparse attention backward (same contract as the bf16
// MFMA kernels; gradient of the sparse forward used for training with dynamic
// sparsity, DSV page, Abstract).
//
// Plain fp32 FMA arithmetic for checking against the float64 oracle at 1e-5.
// dq32: one workgroup per mask row, TPQ = D/32 threads per query.
// dkv32: one workgroup per key block (CSC column), TPQ threads per key.
// Key (or query) blocks stream through LDS in 32-row chunks.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kChunk = 32;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__global__ void dq32_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                            const float* __restrict__ dout, const float* __restrict__ delta,
                            const float* __restrict__ lse2, const int32_t* __restrict__ row_ptr,
                            const int32_t* __restrict__ col_idx, int64_t cap, float* __restrict__ dq, int N, int bs,
                            int nb, float scale) {
  constexpr int TPQ = D / 32;
  __shared__ float ks[kChunk][D + 1];
  __shared__ float vs[kChunk][D + 1];
  const int r = blockIdx.x;
  const int bh = r / nb, i = r - bh * nb;
  const int tid = threadIdx.x;
  const int ql = tid / TPQ, sl = tid % TPQ;
  const int qq = i * bs + ql;
  const bool qvalid = qq < N;
  int64_t e0 = row_ptr[r], e1 = row_ptr[r + 1];
  if (e1 > cap) e1 = cap;
  if (e0 < 0) e0 = 0;
  if (e0 > e1) e0 = e1;
  const size_t head = (size_t)bh * N * D;
  float qv[32], gv[32], acc[32];
  for (int d = 0; d < 32; ++d) {
    qv[d] = qvalid ? q[head + (size_t)qq * D + sl * 32 + d] : 0.f;
    gv[d] = qvalid ? dout[head + (size_t)qq * D + sl * 32 + d] : 0.f;
    acc[d] = 0.f;
  }
  const size_t prow = (size_t)bh * nb * bs + (size_t)i * bs + ql;
  const float my_lse2 = lse2[prow], my_delta = delta[prow];
  const float c2 = scale * kLog2e;
  for (int64_t e = e0; e < e1; ++e) {
    const int j = col_idx[e];
    if (j < 0 || j >= nb) continue;
    for (int c0 = 0; c0 < bs; c0 += kChunk) {
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
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < 32; ++d) {
          s = fmaf(qv[d], ks[kr][sl * 32 + d], s);
          dp = fmaf(gv[d], vs[kr][sl * 32 + d], dp);
        }
        for (int off = 1; off < TPQ; off <<= 1) {
          s += __shfl_xor(s, off);
          dp += __shfl_xor(dp, off);
        }
        if (c0 + kr >= bs || key >= N || !qvalid) continue;
        const float p = exp2f(s * c2 - my_lse2);
        const float ds = p * (dp - my_delta);
        for (int d = 0; d < 32; ++d) acc[d] = fmaf(ds, ks[kr][sl * 32 + d], acc[d]);
      }
    }
  }
  if (qvalid)
    for (int d = 0; d < 32; ++d) dq[head + (size_t)qq * D + sl * 32 + d] = acc[d] * scale;
}

template <int D>
__global__ void dkv32_kernel(const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                             const float* __restrict__ dout, const float* __restrict__ delta,
                             const float* __restrict__ lse2, const int32_t* __restrict__ csc_start,
                             const int32_t* __restrict__ csc_count, const int32_t* __restrict__ csc_row,
                             float* __restrict__ dk, float* __restrict__ dv, int N, int bs, int nb, float scale) {
  constexpr int TPQ = D / 32;
  __shared__ float qs[kChunk][D + 1];
  __shared__ float gs[kChunk][D + 1];
  __shared__ float ls[kChunk], dl[kChunk];
  const int c = blockIdx.x;
  const int bh = c / nb, j = c - bh * nb;
  const int tid = threadIdx.x;
  const int kl = tid / TPQ, sl = tid % TPQ;
  const int kk = j * bs + kl;
  const bool kvalid = kk < N;
  const size_t head = (size_t)bh * N * D;
  float kv[32], vv[32], ak[32], av[32];
  for (int d = 0; d < 32; ++d) {
    kv[d] = kvalid ? k[head + (size_t)kk * D + sl * 32 + d] : 0.f;
    vv[d] = kvalid ? v[head + (size_t)kk * D + sl * 32 + d] : 0.f;
    ak[d] = 0.f;
    av[d] = 0.f;
  }
  const float c2 = scale * kLog2e;
  const int start = csc_start[c], n = csc_count[c];
  for (int it = 0; it < n; ++it) {
    const int i = csc_row[start + it];
    if (i < 0 || i >= nb) continue;
    for (int c0 = 0; c0 < bs; c0 += kChunk) {
      __syncthreads();
      for (int x = tid; x < kChunk * D; x += blockDim.x) {
        const int qr = x / D, d = x % D;
        const int qq = i * bs + c0 + qr;
        const bool in = c0 + qr < bs && qq < N;
        qs[qr][d] = in ? q[head + (size_t)qq * D + d] : 0.f;
        gs[qr][d] = in ? dout[head + (size_t)qq * D + d] : 0.f;
      }
      for (int x = tid; x < kChunk; x += blockDim.x) {
        const size_t prow = (size_t)bh * nb * bs + (size_t)i * bs + c0 + x;
        const bool in = c0 + x < bs;
        ls[x] = in ? lse2[prow] : INFINITY;
        dl[x] = in ? delta[prow] : 0.f;
      }
      __syncthreads();
      for (int qr = 0; qr < kChunk; ++qr) {
        float s = 0.f, dp = 0.f;
        for (int d = 0; d < 32; ++d) {
          s = fmaf(kv[d], qs[qr][sl * 32 + d], s);
          dp = fmaf(vv[d], gs[qr][sl * 32 + d], dp);
        }
        for (int off = 1; off < TPQ; off <<= 1) {
          s += __shfl_xor(s, off);
          dp += __shfl_xor(dp, off);
        }
        if (!kvalid || c0 + qr >= bs || i * bs + c0 + qr >= N) continue;
        const float p = exp2f(s * c2 - ls[qr]);
        const float ds = p * (dp - dl[qr]);
        for (int d = 0; d < 32; ++d) {
          av[d] = fmaf(p, gs[qr][sl * 32 + d], av[d]);
          ak[d] = fmaf(ds, qs[qr][sl * 32 + d], ak[d]);
        }
      }
    }
  }
  if (kvalid)
    for (int d = 0; d < 32; ++d) {
      dk[head + (size_t)kk * D + sl * 32 + d] = ak[d] * scale;
      dv[head + (size_t)kk * D + sl * 32 + d] = av[d];
    }
}

}  // namespace

hipError_t launch_backward_fp32(const Problem& p, const void* q, const void* k, const void* v, const void* d_o,
                                float scale, const bsa_csr* mask, void* dq, void* dk, void* dv,
                                const BackwardWs& w, hipStream_t s) {
  const int threads = p.bs * (p.D / 32);
  const float* fq = static_cast<const float*>(q);
  const float* fk = static_cast<const float*>(k);
  const float* fv = static_cast<const float*>(v);
  const float* fg = static_cast<const float*>(d_o);
  if (p.D == 64) {
    dq32_kernel<64><<<p.R, threads, 0, s>>>(fq, fk, fv, fg, w.delta, w.lse2, mask->row_ptr, mask->col_idx,
                                            mask->capacity, static_cast<float*>(dq), p.N, p.bs, p.nb, scale);
    dkv32_kernel<64><<<p.R, threads, 0, s>>>(fq, fk, fv, fg, w.delta, w.lse2, w.csc_start, w.csc_count, w.csc_row,
                                             static_cast<float*>(dk), static_cast<float*>(dv), p.N, p.bs, p.nb,
                                             scale);
  } else {
    dq32_kernel<128><<<p.R, threads, 0, s>>>(fq, fk, fv, fg, w.delta, w.lse2, mask->row_ptr, mask->col_idx,
                                             mask->capacity, static_cast<float*>(dq), p.N, p.bs, p.nb, scale);
    dkv32_kernel<128><<<p.R, threads, 0, s>>>(fq, fk, fv, fg, w.delta, w.lse2, w.csc_start, w.csc_count, w.csc_row,
                                              static_cast<float*>(dk), static_cast<float*>(dv), p.N, p.bs, p.nb,
                                              scale);
  }
  return hipGetLastError();
}

}  // namespace bsa
