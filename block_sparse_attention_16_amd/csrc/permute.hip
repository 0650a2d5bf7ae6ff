// Token permutation (layout transformation), an HBM-streaming gather/scatter.
//
// Reordering tokens along a space-filling curve keeps space-time neighbours
// in the same block (DFSAttn page, Abstract; GSRS page, Figure 1, 3 and 6
// captions); the SVG page (Abstract) pairs its kernels with a layout
// transformation of the tensors.  The reorder is a pure data movement of
// [heads, n, row_bytes] slabs: gather dst[h, t] = src[h, perm[t]] into the
// new order, scatter dst[h, perm[t]] = src[h, t] back.
//
// Each thread moves VEC bytes (16 when rows and pointers allow it); a unit
// index enumerates the destination (gather) or the source (scatter) in memory
// order, so one side streams contiguously and the other reads or writes whole
// rows.
#include "bsa_internal.h"

namespace bsa {
namespace {

template <int VEC>
struct Vec;
template <>
struct Vec<16> { typedef uint32_t T __attribute__((ext_vector_type(4))); };
template <>
struct Vec<4> { using T = uint32_t; };

template <int VEC, bool INVERSE>
__global__ __launch_bounds__(256) void permute_kernel(const char* __restrict__ src, const int32_t* __restrict__ perm,
                                                      char* __restrict__ dst, int n, int upr, int total_units) {
  using T = typename Vec<VEC>::T;
  constexpr int K = 4;                               // units per thread per step, loads before stores
  const int stride = gridDim.x * 256;
  for (int u0 = blockIdx.x * 256 + threadIdx.x; u0 < total_units; u0 += K * stride) {
    T v[K];
    size_t to[K];
    bool ok[K];
#pragma unroll
    for (int x = 0; x < K; ++x) {
      const int u = u0 + x * stride;
      ok[x] = false;
      to[x] = 0;
      v[x] = T{};
      if (u < total_units) {
        const int row = u / upr, c = u - row * upr;      // row = h * n + t
        const int h = row / n, t = row - h * n;
        const int p = perm[t];
        const bool okp = p >= 0 && p < n;
        const size_t other = ((size_t)h * n + (okp ? p : 0)) * upr + c;
        if constexpr (!INVERSE) {
          if (okp) v[x] = __builtin_nontemporal_load(reinterpret_cast<const T*>(src) + other);
          to[x] = (size_t)u;
          ok[x] = true;
        } else {
          v[x] = __builtin_nontemporal_load(reinterpret_cast<const T*>(src) + u);
          to[x] = other;
          ok[x] = okp;
        }
      }
    }
#pragma unroll
    for (int x = 0; x < K; ++x)
      if (ok[x]) __builtin_nontemporal_store(v[x], reinterpret_cast<T*>(dst) + to[x]);
  }
}

template <int VEC>
hipError_t launch_vec(int64_t heads, int n, int row_bytes, const void* src, const int32_t* perm, bool inverse,
                      void* dst, hipStream_t s) {
  const int upr = row_bytes / VEC;
  const int64_t total = heads * n * upr;
  const int blocks = (int)std::min<int64_t>((total + 255) / 256, 256 * 64);
  if (inverse)
    permute_kernel<VEC, true><<<blocks, 256, 0, s>>>(static_cast<const char*>(src), perm, static_cast<char*>(dst), n,
                                                     upr, (int)total);
  else
    permute_kernel<VEC, false><<<blocks, 256, 0, s>>>(static_cast<const char*>(src), perm, static_cast<char*>(dst),
                                                      n, upr, (int)total);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute_rows(int64_t heads, int n, int row_bytes, const void* src, const int32_t* perm,
                               bool inverse, void* dst, hipStream_t s) {
  const bool v16 = row_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(src) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
  return v16 ? launch_vec<16>(heads, n, row_bytes, src, perm, inverse, dst, s)
             : launch_vec<4>(heads, n, row_bytes, src, perm, inverse, dst, s);
}

}  // namespace bsa
