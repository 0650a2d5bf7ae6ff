// Longest-first dispatch of the last rows of a row-parallel grid.
//
// The sparse kernels run one workgroup per mask row, and the rows of a
// dynamic mask differ widely in length (at the HunyuanVideo-like size from 4
// to 631 entries, mean 103).  Dispatched in index order, long rows that fall
// at the end of the grid finish alone while most of the chip idles.  Sorting
// the whole grid longest first removes that tail but interleaves the rows of
// every head, so that rows running at the same time no longer share their K/V
// blocks in the caches: measured slower on every workload.  Only the last T
// rows are therefore reordered: the grid stays head-major up to R - T, and the
// final few rounds of resident workgroups take the long rows first.  Rows are
// independent, so the order never changes a result.
//
// tail_order_kernel: one workgroup counting-sorts the lengths of rows
// [r0, r0 + T) in descending order and writes their row indices to
// order[0, T); rows of equal length keep no particular order.  A row's length
// is counts[r] when counts is given (the columns of a transposed mask), else
// its CSR extent clamped to [0, cap]; either is clamped to 4095 for the sort.
#include "bsa_internal.h"

namespace bsa {
namespace {

constexpr int kBuckets = 4096;
constexpr int kThreads = 1024;   // kBuckets / 4: each thread scans four buckets

__global__ __launch_bounds__(kThreads) void tail_order_kernel(const int32_t* __restrict__ row_ptr, int64_t cap,
                                                              const int32_t* __restrict__ counts, int r0, int T,
                                                              int32_t* __restrict__ order) {
  __shared__ int cnt[kBuckets];
  __shared__ int wsum[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int b = tid; b < kBuckets; b += kThreads) cnt[b] = 0;
  __syncthreads();
  auto len = [&](int r) {
    int64_t n;
    if (counts) {
      n = counts[r];
    } else {
      int64_t a = row_ptr[r], e = row_ptr[r + 1];
      if (e > cap) e = cap;
      if (a < 0) a = 0;
      n = e - a;
    }
    return (int)(n < 0 ? 0 : (n > kBuckets - 1 ? kBuckets - 1 : n));
  };
  for (int t = tid; t < T; t += kThreads) atomicAdd(&cnt[len(r0 + t)], 1);
  __syncthreads();
  // Exclusive scan over the buckets from the longest length down: thread t
  // owns buckets kBuckets-1-4t .. kBuckets-4-4t.
  int loc[4], s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    loc[j] = cnt[kBuckets - 1 - (4 * tid + j)];
    s += loc[j];
  }
  int x = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  int run = x - s;
  for (int w = 0; w < wid; ++w) run += wsum[w];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    cnt[kBuckets - 1 - (4 * tid + j)] = run;
    run += loc[j];
  }
  __syncthreads();
  for (int t = tid; t < T; t += kThreads) order[atomicAdd(&cnt[len(r0 + t)], 1)] = r0 + t;
}

}  // namespace

void launch_tail_order(const int32_t* row_ptr, int64_t cap, const int32_t* counts, int r0, int T, int32_t* order,
                       hipStream_t s) {
  if (T > 0) tail_order_kernel<<<1, kThreads, 0, s>>>(row_ptr, cap, counts, r0, T, order);
}

}  // namespace bsa
