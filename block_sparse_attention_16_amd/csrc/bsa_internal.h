// Internal declarations shared by the host API and the HIP kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "bsa.h"

namespace bsa {

// Problem description after host-side validation.
struct Problem {
  int B, H, N, D, bs, nb, R;     // R = B*H*nb mask rows
  int dtype;                     // bsa_dtype
  size_t elem;                   // bytes per element of q/k/v/o
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace carving: every sub-buffer starts on a 256-byte boundary.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <class T>
  T* take(size_t count) {
    off = align_up(off, 256);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

// ---- estimator (estimate.hip) ----
struct EstimateWs {
  float* qbar;       // [R, D] pooled query means
  float* kbar;       // [R * sub_blocks, D] pooled key means (per sub-block)
  int32_t* counts;   // [R] selected blocks per row
  uint32_t* bits;    // [R, words] selection bitmask
  float* logits;     // [R, nb] pooled logits
  int words;         // ceil(nb / 32)
};
EstimateWs carve_estimate(const Problem& p, int sub_blocks, void* ws, size_t* bytes);
// sub_blocks: 1 (mean-pool logits) or 2, 4, 8 (hierarchical block scoring)
hipError_t launch_estimate(const Problem& p, const void* q, const void* k, float top_p, float scale,
                           const bsa_csr* cand, int keep_prefix_tokens, int sub_blocks, const bsa_csr* out,
                           const EstimateWs& w, hipStream_t s);

// ---- mask narrowing from block masses (estimate.hip) ----
struct SelectWs {
  int32_t* counts;   // [R] kept entries per row
  uint32_t* bits;    // [R, words] kept-block bitmask
  int words;
};
SelectWs carve_select(const Problem& p, void* ws, size_t* bytes);
hipError_t launch_select_from_mass(const Problem& p, const bsa_csr* mask, const float* mass, float top_p,
                                   int keep_prefix_tokens, const bsa_csr* out, const SelectWs& w, hipStream_t s);
// Narrowing without a caller workspace: the device address of the library's
// static scratch array on the stream's device (the current device for the
// null stream), looked up once per device.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;   // 16 MiB per GPU
hipError_t scratch_for_stream(hipStream_t stream, void** ptr);

// ---- structured head masks (estimate.hip); same workspace as narrowing ----
hipError_t launch_structured_mask(const Problem& p, const int32_t* head_kind, const bsa_pattern_params& prm,
                                  const bsa_csr* out, const SelectWs& w, hipStream_t s);

// ---- token permutation (permute.hip) ----
hipError_t launch_permute_rows(int64_t heads, int n, int row_bytes, const void* src, const int32_t* perm,
                               bool inverse, void* dst, hipStream_t s);

// ---- longest-first order of a grid's last rows (order.hip) ----
// Rows [R - T, R), T = tail_rows(R), run longest first; order[t] is the row
// that workgroup R - T + t takes.  2048 rows measured best of 1024/2048/4096
// on the four video workloads (four rounds of the 512 resident 128-token
// forward workgroups).
constexpr int kTailRows = 2048;
inline int tail_rows(int R) { return R < kTailRows ? R : kTailRows; }
// Tail of a grid with one workgroup per query block (forward, dQ).  With
// 64-token blocks (two-wave workgroups) 1024 rows measured best on the
// training workload: forward 3 % faster than with 2048 (3072 and 4096
// slower), dQ ~1 % (the dK/dV grid keeps 2048).  With 128-token blocks 2048
// stays best.  At most tail_rows(R), the size of the order arrays.
inline int query_tail_rows(int R, int bs) { return bs == 64 ? (R < 1024 ? R : 1024) : tail_rows(R); }
// Lengths are counts[r] when counts is non-null, else the CSR extents of
// row_ptr clamped to [0, cap].
// Unit lists of the pair grid for 64-token blocks (forward_bf16.hip): P =
// B*H*ceil(nb/2) pairs of rows; units [capacity], ulen [P].
void launch_pair_units(const int32_t* row_ptr, const int32_t* col_idx, int64_t cap, int nb, int P, uint32_t* units,
                       int32_t* ulen, hipStream_t s);
void launch_tail_order(const int32_t* row_ptr, int64_t cap, const int32_t* counts, int r0, int T, int32_t* order,
                       hipStream_t s);

// ---- forward (forward_bf16.hip, forward_fp32.hip) ----
struct ForwardWs {
  float* part;       // [capacity, bs] per-entry, per-query block log-sum-exp (block mass)
  int32_t* order;    // [tail_rows(R)] rows of the grid's tail, longest first
  uint32_t* units;   // bf16, block 64: [capacity] unit lists of the pair grid
  int32_t* ulen;     // bf16, block 64: [B*H*ceil(nb/2)] their lengths
};
ForwardWs carve_forward(const Problem& p, int64_t capacity, bool want_mass, void* ws, size_t* bytes);
hipError_t launch_forward_bf16(const Problem& p, const void* q, const void* k, const void* v, float scale,
                               const bsa_csr* mask, void* o, float* lse, float* mass, float* o32,
                               const ForwardWs& w, hipStream_t s);
hipError_t launch_forward_fp32(const Problem& p, const void* q, const void* k, const void* v, float scale,
                               const bsa_csr* mask, void* o, float* lse, float* mass,
                               const ForwardWs& w, hipStream_t s);

// ---- backward (backward.hip) ----
struct BackwardWs {
  float* delta;        // [B*H, nb*bs] rowsum(dO * O), 0 on padding rows
  float* lse2;         // [B*H, nb*bs] LSE * log2(e), +inf on padding rows
  int32_t* csc_start;  // [B*H*nb] first transposed entry of key-block column (bh, j)
  int32_t* csc_count;  // [B*H*nb] query blocks in that column
  int32_t* csc_row;    // [capacity] query block of each transposed entry
  int32_t* order_q;    // [tail_rows(R)] dQ grid's last rows, longest first
  int32_t* order_k;    // [tail_rows(R)] dK/dV grid's last columns, longest first
  uint32_t* units;     // bf16, block 64: [capacity] unit lists of the dQ pair grid
  int32_t* ulen;       // bf16, block 64: [B*H*ceil(nb/2)] their lengths
};
BackwardWs carve_backward(const Problem& p, int64_t capacity, void* ws, size_t* bytes);
hipError_t launch_backward(const Problem& p, const void* q, const void* k, const void* v, const void* o,
                           const float* o32, const void* d_o, const float* lse, float scale, const bsa_csr* mask,
                           void* dq, void* dk, void* dv, const BackwardWs& w, hipStream_t s);

}  // namespace bsa
