// Sparse attention backward over a block mask, bf16 MFMA (gfx950).
//
// The DSV page (Abstract) trains video DiTs with dynamic sparse attention;
// this is the gradient of the sparse forward for a loss with dL/dO = dO,
// over the same CSR block mask.  With P = exp(scale Q_i K_j^T - LSE):
//   dV_j += P^T dO_i,  dP = dO_i V_j^T,  dS = P * (dP - delta),
//   dQ_i += scale dS K_j,  dK_j += scale dS^T Q_i,  delta_q = dO_q . O_q.
// Deterministic, no floating-point atomics: dQ is produced query-major over
// the CSR rows, dK/dV key-major over a transposed (CSC) copy of the mask.
//
// Kernels, in launch order:
//   delta_kernel  lse2 = LSE * log2(e), padded per head to nb*BS rows (padding
//                 +inf -> P = 0); with an fp32 O (the fp32 path, or the
//                 forward's fp32 copy of a bf16 O) also delta = rowsum(dO * O)
//   csc_kernel    one workgroup per head: counting transpose of the mask, rows
//                 visited in order so every column lists query blocks ascending
//   dq_kernel     per query block: S^T = K Q^T, dP^T = V dO^T; without a
//                 given delta, pass 1 computes delta = sum_k P dP; then
//                 dQ^T += K^T dS^T
//   dkv_kernel    per key block:   S = Q K^T,   dP = dO V^T,
//                 dV^T += dO^T P,  dK^T += Q^T dS
//
// MFMA layouts are those of the forward kernel: v_mfma_f32_32x32x16_bf16,
// operands read from LDS tiles either row-wise (ds_read_b128) or transposed
// (two ds_read_b64_tr_b16), the 32x32 accumulator of a lane holding one
// column and 16 rows {8a + 4h + r}, and the k-slot permutation that lets an
// accumulator, rounded to bf16, feed the next MFMA as its B operand.
//
// Like the forward, both MFMA kernels stream their operand through LDS with
// buffer loads straight into LDS (exact LDS wait counts while a copy is in
// flight; reads past the end return zeros); block ids come ahead through
// vector loads; operand reads run ahead of the MFMAs under scheduling fences.
// dq_kernel double-buffers units of SUB keys at two waves per SIMD.
// dkv_kernel streams 32-query tiles through three LDS slots and is
// software-pipelined one tile deep (at D = 128 its registers allow one wave
// per SIMD, so its VALU work must run under its own MFMAs).  Both grids
// dispatch their last rows longest first (order.hip).
#include <type_traits>

#include "bsa_internal.h"

namespace bsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef short short4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// One XOR swizzle of 16-byte chunks that is bank-conflict free both for
// ds_read_b128 down 16 consecutive rows and for ds_read_b64_tr_b16 over
// 4 consecutive rows x 4 chunks (rows of CPR = 16 or 8 chunks).
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  static_assert(CPR == 16 || CPR == 8, "row must be 128 or 256 bytes");
  return CPR == 16 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

__device__ __forceinline__ short4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
}

// Raw buffer resource over `bytes` bytes at base; reads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// 16 (or 4) bytes per lane from buffer offset `off` into LDS at
// lds_wave_base + 16 (or 4) * lane.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t off, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16, off, 0,
                                           0, 0);
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t off, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 4, off, 0,
                                           0, 0);
}

template <int BS, int D>
struct BCfg {
  static constexpr int NW = BS / 32;          // waves; wave w owns 32 rows (queries or keys)
  static constexpr int THREADS = NW * 64;
  static constexpr int SUB = (BS == 64 && D == 128) ? 32 : 64;   // streamed rows per unit
  static constexpr int KC = SUB / 32;         // 32-row tiles per unit
  static constexpr int U = BS / SUB;          // units per block
  static constexpr int DS = D / 16, DT = D / 32;
  static constexpr int CPR = D / 8;
  static constexpr int TILE_BYTES = SUB * D * 2;
  static constexpr int LOADS = TILE_BYTES / (16 * THREADS);
  static_assert(LOADS * 16 * THREADS == TILE_BYTES, "tile must split evenly over the waves");
  static_assert(4 * TILE_BYTES * (8 / NW) <= 160 * 1024, "LDS of two waves per SIMD");
};

// Per-lane byte offset, within a SUB-row window of a [N, D] bf16 matrix, of
// the 16-byte chunk that dma op `it` of this lane stores (lane l of a wave
// writes LDS chunk base + l; the swizzle decides which logical chunk lands there).
template <int BS, int D>
__device__ __forceinline__ uint32_t dma_src_off(int it, int wave, int lane) {
  using C = BCfg<BS, D>;
  const int L = (it * C::NW + wave) * 64 + lane;
  const int row = L / C::CPR, pos = L % C::CPR;
  return (uint32_t)((row * D + (pos ^ swz<C::CPR>(row)) * 8) * 2);
}

// DMA rows [row0, row0 + SUB) of two heads' [N, D] bf16 matrices into
// swizzled LDS tiles (rows past N read as zeros).
template <int BS, int D>
__device__ __forceinline__ void dma_tiles(__amdgpu_buffer_rsrc_t a, __amdgpu_buffer_rsrc_t b, int row0, char* ta,
                                          char* tb, int wave, const uint32_t (&off)[BCfg<BS, D>::LOADS]) {
  using C = BCfg<BS, D>;
  const uint32_t base = (uint32_t)row0 * (D * 2);
#pragma unroll
  for (int it = 0; it < C::LOADS; ++it) {
    lds_dma16(a, base + off[it], ta + (it * C::NW + wave) * 64 * 16);
    lds_dma16(b, base + off[it], tb + (it * C::NW + wave) * 64 * 16);
  }
}

// 8 bf16 of row `row`, logical chunk `c`, of a swizzled tile (MFMA A operand).
template <int CPR>
__device__ __forceinline__ bf16x8 read_row8(const char* t, int row, int c) {
  return *reinterpret_cast<const bf16x8*>(t + (row * CPR + (c ^ swz<CPR>(row))) * 16);
}

// Transposed A operand: lane L receives tile[r0 + 8x + 4(L/32) + t][d0 + L%32]
// in k-slot 4x + t (the slot order of an accumulator used as B operand).
template <int CPR>
__device__ __forceinline__ bf16x8 read_tr8(const char* t, int r0, int d0, int lane) {
  const int G = lane >> 4, tr = (lane >> 2) & 3, g4 = lane & 3;
  const int dcol = d0 + 16 * (G & 1) + 4 * g4;
  short4_t h[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int row = r0 + 8 * x + 4 * (G >> 1) + tr;
    h[x] = lds_read_tr16(t + (row * CPR + ((dcol >> 3) ^ swz<CPR>(row))) * 16 + (dcol & 7) * 2);
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ bf16x8 to_bf16x8(const floatx16& a, int half) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)a[half * 8 + e];
  return r;
}

// Two 32x32 accumulators of one 32-row tile: X = A1 B1 and Y = A2 B2 over
// the d dimension, A operands read row-wise from tiles ta / tb (rows
// r0 + l32), B operands in registers.  Reads run AHEAD k-steps in front.
template <int D>
__device__ __forceinline__ void two_products(const char* ta, const char* tb, const bf16x8 (&ba)[D / 16],
                                             const bf16x8 (&bb)[D / 16], floatx16& x, floatx16& y, int r0, int l32,
                                             int hf) {
  constexpr int DS = D / 16, CPR = D / 8, AHEAD = 2;
  const floatx16 zero = {};
  bf16x8 fa[DS], fb[DS];
#pragma unroll
  for (int ds = 0; ds < AHEAD; ++ds) {
    fa[ds] = read_row8<CPR>(ta, r0 + l32, ds * 2 + hf);
    fb[ds] = read_row8<CPR>(tb, r0 + l32, ds * 2 + hf);
  }
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    __builtin_amdgcn_sched_barrier(0);
    if (ds + AHEAD < DS) {
      fa[ds + AHEAD] = read_row8<CPR>(ta, r0 + l32, (ds + AHEAD) * 2 + hf);
      fb[ds + AHEAD] = read_row8<CPR>(tb, r0 + l32, (ds + AHEAD) * 2 + hf);
    }
    x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ds], ba[ds], ds == 0 ? zero : x, 0, 0, 0);
    y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ds], bb[ds], ds == 0 ? zero : y, 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// delta = rowsum(dO * O), lse2 = LSE * log2(e); [BH, nb*BS] with padding rows.
// ---------------------------------------------------------------------------
template <class TO, class TG, int D>
__global__ __launch_bounds__(256) void delta_kernel(const TO* __restrict__ o, const TG* __restrict__ dout,
                                                    const float* __restrict__ lse, float* __restrict__ delta,
                                                    float* __restrict__ lse2, int N, int npad, int BH,
                                                    int with_delta) {
  constexpr int LPR = D / 8;                       // lanes per row, 8 elements each
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int row = gid / LPR, part = gid % LPR;     // row over BH * npad
  if (row >= BH * npad) return;
  const int bh = row / npad, t = row % npad;
  float s = 0.f;
  if (with_delta && t < N) {
    const size_t off = ((size_t)bh * N + t) * D + part * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += (float)o[off + e] * (float)dout[off + e];
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) s += __shfl_xor(s, m);
  if (part == 0) {
    if (with_delta) delta[row] = s;
    lse2[row] = t < N ? lse[(size_t)bh * N + t] * kLog2e : INFINITY;
  }
}

// ---------------------------------------------------------------------------
// CSC transpose: column (bh, j) lists the query blocks i whose row holds j,
// ascending; csc_start/csc_count index csc_row.  One workgroup of 1024
// threads per head.  The head's rows split into T contiguous chunks, one per
// wavefront (T = 16, fewer when nb > 1024, so the per-chunk column counts fit
// in LDS).  Each wavefront counts its chunk's entries per column.  One scan
// over (column, chunk) gives every chunk its cursor into each column.  Each
// wavefront then writes its rows in order, so every column lists its rows
// ascending without a barrier per row.
// ---------------------------------------------------------------------------
constexpr int kCscThreads = 1024;
constexpr int kCscLds = 16384;            // ints of per-chunk column counters

__global__ __launch_bounds__(kCscThreads) void csc_kernel(const int32_t* __restrict__ row_ptr,
                                                          const int32_t* __restrict__ col_idx, int64_t cap, int nb,
                                                          int32_t* __restrict__ csc_start,
                                                          int32_t* __restrict__ csc_count,
                                                          int32_t* __restrict__ csc_row) {
  __shared__ int cnt[kCscLds];            // [T][nb]: counts, then cursors
  __shared__ int64_t rp[4097];            // the head's clamped row offsets
  __shared__ int wsum[kCscThreads / 64];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int T = min(kCscThreads / 64, kCscLds / nb);     // row chunks (>= 4 for nb <= 4096)
  const int rows_per = (nb + T - 1) / T;
  auto clampe = [&](int64_t e) { return e < 0 ? (int64_t)0 : (e > cap ? cap : e); };
  for (int i = tid; i <= nb; i += kCscThreads) rp[i] = clampe(row_ptr[(size_t)bh * nb + i]);
  for (int x = tid; x < T * nb; x += kCscThreads) cnt[x] = 0;
  __syncthreads();
  const int64_t hb = rp[0], he = rp[nb];
  const int r0 = w * rows_per, r1 = min(nb, r0 + rows_per);
  if (w < T) {
    int* mine = cnt + w * nb;
    for (int i = r0; i < r1; ++i) {
      const int64_t a = max(rp[i], hb), b = min(rp[i + 1], he);
      for (int64_t e = a + lane; e < b; e += 64) {
        const int j = col_idx[e];
        if (j >= 0 && j < nb) atomicAdd(&mine[j], 1);
      }
    }
  }
  __syncthreads();
  // column totals and their exclusive scan; each thread owns consecutive columns
  const int chunk = (nb + kCscThreads - 1) / kCscThreads;
  const int c0 = tid * chunk;
  int run = 0;
  for (int j = c0; j < c0 + chunk && j < nb; ++j)
    for (int c = 0; c < T; ++c) run += cnt[c * nb + j];
  int x = run;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int base = (int)hb + x - run;
  for (int ww = 0; ww < w; ++ww) base += wsum[ww];
  for (int j = c0; j < c0 + chunk && j < nb; ++j) {
    int pos = base;
    for (int c = 0; c < T; ++c) {          // chunk c's cursor into column j
      const int v = cnt[c * nb + j];
      cnt[c * nb + j] = pos;
      pos += v;
    }
    csc_start[(size_t)bh * nb + j] = base;
    csc_count[(size_t)bh * nb + j] = pos - base;
    base = pos;
  }
  __syncthreads();
  // fill: each wavefront writes its rows in ascending order
  if (w < T) {
    int* cur = cnt + w * nb;
    for (int i = r0; i < r1; ++i) {
      const int64_t a = max(rp[i], hb), b = min(rp[i + 1], he);
      for (int64_t e = a + lane; e < b; e += 64) {
        const int j = col_idx[e];
        if (j >= 0 && j < nb) {
          const int pos = atomicAdd(&cur[j], 1);       // distinct slots even for a repeated id
          if (pos >= hb && pos < he) csc_row[pos] = i;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per query block (mask row).  Wave w owns queries
// [32w, 32w+32); per unit (SUB keys of a visited key block, tiles K, V in LDS):
//   S^T = K Q^T, P^T = exp2(c2 S^T - lse2_q), dP^T = V dO^T.
// Without a given delta (delta_given = 0), pass 1 accumulates
// delta_q = sum_k P dP over the row in fp32 (equal to dO_q . O_q for the
// exact O, without the rounding of a bf16 O) and stores it for the dK/dV
// kernel; the last pass forms dS^T = P^T (dP^T - delta_q) and
// dQ^T += K^T dS^T.
// ---------------------------------------------------------------------------
// PAIR (64-token blocks): as in the forward, a 128-query workgroup takes the
// mask rows of query blocks 2m and 2m + 1 (waves 0-1 and 2-3) and walks the
// pair's unit list (64-key blocks flagged with the rows that list them); a
// wave takes P = 0 on a unit its row does not list, which adds exact zeros.
template <int BS, int D, bool PAIR = false>
__global__ __launch_bounds__(2 * BS, 2) void dq_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, float* __restrict__ delta, const float* __restrict__ lse2,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t cap,
    __bf16* __restrict__ dq, int N, int nb, float scale, int delta_given, const int32_t* __restrict__ order,
    int t0, const uint32_t* __restrict__ units, const int32_t* __restrict__ ulen) {
  using C = BCfg<BS, D>;
  static_assert(!PAIR || BS == 128, "a pair of 64-token query blocks fills a 128-query workgroup");
  constexpr int KB = PAIR ? 64 : BS;          // tokens per key block and per mask row's query block
  constexpr int UPE = PAIR ? 1 : C::U;        // units per listed key block
  __shared__ __attribute__((aligned(1024))) char k0s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILE_BYTES];

  // head-major rows up to t0, the grid's last rows longest first (order)
  const int r = (int)blockIdx.x < t0 ? (int)blockIdx.x : order[blockIdx.x - t0];
  const int nbw = PAIR ? (nb + 1) / 2 : nb;  // workgroup rows per head
  const int bh = r / nbw, i = r - bh * nbw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int qloc = wave * 32 + l32;
  const int qq = i * BS + qloc;
  const int wrow = PAIR ? (wave >> 1) : 0;    // pair: row 2i (waves 0-1) or 2i + 1 (waves 2-3)
  const bool row_ok = !PAIR || 2 * i + wrow < nb;
  const int32_t* ids;                          // unit ids: the row's entries or the pair's unit list
  int n_u;
  if constexpr (PAIR) {
    int64_t a = row_ptr[(int64_t)bh * nb + 2 * i];
    a = a < 0 ? 0 : (a > cap ? cap : a);
    ids = reinterpret_cast<const int32_t*>(units) + a;
    n_u = ulen[r];
  } else {
    int64_t e_begin = row_ptr[r], e_end = row_ptr[r + 1];
    if (e_end > cap) e_end = cap;
    if (e_begin < 0) e_begin = 0;
    if (e_begin > e_end) e_begin = e_end;
    ids = col_idx + e_begin;
    n_u = (int)(e_end - e_begin) * C::U;
  }
  const auto kh = raw_rsrc(k + (size_t)bh * N * D, N * D * 2);
  const auto vh = raw_rsrc(v + (size_t)bh * N * D, N * D * 2);
  const auto colr = raw_rsrc(ids, (n_u / UPE) * 4);

  bf16x8 qf[C::DS], gf[C::DS];     // Q^T and dO^T as B operands (query column qloc)
  {
    const int qr = min(qq, N - 1);
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
      qf[ds] = *reinterpret_cast<const bf16x8*>(q + ((size_t)bh * N + qr) * D + ds * 16 + hf * 8);
      gf[ds] = *reinterpret_cast<const bf16x8*>(dout + ((size_t)bh * N + qr) * D + ds * 16 + hf * 8);
    }
  }
  const size_t prow = (size_t)bh * nb * KB + qq;   // padded per-head row
  const float my_lse2 = row_ok ? lse2[prow] : INFINITY;   // +inf for padding queries -> P = 0
  const float c2 = scale * kLog2e;
  float my_delta = 0.f;

  uint32_t off[C::LOADS];
#pragma unroll
  for (int it = 0; it < C::LOADS; ++it) off[it] = dma_src_off<BS, D>(it, wave, lane);

  floatx16 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[dt][e] = 0.f;

  // first key and valid-key count of unit u from its block id (pair: 0 keys
  // for a unit this wave's row does not list)
  auto unit_key = [&](int j_raw, int u, int& nvk) {
    bool mine = true;
    if constexpr (PAIR) {
      mine = (((uint32_t)j_raw >> (30 + wrow)) & 1u) != 0u;
      j_raw &= 0x3fffffff;
    }
    const bool valid = j_raw >= 0 && j_raw < nb;
    const int key0 = (valid ? j_raw : 0) * KB + (u % UPE) * C::SUB;
    nvk = valid && mine ? max(0, min(C::SUB, N - key0)) : 0;
    return key0;
  };
  auto col_load = [&](int u) { return __builtin_amdgcn_raw_buffer_load_b32(colr, (u / UPE) * 4, 0, 0); };

  // SECOND = false: accumulate sum_k P dP into dsum; true: dS and dQ.
  auto pass = [&](auto second, float& dsum) __attribute__((always_inline)) {
    constexpr bool SECOND = decltype(second)::value;
    int jv0 = 0, jv1 = 0;
    if (n_u > 0) {
      jv0 = ids[0];
      int nv;
      dma_tiles<BS, D>(kh, vh, unit_key(jv0, 0, nv), k0s, v0s, wave, off);
      jv1 = col_load(1);
    }
    auto unit = [&](int u, const char* ks, const char* vs, char* kn, char* vn) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies (and the next id) landed
      __syncthreads();                      // ... and every wave's; the other slot is free
      int nvk, nn;
      unit_key(__builtin_amdgcn_readfirstlane(jv0), u, nvk);
      const int key1 = unit_key(__builtin_amdgcn_readfirstlane(jv1), u + 1, nn);
      if (u + 1 < n_u) dma_tiles<BS, D>(kh, vh, key1, kn, vn, wave, off);
      jv0 = jv1;
      jv1 = col_load(u + 2);
      const int lim = nvk - 4 * hf;         // key 32t + 8(x/4) + 4hf + x%4 is valid iff below nvk
#pragma unroll
      for (int t = 0; t < C::KC; ++t) {
        floatx16 st, dpt;
        two_products<D>(ks, vs, qf, gf, st, dpt, t * 32, l32, hf);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int kl = t * 32 + 8 * (x >> 2) + (x & 3);
          const float p = kl < lim ? __builtin_amdgcn_exp2f(fmaf(st[x], c2, -my_lse2)) : 0.f;
          if constexpr (SECOND) st[x] = p * (dpt[x] - my_delta);
          else dsum = fmaf(p, dpt[x], dsum);
        }
        if constexpr (SECOND) {
          const bf16x8 ds0 = to_bf16x8(st, 0), ds1 = to_bf16x8(st, 1);
          // step s: d tile s % DT, 16-key half s / DT (consecutive MFMAs, different accumulators)
          constexpr int NS = 2 * C::DT, AHEAD = 2;
          auto rd = [&](int st) { return read_tr8<C::CPR>(ks, t * 32 + 16 * (st / C::DT), (st % C::DT) * 32, lane); };
          bf16x8 a[NS];
#pragma unroll
          for (int s = 0; s < AHEAD; ++s) a[s] = rd(s);
#pragma unroll
          for (int s = 0; s < NS; ++s) {
            __builtin_amdgcn_sched_barrier(0);
            if (s + AHEAD < NS) a[s + AHEAD] = rd(s + AHEAD);
            const int dt = s % C::DT;
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], (s / C::DT) ? ds1 : ds0, acc[dt], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    int u = 0;
    for (; u + 1 < n_u; u += 2) {
      unit(u, k0s, v0s, k1s, v1s);
      unit(u + 1, k1s, v1s, k0s, v0s);
    }
    if (u < n_u) unit(u, k0s, v0s, k1s, v1s);
  };

  using first_t = std::integral_constant<bool, false>;
  using second_t = std::integral_constant<bool, true>;
  float dsum = 0.f;
  if (delta_given) {
    my_delta = row_ok ? delta[prow] : 0.f;
  } else {
    pass(first_t{}, dsum);
    my_delta = dsum + __shfl_xor(dsum, 32);
    if (hf == 0 && row_ok) delta[prow] = my_delta;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // the last unit's prefetched id
    __syncthreads();                      // every wave is done with the tiles
  }
  pass(second_t{}, dsum);

  if (qq < N) {
    __bf16* row = dq + ((size_t)bh * N + qq) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 out4;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) out4[r4] = (__bf16)(acc[dt][g * 4 + r4] * scale);
        *reinterpret_cast<bf16x4*>(row + dt * 32 + 8 * g + 4 * hf) = out4;
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per key block (bh, j).  Wave w owns keys
// [32w, 32w+32); the column's query blocks stream through LDS as 32-query
// tiles (Q, dO and their lse2 / delta rows).  Per tile:
//   S = Q K^T, P = exp2(c2 S - lse2_q), dP = dO V^T, dS = P (dP - delta_q),
//   dV^T += dO^T P, dK^T += Q^T dS.
// Software pipeline one tile deep: iteration t computes S and dP of tile
// t + 1 with the P / dS arithmetic of tile t interleaved under those MFMAs,
// then the dV / dK MFMAs of tile t.  Tiles t and t + 1 are read while tile
// t + 2 is copied in, so three LDS slots rotate (three distinct objects at
// fixed places of a 3x-unrolled loop).  At D = 128 the K, V fragments and
// both accumulators fill the register file for one wave per SIMD, with no
// other wave to hide the VALU work; the pipeline puts it under the MFMAs.
// ---------------------------------------------------------------------------
template <int BS, int D>
struct KvCfg {
  static constexpr int NW = BS / 32;                  // waves, 32 keys each
  static constexpr int THREADS = NW * 64;
  static constexpr int TPB = BS / 32;                 // 32-query tiles per query block
  static constexpr int DS = D / 16, DT = D / 32, CPR = D / 8;
  static constexpr int TILE_BYTES = 32 * D * 2;       // one Q or dO tile
  static constexpr int LOADS = TILE_BYTES / (16 * THREADS);
  static constexpr int WAVES_PER_SIMD = D == 128 ? 1 : 2;
  static_assert(LOADS >= 1 && LOADS * 16 * THREADS == TILE_BYTES, "tile must split evenly over the waves");
  static_assert(3 * (2 * TILE_BYTES + 256) * (4 * WAVES_PER_SIMD / NW) <= 160 * 1024, "LDS of the resident groups");
};

template <class C>
__device__ __forceinline__ uint32_t kv_src_off(int it, int wave, int lane) {
  const int L = (it * C::NW + wave) * 64 + lane;
  const int row = L / C::CPR, pos = L % C::CPR;
  return (uint32_t)((row * (C::CPR * 8) + (pos ^ swz<C::CPR>(row)) * 8) * 2);
}

// Phase A of a dK/dV iteration: S and dP of the next tile (A operands read
// row-wise from tiles ta / tb, K^T / V^T fragments in registers), with the
// current tile's s -> P and dp -> dS interleaved, NE / DS elements per k-step.
template <int D>
__device__ __forceinline__ void kv_phase_a(const char* ta, const char* tb, const bf16x8 (&kf)[D / 16],
                                           const bf16x8 (&vf)[D / 16], floatx16& sn, floatx16& dpn, floatx16& s,
                                           floatx16& dp, const float (&lv)[16], const float (&dv)[16], bool valid,
                                           float c2, int l32, int hf) {
  constexpr int DS = D / 16, CPR = D / 8, AHEAD = 2, EPS = 16 / DS;
  const floatx16 zero = {};
  bf16x8 fa[DS], fb[DS];
#pragma unroll
  for (int ds = 0; ds < AHEAD; ++ds) {
    fa[ds] = read_row8<CPR>(ta, l32, ds * 2 + hf);
    fb[ds] = read_row8<CPR>(tb, l32, ds * 2 + hf);
  }
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    __builtin_amdgcn_sched_barrier(0);
    if (ds + AHEAD < DS) {
      fa[ds + AHEAD] = read_row8<CPR>(ta, l32, (ds + AHEAD) * 2 + hf);
      fb[ds + AHEAD] = read_row8<CPR>(tb, l32, (ds + AHEAD) * 2 + hf);
    }
    sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ds], kf[ds], ds == 0 ? zero : sn, 0, 0, 0);
    dpn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ds], vf[ds], ds == 0 ? zero : dpn, 0, 0, 0);
#pragma unroll
    for (int x = ds * EPS; x < (ds + 1) * EPS; ++x) {
      const float p = valid ? __builtin_amdgcn_exp2f(fmaf(s[x], c2, -lv[x])) : 0.f;
      s[x] = p;
      dp[x] = p * (dp[x] - dv[x]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <int BS, int D>
__global__ __launch_bounds__(2 * BS, D == 128 ? 1 : 2) void dkv_kernel(   // KvCfg::WAVES_PER_SIMD
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ delta, const float* __restrict__ lse2,
    const int32_t* __restrict__ csc_start, const int32_t* __restrict__ csc_count,
    const int32_t* __restrict__ csc_row, __bf16* __restrict__ dk, __bf16* __restrict__ dv, int N, int nb,
    float scale, const int32_t* __restrict__ order, int t0) {
  using C = KvCfg<BS, D>;
  __shared__ __attribute__((aligned(1024))) char qa[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char qb[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char qc[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char ga[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char gb[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char gc[C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) float la[64];   // lse2 of the tile's 32 rows, then their delta
  __shared__ __attribute__((aligned(16))) float lb[64];
  __shared__ __attribute__((aligned(16))) float lc[64];

  // column = bh * nb + j: head-major up to t0, the last columns longest first
  const int c = (int)blockIdx.x < t0 ? (int)blockIdx.x : order[blockIdx.x - t0];
  const int bh = c / nb, j = c - bh * nb;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int kloc = wave * 32 + l32;
  const int kk = j * BS + kloc;
  const int start = csc_start[c];
  const int n_e = csc_count[c];
  const int n_t = n_e * C::TPB;                     // 32-query tiles of the column
  const auto qh = raw_rsrc(q + (size_t)bh * N * D, N * D * 2);
  const auto gh = raw_rsrc(dout + (size_t)bh * N * D, N * D * 2);
  const auto lr = raw_rsrc(lse2 + (size_t)bh * nb * BS, nb * BS * 4);
  const auto dr = raw_rsrc(delta + (size_t)bh * nb * BS, nb * BS * 4);
  const auto rowr = raw_rsrc(csc_row + start, n_e * 4);

  bf16x8 kf[C::DS], vf[C::DS];     // K^T and V^T as B operands (key column kloc)
  {
    const int kr = min(kk, N - 1);
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
      kf[ds] = *reinterpret_cast<const bf16x8*>(k + ((size_t)bh * N + kr) * D + ds * 16 + hf * 8);
      vf[ds] = *reinterpret_cast<const bf16x8*>(v + ((size_t)bh * N + kr) * D + ds * 16 + hf * 8);
    }
  }
  const bool kvalid = kk < N;
  const float c2 = scale * kLog2e;

  uint32_t off[C::LOADS];
#pragma unroll
  for (int it = 0; it < C::LOADS; ++it) off[it] = kv_src_off<C>(it, wave, lane);

  floatx16 adk[C::DT], adv[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int e = 0; e < 16; ++e) { adk[dt][e] = 0.f; adv[dt][e] = 0.f; }

  // first padded query row of tile t of entry id ib (-1: invalid entry)
  auto tile_row = [&](int ib, int t) { return (ib >= 0 && ib < nb) ? ib * BS + (t % C::TPB) * 32 : -1; };
  auto id_load = [&](int t) { return __builtin_amdgcn_raw_buffer_load_b32(rowr, (t / C::TPB) * 4, 0, 0); };
  // Q and dO rows [row0, row0 + 32) and (wave 0) their lse2 and delta
  auto dma = [&](int row0, char* qs, char* gs, float* ls) __attribute__((always_inline)) {
    const uint32_t r0 = (uint32_t)(row0 < 0 ? 0 : row0);
    const uint32_t base = r0 * (D * 2);
#pragma unroll
    for (int it = 0; it < C::LOADS; ++it) {
      lds_dma16(qh, base + off[it], qs + (it * C::NW + wave) * 64 * 16);
      lds_dma16(gh, base + off[it], gs + (it * C::NW + wave) * 64 * 16);
    }
    if (wave == 0) {
      // lanes 0-31: lse2 rows, lanes 32-63: delta rows
      const uint32_t o = (r0 + l32) * 4;
      if (hf == 0) lds_dma4(lr, o, ls);
      else lds_dma4(dr, o, ls);
    }
  };

  floatx16 s, dp;                  // S and dP of the current tile
  int id0 = 0, id1 = 0, id2 = 0;   // entry ids of tiles t, t + 1, t + 2
  if (n_t > 0) {
    id0 = csc_row[start];
    dma(tile_row(id0, 0), qa, ga, la);
    if (n_t > 1) {
      id1 = csc_row[start + 1 / C::TPB];
      dma(tile_row(id1, 1), qb, gb, lb);
    }
    id2 = id_load(2);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    two_products<D>(qa, ga, kf, vf, s, dp, 0, l32, hf);
  }

  // Iteration t: tile t in slot (qs, gs, ls), tile t + 1 in (qn, gn), tile
  // t + 2 copied into (qd, gd, ld), the slot of tile t - 1.  For the last
  // tile the next tile's S and dP come from a stale slot and are discarded.
  auto iter = [&](int t, const char* qs, const char* gs, const float* ls, const char* qn, const char* gn, char* qd,
                  char* gd, float* ld) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): tile t + 1 and id2 landed
    __syncthreads();                      // every wave is past tile t - 1
    const bool valid = tile_row(__builtin_amdgcn_readfirstlane(id0), t) >= 0 && kvalid;
    if (t + 2 < n_t) dma(tile_row(__builtin_amdgcn_readfirstlane(id2), t + 2), qd, gd, ld);
    const int id3 = id_load(t + 3);
    float lv[16], dvv[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int qr = 8 * g + 4 * hf;      // 4 consecutive query rows of the tile
      const float4 l4 = *reinterpret_cast<const float4*>(ls + qr);
      const float4 d4 = *reinterpret_cast<const float4*>(ls + 32 + qr);
      lv[4 * g] = l4.x; lv[4 * g + 1] = l4.y; lv[4 * g + 2] = l4.z; lv[4 * g + 3] = l4.w;
      dvv[4 * g] = d4.x; dvv[4 * g + 1] = d4.y; dvv[4 * g + 2] = d4.z; dvv[4 * g + 3] = d4.w;
    }
    floatx16 sn, dpn;
    kv_phase_a<D>(qn, gn, kf, vf, sn, dpn, s, dp, lv, dvv, valid, c2, l32, hf);
    const bf16x8 p0 = to_bf16x8(s, 0), p1 = to_bf16x8(s, 1);
    const bf16x8 d0 = to_bf16x8(dp, 0), d1 = to_bf16x8(dp, 1);
    // dV, dK: step st = d tile st % DT, 16-query half (st / DT) & 1, dV for
    // st < 2 DT, then dK; consecutive MFMAs update different accumulators
    constexpr int NS = 4 * C::DT, AHEAD = 2;
    auto rd = [&](int st) {
      const char* tt = st >= 2 * C::DT ? qs : gs;
      return read_tr8<C::CPR>(tt, 16 * ((st / C::DT) & 1), (st % C::DT) * 32, lane);
    };
    bf16x8 a[NS];
#pragma unroll
    for (int st = 0; st < AHEAD; ++st) a[st] = rd(st);
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      if (st + AHEAD < NS) a[st + AHEAD] = rd(st + AHEAD);
      const int dt = st % C::DT, half = (st / C::DT) & 1;
      if (st >= 2 * C::DT)
        adk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[st], half ? d1 : d0, adk[dt], 0, 0, 0);
      else
        adv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[st], half ? p1 : p0, adv[dt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    s = sn;
    dp = dpn;
    id0 = id1;
    id1 = id2;
    id2 = id3;
  };

  int t = 0;
  for (; t + 2 < n_t; t += 3) {
    iter(t, qa, ga, la, qb, gb, qc, gc, lc);
    iter(t + 1, qb, gb, lb, qc, gc, qa, ga, la);
    iter(t + 2, qc, gc, lc, qa, ga, qb, gb, lb);
  }
  if (t < n_t) {
    iter(t, qa, ga, la, qb, gb, qc, gc, lc);
    if (t + 1 < n_t) iter(t + 1, qb, gb, lb, qc, gc, qa, ga, la);
  }

  if (kk < N) {
    __bf16* krow = dk + ((size_t)bh * N + kk) * D;
    __bf16* vrow = dv + ((size_t)bh * N + kk) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 ok, ov;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          ok[r4] = (__bf16)(adk[dt][g * 4 + r4] * scale);
          ov[r4] = (__bf16)adv[dt][g * 4 + r4];
        }
        *reinterpret_cast<bf16x4*>(krow + dt * 32 + 8 * g + 4 * hf) = ok;
        *reinterpret_cast<bf16x4*>(vrow + dt * 32 + 8 * g + 4 * hf) = ov;
      }
  }
}

template <int BS, int D>
hipError_t launch_bwd_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* d_o,
                           float scale, const bsa_csr* mask, void* dq, void* dk, void* dv, bool delta_given,
                           const BackwardWs& w, hipStream_t s) {
  const int Tk = tail_rows(p.R), t0k = p.R - Tk;              // dK/dV grid: columns
  launch_tail_order(nullptr, 0, w.csc_count, t0k, Tk, w.order_k, s);
  if constexpr (BS == 64) {                                   // dQ grid: pairs of rows
    const int P = p.B * p.H * ((p.nb + 1) / 2);
    launch_pair_units(mask->row_ptr, mask->col_idx, mask->capacity, p.nb, P, w.units, w.ulen, s);
    const int Tq = tail_rows(P), t0 = P - Tq;
    launch_tail_order(nullptr, 0, w.ulen, t0, Tq, w.order_q, s);
    dq_kernel<128, D, true><<<P, 256, 0, s>>>(
        static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
        static_cast<const __bf16*>(d_o), w.delta, w.lse2, mask->row_ptr, mask->col_idx, mask->capacity,
        static_cast<__bf16*>(dq), p.N, p.nb, scale, delta_given ? 1 : 0,   // writes delta when not given
        w.order_q, t0, w.units, w.ulen);
  } else {                                                    // dQ grid: rows
    const int Tq = query_tail_rows(p.R, BS), t0 = p.R - Tq;
    launch_tail_order(mask->row_ptr, mask->capacity, nullptr, t0, Tq, w.order_q, s);
    dq_kernel<BS, D><<<p.R, 2 * BS, 0, s>>>(
        static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
        static_cast<const __bf16*>(d_o), w.delta, w.lse2, mask->row_ptr, mask->col_idx, mask->capacity,
        static_cast<__bf16*>(dq), p.N, p.nb, scale, delta_given ? 1 : 0,   // writes delta when not given
        w.order_q, t0, nullptr, nullptr);
  }
  dkv_kernel<BS, D><<<p.R, 2 * BS, 0, s>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
      static_cast<const __bf16*>(d_o), w.delta, w.lse2, w.csc_start, w.csc_count, w.csc_row,
      static_cast<__bf16*>(dk), static_cast<__bf16*>(dv), p.N, p.nb, scale, w.order_k, t0k);
  return hipGetLastError();
}

template <class TO, class TG>
void launch_delta(const Problem& p, const void* o, const void* d_o, const float* lse, int with_delta,
                  const BackwardWs& w, hipStream_t s) {
  const int BH = p.B * p.H;
  const int npad = p.nb * p.bs;
  const long long rows = (long long)BH * npad;
  const unsigned grid = (unsigned)((rows * (p.D / 8) + 255) / 256);
  if (p.D == 64)
    delta_kernel<TO, TG, 64><<<grid, 256, 0, s>>>(static_cast<const TO*>(o), static_cast<const TG*>(d_o), lse,
                                                  w.delta, w.lse2, p.N, npad, BH, with_delta);
  else
    delta_kernel<TO, TG, 128><<<grid, 256, 0, s>>>(static_cast<const TO*>(o), static_cast<const TG*>(d_o), lse,
                                                   w.delta, w.lse2, p.N, npad, BH, with_delta);
}

}  // namespace

BackwardWs carve_backward(const Problem& p, int64_t capacity, void* ws, size_t* bytes) {
  Carver c(ws);
  BackwardWs w{};
  const size_t padded = (size_t)p.B * p.H * p.nb * p.bs;
  w.delta = c.take<float>(padded);
  w.lse2 = c.take<float>(padded);
  w.csc_start = c.take<int32_t>((size_t)p.R);
  w.csc_count = c.take<int32_t>((size_t)p.R);
  w.csc_row = c.take<int32_t>((size_t)(capacity > 0 ? capacity : 1));
  if (p.dtype == BSA_BF16) {
    w.order_q = c.take<int32_t>(tail_rows(p.R));
    w.order_k = c.take<int32_t>(tail_rows(p.R));
  }
  if (p.dtype == BSA_BF16 && p.bs == 64) {   // the dQ pair grid's unit lists
    w.units = c.take<uint32_t>((size_t)(capacity > 0 ? capacity : 1));
    w.ulen = c.take<int32_t>((size_t)p.B * p.H * ((p.nb + 1) / 2));
  }
  *bytes = align_up(c.off, 256);
  return w;
}

hipError_t launch_backward_fp32(const Problem& p, const void* q, const void* k, const void* v, const void* d_o,
                                float scale, const bsa_csr* mask, void* dq, void* dk, void* dv,
                                const BackwardWs& w, hipStream_t s);

hipError_t launch_backward(const Problem& p, const void* q, const void* k, const void* v, const void* o,
                           const float* o32, const void* d_o, const float* lse, float scale, const bsa_csr* mask,
                           void* dq, void* dk, void* dv, const BackwardWs& w, hipStream_t s) {
  const bool bf = p.dtype == BSA_BF16;
  const bool delta_given = bf && o32 != nullptr;
  if (!bf) launch_delta<float, float>(p, o, d_o, lse, 1, w, s);
  else if (delta_given) launch_delta<float, __bf16>(p, o32, d_o, lse, 1, w, s);
  else launch_delta<__bf16, __bf16>(p, o, d_o, lse, 0, w, s);
  csc_kernel<<<p.B * p.H, kCscThreads, 0, s>>>(mask->row_ptr, mask->col_idx, mask->capacity, p.nb, w.csc_start,
                                      w.csc_count, w.csc_row);
  if (!bf) return launch_backward_fp32(p, q, k, v, d_o, scale, mask, dq, dk, dv, w, s);
  if (p.bs == 128 && p.D == 128)
    return launch_bwd_bf16<128, 128>(p, q, k, v, d_o, scale, mask, dq, dk, dv, delta_given, w, s);
  if (p.bs == 128 && p.D == 64)
    return launch_bwd_bf16<128, 64>(p, q, k, v, d_o, scale, mask, dq, dk, dv, delta_given, w, s);
  if (p.bs == 64 && p.D == 128)
    return launch_bwd_bf16<64, 128>(p, q, k, v, d_o, scale, mask, dq, dk, dv, delta_given, w, s);
  return launch_bwd_bf16<64, 64>(p, q, k, v, d_o, scale, mask, dq, dk, dv, delta_given, w, s);
}

}  // namespace bsa
