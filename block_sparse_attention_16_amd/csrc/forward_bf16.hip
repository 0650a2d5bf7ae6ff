// Sparse attention forward with exact per-block attention mass, bf16 MFMA (gfx950).
//
// Stage two of the estimate-then-attend scheme (DSV page, Abstract): a
// FlashAttention-style online-softmax forward that visits only the key blocks
// of each query block's CSR row, and obtains the exact attention weight of
// every visited block inside the same pass (GSRS page, Abstract; the
// block-level attention map of its Figure 3 caption).
//
// Workgroup = one mask row (query block i of head bh), BS/32 waves.  Wave w
// owns queries [32w, 32w + 32) of the block and every key of each visited key
// block, with its own online-softmax state.  Two waves share each SIMD.  With
// 64-token blocks a workgroup takes two adjacent mask rows instead (the pair
// grid, PAIR below), so that every workgroup has 128 queries and 64-key units.
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// A = K rows from LDS, B = Q^T held in registers.  In the 32x32 accumulator a
// lane holds one query column and 16 key rows, so a query's row max and sum
// need one cross-half exchange (lane ^ 32).  The same registers, rounded to
// bf16, are the B operand of O^T += V^T P^T: the MFMA k-slots of lane half h
// hold key rows {16g + 8a + 4h + r}.  The matching A operand (V^T) is read
// from the row-major V tile with two ds_read_b64_tr_b16, which transpose
// 4x4 blocks of bf16 across each 16-lane group.
//
// Keys are consumed in units of SUB keys (a sub-block of one CSR entry).  The
// loop is software-pipelined by one unit inside each wave: while the matrix
// cores compute the scores of unit u+1, the VALU turns the scores of unit u
// into probabilities; while they accumulate unit u's P V, the VALU takes the
// row max of unit u+1 (D = 64) or has nothing to do (D = 128, see below).  So
// the softmax runs under the MFMAs of the same wave.
//
// Running max, exact for any value it takes.  D = 64: the row max of the next
// unit (taken under the PV MFMAs, where the VALU is otherwise idle) raises it
// lazily, only by more than kTau.  D = 128: no max on the common path; a
// unit's probabilities are taken against the running max as it stands, and
// only when it is still -inf or some lane's sum over the unit exceeds 2^64 is
// the unit's exact max folded in, the accumulators rescaled and the unit's
// probabilities taken again (measured 2-3 % faster at D = 128; at D = 64 the
// check after the exponentials sits on the critical path and costs more than
// the max it saves).
//
// K and V tiles stream from HBM/L2 straight into LDS with buffer loads (two
// K slots, two V slots).  At the top of iteration u one barrier frees the K
// slot of unit u (scored in iteration u-1) and the V slot of unit u-1; the
// DMAs of K[u+2] and V[u+1] then have a whole iteration to land.  LDS rows are
// XOR-swizzled in 16-byte chunks so the MFMA operand reads are conflict free.
//
// Block mass: for every visited entry e and query q the kernel stores the
// block-local log2-sum-exp m + log2(l_block) (exact whatever the running max
// m is); once the row's final LSE is known the epilogue turns these into
// mean_q exp2(c_e(q) - lse2(q)).
#include "bsa_internal.h"

#include <type_traits>

namespace bsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef short short4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 8.0f;     // lazy-rescale threshold of the running max, log2 units (D = 64)
constexpr float kSumMax = 1.8446744e19f;   // 2^64: largest lane sum over a unit kept without rescale (D = 128)

// Where the running max is kept current (see the file comment).
template <int D>
constexpr bool max_under_pv() { return D == 64; }

// 16-byte chunk swizzles of a [key][D] bf16 tile whose rows are CPR chunks long.
// K is read with ds_read_b128 down 16 consecutive rows; V with ds_read_b64_tr_b16
// over 4 consecutive rows x 4 chunks per 32 lanes.
template <int CPR>
__device__ __forceinline__ int swz_k(int row) {
  static_assert(CPR == 16 || CPR == 8, "row must be 128 or 256 bytes");
  return CPR == 16 ? (row & 15) : ((row >> 1) & 7);
}
template <int CPR>
__device__ __forceinline__ int swz_v(int row) {
  static_assert(CPR == 16 || CPR == 8, "row must be 128 or 256 bytes");
  return CPR == 16 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

// Transposing LDS read: within each 16-lane group, result lane 4g+c, element t
// is element c of the 8-byte row addressed by lane 4t+g.
__device__ __forceinline__ short4_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p));
}

// Combine a value with its partner in the other half of the wave (lane ^ 32)
// with v_permlane32_swap, a VALU op: swapping x with itself yields
// [x_lo, x_lo] and [x_hi, x_hi], so op(r0, r1) = op(x[l%32], x[l%32 + 32]) on
// every lane, identically on both halves.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer resource over one head's [N, D] bf16 matrix: raw (stride 0), its
// record count the matrix size in bytes, so that reads past the last key
// return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const __bf16* base, int N, int D) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(base), (short)0, N * D * 2, 0x00020000);
}

// 16 bytes per lane from buffer offset `off` into LDS at lds_wave_base + 16 * lane.
// The buffer form (not global_load_lds) lets the compiler keep exact LDS
// wait counts while the copy is in flight.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t off, void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds_wave_base, 16, off, 0,
                                           0, 0);
}

template <int BS, int D>
struct Cfg {
  static constexpr int NW = BS / 32;                  // waves; wave w owns 32 queries
  static constexpr int THREADS = NW * 64;
  static constexpr int WG_PER_CU = 8 / NW;            // two waves per SIMD
  // Keys stream through LDS in units of SUB keys (KC 32-key tiles).
  static constexpr int SUB = (BS == 64 && D == 128) ? 32 : 64;
  static constexpr int KC = SUB / 32;
  static constexpr int U = BS / SUB;                  // units per key block
  static constexpr int DS = D / 16, DT = D / 32;      // MFMA k-steps over d, d tiles
  static constexpr int CPR = D / 8;                   // 16-byte chunks per K or V row
  static constexpr int TILE_BYTES = SUB * D * 2;      // one K or V tile
  static constexpr int LOADS = TILE_BYTES / (16 * THREADS);  // dma ops per thread per tile
  static_assert(LOADS * 16 * THREADS == TILE_BYTES, "tile must split evenly over the waves");
  static_assert(4 * TILE_BYTES * WG_PER_CU <= 160 * 1024, "LDS of the resident workgroups");
};

// Per-lane byte offset, within a SUB-row window of a [N, D] bf16 matrix, of
// the 16-byte source chunk that dma op `it` of this lane stores.  Lane l of a
// wave writes LDS chunk (wave chunk base + l); the swizzle decides which
// logical chunk lands there.
template <int BS, int D, bool IS_V>
__device__ __forceinline__ uint32_t dma_src_off(int it, int wave, int lane) {
  using C = Cfg<BS, D>;
  const int L = (it * C::NW + wave) * 64 + lane;
  const int row = L / C::CPR, pos = L % C::CPR;
  const int c = pos ^ (IS_V ? swz_v<C::CPR>(row) : swz_k<C::CPR>(row));
  return (uint32_t)((row * D + c * 8) * 2);
}

// DMA of rows [key0, key0 + SUB) of a head's [N, D] bf16 matrix into a
// swizzled LDS tile.  Rows past N read as zeros (their scores are masked to
// -inf, so they carry no weight).
template <int BS, int D>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rsrc, int key0, char* tile, int wave,
                                         const uint32_t (&off)[Cfg<BS, D>::LOADS]) {
  using C = Cfg<BS, D>;
  const uint32_t base = (uint32_t)key0 * (D * 2);
#pragma unroll
  for (int it = 0; it < C::LOADS; ++it) lds_dma16(rsrc, base + off[it], tile + (it * C::NW + wave) * 64 * 16);
}

// K operand of score step s = ds * KC + t: rows 32t + l32 of the tile, d
// columns 16 ds + 8 hf .. +8.
template <int BS, int D, class C = Cfg<BS, D>>
__device__ __forceinline__ bf16x8 read_k(const char* ks, int s, int l32, int hf) {
  const int ds = s / C::KC, t = s % C::KC;
  const int row = t * 32 + l32;
  const int c = (ds * 2 + hf) ^ swz_k<C::CPR>(row);
  return *reinterpret_cast<const bf16x8*>(ks + (row * C::CPR + c) * 16);
}

// V^T operand of PV step s, steps ordered (t, h2, dt) so that consecutive
// MFMAs update different accumulators.  Source-lane role in the transposing
// read: lane 16G + 4r + g points at key row (32t + 16h2 + 8x + 4(G/2) + r),
// dims 32dt + 16(G&1) + 4g .. +3, so that result lane L receives
// V[32t + 16h2 + 8x + 4(L/32) + r][32dt + L%32] for r = 0..3.
template <int BS, int D, class C = Cfg<BS, D>>
__device__ __forceinline__ bf16x8 read_v(const char* vs, int s, int lane) {
  const int G = lane >> 4, tr = (lane >> 2) & 3, g4 = lane & 3;
  const int dt = s % C::DT, h2 = (s / C::DT) & 1, t = s / (2 * C::DT);
  const int dcol = dt * 32 + 16 * (G & 1) + 4 * g4;
  short4_t t4[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int row = t * 32 + h2 * 16 + 8 * x + 4 * (G >> 1) + tr;
    const int c = (dcol >> 3) ^ swz_v<C::CPR>(row);
    t4[x] = lds_read_tr16(vs + (row * C::CPR + c) * 16 + (dcol & 7) * 2);
  }
  // whole-register reinterpretation (element-wise casts of the transposed
  // halves are mis-assembled by the compiler)
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t4[0], t4[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Keys past the valid count of a unit (end of the sequence, or an invalid
// entry) get score -inf.  nvk is wave-uniform.
template <int BS, int D, class C = Cfg<BS, D>>
__device__ __forceinline__ void mask_scores(floatx16 (&s)[C::KC], int nvk, int hf) {
  const int lim = nvk - 4 * hf;        // key 32t + 8(v/4) + 4hf + v%4 is valid iff below nvk
#pragma unroll
  for (int t = 0; t < C::KC; ++t)
#pragma unroll
    for (int v2 = 0; v2 < 16; ++v2) {
      const int kl = t * 32 + 8 * (v2 >> 2) + (v2 & 3);
      s[t][v2] = kl < lim ? s[t][v2] : -INFINITY;
    }
}

// Scores of one unit alone (pipeline prologue).
template <int BS, int D, class C = Cfg<BS, D>>
__device__ __forceinline__ void scores_only(const char* ks, const bf16x8 (&qf)[C::DS], floatx16 (&sn)[C::KC],
                                            int l32, int hf) {
  constexpr int NS = C::DS * C::KC;
  const floatx16 zero = {};
  bf16x8 kf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) kf[s] = read_k<BS, D>(ks, s, l32, hf);
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int ds = s / C::KC, t = s % C::KC;
    sn[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[ds], ds == 0 ? zero : sn[t], 0, 0, 0);
  }
}

// Probabilities j in [j0, j1) of the current unit: exp2 of the scaled,
// max-shifted scores (in place), their running sum ls, and bf16 copies
// (pairs) for the PV MFMAs with the running sum lt of those rounded copies
// (one v_dot2 against (1, 1) per pair).  O is normalised by lt, the weights
// its PV product actually used, so that O is a weighted mean of V rows and
// the rounding of P moves it only by the weighted spread of V around O;
// normalising by ls instead lets the rounding of the largest probabilities
// scale O as a whole (up to ~2.5 times the error on the video workloads).
// LSE and block mass use the exact sum ls.
// With max_under_pv the scores are overwritten by their probabilities;
// otherwise they are kept for a possible second pass (rescale_redo).
template <int BS, int D, class C = Cfg<BS, D>>
__device__ __forceinline__ void probs(floatx16 (&sc)[C::KC], bf16x8 (&pb)[C::KC][2], float c2, float m_use,
                                      float& ls, float& lt, int j0, int j1) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float prev = 0.f;
#pragma unroll
  for (int j = j0; j < j1; ++j) {
    const int t = j / 16, v2 = j % 16;
    const float p = __builtin_amdgcn_exp2f(fmaf(sc[t][v2], c2, -m_use));
    ls += p;
    if constexpr (max_under_pv<D>()) {
      sc[t][v2] = p;
      if (j & 1) {
        // kept in place (empty asm): sunk past the next unit's max fold,
        // the conversions and sums run uncovered (measured 8 % slower)
        bf16x2 pr = {(__bf16)sc[t][v2 - 1], (__bf16)p};
        asm volatile("" : "+v"(pr));
        pb[t][v2 / 8][(v2 - 1) % 8] = pr[0];
        pb[t][v2 / 8][v2 % 8] = pr[1];
        lt = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lt, false);
        asm volatile("" : "+v"(lt));
      }
    } else {
      if (j & 1) {
        const bf16x2 pr = {(__bf16)prev, (__bf16)p};
        pb[t][v2 / 8][(v2 - 1) % 8] = pr[0];
        pb[t][v2 / 8][v2 % 8] = pr[1];
        lt = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lt, false);
      }
      prev = p;
    }
  }
}

// Phase B of an iteration: probabilities of the current unit, interleaved
// with the score MFMAs of the next unit when NEXT.  Scheduling
// fences pin the interleave: per MFMA step one K read (AHEAD steps ahead)
// and an equal share of the exponentials.
template <int BS, int D, bool NEXT, class C = Cfg<BS, D>>
__device__ __forceinline__ void phase_b(const char* ks, const bf16x8 (&qf)[C::DS], floatx16 (&sc)[C::KC],
                                        floatx16 (&sn)[C::KC], bf16x8 (&pb)[C::KC][2], float c2, float m_use,
                                        float& ls, float& lt, int l32, int hf) {
  constexpr int NS = C::DS * C::KC;            // score MFMAs of the next unit
  constexpr int NE = C::KC * 16;               // probabilities per lane
  constexpr int NSEG = NEXT ? NS : 1;
  constexpr int EPS = (NE + NSEG - 1) / NSEG;
  constexpr int AHEAD = NS < 2 ? NS : 2;
  const floatx16 zero = {};
  bf16x8 kf[NS];
  if constexpr (NEXT) {
#pragma unroll
    for (int s = 0; s < AHEAD; ++s) kf[s] = read_k<BS, D>(ks, s, l32, hf);
  }
#pragma unroll
  for (int g = 0; g < NSEG; ++g) {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) {
      if (g + AHEAD < NS) kf[g + AHEAD] = read_k<BS, D>(ks, g + AHEAD, l32, hf);
      const int ds = g / C::KC, t = g % C::KC;
      sn[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[g], qf[ds], ds == 0 ? zero : sn[t], 0, 0, 0);
    }
    probs<BS, D>(sc, pb, c2, m_use, ls, lt, g * EPS, (g + 1) * EPS < NE ? (g + 1) * EPS : NE);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Phase C: O^T += V^T P^T for the current unit, interleaved with the row max
// of the next unit's scores when NEXT and max_under_pv.  V operands are read
// AHEAD steps ahead.
template <int BS, int D, bool NEXT, class C = Cfg<BS, D>>
__device__ __forceinline__ void phase_c(const char* vs, const bf16x8 (&pb)[C::KC][2], floatx16 (&acc)[C::DT],
                                        const floatx16 (&sn)[C::KC], float& mx, int lane) {
  constexpr int NSTEP = C::KC * 2 * C::DT;
  constexpr int NM = C::KC * 16;
  constexpr int MPS = (NM + NSTEP - 1) / NSTEP;   // max operands per step
  constexpr int AHEAD = NSTEP < 3 ? NSTEP : 3;
  bf16x8 vf[NSTEP];
#pragma unroll
  for (int s = 0; s < AHEAD; ++s) vf[s] = read_v<BS, D>(vs, s, lane);
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    __builtin_amdgcn_sched_barrier(0);
    if (s + AHEAD < NSTEP) vf[s + AHEAD] = read_v<BS, D>(vs, s + AHEAD, lane);
    const int dt = s % C::DT, h2 = (s / C::DT) & 1, t = s / (2 * C::DT);
    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[s], pb[t][h2], acc[dt], 0, 0, 0);
    if constexpr (NEXT && max_under_pv<D>()) {
#pragma unroll
      for (int j = s * MPS; j < (s + 1) * MPS && j < NM; ++j) mx = fmaxf(mx, sn[j / 16][j % 16]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// WRITE_O32: also store O in fp32 (a separate instantiation, so that the
// common kernel is compiled without the extra epilogue).
// PAIR (64-token blocks): a 128-query workgroup takes the two mask rows of
// query blocks 2m and 2m + 1 of a head (waves 0-1 and 2-3), walking the unit
// list built by pair_units_kernel: one 64-key block per unit, with flags for
// the rows that list it.  Every unit's K/V tiles are copied once for both
// rows; a wave scores a unit its row does not list as -inf throughout, which
// adds exact zeros, so each row's results are those of a walk over its own
// list.  On the video training masks adjacent rows share ~89 % of their
// blocks.
template <int BS, int D, bool WRITE_O32, bool PAIR = false>
__global__ __launch_bounds__(2 * BS, 2) void fwd_kernel(   // Cfg::THREADS; two waves per SIMD
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t cap, __bf16* __restrict__ o,
    float* __restrict__ lse, float* __restrict__ mass, float* __restrict__ part, float* __restrict__ o32, int N,
    int nb, float scale, const int32_t* __restrict__ order, int t0, const uint32_t* __restrict__ units,
    const int32_t* __restrict__ ulen) {
  using C = Cfg<BS, D>;
  static_assert(!PAIR || BS == 128, "a pair of 64-token query blocks fills a 128-query workgroup");
  constexpr int KB = PAIR ? 64 : BS;          // tokens per key block and per mask row's query block
  constexpr int UPE = PAIR ? 1 : C::U;        // units per listed key block
  // LDS tiles.  Distinct objects, each used at a fixed place of the loop, let
  // the compiler see that reads of one tile do not wait on the DMA into another.
  __shared__ __attribute__((aligned(1024))) char k0s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k1s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) float lse2_s[BS];

  // blockIdx -> mask row, dealt to the 8 XCDs round-robin by the dispatcher
  // (finer-grained than any contiguous split, which balances rows of unequal
  // length; keeping neighbouring rows on one XCD's L2 measured no faster).
  // Head-major up to t0, so that rows running together share K/V in the
  // caches; the last rows of the grid longest first (order).
  const int r = (int)blockIdx.x < t0 ? (int)blockIdx.x : order[blockIdx.x - t0];
  const int nbw = PAIR ? (nb + 1) / 2 : nb;  // workgroup rows per head
  const int bh = r / nbw, i = r - bh * nbw;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
  const int l32 = lane & 31, hf = lane >> 5;
  const int q0 = i * BS;
  const int nq = min(BS, N - q0);
  const int qloc = wave * 32 + l32;          // this lane's query within the block
  const int qq = q0 + qloc;

  // This wave's mask row: the workgroup's row, or in a pair row 2i (waves
  // 0-1) or 2i + 1 (waves 2-3, absent when 2i + 1 = nb).
  const int wrow = PAIR ? (wave >> 1) : 0;
  const int64_t rrow = PAIR ? (int64_t)bh * nb + 2 * i + wrow : r;
  int64_t e_begin = 0, e_end = 0;
  if (!PAIR || 2 * i + wrow < nb) {
    e_begin = row_ptr[rrow];
    e_end = row_ptr[rrow + 1];
    if (e_end > cap) e_end = cap;
    if (e_begin < 0) e_begin = 0;
    if (e_begin > e_end) e_begin = e_end;
  }
  const int n_e = (int)(e_end - e_begin);

  const auto kh = head_rsrc(k + (size_t)bh * N * D, N, D);
  const auto vh = head_rsrc(v + (size_t)bh * N * D, N, D);

  // Q^T fragments (B operand): lane holds query qloc, d = ds*16 + hf*8 .. +8
  bf16x8 qf[C::DS];
#pragma unroll
  for (int ds = 0; ds < C::DS; ++ds) {
    if (qq < N) {
      qf[ds] = *reinterpret_cast<const bf16x8*>(q + ((size_t)bh * N + qq) * D + ds * 16 + hf * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ds][e] = (__bf16)0.f;
    }
  }

  floatx16 acc[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int v2 = 0; v2 < 16; ++v2) acc[dt][v2] = 0.f;
  // Running sums.  D = 128: of this lane's half of the keys (lanes l and
  // l ^ 32 hold the same query and the same m_run, so the two halves are
  // combined only where a sum is used: the block-mass partial at each entry's
  // end, LSE and O at the end of the row; measured 0.6 % faster).  D = 64:
  // combined every unit (deferring measured 6 % slower there).
  constexpr bool kHalfSums = !max_under_pv<D>();
  float m_run = -INFINITY, l_run = 0.f;
  float lt_run = 0.f;      // sum of the bf16-rounded probabilities (normalises O)
  float ls_blk = 0.f;      // current entry's sum of exp2(s - m_run), for the block mass
  const float c2 = scale * kLog2e;   // logits in base-2 units

  // Unit u = sub-block (u % U) of CSR entry (u / U).  The loop reads the
  // entries' key-block ids with vector buffer loads one iteration ahead (so
  // they land under the same wait as the tile DMAs, and ids past the row read
  // as 0 without a bounds test); the prologue reads its first ids directly.
  // Ids of the units: the row's CSR entries, or the pair's unit list (which
  // starts where row 2i's entries start).
  const int32_t* ids = col_idx + e_begin;
  int n_u = n_e * UPE;
  if constexpr (PAIR) {
    int64_t a = row_ptr[(int64_t)bh * nb + 2 * i];
    a = a < 0 ? 0 : (a > cap ? cap : a);
    ids = reinterpret_cast<const int32_t*>(units) + a;
    n_u = ulen[r];
  }
  const auto colr = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(ids), (short)0, (n_u / UPE) * 4,
                                                      0x00020000);
  auto col_load = [&](int u) { return __builtin_amdgcn_raw_buffer_load_b32(colr, (u / UPE) * 4, 0, 0); };
  // first key of unit u; nvk = its valid keys for this wave (0 for a unit
  // that this wave's row does not list)
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
  auto unit_mine = [&](int j_raw) { return !PAIR || ((((uint32_t)j_raw >> (30 + wrow)) & 1u) != 0u); };
  auto unit_src = [&](int u, int& nvk) { return unit_key(ids[u / UPE], u, nvk); };
  uint32_t koff[C::LOADS], voff[C::LOADS];
#pragma unroll
  for (int it = 0; it < C::LOADS; ++it) {
    koff[it] = dma_src_off<BS, D, false>(it, wave, lane);
    voff[it] = dma_src_off<BS, D, true>(it, wave, lane);
  }

  // This lane's max over a unit's (masked) scores, in raw score units.
  auto unit_max = [&](const floatx16 (&sc)[C::KC]) __attribute__((always_inline)) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < C::KC; ++t)
#pragma unroll
      for (int v2 = 0; v2 < 16; ++v2) mx = fmaxf(mx, sc[t][v2]);
    return mx;
  };
  // D = 64: fold a unit's row max (raw score units, this lane's half) into
  // the running max.  It is only raised when some lane's new max exceeds it
  // by more than kTau (log2 units): p <= 2^kTau stays safe in bf16/fp32 and
  // most updates skip the rescale of the output accumulators.
  auto fold_max = [&](float mx) __attribute__((always_inline)) {
    mx = xhalf_max(mx) * c2;
    if (__any(mx > m_run + kTau)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int v2 = 0; v2 < 16; ++v2) acc[dt][v2] *= alpha;
      l_run *= alpha;
      lt_run *= alpha;
      ls_blk *= alpha;
    }
  };
  // D = 128: the unit's probabilities overflowed the safe range, or nothing
  // is accumulated yet: fold in the unit's exact max, rescale what is
  // accumulated (nothing when m_run was -inf), take the probabilities again.
  auto rescale_redo = [&](floatx16 (&sc)[C::KC], bf16x8 (&pb)[C::KC][2], float& ls, float& lt)
                          __attribute__((always_inline)) {
    const float m_new = fmaxf(m_run, xhalf_max(unit_max(sc)) * c2);
    if (m_new != m_run) {
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int v2 = 0; v2 < 16; ++v2) acc[dt][v2] *= alpha;
      l_run *= alpha;
      lt_run *= alpha;
      ls_blk *= alpha;
      m_run = m_new;
    }
    ls = 0.f;
    lt = 0.f;
    probs<BS, D>(sc, pb, c2, m_run == -INFINITY ? 0.f : m_run, ls, lt, 0, C::KC * 16);
  };

  floatx16 sa[C::KC], sb[C::KC];     // scores of the current and the next unit
  int jv1 = col_load(1), jv2 = col_load(2);   // key-block ids of units u+1, u+2 (VGPR, uniform)
  bool mine_u = n_u > 0 && unit_mine(ids[0]);  // PAIR: this wave's row lists the current unit
  int k_row = 0;                               // PAIR: entries of this wave's row walked so far
  if (n_u > 0) {
    int nv0;
    const int key0 = unit_src(0, nv0);
    dma_tile<BS, D>(kh, key0, k0s, wave, koff);
    dma_tile<BS, D>(vh, key0, v0s, wave, voff);
    if (n_u > 1) {
      int nv1;
      dma_tile<BS, D>(kh, unit_src(1, nv1), k1s, wave, koff);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    scores_only<BS, D>(k0s, qf, sa, l32, hf);
    if (nv0 < C::SUB) mask_scores<BS, D>(sa, nv0, hf);
    if constexpr (max_under_pv<D>()) fold_max(unit_max(sa));
  }

  // Iteration u: K[u+1] sits in slot (u+1)%2, V[u] in slot u%2.  sc holds
  // unit u's scores (masked; max folded in at D = 64); sn receives unit u+1's.  Inside
  // the unrolled loop the next unit's scores are always computed (for the
  // last unit from a stale K slot, then discarded), which keeps one code path.
  auto iter = [&](auto next_tag, int u, floatx16 (&sc)[C::KC], floatx16 (&sn)[C::KC], const char* ks_next,
                  const char* vs_cur, char* k_free, char* v_free) __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_tag)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMAs of K[u+1], V[u] (and ids) landed
    __syncthreads();                      // ... and every other wave's; slots of K[u], V[u-1] are free
    const bool has_next = u + 1 < n_u;
    int nvn, nn;
    const int jr1 = __builtin_amdgcn_readfirstlane(jv1);
    const int key1 = unit_key(jr1, u + 1, nvn);
    const bool mine_cur = mine_u;
    mine_u = unit_mine(jr1);
    const int key2 = unit_key(__builtin_amdgcn_readfirstlane(jv2), u + 2, nn);
    if (u + 2 < n_u) dma_tile<BS, D>(kh, key2, k_free, wave, koff);
    if (has_next) dma_tile<BS, D>(vh, key1, v_free, wave, voff);
    jv1 = jv2;
    jv2 = col_load(u + 3);
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    bf16x8 pb[C::KC][2];
    float ls = 0.f, lt = 0.f;
    phase_b<BS, D, NEXT>(ks_next, qf, sc, sn, pb, c2, m_use, ls, lt, l32, hf);
    if constexpr (!max_under_pv<D>()) {
      if (__any(m_run == -INFINITY || ls > kSumMax)) rescale_redo(sc, pb, ls, lt);
    }
    if constexpr (!kHalfSums) {
      ls = xhalf_sum(ls);
      lt = xhalf_sum(lt);
    }
    l_run += ls;
    lt_run += lt;
    ls_blk += ls;
    if (u % UPE == UPE - 1) {           // last unit of the entry
      if constexpr (PAIR) {
        if (part != nullptr && mine_cur) {
          const float lb = kHalfSums ? xhalf_sum(ls_blk) : ls_blk;
          if (hf == 0)
            part[(e_begin + k_row) * KB + (qloc & 63)] = lb > 0.f ? m_run + __builtin_amdgcn_logf(lb) : -INFINITY;
        }
        k_row += mine_cur ? 1 : 0;
      } else if (part != nullptr) {
        const int it = u / C::U;
        const float lb = kHalfSums ? xhalf_sum(ls_blk) : ls_blk;
        if (hf == 0) part[(e_begin + it) * BS + qloc] = lb > 0.f ? m_run + __builtin_amdgcn_logf(lb) : -INFINITY;
      }
      ls_blk = 0.f;
    }
    float mx = -INFINITY;
    if constexpr (NEXT) {
      if (has_next && nvn < C::SUB) mask_scores<BS, D>(sn, nvn, hf);
    }
    phase_c<BS, D, NEXT>(vs_cur, pb, acc, sn, mx, lane);
    if constexpr (NEXT && max_under_pv<D>()) fold_max(has_next ? mx : -INFINITY);   // a stale next unit adds nothing
  };
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  int u = 0;
  for (; u + 1 < n_u; u += 2) {
    iter(Yes{}, u, sa, sb, k1s, v0s, k0s, v1s);
    iter(Yes{}, u + 1, sb, sa, k0s, v1s, k1s, v0s);
  }
  if (u < n_u) iter(No{}, u, sa, sb, k1s, v0s, k0s, v1s);

  // ---- normalise, write O and LSE ----
  if constexpr (kHalfSums) {
    l_run = xhalf_sum(l_run);
    lt_run = xhalf_sum(lt_run);
  }
  const float inv = l_run > 0.f && lt_run > 0.f ? 1.f / lt_run : 0.f;
  const float mu = m_run == -INFINITY ? 0.f : m_run;
  const float lse2 = l_run > 0.f ? mu + __builtin_amdgcn_logf(l_run) : -INFINITY;
  if (hf == 0) lse2_s[qloc] = lse2;
  if (qq < N) {
    if (hf == 0) lse[(size_t)bh * N + qq] = lse2 * kLn2;
    __bf16* orow = o + ((size_t)bh * N + qq) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 out4;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) out4[r4] = (__bf16)(acc[dt][g * 4 + r4] * inv);
        *reinterpret_cast<bf16x4*>(orow + dt * 32 + 8 * g + 4 * hf) = out4;
      }
    }
    if constexpr (WRITE_O32) {         // O before its rounding to bf16
      float* frow = o32 + ((size_t)bh * N + qq) * D;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<float4*>(frow + dt * 32 + 8 * g + 4 * hf) =
              make_float4(acc[dt][g * 4] * inv, acc[dt][g * 4 + 1] * inv, acc[dt][g * 4 + 2] * inv,
                          acc[dt][g * 4 + 3] * inv);
    }
  }
  if (mass == nullptr || (!PAIR && n_e == 0)) return;   // uniform over the workgroup
  __syncthreads();

  // ---- exact block mass: mean over valid queries of exp2(part - lse2) ----
  if constexpr (PAIR) {
    // each row's entries by its two waves; n_e = 0 for an absent row
    const int qr = 64 * wrow;                  // the row's first query in the workgroup
    const int nq_row = max(0, min(64, N - (q0 + qr)));
    for (int it = wave & 1; it < n_e; it += 2) {
      const int64_t e = e_begin + it;
      const int j_raw = col_idx[e];
      float s = 0.f;
      if (j_raw >= 0 && j_raw < nb && lane < nq_row) s = __builtin_amdgcn_exp2f(part[e * KB + lane] - lse2_s[qr + lane]);
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0) mass[e] = s / (float)nq_row;
    }
  } else if constexpr (D == 128 && BS == 128) {
    // Four entries per wavefront at a time, 16 lanes each: lane c of a group
    // sums queries [QPL c, QPL c + QPL) (16-byte loads of part and lse2),
    // then four xor-shuffles within the group.  (Measured slower elsewhere:
    // ~4 % for the whole kernel at D = 64 with the main loop unchanged, 1 %
    // with 64-token blocks; those keep one entry per wavefront.)
    constexpr int QPL = BS / 16;               // queries per lane
    const int grp = lane >> 4, c = lane & 15;
    float l2[QPL];
#pragma unroll
    for (int x = 0; x < QPL; x += 4) {
      const float4 v4 = *reinterpret_cast<const float4*>(lse2_s + QPL * c + x);
      l2[x] = v4.x; l2[x + 1] = v4.y; l2[x + 2] = v4.z; l2[x + 3] = v4.w;
    }
    for (int base = wave * 4; base < n_e; base += C::NW * 4) {
      const int it = base + grp;
      const bool live = it < n_e;
      const int64_t e = e_begin + (live ? it : 0);
      const int j_raw = live ? col_idx[e] : -1;
      float s = 0.f;
      if (j_raw >= 0 && j_raw < nb) {
        const float* pe = part + e * BS + QPL * c;
#pragma unroll
        for (int x = 0; x < QPL; x += 4) {
          const float4 p4 = *reinterpret_cast<const float4*>(pe + x);
          const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
          for (int y = 0; y < 4; ++y)
            if (QPL * c + x + y < nq) s += __builtin_amdgcn_exp2f(pv[y] - l2[x + y]);
        }
      }
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) s += __shfl_xor(s, off);
      if (live && c == 0) mass[e] = s / (float)nq;
    }
  } else {
    for (int it = wave; it < n_e; it += C::NW) {
      const int64_t e = e_begin + it;
      const int j_raw = col_idx[e];
      float s = 0.f;
      if (j_raw >= 0 && j_raw < nb) {
        for (int t = lane; t < nq; t += 64) s += __builtin_amdgcn_exp2f(part[e * BS + t] - lse2_s[t]);
      }
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
      if (lane == 0) mass[e] = s / (float)nq;
    }
  }
}

// Unit lists of the pair grid (fwd_kernel, PAIR): pair p is query blocks 2m
// and 2m + 1 of head bh (rows A and B).  When both rows list strictly
// ascending ids in [0, nb), the pair walks their union in ascending order,
// bit 30 marking a block of A and bit 31 one of B; otherwise A's entries then
// B's, as listed (ids outside [0, nb) kept outside).  Pair p's list goes over
// the pair's own entries [row_ptr[A], row_ptr[B + 1]) of the unit array,
// which hold |A| + |B| slots, at least its length; a pair whose rows are not
// adjacent in col_idx (a decreasing row_ptr) gets no units.  One wavefront per
// pair, the union through two LDS bitmasks.
constexpr uint32_t kUnitA = 1u << 30, kUnitB = 1u << 31, kUnitNone = kUnitA - 1u;
constexpr int kPairWaves = 4;
__global__ __launch_bounds__(64 * kPairWaves) void pair_units_kernel(const int32_t* __restrict__ row_ptr,
                                                                     const int32_t* __restrict__ col_idx,
                                                                     int64_t cap, int nb, int P,
                                                                     uint32_t* __restrict__ units,
                                                                     int32_t* __restrict__ ulen) {
  __shared__ uint32_t bits[kPairWaves][2][4096 / 32];   // nb <= 4096
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int p = blockIdx.x * kPairWaves + wid;
  if (p >= P) return;                        // whole wavefront leaves together
  const int np = (nb + 1) / 2;
  const int bh = p / np, m = p - bh * np;
  const int64_t rA = (int64_t)bh * nb + 2 * m;
  const bool hasB = 2 * m + 1 < nb;
  auto clampc = [&](int64_t x) { return x < 0 ? (int64_t)0 : (x > cap ? cap : x); };
  const int64_t sA = clampc(row_ptr[rA]);
  int64_t eA = clampc(row_ptr[rA + 1]);
  if (eA < sA) eA = sA;
  int64_t sB = eA, eB = eA;
  if (hasB) {
    sB = clampc(row_ptr[rA + 1]);
    eB = clampc(row_ptr[rA + 2]);
    if (eB < sB) eB = sB;
  }
  if (sB != eA) {
    if (lane == 0) ulen[p] = 0;
    return;
  }
  constexpr int64_t kRowMax = 1 << 30;       // entries read per row (the sum stays an int)
  const int64_t nA = min(eA - sA, kRowMax), nB = min(eB - sB, kRowMax);
  bool bad = false;
  for (int64_t t = lane; t < nA; t += 64) {
    const int x = col_idx[sA + t];
    bad = bad || x < 0 || x >= nb || (t > 0 && col_idx[sA + t - 1] >= x);
  }
  for (int64_t t = lane; t < nB; t += 64) {
    const int x = col_idx[sB + t];
    bad = bad || x < 0 || x >= nb || (t > 0 && col_idx[sB + t - 1] >= x);
  }
  if (!__any(bad)) {
    uint32_t* ba = bits[wid][0];
    uint32_t* bb = bits[wid][1];
    const int words = (nb + 31) / 32;
    for (int w = lane; w < words; w += 64) {
      ba[w] = 0u;
      bb[w] = 0u;
    }
    __builtin_amdgcn_wave_barrier();
    for (int64_t t = lane; t < nA; t += 64) {
      const int x = col_idx[sA + t];
      atomicOr(&ba[x >> 5], 1u << (x & 31));
    }
    for (int64_t t = lane; t < nB; t += 64) {
      const int x = col_idx[sB + t];
      atomicOr(&bb[x >> 5], 1u << (x & 31));
    }
    __builtin_amdgcn_wave_barrier();
    int64_t out = sA;
    for (int c = 0; c < (nb + 63) / 64; ++c) {
      const int j = 64 * c + lane;
      const bool inA = j < nb && ((ba[j >> 5] >> (j & 31)) & 1u);
      const bool inB = j < nb && ((bb[j >> 5] >> (j & 31)) & 1u);
      const uint64_t mk = __ballot(inA || inB);
      if (inA || inB) {
        const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
        units[out + rank] = (uint32_t)j | (inA ? kUnitA : 0u) | (inB ? kUnitB : 0u);
      }
      out += __popcll(mk);
    }
    if (lane == 0) ulen[p] = (int)(out - sA);
  } else {
    for (int64_t t = lane; t < nA; t += 64) {
      const int x = col_idx[sA + t];
      units[sA + t] = (x >= 0 && x < nb ? (uint32_t)x : kUnitNone) | kUnitA;
    }
    for (int64_t t = lane; t < nB; t += 64) {
      const int x = col_idx[sB + t];
      units[sA + nA + t] = (x >= 0 && x < nb ? (uint32_t)x : kUnitNone) | kUnitB;
    }
    if (lane == 0) ulen[p] = (int)(nA + nB);
  }
}

// 64-token blocks: pairs of query blocks in 128-query workgroups.
template <int D>
hipError_t launch_pairs(const Problem& p, const void* q, const void* k, const void* v, float scale,
                        const bsa_csr* mask, void* o, float* lse, float* mass, float* o32, const ForwardWs& w,
                        hipStream_t s) {
  using C = Cfg<128, D>;
  const int P = p.B * p.H * ((p.nb + 1) / 2);
  launch_pair_units(mask->row_ptr, mask->col_idx, mask->capacity, p.nb, P, w.units, w.ulen, s);
  const int T = tail_rows(P), t0 = P - T;
  launch_tail_order(nullptr, 0, w.ulen, t0, T, w.order, s);
  if (o32 != nullptr)
    fwd_kernel<128, D, true, true><<<P, C::THREADS, 0, s>>>(
        static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), mask->row_ptr,
        mask->col_idx, mask->capacity, static_cast<__bf16*>(o), lse, mass, mass ? w.part : nullptr, o32, p.N, p.nb,
        scale, w.order, t0, w.units, w.ulen);
  else
    fwd_kernel<128, D, false, true><<<P, C::THREADS, 0, s>>>(
        static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), mask->row_ptr,
        mask->col_idx, mask->capacity, static_cast<__bf16*>(o), lse, mass, mass ? w.part : nullptr, nullptr, p.N,
        p.nb, scale, w.order, t0, w.units, w.ulen);
  return hipGetLastError();
}

template <int BS, int D>
hipError_t launch_bs_d(const Problem& p, const void* q, const void* k, const void* v, float scale,
                       const bsa_csr* mask, void* o, float* lse, float* mass, float* o32, const ForwardWs& w,
                       hipStream_t s) {
  using C = Cfg<BS, D>;
  const int T = query_tail_rows(p.R, BS), t0 = p.R - T;
  launch_tail_order(mask->row_ptr, mask->capacity, nullptr, t0, T, w.order, s);
  if (o32 != nullptr)
    fwd_kernel<BS, D, true><<<p.R, C::THREADS, 0, s>>>(
        static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), mask->row_ptr,
        mask->col_idx, mask->capacity, static_cast<__bf16*>(o), lse, mass, mass ? w.part : nullptr, o32, p.N, p.nb,
        scale, w.order, t0, nullptr, nullptr);
  else
    fwd_kernel<BS, D, false><<<p.R, C::THREADS, 0, s>>>(
        static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v), mask->row_ptr,
        mask->col_idx, mask->capacity, static_cast<__bf16*>(o), lse, mass, mass ? w.part : nullptr, nullptr, p.N,
        p.nb, scale, w.order, t0, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace

void launch_pair_units(const int32_t* row_ptr, const int32_t* col_idx, int64_t cap, int nb, int P, uint32_t* units,
                       int32_t* ulen, hipStream_t s) {
  if (P > 0)
    pair_units_kernel<<<(P + kPairWaves - 1) / kPairWaves, 64 * kPairWaves, 0, s>>>(row_ptr, col_idx, cap, nb, P,
                                                                                     units, ulen);
}

hipError_t launch_forward_bf16(const Problem& p, const void* q, const void* k, const void* v, float scale,
                               const bsa_csr* mask, void* o, float* lse, float* mass, float* o32, const ForwardWs& w,
                               hipStream_t s) {
  if (p.bs == 128 && p.D == 128) return launch_bs_d<128, 128>(p, q, k, v, scale, mask, o, lse, mass, o32, w, s);
  if (p.bs == 128 && p.D == 64) return launch_bs_d<128, 64>(p, q, k, v, scale, mask, o, lse, mass, o32, w, s);
  if (p.bs == 64 && p.D == 128) return launch_pairs<128>(p, q, k, v, scale, mask, o, lse, mass, o32, w, s);
  return launch_pairs<64>(p, q, k, v, scale, mask, o, lse, mass, o32, w, s);
}

ForwardWs carve_forward(const Problem& p, int64_t capacity, bool want_mass, void* ws, size_t* bytes) {
  Carver c(ws);
  ForwardWs w{};
  if (want_mass) w.part = c.take<float>((size_t)capacity * p.bs);
  if (p.dtype == BSA_BF16) w.order = c.take<int32_t>(tail_rows(p.R));
  if (p.dtype == BSA_BF16 && p.bs == 64) {   // the pair grid's unit lists
    w.units = c.take<uint32_t>((size_t)capacity);
    w.ulen = c.take<int32_t>((size_t)p.B * p.H * ((p.nb + 1) / 2));
  }
  *bytes = align_up(c.off, 256);
  return w;
}

}  // namespace bsa
