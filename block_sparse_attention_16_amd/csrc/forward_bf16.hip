// Sparse attention forward with exact per-block attention mass, bf16 MFMA (gfx950).
//
// Stage two of the estimate-then-attend scheme (DSV page, Abstract): a
// FlashAttention-style online-softmax forward that visits only the key blocks
// of each query block's CSR row, and obtains the exact attention weight of
// every visited block inside the same pass (GSRS page, Abstract; the
// block-level attention map of its Figure 3 caption).
//
// Workgroup = one mask row (query block i of head bh), 4 waves.  Wave
// w = 2*qg + kg owns queries [qg*BS/2, (qg+1)*BS/2) of the block and keys
// [kg*BS/2, (kg+1)*BS/2) of every visited key block, with its own online
// softmax state; the two key halves are merged once at the end.
//
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// A = K rows from LDS, B = Q^T held in registers.  In the 32x32 accumulator a
// lane holds one query column and 16 key rows, so a query's row max and sum
// need one cross-half exchange (lane ^ 32).  The same registers, rounded to
// bf16, are the B operand of O^T += V^T P^T: the MFMA k-slots of a lane half
// map to key rows {16g + 8a + 4h + r}, so V^T is stored with bits 2 and 3 of
// the key index swapped inside every 16-key group (done by vt_kernel).
//
// K and V^T tiles stream from HBM/L2 straight into LDS with
// global_load_lds_dwordx4, double-buffered: block t+1 is in flight while
// block t is computed.  LDS rows are XOR-swizzled in 16-byte chunks so the
// MFMA operand reads are bank-conflict free.
#include "bsa_internal.h"

namespace bsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kThreads = 256;

__device__ __forceinline__ int key_slot(int key) {  // swap bits 2 and 3
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// 16-byte chunk swizzle for an LDS tile whose rows are `cpr` chunks long.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  static_assert(CPR == 16 || CPR == 8, "row must be 128 or 256 bytes");
  return CPR == 16 ? (row & 15) : ((row >> 1) & 7);
}

// V [BH, N, D] -> vt [BH, nb, D, BS]: each key block transposed, keys permuted
// by key_slot inside 16-key groups, keys >= N zero.  grid (nb, BH), 256 threads.
template <int BS, int D>
__global__ __launch_bounds__(kThreads) void vt_kernel(const __bf16* __restrict__ v, __bf16* __restrict__ vt, int N,
                                                      int nb) {
  __shared__ uint16_t tile[BS][D + 2];
  const int jb = blockIdx.x, bh = blockIdx.y;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(v) + ((size_t)bh * N + (size_t)jb * BS) * D;
  // coalesced read: 8 elements per thread step
  for (int c = threadIdx.x; c < BS * D / 8; c += kThreads) {
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (jb * BS + row < N) u = *reinterpret_cast<const uint4*>(src + (size_t)row * D + col);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[row][col + 2 * e] = (uint16_t)(w[e] & 0xffff);
      tile[row][col + 2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
  uint16_t* dst = reinterpret_cast<uint16_t*>(vt) + ((size_t)bh * nb + jb) * (size_t)D * BS;
  for (int c = threadIdx.x; c < D * BS / 2; c += kThreads) {
    const int d = c / (BS / 2), s2 = (c % (BS / 2)) * 2;      // slots s2, s2+1 hold keys key_slot(s2), +1
    const int k0 = key_slot(s2);
    const uint32_t lo = tile[k0][d], hi = tile[k0 + 1][d];
    reinterpret_cast<uint32_t*>(dst)[(d * BS + s2) / 2] = lo | (hi << 16);
  }
}

__device__ __forceinline__ void lds_dma16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

template <int BS, int D>
struct Cfg {
  static constexpr int QPW = BS / 2, KPW = BS / 2;    // queries / keys per wave
  static constexpr int QT = QPW / 32, KT = KPW / 32;  // 32-wide tiles
  static constexpr int DS = D / 16, DT = D / 32;      // MFMA k-steps over d, d tiles
  static constexpr int CPR_K = D / 8;                 // 16-byte chunks per K row
  static constexpr int CPR_V = BS / 8;                // 16-byte chunks per V^T row
  static constexpr int TILE_BYTES = BS * D * 2;       // one K or V^T tile
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  static constexpr int LOADS = TILE_BYTES / (16 * kThreads);  // dma ops per thread per tile
  static constexpr int MERGE_BYTES = 2 * DT * QT * 16 * 64 * 4 + 2 * 2 * QT * 64 * 4;
  static constexpr int LDS_BYTES = (2 * STAGE_BYTES > MERGE_BYTES ? 2 * STAGE_BYTES : MERGE_BYTES) + BS * 4;
};

// Issue the DMA of K block j and V^T block j into one LDS stage.
template <int BS, int D>
__device__ __forceinline__ void issue_tile_loads(const __bf16* __restrict__ kh, const __bf16* __restrict__ vth,
                                                 int j, int N, char* stage, int wave, int lane) {
  using C = Cfg<BS, D>;
  const int key0 = j * BS;
#pragma unroll
  for (int it = 0; it < C::LOADS; ++it) {
    const int chunk0 = (it * 4 + wave) * 64;   // first LDS chunk of this wave's 1 KB
    const int L = chunk0 + lane;
    const int row = L / C::CPR_K, pos = L % C::CPR_K;
    const int c = pos ^ swz<C::CPR_K>(row);
    const int key = min(key0 + row, N - 1);
    lds_dma16(kh + (size_t)key * D + c * 8, stage + chunk0 * 16);
  }
  const __bf16* vtile = vth + (size_t)j * D * BS;
#pragma unroll
  for (int it = 0; it < C::LOADS; ++it) {
    const int chunk0 = (it * 4 + wave) * 64;
    const int L = chunk0 + lane;
    const int row = L / C::CPR_V, pos = L % C::CPR_V;
    const int c = pos ^ swz<C::CPR_V>(row);
    lds_dma16(vtile + (size_t)row * BS + c * 8, stage + C::TILE_BYTES + chunk0 * 16);
  }
}

template <int BS, int D>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ vt,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx, int64_t cap, __bf16* __restrict__ o,
    float* __restrict__ lse, float* __restrict__ mass, float* __restrict__ part, int N, int nb, int R, float scale,
    int xcd_remap) {
  using C = Cfg<BS, D>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // blockIdx -> mask row.  Workgroups are dealt to the 8 XCDs round-robin;
  // with xcd_remap each XCD takes a contiguous range of rows instead.
  int r = blockIdx.x;
  if (xcd_remap) {
    const int per = (R + 7) / 8;
    r = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (r >= R) return;
  }
  const int bh = r / nb, i = r - bh * nb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qg = wave >> 1, kg = wave & 1;
  const int l32 = lane & 31, hf = lane >> 5;
  const int q0 = i * BS;
  const int nq = min(BS, N - q0);

  int64_t e_begin = row_ptr[r], e_end = row_ptr[r + 1];
  if (e_end > cap) e_end = cap;
  if (e_begin < 0) e_begin = 0;
  if (e_begin > e_end) e_begin = e_end;
  const int n_e = (int)(e_end - e_begin);

  const __bf16* kh = k + (size_t)bh * N * D;
  const __bf16* vth = vt + (size_t)bh * nb * D * BS;

  // Q^T fragments (B operand): lane holds query (qg*QPW + qt*32 + l32), d = ds*16 + hf*8 .. +8
  bf16x8 qf[C::QT][C::DS];
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) {
    const int qq = q0 + qg * C::QPW + qt * 32 + l32;
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
      if (qq < N) {
        qf[qt][ds] = *reinterpret_cast<const bf16x8*>(q + ((size_t)bh * N + qq) * D + ds * 16 + hf * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[qt][ds][e] = (__bf16)0.f;
      }
    }
  }

  floatx16 acc[C::DT][C::QT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[dt][qt][v] = 0.f;
  float m_run[C::QT], l_run[C::QT];
#pragma unroll
  for (int qt = 0; qt < C::QT; ++qt) { m_run[qt] = -INFINITY; l_run[qt] = 0.f; }

  const float c2 = scale * kLog2e;   // logits in base-2 units

  if (n_e > 0) {
    int j_next = col_idx[e_begin];
    issue_tile_loads<BS, D>(kh, vth, (j_next >= 0 && j_next < nb) ? j_next : 0, N, smem, wave, lane);
  }

  for (int it = 0; it < n_e; ++it) {
    const int64_t e = e_begin + it;
    const int j_raw = col_idx[e];
    const bool valid = j_raw >= 0 && j_raw < nb;
    const int j = valid ? j_raw : 0;
    char* stage = smem + (it & 1) * C::STAGE_BYTES;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (it + 1 < n_e) {
      const int jn = col_idx[e + 1];
      issue_tile_loads<BS, D>(kh, vth, (jn >= 0 && jn < nb) ? jn : 0, N, smem + ((it + 1) & 1) * C::STAGE_BYTES,
                              wave, lane);
    }
    const char* ks = stage;
    const char* vs = stage + C::TILE_BYTES;

    // S^T = K Q^T for this wave's key half
    floatx16 st[C::KT][C::QT];
#pragma unroll
    for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
      for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
        for (int v = 0; v < 16; ++v) st[kt][qt][v] = 0.f;
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt) {
        const int row = kg * C::KPW + kt * 32 + l32;
        const int c = (ds * 2 + hf) ^ swz<C::CPR_K>(row);
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (row * C::CPR_K + c) * 16);
#pragma unroll
        for (int qt = 0; qt < C::QT; ++qt)
          st[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qt][ds], st[kt][qt], 0, 0, 0);
      }
    }

    // mask keys past the end of the sequence (partial last block) or of an invalid entry
    const int key_base = j * BS + kg * C::KPW;
    if (!valid || key_base + C::KPW > N) {
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = key_base + kt * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
          if (!valid || key >= N) {
#pragma unroll
            for (int qt = 0; qt < C::QT; ++qt) st[kt][qt][v] = -INFINITY;
          }
        }
    }

    // online softmax per query column
    bf16x8 pb[C::KT][C::QT][2];
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, st[kt][qt][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[qt], mx * c2);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_use);
      m_run[qt] = m_new;
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(st[kt][qt][v], c2, -m_use));
          st[kt][qt][v] = p;
          ls += p;
        }
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int e2 = 0; e2 < 8; ++e2) pb[kt][qt][h2][e2] = (__bf16)st[kt][qt][h2 * 8 + e2];
      }
      ls += __shfl_xor(ls, 32);
      l_run[qt] = l_run[qt] * alpha + ls;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[dt][qt][v] *= alpha;
      if (part != nullptr && hf == 0) {
        // log2 of this wave's key-half sum for this block: m + log2(l_block)
        const float cval = ls > 0.f ? m_use + __builtin_amdgcn_logf(ls) : -INFINITY;
        part[(e * 2 + kg) * BS + qg * C::QPW + qt * 32 + l32] = cval;
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int row = dt * 32 + l32;
#pragma unroll
      for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int slot = kg * C::KPW + kt * 32 + h2 * 16 + hf * 8;
          const int c = (slot >> 3) ^ swz<C::CPR_V>(row);
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vs + (row * C::CPR_V + c) * 16);
#pragma unroll
          for (int qt = 0; qt < C::QT; ++qt)
            acc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kt][qt][h2], acc[dt][qt], 0, 0, 0);
        }
      }
    }
  }

  // ---- merge the two key halves, normalise, write O and LSE ----
  __syncthreads();   // all waves done with the stage buffers
  float* mo = reinterpret_cast<float*>(smem);                       // [qg][DT][QT][16][64]
  float* mml = mo + 2 * C::DT * C::QT * 16 * 64;                    // [qg][2][QT][64]
  float* lse2_s = reinterpret_cast<float*>(smem + C::LDS_BYTES - BS * 4);
  if (kg == 1) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int qt = 0; qt < C::QT; ++qt)
#pragma unroll
        for (int v = 0; v < 16; ++v) mo[(((qg * C::DT + dt) * C::QT + qt) * 16 + v) * 64 + lane] = acc[dt][qt][v];
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt) {
      mml[((qg * 2 + 0) * C::QT + qt) * 64 + lane] = m_run[qt];
      mml[((qg * 2 + 1) * C::QT + qt) * 64 + lane] = l_run[qt];
    }
  }
  __syncthreads();
  if (kg == 0) {
#pragma unroll
    for (int qt = 0; qt < C::QT; ++qt) {
      const float m1 = mml[((qg * 2 + 0) * C::QT + qt) * 64 + lane];
      const float l1 = mml[((qg * 2 + 1) * C::QT + qt) * 64 + lane];
      const float m0 = m_run[qt], l0 = l_run[qt];
      const float mm = fmaxf(m0, m1);
      const float mu = mm == -INFINITY ? 0.f : mm;
      const float a0 = __builtin_amdgcn_exp2f(m0 - mu), a1 = __builtin_amdgcn_exp2f(m1 - mu);
      const float l = l0 * a0 + l1 * a1;
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int qloc = qg * C::QPW + qt * 32 + l32;
      const int qq = q0 + qloc;
      const float lse2 = l > 0.f ? mu + __builtin_amdgcn_logf(l) : -INFINITY;
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
            for (int r4 = 0; r4 < 4; ++r4) {
              const int v = g * 4 + r4;
              const float x1 = mo[(((qg * C::DT + dt) * C::QT + qt) * 16 + v) * 64 + lane];
              out4[r4] = (__bf16)((acc[dt][qt][v] * a0 + x1 * a1) * inv);
            }
            *reinterpret_cast<bf16x4*>(orow + dt * 32 + 8 * g + 4 * hf) = out4;
          }
        }
      }
    }
  }
  if (mass == nullptr || n_e == 0) return;
  __syncthreads();

  // ---- exact block mass: mean over valid queries of exp2(part - lse2) ----
  for (int it = wave; it < n_e; it += 4) {
    const int64_t e = e_begin + it;
    const int j_raw = col_idx[e];
    float s = 0.f;
    if (j_raw >= 0 && j_raw < nb) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        for (int qq = lane; qq < nq; qq += 64)
          s += __builtin_amdgcn_exp2f(part[(e * 2 + h2) * BS + qq] - lse2_s[qq]);
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) mass[e] = s / (float)nq;
  }
}

template <int BS, int D>
hipError_t launch_bs_d(const Problem& p, const void* q, const void* k, const void* v, float scale,
                       const bsa_csr* mask, void* o, float* lse, float* mass, const ForwardWs& w, hipStream_t s) {
  using C = Cfg<BS, D>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t err = hipFuncSetAttribute((const void*)fwd_kernel<BS, D>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (err != hipSuccess) return err;
    attr_set = true;
  }
  vt_kernel<BS, D><<<dim3(p.nb, p.B * p.H), kThreads, 0, s>>>(static_cast<const __bf16*>(v),
                                                                static_cast<__bf16*>(w.vt), p.N, p.nb);
  const int xcd = 0;
  const int grid = xcd ? ((p.R + 7) / 8) * 8 : p.R;
  fwd_kernel<BS, D><<<grid, kThreads, C::LDS_BYTES, s>>>(
      static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(w.vt), mask->row_ptr,
      mask->col_idx, mask->capacity, static_cast<__bf16*>(o), lse, mass, mass ? w.part : nullptr, p.N, p.nb, p.R,
      scale, xcd);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_bf16(const Problem& p, const void* q, const void* k, const void* v, float scale,
                               const bsa_csr* mask, void* o, float* lse, float* mass, const ForwardWs& w,
                               hipStream_t s) {
  if (p.bs == 128 && p.D == 128) return launch_bs_d<128, 128>(p, q, k, v, scale, mask, o, lse, mass, w, s);
  if (p.bs == 128 && p.D == 64) return launch_bs_d<128, 64>(p, q, k, v, scale, mask, o, lse, mass, w, s);
  if (p.bs == 64 && p.D == 128) return launch_bs_d<64, 128>(p, q, k, v, scale, mask, o, lse, mass, w, s);
  return launch_bs_d<64, 64>(p, q, k, v, scale, mask, o, lse, mass, w, s);
}

}  // namespace bsa

namespace bsa {

ForwardWs carve_forward(const Problem& p, int64_t capacity, bool want_mass, void* ws, size_t* bytes) {
  Carver c(ws);
  ForwardWs w{};
  if (p.dtype == BSA_BF16) w.vt = c.take<uint16_t>((size_t)p.B * p.H * p.nb * p.D * p.bs);
  if (want_mass) w.part = c.take<float>((size_t)capacity * 2 * p.bs);
  *bytes = align_up(c.off, 256);
  return w;
}

}  // namespace bsa
