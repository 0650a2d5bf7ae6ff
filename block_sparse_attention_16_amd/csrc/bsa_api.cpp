// C ABI of the block-sparse attention library: argument validation, workspace
// layout and dispatch to the HIP kernels.  Nothing here allocates device
// memory or synchronises the host.
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "bsa_internal.h"

namespace {

thread_local char g_err[512] = "";
constexpr int kMaxSubBlocks = 8;   // hierarchical block scoring: sub-blocks per key block

bsa_status fail(bsa_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bsa_status fail(bsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BSA_OK;
  return fail(BSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates the shape and fills the problem description.
bsa_status make_problem(const bsa_shape* s, bsa::Problem* p) {
  if (!s) return fail(BSA_ERR_INVALID_ARG, "shape is NULL");
  if (s->B < 1 || s->H < 1 || s->N < 1) return fail(BSA_ERR_INVALID_ARG, "B, H and N must be >= 1");
  if (s->D != 64 && s->D != 128) return fail(BSA_ERR_UNSUPPORTED, "D=%d: only 64 and 128 are built", s->D);
  if (s->block != 64 && s->block != 128)
    return fail(BSA_ERR_UNSUPPORTED, "block=%d: only 64 and 128 are built", s->block);
  if (s->dtype != BSA_BF16 && s->dtype != BSA_FP32) return fail(BSA_ERR_UNSUPPORTED, "dtype %d", s->dtype);
  const int64_t nb = ((int64_t)s->N + s->block - 1) / s->block;
  if (nb > 4096) return fail(BSA_ERR_UNSUPPORTED, "%lld blocks per sequence exceed 4096", (long long)nb);
  const int64_t elems = (int64_t)s->B * s->H * s->N * s->D;
  if (elems >= (int64_t(1) << 31)) return fail(BSA_ERR_UNSUPPORTED, "B*H*N*D must be below 2^31");
  const int64_t R = (int64_t)s->B * s->H * nb;
  if (R * nb >= (int64_t(1) << 31)) return fail(BSA_ERR_UNSUPPORTED, "B*H*nb*nb must be below 2^31");
  p->B = s->B; p->H = s->H; p->N = s->N; p->D = s->D; p->bs = s->block;
  p->nb = (int)nb; p->R = (int)R; p->dtype = s->dtype;
  p->elem = s->dtype == BSA_BF16 ? 2 : 4;
  return BSA_OK;
}

bsa_status check_tensor(const void* t, const char* name) {
  if (!t) return fail(BSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(t)) return fail(BSA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return BSA_OK;
}

bsa_status check_csr(const bsa_csr* c, const char* name) {
  if (!c) return fail(BSA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!c->row_ptr) return fail(BSA_ERR_INVALID_ARG, "%s->row_ptr is NULL", name);
  if (c->capacity < 0) return fail(BSA_ERR_INVALID_ARG, "%s->capacity is negative", name);
  if (c->capacity > 0 && !c->col_idx) return fail(BSA_ERR_INVALID_ARG, "%s->col_idx is NULL", name);
  return BSA_OK;
}

float resolve_scale(float scale, int D) {
  return scale > 0.f ? scale : (float)(1.0 / std::sqrt((double)D));
}

#define BSA_TRY(x)                      \
  do {                                  \
    bsa_status st_ = (x);               \
    if (st_ != BSA_OK) return st_;      \
  } while (0)

}  // namespace

extern "C" {

size_t bsa_workspace_size(const bsa_shape* shape, int32_t kind, int64_t capacity) {
  bsa::Problem p;
  if (make_problem(shape, &p) != BSA_OK || capacity < 0) return 0;
  size_t bytes = 0;
  switch (kind) {
    case BSA_WS_ESTIMATE: bsa::carve_estimate(p, 1, nullptr, &bytes); break;
    case BSA_WS_ESTIMATE_HIER: bsa::carve_estimate(p, kMaxSubBlocks, nullptr, &bytes); break;
    case BSA_WS_FORWARD: bsa::carve_forward(p, capacity, true, nullptr, &bytes); break;
    case BSA_WS_BACKWARD: bsa::carve_backward(p, capacity, nullptr, &bytes); break;
    case BSA_WS_SELECT_FROM_MASS:
    case BSA_WS_STRUCTURED: bsa::carve_select(p, nullptr, &bytes); break;
    default: return 0;
  }
  return bytes;
}

static bsa_status estimate_common(const bsa_shape* shape, const void* q, const void* k, float top_p, float scale,
                                  const bsa_csr* candidate, int32_t keep_prefix_tokens, int32_t sub_blocks,
                                  bsa_csr* out, void* ws, size_t ws_bytes, void* stream, size_t need_for) {
  g_err[0] = 0;
  bsa::Problem p;
  BSA_TRY(make_problem(shape, &p));
  BSA_TRY(check_tensor(q, "q"));
  BSA_TRY(check_tensor(k, "k"));
  if (!(top_p > 0.f && top_p <= 1.f)) return fail(BSA_ERR_INVALID_ARG, "top_p=%g is outside (0, 1]", top_p);
  if (!std::isfinite(scale)) return fail(BSA_ERR_INVALID_ARG, "scale is not finite");
  if (keep_prefix_tokens < 0 || keep_prefix_tokens > p.N)
    return fail(BSA_ERR_INVALID_ARG, "keep_prefix_tokens=%d is outside [0, N]", keep_prefix_tokens);
  if (sub_blocks != 1 && sub_blocks != 2 && sub_blocks != 4 && sub_blocks != 8)
    return fail(BSA_ERR_INVALID_ARG, "sub_blocks=%d is not 1, 2, 4 or 8", sub_blocks);
  BSA_TRY(check_csr(out, "out"));
  if (candidate) {
    BSA_TRY(check_csr(candidate, "candidate"));
    if (candidate->row_ptr == out->row_ptr || (candidate->col_idx && candidate->col_idx == out->col_idx))
      return fail(BSA_ERR_INVALID_ARG, "candidate aliases out");
  }
  size_t need = 0;
  bsa::carve_estimate(p, (int)need_for, nullptr, &need);
  if (ws_bytes < need || (need && !ws))
    return fail(BSA_ERR_WORKSPACE, "estimate workspace needs %zu bytes, got %zu", need, ws_bytes);
  bsa::EstimateWs w = bsa::carve_estimate(p, (int)need_for, ws, &need);
  return hip_status(bsa::launch_estimate(p, q, k, top_p, resolve_scale(scale, p.D), candidate, keep_prefix_tokens,
                                         sub_blocks, out, w, static_cast<hipStream_t>(stream)),
                    "estimate launch");
}

bsa_status bsa_estimate_mask(const bsa_shape* shape, const void* q, const void* k, float top_p, float scale,
                             const bsa_csr* candidate, int32_t keep_prefix_tokens, bsa_csr* out, void* ws,
                             size_t ws_bytes, void* stream) {
  return estimate_common(shape, q, k, top_p, scale, candidate, keep_prefix_tokens, 1, out, ws, ws_bytes, stream, 1);
}

bsa_status bsa_estimate_mask_hierarchical(const bsa_shape* shape, const void* q, const void* k, float top_p,
                                          float scale, const bsa_csr* candidate, int32_t keep_prefix_tokens,
                                          int32_t sub_blocks, bsa_csr* out, void* ws, size_t ws_bytes,
                                          void* stream) {
  return estimate_common(shape, q, k, top_p, scale, candidate, keep_prefix_tokens, sub_blocks, out, ws, ws_bytes,
                         stream, kMaxSubBlocks);
}

// Argument checks shared by the two narrowing entry points.
static bsa_status check_select_args(const bsa_shape* shape, const bsa_csr* mask, const float* block_mass,
                                    float top_p, int32_t keep_prefix_tokens, const bsa_csr* out, bsa::Problem* p) {
  BSA_TRY(make_problem(shape, p));
  BSA_TRY(check_csr(mask, "mask"));
  BSA_TRY(check_csr(out, "out"));
  if (mask->capacity > 0 && !block_mass) return fail(BSA_ERR_INVALID_ARG, "block_mass is NULL");
  if (!(top_p > 0.f && top_p <= 1.f)) return fail(BSA_ERR_INVALID_ARG, "top_p=%g is outside (0, 1]", top_p);
  if (keep_prefix_tokens < 0 || keep_prefix_tokens > p->N)
    return fail(BSA_ERR_INVALID_ARG, "keep_prefix_tokens=%d is outside [0, N]", keep_prefix_tokens);
  if (mask->row_ptr == out->row_ptr || (mask->col_idx && mask->col_idx == out->col_idx))
    return fail(BSA_ERR_INVALID_ARG, "mask aliases out");
  return BSA_OK;
}

bsa_status bsa_select_from_mass(const bsa_shape* shape, const bsa_csr* mask, const float* block_mass, float top_p,
                                int32_t keep_prefix_tokens, bsa_csr* out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  bsa::Problem p;
  BSA_TRY(check_select_args(shape, mask, block_mass, top_p, keep_prefix_tokens, out, &p));
  size_t need = 0;
  bsa::carve_select(p, nullptr, &need);
  if (ws_bytes < need || (need && !ws))
    return fail(BSA_ERR_WORKSPACE, "select workspace needs %zu bytes, got %zu", need, ws_bytes);
  bsa::SelectWs w = bsa::carve_select(p, ws, &need);
  return hip_status(bsa::launch_select_from_mass(p, mask, block_mass, top_p, keep_prefix_tokens, out, w,
                                                 static_cast<hipStream_t>(stream)),
                    "select-from-mass launch");
}

bsa_status bsa_select_from_mass_noalloc(const bsa_shape* shape, const bsa_csr* mask, const float* block_mass,
                                        float top_p, int32_t keep_prefix_tokens, bsa_csr* out, void* stream) {
  g_err[0] = 0;
  bsa::Problem p;
  BSA_TRY(check_select_args(shape, mask, block_mass, top_p, keep_prefix_tokens, out, &p));
  size_t need = 0;
  bsa::carve_select(p, nullptr, &need);
  if (need > bsa::kNoAllocScratchBytes)
    return fail(BSA_ERR_WORKSPACE, "narrowing needs %zu bytes of scratch; the built-in scratch holds %zu",
                need, bsa::kNoAllocScratchBytes);
  void* scratch = nullptr;
  BSA_TRY(hip_status(bsa::scratch_for_stream(static_cast<hipStream_t>(stream), &scratch), "scratch lookup"));
  bsa::SelectWs w = bsa::carve_select(p, scratch, &need);
  return hip_status(bsa::launch_select_from_mass(p, mask, block_mass, top_p, keep_prefix_tokens, out, w,
                                                 static_cast<hipStream_t>(stream)),
                    "select-from-mass launch");
}

bsa_status bsa_structured_mask(const bsa_shape* shape, const int32_t* head_kind, const bsa_pattern_params* params,
                               bsa_csr* out, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  bsa::Problem p;
  BSA_TRY(make_problem(shape, &p));
  if (!head_kind) return fail(BSA_ERR_INVALID_ARG, "head_kind is NULL");
  if (!params) return fail(BSA_ERR_INVALID_ARG, "params is NULL");
  BSA_TRY(check_csr(out, "out"));
  const bsa_pattern_params& q = *params;
  if (q.prefix_tokens < 0 || q.prefix_tokens > p.N)
    return fail(BSA_ERR_INVALID_ARG, "prefix_tokens=%d is outside [0, N]", q.prefix_tokens);
  if (q.frame_tokens < 1) return fail(BSA_ERR_INVALID_ARG, "frame_tokens=%d must be >= 1", q.frame_tokens);
  if (q.band < 0) return fail(BSA_ERR_INVALID_ARG, "band=%d must be >= 0", q.band);
  if (q.period < 1) return fail(BSA_ERR_INVALID_ARG, "period=%d must be >= 1", q.period);
  if (q.n_stripes < 0 || (q.n_stripes > 0 && !q.stripes))
    return fail(BSA_ERR_INVALID_ARG, "stripes: n_stripes=%d with %s array", q.n_stripes,
                q.stripes ? "an" : "no");
  size_t need = 0;
  bsa::carve_select(p, nullptr, &need);
  if (ws_bytes < need || (need && !ws))
    return fail(BSA_ERR_WORKSPACE, "structured-mask workspace needs %zu bytes, got %zu", need, ws_bytes);
  bsa::SelectWs w = bsa::carve_select(p, ws, &need);
  return hip_status(bsa::launch_structured_mask(p, head_kind, q, out, w, static_cast<hipStream_t>(stream)),
                    "structured-mask launch");
}

bsa_status bsa_permute_rows(int64_t heads, int32_t n, int32_t row_bytes, const void* src, const int32_t* perm,
                            int32_t inverse, void* dst, void* stream) {
  g_err[0] = 0;
  if (heads < 1 || n < 1) return fail(BSA_ERR_INVALID_ARG, "heads=%lld and n=%d must be >= 1", (long long)heads, n);
  if (row_bytes < 4 || row_bytes % 4 != 0)
    return fail(BSA_ERR_INVALID_ARG, "row_bytes=%d must be a positive multiple of 4", row_bytes);
  if (!src || !dst || !perm) return fail(BSA_ERR_INVALID_ARG, "src, dst and perm must not be NULL");
  if ((reinterpret_cast<uintptr_t>(src) & 3u) || (reinterpret_cast<uintptr_t>(dst) & 3u))
    return fail(BSA_ERR_INVALID_ARG, "src and dst must be 4-byte aligned");
  if (inverse != 0 && inverse != 1) return fail(BSA_ERR_INVALID_ARG, "inverse must be 0 or 1");
  const int64_t words = heads * (int64_t)n * (row_bytes / 4);
  if (heads > (int64_t(1) << 31) / n || words >= (int64_t(1) << 31))
    return fail(BSA_ERR_UNSUPPORTED, "heads*n*row_bytes/4 must be below 2^31");
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t bytes = (uintptr_t)words * 4;
  if (a < b + bytes && b < a + bytes) return fail(BSA_ERR_INVALID_ARG, "src and dst overlap");
  return hip_status(bsa::launch_permute_rows(heads, n, row_bytes, src, perm, inverse == 1, dst,
                                             static_cast<hipStream_t>(stream)),
                    "permute launch");
}

bsa_status bsa_forward(const bsa_shape* shape, const void* q, const void* k, const void* v, float scale,
                       const bsa_csr* mask, void* o, float* lse, float* block_mass, float* o_f32, void* ws,
                       size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  bsa::Problem p;
  BSA_TRY(make_problem(shape, &p));
  BSA_TRY(check_tensor(q, "q"));
  BSA_TRY(check_tensor(k, "k"));
  BSA_TRY(check_tensor(v, "v"));
  BSA_TRY(check_tensor(o, "o"));
  BSA_TRY(check_tensor(lse, "lse"));
  if (o_f32) {
    if (p.dtype != BSA_BF16) return fail(BSA_ERR_INVALID_ARG, "o_f32 is for bf16 data only");
    BSA_TRY(check_tensor(o_f32, "o_f32"));
  }
  if (!std::isfinite(scale)) return fail(BSA_ERR_INVALID_ARG, "scale is not finite");
  BSA_TRY(check_csr(mask, "mask"));
  size_t need = 0;
  bsa::carve_forward(p, mask->capacity, block_mass != nullptr, nullptr, &need);
  if (ws_bytes < need || (need && !ws))
    return fail(BSA_ERR_WORKSPACE, "forward workspace needs %zu bytes, got %zu", need, ws_bytes);
  bsa::ForwardWs w = bsa::carve_forward(p, mask->capacity, block_mass != nullptr, ws, &need);
  const float sc = resolve_scale(scale, p.D);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = p.dtype == BSA_BF16 ? bsa::launch_forward_bf16(p, q, k, v, sc, mask, o, lse, block_mass, o_f32, w, s)
                                     : bsa::launch_forward_fp32(p, q, k, v, sc, mask, o, lse, block_mass, w, s);
  return hip_status(e, "forward launch");
}

bsa_status bsa_backward(const bsa_shape* shape, const void* q, const void* k, const void* v, const void* o,
                        const float* o_f32, const void* d_o, const float* lse, float scale, const bsa_csr* mask,
                        void* dq, void* dk, void* dv, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  bsa::Problem p;
  BSA_TRY(make_problem(shape, &p));
  BSA_TRY(check_tensor(q, "q"));
  BSA_TRY(check_tensor(k, "k"));
  BSA_TRY(check_tensor(v, "v"));
  BSA_TRY(check_tensor(o, "o"));
  BSA_TRY(check_tensor(d_o, "d_o"));
  BSA_TRY(check_tensor(lse, "lse"));
  BSA_TRY(check_tensor(dq, "dq"));
  BSA_TRY(check_tensor(dk, "dk"));
  BSA_TRY(check_tensor(dv, "dv"));
  if (o_f32) {
    if (p.dtype != BSA_BF16) return fail(BSA_ERR_INVALID_ARG, "o_f32 is for bf16 data only");
    BSA_TRY(check_tensor(o_f32, "o_f32"));
  }
  if (!std::isfinite(scale)) return fail(BSA_ERR_INVALID_ARG, "scale is not finite");
  BSA_TRY(check_csr(mask, "mask"));
  size_t need = 0;
  bsa::carve_backward(p, mask->capacity, nullptr, &need);
  if (ws_bytes < need || (need && !ws))
    return fail(BSA_ERR_WORKSPACE, "backward workspace needs %zu bytes, got %zu", need, ws_bytes);
  bsa::BackwardWs w = bsa::carve_backward(p, mask->capacity, ws, &need);
  return hip_status(bsa::launch_backward(p, q, k, v, o, o_f32, d_o, lse, resolve_scale(scale, p.D), mask, dq, dk, dv, w,
                                         static_cast<hipStream_t>(stream)),
                    "backward launch");
}

const char* bsa_status_string(bsa_status status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_ERR_INVALID_ARG: return "invalid argument";
    case BSA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case BSA_ERR_WORKSPACE: return "workspace or capacity too small";
    case BSA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* bsa_last_error(void) { return g_err; }

int32_t bsa_version(void) { return 100; }

}  // extern "C"
