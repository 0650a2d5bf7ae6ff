/*
 * bsa.h -- C ABI of the MI355X (gfx950) dynamic block-sparse attention library.
 *
 * The library computes, on one GPU, the two-stage estimate-then-attend scheme
 * for video diffusion transformers:
 *
 *   1. a block-importance estimator: mean-pool Q and K over each token block,
 *      score every (query block, key block) pair with the pooled dot product,
 *      take a softmax over each query block's row and keep, per row, the
 *      fewest highest-scoring key blocks whose probability reaches top_p.
 *      Two-stage estimation of critical key-value pairs: DSV page, Abstract.
 *      Top-p selection: GSRS page ("Sparse Attention for Video Generation
 *      Acceleration via Growing Sparsity and Reduced Search"), Abstract.
 *      Restricting a later search to an earlier step's blocks ("reduced
 *      search"): GSRS page, Abstract and Figure 4 caption.
 *   2. a FlashAttention-style forward over the selected key blocks that also
 *      returns the exact attention mass of every selected block (the block-
 *      level attention map of the GSRS page, Figure 3 caption, computed inside
 *      the attention kernel as the GSRS abstract describes), and
 *   3. the matching backward pass (dQ, dK, dV) over the same block mask, for
 *      training with dynamic sparsity (DSV page, Abstract).
 *
 * Conventions shared by every entry point
 *   - Tensors Q, K, V, O, dO, dQ, dK, dV are contiguous [B, H, N, D] device
 *     arrays of the dtype in bsa_shape (bf16 or fp32); LSE is [B, H, N] fp32.
 *   - Token block i of a sequence covers tokens [i*block, min((i+1)*block, N));
 *     nb = ceil(N / block) query blocks = key blocks; the last one may be
 *     partial.  Mask rows are ordered r = (b*H + h)*nb + i; R = B*H*nb.
 *   - Every pointer is a device pointer owned by the caller.  The library
 *     never allocates or frees device memory and never synchronises the host;
 *     all work is enqueued on `stream` (a hipStream_t; NULL = null stream).
 *   - Arguments are validated on the host before anything is launched; a
 *     failed check returns an error status and enqueues nothing.  A HIP launch
 *     error returns BSA_ERR_HIP.  No C++ exception crosses this interface.
 *     bsa_last_error() describes the latest failure on the calling thread.
 *   - Supported: D in {64, 128}, block in {64, 128}, nb <= 4096, B*H*N*D < 2^31.
 */
#ifndef BSA_H_
#define BSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, p outside (0,1], ... */
  BSA_ERR_UNSUPPORTED = 2,   /* D, block or dtype the kernels are not built for */
  BSA_ERR_WORKSPACE = 3,     /* workspace or CSR capacity too small */
  BSA_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed */
} bsa_status;

typedef enum { BSA_BF16 = 0, BSA_FP32 = 1 } bsa_dtype;

/* Problem shape.  dtype selects the element type of every [B,H,N,D] tensor:
 * BSA_BF16 is the production path (bf16 MFMA, fp32 accumulation);
 * BSA_FP32 is the debug path (fp32 arithmetic throughout). */
typedef struct {
  int32_t B, H, N, D, block;
  int32_t dtype; /* bsa_dtype */
} bsa_shape;

/* Block mask in CSR form over the R mask rows.
 *   row_ptr [R+1]  int32, row_ptr[0] = 0, non-decreasing; row r's key blocks
 *                  are col_idx[row_ptr[r] .. row_ptr[r+1]).
 *   col_idx [capacity] int32 key-block ids, strictly ascending within a row.
 *   capacity       number of int32 slots col_idx (and a block_mass array)
 *                  can hold.  R*nb always suffices.
 * Kernels never touch col_idx at or beyond capacity: entries there are
 * ignored, and ids outside [0, nb) are ignored. */
typedef struct {
  int32_t* row_ptr;
  int32_t* col_idx;
  int64_t capacity;
} bsa_csr;

/* Which call a workspace is sized for. */
typedef enum {
  BSA_WS_ESTIMATE = 0,
  BSA_WS_FORWARD = 1,
  BSA_WS_BACKWARD = 2,
  BSA_WS_SELECT_FROM_MASS = 3,
  BSA_WS_STRUCTURED = 4,
  BSA_WS_ESTIMATE_HIER = 5    /* bsa_estimate_mask_hierarchical, any sub_blocks */
} bsa_ws_kind;

/* Bytes of device workspace `kind` needs for `shape` and a CSR of `capacity`
 * entries (the forward stores per-entry partial sums for the block mass).
 * Returns 0 for an invalid shape. */
size_t bsa_workspace_size(const bsa_shape* shape, int32_t kind, int64_t capacity);

/* Block-importance estimator (see the header comment, stage 1).
 *   q, k       [B,H,N,D] device tensors of shape->dtype.
 *   top_p      in (0, 1]; 1 keeps every candidate block.
 *   scale      score temperature; <= 0 selects 1/sqrt(D) (the attention scale).
 *   candidate  NULL: every key block is scored.  Otherwise a CSR over the same
 *              R rows; row r scores, softmaxes and ranks only its candidate
 *              blocks (reduced search).  An empty candidate row selects only
 *              the forced blocks.  Every entry of a row is read (up to
 *              2^31 - 1 per row), in any order; repeated ids count once and
 *              ids outside [0, nb) are ignored.  Must not alias `out`.
 *   keep_prefix_tokens  in [0, N]: key blocks j with j*block < keep_prefix_tokens
 *              (e.g. a text prefix) join every row after the Top-p cut.
 *   out        CSR written by the call.  out->row_ptr receives exact offsets
 *              even when the total exceeds out->capacity; entries past the
 *              capacity are dropped, so a caller checks row_ptr[R] <= capacity.
 *   ws         device workspace of at least
 *              bsa_workspace_size(shape, BSA_WS_ESTIMATE, 0) bytes.
 * Ranking is by pooled logit, larger first, lower block id first on ties; the
 * kept prefix is the shortest whose fp32 cumulative probability reaches top_p.
 * Each output row is ascending. */
bsa_status bsa_estimate_mask(const bsa_shape* shape, const void* q, const void* k,
                             float top_p, float scale, const bsa_csr* candidate,
                             int32_t keep_prefix_tokens, bsa_csr* out,
                             void* ws, size_t ws_bytes, void* stream);

/* Hierarchical block scoring.  The DFSAttn page (Abstract) names hierarchical
 * block scoring for block importance without defining it; this library reads
 * it as: each key block j splits into sub_blocks sub-blocks of
 * block / sub_blocks tokens (sub-blocks past N are left out), the query block
 * mean is scored against each sub-block mean, scale * <Qbar_i, Kbar_{j,m}>,
 * and block j's logit is the natural log-sum-exp over its sub-blocks.  A
 * block's softmax probability is then the sum of its sub-blocks'
 * probabilities, so one strongly matched sub-block (a vertical stripe, a
 * small object) is not averaged away.  Softmax, Top-p, ranking, candidates,
 * forced blocks and the output are those of bsa_estimate_mask.
 *   sub_blocks 1, 2, 4 or 8 (1: the logits of bsa_estimate_mask).
 *   ws         at least bsa_workspace_size(shape, BSA_WS_ESTIMATE_HIER, 0)
 *              bytes (sized for 8 sub-blocks).
 * Errors: BSA_ERR_INVALID_ARG for any other sub_blocks, otherwise as
 * bsa_estimate_mask. */
bsa_status bsa_estimate_mask_hierarchical(const bsa_shape* shape, const void* q, const void* k,
                                          float top_p, float scale, const bsa_csr* candidate,
                                          int32_t keep_prefix_tokens, int32_t sub_blocks,
                                          bsa_csr* out, void* ws, size_t ws_bytes, void* stream);

/* Mask narrowing from exact block attention weights.  The GSRS page
 * (Abstract) obtains exact attention weights inside the attention computation
 * and restricts later search steps to the blocks of an earlier step
 * (Abstract; Figure 4 caption); its Figure 3 caption describes the
 * block-level attention map those weights form.  This call applies the
 * estimator's Top-p rule to such weights: row r of `mask` is ranked by the
 * block masses aligned with it (larger first, lower block id first on equal
 * masses) and keeps the shortest prefix whose share of the row's total mass
 * reaches top_p; forced blocks (keep_prefix_tokens, as in bsa_estimate_mask)
 * join after the cut.
 *   mask       CSR over the R rows, e.g. the one a forward ran on.
 *   block_mass [mask->capacity] fp32 device array aligned with mask->col_idx,
 *              e.g. bsa_forward's block_mass.  A negative or NaN mass counts
 *              as 0; a row whose masses sum to 0 keeps every entry; a block
 *              listed twice in a row counts once, with the mass of its first
 *              listing; ids outside [0, nb) are ignored.  Every entry of a
 *              row is read (up to 2^31 - 1 per row), in any order.
 *   top_p      in (0, 1]; 1 keeps every entry.
 *   out        CSR written by the call (a subset of mask plus forced blocks),
 *              rows ascending; exact row_ptr offsets, entries past
 *              out->capacity dropped, as in bsa_estimate_mask.  Must not alias
 *              mask.
 *   ws         at least bsa_workspace_size(shape, BSA_WS_SELECT_FROM_MASS, 0) bytes. */
bsa_status bsa_select_from_mass(const bsa_shape* shape, const bsa_csr* mask, const float* block_mass,
                                float top_p, int32_t keep_prefix_tokens, bsa_csr* out,
                                void* ws, size_t ws_bytes, void* stream);

/* bsa_select_from_mass without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, result and errors as
 * bsa_select_from_mass, except that the kernels' scratch (R row counts and
 * an R x ceil(nb/32) word bitmask, 4 bytes each) lives in a 16 MiB array
 * that the library holds on each GPU until the process ends; a shape that
 * needs more returns BSA_ERR_WORKSPACE.  Every call on one GPU shares that
 * array, so calls that overlap on one GPU (e.g. on two streams) race; calls
 * in one stream are safe.  The array used is that of the stream's device
 * (the current device for the NULL stream); the first call on a device
 * looks its address up, making that device current for the lookup and
 * restoring the caller's current device (a HIP failure there returns
 * BSA_ERR_HIP).  Allocates nothing. */
bsa_status bsa_select_from_mass_noalloc(const bsa_shape* shape, const bsa_csr* mask, const float* block_mass,
                                        float top_p, int32_t keep_prefix_tokens, bsa_csr* out, void* stream);

/* Structured (static) head patterns.  The SVG page (Abstract) sorts heads
 * into spatial heads, where tokens of the same frame dominate, and temporal
 * heads, where tokens at the same position in other frames dominate; the
 * Sparse-vDiT page (Abstract) finds diagonal, multi-diagonal and
 * vertical-stripe patterns.  Token geometry: tokens [0, prefix_tokens) are
 * text; video token n >= prefix_tokens is in frame (n - prefix)/frame_tokens
 * at spatial index (n - prefix) % frame_tokens.
 *   SPATIAL        a video query token relates to the video keys of its frame;
 *   TEMPORAL       ... to the video keys at its spatial index, in every frame;
 *   DIAGONAL       query block i relates to key block j when |i - j| <= band;
 *   MULTI_DIAGONAL ... when |i - j - k*period| <= band for some integer k;
 *   STRIPES        ... when j is one of `stripes` or |i - j| <= band;
 *   DENSE          every pair.
 * In every pattern pairs with a text token are related, and a block pair is
 * kept when any of its token pairs is related. */
typedef enum {
  BSA_PATTERN_DENSE = 0,
  BSA_PATTERN_SPATIAL = 1,
  BSA_PATTERN_TEMPORAL = 2,
  BSA_PATTERN_DIAGONAL = 3,
  BSA_PATTERN_MULTI_DIAGONAL = 4,
  BSA_PATTERN_STRIPES = 5
} bsa_pattern;

typedef struct {
  int32_t prefix_tokens;   /* text tokens at the start, in [0, N] */
  int32_t frame_tokens;    /* video tokens per frame, >= 1 */
  int32_t band;            /* half-width of the diagonal bands in blocks, >= 0 */
  int32_t period;          /* spacing of the multi-diagonal bands in blocks, >= 1 */
  const int32_t* stripes;  /* device array of key-block ids (ids outside [0, nb) ignored), or NULL */
  int32_t n_stripes;       /* entries of stripes, >= 0 */
} bsa_pattern_params;

/* Builds the CSR mask of structured head patterns.
 *   head_kind  [B*H] int32 device array, one bsa_pattern per head (b, h);
 *              an unknown value gives that head dense rows.
 *   params     pattern parameters shared by all heads (host struct).
 *   out        CSR written by the call, rows ascending, exact row_ptr
 *              offsets and entries past out->capacity dropped, as in
 *              bsa_estimate_mask (R*nb always suffices).
 *   ws         at least bsa_workspace_size(shape, BSA_WS_STRUCTURED, 0) bytes.
 * Only shape->B, H, N and block are used (D and dtype must still be valid). */
bsa_status bsa_structured_mask(const bsa_shape* shape, const int32_t* head_kind, const bsa_pattern_params* params,
                               bsa_csr* out, void* ws, size_t ws_bytes, void* stream);

/* Token permutation of [heads, n, row_bytes] slabs.  Reordering tokens along
 * a space-filling curve keeps space-time neighbours in the same block (DFSAttn
 * page, Abstract; GSRS page, Figure 1, 3 and 6 captions); the SVG page
 * (Abstract) pairs its kernels with such a layout transformation.
 *   heads      number of slabs (e.g. B*H), >= 1.
 *   n          token rows per slab (e.g. N), >= 1.
 *   row_bytes  bytes per row, a positive multiple of 4 (D * element size for
 *              q, k, v, o; 4 for lse).
 *   perm       [n] int32 device array, normally a permutation of [0, n).
 *   inverse    0: gather, dst[h, t] = src[h, perm[t]] (into the new order);
 *              1: scatter, dst[h, perm[t]] = src[h, t] (undoes the gather).
 *              An entry outside [0, n) gives a zero row in a gather and is
 *              skipped in a scatter; a perm with repeated entries leaves the
 *              scatter's result for those rows unspecified.
 *   src, dst   device arrays of heads*n*row_bytes bytes, 4-byte aligned, not
 *              overlapping; heads*n*row_bytes/4 must be below 2^31.
 * 16-byte moves are used when row_bytes and both pointers allow. */
bsa_status bsa_permute_rows(int64_t heads, int32_t n, int32_t row_bytes, const void* src, const int32_t* perm,
                            int32_t inverse, void* dst, void* stream);

/* Sparse attention forward over a block mask (see the header comment, stage 2).
 *   q, k, v    [B,H,N,D] device tensors of shape->dtype.
 *   scale      logit scale; <= 0 selects 1/sqrt(D).
 *   mask       CSR over the R rows (e.g. from bsa_estimate_mask).  Each row's
 *              entries are attended as listed.  With block 64 (bf16) rows 2m
 *              and 2m + 1 must be adjacent in col_idx (a non-decreasing
 *              row_ptr, as every CSR this library writes); a pair of rows
 *              that is not gets no entries.
 *   o          [B,H,N,D] output of shape->dtype: softmax(scale*Q_i K_S^T) V_S
 *              over the keys S of the row's selected blocks.
 *   lse        [B,H,N] fp32 output: natural log of sum over S of exp(scale*q.k).
 *              A row with no selected block gets O = 0 and lse = -inf.
 *   block_mass NULL, or [mask->capacity] fp32 output aligned with col_idx:
 *              for entry (i, j), the mean over the valid queries of block i of
 *              the softmax probability that falls on key block j (each row
 *              sums to 1).
 *   o_f32      NULL, or (BSA_BF16 only) a [B,H,N,D] fp32 output receiving O
 *              before its rounding to bf16, for bsa_backward's single-pass
 *              delta.  Must be NULL for BSA_FP32 (o is already fp32).
 *   ws         at least bsa_workspace_size(shape, BSA_WS_FORWARD, capacity) bytes. */
bsa_status bsa_forward(const bsa_shape* shape, const void* q, const void* k, const void* v,
                       float scale, const bsa_csr* mask, void* o, float* lse,
                       float* block_mass, float* o_f32, void* ws, size_t ws_bytes, void* stream);

/* Backward of the sparse forward for a loss L with dL/dO = d_o.
 *   o, lse     the forward's outputs for the same q, k, v, scale and mask
 *              (the same conditions on the mask: with block 64, bf16, rows
 *              2m and 2m + 1 adjacent in col_idx).
 *   o_f32      NULL, or (BSA_BF16 only) the forward's o_f32 output: then
 *              delta_q = dO_q . O_q is taken from it and dQ needs one pass
 *              over the row.  With NULL (or for BSA_FP32 data) delta is
 *              computed exactly as sum_k P dP in a first pass, because the
 *              rounding of a bf16 O moves it by more than the gradients can
 *              absorb.
 *   dq, dk, dv [B,H,N,D] outputs of shape->dtype (overwritten, not accumulated).
 *   ws         at least bsa_workspace_size(shape, BSA_WS_BACKWARD, capacity) bytes.
 * Deterministic: no floating-point atomics. */
bsa_status bsa_backward(const bsa_shape* shape, const void* q, const void* k, const void* v,
                        const void* o, const float* o_f32, const void* d_o, const float* lse, float scale,
                        const bsa_csr* mask, void* dq, void* dk, void* dv,
                        void* ws, size_t ws_bytes, void* stream);

/* Static description of a status code. */
const char* bsa_status_string(bsa_status status);

/* Message for the most recent failed call on the calling thread ("" if none). */
const char* bsa_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t bsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H_ */
