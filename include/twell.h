/*
 * libtwell: the ReLU-gated transformer FFN that skips exact-zero gate
 * activations through the Tile-wise ELLPACK (TwELL) format, on AMD Instinct
 * MI355X (gfx950).
 *
 * Sources, cited by page and section:
 *   intellectnews.ru article on the Sakana AI + NVIDIA TwELL work
 *   ("...twell-uskorenie-llm-do-20-procentov"), sections
 *     "Формат TwELL вместо классической sparse-упаковки"   (TwELL format),
 *     "Слитые CUDA-ядра для инференса и гибрид для обучения" (fused inference
 *        kernel, hybrid sparse/dense format for training),
 *     "Минимальные изменения в рецепте обучения"            (ReLU gate),
 *     "Ограничения и открытые вопросы"                      (gated FFN);
 *   gate.com/es post 20977915, paragraph 3 (per-tile packing inside the GPU's
 *   compute units); gate.com/id post 20978418, paragraphs 4-5 (same).
 *
 * The layer computed everywhere below, with weights stored neuron-major
 * (WgT, WuT and Wd are each [F][d] row-major, F = d_ff):
 *     g = x . WgT^T + bg        h = ReLU(g)   (exact zeros where g <= 0)
 *     u = x . WuT^T             a = h * u
 *     y = a . Wd
 *
 * Conventions shared by every call:
 *   - Every pointer argument is a DEVICE pointer, except the twell_mat and
 *     twell_ffn_shape structs themselves, which live in host memory (their
 *     array members are device pointers).
 *   - Every call is asynchronous on the caller's HIP stream.  No call
 *     synchronises the device, allocates or frees memory; the caller owns
 *     every buffer, including the workspace.
 *   - Outputs are overwritten, never accumulated into.
 *   - Arguments are checked on the host before anything is launched: a NULL
 *     pointer or an inconsistent shape returns TWELL_EINVAL, a shape or layout
 *     the GPU path does not handle returns TWELL_EUNSUPPORTED, a workspace that
 *     is too small returns TWELL_EWORKSPACE, and a failed launch returns
 *     TWELL_EHIP.  twell_last_error() then gives a thread-local description.
 *   - Device arrays must be 16-byte aligned.  Dense matrices are row-major.
 *   - The GPU path needs d % 64 == 0 and F % 64 == 0 (64 <= F <= 65472); T may
 *     be any value >= 0 (ragged last tiles are handled).  T*d, F*d and T*F
 *     must each be below 2^31 (the GEMM mainloops address every 16-bit
 *     operand with 32-bit byte offsets); a larger shape returns
 *     TWELL_EUNSUPPORTED before anything is launched.
 */
#ifndef TWELL_H
#define TWELL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TWELL_OK = 0,
  TWELL_EINVAL = 1,
  TWELL_EUNSUPPORTED = 2,
  TWELL_EWORKSPACE = 3,
  TWELL_EHIP = 4
} twell_status;

typedef enum { TWELL_F32 = 0, TWELL_BF16 = 1 } twell_dtype;

/*
 * A [T x F] matrix of ReLU outputs in TwELL form (intellectnews.ru TwELL
 * article, section "Формат TwELL вместо классической sparse-упаковки"):
 * the matrix is cut into R x C tiles (R = 16 rows, C = 64 columns on the GPU;
 * NR = ceil(T/R) row tiles, NT = F/C column tiles) and inside each tile every
 * row keeps only its entries > 0, compacted in ascending column order
 * (ELLPACK per tile).
 *   cnt   uint8  [T][NT]        number of kept entries of row t in tile j
 *   width uint8  [NR][NT]       ELL width of tile (i, j): max cnt of its rows
 *   val   vdtype [NR][NT][C][R] value of slot s of row r of tile (i, j)
 *   idx   uint8  [NR][NT][C][R] its column inside the tile (0..C-1)
 *   mask  uint64 [T][NT]        optional (may be NULL): bit c set iff column
 *                               j*C + c of row t is kept; the same information
 *                               as idx, in the form the kernels consume
 * Slots s < cnt hold the row's entries; slots cnt <= s < width hold value
 * +0.0 and index 0; slots >= width are left unwritten.  Row positions past T
 * in the last row tile behave as empty rows.  The caller allocates every
 * array (twell_mat_bytes gives the sizes).
 */
typedef struct {
  int32_t T, F, R, C;
  twell_dtype vdtype;
  uint8_t *cnt;
  uint8_t *width;
  void *val;
  uint8_t *idx;
  uint64_t *mask;
} twell_mat;

/* Shape and dtypes of one FFN layer call. in_dt is the dtype of x, the three
 * weight matrices, bg and dY; out_dt the dtype of y. */
typedef struct {
  int32_t T, d, F;
  twell_dtype in_dt, out_dt;
} twell_ffn_shape;

/* Bytes of each TwELL array (parts: cnt, width, val, idx, mask) for a T x F
 * matrix with R x C tiles and value dtype vdtype; returns their sum.  parts
 * may be NULL.  Pure host arithmetic. */
size_t twell_mat_bytes(int32_t T, int32_t F, int32_t R, int32_t C, twell_dtype vdtype, size_t parts[5]);

/*
 * twell_pack: G (device, [T][ldg] row-major, dtype gdtype, the first F
 * columns used) -> out, the TwELL form of ReLU(G); entries > 0 are kept and
 * their values are bit copies of G (out->vdtype must equal gdtype).  Shape is
 * taken from out (T, F); R must be 16 and C 64.  out->mask may be NULL.
 * One pass over G in HBM (intellectnews.ru TwELL article, TwELL section).
 */
twell_status twell_pack(const void *G, twell_dtype gdtype, int64_t ldg, twell_mat *out, hipStream_t stream);

/* twell_unpack: dense H ([T][ldh], dtype in->vdtype) = the matrix in holds:
 * kept entries at their columns, +0.0 elsewhere.  A test helper. */
twell_status twell_unpack(const twell_mat *in, void *H, int64_t ldh, hipStream_t stream);

/* Workspace bytes for twell_ffn_fwd with this shape (training != 0: the
 * hybrid forward with a dense-row threshold).  0 for an invalid shape. */
size_t twell_ffn_fwd_workspace(const twell_ffn_shape *sh, int32_t training);

/*
 * twell_ffn_fwd: y = (ReLU(x.WgT^T + bg) * (x.WuT^T)) . Wd through TwELL
 * (intellectnews.ru TwELL article, section "Слитые CUDA-ядра для инференса и
 * гибрид для обучения"): the gate GEMM packs h into TwELL in its epilogue
 * (no pass over a dense h), then the up-projection and the down-projection
 * visit only the stored (token, neuron) pairs.
 *   x    [T][d]   in_dt
 *   WgT, WuT, Wd  [F][d] in_dt
 *   bg   [F]      in_dt, may be NULL (no bias)
 *   y    [T][d]   out_dt
 *   saved_h       NULL, or a caller-allocated twell_mat (vdtype TWELL_F32,
 *                 R=16, C=64, T and F of the shape, mask required) that
 *                 receives h for the backward pass
 *   dense_row_threshold   < 0: every row takes the sparse path (inference).
 *                 >= 0: hybrid forward; rows whose nnz exceeds it take the
 *                 dense branch, gathered-row MFMA GEMMs (requires saved_h)
 *   ws, ws_bytes  workspace of at least twell_ffn_fwd_workspace(sh, thr >= 0)
 * Stored pairs are exactly the (t, n) with g > 0 in fp32; accumulation is
 * fp32.  bf16 inputs: the up- and down-projections run as MFMA GEMMs over each
 * 128-token block's union of active neurons, with a = h*u passed between them
 * in fp16 (if any |a| exceeds the fp16 range the layer is recomputed with a in
 * fp32 automatically); fp32 inputs keep h, u and a in fp32 throughout.
 */
twell_status twell_ffn_fwd(const twell_ffn_shape *sh, const void *x, const void *WgT, const void *bg,
                           const void *WuT, const void *Wd, void *y, twell_mat *saved_h,
                           int32_t dense_row_threshold, void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for twell_ffn_bwd_hybrid with this shape and threshold
 * (the sparse branch's pair index is sized by min(F, threshold) pairs per
 * row; the dense rows go in rounds of half the tokens, all of them up to
 * 1024, and the sparse branch's buffers reuse the dense branch's memory).
 * 0 for an invalid shape.  The forward's workspace is free once it returns,
 * so one buffer of the larger size serves both calls. */
size_t twell_ffn_bwd_workspace(const twell_ffn_shape *sh, int32_t dense_row_threshold);

/*
 * twell_ffn_bwd_hybrid: gradients of L = <y, dY> for the layer of
 * twell_ffn_fwd, in the hybrid sparse/dense training format
 * (intellectnews.ru TwELL article, section "Слитые CUDA-ядра для инференса и
 * гибрид для обучения": well-sparse rows are handled in the compact sparse
 * format, rows with many active values in a dense branch).
 *   x, WgT, bg, WuT, Wd   as for twell_ffn_fwd (bg may be NULL)
 *   dY       [T][d] in_dt, the gradient of the output
 *   saved_h  the TwELL of h written by twell_ffn_fwd (fp32 values, mask
 *            required); it fixes the pattern of the sparse rows
 *   dense_row_threshold   rows whose non-zero count exceeds it take the dense
 *            branch, the others the sparse branch (any value; < 0: all dense)
 *   dX       [T][d] fp32;  dWgT, dWuT, dWd  [F][d] fp32;  dbg [F] fp32 or NULL
 *            -- all overwritten
 *   n_dense_rows  NULL or one device int32 that receives the number of rows
 *            taken by the dense branch
 *   ws, ws_bytes  workspace of at least twell_ffn_bwd_workspace(sh, thr)
 * ReLU'(g) is 1 for g > 0 and 0 otherwise.  Sparse rows: per stored pair,
 * u = x_t.WuT[n], da = dY_t.Wd[n], dg = da*u, du = da*h; dX_t = sum dg*WgT[n]
 * + du*WuT[n]; dWd[n] += h*u*dY_t, dWgT[n] += dg*x_t, dWuT[n] += du*x_t,
 * summed per neuron over its tokens in ascending order (deterministic).
 * Dense rows: the same gradient from gathered-row GEMMs.  fp32 accumulation
 * throughout; needs 3*T*F < 2^32 (TWELL_EUNSUPPORTED otherwise).
 */
twell_status twell_ffn_bwd_hybrid(const twell_ffn_shape *sh, const void *x, const void *WgT, const void *bg,
                                  const void *WuT, const void *Wd, const void *dY, const twell_mat *saved_h,
                                  int32_t dense_row_threshold, float *dX, float *dWgT, float *dWuT, float *dWd,
                                  float *dbg, int32_t *n_dense_rows, void *ws, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * twell_ffn_bwd_hybrid_l1: twell_ffn_bwd_hybrid for the loss with the
 * activation penalty of the training recipe (intellectnews.ru TwELL article,
 * section "Минимальные изменения в рецепте обучения": a small L1 term on the
 * FFN activations, weight about 2e-5):
 *   L = <y, dY> + lambda * sum_{t,n} h[t,n]          (l1_per_token_mean = 0)
 *   L = <y, dY> + lambda / T * sum_{t,n} h[t,n]      (l1_per_token_mean = 1)
 * The pages do not fix the normalisation; both are offered.  h >= 0, so the
 * term adds c * 1[g > 0] to dG (c = lambda or lambda / T) on both branches,
 * and through dG to dX, dWgT and dbg; dWuT and dWd are unchanged.
 * lambda = 0 gives exactly twell_ffn_bwd_hybrid.  Other arguments, outputs
 * and errors as for twell_ffn_bwd_hybrid; EINVAL also for a negative or
 * non-finite lambda or a mean flag other than 0 or 1.
 */
twell_status twell_ffn_bwd_hybrid_l1(const twell_ffn_shape *sh, const void *x, const void *WgT, const void *bg,
                                     const void *WuT, const void *Wd, const void *dY, const twell_mat *saved_h,
                                     int32_t dense_row_threshold, float l1_lambda, int32_t l1_per_token_mean,
                                     float *dX, float *dWgT, float *dWuT, float *dWd, float *dbg,
                                     int32_t *n_dense_rows, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Compact TwELL for the saved state of training (intellectnews.ru TwELL
 * article, section "Слитые CUDA-ядра для инференса и гибрид для обучения":
 * well-sparse rows in a compact sparse matrix, the others in a dense branch;
 * gate.com ES / ID, first paragraph: lower peak memory).  The same tiles as
 * twell_mat (R = 16, C = 64, fp32 values) with room for only W slots per
 * tile, so that tile (i, j) starts at (i*NT + j)*W*16 with no offset table:
 *   cnt   uint8  [T][NT]        true number of entries of row t in tile j
 *   width uint8  [NR][NT]       min(ELL width of the tile, W)
 *   val   float  [NR][NT][W][R] slots 0..W-1 of the capacity-64 layout
 *   idx   uint8  [NR][NT][W][R]
 *   mask  uint64 [T][NT]        as in twell_mat (required)
 *   ovf   uint8  [T]            1 iff some tile of row t holds more than W
 *                               entries: the row's stored slots are then
 *                               incomplete and its backward takes the dense
 *                               branch, which recomputes h from x
 * A row with ovf = 0 keeps every entry, bit for bit.  1 <= W <= 64; W = 64
 * is the full form.  The caller allocates every array (twell_cmat_bytes).
 */
typedef struct {
  int32_t T, F, W;
  uint8_t *cnt;
  uint8_t *width;
  float *val;
  uint8_t *idx;
  uint64_t *mask;
  uint8_t *ovf;
} twell_cmat;

/* Bytes of each compact array (parts: cnt, width, val, idx, mask, ovf) for a
 * T x F matrix of capacity W; returns their sum, 0 for an invalid shape.
 * parts may be NULL.  Pure host arithmetic. */
size_t twell_cmat_bytes(int32_t T, int32_t F, int32_t W, size_t parts[6]);

/*
 * twell_compact: full (fp32 values, mask required, same T and F) -> out.
 *   Writes every array of out (val and idx slots >= out->width excepted).
 * twell_expand: in -> full, the capacity-64 form: cnt, width and mask copied,
 *   the W stored slots of each tile moved to their capacity-64 positions,
 *   slots >= width unwritten.  For a row with ovf = 1, cnt stays the true
 *   count while only W slots of a tile survive.
 * Both are one pass over the stored arrays; EINVAL for NULL arrays, shape
 * mismatch, W outside 1..64 or misaligned (16 bytes) val / mask.
 */
twell_status twell_compact(const twell_mat *full, twell_cmat *out, hipStream_t stream);
twell_status twell_expand(const twell_cmat *in, twell_mat *full, hipStream_t stream);

/* Workspace bytes for twell_ffn_bwd_hybrid_compact with a saved state of
 * capacity W: that of twell_ffn_bwd_workspace with its per-pair value arrays
 * at W slots per tile instead of 64.  0 for an invalid shape or W. */
size_t twell_ffn_bwd_compact_workspace(const twell_ffn_shape *sh, int32_t dense_row_threshold, int32_t W);

/*
 * twell_ffn_bwd_hybrid_compact: twell_ffn_bwd_hybrid_l1 with the saved state
 * in compact form (saved: T x F, written by twell_ffn_fwd_compact or by
 * twell_compact of a forward's saved_h), read in place.  Row t takes the
 * dense branch when its count exceeds dense_row_threshold or when
 * saved->ovf[t] is set; every other row keeps all its entries and takes the
 * sparse branch as before, so the gradients equal those of
 * twell_ffn_bwd_hybrid_l1 up to fp32 rounding.  n_dense_rows counts both
 * kinds.  ws: at least twell_ffn_bwd_compact_workspace(sh, thr, saved->W)
 * bytes.  Other arguments, outputs and errors as for twell_ffn_bwd_hybrid_l1.
 */
twell_status twell_ffn_bwd_hybrid_compact(const twell_ffn_shape *sh, const void *x, const void *WgT,
                                          const void *bg, const void *WuT, const void *Wd, const void *dY,
                                          const twell_cmat *saved, int32_t dense_row_threshold, float l1_lambda,
                                          int32_t l1_per_token_mean, float *dX, float *dWgT, float *dWuT,
                                          float *dWd, float *dbg, int32_t *n_dense_rows, void *ws,
                                          size_t ws_bytes, hipStream_t stream);

/*
 * twell_ffn_fwd_compact: the hybrid training forward (twell_ffn_fwd with
 * dense_row_threshold >= 0) that saves h straight into compact form: the
 * gate GEMM's epilogue packs every tile into the W slots of saved (keeping
 * the first W entries of each row and the true counts and masks), then each
 * row with more than W entries in some tile is flagged (saved->ovf) and
 * joins the dense branch with the rows above the threshold; tile widths are
 * clamped to W.  No capacity-64 form is ever held.  y is the same layer as
 * twell_ffn_fwd's (the dense branch computes the same function), and saved
 * equals twell_compact of twell_ffn_fwd's saved_h.
 *   saved  caller-allocated twell_cmat (T and F of the shape; any W in 1..64)
 *   dense_row_threshold  >= 0 (EINVAL otherwise)
 *   ws, ws_bytes  at least twell_ffn_fwd_compact_workspace(sh, saved->W)
 * Other arguments and errors as for twell_ffn_fwd.
 */
size_t twell_ffn_fwd_compact_workspace(const twell_ffn_shape *sh, int32_t W);
twell_status twell_ffn_fwd_compact(const twell_ffn_shape *sh, const void *x, const void *WgT, const void *bg,
                                   const void *WuT, const void *Wd, void *y, twell_cmat *saved,
                                   int32_t dense_row_threshold, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * twell_ffn_fwd_ex: twell_ffn_fwd that also records up to n_events caller-
 * created HIP events on the stream at its stage boundaries, for timing:
 *   [0] start
 *   [1] gate GEMM + TwELL pack done (and the row classification, training)
 *   [2] row-block neuron unions and the fp16 copy of Wd done (bf16 inputs;
 *       for fp32 inputs recorded right after [1])
 *   [3] up-projection done   [4] down-projection done
 *   [5] sparse phases done (for bf16 inputs right after [4]: the fp16-
 *       overflow fallback runs inside the down-projection kernel)
 *   [6] end (after the dense-row forward, training)
 * Arguments otherwise as for twell_ffn_fwd; events past n_events are not
 * recorded.
 */
twell_status twell_ffn_fwd_ex(const twell_ffn_shape *sh, const void *x, const void *WgT, const void *bg,
                              const void *WuT, const void *Wd, void *y, twell_mat *saved_h,
                              int32_t dense_row_threshold, void *ws, size_t ws_bytes, hipStream_t stream,
                              hipEvent_t *stage_events, int32_t n_events);

/*
 * Capacity-bounded inference forward (intellectnews.ru TwELL article, section
 * "Слитые CUDA-ядра для инференса и гибрид для обучения": intermediates are
 * not written to global memory beyond need; gate.com ES / ID, first
 * paragraph: lower peak memory).  The same layer and the same kernels as
 * twell_ffn_fwd for bf16 inputs, with the two per-call buffers that grow with
 * T x F sized by capacities the caller picks instead of for the worst case:
 *   tile_cap   slots per 16 x 64 TwELL tile of h (a multiple of 4, 4..64; the
 *              full form has 64): h takes 5 * tile_cap / 64 bytes per (t, n)
 *              instead of 5
 *   union_cap  union positions per 128-token block that the fp16 buffer of
 *              a = h * u holds (a multiple of 64, 64..F): 2 * union_cap bytes
 *              per token instead of 2 * F
 * A 128-token block with a tile wider than tile_cap whose union fits takes
 * h from a gate GEMM over its union instead of its incomplete TwELL (about
 * one more GEMM over the union for that block); a block with more than
 * union_cap neurons active in its tokens is computed per stored pair in fp32
 * inside the down-projection, with h recomputed from x, WgT and bg for its
 * pairs (the mask keeps every pair).  Both are exact for any input; the
 * second is slow.  The caller picks the capacities from its activation
 * statistics (e.g. the largest per-tile count and block union seen in
 * calibration).
 *   n_over_blocks  NULL, or a device int32 that receives the number of
 *                  128-token blocks over either capacity (0: every block fit)
 *   Other arguments as for twell_ffn_fwd with saved_h NULL and
 *   dense_row_threshold < 0.  bf16 inputs only (EUNSUPPORTED otherwise);
 *   EINVAL for capacities outside the ranges above.  For T <= 256 the call is
 *   twell_ffn_fwd's few-token path, whose workspace is small already.
 *   ws, ws_bytes  at least twell_ffn_fwd_bounded_workspace(sh, tile_cap,
 *   union_cap) bytes (0 for an invalid shape or capacities).
 */
size_t twell_ffn_fwd_bounded_workspace(const twell_ffn_shape *sh, int32_t tile_cap, int32_t union_cap);
twell_status twell_ffn_fwd_bounded(const twell_ffn_shape *sh, const void *x, const void *WgT, const void *bg,
                                   const void *WuT, const void *Wd, void *y, int32_t tile_cap, int32_t union_cap,
                                   int32_t *n_over_blocks, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The three stages of the forward, callable one by one: the same layer as
 * twell_ffn_fwd, computed by the per-pair kernels that twell_ffn_fwd keeps
 * for fp32 inputs.  For bf16 inputs
 * twell_ffn_fwd itself runs other kernels (the union GEMMs with a in fp16, or
 * the few-token kernels), so its bits differ from this sequence's; both meet
 * the same tolerance against the definition.
 *
 * twell_gate_pack: gate GEMM g = x.WgT^T + bg with ReLU and the TwELL pack in
 *   its epilogue (intellectnews.ru TwELL article, TwELL section: the format is
 *   assembled at the end of the kernel that produces it).  h must be T x F,
 *   vdtype TWELL_F32, R=16, C=64, mask required; every array of h is written
 *   (slots >= width excepted).  sh->out_dt is ignored.
 */
twell_status twell_gate_pack(const twell_ffn_shape *sh, const void *x, const void *WgT, const void *bg,
                             twell_mat *h, hipStream_t stream);

/*
 * twell_sparse_up: a[t,n] = h[t,n] * (x_t . WuT[n]) for every (t, n) stored
 *   in h, fp32, written at the same slot positions as h->val into aval
 *   ([NR][NT][64][16] floats; aval may be h->val itself, which is then
 *   overwritten).  Slots that hold no stored pair are not written.
 */
twell_status twell_sparse_up(const twell_ffn_shape *sh, const void *x, const void *WuT, const twell_mat *h,
                             float *aval, hipStream_t stream);

/*
 * twell_sparse_down: y_t = sum over the pairs (t, n) stored in pattern of
 *   a[t,n] * Wd[n] (a read from aval at pattern's slot positions), for every
 *   row t; y is [T][d] in sh->out_dt.  fp32 accumulation; a enters the bf16
 *   matrix cores as a hi + lo pair of bf16 values.
 */
twell_status twell_sparse_down(const twell_ffn_shape *sh, const float *aval, const void *Wd,
                               const twell_mat *pattern, void *y, hipStream_t stream);

/* Workspace bytes for twell_ffn_dense_fwd. */
size_t twell_ffn_dense_fwd_workspace(const twell_ffn_shape *sh);

/*
 * twell_ffn_dense_fwd: the same layer computed densely (the library's own
 * dense MFMA baseline, bf16 only): a fused gate/up GEMM writes
 * act = bf16(ReLU(g) * u) for every (t, n), then y = act . Wd.  For
 * 0 < T <= 256 every GEMM is split along K over many workgroups, with the
 * same blocks as the few-token TwELL forward's gate (partial sums added in
 * a fixed order).
 * Arguments as for twell_ffn_fwd.
 */
twell_status twell_ffn_dense_fwd(const twell_ffn_shape *sh, const void *x, const void *WgT, const void *bg,
                                 const void *WuT, const void *Wd, void *y, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/* Workspace bytes for twell_relu_ffn_fwd (0 for an invalid shape). */
size_t twell_relu_ffn_fwd_workspace(const twell_ffn_shape *sh);

/*
 * twell_relu_ffn_fwd: the non-gated ReLU FFN y = ReLU(x.W1T^T + b1) . W2
 * through TwELL.  The pages' method targets gated FFNs (intellectnews.ru
 * TwELL article, section "Ограничения и открытые вопросы"); a plain ReLU FFN
 * has the same exact zeros in its hidden layer but no up-projection to skip.
 * The gate GEMM packs h = ReLU(x.W1T^T + b1) into TwELL in its epilogue (as
 * in twell_ffn_fwd), then the down-projection visits only the stored pairs:
 * for bf16 inputs an fp16 MFMA GEMM over each 128-token block's union of
 * active neurons with h in fp16 (h beyond the fp16 range: recomputed per pair
 * in fp32), for fp32 inputs the per-pair kernel in fp32.
 *   x    [T][d] in_dt;  W1T, W2 [F][d] in_dt (neuron-major);  b1 [F] or NULL
 *   y    [T][d] out_dt (overwritten)
 *   saved_h  NULL or a caller-allocated twell_mat (fp32 values, mask
 *            required) that receives h
 *   ws, ws_bytes  workspace of at least twell_relu_ffn_fwd_workspace(sh)
 * Errors as for twell_ffn_fwd.
 */
twell_status twell_relu_ffn_fwd(const twell_ffn_shape *sh, const void *x, const void *W1T, const void *b1,
                                const void *W2, void *y, twell_mat *saved_h, void *ws, size_t ws_bytes,
                                hipStream_t stream);

/*
 * twell_relu_ffn_fwd_bounded: the non-gated layer of twell_relu_ffn_fwd with
 * the capacities of twell_ffn_fwd_bounded (gate.com ES / ID, first paragraph:
 * lower peak memory): h in a TwELL of tile_cap slots per tile, a = h over at
 * most union_cap union positions per 128-token block.  A block with a tile
 * wider than tile_cap whose union fits takes h from a GEMM of x with its
 * union's W1T rows; a block with a longer union is computed per stored pair
 * in fp32 with h recomputed.  Exact for any input.  bf16 inputs only;
 * capacities, n_over_blocks and errors as for twell_ffn_fwd_bounded, other
 * arguments as for twell_relu_ffn_fwd (no saved_h).  ws: at least
 * twell_relu_ffn_fwd_bounded_workspace(sh, tile_cap, union_cap) bytes.
 */
size_t twell_relu_ffn_fwd_bounded_workspace(const twell_ffn_shape *sh, int32_t tile_cap, int32_t union_cap);
twell_status twell_relu_ffn_fwd_bounded(const twell_ffn_shape *sh, const void *x, const void *W1T, const void *b1,
                                        const void *W2, void *y, int32_t tile_cap, int32_t union_cap,
                                        int32_t *n_over_blocks, void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for twell_relu_ffn_dense_fwd. */
size_t twell_relu_ffn_dense_fwd_workspace(const twell_ffn_shape *sh);

/*
 * twell_relu_ffn_dense_fwd: the same non-gated layer computed densely (the
 * library's own dense MFMA baseline for it, bf16 only): a GEMM writes
 * act = bf16(ReLU(x.W1T^T + b1)) for every (t, n), then y = act . W2.
 * EUNSUPPORTED unless F % 128 == 0.  Other arguments as twell_relu_ffn_fwd.
 */
twell_status twell_relu_ffn_dense_fwd(const twell_ffn_shape *sh, const void *x, const void *W1T, const void *b1,
                                      const void *W2, void *y, void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for twell_ffn_dense_bwd. */
size_t twell_ffn_dense_bwd_workspace(const twell_ffn_shape *sh);

/*
 * twell_ffn_dense_bwd: the library's own dense training step of the same
 * layer, the denominator for the hybrid training path ([IN] "Слитые
 * CUDA-ядра для инференса и гибрид для обучения" describes the hybrid; this
 * is its plain dense counterpart).  Runs the dense forward, keeping
 * h = ReLU(g), u and a = h*u as bf16 [T][F] in the workspace, writes y, then
 * the backward: dA = dY.Wd^T, dG = dA*u*[g > 0], dU = dA*h (bf16),
 * dX = dG.WgT + dU.WuT, dWgT = dG^T.x, dWuT = dU^T.x, dWd = a^T.dY,
 * dbg = column sums of dG.  bf16 inputs only; fp32 accumulation; the bf16
 * intermediates make it the fastest dense variant, not an fp32-accurate one.
 *   x, dY     [T][d] bf16;  WgT, WuT, Wd [F][d] bf16;  bg [F] bf16 or NULL
 *   y         [T][d] in sh->out_dt (overwritten)
 *   dX        [T][d] fp32;  dWgT, dWuT, dWd [F][d] fp32;  dbg [F] fp32 or NULL
 *             (all overwritten; with T == 0 the weight gradients are zeros)
 *   ws        twell_ffn_dense_bwd_workspace(sh) bytes
 * Errors: EINVAL for NULL or misaligned arguments, EUNSUPPORTED unless
 * T % 64 == 0, d % 256 == 0 and F % 256 == 0 (or for fp32 inputs),
 * EWORKSPACE, EHIP.
 */
twell_status twell_ffn_dense_bwd(const twell_ffn_shape *sh, const void *x, const void *WgT, const void *bg,
                                 const void *WuT, const void *Wd, const void *dY, void *y, float *dX, float *dWgT,
                                 float *dWuT, float *dWd, float *dbg, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/*
 * twell_ffn_fwd_noalloc: twell_ffn_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a static device array inside the
 * library, TWELL_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held by each GPU the
 * call runs on until the process ends; its device address is looked up on the
 * first call on a device.  The call allocates and frees nothing.
 *   Arguments as for twell_ffn_fwd, without ws and ws_bytes; the output and
 *   numerics are those of twell_ffn_fwd with the same arguments.
 *   TWELL_EWORKSPACE (nothing launched) when the shape needs more than the
 *   scratch holds, i.e. when twell_ffn_fwd_workspace(sh, thr >= 0) would ask
 *   for more than TWELL_NOALLOC_SCRATCH_BYTES: decode-shaped and small
 *   batches fit (e.g. T = 64 tokens at d = 2304, F = 9216).
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind; nothing in it needs to start at zero.  Calls that overlap on one GPU
 * (two streams, or two host threads) race on it: the caller serialises them.
 */
#define TWELL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
twell_status twell_ffn_fwd_noalloc(const twell_ffn_shape *sh, const void *x, const void *WgT, const void *bg,
                                   const void *WuT, const void *Wd, void *y, twell_mat *saved_h,
                                   int32_t dense_row_threshold, hipStream_t stream);

/* Static description of a status code. */
const char *twell_status_string(twell_status st);
/* Thread-local description of the last error returned on this thread. */
const char *twell_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TWELL_H */
