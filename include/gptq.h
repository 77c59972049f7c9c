/*
 * gptq.h -- C ABI of the MI355X (gfx950) GPTQ layer-quantization library
 * (libgptq_mi355x.so).
 *
 * One linear layer W (rows x cols, out x in) and its calibration inputs X
 * (cols features x n tokens) go through four calls, in the order the method
 * is stated on the pages:
 *
 *   1. gptq_hessian_accumulate -- collect the layer's inputs into H = 2 X X^T
 *      ("GPTQ implementation with tensor subclasses", section Background:
 *      track the activations reaching the linear; "GPTQ", section Komponenty:
 *      the Hessian of the layer inputs).
 *   2. gptq_prepare_hinv -- damping, activation order and the Cholesky factor
 *      of the inverse Hessian ("GPTQ", sections Komponenty and
 *      Hiperparametry).
 *   3. gptq_quantize_layer -- column-by-column quantization with Optimal
 *      Brain Surgeon error compensation and block updates, producing the
 *      codes and the updated (dequantized) weight the layer goes on with
 *      ("GPTQ", section Jak dziala; "GPTQ implementation with tensor
 *      subclasses", section Background: use the updated weight).
 *   4. gptq_pack -- b-bit codes to a bit stream ("GPTQ", section
 *      Zlozonosc obliczeniowa: about 4.x bits per weight as stored).
 *
 * The stored 4-bit layer then runs as y = x W^T through gptq_w4a16_prepare
 * and gptq_w4a16_gemm (at the end of this header).
 *
 * Conventions shared by every call:
 *  - Every pointer except `params` and the profiling outputs is a DEVICE
 *    pointer on the current HIP device, owned by the caller.  Buffers must
 *    not overlap unless stated.  Matrices are row-major and contiguous
 *    unless a leading dimension is given.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = legacy default
 *    stream) and is asynchronous, except where stated.  The library keeps no
 *    device state between calls; calls on different streams, from one or
 *    several host threads, may run concurrently as long as their buffers are
 *    distinct.  Its only host state is a lock-guarded cache of per-device
 *    attributes (kernel LDS limits, compute-unit count), the thread-local
 *    error text and the profiler (which is single-threaded).
 *  - The library never allocates device memory.  Scratch memory is the
 *    caller's `ws` buffer of `ws_bytes` bytes, sized by
 *    gptq_workspace_bytes() and 256-byte aligned.
 *  - Errors are returned as gptq_status, never thrown.  All argument checks
 *    run on the host before any launch; on GPTQ_ERR_INVALID_ARG or
 *    GPTQ_ERR_WORKSPACE nothing has been enqueued and no output was written.
 *    gptq_last_error() then gives a message (thread-local).  A failed launch
 *    returns GPTQ_ERR_DEVICE; outputs are then undefined.
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = 1, /* bad size, pointer, alignment or parameter      */
  GPTQ_ERR_NOT_SPD = 2,     /* damped Hessian not positive definite          */
  GPTQ_ERR_DEVICE = 3,      /* a HIP call or kernel launch failed            */
  GPTQ_ERR_WORKSPACE = 4    /* ws NULL, misaligned or smaller than required  */
} gptq_status;

typedef enum { GPTQ_DT_F32 = 0, GPTQ_DT_BF16 = 1 } gptq_dtype;

typedef enum {
  GPTQ_GRID_AFFINE = 0, /* asymmetric min-max scale + integer zero per group  */
  GPTQ_GRID_Q4K = 1     /* two-level k-quant grid: sub-block scale/min codes
                           (32 weights) under fp16 super-scale/super-min (256
                           weights); Q4_K for bits = 4                        */
} gptq_grid;

/* Factor that carries the compensation between gptq_prepare_hinv and
 * gptq_quantize_layer ("GPTQ", section Komponenty: the not yet quantized
 * weights are corrected through the Cholesky factor of the inverse Hessian).
 *
 * INVERSE: U, the upper Cholesky factor of Hp^-1 (U^T U = Hp^-1), the pages'
 *   own object; after column j the later columns take w_k -= e_j U_jk with
 *   e_j = (w_j - w^_j) / U_jj.
 * HESSIAN: the same compensation without the inverse of the whole factor.
 *   With Hp = R R^T (R upper, R = U^-1) the errors satisfy W - W^ = E U, so
 *   E = (W - W^) R, and the compensated weights of a block B of 128 columns
 *   at its turn are c_B = o_B + (o - w^)_{<B} R_{<B,B} U_BB, o being the
 *   weights before compensation and U_BB U's diagonal block (the inverse of
 *   R's, which the blocked Cholesky forms anyway).  So the updates between
 *   blocks go through M = R_{<B,B} U_BB with the error w^_j - o_j, and the
 *   pages' rule runs inside each block on U_BB.  Needs cols % 128 == 0,
 *   block = 128 and the affine grid with group dividing 128 (a group's grid
 *   is then chosen inside one block). */
typedef enum { GPTQ_ROUTE_INVERSE = 0, GPTQ_ROUTE_HESSIAN = 1 } gptq_route;

/* Hyper-parameters ("GPTQ", section Hiperparametry: target precision, weights
 * per scale, activation order, value added to the Hessian diagonal). */
typedef struct {
  int32_t bits;      /* AFFINE: 2..8; Q4K: 2..6 (the sub-block scale/min codes
                        are 4 bits wide for bits = 2, 6 for 3..5, 8 for 6:
                        "Add gguf q4_k quantization", review thread)         */
  int32_t group;     /* AFFINE: weights per scale, divides cols (cols = one
                        group per row); Q4K: must be 256                      */
  int32_t block;     /* lazy-update block B, 1..128; group % B == 0 or
                        B % group == 0                                        */
  int32_t act_order; /* 0: original column order; 1: decreasing diag(H)      */
  float percdamp;    /* damping = percdamp * mean(diag H), >= 0 (0.01 usual)   */
  int32_t grid;      /* gptq_grid                                             */
  int32_t search;    /* 0: min-max grids.  1: importance-weighted search,
                        the importance of a column being its activation
                        energy hdiag ("Add gguf q4_k quantization", review
                        thread: weighted search, activation-aware
                        importance).  AFFINE: the group's scale of least
                        weighted squared error among (1 - k/32) x the min-max
                        scale, k = 0..15, at the min-max zero point.  Q4K:
                        each sub-block's (scale, min) among (1 - k/32) x its
                        min-max pair, before the super-block level codes
                        them.                                                 */
  int32_t route;     /* gptq_route: which triangular factor carries the
                        compensation (same codes and W^ in exact arithmetic) */
} gptq_params;

/* Message of the last failing call on this thread ("" if none). */
const char *gptq_last_error(void);

/* Bytes of `ws` needed by gptq_prepare_hinv (for cols) and by
 * gptq_quantize_layer (for rows x cols) with these parameters, and wanted by
 * gptq_hessian_accumulate (for cols features); the largest of the three, so
 * one buffer serves all three calls.  Returns 0 on invalid arguments. */
size_t gptq_workspace_bytes(int64_t rows, int64_t cols, const gptq_params *p);

/*
 * H += 2 * X * X^T and hdiag += 2 * sum_t X[i,t]^2.
 *
 * ("GPTQ", section Komponenty: the Hessian of a linear layer is 2 X X^T of
 * its input activations; section Zlozonosc obliczeniowa: the cost grows with
 * calibration tokens times d^2, so X arrives in token chunks and the sums
 * are accumulated across calls.)
 *
 *  H      d x d float, row-major.  Only the upper triangle including the
 *         diagonal (j >= i) is read and written; the strict lower triangle is
 *         never touched.  Zero it before the first chunk.
 *  hdiag  d doubles: the activation energy of each feature, accumulated in
 *         float64 (the column order under act-order is decided on it).  Zero
 *         it before the first chunk.
 *  X      d rows (features) x n_tok tokens, row stride ld_x elements
 *         (ld_x >= n_tok), dtype x_dtype (BF16 = raw bfloat16 bits, or
 *         F32).  16-byte aligned, and ld_x a multiple of 8 (BF16) or 4 (F32).
 *  n_tok  tokens in this chunk (0 is a no-op).
 *  ws     optional scratch (NULL with ws_bytes 0, or 256-byte aligned): with
 *         room for it, the bf16 path splits the tiles of its last, partly
 *         filled round of workgroups into token parts whose sums are added
 *         into H in a fixed order, so that the round fills the GPU.  More
 *         room allows finer parts, up to what gptq_workspace_bytes asks for
 *         and beyond; none at all gives one workgroup per tile.
 *
 * Products of bf16 inputs are exact in float32; sums are float32 in H.  For
 * given sizes, compute-unit count and ws_bytes the result is the same bits
 * on every call.
 */
gptq_status gptq_hessian_accumulate(float *H, double *hdiag, int64_t d,
                                    const void *X, int32_t x_dtype,
                                    int64_t n_tok, int64_t ld_x, void *ws,
                                    size_t ws_bytes, void *stream);

/*
 * Damping, order and inverse-Hessian factor.
 *
 * ("GPTQ", section Komponenty: Cholesky decomposition of the inverse
 * Hessian; section Hiperparametry: column order by activation importance
 * and a value added to the diagonal; section Implementacja: inverting an
 * ill-conditioned Hessian is unstable.)
 *
 *  H, hdiag  as left by gptq_hessian_accumulate; read only.
 *  dead      out, d bytes: 1 where hdiag[i] == 0 (a feature that never fires;
 *            its H_ii is taken as 1 and its weights as 0).
 *  perm      out, d int32: perm[p] = original column processed at position p.
 *            act_order: decreasing hdiag, ties by lower index; else identity.
 *  U         out, d x d float, row-major, in processing order, strict lower
 *            triangle written as 0.  Hp = P (H with dead fix) P^T + percdamp *
 *            mean(diag) * I.  route INVERSE: the upper triangular factor with
 *            positive diagonal and U^T U = Hp^-1.  route HESSIAN (d % 128 ==
 *            0): U's entries inside the 128 x 128 diagonal blocks, and above
 *            each diagonal block B the product R_{<B,B} U_BB, where Hp =
 *            R R^T with R upper triangular (R = U^-1).
 *  ws        scratch, >= gptq_workspace_bytes(., d, p).
 *
 * Synchronizes `stream` once at the end to read the positive-definiteness
 * flag: GPTQ_ERR_NOT_SPD when a Cholesky pivot is <= 0 or not finite (U is
 * then undefined; the caller may retry with a larger percdamp).
 */
gptq_status gptq_prepare_hinv(const float *H, const double *hdiag, int64_t d,
                              const gptq_params *p, float *U, int32_t *perm,
                              uint8_t *dead, void *ws, size_t ws_bytes,
                              void *stream);

/*
 * Quantize W column by column in processing order with OBS compensation.
 *
 * ("GPTQ", section Jak dziala: columns in a fixed order, the not yet
 * quantized weights corrected through the inverse Hessian after each
 * column, block updates, a scale per group, 4- or 3-bit result; "Add gguf
 * q4_k quantization", summary: the two-level grid w = q * block_scale +
 * block_min with a super-block scale, by a simple min-max choice.)
 *
 *  W        in/out, rows x cols float, original column order.  On return it
 *           holds the dequantized weights W^ (what the layer uses next).
 *  U, perm, dead  from gptq_prepare_hinv with the same d and params (the
 *           same route).
 *  hdiag    the activation energy from gptq_hessian_accumulate (cols doubles,
 *           original order); read only when params->search is 1, else may be
 *           NULL.
 *  q        out, rows x cols bytes, codes in original column order.
 *  g_idx    out, cols int32: group of each original column (AFFINE:
 *           processing position / group; Q4K: processing position / 32).
 *  AFFINE (else pass NULL):
 *   scale   out, rows x (cols/group) float, groups in processing order.
 *   zero    out, rows x (cols/group) bytes, integer zero point in [0, 2^bits).
 *           w^ = scale * (q - zero).
 *  Q4K (else pass NULL):
 *   q4k_super_scale, q4k_super_min  out, rows x (cols/256) fp16 bit patterns.
 *   q4k_sub_scale, q4k_sub_min      out, rows x (cols/32) bytes in
 *                                   [0, kmax], kmax = 15, 63 or 255 for
 *                                   4-, 6- or 8-bit sub-block codes.
 *           w^ = (D * sc) * q - (Dm * mc).
 *  ws       scratch, >= gptq_workspace_bytes(rows, cols, p).
 */
gptq_status gptq_quantize_layer(float *W, int64_t rows, int64_t cols,
                                const float *U, const int32_t *perm,
                                const uint8_t *dead, const double *hdiag,
                                const gptq_params *p,
                                uint8_t *q, int32_t *g_idx, float *scale,
                                uint8_t *zero, uint16_t *q4k_super_scale,
                                uint16_t *q4k_super_min, uint8_t *q4k_sub_scale,
                                uint8_t *q4k_sub_min, void *ws, size_t ws_bytes,
                                void *stream);

/*
 * Pack b-bit codes into a bit stream per row.
 *
 * ("GPTQ", sections Jak dziala and Zlozonosc obliczeniowa: 4- or 3-bit
 * weights, about 4.x bits per weight as stored.)
 *
 *  codes   rows x cols bytes, every value < 2^bits (larger values are masked
 *          to their low `bits` bits).
 *  packed  out, rows x (cols*bits/32) uint32.  Least significant bit first:
 *          code k of a row occupies stream bits [k*bits, (k+1)*bits), and
 *          stream bit t is bit (t mod 32) of word t / 32.
 *  bits 1..8; cols*bits must be a multiple of 32 (pack zero points of a
 *  whole layer as one row of rows*groups codes when a row alone is not).
 */
gptq_status gptq_pack(const uint8_t *codes, int64_t rows, int64_t cols,
                      int32_t bits, uint32_t *packed, void *stream);

/* ------------------------------------------------- sequential calibration
 * Outputs of a quantized layer, made with its updated weight, become the next
 * layer's calibration inputs ("GPTQ implementation with tensor subclasses",
 * section Background: for each linear, track its activations, update its
 * weight, use the updated weight to generate its outputs, then go on to the
 * next linear).  Activations keep the layout gptq_hessian_accumulate reads:
 * features x tokens, bf16 bit patterns, tokens contiguous.
 */

/* Scratch bytes of gptq_linear_forward (0 on invalid sizes). */
size_t gptq_linear_forward_ws_bytes(int64_t rows, int64_t cols, int64_t n_tok);

/*
 * Y = bf16(W X): W rows x cols float (e.g. W^ as gptq_quantize_layer leaves
 * it), X cols x n_tok bf16 (row stride ld_x), Y rows x n_tok bf16 (row
 * stride ld_y).  Products and sums in float32 (bf16 inputs widen exactly),
 * one rounding to bf16 (nearest, ties to even) per output.  ws >=
 * gptq_linear_forward_ws_bytes, 256-byte aligned.  n_tok = 0 is a no-op.
 */
gptq_status gptq_linear_forward(const float *W, int64_t rows, int64_t cols,
                                const uint16_t *X, int64_t n_tok, int64_t ld_x,
                                uint16_t *Y, int64_t ld_y, void *ws,
                                size_t ws_bytes, void *stream);

/*
 * A = bf16(silu(G) * U) elementwise, silu(g) = g / (1 + e^-g), in float32:
 * the gated activation between a gated MLP's gate/up linears and its down
 * linear.  G, U rows x n_tok bf16 with row stride ld; A with row stride ld_a.
 */
gptq_status gptq_silu_mul(const uint16_t *G, const uint16_t *U, int64_t rows,
                          int64_t n_tok, int64_t ld, uint16_t *A, int64_t ld_a,
                          void *stream);

/* ------------------------------------------------------------------ W4A16
 * Running the stored layer: y = x W^T, with W^ rebuilt from 4-bit codes,
 * per-group scale and zero inside the product kernel, activations in fp16
 * ("Hugging Face AutoGPTQ and Transformers Integration", section Mixed
 * Precision Scheme: int4 weights, fp16 activations, dequantization on the
 * fly in a fused kernel; "GPTQ", section Waskie gardla: in inference the
 * cost is reading memory).
 *
 * The stored layer is what gptq_quantize_layer (affine grid, bits = 4) and
 * gptq_pack produce.  gptq_w4a16_prepare turns it once into the product
 * kernel's layout; gptq_w4a16_gemm then runs any number of products.
 */

/* Host-side description of a prepared layer, filled by gptq_w4a16_prepare.
 * The caller owns the struct and `mem`; treat the fields as read-only. */
typedef struct {
  int64_t rows;      /* out features                                         */
  int64_t cols;      /* in features                                          */
  int32_t group;     /* columns per group                                    */
  int32_t permuted;  /* 1 when g_idx is not column / group (activation
                        order): each product then first gathers x into
                        group order in the workspace                        */
  int64_t rows_pad;  /* rows rounded up to 16                                */
  int64_t k_pad;     /* cols rounded up to 128                               */
  void *mem;         /* device buffer given to gptq_w4a16_prepare            */
  size_t mem_bytes;
} gptq_w4a16_layer;

/* Bytes of device memory a prepared layer needs (0 on invalid sizes). */
size_t gptq_w4a16_layer_bytes(int64_t rows, int64_t cols, int32_t group);

/*
 * Prepare a 4-bit affine layer for gptq_w4a16_gemm.  SYNCHRONOUS: it waits
 * for `stream`, because it validates g_idx on the device and reads the
 * verdict back.
 *
 *  packed       rows x (cols/8) uint32: the codes as gptq_pack(bits = 4)
 *               lays them out (original column order, LSB first).
 *  g_idx        cols int32: group of each original column, in [0, cols/group);
 *               every group must hold exactly `group` columns.
 *  scale        rows x (cols/group) float, indexed by group.
 *  zero_packed  the rows x (cols/group) zero points in [0, 16) as one 4-bit
 *               LSB-first stream in row-major order (gptq_pack of the zero
 *               matrix, as one row when a row alone is not 32-bit aligned);
 *               ceil(rows*(cols/group)/8) uint32.
 *  group        32, 64, or a multiple of 128; cols a multiple of group.
 *  mem          device buffer, 256-byte aligned, >= gptq_w4a16_layer_bytes;
 *               read-only for the products, which may run concurrently.
 *  layer        out, host struct describing the prepared layer.
 * The weight each product uses is w^[r][c] = scale[r][g] * (q[r][c] - z[r][g])
 * with g = g_idx[c].  Returns GPTQ_ERR_INVALID_ARG when g_idx is out of range
 * or a group's size differs from `group` (then `layer` is not filled).
 */
gptq_status gptq_w4a16_prepare(const uint32_t *packed, const int32_t *g_idx,
                               const float *scale, const uint32_t *zero_packed,
                               int64_t rows, int64_t cols, int32_t group,
                               void *mem, size_t mem_bytes,
                               gptq_w4a16_layer *layer, void *stream);

/* Scratch bytes gptq_w4a16_gemm needs for `batch` rows of x. */
size_t gptq_w4a16_workspace_bytes(const gptq_w4a16_layer *layer, int64_t batch);

/*
 * y = x W^T on the prepared layer.
 *
 *  x      batch x cols fp16 bit patterns, row-major, 16-byte aligned.
 *  y      out, batch x rows fp16 (round to nearest even), row-major.
 *  batch  1..4096.
 *  ws     scratch, 256-byte aligned, >= gptq_w4a16_workspace_bytes.
 * Products are formed exactly (fp16 activation times the integer q - z) and
 * summed in float32; each group's sum is scaled by its float32 scale.  The
 * summation order is fixed, so results are reproducible bit for bit.
 */
gptq_status gptq_w4a16_gemm(const gptq_w4a16_layer *layer, const uint16_t *x,
                            int64_t batch, uint16_t *y, void *ws,
                            size_t ws_bytes, void *stream);

/* Size of the static device scratch of gptq_w4a16_gemm_noalloc (per GPU). */
#define GPTQ_W4A16_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * y = x W^T exactly as gptq_w4a16_gemm computes it (same kernels, same
 * bits), for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace and calls no allocator; its scratch memory (the
 * gathered activations of an activation-ordered layer, split-K partial
 * sums) is a static device array of GPTQ_W4A16_STATIC_SCRATCH_BYTES inside
 * the library, one per GPU, held from the library's load until the process
 * ends.  Its address on a device is looked up once, on the first call on
 * that device.
 *
 * Every call on a GPU shares that GPU's array, and each call writes its
 * scratch in full before reading it (nothing in it needs to start at zero).
 * Calls whose execution overlaps on one GPU -- on different streams, or
 * from different host threads without ordering -- race on the array and
 * must not be issued; calls on one stream are ordered and safe.
 *
 * Arguments as for gptq_w4a16_gemm.  Returns GPTQ_ERR_WORKSPACE, with
 * nothing enqueued, when gptq_w4a16_workspace_bytes(layer, batch) exceeds
 * GPTQ_W4A16_STATIC_SCRATCH_BYTES (large batches on wide layers).
 */
gptq_status gptq_w4a16_gemm_noalloc(const gptq_w4a16_layer *layer, const uint16_t *x,
                                    int64_t batch, uint16_t *y, void *stream);

/*
 * Per-kernel timing with HIP events (for measurement, off by default).
 * When enabled, every kernel launch of the library is bracketed by a pair of
 * events on its stream.  gptq_profile_query synchronizes those events and
 * returns the number of launches and their summed duration for the kernel
 * `name` (e.g. "hessian_syrk_bf16"); 0 launches if unknown.  reset drops all
 * records.  Not thread-safe; use from one host thread.
 */
void gptq_profile_enable(int on);
void gptq_profile_reset(void);
gptq_status gptq_profile_query(const char *name, int64_t *launches,
                               double *total_ms);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
