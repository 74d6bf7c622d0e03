/*
 * gptq.h - C ABI of the GPTQ layer quantizer for AMD Instinct MI355X (gfx950).
 *
 * One linear layer y = W x with W of shape d_row x d_col is quantized to
 * int4 / int3 (or int8) codes with one fp16 scale and zero point per group of
 * consecutive weights of a row, guided by the Hessian of the layer-wise
 * reconstruction objective built from calibration activations X.
 *
 * Method: GPTQ paper summary page (azimuth.plus, "GPTQ: accurate post-training
 * quantization for generative pre-trained transformers"): layer-wise objective,
 * OBQ-style compensation through the inverse Hessian, one fixed column order
 * shared by all rows ("Innovation 1"), lazy batched updates in blocks of 128
 * columns ("Innovation 2"), Cholesky factor of the inverse Hessian computed once
 * with a small dampening term ("Innovation 3").  Quantizer and storage format:
 * Hugging Face Transformers "Quantization concepts" guide ("Mapping values to
 * fewer bits", "Choose granularity", "Data types - int8 and int4").
 *
 * Conventions shared by every entry point
 *  - Every pointer argument named as a matrix or buffer is a DEVICE pointer
 *    unless its comment says "host".  The caller owns every buffer; the library
 *    never allocates or frees device memory.  It keeps no state between calls:
 *    the extra HIP streams and events with which gptq_prepare_hinv and
 *    gptq_quantize_layers overlap their own phases live in a gptq_context that the
 *    caller creates, passes and destroys (NULL: everything runs on `stream`).
 *  - Matrices are row-major.  All work is enqueued asynchronously on `stream`
 *    (a hipStream_t; NULL = the default stream); no call synchronizes.
 *  - Argument errors (null pointers, bad sizes, unsupported settings, a
 *    workspace that is too small) are detected on the host before anything is
 *    enqueued and returned immediately; nothing is written then.
 *  - Conditions that only the device can see are reported through `*info`
 *    (device int32), readable after the stream is synchronized: 0 = success,
 *    k > 0 = a matrix that must be positive definite is not (see
 *    gptq_prepare_hinv), -1 = a non-finite input or a scale that is not a
 *    normal fp16 number, -2 = a bounded wait between workgroups expired (see
 *    gptq_prepare_hinv).  The call itself still returns GPTQ_OK.
 *  - Calls on one stream are ordered; concurrent calls on different streams
 *    must not share output or workspace buffers, nor a gptq_context.
 *  - Size limits (beyond them GPTQ_ERR_UNSUPPORTED): d_col at most 65536 for
 *    gptq_hessian_accumulate and 65535 for the factorization and the quantizers
 *    (gptq_obq_layer: 2048); d_row at most 65535 * 128 = 8388480 for
 *    gptq_quantize_layer, its _noalloc variant and gptq_quantize_layers, 2^31 / 64 for
 *    gptq_obq_layer; for the quantized linear d_row and d_col at most 2^31 / 64 and
 *    n_tokens at most 65535 * 64 = 4194240.  Dequantization takes any number of rows.
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
    GPTQ_ERR_INVALID_ARG = 1,   /* null pointer, negative or inconsistent size */
    GPTQ_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement */
    GPTQ_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    GPTQ_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed */
    GPTQ_ERR_NOT_PD = 5,        /* used by bindings to report info > 0 */
    GPTQ_ERR_NONFINITE = 6      /* used by bindings to report info == -1 */
} gptq_status;

typedef enum {
    GPTQ_F32 = 0,
    GPTQ_BF16 = 1,
    GPTQ_F16 = 2
} gptq_dtype;

/*
 * Execution context (host object owned by the caller): HIP streams and events, all at
 * the default priority, with which one call overlaps its own phases -- an auxiliary
 * stream for the factorization's triangular inverse, and for gptq_quantize_layers a
 * Hessian stream plus n_slots slot streams, each with its own auxiliary stream.
 * gptq_context_create makes them on the current device; gptq_context_destroy waits for
 * the work already queued on them and releases them (with that device made current for
 * the call).  A context serves one call at a time: calls that share one must not
 * overlap on the host.  Different contexts are independent, so calls from several host
 * threads, each with its own context and stream, run concurrently.
 *
 *  n_slots   1 .. GPTQ_LAYERS_MAX_SLOTS: the most slots a gptq_quantize_layers call with
 *            this context may use.
 *  ctx       host pointer that receives the context.
 * Errors: n_slots out of range or ctx NULL -> GPTQ_ERR_INVALID_ARG (nothing is made);
 * a failing HIP call -> GPTQ_ERR_HIP (what was made is released).  Destroying NULL is a
 * no-op.
 */
#define GPTQ_LAYERS_MAX_SLOTS 4
typedef struct gptq_context gptq_context;
gptq_status gptq_context_create(int32_t n_slots, gptq_context** ctx);
gptq_status gptq_context_destroy(gptq_context* ctx);

/*
 * Bound of the factorization's wait (see gptq_prepare_hinv's info = -2) in calls made
 * with this context (gptq_prepare_hinv and gptq_quantize_layers), in polls of about 128
 * clocks; a new context has 1 << 25 (about 2 s).  0 gives up before the first poll, so
 * that every factorization wider than 128 columns reports info = -2 with all its
 * kernels ending normally: a way to exercise a caller's handling of that error.
 * Errors: ctx NULL or polls < 0 -> GPTQ_ERR_INVALID_ARG.
 */
gptq_status gptq_context_set_wait_limit(gptq_context* ctx, int32_t polls);

/* Quantizer settings (host struct). */
typedef struct {
    int32_t bits;        /* 3 (codes as a bitstream, eight in three bytes; d_col a multiple
                            of 8), 4 (two per byte) or 8 (one per byte) */
    int32_t group_size;  /* weights per scale/zero group along a row; must divide
                            block_size and d_col; 0 = one group per row; -1 = one range
                            for the whole matrix (per tensor: every row stores the same
                            S16 and zero, laid out as one group per row; dequantize and
                            the quantized linear take -1 or 0 for it).  Quantization
                            concepts guide, "Choose granularity". */
    int32_t sym;         /* 0: asymmetric grid [0, 2^bits-1], S = (max-min)/(2^bits-1),
                               Z = -round(min/S16);
                            1: symmetric grid +-(2^(bits-1)-1), S = absmax/(2^(bits-1)-1),
                               stored codes shifted by 2^(bits-1), stored zero 2^(bits-1)
                         2: FP4 E2M1 grid (bits 4): values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6},
                            S = absmax / 6 per group, nearest value with ties to the even
                            mantissa, code = sign bit 8 | magnitude index, stored zero 0;
                            dequantize with gptq_dequantize_e2m1;
                         3: as 2 with S rounded up to a power of two (MXFP4).
                            Quantization concepts guide, "FP4 with block scales". */
    int32_t block_size;  /* lazy-update block width; the library supports 128 */
} gptq_params;

/*
 * H += 2 * X^T X   (Hessian of the layer objective ||X (W - What)^T||^2)
 *
 * Source: GPTQ summary page, statement of the one-layer procedure (H = 2 X X^T
 * with the page's d_col x tokens X; the same matrix for the tokens x d_col X used
 * here).  Call once per chunk of calibration tokens; zero H before the first call.
 *
 *  H        d_col x d_col fp32, read and written.  H is kept symmetric: both
 *           triangles are written with the same values.
 *  X        n_tokens x d_col, row stride ldx elements (ldx >= d_col), dtype x_dtype.
 *           GPTQ_BF16 and GPTQ_F16 products are exact in fp32; with X 16-byte aligned
 *           and ldx a multiple of 8 they run on the 16-bit matrix cores (fp16
 *           subnormals taken as they are), otherwise, like GPTQ_F32, on fp32 MFMA.
 *  ws       device workspace of at least gptq_hessian_workspace_size(n_tokens, d_col)
 *           bytes (the fp32 partial sums of the token splits); contents on entry are
 *           ignored.  May be NULL when the size is 0.
 * The accumulation order is fixed, so results are bitwise reproducible.
 * n_tokens == 0 or d_col == 0 is a no-op.
 */
size_t gptq_hessian_workspace_size(int64_t n_tokens, int64_t d_col);
gptq_status gptq_hessian_accumulate(float* H, const void* X, gptq_dtype x_dtype,
                                    int64_t n_tokens, int64_t d_col, int64_t ldx,
                                    void* ws, size_t ws_bytes, void* stream);

/*
 * U = upper Cholesky factor of (H + lambda I)^-1, lambda = percdamp * mean(diag H):
 * (H + lambda I)^-1 = U^T U, U upper triangular with a positive diagonal.
 *
 * Source: GPTQ summary page, "Innovation 3" (Cholesky decomposition of the inverse
 * Hessian computed once in advance, entries read row by row; dampening term
 * lambda I for near-singular H).  Computed as U = T^-1 where H + lambda I = T T^T
 * with T upper triangular (a Cholesky factorization that starts from the last
 * column), in fp64, then rounded to fp32.
 *
 *  H        d_col x d_col fp32 (only the upper triangle is read).
 *  U        d_col x d_col fp32 output; the strictly lower triangle is written as 0.
 *  ws       at least gptq_prepare_hinv_workspace_size(d_col) bytes.
 *  ctx      NULL: every kernel runs on `stream`.  Otherwise a context made on the
 *           current device: the inverse of the leading row blocks then runs on its
 *           auxiliary stream beside the factorization's chain, ordered after the
 *           earlier work of `stream` and joined back into `stream` by its events, so
 *           `stream` sees the call as one ordered operation (also under stream
 *           capture).  The result is bit-identical either way.
 * `stream` must belong to the current device.
 *
 *  info     device int32: 0, or k > 0 when the trailing principal submatrix of
 *           H + lambda I of order k is not positive definite (U is then undefined),
 *           or -1 when diag(H) holds a non-finite value, or -2 when a workgroup of
 *           the factorization waited longer than its bound (about 2 s, or what
 *           gptq_context_set_wait_limit set) for the diagonal block that another
 *           workgroup of the same launch publishes (U is then undefined).  The
 *           publishing workgroup is dispatched before every workgroup that waits for
 *           it and depends on no other, so it runs whenever one waits, also beside
 *           concurrent work on the device: with the default bound -2 means a device
 *           slowed some 10^5-fold.
 */
size_t gptq_prepare_hinv_workspace_size(int64_t d_col);
/* The same size under the name with a U type: u_dtype must be GPTQ_F32 (U is fp32; any
 * other value gives 0). */
size_t gptq_prepare_hinv_workspace(int64_t d_col, gptq_dtype u_dtype);
gptq_status gptq_prepare_hinv(const float* H, float* U, int64_t d_col, float percdamp,
                              void* ws, size_t ws_bytes, int32_t* info, gptq_context* ctx, void* stream);

/*
 * Quantize W column by column in natural order with error compensation through U.
 *
 * Sources: GPTQ summary page (OBQ background; "Innovation 1" fixed order;
 * "Innovation 2" lazy blocks of 128 columns; "Innovation 3" rows of U);
 * Quantization concepts guide ("Mapping values to fewer bits", "Choose
 * granularity", "Data types - int8 and int4").
 *
 * For every row r and column c = 0..d_col-1: at the first column of a group the
 * group's scale S and zero point Z are computed from the group's current
 * (compensated) values and S16 = fp16(S); then
 *     q = clamp(rne(w / S16 + Z))  (fp32, IEEE division), what = S16 (q - Z),
 *     err = (w - what) / U[c][c],  w[c+1:] -= err * U[c][c+1:].
 * Updates stay inside the current 128-column block; the block's errors are applied
 * to the later columns in one matrix product per block.
 *
 *  W          d_row x d_col, dtype w_dtype (read only).
 *  U          d_col x d_col fp32 from gptq_prepare_hinv (upper triangle read; the
 *             strictly lower triangle of each 128x128 diagonal block must be 0).
 *  p          host pointer to the settings.
 *  codes      bits == 4: d_row x d_col/2 bytes, column 2k in the low nibble of byte k,
 *             column 2k+1 in the high nibble (d_col must be even);
 *             bits == 3: d_row x 3 d_col/8 bytes, each row a bitstream with column c in
 *             stream bits 3c .. 3c+2 (lowest bit first) and stream bit i in bit i % 8
 *             of byte i / 8 (d_col must be a multiple of 8; the concepts guide's
 *             first-value-lowest order of "Data types - int8 and int4" continued);
 *             bits == 8: d_row x d_col bytes.  Codes are unsigned (see gptq_params).
 *  scales_f16 d_row x n_groups fp16 bit patterns (S16); n_groups = d_col/group_size,
 *             or 1 when group_size is 0 or -1.
 *  zeros_f16  d_row x n_groups fp16 bit patterns of the stored (integer) zero point.
 *  ws         at least gptq_quantize_workspace_size(d_row, d_col, p) bytes.
 *  info       device int32: 0, or -1 when W holds a non-finite value or a scale is
 *             not a normal fp16 number.
 * Rows are independent given U; d_row == 0 is a no-op.
 */
size_t gptq_quantize_workspace_size(int64_t d_row, int64_t d_col, const gptq_params* p);
/* The same size under the shorter name. */
size_t gptq_quantize_workspace(int64_t d_row, int64_t d_col, const gptq_params* p);
gptq_status gptq_quantize_layer(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col,
                                const float* U, const gptq_params* p,
                                uint8_t* codes, uint16_t* scales_f16, uint16_t* zeros_f16,
                                void* ws, size_t ws_bytes, int32_t* info, void* stream);

/*
 * gptq_quantize_layer without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  It computes exactly what gptq_quantize_layer computes (the same
 * kernels), with the library's own scratch in place of `ws`: a fixed array of
 * GPTQ_NOALLOC_SCRATCH_BYTES in each GPU's memory, held from the library's first use of
 * that GPU until the process ends.  The call allocates and frees nothing.
 *
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time on one GPU
 * (different streams, or several host threads) race and must be serialized by the
 * caller; calls ordered on one stream are fine.
 *
 *  W, U, p, codes, scales_f16, zeros_f16, info, stream   as for gptq_quantize_layer.
 * Errors as gptq_quantize_layer, and GPTQ_ERR_UNSUPPORTED when the layer needs more than
 * the scratch holds (gptq_quantize_workspace_size(d_row, d_col, p) >
 * GPTQ_NOALLOC_SCRATCH_BYTES: up to 4096 x 4096 fits), decided before anything is queued.
 */
#define GPTQ_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
gptq_status gptq_quantize_layer_noalloc(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col,
                                        const float* U, const gptq_params* p,
                                        uint8_t* codes, uint16_t* scales_f16, uint16_t* zeros_f16,
                                        int32_t* info, void* stream);

/*
 * Several layers in one call, with the phases of different layers overlapped: for
 * every layer, H = 2 X^T X over its own calibration inputs, U as gptq_prepare_hinv
 * makes it, and codes, scales and zeros as gptq_quantize_layer writes them; each
 * layer's outputs are bit-identical to those three calls'.  Consecutive layers with
 * the same inputs (X, x_dtype, n_tokens, ldx, d_col all equal: a block's q, k and v,
 * or gate and up) share one H and one U.
 *
 * Source: GPTQ summary page, the statement of the procedure (the model is quantized
 * layer by layer, each layer from the inputs it receives; H depends only on a layer's
 * inputs) and "Innovation 3" (the factorization is computed once per H).
 *
 * Schedule: groups start widest first (ties in the given order; no layer's result
 * depends on the order).  With a context, their Hessians run one after another on the
 * context's Hessian stream and the k-th started group's factorization and sweeps on
 * slot stream k mod n_slots, so the next group's Hessian overlaps the running
 * factorizations and sweeps, and the factorizations of up to n_slots groups overlap
 * each other; the call is ordered after the work already queued on `stream`, and later
 * work on `stream` after it.  With ctx NULL every group runs on `stream`, one after
 * another.
 *
 *  layers     host array of n_layers descriptors (device pointers inside); the
 *             quantizer settings p apply to every layer (group size dividing each d_col).
 *  n_slots    1 .. GPTQ_LAYERS_MAX_SLOTS, and at most the context's: groups in flight at
 *             once (memory grows with it; without a context 1 is enough).
 *  ws         at least gptq_quantize_layers_workspace_size(layers, n_layers, n_slots)
 *             bytes, 256-byte aligned: n_slots x (H, U, factorization and sweep
 *             workspaces of the largest layer) + one Hessian workspace.
 *  info       device int32[2 * n_layers], set to 0 first: info[2l] = the factorization's
 *             status for layer l's group (on the group's first layer; as
 *             gptq_prepare_hinv), info[2l + 1] = layer l's sweep status (as
 *             gptq_quantize_layer).
 * Errors (checked for every layer before anything is queued): as the per-phase calls;
 * n_tokens < 1, d_row < 1 or d_col < 1 -> GPTQ_ERR_INVALID_ARG; n_slots out of range
 * (or above the context's) -> GPTQ_ERR_INVALID_ARG.  n_layers = 0 is a no-op.
 */
typedef struct gptq_layer {
    const void* X; gptq_dtype x_dtype; int64_t n_tokens; int64_t ldx;   /* n_tokens x d_col inputs */
    const void* W; gptq_dtype w_dtype; int64_t d_row; int64_t d_col;    /* d_row x d_col weights */
    uint8_t* codes; uint16_t* scales_f16; uint16_t* zeros_f16;          /* outputs, as gptq_quantize_layer */
} gptq_layer;
size_t gptq_quantize_layers_workspace_size(const gptq_layer* layers, int32_t n_layers, int32_t n_slots);  /* reads shapes only */
gptq_status gptq_quantize_layers(const gptq_layer* layers, int32_t n_layers, float percdamp,
                                 const gptq_params* p, int32_t n_slots, void* ws, size_t ws_bytes,
                                 int32_t* info, gptq_context* ctx, void* stream);

/*
 * OBQ, the method GPTQ is compared with: every row on its own, its weights quantized
 * in a greedy order (next: the remaining weight whose quantization adds the least
 * error, (w_j - q(w_j))^2 / [F]_jj), each followed by the update of the row's other
 * remaining weights and the removal of that weight from F, the inverse Hessian of the
 * remaining weights (starting from (H + lambda I)^-1 = U^T U).  The row's grid is
 * fixed first from its original values (one group per row).  O(d_row d_col^3); a
 * baseline for timing, not a production path.
 *
 * Source: GPTQ summary page, OBQ background (greedy order, update of the remaining
 * weights and of the inverse Hessian after each weight) and the runtime comparison
 * with GPTQ.
 *
 *  W, U, p, codes, scales_f16, zeros_f16, info   as for gptq_quantize_layer; p must have
 *             group_size 0 and an integer grid, sym 0 or 1 (else GPTQ_ERR_UNSUPPORTED).
 *  ws         at least gptq_obq_workspace_size(d_row, d_col) bytes: H^-1 and one
 *             d_col x d_col copy per row in flight (at most 256).
 * Errors as gptq_quantize_layer; d_col > 2048 -> GPTQ_ERR_UNSUPPORTED.  Arithmetic is
 * fp32, so where two candidates' added errors are nearly equal the order can differ
 * from an fp64 evaluation.
 */
size_t gptq_obq_workspace_size(int64_t d_row, int64_t d_col);
gptq_status gptq_obq_layer(const void* W, gptq_dtype w_dtype, int64_t d_row, int64_t d_col,
                           const float* U, const gptq_params* p,
                           uint8_t* codes, uint16_t* scales_f16, uint16_t* zeros_f16,
                           void* ws, size_t ws_bytes, int32_t* info, void* stream);

/*
 * W_out = S16 * (u - z) for every weight (computed in fp32, exact, then rounded
 * to out_dtype with round-to-nearest-even).
 *
 * Source: Quantization concepts guide, "Mapping values to fewer bits"
 * (x ~= S (q - Z)) and "Data types - int8 and int4" (unpacking two codes per byte).
 *
 *  codes, scales_f16, zeros_f16   as written by gptq_quantize_layer (bits 3: the 3-bit
 *             stream, d_col a multiple of 8, else GPTQ_ERR_INVALID_ARG).
 *  W_out      d_row x d_col, dtype out_dtype.
 */
gptq_status gptq_dequantize(const uint8_t* codes, const uint16_t* scales_f16,
                            const uint16_t* zeros_f16, int64_t d_row, int64_t d_col,
                            int32_t bits, int32_t group_size,
                            void* W_out, gptq_dtype out_dtype, void* stream);

/*
 * W_out = S16 * e2m1(u) for every weight of a layer quantized on the FP4 E2M1 grid
 * (gptq_params.sym = 2): e2m1(u) = +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}[u & 7], negative when
 * u & 8.  Same layout and errors as gptq_dequantize (no zero array: the grid has none).
 *
 * Source: Quantization concepts guide, "FP4 with block scales".
 */
gptq_status gptq_dequantize_e2m1(const uint8_t* codes, const uint16_t* scales_f16, int64_t d_row,
                                 int64_t d_col, int32_t group_size, void* W_out, gptq_dtype out_dtype,
                                 void* stream);

/*
 * The layer's product on its quantized weights, read from the stored format:
 *   y[t][r] = sum_c x[t][c] * What[r][c],  What[r][c] = S16[r][g] * (u[r][c] - z[r][g]),
 * accumulated in fp32 (per piece of one group: sum of x * (u - z), then times S16),
 * rounded once to y_dtype.
 *
 * Sources: GPTQ summary page, layer-wise objective (the layer computes W X; with
 * activations stored tokens x d_col the output is X W^T) and its results on
 * inference with the packed weights; Quantization concepts guide, "Mapping values to
 * fewer bits" (x ~= S (q - Z)) and "Data types - int8 and int4".
 *
 *  codes, scales_f16, zeros_f16   as written by gptq_quantize_layer (bits, group_size
 *             as there: 3 the 3-bit stream, 4 two per byte, 8 one per byte; group 0 = per
 *             row).
 *  x          n_tokens x d_col, row pitch ldx >= d_col elements, dtype x_dtype.
 *  y          n_tokens x d_row (row pitch d_row), dtype y_dtype; written, not read.
 * Any even d_col works (3-bit: a multiple of 8); d_col a multiple of 32 with 16-byte
 * aligned code rows (3-bit: 4-byte) and x rows takes the fast kernels: a single token
 * streams the codes with fp32 multiply-adds; from two tokens on, 3- or 4-bit codes with
 * bf16/f16 x and d_col and the group width multiples of 128 go to the matrix cores (u - z decoded once per 16 tokens, exact in
 * x's 16-bit type for integer zeros, else completed by a second product of the
 * remainder), otherwise the codes are streamed once per four tokens.
 * Integer grids only (a layer on the E2M1 grid is dequantized with gptq_dequantize_e2m1).
 * Errors: negative sizes, bad dtypes or group width, or bits 3 with d_col not a multiple
 * of 8 -> GPTQ_ERR_INVALID_ARG; bits not 3/4/8 -> GPTQ_ERR_UNSUPPORTED; zero sizes are a
 * no-op.
 */
gptq_status gptq_quantized_linear(const uint8_t* codes, const uint16_t* scales_f16,
                                  const uint16_t* zeros_f16, int64_t d_row, int64_t d_col,
                                  int32_t bits, int32_t group_size,
                                  const void* x, gptq_dtype x_dtype, int64_t n_tokens, int64_t ldx,
                                  void* y, gptq_dtype y_dtype, void* stream);

/* Host: a static message for a status code. */
const char* gptq_status_string(gptq_status s);

#ifdef __cplusplus
}
#endif
#endif /* GPTQ_MI355X_H */
