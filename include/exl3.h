/*
 * exl3.h -- C ABI of the MI355X (gfx950) EXL3 trellis tile encoder.
 *
 * Sources of the operations (cited by page title and section):
 *   [P1] "EXL3 Intel Arc Quantizer" README, Core Implemented Architecture:
 *        section 1 (tile encoder: add-compare-select dynamic program, two-pass
 *        tail-biting closure), section 4 (16-bit state algebra), section 5
 *        (mul1 codebook, MSB-first container with SWAP16), section 7 (blockwise
 *        Sylvester Hadamard), section 8 (regularization and scale search over a
 *        wrapped-diagonal tile sample; out-channel normalization), section 2
 *        (bounded scratch, admission before work, batch halving that keeps
 *        results identical).
 *   [P2] "JEV-9B EXL3 K=2 (mul1) Checkpoint" model card, section 2
 *        (golden-section scale search).
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer on the context's device unless
 *     stated otherwise; the caller owns it.  The library never frees it and
 *     never keeps it beyond the work it enqueued on the context's stream.
 *     Before any launch each array is checked to lie inside one allocation
 *     the context's GPU can address (device memory of that device, managed
 *     memory, or pinned host memory) that holds every byte the call touches;
 *     otherwise (plain host memory, another device's memory, a buffer ending
 *     too early) the call returns EXL3_EINVAL.  A sub-range of a larger
 *     allocation, such as a caching allocator's segment, is measured against
 *     that allocation.  Arrays documented as host arrays must not be device
 *     memory.
 *   - Calls return EXL3_OK (0) or a negative EXL3_E* code and never throw.
 *     exl3_last_error() gives the message.  Arguments are validated before
 *     anything is enqueued: on a validation error no output has been
 *     written; a failure later in the call (EXL3_ENOMEM, EXL3_EHIP) may leave
 *     outputs partly written.
 *   - Arithmetic contract: binary32, each subtract / multiply / add rounded on
 *     its own (no fused multiply-add), lowest index on equal costs (the *_f16
 *     entry points state their binary16 contract).  Outputs are bit-identical
 *     for any batch size and scratch limit.
 *   - A context is not thread-safe; use one per host thread / stream.  Every
 *     call makes the context's device current on the calling thread.
 *   - Tiles: a 16x16 tile is 256 consecutive values in trellis order: position
 *     t holds the tile's element order[t] (element 16*row + col), order being
 *     the context's within-tile order (exl3_set_tile_order; by default the
 *     identity, position t = element t); tile tau = tr * (cols/16) + tc of a
 *     rows x cols matrix.
 */
#ifndef EXL3_H
#define EXL3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    EXL3_OK = 0,
    EXL3_EINVAL = -1,        /* bad argument (null pointer, shape, sign vector, ...) */
    EXL3_ENOMEM = -2,        /* scratch limit below one tile, or device allocation failed */
    EXL3_ENONFINITE = -3,    /* NaN or Inf in the weight matrix */
    EXL3_EHIP = -4,          /* a HIP runtime call failed; the context stays usable */
    EXL3_EUNSUPPORTED = -5   /* K or Hadamard block not supported */
};

enum { EXL3_F32 = 0, EXL3_BF16 = 1 };              /* weight storage type */
enum { EXL3_ROW_MAJOR = 0, EXL3_TILE_MAJOR = 1 };  /* layout of regularized output */

typedef struct exl3_ctx exl3_ctx;

/* Golden-section scale search [P2 section 2; P1 section 8]: bracket
 * [lo * rms, hi * rms], two initial probes, then `iters` reductions. */
typedef struct {
    int iters;
    double lo;
    double hi;
} exl3_gss;

/* Library version string (static storage). */
const char *exl3_version(void);

/*
 * Create a context on HIP device `device`.  `hip_stream` is a hipStream_t the
 * caller owns (NULL = the null stream); every call enqueues on it.
 * `scratch_bytes` bounds the backpointer scratch the context may allocate
 * (0 = a default of 64 GiB, about a fifth of an MI355X's HBM: the final
 * encode of a 4096 x 4096 matrix in one batch); batches are sized to fit it
 * and the scratch grows only to what a call needs [P1 section 2].
 * The context uploads the mul1 level table (65,536 fp16 values, 128 KiB).
 * Errors: EXL3_EINVAL (out == NULL), EXL3_EHIP (device unusable).
 */
int exl3_ctx_create(exl3_ctx **out, int device, void *hip_stream, size_t scratch_bytes);

/* Destroy a context: waits for its stream, frees what it allocated.  NULL is ignored. */
void exl3_ctx_destroy(exl3_ctx *ctx);

/* Last error message of this context ("" if none); never NULL.  ctx may be NULL. */
const char *exl3_last_error(const exl3_ctx *ctx);

/*
 * Change the stream later calls enqueue on (the caller still owns it).  The new
 * stream is made to wait (through an event, without blocking the host) for the
 * work already enqueued on the old one, since that work may still use the
 * context's buffers.  Errors: EXL3_EINVAL, EXL3_EHIP.
 */
int exl3_ctx_set_stream(exl3_ctx *ctx, void *hip_stream);

/*
 * Replace the level table with caller-supplied fp16 values (HOST pointer,
 * 65,536 uint16 bit patterns, copied before return).  NULL restores mul1.
 * Used to run other procedural codebooks or synthetic tables through the
 * same kernels.  Errors: EXL3_EINVAL (a value is NaN or Inf), EXL3_EHIP.
 */
int exl3_set_codebook(exl3_ctx *ctx, const uint16_t *levels_fp16_host);

/* Copy the current level table to a HOST buffer of 65,536 uint16. */
int exl3_get_codebook(exl3_ctx *ctx, uint16_t *levels_fp16_host);

/*
 * Within-tile order of every tile-major array of this context [P1 section 5:
 * a fixed 256-element permutation of the positions within a tile, and its
 * inverse, for the tensor-core decoder; P1 section 3: LDLQ encodes permuted
 * tiles and reconstructs in matrix order].  The pages do not print the
 * table, so the caller supplies it:
 *   order_host  host uint8 [256], a permutation of 0..255: trellis position t
 *               of a tile holds the tile's element order[t] = 16*row + col.
 *               NULL (or the identity) restores the natural order.
 * It applies where tiles meet matrix order: the tile-major layouts of
 * exl3_regularize (output and per-tile energies, summed in trellis order)
 * and exl3_unregularize (input), and the whole-matrix calls (their tiles,
 * w_hat, per-tile outputs and container, and LDLQ's feedback in matrix
 * order).  exl3_encode_tiles / exl3_decode_tiles take tiles already in
 * trellis order and are unaffected.  Work enqueued before the call keeps the
 * previous order.  Errors: EXL3_EINVAL (not a permutation, device memory),
 * EXL3_ENOMEM, EXL3_EHIP.
 */
int exl3_set_tile_order(exl3_ctx *ctx, const uint8_t *order_host);

/*
 * Select one of the procedural codebooks [P1 section 5: mul1, mcg, 3INST; the
 * pages print their counts of distinct levels, 913, 10,746 and 10,598] as the
 * level table of later calls (binary32 and binary16 modes, encode and decode).
 *   EXL3_CB_MUL1   the default table (see exl3_set_codebook)
 *   EXL3_CB_MCG    w = 0x9E378FED * s mod 2^32 (the first odd multiplier from
 *                  0x9E3779B1 up whose table has the printed 10,746 levels)
 *   EXL3_CB_3INST  w = 89226354 * s + 64248484 mod 2^32 (the QTIP three-
 *                  instruction decoder)
 * For mcg and 3INST, w = (w & 0x8FFF8FFF) ^ 0x3B603B60 and the level is the
 * binary16 sum (round to nearest even) of w's two halves read as binary16.
 * Levels of mcg and 3INST have a standard deviation near 1.24 (mul1: 1), so
 * the best scale is near rms / 1.24, inside the default search bracket.
 * Synchronizes the stream.  Errors: EXL3_EUNSUPPORTED (unknown kind), EXL3_EHIP.
 */
enum { EXL3_CB_MUL1 = 0, EXL3_CB_MCG = 1, EXL3_CB_3INST = 2 };
int exl3_set_codebook_kind(exl3_ctx *ctx, int kind);

/*
 * Regularize a weight matrix [P1 sections 7 and 8]:
 *   W_reg = H_l diag(su) W diag(sv) H_r
 * where H_l / H_r apply the natural-order Sylvester Hadamard of size had_block
 * to each block of had_block rows / columns, each normalised by the binary32
 * value of 1/sqrt(had_block).  Order of evaluation: sign flips, left
 * transform, normalisation, right transform, normalisation.
 *   w          [rows][cols] row-major, w_dtype EXL3_F32 or EXL3_BF16
 *   su, sv     float [rows], float [cols]; every entry exactly +1 or -1
 *   w_reg      float [rows*cols]; row-major or tile-major (out_layout)
 *   tile_sumsq optional float [(rows/16)*(cols/16)]: per tile, the sequential
 *              binary32 sum over t = 0..255 of rn(w_t * w_t)
 *   nonfinite  optional int [1]: set to 1 if W holds NaN/Inf (left unchanged
 *              otherwise; the caller clears it)
 * rows and cols must be multiples of had_block (64 or 128).  Asynchronous.
 * Errors: EXL3_EINVAL, EXL3_EUNSUPPORTED, EXL3_EHIP.
 */
int exl3_regularize(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                    int had_block, const float *su, const float *sv, float *w_reg,
                    int out_layout, float *tile_sumsq, int *nonfinite);

/*
 * Inverse of exl3_regularize [P1 section 7: decode applies H_l, x su, H_r,
 * x sv; H is its own inverse]: W = diag(su) H_l W_reg H_r diag(sv), evaluated
 * as left transform, x rn32(1/sqrt(had_block)), right transform, the same
 * factor, then x su[row], x sv[col].  su and sv may be any finite values (the
 * folded signs of exl3_channel_normalize), so dequantized tiles go back to the
 * original weights' domain.
 *   w_reg     float [rows*cols], tile-major (as exl3_decode_tiles and the
 *             w_hat outputs write it) or row-major (in_layout)
 *   su, sv    float [rows], float [cols]
 *   out       float [rows][cols] row-major; must not overlap w_reg
 * rows and cols multiples of had_block (64 or 128).  Asynchronous.
 * Errors: EXL3_EINVAL, EXL3_EUNSUPPORTED, EXL3_EHIP.
 */
int exl3_unregularize(exl3_ctx *ctx, const float *w_reg, int in_layout, int rows, int cols,
                      int had_block, const float *su, const float *sv, float *out);

/*
 * Out-channel RMS normalization with the scale folded into the row signs
 * [P1 section 8: out-channel RMS normalization, sign + scale folding, the
 * zero-channel floor, a zero sign for all-zero channels].  The output channels
 * are the rows of W (the LDLQ factor of exl3_quantize_matrix_ldlq acts on the
 * columns, the input side).  Per row i:
 *   r_i        = sqrt(sum_j w_ij^2 / cols) in binary64, j ascending
 *   f_i        = (float)(1.0 / r_i), with r_i replaced by `floor` (the pages:
 *                0.1) when it is 0
 *   w_norm_ij  = rn32(w_ij * f_i)
 *   su_folded_i = su_i * (float)r_i, or +0 when r_i is 0
 * Quantizing w_norm with the +-1 signs su and decoding with su_folded in
 * place of su gives back W (up to the roundings above).
 *   w          [rows][cols] row-major, w_dtype EXL3_F32 or EXL3_BF16
 *   su         float [rows], every entry exactly +1 or -1
 *   w_norm     float [rows][cols] row-major; must not overlap w
 *   su_folded  float [rows]
 *   row_rms    optional double [rows]: r_i before the floor
 * Non-finite weights give non-finite rows of w_norm (exl3_quantize_matrix
 * then rejects them).  rows, cols >= 1; floor finite and > 0.  Asynchronous.
 * Errors: EXL3_EINVAL, EXL3_EHIP.
 */
int exl3_channel_normalize(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                           const float *su, double floor, float *w_norm, float *su_folded,
                           double *row_rms);

/*
 * Encode n tiles at a fixed binary32 scale [P1 sections 1, 4, 5]:
 * a two-pass tail-biting Viterbi search over the 16-bit bitshift trellis that
 * shifts in K bits per step, comparing each input with v[s] = rn(scale*c[s]).
 *   x         float [n][256] tile-major inputs (finite; otherwise the output is
 *             unspecified but the call stays memory-safe)
 *   packed    uint16 [n][16*K]: the low K bits of each state, MSB-first, then
 *             words 2i and 2i+1 swapped
 *   states    optional uint16 [n][256]: the state sequence S_0..S_255
 *   tile_sse  optional float [n]: sequential binary32 sum of squared errors of
 *             the decoded tile, which equals the search's own path cost
 * K in {1, 2, 3, 4}.  n may be 0.  Asynchronous (uses the context's scratch).
 * Errors: EXL3_EINVAL, EXL3_EUNSUPPORTED, EXL3_ENOMEM, EXL3_EHIP.
 */
int exl3_encode_tiles(exl3_ctx *ctx, const float *x, int64_t n, int K, float scale,
                      uint16_t *packed, uint16_t *states, float *tile_sse);

/* Most tiles one exl3_encode_tiles_noalloc call takes (its static scratch). */
enum { EXL3_NOALLOC_MAX_TILES = 256, EXL3_NOALLOC_MAX_TILES_K4 = 512 };

/*
 * exl3_encode_tiles without any device allocation, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, outputs and results, bit for bit, as
 * exl3_encode_tiles; the chain's scratch (backpointers and per-tile
 * bookkeeping) is a fixed array in the library's device code, 267,390,976 B
 * (255 MiB) that every GPU the library is loaded on holds until the process
 * ends, looked up once per device when a context is created there.
 *   n <= EXL3_NOALLOC_MAX_TILES (K = 1, 2, 3) or EXL3_NOALLOC_MAX_TILES_K4
 *   (K = 4) per call; larger n is rejected with EXL3_EINVAL before any launch
 *   (encode the rest in further calls).
 * The call enqueues four kernels on the context's stream and calls no
 * hipMalloc / hipFree.  All calls on one GPU share that GPU's array, which
 * keeps the last call's contents (nothing in it needs to start at zero):
 * calls that overlap on one GPU -- on different streams or contexts, or from
 * different threads -- race; order them on one stream.
 * Errors: EXL3_EINVAL, EXL3_EUNSUPPORTED, EXL3_EHIP (also when the array's
 * address could not be looked up for this device).
 */
int exl3_encode_tiles_noalloc(exl3_ctx *ctx, const float *x, int64_t n, int K, float scale,
                              uint16_t *packed, uint16_t *states, float *tile_sse);

/*
 * Encode n tiles in binary16 arithmetic [P1 sections 1 and 4: the half-precision
 * add-compare-select]: the same two-pass tail-biting search, with inputs, code
 * values and path costs in IEEE binary16.  Per state and step the difference
 * x_t - c[s] is rounded once to binary16 and the cost d*d + M is one fused
 * multiply-add rounded once to binary16 (nearest-even, subnormals kept,
 * overflow to +inf); among equal costs the lowest branch index wins, and the
 * pass-1 end state is the lowest-index state of least cost.  The code values
 * are the context's codebook as binary16 bit patterns, unscaled.
 *   x         uint16 [n][256]: binary16 bit patterns, tile-major (finite;
 *             otherwise the output is unspecified but the call stays
 *             memory-safe)
 *   packed    uint16 [n][16*K]: container as for exl3_encode_tiles
 *   states    optional uint16 [n][256]: the state sequence S_0..S_255
 *   cost      optional uint16 [n]: the path cost as binary16 bits (the
 *             binary16 sequential sum over the tile of fp16(fp16(x_t - c)^2 + acc))
 * K in {1, 2, 3, 4}.  n may be 0.  Asynchronous (uses the context's scratch).
 * Errors: EXL3_EINVAL, EXL3_EUNSUPPORTED, EXL3_ENOMEM, EXL3_EHIP.
 */
int exl3_encode_tiles_f16(exl3_ctx *ctx, const uint16_t *x, int64_t n, int K, uint16_t *packed,
                          uint16_t *states, uint16_t *cost);

/*
 * Decode n packed tiles [P1 section 5]: S_t = the 16-bit window of the
 * circular bit stream that ends at bit (t+1)*K - 1; out[t] = rn(scale*c[S_t]).
 *   packed uint16 [n][16*K] (as written by exl3_encode_tiles), out float [n][256].
 * K in 1..8.  Asynchronous.  Errors: EXL3_EINVAL, EXL3_EUNSUPPORTED, EXL3_EHIP.
 */
int exl3_decode_tiles(exl3_ctx *ctx, const uint16_t *packed, int64_t n, int K, float scale,
                      float *out);

/*
 * Whole-matrix quantization [P1 sections 1, 7, 8; P2 section 2]:
 * regularize, per-tile energy, rms = sqrt(sum / (rows*cols)) in binary64,
 * then either the fixed scale (gss == NULL) or a golden-section search for the
 * scale on the tile sample (wrapped diagonal plus the highest- and
 * lowest-energy tiles), whose objective is the binary64 sum, in ascending tile
 * order, of the sample tiles' squared errors; the result is the midpoint of the
 * final bracket rounded to binary32 (0 when rms is 0).  The sample is encoded
 * iters + 1 times: the last reduction's new point is never scored, since the
 * bracket it narrows already fixes the result.  Then every tile is encoded at
 * that scale.
 *   w, w_dtype, rows, cols, had_block, su, sv : as exl3_regularize
 *   packed    uint16 [rows/16][cols/16][16*K]
 *   scale_out HOST float [1]: the scale used
 *   mse_out   optional HOST double [1]: binary64 sum of tile errors / (rows*cols)
 *   w_hat     optional float [rows*cols]: dequantized weights in the
 *             regularized domain, tile-major
 *   tile_sse  optional float [tiles]: per-tile squared error
 * Synchronizes the stream: the tile energies are read back to pick the sample,
 * the search's probes and reductions then run on the device without a host
 * round trip, and its result and the errors are read back; returns after all
 * work is complete.  Errors: EXL3_EINVAL, EXL3_EUNSUPPORTED, EXL3_ENOMEM,
 * EXL3_ENONFINITE (before any encode), EXL3_EHIP.
 */
int exl3_quantize_matrix(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                         int K, int had_block, const float *su, const float *sv,
                         const exl3_gss *gss, float fixed_scale, uint16_t *packed,
                         float *scale_out, double *mse_out, float *w_hat, float *tile_sse);

/*
 * Whole-matrix quantization with the binary16 encoder [P1 sections 1 and 4:
 * the search runs in half precision; section 8: scale search] -- the
 * exl3_quantize_matrix path with exl3_encode_tiles_f16 inside: at a scale s
 * the encoder inputs are fp16(rn32(w / s)) (all zero at s = 0), the binary16
 * two-pass search gives the states, and each tile is dequantized and scored
 * as in exl3_quantize_matrix (w_hat = rn32(s * c[state]), sequential binary32
 * squared error).  The golden-section objective is the binary64 ascending sum
 * of those errors over the tile sample; gss == NULL uses fixed_scale.
 * Arguments, outputs and errors as exl3_quantize_matrix (tile_sse: the
 * binary32 squared errors).  Synchronizes the stream.
 */
int exl3_quantize_matrix_f16(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                             int K, int had_block, const float *su, const float *sv,
                             const exl3_gss *gss, float fixed_scale, uint16_t *packed,
                             float *scale_out, double *mse_out, float *w_hat, float *tile_sse);

/*
 * Whole-matrix quantization with the pages' grid + parabolic scale search
 * [P1 section 8] instead of the golden section: the search runs over a
 * multiplier g of the matrix rms.  Coarse points g = coarse_lo + k*coarse_step,
 * k = 0 .. round((coarse_hi - coarse_lo) / coarse_step), are scored on every
 * stride-th tile of the scale-search tile set (the set of exl3_quantize_matrix),
 * fine points g_c + m*fine_step, |m| <= round(fine_radius / fine_step), around
 * the best coarse point g_c on the whole set; the objective is the binary64
 * sum, in ascending tile order, of the path costs at scale (float)(g * rms);
 * the least value wins (lowest g on ties).  If the best fine point is interior,
 * the vertex of the parabola through it and its two neighbours replaces it; the
 * result is at least `floor`, and the scale is (float)(g * rms) (0 when rms is 0).
 * The pages' values: {0.1, 1.9, 0.1, 2, 0.075, 0.025, 0.01}.
 * Outputs and errors as exl3_quantize_matrix; EXL3_EINVAL for a null or
 * malformed grid (coarse_lo <= 0, steps <= 0, stride < 1, floor < 0, more than
 * 1000 points per stage).
 */
typedef struct {
    double coarse_lo, coarse_hi, coarse_step;
    int stride;
    double fine_radius, fine_step;
    double floor;
} exl3_grid;

int exl3_quantize_matrix_grid(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                              int K, int had_block, const float *su, const float *sv,
                              const exl3_grid *grid, uint16_t *packed, float *scale_out,
                              double *mse_out, float *w_hat, float *tile_sse);

/*
 * Whole-matrix quantization with LDLQ error feedback [P1 section 3: one-sided
 * block LDLQ].  Regularization and the scale exactly as exl3_quantize_matrix
 * (the scale is chosen on the matrix without feedback); then the 16-column
 * tile spans are quantized from the last to the first, span j at the target
 *     T_j = W_j + sum_{i > j} (W_i - What_i) L_ij
 * (W the regularized matrix, L_ij the 16x16 block of L at rows 16i.., columns
 * 16j..), summed per element over i ascending, then the block row ascending,
 * each product and sum rounded to binary32 on its own.
 *   L        float [cols][cols] row-major, device: unit block-lower-triangular
 *            factor of H = L D L^T over the regularized columns; only the
 *            blocks below the diagonal are read
 *   packed, scale_out, w_hat : as exl3_quantize_matrix
 *   mse_out  optional HOST double [1]: binary64 ascending sum over tiles of
 *            tile_err, / (rows*cols)
 *   tile_err optional float [tiles]: per tile, the sequential binary32 sum of
 *            (W - What)^2 (squared error against the weight, not the target)
 * Synchronizes the stream.  Errors: as exl3_quantize_matrix; EXL3_EINVAL for a
 * null L.
 */
int exl3_quantize_matrix_ldlq(exl3_ctx *ctx, const void *w, int w_dtype, int rows, int cols,
                              int K, int had_block, const float *su, const float *sv,
                              const exl3_gss *gss, float fixed_scale, const float *L,
                              uint16_t *packed, float *scale_out, double *mse_out, float *w_hat,
                              float *tile_err);

/* Kernel kinds for exl3_ctx_read_timing. */
enum {
    EXL3_KERNEL_FWD1 = 0,        /* forward pass 1 (rotated input, free start) */
    EXL3_KERNEL_FWD2 = 1,        /* forward pass 2 (start pinned to X) with
                                    backpointers */
    EXL3_KERNEL_TB1 = 2,         /* traceback to X */
    EXL3_KERNEL_TB2 = 3,         /* traceback, packing, squared error */
    EXL3_KERNEL_REGULARIZE = 4,
    EXL3_KERNEL_FWD_SIDE = 5,    /* forward passes of a scale-search probe's last
                                    partial round, run on a second stream beside
                                    the main part (their durations overlap) */
    EXL3_KERNEL_FWD_COST = 6,    /* pass 2's cost-only form (scale-search probes,
                                    on the context's stream) */
    EXL3_KERNEL_CHANNEL = 7,     /* out-channel normalization (tile count 0) */
    EXL3_KERNEL_DECODE = 8       /* exl3_decode_tiles */
};

/*
 * Per-launch timing for measurement.  With timing on, every launch of the
 * kinds above is bracketed by two HIP events on the context's stream
 * (a small overhead per launch).  Turning it on or off clears the records.
 */
int exl3_ctx_set_timing(exl3_ctx *ctx, int enable);

/*
 * Sum of the durations (ms) of the recorded launches of one kind, their count
 * and the number of tiles they processed.  Synchronizes the stream.
 */
int exl3_ctx_read_timing(exl3_ctx *ctx, int kind, double *total_ms, int64_t *launches,
                         int64_t *tiles);

/*
 * Scratch bytes one tile needs in flight at this K (backpointers of the
 * longer pass plus per-tile bookkeeping).  0 for an unsupported K.
 */
size_t exl3_scratch_per_tile(int K);

#ifdef __cplusplus
}
#endif

#endif /* EXL3_H */
