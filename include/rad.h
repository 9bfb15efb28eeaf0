/*
 * rad.h -- C ABI of librad.so: the rotated W8A8 int8 linear layer on AMD
 * MI355X (gfx950).
 *
 * The layer is the one on the model card "Qwen3.8-27B IQ8R + DFlash2 --
 * radiance container":
 *   - table row "Weights": trunk linears hold int8 codes in -127..127, one u8
 *     scale for every (row, 256 of K) under one bf16 scale per row, and every
 *     128 of K is rotated by the unnormalised Hadamard transform; the lm_head
 *     holds int8 codes with one bf16 scale for every (row, 128 of K);
 *   - table row "Activations": activations are int8 in the same rotated
 *     domain (W8A8);
 *   - section "How this file was made": the recipe rules that name these two
 *     formats and the fwht128 transform.
 * The card gives no code and no interface; the calls below are this
 * library's own.
 *
 * Conventions for every call:
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates nothing, keeps no pointer after it returns, and holds no state.
 *   - Every call only enqueues kernels on `stream` (a hipStream_t; NULL is the
 *     default stream) and returns without synchronising.  The caller keeps the
 *     buffers alive until that stream's work completes.  Calls on different
 *     streams may run concurrently; the library is thread-safe.
 *   - Every argument is validated on the host BEFORE any HIP call, so a bad
 *     argument returns an error status and enqueues nothing.  A HIP error
 *     reported by the launch is returned as RAD_E_HIP.
 *   - Sizes of zero (rows, M or N) are valid and enqueue nothing.
 *   - Data values are not checked: NaN or infinite activations, and weight
 *     codes of -128, give unspecified results.
 *   - Layouts are row-major and dense (no strides).
 */
#ifndef RAD_H
#define RAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *rad_stream_t; /* hipStream_t */

/* Status codes returned by every call. */
enum rad_status {
    RAD_OK = 0,
    RAD_E_NULL = -1,   /* a required pointer is NULL                          */
    RAD_E_SHAPE = -2,  /* a size is negative, or K is not a multiple of the
                          rotation block (128) or of the format's group width */
    RAD_E_ALIGN = -3,  /* a pointer is not aligned as the call requires       */
    RAD_E_FMT = -4,    /* unknown weight format, or a scale pointer that the
                          format requires is missing / forbids is present     */
    RAD_E_RANGE = -5,  /* a size is beyond what the call supports             */
    RAD_E_ALIAS = -6,  /* an output overlaps another argument                  */
    RAD_E_HIP = -7     /* the HIP runtime reported an error at launch          */
};

/* Weight formats. */
enum rad_format {
    /* Trunk linears: codes int8 [N][K]; gscale uint8 [N][K/256] (a plain
       integer multiplier per (row, 256 of K)); rscale bf16 bits [N]. */
    RAD_FMT_U8G256_BF16ROW = 0,
    /* Vocabulary head: codes int8 [N][K]; gscale bf16 bits [N][K/128];
       rscale must be NULL. */
    RAD_FMT_BF16G128 = 1,
    /* The drafter's linears (model card, table row "Speculator": a 16-level
       integer codebook, four bits, in the same rotated domain; section "How
       this file was made": rules with table=-127;-97;-75;-58;-43;-30;-18;-6;
       6;18;30;43;58;75;97;127 group=128 scale=bf16 transform=fwht128):
       codes are 4-bit indices into that table, packed uint8 [N][K/2] -- in
       each 16-byte run of a row, byte b holds element 32c + b in its low
       nibble and element 32c + 16 + b in its high nibble (c the run's index);
       gscale bf16 bits [N][K/128]; rscale must be NULL.  The layer is the
       head format applied to the table values.  Accepted by rad_w8a8_gemv,
       rad_w8a8_gemm (which runs it through the M <= 128 kernels in chunks of
       128 tokens), rad_w8a8_linear and rad_quant_weight_i8; not by
       rad_w8a8_rescore. */
    RAD_FMT_TBL4_BF16G128 = 2
};

/* Largest K that rad_quant_act_i8 accepts (its rows are held on chip). */
#define RAD_QUANT_MAX_K 65536
/* Largest M that rad_w8a8_gemv accepts. */
#define RAD_GEMV_MAX_M 128
/* Largest K that rad_quant_weight_i8 accepts (a rotated row is held on chip). */
#define RAD_QUANT_WEIGHT_MAX_K 32768
/* Largest K that the contraction calls (rad_w8a8_gemv, rad_w8a8_gemm,
   rad_w8a8_linear, rad_w8a8_rescore) accept: the kernels address a tile of
   up to 256 weight or token rows with 32-bit byte offsets row * K + column.
   The same calls also return RAD_E_RANGE when the group-scale array
   (N * (K / group width) * scale size) reaches 2^31 bytes, when a buffer's
   byte count does not fit int64, or, for more than RAD_GEMV_MAX_M tokens,
   when the output has 2^31 or more tiles of 256 x 128. */
#define RAD_LINEAR_MAX_K 16777216

/*
 * A quantised weight in the rotated domain.  Codes are int8 in -127..127 and
 * each contiguous 128 of a row's K has already been rotated by H (the
 * 128x128 Sylvester Hadamard matrix, H[i][j] = (-1)^popcount(i&j), no
 * normalisation).  codes must be 16-byte aligned; gscale and rscale must be
 * 4-byte aligned (the kernels read scales a 32-bit word at a time, never past
 * the end of either array).
 */
typedef struct rad_w8a8_weight {
    const int8_t *codes;     /* int8 [N][K] (packed uint8 [N][K/2] for fmt 2)  */
    const void *gscale;      /* see enum rad_format                           */
    const uint16_t *rscale;  /* bf16 bits [N], or NULL for RAD_FMT_BF16G128    */
    int64_t N;               /* output features                               */
    int64_t K;               /* input features                                */
    int32_t fmt;             /* enum rad_format                               */
} rad_w8a8_weight;

/*
 * rad_fwht128 -- y = x rotated block by block: each contiguous 128 of a row
 * of x is multiplied by H (model card, table row "Weights": every 128 of K is
 * rotated by the unnormalised Hadamard transform; table row "Activations":
 * the same rotation applies to activations).
 *
 *   x, y   f32 [rows][K], 16-byte aligned.  y == x (in place) is allowed; any
 *          other overlap returns RAD_E_ALIAS.
 *   rows   >= 0.  K > 0 and K % 128 == 0.
 *
 * The f32 result is the butterfly network with stage widths 1, 2, 4, ..., 64
 * in that order, the sum of each butterfly going to the lower index and the
 * difference (lower minus upper) to the upper; it equals x.H exactly whenever
 * no partial sum rounds.
 */
int rad_fwht128(const float *x, float *y, int64_t rows, int64_t K, rad_stream_t stream);

/*
 * rad_quant_act_i8 -- per-token symmetric int8 quantisation of activations,
 * optionally rotated first (model card, table row "Activations": int8 under
 * the same rotation as the weights; codes are symmetric in -127..127 as the
 * weights' are, table row "Weights").
 *
 *   x      f32 [M][K], 16-byte aligned.
 *   q      int8 [M][K] output, 16-byte aligned.
 *   scale  f32 [M] output, 4-byte aligned.
 *   rotate 1: x~ = x rotated as by rad_fwht128 (bit-identical); 0: x~ = x.
 *   M >= 0; K > 0, K % 128 == 0, K <= RAD_QUANT_MAX_K.
 *
 * Per token m: amax = max_k |x~[m][k]|; scale[m] = amax / 127 (f32 division);
 * q[m][k] = clamp(rne(x~[m][k] / scale[m]), -127, 127) with an f32 division and
 * ties to even.  amax == 0 gives scale[m] = 0 and q[m][:] = 0.  No output may
 * overlap x or the other output (RAD_E_ALIAS).
 */
int rad_quant_act_i8(const float *x, int8_t *q, float *scale, int64_t M, int64_t K, int rotate,
                     rad_stream_t stream);

/*
 * rad_w8a8_gemv -- the rotated W8A8 contraction and epilogue for decode and
 * verify sized batches, 1 <= M <= RAD_GEMV_MAX_M (model card, table row
 * "Weights": int8 codes under a u8 scale per (row, 256 of K) and a bf16 row
 * scale, or for the lm_head a bf16 scale per (row, 128 of K); table row
 * "Activations": int8 activations in the same rotated domain).
 *
 *   q         int8 [M][K] activation codes (from rad_quant_act_i8), 16-byte aligned.
 *   scale     f32 [M] activation scales.
 *   w         host pointer to the weight descriptor (its fields point to device
 *             memory); w->K is the K of q.
 *   y         f32 [M][N] output, 4-byte aligned.
 *   partials  NULL, or int32 [M][N][G] output (G = K / group width, 4-byte
 *             aligned) that receives every group partial; a debug aid, slower.
 *
 * P[m][n][g] = sum over the K indices k of group g of q[m][k] * codes[n][k]
 * (exact int32).  Output:
 *   RAD_FMT_U8G256_BF16ROW: y = scale[m] * r[n] * 2^-7 * sum_g u8[n][g] * P[m][n][g]
 *   RAD_FMT_BF16G128:       y = scale[m] * 2^-7 * sum_g b[n][g] * P[m][n][g]
 * 2^-7 undoes H.H^T = 128 I, since both operands were rotated.  The f32 sum
 * order of the epilogue is unspecified.  M > RAD_GEMV_MAX_M returns
 * RAD_E_RANGE.  y and partials may not overlap each other or any input.
 */
int rad_w8a8_gemv(const int8_t *q, const float *scale, const rad_w8a8_weight *w, float *y,
                  int64_t M, int32_t *partials, rad_stream_t stream);

/*
 * rad_w8a8_gemm -- the same contraction and epilogue as rad_w8a8_gemv for any
 * M >= 0 (prefill sized batches), on int8 matrix cores.  Same arguments,
 * layouts and errors, without the limit on M.  For equal inputs both calls
 * produce identical partials.
 */
int rad_w8a8_gemm(const int8_t *q, const float *scale, const rad_w8a8_weight *w, float *y,
                  int64_t M, int32_t *partials, rad_stream_t stream);

/*
 * rad_w8a8_linear -- the whole layer on f32 activations (model card, table
 * rows "Weights" and "Activations"): rotate and quantise x exactly as
 * rad_quant_act_i8 with rotate = 1, then contract exactly as rad_w8a8_gemv
 * (M <= RAD_GEMV_MAX_M) or rad_w8a8_gemm (larger M).  The activation codes
 * and scales are written out as well as y, and all three equal, bit for bit,
 * what the separate calls produce.
 *
 *   x      f32 [M][K], 16-byte aligned, K <= RAD_QUANT_MAX_K.
 *   q      int8 [M][K] output, 16-byte aligned.
 *   scale  f32 [M] output, 4-byte aligned.
 *   w, y   as for rad_w8a8_gemv.
 *
 * For a single token (M == 1, K <= 20480) the three steps run as one kernel:
 * each workgroup rotates and quantises the token itself while its first
 * weight rows are already in flight, so no separate quantisation launch
 * stands in front of the weight stream.  Errors as for the separate calls;
 * q, scale and y may not overlap each other or any input (RAD_E_ALIAS).
 */
int rad_w8a8_linear(const float *x, int8_t *q, float *scale, const rad_w8a8_weight *w, float *y,
                    int64_t M, rad_stream_t stream);

/*
 * rad_quant_weight_i8 -- quantise float weights into either format above:
 * rotate, then round to nearest with a scale searched per group for least
 * error (model card "Qwen3.8-Flash-Next, IQR-V4 -- radiance container",
 * section "How this file was made": recipe rules with int8 codes, group 128,
 * bf16 scale, fwht128 transform, clamp=sym, rule=search, and table row
 * "Trunk": a scale per 128 columns searched for least error; model card
 * "Qwen3.8-27B IQ8R + DFlash2 -- radiance container", same section: int8
 * codes, group 256, u8 scale under a bf16 scale per row, clamp=sym,
 * rule=search.  Those cards then fit the codes by GPTQ, which needs
 * calibration Hessians; this call is the round-to-nearest form.)
 *
 *   W       f32 [N][K] weights (unrotated), 16-byte aligned.
 *   codes   int8 [N][K] output (packed 4-bit indices uint8 [N][K/2] for
 *           RAD_FMT_TBL4_BF16G128), 16-byte aligned.
 *   gscale  output: uint8 [N][K/256] (RAD_FMT_U8G256_BF16ROW) or bf16 bits
 *           [N][K/128] (the other two formats), 4-byte aligned.
 *   rscale  output bf16 bits [N] for RAD_FMT_U8G256_BF16ROW (4-byte aligned);
 *           must be NULL for RAD_FMT_BF16G128.
 *   N >= 0; K > 0, K % group width == 0, K <= RAD_QUANT_WEIGHT_MAX_K.
 *
 * Per row: w~ = W rotated as by rad_fwht128 (bit-identical).  Per group g with
 * amax = max |w~| over the group, candidate c = 0..15 aims at the scale
 * t_c = (amax * (64 - c) / 64) / 127 (f32 product, then f32 division):
 *   RAD_FMT_BF16G128: stored b = bf16(t_c) (nearest, ties to even), d = b;
 *   RAD_FMT_U8G256_BF16ROW: r = bf16((amax_row / 127) / 255) with amax_row
 *     = max |w~| over the row, stored u8 = clamp(rne(t_c / r), 1, 255),
 *     d = r * u8 (r = 0, an all-zero row, stores u8 = 1 and zero codes).
 *   RAD_FMT_TBL4_BF16G128: as the head format; each index picks the table
 *     entry nearest to w~ / d (f32 division), a tie going to the entry of
 *     smaller magnitude and 0 to +6 (d = 0: the index of +6); the error below
 *     uses d * entry.
 * Codes are clamp(rne(w~ / d), -127, 127) (f32 division; d = 0 gives 0).  The
 * candidate with the least f64 sum of (w~ - d * code)^2 over the group wins
 * (the sum taken as a balanced pairwise tree in index order; ties go to the
 * smaller c).  The result is deterministic and bit-identical across calls.
 * The outputs feed rad_w8a8_gemv / rad_w8a8_gemm directly.  No output may
 * overlap W or another output (RAD_E_ALIAS).  Non-finite weights give
 * unspecified results.
 */
int rad_quant_weight_i8(const float *W, int8_t *codes, void *gscale, uint16_t *rscale, int64_t N,
                        int64_t K, int32_t fmt, rad_stream_t stream);

/*
 * rad_w8a8_rescore -- the layer's output at candidate rows only (model card
 * "Qwen3.8-27B IQ8R + DFlash2 -- radiance container", table row "Speculator":
 * the drafter's top 32 candidates are rescored against the model's own int8
 * head, table row "Weights").
 *
 *   q, scale  activation codes [M][K] and scales [M] as for rad_w8a8_gemv.
 *   w         the weight descriptor (either format).
 *   ids       int32 [M][C] candidate rows per token, 4-byte aligned.
 *   y         f32 [M][C] output, 4-byte aligned.
 *   M, C >= 0, M * C < 2^33.
 *
 * y[m][j] equals the output rad_w8a8_gemv / rad_w8a8_gemm would give at row
 * ids[m][j] (same exact partials and epilogue; for the u8 format the very same
 * bits as the one-token path, rounded once from f64).  An id outside 0..N-1
 * reads nothing and gives NaN.  y may not overlap any input (RAD_E_ALIAS).
 */
int rad_w8a8_rescore(const int8_t *q, const float *scale, const rad_w8a8_weight *w, const int32_t *ids,
                     int64_t C, float *y, int64_t M, rad_stream_t stream);

/*
 * rad_kv_quant_i8 / rad_kv_dequant_i8 -- the int8 attention-cache codec
 * (model card "Qwen3.8-27B IQ8R + DFlash2 -- radiance container", section
 * "Serve": kv-cache-dtype i8 stores the attention cache as int8 with an f16
 * scale per token and head, half of bf16's bytes).  A row is one head's
 * vector of one token.
 *
 *   x       bf16 bits [rows][D] (encode input; decode output y), 16-byte aligned.
 *   codes   int8 [rows][D], 8-byte aligned.
 *   scale   f16 bits [rows], 2-byte aligned.
 *   rows >= 0; D is 64, 128 or 256 (other head sizes return RAD_E_SHAPE).
 *
 * Encode: s = f16(amax / 127) with amax the row's largest |x| (f32 division,
 * rounded to the nearest f16, ties to even, subnormals kept, saturating at
 * 65504); codes = clamp(rne(x / s), -127, 127) with s the stored value (f32
 * division), s = 0 giving zero codes.  Decode: y = bf16(code * s) (the product
 * is exact in f32; rounded to nearest even).  Outputs may not overlap inputs
 * or each other (RAD_E_ALIAS).  Non-finite inputs give unspecified results.
 */
int rad_kv_quant_i8(const uint16_t *x, int8_t *codes, uint16_t *scale, int64_t rows, int64_t D,
                    rad_stream_t stream);
int rad_kv_dequant_i8(const int8_t *codes, const uint16_t *scale, uint16_t *y, int64_t rows,
                      int64_t D, rad_stream_t stream);

/*
 * rad_probe_mfma_i8 -- a measurement aid, not a step of the layer: what the
 * int8 matrix cores sustain on given operand bytes.  Its callers are
 * benchmarks that price a contraction against the rate the chip reaches on
 * the same kind of data within its power budget (on random codes the core
 * clock stays well below its maximum).
 *
 * Launches `blocks` workgroups of 8 waves (one per CU at most: each takes
 * 96 KiB of LDS).  Block b copies its RAD_PROBE_BLOCK_BYTES of `src` (bytes
 * b * RAD_PROBE_BLOCK_BYTES ..) into LDS; each wave then runs `ksteps`
 * k-steps of a 64 x 64 tile, four v_mfma_i32_32x32x32_i8 a k-step (32 x 32
 * outputs over 32 of K each), on 16-byte fragments of those bytes.
 * lds_fed = 0: the fragments are loaded once and the wave alternates between
 * two sets; lds_fed = 1: every k-step's four fragments are read from LDS
 * first, as an LDS-staged GEMM with this wave tile must.  The int8 operations
 * performed are blocks * 8 * ksteps * 4 * 65536.
 *
 *   src     int8 [blocks * RAD_PROBE_BLOCK_BYTES], 16-byte aligned.
 *   out     int32 [blocks * 512]: each lane's 64 accumulator elements summed
 *           with 32-bit wrap-around.  With every src byte equal to c each
 *           word is 2048 * ksteps * c * c (mod 2^32).
 *   blocks  0 .. RAD_PROBE_MAX_BLOCKS; ksteps even, 0 .. RAD_PROBE_MAX_KSTEPS.
 *
 * Errors: RAD_E_SHAPE (negative or odd ksteps, negative blocks), RAD_E_RANGE
 * (sizes above the maxima, lds_fed not 0 or 1), RAD_E_NULL, RAD_E_ALIGN,
 * RAD_E_ALIAS (out overlaps src).
 */
#define RAD_PROBE_BLOCK_BYTES 98304
#define RAD_PROBE_MAX_BLOCKS 65536
#define RAD_PROBE_MAX_KSTEPS 1073741824
int rad_probe_mfma_i8(const int8_t *src, int32_t *out, int64_t blocks, int64_t ksteps, int lds_fed,
                      rad_stream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *rad_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* RAD_H */
