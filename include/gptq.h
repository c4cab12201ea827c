/*
 * gptq.h -- C ABI of the GPTQ per-layer quantization solver for AMD gfx950.
 *
 * The solver finds, for one linear layer with weights W [d_row x d_col] and
 * calibration inputs X [n x d_col], integer codes on an asymmetric k-bit
 * min/max grid (one grid per row, or one per group of g consecutive columns)
 * that approximately minimise ||W X^T - What X^T||^2 (the layer objective of
 * the itwiki "GPTQ" page, section "문제 설정").  It runs in three calls:
 *
 *   gptq_hessian_accumulate   H += 2 X_c^T X_c for each calibration chunk
 *   gptq_prepare_hinv         damping, then U = upper Cholesky factor of H^-1
 *   gptq_quantize_layer       the lazy-batch column loop; codes, grid, error
 *
 * Conventions shared by every call:
 *   - All matrices are row-major.  A "leading dimension" (ld_*) is the
 *     distance in elements between consecutive rows and must be >= the row
 *     width.
 *   - Pointers marked [device] are device (HBM) addresses on the current HIP
 *     device; [host] pointers are host addresses.  The caller owns every
 *     buffer; the library allocates no device memory.  Its only state kept
 *     between calls is a host-side memo, one per calling thread, of the
 *     Hessian launch's work-group tile order for the last tile count seen (a
 *     pure function of the shape, so no result depends on it).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on that stream and returns; results are valid once the
 *     stream has been synchronised.  Calls on different streams are
 *     independent; the caller orders calls that share buffers.
 *   - `ws` is a caller-provided device workspace of at least the size that the
 *     matching *_workspace_size() query returns for the same shape.  Its
 *     contents are scratch on entry and exit.
 *   - The return value reports argument validation (done on the host, before
 *     anything is enqueued) and launch errors.  Numerical failures are
 *     reported through device words (`info`, NaN error) documented per call.
 */
#ifndef GPTQ_H_
#define GPTQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_ERR_NULL_POINTER = 1,    /* a required pointer is NULL            */
  GPTQ_ERR_BAD_SIZE = 2,        /* a size is negative or zero             */
  GPTQ_ERR_BAD_LEADING_DIM = 3, /* ld_* smaller than the row width        */
  GPTQ_ERR_BAD_DTYPE = 4,       /* element type not GPTQ_F32 / GPTQ_F16   */
  GPTQ_ERR_BAD_BITS = 5,        /* bits outside [2, 8]                    */
  GPTQ_ERR_BAD_BLOCK = 6,       /* block_size not one of 16, 32, 64, 128  */
  GPTQ_ERR_BAD_GROUP = 7,       /* group_size not 0 / 16k aligned with B  */
  GPTQ_ERR_WORKSPACE = 8,       /* ws NULL or smaller than the query      */
  GPTQ_ERR_BAD_DAMP = 9,        /* percdamp negative or not finite        */
  GPTQ_ERR_LAUNCH = 10,         /* a HIP launch or runtime call failed    */
  GPTQ_ERR_TOO_LARGE = 11,      /* a size exceeds the library's limits    */
  GPTQ_ERR_SCRATCH = 12         /* shape too large for the no-allocation  */
                                /* entry point's fixed workspace          */
} gptq_status;

typedef enum {
  GPTQ_F32 = 0, /* IEEE binary32 */
  GPTQ_F16 = 1  /* IEEE binary16 */
} gptq_dtype;

/*
 * Hessian accumulation: H += 2 * X^T X   (blog "GPTQ를 밑바닥부터 구현하며 배운
 * 것들", section 3, formula H = 2 X^T X; itwiki "GPTQ", minimal implementation).
 *
 *   H      [device] float [d_col x d_col], row-major, leading dimension d_col.
 *          Accumulated in place, both triangles written (H stays exactly
 *          symmetric).  The caller zeroes H before the first chunk; the call
 *          may be repeated for any number of chunks (the sum is over all rows
 *          of all chunks -- a sum, not a mean).
 *   d_col  number of input features (columns of X, rows/cols of H); >= 1.
 *   X      [device] n_rows x d_col chunk, row-major, element type x_dtype,
 *          leading dimension ld_x >= d_col.  Read only.
 *   n_rows rows in this chunk; 0 is a no-op that returns GPTQ_OK.
 *   ws     [device] workspace, >= gptq_hessian_accumulate_workspace_size().
 *
 * Products of fp16 values are exact in fp32; accumulation is fp32 on the
 * matrix cores, split over row ranges whose partial sums are added in a fixed
 * order, so results are bitwise reproducible for a given shape.
 */
gptq_status gptq_hessian_accumulate(float* H, int64_t d_col, const void* X, int32_t x_dtype,
                                    int64_t n_rows, int64_t ld_x, void* ws, size_t ws_bytes,
                                    void* stream);
size_t gptq_hessian_accumulate_workspace_size(int64_t d_col, int64_t n_rows, int32_t x_dtype);

/*
 * Inverse-Hessian factor (itwiki "GPTQ": three-changes table, change 3;
 * Algorithm 1, first line; minimal implementation, damping and factor lines):
 *
 *   lambda = percdamp * mean(diag H);   H_l = H + lambda * I
 *   U      = upper-triangular factor with U^T U = H_l^-1 and diag(U) > 0
 *
 * computed as U = Ut^-1 where H_l = Ut Ut^T, Ut upper (the reverse-order
 * Cholesky factor): the Cholesky runs in fp64, the triangular inverse in fp32.
 *
 *   H          [device] float [d_col x d_col] row-major; read only (the
 *              undamped H is preserved for the error of gptq_quantize_layer).
 *   percdamp   damping fraction (0.01 in the pages); finite and >= 0.
 *   U          [device] float [d_col x d_col] row-major output; the strictly
 *              lower triangle is written as zeros.
 *   lambda_out [device] one float: the lambda used.
 *   info       [device] one int32: 0 on success; k + 1 if H_l is not
 *              positive definite, with k the first failing pivot in the
 *              natural column order.  U is unspecified when info != 0.
 *   ws         [device] workspace, >= gptq_prepare_hinv_workspace_size().
 */
gptq_status gptq_prepare_hinv(const float* H, int64_t d_col, float percdamp, float* U,
                              float* lambda_out, int32_t* info, void* ws, size_t ws_bytes,
                              void* stream);
size_t gptq_prepare_hinv_workspace_size(int64_t d_col);

/*
 * Lazy-batch quantization loop (itwiki "GPTQ", Algorithm 1 and the minimal
 * implementation; group quantization from the "practical variants" section),
 * natural column order:
 *
 *   grid: scale = max(max - min, 1e-8) / (2^bits - 1), zero = round(-min/scale)
 *         per row from W0 (group_size == 0), or per group of group_size
 *         columns from the then-current weights when the group's first column
 *         is reached;
 *   for each block [i, i + block_size):
 *     for each column j: c = clamp(round(w_j / scale) + zero, 0, 2^bits - 1)
 *                        e = (w_j - scale * (c - zero)) / U[j, j]
 *                        W[:, j:i+B] -= e * U[j, j:i+B]
 *     W[:, i+B:] -= E * U[i:i+B, i+B:]
 *   round() is round-half-to-even.
 *
 *   W0         [device] d_row x d_col weights, element type w_dtype, leading
 *              dimension ld_w >= d_col; read only (the fp32 working copy
 *              lives in ws).
 *   U          [device] float [d_col x d_col], the factor from
 *              gptq_prepare_hinv (only the upper triangle is read).
 *   lambda     [device] one float from gptq_prepare_hinv, or NULL.
 *   bits       2..8.
 *   group_size 0 (one grid per row) or a positive multiple of 16 with
 *              group_size % block_size == 0 or block_size % group_size == 0
 *              (so a group never starts inside a block except at a
 *              multiple of its size, and its parameters come from fully
 *              updated weights).
 *   block_size 16, 32, 64 or 128 (the pages use 128); the last block may be
 *              partial.
 *   codes      [device] uint8 [d_row x d_col] row-major output codes.
 *   scales     [device] float [d_row x n_groups] output, n_groups =
 *              ceil(d_col / group_size) or 1.
 *   zeros      [device] int32 [d_row x n_groups] output zero-points.
 *   out_err    [device] one double: ||X (W0 - What)^T||^2 with What =
 *              scale * (codes - zero), evaluated as 1/2 ||E||^2 -
 *              lambda/2 ||W0 - What||^2 from the scaled errors E of the loop
 *              (exact for the undamped H given U of the damped one); when
 *              lambda is NULL it is 1/2 ||E||^2 (the damped objective).  NaN
 *              or Inf if an input was not finite.
 *   ws         [device] workspace, >= gptq_quantize_layer_workspace_size().
 */
gptq_status gptq_quantize_layer(const void* W0, int32_t w_dtype, int64_t d_row, int64_t d_col,
                                int64_t ld_w, const float* U, const float* lambda, int32_t bits,
                                int64_t group_size, int64_t block_size, uint8_t* codes,
                                float* scales, int32_t* zeros, double* out_err, void* ws,
                                size_t ws_bytes, void* stream);
size_t gptq_quantize_layer_workspace_size(int64_t d_row, int64_t d_col, int64_t block_size);

/*
 * gptq_quantize_layer without a workspace argument, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, results and kernels
 * as gptq_quantize_layer (bitwise the same outputs) minus ws / ws_bytes; the
 * call allocates nothing.  Its workspace is a fixed device array of
 * GPTQ_NOALLOC_SCRATCH_BYTES bytes inside the library, one per device, which
 * each device holds from the library's load until the process ends.
 *
 *   Limit: shapes with gptq_quantize_layer_workspace_size(d_row, d_col,
 *          block_size) > GPTQ_NOALLOC_SCRATCH_BYTES are rejected with
 *          GPTQ_ERR_SCRATCH before anything is enqueued (4096 x 4096 with
 *          blocks of 128 fits).
 *   Races: every call on one device shares that device's array, which keeps
 *          the last call's contents (each call clears what it needs zeroed
 *          with a kernel).  Calls that can overlap on one device -- on
 *          different streams, or from different host threads without
 *          ordering -- race on it; order them on one stream.
 *   The first call on a device looks up the array's address there
 *   (hipGetSymbolAddress, under a lock); later calls reuse it.
 */
#define GPTQ_NOALLOC_SCRATCH_BYTES (96ull << 20)
gptq_status gptq_quantize_layer_noalloc(const void* W0, int32_t w_dtype, int64_t d_row,
                                        int64_t d_col, int64_t ld_w, const float* U,
                                        const float* lambda, int32_t bits, int64_t group_size,
                                        int64_t block_size, uint8_t* codes, float* scales,
                                        int32_t* zeros, double* out_err, void* stream);

/*
 * Act-order (itwiki "GPTQ", section "실무 변형" (practical variants): an option of
 * later implementations quantizes the columns with the largest Hessian
 * diagonal -- the largest input activations -- first; combined with groups it
 * needs a column-to-group map).  Three calls mirror the natural-order ones:
 *
 * gptq_act_order_perm: the quantization order.
 *   H      [device] float [d_col x d_col] (only the diagonal is read).
 *   perm   [device] int32 [d_col] output: position i quantizes original column
 *          perm[i].  Columns by descending diag(H) compared as fp32; equal
 *          diagonals keep ascending column index; a NaN diagonal counts as
 *          -inf.  Always a permutation of 0 .. d_col-1.  Needs no workspace.
 *
 * gptq_prepare_hinv_perm: as gptq_prepare_hinv for the Hessian with rows and
 *   columns in that order, Hp[a][b] = H[perm[a]][perm[b]] (H is not modified
 *   and not copied).  U is the factor of the damped Hp, in the quantization
 *   order; info's pivot index counts positions of that order.  lambda is the
 *   same as for H.  perm [device] int32 [d_col], a permutation of
 *   0 .. d_col-1 (entries out of range are clamped, giving unspecified
 *   results but no out-of-bounds access).  Workspace as gptq_prepare_hinv.
 *
 * gptq_quantize_layer_perm: as gptq_quantize_layer with the columns of W0
 *   quantized in the order perm, using the U of gptq_prepare_hinv_perm.
 *   codes  are written in the ORIGINAL column order.
 *   groups are runs of group_size consecutive positions of the quantization
 *          order: scales / zeros [d_row x n_groups] are indexed by that run,
 *          and original column j belongs to run
 *   g_idx  [device] int32 [d_col] output: g_idx[j] = (position of j) /
 *          group_size (0 for every column when group_size == 0).
 *   out_err is the same order-free quantity as in gptq_quantize_layer.
 *   Workspace as gptq_quantize_layer.
 */
gptq_status gptq_act_order_perm(const float* H, int64_t d_col, int32_t* perm, void* stream);
gptq_status gptq_prepare_hinv_perm(const float* H, int64_t d_col, const int32_t* perm,
                                   float percdamp, float* U, float* lambda_out, int32_t* info,
                                   void* ws, size_t ws_bytes, void* stream);
gptq_status gptq_quantize_layer_perm(const void* W0, int32_t w_dtype, int64_t d_row,
                                     int64_t d_col, int64_t ld_w, const float* U,
                                     const float* lambda, const int32_t* perm, int32_t bits,
                                     int64_t group_size, int64_t block_size, uint8_t* codes,
                                     float* scales, int32_t* zeros, int32_t* g_idx,
                                     double* out_err, void* ws, size_t ws_bytes, void* stream);

/*
 * Packed codes and the dequantizing product -- the consumer of the codes (itwiki
 * "GPTQ", section "결과": kernels that unpack the weights on the fly).
 *
 * Layout (packed): each row is a little-endian bitstream of `bits`-bit fields
 * in 32-bit words; position i of a row occupies bits [bits*i, bits*i + bits)
 * of the stream (bit b of the stream = bit b % 32 of word b / 32).  Rows are
 * padded to whole chunks of 32 codes (a chunk is exactly `bits` words);
 * gptq_packed_words_per_row() = ceil(d_col / 32) * bits.  bits is 2, 3, 4 or 8.
 *
 * gptq_pack_codes: codes [device] uint8 [d_row x d_col] (leading dimension
 *   ld_codes >= d_col, values < 2^bits; higher bits are dropped) -> packed
 *   [device] uint32 [d_row x ld_packed], ld_packed >= words per row.  perm:
 *   NULL, or [device] int32 [d_col] with position i holding column perm[i]
 *   (pass the act-order permutation so that groups of positions are
 *   contiguous; entries out of range are clamped).  Needs no workspace.
 *
 * gptq_dequant_matmul: Y [device] float [m x d_row] (leading dimension ld_y >=
 *   d_row) = X What^T for 1 <= m <= 8 rows of X [device] [m x d_col]
 *   (x_dtype GPTQ_F16 or GPTQ_F32, leading dimension ld_x >= d_col), with
 *     What by position i = scales[r][g] * (code_i - zeros[r][g]),
 *     g = i / group_size (0 when group_size == 0; group_size a multiple of 16),
 *   and position i multiplying column perm[i] of X (or column i when perm is
 *   NULL).  scales / zeros as written by gptq_quantize_layer(_perm).  fp32
 *   accumulation; no workspace.
 */
int64_t gptq_packed_words_per_row(int64_t d_col, int32_t bits);
gptq_status gptq_pack_codes(const uint8_t* codes, int64_t d_row, int64_t d_col, int64_t ld_codes,
                            int32_t bits, const int32_t* perm, uint32_t* packed, int64_t ld_packed,
                            void* stream);
gptq_status gptq_dequant_matmul(const uint32_t* packed, int64_t ld_packed, int32_t bits,
                                const float* scales, const int32_t* zeros, int64_t group_size,
                                const int32_t* perm, int64_t d_row, int64_t d_col, const void* X,
                                int32_t x_dtype, int64_t m, int64_t ld_x, float* Y, int64_t ld_y,
                                void* stream);

/*
 * Dequantized weights -- What as the model uses it between quantized layers
 * (itwiki "GPTQ", algorithm section: the loop's output is What = scale * (q - zero)
 * on the grid; the model-level procedure feeds the quantized block's outputs on).
 *
 * gptq_dequantize: out [device] [d_row x d_col] (out_dtype GPTQ_F32 or GPTQ_F16,
 *   leading dimension ld_out >= d_col) = scales[r][g] * (codes[r][j] - zeros[r][g]),
 *   computed in fp32 and rounded once to out_dtype.  codes [device] uint8
 *   [d_row x ld_codes]; scales / zeros [device] [d_row x n_groups] as written by
 *   gptq_quantize_layer(_perm), n_groups = ceil(d_col / group_size) (1 when
 *   group_size == 0).  g: g_idx[j] when g_idx ([device] int32 [d_col], the
 *   act-order column-to-group map; entries clamped to [0, n_groups)) is given,
 *   else j / group_size, else 0.  No workspace.
 */
gptq_status gptq_dequantize(const uint8_t* codes, int64_t d_row, int64_t d_col, int64_t ld_codes,
                            const float* scales, const int32_t* zeros, int64_t group_size, const int32_t* g_idx,
                            void* out, int32_t out_dtype, int64_t ld_out, void* stream);

/*
 * Two-sided adaptive rounding (blog.secrett2633.cloud, "[논문리뷰] GPTQ-2D:
 * Cubic-Time Two-Sided Adaptive Rounding", sections 1-3): round X [m x n] on one
 * asymmetric k-bit grid so as to minimise ||A (Z - X) B||_F^2, entry by entry with
 * error feedback, swept by anti-diagonals.
 *
 * gptq2d_quantize: X [device] [m x n] (x_dtype GPTQ_F32 or GPTQ_F16, leading
 *   dimension ldx >= n); U_Q [device] fp32 [m x m] and U_P [device] fp32 [n x n]:
 *   upper factors with U_Q^T U_Q = (A^T A)^-1 and U_P^T U_P = (B B^T)^-1 (for
 *   example gptq_prepare_hinv of A^T A and of B B^T; only the upper triangles are
 *   read); bits in [2, 8].  Writes codes [device] uint8 [m x ld_codes] (ld_codes >=
 *   n), scale [device] one float and zero [device] one int32 (the grid: scale =
 *   max(max X - min X, 1e-8) / (2^bits - 1), zero = round(-min X / scale); What =
 *   scale * (code - zero)) and out_err [device] one double: sum of the squared
 *   scaled errors, which is ||A (What - X) B||_F^2 for the A^T A and B B^T the
 *   factors come from.  Workspace: gptq2d_quantize_workspace_size(m, n) bytes
 *   (M, m x n fp32, and per-tile partial sums); m + n - 1 launches of 32 x 32 tiles.
 */
size_t gptq2d_quantize_workspace_size(int64_t m, int64_t n);
gptq_status gptq2d_quantize(const void* X, int32_t x_dtype, int64_t m, int64_t n, int64_t ldx, const float* U_Q,
                            const float* U_P, int32_t bits, uint8_t* codes, int64_t ld_codes, float* scale,
                            int32_t* zero, double* out_err, void* ws, size_t ws_bytes, void* stream);

/*
 * Per-launch timing of the quantization loop -- a measurement aid, off by
 * default.  gptq_launch_timing(1) switches it on for the calling host thread:
 * every later gptq_quantize_layer / _perm / _noalloc call made from that
 * thread brackets each of its in-block panel launches (kind 0) and each
 * out-of-block product launch (kind 1) with a pair of HIP events recorded on
 * the call's stream (so it also times any gaps the stream has between them),
 * and notes the launch's algorithmic work.  gptq_launch_timing(0) switches it
 * off; events already recorded stay readable.
 *
 * gptq_launch_timing_read(kind, ms, launches, work) waits for the recorded
 * events of that kind, returns [host] their summed duration in milliseconds,
 * the number of launches and their summed work, and forgets them.  Work of a
 * panel launch (kind 0): the bytes the block's step must move at least --
 * W block read (4 d_row w), its scaled errors E written (4 d_row w), codes
 * written (d_row w), U's diagonal block read (4 w^2) and the grid parameters of
 * groups starting in the block written (8 d_row per group), w the block width.
 * Work of a product launch (kind 1): 2 M N K flop.  Uses HIP events, created on
 * first use and kept per thread for reuse; not for the no-allocation path's
 * callers that forbid event creation.
 */
gptq_status gptq_launch_timing(int32_t enable);
gptq_status gptq_launch_timing_read(int32_t kind, double* ms, int64_t* launches, double* work);

/* [host] static description of a status code; never NULL. */
const char* gptq_status_string(int32_t status);
/* [host] library version string, e.g. "gptq-gfx950 0.1.0". */
const char* gptq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_H_ */
