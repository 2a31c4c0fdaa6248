/*
 * fp8q.h -- C ABI of the fine-grained FP8 quantization and block-scaled FP8
 * GEMM library for AMD Instinct MI355X (gfx950).
 *
 * The method is the FP8 mixed-precision scheme quoted on the pages:
 *   - GEMM operands are E4M3 on all tensors (page "Deepseek Ai News Expert
 *     Interview", passage adopting E4M3 on all tensors);
 *   - activations are grouped and scaled per 1x128 tile (per token per 128
 *     channels) and weights per 128x128 block (per 128 input channels per 128
 *     output channels) (page dssusan.co.kr Q&A board, passage on Figure 7(a));
 *   - the three GEMMs of a Linear operator -- Fprop, Dgrad and Wgrad -- all
 *     consume FP8 (same page, passage on Figure 6);
 *   - partial products are promoted to full FP32 accumulation once per
 *     128-element interval along K, where the per-group scales are applied
 *     (page "Deepseek Ai News Expert Interview", passage on copying partial
 *     results to FP32 registers; page inprokorea.com free board, passage on
 *     the 128-element, four-WGMMA accumulation interval; page "Is aI Hitting
 *     a Wall?", passage on the dequantization overhead);
 *   - the GEMMs take FP8 tensors and produce BF16 or FP32 (page "Deepseek Ai
 *     News Expert Interview", passage on GEMM inputs and outputs);
 *   - MoE activations are quantized before dispatch, compatible with the FP8
 *     Fprop of the expert up-projections (page "Eliminate Deepseek Ai News For
 *     Good", passage on quantizing before the MoE up-projections).
 *
 * Numeric contract (readings where the pages are silent):
 *   E4M3 is OCP E4M3FN (bias 7, no infinities, largest finite 448). For each
 *   group: amax = max |x| (exact), scale s = fl32(amax / 448) (IEEE binary32
 *   division), code q = E4M3(fl32(x / s)) rounded to nearest, ties to the even
 *   code, saturating to +-448; an all-zero group stores s = 0 and signed-zero
 *   codes; the sign bit of q is the sign of x. Dequantized value = dec(q) * s.
 *   bf16 and fp32 subnormals are honoured. NaN/Inf inputs are out of contract
 *   (the kernels finish, the output is unspecified).
 *
 * Conventions for every entry point:
 *   - all data pointers are device memory (HBM) owned by the caller; the
 *     library never allocates, frees or synchronizes, and inputs are const
 *     (its one device array is the scratch of fp8_grouped_gemm_noalloc);
 *   - bf16 tensors are passed as their uint16 bit patterns; FP8 tensors as
 *     uint8 E4M3 codes; matrices are row-major with a leading dimension (ld)
 *     counted in elements;
 *   - work is enqueued asynchronously on `stream` (NULL = the default stream);
 *     the call returns once the launch is enqueued;
 *   - arguments are validated on the host before anything is launched; on any
 *     error nothing is launched and nothing is written;
 *   - calls are thread-safe and keep no state besides the last HIP error code
 *     (and fp8_grouped_gemm_noalloc's per-device scratch address);
 *   - FP8Q_DEBUG=1 in the environment adds host-side checks of the device
 *     arrays the grouped GEMMs trust (fp8_grouped_gemm, fp8_grouped_gemm_wgrad):
 *     they are copied to the host on `stream`, which is then synchronized, and a
 *     contract violation returns FP8Q_ERR_SHAPE before anything is launched.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
#define FP8Q_OK         0 /* launched (or nothing to do)                          */
#define FP8Q_ERR_NULL   1 /* a required pointer is NULL                           */
#define FP8Q_ERR_SHAPE  2 /* negative size, bad divisibility, ld below the width  */
#define FP8Q_ERR_ALIGN  3 /* a pointer or leading dimension breaks the alignment  */
#define FP8Q_ERR_ENUM   4 /* an enum argument is out of range                     */
#define FP8Q_ERR_HIP    5 /* the HIP launch failed; see fp8q_last_hip_error()     */

/* ---------------------------------------------------------------- enums */
#define FP8Q_TILE_1x128       0 /* one scale per row per 128 consecutive columns  */
#define FP8Q_TILE_128x1       1 /* one scale per column per 128 consecutive rows  */
#define FP8Q_BSCALE_BLOCK128  0 /* B scales per 128x128 block: [ceil(n/128)][ld]  */
#define FP8Q_BSCALE_ROW128    1 /* B scales per (128-slab, row): [k/128][ld]      */
#define FP8Q_OUT_BF16         0 /* output rounded to bf16, nearest-even           */
#define FP8Q_OUT_F32          1 /* output as fp32                                 */

/*
 * Limits of the GEMM entry points (fp8_gemm, fp8_grouped_gemm,
 * fp8_grouped_gemm_wgrad, fp8_gemm_mx, fp8_gemm_tensor). A block addresses
 * its operand tiles and their scales through buffer ranges of at most
 * 2^31 - 1 bytes from the tile origin, so:
 *   lda, ldb <= FP8Q_MAX_GEMM_LD (elements = bytes of FP8 codes);
 *   every scale array spans fewer than FP8Q_MAX_SCALE_SPAN floats:
 *   (k/128) * ld_as, and (k/128) * ld_bs (per-row B scales) or
 *   ceil(n/128) * ld_bs (128x128 B block scales).
 * Larger values return FP8Q_ERR_SHAPE before anything is launched.
 */
#define FP8Q_MAX_GEMM_LD      8388480LL    /* 2^23 - 128 */
#define FP8Q_MAX_SCALE_SPAN   536870912LL  /* 2^29 floats (2 GiB) */

/*
 * fp8_quantize_act -- fine-grained activation quantization.
 *
 * Tiles: page dssusan.co.kr Q&A board, passage on Figure 7(a) (1x128 tiles,
 * per token per 128 channels); the 128x1 token tiles for the Wgrad operands
 * are a reading (the Wgrad GEMM in FP8: same page, passage on Figure 6).
 *
 * x       bf16 input [rows][ld_x], ld_x >= cols.
 * tiling  FP8Q_TILE_1x128: cols % 128 == 0. Writes codes q[rows][ld_q]
 *           (ld_q >= cols, same layout as x) and scales scale[cols/128][ld_s]
 *           with ld_s >= rows (slab-major: one row of scales per 128 columns).
 *         FP8Q_TILE_128x1: rows % 128 == 0, cols % 8 == 0. Writes codes
 *           TRANSPOSED, q[cols][ld_q] with ld_q >= rows (row c of q holds
 *           column c of x, token-contiguous, ready to be a K-contiguous GEMM
 *           operand), and scales scale[rows/128][ld_s] with ld_s >= cols.
 * Alignment: x and q 16-byte aligned; ld_x % 8 == 0; ld_q % 16 == 0; scale
 *         4-byte aligned.
 * rows == 0 or cols == 0: returns FP8Q_OK without launching.
 * Errors: FP8Q_ERR_NULL, FP8Q_ERR_SHAPE, FP8Q_ERR_ALIGN, FP8Q_ERR_ENUM,
 *         FP8Q_ERR_HIP.
 */
int fp8_quantize_act(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x, int tiling,
                     uint8_t *q, int64_t ld_q, float *scale, int64_t ld_s, hipStream_t stream);

/*
 * fp8_quantize_act_scatter -- quantize before the MoE dispatch.
 *
 * Page "Eliminate Deepseek Ai News For Good", passage on quantizing the
 * activations into FP8 before the MoE dispatch, compatible with the FP8 Fprop
 * of the expert up-projections; 1x128 tiles as in fp8_quantize_act. Each
 * token row of x is quantized once; its codes and scales are stored to every
 * row of the expert-sorted layout (the A operand of fp8_grouped_gemm) that
 * the routing sends it to. Row r of q then equals what fp8_quantize_act
 * writes for the token routed to r (quantization commutes with row moves).
 *
 * x        bf16 tokens [tokens][ld_x], ld_x >= cols, cols % 128 == 0.
 * topk     destinations per token, 1..8.
 * dst_rows device int32 [tokens][topk]: the destination row in q of token t's
 *          k-th route, or -1 (not routed to this layout). Values >= m_total
 *          are ignored. Each destination row should be named once; a row
 *          named by several tokens ends up with one of their codes.
 * q        codes [m_total][ld_q], ld_q >= cols. scale [cols/128][ld_s] with
 *          ld_s >= m_total. Rows named by no route (the 128-row padding of
 *          each expert segment) are not written; fp8_grouped_gemm never lets
 *          their contents reach a stored output.
 * Alignment: x and q 16-byte aligned; ld_x % 8 == 0; ld_q % 16 == 0; scale
 *          and dst_rows 4-byte aligned.
 * tokens, cols or m_total == 0: returns FP8Q_OK without launching.
 * Errors: FP8Q_ERR_NULL, FP8Q_ERR_SHAPE (also topk outside 1..8),
 *         FP8Q_ERR_ALIGN, FP8Q_ERR_HIP.
 */
int fp8_quantize_act_scatter(const uint16_t *x, int64_t tokens, int64_t cols, int64_t ld_x,
                             int32_t topk, const int32_t *dst_rows, int64_t m_total, uint8_t *q,
                             int64_t ld_q, float *scale, int64_t ld_s, hipStream_t stream);

/*
 * fp8_quantize_weight -- 128x128 block weight quantization.
 *
 * Blocks: page dssusan.co.kr Q&A board, passage on Figure 7(a) (per 128 input
 * channels per 128 output channels). The optional transposed copy feeds the
 * Dgrad GEMM (same page, passage on Figure 6); block quantization commutes
 * with transposition, so it is the exact transpose of q and scale.
 *
 * w        bf16 weight [n][ld_w] (n output channels x k input channels),
 *          n % 128 == 0, k % 128 == 0, ld_w >= k.
 * q        codes [n][ld_q], ld_q >= k; scale [n/128][ld_s], ld_s >= k/128.
 * q_t      NULL, or the transposed codes [k][ld_qt] with ld_qt >= n; then
 *          scale_t [k/128][ld_st] with ld_st >= n/128 must be non-NULL.
 * Alignment: w, q, q_t 16-byte aligned; ld_w % 8 == 0; ld_q, ld_qt % 16 == 0.
 * n == 0 or k == 0: returns FP8Q_OK without launching.
 * Errors: FP8Q_ERR_NULL, FP8Q_ERR_SHAPE, FP8Q_ERR_ALIGN, FP8Q_ERR_HIP.
 */
int fp8_quantize_weight(const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                        uint8_t *q, int64_t ld_q, float *scale, int64_t ld_s,
                        uint8_t *q_t, int64_t ld_qt, float *scale_t, int64_t ld_st,
                        hipStream_t stream);

/*
 * fp8_quantize_act_weight -- a Linear layer's two GEMM operands in one launch:
 * fp8_quantize_act with FP8Q_TILE_1x128 on x, and fp8_quantize_weight on w
 * (with the transposed copy when wq_t is given). Same groups, passages,
 * layouts, alignment rules and results, bit for bit. One launch instead of
 * two saves a launch gap and overlaps the two kernels' ramps and tails.
 * Either operand may be empty (rows or cols == 0; n or k == 0): it is then
 * skipped and its pointers are not read. x and w may overlap (both are only
 * read). The two halves of the launch run concurrently, so no output of the
 * activation (q, scale) may share a byte with an output of the weight (wq,
 * wscale, wq_t, wscale_t).
 * Errors: those of the two calls (FP8Q_ERR_NULL, FP8Q_ERR_SHAPE,
 *         FP8Q_ERR_ALIGN, FP8Q_ERR_HIP); FP8Q_ERR_SHAPE also when an
 *         activation output overlaps a weight output.
 */
int fp8_quantize_act_weight(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *q,
                            int64_t ld_q, float *scale, int64_t ld_s, const uint16_t *w, int64_t n,
                            int64_t k, int64_t ld_w, uint8_t *wq, int64_t ld_wq, float *wscale,
                            int64_t ld_ws, uint8_t *wq_t, int64_t ld_wqt, float *wscale_t, int64_t ld_wst,
                            hipStream_t stream);

/*
 * fp8_quantize_act_128x1_pair -- the two Wgrad operands in one launch:
 * fp8_quantize_act with FP8Q_TILE_128x1 on x0[tokens][cols0] and on
 * x1[tokens][cols1] (dY and X of one token count), page dssusan.co.kr Q&A
 * board, Figure 6 (Wgrad in FP8). Same tiles, layouts (q transposed
 * [cols][ld_q], scale [tokens/128][ld_s]), alignment rules and results, bit
 * for bit, as the two separate calls. One launch instead of two removes a
 * launch gap and overlaps the two kernels' ramps and tails.
 * An operand with cols == 0 (or tokens == 0) is skipped and its pointers
 * are not read. The two halves of the launch run concurrently, so no output
 * of one operand (q, scale) may share a byte with an output of the other.
 * Errors: those of fp8_quantize_act (FP8Q_ERR_NULL, FP8Q_ERR_SHAPE,
 *         FP8Q_ERR_ALIGN, FP8Q_ERR_HIP); FP8Q_ERR_SHAPE also when the outputs
 *         of the two operands overlap.
 */
int fp8_quantize_act_128x1_pair(int64_t tokens, const uint16_t *x0, int64_t cols0, int64_t ld_x0, uint8_t *q0,
                                int64_t ld_q0, float *scale0, int64_t ld_s0, const uint16_t *x1, int64_t cols1,
                                int64_t ld_x1, uint8_t *q1, int64_t ld_q1, float *scale1, int64_t ld_s1,
                                hipStream_t stream);

/*
 * fp8_quantize_act_128x1_retile -- the two Wgrad operands in one launch when
 * X comes from the FP8 activation cache: fp8_quantize_act with
 * FP8Q_TILE_128x1 on x0[tokens][cols0] (dY), and fp8_retile_act_128x1 on the
 * cached 1x128 codes xq[tokens][ld_xq] and scales xs[cols1/128][ld_xs] of X
 * (page "Is aI Hitting a Wall?", passage on keeping activations in FP8 for
 * the backward pass; page dssusan.co.kr Q&A board, Figure 6). Same tiles,
 * layouts, alignment rules and results, bit for bit, as the two calls; one
 * launch instead of two.
 * An operand with no columns (or tokens == 0) is skipped and its pointers
 * are not read. The two halves of the launch run concurrently, so no output
 * of one operand (q, scale) may share a byte with an output of the other.
 * Errors: those of the two calls (FP8Q_ERR_NULL, FP8Q_ERR_SHAPE,
 *         FP8Q_ERR_ALIGN, FP8Q_ERR_HIP); FP8Q_ERR_SHAPE also when the outputs
 *         of the two operands overlap.
 */
int fp8_quantize_act_128x1_retile(int64_t tokens, const uint16_t *x0, int64_t cols0, int64_t ld_x0, uint8_t *q0,
                                  int64_t ld_q0, float *scale0, int64_t ld_s0, const uint8_t *xq, int64_t cols1,
                                  int64_t ld_xq, const float *xs, int64_t ld_xs, uint8_t *q1, int64_t ld_q1,
                                  float *scale1, int64_t ld_s1, hipStream_t stream);

/*
 * fp8_quantize_weight_grouped -- fp8_quantize_weight over several weight
 * matrices of one shape (say the experts of an MoE layer) in one launch.
 *
 * Group e reads w + e*stride_w and writes q + e*stride_q, scale +
 * e*stride_s and, when q_t is given, q_t + e*stride_qt and scale_t +
 * e*stride_st (strides in elements), each exactly as fp8_quantize_weight
 * with the same n, k and leading dimensions. One launch for all experts
 * instead of one each; the per-expert transposed copies (Dgrad's B) come out
 * contiguous. Blocks and passages as fp8_quantize_weight.
 *
 * groups   number of matrices, >= 0 (0: returns FP8Q_OK).
 * Strides: all >= 0. The inputs may overlap (they are only read); for
 *          groups > 1 the outputs may not: stride_q >= n*ld_q,
 *          stride_s >= (n/128)*ld_s and, with q_t, stride_qt >= k*ld_qt,
 *          stride_st >= (k/128)*ld_st.
 * Alignment: as fp8_quantize_weight, and stride_w % 8 == 0,
 *          stride_q % 16 == 0, stride_qt % 16 == 0.
 * Errors: FP8Q_ERR_NULL, FP8Q_ERR_SHAPE, FP8Q_ERR_ALIGN, FP8Q_ERR_HIP.
 */
int fp8_quantize_weight_grouped(int32_t groups, const uint16_t *w, int64_t n, int64_t k, int64_t ld_w,
                                int64_t stride_w, uint8_t *q, int64_t ld_q, int64_t stride_q,
                                float *scale, int64_t ld_s, int64_t stride_s, uint8_t *q_t,
                                int64_t ld_qt, int64_t stride_qt, float *scale_t, int64_t ld_st,
                                int64_t stride_st, hipStream_t stream);

/*
 * fp8_gemm -- C = dequant(A) * dequant(B)^T with per-128-slab promotion.
 *
 * For each 128-element K slab j the FP8 products of the slab are summed into
 * an FP32 partial P_j, and the FP32 accumulator takes acc += P_j * sA * sB,
 * the scales of the slab's tiles/blocks (pages: see the file header).
 *   Fprop:  A = X codes [m][k] (1x128),   B = W codes [n][k] (BLOCK128).
 *   Dgrad:  A = dY codes [m][k] (1x128),  B = W^T codes [n][k] (BLOCK128,
 *           the transposed copy of fp8_quantize_weight).
 *   Wgrad:  A = dY^T codes [m][k], B = X^T codes [n][k], both from the 128x1
 *           token tiling (ROW128); K is the token dimension.
 *
 * a        codes [m][lda], K contiguous, lda >= k.
 * a_scale  [k/128][ld_as], ld_as >= m (slab-major, as written by
 *          fp8_quantize_act in either tiling).
 * b        codes [n][ldb], K contiguous, ldb >= k.
 * b_scale  FP8Q_BSCALE_BLOCK128: [ceil(n/128)][ld_bs], ld_bs >= k/128.
 *          FP8Q_BSCALE_ROW128:   [k/128][ld_bs], ld_bs >= n.
 * c        [m][ldc], ldc >= n; out_dtype FP8Q_OUT_BF16 (uint16 bf16, rounded
 *          to nearest even) or FP8Q_OUT_F32. Every element of the m x n
 *          window is written; k == 0 writes zeros (A, B and their scales
 *          are then not read and may be NULL).
 * Shapes:  m, n >= 0 (any value; ragged tiles are handled), k % 128 == 0;
 *          lda, ldb and the scale spans within the limits above.
 * Alignment: a, b, c 16-byte aligned; lda, ldb % 16 == 0; ldc % 8 == 0;
 *          scales 4-byte aligned.
 * m == 0 or n == 0: returns FP8Q_OK without launching.
 * Errors: FP8Q_ERR_NULL, FP8Q_ERR_SHAPE, FP8Q_ERR_ALIGN, FP8Q_ERR_ENUM,
 *         FP8Q_ERR_HIP.
 */
int fp8_gemm(int64_t m, int64_t n, int64_t k,
             const uint8_t *a, int64_t lda, const float *a_scale, int64_t ld_as,
             const uint8_t *b, int64_t ldb, const float *b_scale, int64_t ld_bs, int b_scale_kind,
             void *c, int64_t ldc, int out_dtype, hipStream_t stream);

/*
 * fp8_grouped_gemm -- MoE expert Fprop over an expert-sorted row layout.
 *
 * Expert e owns rows [group_offsets[e], group_offsets[e+1]) of A and C; its
 * first group_rows[e] rows are real tokens and the rest is padding. Real rows
 * get C_e = dequant(A_e) * dequant(W_e)^T exactly as fp8_gemm with
 * FP8Q_BSCALE_BLOCK128; padding rows of C are written as zeros. A is the FP8
 * activation quantized once before dispatch (page "Eliminate Deepseek Ai News
 * For Good", passage on quantizing before the MoE up-projections), with
 * slab-major 1x128 scales.
 *
 * groups        number of experts, >= 0.
 * group_offsets DEVICE int32[groups + 1]: non-decreasing multiples of 128,
 *               group_offsets[0] == 0, group_offsets[groups] == m_total.
 * group_rows    DEVICE int32[groups] real rows per expert,
 *               0 <= group_rows[e] <= group_offsets[e+1] - group_offsets[e];
 *               NULL means every row is real.
 * m_total       rows of A and C (host copy of group_offsets[groups]),
 *               m_total % 128 == 0.
 * a, a_scale    codes [m_total][lda], scales [k/128][ld_as], ld_as >= m_total.
 *               The codes and scales of padding rows may hold any bytes: they
 *               feed only padding rows of C, which are written as zeros.
 * b             expert weights: expert e at b + e * stride_b, codes [n][ldb].
 * b_scale       expert e at b_scale + e * stride_bs, [n/128][ld_bs].
 *               The experts' weights are only read, so their rows may
 *               interleave: stride_b and stride_bs need only be >= 0. For
 *               Dgrad, quantizing all experts' W as one [E*N][K] matrix
 *               gives the transposed copy [K][E*N]; expert e's W_e^T is
 *               then b + e*N with ldb = E*N (stride_b = N), and its block
 *               scales b_scale + e*N/128 with ld_bs = E*N/128.
 * c             [m_total][ldc]; out_dtype as in fp8_gemm.
 * workspace     DEVICE scratch of workspace_bytes bytes owned by the caller,
 *               or NULL. The 256 x 256 output tiles run in rounds of the 256
 *               compute units; when the last round is less than half full,
 *               each of its tiles is cut along K into pieces that run on the
 *               otherwise idle units and leave FP32 partial tiles here, and a
 *               second kernel on `stream` adds each tile's pieces in a fixed
 *               order and writes C (the result is deterministic; it differs
 *               from the unsplit sum by FP32 rounding only). A workspace of
 *               FP8Q_GROUPED_WORKSPACE_BYTES allows every split; a smaller
 *               one limits it, and NULL (or fewer bytes than two partial
 *               tiles need) turns it off. Its contents need no
 *               initialisation and are left unspecified; calls whose work
 *               overlaps in time must not share a workspace.
 * Shapes:       n % 128 == 0, k % 128 == 0; lda, ldb and the scale
 *               spans within the GEMM limits above; workspace_bytes >= 0.
 * Alignment:    as fp8_gemm; stride_b % 16 == 0; workspace 256-byte aligned.
 * The device arrays are trusted: offsets that break the contract give
 * unspecified output (the kernels still stay within the m_total rows and
 * the workspace); with FP8Q_DEBUG=1 they are checked on the host first (see
 * above).
 * Errors: FP8Q_ERR_NULL, FP8Q_ERR_SHAPE, FP8Q_ERR_ALIGN, FP8Q_ERR_ENUM,
 *         FP8Q_ERR_HIP.
 */
#define FP8Q_GROUPED_WORKSPACE_BYTES 67117056LL /* 64 MiB of partial tiles + 8 KiB of records */

int fp8_grouped_gemm(int32_t groups, const int32_t *group_offsets, const int32_t *group_rows,
                     int64_t m_total, int64_t n, int64_t k,
                     const uint8_t *a, int64_t lda, const float *a_scale, int64_t ld_as,
                     const uint8_t *b, int64_t ldb, int64_t stride_b,
                     const float *b_scale, int64_t ld_bs, int64_t stride_bs,
                     void *c, int64_t ldc, int out_dtype,
                     void *workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * fp8_grouped_gemm_noalloc -- fp8_grouped_gemm for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *
 * Arguments, results and errors are those of fp8_grouped_gemm with a
 * workspace of FP8Q_GROUPED_WORKSPACE_BYTES. The workspace is the library's
 * own scratch: a file-scope device array of FP8Q_GROUPED_WORKSPACE_BYTES
 * (64 MiB + 8 KiB) that each GPU the library runs on holds until the process
 * ends. That is the largest workspace any call uses, so no shape is refused
 * for its size; shapes past the limits of fp8_grouped_gemm return
 * FP8Q_ERR_SHAPE as there. The call allocates nothing (no hipMalloc, hipFree
 * or allocating library routine). Its first call on a device looks up the
 * array's address there with that device current (make it before a graph
 * capture); a device id of 64 or more returns FP8Q_ERR_HIP. Nothing in the
 * scratch needs to start at zero, and it keeps the last call's partial
 * tiles. All calls on one GPU share it: calls whose work overlaps in time on
 * one GPU (on several streams, or graph replays in flight together) race and
 * give unspecified output.
 */
int fp8_grouped_gemm_noalloc(int32_t groups, const int32_t *group_offsets, const int32_t *group_rows,
                             int64_t m_total, int64_t n, int64_t k,
                             const uint8_t *a, int64_t lda, const float *a_scale, int64_t ld_as,
                             const uint8_t *b, int64_t ldb, int64_t stride_b,
                             const float *b_scale, int64_t ld_bs, int64_t stride_bs,
                             void *c, int64_t ldc, int out_dtype, hipStream_t stream);

/*
 * fp8_grouped_gemm_wgrad -- MoE expert Wgrad: one weight gradient per expert,
 * each contracting over that expert's own token segment.
 *
 * The Wgrad GEMM in FP8 (page dssusan.co.kr Q&A board, passage on Figure 6)
 * applied to every expert of a MoE layer; the per-(slab, row) scales come
 * from 128x1 token tiles, as for fp8_gemm with FP8Q_BSCALE_ROW128.
 *   dW_e[i][j] = sum over tokens t in [group_offsets[e], group_offsets[e+1])
 *                of dequant(A)[i][t] * dequant(B)[j][t],
 * with the same per-slab promotion as fp8_gemm: A = dY^T codes, B = X^T codes
 * of the expert-sorted token layout, both quantized with FP8Q_TILE_128x1 over
 * all k_total tokens. Segments are multiples of 128 tokens, so no 128-token
 * tile straddles two experts; padding tokens must be zero in the bf16 inputs
 * (their codes are then zero and add nothing).
 *
 * groups        number of experts, >= 0.
 * group_offsets DEVICE int32[groups + 1]: non-decreasing multiples of 128,
 *               group_offsets[0] == 0, group_offsets[groups] == k_total.
 * k_total       tokens of the layout (host copy of group_offsets[groups]).
 * m, n          rows and columns of each dW_e (n_out x k_in).
 * a, a_scale    codes [m][lda], lda >= k_total; scales [k_total/128][ld_as],
 *               ld_as >= m.
 * b, b_scale    codes [n][ldb], ldb >= k_total; scales [k_total/128][ld_bs],
 *               ld_bs >= n.
 * c             dW_e at c + e * stride_c (elements of out_dtype), [m][ldc],
 *               ldc >= n, stride_c >= m * ldc, stride_c % 8 == 0. An expert
 *               with an empty segment gets dW_e = 0 (k_total == 0: all are
 *               zero, and A, B and their scales may be NULL).
 * Shapes:       lda, ldb and the scale spans within the GEMM limits above.
 * Alignment:    as fp8_gemm.
 * The device array is trusted: segments outside [0, k_total] are skipped
 * (their dW_e is not written); with FP8Q_DEBUG=1 it is checked on the host
 * first (see above).
 * Errors: FP8Q_ERR_NULL, FP8Q_ERR_SHAPE, FP8Q_ERR_ALIGN, FP8Q_ERR_ENUM,
 *         FP8Q_ERR_HIP.
 */
int fp8_grouped_gemm_wgrad(int32_t groups, const int32_t *group_offsets, int64_t k_total,
                           int64_t m, int64_t n,
                           const uint8_t *a, int64_t lda, const float *a_scale, int64_t ld_as,
                           const uint8_t *b, int64_t ldb, const float *b_scale, int64_t ld_bs,
                           void *c, int64_t ldc, int64_t stride_c, int out_dtype,
                           hipStream_t stream);

/*
 * fp8_quantize_mx -- microscaling (OCP MX) quantization with E4M3 elements.
 *
 * The variant the pages liken their fine-grained groups to (page "Deepseek
 * Ai News Expert Interview", passage on microscaling formats with smaller
 * quantization granularity). A different numeric contract from
 * fp8_quantize_act: every 32 consecutive elements of a row share a power-
 * of-two scale 2^e, e = floor(log2(amax)) - 8 clamped to [-127, 127] (-127
 * for an all-zero block), stored as the E8M0 byte e + 127; each code is
 * E4M3(x / 2^e) rounded to nearest, ties to the even code, saturating to
 * +-448. Dequantized value = dec(q) * 2^e.
 *
 * x      bf16 [rows][ld_x], ld_x >= cols, cols % 128 == 0.
 * q      codes [rows][ld_q], ld_q >= cols (the layout of x).
 * scale  uint32 [cols/128][ld_s], ld_s >= rows: word (j, r) holds the four
 *        E8M0 bytes of row r's blocks 4j .. 4j+3, byte b for block 4j + b.
 * Alignment: x and q 16-byte aligned; ld_x % 8 == 0; ld_q % 16 == 0; scale
 *        4-byte aligned. rows == 0 or cols == 0: returns FP8Q_OK.
 * Errors: FP8Q_ERR_NULL, FP8Q_ERR_SHAPE, FP8Q_ERR_ALIGN, FP8Q_ERR_HIP.
 */
int fp8_quantize_mx(const uint16_t *x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t *q,
                    int64_t ld_q, uint32_t *scale, int64_t ld_s, hipStream_t stream);

/*
 * fp8_quantize_mx_pair -- fp8_quantize_mx on the two operands of the
 * microscaling GEMM (x0[rows0][cols0] and x1[rows1][cols1]) in one launch,
 * page "Deepseek Ai News Expert Interview", same passage. Same layouts,
 * alignment rules and results, bit for bit, as the two calls; one launch
 * instead of two. A matrix with no rows or columns is skipped and its
 * pointers are not read. The two halves of the launch run concurrently, so
 * no output of one matrix (q, scale) may share a byte with an output of the
 * other.
 * Errors: those of fp8_quantize_mx; FP8Q_ERR_SHAPE also when the outputs of
 *         the two matrices overlap.
 */
int fp8_quantize_mx_pair(const uint16_t *x0, int64_t rows0, int64_t cols0, int64_t ld_x0, uint8_t *q0,
                         int64_t ld_q0, uint32_t *scale0, int64_t ld_s0, const uint16_t *x1, int64_t rows1,
                         int64_t cols1, int64_t ld_x1, uint8_t *q1, int64_t ld_q1, uint32_t *scale1,
                         int64_t ld_s1, hipStream_t stream);

/*
 * fp8_gemm_mx -- C = dequant_mx(A) * dequant_mx(B)^T.
 *
 * Both operands are K-contiguous MX codes with their scale words (as written
 * by fp8_quantize_mx along K). The gfx950 scaled MFMA applies every 32-element
 * block's two power-of-two scales and accumulates in FP32 inside the matrix
 * core; there is no separate promotion step.
 * a, a_scale  [m][lda], lda >= k; words [k/128][ld_as], ld_as >= m.
 * b, b_scale  [n][ldb], ldb >= k; words [k/128][ld_bs], ld_bs >= n.
 * c           [m][ldc], ldc >= n; out_dtype FP8Q_OUT_BF16 or FP8Q_OUT_F32.
 * Shapes:     m, n >= 0, k % 128 == 0 (k == 0 writes zeros); lda, ldb
 *             within the GEMM limits above.
 * Alignment:  as fp8_gemm.
 * Errors: FP8Q_ERR_NULL, FP8Q_ERR_SHAPE, FP8Q_ERR_ALIGN, FP8Q_ERR_ENUM,
 *         FP8Q_ERR_HIP.
 */
int fp8_gemm_mx(int64_t m, int64_t n, int64_t k,
                const uint8_t *a, int64_t lda, const uint32_t *a_scale, int64_t ld_as,
                const uint8_t *b, int64_t ldb, const uint32_t *b_scale, int64_t ld_bs,
                void *c, int64_t ldc, int out_dtype, hipStream_t stream);

/*
 * fp8_retile_act_128x1 -- a cached FP8 activation re-tiled for Wgrad.
 *
 * The FP8 Wgrad GEMM lets the forward activations be kept in FP8 for the
 * backward pass (page "Is aI Hitting a Wall?", passage on storing
 * activations in FP8 for the backward pass). The forward pass holds them as
 * 1x128 codes and scales (fp8_quantize_act, FP8Q_TILE_1x128); Wgrad takes
 * 128x1 token tiles. Each value is dequantized to binary32,
 * v = fl32(dec(q) * s), and the v are quantized in 128x1 tiles exactly as
 * FP8Q_TILE_128x1 quantizes bf16 input (s' = fl32(amax / 448),
 * q' = E4M3(fl32(v / s')), RNE, saturating; all-zero tile: s' = 0). The
 * result is bit-identical to that definition; it is not, in general, the
 * 128x1 quantization of the original bf16 activation.
 *
 * q        codes [tokens][ld_q], ld_q >= cols (1x128 layout).
 * scale    fp32 [cols/128][ld_s], ld_s >= tokens (slab-major 1x128 scales).
 * q_t      codes [cols][ld_qt], ld_qt >= tokens (token-contiguous).
 * scale_t  fp32 [tokens/128][ld_st], ld_st >= cols.
 * Shapes: tokens % 128 == 0, cols % 128 == 0; either 0: returns FP8Q_OK.
 * Alignment: q, q_t and scale 16-byte aligned; ld_q % 16 == 0,
 *         ld_qt % 16 == 0, ld_s % 4 == 0; scale_t 4-byte aligned.
 * Codes 0x7F / 0xFF (NaN) are outside the contract.
 * Errors: FP8Q_ERR_NULL, FP8Q_ERR_SHAPE, FP8Q_ERR_ALIGN, FP8Q_ERR_HIP.
 */
int fp8_retile_act_128x1(const uint8_t *q, int64_t tokens, int64_t cols, int64_t ld_q,
                         const float *scale, int64_t ld_s, uint8_t *q_t, int64_t ld_qt,
                         float *scale_t, int64_t ld_st, hipStream_t stream);

/*
 * fp8_gemm_tensor -- C = sA * sB * sum_k dec(A[m][k]) * dec(B[n][k]), with one
 * scale per operand and the whole K sum accumulated inside the matrix core.
 *
 * The arm of the accumulation study (page "Eliminate Deepseek Ai News For
 * Good", passage on limited accumulation precision in a K = 4096 GEMM of
 * random matrices): no per-interval promotion, the MFMA accumulators carry
 * the sum over all K, and fl32(sA * sB) scales the result once. Compare
 * fp8_gemm, which promotes every 128-element slab.
 * a        codes [m][lda], lda >= k.    a_scale  one fp32 (device).
 * b        codes [n][ldb], ldb >= k.    b_scale  one fp32 (device).
 * c        [m][ldc], ldc >= n; out_dtype FP8Q_OUT_BF16 or FP8Q_OUT_F32.
 * Shapes:  m, n >= 0, k % 128 == 0 (k == 0 writes zeros; a, b and the
 *          scales are then not read and may be NULL); lda, ldb within the
 *          GEMM limits above.
 * Alignment: as fp8_gemm.
 * Errors: FP8Q_ERR_NULL, FP8Q_ERR_SHAPE, FP8Q_ERR_ALIGN, FP8Q_ERR_ENUM,
 *         FP8Q_ERR_HIP.
 */
int fp8_gemm_tensor(int64_t m, int64_t n, int64_t k, const uint8_t *a, int64_t lda,
                    const float *a_scale, const uint8_t *b, int64_t ldb, const float *b_scale,
                    void *c, int64_t ldc, int out_dtype, hipStream_t stream);

/* Text for a status code (static storage; never NULL). */
const char *fp8q_status_string(int status);

/* hipError_t of the most recent FP8Q_ERR_HIP in this thread (0 if none). */
int fp8q_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
