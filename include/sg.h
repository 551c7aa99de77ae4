/*
 * sg.h -- C ABI of sparse_gemm_layers_amd: FP8 (OCP e4m3) groupwise-scaled and
 * 2:4-sparse linear-layer GEMMs for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * Sources (web pages; cited by title and by position in the thread):
 *   [I2029] CUTLASS issue #2029, "[QST] CUTLASS support for fp8 sparse matrix
 *           (for W) multiplication for A*W=Y with GPU (SM90a/89) sparse tensor core"
 *   [P2095] CUTLASS PR #2095, "Improvements for: Groupwise scaling along M for
 *           FP8 gemm"
 *   [I2058] CUTLASS issue #2058, "[QST] How to implement a fused mixed precision
 *           matrix multiplication such as w4a4 + w16a16?"
 *   [T3258] torchao PR #3258, "Introduce new W8A8-FP-CSR quantization API"
 *
 * Conventions for every entry point
 *   - All matrices are row-major.  A leading dimension (ld*) is the distance in
 *     ELEMENTS between consecutive rows (bytes for uint8 buffers; for packed int4
 *     buffers it is in bytes, i.e. pairs of elements).
 *   - Scale arrays are fp32 and addressed through two strides in floats, so both
 *     the "M-major" layout of [P2095] (PR description: scales contiguous along M,
 *     one column per K tile) and a row-major layout can be passed.
 *   - Every pointer is caller-owned device memory.  The library allocates
 *     nothing, needs no workspace, keeps no mutable global state, and may be
 *     called from several host threads at once.
 *   - Work is enqueued on `stream` (0 = the null stream) and runs asynchronously;
 *     nothing is copied back to the host and no call synchronises.
 *   - Arguments are validated on the host BEFORE any HIP call; an invalid call
 *     returns an error status and enqueues nothing.  A launch failure reported
 *     by the HIP runtime returns SG_ERR_HIP.
 *   - Every size argument (rows, cols, M, N, K, L, G) must be at least 1: a
 *     zero or negative size is SG_ERR_SHAPE and enqueues nothing.  The pages
 *     describe no empty problem; a caller with nothing to do makes no call.
 *     (Only single groups of the grouped GEMM may be empty.)  The mixed GEMM's
 *     K2 may be 0.
 *   - Non-finite inputs (the pages say nothing of them) follow IEEE arithmetic
 *     through the documented formulas: a quantiser block holding a NaN gets a
 *     NaN scale and one holding an infinity an infinite scale; e4m3 encoding
 *     saturates infinities to +-448 and gives every NaN the code 0x7F; an int8
 *     or int4 code of a NaN is 0; bf16 outputs keep NaN as NaN; pruning ranks
 *     NaN above every number.  Every access stays within the described buffers.
 */
#ifndef SPARSE_GEMM_LAYERS_AMD_SG_H
#define SPARSE_GEMM_LAYERS_AMD_SG_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status, dtype and output-form codes are plain 32-bit ints with named
 * values, so that any int a caller passes is a valid argument (an unknown
 * value is rejected with SG_ERR_UNSUPPORTED, never undefined behaviour). */
typedef int32_t sg_status;
enum {
  SG_OK = 0,
  SG_ERR_NULL = 1,        /* a required pointer is NULL                          */
  SG_ERR_SHAPE = 2,       /* a size or leading dimension is out of range         */
  SG_ERR_UNSUPPORTED = 3, /* granularity, dtype or output form not supported     */
  SG_ERR_ALIGN = 4,       /* a pointer or leading dimension is misaligned        */
  SG_ERR_HIP = 5          /* the HIP runtime reported an error at launch         */
};

typedef int32_t sg_dtype;
enum { SG_F32 = 0, SG_BF16 = 1, SG_E4M3 = 2, SG_I8 = 3 };

/* Output form of the GEMMs.  Both compute the same numbers.
 *   SG_OUT_Y : Y   [M, N] row-major, element (m, n) at y[m * ldy + n]
 *   SG_OUT_YT: Y^T [N, M] row-major, element (m, n) at y[n * ldy + m]
 * SG_OUT_YT is the swap+transpose form C^T = B^T . A^T of [I2029] (klevzoff's
 * answer: swap the operands and flip the layout of C/D), which puts the sparse
 * weight on the left. */
typedef int32_t sg_form;
enum { SG_OUT_Y = 0, SG_OUT_YT = 1 };

/* Human-readable name of a status code (static string, never NULL; any value). */
const char* sg_status_str(sg_status s);

/* Version of this ABI; bumped on any incompatible change (2: the int4
 * quantiser takes its group width; 3: empty problems are SG_ERR_SHAPE). */
int sg_abi_version(void);

/*
 * sg_fp8_quant_groupwise -- per-block amax -> scale -> e4m3 codes.
 * [P2095] hwu36's comment (ScaleGranularityM/N: 1 or 128 rows share one scale
 * per 128-wide K block); [T3258] jcaip's review (scale must be positive, an
 * all-zero tensor must be supported, activations are scaled then cast to
 * float8_e4m3fn).
 *
 * For each block of gr rows x gc columns (the last row block may be partial):
 *   amax = max |x|;  s = amax / 448 in fp32 (s = 1 if amax == 0; NaN if the
 *          block holds a NaN);
 *   q    = e4m3(x / s): IEEE fp32 divide, round to nearest even, saturate at
 *          +-448, a negative value that rounds to zero gives -0 (0x80).
 *   x   : [rows, cols], dtype x_dt (SG_F32 or SG_BF16), leading dim ldx.
 *   gr  : 1 or 128.   gc: 128 or 64 (64 serves the compressed 2:4 values, whose
 *         128 x 64 blocks are the 128 x 128 blocks of the dense weight).
 *         Or one block per row (gr = 1, gc = cols) or one for the tensor
 *         (gr = rows, gc = cols), with cols a multiple of 16: the rowwise and
 *         tensorwise scales that the GEMMs take as scales constant along K
 *         ([T3258]: its quoted weight quantisation keeps one scale per row).
 *   q   : [rows, cols] e4m3 codes (uint8), leading dim ldq (bytes).
 *   s   : block (rb, cb) at s[rb * s_stride_r + cb * s_stride_c],
 *         rb < ceil(rows / gr), cb < cols / gc.
 * Requires cols % gc == 0, ldx >= cols, ldq >= cols; x, q 16-byte aligned,
 * ldx * sizeof(x_dt) and ldq multiples of 16; s 4-byte aligned.
 */
sg_status sg_fp8_quant_groupwise(const void* x, sg_dtype x_dt, int64_t rows, int64_t cols,
                                 int64_t ldx, int gr, int gc, uint8_t* q, int64_t ldq, float* s,
                                 int64_t s_stride_r, int64_t s_stride_c, hipStream_t stream);

/*
 * sg_int4_quant_groupwise -- symmetric int4 codes with one fp32 scale per
 * (row, gc-column group), the input format of sg_mixed_gemm_add (gc = 128;
 * [I2058] hyx1999: X1 and W1 are quantised to 4 bit; the page fixes no
 * scheme) and, over 2:4-compressed values (gc = 64 = one 128-wide K block),
 * of sg_w4a16_sparse24_gemm_groupwise.
 *   s = amax / 7 in fp32 (1 if amax == 0);  q = clamp(rint(x / s), -7, 7),
 *   rint = round half to even, IEEE fp32 divide.
 *   Packed two's-complement nibbles: element 2j in the low nibble of byte j.
 *   x : [rows, cols] (SG_F32 or SG_BF16), ld ldx.  q: [rows, cols/2] bytes, ld ldq.
 *   gc: 128 or 64.
 *   s : (r, cb) at s[r * s_stride_r + cb * s_stride_c], cb < cols / gc.
 * Requires cols % gc == 0; x 16-byte aligned, ldx * sizeof(x_dt) % 16 == 0;
 * q 4-byte aligned, ldq % 4 == 0, ldq >= cols / 2.
 */
sg_status sg_int4_quant_groupwise(const void* x, sg_dtype x_dt, int64_t rows, int64_t cols,
                                  int64_t ldx, int gc, uint8_t* q, int64_t ldq, float* s,
                                  int64_t s_stride_r, int64_t s_stride_c, hipStream_t stream);

/*
 * sg_sparse24_prune_compress -- 2:4 magnitude pruning along K, then packing of
 * the kept values and their metadata.  [T3258] jcaip's review: groups of 4
 * along a row, the two smallest |w| are dropped; store only the specified
 * values and the sparsity metadata.  [I2029] klevzoff: the sparse operand is
 * passed as values + metadata E.
 *   Kept: the two largest |w| of each group; equal magnitudes -> lower index
 *   (+0 and -0 are equal); NaN ranks above every number, NaNs are equal.
 *   vals[r, 2g + j] = w[r, 4g + i_j] with i_0 < i_1 (bits copied unchanged);
 *   meta[r, b]      = nib(2b) | nib(2b + 1) << 4,  nib(g) = i_0 | i_1 << 2.
 *   w    : [rows, k], dtype dt (SG_F32, SG_BF16, or SG_E4M3 codes: a weight
 *          already quantised, whose codes' magnitudes are ranked), leading dim ldw.
 *   vals : [rows, k/2], same dtype, leading dim ldv.
 *   meta : [rows, k/8] bytes, leading dim ldm.
 * Requires k % 8 == 0, ldw >= k, ldv >= k/2, ldm >= k/8; w and vals 16-byte
 * aligned, ldw * sizeof(dt) a multiple of 16 and ldv a multiple of 4.
 */
sg_status sg_sparse24_prune_compress(const void* w, sg_dtype dt, int64_t rows, int64_t k,
                                     int64_t ldw, void* vals, int64_t ldv, uint8_t* meta,
                                     int64_t ldm, hipStream_t stream);

/*
 * sg_fp8_gemm_groupwise -- Y = X . W^T with groupwise dequantisation scales.
 * [P2095] hwu36's comment (the four ScaleGranularityM/N modes) and the
 * promotion-interval review (products of a K tile start from zero and are
 * promoted into fp32 accumulators with the tile's scales); here once per
 * 128-wide K block:
 *   y[m, n] = sum_kb sx[m/gran_m, kb] * sw[n/gran_n, kb] * sum_{k in kb} x[m,k] w[n,k]
 *   xq : [M, K] e4m3, ld ldx.   sx: (m/gran_m, kb) at sx[(m/gran_m)*sx_sm + kb*sx_sk].
 *   wq : [N, K] e4m3, ld ldw.   sw: (n/gran_n, kb) at sw[(n/gran_n)*sw_sn + kb*sw_sk].
 *   gran_m, gran_n : 1 or 128.
 *   y  : SG_F32 or SG_BF16 (round to nearest even) in the layout `form` selects.
 * Requires K % 128 == 0, K > 0, M, N >= 1, ldx, ldw >= K; xq, wq 16-byte aligned,
 * ldx, ldw multiples of 16; ldy >= N (SG_OUT_Y) or >= M (SG_OUT_YT); y aligned to
 * its element size.  M and N need not be multiples of any tile (the partial M
 * and N tiles of [P2095] are predicated).
 * Scales constant along K (sx_sk == 0 and sw_sk == 0): rowwise scales (gran 1,
 * one per X row and per W row) or tensorwise ones (also sx_sm == 0, sw_sn ==
 * 0), as in [T3258] (its quoted weight quantisation expands one scale per
 * weight row over the whole row; jcaip's review asks for kernels that fuse
 * the scale multiplication).  Then y = sx * sw * sum_k x w, and for M > 64
 * the kernels add all of K in the matrix core's fp32 accumulator and apply
 * the scale product once, after the K loop (the same result within rounding;
 * the int8 GEMMs keep an exact int32 sum while K <= 131072).  This holds for
 * every GEMM entry point below.
 */
sg_status sg_fp8_gemm_groupwise(int64_t M, int64_t N, int64_t K, const uint8_t* xq, int64_t ldx,
                                const float* sx, int64_t sx_sm, int64_t sx_sk, int gran_m,
                                const uint8_t* wq, int64_t ldw, const float* sw, int64_t sw_sn,
                                int64_t sw_sk, int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                                sg_form form, hipStream_t stream);

/*
 * sg_fp8_sparse24_gemm_groupwise -- the same GEMM with W stored 2:4-compressed
 * (values + metadata as produced by sg_sparse24_prune_compress then quantised
 * with sg_fp8_quant_groupwise at gr = 128, gc = 64).  The result equals
 * sg_fp8_gemm_groupwise on the decompressed weight.  [I2029] (hwu36: the sparse
 * FP8 operand must be the row-major left operand; klevzoff: swap+transpose);
 * [T3258] jcaip's review (fused scale multiplication in the sparse FP8 kernel).
 *   wv    : [N, K/2] e4m3 codes, ld ldwv (bytes).
 *   wmeta : [N, K/8] metadata bytes, ld ldwm.
 *   other arguments as sg_fp8_gemm_groupwise.
 * Requires in addition ldwv >= K/2, ldwm >= K/8, wv and wmeta 16-byte aligned,
 * ldwv and ldwm multiples of 16.  Metadata nibbles must be legal
 * (0x4, 0x8, 0x9, 0xC, 0xD, 0xE); others give unspecified values in range.
 */
sg_status sg_fp8_sparse24_gemm_groupwise(int64_t M, int64_t N, int64_t K, const uint8_t* xq,
                                         int64_t ldx, const float* sx, int64_t sx_sm,
                                         int64_t sx_sk, int gran_m, const uint8_t* wv,
                                         int64_t ldwv, const uint8_t* wmeta, int64_t ldwm,
                                         const float* sw, int64_t sw_sn, int64_t sw_sk,
                                         int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                                         sg_form form, hipStream_t stream);

/*
 * sg_sparse24_packed_bytes -- size in bytes of the gfx950 packed form of an
 * N x K 2:4-compressed weight: ceil(N / 16) * (K / 128) * 1280.  Returns -1 if
 * N < 0, K <= 0 or K % 128 != 0.
 */
int64_t sg_sparse24_packed_bytes(int64_t N, int64_t K);

/*
 * sg_sparse24_pack_gfx950 -- rearranges a 2:4-compressed FP8 weight (codes
 * wv [N, K/2], metadata wmeta [N, K/8], as produced by
 * sg_sparse24_prune_compress + sg_fp8_quant_groupwise) into the layout the
 * sparse GEMM kernels stream from HBM straight into LDS.  [T3258] jcaip's
 * review (FP8 semi-structured weights are packed by the hardware's packing
 * kernel); [I2029] klevzoff (values and metadata E reach the mainloop in the
 * hardware's layout).  A pure byte permutation:
 *   for 16-row block R (rows 16 R .. 16 R + 15) and 128-wide K block kb the
 *   1280-byte chunk at (R * K/128 + kb) * 1280 (one row block's chunks follow
 *   each other along K) holds, for local row lr and lane group g = 0..3
 *   (b = 32 (g & 1) + 8 (g >> 1)):
 *     - at lr*64 + 16 (g ^ ((lr >> 1) & 3)): compressed bytes [b, b+8) and
 *       [b+16, b+24) of the row's 64 bytes of block kb;
 *     - at 1024 + lr*16 + 4 ((g + 2 ((lr >> 3) & 1)) & 3): metadata bytes b/4,
 *       b/4+1, b/4+4, b/4+5 of the row's 16 bytes of block kb;
 *   rows past N (up to the next multiple of 16) are zero.
 *   packed : sg_sparse24_packed_bytes(N, K) bytes, 16-byte aligned, written fully.
 * Requires K % 128 == 0, ldwv >= K/2, ldwm >= K/8, multiples of 16; wv, wmeta
 * 16-byte aligned.
 */
sg_status sg_sparse24_pack_gfx950(const uint8_t* wv, int64_t ldwv, const uint8_t* wmeta, int64_t ldwm,
                                  int64_t N, int64_t K, uint8_t* packed, hipStream_t stream);

/*
 * sg_fp8_sparse24_gemm_groupwise_packed -- sg_fp8_sparse24_gemm_groupwise with
 * the weight given in the packed form of sg_sparse24_pack_gfx950 (same
 * results; the form whose loads are contiguous 1 KB per wave instruction, and
 * that the M <= 64 path streams row block by row block).
 *   wpacked : sg_sparse24_packed_bytes(N, K) bytes, 16-byte aligned.
 *   other arguments as sg_fp8_sparse24_gemm_groupwise.
 * Requires in addition (K / 128) * 16 * 1280 < 2^31.
 */
sg_status sg_fp8_sparse24_gemm_groupwise_packed(int64_t M, int64_t N, int64_t K, const uint8_t* xq,
                                                int64_t ldx, const float* sx, int64_t sx_sm,
                                                int64_t sx_sk, int gran_m, const uint8_t* wpacked,
                                                const float* sw, int64_t sw_sn, int64_t sw_sk,
                                                int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                                                sg_form form, hipStream_t stream);

/*
 * sg_mixed_gemm_add -- Y = X1 . W1^T + X2 . W2^T in one kernel ([I2058],
 * hyx1999: a w4a4 GEMM plus a small w16a16 GEMM whose results are added, with
 * L = 2048, D1 = 4096, D2 = 64, D = 4096 as the example shape).
 *   y[m, n] = sum_kb sx1[m, kb] sw1[n, kb] sum_{k in kb} int4(x1) int4(w1)
 *           + sum_{k < K2} bf16(x2[m, k]) bf16(w2[n, k]),   fp32 accumulation.
 *   x1 : [M, K1/2] packed int4 (sg_int4_quant_groupwise), ld ldx1 bytes;
 *        sx1 (m, kb) at sx1[m * sx1_sm + kb * sx1_sk].
 *   w1 : [N, K1/2] packed int4, ld ldw1; sw1 (n, kb) at sw1[n * sw1_sn + kb * sw1_sk].
 *   x2 : [M, K2] bf16 bits, ld ldx2.   w2: [N, K2] bf16 bits, ld ldw2.
 *   y  : [M, N] bf16 (round to nearest even), ld ldy.
 * Requires K1 % 128 == 0, K1 > 0, K2 % 32 == 0, K2 >= 0; ldx1, ldw1 >= K1/2,
 * multiples of 16 and below 2^23; ldx2, ldw2 >= K2, below 2^22, with rows a
 * multiple of 16 bytes; x1, w1, x2, w2 16-byte aligned (x2, w2 may be NULL when
 * K2 == 0); y 2-byte aligned; the scale arrays' byte extents below 2^31.
 */
sg_status sg_mixed_gemm_add(int64_t M, int64_t N, int64_t K1, int64_t K2, const uint8_t* x1,
                            int64_t ldx1, const float* sx1, int64_t sx1_sm, int64_t sx1_sk,
                            const uint8_t* w1, int64_t ldw1, const float* sw1, int64_t sw1_sn,
                            int64_t sw1_sk, const uint16_t* x2, int64_t ldx2, const uint16_t* w2,
                            int64_t ldw2, uint16_t* y, int64_t ldy, hipStream_t stream);

/*
 * sg_fp8_sparse24_gemm_packed_quant_x -- the packed 2:4 FP8 GEMM with the
 * activation quantisation done inside it.  [T3258] jcaip's review: the
 * activation is scaled and cast to float8_e4m3fn on its way into the sparse
 * FP8 kernel.  X (fp32 or bf16) is quantised per 1 x 128 block exactly as
 * sg_fp8_quant_groupwise(x, gr = 1, gc = 128) does it (block amax, s =
 * amax / 448 by IEEE divide, codes = e4m3(x / s)), and the GEMM is
 * sg_fp8_sparse24_gemm_groupwise_packed with those codes, gran_m = 1 and the
 * same W operands: the result is bit for bit that of the two calls, without
 * writing the codes and scales to memory.
 *   x   : [M, K], x_dt SG_F32 or SG_BF16, leading dim ldx (elements).
 *   wpacked, sw, sw_sn, sw_sk: as for sg_fp8_sparse24_gemm_groupwise_packed,
 *         gran_n = 128 only.
 *   y, y_dt, ldy, form: as for the other GEMMs.
 * Decode sizes only: 1 <= M <= 64 (SG_ERR_UNSUPPORTED above; every workgroup
 * quantises all of X, which pays off only while X is small against the
 * weight).  Requires K % 128 == 0, ldx >= K, x 16-byte aligned with rows of a
 * multiple of 16 bytes, 64 * ldx * sizeof(x_dt) < 2^32.
 */
sg_status sg_fp8_sparse24_gemm_packed_quant_x(int64_t M, int64_t N, int64_t K, const void* x, sg_dtype x_dt,
                                              int64_t ldx, const uint8_t* wpacked, const float* sw, int64_t sw_sn,
                                              int64_t sw_sk, int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                                              sg_form form, hipStream_t stream);

/*
 * int8 x int8 2:4-sparse GEMM ([T3258], jcaip: the existing 2:4 kernels are
 * int8 x int8 and fp8 x fp8).  The page fixes no int8 scheme; this one keeps
 * the FP8 path's groupwise blocks and uses the symmetric int8 grid.
 *
 * sg_int8_quant_groupwise -- as sg_fp8_quant_groupwise (same arguments, blocks,
 * layouts, requirements and errors) with int8 codes:
 *   s = fl32(amax / 127) (1 when amax == 0); q = clamp(rint_even(fl32(v / s)), -127, 127).
 */
sg_status sg_int8_quant_groupwise(const void* x, sg_dtype x_dt, int64_t rows, int64_t cols,
                                  int64_t ldx, int gr, int gc, int8_t* q, int64_t ldq, float* s,
                                  int64_t s_stride_r, int64_t s_stride_c, hipStream_t stream);

/*
 * sg_int8_sparse24_gemm_groupwise -- as sg_fp8_sparse24_gemm_groupwise (same
 * arguments, scale modes, output forms, requirements and errors) with int8
 * codes for X and for the compressed W values (W pruned with
 * sg_sparse24_prune_compress, then quantised with sg_int8_quant_groupwise at
 * gr = 128, gc = 64):
 *   y[m, n] = sum_kb sx[m / gran_m, kb] * sw[n / gran_n, kb] * P[m, n, kb],
 *   P = the exact integer sum over the K block of x * w (int32 on the matrix core).
 */
sg_status sg_int8_sparse24_gemm_groupwise(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                                          int64_t ldx, const float* sx, int64_t sx_sm,
                                          int64_t sx_sk, int gran_m, const int8_t* wv,
                                          int64_t ldwv, const uint8_t* wmeta, int64_t ldwm,
                                          const float* sw, int64_t sw_sn, int64_t sw_sk,
                                          int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                                          sg_form form, hipStream_t stream);

/*
 * sg_int8_sparse24_gemm_groupwise_packed -- the same with the weight in the
 * packed form of sg_sparse24_pack_gfx950 (which moves bytes and so packs int8
 * codes as it packs e4m3 codes); arguments as
 * sg_fp8_sparse24_gemm_groupwise_packed.
 */
sg_status sg_int8_sparse24_gemm_groupwise_packed(int64_t M, int64_t N, int64_t K, const int8_t* xq,
                                                 int64_t ldx, const float* sx, int64_t sx_sm,
                                                 int64_t sx_sk, int gran_m, const uint8_t* wpacked,
                                                 const float* sw, int64_t sw_sn, int64_t sw_sk,
                                                 int gran_n, void* y, sg_dtype y_dt, int64_t ldy,
                                                 sg_form form, hipStream_t stream);

/*
 * Batched ("L" mode) forms: L problems of one shape (M, N, K), problem z
 * reading and writing its operands at these offsets from problem 0's:
 *   xq + z * x_bs, wq / wv / wpacked + z * (w_bs / wv_bs / wp_bs), wmeta +
 *   z * wm_bs (bytes); sx + z * sx_bs, sw + z * sw_bs (floats); y + z * y_bs
 *   (elements of y_dt).
 * [P2095] PR description: the scale layout (M / ScaleGranularityM, K_TILES, L)
 * carries the batch L as its outermost mode.  Every problem follows its
 * single-problem entry point; L == 1 with zero strides is that call.
 * bias (may be NULL: no bias): fp32 [N] per problem, at bias + z * bias_bs,
 * 4-byte aligned; bias[n] is added to output row n of every column after the
 * scales and before the output rounding (the `bias` argument of the sparse
 * FP8 linear that jcaip's review in [T3258] points to).
 * Requires in addition 1 <= L <= 65535,
 * every batch stride >= 0, and x_bs, w_bs / wv_bs / wp_bs, wm_bs multiples of 16
 * (SG_ERR_ALIGN otherwise).  Outputs of different problems must not overlap;
 * inputs may (a zero weight stride shares one weight among the problems).
 */
sg_status sg_fp8_gemm_groupwise_batched(int64_t L, int64_t M, int64_t N, int64_t K, const uint8_t* xq,
                                        int64_t ldx, int64_t x_bs, const float* sx, int64_t sx_sm,
                                        int64_t sx_sk, int64_t sx_bs, int gran_m, const uint8_t* wq,
                                        int64_t ldw, int64_t w_bs, const float* sw, int64_t sw_sn,
                                        int64_t sw_sk, int64_t sw_bs, int gran_n, const float* bias,
                                        int64_t bias_bs, void* y, sg_dtype y_dt, int64_t ldy, int64_t y_bs,
                                        sg_form form, hipStream_t stream);

sg_status sg_fp8_sparse24_gemm_groupwise_batched(int64_t L, int64_t M, int64_t N, int64_t K, const uint8_t* xq,
                                                 int64_t ldx, int64_t x_bs, const float* sx, int64_t sx_sm,
                                                 int64_t sx_sk, int64_t sx_bs, int gran_m, const uint8_t* wv,
                                                 int64_t ldwv, int64_t wv_bs, const uint8_t* wmeta,
                                                 int64_t ldwm, int64_t wm_bs, const float* sw, int64_t sw_sn,
                                                 int64_t sw_sk, int64_t sw_bs, int gran_n, const float* bias,
                                                 int64_t bias_bs, void* y, sg_dtype y_dt, int64_t ldy,
                                                 int64_t y_bs, sg_form form, hipStream_t stream);

sg_status sg_fp8_sparse24_gemm_groupwise_packed_batched(int64_t L, int64_t M, int64_t N, int64_t K,
                                                        const uint8_t* xq, int64_t ldx, int64_t x_bs,
                                                        const float* sx, int64_t sx_sm, int64_t sx_sk,
                                                        int64_t sx_bs, int gran_m, const uint8_t* wpacked,
                                                        int64_t wp_bs, const float* sw, int64_t sw_sn,
                                                        int64_t sw_sk, int64_t sw_bs, int gran_n,
                                                        const float* bias, int64_t bias_bs, void* y,
                                                        sg_dtype y_dt, int64_t ldy, int64_t y_bs, sg_form form,
                                                        hipStream_t stream);

/*
 * sg_w8a16_sparse24_gemm_groupwise -- weight-only 2:4 GEMM: bf16 activations
 * (not quantised) times a 2:4 weight of 8-bit codes with groupwise scales.
 * [T3258] jcaip's review (weight-only sparsity configs for int8 and float8
 * have no mixed-dtype kernel); [P2095] hwu36's comment (scale blocks):
 *   y[m, n] = sum_kb sw[n/gran_n, kb] * sum_{k in kb} x[m, k] * dec(w[n, k])  (+ bias[n])
 *   x     : [M, K] bf16 bits, leading dim ldx (elements).
 *   wv    : [N, K/2] codes, w_dt = SG_E4M3 or SG_I8, as produced by
 *           sg_sparse24_prune_compress then sg_fp8_quant_groupwise or
 *           sg_int8_quant_groupwise at gr = 128 (or 1), gc = 64; ld ldwv (bytes).
 *   wmeta : [N, K/8] metadata, ld ldwm.   sw, gran_n: as sg_fp8_gemm_groupwise.
 *   bias  : [N] fp32 or NULL.   y, y_dt, ldy, form: as sg_fp8_gemm_groupwise.
 * The codes are widened to bf16 (exactly) in registers and multiplied with the
 * sparse bf16 matrix-core instruction, which reads the metadata as stored.
 * Decode-sized M streams the weight once per call; large M runs on 256 x 128
 * output tiles staged in LDS (the faster of the two is picked per shape).
 * Requires K % 128 == 0, ldx >= K, ldwv >= K/2, ldwm >= K/8, ldx, ldwv, ldwm <
 * 2^24, ceil(M/16) <= 65535; x, wv 16-byte aligned, ldx * 2 and ldwv multiples
 * of 16, wmeta 16-byte aligned and ldwm a multiple of 16.
 */
sg_status sg_w8a16_sparse24_gemm_groupwise(int64_t M, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                                           const uint8_t* wv, int64_t ldwv, const uint8_t* wmeta, int64_t ldwm,
                                           sg_dtype w_dt, const float* sw, int64_t sw_sn, int64_t sw_sk, int gran_n,
                                           const float* bias, void* y, sg_dtype y_dt, int64_t ldy, sg_form form,
                                           hipStream_t stream);

/*
 * sg_w8a16_sparse24_gemm_groupwise_packed -- sg_w8a16_sparse24_gemm_groupwise
 * with the weight in the packed form of sg_sparse24_pack_gfx950 (a byte
 * permutation, so it packs int8 codes as it packs e4m3 ones).  The same
 * arithmetic in the same order: results equal the unpacked call's bit for
 * bit.  The packed chunks reach LDS as contiguous 1 KB and 256 B pieces per
 * wave instruction, where the row-major codes and metadata take 64-byte and
 * 16-byte pieces of 16 rows.  [T3258] jcaip's review; [I2029] klevzoff (the
 * hardware's layout straight into the mainloop).
 *   wpacked : sg_sparse24_packed_bytes(N, K) bytes, 16-byte aligned; w_dt =
 *             SG_E4M3 or SG_I8, the code type that was packed.
 *   other arguments as sg_w8a16_sparse24_gemm_groupwise.
 * Requires K % 128 == 0, ldx >= K, ldx < 2^24, (K / 128) * 16 * 1280 < 2^31,
 * ceil(M/16) <= 65535; x 16-byte aligned, ldx * 2 a multiple of 16.
 */
sg_status sg_w8a16_sparse24_gemm_groupwise_packed(int64_t M, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                                                  const uint8_t* wpacked, sg_dtype w_dt, const float* sw,
                                                  int64_t sw_sn, int64_t sw_sk, int gran_n, const float* bias,
                                                  void* y, sg_dtype y_dt, int64_t ldy, sg_form form,
                                                  hipStream_t stream);

/*
 * sg_w4a16_sparse24_gemm_groupwise -- the same with int4 weight codes: the
 * 2:4-compressed values quantised by sg_int4_quant_groupwise with gc = 64 (one
 * scale per row and 128-wide K block), two per byte.
 *   wv4 : [N, K/4] packed int4, element 2j in the low nibble of byte j; ld ldwv4 (bytes).
 *   sw  : (n, kb) at sw[n * sw_sn + kb * sw_sk].   Other arguments as the W8A16 GEMM.
 * Requires ldwv4 >= K/4, wv4 16-byte aligned and ldwv4 a multiple of 16.
 */
sg_status sg_w4a16_sparse24_gemm_groupwise(int64_t M, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                                           const uint8_t* wv4, int64_t ldwv4, const uint8_t* wmeta, int64_t ldwm,
                                           const float* sw, int64_t sw_sn, int64_t sw_sk, const float* bias,
                                           void* y, sg_dtype y_dt, int64_t ldy, sg_form form, hipStream_t stream);

/*
 * sg_sparse24_w4_packed_bytes -- bytes of the blocked form of an N x K 2:4
 * int4 weight: ceil(N/16) * (K/128) * 768, or -1 unless N >= 1, K >= 1 and
 * K % 128 == 0.
 *
 * sg_sparse24_pack_w4 -- the blocked form the weight-only kernels stream: for
 * 16-row block R and 128-wide K block kb the 768-byte chunk at
 * (R * K/128 + kb) * 768 holds local row lr's 32 code bytes of block kb at
 * lr*32 (as stored in wv4) and its 16 metadata bytes at 512 + lr*16; rows past
 * N (up to the next multiple of 16) are zero.  The chunking of
 * sg_sparse24_pack_gfx950 without the permutation inside a chunk ([T3258]
 * jcaip's review: the weight arranged by a packing kernel; [I2029] klevzoff).
 *   wv4   : [N, K/4] int4 codes as sg_w4a16_sparse24_gemm_groupwise takes them, ld ldwv4.
 *   wmeta : [N, K/8] metadata, ld ldwm.
 *   packed: sg_sparse24_w4_packed_bytes(N, K) bytes, 16-byte aligned, written fully.
 * Requires K % 128 == 0, ldwv4 >= K/4, ldwm >= K/8, multiples of 16; wv4,
 * wmeta 16-byte aligned.
 *
 * sg_w4a16_sparse24_gemm_groupwise_packed -- sg_w4a16_sparse24_gemm_groupwise
 * with the weight in that blocked form: the same arithmetic in the same order
 * (results equal the unpacked call's bit for bit), with each chunk reaching
 * LDS in 256-byte pieces per wave instruction instead of 32- and 16-byte row
 * pieces.
 *   wpacked : sg_sparse24_w4_packed_bytes(N, K) bytes, 16-byte aligned.
 *   other arguments as sg_w4a16_sparse24_gemm_groupwise.
 * Requires K % 128 == 0, ldx >= K, ldx < 2^24, (K / 128) * 16 * 768 < 2^31,
 * ceil(M/16) <= 65535; x 16-byte aligned, ldx * 2 a multiple of 16.
 */
int64_t sg_sparse24_w4_packed_bytes(int64_t N, int64_t K);

sg_status sg_sparse24_pack_w4(const uint8_t* wv4, int64_t ldwv4, const uint8_t* wmeta, int64_t ldwm, int64_t N,
                              int64_t K, uint8_t* packed, hipStream_t stream);

sg_status sg_w4a16_sparse24_gemm_groupwise_packed(int64_t M, int64_t N, int64_t K, const uint16_t* x, int64_t ldx,
                                                  const uint8_t* wpacked, const float* sw, int64_t sw_sn,
                                                  int64_t sw_sk, const float* bias, void* y, sg_dtype y_dt,
                                                  int64_t ldy, sg_form form, hipStream_t stream);

/*
 * sg_fp8_sparse24_gemm_groupwise_packed_grouped -- G problems that share N and
 * K but not M (e.g. tokens routed to experts): group g multiplies rows
 * row_off[g] .. row_off[g] + m_sizes[g] - 1 of X (row_off = prefix sums of
 * m_sizes) with its own packed weight wpacked + g * wp_bs (bytes), W scales
 * sw + g * sw_bs (floats) and bias + g * bias_bs, and writes the same rows of Y
 * (SG_OUT_Y) or columns of Y^T (SG_OUT_YT).  X scales are per X row (gran_m 1):
 * row r's scale of K block kb at sx[r * sx_sm + kb * sx_sk].  Every group follows
 * sg_fp8_sparse24_gemm_groupwise_packed (scales constant along K included); one
 * launch covers every group's 128-row tiles ([P2095] PR description: the L mode
 * of the scale layout; this form lets L's problems differ in M).
 *   m_sizes : HOST array of G entries >= 0 (0: an empty group).
 * Requires 1 <= G <= 64, sum(m_sizes) >= 1 as M and all requirements of the packed
 * entry point and of the batched forms' strides; bias may be NULL.
 */
sg_status sg_fp8_sparse24_gemm_groupwise_packed_grouped(int64_t G, const int64_t* m_sizes, int64_t N, int64_t K,
                                                        const uint8_t* xq, int64_t ldx, const float* sx,
                                                        int64_t sx_sm, int64_t sx_sk, const uint8_t* wpacked,
                                                        int64_t wp_bs, const float* sw, int64_t sw_sn,
                                                        int64_t sw_sk, int64_t sw_bs, int gran_n, const float* bias,
                                                        int64_t bias_bs, void* y, sg_dtype y_dt, int64_t ldy,
                                                        sg_form form, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_GEMM_LAYERS_AMD_SG_H */
