/*
 * mxfp4.h -- C ABI of libmxfp4: MXFP4 block quantization of bf16 tensors and
 * the block-scaled FP4 x FP4 ("a4w4") GEMM that consumes the blobs, for
 * MI355X (gfx950).
 *
 * Formats follow the OCP Microscaling Formats (MX) Specification v1.0:
 * 32-element blocks, one E8M0 scale byte per block (2^(byte-127), 0xFF = NaN)
 * and E2M1 elements (sign, 2 exponent bits, 1 mantissa bit: magnitudes
 * 0, .5, 1, 1.5, 2, 3, 4, 6).  Blob shapes, the 128-padding of the quantized
 * axis and the row/col option triplets follow the page
 * "primus_turbo_mxfp4_local.py" (ROCm docs download of Primus): its fake
 * (shape-only) dual-quantize op and the arguments of its dual-quantize and
 * FP4 GEMM calls.
 *
 * Conventions shared by every entry point:
 *  - All tensors live in device memory the caller owns; the library allocates
 *    nothing and keeps no state between calls.
 *  - Work is enqueued on `stream` (NULL = the null stream) and runs
 *    asynchronously.  Returned status reflects argument validation and
 *    the launch only; kernels never report errors after launch.
 *  - Validation happens before any launch.  Nothing is written on error, and
 *    there is no fallback path: an unsupported request is an error.
 *  - Sizes are element counts (int64_t); strides are in elements.
 *  - bf16 input x is M x N row-major with row stride ldx >= N elements.
 *  - Thread-safe: calls on different streams may overlap.  Calls that write
 *    the same output buffers race, as with any kernel.
 *
 * Error behaviour: every function returns an mx_status.  mx_last_error()
 * gives a human-readable detail string for the calling thread's last failed
 * call.
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>   /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mx_status {
    MX_SUCCESS = 0,
    MX_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, stride < row length */
    MX_ERR_MISALIGNED = 2,         /* pointer not 16-byte aligned, ldx or ldc not a multiple of 8 */
    MX_ERR_UNSUPPORTED = 3,        /* option combination not implemented (e.g. transposes) */
    MX_ERR_DEVICE_UNSUPPORTED = 4, /* current device is not gfx950 */
    MX_ERR_HIP = 5                 /* HIP runtime error; detail in mx_last_error() */
} mx_status;

/*
 * Blob layouts.
 *
 * MX_LAYOUT_CANONICAL -- the interchange layout of the fake dual-quantize op
 * on the page "primus_turbo_mxfp4_local.py".  For a blob of R rows quantized
 * along an axis of length L, L_pad = cdiv(L,128)*128:
 *   data:  R x L_pad/2 bytes, row-major; element k of a row in byte k/2,
 *          low nibble for even k, high nibble for odd k.
 *   scale: R x L_pad/32 bytes, row-major; byte b scales elements [32b, 32b+32).
 *   Row-wise blob of x: R = M, L = N.  Column-wise blob: R = N, L = M (the
 *   transpose of x, quantized along M).  Padding elements are +0 (nibble 0);
 *   pad-only blocks have scale byte 0.
 *
 * MX_LAYOUT_TILED -- this library's MFMA-native layout, written directly by
 * the quantizers and read by the GEMM with one 16-byte load per lane.
 * Rows are padded to R16 = cdiv(R,16)*16 (pad rows are zero bytes).
 *   data: 1024-byte atoms.  Atom (g, c) holds rows [16g, 16g+16) x k in
 *         [128c, 128c+128) and sits at byte (g * (L_pad/128) + c) * 1024.
 *         Inside an atom, lane = (r%16) + 16*((k%128)/32) owns bytes
 *         [16*lane, 16*lane+16); element k is in byte (k%32)/2 of that slice,
 *         low nibble for even k.  (Lane L holds the 32 elements of row L%16,
 *         k-block L/16: exactly the A/B operand of one 16x16x128 scaled MFMA.)
 *         Total R16 * L_pad/2 bytes.
 *   scale: 256-byte atoms.  Atom (g, h) holds the scales of rows [16g, 16g+16)
 *         and k-blocks [16h, 16h+16) and sits at byte
 *         (g * cdiv(L_pad,512) + h) * 256.  The scale of k-block kb of row r
 *         is byte 4*lane + (kb%16)/4 with lane = (r%16) + 16*(kb%4): each
 *         lane's dword packs its scales for 4 consecutive 128-wide k steps.
 *         Bytes beyond L_pad/32 blocks are 0.  Total R16 * cdiv(L_pad,512) * 16 bytes.
 */
typedef enum mx_layout {
    MX_LAYOUT_CANONICAL = 0,
    MX_LAYOUT_TILED = 1
} mx_layout;

typedef enum mx_dtype {
    MX_BF16 = 0,   /* bfloat16, round to nearest even */
    MX_F32 = 1     /* float32 (verification output of the GEMM) */
} mx_dtype;

/*
 * Per-direction quantization options; the row/col pairs mirror the flag
 * triplets of the dual-quantize op on the page "primus_turbo_mxfp4_local.py"
 * (2D block, stochastic rounding; its Hadamard and shuffle flags have no
 * counterpart here).
 *
 * use_2d_block: 0 = 32-element blocks along the quantized axis; 1 = aligned
 *   32x32 tiles of x share one scale (tile amax), replicated into every
 *   blob row the tile covers; blob shapes are unchanged.
 * use_sr: 0 = round to nearest, ties to even; 1 = stochastic rounding.  The
 *   element with row-major index n = index_base + i*N + j of the logical M x N
 *   tensor draws byte n%16 (little-endian) of Philox-4x32-10 (Salmon et al.,
 *   SC'11) with counter (lo32(n>>4), hi32(n>>4), tensor_id, dir) and key
 *   (lo32(seed), hi32(seed)); dir = 0 for the row-wise blob, 1 for the
 *   column-wise blob.  With neighbouring grid values lo <= v < hi of the scaled
 *   magnitude v, it rounds up iff byte < floor(256*(v-lo)/(hi-lo)).
 * rht: 0 = off; otherwise each 32-element block along the quantized axis is
 *   replaced, before its scale and codes are taken, by the random Hadamard
 *   transform y = c * H32 * D * x evaluated in fp32 (the page
 *   "primus_turbo_mxfp4_local.py" switches "rht" on for the column-wise blobs
 *   of the activation and the gradient, the two wgrad operands, and defines
 *   nothing more; this definition is the library's): D negates position p
 *   when bit p of the first word of Philox-4x32-10 at counter (0, 0, 0, 2),
 *   key (rht, 0) is set; H32 = Sylvester Hadamard matrix, applied as a fast
 *   Walsh-Hadamard transform over position bits 0..4, each (a, b) -> (a + b,
 *   a - b) rounded to fp32; c = fp32(1/sqrt(32)).  Pads count as +0 before
 *   the transform, so pad positions of a block that holds real elements get
 *   codes too.  With use_sr their byte uses the same index formula on padded
 *   coordinates in a counter space of their own: counter word 3 is 2 + dir,
 *   so no pad shares a byte with a real element (and, for the row-wise blob
 *   with N >= 64 and for the column-wise blob, with another pad).  Both
 *   operands of a GEMM must be transformed with the same
 *   rht value along the shared K axis: (H D)^T (H D) c^2 ~= I leaves the
 *   product unchanged.  Not combined with use_2d_block (MX_ERR_UNSUPPORTED).
 * The scale never depends on use_sr.  NULL options = all zero.
 */
typedef struct mx_quant_opts {
    uint32_t use_2d_block;
    uint32_t use_sr;
    uint64_t seed;
    uint32_t tensor_id;
    uint64_t index_base;   /* global element-index offset of x (shards, chunks) */
    uint32_t rht;          /* random Hadamard transform seed, 0 = off */
} mx_quant_opts;

/*
 * Byte sizes of one blob (rows blob rows, quantized along `length`) in
 * `layout`.  Either output pointer may be NULL.  Canonical sizes equal the
 * fake dual-quantize op's shapes: rows * L_pad/2 and rows * L_pad/32.
 * Errors: MX_ERR_INVALID_ARGUMENT (negative size), MX_ERR_UNSUPPORTED (layout).
 */
mx_status mx_blob_bytes(int64_t rows, int64_t length, mx_layout layout,
                        size_t *data_bytes, size_t *scale_bytes);

/*
 * Row-wise MXFP4 quantization of x (M x N bf16, stride ldx): blocks of 32
 * along N, the row-only packer a forward pass with no backward behind it needs
 * (page "Primus PR 1107", the commit that packs rows only when no backward will
 * read the columns; the caller decides, the library never infers grad mode).
 * Outputs: q (data) and s (scales) of the row-wise blob (R = M, L = N) in
 * `layout`, sized by mx_blob_bytes.  Every output byte is written, padding
 * included.  M == 0 or N == 0 is a no-op.
 * Requires x and the outputs 16-byte aligned and ldx % 8 == 0.
 * Errors: INVALID_ARGUMENT, MISALIGNED, UNSUPPORTED, DEVICE_UNSUPPORTED, HIP.
 */
mx_status mx_quantize_rowwise(const void *x, int64_t M, int64_t N, int64_t ldx,
                              const mx_quant_opts *opts, mx_layout layout,
                              void *q, void *s, hipStream_t stream);

/*
 * Dual quantization: the row-wise blob (R = M, L = N) and the column-wise blob
 * (R = N, L = M: x transposed, blocks of 32 along M) from one read of x, as the
 * dual-quantize op on the page "primus_turbo_mxfp4_local.py" returns them
 * (row data, row scale, col data, col scale).  Options are per direction.
 * Same requirements and errors as mx_quantize_rowwise.
 */
mx_status mx_quantize_dual(const void *x, int64_t M, int64_t N, int64_t ldx,
                           const mx_quant_opts *row_opts, const mx_quant_opts *col_opts,
                           mx_layout layout, void *q_row, void *s_row,
                           void *q_col, void *s_col, hipStream_t stream);

/*
 * Quantizer with a multiply prologue: quantizes y = bf16(x * g) (elementwise,
 * each product formed in fp32 and rounded to bf16 nearest-even) exactly as
 * mx_quantize_dual / mx_quantize_rowwise would quantize a stored y, but y is
 * formed in the staging read and never written to memory.  It fuses the
 * last elementwise step of a producer's backward into the packer, the
 * pattern of the page "Primus PR 1107" (its QKV packer computes the
 * gradient during its staging read instead of reading it back from HBM);
 * that page's norm+RoPE backward itself is not part of this library, g
 * carries any elementwise factor (an activation derivative, a mask, a gate).
 * x: M x N bf16, stride ldx; g: M x N bf16, stride ldg.  q_col = s_col =
 * NULL: row-wise blob only.  Options as mx_quantize_dual except rht
 * (MX_ERR_UNSUPPORTED).  Same alignment rules for g as for x.
 * Errors: INVALID_ARGUMENT, MISALIGNED, UNSUPPORTED, DEVICE_UNSUPPORTED, HIP.
 */
mx_status mx_quantize_dual_mul(const void *x, const void *g, int64_t M, int64_t N, int64_t ldx, int64_t ldg,
                               const mx_quant_opts *row_opts, const mx_quant_opts *col_opts,
                               mx_layout layout, void *q_row, void *s_row,
                               void *q_col, void *s_col, hipStream_t stream);

/*
 * Block-scaled FP4 x FP4 GEMM with fp32 accumulation:
 *   C[i][j] = sum_k A[i][k] * B[j][k]   (i < M, j < N, k over the padded K)
 * where A (M rows) and B (N rows) are blobs quantized along K and each
 * element is e2m1(code) * 2^(scale-127).  This is the NT call that the
 * forward (X_row . W_row^T), dgrad (dY_row . W_col^T) and wgrad
 * (dY_col . X_col^T) of the MXFP4 linear on the page
 * "primus_turbo_mxfp4_local.py" all make.
 * transA must be 0 and transB must be 1 (both operands K-contiguous); any
 * other combination returns MX_ERR_UNSUPPORTED.  layout must be
 * MX_LAYOUT_TILED.  K is the logical K; the blobs carry cdiv(K,128)*128.
 * C is M x N row-major with stride ldc >= N, out_dtype MX_BF16 (round to
 * nearest even; overflow to +-Inf) or MX_F32.  A NaN scale byte yields NaN in
 * the affected outputs (hardware-defined propagation).  M == 0 or N == 0 is a
 * no-op; K == 0 writes zeros.
 * Requires 16-byte aligned pointers and ldc % 8 == 0.  Each operand's tiled
 * data blob (cdiv(rows,16)*16 * K_pad/2 bytes) must stay below 2 GiB: the
 * kernels address it with 32-bit buffer offsets (MX_ERR_UNSUPPORTED
 * otherwise, before anything is launched; split the product instead).
 */
mx_status mx_gemm_a4w4(int transA, int transB, int64_t M, int64_t N, int64_t K,
                       const void *A, const void *A_scale,
                       const void *B, const void *B_scale,
                       mx_layout layout, mx_dtype out_dtype,
                       void *C, int64_t ldc, hipStream_t stream);

/*
 * mx_gemm_a4w4 with the linear layer's bias added in the epilogue:
 *   C[i][j] = round(sum_k A[i][k] * B[j][k] + bias[j])
 * bias: N bf16 values (device pointer, 16-byte aligned, caller-owned), added
 * to the fp32 accumulator before the one rounding to out_dtype.  This fuses
 * the separate `output + bias` that the parallel linear layers on the page
 * "primus_turbo_mxfp4_local.py" apply after the FP4 GEMM (there the sum is
 * rounded to bf16 twice; here once).  K == 0 writes bias broadcast over the
 * rows.  Arguments and errors otherwise as mx_gemm_a4w4 (NULL bias:
 * MX_ERR_INVALID_ARGUMENT; misaligned bias: MX_ERR_MISALIGNED).
 */
mx_status mx_gemm_a4w4_bias(int transA, int transB, int64_t M, int64_t N, int64_t K,
                            const void *A, const void *A_scale,
                            const void *B, const void *B_scale,
                            mx_layout layout, mx_dtype out_dtype, const void *bias,
                            void *C, int64_t ldc, hipStream_t stream);

/*
 * ---- Hybrid backward: tensorwise FP8 (E5M2) ----
 * The page "primus_turbo_mxfp4_local.py" offers a backward that re-quantizes
 * the saved bf16 activation, weight and gradient to FP8 E5M2 with one scale
 * per tensor and runs FP8 GEMMs that multiply by both inverse scales.  E5M2
 * per the OCP 8-bit floating point spec (bias 15, 2 mantissa bits, largest
 * finite 57344).  The scale rule is the library's reading (the quantizer's
 * code is not on the pages):
 *   amax = max |x|;  scale = 57344 / amax as an fp32 division (1 if amax is 0
 *   or not finite);  code = E5M2 of the fp32 product x * scale, round to
 *   nearest even, finite overflow saturating to 57344, Inf kept, NaN -> 0x7F
 *   with its sign;  scale_inv = 1 / scale (fp32).
 * FP8 blobs: rows x L_pad bytes (L_pad = cdiv(length,128)*128, pads code 0).
 *   MX_LAYOUT_CANONICAL: row-major.  MX_LAYOUT_TILED: rows padded to 16;
 *   atom (row group g, k-step s of 64) = 1 KB at (g * L_pad/64 + s) * 1024;
 *   lane = (r%16) + 16*((k%64)/16) owns bytes [16 lane, 16 lane + 16),
 *   element k at byte k%16.
 */

/* Bytes of one FP8 blob.  Errors: MX_ERR_INVALID_ARGUMENT, MX_ERR_UNSUPPORTED. */
mx_status mx_fp8_blob_bytes(int64_t rows, int64_t length, mx_layout layout, size_t *bytes);

/*
 * Tensorwise E5M2 quantization of x (M x N bf16, row stride ldx).  q_row
 * (M rows along N) and q_col (N rows along M, the transpose) may each be NULL
 * (not both).  info: device float[2], caller-owned: receives amax in [0] and
 * scale_inv in [1]; [0] is also the reduction's working word, so calls that
 * share an info buffer must not overlap.  Three launches on `stream`.
 * Errors: MX_ERR_INVALID_ARGUMENT (NULL x/info, both outputs NULL, negative
 * sizes, ldx < N), MX_ERR_MISALIGNED (x, outputs or info not 16-byte
 * aligned, ldx % 8), MX_ERR_UNSUPPORTED (layout), MX_ERR_DEVICE_UNSUPPORTED,
 * MX_ERR_HIP.  M == 0 or N == 0 is a no-op.
 */
mx_status mx_quantize_fp8_tw(const void *x, int64_t M, int64_t N, int64_t ldx, mx_layout layout,
                             void *q_row, void *q_col, float *info, hipStream_t stream);

/*
 * C = (A . B^T) * a_scale_inv[0] * b_scale_inv[0] on tensorwise E5M2 blobs
 * (MX_LAYOUT_TILED, both K-contiguous: the NT form of the hybrid backward's
 * dgrad dY_row . W_col^T and wgrad dY_col . X_col^T), fp32 accumulation,
 * bf16 (RNE) or fp32 output.  a_scale_inv / b_scale_inv: device pointers to
 * the inverse scales (the [1] entries of the quantizer's info), read by the
 * kernel, so no host synchronization.  Arguments and errors otherwise as
 * mx_gemm_a4w4 (each FP8 operand blob, cdiv(rows,16)*16 * K_pad bytes, must
 * stay below 2 GiB).
 */
mx_status mx_gemm_f8_tw(int transA, int transB, int64_t M, int64_t N, int64_t K,
                        const void *A, const float *a_scale_inv,
                        const void *B, const float *b_scale_inv,
                        mx_layout layout, mx_dtype out_dtype,
                        void *C, int64_t ldc, hipStream_t stream);

/* ------------------------------------------------------------------ MXFP6
 *
 * MXFP6: the same 32-element blocks and E8M0 scales with 6-bit elements.
 * The pages name an MXFP6 Flux training campaign (Primus PR 1107) and define
 * none of it; the formats are the OCP MX v1.0 FP6 elements (sec. 5.3.2):
 *   MX_FP6_E2M3: sign, 2 exponent bits (bias 1), 3 mantissa bits; magnitudes
 *     k/8 for k < 8 (subnormal), up to 7.5; emax_elem = 2.
 *   MX_FP6_E3M2: sign, 3 exponent bits (bias 3), 2 mantissa bits; magnitudes
 *     k/16 for k < 4 (subnormal), up to 28; emax_elem = 4.
 * Code = sign << 5 | exponent << mbits | mantissa; no Inf/NaN codes.  Scale
 * byte = max(E(amax) - emax_elem, 0) (0xFF and all-zero codes for a block
 * holding Inf/NaN); elements round to nearest even, or stochastically by the
 * rule of mx_quant_opts, saturating at the largest magnitude.
 *
 * Blob layouts (R rows, quantized axis L, L_pad = cdiv(L,128)*128):
 *   canonical data: R x L_pad*3/4 bytes; element k of a row occupies bits
 *     [6k, 6k+6) of the row read as a little-endian bit string (a 32-element
 *     block is 24 bytes); scales as MX_LAYOUT_CANONICAL.
 *   tiled data: 1536-byte atoms; atom (g, c) = rows [16g, 16g+16) x k in
 *     [128c, 128c+128) at byte (g * (L_pad/128) + c) * 1536.  Lane
 *     (r%16) + 16*((k%128)/32) owns the 24 canonical bytes of its row's
 *     k-block: bytes 0..15 at 16*lane, bytes 16..23 at 1024 + 8*lane (the
 *     six-register operand of the f8f6f4 matrix instruction, split so that
 *     both parts load aligned).  Rows padded to cdiv(R,16)*16 with zeros;
 *     scales exactly as MX_LAYOUT_TILED.
 */
typedef enum mx_fp6_format {
    MX_FP6_E2M3 = 2,
    MX_FP6_E3M2 = 3
} mx_fp6_format;

/* Byte sizes of one MXFP6 blob in `layout` (either output may be NULL).
 * Errors: MX_ERR_INVALID_ARGUMENT (negative size), MX_ERR_UNSUPPORTED (layout). */
mx_status mx_fp6_blob_bytes(int64_t rows, int64_t length, mx_layout layout,
                            size_t *data_bytes, size_t *scale_bytes);

/*
 * MXFP6 quantization of x (M x N bf16, stride ldx): the row-wise blob (R = M,
 * L = N) in row_fmt, and, when q_col / s_col are given, the column-wise blob
 * (R = N, L = M) in col_fmt from the same read of x (q_col = s_col = NULL:
 * row-wise only, as a forward pass with no backward behind it needs).  Options
 * per direction as for mx_quantize_dual, except rht (MX_ERR_UNSUPPORTED).
 * Outputs sized by mx_fp6_blob_bytes; every output byte is written.
 * Requires x and the outputs 16-byte aligned and ldx % 8 == 0.  M == 0 or
 * N == 0 is a no-op.
 * Errors: INVALID_ARGUMENT, MISALIGNED, UNSUPPORTED (format, layout, rht),
 * DEVICE_UNSUPPORTED, HIP.
 */
mx_status mx_quantize_fp6(const void *x, int64_t M, int64_t N, int64_t ldx,
                          int row_fmt, const mx_quant_opts *row_opts,
                          int col_fmt, const mx_quant_opts *col_opts,
                          mx_layout layout, void *q_row, void *s_row,
                          void *q_col, void *s_col, hipStream_t stream);

/*
 * Block-scaled FP6 x FP6 GEMM with fp32 accumulation on tiled MXFP6 blobs:
 *   C[i][j] = sum_k A[i][k] * B[j][k],  element = fp6(code) * 2^(scale-127)
 * with A in fmt_a and B in fmt_b (MX_FP6_E2M3 or MX_FP6_E3M2, mixed allowed).
 * Arguments, layout (MX_LAYOUT_TILED of the MXFP6 blobs), output and errors
 * as mx_gemm_a4w4; MX_ERR_UNSUPPORTED also for an unknown format and when an
 * operand blob (cdiv(rows,16)*16 * K_pad*3/4 bytes) reaches 2 GiB.  The matrix instruction's sum of 64
 * E3M2 x E3M2 products keeps fewer bits than fp32 (measured on MI355X: error
 * up to about 2^-14 of the sum of |products|); E2M3 operands sum exactly.
 */
mx_status mx_gemm_fp6(int transA, int transB, int64_t M, int64_t N, int64_t K,
                      int fmt_a, const void *A, const void *A_scale,
                      int fmt_b, const void *B, const void *B_scale,
                      mx_layout layout, mx_dtype out_dtype,
                      void *C, int64_t ldc, hipStream_t stream);

/*
 * Device-side layout conversion of one blob (rows, length) between the two
 * layouts, asynchronous on `stream`: the tiled layout is the one this
 * library's GEMM reads, the canonical one the interchange shapes of the page
 * "primus_turbo_mxfp4_local.py" (its fake dual-quantize op), so blobs made
 * elsewhere can be fed in and blobs made here handed out.  to_tiled = 1:
 * canonical -> tiled (padding rows and unused scale slots are written as 0);
 * 0: tiled -> canonical.  Device pointers, caller-owned, sized by
 * mx_blob_bytes for their layout; source and destination must not overlap.
 * Errors: MX_ERR_INVALID_ARGUMENT (negative shape, NULL pointer),
 * MX_ERR_MISALIGNED (data or scale pointers not 16-byte aligned),
 * MX_ERR_DEVICE_UNSUPPORTED, MX_ERR_HIP (launch failure).  rows == 0 or
 * length == 0 is a no-op.
 */
mx_status mx_layout_convert(int to_tiled, int64_t rows, int64_t length, const void *q_src,
                            const void *s_src, void *q_dst, void *s_dst, hipStream_t stream);

/*
 * Host-side layout conversion of one blob (rows, length) between the two
 * layouts; plain host pointers, synchronous.  to_tiled = 1: canonical ->
 * tiled; 0: tiled -> canonical.  Destination buffers are sized by
 * mx_blob_bytes for their layout.
 */
mx_status mx_layout_convert_host(int to_tiled, int64_t rows, int64_t length,
                                 const void *q_src, const void *s_src,
                                 void *q_dst, void *s_dst);

/*
 * Device dequantization (a test aid): out[r][k] = element value as float32
 * for r < rows, k < length (logical, unpadded), row stride ldo >= length.
 * Values are exact in float32 for scale bytes <= 252 (the quantizers never
 * emit more for finite input); byte 0xFF gives NaN.
 */
mx_status mx_dequantize(const void *q, const void *s, int64_t rows, int64_t length,
                        mx_layout layout, void *out_f32, int64_t ldo, hipStream_t stream);

/*
 * Measurement aid (not a step of the path): the sustained rate of the
 * block-scaled matrix instruction the GEMMs issue
 * (V_MFMA_SCALE_F32_32X32X64_F8F6F4 with unit scales) for element formats
 * fmt_a x fmt_b (0 E4M3, 1 E5M2, 2 E2M3, 3 E3M2, 4 E2M1: the instruction's own
 * codes), with no memory traffic in its loop, i.e. the ceiling that the
 * chip's clock under matrix work leaves for GEMMs on operands like the given
 * ones (the dense specs assume 2.4 GHz throughout).
 *   operands: device buffer of 64 x 64 uint32 words (16 KB, caller-owned,
 *     16-byte aligned): lane L of every wave uses words [64 L, 64 L + 64) as
 *     4 operand pairs (pair k: A = words 16k..16k+7, B = words 16k+8..16k+15;
 *     an E2M1 operand uses the first 4 words of its 8, an FP6 one the first 6),
 *     one per accumulator chain.
 *   workgroups: >= 1 workgroups of 8 waves (two per SIMD); each wave issues
 *     4 * iters instructions, so one launch performs
 *     workgroups * 8 * 4 * iters * 131072 flops.
 *   out: device float[workgroups * 512] (caller-owned): one sum per lane,
 *     stored so that the work is kept.
 * Asynchronous on `stream`.  Errors: MX_ERR_UNSUPPORTED (format code),
 * MX_ERR_INVALID_ARGUMENT (NULL, workgroups < 1, iters < 1),
 * MX_ERR_MISALIGNED, MX_ERR_DEVICE_UNSUPPORTED, MX_ERR_HIP.
 */
mx_status mx_measure_mfma(int fmt_a, int fmt_b, const void *operands, int workgroups, int64_t iters, float *out,
                          hipStream_t stream);

/*
 * 1 if device `device` is gfx950 (the only target), else 0.  The page
 * "primus_turbo_mxfp4_local.py" has check_mxfp4_support() decide, when a
 * layer is built, whether the FP4 path can run at all, and refuses to build
 * the layer otherwise; this is that check.  Every entry point that launches
 * work repeats it (cached per device) and returns MX_ERR_DEVICE_UNSUPPORTED
 * instead of launching on another device.
 */
int mx_device_supported(int device);

/*
 * Test aid: replaces the device query of every entry point by a fixed
 * architecture name, so that the failure paths can be exercised on any
 * machine.  arch = NULL restores the real query.  With a name other than
 * "gfx950", calls fail with MX_ERR_DEVICE_UNSUPPORTED after validation; with
 * "gfx950" on a machine whose runtime has no usable device, the launch fails
 * and the call returns MX_ERR_HIP with HIP's error text.  The name applies to
 * every device index and to mx_device_supported.  Process-wide; not for use
 * while other threads call the library.  Errors: MX_ERR_INVALID_ARGUMENT (a
 * name of 64 characters or more).
 */
mx_status mx_set_device_arch_override(const char *arch);

/* Static name of a status code. */
const char *mx_status_string(mx_status status);

/* Detail of the calling thread's last failed call ("" if none). */
const char *mx_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
