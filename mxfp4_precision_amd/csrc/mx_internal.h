// Internal declarations shared by the libmxfp4 translation units (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mxfp4.h"

namespace mx {

constexpr int64_t kBlock = 32;   // elements per scale block
constexpr int64_t kPad = 128;    // quantized-axis padding

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t padded(int64_t n) { return cdiv(n, kPad) * kPad; }

// Per-direction options in the form the kernels take them.
struct DirOpts {
    uint32_t use_2d;
    uint32_t use_sr;
    uint32_t key0, key1;        // Philox key = seed
    uint32_t tensor_id;
    uint64_t index_base;
    uint32_t rht;               // random Hadamard transform seed, 0 = off
    uint32_t fmt;               // MXFP6 element format (2 = E2M3, 3 = E3M2); unused for MXFP4
};

struct QuantArgs {
    const uint16_t *x;
    int64_t M, N, ldx;
    const uint16_t *g;          // second factor of the multiply prologue (same shape), or NULL
    int64_t ldg;
    int64_t M_pad, N_pad;       // padded quantized axes (col blob, row blob)
    DirOpts row, col;
    uint32_t sr_pairs;          // 1: N and both index bases are multiples of 16
    uint8_t *q_row, *s_row, *q_col, *s_col;
    int64_t row_tile0;          // first 128-row tile of this launch (set by the launchers)
};

// Grid dimension y of one launch holds at most 65536 workgroups on gfx950
// (hipDeviceAttributeMaxGridDimY); the quantize launchers cover taller inputs
// with several launches of kMaxRowTiles row tiles each.
constexpr int64_t kMaxRowTiles = 65535;

// Kernel launchers (quantize.hip, gemm.hip, convert.hip, dequantize.hip).  They assume validated arguments.
hipError_t launch_quantize(const QuantArgs &a, bool dual, mx_layout layout, hipStream_t stream);
hipError_t launch_quantize_fp6(const QuantArgs &a, bool dual, mx_layout layout, hipStream_t stream);
hipError_t launch_quantize_mul(const QuantArgs &a, bool dual, mx_layout layout, hipStream_t stream);
hipError_t launch_gemm_fp6(int64_t M, int64_t N, int64_t K, int fmt_a, const uint8_t *A, const uint8_t *As,
                           int fmt_b, const uint8_t *B, const uint8_t *Bs, mx_dtype out_dtype, void *C, int64_t ldc,
                           hipStream_t stream);
hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t *A, const uint8_t *As,
                       const uint8_t *B, const uint8_t *Bs, const uint16_t *bias, mx_dtype out_dtype, void *C,
                       int64_t ldc, hipStream_t stream);
int device_cu_count();   // compute units of the current device (cached), 0 if unknown
hipError_t launch_gemm_fp8(int64_t M, int64_t N, int64_t K, const uint8_t *A, const float *a_scale_inv,
                           const uint8_t *B, const float *b_scale_inv, mx_dtype out_dtype, void *C, int64_t ldc,
                           hipStream_t stream);
hipError_t launch_quantize_fp8(const uint16_t *x, int64_t M, int64_t N, int64_t ldx, mx_layout layout,
                               uint8_t *q_row, uint8_t *q_col, float *info, hipStream_t stream);
hipError_t launch_layout_convert(bool to_tiled, int64_t rows, int64_t length, const uint8_t *q_src,
                                 const uint8_t *s_src, uint8_t *q_dst, uint8_t *s_dst, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t length,
                             mx_layout layout, float *out, int64_t ldo, hipStream_t stream);
hipError_t launch_measure_mfma(int fmt_a, int fmt_b, const void *ops, int workgroups, int64_t iters, float *out,
                               hipStream_t stream);

}  // namespace mx
