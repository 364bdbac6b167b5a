// Tensorwise FP8 E5M2 quantization for the hybrid backward of the page
// "primus_turbo_mxfp4_local.py": the saved bf16 tensors are re-quantized to
// E5M2 with one scale per tensor and the FP8 GEMM multiplies by both inverse
// scales.  E5M2 per the OCP 8-bit floating point spec (bias 15, 2 mantissa
// bits, largest finite 57344).  The scale rule is not on the pages; this
// library's: amax = max |x| over the tensor, scale = 57344 / amax (fp32
// division; 1 if amax is 0 or not finite), code = E5M2 of the fp32 product
// x * scale rounded to nearest even, finite overflow saturating to 57344,
// Inf kept, NaN -> 0x7F with its sign; scale_inv = 1 / scale (fp32).
//
// Three launches on the caller's stream: clear the amax word, reduce |x| into
// it (atomic max on the fp32 bits, which order like the values for
// non-negative numbers and put NaN above Inf), then quantize, each workgroup
// deriving the scale from the reduced amax; one thread stores scale_inv.  A
// tensor with a finite amax is encoded by the hardware converter (every
// product then lies where it rounds as the rule above), any other by the
// software encode.
// Output: row-wise blob (M rows along N) and/or column-wise blob (N rows along
// M, the transpose), K axis padded to a multiple of 128 with code 0; layout
// canonical (rows x L_pad bytes) or tiled (16-row groups, 64-element k-steps:
// atom (g, s) = 1 KB at (g * L_pad/64 + s) * 1024, lane (r%16) + 16*((k%64)/16)
// owns 16 bytes, element k at byte k%16; the MFMA operand layout of
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 with FP8 inputs).

#include "mx_internal.h"

namespace mx {
namespace {

constexpr int kTile = 64;   // 64 x 64 elements per workgroup

__global__ void fp8_clear_kernel(float *info) {
    if (threadIdx.x == 0 && blockIdx.x == 0) reinterpret_cast<uint32_t *>(info)[0] = 0u;
}

// amax of |x| into info[0] (fp32 bits of a bf16 magnitude, atomic max).  Each
// thread walks 16-byte chunks (row i, columns jc*8..) with a grid stride; the
// (row, chunk) position advances by adding the stride's quotient and
// remainder instead of dividing per chunk.  The block reduces in LDS and
// issues one atomic, skipped when the stored maximum is already as large.
__global__ __launch_bounds__(256) void fp8_amax_kernel(const uint16_t *__restrict__ x, int64_t M, int64_t N,
                                                       int64_t ldx, float *info) {
    __shared__ uint32_t s_max[4];
    const int64_t cpr = cdiv(N, 8);
    const int64_t total = M * cpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t sq = stride / cpr, sr = stride % cpr;
    int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t i = c / cpr, jc = c % cpr;
    uint32_t m = 0;
    for (; c < total; c += stride) {
        const int64_t j0 = jc * 8;
        const uint16_t *p = x + i * ldx + j0;
        if (j0 + 8 <= N) {
            const uint4 v = *reinterpret_cast<const uint4 *>(p);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = w[e] & 0x7FFFu, hi = (w[e] >> 16) & 0x7FFFu;
                m = m > lo ? m : lo;
                m = m > hi ? m : hi;
            }
        } else {
            for (int64_t j = j0; j < N; ++j) {
                const uint32_t b = p[j - j0] & 0x7FFFu;
                m = m > b ? m : b;
            }
        }
        jc += sr;
        i += sq;
        if (jc >= cpr) {
            jc -= cpr;
            ++i;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
        m = m > o ? m : o;
    }
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = s_max[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) m = m > s_max[w] ? m : s_max[w];
        uint32_t *word = reinterpret_cast<uint32_t *>(info);
        const uint32_t bits = m << 16;
        if (bits > __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(word, bits);
    }
}

// E5M2 code of an fp32 value (see the file comment).
__device__ __forceinline__ uint32_t e5m2_code(float v) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return sign | 0x7Fu;              // NaN
    if (a == 0x7F800000u) return sign | 0x7Cu;             // Inf
    uint32_t code;
    if (a >= 0x38800000u) {                                // |v| >= 2^-14: E5M2 normal range
        const uint32_t r = (a + 0xFFFFFu + ((a >> 21) & 1u)) >> 21;   // fp32 exponent and 2 mantissa bits, RNE
        const int32_t e = (int32_t)(r >> 2) - 127 + 15;
        code = e > 30 ? 0x7Bu : (((uint32_t)e << 2) | (r & 3u));
        code = code > 0x7Bu ? 0x7Bu : code;                // saturate finite overflow
    } else {                                               // subnormal spacing 2^-16, RNE (4 -> 2^-14)
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 65536.0f);
    }
    return sign | code;
}

// tiled byte offset of 16-element chunk (r, k..k+15), k % 16 == 0
__device__ __forceinline__ int64_t fp8_tiled_off(int64_t r, int64_t k, int64_t Lp) {
    return ((r / 16) * (Lp / 64) + k / 64) * 1024 + ((r % 16) + 16 * ((k % 64) / 16)) * 16;
}

template <int LAYOUT>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(const uint16_t *__restrict__ x, int64_t M, int64_t N,
                                                           int64_t ldx, const float *__restrict__ info_in,
                                                           float *info_out, uint8_t *__restrict__ q_row,
                                                           uint8_t *__restrict__ q_col, int64_t tile0) {
    __shared__ __attribute__((aligned(16))) uint8_t s_t[kTile][kTile + 16];   // transposed codes
    const float amax = __uint_as_float(reinterpret_cast<const uint32_t *>(info_in)[0]);
    const bool finite = __float_as_uint(amax) < 0x7F800000u;
    const float scale = (finite && amax > 0.0f) ? __fdiv_rn(57344.0f, amax) : 1.0f;
    if (tile0 == 0 && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) info_out[1] = __frcp_rn(scale);

    const int64_t N_pad = padded(N), M_pad = padded(M);
    const int64_t r0 = ((int64_t)blockIdx.y + tile0) * kTile, c0 = (int64_t)blockIdx.x * kTile;
    const int tr = threadIdx.x >> 2, tc = (threadIdx.x & 3) * 16;   // 64 rows x 4 chunks of 16
    const int64_t i = r0 + tr, j0 = c0 + tc;
    uint32_t codes[4] = {0u, 0u, 0u, 0u};                             // 16 bytes, element e in byte e
    if (i < M) {
        const uint16_t *p = x + i * ldx + j0;
        uint32_t w[8];
        if (j0 + 16 <= N) {
            const uint4 v0 = *reinterpret_cast<const uint4 *>(p);
            const uint4 v1 = *reinterpret_cast<const uint4 *>(p + 8);
            w[0] = v0.x; w[1] = v0.y; w[2] = v0.z; w[3] = v0.w; w[4] = v1.x; w[5] = v1.y; w[6] = v1.z; w[7] = v1.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t lo = j0 + 2 * e < N ? p[2 * e] : 0u, hi = j0 + 2 * e + 1 < N ? p[2 * e + 1] : 0u;
                w[e] = lo | (hi << 16);
            }
        }
        if (finite) {
            // a finite tensor: every product is finite and at most 57344 in
            // magnitude (plus rounding), where V_CVT_PK_BF8_F32 rounds exactly
            // as e5m2_code (compared on MI355X over every fp32 pattern: it
            // differs only for NaN and for magnitudes of 61440 and above, which
            // it turns into Inf instead of saturating)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = w[2 * k], hi = w[2 * k + 1];
                const float v0 = __uint_as_float(lo << 16) * scale, v1 = __uint_as_float(lo & 0xFFFF0000u) * scale;
                const float v2 = __uint_as_float(hi << 16) * scale, v3 = __uint_as_float(hi & 0xFFFF0000u) * scale;
                const int c01 = __builtin_amdgcn_cvt_pk_bf8_f32(v0, v1, 0, false);
                codes[k] = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(v2, v3, c01, true);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t b = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                const float v = __uint_as_float(b << 16) * scale;    // fp32 product, one rounding
                codes[e >> 2] |= e5m2_code(v) << (8 * (e & 3));
            }
        }
    }
    // row-wise blob: row i, elements j0..j0+15
    if (q_row && j0 < N_pad) {
        const int64_t rows_out = LAYOUT == MX_LAYOUT_TILED ? cdiv(M, 16) * 16 : M;
        if (i < rows_out) {
            const int64_t off = LAYOUT == MX_LAYOUT_TILED ? fp8_tiled_off(i, j0, N_pad) : i * N_pad + j0;
            *reinterpret_cast<uint4 *>(q_row + off) = uint4{codes[0], codes[1], codes[2], codes[3]};
        }
    }
    if (q_col) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s_t[tc + e][tr] = (uint8_t)(codes[e >> 2] >> (8 * (e & 3)));
        __syncthreads();
        // column-wise blob: blob row = x column c0 + tr, elements (x rows) r0 + tc .. +15
        const int64_t br = c0 + tr, bk = r0 + tc;
        const int64_t rows_out = LAYOUT == MX_LAYOUT_TILED ? cdiv(N, 16) * 16 : N;
        if (br < rows_out && bk < M_pad) {
            const uint4 v = *reinterpret_cast<const uint4 *>(&s_t[tr][tc]);
            const int64_t off = LAYOUT == MX_LAYOUT_TILED ? fp8_tiled_off(br, bk, M_pad) : br * M_pad + bk;
            *reinterpret_cast<uint4 *>(q_col + off) = v;
        }
    }
}

}  // namespace

hipError_t launch_quantize_fp8(const uint16_t *x, int64_t M, int64_t N, int64_t ldx, mx_layout layout,
                               uint8_t *q_row, uint8_t *q_col, float *info, hipStream_t stream) {
    hipLaunchKernelGGL(fp8_clear_kernel, dim3(1), dim3(64), 0, stream, info);
    const int64_t chunks = M * cdiv(N, 8);
    const unsigned ablocks = (unsigned)(cdiv(chunks, 256) < 1024 ? cdiv(chunks, 256) : 1024);
    hipLaunchKernelGGL(fp8_amax_kernel, dim3(ablocks), dim3(256), 0, stream, x, M, N, ldx, info);
    // the grids cover both padded axes: pad columns of the row blob, pad rows
    // of the column blob; one launch per kMaxRowTiles row tiles (grid y is limited)
    const int64_t row_tiles = padded(M) / kTile;
    for (int64_t t0 = 0; t0 < row_tiles; t0 += kMaxRowTiles) {
        const int64_t n = row_tiles - t0 < kMaxRowTiles ? row_tiles - t0 : kMaxRowTiles;
        dim3 grid((unsigned)(padded(N) / kTile), (unsigned)n);
        if (layout == MX_LAYOUT_TILED)
            hipLaunchKernelGGL(fp8_quantize_kernel<MX_LAYOUT_TILED>, grid, dim3(256), 0, stream, x, M, N, ldx, info,
                               info, q_row, q_col, t0);
        else
            hipLaunchKernelGGL(fp8_quantize_kernel<MX_LAYOUT_CANONICAL>, grid, dim3(256), 0, stream, x, M, N, ldx,
                               info, info, q_row, q_col, t0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace mx
