// Block-scaled FP4 x FP4 GEMM (C = A . B^T) for gfx950 on tiled-layout blobs.
//
// C[i][j] = sum_k e2m1(A[i][k]) 2^(sa[i][k/32]-127) * e2m1(B[j][k]) 2^(sb[j][k/32]-127),
// fp32 accumulation, bf16 (RNE) or fp32 output: the NT product that the
// forward, dgrad and wgrad of the MXFP4 linear on the page
// "primus_turbo_mxfp4_local.py" compute.
//
// Each 16x16x128 step is one V_MFMA_SCALE_F32_16X16X128_F8F6F4 with both
// formats FP4: lane L supplies 16 bytes (32 elements) of row L%16, k-block
// L/16 of each operand plus that block's E8M0 scale in byte 0 of a VGPR.
// The tiled layout stores exactly those 16 bytes at lane*16 of a 1 KB atom,
// so every operand fetch is one coalesced 16-byte load per lane.

#include "mx_internal.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kFmtFp4 = 4;      // MFMA f8f6f4 format code for E2M1

// Workgroup: 4 waves in a 2x2 grid, 128x128 output tile; each wave 64x64 =
// 4x4 MFMA tiles of 16x16.
constexpr int kWgM = 128, kWgN = 128;
constexpr int kWaveM = 64, kWaveN = 64;
constexpr int kTm = kWaveM / 16, kTn = kWaveN / 16;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_a4w4_kernel(int64_t M, int64_t N, int64_t K_pad,
                                                        const uint8_t *__restrict__ A,
                                                        const uint8_t *__restrict__ As,
                                                        const uint8_t *__restrict__ B,
                                                        const uint8_t *__restrict__ Bs,
                                                        void *__restrict__ C, int64_t ldc) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * kWgM + (wave >> 1) * kWaveM;
    const int64_t n0 = (int64_t)blockIdx.x * kWgN + (wave & 1) * kWaveN;
    const int64_t ksteps = K_pad / 128;
    const int64_t kgroups = cdiv(K_pad, 512);
    const int64_t gA = cdiv(M, 16), gB = cdiv(N, 16);   // row groups present in memory

    v4f acc[kTm][kTn];
#pragma unroll
    for (int i = 0; i < kTm; ++i)
#pragma unroll
        for (int j = 0; j < kTn; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const uint4 zero4 = {0u, 0u, 0u, 0u};
    for (int64_t s = 0; s < ksteps; ++s) {
        uint4 a[kTm], b[kTn];
        uint32_t sa[kTm], sb[kTn];
        const int64_t h = s / 4;
        const int sh = (int)(s % 4) * 8;
#pragma unroll
        for (int i = 0; i < kTm; ++i) {
            const int64_t g = m0 / 16 + i;
            if (g < gA) {
                a[i] = *reinterpret_cast<const uint4 *>(A + (g * ksteps + s) * 1024 + lane * 16);
                sa[i] = (*reinterpret_cast<const uint32_t *>(As + (g * kgroups + h) * 256 + lane * 4) >> sh) & 0xFFu;
            } else {
                a[i] = zero4;
                sa[i] = 0;
            }
        }
#pragma unroll
        for (int j = 0; j < kTn; ++j) {
            const int64_t g = n0 / 16 + j;
            if (g < gB) {
                b[j] = *reinterpret_cast<const uint4 *>(B + (g * ksteps + s) * 1024 + lane * 16);
                sb[j] = (*reinterpret_cast<const uint32_t *>(Bs + (g * kgroups + h) * 256 + lane * 4) >> sh) & 0xFFu;
            } else {
                b[j] = zero4;
                sb[j] = 0;
            }
        }
#pragma unroll
        for (int i = 0; i < kTm; ++i) {
            v8i av = {(int)a[i].x, (int)a[i].y, (int)a[i].z, (int)a[i].w, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < kTn; ++j) {
                v8i bv = {(int)b[j].x, (int)b[j].y, (int)b[j].z, (int)b[j].w, 0, 0, 0, 0};
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    av, bv, acc[i][j], kFmtFp4, kFmtFp4, 0, (int)sa[i], 0, (int)sb[j]);
            }
        }
    }

    // Epilogue: lane holds C[16i + 4*(lane/16) + r][16j + lane%16], r = 0..3.
#pragma unroll
    for (int i = 0; i < kTm; ++i)
#pragma unroll
        for (int j = 0; j < kTn; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 16 * i + 4 * (lane >> 4) + r;
                const int64_t col = n0 + 16 * j + (lane & 15);
                if (row < M && col < N) {
                    if (OUT_BF16)
                        reinterpret_cast<uint16_t *>(C)[row * ldc + col] = f32_to_bf16_rne(acc[i][j][r]);
                    else
                        reinterpret_cast<float *>(C)[row * ldc + col] = acc[i][j][r];
                }
            }
}

template <typename T>
__global__ void fill_zero_kernel(T *C, int64_t M, int64_t N, int64_t ldc) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx < M * N) C[(idx / N) * ldc + idx % N] = T(0);
}

}  // namespace

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t *A, const uint8_t *As,
                       const uint8_t *B, const uint8_t *Bs, mx_dtype out_dtype, void *C,
                       int64_t ldc, hipStream_t stream) {
    const int64_t K_pad = padded(K);
    if (K_pad == 0) {
        const int64_t n = M * N;
        dim3 grid((unsigned)cdiv(n, 256));
        if (out_dtype == MX_BF16)
            hipLaunchKernelGGL(fill_zero_kernel<uint16_t>, grid, dim3(256), 0, stream,
                               reinterpret_cast<uint16_t *>(C), M, N, ldc);
        else
            hipLaunchKernelGGL(fill_zero_kernel<float>, grid, dim3(256), 0, stream,
                               reinterpret_cast<float *>(C), M, N, ldc);
        return hipGetLastError();
    }
    dim3 grid((unsigned)cdiv(N, kWgN), (unsigned)cdiv(M, kWgM));
    if (out_dtype == MX_BF16)
        hipLaunchKernelGGL(gemm_a4w4_kernel<true>, grid, dim3(256), 0, stream, M, N, K_pad, A, As, B, Bs,
                           C, ldc);
    else
        hipLaunchKernelGGL(gemm_a4w4_kernel<false>, grid, dim3(256), 0, stream, M, N, K_pad, A, As, B,
                           Bs, C, ldc);
    return hipGetLastError();
}

}  // namespace mx
