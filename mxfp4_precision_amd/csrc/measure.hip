// Measurement aid: the sustained rate of the block-scaled FP4 matrix
// instruction the GEMM issues (V_MFMA_SCALE_F32_32X32X64_F8F6F4 with E2M1 x
// E2M1 operands, unit scales), with no memory traffic inside the loop.  Its
// rate on a given operand pattern is the ceiling that the chip's power limit
// and clock leave for any FP4 GEMM on data like it, next to the 10.1 PF/s
// dense spec.
//
// Each workgroup is 8 waves (two per SIMD, as in the GEMM).  A lane holds 8
// operand pairs read once from `ops` (lane L: words [64 L, 64 L + 64), pair k
// = A words 8k..8k+3 and B words 8k+4..8k+7) and runs 8 accumulator chains,
// chain k on pair k, so consecutive instructions switch operands as a GEMM's
// do.  One float per lane (the sum of its accumulators) is stored at the end
// so that the work is kept.

#include "mx_internal.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kMeasureThreads = 512;
constexpr int kChains = 8;
constexpr int kFmtFp4 = 4;          // f8f6f4 format code for E2M1
constexpr int kUnitScale = 127;     // E8M0 2^0

__global__ __launch_bounds__(kMeasureThreads) void mfma_rate_kernel(const uint4 *__restrict__ ops, int64_t iters,
                                                                    float *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    v8i a[kChains], b[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
        const uint4 x = ops[16 * lane + 2 * k];
        const uint4 y = ops[16 * lane + 2 * k + 1];
        a[k] = v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
        b[k] = v8i{(int)y.x, (int)y.y, (int)y.z, (int)y.w, 0, 0, 0, 0};
    }
    v16f acc[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) acc[k] = v16f{};
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kChains; ++k)
            acc[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[k], b[k], acc[k], kFmtFp4, kFmtFp4, 0,
                                                                      kUnitScale, 0, kUnitScale);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kChains; ++k)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[k][e];
    out[(int64_t)blockIdx.x * kMeasureThreads + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_measure_mfma_fp4(const void *ops, int workgroups, int64_t iters, float *out, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)workgroups), dim3(kMeasureThreads), 0, stream,
                       static_cast<const uint4 *>(ops), iters, out);
    return hipGetLastError();
}

}  // namespace mx
