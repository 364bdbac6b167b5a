// Measurement aid: the sustained rate of the block-scaled matrix instruction
// the GEMMs issue (V_MFMA_SCALE_F32_32X32X64_F8F6F4, unit scales) for a pair
// of element formats, with no memory traffic inside the loop.  Its rate on a
// given operand pattern is the ceiling that the chip's clock under MFMA work
// leaves for any GEMM on data like it, next to the dense spec.
//
// Each workgroup is 8 waves (two per SIMD, as in the GEMMs).  A lane holds 4
// operand pairs read once from `ops` (lane L: words [64 L, 64 L + 64), pair k
// = A words 16k..16k+7 and B words 16k+8..16k+15; a format of fewer than 8
// bits per element uses the first 4 (E2M1) or 6 (FP6) words of each) and
// runs 4 accumulator chains, chain k on pair k, so consecutive instructions
// switch operands as a GEMM's do.  One float per lane (the sum of its
// accumulators) is stored at the end so that the work is kept.

#include "mx_internal.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kMeasureThreads = 512;
constexpr int kChains = 4;
constexpr int kUnitScale = 127;     // E8M0 2^0

// f8f6f4 format codes: 0 E4M3, 1 E5M2, 2 E2M3, 3 E3M2, 4 E2M1
template <int FA, int FB>
__global__ __launch_bounds__(kMeasureThreads) void mfma_rate_kernel(const uint4 *__restrict__ ops, int64_t iters,
                                                                    float *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    v8i a[kChains], b[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
        const uint4 a0 = ops[16 * lane + 4 * k], a1 = ops[16 * lane + 4 * k + 1];
        const uint4 b0 = ops[16 * lane + 4 * k + 2], b1 = ops[16 * lane + 4 * k + 3];
        a[k] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        b[k] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    }
    v16f acc[kChains];
#pragma unroll
    for (int k = 0; k < kChains; ++k) acc[k] = v16f{};
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kChains; ++k)
            acc[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[k], b[k], acc[k], FA, FB, 0, kUnitScale, 0,
                                                                      kUnitScale);
    }
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < kChains; ++k)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[k][e];
    out[(int64_t)blockIdx.x * kMeasureThreads + threadIdx.x] = s;
}

template <int FA>
void *kernel_for_b(int fb) {
    switch (fb) {
        case 0: return reinterpret_cast<void *>(mfma_rate_kernel<FA, 0>);
        case 1: return reinterpret_cast<void *>(mfma_rate_kernel<FA, 1>);
        case 2: return reinterpret_cast<void *>(mfma_rate_kernel<FA, 2>);
        case 3: return reinterpret_cast<void *>(mfma_rate_kernel<FA, 3>);
        default: return reinterpret_cast<void *>(mfma_rate_kernel<FA, 4>);
    }
}

}  // namespace

hipError_t launch_measure_mfma(int fmt_a, int fmt_b, const void *ops, int workgroups, int64_t iters, float *out,
                               hipStream_t stream) {
    void *k = fmt_a == 0 ? kernel_for_b<0>(fmt_b) : fmt_a == 1 ? kernel_for_b<1>(fmt_b)
              : fmt_a == 2 ? kernel_for_b<2>(fmt_b) : fmt_a == 3 ? kernel_for_b<3>(fmt_b) : kernel_for_b<4>(fmt_b);
    const uint4 *o = static_cast<const uint4 *>(ops);
    void *args[] = {&o, &iters, &out};
    return hipLaunchKernel(k, dim3((unsigned)workgroups), dim3(kMeasureThreads), args, 0, stream);
}

}  // namespace mx
