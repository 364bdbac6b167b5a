// Device dequantization of one blob to float32 (a test aid): element value
// (-1)^s * e2m1(code) * 2^(scale-127) per OCP Microscaling Formats v1.0,
// sec. 5.3.3 (E2M1) and 5.4.1 (E8M0, 0xFF = NaN).

#include "mx_internal.h"

namespace mx {
namespace {

__device__ __forceinline__ float e2m1_value(uint32_t nib) {
    // magnitudes of codes 0..7 in units of 0.5: 0 1 2 3 4 6 8 12
    const uint32_t c = nib & 7u;
    const uint32_t half_units = c < 4u ? c : (c == 7u ? 12u : 2u * c - 4u);
    float m = 0.5f * (float)half_units;
    return (nib & 8u) ? -m : m;
}

__global__ void dequantize_kernel(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t length,
                                  int tiled, float *out, int64_t ldo) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * length) return;
    const int64_t r = idx / length, k = idx % length;
    const int64_t Lp = padded(length);
    int64_t qoff, soff;
    if (!tiled) {
        qoff = r * (Lp / 2) + k / 2;
        soff = r * (Lp / 32) + k / 32;
    } else {
        const int64_t lane = r % 16 + 16 * ((k % 128) / 32);
        qoff = ((r / 16) * (Lp / 128) + k / 128) * 1024 + 16 * lane + (k % 32) / 2;
        const int64_t kb = k / 32;
        const int64_t slane = r % 16 + 16 * (kb % 4);
        soff = ((r / 16) * cdiv(Lp, 512) + kb / 16) * 256 + 4 * slane + (kb % 16) / 4;
    }
    const uint32_t byte = q[qoff];
    const uint32_t nib = (k & 1) ? (byte >> 4) : (byte & 0xFu);
    const uint32_t sb = s[soff];
    float v;
    if (sb == 0xFFu) v = __builtin_nanf("");
    else v = ldexpf(e2m1_value(nib), (int)sb - 127);
    out[r * ldo + k] = v;
}

}  // namespace

hipError_t launch_dequantize(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t length,
                             mx_layout layout, float *out, int64_t ldo, hipStream_t stream) {
    const int64_t n = rows * length;
    if (n == 0) return hipSuccess;
    dim3 grid((unsigned)cdiv(n, 256));
    hipLaunchKernelGGL(dequantize_kernel, grid, dim3(256), 0, stream, q, s, rows, length,
                       layout == MX_LAYOUT_TILED ? 1 : 0, out, ldo);
    return hipGetLastError();
}

}  // namespace mx
