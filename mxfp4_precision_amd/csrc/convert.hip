// Device-side conversion of one blob between MX_LAYOUT_CANONICAL and
// MX_LAYOUT_TILED (layouts defined in include/mxfp4.h).  A 16-byte lane slice
// is 32 consecutive elements (one k-block) of one row in both layouts, so data
// moves as 16-byte copies; every destination byte is written exactly once
// (tiled padding rows and scale slots past the last k-block are written as 0),
// so the destination needs no clearing beforehand.

#include "mx_internal.h"

namespace mx {
namespace {

struct Geom {
    int64_t rows, Lp, nblk, ksteps, kgroups, r16;
};

__device__ __forceinline__ int64_t tiled_q(const Geom &g, int64_t row, int64_t kb) {
    return ((row / 16) * g.ksteps + kb / 4) * 1024 + ((row % 16) + 16 * (kb % 4)) * 16;
}
__device__ __forceinline__ int64_t tiled_s(const Geom &g, int64_t row, int64_t kb) {
    return ((row / 16) * g.kgroups + kb / 16) * 256 + 4 * ((row % 16) + 16 * (kb % 4)) + (kb % 16) / 4;
}

// One thread per destination 16-byte data slice, then per destination scale byte.
__global__ void to_tiled_kernel(Geom g, const uint8_t *__restrict__ qs, const uint8_t *__restrict__ ss,
                                uint8_t *__restrict__ qd, uint8_t *__restrict__ sd) {
    const int64_t nslices = g.r16 * g.nblk;            // tiled data = r16 rows x nblk slices
    const int64_t nscale = g.r16 * g.kgroups * 16;     // tiled scale bytes
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < nslices; d += stride) {
        // slice d of the tiled blob: atom d / 64 = (row group, k-step), lane d % 64
        const int64_t atom = d / 64, lane = d % 64;
        const int64_t row = (atom / g.ksteps) * 16 + lane % 16;
        const int64_t kb = (atom % g.ksteps) * 4 + lane / 16;
        uint4 v = {0u, 0u, 0u, 0u};
        if (row < g.rows) v = *reinterpret_cast<const uint4 *>(qs + row * (g.Lp / 2) + kb * 16);
        *reinterpret_cast<uint4 *>(qd + d * 16) = v;
    }
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < nscale; e += stride) {
        // byte e of the tiled scales: atom e / 256 = (row group, k-group); byte 4*(r%16 + 16*(kb%4)) + (kb%16)/4
        const int64_t atom = e / 256, b = e % 256;
        const int64_t lane = b / 4;
        const int64_t row = (atom / g.kgroups) * 16 + lane % 16;
        const int64_t kb = (atom % g.kgroups) * 16 + 4 * (b % 4) + lane / 16;
        sd[e] = (row < g.rows && kb < g.nblk) ? ss[row * g.nblk + kb] : (uint8_t)0;
    }
}

// One thread per canonical 16-byte data slice and scale byte.
__global__ void to_canonical_kernel(Geom g, const uint8_t *__restrict__ qs, const uint8_t *__restrict__ ss,
                                    uint8_t *__restrict__ qd, uint8_t *__restrict__ sd) {
    const int64_t n = g.rows * g.nblk;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n; c += stride) {
        const int64_t row = c / g.nblk, kb = c % g.nblk;
        *reinterpret_cast<uint4 *>(qd + row * (g.Lp / 2) + kb * 16) =
            *reinterpret_cast<const uint4 *>(qs + tiled_q(g, row, kb));
        sd[c] = ss[tiled_s(g, row, kb)];
    }
}

}  // namespace

hipError_t launch_layout_convert(bool to_tiled, int64_t rows, int64_t length, const uint8_t *qs,
                                 const uint8_t *ss, uint8_t *qd, uint8_t *sd, hipStream_t stream) {
    Geom g;
    g.rows = rows;
    g.Lp = padded(length);
    g.nblk = g.Lp / 32;
    g.ksteps = g.Lp / 128;
    g.kgroups = cdiv(g.Lp, 512);
    g.r16 = cdiv(rows, 16) * 16;
    const int64_t work = to_tiled ? g.r16 * g.nblk : rows * g.nblk;
    const unsigned blocks = (unsigned)(cdiv(work, 256) < 8192 ? cdiv(work, 256) : 8192);
    if (to_tiled)
        hipLaunchKernelGGL(to_tiled_kernel, dim3(blocks), dim3(256), 0, stream, g, qs, ss, qd, sd);
    else
        hipLaunchKernelGGL(to_canonical_kernel, dim3(blocks), dim3(256), 0, stream, g, qs, ss, qd, sd);
    return hipGetLastError();
}

}  // namespace mx
