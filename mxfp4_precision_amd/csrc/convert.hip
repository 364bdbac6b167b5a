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

// 4 x 4 byte transpose: out[j] byte b = in[b] byte j.  Canonical scale bytes
// kb = 16*kg + 4*b + j travel as dword b; in a tiled scale atom lane
// (r % 16) + 16*j holds them as dword j, byte b.
__device__ __forceinline__ void transpose4x4(const uint32_t (&in)[4], uint32_t (&out)[4]) {
    const uint32_t lo01 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);   // b0: in0.b0 in1.b0 in0.b1 in1.b1
    const uint32_t hi01 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);   // in0.b2 in1.b2 in0.b3 in1.b3
    const uint32_t lo23 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
    out[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);   // in0.b0 in1.b0 in2.b0 in3.b0
    out[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);   // in0.b1 in1.b1 in2.b1 in3.b1
    out[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
}

// Work items in tiled order, one thread each: first the tiled data slices
// (r16 rows x nblk 16-byte slices; slice d is atom d / 64 = (row group,
// k-step), lane d % 64), then the tiled scale lanes (16 per 256-byte atom;
// item e = atom e / 16 = (row group, k-group), row e % 16, carrying that row's
// 16 scale bytes of the k-group).  The tiled side is read or written
// contiguously; the canonical side moves in 16-byte (data) and 4-byte (scale)
// pieces.  Tiled padding (rows >= rows, scale slots with kb >= nblk) is
// written as 0 and skipped on the way back.
template <bool TO_TILED>
__global__ __launch_bounds__(256) void convert_kernel(Geom g, const uint8_t *__restrict__ qs,
                                                      const uint8_t *__restrict__ ss, uint8_t *__restrict__ qd,
                                                      uint8_t *__restrict__ sd) {
    const int64_t nd = g.r16 * g.nblk;
    const int64_t ns = (g.r16 / 16) * g.kgroups * 16;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < nd) {
        const int64_t atom = t >> 6;
        const int lane = (int)(t & 63);
        const int64_t row = (atom / g.ksteps) * 16 + (lane & 15);
        const int64_t kb = (atom % g.ksteps) * 4 + (lane >> 4);
        const int64_t coff = row * (g.Lp / 2) + kb * 16;
        if (TO_TILED) {
            uint4 v = {0u, 0u, 0u, 0u};
            if (row < g.rows) v = *reinterpret_cast<const uint4 *>(qs + coff);
            *reinterpret_cast<uint4 *>(qd + t * 16) = v;
        } else if (row < g.rows) {
            *reinterpret_cast<uint4 *>(qd + coff) = *reinterpret_cast<const uint4 *>(qs + t * 16);
        }
    } else if (t < nd + ns) {
        const int64_t e = t - nd;
        const int64_t atom = e >> 4;
        const int r = (int)(e & 15);
        const int64_t row = (atom / g.kgroups) * 16 + r;
        const int64_t kb0 = (atom % g.kgroups) * 16;
        uint32_t in[4], out[4];
        if (TO_TILED) {
            // canonical row: nblk is a multiple of 4, so each dword is all in or all out
#pragma unroll
            for (int b = 0; b < 4; ++b)
                in[b] = (row < g.rows && kb0 + 4 * b < g.nblk)
                            ? *reinterpret_cast<const uint32_t *>(ss + row * g.nblk + kb0 + 4 * b)
                            : 0u;
            transpose4x4(in, out);
#pragma unroll
            for (int j = 0; j < 4; ++j) *reinterpret_cast<uint32_t *>(sd + atom * 256 + 4 * (r + 16 * j)) = out[j];
        } else if (row < g.rows) {
#pragma unroll
            for (int j = 0; j < 4; ++j) in[j] = *reinterpret_cast<const uint32_t *>(ss + atom * 256 + 4 * (r + 16 * j));
            transpose4x4(in, out);
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (kb0 + 4 * b < g.nblk) *reinterpret_cast<uint32_t *>(sd + row * g.nblk + kb0 + 4 * b) = out[b];
        }
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
    const int64_t work = g.r16 * g.nblk + (g.r16 / 16) * g.kgroups * 16;
    const dim3 grid((unsigned)cdiv(work, 256));
    if (to_tiled)
        hipLaunchKernelGGL(convert_kernel<true>, grid, dim3(256), 0, stream, g, qs, ss, qd, sd);
    else
        hipLaunchKernelGGL(convert_kernel<false>, grid, dim3(256), 0, stream, g, qs, ss, qd, sd);
    return hipGetLastError();
}

}  // namespace mx
