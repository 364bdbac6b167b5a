// MXFP4 block quantization kernels for gfx950.
//
// What is computed (OCP Microscaling Formats v1.0, sec. 6.3; blob shapes and
// the 128-padding from the page "primus_turbo_mxfp4_local.py"):
//   per 32-element block (or aligned 32x32 tile in 2D mode) the scale byte is
//   max(E(amax) - 2, 0), E = biased exponent of the block's bf16 amax, or 0xFF
//   if the block holds Inf/NaN; each element becomes the E2M1 code of
//   |x| / 2^(byte-127), rounded to nearest even (or stochastically) and
//   saturated at 6, with x's sign bit.
//
// Work decomposition: one wave owns a 32-row x 128-column tile of x; lane
// (c = lane%16, q = lane/16) holds the 8x8 sub-block rows 8q..8q+7,
// columns 8c..8c+7, loaded as eight 16-byte row segments (each load
// instruction reads 4 rows x 256 contiguous bytes).  Both directions' blocks
// are complete inside the wave: a row block (32 columns) spans lanes
// c = 4b..4b+3, a column block (32 rows) spans lanes q = 0..3, so the amax
// reductions are two cross-lane steps each and x is read from HBM once.
// A workgroup stacks 4 waves (128 x 128) so column-blob writes form 64-byte
// runs in the canonical layout and whole 1 KB atoms in the tiled layout.
//
// Encoding, round to nearest even: V_CVT_SCALEF32_PK_FP4_BF16 converts a bf16
// pair divided by the fp32 scale 2^(byte-127) to two E2M1 nibbles.  Its
// rounding (ties to even, saturation at 6, sign kept, subnormal inputs and the
// subnormal scale 2^-127 included) was checked exhaustively against the
// definition for every finite bf16 value at every scale byte that can hold it;
// the GPU parity tests repeat that sweep through this kernel.
//
// Encoding, stochastic: with u = |x| * 2^(1-c) as an fp32 bit pattern, the
// E2M1 normal numbers (1 <= v < 8) coincide with fp32 normal numbers and the
// E2M1 subnormal step (0.5) with the fp32 subnormal range, so the code is
// the truncation u >> 22 plus 1 iff the element's random byte is below the
// next 8 bits (u >> 14) & 0xFF, which equal floor(256 (v-lo)/(hi-lo)).

#include "mx_internal.h"

namespace mx {
namespace {

constexpr int kWaveRows = 32;
constexpr int kTileCols = 128;
constexpr int kWaves = 4;
constexpr int kTileRows = kWaveRows * kWaves;

__device__ __forceinline__ uint32_t scale_code(uint32_t amax16) {
    if (amax16 >= 0x7F80u) return 0xFFu;            // Inf or NaN in the block
    uint32_t e = amax16 >> 7;
    return e > 2u ? e - 2u : 0u;
}

// |x| * 2^(1-c) as fp32 bits (exact whenever the code can be non-zero).
__device__ __forceinline__ uint32_t scaled_u(uint32_t x16, uint32_t c) {
    float xf = __uint_as_float((x16 & 0x7FFFu) << 16);
    return __float_as_uint(__builtin_ldexpf(xf, 1 - (int)c));
}

__device__ __forceinline__ uint32_t code_sr(uint32_t u, uint32_t rbyte) {
    uint32_t r = (u >> 22) + (rbyte < ((u >> 14) & 0xFFu) ? 1u : 0u);
    return r < 7u ? r : 7u;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 2^(c-127) as fp32 (c = 0 is the subnormal 2^-127).
__device__ __forceinline__ float scale_f32(uint32_t c) {
    return __uint_as_float(c ? (c << 23) : 0x00400000u);
}

// Four bf16 pairs (element 2i in the low half of p_i) -> 8 nibbles, RNE, saturating.
__device__ __forceinline__ uint32_t pack8_rne(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3,
                                              uint32_t c) {
    const float sf = scale_f32(c);
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, p0), sf, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, p1), sf, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, p2), sf, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, p3), sf, 3);
    return c == 0xFFu ? 0u : r;      // Inf/NaN block: all nibbles 0
}

// bf16 pair (lo, hi) from the same half of two words: half 0 = low halves.
__device__ __forceinline__ uint32_t pair_of(uint32_t lo_word, uint32_t hi_word, int half) {
    return __builtin_amdgcn_perm(hi_word, lo_word, half ? 0x07060302u : 0x05040100u);
}

__device__ __forceinline__ uint32_t nibble_sr(uint32_t x16, uint32_t c, uint32_t rbyte) {
    if (c == 0xFFu) return 0u;
    return code_sr(scaled_u(x16, c), rbyte) | ((x16 >> 12) & 8u);
}

// ------------------------------------------------------------------ Philox
// Philox-4x32-10 (Salmon et al., SC'11, sec. 4.2).
__device__ __forceinline__ void philox10(uint32_t &c0, uint32_t &c1, uint32_t &c2, uint32_t &c3,
                                         uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
        uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
        uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
        k0 += 0x9E3779B9u; k1 += 0xBB67AE85u;
    }
}

// The 8 random bytes of elements n0 .. n0+7 for one direction, little-endian
// in (lo, hi): byte e is the SR byte of element n0+e.
__device__ __forceinline__ void rand8(uint64_t n0, const DirOpts &o, uint32_t dir,
                                      uint32_t &lo, uint32_t &hi) {
    uint64_t g = n0 >> 4;
    uint32_t off = (uint32_t)(n0 & 15u);
    uint32_t a0 = (uint32_t)g, a1 = (uint32_t)(g >> 32), a2 = o.tensor_id, a3 = dir;
    philox10(a0, a1, a2, a3, o.key0, o.key1);
    if (off == 0u) { lo = a0; hi = a1; return; }
    if (off == 8u) { lo = a2; hi = a3; return; }
    // Unaligned: window of 32 bytes across two consecutive counters.
    uint64_t g1 = g + 1;
    uint32_t b0 = (uint32_t)g1, b1 = (uint32_t)(g1 >> 32), b2 = o.tensor_id, b3 = dir;
    if (off > 8u) philox10(b0, b1, b2, b3, o.key0, o.key1);
    uint32_t w[8] = {a0, a1, a2, a3, b0, b1, b2, b3};
    uint32_t s = (off & 3u) * 8u;
    uint32_t i = off >> 2;
    uint32_t x0 = 0, x1 = 0, x2 = 0;
#pragma unroll
    for (uint32_t t = 0; t < 6; ++t) {
        if (t == i) { x0 = w[t]; x1 = w[t + 1]; x2 = w[t + 2]; }
    }
    lo = s ? (x0 >> s) | (x1 << (32u - s)) : x0;
    hi = s ? (x1 >> s) | (x2 << (32u - s)) : x1;
}

__device__ __forceinline__ uint32_t max_abs_pair(uint32_t d) {
    uint32_t lo = d & 0x7FFFu, hi = (d >> 16) & 0x7FFFu;
    return lo > hi ? lo : hi;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint32_t xor_max(uint32_t v, int mask) {
    return umax(v, (uint32_t)__shfl_xor((int)v, mask, 64));
}

template <int LAYOUT, bool DUAL>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;
    const int q = lane >> 4;
    const int64_t row0 = (int64_t)blockIdx.y * kTileRows + wave * kWaveRows;
    const int64_t col0 = (int64_t)blockIdx.x * kTileCols;
    const int64_t M = a.M, N = a.N;

    // ---- staging read: d[t][w] = bf16 pair (cols 2w, 2w+1 of the lane's 8) of row 8q+t
    uint32_t d[8][4];
    const int64_t j0 = col0 + 8 * c;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int64_t i = row0 + 8 * q + t;
        const uint16_t *p = a.x + i * a.ldx + j0;
        if (i < M && j0 + 8 <= N) {
            uint4 v = *reinterpret_cast<const uint4 *>(p);
            d[t][0] = v.x; d[t][1] = v.y; d[t][2] = v.z; d[t][3] = v.w;
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t lo = (i < M && j0 + 2 * w < N) ? p[2 * w] : 0u;
                uint32_t hi = (i < M && j0 + 2 * w + 1 < N) ? p[2 * w + 1] : 0u;
                d[t][w] = lo | (hi << 16);
            }
        }
    }

    // ---- block amax, row direction: per row t over the lane's 8 columns, then lanes c^1, c^2
    uint32_t ramax[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        uint32_t m = umax(umax(max_abs_pair(d[t][0]), max_abs_pair(d[t][1])),
                          umax(max_abs_pair(d[t][2]), max_abs_pair(d[t][3])));
        ramax[t] = m;
    }
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        uint32_t pk = ramax[t] | (ramax[t + 1] << 16);
        uint32_t o1 = (uint32_t)__shfl_xor((int)pk, 1, 64);
        uint32_t lo = umax(pk & 0xFFFFu, o1 & 0xFFFFu), hi = umax(pk >> 16, o1 >> 16);
        pk = lo | (hi << 16);
        uint32_t o2 = (uint32_t)__shfl_xor((int)pk, 2, 64);
        ramax[t] = umax(pk & 0xFFFFu, o2 & 0xFFFFu);
        ramax[t + 1] = umax(pk >> 16, o2 >> 16);
    }
    // 32x32 tile amax (2D mode): rows of the lane, then the 4 q-lanes
    uint32_t tile_amax = 0;
    if (a.row.use_2d || (DUAL && a.col.use_2d)) {
        uint32_t m = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) m = umax(m, ramax[t]);
        m = xor_max(m, 16);
        m = xor_max(m, 32);
        tile_amax = m;
    }

    // ---- row-wise blob
    {
        const int64_t Lp = a.N_pad;
        const int64_t rows_out = (LAYOUT == MX_LAYOUT_TILED) ? cdiv(M, 16) * 16 : M;
        const int64_t kb = col0 / 32 + c / 4;        // k-block of this lane's columns
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int64_t i = row0 + 8 * q + t;
            // rows past M exist only as zero padding of the tiled layout: scale 0 there
            const uint32_t sc = i < M ? scale_code(a.row.use_2d ? tile_amax : ramax[t]) : 0u;
            uint32_t packed = 0;
            if (a.row.use_sr) {
                uint32_t rlo = 0, rhi = 0;
                if (i < M && j0 < N) rand8(a.row.index_base + (uint64_t)i * (uint64_t)N + (uint64_t)j0,
                                           a.row, 0u, rlo, rhi);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint32_t x16 = (d[t][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    uint32_t rb = ((e < 4 ? rlo : rhi) >> (8 * (e & 3))) & 0xFFu;
                    packed |= nibble_sr(x16, sc, rb) << (4 * e);
                }
            } else {
                packed = pack8_rne(d[t][0], d[t][1], d[t][2], d[t][3], sc);
            }
            if (i < rows_out) {
                if (LAYOUT == MX_LAYOUT_CANONICAL) {
                    *reinterpret_cast<uint32_t *>(a.q_row + i * (Lp / 2) + col0 / 2 + 4 * c) = packed;
                    if ((c & 3) == 0) a.s_row[i * (Lp / 32) + kb] = (uint8_t)sc;
                } else {
                    const int64_t ksteps = Lp / 128, kgroups = cdiv(Lp, 512);
                    const int64_t g = i / 16;
                    const int64_t atom = (g * ksteps + col0 / 128) * 1024;
                    const int lane_t = (int)(i % 16) + 16 * (c / 4);
                    *reinterpret_cast<uint32_t *>(a.q_row + atom + lane_t * 16 + 4 * (c & 3)) = packed;
                    if ((c & 3) == 0) {
                        const int64_t satom = (g * kgroups + kb / 16) * 256;
                        const int slane = (int)(i % 16) + 16 * (int)(kb % 4);
                        a.s_row[satom + 4 * slane + (kb % 16) / 4] = (uint8_t)sc;
                    }
                    // zero the unused tail of the last scale atom (blocks past L_pad/32)
                    const int64_t nblk = Lp / 32;
                    const int64_t tail = (16 - nblk % 16) % 16;
                    if (col0 + kTileCols == Lp && c < tail) {
                        const int64_t zb = nblk + c;
                        const int64_t zatom = (g * kgroups + zb / 16) * 256;
                        const int zl = (int)(i % 16) + 16 * (int)(zb % 4);
                        a.s_row[zatom + 4 * zl + (zb % 16) / 4] = 0;
                    }
                }
            }
        }
    }

    if (!DUAL) return;

    // ---- column-wise blob: per column u of the lane, 8 rows in-lane, then lanes q^1, q^2
    uint32_t camax[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            lo = umax(lo, d[t][w] & 0x7FFFu);
            hi = umax(hi, (d[t][w] >> 16) & 0x7FFFu);
        }
        uint32_t pk = lo | (hi << 16);
        uint32_t o1 = (uint32_t)__shfl_xor((int)pk, 16, 64);
        lo = umax(pk & 0xFFFFu, o1 & 0xFFFFu); hi = umax(pk >> 16, o1 >> 16);
        pk = lo | (hi << 16);
        uint32_t o2 = (uint32_t)__shfl_xor((int)pk, 32, 64);
        camax[2 * w] = umax(pk & 0xFFFFu, o2 & 0xFFFFu);
        camax[2 * w + 1] = umax(pk >> 16, o2 >> 16);
    }
    {
        const int64_t Lp = a.M_pad;
        const int64_t rows_out = (LAYOUT == MX_LAYOUT_TILED) ? cdiv(N, 16) * 16 : N;
        const int64_t kb = (row0) / 32;              // k-block along M of this wave
        // SR bytes: element (i, j) with i = row0+8q+t, j = j0+u: n = base + i*N + j
        uint32_t rl[8], rh[8];
        if (a.col.use_sr) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int64_t i = row0 + 8 * q + t;
                rl[t] = rh[t] = 0;
                if (i < M && j0 < N)
                    rand8(a.col.index_base + (uint64_t)i * (uint64_t)N + (uint64_t)j0, a.col, 1u,
                          rl[t], rh[t]);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t j = j0 + u;
            const uint32_t sc = j < N ? scale_code(a.col.use_2d ? tile_amax : camax[u]) : 0u;
            uint32_t packed = 0;
            if (a.col.use_sr) {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    uint32_t x16 = (d[t][u >> 1] >> (16 * (u & 1))) & 0xFFFFu;
                    uint32_t rb = ((u < 4 ? rl[t] : rh[t]) >> (8 * (u & 3))) & 0xFFu;
                    packed |= nibble_sr(x16, sc, rb) << (4 * t);
                }
            } else {
                const int w = u >> 1, h = u & 1;
                packed = pack8_rne(pair_of(d[0][w], d[1][w], h), pair_of(d[2][w], d[3][w], h),
                                   pair_of(d[4][w], d[5][w], h), pair_of(d[6][w], d[7][w], h), sc);
            }
            if (j < rows_out) {
                if (LAYOUT == MX_LAYOUT_CANONICAL) {
                    *reinterpret_cast<uint32_t *>(a.q_col + j * (Lp / 2) + row0 / 2 + 4 * q) = packed;
                    if (q == 0) a.s_col[j * (Lp / 32) + kb] = (uint8_t)sc;
                } else {
                    const int64_t ksteps = Lp / 128, kgroups = cdiv(Lp, 512);
                    const int64_t g = j / 16;
                    const int64_t atom = (g * ksteps + row0 / 128) * 1024;
                    const int lane_t = (int)(j % 16) + 16 * wave;   // (row%128)/32 == wave
                    *reinterpret_cast<uint32_t *>(a.q_col + atom + lane_t * 16 + 4 * q) = packed;
                    if (q == 0) {
                        const int64_t satom = (g * kgroups + kb / 16) * 256;
                        const int slane = (int)(j % 16) + 16 * (int)(kb % 4);
                        a.s_col[satom + 4 * slane + (kb % 16) / 4] = (uint8_t)sc;
                    }
                    const int64_t nblk = Lp / 32;
                    const int64_t tail = (16 - nblk % 16) % 16;
                    if (wave == 0 && (int64_t)blockIdx.y * kTileRows + kTileRows == Lp) {
                        for (int64_t z = q; z < tail; z += 4) {
                            const int64_t zb = nblk + z;
                            const int64_t zatom = (g * kgroups + zb / 16) * 256;
                            const int zl = (int)(j % 16) + 16 * (int)(zb % 4);
                            a.s_col[zatom + 4 * zl + (zb % 16) / 4] = 0;
                        }
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_quantize(const QuantArgs &a, bool dual, mx_layout layout, hipStream_t stream) {
    dim3 grid((unsigned)cdiv(a.N, kTileCols), (unsigned)cdiv(a.M, kTileRows));
    dim3 block(256);
    if (layout == MX_LAYOUT_CANONICAL) {
        if (dual) hipLaunchKernelGGL((quantize_kernel<MX_LAYOUT_CANONICAL, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((quantize_kernel<MX_LAYOUT_CANONICAL, false>), grid, block, 0, stream, a);
    } else {
        if (dual) hipLaunchKernelGGL((quantize_kernel<MX_LAYOUT_TILED, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((quantize_kernel<MX_LAYOUT_TILED, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace mx
