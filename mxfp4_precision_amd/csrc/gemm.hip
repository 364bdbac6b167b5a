// Block-scaled FP4 x FP4 GEMM (C = A . B^T) for gfx950 on tiled-layout blobs.
//
// C[i][j] = sum_k e2m1(A[i][k]) 2^(sa[i][k/32]-127) * e2m1(B[j][k]) 2^(sb[j][k/32]-127),
// fp32 accumulation, bf16 (RNE) or fp32 output: the NT product that the
// forward, dgrad and wgrad of the MXFP4 linear on the page
// "primus_turbo_mxfp4_local.py" compute.
//
// Each 16x16x128 step is one V_MFMA_SCALE_F32_16X16X128_F8F6F4 with both
// formats FP4: lane L supplies 16 bytes (32 elements) of row L%16, k-block
// L/16 of each operand, and that block's E8M0 scale as one byte of a VGPR
// chosen by OPSEL.  The tiled layout stores exactly those 16 bytes at
// lane*16 of a 1 KB atom and packs a lane's scales for 4 consecutive k-steps
// into one dword, so operands move with 16-byte loads and ds_read_b128 that
// never conflict, and a k-group of 4 steps needs one scale dword per lane.
//
// Tiling: a 256-thread workgroup computes a 256x256 tile of C; its 4 waves
// each own 128x128 (8x8 MFMA tiles, 256 fp32 accumulators per lane).  Per
// 128-wide k-step the workgroup stages 16 A atoms and 16 B atoms (32 KB) in
// LDS, double-buffered: the next step's global loads are in flight while the
// current step's 64 MFMAs per wave run.  The MFMA is issued with B as the
// "A" operand, so each lane's 4 accumulators are 4 consecutive columns of one
// row of C and the epilogue stores 8 contiguous bytes per lane.
// Workgroups are ordered so that each XCD (8 on MI355X, dispatched
// round-robin) works on a compact band of output tiles, keeping the A rows
// and B columns it shares within its own L2.

#include "mx_internal.h"


namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kFmtFp4 = 4;              // MFMA f8f6f4 format code for E2M1
constexpr int kBM = 256, kBN = 256;     // workgroup tile
constexpr int kWM = 128, kWN = 128;     // wave tile
constexpr int kGA = kBM / 16;           // A atoms (row groups) per k-step per workgroup
constexpr int kGB = kBN / 16;
constexpr int kTA = kWM / 16;           // A atoms per wave
constexpr int kTB = kWN / 16;
constexpr int kMA = kWM / 32;           // 32x32 MFMA tiles per wave along M (A rows)
constexpr int kMB = kWN / 32;           // ... along N (B rows)
constexpr int kAtoms = kGA + kGB;       // atoms per stage
constexpr int kLoadsPerThread = kAtoms / 4;   // 4 waves, one atom per wave instruction
constexpr int kXcds = 8;
constexpr int kGroupM = 8;              // tile rows per band in the tile order

__device__ __forceinline__ uint32_t bf16_rne_pair(float lo, float hi) {
    uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
    uint32_t ra = (a & 0x7FFFFFFFu) > 0x7F800000u ? ((a >> 16) | 0x40u) : ((a + 0x7FFFu + ((a >> 16) & 1u)) >> 16);
    uint32_t rb = (b & 0x7FFFFFFFu) > 0x7F800000u ? ((b >> 16) | 0x40u) : ((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
    return (ra & 0xFFFFu) | (rb << 16);
}

// Buffer resource over [p, p + bytes).  Loads address it with a per-lane
// byte offset; an offset at or past `bytes` reads zeros (the hardware range
// check of raw buffers), which is how k-steps past K_pad become zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// LDS: 4 k-step stages of 32 atoms (the stage of step k is k % 4, which is
// also its OPSEL scale byte) and one k-group buffer of 32 scale atoms.  A
// group's scales are read into registers at its first step; the next group's
// scales are queued one step later, after every wave passed that read.
// Separate arrays keep every LDS address a compile-time constant plus lane.
__shared__ __attribute__((aligned(1024))) uint8_t g_stage0[kAtoms * 1024];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage1[kAtoms * 1024];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage2[kAtoms * 1024];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage3[kAtoms * 1024];
__shared__ __attribute__((aligned(1024))) uint8_t g_scale[kAtoms * 256];

template <int S>
__device__ __forceinline__ uint8_t *stage_buf() {
    return S == 0 ? g_stage0 : S == 1 ? g_stage1 : S == 2 ? g_stage2 : g_stage3;
}

#define MX_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Offset that lies past every operand buffer: a buffer load there returns 0.
constexpr uint32_t kOutOfRange = 0x80000000u;

struct GemmCtx {
    __amdgpu_buffer_rsrc_t rA, rB, rAs, rBs;
    int ld_row[kLoadsPerThread];    // byte offset of this wave's r-th atom row (k-step 0)
    int sc_row[kLoadsPerThread];    // byte offset of this wave's r-th scale-atom row (k-group 0)
    int64_t ksteps, kgroups;
    int wave, lane16, lane4;
};

// DMA k-step k into stage S (global -> LDS, no registers): wave w copies atoms
// 4r + w.  Steps past K_pad read out of range and land as zeros.  When k
// opens a k-group, that group's 32 scale atoms go to the scale buffer.
template <int S>
__device__ __forceinline__ void issue_step(const GemmCtx &c, int64_t k) {
    const bool valid = k < c.ksteps;
    const uint32_t koff = (uint32_t)(k * 1024);
#pragma unroll
    for (int r = 0; r < kLoadsPerThread; ++r) {
        const int a = 4 * r + c.wave;
        const uint32_t voff = valid ? (uint32_t)c.ld_row[r] + koff + c.lane16 : kOutOfRange + c.lane16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a < kGA ? c.rA : c.rB, MX_LDS(stage_buf<S>() + a * 1024), 16,
                                                 voff, 0, 0, 0);
    }
    if (S == 0) {
        const int64_t h = k / 4;
        const bool hvalid = h < c.kgroups;
        const uint32_t hoff = (uint32_t)(h * 256);
#pragma unroll
        for (int r = 0; r < kLoadsPerThread; ++r) {
            const int a = 4 * r + c.wave;
            const uint32_t voff = hvalid ? (uint32_t)c.sc_row[r] + hoff + c.lane4 : kOutOfRange + c.lane4;
            uint8_t *dst = g_scale + a * 256;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(a < kGA ? c.rAs : c.rBs, MX_LDS(dst), 4, voff, 0, 0, 0);
        }
    }
}

// Vector-memory instructions a wave issues for k-step j (data, plus scales at a group start).
__host__ __device__ constexpr int issued_for(int j_mod4) { return kLoadsPerThread * (j_mod4 == 0 ? 2 : 1); }

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_a4w4_kernel(int64_t M, int64_t N, int64_t K_pad, int tiles_m,
                                                        int tiles_n, const uint8_t *__restrict__ A,
                                                        const uint8_t *__restrict__ As,
                                                        const uint8_t *__restrict__ B,
                                                        const uint8_t *__restrict__ Bs,
                                                        void *__restrict__ C, int64_t ldc) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int wm = wave >> 1, wn = wave & 1;

    // ---- tile order: XCD-contiguous ranges, bands of kGroupM tile rows
    const int nb = gridDim.x;
    const int b = blockIdx.x;
    const int xcd = b % kXcds, local = b / kXcds;
    const int per = nb / kXcds, rem = nb % kXcds;
    const int id = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int band = kGroupM * tiles_n;
    const int first_m = (id / band) * kGroupM;
    const int gsz = min(tiles_m - first_m, kGroupM);
    const int tm = first_m + (id % band) % gsz;
    const int tn = (id % band) / gsz;

    GemmCtx c;
    c.ksteps = K_pad / 128;
    c.kgroups = cdiv(K_pad, 512);
    c.wave = wave;
    c.lane16 = lane * 16;
    c.lane4 = lane * 4;
    const int64_t nGA = cdiv(M, 16), nGB = cdiv(N, 16);   // row groups present in memory
    const int64_t gA0 = (int64_t)tm * kGA, gB0 = (int64_t)tn * kGB;
    c.rA = make_rsrc(A, nGA * c.ksteps * 1024);
    c.rB = make_rsrc(B, nGB * c.ksteps * 1024);
    c.rAs = make_rsrc(As, nGA * c.kgroups * 256);
    c.rBs = make_rsrc(Bs, nGB * c.kgroups * 256);
    // Row groups past an operand are clamped to its last group: those rows of C
    // are never stored, so their contents do not matter.
#pragma unroll
    for (int r = 0; r < kLoadsPerThread; ++r) {
        const int a = 4 * r + wave;
        const bool isA = a < kGA;
        int64_t g = isA ? gA0 + a : gB0 + (a - kGA);
        const int64_t gmax = (isA ? nGA : nGB) - 1;
        g = g < gmax ? g : gmax;
        c.ld_row[r] = (int)(g * c.ksteps * 1024);
        c.sc_row[r] = (int)(g * c.kgroups * 256);
    }

    v16f acc[kMB][kMA];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kMA; ++j) acc[i][j] = v16f{};

    issue_step<0>(c, 0);
    issue_step<1>(c, 1);
    issue_step<2>(c, 2);

    // Lane L of a 32-row operand tile takes row L%32, k-block 2*half + L/32 of
    // V_MFMA_SCALE_F32_32X32X64_F8F6F4: in the tiled layout that is atom
    // (L%32)/16, slice (L%16) + 16*(2*half + L/32) -- four contiguous 256-byte
    // runs per ds_read_b128, so the reads stay conflict-free.  Its scale is
    // byte (k-step % 4) of the dword at the same slice of the scale atom.
    const int lrow = lane & 31, lhi = lane >> 5;
    const int frag_off = ((lrow >> 4) * 1024) + ((lrow & 15) + 16 * lhi) * 16;   // half 0; half 1 adds 512
    const int sc_off = ((lrow >> 4) * 256) + ((lrow & 15) + 16 * lhi) * 4;       // half 0; half 1 adds 128

    uint32_t sa[kMA][2], sb[kMB][2], sa_n[kMA][2], sb_n[kMB][2];
    uint4 fa0[kMA], fb0[kMB], fa1[kMA], fb1[kMB];
    auto read_scales = [&](uint32_t (&xa)[kMA][2], uint32_t (&xb)[kMB][2]) {
#pragma unroll
        for (int t = 0; t < kMA; ++t)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                xa[t][hh] = *reinterpret_cast<const uint32_t *>(g_scale + (wm * kTA + 2 * t) * 256 + sc_off + hh * 128);
#pragma unroll
        for (int t = 0; t < kMB; ++t)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                xb[t][hh] = *reinterpret_cast<const uint32_t *>(g_scale + (kGA + wn * kTB + 2 * t) * 256 + sc_off + hh * 128);
    };
    auto read_frags = [&](const uint8_t *stage, int hh, uint4 (&xa)[kMA], uint4 (&xb)[kMB]) {
        const uint8_t *a_lds = stage + (wm * kTA) * 1024 + frag_off + hh * 512;
        const uint8_t *b_lds = stage + (kGA + wn * kTB) * 1024 + frag_off + hh * 512;
#pragma unroll
        for (int t = 0; t < kMA; ++t) xa[t] = *reinterpret_cast<const uint4 *>(a_lds + t * 2048);
#pragma unroll
        for (int t = 0; t < kMB; ++t) xb[t] = *reinterpret_cast<const uint4 *>(b_lds + t * 2048);
    };
    auto mfmas = [&](auto s_tag, int hh, const uint4 (&xa)[kMA], const uint4 (&xb)[kMB]) {
        constexpr int S = decltype(s_tag)::value;
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
            const v8i bop = {(int)xb[i].x, (int)xb[i].y, (int)xb[i].z, (int)xb[i].w, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < kMA; ++j) {
                const v8i aop = {(int)xa[j].x, (int)xa[j].y, (int)xa[j].z, (int)xa[j].w, 0, 0, 0, 0};
                // MFMA "A" operand = B rows (columns of C), "B" operand = A rows (rows of C)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    bop, aop, acc[i][j], kFmtFp4, kFmtFp4, S, (int)sb[i][hh], S, (int)sa[j][hh]);
            }
        }
    };

    // Prologue: step 0 landed, group 0 scales and step 0's first half in registers.
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(issued_for(1) + issued_for(2)) : "memory");
    read_scales(sa, sb);
    read_frags(stage_buf<0>(), 0, fa0, fb0);

    // One 128-wide k-step (stage S = k % 4 = OPSEL), software-pipelined so the
    // MFMA pipe never drains: the first half's 16 MFMAs are interleaved with
    // the reads of the second half's operands; then the workgroup meets at the
    // barrier that publishes step k+1 (each wave waits for its own DMA of step
    // k+1 first) and frees stage k-1; the second half's 16 MFMAs are
    // interleaved with the DMA of step k+3 into stage k-1 and the reads of
    // step k+1's first half.  Every memory instruction issues in the shadow of
    // an MFMA (sched_group_barrier masks: 0x008 MFMA, 0x020 VMEM read,
    // 0x100 DS read).
    auto one_step = [&](int64_t k, auto s_tag) {
        constexpr int S = decltype(s_tag)::value;
        mfmas(s_tag, 0, fa0, fb0);
        read_frags(stage_buf<S>(), 1, fa1, fb1);
#pragma unroll
        for (int t = 0; t < kMA + kMB; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kMA * kMB - (kMA + kMB), 0);
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(issued_for((S + 2) & 3)) : "memory");
        __builtin_amdgcn_sched_barrier(0);
        issue_step<(S + 3) & 3>(c, k + 3);
        mfmas(s_tag, 1, fa1, fb1);
        if (S == 3) read_scales(sa_n, sb_n);
        read_frags(stage_buf<(S + 1) & 3>(), 0, fa0, fb0);
        constexpr int kDma = issued_for((S + 3) & 3);
#pragma unroll
        for (int t = 0; t < kDma; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);
        }
        constexpr int kDs = (kMA + kMB) + (S == 3 ? 2 * (kMA + kMB) : 0);
        constexpr int kMfmaLeft = kMA * kMB - kDma;
        constexpr int kPairs = kDs < kMfmaLeft ? kDs : kMfmaLeft;
#pragma unroll
        for (int t = 0; t < kPairs; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        }
        if (kMfmaLeft > kPairs) __builtin_amdgcn_sched_group_barrier(0x008, kMfmaLeft - kPairs, 1);
        if (kDs > kPairs) __builtin_amdgcn_sched_group_barrier(0x100, kDs - kPairs, 1);
        __builtin_amdgcn_sched_barrier(0);
        if (S == 3) {
#pragma unroll
            for (int t = 0; t < kMA; ++t) { sa[t][0] = sa_n[t][0]; sa[t][1] = sa_n[t][1]; }
#pragma unroll
            for (int t = 0; t < kMB; ++t) { sb[t][0] = sb_n[t][0]; sb[t][1] = sb_n[t][1]; }
        }
    };

    for (int64_t h = 0; h < c.kgroups; ++h) {
        const int64_t k0 = 4 * h;
        one_step(k0, std::integral_constant<int, 0>{});
        one_step(k0 + 1, std::integral_constant<int, 1>{});
        one_step(k0 + 2, std::integral_constant<int, 2>{});
        one_step(k0 + 3, std::integral_constant<int, 3>{});
    }
    // drain the trailing (out-of-range) DMAs before the workgroup exits
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue: acc[i][j][r] = C[m0 + 32j + lane%32][n0 + 32i + 8(r/4) + 4(lane/32) + r%4]
    const int64_t m0 = (int64_t)tm * kBM + wm * kWM;
    const int64_t n0 = (int64_t)tn * kBN + wn * kWN;
#pragma unroll
    for (int j = 0; j < kMA; ++j) {
        const int64_t row = m0 + 32 * j + lrow;
        if (row >= M) continue;
#pragma unroll
        for (int i = 0; i < kMB; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t col = n0 + 32 * i + 8 * q + 4 * lhi;
                const v4f v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                if (OUT_BF16) {
                    uint16_t *dst = reinterpret_cast<uint16_t *>(C) + row * ldc + col;
                    const uint32_t p01 = bf16_rne_pair(v[0], v[1]), p23 = bf16_rne_pair(v[2], v[3]);
                    if (col + 3 < N) {
                        *reinterpret_cast<uint2 *>(dst) = uint2{p01, p23};
                    } else {
                        if (col < N) dst[0] = (uint16_t)p01;
                        if (col + 1 < N) dst[1] = (uint16_t)(p01 >> 16);
                        if (col + 2 < N) dst[2] = (uint16_t)p23;
                    }
                } else {
                    float *dst = reinterpret_cast<float *>(C) + row * ldc + col;
                    if (col + 3 < N) {
                        *reinterpret_cast<v4f *>(dst) = v;
                    } else {
#pragma unroll
                        for (int r = 0; r < 3; ++r)
                            if (col + r < N) dst[r] = v[r];
                    }
                }
            }
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
    // buffer offsets are 32-bit: each operand blob must stay below 2 GiB
    if (cdiv(M, 16) * K_pad / 2 >= (int64_t(1) << 31) || cdiv(N, 16) * K_pad / 2 >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
    const int tiles_m = (int)cdiv(M, kBM), tiles_n = (int)cdiv(N, kBN);
    dim3 grid((unsigned)(tiles_m * tiles_n));
    if (out_dtype == MX_BF16)
        hipLaunchKernelGGL(gemm_a4w4_kernel<true>, grid, dim3(256), 0, stream, M, N, K_pad, tiles_m, tiles_n,
                           A, As, B, Bs, C, ldc);
    else
        hipLaunchKernelGGL(gemm_a4w4_kernel<false>, grid, dim3(256), 0, stream, M, N, K_pad, tiles_m,
                           tiles_n, A, As, B, Bs, C, ldc);
    return hipGetLastError();
}

}  // namespace mx

