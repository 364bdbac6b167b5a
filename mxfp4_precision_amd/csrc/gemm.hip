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

constexpr int kFmtFp4 = 4;              // MFMA f8f6f4 format code for E2M1
constexpr int kBM = 256, kBN = 256;     // workgroup tile
constexpr int kWM = 128, kWN = 128;     // wave tile
constexpr int kGA = kBM / 16;           // A atoms (row groups) per k-step per workgroup
constexpr int kGB = kBN / 16;
constexpr int kTA = kWM / 16;           // A atoms per wave
constexpr int kTB = kWN / 16;
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

// Buffer resource over [p, p + bytes): loads take a wave-uniform SGPR offset
// plus the lane's VGPR offset.  Every offset the kernel forms is clamped
// inside the buffer, so no access relies on the range check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_a4w4_kernel(int64_t M, int64_t N, int64_t K_pad, int tiles_m,
                                                        int tiles_n, const uint8_t *__restrict__ A,
                                                        const uint8_t *__restrict__ As,
                                                        const uint8_t *__restrict__ B,
                                                        const uint8_t *__restrict__ Bs,
                                                        void *__restrict__ C, int64_t ldc) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][kAtoms * 1024];

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

    const int64_t ksteps = K_pad / 128;
    const int64_t kgroups = cdiv(K_pad, 512);
    const int64_t nGA = cdiv(M, 16), nGB = cdiv(N, 16);   // row groups present in memory
    const int64_t gA0 = (int64_t)tm * kGA, gB0 = (int64_t)tn * kGB;

    // ---- global -> register staging of one k-step: wave w loads atoms 4r + w.
    // Row groups past the operand are clamped to its last group (their results
    // are never stored); k-steps past K_pad (the tail of the last k-group) are
    // loaded clamped and zeroed, so every k-group runs 4 branch-free steps and
    // the padding contributes exact zeros (the layout's pad scale bytes are 0).
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(A, nGA * ksteps * 1024);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(B, nGB * ksteps * 1024);
    const __amdgpu_buffer_rsrc_t rAs = make_rsrc(As, nGA * kgroups * 256);
    const __amdgpu_buffer_rsrc_t rBs = make_rsrc(Bs, nGB * kgroups * 256);
    int ld_row[kLoadsPerThread];                 // wave-uniform atom-row offsets (bytes)
#pragma unroll
    for (int r = 0; r < kLoadsPerThread; ++r) {
        const int a = 4 * r + wave;
        const bool isA = a < kGA;
        int64_t g = isA ? gA0 + a : gB0 + (a - kGA);
        const int64_t gmax = (isA ? nGA : nGB) - 1;
        g = g < gmax ? g : gmax;
        ld_row[r] = (int)(g * ksteps * 1024);
    }
    int sa_row[kTA], sb_row[kTB];                // wave-uniform scale-row offsets (bytes)
#pragma unroll
    for (int j = 0; j < kTA; ++j) {
        int64_t g = gA0 + wm * kTA + j;
        g = g < nGA - 1 ? g : nGA - 1;
        sa_row[j] = (int)(g * kgroups * 256);
    }
#pragma unroll
    for (int i = 0; i < kTB; ++i) {
        int64_t g = gB0 + wn * kTB + i;
        g = g < nGB - 1 ? g : nGB - 1;
        sb_row[i] = (int)(g * kgroups * 256);
    }
    const int lane16 = lane * 16, lane4 = lane * 4;

    uint4 stage[kLoadsPerThread];
    // Issue the 8 global loads of k-step k (clamped into the operand); the data
    // is consumed only by store_step, after this step's MFMAs.
    auto load_step = [&](int64_t k) {
        const int kc = (int)(k < ksteps ? k : ksteps - 1);
#pragma unroll
        for (int r = 0; r < kLoadsPerThread; ++r) {
            const bool isA = 4 * r + wave < kGA;
            stage[r] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(isA ? rA : rB, lane16, ld_row[r] + kc * 1024, 0));
        }
    };
    // Write the staged step into LDS buffer buf; steps past K_pad become zeros.
    auto store_step = [&](int buf, bool keep) {
        const uint32_t m = keep ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int r = 0; r < kLoadsPerThread; ++r)
            *reinterpret_cast<uint4 *>(&lds[buf][(4 * r + wave) * 1024 + lane16]) =
                uint4{stage[r].x & m, stage[r].y & m, stage[r].z & m, stage[r].w & m};
    };

    uint32_t sa_cur[kTA], sb_cur[kTB], sa_nxt[kTA], sb_nxt[kTB];
    auto load_scales = [&](int64_t h, uint32_t (&sa)[kTA], uint32_t (&sb)[kTB]) {
        const int hc = (int)(h < kgroups ? h : kgroups - 1);
#pragma unroll
        for (int j = 0; j < kTA; ++j) sa[j] = __builtin_amdgcn_raw_buffer_load_b32(rAs, lane4, sa_row[j] + hc * 256, 0);
#pragma unroll
        for (int i = 0; i < kTB; ++i) sb[i] = __builtin_amdgcn_raw_buffer_load_b32(rBs, lane4, sb_row[i] + hc * 256, 0);
    };

    v4f acc[kTB][kTA];
#pragma unroll
    for (int i = 0; i < kTB; ++i)
#pragma unroll
        for (int j = 0; j < kTA; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    load_scales(0, sa_cur, sb_cur);
    load_step(0);
    store_step(0, true);
    __syncthreads();

    // One 128-wide k-step from LDS buffer buf; OPSEL picks the step's scale byte.
    // The next step's loads are in flight meanwhile; sched_barriers keep the
    // compiler from sinking MFMAs past the buffer hand-over.
    auto one_step = [&](int64_t k, auto opsel_tag) {
        constexpr int OPSEL = decltype(opsel_tag)::value;
        const int buf = (int)(k & 1);
        load_step(k + 1);
        const uint8_t *a_lds = &lds[buf][(wm * kTA) * 1024 + lane16];
        const uint8_t *b_lds = &lds[buf][(kGA + wn * kTB) * 1024 + lane16];
        uint4 af[kTA];
#pragma unroll
        for (int j = 0; j < kTA; ++j) af[j] = *reinterpret_cast<const uint4 *>(a_lds + j * 1024);
        uint4 bnext = *reinterpret_cast<const uint4 *>(b_lds);
#pragma unroll
        for (int i = 0; i < kTB; ++i) {
            const uint4 bcur = bnext;
            if (i + 1 < kTB) bnext = *reinterpret_cast<const uint4 *>(b_lds + (i + 1) * 1024);
            const v8i bop = {(int)bcur.x, (int)bcur.y, (int)bcur.z, (int)bcur.w, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < kTA; ++j) {
                const v8i aop = {(int)af[j].x, (int)af[j].y, (int)af[j].z, (int)af[j].w, 0, 0, 0, 0};
                // MFMA "A" operand = B rows (columns of C), "B" operand = A rows (rows of C)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bop, aop, acc[i][j], kFmtFp4, kFmtFp4, OPSEL, (int)sb_cur[i], OPSEL, (int)sa_cur[j]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();                // every wave is done reading the buffer about to be refilled
        store_step(buf ^ 1, k + 1 < ksteps);
        __syncthreads();                // the refilled buffer is visible
        __builtin_amdgcn_sched_barrier(0);
    };

    for (int64_t h = 0; h < kgroups; ++h) {
        const int64_t k0 = 4 * h;
        load_scales(h + 1, sa_nxt, sb_nxt);
        one_step(k0, std::integral_constant<int, 0>{});
        one_step(k0 + 1, std::integral_constant<int, 1>{});
        one_step(k0 + 2, std::integral_constant<int, 2>{});
        one_step(k0 + 3, std::integral_constant<int, 3>{});
#pragma unroll
        for (int j = 0; j < kTA; ++j) sa_cur[j] = sa_nxt[j];
#pragma unroll
        for (int i = 0; i < kTB; ++i) sb_cur[i] = sb_nxt[i];
    }

    // ---- epilogue: acc[i][j][r] = C[m0 + 16j + lane%16][n0 + 16i + 4*(lane/16) + r]
    const int64_t m0 = (int64_t)tm * kBM + wm * kWM;
    const int64_t n0 = (int64_t)tn * kBN + wn * kWN;
#pragma unroll
    for (int j = 0; j < kTA; ++j) {
        const int64_t row = m0 + 16 * j + (lane & 15);
        if (row >= M) continue;
#pragma unroll
        for (int i = 0; i < kTB; ++i) {
            const int64_t col = n0 + 16 * i + 4 * (lane >> 4);
            const v4f v = acc[i][j];
            if (OUT_BF16) {
                uint16_t *dst = reinterpret_cast<uint16_t *>(C) + row * ldc + col;
                if (col + 3 < N) {
                    uint2 p = {bf16_rne_pair(v[0], v[1]), bf16_rne_pair(v[2], v[3])};
                    *reinterpret_cast<uint2 *>(dst) = p;
                } else {
                    const uint32_t p01 = bf16_rne_pair(v[0], v[1]), p23 = bf16_rne_pair(v[2], v[3]);
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
