// Block-scaled FP6 x FP6 GEMM (C = A . B^T) for gfx950 on tiled MXFP6 blobs.
//
// C[i][j] = sum_k fp6(A[i][k]) 2^(sa[i][k/32]-127) * fp6(B[j][k]) 2^(sb[j][k/32]-127),
// fp32 accumulation, bf16 (RNE) or fp32 output; each operand E2M3 or E3M2
// (OCP MX v1.0 sec. 5.3.2).  The NT product of the MXFP4 linear's forward,
// dgrad and wgrad, with 6-bit elements.
//
// MFMA: V_MFMA_SCALE_F32_32X32X64_F8F6F4 with FP6 formats (2 = E2M3,
// 3 = E3M2).  Lane L of a 32-row operand tile supplies six registers: the
// 24 bytes (32 elements, element i at bits 6i) of row L%32, k-block
// 2*half + L/32, and that block's E8M0 scale through OPSEL.  A tiled atom
// (16 rows x 128 k, 1536 bytes) stores each lane's first 16 bytes in its
// first kilobyte and the last 8 in the remaining 512 bytes, so both parts
// load with aligned ds_read_b128 / ds_read_b64.
//
// Same workgroup shape as the FP4 kernel: 8 waves (two per SIMD), 256x256
// tile, wave tile 128x64 (4x2 MFMA tiles, 128 fp32 accumulators per lane).
// A k-step's 32 atoms take 48 KB of LDS, so the pipeline has 3 stages (plus
// one k-group of scale atoms, 8 KB): step k+2 is in flight while step k
// computes, with the FP4 kernel's schedule (half 0 of step k issues the
// second part of step k+2's DMA, half 1 the first part of step k+3's, whose
// stage is the one step k finished reading at the barrier between the
// halves).  The stage index runs mod 3 and the position in the 4-step scale
// group mod 4, so the k-loop body is 12 steps.  DMA per wave and step: four
// 1 KB low parts and two 1 KB units each holding the high parts of the two
// atoms of one 32-row operand tile, interleaved in 16-byte chunks (chunk c of
// atom 2h+a at position 2c+a), so that the 8-byte reads of a half-wave (16
// rows of each atom) fall on 64 different banks.

#include "mx_internal.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef uint32_t v6u __attribute__((ext_vector_type(6)));   // one lane's FP6 operand
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 256, kBN = 256;        // workgroup tile
constexpr int kWM = 128, kWN = 64;         // wave tile
constexpr int kWavesM = kBM / kWM;         // wave grid 2 x 4
constexpr int kGA = kBM / 16;              // A atoms per k-step per workgroup
constexpr int kGB = kBN / 16;
constexpr int kTA = kWM / 16;
constexpr int kTB = kWN / 16;
constexpr int kMA = kWM / 32;
constexpr int kMB = kWN / 32;
constexpr int kAtoms = kGA + kGB;          // 32 atoms per stage
constexpr int kAtomBytes = 1536;
constexpr int kLoLoads = kAtoms / kWaves;          // 4 low-part DMAs per wave per step
constexpr int kHiLoads = kAtoms / 2 / kWaves;      // 2 high-part DMAs (two atoms each)
constexpr int kLoads = kLoLoads + kHiLoads;        // 6
constexpr int kScaleLoads = kAtoms / kWaves;       // 4 scale atoms per wave per k-group
constexpr int kHalfLoads = kLoads / 2;
constexpr int kHalfScale = kScaleLoads / 2;
constexpr int kSlots = kMA * kMB;                  // MFMAs per wave per half-step
constexpr int kStages = 3;
constexpr int kHiBase = kAtoms * 1024;             // high parts follow the 32 low parts
constexpr int kStageBytes = kAtoms * kAtomBytes;   // 48 KB
constexpr int kRowsPerStage = kStageBytes / (kBN * 2);   // bf16 C rows one stage holds (96)
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

static_assert(kLoads % 2 == 0 && kScaleLoads % 2 == 0, "DMA split");
static_assert(kRowsPerStage * kStages >= kBM, "the bf16 C tile fits the stages");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__shared__ __attribute__((aligned(1024))) uint8_t f6_stage0[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t f6_stage1[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t f6_stage2[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t f6_scale[kAtoms * 256];

template <int S>
__device__ __forceinline__ uint8_t *stage_buf() {
    return S == 0 ? f6_stage0 : S == 1 ? f6_stage1 : f6_stage2;
}
__device__ __forceinline__ uint8_t *stage_dyn(int s) {
    return s == 0 ? f6_stage0 : s == 1 ? f6_stage1 : f6_stage2;
}
// byte address of bf16 C element (r, col) of the staged tile, col % 4 == 0:
// rows [96s, 96s + 96) in stage s, 512 bytes per row, 16-byte chunk c of row
// r at chunk c ^ (r % 32)
__device__ __forceinline__ uint8_t *c_stage(int r, int col) {
    const int s = r / kRowsPerStage, rr = r - s * kRowsPerStage;
    const int chunk = (col >> 3) ^ (r & 31);
    return stage_dyn(s) + rr * (kBN * 2) + chunk * 16 + (col & 7) * 2;
}

#define MX_LDS(p) ((__attribute__((address_space(3))) void *)(p))

constexpr uint32_t kOutOfRange = 0x80000000u;

struct Ctx {
    __amdgpu_buffer_rsrc_t rA, rB, rAs, rBs;
    int lo_row[kLoLoads];   // byte offset of this wave's low-part atom rows (k-step 0)
    uint32_t hi_off[kHiLoads];   // per lane: its atom row's high part (k-step 0)
    int sc_row[kScaleLoads];
    int64_t ksteps, kgroups;
    int wave, lane16, lane4;
};

struct Regs {
    v6u a0[kMA], b0[kMB], a1[kMA], b1[kMB];          // operands of half 0 / half 1
    uint32_t sa[kMA][2], sb[kMB][2];                 // scales of the k-group in use, per half
};

// 24 operand bytes: 16 from the low kilobyte, 8 from the high part
__device__ __forceinline__ v6u read_op(const uint8_t *lo, const uint8_t *hi) {
    const uint4 v = *reinterpret_cast<const uint4 *>(lo);
    const uint2 h = *reinterpret_cast<const uint2 *>(hi);
    return v6u{v.x, v.y, v.z, v.w, h.x, h.y};
}

// DMA instruction V of k-step k into stage S: V < kLoLoads copies the low
// kilobyte of atom kWaves*V + wave; V < kLoads copies the high parts of atoms
// 2h, 2h+1 (h = kWaves*(V - kLoLoads) + wave; lane p fetches chunk p/2 of
// atom 2h + p%2); otherwise (only when k opens a k-group) scale atom
// kWaves*(V - kLoads) + wave.
template <int S, int V>
__device__ __forceinline__ void dma_op(const Ctx &c, int64_t k) {
    if constexpr (V < kLoLoads) {
        const int a = kWaves * V + c.wave;
        const uint32_t base = k < c.ksteps ? (uint32_t)c.lo_row[V] + (uint32_t)(k * kAtomBytes) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a < kGA ? c.rA : c.rB, MX_LDS(stage_buf<S>() + a * 1024), 16,
                                                 base + c.lane16, 0, 0, 0);
    } else if constexpr (V < kLoads) {
        constexpr int R = V - kLoLoads;
        const int h = kWaves * R + c.wave;
        const uint32_t off = k < c.ksteps ? c.hi_off[R] + (uint32_t)(k * kAtomBytes) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(2 * h < kGA ? c.rA : c.rB,
                                                 MX_LDS(stage_buf<S>() + kHiBase + h * 1024), 16, off, 0, 0, 0);
    } else {
        constexpr int R = V - kLoads;
        const int a = kWaves * R + c.wave;
        const int64_t g = k / 4;
        const uint32_t base = g < c.kgroups ? (uint32_t)c.sc_row[R] + (uint32_t)(g * 256) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a < kGA ? c.rAs : c.rBs, MX_LDS(f6_scale + a * 256), 4,
                                                 base + c.lane4, 0, 0, 0);
    }
}

// A k-step's DMA in two parts: part P holds data instructions
// [P*kHalfLoads, (P+1)*kHalfLoads) and, when the step opens a k-group
// (position G == 0), scale instructions [P*kHalfScale, (P+1)*kHalfScale).
__host__ __device__ constexpr int part_ops(int G) { return G == 0 ? kHalfLoads + kHalfScale : kHalfLoads; }
__host__ __device__ constexpr int part_op(int P, int n) {
    return n < kHalfLoads ? kHalfLoads * P + n : kLoads + kHalfScale * P + (n - kHalfLoads);
}
__host__ __device__ constexpr int issued_for(int G) { return 2 * part_ops(G); }
__host__ __device__ constexpr int dma_slot(int n, int nv) {
    const int s = 1 + (n * kSlots) / nv;
    return s > kSlots - 1 ? kSlots - 1 : s;
}

template <int S, int G, int P, int n = 0>
__device__ __forceinline__ void dma_part(const Ctx &c, int64_t k) {
    if constexpr (n < part_ops(G)) {
        dma_op<S, part_op(P, n)>(c, k);
        dma_part<S, G, P, n + 1>(c, k);
    }
}

template <int FA, int FB, int G>
__device__ __forceinline__ void mfma_tile(v16f &acc, const v6u &xb, const v6u &xa, uint32_t sbv, uint32_t sav) {
    const v8i bop = {(int)xb[0], (int)xb[1], (int)xb[2], (int)xb[3], (int)xb[4], (int)xb[5], 0, 0};
    const v8i aop = {(int)xa[0], (int)xa[1], (int)xa[2], (int)xa[3], (int)xa[4], (int)xa[5], 0, 0};
    // MFMA "A" operand = B rows (columns of C), "B" operand = A rows (rows of C)
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bop, aop, acc, FB, FA, G, (int)sbv, G, (int)sav);
}

// Per-lane LDS byte offsets of this wave's first A and B operand tiles
// (half 0): the wave-dependent part is folded in once, so that every read
// adds only a compile-time constant (tile, half) that fits the instruction's
// offset field, and the stages need one base register per part and operand.
struct Lds {
    int lo_a, lo_b;   // low 16 bytes in a stage's low region
    int hi_a, hi_b;   // high 8 bytes in a stage's interleaved high-part units
    int sc_a, sc_b;   // scale dword in the scale atoms
};

// Slot T of half H of the k-step with stage S and k-group position G: MFMA
// T, the LDS reads (low and high part) of operand T of the other half (half 0
// reads the second half of stage S, half 1 the first half of stage S+1), the
// next k-group's scales at G == 3, and this slot's share of the DMA (half 0:
// part 1 of step k+2, half 1: part 0 of step k+3).
template <int FA, int FB, int S, int G, int H, int T>
__device__ __forceinline__ void slot(const Ctx &c, int64_t k, v16f (&acc)[kMB][kMA], Regs &r, const Lds &l) {
    constexpr int i = T / kMA, j = T % kMA;
    if constexpr (H == 0) mfma_tile<FA, FB, G>(acc[i][j], r.b0[i], r.a0[j], r.sb[i][0], r.sa[j][0]);
    else mfma_tile<FA, FB, G>(acc[i][j], r.b1[i], r.a1[j], r.sb[i][1], r.sa[j][1]);

    if constexpr (T < kMA + kMB) {
        constexpr int RS = H == 0 ? S : (S + 1) % kStages;
        constexpr int RH = H == 0 ? 1 : 0;
        const uint8_t *st = stage_buf<RS>();
        if constexpr (T == 0 || T > kMA) {
            constexpr int bi = T == 0 ? 0 : T - kMA;
            const v6u v = read_op(st + l.lo_b + (2 * bi * 1024 + RH * 512), st + kHiBase + l.hi_b + (bi * 1024 + RH * 512));
            if constexpr (H == 0) r.b1[bi] = v; else r.b0[bi] = v;
        } else {
            constexpr int ai = T - 1;
            const v6u v = read_op(st + l.lo_a + (2 * ai * 1024 + RH * 512), st + kHiBase + l.hi_a + (ai * 1024 + RH * 512));
            if constexpr (H == 0) r.a1[ai] = v; else r.a0[ai] = v;
        }
    }
    // Scales of the next k-group: the half-0 entries are free once half 1 of the
    // group's last step runs, the half-1 entries once half 0 of the next
    // group's first step runs; the scale atoms stay in LDS until step 4 of
    // that group issues the following group's DMA.
    constexpr int kScStart = kSlots - (kMA + kMB);
    if constexpr ((H == 1 && G == 3) || (H == 0 && G == 0)) {
        if constexpr (T >= kScStart) {
            constexpr int t = T - kScStart, hh = 1 - H;   // the half whose MFMAs are not running
            if constexpr (t < kMA)
                r.sa[t][hh] = *reinterpret_cast<const uint32_t *>(f6_scale + l.sc_a + (2 * t * 256 + hh * 128));
            else
                r.sb[t - kMA][hh] = *reinterpret_cast<const uint32_t *>(f6_scale + l.sc_b + (2 * (t - kMA) * 256 + hh * 128));
        }
    }

    constexpr int DS = H == 0 ? (S + 2) % kStages : (S + 3) % kStages;
    constexpr int DG = H == 0 ? (G + 2) % 4 : (G + 3) % 4;
    constexpr int P = H == 0 ? 1 : 0;
    constexpr int nv = part_ops(DG);
    const int64_t dk = H == 0 ? k + 2 : k + 3;
    if constexpr (dma_slot(0, nv) == T) dma_op<DS, part_op(P, 0)>(c, dk);
    if constexpr (nv > 1 && dma_slot(1, nv) == T) dma_op<DS, part_op(P, 1)>(c, dk);
    if constexpr (nv > 2 && dma_slot(2, nv) == T) dma_op<DS, part_op(P, 2)>(c, dk);
    if constexpr (nv > 3 && dma_slot(3, nv) == T) dma_op<DS, part_op(P, 3)>(c, dk);
    if constexpr (nv > 4 && dma_slot(4, nv) == T) dma_op<DS, part_op(P, 4)>(c, dk);
    static_assert(part_ops(0) <= 5, "dma slots");
    __builtin_amdgcn_sched_barrier(0);
}

template <int FA, int FB, int S, int G, int H, int T = 0>
__device__ __forceinline__ void half_step(const Ctx &c, int64_t k, v16f (&acc)[kMB][kMA], Regs &r, const Lds &l) {
    if constexpr (T < kSlots) {
        slot<FA, FB, S, G, H, T>(c, k, acc, r, l);
        half_step<FA, FB, S, G, H, T + 1>(c, k, acc, r, l);
    }
}

// One 128-wide k-step; the barrier between the halves waits for this wave's
// DMA of step k+1 (only step k+2's may still be outstanding) and for every
// wave, which publishes step k+1 and frees stage S for step k+3.
template <int FA, int FB, int S, int G>
__device__ __forceinline__ void k_step(const Ctx &c, int64_t k, v16f (&acc)[kMB][kMA], Regs &r, const Lds &l) {
    // an opaque step index keeps the compiler from precomputing every step's
    // addresses of the 12-step loop body into registers
    asm volatile("" : "+s"(k));
    __builtin_amdgcn_sched_barrier(0);
    half_step<FA, FB, S, G, 0>(c, k, acc, r, l);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(issued_for((G + 2) & 3)) : "memory");
    __builtin_amdgcn_sched_barrier(0);
    half_step<FA, FB, S, G, 1>(c, k, acc, r, l);
}

// Epilogue as in the FP4 kernel (bf16: rounded, staged through LDS, written
// as 512-byte row segments; fp32: straight from registers), masked at the edges.
template <bool OUT_BF16>
__device__ __forceinline__ void store_tile(v16f (&acc)[kMB][kMA], int tm, int tn, int64_t M, int64_t N, void *C,
                                           int64_t ldc, int wave, int lane) {
    const int wm = wave % kWavesM, wn = wave / kWavesM;
    const int lrow = lane & 31, lhi = lane >> 5;
    const int64_t tm0 = (int64_t)tm * kBM, tn0 = (int64_t)tn * kBN;
    if (OUT_BF16) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kMA; ++j)
#pragma unroll
            for (int i = 0; i < kMB; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int rl = wm * kWM + 32 * j + lrow, cl = wn * kWN + 32 * i + 8 * q + 4 * lhi;
                    const uint32_t p01 = __builtin_bit_cast(
                        uint32_t, __builtin_convertvector((f32x2_t{acc[i][j][4 * q], acc[i][j][4 * q + 1]}), bf16x2_t));
                    const uint32_t p23 = __builtin_bit_cast(
                        uint32_t, __builtin_convertvector((f32x2_t{acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]}), bf16x2_t));
                    *reinterpret_cast<uint2 *>(c_stage(rl, cl)) = uint2{p01, p23};
                }
        __syncthreads();
        constexpr int kRowsPerWave = kBM / kWaves;
        const int cl = (lane & 31) * 8;
        const int64_t col = tn0 + cl;
        uint4 v[kRowsPerWave / 2];
#pragma unroll
        for (int it = 0; it < kRowsPerWave / 2; ++it)
            v[it] = *reinterpret_cast<const uint4 *>(c_stage(kRowsPerWave * wave + 2 * it + (lane >> 5), cl));
        uint16_t *dst0 = reinterpret_cast<uint16_t *>(C) + (tm0 + kRowsPerWave * wave + (lane >> 5)) * ldc + col;
        if (tm0 + kBM <= M && tn0 + kBN <= N) {
#pragma unroll
            for (int it = 0; it < kRowsPerWave / 2; ++it)
                __builtin_nontemporal_store(__builtin_bit_cast(v4u_t, v[it]), reinterpret_cast<v4u_t *>(dst0 + 2 * it * ldc));
        } else {
#pragma unroll
            for (int it = 0; it < kRowsPerWave / 2; ++it) {
                const int64_t row = tm0 + kRowsPerWave * wave + 2 * it + (lane >> 5);
                if (row >= M || col >= N) continue;
                uint16_t *dst = dst0 + 2 * it * ldc;
                if (col + 7 < N) {
                    *reinterpret_cast<uint4 *>(dst) = v[it];
                } else {
                    const uint32_t w4[4] = {v[it].x, v[it].y, v[it].z, v[it].w};
#pragma unroll
                    for (int e = 0; e < 7; ++e)
                        if (col + e < N) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
    } else {
        const int64_t m0 = tm0 + wm * kWM, n0 = tn0 + wn * kWN;
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
                    float *dst = reinterpret_cast<float *>(C) + row * ldc + col;
                    if (col + 3 < N) {
                        *reinterpret_cast<v4f *>(dst) = v;
                    } else {
#pragma unroll
                        for (int e = 0; e < 3; ++e)
                            if (col + e < N) dst[e] = v[e];
                    }
                }
            }
        }
    }
}

template <bool OUT_BF16, int FA, int FB>
__global__ __launch_bounds__(kThreads) void gemm_fp6_kernel(int64_t M, int64_t N, int64_t K_pad, int tiles_m,
                                                            int tiles_n, const uint8_t *__restrict__ A,
                                                            const uint8_t *__restrict__ As,
                                                            const uint8_t *__restrict__ B,
                                                            const uint8_t *__restrict__ Bs, void *__restrict__ C,
                                                            int64_t ldc) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % kWavesM, wn = wave / kWavesM;

    // tile order: XCD-contiguous ranges, bands of kGroupM tile rows
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

    Ctx c;
    c.ksteps = K_pad / 128;
    c.kgroups = cdiv(K_pad, 512);
    c.wave = wave;
    c.lane16 = lane * 16;
    c.lane4 = lane * 4;
    const int64_t nGA = cdiv(M, 16), nGB = cdiv(N, 16);
    const int64_t gA0 = (int64_t)tm * kGA, gB0 = (int64_t)tn * kGB;
    c.rA = make_rsrc(A, nGA * c.ksteps * kAtomBytes);
    c.rB = make_rsrc(B, nGB * c.ksteps * kAtomBytes);
    c.rAs = make_rsrc(As, nGA * c.kgroups * 256);
    c.rBs = make_rsrc(Bs, nGB * c.kgroups * 256);
    // Row groups past an operand are clamped to its last group (those rows of
    // C are never stored).
    auto group_of = [&](int a) -> int64_t {
        const bool isA = a < kGA;
        int64_t g = isA ? gA0 + a : gB0 + (a - kGA);
        const int64_t gmax = (isA ? nGA : nGB) - 1;
        return g < gmax ? g : gmax;
    };
#pragma unroll
    for (int r = 0; r < kLoLoads; ++r) c.lo_row[r] = (int)(group_of(kWaves * r + wave) * c.ksteps * kAtomBytes);
#pragma unroll
    for (int r = 0; r < kHiLoads; ++r) {
        const int h = kWaves * r + wave;
        const int a = 2 * h + (lane & 1);
        c.hi_off[r] = (uint32_t)(group_of(a) * c.ksteps * kAtomBytes) + 1024u + (uint32_t)((lane >> 1) * 16);
    }
#pragma unroll
    for (int r = 0; r < kScaleLoads; ++r) c.sc_row[r] = (int)(group_of(kWaves * r + wave) * c.kgroups * 256);

    v16f acc[kMB][kMA];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kMA; ++j) acc[i][j] = v16f{};

    // Prologue: steps 0 and 1 whole, the first part of step 2.
    dma_part<0, 0, 0>(c, 0);
    dma_part<0, 0, 1>(c, 0);
    dma_part<1, 1, 0>(c, 1);
    dma_part<1, 1, 1>(c, 1);
    dma_part<2, 2, 0>(c, 2);

    const int lrow = lane & 31, lhi = lane >> 5;
    Lds l;
    {
        // lane L of a 32-row tile: row L%32 = atom (L%32)/16, slice s = L%16 + 16*(L/32) (half 0)
        const int sl = (lrow & 15) + 16 * lhi;
        const int frag_off = ((lrow >> 4) * 1024) + sl * 16;
        // high parts: slice s of atom 2t + a at chunk position 2(s/2) + a, 8 bytes in per s%2
        const int frag_hi = 32 * (sl >> 1) + 16 * (lrow >> 4) + 8 * (sl & 1);
        const int sc_off = ((lrow >> 4) * 256) + sl * 4;
        const int a0 = wm * kTA, b0 = kGA + wn * kTB;     // first atoms of the wave's A and B tiles
        l.lo_a = frag_off + a0 * 1024;
        l.lo_b = frag_off + b0 * 1024;
        l.hi_a = frag_hi + (a0 / 2) * 1024;
        l.hi_b = frag_hi + (b0 / 2) * 1024;
        l.sc_a = sc_off + a0 * 256;
        l.sc_b = sc_off + b0 * 256;
    }

    Regs r;
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(issued_for(1) + part_ops(2)) : "memory");
#pragma unroll
    for (int t = 0; t < kMA; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            r.sa[t][hh] = *reinterpret_cast<const uint32_t *>(f6_scale + l.sc_a + t * 512 + hh * 128);
#pragma unroll
    for (int t = 0; t < kMB; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            r.sb[t][hh] = *reinterpret_cast<const uint32_t *>(f6_scale + l.sc_b + t * 512 + hh * 128);
#pragma unroll
    for (int t = 0; t < kMA; ++t)
        r.a0[t] = read_op(f6_stage0 + l.lo_a + t * 2048, f6_stage0 + kHiBase + l.hi_a + t * 1024);
#pragma unroll
    for (int t = 0; t < kMB; ++t)
        r.b0[t] = read_op(f6_stage0 + l.lo_b + t * 2048, f6_stage0 + kHiBase + l.hi_b + t * 1024);

    // 12 steps per iteration: stage k % 3, k-group position k % 4.  Steps past
    // K_pad load zeros (out-of-range DMA) and add nothing.
    for (int64_t k = 0; k < c.ksteps; k += 12) {
        k_step<FA, FB, 0, 0>(c, k, acc, r, l);
        k_step<FA, FB, 1, 1>(c, k + 1, acc, r, l);
        k_step<FA, FB, 2, 2>(c, k + 2, acc, r, l);
        k_step<FA, FB, 0, 3>(c, k + 3, acc, r, l);
        k_step<FA, FB, 1, 0>(c, k + 4, acc, r, l);
        k_step<FA, FB, 2, 1>(c, k + 5, acc, r, l);
        k_step<FA, FB, 0, 2>(c, k + 6, acc, r, l);
        k_step<FA, FB, 1, 3>(c, k + 7, acc, r, l);
        k_step<FA, FB, 2, 0>(c, k + 8, acc, r, l);
        k_step<FA, FB, 0, 1>(c, k + 9, acc, r, l);
        k_step<FA, FB, 1, 2>(c, k + 10, acc, r, l);
        k_step<FA, FB, 2, 3>(c, k + 11, acc, r, l);
    }
    // drain the DMAs still in flight before LDS is reused
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    store_tile<OUT_BF16>(acc, tm, tn, M, N, C, ldc, wave, lane);
}

template <typename T>
__global__ void fill_zero_kernel(T *C, int64_t M, int64_t N, int64_t ldc) {
    const int64_t n = M * N;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x)
        C[(e / N) * ldc + e % N] = T(0);
}

template <bool OUT_BF16>
auto pick_kernel(int fa, int fb) {
    if (fa == 2) return fb == 2 ? gemm_fp6_kernel<OUT_BF16, 2, 2> : gemm_fp6_kernel<OUT_BF16, 2, 3>;
    return fb == 2 ? gemm_fp6_kernel<OUT_BF16, 3, 2> : gemm_fp6_kernel<OUT_BF16, 3, 3>;
}

}  // namespace

hipError_t launch_gemm_fp6(int64_t M, int64_t N, int64_t K, int fmt_a, const uint8_t *A, const uint8_t *As,
                           int fmt_b, const uint8_t *B, const uint8_t *Bs, mx_dtype out_dtype, void *C, int64_t ldc,
                           hipStream_t stream) {
    const int64_t K_pad = padded(K);
    if (K_pad == 0) {
        const int64_t n = M * N;
        dim3 grid((unsigned)(cdiv(n, 256) < 65536 ? cdiv(n, 256) : 65536));
        if (out_dtype == MX_BF16)
            hipLaunchKernelGGL(fill_zero_kernel<uint16_t>, grid, dim3(256), 0, stream,
                               reinterpret_cast<uint16_t *>(C), M, N, ldc);
        else
            hipLaunchKernelGGL(fill_zero_kernel<float>, grid, dim3(256), 0, stream, reinterpret_cast<float *>(C), M,
                               N, ldc);
        return hipGetLastError();
    }
    // buffer offsets are 32-bit: each operand blob must stay below 2 GiB
    if (cdiv(M, 16) * (K_pad / 128) * kAtomBytes >= (int64_t(1) << 31) ||
        cdiv(N, 16) * (K_pad / 128) * kAtomBytes >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
    const int tiles_m = (int)cdiv(M, kBM), tiles_n = (int)cdiv(N, kBN);
    const int tiles = tiles_m * tiles_n;
    // whole rounds here; a last round that would fill at most a quarter of the
    // CUs goes to the 128x128 tail kernel (gemm_fp6_tail.hip).  (Same-box A/B
    // on the fc2 shapes: 64 leftover tiles -7.5%; 96 no gain; 128 +1%.)
    const int cus = device_cu_count();
    const int tail = (cus > 0 && tiles > cus && tiles % cus <= cus / 4) ? tiles % cus : 0;
    auto kernel = out_dtype == MX_BF16 ? pick_kernel<true>(fmt_a, fmt_b) : pick_kernel<false>(fmt_a, fmt_b);
    hipLaunchKernelGGL(kernel, dim3((unsigned)(tiles - tail)), dim3(kThreads), 0, stream, M, N, K_pad, tiles_m,
                       tiles_n, A, As, B, Bs, C, ldc);
    if (tail) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_gemm_fp6_tail(M, N, K_pad, tiles_m, tiles_n, tiles - tail, tail, fmt_a, A, As, fmt_b, B, Bs,
                                    out_dtype, C, ldc, stream);
    }
    return hipGetLastError();
}

}  // namespace mx
