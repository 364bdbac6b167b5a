// Tail kernel of the block-scaled FP4 x FP4 GEMM (C = A . B^T): the same
// product as the main kernel in gemm.hip, on 128x128 output tiles.
//
// The main kernel's 256x256 tiles run in rounds of one tile per CU; when the
// tile count is not a multiple of the CU count, its last round leaves most
// CUs idle (the fc2 forward's 864 tiles fill 256 CUs 3.375 times, the wgrad's
// 576 2.25 times).  The launcher gives the main kernel the whole rounds and
// this kernel the leftover 256x256 tiles, each as four 128x128 tiles, so the
// last round is spread over the chip.  Same MFMA, operand layout, DMA
// pipeline and slot schedule as the main kernel, scaled down: 4 waves of
// 64x64 (2x2 MFMA tiles), 16 atoms (16 KB) per LDS stage, so two workgroups
// fit one CU and each SIMD still interleaves two waves.
//
// When the leftover tiles give at most one 128x128 tile per CU (the fc2 and
// fc1 wgrad: 64 leftover 256x256 tiles on 256 CUs), a lone 4-wave workgroup
// would leave each SIMD one wave with nothing to hide its waits behind.  The
// split form then runs two groups of 4 waves per workgroup on the same tile,
// each group the pipeline above over one half of K (its own LDS stages), and
// adds the two fp32 partial tiles through LDS before the epilogue.

#include <type_traits>

#include "mx_internal.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));

constexpr int kFmtFp4 = 4;                 // MFMA f8f6f4 format code for E2M1
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 128, kBN = 128;        // workgroup tile
constexpr int kWM = 64, kWN = 64;          // wave tile
constexpr int kWavesM = kBM / kWM;         // wave grid 2 x 2
constexpr int kGA = kBM / 16;              // A atoms (16-row groups) per k-step per workgroup
constexpr int kGB = kBN / 16;
constexpr int kTA = kWM / 16;              // A atoms per wave
constexpr int kTB = kWN / 16;
constexpr int kMA = kWM / 32;              // 32x32 MFMA tiles per wave along M (A rows)
constexpr int kMB = kWN / 32;              // ... along N (B rows)
constexpr int kAtoms = kGA + kGB;          // atoms per stage
constexpr int kLoads = kAtoms / kWaves;    // data DMAs per wave per k-step
constexpr int kHalfLoads = kLoads / 2;
constexpr int kSlots = kMA * kMB;          // MFMAs per wave per half-step
constexpr int kGroupM = 8;                 // tile rows per band in the tile order

static_assert(kAtoms % kWaves == 0 && kLoads % 2 == 0, "DMA split");
static_assert(kMA + kMB <= kSlots, "one operand read per slot");

// Buffer resource over [p, p + bytes).  Loads address it with a per-lane
// byte offset; an offset at or past `bytes` reads zeros (the hardware range
// check of raw buffers), which is how k-steps past K_pad become zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// LDS: 4 k-step stages of 16 atoms and one k-group of scale atoms, as
// separate arrays so that the compiler can tell a DMA into one stage from a
// read of another.  After the k-loop the stages hold the bf16 C tile: rows
// [32s, 32s + 32) in stage s, 256 bytes per row, 16-byte chunk c of row r at
// chunk c ^ (r % 16) so that reads and writes of a column of rows spread
// over all banks.
constexpr int kStageBytes = kAtoms * 1024;
static_assert(kBN * 2 * (kBM / 4) <= kStageBytes, "a quarter of the bf16 C tile fits one stage");
__shared__ __attribute__((aligned(1024))) uint8_t g_stage0[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage1[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage2[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage3[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_scale[kAtoms * 256];
// the second K group's pipeline (split form only)
__shared__ __attribute__((aligned(1024))) uint8_t g_stage4[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage5[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage6[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage7[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_scale1[kAtoms * 256];

// stage S of K group G (G = 0 in the plain form)
template <int S, int G = 0>
__device__ __forceinline__ uint8_t *stage_buf() {
    if constexpr (G == 0) return S == 0 ? g_stage0 : S == 1 ? g_stage1 : S == 2 ? g_stage2 : g_stage3;
    else return S == 0 ? g_stage4 : S == 1 ? g_stage5 : S == 2 ? g_stage6 : g_stage7;
}
template <int G = 0>
__device__ __forceinline__ uint8_t *scale_buf() { return G == 0 ? g_scale : g_scale1; }
__device__ __forceinline__ uint8_t *stage_dyn(int s) {
    return s == 0 ? g_stage0 : s == 1 ? g_stage1 : s == 2 ? g_stage2 : g_stage3;
}
// byte address of bf16 C element (r, col) of the staged tile, col % 4 == 0
__device__ __forceinline__ uint8_t *c_stage(int r, int col) {
    const int chunk = (col >> 3) ^ (r & 15);
    return stage_dyn(r >> 5) + (r & 31) * (kBN * 2) + chunk * 16 + (col & 7) * 2;
}

#define MX_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Offset that lies past every operand buffer: a buffer load there returns 0.
constexpr uint32_t kOutOfRange = 0x80000000u;

struct GemmCtx {
    __amdgpu_buffer_rsrc_t rA, rB, rAs, rBs;
    int ld_row[kLoads];    // byte offset of this wave's r-th atom row (k-step 0)
    int sc_row[kLoads];    // byte offset of this wave's r-th scale-atom row (k-group 0)
    int64_t ksteps, kgroups;
    int wave, lane16, lane4;
};

struct Regs {
    uint4 a0[kMA], b0[kMB], a1[kMA], b1[kMB];       // operands of half 0 / half 1
    uint32_t sa[kMA][2], sb[kMB][2];                // scales of the current k-group
    uint32_t sa_n[kMA][2], sb_n[kMB][2];            // ... of the next one
};

// DMA instruction V of k-step k into stage S = k % 4: V < kLoads copies data
// atom kWaves*V + wave; V >= kLoads (only when k opens a k-group) copies scale
// atom kWaves*(V - kLoads) + wave.  Past K_pad the offset is out of range and
// the atom lands as zeros.
template <int S, int V, int G>
__device__ __forceinline__ void dma_op(const GemmCtx &c, int64_t k) {
    if constexpr (V < kLoads) {
        const int a = kWaves * V + c.wave;
        const uint32_t base = k < c.ksteps ? (uint32_t)c.ld_row[V] + (uint32_t)(k * 1024) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a < kGA ? c.rA : c.rB, MX_LDS((stage_buf<S, G>() + a * 1024)), 16,
                                                 base + c.lane16, 0, 0, 0);
    } else {
        constexpr int R = V - kLoads;
        const int a = kWaves * R + c.wave;
        const int64_t h = k / 4;
        const uint32_t base = h < c.kgroups ? (uint32_t)c.sc_row[R] + (uint32_t)(h * 256) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a < kGA ? c.rAs : c.rBs, MX_LDS(scale_buf<G>() + a * 256), 4,
                                                 base + c.lane4, 0, 0, 0);
    }
}

// A k-step's DMA is issued in two parts: part P holds data atoms
// [P*kHalfLoads, (P+1)*kHalfLoads) and, when the step opens a k-group, the
// scale atoms with the same indices.
__host__ __device__ constexpr int part_ops(int S) { return S == 0 ? 2 * kHalfLoads : kHalfLoads; }
__host__ __device__ constexpr int part_op(int S, int P, int n) {
    return n < kHalfLoads ? kHalfLoads * P + n : kLoads + kHalfLoads * P + (n - kHalfLoads);
}
// vector-memory instructions a wave issues for a k-step with stage S
__host__ __device__ constexpr int issued_for(int S) { return 2 * part_ops(S); }
// slot of the n-th of nv DMA instructions in a half-step
__host__ __device__ constexpr int dma_slot(int n, int nv) {
    const int s = 1 + (n * kSlots) / nv;
    return s > kSlots - 1 ? kSlots - 1 : s;
}

template <int S, int P, int G, int n = 0>
__device__ __forceinline__ void dma_part(const GemmCtx &c, int64_t k) {
    if constexpr (n < part_ops(S)) {
        dma_op<S, part_op(S, P, n), G>(c, k);
        dma_part<S, P, G, n + 1>(c, k);
    }
}

template <int S>
__device__ __forceinline__ void mfma_tile(v16f &acc, const uint4 &xb, const uint4 &xa, uint32_t sbv, uint32_t sav) {
    const v8i bop = {(int)xb.x, (int)xb.y, (int)xb.z, (int)xb.w, 0, 0, 0, 0};
    const v8i aop = {(int)xa.x, (int)xa.y, (int)xa.z, (int)xa.w, 0, 0, 0, 0};
    // MFMA "A" operand = B rows (columns of C), "B" operand = A rows (rows of C)
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bop, aop, acc, kFmtFp4, kFmtFp4, S, (int)sbv, S,
                                                          (int)sav);
}

struct Lds {
    int frag_off;   // this lane's slice within a 32-row pair of atoms (half 0)
    int sc_off;     // ... within a pair of scale atoms
    int a_atom0;    // first A atom of this wave's rows
    int b_atom0;    // first B atom of this wave's columns
};

// Slot T of half H of the k-step with stage S.
//  - MFMA T: tile (i, j) = (T / kMA, T % kMA) with the operands of half H.
//  - LDS read T (T < kMA + kMB) of the other operand set: half 0 reads the
//    second half of stage S, half 1 the first half of stage S+1, in order of
//    first use (b[0], a[0..kMA), b[1..kMB)).
//  - at S == 3, half 1 also reads the next k-group's scales, two per slot.
//  - the DMA instructions this slot carries (half 0: part 1 of step k+2,
//    half 1: part 0 of step k+3).
template <int S, int H, int T, int G>
__device__ __forceinline__ void slot(const GemmCtx &c, int64_t k, v16f (&acc)[kMB][kMA], Regs &r, const Lds &l) {
    constexpr int i = T / kMA, j = T % kMA;
    if constexpr (H == 0) mfma_tile<S>(acc[i][j], r.b0[i], r.a0[j], r.sb[i][0], r.sa[j][0]);
    else mfma_tile<S>(acc[i][j], r.b1[i], r.a1[j], r.sb[i][1], r.sa[j][1]);

    if constexpr (T < kMA + kMB) {
        constexpr int RS = H == 0 ? S : ((S + 1) & 3);
        constexpr int RH = H == 0 ? 1 : 0;
        const uint8_t *st = stage_buf<RS, G>() + l.frag_off + RH * 512;
        if constexpr (T == 0 || T > kMA) {
            constexpr int bi = T == 0 ? 0 : T - kMA;
            const uint4 v = *reinterpret_cast<const uint4 *>(st + (l.b_atom0 + 2 * bi) * 1024);
            if constexpr (H == 0) r.b1[bi] = v; else r.b0[bi] = v;
        } else {
            constexpr int ai = T - 1;
            const uint4 v = *reinterpret_cast<const uint4 *>(st + (l.a_atom0 + 2 * ai) * 1024);
            if constexpr (H == 0) r.a1[ai] = v; else r.a0[ai] = v;
        }
    }
    constexpr int kScStart = kSlots - (kMA + kMB);
    if constexpr (H == 1 && S == 3 && T >= kScStart) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int q = 2 * (T - kScStart) + e;
            const int hh = q & 1, t = q >> 1;
            if (t < kMA)
                r.sa_n[t][hh] = *reinterpret_cast<const uint32_t *>(scale_buf<G>() + (l.a_atom0 + 2 * t) * 256 + l.sc_off + hh * 128);
            else
                r.sb_n[t - kMA][hh] =
                    *reinterpret_cast<const uint32_t *>(scale_buf<G>() + (l.b_atom0 + 2 * (t - kMA)) * 256 + l.sc_off + hh * 128);
        }
    }

    constexpr int DS = H == 0 ? ((S + 2) & 3) : ((S + 3) & 3);
    constexpr int P = H == 0 ? 1 : 0;
    constexpr int nv = part_ops(DS);
    const int64_t dk = H == 0 ? k + 2 : k + 3;
    if constexpr (dma_slot(0, nv) == T) dma_op<DS, part_op(DS, P, 0), G>(c, dk);
    if constexpr (nv > 1 && dma_slot(1, nv) == T) dma_op<DS, part_op(DS, P, 1), G>(c, dk);
    if constexpr (nv > 2 && dma_slot(2, nv) == T) dma_op<DS, part_op(DS, P, 2), G>(c, dk);
    if constexpr (nv > 3 && dma_slot(3, nv) == T) dma_op<DS, part_op(DS, P, 3), G>(c, dk);
    static_assert(part_ops(0) <= 4, "dma slots");
    // keep this slot's instructions in this slot
    __builtin_amdgcn_sched_barrier(0);
}

template <int S, int H, int G, int T = 0>
__device__ __forceinline__ void half_step(const GemmCtx &c, int64_t k, v16f (&acc)[kMB][kMA], Regs &r, const Lds &l) {
    if constexpr (T < kSlots) {
        slot<S, H, T, G>(c, k, acc, r, l);
        half_step<S, H, G, T + 1>(c, k, acc, r, l);
    }
}

// One 128-wide k-step.  The barrier waits for this wave's DMA of step k+1
// (only step k+2's instructions may still be outstanding) and then for every
// wave, which publishes step k+1 and certifies that all reads of step k-1's
// stage are done before half 1 starts overwriting it.
template <int S, int G>
__device__ __forceinline__ void k_step(const GemmCtx &c, int64_t k, v16f (&acc)[kMB][kMA], Regs &r, const Lds &l) {
    __builtin_amdgcn_sched_barrier(0);
    half_step<S, 0, G>(c, k, acc, r, l);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(issued_for((S + 2) & 3)) : "memory");
    __builtin_amdgcn_sched_barrier(0);
    half_step<S, 1, G>(c, k, acc, r, l);
    if constexpr (S == 3) {
#pragma unroll
        for (int t = 0; t < kMA; ++t) { r.sa[t][0] = r.sa_n[t][0]; r.sa[t][1] = r.sa_n[t][1]; }
#pragma unroll
        for (int t = 0; t < kMB; ++t) { r.sb[t][0] = r.sb_n[t][0]; r.sb[t][1] = r.sb_n[t][1]; }
    }
}

// Epilogue: write the 128x128 tile (tm, tn) of C from the accumulators;
// acc[i][j][r] = C[m0 + 32j + lane%32][n0 + 32i + 8(r/4) + 4(lane/32) + r%4].
// bf16: rounded (V_CVT_PK_BF16_F32, nearest even), staged in LDS, then
// written as whole 256-byte row segments (each store instruction covers 4
// rows with 16 bytes per lane; non-temporal, as C is not read again here);
// fp32: 16 bytes per lane straight from registers.  Masked at the M/N edges.
// NG K groups share the workgroup: group 0 holds the summed accumulators
// (wave = its index in the group); all NG * kWaves waves (index wave_all)
// take part in the bf16 stores.
template <bool OUT_BF16, int NG>
__device__ __forceinline__ void store_tile(v16f (&acc)[kMB][kMA], int tm, int tn, int64_t M, int64_t N, void *C,
                                           int64_t ldc, int group, int wave, int wave_all, int lane) {
    const int wm = wave % kWavesM, wn = wave / kWavesM;
    const int lrow = lane & 31, lhi = lane >> 5;
    const int64_t tm0 = (int64_t)tm * kBM, tn0 = (int64_t)tn * kBN;
    if (OUT_BF16) {
        // Every wave waited for its own DMAs; the barrier makes sure all of
        // them have landed and every stage read is done before the tile
        // overwrites the stages.
        __syncthreads();
        if (group == 0) {
#pragma unroll
            for (int j = 0; j < kMA; ++j)
#pragma unroll
                for (int i = 0; i < kMB; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int rl = wm * kWM + 32 * j + lrow, cl = wn * kWN + 32 * i + 8 * q + 4 * lhi;
                        const uint32_t p01 = __builtin_bit_cast(
                            uint32_t,
                            __builtin_convertvector((f32x2_t{acc[i][j][4 * q], acc[i][j][4 * q + 1]}), bf16x2_t));
                        const uint32_t p23 = __builtin_bit_cast(
                            uint32_t,
                            __builtin_convertvector((f32x2_t{acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]}), bf16x2_t));
                        *reinterpret_cast<uint2 *>(c_stage(rl, cl)) = uint2{p01, p23};
                    }
        }
        __syncthreads();
        constexpr int kRowsPerWave = kBM / (kWaves * NG);   // 32 or 16: instructions of 4 rows
        const int cl = (lane & 15) * 8;
        const int64_t col = tn0 + cl;
        uint4 v[kRowsPerWave / 4];
#pragma unroll
        for (int it = 0; it < kRowsPerWave / 4; ++it)
            v[it] = *reinterpret_cast<const uint4 *>(c_stage(kRowsPerWave * wave_all + 4 * it + (lane >> 4), cl));
        uint16_t *dst0 = reinterpret_cast<uint16_t *>(C) + (tm0 + kRowsPerWave * wave_all + (lane >> 4)) * ldc + col;
        if (tm0 + kBM <= M && tn0 + kBN <= N) {
#pragma unroll
            for (int it = 0; it < kRowsPerWave / 4; ++it)
                __builtin_nontemporal_store(__builtin_bit_cast(v4u_t, v[it]), reinterpret_cast<v4u_t *>(dst0 + 4 * it * ldc));
        } else {
#pragma unroll
            for (int it = 0; it < kRowsPerWave / 4; ++it) {
                const int64_t row = tm0 + kRowsPerWave * wave_all + 4 * it + (lane >> 4);
                if (row >= M || col >= N) continue;
                uint16_t *dst = dst0 + 4 * it * ldc;
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
        if (group != 0) return;
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

// The k-loop of K group G: prologue DMAs, then `iters` k-groups of 4 k-steps
// (k-steps at or past c.ksteps land as zeros), then the drain of the trailing
// DMAs.  Every wave of the workgroup runs the same number of k-steps, so the
// per-step barriers line up across groups.
template <int G>
__device__ __forceinline__ void run_k(const GemmCtx &c, v16f (&acc)[kMB][kMA], const Lds &l, int64_t iters) {
    // Prologue: steps 0 and 1 whole, the first part of step 2 (its second
    // part goes out in step 0's first half).
    dma_part<0, 0, G>(c, 0);
    dma_part<0, 1, G>(c, 0);
    dma_part<1, 0, G>(c, 1);
    dma_part<1, 1, G>(c, 1);
    dma_part<2, 0, G>(c, 2);

    Regs r;
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(issued_for(1) + part_ops(2)) : "memory");
#pragma unroll
    for (int t = 0; t < kMA; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            r.sa[t][hh] =
                *reinterpret_cast<const uint32_t *>(scale_buf<G>() + (l.a_atom0 + 2 * t) * 256 + l.sc_off + hh * 128);
#pragma unroll
    for (int t = 0; t < kMB; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            r.sb[t][hh] =
                *reinterpret_cast<const uint32_t *>(scale_buf<G>() + (l.b_atom0 + 2 * t) * 256 + l.sc_off + hh * 128);
#pragma unroll
    for (int t = 0; t < kMA; ++t)
        r.a0[t] = *reinterpret_cast<const uint4 *>(stage_buf<0, G>() + (l.a_atom0 + 2 * t) * 1024 + l.frag_off);
#pragma unroll
    for (int t = 0; t < kMB; ++t)
        r.b0[t] = *reinterpret_cast<const uint4 *>(stage_buf<0, G>() + (l.b_atom0 + 2 * t) * 1024 + l.frag_off);

    for (int64_t h = 0; h < iters; ++h) {
        const int64_t k0 = 4 * h;
        k_step<0, G>(c, k0, acc, r, l);
        k_step<1, G>(c, k0 + 1, acc, r, l);
        k_step<2, G>(c, k0 + 2, acc, r, l);
        k_step<3, G>(c, k0 + 3, acc, r, l);
    }
    // drain the trailing (out-of-range) DMAs before LDS is reused
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Split form: 4 KB of the second group's stages per accumulator tile of a
// wave (wave w of the group owns stage 4 + w), float e of lane L at
// (e * 64 + L) * 4, so consecutive lanes touch consecutive banks.
__device__ __forceinline__ float *partial_slot(int wave, int tile) {
    uint8_t *base = wave == 0 ? g_stage4 : wave == 1 ? g_stage5 : wave == 2 ? g_stage6 : g_stage7;
    return reinterpret_cast<float *>(base + tile * 4096);
}

// BIAS: C[i][j] = (sum) + bias[j], bias a bf16 vector of N, added in fp32
// before the output rounding.
// Workgroup b computes quarter b % 4 of 256x256 tile first + b / 4 of the
// main kernel's tile order (tiles_m x tiles_n 256x256 tiles, bands of 8 rows).
// SPLIT: 8 waves, K group g = wave / 4 takes k-groups [g * kg0, ...) of the
// tile (kg0 = half of them, rounded up); group 1's partial tile is added into
// group 0's through LDS before the epilogue.
template <bool OUT_BF16, bool BIAS, bool SPLIT>
__global__ __launch_bounds__(SPLIT ? 2 * kThreads : kThreads) void gemm_a4w4_tail_kernel(
    int64_t M, int64_t N, int64_t K_pad, int tiles_m, int tiles_n, int first, const uint8_t *__restrict__ A,
    const uint8_t *__restrict__ As, const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
    const uint16_t *__restrict__ bias, void *__restrict__ C, int64_t ldc) {
    constexpr int NG = SPLIT ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int group = SPLIT ? wave_all / kWaves : 0;
    const int wave = wave_all % kWaves;
    const int wm = wave % kWavesM, wn = wave / kWavesM;

    // ---- which 128x128 tile: quarter of a leftover 256x256 tile of the main order
    const int id = first + (int)(blockIdx.x >> 2), quarter = (int)(blockIdx.x & 3);
    const int band = kGroupM * tiles_n;
    const int first_m = (id / band) * kGroupM;
    const int gsz = min(tiles_m - first_m, kGroupM);
    const int tm = 2 * (first_m + (id % band) % gsz) + (quarter >> 1);
    const int tn = 2 * ((id % band) / gsz) + (quarter & 1);

    const int64_t ksteps = K_pad / 128, kgroups = cdiv(K_pad, 512);
    // k-groups of group 0 (all of them without the split); group 1 starts at k-group kg0
    const int64_t kg0 = SPLIT ? (kgroups + 1) / 2 : kgroups;
    const int64_t kfirst = group ? 4 * kg0 : 0;
    GemmCtx c;
    c.ksteps = group ? ksteps - kfirst : (SPLIT ? (ksteps < 4 * kg0 ? ksteps : 4 * kg0) : ksteps);
    c.kgroups = group ? kgroups - kg0 : kg0;
    c.wave = wave;
    c.lane16 = lane * 16;
    c.lane4 = lane * 4;
    const int64_t nGA = cdiv(M, 16), nGB = cdiv(N, 16);   // row groups present in memory
    const int64_t gA0 = (int64_t)tm * kGA, gB0 = (int64_t)tn * kGB;
    c.rA = make_rsrc(A, nGA * ksteps * 1024);
    c.rB = make_rsrc(B, nGB * ksteps * 1024);
    c.rAs = make_rsrc(As, nGA * kgroups * 256);
    c.rBs = make_rsrc(Bs, nGB * kgroups * 256);

    // This lane's bias values (columns n0 + 32i + 8q + 4(lane/32) + 0..3 of its
    // tile, 4 bf16 per (i, q)), loaded before the k-loop so they have long
    // arrived by the epilogue.  The range check of a buffer load zeroes whole
    // dwords, so the range ends at the 16-byte boundary after the last entry
    // (the bias is 16-byte aligned, so that block is inside the caller's
    // allocation's last page); columns past it read 0, columns past N are
    // never stored.
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    v2u bias_bits[BIAS ? kMB * 4 : 1];
    if constexpr (BIAS) {
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias, cdiv(N * 2, 16) * 16);
        const int col0 = tn * kBN + wn * kWN + 4 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                bias_bits[i * 4 + q] = __builtin_amdgcn_raw_buffer_load_b64(rb, (col0 + 32 * i + 8 * q) * 2, 0, 0);
    }
    // Row groups past an operand are clamped to its last group: those rows of C
    // are never stored, so their contents do not matter.  A group's offsets
    // start at its first k-step.
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
        const int a = kWaves * r + wave;
        const bool isA = a < kGA;
        int64_t g = isA ? gA0 + a : gB0 + (a - kGA);
        const int64_t gmax = (isA ? nGA : nGB) - 1;
        g = g < gmax ? g : gmax;
        c.ld_row[r] = (int)((g * ksteps + kfirst) * 1024);
        c.sc_row[r] = (int)((g * kgroups + kfirst / 4) * 256);
    }

    v16f acc[kMB][kMA];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kMA; ++j) acc[i][j] = v16f{};

    // Lane L of a 32-row operand tile takes row L%32, k-block 2*half + L/32:
    // atom (L%32)/16, slice (L%16) + 16*(2*half + L/32).  Its scale is byte
    // (k-step % 4) of the dword at the same slice of the scale atom.
    const int lrow = lane & 31, lhi = lane >> 5;
    Lds l;
    l.frag_off = ((lrow >> 4) * 1024) + ((lrow & 15) + 16 * lhi) * 16;
    l.sc_off = ((lrow >> 4) * 256) + ((lrow & 15) + 16 * lhi) * 4;
    l.a_atom0 = wm * kTA;
    l.b_atom0 = kGA + wn * kTB;

    if (SPLIT && group == 1) run_k<1>(c, acc, l, kg0);
    else run_k<0>(c, acc, l, kg0);

    if constexpr (SPLIT) {
        // every wave is past its last stage read; group 1's stages take its partial tile
        __syncthreads();
        if (group == 1) {
#pragma unroll
            for (int i = 0; i < kMB; ++i)
#pragma unroll
                for (int j = 0; j < kMA; ++j) {
                    float *p = partial_slot(wave, i * kMA + j) + lane;
#pragma unroll
                    for (int e = 0; e < 16; ++e) p[e * 64] = acc[i][j][e];
                }
        }
        __syncthreads();
        if (group == 0) {
#pragma unroll
            for (int i = 0; i < kMB; ++i)
#pragma unroll
                for (int j = 0; j < kMA; ++j) {
                    const float *p = partial_slot(wave, i * kMA + j) + lane;
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[i][j][e] += p[e * 64];
                }
        }
    }

    // ---- epilogue
    if constexpr (BIAS) {
        if (group == 0) {
#pragma unroll
            for (int i = 0; i < kMB; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const v2u bb = bias_bits[i * 4 + q];
                    const float b0 = __uint_as_float(bb[0] << 16), b1 = __uint_as_float(bb[0] & 0xFFFF0000u);
                    const float b2 = __uint_as_float(bb[1] << 16), b3 = __uint_as_float(bb[1] & 0xFFFF0000u);
#pragma unroll
                    for (int j = 0; j < kMA; ++j) {
                        acc[i][j][4 * q] += b0;
                        acc[i][j][4 * q + 1] += b1;
                        acc[i][j][4 * q + 2] += b2;
                        acc[i][j][4 * q + 3] += b3;
                    }
                }
        }
    }
    store_tile<OUT_BF16, NG>(acc, tm, tn, M, N, C, ldc, group, wave, wave_all, lane);
}

}  // namespace

hipError_t launch_gemm_tail(int64_t M, int64_t N, int64_t K_pad, int tiles_m, int tiles_n, int first, int count,
                            const uint8_t *A, const uint8_t *As, const uint8_t *B, const uint8_t *Bs,
                            const uint16_t *bias, mx_dtype out_dtype, void *C, int64_t ldc, hipStream_t stream) {
    // at most one 128x128 tile per CU (and K long enough to halve): the split form
    const int cus = device_cu_count();
    const bool split = cus > 0 && 4 * count <= cus && K_pad >= 8 * 128;
    const bool bf = out_dtype == MX_BF16;
    auto kernel = split ? (bf ? (bias ? gemm_a4w4_tail_kernel<true, true, true> : gemm_a4w4_tail_kernel<true, false, true>)
                              : (bias ? gemm_a4w4_tail_kernel<false, true, true> : gemm_a4w4_tail_kernel<false, false, true>))
                        : (bf ? (bias ? gemm_a4w4_tail_kernel<true, true, false> : gemm_a4w4_tail_kernel<true, false, false>)
                              : (bias ? gemm_a4w4_tail_kernel<false, true, false> : gemm_a4w4_tail_kernel<false, false, false>));
    hipLaunchKernelGGL(kernel, dim3((unsigned)(4 * count)), dim3(split ? 2 * kThreads : kThreads), 0, stream, M, N,
                       K_pad, tiles_m, tiles_n, first, A, As, B, Bs, bias, C, ldc);
    return hipGetLastError();
}

}  // namespace mx
