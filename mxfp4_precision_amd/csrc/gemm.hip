// Block-scaled FP4 x FP4 GEMM (C = A . B^T) for gfx950 on tiled-layout blobs.
//
// C[i][j] = sum_k e2m1(A[i][k]) 2^(sa[i][k/32]-127) * e2m1(B[j][k]) 2^(sb[j][k/32]-127),
// fp32 accumulation, bf16 (RNE) or fp32 output: the NT product that the
// forward, dgrad and wgrad of the MXFP4 linear on the page
// "primus_turbo_mxfp4_local.py" compute.
//
// MFMA: V_MFMA_SCALE_F32_32X32X64_F8F6F4 with both formats FP4.  Lane L of a
// 32-row operand tile supplies 16 bytes (32 elements) of row L%32, k-block
// 2*half + L/32 of a 128-wide k-step, and that block's E8M0 scale as the byte
// of a VGPR that OPSEL picks.  The tiled layout puts exactly those 16 bytes at
// a fixed slice of a 1 KB atom (16 rows x 128 k) and a lane's scales for 4
// consecutive k-steps in one dword of a 256-byte scale atom, so operands move
// as whole atoms and are read from LDS with conflict-free ds_read_b128.
//
// Workgroup: 8 waves (two per SIMD), 256x256 tile of C; wave w owns the
// 128x64 block at rows 128*(w%2), columns 64*(w/2): 4x2 MFMA tiles, 128 fp32
// accumulators per lane, under 256 registers so two waves share each SIMD.
// Every LDS read or DMA instruction a wave issues stalls that wave's MFMA
// stream for tens of cycles; with two waves per SIMD the other wave's MFMAs
// fill that gap.
//
// Pipeline: LDS holds 4 k-step stages of 32 atoms (16 A + 16 B, 32 KB) and one
// k-group (4 steps) of scale atoms.  Atoms travel global -> LDS by DMA
// (buffer_load ... lds, no registers); step k+3 is in flight while step k
// computes.  Each k-step is two halves of 8 MFMAs per wave; one slot = one
// MFMA plus, in fixed order, the LDS read of an operand of the next half and
// the DMA instructions assigned to that slot, so memory instructions are
// spread evenly between MFMAs.  Half 0 of step k issues the second part of
// step k+2's DMA, half 1 the first part of step k+3's; the barrier between
// the halves publishes step k+1 and frees the stage of step k-1.
//
// The MFMA is issued with B as the "A" operand, so each lane's accumulators
// are 4 consecutive columns of one row of C.  Workgroups are ordered so that
// each XCD (8 on MI355X, dispatched round-robin) works on a compact band of
// output tiles, keeping the A rows and B columns it shares within its own L2.
//
// With a short K and several rounds of tiles, a persistent form runs one
// workgroup per CU over its tiles as one stream of k-steps: the next tile's
// first steps are fetched during the current tile's last ones, and the
// epilogue's stores drain while the next tile computes instead of holding
// the CU (at 24 k-steps per tile the bf16 stores alone cost ~10% otherwise).

#include <atomic>
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
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = 256, kBN = 256;        // workgroup tile
constexpr int kWM = 128, kWN = 64;         // wave tile
constexpr int kWavesM = kBM / kWM;         // wave grid 2 x 4
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
constexpr int kXcds = 8;
constexpr int kGroupM = 8;                 // tile rows per band in the tile order

static_assert(kAtoms % kWaves == 0 && kLoads % 2 == 0, "DMA split");
// 16-byte stores per wave per tile in the stream kernel's epilogue: kMA
// passes of the wave's own 32 rows x kWN bf16 columns, 64 lanes x 16 bytes
// per store instruction
constexpr int kEpiStoresPerTile = kMA * (32 * kWN * 2) / (64 * 16);
static_assert(kMA + kMB <= kSlots, "one operand read per slot");

// Buffer resource over [p, p + bytes).  Loads address it with a per-lane
// byte offset; an offset at or past `bytes` reads zeros (the hardware range
// check of raw buffers), which is how k-steps past K_pad become zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// LDS: 4 k-step stages of 32 atoms and one k-group of scale atoms, as
// separate arrays so that the compiler can tell a DMA into one stage from a
// read of another.  After the k-loop the stages hold the bf16 C tile: rows
// [64s, 64s + 64) in stage s, 512 bytes per row, 16-byte chunk c of row r at
// chunk c ^ (r % 32) so that reads and writes of a column of rows spread
// over all banks.
constexpr int kStageBytes = kAtoms * 1024;
static_assert(kBN * 2 * (kBM / 4) == kStageBytes, "a quarter of the bf16 C tile fills one stage");
__shared__ __attribute__((aligned(1024))) uint8_t g_stage0[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage1[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage2[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_stage3[kStageBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_scale[kAtoms * 256];

template <int S>
__device__ __forceinline__ uint8_t *stage_buf() {
    return S == 0 ? g_stage0 : S == 1 ? g_stage1 : S == 2 ? g_stage2 : g_stage3;
}
__device__ __forceinline__ uint8_t *scale_buf() { return g_scale; }
__device__ __forceinline__ uint8_t *stage_dyn(int s) {
    return s == 0 ? g_stage0 : s == 1 ? g_stage1 : s == 2 ? g_stage2 : g_stage3;
}
// byte address of bf16 C element (r, col) of the staged tile, col % 4 == 0
__device__ __forceinline__ uint8_t *c_stage(int r, int col) {
    const int chunk = (col >> 3) ^ (r & 31);
    return stage_dyn(r >> 6) + (r & 63) * (kBN * 2) + chunk * 16 + (col & 7) * 2;
}

#define MX_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// Offset that lies past every operand buffer: a buffer load there returns 0.
constexpr uint32_t kOutOfRange = 0x80000000u;
// buffer-store cache policy: non-temporal (C is not read again by the kernel)
constexpr int kCachePolicyNT = 2;
// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their
// maxima (no wait): vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
constexpr int kWaitVmcnt0 = 0x0F70;

// STREAM: the workgroup runs several output tiles back to back as one stream
// of k-steps; a tile occupies kstream = 4 * kgroups steps of it, and a DMA
// for step kstream + j (j < 3) fetches step j of the next tile (ld_next /
// sc_next; knext = its k-steps, 0 when there is none).
template <bool STREAM>
struct GemmCtxT {
    static constexpr bool kStream = STREAM;
    // k-step counter type: the stream kernel keeps k-steps in 32 bits (operand
    // blobs stay below 2 GiB, so K_pad / 128 < 2^24) to spare scalar registers
    using kint = typename std::conditional<STREAM, int, int64_t>::type;
    __amdgpu_buffer_rsrc_t rA, rB, rAs, rBs;
    int ld_row[kLoads];    // byte offset of this wave's r-th atom row (k-step 0)
    int sc_row[kLoads];    // byte offset of this wave's r-th scale-atom row (k-group 0)
    kint ksteps, kgroups;
    int wave, lane16, lane4;
    int ld_next[STREAM ? kLoads : 1], sc_next[STREAM ? kLoads : 1];
    kint kstream, knext;
};
using GemmCtx = GemmCtxT<false>;

struct Regs {
    uint4 a0[kMA], b0[kMB], a1[kMA], b1[kMB];       // operands of half 0 / half 1
    uint32_t sa[kMA][2], sb[kMB][2];                // scales of the current k-group
    uint32_t sa_n[kMA][2], sb_n[kMB][2];            // ... of the next one
};

// DMA instruction V of k-step k into stage S = k % 4: V < kLoads copies data
// atom kWaves*V + wave; V >= kLoads (only when k opens a k-group) copies scale
// atom kWaves*(V - kLoads) + wave.  Past K_pad the offset is out of range and
// the atom lands as zeros.  INNER: the caller guarantees k < ksteps (a step
// of the current tile inside K_pad), so the offset is the row's plus k's
// with no test: a wave issues its instructions in order, and the tests and
// selects in front of every DMA otherwise hold back its next MFMA.
template <int S, int V, bool INNER = false, class Ctx>
__device__ __forceinline__ void dma_op(const Ctx &c, typename Ctx::kint k) {
    using kint = typename Ctx::kint;
    if constexpr (V < kLoads) {
        // atom kWaves*V + wave: an A atom for every wave or a B atom for every wave
        constexpr bool isA = kWaves * (V + 1) <= kGA;
        static_assert(isA || kWaves * V >= kGA, "A/B split falls on a DMA instruction");
        const int a = kWaves * V + c.wave;
        uint32_t base;
        if constexpr (INNER) {
            base = (uint32_t)c.ld_row[V] + (uint32_t)(k * 1024);
        } else if constexpr (Ctx::kStream) {
            // steps of the tile, then the next tile's first steps
            const bool cur = k < c.kstream;
            const kint kk = cur ? k : k - c.kstream;
            const int row = cur ? c.ld_row[V] : c.ld_next[V];
            base = kk < (cur ? c.ksteps : c.knext) ? (uint32_t)row + (uint32_t)(kk * 1024) : kOutOfRange;
        } else {
            base = k < c.ksteps ? (uint32_t)c.ld_row[V] + (uint32_t)(k * 1024) : kOutOfRange;
        }
        // (plain-typed locals: a builtin call on template-dependent operands
        // does not resolve in the host compilation pass)
        const __amdgpu_buffer_rsrc_t rsrc = isA ? c.rA : c.rB;
        const uint32_t off = base + (uint32_t)c.lane16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, MX_LDS(stage_buf<S>() + a * 1024), 16, off, 0, 0, 0);
    } else {
        constexpr int R = V - kLoads;
        constexpr bool isA = kWaves * (R + 1) <= kGA;
        static_assert(isA || kWaves * R >= kGA, "A/B split falls on a DMA instruction");
        const int a = kWaves * R + c.wave;
        const kint h = k / 4;
        uint32_t base;
        if constexpr (INNER) {
            base = (uint32_t)c.sc_row[R] + (uint32_t)(h * 256);
        } else {
            base = h < c.kgroups ? (uint32_t)c.sc_row[R] + (uint32_t)(h * 256) : kOutOfRange;
            // only step kstream (the next tile's first) opens a k-group past the tile
            if constexpr (Ctx::kStream)
                if (k >= c.kstream) base = c.knext > 0 ? (uint32_t)c.sc_next[R] : kOutOfRange;
        }
        const __amdgpu_buffer_rsrc_t rsrc = isA ? c.rAs : c.rBs;
        const uint32_t off = base + (uint32_t)c.lane4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, MX_LDS(scale_buf() + a * 256), 4, off, 0, 0, 0);
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

template <int S, int P, int n = 0, class Ctx>
__device__ __forceinline__ void dma_part(const Ctx &c, typename Ctx::kint k) {
    if constexpr (n < part_ops(S)) {
        dma_op<S, part_op(S, P, n)>(c, k);
        dma_part<S, P, n + 1>(c, k);
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
//    half 1: part 0 of step k+3); INNER: both steps lie inside the tile's K.
template <int S, int H, int T, bool FRESH, bool INNER, class Ctx>
__device__ __forceinline__ void slot(const Ctx &c, typename Ctx::kint k, v16f (&acc)[kMB][kMA], Regs &r,
                                     const Lds &l) {
    constexpr int i = T / kMA, j = T % kMA;
    if constexpr (H == 0) mfma_tile<S>(acc[i][j], r.b0[i], r.a0[j], r.sb[i][0], r.sa[j][0]);
    else mfma_tile<S>(acc[i][j], r.b1[i], r.a1[j], r.sb[i][1], r.sa[j][1]);

    if constexpr (T < kMA + kMB) {
        constexpr int RS = H == 0 ? S : ((S + 1) & 3);
        constexpr int RH = H == 0 ? 1 : 0;
        const uint8_t *st = stage_buf<RS>() + l.frag_off + RH * 512;
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
                r.sa_n[t][hh] = *reinterpret_cast<const uint32_t *>(scale_buf() + (l.a_atom0 + 2 * t) * 256 + l.sc_off + hh * 128);
            else
                r.sb_n[t - kMA][hh] =
                    *reinterpret_cast<const uint32_t *>(scale_buf() + (l.b_atom0 + 2 * (t - kMA)) * 256 + l.sc_off + hh * 128);
        }
    }

    constexpr int DS = H == 0 ? ((S + 2) & 3) : ((S + 3) & 3);
    constexpr int P = H == 0 ? 1 : 0;
    // FRESH (a tile's first k-step in the stream kernel): the second part of
    // step 2 already went out before the previous tile's stores
    constexpr int nv = (FRESH && S == 0 && H == 0) ? 0 : part_ops(DS);
    const typename Ctx::kint dk = H == 0 ? k + 2 : k + 3;
    if constexpr (nv > 0 && dma_slot(0, nv) == T) dma_op<DS, part_op(DS, P, 0), INNER>(c, dk);
    if constexpr (nv > 1 && dma_slot(1, nv) == T) dma_op<DS, part_op(DS, P, 1), INNER>(c, dk);
    if constexpr (nv > 2 && dma_slot(2, nv) == T) dma_op<DS, part_op(DS, P, 2), INNER>(c, dk);
    if constexpr (nv > 3 && dma_slot(3, nv) == T) dma_op<DS, part_op(DS, P, 3), INNER>(c, dk);
    static_assert(part_ops(0) <= 4, "dma slots");
    // keep this slot's instructions in this slot
    __builtin_amdgcn_sched_barrier(0);
}

template <int S, int H, int T = 0, bool FRESH = false, bool INNER = false, class Ctx>
__device__ __forceinline__ void half_step(const Ctx &c, typename Ctx::kint k, v16f (&acc)[kMB][kMA], Regs &r,
                                          const Lds &l) {
    if constexpr (T < kSlots) {
        slot<S, H, T, FRESH, INNER>(c, k, acc, r, l);
        half_step<S, H, T + 1, FRESH, INNER>(c, k, acc, r, l);
    }
}

// One 128-wide k-step.  The barrier waits for this wave's DMA of step k+1
// (only step k+2's instructions may still be outstanding) and then for every
// wave, which publishes step k+1 and certifies that all reads of step k-1's
// stage are done before half 1 starts overwriting it.  Vector memory
// instructions complete in issue order (loads and stores alike), so the
// count is exact.  FRESH: the first k-group of a tile in the stream kernel,
// where EXTRA vector-memory instructions (the previous tile's stores and
// this tile's bias loads) were issued after all of step 2's DMA; the first
// two waits count past them instead of draining them.  INNER: steps k+2 and
// k+3 are both below ksteps (see dma_op).
template <int S, bool FRESH = false, int EXTRA = 0, bool INNER = false, class Ctx>
__device__ __forceinline__ void k_step(const Ctx &c, typename Ctx::kint k, v16f (&acc)[kMB][kMA], Regs &r,
                                       const Lds &l) {
    constexpr int kStores = FRESH && S < 2 ? EXTRA : 0;
    __builtin_amdgcn_sched_barrier(0);
    half_step<S, 0, 0, FRESH, INNER>(c, k, acc, r, l);
    static_assert(issued_for((S + 2) & 3) + kStores <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(issued_for((S + 2) & 3) + kStores) : "memory");
    __builtin_amdgcn_sched_barrier(0);
    half_step<S, 1, 0, FRESH, INNER>(c, k, acc, r, l);
    if constexpr (S == 3) {
#pragma unroll
        for (int t = 0; t < kMA; ++t) { r.sa[t][0] = r.sa_n[t][0]; r.sa[t][1] = r.sa_n[t][1]; }
#pragma unroll
        for (int t = 0; t < kMB; ++t) { r.sb[t][0] = r.sb_n[t][0]; r.sb[t][1] = r.sb_n[t][1]; }
    }
}

// Epilogue: write the 256x256 tile (tm, tn) of C from the accumulators;
// acc[i][j][r] = C[m0 + 32j + lane%32][n0 + 32i + 8(r/4) + 4(lane/32) + r%4].
// bf16: rounded (V_CVT_PK_BF16_F32, nearest even), staged in LDS, then
// written as whole 512-byte row segments (each store instruction covers 2
// rows with 16 bytes per lane; non-temporal, as C is not read again here);
// fp32: 16 bytes per lane straight from registers.  Masked at the M/N edges.
template <bool OUT_BF16>
__device__ __forceinline__ void store_tile(v16f (&acc)[kMB][kMA], int tm, int tn, int64_t M, int64_t N, void *C,
                                           int64_t ldc, int wave, int lane) {
    const int wm = wave % kWavesM, wn = wave / kWavesM;
    const int lrow = lane & 31, lhi = lane >> 5;
    const int64_t tm0 = (int64_t)tm * kBM, tn0 = (int64_t)tn * kBN;
    if (OUT_BF16) {
        // Every wave waited for its own DMAs; the barrier makes sure all of
        // them have landed and every stage read is done before the tile
        // overwrites the stages.
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
        constexpr int kRowsPerWave = kBM / kWaves;        // 32: 16 instructions of 2 rows
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

// Tile of block index b in a launch of nb blocks: XCD-contiguous ranges of
// the tile order (blocks are dispatched to the XCDs round-robin), the order
// walking bands of kGroupM tile rows column by column.
__device__ __forceinline__ void tile_of(int b, int nb, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int xcd = b % kXcds, local = b / kXcds;
    const int per = nb / kXcds, rem = nb % kXcds;
    const int id = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int band = kGroupM * tiles_n;
    const int first_m = (id / band) * kGroupM;
    const int gsz = min(tiles_m - first_m, kGroupM);
    tm = first_m + (id % band) % gsz;
    tn = (id % band) / gsz;
}

// Byte offsets of this wave's atom rows and scale-atom rows for tile (tm, tn).
// Row groups past an operand are clamped to its last group: those rows of C
// are never stored, so their contents do not matter.
template <class Ctx>
__device__ __forceinline__ void tile_rows(const Ctx &c, int tm, int tn, int64_t nGA, int64_t nGB, int (&ld)[kLoads],
                                          int (&sc)[kLoads]) {
    const int64_t gA0 = (int64_t)tm * kGA, gB0 = (int64_t)tn * kGB;
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
        const int a = kWaves * r + c.wave;
        const bool isA = a < kGA;
        int64_t g = isA ? gA0 + a : gB0 + (a - kGA);
        const int64_t gmax = (isA ? nGA : nGB) - 1;
        g = g < gmax ? g : gmax;
        ld[r] = (int)(g * c.ksteps * 1024);
        sc[r] = (int)(g * c.kgroups * 256);
    }
}

// BIAS: C[i][j] = (sum) + bias[j], bias a bf16 vector of N, added in fp32
// before the output rounding.
template <bool OUT_BF16, bool BIAS>
__global__ __launch_bounds__(kThreads) void gemm_a4w4_kernel(int64_t M, int64_t N, int64_t K_pad, int tiles_m,
                                                             int tiles_n, const uint8_t *__restrict__ A,
                                                             const uint8_t *__restrict__ As,
                                                             const uint8_t *__restrict__ B,
                                                             const uint8_t *__restrict__ Bs,
                                                             const uint16_t *__restrict__ bias,
                                                             void *__restrict__ C, int64_t ldc) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int wm = wave % kWavesM, wn = wave / kWavesM;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);

    GemmCtx c;
    c.ksteps = K_pad / 128;
    c.kgroups = cdiv(K_pad, 512);
    c.wave = wave;
    c.lane16 = lane * 16;
    c.lane4 = lane * 4;
    const int64_t nGA = cdiv(M, 16), nGB = cdiv(N, 16);   // row groups present in memory
    c.rA = make_rsrc(A, nGA * c.ksteps * 1024);
    c.rB = make_rsrc(B, nGB * c.ksteps * 1024);
    c.rAs = make_rsrc(As, nGA * c.kgroups * 256);
    c.rBs = make_rsrc(Bs, nGB * c.kgroups * 256);

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
    tile_rows(c, tm, tn, nGA, nGB, c.ld_row, c.sc_row);

    v16f acc[kMB][kMA];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kMA; ++j) acc[i][j] = v16f{};

    // Prologue: steps 0 and 1 whole, the first part of step 2 (its second
    // part goes out in step 0's first half).
    dma_part<0, 0>(c, 0);
    dma_part<0, 1>(c, 0);
    dma_part<1, 0>(c, 1);
    dma_part<1, 1>(c, 1);
    dma_part<2, 0>(c, 2);

    // Lane L of a 32-row operand tile takes row L%32, k-block 2*half + L/32:
    // atom (L%32)/16, slice (L%16) + 16*(2*half + L/32).  Its scale is byte
    // (k-step % 4) of the dword at the same slice of the scale atom.
    const int lrow = lane & 31, lhi = lane >> 5;
    Lds l;
    l.frag_off = ((lrow >> 4) * 1024) + ((lrow & 15) + 16 * lhi) * 16;
    l.sc_off = ((lrow >> 4) * 256) + ((lrow & 15) + 16 * lhi) * 4;
    l.a_atom0 = wm * kTA;
    l.b_atom0 = kGA + wn * kTB;

    Regs r;
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(issued_for(1) + part_ops(2)) : "memory");
#pragma unroll
    for (int t = 0; t < kMA; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            r.sa[t][hh] = *reinterpret_cast<const uint32_t *>(scale_buf() + (l.a_atom0 + 2 * t) * 256 + l.sc_off + hh * 128);
#pragma unroll
    for (int t = 0; t < kMB; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            r.sb[t][hh] = *reinterpret_cast<const uint32_t *>(scale_buf() + (l.b_atom0 + 2 * t) * 256 + l.sc_off + hh * 128);
#pragma unroll
    for (int t = 0; t < kMA; ++t)
        r.a0[t] = *reinterpret_cast<const uint4 *>(stage_buf<0>() + (l.a_atom0 + 2 * t) * 1024 + l.frag_off);
#pragma unroll
    for (int t = 0; t < kMB; ++t)
        r.b0[t] = *reinterpret_cast<const uint4 *>(stage_buf<0>() + (l.b_atom0 + 2 * t) * 1024 + l.frag_off);

    // k-group h fetches steps 4h+2 .. 4h+6: inside K while 4h+6 < ksteps
    int64_t h = 0;
    for (; 4 * h + 6 < c.ksteps; ++h) {
        const int64_t k0 = 4 * h;
        k_step<0, false, 0, true>(c, k0, acc, r, l);
        k_step<1, false, 0, true>(c, k0 + 1, acc, r, l);
        k_step<2, false, 0, true>(c, k0 + 2, acc, r, l);
        k_step<3, false, 0, true>(c, k0 + 3, acc, r, l);
    }
    for (; h < c.kgroups; ++h) {
        const int64_t k0 = 4 * h;
        k_step<0>(c, k0, acc, r, l);
        k_step<1>(c, k0 + 1, acc, r, l);
        k_step<2>(c, k0 + 2, acc, r, l);
        k_step<3>(c, k0 + 3, acc, r, l);
    }
    // drain the trailing (out-of-range) DMAs before LDS is reused
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---- epilogue
    if constexpr (BIAS) {
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
    store_tile<OUT_BF16>(acc, tm, tn, M, N, C, ldc, wave, lane);
}

// Epilogue of the stream kernel (bf16 output).  Stages 0-2 already hold the
// next tile's first k-steps, so only stage 3 is free.  Each wave takes a
// 4 KB slot of it: in pass p (kMA passes) the wave stages its own 32 x 64
// block (MFMA row tile p: tile rows 128 wm + 32p + [0, 32), columns
// 64 wn + [0, 64)), 128 bytes per row with 16-byte chunk c of row r at c ^
// (r % 8), and reads it back as whole 128-byte row segments, 8 rows per store
// instruction.  After the first barrier (every wave done with stage 3's last
// k-step) no wave waits for another: a wave's LDS operations complete in
// order, so its next pass may overwrite the slot it has just read.  Each wave
// issues exactly kEpiStoresPerTile 16-byte buffer stores per tile whatever
// the edges: a chunk past row M or column N gets an out-of-range offset, which
// the buffer range check drops (N % 8 == 0, so a chunk is all in or all out).
// The fixed count is what lets the next tile's first waits count past the
// stores instead of draining them.  Before the stores, the epilogue issues
// the second part of the next tile's step 2 (its first k-step would otherwise
// issue it after them), into stage 2, free since the tile's last k-step.
constexpr int kSlotBytes = 32 * kWN * 2;                  // 4 KB per wave
static_assert(kSlotBytes * kWaves == kStageBytes, "one slot per wave fills stage 3");
static_assert(kEpiStoresPerTile == kMA * 4, "store count: 4 instructions of 8 rows per pass");

__device__ __forceinline__ uint8_t *c_slot(int wave, int r, int chunk) {
    return g_stage3 + wave * kSlotBytes + r * (kWN * 2) + ((chunk ^ (r & 7)) * 16);
}

__device__ __forceinline__ void store_tile_stream(const GemmCtxT<true> &c, v16f (&acc)[kMB][kMA], int tm, int tn,
                                                  int M, int N, __amdgpu_buffer_rsrc_t rC, int ldc, int wave,
                                                  int lane) {
    dma_part<2, 1>(c, c.kstream + 2);
    const int wm = wave % kWavesM, wn = wave / kWavesM;
    const int lrow = lane & 31, lhi = lane >> 5;
    const int row_w = tm * kBM + kWM * wm;                     // first C row of this wave's block
    const int col = tn * kBN + kWN * wn + 8 * (lane & 7);      // this lane's 8 columns on the way out
    // every wave is done reading stage 3 (the tile's last k-step); a bare
    // barrier: a __syncthreads() fence would also wait for the next tile's DMAs
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int p = 0; p < kMA; ++p) {
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t p01 = __builtin_bit_cast(
                    uint32_t, __builtin_convertvector((f32x2_t{acc[i][p][4 * q], acc[i][p][4 * q + 1]}), bf16x2_t));
                const uint32_t p23 = __builtin_bit_cast(
                    uint32_t, __builtin_convertvector((f32x2_t{acc[i][p][4 * q + 2], acc[i][p][4 * q + 3]}), bf16x2_t));
                *reinterpret_cast<uint2 *>(c_slot(wave, lrow, 4 * i + q) + 8 * lhi) = uint2{p01, p23};
            }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int r = 8 * s + (lane >> 3);
            const v4u_t v = *reinterpret_cast<const v4u_t *>(c_slot(wave, r, lane & 7));
            const int row = row_w + 32 * p + r;
            const uint32_t off = row < M && col < N ? (uint32_t)(row * ldc + col) * 2u : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(v, rC, off, 0, kCachePolicyNT);
        }
    }
}

typedef uint32_t v2u_t __attribute__((ext_vector_type(2)));

// This lane's bias values for tile column tn: columns n0 + 32i + 8q +
// 4(lane/32) + 0..3 of the tile, 4 bf16 per (i, q), one 8-byte buffer load
// each (the range ends at the 16-byte boundary after the last entry; the
// bias is 16-byte aligned, so that block is inside its allocation; columns
// past it read 0 and are never stored).
__device__ __forceinline__ void load_bias(__amdgpu_buffer_rsrc_t rb, int tn, int wn, int lane,
                                          v2u_t (&bias_bits)[kMB * 4]) {
    const int col0 = tn * kBN + wn * kWN + 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            bias_bits[i * 4 + q] = __builtin_amdgcn_raw_buffer_load_b64(rb, (col0 + 32 * i + 8 * q) * 2, 0, 0);
}

__device__ __forceinline__ void add_bias(v16f (&acc)[kMB][kMA], const v2u_t (&bias_bits)[kMB * 4]) {
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const v2u_t bb = bias_bits[i * 4 + q];
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

// Persistent form of gemm_a4w4_kernel for bf16 output:
// gridDim.x workgroups, block b runs tiles b, b + gridDim.x, ... of the first
// `tiles` of the tile order as one stream of k-steps.  A tile's last k-steps
// already fetch the next tile's first three and its first operands and
// scales, so the pipeline never drains between tiles; the epilogue's stores
// then overlap the next tile's first k-steps (its first two waits count past
// them, only the third one needs them done).  The k-loop is the one-tile
// kernel's, DMA schedule included.  BIAS: a tile's bias values are loaded
// right after the previous tile's stores (8 more instructions for those
// waits to count past).  Needs N % 8 == 0 and M * ldc * 2 < 2^31 (32-bit
// store offsets).
template <bool BIAS>
__global__ __launch_bounds__(kThreads) void gemm_a4w4_stream_kernel(int M, int N, int K_pad, int tiles_m, int tiles_n,
                                                                    int tiles, const uint8_t *__restrict__ A,
                                                                    const uint8_t *__restrict__ As,
                                                                    const uint8_t *__restrict__ B,
                                                                    const uint8_t *__restrict__ Bs,
                                                                    const uint16_t *__restrict__ bias,
                                                                    void *__restrict__ C, int ldc) {
    constexpr int kBiasLoads = BIAS ? kMB * 4 : 0;
    constexpr int kFreshOps = kEpiStoresPerTile + kBiasLoads;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % kWavesM, wn = wave / kWavesM;
    const int P = gridDim.x;

    GemmCtxT<true> c;
    c.ksteps = K_pad / 128;
    c.kgroups = (K_pad + 511) / 512;
    c.kstream = 4 * c.kgroups;
    c.wave = wave;
    c.lane16 = lane * 16;
    c.lane4 = lane * 4;
    const int nGA = (M + 15) / 16, nGB = (N + 15) / 16;
    c.rA = make_rsrc(A, (int64_t)nGA * c.ksteps * 1024);
    c.rB = make_rsrc(B, (int64_t)nGB * c.ksteps * 1024);
    c.rAs = make_rsrc(As, (int64_t)nGA * c.kgroups * 256);
    c.rBs = make_rsrc(Bs, (int64_t)nGB * c.kgroups * 256);
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(C, (int64_t)M * ldc * 2);
    const __amdgpu_buffer_rsrc_t rBias = make_rsrc(bias, BIAS ? ((int64_t)N * 2 + 15) / 16 * 16 : 0);

    int vb = blockIdx.x;
    int tm, tn, tm_next = 0, tn_next = 0;
    tile_of(vb, tiles, tiles_m, tiles_n, tm, tn);
    tile_rows(c, tm, tn, nGA, nGB, c.ld_row, c.sc_row);
    c.knext = 0;
    if (vb + P < tiles) {
        tile_of(vb + P, tiles, tiles_m, tiles_n, tm_next, tn_next);
        tile_rows(c, tm_next, tn_next, nGA, nGB, c.ld_next, c.sc_next);
        c.knext = c.ksteps;
    }

    v16f acc[kMB][kMA];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kMA; ++j) acc[i][j] = v16f{};
    v2u_t bias_bits[BIAS ? kMB * 4 : 1];
    if constexpr (BIAS) load_bias(rBias, tn, wn, lane, bias_bits);

    // Prologue: steps 0-2 whole (a tile's first k-step does not issue step
    // 2's second part), all landed before the first k-step, so the first
    // tile's first two waits (which count past stores that this tile does not
    // have) wait for nothing.
    dma_part<0, 0>(c, 0);
    dma_part<0, 1>(c, 0);
    dma_part<1, 0>(c, 1);
    dma_part<1, 1>(c, 1);
    dma_part<2, 0>(c, 2);
    dma_part<2, 1>(c, 2);

    const int lrow = lane & 31, lhi = lane >> 5;
    Lds l;
    l.frag_off = ((lrow >> 4) * 1024) + ((lrow & 15) + 16 * lhi) * 16;
    l.sc_off = ((lrow >> 4) * 256) + ((lrow & 15) + 16 * lhi) * 4;
    l.a_atom0 = wm * kTA;
    l.b_atom0 = kGA + wn * kTB;

    Regs r;
    // vmcnt(0) as a builtin (not asm), so that the compiler's own wait
    // tracking also knows that nothing is outstanding past this point
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int t = 0; t < kMA; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            r.sa[t][hh] = *reinterpret_cast<const uint32_t *>(scale_buf() + (l.a_atom0 + 2 * t) * 256 + l.sc_off + hh * 128);
#pragma unroll
    for (int t = 0; t < kMB; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            r.sb[t][hh] = *reinterpret_cast<const uint32_t *>(scale_buf() + (l.b_atom0 + 2 * t) * 256 + l.sc_off + hh * 128);
#pragma unroll
    for (int t = 0; t < kMA; ++t)
        r.a0[t] = *reinterpret_cast<const uint4 *>(stage_buf<0>() + (l.a_atom0 + 2 * t) * 1024 + l.frag_off);
#pragma unroll
    for (int t = 0; t < kMB; ++t)
        r.b0[t] = *reinterpret_cast<const uint4 *>(stage_buf<0>() + (l.b_atom0 + 2 * t) * 1024 + l.frag_off);

    for (;;) {
        // first k-group: its first two waits count past the previous tile's
        // stores and this tile's bias loads
        k_step<0, true, kFreshOps>(c, 0, acc, r, l);
        k_step<1, true, kFreshOps>(c, 1, acc, r, l);
        k_step<2>(c, 2, acc, r, l);
        k_step<3>(c, 3, acc, r, l);
        // k-group h fetches steps 4h+2 .. 4h+6: all of this tile while
        // 4h+6 < ksteps; the last group (or two) also fetch the next tile's
        int h = 1;
        for (; 4 * h + 6 < c.ksteps; ++h) {
            const int k0 = 4 * h;
            k_step<0, false, 0, true>(c, k0, acc, r, l);
            k_step<1, false, 0, true>(c, k0 + 1, acc, r, l);
            k_step<2, false, 0, true>(c, k0 + 2, acc, r, l);
            k_step<3, false, 0, true>(c, k0 + 3, acc, r, l);
        }
        for (; h < c.kgroups; ++h) {
            const int k0 = 4 * h;
            k_step<0>(c, k0, acc, r, l);
            k_step<1>(c, k0 + 1, acc, r, l);
            k_step<2>(c, k0 + 2, acc, r, l);
            k_step<3>(c, k0 + 3, acc, r, l);
        }
        // r now holds the next tile's first operands and scales
        if constexpr (BIAS) add_bias(acc, bias_bits);
        store_tile_stream(c, acc, tm, tn, M, N, rC, ldc, wave, lane);
        if constexpr (BIAS) {
            // The next tile's bias, after the stores in issue order as the
            // first waits assume.  (The compiler moves these loads past the
            // exit test below; its own wait before the first read of the
            // next tile then merges the paths with and without them and
            // comes out at 20-21 instead of 28, draining a few of the oldest
            // stores: correct, slightly conservative.)
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            load_bias(rBias, tn_next, wn, lane, bias_bits);
            __builtin_amdgcn_sched_barrier(0);
        }
        vb += P;
        if (vb >= tiles) break;
        tm = tm_next;
        tn = tn_next;
#pragma unroll
        for (int q = 0; q < kLoads; ++q) {
            c.ld_row[q] = c.ld_next[q];
            c.sc_row[q] = c.sc_next[q];
        }
        c.knext = 0;
        if (vb + P < tiles) {
            tile_of(vb + P, tiles, tiles_m, tiles_n, tm_next, tn_next);
            tile_rows(c, tm_next, tn_next, nGA, nGB, c.ld_next, c.sc_next);
            c.knext = c.ksteps;
        }
#pragma unroll
        for (int i = 0; i < kMB; ++i)
#pragma unroll
            for (int j = 0; j < kMA; ++j) acc[i][j] = v16f{};
    }
    // drain the stores and the trailing (out-of-range) DMAs
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ------------------------------------------------------------ FP8 (E5M2)
// The hybrid backward's GEMM: tensorwise E5M2 operands in the FP8 tiled
// layout (16-row groups, 64-element k-steps, 1 KB atoms; lane
// (r%16) + 16*((k%64)/16) owns 16 bytes), C = (A . B^T) * sa_inv * sb_inv.
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 with both formats E5M2 and unit block
// scales (127): lane L of a 32-row operand tile supplies 32 bytes, row L%32,
// elements [32*(L/32), 32*(L/32) + 32) of the 64-wide step = two 16-byte
// slices of the atom, 256 bytes apart.  Same workgroup, wave tiles, XCD
// order and LDS stages as the FP4 kernel; a k-step is 64 elements, its 32
// atoms fill one 32 KB stage, step k+3 is in flight while step k computes.
constexpr int kFmtBf8 = 1;          // MFMA f8f6f4 format code for E5M2
constexpr int kUnitScale = 127;     // E8M0 2^0

template <int S>
__device__ __forceinline__ void fp8_dma_step(const GemmCtx &c, int64_t k) {
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
        const int a = kWaves * r + c.wave;
        const uint32_t base = k < c.ksteps ? (uint32_t)c.ld_row[r] + (uint32_t)(k * 1024) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(a < kGA ? c.rA : c.rB, MX_LDS(stage_buf<S>() + a * 1024), 16,
                                                 base + c.lane16, 0, 0, 0);
    }
}

template <int S>
__device__ __forceinline__ void fp8_step(const GemmCtx &c, int64_t k, v16f (&acc)[kMB][kMA], int frag_off,
                                         int a_atom0, int b_atom0) {
    // step k landed for every wave (only steps k+1, k+2 may still be in flight),
    // and every wave is done reading step k-1's stage
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kLoads) : "memory");
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t *st = stage_buf<S>() + frag_off;
    uint4 b[kMB][2], a[kMA][2];
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
        b[i][0] = *reinterpret_cast<const uint4 *>(st + (b_atom0 + 2 * i) * 1024);
        b[i][1] = *reinterpret_cast<const uint4 *>(st + (b_atom0 + 2 * i) * 1024 + 256);
    }
#pragma unroll
    for (int j = 0; j < kMA; ++j) {
        a[j][0] = *reinterpret_cast<const uint4 *>(st + (a_atom0 + 2 * j) * 1024);
        a[j][1] = *reinterpret_cast<const uint4 *>(st + (a_atom0 + 2 * j) * 1024 + 256);
    }
    fp8_dma_step<(S + 3) & 3>(c, k + 3);
#pragma unroll
    for (int i = 0; i < kMB; ++i) {
        const v8i bop = {(int)b[i][0].x, (int)b[i][0].y, (int)b[i][0].z, (int)b[i][0].w,
                         (int)b[i][1].x, (int)b[i][1].y, (int)b[i][1].z, (int)b[i][1].w};
#pragma unroll
        for (int j = 0; j < kMA; ++j) {
            const v8i aop = {(int)a[j][0].x, (int)a[j][0].y, (int)a[j][0].z, (int)a[j][0].w,
                             (int)a[j][1].x, (int)a[j][1].y, (int)a[j][1].z, (int)a[j][1].w};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bop, aop, acc[i][j], kFmtBf8, kFmtBf8, 0,
                                                                        kUnitScale, 0, kUnitScale);
        }
    }
    // reads first (the MFMAs need them), each DMA after an MFMA
#pragma unroll
    for (int t = 0; t < kLoads; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMA * kMB - kLoads, 0);
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void gemm_fp8_kernel(int64_t M, int64_t N, int64_t K_pad, int tiles_m,
                                                            int tiles_n, const uint8_t *__restrict__ A,
                                                            const float *__restrict__ a_scale_inv,
                                                            const uint8_t *__restrict__ B,
                                                            const float *__restrict__ b_scale_inv,
                                                            void *__restrict__ C, int64_t ldc) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave % kWavesM, wn = wave / kWavesM;
    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);

    GemmCtx c;
    c.ksteps = K_pad / 64;
    c.kgroups = 0;
    c.wave = wave;
    c.lane16 = lane * 16;
    c.lane4 = 0;
    const int64_t nGA = cdiv(M, 16), nGB = cdiv(N, 16);
    c.rA = make_rsrc(A, nGA * c.ksteps * 1024);
    c.rB = make_rsrc(B, nGB * c.ksteps * 1024);
    const int64_t gA0 = (int64_t)tm * kGA, gB0 = (int64_t)tn * kGB;
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
        const int a = kWaves * r + wave;
        const bool isA = a < kGA;
        int64_t g = isA ? gA0 + a : gB0 + (a - kGA);
        const int64_t gmax = (isA ? nGA : nGB) - 1;
        g = g < gmax ? g : gmax;
        c.ld_row[r] = (int)(g * c.ksteps * 1024);
    }
    const float scale = a_scale_inv[0] * b_scale_inv[0];

    v16f acc[kMB][kMA];
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kMA; ++j) acc[i][j] = v16f{};

    fp8_dma_step<0>(c, 0);
    fp8_dma_step<1>(c, 1);
    fp8_dma_step<2>(c, 2);
    const int lrow = lane & 31, lhi = lane >> 5;
    const int frag_off = ((lrow >> 4) * 1024) + ((lrow & 15) + 32 * lhi) * 16;
    const int a_atom0 = wm * kTA, b_atom0 = kGA + wn * kTB;
    for (int64_t k = 0; k < c.ksteps; k += 4) {
        fp8_step<0>(c, k, acc, frag_off, a_atom0, b_atom0);
        fp8_step<1>(c, k + 1, acc, frag_off, a_atom0, b_atom0);
        fp8_step<2>(c, k + 2, acc, frag_off, a_atom0, b_atom0);
        fp8_step<3>(c, k + 3, acc, frag_off, a_atom0, b_atom0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < kMB; ++i)
#pragma unroll
        for (int j = 0; j < kMA; ++j) acc[i][j] *= scale;
    store_tile<OUT_BF16>(acc, tm, tn, M, N, C, ldc, wave, lane);
}

// K == 0: C[i][j] = 0, or bias[j] (bf16 bits; exact in either output type).
template <typename T>
__global__ void fill_kernel(T *C, int64_t M, int64_t N, int64_t ldc, const uint16_t *bias) {
    int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= M * N) return;
    const int64_t j = idx % N;
    const uint16_t b = bias ? bias[j] : (uint16_t)0;
    if constexpr (sizeof(T) == 2) C[(idx / N) * ldc + j] = b;
    else C[(idx / N) * ldc + j] = __uint_as_float((uint32_t)b << 16);
}

}  // namespace

// Compute units of the current device (cached per device; 0 if unknown).
int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0) n = 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t *A, const uint8_t *As,
                       const uint8_t *B, const uint8_t *Bs, const uint16_t *bias, mx_dtype out_dtype, void *C,
                       int64_t ldc, hipStream_t stream) {
    const int64_t K_pad = padded(K);
    if (K_pad == 0) {
        const int64_t n = M * N;
        dim3 grid((unsigned)cdiv(n, 256));
        if (out_dtype == MX_BF16)
            hipLaunchKernelGGL(fill_kernel<uint16_t>, grid, dim3(256), 0, stream, reinterpret_cast<uint16_t *>(C),
                               M, N, ldc, bias);
        else
            hipLaunchKernelGGL(fill_kernel<float>, grid, dim3(256), 0, stream, reinterpret_cast<float *>(C), M, N,
                               ldc, bias);
        return hipGetLastError();
    }
    // buffer offsets are 32-bit: each operand blob (16-row groups of K_pad/2
    // bytes per row) must stay below 2 GiB
    if (cdiv(M, 16) * 16 * (K_pad / 2) >= (int64_t(1) << 31) || cdiv(N, 16) * 16 * (K_pad / 2) >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
    const int tiles_m = (int)cdiv(M, kBM), tiles_n = (int)cdiv(N, kBN);
    const int tiles = tiles_m * tiles_n;
    // Whole rounds of 256x256 tiles here; a last round that would fill at most
    // half of the CUs goes to the tail kernel as 128x128 tiles instead.
    const int cus = device_cu_count();
    const int tail = (cus > 0 && tiles > cus && tiles % cus <= cus / 2) ? tiles % cus : 0;
    // Several tiles per workgroup: one persistent workgroup per CU.  Same-box
    // timings at 18432 rows: the stream form takes 7% off at 12-24 k-steps per
    // tile and 3.5% at 48, ties at 96, and with its wave-private epilogue
    // takes 0.9% off at 144 (the fc2 wgrad; with the earlier epilogue it lost
    // 1-2% there).  Longer K is not measured, so it keeps one tile per
    // workgroup.
    if (out_dtype == MX_BF16 && N % 8 == 0 && M * ldc * 2 < (int64_t(1) << 31) && K_pad <= 144 * 128 && cus > 0 &&
        tiles - tail > cus) {
        auto kernel = bias ? gemm_a4w4_stream_kernel<true> : gemm_a4w4_stream_kernel<false>;
        hipLaunchKernelGGL(kernel, dim3((unsigned)cus), dim3(kThreads), 0, stream, (int)M, (int)N, (int)K_pad,
                           tiles_m, tiles_n, tiles - tail, A, As, B, Bs, bias, C, (int)ldc);
    } else {
        auto kernel = out_dtype == MX_BF16 ? (bias ? gemm_a4w4_kernel<true, true> : gemm_a4w4_kernel<true, false>)
                                           : (bias ? gemm_a4w4_kernel<false, true> : gemm_a4w4_kernel<false, false>);
        hipLaunchKernelGGL(kernel, dim3((unsigned)(tiles - tail)), dim3(kThreads), 0, stream, M, N, K_pad, tiles_m,
                           tiles_n, A, As, B, Bs, bias, C, ldc);
    }
    if (tail) {
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_gemm_tail(M, N, K_pad, tiles_m, tiles_n, tiles - tail, tail, A, As, B, Bs, bias, out_dtype, C,
                                ldc, stream);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_fp8(int64_t M, int64_t N, int64_t K, const uint8_t *A, const float *a_scale_inv,
                           const uint8_t *B, const float *b_scale_inv, mx_dtype out_dtype, void *C, int64_t ldc,
                           hipStream_t stream) {
    const int64_t K_pad = padded(K);
    if (K_pad == 0) {
        const int64_t n = M * N;
        dim3 grid((unsigned)cdiv(n, 256));
        if (out_dtype == MX_BF16)
            hipLaunchKernelGGL(fill_kernel<uint16_t>, grid, dim3(256), 0, stream, reinterpret_cast<uint16_t *>(C),
                               M, N, ldc, nullptr);
        else
            hipLaunchKernelGGL(fill_kernel<float>, grid, dim3(256), 0, stream, reinterpret_cast<float *>(C), M, N,
                               ldc, nullptr);
        return hipGetLastError();
    }
    // buffer offsets are 32-bit: each operand blob must stay below 2 GiB
    if (cdiv(M, 16) * 16 * K_pad >= (int64_t(1) << 31) || cdiv(N, 16) * 16 * K_pad >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
    const int tiles_m = (int)cdiv(M, kBM), tiles_n = (int)cdiv(N, kBN);
    dim3 grid((unsigned)(tiles_m * tiles_n));
    auto kernel = out_dtype == MX_BF16 ? gemm_fp8_kernel<true> : gemm_fp8_kernel<false>;
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, M, N, K_pad, tiles_m, tiles_n, A, a_scale_inv, B,
                       b_scale_inv, C, ldc);
    return hipGetLastError();
}

}  // namespace mx
