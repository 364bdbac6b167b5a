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
// next 8 bits (u >> 14) & 0xFF, which equal floor(256 (v-lo)/(hi-lo)); the
// kernel gets that sum as one carry (see pack8_sr).

// Random Hadamard transform (when a direction's rht seed is non-zero): the
// page's dual-quantize op has an "rht" switch for the column-wise blobs of
// the activation and the gradient (the wgrad operands) and defines nothing
// more.  Here each 32-element block along the quantized axis becomes
// c * H32 * D * x in fp32: D negates the positions whose bit is set in a
// sign word drawn from the seed (Philox-4x32-10, counter (0,0,0,2), key
// (seed, 0), first word), H32 is the Sylvester Hadamard matrix applied as a
// fast Walsh-Hadamard transform (pairs differing in position bit k = 0..4,
// (a, b) -> (a + b, a - b)), c = fp32(1/sqrt(32)).  A lane holds 8 positions
// of a block, so bits 0..2 are in-lane butterflies and bits 3, 4 exchange
// with the lanes that hold the other 8-position slices.  Pads are +0 before
// the transform.  Scale and codes then come from the fp32 values: RNE with
// V_CVT_SCALEF32_PK_FP4_F32 (a probe compared it with the comparison rule
// below on every non-negative finite fp32 pattern at scale bytes 0, 1, 127,
// 130, 200 and 254: no difference), SR from exact fraction bits of
// |y| 2^(127-c).

#include "mx_internal.h"

namespace mx {
namespace {

constexpr int kWaveRows = 32;
constexpr int kTileCols = 128;
constexpr int kWaves = 4;
constexpr int kTileRows = kWaveRows * kWaves;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// 2^(c-127) as fp32 (c = 0 is the subnormal 2^-127, c = 255 gives +Inf):
// one exact ldexp of 2^-127 (fp32 denormals are kept in this build).
__device__ __forceinline__ float scale_f32(uint32_t c) {
    return __builtin_ldexpf(__uint_as_float(0x00400000u), (int)c);
}

// Scale byte of a block amax and whether the block holds Inf/NaN.  FINITE:
// the caller knows no element of the wave's tile is Inf/NaN.
template <bool FINITE = false>
__device__ __forceinline__ uint32_t scale_code_nf(uint32_t amax16, bool &nonfinite) {
    nonfinite = FINITE ? false : amax16 >= 0x7F80u;
    return nonfinite ? 0xFFu : __builtin_elementwise_sub_sat(amax16 >> 7, 2u);
}

// compile-time flag for the two instances of an encode
template <bool B>
struct FiniteTag {
    static constexpr bool value = B;
};

// Four bf16 pairs (element 2i in the low half of p_i) -> 8 nibbles, RNE,
// saturating; a block holding Inf/NaN (scale byte 0xFF) gives all nibbles 0.
__device__ __forceinline__ uint32_t pack8_rne(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3,
                                              uint32_t c, bool nonfinite) {
    const float sf = scale_f32(c);
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, p0), sf, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, p1), sf, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, p2), sf, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, p3), sf, 3);
    return nonfinite ? 0u : r;
}

// bf16 pair (lo, hi) from the same half of two words: half 0 = low halves.
__device__ __forceinline__ uint32_t pair_of(uint32_t lo_word, uint32_t hi_word, int half) {
    return __builtin_amdgcn_perm(hi_word, lo_word, half ? 0x07060302u : 0x05040100u);
}

// Element h (0 = low half) of a bf16 pair word as an fp32 pattern: the bf16
// in the high 16 bits, zeros below.
__device__ __forceinline__ uint32_t elem_hi(uint32_t w, int h) {
    return h ? (w & 0xFFFF0000u) : (w << 16);
}

// Sign masks of eight elements held as bf16 pairs: element 2i is the low half
// of p_i, 2i+1 the high half.  Byte i of `even` is 0xFF iff element 2i is
// negative (0x00 otherwise), byte i of `odd` likewise for element 2i+1.
// V_PERM_B32 selectors 8..11 replicate bit 15 or 31 of either source across
// a byte.
__device__ __forceinline__ void sign_masks(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3,
                                           uint32_t &even, uint32_t &odd) {
    const uint32_t a = __builtin_amdgcn_perm(p1, p0, 0x0B090A08u);   // signs of elements 0 2 1 3
    const uint32_t b = __builtin_amdgcn_perm(p3, p2, 0x0B090A08u);   // signs of elements 4 6 5 7
    even = __builtin_amdgcn_perm(b, a, 0x05040100u);
    odd = __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Stochastic E2M1 nibbles of eight elements that share the scale byte c.
// xw(e) is element e as an fp32 pattern (elem_hi); nb(e) holds 255 minus its
// random byte in bits 16..23 and zeros elsewhere; even/odd are the sign
// masks of sign_masks; nonfinite: the block holds Inf/NaN (c = 0xFF).  With
// u = |x| 2^(1-c) clamped at code 7, (u << 2) +
// nb(e) carries into bit 24 iff the byte is below u's bits 14..21, so byte 3
// of the sum is the code (0..7).  Four byte permutes gather the eight codes
// (even elements to the low nibbles, odd ones to the high nibbles), the sign
// masks supply bit 3 of each nibble, and a block holding Inf/NaN (c = 0xFF)
// is zeroed once for all eight.
template <typename XW, typename NB>
__device__ __forceinline__ uint32_t pack8_sr(XW xw, uint32_t c, NB nb, uint32_t even, uint32_t odd, bool nonfinite) {
    const int sh = 1 - (int)c;
    constexpr uint32_t top = 7u << 22;
    uint32_t s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t u = __float_as_uint(__builtin_ldexpf(__builtin_fabsf(__uint_as_float(xw(e))), sh));
        u = u < top ? u : top;
        s[e] = (u << 2) + nb(e);
    }
    // byte 3 of two sums into bytes 0, 1 (selector 0x0C0C0703) or 2, 3 (0x07030C0C)
    const uint32_t lo = __builtin_amdgcn_perm(s[2], s[0], 0x0C0C0703u) | __builtin_amdgcn_perm(s[6], s[4], 0x07030C0Cu) |
                        (even & 0x08080808u);
    const uint32_t hi = __builtin_amdgcn_perm(s[3], s[1], 0x0C0C0703u) | __builtin_amdgcn_perm(s[7], s[5], 0x07030C0Cu) |
                        (odd & 0x08080808u);
    return nonfinite ? 0u : (lo | (hi << 4));
}

// Byte k of w moved to bits 16..23, zeros elsewhere (selector 0x0C gives 0x00).
__device__ __forceinline__ uint32_t byte_to_b2(uint32_t w, int k) {
    return __builtin_amdgcn_perm(w, w, 0x0C000C0Cu | ((uint32_t)k << 16));
}

// ------------------------------------------------------------------ Philox
// Philox-4x32-10 (Salmon et al., SC'11, sec. 4.2).
__device__ __forceinline__ void philox10(uint32_t &c0, uint32_t &c1, uint32_t &c2, uint32_t &c3,
                                         uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;    // one v_mad_u64_u32 each
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // three-input xors as one V_BITOP3_B32 each (truth table 0x96 = a ^ b ^ c)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c0 = n0; c1 = (uint32_t)p1; c2 = n2; c3 = (uint32_t)p0;
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

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// max of each 16-bit half (one packed instruction for two magnitudes)
__device__ __forceinline__ uint32_t pk_umax(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a), __builtin_bit_cast(u16x2_t, b)));
}

// Maximum with lane l^M, without an LDS round trip: l^1 and l^2 through DPP
// quad permutes ([1,0,3,2], [2,3,0,1]), l^16 and l^32 through the lane-swap
// instructions, whose two results hold this lane's value and the other
// lane's in an order that depends on the lane (so both go into the max).
// Every lane of the wave must be active.  PK: two 16-bit halves (pk_umax).
template <int M, bool PK>
__device__ __forceinline__ uint32_t lane_max(uint32_t v) {
    const auto mx = [](uint32_t a, uint32_t b) { return PK ? pk_umax(a, b) : umax(a, b); };
    static_assert(M == 1 || M == 2 || M == 16 || M == 32, "lane distance");
    if constexpr (M == 1) return mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    else if constexpr (M == 2) return mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return mx(r[0], r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return mx(r[0], r[1]);
    }
}

// ------------------------------------------------------------------ RHT
constexpr uint32_t kRhtScaleBits = 0x3E3504F3u;   // fp32 nearest to 1/sqrt(32)

__device__ __forceinline__ uint32_t rht_sign_word(uint32_t seed) {
    uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 2;
    philox10(c0, c1, c2, c3, seed, 0u);
    return c0;
}

// One butterfly stage between lane pairs (lane, lane ^ MASK) on 8 values:
// the lane with the bit clear (holding a) keeps a + b, its partner (holding
// b) keeps a - b.
//  MASK 16 / 32: V_PERMLANE16_SWAP / V_PERMLANE32_SWAP of a value with itself
//    returns (a, b) in both lanes of a pair (checked on MI355X: the first
//    result is the lower row / half's value, the second the upper one's), so
//    both lanes compute fma(+-1, b, a), which rounds exactly like a +- b.
//  MASK 1 / 2: DPP quad permutations [1,0,3,2] / [2,3,0,1] fetch the partner.
template <int MASK>
__device__ __forceinline__ void rht_cross_stage(float (&v)[8], bool hi) {
#pragma clang fp contract(off)
    if constexpr (MASK == 16 || MASK == 32) {
        const float sgn = hi ? -1.0f : 1.0f;
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            const uint32_t x = __float_as_uint(v[a]);
            uint32_t lo, up;
            if constexpr (MASK == 16) {
                const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
                lo = r[0]; up = r[1];
            } else {
                const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
                lo = r[0]; up = r[1];
            }
            v[a] = __builtin_fmaf(sgn, __uint_as_float(up), __uint_as_float(lo));
        }
    } else {
        static_assert(MASK == 1 || MASK == 2, "lane exchange");
        constexpr int kCtl = MASK == 1 ? 0xB1 : 0x4E;
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            const float p = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[a]), kCtl, 0xF, 0xF, false));
            v[a] = hi ? p - v[a] : v[a] + p;
        }
    }
}

// The transform of one block, of which this lane holds positions
// 8*slice .. 8*slice+7 in v[0..7]; the slices differing in position bit 3 /
// bit 4 sit in lanes lane^MASK3 / lane^MASK4.
template <int MASK3, int MASK4>
__device__ __forceinline__ void rht8(float (&v)[8], uint32_t signs, int slice) {
#pragma clang fp contract(off)
    const uint32_t sl = signs >> (8 * slice);
#pragma unroll
    for (int a = 0; a < 8; ++a)
        if ((sl >> a) & 1u) v[a] = -v[a];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int h = 1 << k;
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            if (a & h) continue;
            const float x = v[a], y = v[a + h];
            v[a] = x + y;
            v[a + h] = x - y;
        }
    }
    rht_cross_stage<MASK3>(v, (slice & 1) != 0);
    rht_cross_stage<MASK4>(v, (slice & 2) != 0);
    const float cs = __uint_as_float(kRhtScaleBits);
#pragma unroll
    for (int a = 0; a < 8; ++a) v[a] = v[a] * cs;
}

// Scale byte from the block's max |y| as fp32 bits (NaN sorts above Inf).
__device__ __forceinline__ uint32_t scale_code_f32(uint32_t amax_bits) {
    if (amax_bits >= 0x7F800000u) return 0xFFu;
    const uint32_t e = amax_bits >> 23;
    return e > 2u ? e - 2u : 0u;
}

// Stochastic E2M1 nibbles of eight fp32 values y (element e in nibble e)
// that share the scale byte c: pack8_sr's carry form with u taken exactly
// for fp32 inputs.  With v = |y| 2^(127-c) (below 8 in a finite block), u
// should be the fp32 bits of v 2^-126 with the bits under 2^-149 cut off: that
// pattern itself is exact for v >= 1, while below 1 ldexp rounds into the
// subnormal range (to floor(v 2^23) or one more), so u is the smaller of the
// pattern and the truncating conversion of v 2^23 (equal for v in [1, 2),
// larger above), clamped at code 7 by the same three-way minimum.  Signs as
// in sign_masks, from bit 31 of each value.  A block holding Inf/NaN (c = 0xFF)
// gives all nibbles 0.
template <typename NB>
__device__ __forceinline__ uint32_t pack8_sr_f32(const float (&y)[8], uint32_t c, NB nb) {
    const auto sgn = [&](int e) { return __float_as_uint(y[e]); };
    // byte i of even / odd: 0xFF iff element 2i / 2i+1 is negative (selectors
    // 9, 11: bit 31 of src1, src0), taken first so that each y dies with its sum
    const uint32_t even = __builtin_amdgcn_perm(sgn(2), sgn(0), 0x0C0C0B09u) | __builtin_amdgcn_perm(sgn(6), sgn(4), 0x0B090C0Cu);
    const uint32_t odd = __builtin_amdgcn_perm(sgn(3), sgn(1), 0x0C0C0B09u) | __builtin_amdgcn_perm(sgn(7), sgn(5), 0x0B090C0Cu);
    const int ex = 1 - (int)c;
    constexpr uint32_t top = 7u << 22;
    uint32_t s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float a = __builtin_fabsf(y[e]);
        const uint32_t pat = __float_as_uint(__builtin_ldexpf(a, ex));
        const uint32_t fl = (uint32_t)__builtin_ldexpf(a, ex + 149);
        const uint32_t u = __builtin_elementwise_min(__builtin_elementwise_min(pat, fl), top);
        s[e] = (u << 2) + nb(e);
    }
    const uint32_t lo = __builtin_amdgcn_perm(s[2], s[0], 0x0C0C0703u) | __builtin_amdgcn_perm(s[6], s[4], 0x07030C0Cu) |
                        (even & 0x08080808u);
    const uint32_t hi = __builtin_amdgcn_perm(s[3], s[1], 0x0C0C0703u) | __builtin_amdgcn_perm(s[7], s[5], 0x07030C0Cu) |
                        (odd & 0x08080808u);
    return c == 0xFFu ? 0u : (lo | (hi << 4));
}

// Eight fp32 values (element e in nibble e) -> E2M1 codes of y / 2^(c-127), RNE, saturating, sign kept.
__device__ __forceinline__ uint32_t pack8_rne_f32(float y0, float y1, float y2, float y3, float y4, float y5,
                                                  float y6, float y7, uint32_t c) {
    const float sf = scale_f32(c);
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y0, y1, sf, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y2, y3, sf, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y4, y5, sf, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y6, y7, sf, 3);
    return c == 0xFFu ? 0u : r;
}

// ------------------------------------------------------------------ FP6
// MXFP6 elements (OCP MX v1.0 sec. 5.3.2): fmt 2 = E2M3 (3 mantissa bits,
// emax_elem 2), fmt 3 = E3M2 (2 mantissa bits, emax_elem 4).  As for E2M1,
// u = |x| * 2^(adj-c) as fp32 bits maps the format's smallest normal to the
// smallest fp32 normal (adj = 1 for E2M3, 3 for E3M2), so the code is the
// field u >> sh (sh = 23 - mantissa bits: exponent and mantissa bits in
// place, the subnormal step on the fp32 subnormal grid), exact for bf16
// inputs.  RNE adds half an ulp minus one plus the code's low bit before the
// shift and saturates at code 31; SR clamps u at code 31 and adds
// (255 - byte) << (sh - 8): the carry into bit sh happens iff the byte is
// below the next 8 bits, which equal floor(256 (v-lo)/(hi-lo)).
struct Fp6Dir {
    int sh, adj;
    uint32_t emax;
};
__device__ __forceinline__ Fp6Dir fp6_dir(uint32_t fmt) {
    return fmt == 2u ? Fp6Dir{20, 1, 2u} : Fp6Dir{21, 3, 4u};
}
__device__ __forceinline__ uint32_t scale_code_emax(uint32_t amax16, uint32_t emax) {
    if (amax16 >= 0x7F80u) return 0xFFu;
    const uint32_t e = amax16 >> 7;
    return e > emax ? e - emax : 0u;
}
// 6-bit code (sign in bit 5) of bf16 x16 under scale byte c, round to
// nearest even with saturation (the stochastic code is pack8_sr6's).
__device__ __forceinline__ uint32_t code6(uint32_t x16, uint32_t c, const Fp6Dir &f) {
    const float xf = __uint_as_float((x16 & 0x7FFFu) << 16);
    const uint32_t u = __float_as_uint(__builtin_ldexpf(xf, f.adj - (int)c));
    uint32_t code = (u + (1u << (f.sh - 1)) - 1u + ((u >> f.sh) & 1u)) >> f.sh;
    code = code < 31u ? code : 31u;
    return c == 0xFFu ? 0u : (code | ((x16 >> 10) & 0x20u));
}
// One 32-element block (16 bf16 pairs, element e in half e%2 of w[e/2]) ->
// scale byte and six dwords of codes by V_CVT_SCALEF32_PK32_FP6_BF16 /
// _BF6_BF16 (E2M3 / E3M2), which divide by the fp32 scale and round to
// nearest even with saturation; probed on MI355X against the add-and-shift
// encode below for every finite bf16 at every scale byte a block can have:
// no difference.  A block holding Inf/NaN gets scale 0xFF and zero codes.
typedef __bf16 bf16x32_t __attribute__((ext_vector_type(32)));
typedef uint32_t u32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x6_t __attribute__((ext_vector_type(6)));
__device__ __forceinline__ uint32_t fp6_block_hw(const u32x16_t &w, uint32_t fmt, uint32_t emax, u32x6_t &out) {
    u16x2_t m = {0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w[i] & 0x7FFF7FFFu));
    const uint32_t amax16 = m[0] > m[1] ? m[0] : m[1];
    const uint32_t sc = scale_code_emax(amax16, emax);
    const bf16x32_t x = __builtin_bit_cast(bf16x32_t, w);
    const float sf = scale_f32(sc);
    out = fmt == 2u ? __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(x, sf) : __builtin_amdgcn_cvt_scalef32_pk32_bf6_bf16(x, sf);
    if (sc == 0xFFu) out = u32x6_t{0u, 0u, 0u, 0u, 0u, 0u};
    return sc;
}
__device__ __forceinline__ void lds_put24(uint8_t *p, const u32x6_t &v) {
    *reinterpret_cast<uint2 *>(p) = uint2{v[0], v[1]};
    *reinterpret_cast<uint2 *>(p + 8) = uint2{v[2], v[3]};
    *reinterpret_cast<uint2 *>(p + 16) = uint2{v[4], v[5]};
}

// Eight 6-bit codes -> 48 bits, element e at bits [6e, 6e+6): lo = bits 0..31, hi = 32..47.
__device__ __forceinline__ void pack6(const uint32_t (&k)[8], uint32_t &lo, uint32_t &hi) {
    lo = k[0] | (k[1] << 6) | (k[2] << 12) | (k[3] << 18) | (k[4] << 24) | (k[5] << 30);
    hi = (k[5] >> 2) | (k[6] << 4) | (k[7] << 10);
}

// Four six-bit values in bytes 0..3 -> 24 bits (byte i at bits [6i, 6i+6)).
__device__ __forceinline__ uint32_t pack24(uint32_t x) {
    const uint32_t y = (x & 0x003F003Fu) | ((x >> 2) & 0x0FC00FC0u);
    return (y & 0xFFFu) | ((y >> 4) & 0xFFF000u);
}

// Stochastic MXFP6 codes of eight elements that share the scale byte c, laid
// out as pack6 does.  With u = |x| 2^(adj-c) as fp32 bits clamped at code 31
// (bits [sh, sh+5) hold the lower grid point's code, the 8 bits under them
// floor(256 (v-lo)/(hi-lo))), the code rounds up iff the random byte is
// below those 8 bits: the carry form of pack8_sr with the format's shift,
// (u << (24-sh)) + nb(e) carrying into bit 24, so byte 3 of the sum is the
// code.  xw(e): element e as an fp32
// pattern; nb(e): 255 minus its random byte in bits 16..23; s0123, s4567:
// 0xFF in byte i iff element i (i + 4) is negative.  A block holding Inf/NaN
// (c = 0xFF) gives all codes 0.
template <typename XW, typename NB>
__device__ __forceinline__ void pack8_sr6(XW xw, uint32_t c, const Fp6Dir &f, NB nb, uint32_t s0123, uint32_t s4567,
                                          uint32_t &lo, uint32_t &hi) {
    const int sh = f.sh, ex = f.adj - (int)c;
    const uint32_t top = 31u << sh;
    uint32_t s[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t u = __float_as_uint(__builtin_ldexpf(__builtin_fabsf(__uint_as_float(xw(e))), ex));
        u = u < top ? u : top;
        s[e] = (u << (24 - sh)) + nb(e);
    }
    const uint32_t w0 = __builtin_amdgcn_perm(s[1], s[0], 0x0C0C0703u) | __builtin_amdgcn_perm(s[3], s[2], 0x07030C0Cu) |
                        (s0123 & 0x20202020u);
    const uint32_t w1 = __builtin_amdgcn_perm(s[5], s[4], 0x0C0C0703u) | __builtin_amdgcn_perm(s[7], s[6], 0x07030C0Cu) |
                        (s4567 & 0x20202020u);
    const uint32_t z0 = pack24(w0), z1 = pack24(w1);
    lo = c == 0xFFu ? 0u : z0 | (z1 << 24);
    hi = c == 0xFFu ? 0u : z1 >> 8;
}
// 6 bytes at an even LDS byte offset o.
__device__ __forceinline__ void lds_put6(uint8_t *base, int o, uint32_t lo, uint32_t hi) {
    if ((o & 3) == 0) {
        *reinterpret_cast<uint32_t *>(base + o) = lo;
        *reinterpret_cast<uint16_t *>(base + o + 4) = (uint16_t)hi;
    } else {
        *reinterpret_cast<uint16_t *>(base + o) = (uint16_t)lo;
        *reinterpret_cast<uint32_t *>(base + o + 2) = (lo >> 16) | (hi << 16);
    }
}

// bf16 pair x times bf16 pair y, each product in fp32 (IEEE, denormals kept)
// and rounded to bf16 nearest-even: what a producer that multiplies in fp32
// and stores bf16 would have written.
__device__ __forceinline__ uint32_t mul_bf16_pair(uint32_t x, uint32_t y) {
#pragma clang fp contract(off)
    const f32x2_t p = {__uint_as_float(x << 16) * __uint_as_float(y << 16),
                       __uint_as_float(x & 0xFFFF0000u) * __uint_as_float(y & 0xFFFF0000u)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, bf16x2_t));
}

// Dual stochastic rounding holds both directions' random bytes while the
// staging loads are in flight.  Asking for at least two waves per SIMD (up to
// 256 VGPRs) let the compiler schedule the MXFP4 kernel in 158 VGPRs without
// spills, so three waves fitted a SIMD, where asking for three (168 VGPRs)
// made it spill; with the packed amax and the all-finite encode it now takes
// 121 VGPRs (four waves) under the same request.  Same-box timings of the 18432x3072 dY quantize (before the
// permute gather of pack8_sr): 0.0637 ms, against 0.0688 ms with the spilling
// three-wave request and 0.0711 ms for the earlier form that drew the bytes
// after the loads had landed.  (With the Hadamard transform as well it would
// spill, so that form keeps its registers.)
// MXFP6 draws its bytes after the loads have landed; with both directions
// stochastic it fits three waves (168 VGPRs) without spills, with one
// direction stochastic (the mixed-options forms) two.  The Hadamard-transform
// forms without stochastic rounding would take 133 VGPRs (three waves); asked
// for four they fit 128 (5 spilled before the lane-swap exchanges, none
// since), and the dual quantize of an 18432x12288 activation with its column
// blob transformed ran 0.164 -> 0.157 ms (same box, three alternations).
// Those with stochastic rounding would take 171 (two waves); asked for three
// they fit 168 (4 spilled before the lane-swap exchanges, none since): the
// dual SR quantize of an 18432x3072 gradient with its column blob transformed
// 0.079 (two waves) -> 0.071 ms.
template <int ELEM, bool DUAL, bool ROW_SR, bool COL_SR, bool RHT>
constexpr int kMinWaves = (DUAL && (ROW_SR || COL_SR) && !RHT) ? (ELEM == 6 ? (ROW_SR && COL_SR ? 3 : 2) : 2)
                          : (RHT ? (!ROW_SR && !COL_SR ? 4 : 3) : 1);

// ELEM 4: MXFP4 (E2M1); ELEM 6: MXFP6 with each direction's format in its
// options (no Hadamard transform).  Staged blob-row lines hold 128 elements:
// 64 bytes (FP4) or 96 bytes (FP6), padded by 16 bytes against bank conflicts.
// MUL: the quantized tensor is bf16(x * g) elementwise (the prologue of
// mx_quantize_dual_mul), formed in the staging read.
template <int ELEM, int LAYOUT, bool DUAL, bool ROW_SR, bool COL_SR, bool RHT, bool MUL = false>
__global__ __launch_bounds__(256) __attribute__((
    amdgpu_waves_per_eu(kMinWaves<ELEM, DUAL, ROW_SR, COL_SR, RHT>, 8))) void quantize_kernel(QuantArgs a) {
    static_assert(ELEM == 4 || (ELEM == 6 && !RHT), "element size");
    static_assert(!MUL || (ELEM == 4 && !RHT), "prologue");
    constexpr int kLinePitch = ELEM == 4 ? 80 : 112;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;
    const int q = lane >> 4;
    const int64_t row0 = ((int64_t)blockIdx.y + a.row_tile0) * kTileRows + wave * kWaveRows;
    const int64_t col0 = (int64_t)blockIdx.x * kTileCols;
    const int64_t M = a.M, N = a.N;
    // real rows among the lane's 8 (8q..8q+7) and real columns among its 8 (8c..8c+7)
    const int64_t rl = M - (row0 + 8 * q), cl = N - (col0 + 8 * c);
    const int rows_here = rl < 0 ? 0 : (rl > 8 ? 8 : (int)rl);
    const int cols_here = cl < 0 ? 0 : (cl > 8 ? 8 : (int)cl);

    // ---- staging read: d[t][w] = bf16 pair (cols 2w, 2w+1 of the lane's 8) of row 8q+t.
    // Non-temporal loads: the input is read once, so it should not displace
    // what the caches hold for the GEMMs (same-box fc2 step: X 0.129 -> 0.121 ms,
    // step -1.4%).
    uint32_t d[8][4];
    const int64_t j0 = col0 + 8 * c;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const int64_t i = row0 + 8 * q + t;
        const uint16_t *p = a.x + i * a.ldx + j0;
        if (i < M && j0 + 8 <= N) {
            const v4u_t v = __builtin_nontemporal_load(reinterpret_cast<const v4u_t *>(p));
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
    // the second factor of the prologue, same shape and bounds (positions past
    // M or N read as 0); its loads are issued here and the products formed
    // after the random bytes
    uint32_t gl[MUL ? 8 : 1][4];
    if constexpr (MUL) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int64_t i = row0 + 8 * q + t;
            const uint16_t *p = a.g + i * a.ldg + j0;
            if (i < M && j0 + 8 <= N) {
                const v4u_t v = __builtin_nontemporal_load(reinterpret_cast<const v4u_t *>(p));
                gl[t][0] = v.x; gl[t][1] = v.y; gl[t][2] = v.z; gl[t][3] = v.w;
            } else {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t lo = (i < M && j0 + 2 * w < N) ? p[2 * w] : 0u;
                    const uint32_t hi = (i < M && j0 + 2 * w + 1 < N) ? p[2 * w + 1] : 0u;
                    gl[t][w] = lo | (hi << 16);
                }
            }
        }
    }

    // ---- stochastic-rounding bytes.  They do not depend on x, so MXFP4 draws
    // them while the staging loads above are in flight; MXFP6 draws them after
    // the amax reductions (with its encode, holding the bytes across the loads
    // costs occupancy or spills: same-box SR dual quantize of an 18432x3072
    // gradient 0.078-0.080 ms late, 0.086-0.090 ms early).  One Philox block
    // covers 16 consecutive row-major elements: the columns of lanes c and
    // c^1.  When both
    // directions round stochastically and every group starts on a lane pair
    // (N and both index bases multiples of 16), lane c&1 == d computes the
    // blocks of direction d for its 8 rows and the pair swaps the halves it
    // does not need, halving the Philox work; otherwise each lane computes
    // its own 8-byte windows.
    uint32_t rrow_lo[8], rrow_hi[8], rcol_lo[8], rcol_hi[8];
    auto draw_sr = [&]() {
        if (ROW_SR && COL_SR && a.sr_pairs) {
            const uint32_t p = (uint32_t)(c & 1);
            const DirOpts &o = p ? a.col : a.row;
            const uint64_t jpair = (uint64_t)(col0 + 16 * (c >> 1));
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int64_t i = row0 + 8 * q + t;
                const uint64_t g = (o.index_base + (uint64_t)i * (uint64_t)N + jpair) >> 4;
                // after a Hadamard transform pads carry values and draw from
                // counter word 3 = 2 + dir: the row blob's pads are columns past
                // N (whole 16-blocks, N % 16 == 0 here), the column blob's rows
                // past M (without the transform pads are 0 and round to 0 with
                // any byte, so those kernels skip the distinction)
                const bool pad = RHT && (p ? i >= M : (int64_t)jpair >= N);
                uint32_t w0 = (uint32_t)g, w1 = (uint32_t)(g >> 32), w2 = o.tensor_id, w3 = p + (pad ? 2u : 0u);
                philox10(w0, w1, w2, w3, o.key0, o.key1);
                const uint32_t r0 = (uint32_t)__shfl_xor((int)(p ? w0 : w2), 1, 64);
                const uint32_t r1 = (uint32_t)__shfl_xor((int)(p ? w1 : w3), 1, 64);
                rrow_lo[t] = p ? r0 : w0;
                rrow_hi[t] = p ? r1 : w1;
                rcol_lo[t] = p ? w2 : r0;
                rcol_hi[t] = p ? w3 : r1;
            }
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int64_t i = row0 + 8 * q + t;
                rrow_lo[t] = rrow_hi[t] = rcol_lo[t] = rcol_hi[t] = 0;
                // pads too: after a Hadamard transform they carry values and draw from
                // counter word 3 = 2 + dir (otherwise they are 0 and round to 0 with any byte)
                if (ROW_SR) {
                    const uint64_t n0 = a.row.index_base + (uint64_t)i * (uint64_t)N + (uint64_t)j0;
                    rand8(n0, a.row, 0u, rrow_lo[t], rrow_hi[t]);
                    if (RHT && j0 + 8 > N) {
                        // columns past N among the lane's 8: take their bytes from the pad space
                        uint32_t plo, phi;
                        rand8(n0, a.row, 2u, plo, phi);
                        const int64_t nreal = N - j0;          // real columns of the lane (may be <= 0)
                        const uint64_t keep = nreal <= 0 ? 0ull : (~0ull >> (64 - 8 * nreal));
                        const uint64_t v = (((uint64_t)rrow_hi[t] << 32) | rrow_lo[t]) & keep;
                        const uint64_t w = (((uint64_t)phi << 32) | plo) & ~keep;
                        rrow_lo[t] = (uint32_t)(v | w);
                        rrow_hi[t] = (uint32_t)((v | w) >> 32);
                    }
                }
                if (DUAL && COL_SR)
                    rand8(a.col.index_base + (uint64_t)i * (uint64_t)N + (uint64_t)j0, a.col, RHT && i >= M ? 3u : 1u,
                          rcol_lo[t], rcol_hi[t]);
            }
        }
    };
    if constexpr (ELEM == 4) draw_sr();

    if constexpr (MUL) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int w = 0; w < 4; ++w) d[t][w] = mul_bf16_pair(d[t][w], gl[t][w]);
    }

    // ---- block amax.  A magnitude is the bf16 pattern with its sign cleared,
    // compared as an integer (the order of |x|, Inf and NaN above every finite
    // value), two per packed 16-bit max.  Row direction: per row t over the
    // lane's 8 columns, then lanes c^1, c^2.  For MXFP4 without the Hadamard
    // transform the column maxima are accumulated in the same pass over the
    // magnitudes, so those die before the encode (taken after the row encode,
    // they stayed live through it: 164 -> 202 VGPRs in the stochastic dual
    // kernel).
    constexpr bool kEarlyColAmax = DUAL && ELEM == 4 && !RHT;
    uint32_t ramax[8], rpk[8], cpk[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        uint32_t m[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) m[w] = d[t][w] & 0x7FFF7FFFu;
        rpk[t] = pk_umax(pk_umax(m[0], m[1]), pk_umax(m[2], m[3]));   // (even columns, odd columns)
        if constexpr (kEarlyColAmax) {
#pragma unroll
            for (int w = 0; w < 4; ++w) cpk[w] = t == 0 ? m[w] : pk_umax(cpk[w], m[w]);
        }
    }
    // no Inf/NaN anywhere in the wave's tile (the usual case): the MXFP4
    // encodes then skip the per-block test and selects.  A magnitude of at
    // least 0x7F80 carries into bit 15 of its half when 0x80 is added.
    bool wave_finite = false;
    if constexpr (ELEM == 4) {
        const uint32_t m = pk_umax(pk_umax(pk_umax(rpk[0], rpk[1]), pk_umax(rpk[2], rpk[3])),
                                   pk_umax(pk_umax(rpk[4], rpk[5]), pk_umax(rpk[6], rpk[7])));
        const uint32_t big =
            __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, m) + u16x2_t{0x80, 0x80}) & 0x80008000u;
        wave_finite = __builtin_amdgcn_ballot_w64(big != 0u) == 0u;
    }
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
        // rows t and t+1 in the low and high halves
        uint32_t pk = pk_umax(__builtin_amdgcn_perm(rpk[t + 1], rpk[t], 0x05040100u),
                              __builtin_amdgcn_perm(rpk[t + 1], rpk[t], 0x07060302u));
        pk = lane_max<2, true>(lane_max<1, true>(pk));
        ramax[t] = pk & 0xFFFFu;
        ramax[t + 1] = pk >> 16;
    }
    // 32x32 tile amax (2D mode): rows of the lane, then the 4 q-lanes
    uint32_t tile_amax = 0;
    if (a.row.use_2d || (DUAL && a.col.use_2d)) {
        uint32_t m = 0;
#pragma unroll
        for (int t = 0; t < 8; ++t) m = umax(m, ramax[t]);
        tile_amax = lane_max<32, false>(lane_max<16, false>(m));
    }

    // ---- block amax, column direction: per column u of the lane, 8 rows
    // in-lane (accumulated above for MXFP4 without the transform), then lanes
    // q^1, q^2.  MXFP6 draws its random bytes after this point and takes the
    // column amax later.
    uint32_t camax[8];
    auto col_amax = [&]() {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t pk = cpk[w];   // columns 2w and 2w+1 in the low and high halves
            if constexpr (!kEarlyColAmax) {
#pragma unroll
                for (int t = 0; t < 8; ++t) pk = pk_umax(pk, d[t][w] & 0x7FFF7FFFu);
            }
            pk = lane_max<32, true>(lane_max<16, true>(pk));
            camax[2 * w] = pk & 0xFFFFu;
            camax[2 * w + 1] = pk >> 16;
        }
    };
    if constexpr (kEarlyColAmax) col_amax();

    if constexpr (ELEM == 6) draw_sr();

    // ---- encode both directions into LDS, then write whole 16-byte slices.
    // Staging: one 64-byte line per blob row of this workgroup's tile (128 blob
    // rows per direction, 128 quantized elements each), padded to 80 bytes to
    // spread LDS banks; scales as 4 bytes per blob row.
    // MXFP6, round to nearest, 1D blocks: each 32-element block is gathered
    // into one lane through a 128 x 128 bf16 buffer (rows, then columns) and
    // encoded by the hardware converter.  The codes wait in registers until
    // every gather is done, so the staging lines take the same memory
    // (35 KB of LDS per workgroup instead of 63: four workgroups per CU).
    constexpr int kXPitch = 272;
    constexpr int kDataBytes = 2 * kTileRows * kLinePitch;
    // (only kernels with a round-to-nearest direction can take that path)
    constexpr int kXBytes = (ELEM == 6 && (!ROW_SR || (DUAL && !COL_SR))) ? kTileRows * kXPitch : 0;
    __shared__ __attribute__((aligned(16))) uint8_t s_buf[kXBytes > kDataBytes ? kXBytes : kDataBytes];
    uint8_t(*const s_data)[kTileRows * kLinePitch] = reinterpret_cast<uint8_t(*)[kTileRows * kLinePitch]>(s_buf);
    uint8_t *const s_x = s_buf;
    __shared__ __attribute__((aligned(16))) uint8_t s_scale[2][kTileRows * 4];
    const int r_loc0 = wave * kWaveRows + 8 * q;      // this lane's first tile row
    // the lane's staging addresses for row t / column u of its 8 (MXFP4):
    // kept in registers (opaque to the compiler), so that every write adds
    // only a constant offset instead of recomputing the address per row
    uint32_t row_line = r_loc0 * kLinePitch + 4 * c, row_scale = r_loc0 * 4 + c / 4;
    uint32_t col_line = 8 * c * kLinePitch + 16 * wave + 4 * q, col_scale = 8 * c * 4 + wave;
    asm volatile("" : "+v"(row_line), "+v"(row_scale), "+v"(col_line), "+v"(col_scale));

    if constexpr (ELEM == 4) {
    // row-wise: row r_loc0+t, 8 elements at columns 8c.. -> dword c of the line
    if (RHT && a.row.rht) {
        // per row t: the lane's 8 columns are slice c%4 of their 32-column block
        const uint32_t signs = rht_sign_word(a.row.rht);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = __uint_as_float(((d[t][u >> 1] >> (16 * (u & 1))) & 0xFFFFu) << 16);
            rht8<1, 2>(v, signs, c & 3);
            uint32_t m = 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) m = umax(m, __float_as_uint(v[u]) & 0x7FFFFFFFu);
            m = lane_max<2, false>(lane_max<1, false>(m));
            const int64_t i = row0 + 8 * q + t;
            const uint32_t sc = i < M ? scale_code_f32(m) : 0u;
            uint32_t packed = 0;
            if (ROW_SR) {
                const uint32_t nlo = ~rrow_lo[t], nhi = ~rrow_hi[t];
                packed = pack8_sr_f32(v, sc, [&](int u) { return byte_to_b2(u < 4 ? nlo : nhi, u & 3); });
            } else {
                packed = pack8_rne_f32(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7], sc);
            }
            // rows past M are the tiled layout's zero padding (the transform of an
            // all-zero row can hold -0, whose sign bit must not leak into it)
            if (i >= M) packed = 0;
            *reinterpret_cast<uint32_t *>(&s_data[0][(r_loc0 + t) * kLinePitch + 4 * c]) = packed;
            if ((c & 3) == 0) s_scale[0][(r_loc0 + t) * 4 + c / 4] = (uint8_t)sc;
        }
    } else {
    // each row's block amax: in 2D mode the 32x32 tile's, rows past M taking 0
    // (the tiled layout's zero padding; in 1D mode their amax is 0 already,
    // their data being 0), so that the encode reads one value per row
    if (a.row.use_2d) {
#pragma unroll
        for (int t = 0; t < 8; ++t) ramax[t] = t < rows_here ? tile_amax : 0u;
    }
    auto encode_rows = [&](auto fin) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        bool nonfinite;
        const uint32_t sc = scale_code_nf<decltype(fin)::value>(ramax[t], nonfinite);
        uint32_t packed = 0;
        if (ROW_SR) {
            const uint32_t nlo = ~rrow_lo[t], nhi = ~rrow_hi[t];
            uint32_t even, odd;
            sign_masks(d[t][0], d[t][1], d[t][2], d[t][3], even, odd);
            packed = pack8_sr([&](int e) { return elem_hi(d[t][e >> 1], e & 1); }, sc,
                              [&](int e) { return byte_to_b2(e < 4 ? nlo : nhi, e & 3); }, even, odd, nonfinite);
        } else {
            packed = pack8_rne(d[t][0], d[t][1], d[t][2], d[t][3], sc, nonfinite);
        }
        *reinterpret_cast<uint32_t *>(&s_data[0][row_line + t * kLinePitch]) = packed;
        if ((c & 3) == 0) s_scale[0][row_scale + 4 * t] = (uint8_t)sc;
        // one row at a time: interleaving rows only raises register pressure
        if (ROW_SR) __builtin_amdgcn_sched_barrier(0);
    }
    };
    if (wave_finite) encode_rows(FiniteTag<true>{});
    else encode_rows(FiniteTag<false>{});
    }

    if (DUAL && RHT && a.col.rht) {
        // per column u: the lane's 8 rows are slice q of their 32-row block
        const uint32_t signs = rht_sign_word(a.col.rht);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            float v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = __uint_as_float(((d[t][u >> 1] >> (16 * (u & 1))) & 0xFFFFu) << 16);
            rht8<16, 32>(v, signs, q);
            uint32_t m = 0;
#pragma unroll
            for (int t = 0; t < 8; ++t) m = umax(m, __float_as_uint(v[t]) & 0x7FFFFFFFu);
            m = lane_max<32, false>(lane_max<16, false>(m));
            const int64_t j = j0 + u;
            const uint32_t sc = j < N ? scale_code_f32(m) : 0u;
            uint32_t packed = 0;
            if (COL_SR) {
                packed = pack8_sr_f32(v, sc, [&](int t) { return byte_to_b2(~(u < 4 ? rcol_lo[t] : rcol_hi[t]), u & 3); });
            } else {
                packed = pack8_rne_f32(v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7], sc);
            }
            if (j >= N) packed = 0;    // tiled zero-padding rows of the column blob
            *reinterpret_cast<uint32_t *>(&s_data[1][(8 * c + u) * kLinePitch + 16 * wave + 4 * q]) = packed;
            if (q == 0) s_scale[1][(8 * c + u) * 4 + wave] = (uint8_t)sc;
        }
    } else if (DUAL) {
        if constexpr (!kEarlyColAmax) col_amax();
        // each column's block amax, as for the rows (columns past N take 0)
        if (a.col.use_2d) {
#pragma unroll
            for (int u = 0; u < 8; ++u) camax[u] = u < cols_here ? tile_amax : 0u;
        }
        auto encode_cols = [&](auto fin) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            bool nonfinite;
            const uint32_t sc = scale_code_nf<decltype(fin)::value>(camax[u], nonfinite);
            uint32_t packed = 0;
            if (COL_SR) {
                // element t of the column = row t, half h of word w; the sign
                // masks of the column pair (2w, 2w+1) come from the same four
                // permutes of rows (0,2), (4,6), (1,3), (5,7)
                const int w = u >> 1, h = u & 1;
                const uint32_t s02 = __builtin_amdgcn_perm(d[2][w], d[0][w], 0x0B090A08u);
                const uint32_t s46 = __builtin_amdgcn_perm(d[6][w], d[4][w], 0x0B090A08u);
                const uint32_t s13 = __builtin_amdgcn_perm(d[3][w], d[1][w], 0x0B090A08u);
                const uint32_t s57 = __builtin_amdgcn_perm(d[7][w], d[5][w], 0x0B090A08u);
                const uint32_t half = h ? 0x07060302u : 0x05040100u;
                packed = pack8_sr([&](int t) { return elem_hi(d[t][w], h); }, sc,
                                  [&](int t) { return byte_to_b2(~(u < 4 ? rcol_lo[t] : rcol_hi[t]), u & 3); },
                                  __builtin_amdgcn_perm(s46, s02, half), __builtin_amdgcn_perm(s57, s13, half),
                                  nonfinite);
            } else {
                const int w = u >> 1, h = u & 1;
                packed = pack8_rne(pair_of(d[0][w], d[1][w], h), pair_of(d[2][w], d[3][w], h),
                                   pair_of(d[4][w], d[5][w], h), pair_of(d[6][w], d[7][w], h), sc, nonfinite);
            }
            // blob row = tile column 8c+u; this wave's 32 rows are bytes [16*wave, 16*wave+16)
            *reinterpret_cast<uint32_t *>(&s_data[1][col_line + u * kLinePitch]) = packed;
            if (q == 0) s_scale[1][col_scale + 4 * u] = (uint8_t)sc;
            if (COL_SR) __builtin_amdgcn_sched_barrier(0);
        }
        };
        if (wave_finite) encode_cols(FiniteTag<true>{});
        else encode_cols(FiniteTag<false>{});
    }
    } else {
        // MXFP6: the hardware-converter passes gather through s_x (rows, then
        // columns) into registers; every staging write comes after the last
        // gather, since the staging lines share s_x's memory
        const bool row_hw = !ROW_SR && !a.row.use_2d;
        const bool col_hw = DUAL && !COL_SR && !a.col.use_2d;
        const int th = (int)threadIdx.x, tl = th >> 1;   // tile row / column th/2, blocks 2(th%2), 2(th%2)+1
        u32x6_t hw_codes[2][2];
        uint32_t hw_sc[2][2];
        if (row_hw) {
            // the lane's 8 rows x 8 columns into the row-major buffer
#pragma unroll
            for (int t = 0; t < 8; ++t)
                *reinterpret_cast<uint4 *>(&s_x[(r_loc0 + t) * kXPitch + 16 * c]) =
                    uint4{d[t][0], d[t][1], d[t][2], d[t][3]};
            __syncthreads();
            const uint32_t emax = a.row.fmt == 2u ? 2u : 4u;
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const uint8_t *src = &s_x[tl * kXPitch + 64 * (2 * (th & 1) + bb)];
                u32x16_t w;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint4 x4 = *reinterpret_cast<const uint4 *>(src + 16 * v);
                    w[4 * v] = x4.x; w[4 * v + 1] = x4.y; w[4 * v + 2] = x4.z; w[4 * v + 3] = x4.w;
                }
                hw_sc[0][bb] = fp6_block_hw(w, a.row.fmt, emax, hw_codes[0][bb]);
            }
        }
        if (col_hw) {
            // the lane's 8 columns x 8 rows into the buffer as columns (after
            // every gather of the row pass)
            if (row_hw) __syncthreads();
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int w = u >> 1, h = u & 1;
                *reinterpret_cast<uint4 *>(&s_x[(8 * c + u) * kXPitch + 2 * r_loc0]) =
                    uint4{pair_of(d[0][w], d[1][w], h), pair_of(d[2][w], d[3][w], h), pair_of(d[4][w], d[5][w], h),
                          pair_of(d[6][w], d[7][w], h)};
            }
            __syncthreads();
            const uint32_t emax = a.col.fmt == 2u ? 2u : 4u;
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const uint8_t *src = &s_x[tl * kXPitch + 64 * (2 * (th & 1) + bb)];
                u32x16_t wv;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint4 x4 = *reinterpret_cast<const uint4 *>(src + 16 * v);
                    wv[4 * v] = x4.x; wv[4 * v + 1] = x4.y; wv[4 * v + 2] = x4.z; wv[4 * v + 3] = x4.w;
                }
                hw_sc[1][bb] = fp6_block_hw(wv, a.col.fmt, emax, hw_codes[1][bb]);
            }
        }
        if (row_hw || col_hw) __syncthreads();
        if (row_hw) {
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const int b = 2 * (th & 1) + bb;
                lds_put24(&s_data[0][tl * kLinePitch + 24 * b], hw_codes[0][bb]);
                s_scale[0][tl * 4 + b] = (uint8_t)hw_sc[0][bb];
            }
        } else {
            const Fp6Dir f = fp6_dir(a.row.fmt);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int64_t i = row0 + 8 * q + t;
                const uint32_t sc = i < M ? scale_code_emax(a.row.use_2d ? tile_amax : ramax[t], f.emax) : 0u;
                uint32_t lo, hi;
                if constexpr (ROW_SR) {
                    const uint32_t nlo = ~rrow_lo[t], nhi = ~rrow_hi[t];
                    pack8_sr6([&](int e) { return elem_hi(d[t][e >> 1], e & 1); }, sc, f,
                              [&](int e) { return byte_to_b2(e < 4 ? nlo : nhi, e & 3); },
                              __builtin_amdgcn_perm(d[t][1], d[t][0], 0x0B0A0908u),
                              __builtin_amdgcn_perm(d[t][3], d[t][2], 0x0B0A0908u), lo, hi);
                } else {
                    uint32_t k6[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) k6[e] = code6((d[t][e >> 1] >> (16 * (e & 1))) & 0xFFFFu, sc, f);
                    pack6(k6, lo, hi);
                }
                lds_put6(s_data[0], (r_loc0 + t) * kLinePitch + 6 * c, lo, hi);
                if ((c & 3) == 0) s_scale[0][(r_loc0 + t) * 4 + c / 4] = (uint8_t)sc;
            }
        }
        if (DUAL) {
            col_amax();
            if (col_hw) {
#pragma unroll
                for (int bb = 0; bb < 2; ++bb) {
                    const int b = 2 * (th & 1) + bb;
                    lds_put24(&s_data[1][tl * kLinePitch + 24 * b], hw_codes[1][bb]);
                    s_scale[1][tl * 4 + b] = (uint8_t)hw_sc[1][bb];
                }
            } else {
                const Fp6Dir f = fp6_dir(a.col.fmt);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int64_t j = j0 + u;
                    const uint32_t sc = j < N ? scale_code_emax(a.col.use_2d ? tile_amax : camax[u], f.emax) : 0u;
                    uint32_t lo, hi;
                    const int w = u >> 1, h = u & 1;
                    if constexpr (COL_SR) {
                        // signs of rows 0..3 and 4..7 (bit 15 or 31 of each word, by selector)
                        const uint32_t sa = h ? 0x0C0C0B09u : 0x0C0C0A08u, sb = h ? 0x0B090C0Cu : 0x0A080C0Cu;
                        const uint32_t s0123 = __builtin_amdgcn_perm(d[1][w], d[0][w], sa) |
                                               __builtin_amdgcn_perm(d[3][w], d[2][w], sb);
                        const uint32_t s4567 = __builtin_amdgcn_perm(d[5][w], d[4][w], sa) |
                                               __builtin_amdgcn_perm(d[7][w], d[6][w], sb);
                        pack8_sr6([&](int t) { return elem_hi(d[t][w], h); }, sc, f,
                                  [&](int t) { return byte_to_b2(~(u < 4 ? rcol_lo[t] : rcol_hi[t]), u & 3); }, s0123,
                                  s4567, lo, hi);
                    } else {
                        uint32_t k6[8];
#pragma unroll
                        for (int t = 0; t < 8; ++t) k6[t] = code6((d[t][w] >> (16 * h)) & 0xFFFFu, sc, f);
                        pack6(k6, lo, hi);
                    }
                    // blob row = tile column 8c+u; this wave's 32 rows are bytes [24*wave, 24*wave+24)
                    lds_put6(s_data[1], (8 * c + u) * kLinePitch + 24 * wave + 6 * q, lo, hi);
                    if (q == 0) s_scale[1][(8 * c + u) * 4 + wave] = (uint8_t)sc;
                }
            }
        }
    }
    __syncthreads();

    // ---- write out: direction 0 = row-wise blob, 1 = column-wise blob
#pragma unroll
    for (int dir = 0; dir < (DUAL ? 2 : 1); ++dir) {
        const int64_t R = dir == 0 ? M : N;                      // blob rows
        const int64_t Lp = dir == 0 ? a.N_pad : a.M_pad;         // padded quantized axis
        const int64_t rbase = dir == 0 ? row0 - wave * kWaveRows : col0;   // first blob row of the tile
        const int64_t kbase = dir == 0 ? col0 : row0 - wave * kWaveRows;   // first element along the axis
        uint8_t *qd = dir == 0 ? a.q_row : a.q_col;
        uint8_t *sd = dir == 0 ? a.s_row : a.s_col;
        const int64_t rows_out = (LAYOUT == MX_LAYOUT_TILED) ? cdiv(R, 16) * 16 : R;
        if constexpr (ELEM == 6) {
            if (LAYOUT == MX_LAYOUT_TILED) {
                // 8 atoms of 16 blob rows: lane slot (r%16) + 16*b takes the block's bytes
                // 0..15 at 16*lane and 16..23 at 1024 + 8*lane of a 1536-byte atom
#pragma unroll
                for (int rep = 0; rep < 2; ++rep) {
                    const int slot = (int)threadIdx.x + 256 * rep;
                    const int lane = slot & 63;
                    const int r_loc = 16 * (slot >> 6) + (lane & 15);
                    const int64_t r = rbase + r_loc;
                    if (r < rows_out) {
                        const uint8_t *src = &s_data[dir][r_loc * kLinePitch + 24 * (lane >> 4)];
                        const uint2 v0 = *reinterpret_cast<const uint2 *>(src);
                        const uint2 v1 = *reinterpret_cast<const uint2 *>(src + 8);
                        const uint2 v2 = *reinterpret_cast<const uint2 *>(src + 16);
                        const int64_t atom = ((r / 16) * (Lp / 128) + kbase / 128) * 1536;
                        *reinterpret_cast<uint4 *>(qd + atom + 16 * lane) = uint4{v0.x, v0.y, v1.x, v1.y};
                        *reinterpret_cast<uint2 *>(qd + atom + 1024 + 8 * lane) = v2;
                    }
                }
            } else {
                // 128 blob rows x 96 bytes: six 16-byte chunks per row, consecutive threads along a row
#pragma unroll
                for (int rep = 0; rep < 3; ++rep) {
                    const int ch = (int)threadIdx.x + 256 * rep;
                    const int r_loc = ch / 6, part = ch % 6;
                    const int64_t r = rbase + r_loc;
                    if (r < rows_out) {
                        const uint4 v = *reinterpret_cast<const uint4 *>(&s_data[dir][r_loc * kLinePitch + 16 * part]);
                        *reinterpret_cast<uint4 *>(qd + r * (Lp * 3 / 4) + kbase * 3 / 4 + 16 * part) = v;
                    }
                }
            }
        } else
        // data: 512 slices of 16 bytes (one blob row, one 32-element block each)
#pragma unroll
        for (int rep = 0; rep < 2; ++rep) {
            const int ch = (int)threadIdx.x + 256 * rep;
            int r_loc, part;
            if (LAYOUT == MX_LAYOUT_TILED) {       // consecutive threads fill one 1 KB atom
                const int lt = ch & 63;
                r_loc = 16 * (ch >> 6) + (lt & 15);
                part = lt >> 4;
            } else {                                // consecutive threads fill one 64-byte row run
                r_loc = ch >> 2;
                part = ch & 3;
            }
            const int64_t r = rbase + r_loc;
            if (r < rows_out) {
                const uint4 v = *reinterpret_cast<const uint4 *>(&s_data[dir][r_loc * kLinePitch + 16 * part]);
                int64_t off;
                if (LAYOUT == MX_LAYOUT_TILED)
                    off = ((r / 16) * (Lp / 128) + kbase / 128) * 1024 + ((r % 16) + 16 * part) * 16;
                else
                    off = r * (Lp / 2) + kbase / 2 + 16 * part;
                *reinterpret_cast<uint4 *>(qd + off) = v;
            }
        }
        // scales: 4 bytes per blob row
        if (threadIdx.x < kTileRows) {
            const int r_loc = (int)threadIdx.x;
            const int64_t r = rbase + r_loc;
            if (r < rows_out) {
                const uint32_t s4 = *reinterpret_cast<const uint32_t *>(&s_scale[dir][r_loc * 4]);
                const int64_t kb0 = kbase / 32;
                if (LAYOUT == MX_LAYOUT_CANONICAL) {
                    *reinterpret_cast<uint32_t *>(sd + r * (Lp / 32) + kb0) = s4;
                } else {
                    const int64_t kgroups = cdiv(Lp, 512);
                    const int64_t satom = ((r / 16) * kgroups + kb0 / 16) * 256;
                    const int m = (int)((kb0 % 16) / 4);
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        sd[satom + 4 * ((r % 16) + 16 * b) + m] = (uint8_t)(s4 >> (8 * b));
                    // the last tile along the axis zeroes the scale bytes past L_pad/32
                    // blocks in its final scale atom
                    const int64_t nblk = Lp / 32;
                    if (kbase + kTileCols == Lp && nblk % 16 != 0) {
                        const int64_t zatom = ((r / 16) * kgroups + nblk / 16) * 256;
                        for (int64_t zb = nblk; zb < (nblk / 16 + 1) * 16; ++zb)
                            sd[zatom + 4 * ((r % 16) + 16 * (zb % 4)) + (zb % 16) / 4] = 0;
                    }
                }
            }
        }
    }
}

}  // namespace

// One launch per kMaxRowTiles row tiles (grid y is limited; each launch
// passes its first row tile in the arguments), the same kernel for all.
template <typename L>
hipError_t launch_row_chunks(const QuantArgs &a, L launch) {
    const int64_t row_tiles = cdiv(a.M, kTileRows);
    for (int64_t t0 = 0; t0 < row_tiles; t0 += kMaxRowTiles) {
        QuantArgs b = a;
        b.row_tile0 = t0;
        const int64_t n = row_tiles - t0 < kMaxRowTiles ? row_tiles - t0 : kMaxRowTiles;
        const hipError_t e = launch(b, dim3((unsigned)cdiv(a.N, kTileCols), (unsigned)n));
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int ELEM, int LAYOUT, bool DUAL, bool RHT>
hipError_t launch_sr(const QuantArgs &a, dim3 grid, hipStream_t stream) {
    const bool rs = a.row.use_sr != 0, cs = DUAL && a.col.use_sr != 0;
    if (rs && cs) hipLaunchKernelGGL((quantize_kernel<ELEM, LAYOUT, DUAL, true, true, RHT>), grid, dim3(256), 0, stream, a);
    else if (rs) hipLaunchKernelGGL((quantize_kernel<ELEM, LAYOUT, DUAL, true, false, RHT>), grid, dim3(256), 0, stream, a);
    else if (cs) hipLaunchKernelGGL((quantize_kernel<ELEM, LAYOUT, DUAL, false, true, RHT>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((quantize_kernel<ELEM, LAYOUT, DUAL, false, false, RHT>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int LAYOUT, bool DUAL>
hipError_t launch_rht(const QuantArgs &a, dim3 grid, hipStream_t stream) {
    return (a.row.rht || (DUAL && a.col.rht)) ? launch_sr<4, LAYOUT, DUAL, true>(a, grid, stream)
                                              : launch_sr<4, LAYOUT, DUAL, false>(a, grid, stream);
}

hipError_t launch_quantize(const QuantArgs &a, bool dual, mx_layout layout, hipStream_t stream) {
    return launch_row_chunks(a, [&](const QuantArgs &b, dim3 grid) {
        if (layout == MX_LAYOUT_CANONICAL)
            return dual ? launch_rht<MX_LAYOUT_CANONICAL, true>(b, grid, stream)
                        : launch_rht<MX_LAYOUT_CANONICAL, false>(b, grid, stream);
        return dual ? launch_rht<MX_LAYOUT_TILED, true>(b, grid, stream)
                    : launch_rht<MX_LAYOUT_TILED, false>(b, grid, stream);
    });
}

template <int LAYOUT, bool DUAL>
hipError_t launch_mul(const QuantArgs &a, dim3 grid, hipStream_t stream) {
    const bool rs = a.row.use_sr != 0, cs = DUAL && a.col.use_sr != 0;
    if (rs && cs) hipLaunchKernelGGL((quantize_kernel<4, LAYOUT, DUAL, true, true, false, true>), grid, dim3(256), 0, stream, a);
    else if (rs) hipLaunchKernelGGL((quantize_kernel<4, LAYOUT, DUAL, true, false, false, true>), grid, dim3(256), 0, stream, a);
    else if (cs) hipLaunchKernelGGL((quantize_kernel<4, LAYOUT, DUAL, false, true, false, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((quantize_kernel<4, LAYOUT, DUAL, false, false, false, true>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_quantize_mul(const QuantArgs &a, bool dual, mx_layout layout, hipStream_t stream) {
    return launch_row_chunks(a, [&](const QuantArgs &b, dim3 grid) {
        if (layout == MX_LAYOUT_CANONICAL)
            return dual ? launch_mul<MX_LAYOUT_CANONICAL, true>(b, grid, stream)
                        : launch_mul<MX_LAYOUT_CANONICAL, false>(b, grid, stream);
        return dual ? launch_mul<MX_LAYOUT_TILED, true>(b, grid, stream)
                    : launch_mul<MX_LAYOUT_TILED, false>(b, grid, stream);
    });
}

hipError_t launch_quantize_fp6(const QuantArgs &a, bool dual, mx_layout layout, hipStream_t stream) {
    return launch_row_chunks(a, [&](const QuantArgs &b, dim3 grid) {
        if (layout == MX_LAYOUT_CANONICAL)
            return dual ? launch_sr<6, MX_LAYOUT_CANONICAL, true, false>(b, grid, stream)
                        : launch_sr<6, MX_LAYOUT_CANONICAL, false, false>(b, grid, stream);
        return dual ? launch_sr<6, MX_LAYOUT_TILED, true, false>(b, grid, stream)
                    : launch_sr<6, MX_LAYOUT_TILED, false, false>(b, grid, stream);
    });
}

}  // namespace mx
