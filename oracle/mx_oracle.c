/*
 * mx_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU definition of what the MXFP4 hot path computes.
 * It exists to check the HIP library against; nothing in the product links,
 * imports or calls it.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, tables or headers with the
 * GPU path.
 *
 * Sources it follows (cited per function below):
 *   [OCP-MX]  OCP Microscaling Formats (MX) Specification v1.0:
 *             sec. 5 (E2M1 element and E8M0 scale encodings),
 *             sec. 6.3 (conversion: shared exponent = floor(log2 amax) - emax_elem,
 *             emax_elem = 2 for FP4 E2M1; elements rounded, clamped to +-6).
 *   [P3]      page "primus_turbo_mxfp4_local.py" (ROCm docs download):
 *             block size 32, padding of the quantized axis to 128, the blob
 *             shapes of the fake (shape-only) dual-quantize op, the row/col
 *             flag triplets (2D block, stochastic rounding), and the GEMM
 *             dataflow of the autograd Function (fwd, dgrad, wgrad: all NT).
 *   [PHILOX]  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
 *             as 1, 2, 3", SC'11, sec. 4.2 (Philox-4x32, 10 rounds).
 *   [FP8]     OCP 8-bit Floating Point Specification (OFP8) v1.0, E5M2:
 *             bias 15, 2 mantissa bits, subnormals, Inf and NaN encodings,
 *             largest finite value 57344.  The same page's hybrid backward
 *             re-quantizes the saved bf16 tensors "tensorwise" to E5M2
 *             (one scale per tensor, returned as its inverse) and calls an
 *             FP8 GEMM that multiplies by both inverse scales; the scale
 *             rule itself is not on the pages (reading below).
 *   [OCP-MX] sec. 5.3.2 also defines the FP6 element formats (E2M3, E3M2)
 *             used by the MXFP6 section at the end of this file; the pages
 *             only name an MXFP6 training campaign (Primus PR 1107).
 *   [RHT]     the same page's dual-quantize calls, which switch on a random
 *             Hadamard transform ("rht") for the column-wise blobs of the
 *             activation and of the gradient -- the two operands of wgrad --
 *             and say nothing more about it.  The reading taken here: within
 *             each 32-element block along the quantized axis, y = c * H32 * D * x,
 *             H32 the 32x32 Sylvester Hadamard matrix, D = diag(+-1) a fixed
 *             sign pattern drawn from a seed, c = 1/sqrt(32) rounded to fp32,
 *             evaluated in fp32 as a fast Walsh-Hadamard transform (stages
 *             over index bits 0..4); both wgrad operands use the same D, so
 *             (H D)^T (H D) = 32 I and c^2 * 32 ~ 1 leave the product unchanged.
 *
 * Readings where the pages are silent are listed in the design notes; the
 * ones that shape this file: sign of zero is copied from x; an all-zero or
 * pad-only block gets scale byte 0; a block holding Inf/NaN gets scale byte
 * 0xFF and all-zero nibbles; element 2j sits in the low nibble of byte j;
 * a 2D block is the aligned 32x32 tile whose scale is replicated into every
 * row's block slot; stochastic rounding uses one Philox byte per element.
 *
 * Every value here is computed in fp64 (exact for all the quantizer's
 * arithmetic: bf16 inputs times powers of two), except the random Hadamard
 * transform, which is defined in fp32 (the precision the reading fixes).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define MX_BLOCK 32
#define MX_PAD 128

static int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* bf16 bit pattern -> exact double. */
static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int bf16_is_finite(uint16_t b) { return ((b >> 7) & 0xFF) != 0xFF; }

uint16_t oracle_bf16_from_double(double d);

/* [OCP-MX] sec. 5.3.3: FP4 E2M1 magnitudes of the 3-bit codes 0..7. */
static const double E2M1_MAGNITUDE[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/*
 * [OCP-MX] sec. 6.3: shared exponent of a block.
 * e = floor(log2(amax)) - 2, clamped to the E8M0 range [-127, 127];
 * amax == 0 gives the smallest scale (e = -127).
 */
static int shared_exponent(double amax)
{
    if (amax == 0.0) return -127;
    int ex;
    (void)frexp(amax, &ex);   /* amax = m * 2^ex, 0.5 <= m < 1, so floor(log2 amax) = ex - 1 */
    int e = (ex - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/*
 * Round-to-nearest-even of a scaled magnitude v = |x| * 2^-e onto the E2M1
 * grid {0, .5, 1, 1.5, 2, 3, 4, 6}; anything above 5 goes to 6 (saturation,
 * never NaN).  Each boundary is the midpoint of two neighbours; at a tie the
 * neighbour with the even code wins (codes 0, 2, 4, 6).
 */
static int rne_code(double v)
{
    if (v <= 0.25) return 0;   /* tie 0.25 -> 0   (code 0 even) */
    if (v < 0.75) return 1;    /* tie 0.75 -> 1.0 (code 2 even) */
    if (v <= 1.25) return 2;   /* tie 1.25 -> 1.0 */
    if (v < 1.75) return 3;    /* tie 1.75 -> 2.0 (code 4) */
    if (v <= 2.5) return 4;    /* tie 2.5  -> 2.0 */
    if (v < 3.5) return 5;     /* tie 3.5  -> 4.0 (code 6) */
    if (v <= 5.0) return 6;    /* tie 5.0  -> 4.0 */
    return 7;                  /* (5, inf) -> 6, saturating */
}

/*
 * Stochastic rounding of v onto the E2M1 grid with one random byte r:
 * lo <= v < hi are the neighbouring grid magnitudes; t = floor(256 (v-lo)/(hi-lo));
 * round up iff r < t.  Grid points (t = 0) never move; v >= 6 gives 6.
 */
static int sr_code(double v, unsigned r)
{
    if (v >= 6.0) return 7;
    int lo = 0;
    while (lo < 7 && E2M1_MAGNITUDE[lo + 1] <= v) lo++;
    double frac = (v - E2M1_MAGNITUDE[lo]) / (E2M1_MAGNITUDE[lo + 1] - E2M1_MAGNITUDE[lo]);
    unsigned t = (unsigned)floor(256.0 * frac);
    return (r < t) ? lo + 1 : lo;
}

/* ---------------------------------------------------------------- Philox */

/* [PHILOX] sec. 4.2: Philox-4x32 round constants. */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

/* Philox-4x32-10: 10 rounds of the S-box/P-box network, key bumped by the
 * Weyl constants between rounds. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/*
 * The random byte of logical element n (row-major index into the unpadded
 * M x N tensor, plus the caller's index_base) for one direction:
 * counter = (lo32(n>>4), hi32(n>>4), tensor_id, dir), key = (lo32(seed), hi32(seed)),
 * byte n%16 of the four output words taken little-endian.  (Pad positions,
 * which carry values only after a Hadamard transform, pass dir + 2.)
 */
unsigned oracle_sr_byte(uint64_t seed, uint32_t tensor_id, uint32_t dir, uint64_t n)
{
    uint64_t g = n >> 4;
    uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), tensor_id, dir};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oracle_philox4x32_10(ctr, key, w);
    unsigned idx = (unsigned)(n & 15);
    return (w[idx / 4] >> (8 * (idx % 4))) & 0xFFu;
}

/* ------------------------------------------------------------------- RHT */

/* [RHT] the sign pattern D of seed `rht`: bit p of the first output word of
 * Philox-4x32-10 at counter (0, 0, 0, 2), key (rht, 0); bit set = negate the
 * element at block position p. */
uint32_t oracle_rht_signs(uint32_t rht)
{
    uint32_t ctr[4] = {0, 0, 0, 2};
    uint32_t key[2] = {rht, 0};
    uint32_t w[4];
    oracle_philox4x32_10(ctr, key, w);
    return w[0];
}

/* [RHT] c = the fp32 number nearest to 1/sqrt(32). */
#define RHT_SCALE_BITS 0x3E3504F3u

/*
 * [RHT] one 32-element block: u = D x; then for stage k = 0..4, every pair
 * (i, i + 2^k) with bit k of i clear becomes (u_i + u_(i+2^k), u_i - u_(i+2^k)),
 * each sum rounded to fp32; finally each entry times c in fp32.  The stages
 * build H32 u with H32[j][i] = (-1)^popcount(i & j).
 */
void oracle_rht32(const float in[32], uint32_t signs, float out[32])
{
    float u[32];
    float c;
    uint32_t cb = RHT_SCALE_BITS;
    memcpy(&c, &cb, sizeof c);
    for (int p = 0; p < 32; ++p) u[p] = ((signs >> p) & 1u) ? -in[p] : in[p];
    for (int k = 0; k < 5; ++k) {
        int h = 1 << k;
        for (int i = 0; i < 32; ++i) {
            if (i & h) continue;
            float a = u[i], b = u[i + h];
            u[i] = a + b;
            u[i + h] = a - b;
        }
    }
    for (int p = 0; p < 32; ++p) out[p] = u[p] * c;
}

/* -------------------------------------------------------------- quantize */

/*
 * Quantize one direction of an M x N bf16 tensor x (row stride ldx elements)
 * into the canonical blob layout of [P3] (fake dual-quantize op):
 *   dir 0 (row-wise): blocks run along N;  q is M x N_pad/2 bytes, s is M x N_pad/32.
 *   dir 1 (col-wise): blocks run along M;  q is N x M_pad/2 bytes, s is N x M_pad/32
 *                     (the transpose, quantized along M).
 * The quantized axis L (N or M) is padded with +0 to L_pad = cdiv(L,128)*128.
 * use_2d: the block is the aligned 32x32 tile of x; its scale is written into
 * every blob row slot the tile covers.
 * use_sr: stochastic rounding with the byte oracle_sr_byte(seed, tensor_id, dir, n).
 * rht != 0: each 32-element block along the quantized axis (pads included, as
 * +0) is replaced by its random Hadamard transform with signs
 * oracle_rht_signs(rht) before the scale and the codes are taken; the pad
 * positions of a block that holds real elements then carry codes too, and
 * their stochastic-rounding byte uses the same index formula (n = index_base
 * + i N + j with the padded coordinates).  Not combined with use_2d.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_quantize(const uint16_t *x, int64_t M, int64_t N, int64_t ldx, int dir,
                    int use_2d, int use_sr, uint64_t seed, uint32_t tensor_id,
                    uint64_t index_base, uint32_t rht, uint8_t *q, uint8_t *s)
{
    if (M < 0 || N < 0 || ldx < N || (dir != 0 && dir != 1)) return -1;
    if (rht && use_2d) return -1;
    const uint32_t rht_signs = rht ? oracle_rht_signs(rht) : 0u;
    const int64_t R = dir == 0 ? M : N;        /* blob rows */
    const int64_t L = dir == 0 ? N : M;        /* quantized axis */
    const int64_t L_pad = cdiv64(L, MX_PAD) * MX_PAD;
    const int64_t nblk = L_pad / MX_BLOCK;

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t b = 0; b < nblk; ++b) {
            /* The set of x elements whose amax fixes this block's scale:
             * 1D: this blob row's 32 elements; 2D: the whole aligned 32x32 tile. */
            int64_t i0, i1, j0, j1;  /* x rows [i0,i1), x cols [j0,j1) */
            if (dir == 0) {
                i0 = use_2d ? (r / 32) * 32 : r;
                i1 = use_2d ? i0 + 32 : r + 1;
                j0 = b * MX_BLOCK;
                j1 = j0 + MX_BLOCK;
            } else {
                i0 = b * MX_BLOCK;
                i1 = i0 + MX_BLOCK;
                j0 = use_2d ? (r / 32) * 32 : r;
                j1 = use_2d ? j0 + 32 : r + 1;
            }
            if (i1 > M) i1 = M;
            if (j1 > N) j1 = N;
            if (rht) {
                /* the block's 32 positions along the axis, pads as +0, transformed */
                float xin[32], y[32];
                for (int64_t t = 0; t < MX_BLOCK; ++t) {
                    int64_t k = b * MX_BLOCK + t;
                    xin[t] = 0.0f;
                    if (k < L) {
                        uint16_t bits = dir == 0 ? x[r * ldx + k] : x[k * ldx + r];
                        xin[t] = (float)bf16_value(bits);
                    }
                }
                oracle_rht32(xin, rht_signs, y);
                double amax = 0.0;
                int nonfinite = 0;
                for (int t = 0; t < MX_BLOCK; ++t) {
                    if (!isfinite(y[t])) nonfinite = 1;
                    else if (fabs((double)y[t]) > amax) amax = fabs((double)y[t]);
                }
                int e = shared_exponent(amax);
                s[r * nblk + b] = nonfinite ? 0xFF : (uint8_t)(e + 127);
                for (int64_t t = 0; t < MX_BLOCK; ++t) {
                    int64_t k = b * MX_BLOCK + t;
                    unsigned nibble = 0;
                    if (!nonfinite) {
                        double v = ldexp(fabs((double)y[t]), -e);   /* exact */
                        int code;
                        if (use_sr) {
                            int64_t i = dir == 0 ? r : k;
                            int64_t j = dir == 0 ? k : r;
                            uint64_t n = index_base + (uint64_t)i * (uint64_t)N + (uint64_t)j;
                            /* pad positions (k >= L) draw from their own counter space,
                             * counter word 3 = 2 + dir, so they never share a byte with a
                             * real element */
                            uint32_t word3 = (uint32_t)dir + (k >= L ? 2u : 0u);
                            code = sr_code(v, oracle_sr_byte(seed, tensor_id, word3, n));
                        } else {
                            code = rne_code(v);
                        }
                        nibble = (signbit(y[t]) ? 8u : 0u) | (unsigned)code;
                    }
                    uint8_t *byte = &q[r * (L_pad / 2) + k / 2];
                    if (k % 2 == 0) *byte = (uint8_t)nibble;
                    else *byte = (uint8_t)(*byte | (nibble << 4));
                }
                continue;
            }
            double amax = 0.0;
            int nonfinite = 0;
            for (int64_t i = i0; i < i1; ++i)
                for (int64_t j = j0; j < j1; ++j) {
                    uint16_t bits = x[i * ldx + j];
                    if (!bf16_is_finite(bits)) nonfinite = 1;
                    else {
                        double a = fabs(bf16_value(bits));
                        if (a > amax) amax = a;
                    }
                }
            int e = shared_exponent(amax);
            uint8_t scale_byte = nonfinite ? 0xFF : (uint8_t)(e + 127);
            s[r * nblk + b] = scale_byte;

            for (int64_t t = 0; t < MX_BLOCK; ++t) {
                int64_t k = b * MX_BLOCK + t;      /* position along the quantized axis */
                unsigned nibble = 0;
                if (k < L && !nonfinite) {
                    int64_t i = dir == 0 ? r : k;  /* coordinates in x */
                    int64_t j = dir == 0 ? k : r;
                    uint16_t bits = x[i * ldx + j];
                    double v = ldexp(fabs(bf16_value(bits)), -e);   /* exact */
                    int code;
                    if (use_sr) {
                        uint64_t n = index_base + (uint64_t)i * (uint64_t)N + (uint64_t)j;
                        code = sr_code(v, oracle_sr_byte(seed, tensor_id, (uint32_t)dir, n));
                    } else {
                        code = rne_code(v);
                    }
                    nibble = ((unsigned)(bits >> 15) << 3) | (unsigned)code;
                }
                uint8_t *byte = &q[r * (L_pad / 2) + k / 2];
                if (k % 2 == 0) *byte = (uint8_t)nibble;
                else *byte = (uint8_t)(*byte | (nibble << 4));
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------ dequantize */

/* Exact value of one element of a canonical blob: (-1)^s * mag(code) * 2^(byte-127);
 * scale byte 0xFF (E8M0 NaN) gives NaN. */
static double element_value(const uint8_t *q, const uint8_t *s, int64_t L_pad, int64_t r, int64_t k)
{
    uint8_t sb = s[r * (L_pad / MX_BLOCK) + k / MX_BLOCK];
    if (sb == 0xFF) return NAN;
    uint8_t byte = q[r * (L_pad / 2) + k / 2];
    unsigned nibble = (k % 2 == 0) ? (byte & 0xFu) : (byte >> 4);
    double mag = E2M1_MAGNITUDE[nibble & 7u];
    double v = ldexp(mag, (int)sb - 127);
    return (nibble & 8u) ? -v : v;
}

/* Dequantize a canonical blob of R rows x L logical columns into out (R x L_pad, fp64). */
int oracle_dequantize(const uint8_t *q, const uint8_t *s, int64_t R, int64_t L, double *out)
{
    if (R < 0 || L < 0) return -1;
    const int64_t L_pad = cdiv64(L, MX_PAD) * MX_PAD;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < L_pad; ++k)
            out[r * L_pad + k] = element_value(q, s, L_pad, r, k);
    return 0;
}

/* ------------------------------------------------------------------ GEMM */

/*
 * The block-scaled NT product of [P3] (fwd, dgrad and wgrad all call the FP4
 * GEMM with A untransposed and B transposed, both K-contiguous):
 *   C[i][j] = sum_{k < K_pad} deqA[i][k] * deqB[j][k], summed in fp64 in k order.
 * A and B are canonical blobs (M and N rows, K logical columns).
 * Computes the listed entries (ii[t], jj[t]) into out[t].
 */
int oracle_gemm_entries(const uint8_t *qa, const uint8_t *sa, const uint8_t *qb, const uint8_t *sb,
                        int64_t M, int64_t N, int64_t K, int64_t count,
                        const int64_t *ii, const int64_t *jj, double *out)
{
    if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
    const int64_t K_pad = cdiv64(K, MX_PAD) * MX_PAD;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        int64_t i = ii[t], j = jj[t];
        double acc = 0.0;
        if (i >= 0 && i < M && j >= 0 && j < N)
            for (int64_t k = 0; k < K_pad; ++k)
                acc += element_value(qa, sa, K_pad, i, k) * element_value(qb, sb, K_pad, j, k);
        else
            acc = NAN;
        out[t] = acc;
    }
    return 0;
}

/* Rows [i0, i1) of C (all N columns) into out ((i1-i0) x N, fp64), same definition. */
int oracle_gemm_rows(const uint8_t *qa, const uint8_t *sa, const uint8_t *qb, const uint8_t *sb,
                     int64_t M, int64_t N, int64_t K, int64_t i0, int64_t i1, double *out)
{
    if (M < 0 || N < 0 || K < 0 || i0 < 0 || i1 > M || i0 > i1) return -1;
    const int64_t K_pad = cdiv64(K, MX_PAD) * MX_PAD;
#pragma omp parallel for schedule(static)
    for (int64_t i = i0; i < i1; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            for (int64_t k = 0; k < K_pad; ++k)
                acc += element_value(qa, sa, K_pad, i, k) * element_value(qb, sb, K_pad, j, k);
            out[(i - i0) * N + j] = acc;
        }
    return 0;
}

/* ------------------------------------------------- FP8 E5M2, tensorwise */

#define E5M2_MAX 57344.0

/* [FP8] value of an E5M2 code. */
double oracle_e5m2_value(uint8_t c)
{
    int sign = c >> 7, e = (c >> 2) & 31, m = c & 3;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -16);            /* subnormal: m/4 * 2^-14 */
    else v = ldexp(1.0 + m / 4.0, e - 15);
    return sign ? -v : v;
}

/*
 * [FP8] E5M2 code of v: round to nearest, ties to the even code; finite
 * values beyond 57344 saturate to 57344 (the reading of a saturating cast);
 * +-Inf stays +-Inf; NaN becomes 0x7F with v's sign.
 */
uint8_t oracle_e5m2_from_double(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    double a = fabs(v);
    if (isinf(a)) return (uint8_t)(sign | 0x7C);
    if (a == 0.0) return sign;
    int ex;
    (void)frexp(a, &ex);                 /* a in [2^(ex-1), 2^ex) */
    int unit_exp = (ex - 1) - 2;         /* spacing of 3-significant-bit numbers in this binade */
    if (unit_exp < -16) unit_exp = -16;  /* subnormal spacing 2^-16 */
    double units = ldexp(a, -unit_exp);
    double fl = floor(units), rem = units - fl;
    double n = fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
    double r = ldexp(n, unit_exp);
    if (r > E5M2_MAX) r = E5M2_MAX;
    /* encode the (now representable) magnitude r */
    if (r == 0.0) return sign;
    int rex;
    (void)frexp(r, &rex);
    int e = rex - 1 + 15;                /* biased exponent */
    uint8_t code;
    if (e <= 0) code = (uint8_t)ldexp(r, 16);                      /* subnormal: m = r / 2^-16 */
    else code = (uint8_t)((e << 2) | (int)(ldexp(r, -(rex - 1)) * 4.0 - 4.0));
    return (uint8_t)(sign | code);
}

/*
 * Tensorwise E5M2 quantization of an M x N bf16 tensor (reading of [P3]'s
 * `_quantize_fp8_tw`, whose body is not on the pages):
 *   amax  = max |x| over the tensor (any NaN or Inf: amax is that, not finite)
 *   scale = 57344 / amax as an fp32 division when amax is finite and > 0, else 1
 *   code  = E5M2 of fp32(x * scale)  (the fp32 product is rounded first)
 *   scale_inv = fp32(1 / scale)
 * dir 0 writes the M x N_pad row blob, dir 1 the N x M_pad column blob (the
 * transpose), padding +0 (code 0), row-major bytes.  Returns 0 or -1.
 */
int oracle_quantize_fp8_tw(const uint16_t *x, int64_t M, int64_t N, int64_t ldx, int dir,
                           uint8_t *q, float *scale_inv_out, float *amax_out)
{
    if (M < 0 || N < 0 || ldx < N || (dir != 0 && dir != 1)) return -1;
    double amax = 0.0;
    int nonfinite = 0;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            uint16_t b = x[i * ldx + j];
            if (!bf16_is_finite(b)) nonfinite = 1;
            else if (fabs(bf16_value(b)) > amax) amax = fabs(bf16_value(b));
        }
    /* fp32 arithmetic (correctly rounded float division; amax is a bf16 value, exact in fp32) */
    volatile float famax = (float)amax;
    float scale = 1.0f;
    if (!nonfinite && amax > 0.0) scale = 57344.0f / famax;
    if (scale_inv_out) *scale_inv_out = 1.0f / scale;
    if (amax_out) *amax_out = nonfinite ? INFINITY : (float)amax;
    const int64_t R = dir == 0 ? M : N, L = dir == 0 ? N : M;
    const int64_t L_pad = cdiv64(L, MX_PAD) * MX_PAD;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < L_pad; ++k) {
            uint8_t code = 0;
            if (k < L) {
                uint16_t b = dir == 0 ? x[r * ldx + k] : x[k * ldx + r];
                float v = (float)bf16_value(b) * scale;             /* fp32 product */
                code = oracle_e5m2_from_double((double)v);
            }
            q[r * L_pad + k] = code;
        }
    return 0;
}

/*
 * The FP8 GEMM of the hybrid backward (NT form, both operands K-contiguous):
 *   C[i][j] = (sum_{k < K_pad} e5m2(A[i][k]) * e5m2(B[j][k])) * sa_inv * sb_inv   in fp64.
 */
int oracle_gemm_fp8_entries(const uint8_t *qa, float sa_inv, const uint8_t *qb, float sb_inv,
                            int64_t M, int64_t N, int64_t K, int64_t count,
                            const int64_t *ii, const int64_t *jj, double *out)
{
    if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
    const int64_t K_pad = cdiv64(K, MX_PAD) * MX_PAD;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        int64_t i = ii[t], j = jj[t];
        double acc = 0.0;
        if (i >= 0 && i < M && j >= 0 && j < N)
            for (int64_t k = 0; k < K_pad; ++k)
                acc += oracle_e5m2_value(qa[i * K_pad + k]) * oracle_e5m2_value(qb[j * K_pad + k]);
        else
            acc = NAN;
        out[t] = acc * (double)sa_inv * (double)sb_inv;
    }
    return 0;
}

/*
 * FP8 tiled layout: row groups of 16, k-steps of 64; atom (g, s) is 1 KB at
 * (g * L_pad/64 + s) * 1024; lane = (r%16) + 16*((k%64)/16) owns bytes
 * [16 lane, 16 lane + 16), element k at byte k%16.  Pad rows are zero.
 */
int oracle_fp8_to_tiled(const uint8_t *q, int64_t R, int64_t L, uint8_t *qt)
{
    if (R < 0 || L < 0) return -1;
    const int64_t L_pad = cdiv64(L, MX_PAD) * MX_PAD;
    const int64_t R16 = cdiv64(R, 16) * 16;
    memset(qt, 0, (size_t)(R16 * L_pad));
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < L_pad; ++k) {
            int64_t lane = (r % 16) + 16 * ((k % 64) / 16);
            qt[((r / 16) * (L_pad / 64) + k / 64) * 1024 + 16 * lane + k % 16] = q[r * L_pad + k];
        }
    return 0;
}

/* ----------------------------------------------------------- bf16 cast */

/*
 * Correctly rounded fp64 -> bf16 (round to nearest, ties to even mantissa),
 * done in one rounding step (no detour through fp32).  Overflow gives +-Inf,
 * NaN gives the canonical quiet NaN 0x7FC0 with the sign of the input.
 */
uint16_t oracle_bf16_from_double(double d)
{
    uint16_t sign = signbit(d) ? 0x8000 : 0;
    if (isnan(d)) return (uint16_t)(sign | 0x7FC0);
    double a = fabs(d);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    if (a == 0.0) return sign;
    int ex;
    (void)frexp(a, &ex);             /* a in [2^(ex-1), 2^ex) */
    int unit_exp = (ex - 1) - 7;     /* spacing of 8-significant-bit numbers in this binade */
    if (unit_exp < -133) unit_exp = -133;   /* bf16 subnormal spacing */
    double units = ldexp(a, -unit_exp);     /* exact: a power-of-two rescale */
    double fl = floor(units);
    double rem = units - fl;
    double n = fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
    double rounded = ldexp(n, unit_exp);
    if (rounded >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);
    float f = (float)rounded;        /* exact: rounded has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFF));
}

void oracle_bf16_from_double_array(const double *in, int64_t n, uint16_t *out)
{
    for (int64_t t = 0; t < n; ++t) out[t] = oracle_bf16_from_double(in[t]);
}

/* --------------------------------------------------------- tiled layout */

/*
 * The library's MFMA-native "tiled" blob layout, written out from its
 * definition (the product's own converter is separate code):
 *   rows are padded to R16 = cdiv(R,16)*16 with zero bytes.
 *   data atom (row group g = r/16, k step c = k/128) is 1024 bytes at
 *     offset (g * (L_pad/128) + c) * 1024;
 *     inside it, lane = (r%16) + 16*((k%128)/32) owns bytes [16*lane, 16*lane+16),
 *     element k sits in byte (k%32)/2, low nibble for even k.
 *   scale atom (row group g, k group h = k/512) is 256 bytes at
 *     offset (g * cdiv(L_pad,512) + h) * 256;
 *     inside it, block kb = k/32 of row r is byte 4*lane + (kb%16)/4 with
 *     lane = (r%16) + 16*(kb%4); bytes past L_pad/32 blocks stay zero.
 */
int oracle_to_tiled(const uint8_t *q, const uint8_t *s, int64_t R, int64_t L,
                    uint8_t *qt, uint8_t *st)
{
    if (R < 0 || L < 0) return -1;
    const int64_t L_pad = cdiv64(L, MX_PAD) * MX_PAD;
    const int64_t R16 = cdiv64(R, 16) * 16;
    const int64_t ksteps = L_pad / 128;
    const int64_t kgroups = cdiv64(L_pad, 512);
    memset(qt, 0, (size_t)(R16 * L_pad / 2));
    memset(st, 0, (size_t)(R16 * kgroups * 16));
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t k = 0; k < L_pad; ++k) {
            uint8_t byte = q[r * (L_pad / 2) + k / 2];
            unsigned nibble = (k % 2 == 0) ? (byte & 0xFu) : (byte >> 4);
            int64_t lane = (r % 16) + 16 * ((k % 128) / 32);
            int64_t off = ((r / 16) * ksteps + k / 128) * 1024 + 16 * lane + (k % 32) / 2;
            if (k % 2 == 0) qt[off] = (uint8_t)((qt[off] & 0xF0u) | nibble);
            else qt[off] = (uint8_t)((qt[off] & 0x0Fu) | (nibble << 4));
        }
        for (int64_t kb = 0; kb < L_pad / 32; ++kb) {
            int64_t lane = (r % 16) + 16 * (kb % 4);
            int64_t off = ((r / 16) * kgroups + kb / 16) * 256 + 4 * lane + (kb % 16) / 4;
            st[off] = s[r * (L_pad / 32) + kb];
        }
    }
    return 0;
}

/* ----------------------------------------------------------------- MXFP6 */
/*
 * [OCP-MX] sec. 5.3.2: the two 6-bit element formats, numbered like the
 * format codes of the f8f6f4 matrix instructions: fmt 2 = FP6 E2M3 (2
 * exponent bits, bias 1, 3 mantissa bits), fmt 3 = FP6 E3M2 (3 exponent
 * bits, bias 3, 2 mantissa bits).  Sign in bit 5; no Inf or NaN codes;
 * exponent field 0 holds the subnormals m * 2^(1-bias-mbits).  The pages
 * name an MXFP6 training campaign and define none of it; the element
 * formats, the scale rule (sec. 6.3 with emax_elem = 2 for E2M3, whose
 * largest normal is 1.875 * 2^2, and 4 for E3M2, 1.75 * 2^4), and the
 * rounding rules (as for MXFP4) are this reading's.
 *
 * Canonical FP6 blob: data R x L_pad*3/4 bytes; element k of a row occupies
 * bits [6k, 6k+6) of the row read as a little-endian bit string (byte
 * 6k/8, from bit 6k%8 up, spilling into the next byte); scales exactly as
 * for MXFP4 (R x L_pad/32, byte b scales elements [32b, 32b+32)).
 */
static int fp6_params(int fmt, int *ebits, int *mbits, int *bias, int *emax)
{
    if (fmt == 2) { *ebits = 2; *mbits = 3; *bias = 1; *emax = 2; return 0; }
    if (fmt == 3) { *ebits = 3; *mbits = 2; *bias = 3; *emax = 4; return 0; }
    return -1;
}

/* [OCP-MX] sec. 5.3.2: value of a 6-bit code (NaN for an unknown format). */
double oracle_fp6_value(unsigned code, int fmt)
{
    int ebits, mbits, bias, emax;
    if (fp6_params(fmt, &ebits, &mbits, &bias, &emax) != 0) return NAN;
    unsigned m = code & ((1u << mbits) - 1u);
    unsigned e = (code >> mbits) & ((1u << ebits) - 1u);
    double mag = e == 0 ? ldexp((double)m, 1 - bias - mbits)
                        : ldexp(1.0 + ldexp((double)m, -mbits), (int)e - bias);
    return ((code >> 5) & 1u) ? -mag : mag;
}

/* The 32 non-negative magnitudes of a format, in code order (increasing). */
static void fp6_grid(int fmt, double mag[32])
{
    for (unsigned c = 0; c < 32; ++c) mag[c] = oracle_fp6_value(c, fmt);
}

/* Round to nearest on the grid, ties to the even code; above the largest
 * magnitude saturate to it (code 31). */
static int fp6_rne(double v, const double mag[32])
{
    if (v >= mag[31]) return 31;
    int lo = 0;
    while (mag[lo + 1] <= v) lo++;
    double dlo = v - mag[lo], dhi = mag[lo + 1] - v;
    if (dlo < dhi) return lo;
    if (dhi < dlo) return lo + 1;
    return (lo % 2 == 0) ? lo : lo + 1;
}

/* Stochastic rounding with one random byte r, the MXFP4 rule on this grid:
 * t = floor(256 (v-lo)/(hi-lo)), round up iff r < t; v >= max gives max. */
static int fp6_sr(double v, unsigned r, const double mag[32])
{
    if (v >= mag[31]) return 31;
    int lo = 0;
    while (mag[lo + 1] <= v) lo++;
    double frac = (v - mag[lo]) / (mag[lo + 1] - mag[lo]);
    unsigned t = (unsigned)floor(256.0 * frac);
    return (r < t) ? lo + 1 : lo;
}

static void fp6_put(uint8_t *row, int64_t k, unsigned code)
{
    int64_t bit = 6 * k;
    for (int b = 0; b < 6; ++b, ++bit) {
        uint8_t m = (uint8_t)(1u << (bit % 8));
        if ((code >> b) & 1u) row[bit / 8] |= m;
        else row[bit / 8] &= (uint8_t)~m;
    }
}

static unsigned fp6_get(const uint8_t *row, int64_t k)
{
    unsigned code = 0;
    int64_t bit = 6 * k;
    for (int b = 0; b < 6; ++b, ++bit)
        code |= (unsigned)((row[bit / 8] >> (bit % 8)) & 1u) << b;
    return code;
}

/*
 * MXFP6 quantization of one direction of x (as oracle_quantize, same block,
 * 2D-tile, stochastic-rounding and padding rules; no Hadamard transform):
 * shared exponent e = floor(log2 amax) - emax_elem clamped to [-127, 127]
 * (amax == 0: -127), scale byte e + 127, or 0xFF with all-zero codes when
 * the block holds Inf/NaN; element code = sign | round(|x| * 2^-e) on the
 * format's grid.  q is canonical (R x L_pad*3/4), s is R x L_pad/32.
 */
int oracle_quantize_fp6(const uint16_t *x, int64_t M, int64_t N, int64_t ldx, int dir, int fmt,
                        int use_2d, int use_sr, uint64_t seed, uint32_t tensor_id,
                        uint64_t index_base, uint8_t *q, uint8_t *s)
{
    int ebits, mbits, bias, emax;
    if (M < 0 || N < 0 || ldx < N || (dir != 0 && dir != 1)) return -1;
    if (fp6_params(fmt, &ebits, &mbits, &bias, &emax) != 0) return -1;
    double mag[32];
    fp6_grid(fmt, mag);
    const int64_t R = dir == 0 ? M : N;
    const int64_t L = dir == 0 ? N : M;
    const int64_t L_pad = cdiv64(L, MX_PAD) * MX_PAD;
    const int64_t nblk = L_pad / MX_BLOCK;
    const int64_t row_bytes = L_pad * 3 / 4;

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t b = 0; b < nblk; ++b) {
            int64_t i0, i1, j0, j1;
            if (dir == 0) {
                i0 = use_2d ? (r / 32) * 32 : r;
                i1 = use_2d ? i0 + 32 : r + 1;
                j0 = b * MX_BLOCK;
                j1 = j0 + MX_BLOCK;
            } else {
                i0 = b * MX_BLOCK;
                i1 = i0 + MX_BLOCK;
                j0 = use_2d ? (r / 32) * 32 : r;
                j1 = use_2d ? j0 + 32 : r + 1;
            }
            if (i1 > M) i1 = M;
            if (j1 > N) j1 = N;
            double amax = 0.0;
            int nonfinite = 0;
            for (int64_t i = i0; i < i1; ++i)
                for (int64_t j = j0; j < j1; ++j) {
                    uint16_t bits = x[i * ldx + j];
                    if (!bf16_is_finite(bits)) nonfinite = 1;
                    else if (fabs(bf16_value(bits)) > amax) amax = fabs(bf16_value(bits));
                }
            int e = -127;
            if (amax > 0.0) {
                int ex;
                (void)frexp(amax, &ex);
                e = (ex - 1) - emax;
                if (e < -127) e = -127;
                if (e > 127) e = 127;
            }
            s[r * nblk + b] = nonfinite ? 0xFF : (uint8_t)(e + 127);
            for (int64_t t = 0; t < MX_BLOCK; ++t) {
                int64_t k = b * MX_BLOCK + t;
                unsigned code = 0;
                if (k < L && !nonfinite) {
                    int64_t i = dir == 0 ? r : k;
                    int64_t j = dir == 0 ? k : r;
                    uint16_t bits = x[i * ldx + j];
                    double v = ldexp(fabs(bf16_value(bits)), -e);   /* exact */
                    int c;
                    if (use_sr) {
                        uint64_t n = index_base + (uint64_t)i * (uint64_t)N + (uint64_t)j;
                        c = fp6_sr(v, oracle_sr_byte(seed, tensor_id, (uint32_t)dir, n), mag);
                    } else {
                        c = fp6_rne(v, mag);
                    }
                    code = ((bits >> 15) ? 32u : 0u) | (unsigned)c;
                }
                fp6_put(q + r * row_bytes, k, code);
            }
        }
    }
    return 0;
}

/* Exact fp64 values of a canonical FP6 blob (R x L_pad; NaN under scale 0xFF). */
int oracle_dequantize_fp6(const uint8_t *q, const uint8_t *s, int64_t R, int64_t L, int fmt, double *out)
{
    int ebits, mbits, bias, emax;
    if (R < 0 || L < 0 || fp6_params(fmt, &ebits, &mbits, &bias, &emax) != 0) return -1;
    const int64_t L_pad = cdiv64(L, MX_PAD) * MX_PAD;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t k = 0; k < L_pad; ++k) {
            uint8_t sb = s[r * (L_pad / MX_BLOCK) + k / MX_BLOCK];
            out[r * L_pad + k] = sb == 0xFF ? NAN
                                 : ldexp(oracle_fp6_value(fp6_get(q + r * (L_pad * 3 / 4), k), fmt), (int)sb - 127);
        }
    return 0;
}

/*
 * The block-scaled NT product on FP6 blobs, the same definition as
 * oracle_gemm_entries: C[i][j] = sum over the padded K of deqA[i][k] deqB[j][k]
 * in fp64, k order.  Also returns sum |deqA[i][k] deqB[j][k]| in abs_out (may
 * be NULL), the scale of the hardware's accumulation error.
 */
int oracle_gemm_fp6_entries(const uint8_t *qa, const uint8_t *sa, int fmt_a,
                            const uint8_t *qb, const uint8_t *sb, int fmt_b,
                            int64_t M, int64_t N, int64_t K, int64_t count,
                            const int64_t *ii, const int64_t *jj, double *out, double *abs_out)
{
    int ebits, mbits, bias, emax;
    if (M < 0 || N < 0 || K < 0 || count < 0) return -1;
    if (fp6_params(fmt_a, &ebits, &mbits, &bias, &emax) != 0 || fp6_params(fmt_b, &ebits, &mbits, &bias, &emax) != 0)
        return -1;
    const int64_t K_pad = cdiv64(K, MX_PAD) * MX_PAD;
    const int64_t rb = K_pad * 3 / 4, nblk = K_pad / MX_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t) {
        int64_t i = ii[t], j = jj[t];
        double acc = 0.0, aacc = 0.0;
        if (i >= 0 && i < M && j >= 0 && j < N) {
            for (int64_t k = 0; k < K_pad; ++k) {
                uint8_t ea = sa[i * nblk + k / MX_BLOCK], eb = sb[j * nblk + k / MX_BLOCK];
                double a = ea == 0xFF ? NAN : ldexp(oracle_fp6_value(fp6_get(qa + i * rb, k), fmt_a), (int)ea - 127);
                double b = eb == 0xFF ? NAN : ldexp(oracle_fp6_value(fp6_get(qb + j * rb, k), fmt_b), (int)eb - 127);
                acc += a * b;
                aacc += fabs(a * b);
            }
        } else {
            acc = NAN;
            aacc = NAN;
        }
        out[t] = acc;
        if (abs_out) abs_out[t] = aacc;
    }
    return 0;
}

/*
 * Canonical FP6 blob -> the library's tiled FP6 layout.
 *   data atom (row group g, k-step c = k/128) is 1536 bytes at
 *     (g * (L_pad/128) + c) * 1536; lane = (r%16) + 16*((k%128)/32) owns the
 *     24 bytes of row r's k-block (the canonical bytes of those 32 elements,
 *     in order): bytes 0..15 at 16*lane, bytes 16..23 at 1024 + 8*lane.
 *   scales: the MXFP4 tiled scale atoms (oracle_to_tiled).
 * Pad rows (r >= R) and unused scale bytes are 0.
 */
int oracle_fp6_to_tiled(const uint8_t *q, const uint8_t *s, int64_t R, int64_t L, uint8_t *qt, uint8_t *st)
{
    if (R < 0 || L < 0) return -1;
    const int64_t L_pad = cdiv64(L, MX_PAD) * MX_PAD;
    const int64_t R16 = cdiv64(R, 16) * 16;
    const int64_t ksteps = L_pad / 128;
    const int64_t kgroups = cdiv64(L_pad, 512);
    const int64_t rb = L_pad * 3 / 4;
    memset(qt, 0, (size_t)(R16 * rb));
    memset(st, 0, (size_t)(R16 * kgroups * 16));
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t kb = 0; kb < L_pad / 32; ++kb) {
            int64_t lane = (r % 16) + 16 * (kb % 4);
            int64_t atom = ((r / 16) * ksteps + kb / 4) * 1536;
            const uint8_t *src = q + r * rb + kb * 24;
            for (int b = 0; b < 24; ++b) {
                int64_t off = b < 16 ? atom + 16 * lane + b : atom + 1024 + 8 * lane + (b - 16);
                qt[off] = src[b];
            }
            int64_t soff = ((r / 16) * kgroups + kb / 16) * 256 + 4 * lane + (kb % 16) / 4;
            st[soff] = s[r * (L_pad / 32) + kb];
        }
    }
    return 0;
}

/* ------------------------------------------------------ multiply prologue */
/*
 * The element the multiply prologue quantizes (reading of the page "Primus
 * PR 1107": the packer forms the gradient in its staging read instead of
 * reading back what the producer stored; the producer multiplies in fp32 and
 * stores bf16): y = bf16(fp32(x * g)) -- the exact product of the two bf16
 * values rounded to fp32 nearest-even (IEEE, subnormals kept), then to bf16
 * nearest-even (oracle_bf16_from_double).
 */
void oracle_bf16_mul_array(const uint16_t *x, const uint16_t *g, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) {
        float p = (float)(bf16_value(x[i]) * bf16_value(g[i]));
        out[i] = oracle_bf16_from_double((double)p);
    }
}
