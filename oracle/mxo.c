/*
 * mxo.c -- CPU oracle for OCP-MX block-scaled FP8 (MXFP8) quantize, dequantize and GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this
 * file: only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code, header, table or constant generator with the HIP library; it is
 * plain C99 built with gcc, and it is deliberately slow and literal.
 *
 * Sources (page titles; sections in quotes):
 *   [LPGP] "Low-Precision GPU Programming" (leetllm.com)
 *     - "Format taxonomy: range, spacing, and bitfields": E4M3 max 448, no infinities,
 *       0x7F/0xFF NaN, min normal 2^-6, subnormals down to 2^-9; E5M2 smallest subnormal
 *       2^-16, largest finite 57,344.
 *     - "Numerical hazards" / "Subnormals and flush-to-zero": round-to-nearest-even,
 *       0.75*2^-9 -> 2^-9, 0.5*2^-9 -> signed zero.
 *     - "Numerical hazards" / "Saturation cliffs": conversion rounds first, then a
 *       saturating conversion clamps to +-448 / +-57,344.
 *     - "Scale ownership and the GEMM dataflow": Y = XW, X in R^{MxK}, W in R^{KxN};
 *       with block scaling along K the block-scale product stays inside the outer sum
 *       over blocks b, a partial final block is zero-padded.
 *     - "Scaling architectures" / "One letter, two reciprocal conventions": S is the
 *       reconstruction scale, x_hat = S*q, q = Q(x/S); a zero-only group takes S = 1.
 *     - "Microscaling: the two-row experiment": 32-element blocks, E8M0 byte c means
 *       2^(c-127), 255 is NaN; the conservative power-of-two scale rounds amax/448
 *       upward (exponent = max(-127, ceil(log2(amax/fmax)))), zero block -> 1; the OCP
 *       MX specification describes another scale-selection algorithm (the page names it
 *       without stating it; it is taken from the specification, see mxo_scale_byte_ocp).
 *
 * Readings where the pages are silent (each is listed with its reason in the design notes):
 *   - E5M2 uses the same scale rule with fmax = 57,344.
 *   - A block containing NaN or +-Inf gets scale byte 255 and every code 0x7F.
 *   - Padding positions (k >= K inside the last block) get code 0x00.
 *   - The GEMM epilogue is y = alpha*acc + bias[j] (scale, then bias), done in FP64 here.
 *   - The epilogue activation (SiLU) is applied after the scale and the bias.
 *   - Stochastic rounding: element n (its index line*Kp + k in the padded code array) draws
 *     the 32-bit word n%4 of Philox4x32-10(counter = (n/4 low, n/4 high, 0, 0), key = seed);
 *     its top 24 bits r decide: round up iff r < 2^24 * (|a| - l) / (u - l).  The scale
 *     rule is unchanged.
 *   - Caller-owned (delayed or stale) scales: codes are RNE-satfinite(x / S) with the given
 *     S; NaN -> 0x7F, +-Inf -> +-fmax, a given scale byte 255 makes the block 0x7F; an
 *     element counts as clipped when |x / S| > fmax and as flushed when x != 0 (finite)
 *     and its code has magnitude 0; the exported block amax is max |x| over the real
 *     elements (NaN if any is NaN).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <float.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MXO_F32 0
#define MXO_BF16 1
#define MXO_FMT_E4M3 0
#define MXO_FMT_E5M2 1

/* Number of OpenMP threads the parallel loops below use. */
int mxo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- decode ---------- */

/* FP8 decode straight from the bitfields [LPGP "Format taxonomy"]:
 *   E4M3: sign | 4 exponent bits (bias 7) | 3 mantissa bits; exponent 0 is subnormal
 *         (0.m * 2^-6); S.1111.111 is NaN; there is no infinity.
 *   E5M2: sign | 5 exponent bits (bias 15) | 2 mantissa bits; exponent 0 is subnormal
 *         (0.m * 2^-14); exponent 31 is Inf (m = 0) or NaN.                               */
double mxo_decode(uint8_t code, int fmt)
{
    int s = (code >> 7) & 1;
    double mag;
    if (fmt == MXO_FMT_E4M3) {
        int E = (code >> 3) & 0xF, m = code & 0x7;
        if (E == 15 && m == 7) return NAN;
        if (E == 0) mag = ldexp((double)m / 8.0, -6);
        else        mag = ldexp(1.0 + (double)m / 8.0, E - 7);
    } else {
        int E = (code >> 2) & 0x1F, m = code & 0x3;
        if (E == 31) { if (m == 0) return s ? -INFINITY : INFINITY; return NAN; }
        if (E == 0) mag = ldexp((double)m / 4.0, -14);
        else        mag = ldexp(1.0 + (double)m / 4.0, E - 15);
    }
    return s ? -mag : mag;
}

/* E8M0 scale byte [LPGP "Microscaling: the two-row experiment"]: c in 0..254 is 2^(c-127),
 * 255 is NaN; there is no zero, sign or infinity.                                          */
double mxo_decode_e8m0(uint8_t c)
{
    if (c == 255) return NAN;
    return ldexp(1.0, (int)c - 127);
}

/* Largest finite magnitude of each element format [LPGP "Format taxonomy"]. */
double mxo_fmax(int fmt) { return fmt == MXO_FMT_E4M3 ? 448.0 : 57344.0; }

/* ---------------------------------------------------------------- encode ---------- */

/* Table of the finite non-negative magnitudes, indexed by code.  Because the sign bit is
 * the top bit and exponent sits above mantissa, codes 0x00.. increase with magnitude:
 * E4M3 0x00..0x7E (127 values; 0x7F is NaN), E5M2 0x00..0x7B (124 values; 0x7C is Inf). */
static double g_mag[2][128];
static int g_nmag[2];
static int g_ready;

static void build_tables(void)
{
    if (g_ready) return;
    for (int f = 0; f < 2; ++f) {
        int n = 0;
        for (int c = 0; c < 128; ++c) {
            double v = mxo_decode((uint8_t)c, f);
            if (!isfinite(v)) break;
            g_mag[f][n++] = v;
        }
        g_nmag[f] = n;
    }
    g_ready = 1;
}

int mxo_num_finite_codes(int fmt) { build_tables(); return g_nmag[fmt]; }

/* Round-to-nearest-even, saturating conversion of an exact real value a to an FP8 code
 * [LPGP "Subnormals and flush-to-zero", "Saturation cliffs"].
 *   - |a| at or above fmax gives fmax (rounding first, then saturation, can only land
 *     there: every finite value above fmax either rounds to fmax or overflows).
 *   - otherwise find neighbours lo <= |a| < hi in the table and compare |a| with their
 *     exact midpoint; a tie goes to the even code (mantissa LSB 0), also across the
 *     subnormal/normal seam.
 *   - the sign bit is copied from a, so -0 and negative values that round to zero give
 *     0x80 (signed zero).
 *   - NaN gives 0x7F (the NaN code of both formats with the sign bit clear).            */
uint8_t mxo_encode(double a, int fmt)
{
    build_tables();
    if (isnan(a)) return 0x7F;
    uint8_t sign = signbit(a) ? 0x80 : 0x00;
    double x = fabs(a);
    int n = g_nmag[fmt];
    const double *t = g_mag[fmt];
    if (x >= t[n - 1]) return (uint8_t)(sign | (n - 1));
    /* binary search: largest i with t[i] <= x (t[0] = 0 <= x always) */
    int lo = 0, hi = n - 1;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (t[mid] <= x) lo = mid; else hi = mid;
    }
    /* now t[lo] <= x < t[hi] with hi = lo + 1 */
    double midpoint = (t[lo] + t[hi]) / 2.0; /* exact: both are short dyadic rationals */
    int code;
    if (x < midpoint)      code = lo;
    else if (x > midpoint) code = hi;
    else                   code = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(sign | code);
}

/* Stochastic rounding of an exact real value a to an FP8 code [LPGP "Rounding: RNE
 * versus stochastic rounding"]: with l <= |a| < u the neighbouring finite magnitudes, the
 * result is u with probability (|a| - l) / (u - l), else l; a representable |a| stays.
 * The probability is realised by a uniform 24-bit integer r: up iff r < 2^24 * p.  (p is
 * a dyadic rational here and 2^24 * p is computed exactly in FP64.)  |a| >= fmax gives
 * fmax; sign as in mxo_encode; NaN gives 0x7F.                                           */
uint8_t mxo_encode_sr(double a, int fmt, uint32_t r24)
{
    build_tables();
    if (isnan(a)) return 0x7F;
    uint8_t sign = signbit(a) ? 0x80 : 0x00;
    double x = fabs(a);
    int n = g_nmag[fmt];
    const double *t = g_mag[fmt];
    if (x >= t[n - 1]) return (uint8_t)(sign | (n - 1));
    int lo = 0, hi = n - 1;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (t[mid] <= x) lo = mid; else hi = mid;
    }
    if (x == t[lo]) return (uint8_t)(sign | lo);
    double p = (x - t[lo]) / (t[hi] - t[lo]);
    int code = (double)r24 < p * 16777216.0 ? hi : lo;
    return (uint8_t)(sign | code);
}

/* ---------------------------------------------------------------- random numbers -- */

/* Philox4x32-10 [Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2,
 * 3", SC 2011]: ten rounds of two 32x32->64-bit multiplications (multipliers 0xD2511F53,
 * 0xCD9E8D57) whose high halves are xored with the other counter words and the key; the
 * key is bumped by the Weyl constants 0x9E3779B9, 0xBB67AE85 between rounds.             */
void mxo_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 24-bit uniform integer of element n under a 64-bit seed. */
static uint32_t sr_random24(uint64_t seed, uint64_t n)
{
    uint32_t ctr[4] = {(uint32_t)(n >> 2), (uint32_t)(n >> 34), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    mxo_philox4x32_10(ctr, key, out);
    return out[n & 3] >> 8;
}

/* ---------------------------------------------------------------- scale rule ------ */

/* Conservative power-of-two block scale [LPGP "Microscaling: the two-row experiment";
 * "One letter, two reciprocal conventions"]:
 *   amax == 0         -> S = 1            (byte 127)
 *   amax non-finite   -> byte 255 (NaN)
 *   otherwise         -> S = 2^e with e the smallest integer >= -127 such that
 *                        amax <= fmax * 2^e; byte = e + 127.
 * Written as the literal search; fmax*2^e and the comparison are exact in FP64.         */
int mxo_scale_byte(double amax, int fmt)
{
    if (!isfinite(amax)) return 255;
    if (amax == 0.0) return 127;
    double fmax = mxo_fmax(fmt);
    int e = -127;
    while (ldexp(fmax, e) < amax) ++e;
    return e + 127;
}

/* Scale rule of the OCP Microscaling Formats (MX) Specification v1.0, which the pages
 * cite as the other scale-selection algorithm [LPGP "Microscaling: the two-row
 * experiment"]: the shared exponent is floor(log2(amax)) minus the exponent of the element
 * format's largest normal (E4M3: 448 = 1.75 * 2^8 -> 8; E5M2: 57,344 = 1.75 * 2^15 -> 15),
 * and the elements are then converted with round-to-nearest-even, values past the largest
 * normal clamped to it (satfinite).  Readings shared with the rule above: the exponent is
 * clamped at -127 (E8M0's smallest), a zero block takes S = 1, a non-finite block 255.
 * floor(log2(amax)) is the literal search for the largest E with 2^E <= amax (exact in
 * FP64 for every fp32 / bf16 amax).                                                     */
int mxo_scale_byte_ocp(double amax, int fmt)
{
    if (!isfinite(amax)) return 255;
    if (amax == 0.0) return 127;
    int emax_elem = fmt == MXO_FMT_E4M3 ? 8 : 15;
    int E = -150;                                 /* 2^-150 is below every fp32 value */
    while (ldexp(1.0, E + 1) <= amax) ++E;
    int e = E - emax_elem;
    if (e < -127) e = -127;
    return e + 127;
}

#define MXO_RULE_CEIL 0
#define MXO_RULE_OCP 1

/* ---------------------------------------------------------------- helpers --------- */

static double load_elem(const void *src, int src_type, int64_t idx)
{
    if (src_type == MXO_F32) return (double)((const float *)src)[idx];
    uint16_t h = ((const uint16_t *)src)[idx];
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* bf16 round-to-nearest-even of an FP64 value, by neighbour search: bf16 has 7 stored
 * mantissa bits and fp32's exponent range, so between 2^E and 2^(E+1) (E >= -126) the
 * spacing is 2^(E-7), and below 2^-126 it is 2^-133.  Returns the bf16 bit pattern.    */
uint16_t mxo_round_bf16(double v)
{
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a)) return sign | 0x7F80;
    if (a == 0.0) return sign;
    int E;
    frexp(a, &E);        /* a = f * 2^E, f in [0.5, 1) -> a in [2^(E-1), 2^E) */
    E -= 1;              /* a in [2^E, 2^(E+1)) */
    int q = (E < -126) ? -133 : E - 7;
    double spacing = ldexp(1.0, q);
    double lo = floor(a / spacing) * spacing;
    double hi = lo + spacing;
    double r;
    if (a - lo < hi - a)      r = lo;
    else if (a - lo > hi - a) r = hi;
    else                      r = (fmod(lo / spacing, 2.0) == 0.0) ? lo : hi;
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;       /* rounds past the top: Inf */
    float f = (float)r;   /* r is a bf16 value, so it is exact in fp32 */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* fp32 rounding of an FP64 value that is exactly a (code * power of two): exact unless it
 * is at or beyond 2^128, where IEEE round-to-nearest overflows to Inf.                   */
static float to_f32(double v)
{
    if (isnan(v)) return NAN;
    if (fabs(v) >= ldexp(1.0, 128)) return signbit(v) ? -INFINITY : INFINITY;
    return (float)v;
}

/* ---------------------------------------------------------------- quantize -------- */

/* Quantize one line of K values (element k at src[base + k*stride]) into ceil(K/32)
 * blocks [LPGP "Scale ownership and the GEMM dataflow": block index b along K; partial
 * final block zero-padded].                                                              */
static void quantize_line(const void *src, int src_type, int64_t base, int64_t stride, int64_t K,
                          int fmt, uint8_t *codes, uint8_t *scales, int sr, uint64_t seed, int64_t n0,
                          int rule)
{
    int64_t nb = (K + 31) / 32;
    for (int64_t b = 0; b < nb; ++b) {
        int64_t k0 = 32 * b, k1 = k0 + 32 < K ? k0 + 32 : K;
        double amax = 0.0;
        int nonfinite = 0;
        for (int64_t k = k0; k < k1; ++k) {
            double x = load_elem(src, src_type, base + k * stride);
            if (!isfinite(x)) nonfinite = 1;
            else if (fabs(x) > amax) amax = fabs(x);
        }
        if (nonfinite) {
            scales[b] = 255;
            for (int64_t k = k0; k < k0 + 32; ++k) codes[k] = 0x7F;
            continue;
        }
        int sb = rule == MXO_RULE_OCP ? mxo_scale_byte_ocp(amax, fmt) : mxo_scale_byte(amax, fmt);
        scales[b] = (uint8_t)sb;
        int e = sb - 127;
        for (int64_t k = k0; k < k0 + 32; ++k) {
            if (k < K) {
                double x = load_elem(src, src_type, base + k * stride);
                double a = ldexp(x, -e);                   /* x / S, exact in FP64 */
                codes[k] = sr ? mxo_encode_sr(a, fmt, sr_random24(seed, (uint64_t)(n0 + k)))
                              : mxo_encode(a, fmt);
            } else {
                codes[k] = 0x00;                            /* zero padding */
            }
        }
    }
}

/* axis 0 (rowwise): the lines are the rows of src [rows][ld_src], K = cols.
 * axis 1 (colwise): the lines are the columns of src, K = rows, and the output is stored
 *                   transposed, codes [cols][ld_codes], scales [cols][ld_scales].
 * Writes Kp = 32*ceil(K/32) codes and Kp/32 scale bytes per line.                        */
static void quantize_any(const void *src, int src_type, int64_t rows, int64_t cols, int64_t ld_src,
                         int axis, int fmt, uint8_t *codes, int64_t ld_codes, uint8_t *scales,
                         int64_t ld_scales, int sr, uint64_t seed, int rule)
{
    build_tables();
    int64_t L = axis == 0 ? rows : cols;
    int64_t K = axis == 0 ? cols : rows;
    int64_t Kp = 32 * ((K + 31) / 32);
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t l = 0; l < L; ++l) {
        int64_t base = axis == 0 ? l * ld_src : l;
        int64_t stride = axis == 0 ? 1 : ld_src;
        quantize_line(src, src_type, base, stride, K, fmt, codes + l * ld_codes,
                      scales + l * ld_scales, sr, seed, l * Kp, rule);
    }
}

void mxo_quantize(const void *src, int src_type, int64_t rows, int64_t cols, int64_t ld_src,
                  int axis, int fmt, uint8_t *codes, int64_t ld_codes, uint8_t *scales,
                  int64_t ld_scales)
{
    quantize_any(src, src_type, rows, cols, ld_src, axis, fmt, codes, ld_codes, scales, ld_scales, 0, 0,
                 MXO_RULE_CEIL);
}

/* mxo_quantize with the scale rule chosen: 0 the pages' (ceil), 1 the OCP MX rule.       */
void mxo_quantize_rule(const void *src, int src_type, int64_t rows, int64_t cols, int64_t ld_src,
                       int axis, int fmt, int rule, uint8_t *codes, int64_t ld_codes, uint8_t *scales,
                       int64_t ld_scales)
{
    quantize_any(src, src_type, rows, cols, ld_src, axis, fmt, codes, ld_codes, scales, ld_scales, 0, 0, rule);
}

/* The same blocks and scales with stochastically rounded codes (the readings above give
 * the random-number contract).                                                          */
void mxo_quantize_sr(const void *src, int src_type, int64_t rows, int64_t cols, int64_t ld_src,
                     int axis, int fmt, uint64_t seed, uint8_t *codes, int64_t ld_codes,
                     uint8_t *scales, int64_t ld_scales)
{
    quantize_any(src, src_type, rows, cols, ld_src, axis, fmt, codes, ld_codes, scales, ld_scales, 1, seed,
                 MXO_RULE_CEIL);
}

/* Quantize with caller-owned scale bytes [LPGP "Worked failure: stale delayed scale": a
 * scale from an earlier amax saturates a later spike; "Delayed scaling in Transformer
 * Engine": the quantization pass also records the current amax for the next scale
 * update].  given_scales [L][ld_given]; optional per-block outputs (NULL = not written):
 * amax [L][ld_amax] (FP32 max |x|), clipped and flushed counts [L][ld_diag].           */
void mxo_quantize_scaled(const void *src, int src_type, int64_t rows, int64_t cols, int64_t ld_src,
                         int axis, int fmt, const uint8_t *given_scales, int64_t ld_given,
                         uint8_t *codes, int64_t ld_codes, float *amax_out, int64_t ld_amax,
                         uint8_t *clipped, uint8_t *flushed, int64_t ld_diag)
{
    build_tables();
    int64_t L = axis == 0 ? rows : cols;
    int64_t K = axis == 0 ? cols : rows;
    int64_t nb = (K + 31) / 32;
    double fmax = mxo_fmax(fmt);
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t l = 0; l < L; ++l) {
        int64_t base = axis == 0 ? l * ld_src : l;
        int64_t stride = axis == 0 ? 1 : ld_src;
        for (int64_t b = 0; b < nb; ++b) {
            int sb = given_scales[l * ld_given + b];
            double amax = 0.0;
            int any_nan = 0, nclip = 0, nflush = 0;
            for (int64_t k = 32 * b; k < 32 * b + 32; ++k) {
                uint8_t c = 0x00;                                  /* zero padding */
                if (k < K) {
                    double x = load_elem(src, src_type, base + k * stride);
                    if (isnan(x)) any_nan = 1;
                    else if (fabs(x) > amax) amax = fabs(x);
                    if (sb == 255 || isnan(x)) {
                        c = 0x7F;
                    } else {
                        double a = ldexp(x, 127 - sb);             /* x / S, exact in FP64 */
                        if (fabs(a) > fmax) {
                            ++nclip;
                            a = a < 0 ? -fmax : fmax;              /* saturate */
                        }
                        c = mxo_encode(a, fmt);
                        if (x != 0.0 && (c & 0x7F) == 0) ++nflush;
                    }
                } else if (sb == 255) {
                    c = 0x7F;
                }
                codes[l * ld_codes + k] = c;
            }
            if (amax_out) amax_out[l * ld_amax + b] = any_nan ? NAN : (float)amax;
            if (clipped) clipped[l * ld_diag + b] = (uint8_t)nclip;
            if (flushed) flushed[l * ld_diag + b] = (uint8_t)nflush;
        }
    }
}

/* ---------------------------------------------------------------- dequantize ------ */

/* x_hat = dec(code) * 2^(s-127) [LPGP "One letter, two reciprocal conventions":
 * reconstruction x_hat = S*q], computed exactly in FP64 then rounded to the destination:
 * fp32 (exact unless past 2^128 -> Inf) or bf16 (RNE).  dst_type 0 = fp32, 1 = bf16.   */
void mxo_dequantize(const uint8_t *codes, int64_t ld_codes, const uint8_t *scales,
                    int64_t ld_scales, int fmt, int64_t L, int64_t K, void *dst, int dst_type,
                    int64_t ld_dst)
{
    #pragma omp parallel for schedule(static)
    for (int64_t l = 0; l < L; ++l) {
        for (int64_t k = 0; k < K; ++k) {
            double v = mxo_decode(codes[l * ld_codes + k], fmt) *
                       mxo_decode_e8m0(scales[l * ld_scales + k / 32]);
            if (dst_type == MXO_F32) ((float *)dst)[l * ld_dst + k] = to_f32(v);
            else ((uint16_t *)dst)[l * ld_dst + k] = mxo_round_bf16(v);
        }
    }
}

/* ---------------------------------------------------------------- GEMM ------------ */

/* One output element of the block-K scaled contraction [LPGP "Scale ownership and the
 * GEMM dataflow"]:
 *   acc = sum_b  S_X[i,b] * S_W[b,j] * sum_{k in b, k < K} Xq[i,k] * Wq[k,j]
 *   y   = alpha * acc + bias[j]
 * and the bound T = |alpha| * sum_b S_X S_W sum_k |Xq Wq|.  W is given column-major,
 * i.e. as rows w_codes[j][k] (the kernel contract's "col_major_packed" operand).
 * Every product of two FP8 values and two powers of two is exact in FP64.               */
static void gemm_one(int64_t i, int64_t j, int64_t K,
                     const uint8_t *xc, int64_t ld_x, const uint8_t *xs, int64_t ld_xs, int xf,
                     const uint8_t *wc, int64_t ld_w, const uint8_t *ws, int64_t ld_ws, int wf,
                     double alpha, const float *bias, double *y, double *t)
{
    int64_t nb = (K + 31) / 32;
    double acc = 0.0, bound = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        double inner = 0.0, inner_abs = 0.0;
        for (int64_t k = 32 * b; k < 32 * b + 32 && k < K; ++k) {
            double p = mxo_decode(xc[i * ld_x + k], xf) * mxo_decode(wc[j * ld_w + k], wf);
            inner += p;
            inner_abs += fabs(p);
        }
        double sprod = mxo_decode_e8m0(xs[i * ld_xs + b]) * mxo_decode_e8m0(ws[j * ld_ws + b]);
        acc += sprod * inner;
        bound += sprod * inner_abs;
    }
    *y = alpha * acc + (bias ? (double)bias[j] : 0.0);
    *t = fabs(alpha) * bound;
}

/* Full reference: y_ref and t are dense [M][N] row-major FP64. */
void mxo_gemm(int64_t M, int64_t N, int64_t K,
              const uint8_t *x_codes, int64_t ld_x, const uint8_t *x_scales, int64_t ld_xs, int x_fmt,
              const uint8_t *w_codes, int64_t ld_w, const uint8_t *w_scales, int64_t ld_ws, int w_fmt,
              double alpha, const float *bias, double *y_ref, double *t)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            gemm_one(i, j, K, x_codes, ld_x, x_scales, ld_xs, x_fmt, w_codes, ld_w, w_scales,
                     ld_ws, w_fmt, alpha, bias, &y_ref[i * N + j], &t[i * N + j]);
}

/* Sampled reference: n output elements (ii[s], jj[s]). */
void mxo_gemm_sampled(int64_t K,
                      const uint8_t *x_codes, int64_t ld_x, const uint8_t *x_scales, int64_t ld_xs, int x_fmt,
                      const uint8_t *w_codes, int64_t ld_w, const uint8_t *w_scales, int64_t ld_ws, int w_fmt,
                      double alpha, const float *bias, int64_t n, const int64_t *ii, const int64_t *jj,
                      double *y_ref, double *t)
{
    #pragma omp parallel for schedule(dynamic, 16)
    for (int64_t s = 0; s < n; ++s)
        gemm_one(ii[s], jj[s], K, x_codes, ld_x, x_scales, ld_xs, x_fmt, w_codes, ld_w, w_scales,
                 ld_ws, w_fmt, alpha, bias, &y_ref[s], &t[s]);
}

/* ---------------------------------------------------------------- activation ------ */

/* SiLU, the activation the kernel contract's epilogue names [LPGP "Hardware support and
 * kernel ABI contracts"], by its textbook definition v * sigmoid(v) = v / (1 + e^-v) in
 * FP64 (exact for every purpose here: FP64 keeps ~1e-16 relative error while every
 * comparison is against FP32 or narrower).                                              */
double mxo_silu(double v) { return v / (1.0 + exp(-v)); }

void mxo_silu_array(const double *v, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = mxo_silu(v[i]);
}
