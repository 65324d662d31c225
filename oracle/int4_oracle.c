/*
 * int4_oracle.c -- plain, slow, scalar CPU oracle for block-wise symmetric
 * INT4 weight quantization, two's-complement nibble packing, unpacking and
 * the dequantizing matmul.
 *
 * TEST INFRASTRUCTURE. This file is the correctness reference for the HIP
 * path and nothing else: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may build, load or call it. It shares no code, header or
 * constant with the GPU library, and the GPU library never calls it.
 *
 * Source of the definition: the drill page "Implement INT4 group
 * quantization, nibble packing and a dequantizing matmul"
 * (inferenceinterviews.com), section "statement" (quantize_int4,
 * unpack_int4, int4_matmul) and its two visible tests. Where that statement
 * leaves a step open, the reading taken is named at the step:
 *   - scale: absmax of the group divided by 7 as an IEEE binary32 division,
 *     then rounded to binary16 (round to nearest, ties to even).  This is
 *     what NumPy does for (abs(g).max() / 7).astype(float16) on float32 data,
 *     and the statement runs in NumPy.
 *   - q = round(w / scale): the divisor is the STORED binary16 scale widened
 *     to binary32; the division is binary32; round() is ties-to-even
 *     (NumPy's np.round / np.rint, also used by "Building a Pure-Python INT4
 *     Transformer Weight Quantizer ..." step 4).
 *   - a group whose binary16 scale is zero (all zeros, or an absmax so small
 *     that absmax/7 rounds to zero in binary16) quantizes to all-zero q.
 *   - groups run along K inside each row; the last group may be partial.
 *   - the matmul follows the statement's order: per group, x times the
 *     integer weights first, then that group's scale; accumulated in double
 *     and rounded once to binary32.
 *
 * Also here, each with its own source named where it is defined: the
 * dequantization w_hat = q * scale, the layer epilogue act(y + bias), and the
 * affine (zero-point) variant of the codes from "Build a Blockwise INT4
 * Inference Engine", step 2.
 *
 * Build: cc -O2 -std=c99 -fno-fast-math -ffp-contract=off -shared -fPIC.
 * No SIMD intrinsics, no threads, no blocking or reordering of the loops
 * beyond what the definition states.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>

/* ------------------------------------------------------------------------ */
/* binary16 <-> binary32, written from the IEEE-754 definition.             */
/* ------------------------------------------------------------------------ */

/*
 * Nearest binary16 to a binary32 value, ties to the even significand.
 * binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * For a value a = |f| in [2^e, 2^(e+1)) the spacing of binary16 numbers is
 * 2^(max(e,-14) - 10); below 2^-14 the spacing stays 2^-24 (subnormals).
 * The largest finite binary16 is 65504; the halfway point to the next
 * (unrepresentable) step 65536 is 65520, and a tie there goes to 65536,
 * i.e. to infinity, because 65504 has an odd significand.
 */
uint16_t int4_oracle_half_from_float(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00u);
    double a = fabs((double)f);               /* exact */
    if (a >= 65520.0)                         /* includes +-inf */
        return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0)
        return sign;
    int ex;
    (void)frexp(a, &ex);                      /* a = m * 2^ex, m in [0.5,1) */
    int e = ex - 1;                           /* 2^e <= a < 2^(e+1) */
    if (e < -14)
        e = -14;
    double quantum = ldexp(1.0, e - 10);
    double m = a / quantum;                   /* exact: power-of-two divide */
    double n = nearbyint(m);                  /* round half to even (FE_TONEAREST) */
    /* n is in [0, 2048]; n == 2048 carries into the next exponent, n < 1024
     * only happens for e == -14 (subnormal). One formula covers all cases. */
    long bits = ((long)(e + 15) << 10) + (long)n - 1024;
    return (uint16_t)(sign | (uint16_t)bits);
}

/* Element-wise form of the conversion above, for exhaustive checks. */
void int4_oracle_half_from_float_array(const float *f, int64_t count, uint16_t *h)
{
    for (int64_t i = 0; i < count; ++i)
        h[i] = int4_oracle_half_from_float(f[i]);
}

/* Exact widening of a binary16 bit pattern to binary32. */
float int4_oracle_float_from_half(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                       /* subnormal or zero */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);        /* (1.frac) * 2^(expo-15) */
    return (float)(sign ? -v : v);
}

/* ------------------------------------------------------------------------ */
/* Sizes (drill page, statement: scales [N, G], G = ceil(K / group);        */
/* packed [N, ceil(K / 2)] uint8).                                          */
/* ------------------------------------------------------------------------ */

int64_t int4_oracle_num_groups(int64_t K, int64_t group)
{
    return (K + group - 1) / group;
}

int64_t int4_oracle_packed_row_bytes(int64_t K)
{
    return (K + 1) / 2;
}

/* ------------------------------------------------------------------------ */
/* quantize_int4 (drill page, statement).                                   */
/* ------------------------------------------------------------------------ */

/* Signed 4-bit code of one weight, given its group's widened binary16 scale. */
static int quantize_one(float w, float sf)
{
    if (sf == 0.0f)
        return 0;                               /* a group of zeros gets scale 0 */
    float t = w / sf;                           /* binary32 division, round to nearest */
    float r = rintf(t);                         /* round half to even */
    if (r < -8.0f) r = -8.0f;                   /* clipped to [-8, 7] */
    if (r > 7.0f) r = 7.0f;
    return (int)r;
}

/*
 * w:      [N, K] binary32, row-major.
 * packed: [N, ceil(K/2)] bytes; byte j of a row holds element 2j in its low
 *         nibble and element 2j+1 in its high nibble, each as a 4-bit two's
 *         complement code; an odd K leaves a zero high nibble in the last byte.
 * scales: [N, G] binary16 bit patterns.
 */
void int4_oracle_quantize(const float *w, int64_t N, int64_t K, int64_t group,
                          uint8_t *packed, uint16_t *scales)
{
    int64_t G = int4_oracle_num_groups(K, group);
    int64_t B = int4_oracle_packed_row_bytes(K);
    for (int64_t n = 0; n < N; ++n) {
        const float *row = w + n * K;
        uint8_t *prow = packed + n * B;
        memset(prow, 0, (size_t)B);
        for (int64_t gi = 0; gi < G; ++gi) {
            int64_t k0 = gi * group;
            int64_t k1 = k0 + group < K ? k0 + group : K;
            /* 1. absmax over the (possibly partial) group; exact in binary32 */
            float amax = 0.0f;
            for (int64_t k = k0; k < k1; ++k) {
                float a = fabsf(row[k]);
                if (a > amax)
                    amax = a;
            }
            /* 2. scale = absmax / 7, stored as binary16 */
            float s32 = amax / 7.0f;
            uint16_t s16 = int4_oracle_half_from_float(s32);
            scales[n * G + gi] = s16;
            float sf = int4_oracle_float_from_half(s16);
            /* 3-4. q = clip(round(w / scale), -8, 7), packed as nibbles */
            for (int64_t k = k0; k < k1; ++k) {
                int q = quantize_one(row[k], sf);
                uint8_t nib = (uint8_t)(q & 0xF);     /* two's complement nibble */
                if (k % 2 == 0)
                    prow[k / 2] |= nib;               /* even element: low nibble */
                else
                    prow[k / 2] |= (uint8_t)(nib << 4); /* odd element: high nibble */
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Affine (asymmetric) variant ("Build a Blockwise INT4 Inference Engine",  */
/* step 2: per-group scale and zero point, q = round(w / scale + zp)        */
/* clipped to [0, 15]; "Quantizing a Language Model From Scratch", affine   */
/* quantization: S = (max - min) / 15, w' = S (q - Z)).                     */
/* ------------------------------------------------------------------------ */
/*
 * Readings, where the engine page's listing leaves them open or goes wrong:
 *   - the range is [min(lo, 0), max(hi, 0)] over the group, so that zero is
 *     always inside it and exact (the lmquant page's point about Z); for the
 *     usual group that straddles zero this is the page's min and max;
 *   - scale = (hi - lo) / 15 in binary32, stored as binary16 like the
 *     symmetric scales; every later step uses the stored scale widened;
 *   - zp = clip(round(-lo / scale), 0, 15) with a binary32 division and ties
 *     to even; stored as one byte per group;
 *   - q = clip(round(w / scale + zp), 0, 15): w / scale is a binary32
 *     division, zp is added exactly and the sum rounded half to even (the page
 *     adds an integer zero point to a float32 quotient in NumPy, which widens
 *     the sum to float64);
 *   - a group whose binary16 scale is zero gets zp = 0 and codes 0.
 * Codes are unsigned nibbles in the same layout as the symmetric codes.
 */
static int quantize_one_affine(float w, float sf, int zp)
{
    if (sf == 0.0f)
        return 0;
    float t = w / sf;                           /* binary32 division */
    double r = rint((double)t + (double)zp);    /* exact sum, half to even */
    if (r < 0.0) r = 0.0;
    if (r > 15.0) r = 15.0;
    return (int)r;
}

void int4_oracle_quantize_affine(const float *w, int64_t N, int64_t K, int64_t group,
                                 uint8_t *packed, uint16_t *scales, uint8_t *zeros)
{
    int64_t G = int4_oracle_num_groups(K, group);
    int64_t B = int4_oracle_packed_row_bytes(K);
    for (int64_t n = 0; n < N; ++n) {
        const float *row = w + n * K;
        uint8_t *prow = packed + n * B;
        memset(prow, 0, (size_t)B);
        for (int64_t gi = 0; gi < G; ++gi) {
            int64_t k0 = gi * group;
            int64_t k1 = k0 + group < K ? k0 + group : K;
            float lo = 0.0f, hi = 0.0f;             /* the range includes zero */
            for (int64_t k = k0; k < k1; ++k) {
                if (row[k] < lo) lo = row[k];
                if (row[k] > hi) hi = row[k];
            }
            float s32 = (hi - lo) / 15.0f;
            uint16_t sh = int4_oracle_half_from_float(s32);
            scales[n * G + gi] = sh;
            float sf = int4_oracle_float_from_half(sh);
            int zp = 0;
            if (sf != 0.0f) {
                float z = rintf(-lo / sf);
                zp = z < 0.0f ? 0 : (z > 15.0f ? 15 : (int)z);
            }
            zeros[n * G + gi] = (uint8_t)zp;
            for (int64_t k = k0; k < k1; ++k) {
                uint8_t nib = (uint8_t)quantize_one_affine(row[k], sf, zp);
                prow[k / 2] |= (uint8_t)(nib << (4 * (int)(k & 1)));  /* even: low nibble */
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* unpack_int4 (drill page, statement): int8 [N, K], sign-extended.         */
/* ------------------------------------------------------------------------ */

/* The 4-bit code of element k of a packed row (even k: low nibble). */
static int raw_nibble(const uint8_t *prow, int64_t k)
{
    return (prow[k / 2] >> (4 * (int)(k % 2))) & 0xF;
}

static int nibble_value(const uint8_t *prow, int64_t k)
{
    int v = raw_nibble(prow, k);
    return v >= 8 ? v - 16 : v;                 /* sign extension of a 4-bit code */
}

/* Integer weight of element k of a row: the sign-extended code, or with zero
 * points (zp: that row's array of them, NULL for symmetric codes) the
 * unsigned code minus its group's zero point. */
static int weight_int(const uint8_t *prow, int64_t k, const uint8_t *zp, int64_t group)
{
    if (!zp)
        return nibble_value(prow, k);
    return raw_nibble(prow, k) - (int)zp[k / group];
}

void int4_oracle_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *out)
{
    int64_t B = int4_oracle_packed_row_bytes(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            out[n * K + k] = (int8_t)nibble_value(packed + n * B, k);
}

/* ------------------------------------------------------------------------ */
/* int4_matmul (drill page, statement):                                     */
/*   y = x @ dequantize(W).T, one group at a time: x times the group's      */
/*   integer weights first, then the group's scale on each output column.  */
/* ------------------------------------------------------------------------ */

/*
 * x:     [M, K] binary32 (binary16 inputs are widened exactly by the caller).
 * y:     [M, N] binary32, each entry the double-precision sum rounded once.
 * bound: optional [M, N] binary64, sum over k of |x[m,k] * q[n,k] * scale|,
 *        the magnitude against which the tolerance is stated.
 */
void int4_oracle_matmul_ex(const float *x, int64_t M, const uint8_t *packed,
                           const uint16_t *scales, const uint8_t *zeros, int64_t N, int64_t K,
                           int64_t group, const float *bias, int relu, float *y, double *bound);

void int4_oracle_matmul(const float *x, int64_t M, const uint8_t *packed,
                        const uint16_t *scales, int64_t N, int64_t K, int64_t group,
                        float *y, double *bound)
{
    int4_oracle_matmul_ex(x, M, packed, scales, NULL, N, K, group, NULL, 0, y, bound);
}

/* ------------------------------------------------------------------------ */
/* dequantize (drill page, statement: w_hat = q * scale; "Build a Blockwise */
/* INT4 Inference Engine", the unfused dequantize-then-GEMM baseline):      */
/* out[n, k] = q[n, k] * scale[n, k / group].                               */
/* ------------------------------------------------------------------------ */

/*
 * zeros: NULL for symmetric codes, else [N, G] zero points of affine codes
 * (the value is code - zp). binary32 output: the integer has at most 5
 * significant bits and the widened scale 11, so the product is exact.
 */
void int4_oracle_dequantize(const uint8_t *packed, const uint16_t *scales, const uint8_t *zeros,
                            int64_t N, int64_t K, int64_t group, float *out)
{
    int64_t G = int4_oracle_num_groups(K, group);
    int64_t B = int4_oracle_packed_row_bytes(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            float sf = int4_oracle_float_from_half(scales[n * G + k / group]);
            int q = weight_int(packed + n * B, k, zeros ? zeros + n * G : NULL, group);
            out[n * K + k] = (float)q * sf;
        }
}

/*
 * binary16 output: the exact binary32 product rounded to the nearest
 * binary16 (ties to even); magnitudes of 65520 and more become infinities.
 */
void int4_oracle_dequantize_half(const uint8_t *packed, const uint16_t *scales,
                                 const uint8_t *zeros, int64_t N, int64_t K, int64_t group,
                                 uint16_t *out)
{
    int64_t G = int4_oracle_num_groups(K, group);
    int64_t B = int4_oracle_packed_row_bytes(K);
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            float sf = int4_oracle_float_from_half(scales[n * G + k / group]);
            int q = weight_int(packed + n * B, k, zeros ? zeros + n * G : NULL, group);
            out[n * K + k] = int4_oracle_half_from_float((float)q * sf);
        }
}

/* ------------------------------------------------------------------------ */
/* int4_matmul with the engine page's epilogue ("Build a Blockwise INT4     */
/* Inference Engine", fused GEMM kernel and the Python layer's forward):    */
/*   y = act(x @ dequantize(W).T + bias), act = identity or ReLU.           */
/* ------------------------------------------------------------------------ */

/*
 * The matmul sum follows the statement's order (per group: x times the
 * group's integer codes, then the group's scale), accumulated in double.
 * zeros: NULL for symmetric codes, else [N, G] zero points (affine codes,
 * integer weight = code - zp).
 * bias: optional [N] binary32 (NULL: none), added in double; the result is
 * rounded once to binary32. relu: 0 or 1; ReLU keeps a value greater than
 * zero and gives +0 otherwise (the engine page's `acc > 0 ? acc : 0`).
 * bound: optional [M, N] binary64, sum over k of |x[m,k] * q[n,k] * scale|
 * (the bias is exact and adds nothing to it). int4_oracle_matmul above is
 * this function with no bias and no activation.
 */
void int4_oracle_matmul_ex(const float *x, int64_t M, const uint8_t *packed,
                           const uint16_t *scales, const uint8_t *zeros, int64_t N, int64_t K,
                           int64_t group, const float *bias, int relu, float *y, double *bound)
{
    int64_t G = int4_oracle_num_groups(K, group);
    int64_t B = int4_oracle_packed_row_bytes(K);
    for (int64_t m = 0; m < M; ++m) {
        const float *xrow = x + m * K;
        for (int64_t n = 0; n < N; ++n) {
            const uint8_t *prow = packed + n * B;
            double acc = 0.0, mag = 0.0;
            for (int64_t gi = 0; gi < G; ++gi) {
                int64_t k0 = gi * group;
                int64_t k1 = k0 + group < K ? k0 + group : K;
                double part = 0.0, part_abs = 0.0;
                for (int64_t k = k0; k < k1; ++k) {
                    double p = (double)xrow[k] *
                               (double)weight_int(prow, k, zeros ? zeros + n * G : NULL, group);
                    part += p;
                    part_abs += fabs(p);
                }
                double sf = (double)int4_oracle_float_from_half(scales[n * G + gi]);
                acc += sf * part;
                mag += fabs(sf) * part_abs;
            }
            if (bias)
                acc += (double)bias[n];
            float v = (float)acc;
            if (relu)
                v = v > 0.0f ? v : 0.0f;
            y[m * N + n] = v;
            if (bound)
                bound[m * N + n] = mag;
        }
    }
}
