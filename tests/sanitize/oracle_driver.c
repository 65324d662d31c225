/*
 * oracle_driver.c -- runs the C oracle (oracle/int4_oracle.c) under
 * AddressSanitizer and UndefinedBehaviorSanitizer on the shapes the tests use
 * and on the edge cases of the method: odd K (a pad nibble), a partial last
 * group, group sizes 1, 3, 5, 32 and 128, group larger than K, a zero group,
 * codes of -8 under the smallest binary16 scale, and the affine codes. Every
 * buffer is a heap allocation of exactly the size the call may touch, so a
 * read or write one element past any of them is reported.
 *
 * Besides running clean, each case checks facts that follow from the method
 * itself, independent of any other implementation: the page's printed layout
 * example ("Implement INT4 group quantization, nibble packing and a
 * dequantizing matmul", visible test of the nibble layout), unpack against a
 * direct sign extension of every nibble, the pad nibble being zero, the
 * half-step bound of the round trip, and the matmul against x times the
 * dequantized weights summed here in double.
 *
 * Test infrastructure: built and run only by tests/test_sanitize_cpu.py.
 * Exit status 0 when every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t int4_oracle_half_from_float(float f);
float int4_oracle_float_from_half(uint16_t h);
int64_t int4_oracle_num_groups(int64_t K, int64_t group);
int64_t int4_oracle_packed_row_bytes(int64_t K);
void int4_oracle_quantize(const float *w, int64_t N, int64_t K, int64_t group, uint8_t *packed,
                          uint16_t *scales);
void int4_oracle_quantize_affine(const float *w, int64_t N, int64_t K, int64_t group,
                                 uint8_t *packed, uint16_t *scales, uint8_t *zeros);
void int4_oracle_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *out);
void int4_oracle_dequantize(const uint8_t *packed, const uint16_t *scales, const uint8_t *zeros,
                            int64_t N, int64_t K, int64_t group, float *out);
void int4_oracle_dequantize_half(const uint8_t *packed, const uint16_t *scales,
                                 const uint8_t *zeros, int64_t N, int64_t K, int64_t group,
                                 uint16_t *out);
void int4_oracle_matmul_ex(const float *x, int64_t M, const uint8_t *packed,
                           const uint16_t *scales, const uint8_t *zeros, int64_t N, int64_t K,
                           int64_t group, const float *bias, int relu, float *y, double *bound);

static int failures = 0;
#define CHECK(cond, ...)                                                     \
    do {                                                                     \
        if (!(cond)) {                                                       \
            ++failures;                                                      \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);             \
            fprintf(stderr, __VA_ARGS__);                                    \
            fputc('\n', stderr);                                             \
        }                                                                    \
    } while (0)

/* splitmix64: a fixed, portable stream of test values */
static uint64_t rng_state = 0x243F6A8885A308D3ull;
static uint64_t next_u64(void)
{
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
/* uniform in (-1, 1), a sum of four for a rough bell shape */
static float next_weight(void)
{
    double s = 0.0;
    for (int i = 0; i < 4; ++i) s += (double)(next_u64() >> 11) / 9007199254740992.0 * 2.0 - 1.0;
    return (float)(0.5 * s);
}

static void *xmalloc(size_t n) { void *p = malloc(n ? n : 1); if (!p) abort(); return p; }

static int nibble(const uint8_t *row, int64_t k)
{
    int v = (row[k >> 1] >> (4 * (k & 1))) & 0xF;
    return v >= 8 ? v - 16 : v;
}

/* One symmetric case: quantize, unpack, dequantize (binary32 and binary16) and
 * the matmul with a bias and with ReLU. zero_row / m8_row: rows forced to a
 * zero first group / to -8 * 2^-24 everywhere (or -1 for none). */
static void run_case(int64_t N, int64_t K, int64_t g, int64_t M, int zero_row, int m8_row)
{
    const int64_t G = int4_oracle_num_groups(K, g), B = int4_oracle_packed_row_bytes(K);
    float *w = xmalloc(sizeof(float) * N * K);
    for (int64_t i = 0; i < N * K; ++i) w[i] = next_weight();
    if (zero_row >= 0 && zero_row < N)
        for (int64_t k = 0; k < (g < K ? g : K); ++k) w[zero_row * K + k] = 0.0f;
    if (m8_row >= 0 && m8_row < N)
        for (int64_t k = 0; k < K; ++k) w[m8_row * K + k] = -8.0f * ldexpf(1.0f, -24);
    uint8_t *packed = xmalloc(N * B);
    uint16_t *scales = xmalloc(sizeof(uint16_t) * N * G);
    int8_t *q = xmalloc(N * K);
    float *deq = xmalloc(sizeof(float) * N * K);
    uint16_t *deqh = xmalloc(sizeof(uint16_t) * N * K);
    int4_oracle_quantize(w, N, K, g, packed, scales);
    int4_oracle_unpack(packed, N, K, q);
    int4_oracle_dequantize(packed, scales, NULL, N, K, g, deq);
    int4_oracle_dequantize_half(packed, scales, NULL, N, K, g, deqh);
    for (int64_t n = 0; n < N; ++n) {
        const uint8_t *row = packed + n * B;
        if (K & 1) CHECK((row[B - 1] >> 4) == 0, "pad nibble of row %lld is not zero", (long long)n);
        for (int64_t k = 0; k < K; ++k) {
            const int code = nibble(row, k);
            CHECK(q[n * K + k] == code, "unpack [%lld,%lld]", (long long)n, (long long)k);
            const float sf = int4_oracle_float_from_half(scales[n * G + k / g]);
            CHECK(deq[n * K + k] == (float)code * sf, "dequantize [%lld,%lld]", (long long)n, (long long)k);
            CHECK(deqh[n * K + k] == int4_oracle_half_from_float((float)code * sf), "binary16 dequantize");
            /* half a step of rounding, plus the rounding of the scale itself */
            const double err = fabs((double)code * sf - (double)w[n * K + k]);
            CHECK(err <= 0.5 * sf + 1e-3 * sf + 1e-6, "round trip [%lld,%lld] err %g scale %g",
                  (long long)n, (long long)k, err, (double)sf);
        }
    }
    if (zero_row >= 0 && zero_row < N)
        CHECK(scales[zero_row * G] == 0, "zero group scale bits %04x", scales[zero_row * G]);
    if (m8_row >= 0 && m8_row < N) {
        for (int64_t gi = 0; gi < G; ++gi) CHECK(scales[m8_row * G + gi] == 0x0001, "-8 row scale");
        for (int64_t k = 0; k < K; ++k) CHECK(q[m8_row * K + k] == -8, "-8 row code");
    }

    float *x = xmalloc(sizeof(float) * M * K), *bias = xmalloc(sizeof(float) * N);
    float *y = xmalloc(sizeof(float) * M * N);
    double *bound = xmalloc(sizeof(double) * M * N);
    for (int64_t i = 0; i < M * K; ++i) x[i] = next_weight();
    for (int64_t n = 0; n < N; ++n) bias[n] = next_weight();
    for (int relu = 0; relu < 2; ++relu) {
        int4_oracle_matmul_ex(x, M, packed, scales, NULL, N, K, g, bias, relu, y, bound);
        for (int64_t m = 0; m < M; ++m)
            for (int64_t n = 0; n < N; ++n) {
                double ref = 0.0, b = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    ref += (double)x[m * K + k] * (double)deq[n * K + k];
                    b += fabs((double)x[m * K + k] * (double)deq[n * K + k]);
                }
                ref += bias[n];
                if (relu && ref < 0.0) ref = 0.0;
                const double got = y[m * N + n];
                CHECK(fabs(got - ref) <= 1e-6 * (b + fabs((double)bias[n])) + 1e-30,
                      "matmul [%lld,%lld] %g vs %g", (long long)m, (long long)n, got, ref);
                CHECK(fabs(bound[m * N + n] - b) <= 1e-9 * b, "bound [%lld,%lld]", (long long)m, (long long)n);
            }
    }
    free(x); free(bias); free(y); free(bound);
    free(w); free(packed); free(scales); free(q); free(deq); free(deqh);
}

/* One affine case: codes in [0, 15] with a zero point per group. */
static void run_affine(int64_t N, int64_t K, int64_t g, int64_t M)
{
    const int64_t G = int4_oracle_num_groups(K, g), B = int4_oracle_packed_row_bytes(K);
    float *w = xmalloc(sizeof(float) * N * K);
    for (int64_t i = 0; i < N * K; ++i) w[i] = next_weight() + 0.3f;
    uint8_t *packed = xmalloc(N * B), *zeros = xmalloc(N * G);
    uint16_t *scales = xmalloc(sizeof(uint16_t) * N * G);
    float *deq = xmalloc(sizeof(float) * N * K);
    int4_oracle_quantize_affine(w, N, K, g, packed, scales, zeros);
    int4_oracle_dequantize(packed, scales, zeros, N, K, g, deq);
    for (int64_t n = 0; n < N; ++n) {
        if (K & 1) CHECK((packed[n * B + B - 1] >> 4) == 0, "affine pad nibble");
        for (int64_t gi = 0; gi < G; ++gi) CHECK(zeros[n * G + gi] <= 15, "zero point range");
        for (int64_t k = 0; k < K; ++k) {
            const int u = (packed[n * B + (k >> 1)] >> (4 * (k & 1))) & 0xF;
            const float sf = int4_oracle_float_from_half(scales[n * G + k / g]);
            CHECK(deq[n * K + k] == (float)(u - zeros[n * G + k / g]) * sf, "affine dequantize");
        }
    }
    float *x = xmalloc(sizeof(float) * M * K), *y = xmalloc(sizeof(float) * M * N);
    double *bound = xmalloc(sizeof(double) * M * N);
    for (int64_t i = 0; i < M * K; ++i) x[i] = next_weight();
    int4_oracle_matmul_ex(x, M, packed, scales, zeros, N, K, g, NULL, 0, y, bound);
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double ref = 0.0, b = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                ref += (double)x[m * K + k] * (double)deq[n * K + k];
                b += fabs((double)x[m * K + k] * (double)deq[n * K + k]);
            }
            CHECK(fabs((double)y[m * N + n] - ref) <= 1e-6 * b + 1e-30, "affine matmul");
        }
    free(x); free(y); free(bound); free(w); free(packed); free(zeros); free(scales); free(deq);
}

int main(void)
{
    /* the page's printed layout example: [[1,-1,7,-7]], group 4 -> scale 1.0, bytes F1 97 */
    {
        float *w = xmalloc(4 * sizeof(float));
        const float v[4] = {1.0f, -1.0f, 7.0f, -7.0f};
        memcpy(w, v, sizeof v);
        uint8_t *p = xmalloc(2);
        uint16_t *s = xmalloc(sizeof(uint16_t));
        int4_oracle_quantize(w, 1, 4, 4, p, s);
        CHECK(s[0] == 0x3C00 && p[0] == 0xF1 && p[1] == 0x97, "layout example: %04x %02x %02x", s[0], p[0], p[1]);
        free(w); free(p); free(s);
    }
    /* every byte value unpacks to the sign extension of its two nibbles */
    {
        uint8_t *p = xmalloc(256);
        int8_t *o = xmalloc(512);
        for (int b = 0; b < 256; ++b) p[b] = (uint8_t)b;
        int4_oracle_unpack(p, 1, 512, o);
        for (int b = 0; b < 256; ++b) {
            const int lo = b & 0xF, hi = b >> 4;
            CHECK(o[2 * b] == (lo >= 8 ? lo - 16 : lo) && o[2 * b + 1] == (hi >= 8 ? hi - 16 : hi), "byte %02x", b);
        }
        free(p); free(o);
    }
    run_case(64, 256, 128, 4, -1, -1);      /* the small random configuration */
    run_case(48, 301, 128, 3, 5, 7);        /* odd K, partial group, zero group, -8 codes */
    run_case(7, 33, 1, 2, 0, 3);
    run_case(5, 35, 3, 2, 1, -1);
    run_case(9, 37, 5, 3, 2, 4);
    run_case(6, 96, 32, 5, -1, 5);
    run_case(3, 17, 128, 2, 0, -1);         /* group larger than K */
    run_case(1, 1, 1, 1, -1, -1);           /* the smallest shape */
    run_affine(12, 301, 128, 3);
    run_affine(5, 33, 3, 2);
    run_affine(4, 64, 32, 2);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
