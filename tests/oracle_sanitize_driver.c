/* Runs every entry point of the CPU oracle on the kinds of input its pins use
 * (ragged and padded shapes, empty tensors, both formats and grids, the RHT, all
 * three rounding modes, non-finite and extreme blocks, NaN guide and operand
 * scales) with exactly sized heap buffers, so that an AddressSanitizer /
 * UndefinedBehaviorSanitizer build reports any out-of-bounds access or undefined
 * operation.  A few invariants are checked on the way: guided rounding with the
 * tensor's own RTN guide equals RTN, guide unpack inverts guide pack, and rows
 * quantized on their own equal the same rows of the whole tensor.
 * Test infrastructure: built and run by tests/test_oracle_sanitized.py. */
#include "../oracle/fp4_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {   /* xorshift64* */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}
static double next_unit(void) { return (double)(next_u64() >> 11) * (1.0 / 9007199254740992.0); }

static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static int failures = 0;
#define CHECK(cond, ...)                          \
    do {                                          \
        if (!(cond)) {                            \
            fprintf(stderr, "FAIL: " __VA_ARGS__); \
            fprintf(stderr, "\n");                \
            ++failures;                           \
        }                                         \
    } while (0)

/* rows x ld bf16 tensor (the first cols of each row used); special values in a few blocks */
static uint16_t* make_tensor(int64_t rows, int64_t cols, int64_t ld, int special) {
    uint16_t* x = (uint16_t*)xmalloc((size_t)(rows * ld) * sizeof(uint16_t));
    for (int64_t i = 0; i < rows * ld; ++i) {
        const double g = (next_unit() + next_unit() + next_unit() - 1.5) * 2.0;
        const double out = next_unit() < 0.01 ? 50.0 : 1.0;
        x[i] = to_bf16((float)(g * out));
    }
    if (special && rows > 0 && cols >= 32) {
        x[0] = to_bf16(NAN);
        x[17] = to_bf16(INFINITY);
        if (rows > 1) {
            for (int j = 0; j < 16; ++j) x[ld + j] = 0;                 /* an all-zero block */
            x[ld + 16] = to_bf16(-0.0f);
            x[ld + 20] = to_bf16(3.0e38f);
            x[ld + 21] = to_bf16(1.0e-40f);
        }
    }
    return x;
}

static void run_config(int format, int grid, int rht, int64_t rows, int64_t cols, int64_t pad, int special) {
    const int B = format == ORC_MXFP4 ? 32 : 16;
    if (cols % B) return;
    const int64_t ld = cols + pad, n = rows * cols;
    orc_cfg cfg = {format, grid, rht, 0, 7, 5, 3};
    uint16_t* x = make_tensor(rows, cols, ld, special);
    uint16_t* xr = make_tensor(rows, cols, ld, 0);
    const float ts = format == ORC_NVFP4 ? orc_tensor_scale(&cfg, xr, rows, cols, ld) : 1.0f;
    (void)orc_tensor_scale(&cfg, x, rows, cols, ld);
    uint8_t* codes = (uint8_t*)xmalloc((size_t)(n / 2));
    uint8_t* scales = (uint8_t*)xmalloc((size_t)(n / B));
    uint8_t* bits = (uint8_t*)xmalloc((size_t)(n / 8));
    uint8_t* gcodes = (uint8_t*)xmalloc((size_t)(n / 2));
    uint8_t* gscales = (uint8_t*)xmalloc((size_t)(n / B));
    uint8_t* gbits = (uint8_t*)xmalloc((size_t)(n / 8));
    uint8_t* mant = (uint8_t*)xmalloc((size_t)n);
    uint8_t* so = (uint8_t*)xmalloc((size_t)(n / B));
    float* dq = (float*)xmalloc((size_t)n * sizeof(float));
    uint16_t* dqb = (uint16_t*)xmalloc((size_t)n * sizeof(uint16_t));
    for (int mode = ORC_RTN; mode <= ORC_SR; ++mode) {
        CHECK(orc_quantize(&cfg, mode, x, 0, rows, cols, ld, ts, NULL, NULL, codes, scales, bits) == 0, "quantize");
        orc_dequantize(&cfg, codes, scales, ts, rows, cols, 0, dq);
        orc_dequantize(&cfg, codes, scales, ts, rows, cols, 1, dqb);
        /* rows on their own equal the same rows of the whole tensor */
        if (rows > 2) {
            const int64_t r0 = rows / 2, nr = rows - r0;
            uint8_t* c2 = (uint8_t*)xmalloc((size_t)(nr * cols / 2));
            uint8_t* s2 = (uint8_t*)xmalloc((size_t)(nr * cols / B));
            CHECK(orc_quantize(&cfg, mode, x + r0 * ld, r0, nr, cols, ld, ts, NULL, NULL, c2, s2, NULL) == 0, "rows");
            CHECK(memcmp(c2, codes + r0 * cols / 2, (size_t)(nr * cols / 2)) == 0, "row subset codes");
            CHECK(memcmp(s2, scales + r0 * cols / B, (size_t)(nr * cols / B)) == 0, "row subset scales");
            free(c2);
            free(s2);
        }
    }
    /* rollout RTN with emission, its guide, and guided rounding */
    CHECK(orc_quantize(&cfg, ORC_RTN, xr, 0, rows, cols, ld, ts, NULL, NULL, codes, scales, bits) == 0, "rtn");
    orc_guide_pack(&cfg, codes, scales, rows, cols, gbits, gscales);
    CHECK(memcmp(gbits, bits, (size_t)(n / 8)) == 0, "emission equals guide_pack");
    orc_guide_unpack(&cfg, gbits, gscales, rows, cols, mant, so);
    for (int64_t i = 0; i < n; ++i) CHECK(mant[i] == ((gbits[i / 8] >> (i % 8)) & 1u), "unpack");
    CHECK(memcmp(so, gscales, (size_t)(n / B)) == 0, "unpack scales");
    CHECK(orc_quantize(&cfg, ORC_GUIDED, xr, 0, rows, cols, ld, ts, gbits, gscales, gcodes, scales, NULL) == 0, "g");
    CHECK(memcmp(gcodes, codes, (size_t)(n / 2)) == 0, "own RTN guide reproduces RTN");
    CHECK(orc_quantize(&cfg, ORC_GUIDED, x, 0, rows, cols, ld, ts, gbits, gscales, gcodes, scales, NULL) == 0, "g2");
    /* NaN guide scales */
    if (n / B > 0) gscales[0] = format == ORC_MXFP4 ? 0xFF : 0x7F;
    CHECK(orc_quantize(&cfg, ORC_GUIDED, x, 0, rows, cols, ld, ts, gbits, gscales, gcodes, scales, NULL) == 0, "g3");
    uint64_t counts[3];
    CHECK(orc_guide_mismatch(&cfg, x, rows, cols, ld, ts, codes, gscales, counts) == 0, "mismatch");
    /* standalone RHT, forward and inverse, fp32 and bf16 output */
    if (cols % 16 == 0) {
        orc_rht16(x, rows, cols, ld, cfg.rht_seed, 0, 0, dq);
        orc_rht16(x, rows, cols, ld, cfg.rht_seed, 1, 1, dqb);
    }
    free(x);
    free(xr);
    free(codes);
    free(scales);
    free(bits);
    free(gcodes);
    free(gscales);
    free(gbits);
    free(mant);
    free(so);
    free(dq);
    free(dqb);
}

static void run_gemm(int64_t M, int64_t N, int64_t K) {
    uint8_t* a = (uint8_t*)xmalloc((size_t)(M * K / 2));
    uint8_t* as = (uint8_t*)xmalloc((size_t)(M * K / 32));
    uint8_t* b = (uint8_t*)xmalloc((size_t)(N * K / 2));
    uint8_t* bs = (uint8_t*)xmalloc((size_t)(N * K / 32));
    for (int64_t i = 0; i < M * K / 2; ++i) a[i] = (uint8_t)next_u64();
    for (int64_t i = 0; i < N * K / 2; ++i) b[i] = (uint8_t)next_u64();
    for (int64_t i = 0; i < M * K / 32; ++i) as[i] = (uint8_t)(110 + next_u64() % 40);
    for (int64_t i = 0; i < N * K / 32; ++i) bs[i] = (uint8_t)(110 + next_u64() % 40);
    if (M * K / 32 > 0) as[0] = 0xFF;
    if (N * K / 32 > 1) bs[1] = 0;
    double* c = (double*)xmalloc((size_t)(M * N) * sizeof(double));
    double* mag = (double*)xmalloc((size_t)(M * N) * sizeof(double));
    CHECK(orc_gemm_mx(a, as, b, bs, M, N, K, c, mag) == 0, "gemm");
    CHECK(orc_gemm_mx(a, as, b, bs, M, N, K, c, NULL) == 0, "gemm without magnitudes");
    free(a);
    free(as);
    free(b);
    free(bs);
    free(c);
    free(mag);
}

int main(void) {
    const int64_t shapes[][3] = {{0, 32, 0}, {1, 16, 0}, {1, 32, 8}, {3, 48, 0}, {5, 64, 16},
                                 {37, 544, 24}, {129, 96, 8}, {256, 512, 0}};
    for (int f = 0; f < 2; ++f)
        for (int g = 0; g < 2; ++g)
            for (int r = 0; r < 2; ++r)
                for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s)
                    run_config(f, g, r, shapes[s][0], shapes[s][1], shapes[s][2], s % 2);
    run_gemm(3, 5, 64);
    run_gemm(33, 17, 96);
    run_gemm(1, 1, 32);
    /* codecs and generators over their whole domains */
    for (unsigned c = 0; c < 256; ++c) {
        (void)orc_e4m3_decode(c);
        (void)orc_e8m0_decode(c);
    }
    for (uint32_t p = 0; p < 0x7F800000u; p += 0x3FFu) {
        float f;
        memcpy(&f, &p, 4);
        if (f <= 448.0f) (void)orc_e4m3_encode(f);
    }
    uint32_t brk[64];
    for (int mode = 0; mode < 3; ++mode)
        for (int g = 0; g < 2; ++g) (void)orc_encode_breakpoints(g, mode, 77, 0x3E000000u, 0x3E100000u, brk, 64);
    float v[64];
    uint32_t aux[64];
    uint8_t out[64];
    for (int i = 0; i < 64; ++i) {
        v[i] = (float)(next_unit() * 9.0);
        aux[i] = (uint32_t)(next_u64() & 0xFF);
    }
    for (int mode = 0; mode < 3; ++mode) orc_encode_many(0, mode, v, aux, out, 64);
    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, w[4];
    orc_philox4x32_10(ctr, key, w);
    (void)orc_rht_signs(0xFFFFFFFFFFFFFFFFull);
    if (failures) {
        fprintf(stderr, "%d invariant failures\n", failures);
        return 1;
    }
    printf("oracle sanitize driver ok\n");
    return 0;
}
