/*
 * fp4_oracle.c -- plain, slow, scalar CPU oracle for block-scaled FP4
 * quantization of bf16 tensors.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library. The product library never
 * links, includes or calls it, and it shares no source with the HIP kernels.
 *
 * What it follows (web pages on the method, cited by title and section):
 *   [TRACE-JA]  "TRACE ... ロールアウト誘導型QAT" summary (ai-papers.net):
 *               sections "学習とロールアウトの不一致", "TRACEの仕組み",
 *               "量子化情報キャッシュ".
 *   [TRACE-KO]  "TRACE: 롤아웃 유도형 양자화 인식 학습 ..." (sns.style):
 *               section "작동 원리의 공학적 이해".
 *   [FQT-FP4]   aibr.jp FP4 fully-quantized-training summary, section
 *               "3. 中核となる技術的要素" (NVFP4 = 16-value blocks of E2M1 with
 *               an E4M3 scale; round-to-nearest forward, stochastic rounding
 *               backward).
 *   [TETRAJET]  aibr.jp MXFP4 (TetraJet) summary, section
 *               "3. 中核となる技術的要素" (per-group scale).
 *   [UFP4]      UFP4 recipe page, sections "Random Hadamard Transform（RHT）
 *               の影響" and "UFP4 の設計と実装指針" (uniform E1M2/INT4 grid,
 *               RHT before quantizing).
 * Where the pages leave a step open, the readings are the ones listed in the
 * design notes of this repository; each function below states the one it uses.
 *
 * Arithmetic convention: every floating-point step is evaluated in double,
 * where it is exact, and rounded to fp32 (round-to-nearest-even) exactly at
 * the points the definition places a rounding, via rn32().  For a single
 * +, -, *, / of two fp32 operands, rounding the double result to fp32 gives
 * the correctly rounded fp32 result (double has more than 2*24+2 bits).
 *
 * Parity pins (see tests/test_oracle_*.py): grids, scale codecs, RTN, SR and
 * guided encodes, dequantization, the RHT and the MXFP4 matrix product are
 * pinned against closed forms, brute force and library routines.  Philox4x32-10 is pinned against rocRAND.
 * The RHT butterfly's rounding order is pinned only where every partial sum
 * is exact ("parity unpinned" beyond that: the order is a reading).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <float.h>

#define ORC_NVFP4 0
#define ORC_MXFP4 1
#define ORC_E2M1 0
#define ORC_UNIFORM 1
#define ORC_RTN 0
#define ORC_SR 1
#define ORC_GUIDED 2

typedef struct {
    int32_t format;     /* ORC_NVFP4 or ORC_MXFP4 */
    int32_t grid;       /* ORC_E2M1 or ORC_UNIFORM */
    int32_t rht16;      /* nonzero: 16-point random Hadamard transform first */
    int32_t reserved;
    uint64_t rht_seed;  /* Philox key of the RHT sign diagonal */
    uint64_t sr_seed;   /* Philox key of stochastic rounding */
    uint64_t sr_offset; /* counter offset, in 16-element groups */
} orc_cfg;

/* ------------------------------------------------------------------ */
/* rounding helpers                                                    */
/* ------------------------------------------------------------------ */

static float rn32(double x) { return (float)x; }

float orc_mul32(float a, float b) { return rn32((double)a * (double)b); }
float orc_div32(float a, float b) { return rn32((double)a / (double)b); }
float orc_add32(float a, float b) { return rn32((double)a + (double)b); }
float orc_sub32(float a, float b) { return rn32((double)a - (double)b); }

static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* fp32 -> bf16, round to nearest even; NaN -> canonical 0x7FC0. */
static uint16_t f32_to_bf16(float f) {
    if (isnan(f)) return 0x7FC0;
    uint32_t u;
    memcpy(&u, &f, 4);
    /* exact decision in integers: keep 16 bits, round half to even */
    uint32_t keep = u >> 16, rest = u & 0xFFFF;
    if (rest > 0x8000 || (rest == 0x8000 && (keep & 1))) keep += 1;
    return (uint16_t)keep;
}

/* ------------------------------------------------------------------ */
/* element grids [FQT-FP4 §3: E2M1 = 2 exponent bits, 1 mantissa bit;  */
/* UFP4: uniform E1M2 / INT4 grid]                                     */
/* ------------------------------------------------------------------ */

/* Magnitude of element code k (0..7).  E2M1 is read off its bit fields:
 * exponent bias 1, exponent 0 is subnormal (0.m x 2^0).  The uniform grid
 * is sign-magnitude INT4 with |q| <= 7. */
double orc_grid(int grid, int k) {
    if (grid == ORC_UNIFORM) return (double)k;
    int e = (k >> 1) & 3, m = k & 1;
    if (e == 0) return m * 0.5;
    return ldexp(1.0 + m * 0.5, e - 1);
}

double orc_grid_max(int grid) { return orc_grid(grid, 7); }

/* ------------------------------------------------------------------ */
/* scale codecs                                                        */
/* ------------------------------------------------------------------ */

/* OCP E4M3FN: bias 7, no infinities, S.1111.111 is NaN, max 448. */
double orc_e4m3_decode(unsigned code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = m * ldexp(1.0, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -v : v;
}

/* Non-negative t -> nearest E4M3 value, ties to the even code, anything above
 * the largest finite value saturates to 448.  Brute force over the table. */
unsigned orc_e4m3_encode(float t) {
    if (isnan(t)) return 0x7F;
    if (t >= 448.0f) return 0x7E;
    unsigned best = 0;
    double bestd = INFINITY;
    for (unsigned c = 0; c <= 0x7E; ++c) {
        double d = fabs(orc_e4m3_decode(c) - (double)t);
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            bestd = d;
            best = c;
        }
    }
    return best;
}

/* OCP E8M0: 2^(code-127), 0xFF is NaN. */
double orc_e8m0_decode(unsigned code) {
    if (code == 0xFF) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11)                   */
/* ------------------------------------------------------------------ */

void orc_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * c[0];
        uint64_t p1 = (uint64_t)M1 * c[2];
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
    memcpy(out, c, sizeof c);
}

/* Byte j (0..15) of the Philox output, little-endian across words w0..w3. */
static unsigned philox_byte(const uint32_t w[4], int j) {
    return (w[j >> 2] >> (8 * (j & 3))) & 0xFFu;
}

/* ------------------------------------------------------------------ */
/* 16-point random Hadamard transform [UFP4, RHT section]              */
/* ------------------------------------------------------------------ */

/* Sign diagonal: D_j = -1 iff bit j of word 0 of
 * Philox4x32-10(key = seed, counter = (0, 0, 1, 0)).  Returned as a 16-bit mask. */
uint32_t orc_rht_signs(uint64_t seed) {
    uint32_t ctr[4] = {0, 0, 1, 0};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    orc_philox4x32_10(ctr, key, w);
    return w[0] & 0xFFFFu;
}

/* Sylvester-ordered Hadamard butterfly: stages h = 1, 2, 4, 8, each pair
 * (i, i+h) with (i & h) == 0 replaced by (a_i + a_{i+h}, a_i - a_{i+h}),
 * each sum rounded to fp32. */
static void butterfly16(float a[16]) {
    for (int h = 1; h < 16; h <<= 1) {
        for (int i = 0; i < 16; ++i) {
            if (i & h) continue;
            float s = orc_add32(a[i], a[i + h]);
            float d = orc_sub32(a[i], a[i + h]);
            a[i] = s;
            a[i + h] = d;
        }
    }
}

/* forward: y = 1/4 * H16 * D * x ; inverse: x = D * (1/4 * H16 * y). */
void orc_rht16_vec(const float* x, uint32_t signs, int inverse, float* y) {
    float a[16];
    for (int j = 0; j < 16; ++j) {
        a[j] = x[j];
        if (!inverse && ((signs >> j) & 1)) a[j] = -a[j];
    }
    butterfly16(a);
    for (int j = 0; j < 16; ++j) {
        float v = orc_mul32(a[j], 0.25f);
        if (inverse && ((signs >> j) & 1)) v = -v;
        y[j] = v;
    }
}

/* Standalone transform of a bf16 matrix (rows x cols, row stride ld elements);
 * cols % 16 == 0.  Output is dense: fp32 (out_bf16 == 0) or bf16 RNE. */
void orc_rht16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, uint64_t seed,
               int inverse, int out_bf16, void* out) {
    uint32_t signs = orc_rht_signs(seed);
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c0 = 0; c0 < cols; c0 += 16) {
            float in[16], y[16];
            for (int j = 0; j < 16; ++j) in[j] = bf16_to_f32(x[r * ld + c0 + j]);
            orc_rht16_vec(in, signs, inverse, y);
            for (int j = 0; j < 16; ++j) {
                int64_t i = r * cols + c0 + j;
                if (out_bf16) ((uint16_t*)out)[i] = f32_to_bf16(y[j]);
                else ((float*)out)[i] = y[j];
            }
        }
    }
}

/* Load one row's group of 16 values starting at column c0, widened to fp32
 * and transformed when the configuration asks for the RHT. */
static void load_group(const orc_cfg* cfg, const uint16_t* row, int64_t c0, uint32_t signs, float y[16]) {
    float in[16];
    for (int j = 0; j < 16; ++j) in[j] = bf16_to_f32(row[c0 + j]);
    if (cfg->rht16) orc_rht16_vec(in, signs, 0, y);
    else memcpy(y, in, sizeof in);
}

static int block_size(const orc_cfg* cfg) { return cfg->format == ORC_MXFP4 ? 32 : 16; }

/* ------------------------------------------------------------------ */
/* tensor scale (NVFP4 and uniform grid with the NVFP4 block format)   */
/* ------------------------------------------------------------------ */

/* s_t = amax_t / (Gmax * 448), the denominator rounded first (it is exact),
 * one fp32 rounding of the quotient; amax over finite |y| only; an all-zero
 * (or all non-finite) tensor gives s_t = 1. */
float orc_tensor_scale(const orc_cfg* cfg, const uint16_t* x, int64_t rows, int64_t cols, int64_t ld) {
    uint32_t signs = orc_rht_signs(cfg->rht_seed);
    double amax = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c0 = 0; c0 < cols; c0 += 16) {
            float y[16];
            load_group(cfg, x + r * ld, c0, signs, y);
            for (int j = 0; j < 16; ++j) {
                if (!isfinite(y[j])) continue;
                double a = fabs((double)y[j]);
                if (a > amax) amax = a;
            }
        }
    }
    if (amax == 0.0) return 1.0f;
    float denom = rn32(orc_grid_max(cfg->grid) * 448.0);
    return orc_div32((float)amax, denom);
}

/* ------------------------------------------------------------------ */
/* block scale                                                         */
/* ------------------------------------------------------------------ */

/* From a block's (finite) amax, the stored scale code and the fp32
 * reciprocal multiplier inv used on the elements.
 *   NVFP4: t = RN(amax / RN(Gmax*s_t)); code = E4M3 RNE saturating;
 *          d = dec(code); S = RN(d*s_t); inv = 0 if S == 0 else RN(1/S),
 *          replaced by FLT_MAX when 1/S overflows.
 *   MXFP4: e = clamp(floor(log2 amax) - 2, -127, 127) (e = -127 for amax 0),
 *          code = e + 127, inv = 2^-e.                                      */
static float inv_from_nvfp4_code(unsigned code, float ts) {
    double d = orc_e4m3_decode(code & 0x7F);
    float S = orc_mul32((float)d, ts);
    if (S == 0.0f) return 0.0f;
    float inv = orc_div32(1.0f, S);
    if (isinf(inv)) inv = FLT_MAX;
    return inv;
}

static float inv_from_mx_code(unsigned code) {
    int e = (int)code - 127;
    return (float)ldexp(1.0, -e);
}

void orc_block_params(const orc_cfg* cfg, float amax, float ts, unsigned* code, float* inv) {
    if (cfg->format == ORC_MXFP4) {
        int e;
        if (amax == 0.0f) {
            e = -127;
        } else {
            int ex;
            frexp((double)amax, &ex); /* amax = f * 2^ex, f in [0.5, 1) */
            e = (ex - 1) - 2;         /* floor(log2 amax) - emax(2) */
            if (e < -127) e = -127;
            if (e > 127) e = 127;
        }
        *code = (unsigned)(e + 127);
        *inv = inv_from_mx_code(*code);
    } else {
        float denom = orc_mul32((float)orc_grid_max(cfg->grid), ts);
        float t = orc_div32(amax, denom);
        *code = orc_e4m3_encode(t);
        *inv = inv_from_nvfp4_code(*code, ts);
    }
}

/* Guided mode takes the block scale from the guide; returns 0 when the guide
 * scale is a NaN code. */
int orc_guided_params(const orc_cfg* cfg, unsigned code, float ts, float* inv) {
    if (cfg->format == ORC_MXFP4) {
        if (code == 0xFF) return 0;
        *inv = inv_from_mx_code(code);
    } else {
        if ((code & 0x7F) == 0x7F) return 0;
        *inv = inv_from_nvfp4_code(code, ts);
    }
    return 1;
}

/* ------------------------------------------------------------------ */
/* element encode                                                      */
/* ------------------------------------------------------------------ */

/* v >= 0 is the scaled magnitude RN(|y| * inv).  It is clamped to Gmax and
 * bracketed by the grid: lo = largest codeword <= vc, hi = smallest >= vc.
 *   RTN:    nearest of the two; exact midpoint goes to the even code.
 *           ([FQT-FP4 §3] forward rounding; [TRACE-JA] "nearest" baseline)
 *   SR:     f = (vc - lo) / (hi - lo); up iff (2u + 1) < 512 f, with u the
 *           element's random byte ([FQT-FP4 §3] backward rounding).
 *   GUIDED: of the two neighbours, the one whose code LSB equals the guide
 *           bit b; a value on a codeword keeps it ([TRACE-JA] "TRACEの仕組み":
 *           pick between the upper and lower adjacent codewords following the
 *           rollout; "量子化情報キャッシュ": the mantissa bit identifies it).
 * Returns the 3-bit magnitude code k. */
unsigned orc_encode(int grid, int mode, float v, unsigned aux) {
    double gmax = orc_grid_max(grid);
    double vc = (double)v > gmax ? gmax : (double)v;
    int klo = 0, khi = 7;
    for (int k = 0; k < 8; ++k)
        if (orc_grid(grid, k) <= vc) klo = k;
    for (int k = 7; k >= 0; --k)
        if (orc_grid(grid, k) >= vc) khi = k;
    if (klo == khi) return (unsigned)klo;
    double lo = orc_grid(grid, klo), hi = orc_grid(grid, khi);
    if (mode == ORC_RTN) {
        double mid = (lo + hi) / 2.0;
        if (vc < mid) return (unsigned)klo;
        if (vc > mid) return (unsigned)khi;
        return (unsigned)((klo % 2 == 0) ? klo : khi);
    }
    if (mode == ORC_SR) {
        double f = (vc - lo) / (hi - lo);
        return (double)(2 * aux + 1) < 512.0 * f ? (unsigned)khi : (unsigned)klo;
    }
    /* guided */
    return ((unsigned)klo & 1u) == (aux & 1u) ? (unsigned)klo : (unsigned)khi;
}

/* ------------------------------------------------------------------ */
/* quantize                                                            */
/* ------------------------------------------------------------------ */

/* Quantizes rows [row0, row0 + nrows) of a (rows x cols) bf16 tensor.
 *   x        -> first element of row row0; row stride ld elements
 *   ts       tensor scale (NVFP4 formats; ignored for MXFP4).  In guided
 *            mode it is the guide's tensor scale.
 *   gbits    guided mode: guide bitplane of these rows (bit i%8 of byte i/8)
 *   gscales  guided mode: guide block scales of these rows
 *   codes    nrows*cols/2 bytes: element i in nibble i%2 of byte i/2
 *   scales   nrows*cols/B bytes
 *   emit     optional (NULL): bitplane of the code LSBs (RTN/SR modes)
 * Element indices i are the logical row-major index r*cols + c of the whole
 * tensor (they pick the stochastic-rounding random bytes).
 * Non-finite input in a block: NaN scale code and all-zero codes (RTN/SR);
 * all-zero codes in guided mode, which copies the guide's scale byte. */
int orc_quantize(const orc_cfg* cfg, int mode, const uint16_t* x, int64_t row0, int64_t nrows,
                 int64_t cols, int64_t ld, float ts, const uint8_t* gbits, const uint8_t* gscales,
                 uint8_t* codes, uint8_t* scales, uint8_t* emit) {
    const int B = block_size(cfg);
    if (cols % B != 0) return 1;
    const uint32_t signs = orc_rht_signs(cfg->rht_seed);
    const uint32_t skey[2] = {(uint32_t)cfg->sr_seed, (uint32_t)(cfg->sr_seed >> 32)};
    const unsigned nan_code = cfg->format == ORC_MXFP4 ? 0xFFu : 0x7Fu;
    const int64_t nblk = cols / B;
    memset(codes, 0, (size_t)(nrows * cols / 2));
    if (emit) memset(emit, 0, (size_t)(nrows * cols / 8));
    for (int64_t r = 0; r < nrows; ++r) {
        const uint16_t* row = x + r * ld;
        for (int64_t b = 0; b < nblk; ++b) {
            float y[32];
            for (int g = 0; g < B; g += 16) load_group(cfg, row, b * B + g, signs, y + g);
            int finite = 1;
            float amax = 0.0f;
            for (int j = 0; j < B; ++j) {
                if (!isfinite(y[j])) finite = 0;
                else if (fabsf(y[j]) > amax) amax = fabsf(y[j]);
            }
            unsigned scode;
            float inv = 0.0f;
            int ok;
            const int64_t lblk = r * nblk + b; /* block index within these rows */
            if (mode == ORC_GUIDED) {
                scode = gscales[lblk];
                ok = orc_guided_params(cfg, scode, ts, &inv) && finite;
            } else if (!finite) {
                scode = nan_code;
                ok = 0;
            } else {
                orc_block_params(cfg, amax, ts, &scode, &inv);
                ok = 1;
            }
            scales[lblk] = (uint8_t)scode;
            for (int j = 0; j < B; ++j) {
                const int64_t li = r * cols + b * B + j;          /* local index */
                const int64_t gi = (row0 + r) * cols + b * B + j;  /* tensor index */
                unsigned code = 0;
                if (ok) {
                    float v = orc_mul32(fabsf(y[j]), inv);
                    unsigned aux = 0;
                    if (mode == ORC_SR) {
                        uint64_t g = (uint64_t)(gi / 16) + cfg->sr_offset;
                        uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), 0, 0};
                        uint32_t w[4];
                        orc_philox4x32_10(ctr, skey, w);
                        aux = philox_byte(w, (int)(gi % 16));
                    } else if (mode == ORC_GUIDED) {
                        aux = (gbits[li / 8] >> (li % 8)) & 1u;
                    }
                    unsigned k = orc_encode(cfg->grid, mode, v, aux);
                    code = (signbit(y[j]) ? 8u : 0u) | k;
                }
                codes[li / 2] |= (uint8_t)(code << (4 * (li % 2)));
                if (emit) emit[li / 8] |= (uint8_t)((code & 1u) << (li % 8));
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* dequantize [TRACE-KO: a block shares one scale, each value 4 bits]  */
/* ------------------------------------------------------------------ */

/* NVFP4: val = RN(RN(G[k] * d) * s_t) (the inner product is exact);
 * MXFP4: val = RN(G[k] * 2^e).  The code's sign bit is applied last.
 * A NaN scale code gives canonical NaN for its whole block.
 * out: dense rows*cols of fp32 (out_bf16 == 0) or bf16 (RNE of the fp32). */
void orc_dequantize(const orc_cfg* cfg, const uint8_t* codes, const uint8_t* scales, float ts,
                    int64_t rows, int64_t cols, int out_bf16, void* out) {
    const int B = block_size(cfg);
    const int64_t n = rows * cols;
    for (int64_t i = 0; i < n; ++i) {
        unsigned code = (codes[i / 2] >> (4 * (i % 2))) & 0xFu;
        unsigned s = scales[i / B];
        double g = orc_grid(cfg->grid, (int)(code & 7));
        float val;
        if (cfg->format == ORC_MXFP4) {
            if (s == 0xFF) val = NAN;
            else val = rn32(g * orc_e8m0_decode(s));
        } else {
            if ((s & 0x7F) == 0x7F) val = NAN;
            else {
                float gd = rn32(g * orc_e4m3_decode(s & 0x7F));
                val = orc_mul32(gd, ts);
            }
        }
        if (isnan(val)) {
            uint32_t qnan = 0x7FC00000u;
            memcpy(&val, &qnan, 4);
        } else if (code & 8) {
            val = -val;
        }
        if (out_bf16) ((uint16_t*)out)[i] = f32_to_bf16(val);
        else ((float*)out)[i] = val;
    }
}

/* ------------------------------------------------------------------ */
/* guidance cache [TRACE-JA "量子化情報キャッシュ": 1 mantissa bit +   */
/* the block scale per element]                                        */
/* ------------------------------------------------------------------ */

void orc_guide_pack(const orc_cfg* cfg, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                    int64_t cols, uint8_t* bits, uint8_t* gscales) {
    const int64_t n = rows * cols;
    memset(bits, 0, (size_t)(n / 8));
    for (int64_t i = 0; i < n; ++i) {
        unsigned code = (codes[i / 2] >> (4 * (i % 2))) & 0xFu;
        bits[i / 8] |= (uint8_t)((code & 1u) << (i % 8));
    }
    memcpy(gscales, scales, (size_t)(n / block_size(cfg)));
}

void orc_guide_unpack(const orc_cfg* cfg, const uint8_t* bits, const uint8_t* gscales, int64_t rows,
                      int64_t cols, uint8_t* mant, uint8_t* scales_out) {
    const int64_t n = rows * cols;
    for (int64_t i = 0; i < n; ++i) mant[i] = (bits[i / 8] >> (i % 8)) & 1u;
    memcpy(scales_out, gscales, (size_t)(n / block_size(cfg)));
}

/* ------------------------------------------------------------------ */
/* full-code guided diagnostic [TRACE-JA "量子化情報キャッシュ": one     */
/* mantissa bit names the rollout's codeword only when that codeword is */
/* one of the two that bracket the training value; other cases are the */
/* rare non-adjacent mismatches]                                        */
/* ------------------------------------------------------------------ */

/* The 1-bit guide is the LSB of each rollout code r and the guide scales are
 * the rollout's block scales; g is the guided result for x.  Blocks that
 * guided rounding does not encode (non-finite input after the RHT, NaN guide
 * scale) are left out.
 *   counts[0] = elements of the blocks taken into account,
 *   counts[1] = of those, |g| != |r| (non-adjacent: the bit cannot name r),
 *   counts[2] = of those, g != r (sign included).
 * Returns 0, or 1 for an invalid shape, 2 when out of memory. */
int orc_guide_mismatch(const orc_cfg* cfg, const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                       float ts, const uint8_t* rcodes, const uint8_t* rscales, uint64_t counts[3]) {
    const int B = block_size(cfg);
    if (cols % B != 0) return 1;
    const int64_t n = rows * cols, nblk = cols / B;
    counts[0] = counts[1] = counts[2] = 0;
    uint8_t* gbits = (uint8_t*)calloc((size_t)(n / 8 + 1), 1);
    uint8_t* gcodes = (uint8_t*)malloc((size_t)(n / 2 + 1));
    uint8_t* gscales = (uint8_t*)malloc((size_t)(n / B + 1));
    if (!gbits || !gcodes || !gscales) {
        free(gbits); free(gcodes); free(gscales);
        return 2;
    }
    for (int64_t i = 0; i < n; ++i) {
        unsigned r = (rcodes[i / 2] >> (4 * (i % 2))) & 0xFu;
        gbits[i / 8] |= (uint8_t)((r & 1u) << (i % 8));
    }
    orc_quantize(cfg, ORC_GUIDED, x, 0, rows, cols, ld, ts, gbits, rscales, gcodes, gscales, NULL);
    const uint32_t signs = orc_rht_signs(cfg->rht_seed);
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nblk; ++b) {
            float y[32], inv;
            int finite = 1;
            for (int g = 0; g < B; g += 16) load_group(cfg, x + r * ld, b * B + g, signs, y + g);
            for (int j = 0; j < B; ++j) finite = finite && isfinite(y[j]);
            if (!finite || !orc_guided_params(cfg, rscales[r * nblk + b], ts, &inv)) continue;
            for (int j = 0; j < B; ++j) {
                const int64_t i = r * cols + b * B + j;
                const unsigned rc = (rcodes[i / 2] >> (4 * (i % 2))) & 0xFu;
                const unsigned gc = (gcodes[i / 2] >> (4 * (i % 2))) & 0xFu;
                counts[0] += 1;
                counts[1] += (rc & 7u) != (gc & 7u);
                counts[2] += rc != gc;
            }
        }
    }
    free(gbits); free(gcodes); free(gscales);
    return 0;
}

/* ------------------------------------------------------------------ */
/* MXFP4 matrix product [TETRAJET §3-4: matrix products whose operands  */
/* are both FP4 values with per-group scales]                          */
/* ------------------------------------------------------------------ */

/* Value of element i of an MXFP4 tensor with blocks of 32 along its rows:
 * (-1)^sign * G[k] * 2^(e - 127), exact in double; NaN for a 0xFF scale. */
static double mx_value(const uint8_t* codes, const uint8_t* scales, int64_t i) {
    unsigned code = (codes[i / 2] >> (4 * (i % 2))) & 0xFu;
    double v = orc_grid(ORC_E2M1, (int)(code & 7)) * orc_e8m0_decode(scales[i / 32]);
    return (code & 8) ? -v : v;
}

/* C[m][n] = sum over k of a(m,k) * b(n,k), where a is the [M, K] tensor whose
 * MXFP4 codes and scales are a_codes / a_scales (the layouts the quantizer
 * writes for a row-major [M, K] input) and b likewise the [N, K] tensor of
 * b_codes / b_scales: the product A * B^T with the reduction along the
 * blocked dimension.  Both operands are first decoded to double (exact), then
 * every product is exact in double and the sum runs in k order in double.
 * absdot (may be NULL) receives sum over k of |a(m,k) b(n,k)|, the scale of
 * the rounding error any fp32 summation may make.
 * Returns 0, 1 when K is not a multiple of 32, 2 when out of memory. */
int orc_gemm_mx(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, double* c, double* absdot) {
    if (K % 32 != 0) return 1;
    double* av = (double*)malloc((size_t)(M * K + 1) * sizeof(double));
    double* bv = (double*)malloc((size_t)(N * K + 1) * sizeof(double));
    if (!av || !bv) {
        free(av); free(bv);
        return 2;
    }
    for (int64_t i = 0; i < M * K; ++i) av[i] = mx_value(a_codes, a_scales, i);
    for (int64_t i = 0; i < N * K; ++i) bv[i] = mx_value(b_codes, b_scales, i);
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double prod = av[m * K + k] * bv[n * K + k];
                acc += prod;
                mag += fabs(prod);
            }
            c[m * N + n] = acc;
            if (absdot) absdot[m * N + n] = mag;
        }
    }
    free(av); free(bv);
    return 0;
}

/* ------------------------------------------------------------------ */
/* exhaustive-scan helper for the element encode                       */
/* ------------------------------------------------------------------ */

/* Scans the fp32 bit patterns p in (lo, hi] and writes each p whose encode
 * differs from that of p-1 (breakpoints of the piecewise-constant encode),
 * up to cap entries.  Returns the number found (may exceed cap). */
int64_t orc_encode_breakpoints(int grid, int mode, unsigned aux, uint32_t lo, uint32_t hi,
                               uint32_t* out, int64_t cap) {
    int64_t n = 0;
    float f;
    memcpy(&f, &lo, 4);
    unsigned prev = orc_encode(grid, mode, f, aux);
    for (uint64_t p = (uint64_t)lo + 1; p <= hi; ++p) {
        uint32_t u = (uint32_t)p;
        memcpy(&f, &u, 4);
        unsigned k = orc_encode(grid, mode, f, aux);
        if (k != prev) {
            if (n < cap) out[n] = u;
            ++n;
        }
        prev = k;
    }
    return n;
}

/* Element encode of n pre-scaled magnitudes v[i] >= 0 with aux[i] (SR byte or
 * guide bit); writes the 3-bit magnitude codes. */
void orc_encode_many(int grid, int mode, const float* v, const uint32_t* aux, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_encode(grid, mode, v[i], aux ? aux[i] : 0u);
}
