/*
 * fp4q.h -- C ABI of the MI355X (gfx950) block-scaled FP4 quantization library.
 *
 * The operations follow these web pages on the method:
 *   [TRACE-JA] ai-papers.net summary "TRACE ... ロールアウト誘導型QAT",
 *              sections "TRACEの仕組み" (guided rounding: pick the upper or
 *              lower adjacent codeword the rollout chose) and
 *              "量子化情報キャッシュ" (keep 1 mantissa bit + the block scale,
 *              deep layers only, about 1/6 of the full record).
 *   [TRACE-KO] sns.style summary, section "작동 원리의 공학적 이해": a few
 *              values share one scale, each value is 4 bits, the rounding
 *              direction is a per-value choice; the rollout engine exports its
 *              quantization result and the trainer consumes it.
 *   [FQT-FP4]  aibr.jp FP4 training summary, section 3: NVFP4 = 16-value
 *              blocks of E2M1 with an E4M3 scale; round-to-nearest forward,
 *              stochastic rounding backward.
 *   [TETRAJET] aibr.jp MXFP4 summary, section 3: per-group scale.
 *   [UFP4]     UFP4 recipe page, RHT and uniform-grid sections.
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers owned by the caller; the library
 *     allocates nothing, keeps no pointer after returning and never
 *     synchronizes.  Work is enqueued asynchronously on `stream` (NULL = the
 *     default stream); buffers must stay valid until the stream reaches it.
 *   - bf16 inputs are row-major [rows, cols] with row stride `ld` elements
 *     (ld >= cols, ld % 8 == 0, base 16-byte aligned).  Outputs are dense.
 *   - Element index i = r*cols + c (independent of ld) orders codes, guide
 *     bits and the stochastic-rounding random stream.
 *   - Packed codes: uint8[rows*cols/2], element i in nibble i%2 of byte i/2;
 *     a code is sign<<3 | k, k the 3-bit magnitude index on the grid.
 *   - Block scales: uint8[rows*cols/B], one per block of B consecutive
 *     elements of a row (B = 16 NVFP4, 32 MXFP4).  NVFP4: OCP E4M3FN code;
 *     MXFP4: E8M0 biased exponent.  0x7F (E4M3) / 0xFF (E8M0) mark a block
 *     that held a non-finite value; its codes are all zero.
 *   - Guide bitplane: uint8[rows*cols/8], bit i%8 of byte i/8 = LSB of k_i.
 *   - Device pointer alignment: x, codes, guide bits, dequant output and
 *     unpack output 16 bytes; scales 1 byte; tensor scales 4 bytes.
 *   - Errors are detected on the host before any launch and returned as an
 *     fp4_status; nothing is launched then.  A failed launch returns
 *     FP4_ERR_HIP.  fp4_last_error() gives the message (per thread).
 *   - rows*cols == 0 is a no-op that returns FP4_OK.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP4_OK = 0,
    FP4_ERR_ARG = 1,         /* null pointer, unknown enum, negative size */
    FP4_ERR_SHAPE = 2,       /* cols % B != 0, ld < cols, too many elements */
    FP4_ERR_ALIGN = 3,       /* misaligned pointer or ld % 8 != 0 */
    FP4_ERR_UNSUPPORTED = 4, /* combination not provided */
    FP4_ERR_HIP = 5          /* the HIP runtime reported an error */
} fp4_status;

typedef enum { FP4_NVFP4 = 0, FP4_MXFP4 = 1 } fp4_format;
typedef enum { FP4_GRID_E2M1 = 0, FP4_GRID_UNIFORM = 1 } fp4_grid;
typedef enum { FP4_RTN = 0, FP4_SR = 1 } fp4_rounding;
typedef enum { FP4_OUT_F32 = 0, FP4_OUT_BF16 = 1 } fp4_dtype;
typedef enum { FP4_MODE_RTN = 0, FP4_MODE_SR = 1, FP4_MODE_GUIDED = 2 } fp4_mode;

/* Quantizer configuration (48 bytes: 4 bytes of padding at the end).
 *   format   fp4_format: NVFP4 (16-blocks, E4M3 scale, fp32 tensor scale
 *            [FQT-FP4 §3]) or MXFP4 (32-blocks, E8M0 scale [TETRAJET §3]).
 *   grid     fp4_grid: E2M1 {0,.5,1,1.5,2,3,4,6} or the uniform INT4 grid
 *            {0..7} [UFP4].
 *   rounding fp4_rounding, used by fp4_quantize only.
 *   rht16    nonzero: apply y = 1/4 H16 D x to each 16-group first [UFP4].
 *   sr_seed  Philox4x32-10 key of stochastic rounding; sr_offset is added to
 *            the 16-element group index to form the counter.
 *   rht_seed Philox4x32-10 key of the RHT sign diagonal D.
 *   stream_out  0: the quantizers' outputs (codes, scales, guide bits,
 *            fake-quantized values) are written through the caches, where a
 *            kernel that reads them next finds them (the default).  1: they
 *            are written with non-temporal stores, for outputs that are not
 *            read again soon (a GEMM operand quantized ahead of its product,
 *            gradients quantized with SR): 6-8% faster for a 16384 x 4096
 *            quantize, 8% slower for a chain whose next kernel reads them.
 *            The result is the same bit for bit.  Other values: FP4_ERR_ARG. */
typedef struct {
    int32_t format;
    int32_t grid;
    int32_t rounding;
    int32_t rht16;
    uint64_t sr_seed;
    uint64_t sr_offset;
    uint64_t rht_seed;
    int32_t stream_out;   /* 0 or 1: see below */
} fp4_cfg;

/* Tensor scale for the NVFP4 block format [FQT-FP4 §3 E4M3 block scales
 * under one fp32 tensor scale]: s_t = amax / (Gmax*448), amax the largest
 * finite |y| of the tensor (y = x, or the RHT of x when cfg->rht16), and
 * s_t = 1 for an all-zero tensor.  Writes one float to tensor_scale_out
 * (device, also used as the reduction accumulator). */
fp4_status fp4_tensor_scale(const fp4_cfg* cfg, const void* x_bf16, int64_t rows, int64_t cols,
                            int64_t ld, float* tensor_scale_out, hipStream_t stream);

/* The same tensor scale in one launch [FQT-FP4 §3]: every workgroup stores its
 * partial maximum in a word of `workspace` tagged with the call's epoch, and
 * workgroup 0 waits until all are tagged, reduces them and writes s_t, bit for
 * bit equal to fp4_tensor_scale.
 *   workspace        device memory of at least fp4_tensor_scale_workspace_bytes()
 *                    (FP4_TENSOR_SCALE_WORKSPACE_BYTES), 256-byte aligned, owned by the
 *                    caller and zero-filled before its first use; every call leaves it
 *                    ready for the next one (it advances the epoch count kept there).
 *                    Calls that may run at the same time need workspaces of their own.
 *   workspace_bytes  its size; FP4_ERR_ARG when too small. */
#define FP4_TENSOR_SCALE_WORKSPACE_BYTES 24576
fp4_status fp4_tensor_scale_ws(const fp4_cfg* cfg, const void* x_bf16, int64_t rows, int64_t cols,
                               int64_t ld, float* tensor_scale_out, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);
size_t fp4_tensor_scale_workspace_bytes(void);

/* fp4_tensor_scale_ws without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static array of
 * 16 KiB that the library holds on each GPU it runs on until the process ends;
 * this call allocates nothing.  That size serves every
 * input the other entry points accept (the launch has at most 1024 workgroups);
 * larger inputs fail with FP4_ERR_SHAPE as everywhere.  Calls on one GPU share
 * its array: every completed call leaves it ready for the next, and calls that
 * overlap in time on one GPU (several streams, several host threads) race, with
 * undefined results for them and for later calls.  Same result as
 * fp4_tensor_scale, bit for bit. */
fp4_status fp4_tensor_scale_noalloc(const fp4_cfg* cfg, const void* x_bf16, int64_t rows, int64_t cols,
                                    int64_t ld, float* tensor_scale_out, hipStream_t stream);

/* Block quantization with round-to-nearest-even or stochastic rounding
 * [FQT-FP4 §3; TRACE-KO].  Per block: NVFP4 scale code = E4M3 RNE of
 * amax / RN(Gmax*s_t), saturating at 448, elements multiplied by
 * RN(1/RN(dec(code)*s_t)); MXFP4 scale exponent e = floor(log2 amax) - 2,
 * elements multiplied by 2^-e.  Scaled magnitudes are clamped to Gmax and
 * rounded to the grid: RTN ties to the even code; SR rounds up iff
 * 2u+1 < 512 f, u the element's byte (i%16) of Philox4x32-10(key = sr_seed,
 * counter = (i/16 + sr_offset, 0, 0)), f its position in the bracket.
 *   tensor_scale   NVFP4: device pointer to s_t (positive, finite);
 *                  MXFP4: ignored (may be NULL).
 *   codes, scales  outputs (see conventions).
 *   guide_bits_out NULL, or the guide bitplane of the result, emitted in the
 *                  same pass (rollout side of [TRACE-JA] "量子化情報キャッシュ"). */
fp4_status fp4_quantize(const fp4_cfg* cfg, const void* x_bf16, int64_t rows, int64_t cols,
                        int64_t ld, const float* tensor_scale, void* codes, void* scales,
                        void* guide_bits_out, hipStream_t stream);

/* NVFP4 tensor scale and block quantization of one tensor together
 * [FQT-FP4 §3 E4M3 block scales under one fp32 tensor scale]: writes s_t to
 * tensor_scale_out exactly as fp4_tensor_scale does, and codes, scales (and the
 * guide bits when guide_bits_out is not NULL) exactly as fp4_quantize does with
 * that s_t, RTN or SR.  Without the RHT, and when the device holds every
 * workgroup of the launch at once (up to 2048 workgroups of 512 groups on an
 * MI355X: about 16.7M elements), this is one launch: each workgroup stores the
 * maximum of its own chunk in a word of `workspace`, workgroup 0 reduces those
 * words and publishes s_t, and each workgroup quantizes the chunk it holds in
 * registers.  Otherwise it is fp4_tensor_scale_ws followed by fp4_quantize (two
 * launches).
 *   cfg              NVFP4 (MXFP4: FP4_ERR_UNSUPPORTED), RTN or SR.
 *   workspace        as for fp4_tensor_scale_ws: at least
 *                    FP4_TENSOR_SCALE_WORKSPACE_BYTES, 256-byte aligned, zero-filled
 *                    before first use; concurrent calls need their own.  Every call
 *                    leaves the reduction words of fp4_tensor_scale_ws zeroed; the
 *                    one-launch form keeps an epoch count there and words tagged with
 *                    it, for the next call (zero-filling the workspace again is always
 *                    valid).
 *   launches         NULL, or receives 1 or 2, the number of launches enqueued.
 * The one-launch form needs all its workgroups running together: work that
 * keeps compute units busy for more than about a second while it runs (another
 * stream) makes the waiting workgroups give up (fp4_set_wait_limit): s_t is then
 * NaN, and the codes and scales of the blocks those workgroups quantize under
 * it mean nothing. */
fp4_status fp4_quantize_with_tensor_scale(const fp4_cfg* cfg, const void* x_bf16, int64_t rows, int64_t cols,
                                          int64_t ld, float* tensor_scale_out, void* codes, void* scales,
                                          void* guide_bits_out, void* workspace, size_t workspace_bytes,
                                          int* launches, hipStream_t stream);

/* The number of polls a workgroup that waits on the others of its launch (the
 * gather of fp4_tensor_scale_ws and fp4_tensor_scale_noalloc, and both waits of
 * the one-launch fp4_quantize_with_tensor_scale) makes before it gives up:
 * FP4_WAIT_LIMIT_DEFAULT (2^20 polls, about a second) unless changed.  A wait
 * that gives up writes s_t = NaN instead of hanging (and, in the one-launch
 * quantize, the workgroup goes on with that s_t) and marks the launch in the
 * workspace, so that its workgroups that start later store nothing; the
 * workspace stays valid for the next call.  For tests of that path (0: every wait gives up at once) and
 * for callers that bound their latency.  Applies to launches enqueued after the
 * call, process-wide; returns the previous limit. */
#define FP4_WAIT_LIMIT_DEFAULT 1048576u
uint32_t fp4_set_wait_limit(uint32_t polls);

/* Rollout-guided quantization [TRACE-JA "TRACEの仕組み"; TRACE-KO]: the
 * block scale (and NVFP4 tensor scale) come from the guide; each element is
 * rounded to the one of its two bracketing codewords whose LSB equals its
 * guide bit (a value on a codeword keeps it).  `scales` receives a copy of
 * guide_scales.  A block whose guide scale is a NaN code, or whose input
 * holds a non-finite value, gets all-zero codes. */
fp4_status fp4_quantize_guided(const fp4_cfg* cfg, const void* x_bf16, int64_t rows,
                               int64_t cols, int64_t ld, const void* guide_bits,
                               const void* guide_scales, const float* guide_tensor_scale,
                               void* codes, void* scales, hipStream_t stream);

/* One tensor of a grouped call (fields as in fp4_quantize / fp4_quantize_guided). */
typedef struct {
    const void* x;              /* bf16 [rows, cols], row stride ld elements */
    int64_t rows;
    int64_t cols;
    int64_t ld;
    const float* tensor_scale;  /* NVFP4: s_t, or the guide's s_t when guided; else ignored */
    void* codes;                /* output codes */
    void* scales;               /* output scales */
    void* guide_bits;           /* RTN/SR: fused emission output or NULL; guided: guide bits input */
    const void* guide_scales;   /* guided: guide scales input; otherwise ignored */
} fp4_tensor;

#define FP4_MAX_GROUP 16

/* Several tensors sharing one configuration in a single launch, e.g. the routed
 * experts' weight slices and the activations of one MoE layer [TRACE-JA
 * 実験結果: MoE models; TRACE-JA 量子化情報キャッシュ: every quantization
 * point of a deep layer].  Equivalent to calling fp4_quantize (guided == 0,
 * rounding from cfg) or fp4_quantize_guided (guided != 0) on each tensor in
 * turn with the same cfg: each tensor's element index, and so its
 * stochastic-rounding counter, starts at 0.
 *   n        1 .. FP4_MAX_GROUP
 *   tensors  HOST array of n descriptors; validated like the single calls.
 * With guided == 0 either every tensor gives guide_bits (fused emission) or
 * none does. */
fp4_status fp4_quantize_grouped(const fp4_cfg* cfg, int guided, int n, const fp4_tensor* tensors,
                                hipStream_t stream);

/* Fake quantization for quantization-aware training [TRACE-JA "TRACEの仕組み":
 * the trainer's forward pass uses the chosen quantized value; FQT-FP4 §3]:
 * out = bf16 dequantization of the codes that fp4_quantize (guided == 0,
 * rounding from cfg) or fp4_quantize_guided (guided != 0) would produce,
 * computed in one pass without writing codes.  Bit for bit equal to calling
 * the quantize entry point and then fp4_dequantize with FP4_OUT_BF16.
 *   tensor_scale  NVFP4: s_t (guided: the guide's s_t); MXFP4: ignored
 *   guide_bits, guide_scales  guided only (may be NULL otherwise)
 *   out_bf16      [rows, cols] with row stride ld_out (>= cols, % 8 == 0),
 *                 16-byte aligned. */
fp4_status fp4_fake_quantize(const fp4_cfg* cfg, int guided, const void* x_bf16, int64_t rows,
                             int64_t cols, int64_t ld, const float* tensor_scale,
                             const void* guide_bits, const void* guide_scales, void* out_bf16,
                             int64_t ld_out, hipStream_t stream);

/* Dequantization [TRACE-KO: shared block scale, 4-bit values]:
 * NVFP4 val = RN(RN(G[k]*dec(scale))*s_t); MXFP4 val = G[k]*2^e; the code's
 * sign applied; fp32 output, or bf16 by round-to-nearest-even of that fp32.
 * A NaN scale code gives the canonical quiet NaN for its block.
 * out: [rows, cols] with row stride ld_out elements (ld_out >= cols,
 * ld_out*size % 16 == 0). */
fp4_status fp4_dequantize(const fp4_cfg* cfg, const void* codes, const void* scales,
                          const float* tensor_scale, int64_t rows, int64_t cols, void* out,
                          int64_t ld_out, fp4_dtype dtype, hipStream_t stream);

/* Guidance-cache packing [TRACE-JA "量子化情報キャッシュ"; TRACE-KO
 * "가수와 스케일"]: guide bit i = LSB of code i, guide_scales = scales. */
fp4_status guide_pack(const fp4_cfg* cfg, const void* codes, const void* scales, int64_t rows,
                      int64_t cols, void* guide_bits, void* guide_scales, hipStream_t stream);

/* One tensor of a grouped guide_pack (fields as in guide_pack). */
typedef struct {
    const void* codes;
    const void* scales;
    int64_t rows, cols;
    void* guide_bits;
    void* guide_scales;
} fp4_guide_desc;

/* guide_pack of up to 16 tensors sharing one configuration in one launch, e.g.
 * the routed experts and activations of one deep layer [TRACE-JA
 * "量子化情報キャッシュ": the guide is kept per deep layer].  Same result as
 * guide_pack on each tensor; empty tensors are skipped; every tensor is
 * checked before anything is launched (the message names the tensor). */
fp4_status guide_pack_grouped(const fp4_cfg* cfg, int n, const fp4_guide_desc* tensors, hipStream_t stream);

/* Inverse view of the guide: mant_u8[i] = guide bit i (0 or 1), scales_out =
 * guide_scales. */
fp4_status guide_unpack(const fp4_cfg* cfg, const void* guide_bits, const void* guide_scales,
                        int64_t rows, int64_t cols, void* mant_u8, void* scales_out,
                        hipStream_t stream);

/* Full-code guided diagnostic [TRACE-JA "量子化情報キャッシュ": one mantissa
 * bit names the rollout's codeword only when that codeword brackets the
 * training value; other cases are the rare non-adjacent mismatches].  Guided
 * rounding of x with the guide bits taken from the rollout's full codes
 * (their LSBs) and the rollout's block scales (and tensor scale, NVFP4), the
 * result g compared with the rollout codes r.  Nothing else is written.
 *   counts        device uint64[3], 8-byte aligned, overwritten:
 *                 [0] elements of the blocks guided rounding encodes (finite
 *                     input, finite rollout scale),
 *                 [1] of those, |g| != |r| (non-adjacent: the bit cannot name r),
 *                 [2] of those, g != r (sign included).
 *   rollout_codes, rollout_scales  the rollout's quantization of a tensor of
 *                 the same shape, in the layouts fp4_quantize writes. */
fp4_status fp4_guide_mismatch(const fp4_cfg* cfg, const void* x_bf16, int64_t rows, int64_t cols, int64_t ld,
                              const float* tensor_scale, const void* rollout_codes, const void* rollout_scales,
                              unsigned long long* counts, hipStream_t stream);

/* MXFP4 matrix product on the matrix cores [TETRAJET section 3: FP4 values
 * with one scale per group; section 4: the matrix products of every linear
 * layer take MXFP4 operands]:
 *   C[m][n] = sum over k of a(m,k) * b(n,k),   m < M, n < N, k < K,
 * where a is the [M, K] tensor given by a_codes / a_scales and b the [N, K]
 * tensor given by b_codes / b_scales, each in exactly the layouts fp4_quantize
 * writes for a row-major input with format FP4_MXFP4 and the E2M1 grid:
 * codes K/2 bytes per row, E8M0 scales K/32 bytes per row (blocks of 32
 * along K).  So C = A * B^T; for a linear layer y = x W^T, A holds the
 * activations [tokens, in] and B the weight [out, in].
 *   The products are summed in fp32 by the matrix cores, in an order of
 * their own: |C - C_exact| <= (K + 1) 2^-24 sum_k |a b| + K 2^-149 holds for
 * finite results.  A 0xFF (NaN) scale makes the results of its row of A or
 * B NaN.  Output dense enough for row stride ldc >= N elements: fp32, or
 * bf16 by round-to-nearest-even of the fp32 result.
 *   K % 32 == 0 (K == 0 writes zeros); M == 0 or N == 0 is a no-op;
 *   ldc <= 2^21.
 *   Alignment: codes 16 bytes, scales 1 byte, c 4 (fp32) or 2 (bf16) bytes.
 *   The grid of the codes is E2M1 only: the uniform grid and NVFP4 blocks
 *   are not accepted by this product (the caller keeps them apart). */
fp4_status fp4_gemm_mxfp4(const void* a_codes, const void* a_scales, const void* b_codes, const void* b_scales,
                          int64_t M, int64_t N, int64_t K, void* c, int64_t ldc, fp4_dtype dtype,
                          hipStream_t stream);

/* The MXFP4 product with the rollout's quantization of its result fused into
 * the producing kernel [TRACE-JA "量子化情報キャッシュ": the rollout records the
 * codeword it chose at each quantization point; "実験結果": collecting it costs
 * about as much as plain FP4 rollout; TETRAJET section 4: the next linear
 * layer takes MXFP4 inputs]: C = A * B^T exactly as fp4_gemm_mxfp4 computes it,
 * rounded to bf16, then quantized along its rows as fp4_quantize does with
 * format MXFP4, the E2M1 grid and round to nearest: codes [M, N/2], E8M0 scales
 * [M, N/32] and, when c_guide_bits is not NULL, the guide bitplane [M, N/8].
 * C itself is never written.  Bit for bit equal to fp4_gemm_mxfp4 with bf16
 * output followed by fp4_quantize (MXFP4, RTN, emission) of that output.
 *   N % 32 == 0 (FP4_ERR_SHAPE); K a positive multiple of 512 and both scale
 *   pointers 16-byte aligned (FP4_ERR_UNSUPPORTED otherwise); M == 0 or
 *   N == 0 is a no-op.  c_codes and c_guide_bits 16-byte aligned. */
fp4_status fp4_gemm_mxfp4_quantize(const void* a_codes, const void* a_scales, const void* b_codes,
                                   const void* b_scales, int64_t M, int64_t N, int64_t K, void* c_codes,
                                   void* c_scales, void* c_guide_bits, hipStream_t stream);

/* The same product with its result quantized to NVFP4 instead [TRACE-JA
 * "実験結果": FP4 KV cache; "量子化情報キャッシュ": the rollout's codewords;
 * FQT-FP4 section 3: E4M3 block scales under one fp32 tensor scale], for a
 * producer whose output is stored as NVFP4, such as the K and V projections
 * writing the KV cache: C = A * B^T exactly as fp4_gemm_mxfp4 computes it,
 * rounded to bf16, then quantized along its rows as fp4_quantize does with
 * format NVFP4, the E2M1 grid and round to nearest under the given tensor
 * scale: codes [M, N/2], E4M3 scales [M, N/16] and, when c_guide_bits is not
 * NULL, the guide bitplane [M, N/8].  Bit for bit equal to fp4_gemm_mxfp4 with
 * bf16 output followed by fp4_quantize (NVFP4, RTN, emission, tensor_scale).
 *   tensor_scale   device pointer to s_t (positive and finite), for example
 *                  the previous step's, or a calibrated value: the product's
 *                  own amax is not known until every tile is done.
 *   N % 32 == 0 (FP4_ERR_SHAPE); K and the scale pointers as for
 *   fp4_gemm_mxfp4_quantize; c_codes and c_guide_bits 16-byte aligned,
 *   c_scales 2-byte aligned. */
fp4_status fp4_gemm_mxfp4_quantize_nvfp4(const void* a_codes, const void* a_scales, const void* b_codes,
                                         const void* b_scales, int64_t M, int64_t N, int64_t K,
                                         const float* tensor_scale, void* c_codes, void* c_scales,
                                         void* c_guide_bits, hipStream_t stream);

/* One product of a grouped call (fields as in fp4_gemm_mxfp4). */
typedef struct {
    const void* a_codes;
    const void* a_scales;
    const void* b_codes;
    const void* b_scales;
    int64_t M, N, K;
    void* c;
    int64_t ldc;
} fp4_gemm_desc;

/* Up to 16 MXFP4 products in one launch, e.g. the routed experts of an MoE
 * layer, each with its own token rows and weight [TETRAJET section 4: every
 * linear layer's products take MXFP4 operands; TRACE-JA: MoE models].  Same
 * result as fp4_gemm_mxfp4 on each product in turn; products with M or N of 0
 * are skipped.  Every product is checked before anything is launched (the
 * message names the product).  All products run in one launch when every K is
 * a multiple of 512 with 16-byte aligned scales; otherwise one launch each. */
fp4_status fp4_gemm_mxfp4_grouped(int n, const fp4_gemm_desc* products, fp4_dtype dtype, hipStream_t stream);

/* Standalone 16-point random Hadamard transform [UFP4 RHT section] of each
 * 16-group of a bf16 matrix: forward y = 1/4 H16 D x, inverse x = D 1/4 H16 y,
 * Sylvester order, butterfly stages h = 1,2,4,8 in fp32.  D_j = -1 iff bit j
 * of word 0 of Philox4x32-10(key = seed, counter = (0,0,1,0)).  cols % 16 == 0.
 * Output dense fp32 or bf16 (RNE). */
fp4_status fp4_rht16(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld, uint64_t seed,
                     int inverse, void* out, fp4_dtype dtype, hipStream_t stream);

/* Element encode of n pre-scaled fp32 values (the per-element rounding step
 * on its own, for exhaustive verification): out[i] = sign<<3 | k of v[i]
 * clamped to Gmax; mode FP4_MODE_RTN, FP4_MODE_SR (aux[i] = random byte) or
 * FP4_MODE_GUIDED (aux[i] = guide bit).  aux may be NULL for RTN.  The code
 * of a NaN value is unspecified (quantization zeroes every block holding one).
 * n % 8 == 0; v 16-byte aligned, aux and out 8-byte aligned. */
fp4_status fp4_encode_values(int grid, int mode, const float* v, const uint8_t* aux, int64_t n,
                             uint8_t* out, hipStream_t stream);

/* The NVFP4 block-scale rounding on its own, for exhaustive verification
 * [FQT-FP4 §3: E4M3 block scales]: out[i] = OCP E4M3FN code of min(t[i], 448)
 * rounded to nearest even, for t[i] >= 0 (a NaN gives the code of 448).
 * n % 4 == 0; t 16-byte aligned, out 4-byte aligned. */
fp4_status fp4_encode_scales(const float* t, int64_t n, uint8_t* out, hipStream_t stream);

/* Plain streaming copy of `bytes` (a multiple of 16) from src to dst, one
 * 16-byte load and store per lane: the practical HBM bandwidth reference the
 * quantize kernels are measured against.  Both pointers 16-byte aligned;
 * the ranges must not overlap. */
fp4_status fp4_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/* Buffer sizes in bytes. */
size_t fp4_codes_bytes(int64_t rows, int64_t cols);
size_t fp4_scales_bytes(int format, int64_t rows, int64_t cols);
/* Guide bitplane + guide scales + 4 bytes of tensor scale. */
size_t fp4_guide_bytes(int format, int64_t rows, int64_t cols);

const char* fp4_status_str(fp4_status s);
/* Message of the last error on the calling thread ("" if none). */
const char* fp4_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FP4Q_H */
