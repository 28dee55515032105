// internal.h -- kernel parameter blocks and launchers shared between the C ABI
// (abi.hip) and the kernel translation units.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

// Threads per workgroup for every kernel of the library.
constexpr int kThreads = 256;

// Unsigned division by a runtime constant d (1 <= d < 2^31):
// q = (mulhi(n, m) + n) >> l with l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1.
struct FastDiv {
    uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    uint64_t m = ((((1ull << l) - d) << 32) / d) + 1;
    return FastDiv{d, (uint32_t)m, l};
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, FastDiv f) {
    uint64_t t = __umulhi(n, f.m);
    return (uint32_t)((t + n) >> f.l);
}

// Element offset of half-group hg (logical row-major order) in a tensor with row stride ld.
template <bool CONTIG>
__device__ __forceinline__ int64_t half_offset(uint32_t hg, const FastDiv& gpr, int64_t ld) {
    if constexpr (CONTIG) {
        return (int64_t)hg * 8;
    } else {
        const uint32_t g = hg >> 1;
        const uint32_t row = fastdiv(g, gpr);
        return (int64_t)row * ld + (int64_t)(g - row * gpr.d) * 16 + (hg & 1u) * 8;
    }
}

// 16-element groups are the work unit: group g covers elements 16g..16g+15 of
// the logical row-major order (rows*cols/16 groups; a row holds cols/16).
struct QuantParams {
    const uint16_t* x;          // bf16 input, row stride ld elements
    int64_t ld;
    uint32_t ngroups;
    FastDiv gpr;                // groups per row
    const float* ts;            // NVFP4 tensor scale (device), or guide tensor scale
    uint8_t* codes;
    uint8_t* scales;
    uint8_t* bits_out;          // fused guide emission (RTN / SR), may be null
    const uint8_t* gbits;       // guided: guide bitplane
    const uint8_t* gscales;     // guided: guide scales
    uint32_t key0, key1;        // SR Philox key
    uint64_t sr_offset;         // SR counter offset (groups)
    uint64_t rht_seed;          // RHT: Philox key of the sign diagonal
    uint16_t* fq_out;           // fake quantization: bf16 output (dequantized codes)
    int64_t ld_out;             // its row stride in elements
    const uint8_t* rcodes;      // guide diagnostic: the rollout's full codes (guide bits are their LSBs)
    unsigned long long* counts; // guide diagnostic: elements, non-adjacent, mismatched (zeroed first)
    uint32_t stream_out;        // 1: codes, scales, guide bits and fake-quantized values by non-temporal stores
};

// Up to kMaxGroup tensors sharing one configuration, quantized by one launch.
constexpr int kMaxGroup = 16;

struct GroupedQuantParams {
    QuantParams t[kMaxGroup];
    uint32_t wg_start[kMaxGroup + 1];   // prefix sums of per-tensor workgroup counts
    uint32_t n;
    uint32_t contig_mask;               // bit t: tensor t has ld == cols
};

struct DequantParams {
    const uint8_t* codes;
    const uint8_t* scales;
    const float* ts;
    void* out;
    int64_t ld_out;
    uint32_t ngroups;
    FastDiv gpr;
};

struct GuideParams {
    const uint8_t* in;          // pack: codes;  unpack: guide bits
    const uint8_t* scales_in;
    uint8_t* out;               // pack: guide bits;  unpack: 0/1 bytes
    uint8_t* scales_out;
    uint32_t ngroups;
};

struct RhtParams {
    const uint16_t* x;
    int64_t ld;
    void* out;
    uint32_t ngroups;
    FastDiv gpr;
    uint64_t seed;              // Philox key of the sign diagonal
};

struct AmaxParams {
    const uint16_t* x;
    int64_t ld;
    uint32_t ngroups;
    FastDiv gpr;
    uint64_t rht_seed;
    float* acc;                 // receives max finite |y| (as bits, atomic max)
};

// Workspace of the one-launch tensor scale and of the fused tensor scale and
// quantize, in 32-bit words from a 256-byte aligned base: the epoch word (the
// tag of the last call whose reduction completed), kTsPubCopies copies of the
// fused launch's 64-bit published word (tag << 32 | bits of s_t), each on a
// 256-byte line of its own, and from word kTsGather on one 64-bit word per
// workgroup (tag << 32 | bits of its maximum).  A word counts only when its tag
// is the call's own, so zero is a valid state of all of them: a zero-filled
// workspace suits every call, and every call leaves it ready for the next.
constexpr uint32_t kTsLine = 64;                        // words per 256-byte line
constexpr uint32_t kTsMaxWorkgroups = 1024;             // one-launch tensor scale
constexpr uint32_t kTsEpoch = 0;
constexpr uint32_t kTsPub = kTsLine;                    // 64-bit copies, kTsLine words apart
constexpr uint32_t kTsPubCopies = 16;
constexpr uint32_t kTsGather = 2048;                    // 64-bit words from here on, one per workgroup
constexpr uint32_t kTsGatherMax = 2048;                 // workgroups of the fused launch
constexpr size_t kTsWorkspaceBytes = 4 * kTsGather + 8 * kTsGatherMax;
constexpr uint32_t kTsStaticWords = kTsGather + 2 * kTsMaxWorkgroups;   // what the one-launch tensor scale uses
static_assert(kTsPub + kTsLine * kTsPubCopies <= kTsGather && kTsMaxWorkgroups <= kTsGatherMax,
              "tensor-scale workspace layout");
constexpr int kMaxDevices = 64;                         // devices whose per-device state the library keeps

// Polls a workgroup waiting on others makes before it gives up (fp4_set_wait_limit).
uint32_t wait_limit();
uint32_t set_wait_limit(uint32_t polls);   // returns the previous limit

struct EncodeParams {
    const float* v;
    const uint8_t* aux;
    uint8_t* out;
    uint32_t n8;                // number of 8-element units
};

// MXFP4 matrix product C[M, N] = A[M, K] * B[N, K]^T (codes and E8M0 scales
// along K, as the quantizer writes them); K % 32 == 0, M, N >= 1.
struct GemmParams {
    const uint8_t* a;           // A codes, K/2 bytes per row
    const uint8_t* as;          // A scales, K/32 bytes per row
    const uint8_t* b;
    const uint8_t* bs;
    void* c;                    // fp32 or bf16, row stride ldc elements
    int64_t ldc;
    int64_t M, N, K;
    uint32_t tiles_n;           // column tiles of C
    uint32_t xcd_remap;         // 1: hand out tiles XCD by XCD (grid size a multiple of 8)
    uint32_t staged;            // 1: C and its rows 16-byte aligned (whole tiles stored through LDS)
    uint8_t* qcodes;            // quantize epilogue: codes of the bf16-rounded C, [M, N/2]
    uint8_t* qscales;           // ... E8M0 scales [M, N/32], or E4M3 scales [M, N/16] (NVFP4)
    uint8_t* qbits;             // ... guide bits [M, N/8], or null
    const float* qts;           // ... NVFP4: the tensor scale s_t; null: MXFP4
};

// Launchers (return hipGetLastError() of the launch).
hipError_t launch_quantize(int format, int grid, int mode, bool rht, bool emit, bool contig,
                           const QuantParams& p, hipStream_t s);
// Guided rounding against the rollout's full codes (p.rcodes, p.gscales, p.ts):
// adds the counts of elements, non-adjacent and mismatched codes to p.counts.
hipError_t launch_guide_mismatch(int format, int grid, bool rht, bool contig, const QuantParams& p, hipStream_t s);

// Quantize then dequantize to bf16 in one pass (p.fq_out, p.ld_out); no codes written.
hipError_t launch_fake_quantize(int format, int grid, int mode, bool rht, bool contig,
                                const QuantParams& p, hipStream_t s);
// Workgroups needed to quantize `ngroups` 16-element groups.
uint32_t quantize_chunks(int format, int mode, bool rht, uint32_t ngroups);
hipError_t launch_quantize_grouped(int format, int grid, int mode, bool rht, bool emit,
                                   const GroupedQuantParams& gp, hipStream_t s);
hipError_t launch_tensor_scale(int grid, bool rht, bool contig, const AmaxParams& p, hipStream_t s);
// One-launch tensor scale with its workspace (kTsWorkspaceBytes, 256-byte aligned, counters 0).
hipError_t launch_tensor_scale_1(int grid, bool rht, bool contig, const AmaxParams& p, uint32_t* ws,
                                 hipStream_t s);
// NVFP4 tensor scale and quantization (RTN or SR) of one tensor: one launch when
// there is no RHT and the device can hold every workgroup of it at once, else
// the one-launch tensor scale followed by the quantize launch.  p.ts is ignored
// (the scale goes to ts_out); ws as for launch_tensor_scale_1.  *fused reports
// which.
hipError_t launch_quantize_with_scale(int grid, int mode, bool rht, bool emit, bool contig, const QuantParams& p,
                                      float* ts_out, uint32_t* ws, bool* fused, hipStream_t s);
// Device address of the library's static tensor-scale workspace (kTsWorkspaceBytes)
// on the current device, looked up once per device; NULL with the error in *err
// when the lookup fails.
uint32_t* static_ts_workspace(hipError_t* err);
hipError_t launch_dequantize(int format, int grid, bool bf16_out, const DequantParams& p,
                             hipStream_t s);
hipError_t launch_guide_pack(int format, const GuideParams& p, hipStream_t s);
hipError_t launch_guide_unpack(int format, const GuideParams& p, hipStream_t s);
struct GroupedGuideParams {
    GuideParams t[kMaxGroup];
    uint32_t wg_start[kMaxGroup + 1];   // prefix sums of per-tensor workgroup counts
    uint32_t n;
};
hipError_t launch_guide_pack_grouped(int format, GroupedGuideParams gp, hipStream_t s);
hipError_t launch_rht16(bool inverse, bool bf16_out, bool contig, const RhtParams& p, hipStream_t s);
hipError_t launch_stream_copy(const void* src, void* dst, uint64_t n16, hipStream_t s);
hipError_t launch_encode_values(int grid, int mode, const EncodeParams& p, hipStream_t s);
// E4M3 codes of n4 * 4 values t (NVFP4 block-scale rounding, t clamped to 448).
hipError_t launch_encode_scales(const float* t, uint8_t* out, uint32_t n4, hipStream_t s);
hipError_t launch_gemm_mx(bool bf16_out, const GemmParams& p, hipStream_t s);
// The same product ending in the MXFP4 RTN quantization of its bf16-rounded
// result (p.qcodes, p.qscales, p.qbits; NVFP4 under *p.qts when p.qts is not
// null, else MXFP4); only where gemm_quant_supported(p).
bool gemm_quant_supported(const GemmParams& p);
hipError_t launch_gemm_mx_quant(const GemmParams& p, hipStream_t s);

// Up to kMaxGemmGroup products in one launch (one launch per product when
// some product's K is not a multiple of 512).
constexpr int kMaxGemmGroup = 16;
struct GroupedGemmParams {
    GemmParams g[kMaxGemmGroup];
    uint32_t tile_start[kMaxGemmGroup + 1];   // prefix sums of per-product tile counts
    uint32_t n;
    uint32_t xcd_remap;
};
hipError_t launch_gemm_mx_grouped(bool bf16_out, const GroupedGemmParams& gp, hipStream_t s);

}  // namespace fp4q
