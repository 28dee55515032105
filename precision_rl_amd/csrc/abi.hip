// abi.hip -- the extern "C" entry points of libfp4q: argument validation,
// parameter blocks and kernel launches.  No allocation, no synchronization.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/fp4q.h"
#include "device.h"
#include "internal.h"

namespace {

thread_local char g_err[512] = "";

fp4_status fail(fp4_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

fp4_status ok() {
    g_err[0] = '\0';
    return FP4_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int block_of(int format) { return format == FP4_MXFP4 ? 32 : 16; }

fp4_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Shared checks of a bf16 [rows, cols] input with row stride ld.
fp4_status check_cfg(const fp4_cfg* cfg) {
    if (!cfg) return fail(FP4_ERR_ARG, "cfg is NULL");
    if (cfg->format != FP4_NVFP4 && cfg->format != FP4_MXFP4)
        return fail(FP4_ERR_ARG, "unknown format %d", cfg->format);
    if (cfg->grid != FP4_GRID_E2M1 && cfg->grid != FP4_GRID_UNIFORM)
        return fail(FP4_ERR_ARG, "unknown grid %d", cfg->grid);
    if (cfg->rounding != FP4_RTN && cfg->rounding != FP4_SR)
        return fail(FP4_ERR_ARG, "unknown rounding %d", cfg->rounding);
    if (cfg->stream_out != 0 && cfg->stream_out != 1)
        return fail(FP4_ERR_ARG, "stream_out=%d is neither 0 nor 1", cfg->stream_out);
    return FP4_OK;
}

fp4_status check_matrix(int64_t rows, int64_t cols, int64_t ld, int B, const void* x, uint64_t* ngroups) {
    if (rows < 0 || cols < 0) return fail(FP4_ERR_ARG, "negative shape rows=%lld cols=%lld",
                                          (long long)rows, (long long)cols);
    if (cols % B != 0) return fail(FP4_ERR_SHAPE, "cols=%lld is not a multiple of the block size %d",
                                   (long long)cols, B);
    if (rows > 0 && cols > 0) {
        if (ld < cols) return fail(FP4_ERR_SHAPE, "ld=%lld < cols=%lld", (long long)ld, (long long)cols);
        if (ld % 8 != 0) return fail(FP4_ERR_ALIGN, "ld=%lld is not a multiple of 8 elements", (long long)ld);
        if (!x) return fail(FP4_ERR_ARG, "input pointer is NULL");
        if (!aligned(x, 16)) return fail(FP4_ERR_ALIGN, "input pointer is not 16-byte aligned");
    }
    const uint64_t g = (uint64_t)rows * (uint64_t)cols / 16;
    if (g >= (1ull << 31)) return fail(FP4_ERR_SHAPE, "too many elements (%llu groups of 16)",
                                       (unsigned long long)g);
    if (cols / 16 >= (1ll << 31)) return fail(FP4_ERR_SHAPE, "cols too large");
    *ngroups = g;
    return FP4_OK;
}

fp4_status need(const void* p, uintptr_t align, const char* name) {
    if (!p) return fail(FP4_ERR_ARG, "%s is NULL", name);
    if (!aligned(p, align)) return fail(FP4_ERR_ALIGN, "%s is not %u-byte aligned", name, (unsigned)align);
    return FP4_OK;
}

#define FP4Q_TRY(expr)                       \
    do {                                     \
        fp4_status _s = (expr);              \
        if (_s != FP4_OK) return _s;         \
    } while (0)

}  // namespace

extern "C" {

size_t fp4_codes_bytes(int64_t rows, int64_t cols) { return (size_t)(rows * cols / 2); }

size_t fp4_scales_bytes(int format, int64_t rows, int64_t cols) {
    return (size_t)(rows * cols / block_of(format));
}

size_t fp4_guide_bytes(int format, int64_t rows, int64_t cols) {
    return (size_t)(rows * cols / 8) + fp4_scales_bytes(format, rows, cols) + 4;
}

const char* fp4_status_str(fp4_status s) {
    switch (s) {
        case FP4_OK: return "ok";
        case FP4_ERR_ARG: return "invalid argument";
        case FP4_ERR_SHAPE: return "invalid shape";
        case FP4_ERR_ALIGN: return "misaligned pointer or stride";
        case FP4_ERR_UNSUPPORTED: return "unsupported combination";
        case FP4_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* fp4_last_error(void) { return g_err; }

fp4_status fp4_tensor_scale(const fp4_cfg* cfg, const void* x_bf16, int64_t rows, int64_t cols,
                            int64_t ld, float* tensor_scale_out, hipStream_t stream) {
    FP4Q_TRY(check_cfg(cfg));
    uint64_t ng = 0;
    FP4Q_TRY(check_matrix(rows, cols, ld, 16, x_bf16, &ng));
    FP4Q_TRY(need(tensor_scale_out, 4, "tensor_scale_out"));
    fp4q::AmaxParams p{};
    p.x = static_cast<const uint16_t*>(x_bf16);
    p.ld = ld;
    p.ngroups = (uint32_t)ng;
    p.gpr = fp4q::make_fastdiv(cols > 0 ? (uint32_t)(cols / 16) : 1u);
    p.rht_seed = cfg->rht_seed;
    p.acc = tensor_scale_out;
    return hip_status(fp4q::launch_tensor_scale(cfg->grid, cfg->rht16 != 0, ld == cols, p, stream),
                      "fp4_tensor_scale launch");
}

static_assert(FP4_TENSOR_SCALE_WORKSPACE_BYTES == fp4q::kTsWorkspaceBytes, "workspace size in the header");
static_assert(sizeof(fp4_cfg) == 48, "fp4_cfg layout in the header");
size_t fp4_tensor_scale_workspace_bytes(void) { return fp4q::kTsWorkspaceBytes; }

static_assert(FP4_WAIT_LIMIT_DEFAULT == fp4q::kGatherPolls, "default wait limit in the header");
uint32_t fp4_set_wait_limit(uint32_t polls) { return fp4q::set_wait_limit(polls); }

fp4_status fp4_tensor_scale_ws(const fp4_cfg* cfg, const void* x_bf16, int64_t rows, int64_t cols,
                               int64_t ld, float* tensor_scale_out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
    FP4Q_TRY(check_cfg(cfg));
    uint64_t ng = 0;
    FP4Q_TRY(check_matrix(rows, cols, ld, 16, x_bf16, &ng));
    FP4Q_TRY(need(tensor_scale_out, 4, "tensor_scale_out"));
    FP4Q_TRY(need(workspace, 256, "workspace"));
    if (workspace_bytes < fp4q::kTsWorkspaceBytes)
        return fail(FP4_ERR_ARG, "workspace_bytes=%zu < %zu", workspace_bytes, fp4q::kTsWorkspaceBytes);
    fp4q::AmaxParams p{};
    p.x = static_cast<const uint16_t*>(x_bf16);
    p.ld = ld;
    p.ngroups = (uint32_t)ng;
    p.gpr = fp4q::make_fastdiv(cols > 0 ? (uint32_t)(cols / 16) : 1u);
    p.rht_seed = cfg->rht_seed;
    p.acc = tensor_scale_out;
    return hip_status(fp4q::launch_tensor_scale_1(cfg->grid, cfg->rht16 != 0, ld == cols, p,
                                                  static_cast<uint32_t*>(workspace), stream),
                      "fp4_tensor_scale_ws launch");
}

fp4_status fp4_tensor_scale_noalloc(const fp4_cfg* cfg, const void* x_bf16, int64_t rows, int64_t cols,
                                    int64_t ld, float* tensor_scale_out, hipStream_t stream) {
    FP4Q_TRY(check_cfg(cfg));
    uint64_t ng = 0;
    FP4Q_TRY(check_matrix(rows, cols, ld, 16, x_bf16, &ng));
    FP4Q_TRY(need(tensor_scale_out, 4, "tensor_scale_out"));
    // the launch never exceeds kTsMaxWorkgroups workgroups, whose words the static
    // workspace holds, whatever the input size
    hipError_t e = hipSuccess;
    uint32_t* ws = fp4q::static_ts_workspace(&e);
    if (!ws) return hip_status(e, "fp4_tensor_scale_noalloc: static workspace lookup");
    fp4q::AmaxParams p{};
    p.x = static_cast<const uint16_t*>(x_bf16);
    p.ld = ld;
    p.ngroups = (uint32_t)ng;
    p.gpr = fp4q::make_fastdiv(cols > 0 ? (uint32_t)(cols / 16) : 1u);
    p.rht_seed = cfg->rht_seed;
    p.acc = tensor_scale_out;
    return hip_status(fp4q::launch_tensor_scale_1(cfg->grid, cfg->rht16 != 0, ld == cols, p, ws, stream),
                      "fp4_tensor_scale_noalloc launch");
}

static fp4_status quantize_common(const fp4_cfg* cfg, int mode, const void* x_bf16, int64_t rows,
                                  int64_t cols, int64_t ld, const float* ts, void* codes, void* scales,
                                  void* bits_out, const void* gbits, const void* gscales,
                                  hipStream_t stream) {
    FP4Q_TRY(check_cfg(cfg));
    uint64_t ng = 0;
    FP4Q_TRY(check_matrix(rows, cols, ld, block_of(cfg->format), x_bf16, &ng));
    if (ng == 0) return ok();
    FP4Q_TRY(need(codes, 16, "codes"));
    FP4Q_TRY(need(scales, 1, "scales"));
    if (cfg->format == FP4_NVFP4) FP4Q_TRY(need(ts, 4, "tensor_scale"));
    if (bits_out) FP4Q_TRY(need(bits_out, 16, "guide_bits_out"));
    if (mode == fp4q::MODE_GUIDED) {
        FP4Q_TRY(need(gbits, 16, "guide_bits"));
        FP4Q_TRY(need(gscales, 1, "guide_scales"));
    }
    fp4q::QuantParams p{};
    p.x = static_cast<const uint16_t*>(x_bf16);
    p.ld = ld;
    p.ngroups = (uint32_t)ng;
    p.gpr = fp4q::make_fastdiv((uint32_t)(cols / 16));
    p.ts = ts;
    p.codes = static_cast<uint8_t*>(codes);
    p.scales = static_cast<uint8_t*>(scales);
    p.bits_out = static_cast<uint8_t*>(bits_out);
    p.gbits = static_cast<const uint8_t*>(gbits);
    p.gscales = static_cast<const uint8_t*>(gscales);
    p.key0 = (uint32_t)cfg->sr_seed;
    p.key1 = (uint32_t)(cfg->sr_seed >> 32);
    p.sr_offset = cfg->sr_offset;
    p.rht_seed = cfg->rht_seed;
    p.stream_out = (uint32_t)cfg->stream_out;
    return hip_status(fp4q::launch_quantize(cfg->format, cfg->grid, mode, cfg->rht16 != 0,
                                            bits_out != nullptr, ld == cols, p, stream),
                      "quantize launch");
}

fp4_status fp4_quantize(const fp4_cfg* cfg, const void* x_bf16, int64_t rows, int64_t cols,
                        int64_t ld, const float* tensor_scale, void* codes, void* scales,
                        void* guide_bits_out, hipStream_t stream) {
    FP4Q_TRY(check_cfg(cfg));
    const int mode = cfg->rounding == FP4_SR ? fp4q::MODE_SR : fp4q::MODE_RTN;
    return quantize_common(cfg, mode, x_bf16, rows, cols, ld, tensor_scale, codes, scales,
                           guide_bits_out, nullptr, nullptr, stream);
}

fp4_status fp4_quantize_with_tensor_scale(const fp4_cfg* cfg, const void* x_bf16, int64_t rows, int64_t cols,
                                          int64_t ld, float* tensor_scale_out, void* codes, void* scales,
                                          void* guide_bits_out, void* workspace, size_t workspace_bytes,
                                          int* launches, hipStream_t stream) {
    FP4Q_TRY(check_cfg(cfg));
    if (cfg->format != FP4_NVFP4) return fail(FP4_ERR_UNSUPPORTED, "the tensor scale belongs to the NVFP4 format");
    uint64_t ng = 0;
    FP4Q_TRY(check_matrix(rows, cols, ld, 16, x_bf16, &ng));
    FP4Q_TRY(need(tensor_scale_out, 4, "tensor_scale_out"));
    FP4Q_TRY(need(workspace, 256, "workspace"));
    if (workspace_bytes < fp4q::kTsWorkspaceBytes)
        return fail(FP4_ERR_ARG, "workspace_bytes=%zu < %zu", workspace_bytes, fp4q::kTsWorkspaceBytes);
    if (ng > 0) {
        FP4Q_TRY(need(codes, 16, "codes"));
        FP4Q_TRY(need(scales, 1, "scales"));
        if (guide_bits_out) FP4Q_TRY(need(guide_bits_out, 16, "guide_bits_out"));
    }
    fp4q::QuantParams p{};
    p.x = static_cast<const uint16_t*>(x_bf16);
    p.ld = ld;
    p.ngroups = (uint32_t)ng;
    p.gpr = fp4q::make_fastdiv(cols > 0 ? (uint32_t)(cols / 16) : 1u);
    p.codes = static_cast<uint8_t*>(codes);
    p.scales = static_cast<uint8_t*>(scales);
    p.bits_out = static_cast<uint8_t*>(guide_bits_out);
    p.key0 = (uint32_t)cfg->sr_seed;
    p.key1 = (uint32_t)(cfg->sr_seed >> 32);
    p.sr_offset = cfg->sr_offset;
    p.rht_seed = cfg->rht_seed;
    p.stream_out = (uint32_t)cfg->stream_out;
    const int mode = cfg->rounding == FP4_SR ? fp4q::MODE_SR : fp4q::MODE_RTN;
    bool fused = false;
    const hipError_t e = fp4q::launch_quantize_with_scale(cfg->grid, mode, cfg->rht16 != 0, guide_bits_out != nullptr,
                                                          ld == cols, p, tensor_scale_out,
                                                          static_cast<uint32_t*>(workspace), &fused, stream);
    if (launches) *launches = fused ? 1 : (ng > 0 ? 2 : 1);
    return hip_status(e, "fp4_quantize_with_tensor_scale launch");
}

fp4_status fp4_quantize_grouped(const fp4_cfg* cfg, int guided, int n, const fp4_tensor* tensors,
                                hipStream_t stream) {
    FP4Q_TRY(check_cfg(cfg));
    if (n < 1 || n > FP4_MAX_GROUP) return fail(FP4_ERR_ARG, "n=%d outside 1..%d", n, FP4_MAX_GROUP);
    if (!tensors) return fail(FP4_ERR_ARG, "tensors is NULL");
    static_assert(FP4_MAX_GROUP == fp4q::kMaxGroup, "group size limits differ");
    const int mode = guided ? fp4q::MODE_GUIDED : (cfg->rounding == FP4_SR ? fp4q::MODE_SR : fp4q::MODE_RTN);
    const bool emit = !guided && tensors[0].guide_bits != nullptr;
    fp4q::GroupedQuantParams gp{};
    gp.n = (uint32_t)n;
    uint64_t wg = 0;
    for (int t = 0; t < n; ++t) {
        const fp4_tensor& d = tensors[t];
        uint64_t ng = 0;
        fp4_status st = check_matrix(d.rows, d.cols, d.ld, block_of(cfg->format), d.x, &ng);
        if (st != FP4_OK) {
            char msg[sizeof g_err];
            snprintf(msg, sizeof msg, "%s", g_err);
            return fail(st, "tensor %d: %s", t, msg);
        }
        gp.wg_start[t] = (uint32_t)wg;
        if (ng == 0) continue;
        const char* what = nullptr;
        if (!d.codes || !aligned(d.codes, 16)) what = "codes";
        else if (!d.scales) what = "scales";
        else if (cfg->format == FP4_NVFP4 && (!d.tensor_scale || !aligned(d.tensor_scale, 4))) what = "tensor_scale";
        else if (guided && (!d.guide_bits || !aligned(d.guide_bits, 16))) what = "guide_bits";
        else if (guided && !d.guide_scales) what = "guide_scales";
        else if (!guided && (d.guide_bits != nullptr) != emit) what = "guide_bits (emission must be all or none)";
        else if (!guided && emit && !aligned(d.guide_bits, 16)) what = "guide_bits";
        if (what) return fail(FP4_ERR_ARG, "tensor %d: %s missing or misaligned", t, what);
        fp4q::QuantParams& p = gp.t[t];
        p.x = static_cast<const uint16_t*>(d.x);
        p.ld = d.ld;
        p.ngroups = (uint32_t)ng;
        p.gpr = fp4q::make_fastdiv((uint32_t)(d.cols / 16));
        p.ts = d.tensor_scale;
        p.codes = static_cast<uint8_t*>(d.codes);
        p.scales = static_cast<uint8_t*>(d.scales);
        p.bits_out = guided ? nullptr : static_cast<uint8_t*>(d.guide_bits);
        p.gbits = guided ? static_cast<const uint8_t*>(d.guide_bits) : nullptr;
        p.gscales = guided ? static_cast<const uint8_t*>(d.guide_scales) : nullptr;
        p.key0 = (uint32_t)cfg->sr_seed;
        p.key1 = (uint32_t)(cfg->sr_seed >> 32);
        p.sr_offset = cfg->sr_offset;
        p.rht_seed = cfg->rht_seed;
        p.stream_out = (uint32_t)cfg->stream_out;
        if (d.ld == d.cols) gp.contig_mask |= 1u << t;
        wg += fp4q::quantize_chunks(cfg->format, mode, cfg->rht16 != 0, (uint32_t)ng);
        if (wg >= (1ull << 31)) return fail(FP4_ERR_SHAPE, "grouped call too large");
    }
    gp.wg_start[n] = (uint32_t)wg;
    if (wg == 0) return ok();
    return hip_status(fp4q::launch_quantize_grouped(cfg->format, cfg->grid, mode, cfg->rht16 != 0, emit, gp, stream),
                      "grouped quantize launch");
}

fp4_status fp4_quantize_guided(const fp4_cfg* cfg, const void* x_bf16, int64_t rows,
                               int64_t cols, int64_t ld, const void* guide_bits,
                               const void* guide_scales, const float* guide_tensor_scale,
                               void* codes, void* scales, hipStream_t stream) {
    return quantize_common(cfg, fp4q::MODE_GUIDED, x_bf16, rows, cols, ld, guide_tensor_scale,
                           codes, scales, nullptr, guide_bits, guide_scales, stream);
}

fp4_status fp4_fake_quantize(const fp4_cfg* cfg, int guided, const void* x_bf16, int64_t rows,
                             int64_t cols, int64_t ld, const float* tensor_scale,
                             const void* guide_bits, const void* guide_scales, void* out_bf16,
                             int64_t ld_out, hipStream_t stream) {
    FP4Q_TRY(check_cfg(cfg));
    uint64_t ng = 0;
    FP4Q_TRY(check_matrix(rows, cols, ld, block_of(cfg->format), x_bf16, &ng));
    if (ng == 0) return ok();
    FP4Q_TRY(need(out_bf16, 16, "out_bf16"));
    if (ld_out < cols) return fail(FP4_ERR_SHAPE, "ld_out=%lld < cols=%lld", (long long)ld_out, (long long)cols);
    if (ld_out % 8 != 0) return fail(FP4_ERR_ALIGN, "ld_out=%lld is not a multiple of 8", (long long)ld_out);
    if (cfg->format == FP4_NVFP4) FP4Q_TRY(need(tensor_scale, 4, "tensor_scale"));
    if (guided) {
        FP4Q_TRY(need(guide_bits, 16, "guide_bits"));
        FP4Q_TRY(need(guide_scales, 1, "guide_scales"));
    }
    fp4q::QuantParams p{};
    p.x = static_cast<const uint16_t*>(x_bf16);
    p.ld = ld;
    p.ngroups = (uint32_t)ng;
    p.gpr = fp4q::make_fastdiv((uint32_t)(cols / 16));
    p.ts = tensor_scale;
    p.gbits = static_cast<const uint8_t*>(guide_bits);
    p.gscales = static_cast<const uint8_t*>(guide_scales);
    p.key0 = (uint32_t)cfg->sr_seed;
    p.key1 = (uint32_t)(cfg->sr_seed >> 32);
    p.sr_offset = cfg->sr_offset;
    p.rht_seed = cfg->rht_seed;
    p.stream_out = (uint32_t)cfg->stream_out;
    p.fq_out = static_cast<uint16_t*>(out_bf16);
    p.ld_out = ld_out;
    const int mode = guided ? fp4q::MODE_GUIDED : (cfg->rounding == FP4_SR ? fp4q::MODE_SR : fp4q::MODE_RTN);
    return hip_status(fp4q::launch_fake_quantize(cfg->format, cfg->grid, mode, cfg->rht16 != 0, ld == cols, p, stream),
                      "fake quantize launch");
}

fp4_status fp4_guide_mismatch(const fp4_cfg* cfg, const void* x_bf16, int64_t rows, int64_t cols, int64_t ld,
                              const float* tensor_scale, const void* rollout_codes, const void* rollout_scales,
                              unsigned long long* counts, hipStream_t stream) {
    FP4Q_TRY(check_cfg(cfg));
    FP4Q_TRY(need(counts, 8, "counts"));
    uint64_t ng = 0;
    FP4Q_TRY(check_matrix(rows, cols, ld, block_of(cfg->format), x_bf16, &ng));
    fp4q::QuantParams p{};
    p.counts = counts;
    if (ng == 0) {   // nothing to count: clear the counters and return
        p.ngroups = 0;
        return hip_status(fp4q::launch_guide_mismatch(cfg->format, cfg->grid, cfg->rht16 != 0, true, p, stream),
                          "guide mismatch launch");
    }
    FP4Q_TRY(need(rollout_codes, 16, "rollout_codes"));
    FP4Q_TRY(need(rollout_scales, 1, "rollout_scales"));
    if (cfg->format == FP4_NVFP4) FP4Q_TRY(need(tensor_scale, 4, "tensor_scale"));
    p.x = static_cast<const uint16_t*>(x_bf16);
    p.ld = ld;
    p.ngroups = (uint32_t)ng;
    p.gpr = fp4q::make_fastdiv((uint32_t)(cols / 16));
    p.ts = tensor_scale;
    p.rcodes = static_cast<const uint8_t*>(rollout_codes);
    p.gscales = static_cast<const uint8_t*>(rollout_scales);
    p.rht_seed = cfg->rht_seed;
    return hip_status(fp4q::launch_guide_mismatch(cfg->format, cfg->grid, cfg->rht16 != 0, ld == cols, p, stream),
                      "guide mismatch launch");
}

fp4_status fp4_dequantize(const fp4_cfg* cfg, const void* codes, const void* scales,
                          const float* tensor_scale, int64_t rows, int64_t cols, void* out,
                          int64_t ld_out, fp4_dtype dtype, hipStream_t stream) {
    FP4Q_TRY(check_cfg(cfg));
    if (dtype != FP4_OUT_F32 && dtype != FP4_OUT_BF16) return fail(FP4_ERR_ARG, "unknown dtype %d", (int)dtype);
    uint64_t ng = 0;
    FP4Q_TRY(check_matrix(rows, cols, cols, block_of(cfg->format), codes ? codes : (const void*)16, &ng));
    if (ng == 0) return ok();
    FP4Q_TRY(need(codes, 16, "codes"));
    FP4Q_TRY(need(scales, 1, "scales"));
    FP4Q_TRY(need(out, 16, "out"));
    if (cfg->format == FP4_NVFP4) FP4Q_TRY(need(tensor_scale, 4, "tensor_scale"));
    if (ld_out < cols) return fail(FP4_ERR_SHAPE, "ld_out=%lld < cols=%lld", (long long)ld_out, (long long)cols);
    const int64_t esz = dtype == FP4_OUT_BF16 ? 2 : 4;
    if ((ld_out * esz) % 16 != 0) return fail(FP4_ERR_ALIGN, "output row stride is not a multiple of 16 bytes");
    fp4q::DequantParams p{};
    p.codes = static_cast<const uint8_t*>(codes);
    p.scales = static_cast<const uint8_t*>(scales);
    p.ts = tensor_scale;
    p.out = out;
    p.ld_out = ld_out;
    p.ngroups = (uint32_t)ng;
    p.gpr = fp4q::make_fastdiv((uint32_t)(cols / 16));
    return hip_status(fp4q::launch_dequantize(cfg->format, cfg->grid, dtype == FP4_OUT_BF16, p, stream),
                      "dequantize launch");
}

static fp4_status guide_common(const fp4_cfg* cfg, int64_t rows, int64_t cols, const void* in,
                               const void* scales_in, void* out, void* scales_out, uint64_t* ng) {
    FP4Q_TRY(check_cfg(cfg));
    FP4Q_TRY(check_matrix(rows, cols, cols, block_of(cfg->format), in ? in : (const void*)16, ng));
    if (*ng == 0) return ok();
    FP4Q_TRY(need(in, 16, "input"));
    FP4Q_TRY(need(scales_in, 1, "scales input"));
    FP4Q_TRY(need(out, 16, "output"));
    FP4Q_TRY(need(scales_out, 1, "scales output"));
    return FP4_OK;
}

fp4_status guide_pack(const fp4_cfg* cfg, const void* codes, const void* scales, int64_t rows,
                      int64_t cols, void* guide_bits, void* guide_scales, hipStream_t stream) {
    uint64_t ng = 0;
    FP4Q_TRY(guide_common(cfg, rows, cols, codes, scales, guide_bits, guide_scales, &ng));
    if (ng == 0) return ok();
    fp4q::GuideParams p{static_cast<const uint8_t*>(codes), static_cast<const uint8_t*>(scales),
                        static_cast<uint8_t*>(guide_bits), static_cast<uint8_t*>(guide_scales),
                        (uint32_t)ng};
    return hip_status(fp4q::launch_guide_pack(cfg->format, p, stream), "guide_pack launch");
}

fp4_status guide_pack_grouped(const fp4_cfg* cfg, int n, const fp4_guide_desc* tensors, hipStream_t stream) {
    FP4Q_TRY(check_cfg(cfg));
    if (n < 1 || n > fp4q::kMaxGroup) return fail(FP4_ERR_ARG, "n=%d outside 1..%d", n, fp4q::kMaxGroup);
    if (!tensors) return fail(FP4_ERR_ARG, "tensors is NULL");
    fp4q::GroupedGuideParams gp{};
    for (int t = 0; t < n; ++t) {
        const fp4_guide_desc& d = tensors[t];
        uint64_t ng = 0;
        const fp4_status st = guide_common(cfg, d.rows, d.cols, d.codes, d.scales, d.guide_bits, d.guide_scales, &ng);
        if (st != FP4_OK) {
            char msg[512];
            snprintf(msg, sizeof msg, "%s", g_err);
            return fail(st, "tensor %d: %s", t, msg);
        }
        if (ng == 0) continue;
        gp.t[gp.n++] = fp4q::GuideParams{static_cast<const uint8_t*>(d.codes), static_cast<const uint8_t*>(d.scales),
                                         static_cast<uint8_t*>(d.guide_bits), static_cast<uint8_t*>(d.guide_scales),
                                         (uint32_t)ng};
    }
    if (gp.n == 0) return ok();
    return hip_status(fp4q::launch_guide_pack_grouped(cfg->format, gp, stream), "grouped guide_pack launch");
}

fp4_status guide_unpack(const fp4_cfg* cfg, const void* guide_bits, const void* guide_scales,
                        int64_t rows, int64_t cols, void* mant_u8, void* scales_out,
                        hipStream_t stream) {
    uint64_t ng = 0;
    FP4Q_TRY(guide_common(cfg, rows, cols, guide_bits, guide_scales, mant_u8, scales_out, &ng));
    if (ng == 0) return ok();
    fp4q::GuideParams p{static_cast<const uint8_t*>(guide_bits), static_cast<const uint8_t*>(guide_scales),
                        static_cast<uint8_t*>(mant_u8), static_cast<uint8_t*>(scales_out), (uint32_t)ng};
    return hip_status(fp4q::launch_guide_unpack(cfg->format, p, stream), "guide_unpack launch");
}

}  // extern "C"

namespace {

// Checks one product's arguments and fills its parameter block; *empty is set
// when M or N is 0 (nothing to do).
fp4_status gemm_params(const void* a_codes, const void* a_scales, const void* b_codes, const void* b_scales,
                       int64_t M, int64_t N, int64_t K, void* c, int64_t ldc, fp4_dtype dtype, fp4q::GemmParams* p,
                       bool* empty, bool store_c = true) {
    if (dtype != FP4_OUT_F32 && dtype != FP4_OUT_BF16) return fail(FP4_ERR_ARG, "unknown dtype %d", (int)dtype);
    if (M < 0 || N < 0 || K < 0)
        return fail(FP4_ERR_ARG, "negative shape M=%lld N=%lld K=%lld", (long long)M, (long long)N, (long long)K);
    if (K % 32 != 0) return fail(FP4_ERR_SHAPE, "K=%lld is not a multiple of 32", (long long)K);
    *empty = M == 0 || N == 0;
    if (*empty) return FP4_OK;
    if (M >= (1ll << 31) || N >= (1ll << 31) || K >= (1ll << 40))
        return fail(FP4_ERR_SHAPE, "shape too large M=%lld N=%lld K=%lld", (long long)M, (long long)N, (long long)K);
    if ((uint64_t)((M + 127) / 128) * (uint64_t)((N + 127) / 128) >= (1ull << 31))
        return fail(FP4_ERR_SHAPE, "too many 128 x 128 tiles of C");
    if (store_c) {
        if (ldc < N) return fail(FP4_ERR_SHAPE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
        // the stores address a 256-row band of C with 32-bit offsets
        if (ldc > (1ll << 21)) return fail(FP4_ERR_SHAPE, "ldc=%lld too large", (long long)ldc);
        FP4Q_TRY(need(c, dtype == FP4_OUT_BF16 ? 2 : 4, "c"));
    }
    if (K > 0) {
        FP4Q_TRY(need(a_codes, 16, "a_codes"));
        FP4Q_TRY(need(a_scales, 1, "a_scales"));
        FP4Q_TRY(need(b_codes, 16, "b_codes"));
        FP4Q_TRY(need(b_scales, 1, "b_scales"));
    }
    *p = fp4q::GemmParams{};
    p->a = static_cast<const uint8_t*>(a_codes);
    p->as = static_cast<const uint8_t*>(a_scales);
    p->b = static_cast<const uint8_t*>(b_codes);
    p->bs = static_cast<const uint8_t*>(b_scales);
    p->c = c;
    p->ldc = ldc;
    p->M = M;
    p->N = N;
    p->K = K;
    p->tiles_n = (uint32_t)((N + 127) / 128);
    return FP4_OK;
}

}  // namespace

extern "C" {

fp4_status fp4_gemm_mxfp4(const void* a_codes, const void* a_scales, const void* b_codes, const void* b_scales,
                          int64_t M, int64_t N, int64_t K, void* c, int64_t ldc, fp4_dtype dtype,
                          hipStream_t stream) {
    fp4q::GemmParams p{};
    bool empty = false;
    FP4Q_TRY(gemm_params(a_codes, a_scales, b_codes, b_scales, M, N, K, c, ldc, dtype, &p, &empty));
    if (empty) return ok();
    return hip_status(fp4q::launch_gemm_mx(dtype == FP4_OUT_BF16, p, stream), "gemm launch");
}

static fp4_status gemm_quantize(const void* a_codes, const void* a_scales, const void* b_codes,
                                const void* b_scales, int64_t M, int64_t N, int64_t K, const float* tensor_scale,
                                void* c_codes, void* c_scales, void* c_guide_bits, hipStream_t stream) {
    fp4q::GemmParams p{};
    bool empty = false;
    FP4Q_TRY(gemm_params(a_codes, a_scales, b_codes, b_scales, M, N, K, nullptr, 0, FP4_OUT_BF16, &p, &empty, false));
    if (N % 32 != 0)
        return fail(FP4_ERR_SHAPE, "N=%lld is not a multiple of 32 (the blocks of the result's quantization)",
                    (long long)N);
    if (empty) return ok();
    if ((uint64_t)M * (uint64_t)N / 16 >= (1ull << 31))
        return fail(FP4_ERR_SHAPE, "result too large to quantize (%lld x %lld)", (long long)M, (long long)N);
    FP4Q_TRY(need(c_codes, 16, "c_codes"));
    FP4Q_TRY(need(c_scales, tensor_scale ? 2 : 1, "c_scales"));   // NVFP4: two scale bytes per store
    if (c_guide_bits) FP4Q_TRY(need(c_guide_bits, 16, "c_guide_bits"));
    if (!fp4q::gemm_quant_supported(p))
        return fail(FP4_ERR_UNSUPPORTED, "the quantizing product needs K a positive multiple of 512 (K=%lld) and "
                                         "16-byte aligned scales", (long long)K);
    p.qcodes = static_cast<uint8_t*>(c_codes);
    p.qscales = static_cast<uint8_t*>(c_scales);
    p.qbits = static_cast<uint8_t*>(c_guide_bits);
    p.qts = tensor_scale;
    return hip_status(fp4q::launch_gemm_mx_quant(p, stream), "quantizing gemm launch");
}

fp4_status fp4_gemm_mxfp4_quantize(const void* a_codes, const void* a_scales, const void* b_codes,
                                   const void* b_scales, int64_t M, int64_t N, int64_t K, void* c_codes,
                                   void* c_scales, void* c_guide_bits, hipStream_t stream) {
    return gemm_quantize(a_codes, a_scales, b_codes, b_scales, M, N, K, nullptr, c_codes, c_scales, c_guide_bits,
                         stream);
}

fp4_status fp4_gemm_mxfp4_quantize_nvfp4(const void* a_codes, const void* a_scales, const void* b_codes,
                                         const void* b_scales, int64_t M, int64_t N, int64_t K,
                                         const float* tensor_scale, void* c_codes, void* c_scales,
                                         void* c_guide_bits, hipStream_t stream) {
    FP4Q_TRY(need(tensor_scale, 4, "tensor_scale"));
    return gemm_quantize(a_codes, a_scales, b_codes, b_scales, M, N, K, tensor_scale, c_codes, c_scales,
                         c_guide_bits, stream);
}

fp4_status fp4_gemm_mxfp4_grouped(int n, const fp4_gemm_desc* products, fp4_dtype dtype, hipStream_t stream) {
    if (n < 1 || n > fp4q::kMaxGemmGroup) return fail(FP4_ERR_ARG, "n=%d outside 1..%d", n, fp4q::kMaxGemmGroup);
    if (!products) return fail(FP4_ERR_ARG, "products is NULL");
    fp4q::GroupedGemmParams gp{};
    for (int i = 0; i < n; ++i) {
        const fp4_gemm_desc& d = products[i];
        fp4q::GemmParams p{};
        bool empty = false;
        const fp4_status st = gemm_params(d.a_codes, d.a_scales, d.b_codes, d.b_scales, d.M, d.N, d.K, d.c, d.ldc,
                                          dtype, &p, &empty);
        if (st != FP4_OK) {
            char msg[512];
            snprintf(msg, sizeof msg, "%s", g_err);
            return fail(st, "product %d: %s", i, msg);
        }
        if (!empty) gp.g[gp.n++] = p;
    }
    if (gp.n == 0) return ok();
    return hip_status(fp4q::launch_gemm_mx_grouped(dtype == FP4_OUT_BF16, gp, stream), "grouped gemm launch");
}

fp4_status fp4_rht16(const void* x_bf16, int64_t rows, int64_t cols, int64_t ld, uint64_t seed,
                     int inverse, void* out, fp4_dtype dtype, hipStream_t stream) {
    if (dtype != FP4_OUT_F32 && dtype != FP4_OUT_BF16) return fail(FP4_ERR_ARG, "unknown dtype %d", (int)dtype);
    uint64_t ng = 0;
    FP4Q_TRY(check_matrix(rows, cols, ld, 16, x_bf16, &ng));
    if (ng == 0) return ok();
    FP4Q_TRY(need(out, 16, "out"));
    fp4q::RhtParams p{};
    p.x = static_cast<const uint16_t*>(x_bf16);
    p.ld = ld;
    p.out = out;
    p.ngroups = (uint32_t)ng;
    p.gpr = fp4q::make_fastdiv((uint32_t)(cols / 16));
    p.seed = seed;
    return hip_status(fp4q::launch_rht16(inverse != 0, dtype == FP4_OUT_BF16, ld == cols, p, stream),
                      "rht16 launch");
}

fp4_status fp4_encode_scales(const float* t, int64_t n, uint8_t* out, hipStream_t stream) {
    if (n < 0 || n % 4 != 0) return fail(FP4_ERR_SHAPE, "n=%lld must be a non-negative multiple of 4", (long long)n);
    if (n / 4 >= (1ll << 31)) return fail(FP4_ERR_SHAPE, "n too large");
    if (n == 0) return ok();
    FP4Q_TRY(need(t, 16, "t"));
    FP4Q_TRY(need(out, 4, "out"));
    return hip_status(fp4q::launch_encode_scales(t, out, (uint32_t)(n / 4), stream), "encode_scales launch");
}

fp4_status fp4_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return ok();
    if (bytes % 16 != 0) return fail(FP4_ERR_SHAPE, "bytes=%zu is not a multiple of 16", bytes);
    if (bytes / 16 / fp4q::kThreads >= (1ull << 31)) return fail(FP4_ERR_SHAPE, "copy too large");
    FP4Q_TRY(need(src, 16, "src"));
    FP4Q_TRY(need(dst, 16, "dst"));
    const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
    if (a < b + bytes && b < a + bytes) return fail(FP4_ERR_ARG, "src and dst overlap");
    return hip_status(fp4q::launch_stream_copy(src, dst, bytes / 16, stream), "stream copy launch");
}

fp4_status fp4_encode_values(int grid, int mode, const float* v, const uint8_t* aux, int64_t n,
                             uint8_t* out, hipStream_t stream) {
    if (grid != FP4_GRID_E2M1 && grid != FP4_GRID_UNIFORM) return fail(FP4_ERR_ARG, "unknown grid %d", grid);
    if (mode != FP4_MODE_RTN && mode != FP4_MODE_SR && mode != FP4_MODE_GUIDED)
        return fail(FP4_ERR_ARG, "unknown mode %d", mode);
    if (n < 0 || n % 8 != 0) return fail(FP4_ERR_SHAPE, "n=%lld must be a non-negative multiple of 8", (long long)n);
    if (n / 8 >= (1ll << 31)) return fail(FP4_ERR_SHAPE, "n too large");
    if (n == 0) return ok();
    FP4Q_TRY(need(v, 16, "v"));
    FP4Q_TRY(need(out, 8, "out"));
    if (mode != FP4_MODE_RTN) FP4Q_TRY(need(aux, 8, "aux"));
    if (aux && !aligned(aux, 8)) return fail(FP4_ERR_ALIGN, "aux is not 8-byte aligned");
    fp4q::EncodeParams p{v, aux, out, (uint32_t)(n / 8)};
    return hip_status(fp4q::launch_encode_values(grid, mode, p, stream), "encode_values launch");
}

}  // extern "C"
