// quantize.hip -- block-scaled FP4 quantization kernels for gfx950.
//
// Work mapping: one lane owns one 16-element group of a row (32 bytes of
// bf16 = two 128-bit loads).  A wave covers 64 consecutive groups, so each
// load instruction of a wave spans 2 KiB of the row-major input and the
// 8-byte code stores of a wave are one contiguous 512-byte run.  An NVFP4
// block (16) is one lane; an MXFP4 block (32) is a lane pair whose amax is
// exchanged with one DPP quad permutation.  Each lane processes U groups
// (spaced one workgroup-width apart) with all loads issued first, so every
// lane keeps U*32 bytes in flight.
//
// Per block (scale) [FQT-FP4 §3; TETRAJET §3; TRACE-JA "TRACEの仕組み"]:
//   NVFP4 scale code = E4M3 RNE of amax / RN(Gmax*s_t) (clamped to 448),
//         inv = RN(1/RN(dec(code)*s_t));
//   MXFP4 scale code = max(E(amax) - 2, 0) (E the biased exponent field),
//         inv = 2^-(code-127);
//   guided: the code comes from the guide.
// Per element: v = RN(y*inv), then the grid rounding of device.h.
#include "device.h"
#include "internal.h"

namespace fp4q {

namespace {

#ifndef FP4Q_GROUPS_PER_LANE
#define FP4Q_GROUPS_PER_LANE 1
#endif
constexpr int kGroupsPerLane = FP4Q_GROUPS_PER_LANE;

template <bool CONTIG>
__device__ __forceinline__ int64_t group_offset(uint32_t g, const QuantParams& p) {
    if constexpr (CONTIG) {
        return (int64_t)g * 16;
    } else {
        const uint32_t row = fastdiv(g, p.gpr);
        const uint32_t cg = g - row * p.gpr.d;
        return (int64_t)row * p.ld + (int64_t)cg * 16;
    }
}

__device__ __forceinline__ uint32_t dpp_swap_pair(uint32_t v) {
    // quad_perm [1,0,3,2]: exchange with the neighbouring lane
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}

template <int FMT, int GRID, int MODE, bool RHT, bool EMIT, bool CONTIG>
__global__ __launch_bounds__(kThreads) void k_quantize(const QuantParams p) {
    constexpr int U = kGroupsPerLane;
    constexpr float kGmax = GRID == 0 ? 6.0f : 7.0f;
    const uint32_t g0 = blockIdx.x * (kThreads * U) + threadIdx.x;

    uint32_t w[U][8];
    uint32_t gb[U];
    uint32_t gs[U];
    #pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t g = g0 + u * kThreads;
        if (g < p.ngroups) {
            load32_nt(p.x + group_offset<CONTIG>(g, p), w[u]);
            if constexpr (MODE == MODE_GUIDED) {
                gb[u] = reinterpret_cast<const uint16_t*>(p.gbits)[g];
                gs[u] = p.gscales[FMT == 0 ? g : (g >> 1)];
            }
        }
    }

    const uint32_t signs = RHT ? rht_sign_mask(p.rht_seed) : 0u;   // uniform: scalar unit
    float ts = 1.0f, denom = 1.0f;
    if constexpr (FMT == 0) {
        ts = *p.ts;
        denom = kGmax * ts;
    }

    #pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t g = g0 + u * kThreads;
        if (g >= p.ngroups) continue;

        float y[16];
        widen16<RHT>(w[u], signs, y);

        // block amax (not needed in guided mode except for the finiteness test)
        bool finite;
        uint32_t amax_key;  // monotone key of the amax (bf16 bits, or fp32 bits with RHT)
        if constexpr (RHT) {
            float m = 0.0f;
            #pragma unroll
            for (int j = 0; j < 16; ++j) m = __builtin_elementwise_maximum(m, fabsf(y[j]));
            amax_key = __float_as_uint(m);          // NaN propagates: bits > 0x7F800000
        } else {
            amax_key = amax_bits16(w[u]) << 16;     // as fp32 bits
        }
        if constexpr (FMT == 1) amax_key = max(amax_key, dpp_swap_pair(amax_key));
        finite = amax_key < 0x7F800000u;

        uint32_t sc;
        float inv;
        if constexpr (MODE == MODE_GUIDED) {
            sc = gs[u];
            if constexpr (FMT == 0) {
                finite = finite && ((sc & 0x7Fu) != 0x7Fu);
                inv = nvfp4_inv(sc, ts);
            } else {
                finite = finite && (sc != 0xFFu);
                inv = mx_inv(sc);
            }
        } else if constexpr (FMT == 0) {
            const float t = __uint_as_float(amax_key) / denom;
            sc = e4m3_encode_rne(fminf(t, 448.0f));
            inv = nvfp4_inv(sc, ts);
            if (!finite) sc = 0x7Fu;
        } else {
            const uint32_t e = amax_key >> 23;
            sc = e > 2u ? e - 2u : 0u;
            inv = mx_inv(sc);
            if (!finite) sc = 0xFFu;
        }

        uint32_t r0 = 0, r1 = 0, r2 = 0, r3 = 0;
        if constexpr (MODE == MODE_SR) {
            const uint64_t ctr = (uint64_t)g + p.sr_offset;
            const u32x4 r = philox4x32_10((uint32_t)ctr, (uint32_t)(ctr >> 32), 0u, 0u, p.key0, p.key1);
            r0 = r.w[0]; r1 = r.w[1]; r2 = r.w[2]; r3 = r.w[3];
        }
        const uint32_t gbits = MODE == MODE_GUIDED ? gb[u] : 0u;

        float v[16];
        #pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = y[j] * inv;
        uint32_t c0 = encode8<GRID, MODE>(v, r0, r1, gbits & 0xFFu);
        uint32_t c1 = encode8<GRID, MODE>(v + 8, r2, r3, gbits >> 8);
        if (!finite) { c0 = 0; c1 = 0; }

        st_out2(p.codes, g, c0, c1);
        if constexpr (FMT == 0) {
            st_out(p.scales + g, (uint8_t)sc);
        } else {
            if ((g & 1u) == 0) st_out(p.scales + (g >> 1), (uint8_t)sc);
        }
        if constexpr (EMIT) {
            st_out(reinterpret_cast<uint16_t*>(p.bits_out) + g,
                   (uint16_t)(gather_nibble_lsbs(c0) | (gather_nibble_lsbs(c1) << 8)));
        }
    }
}

template <int FMT, int GRID, int MODE, bool RHT, bool EMIT, bool CONTIG>
hipError_t launch_t(const QuantParams& p, hipStream_t s) {
    const uint32_t per_block = kThreads * kGroupsPerLane;
    const uint32_t blocks = (p.ngroups + per_block - 1) / per_block;
    hipLaunchKernelGGL((k_quantize<FMT, GRID, MODE, RHT, EMIT, CONTIG>), dim3(blocks), dim3(kThreads),
                       0, s, p);
    return hipGetLastError();
}

template <int FMT, int GRID, int MODE, bool RHT, bool EMIT>
hipError_t launch_c(bool contig, const QuantParams& p, hipStream_t s) {
    return contig ? launch_t<FMT, GRID, MODE, RHT, EMIT, true>(p, s)
                  : launch_t<FMT, GRID, MODE, RHT, EMIT, false>(p, s);
}

template <int FMT, int GRID, int MODE, bool RHT>
hipError_t launch_e(bool emit, bool contig, const QuantParams& p, hipStream_t s) {
    if constexpr (MODE == MODE_GUIDED) {
        return launch_c<FMT, GRID, MODE, RHT, false>(contig, p, s);
    } else {
        return emit ? launch_c<FMT, GRID, MODE, RHT, true>(contig, p, s)
                    : launch_c<FMT, GRID, MODE, RHT, false>(contig, p, s);
    }
}

template <int FMT, int GRID, int MODE>
hipError_t launch_r(bool rht, bool emit, bool contig, const QuantParams& p, hipStream_t s) {
    return rht ? launch_e<FMT, GRID, MODE, true>(emit, contig, p, s)
               : launch_e<FMT, GRID, MODE, false>(emit, contig, p, s);
}

template <int FMT, int GRID>
hipError_t launch_m(int mode, bool rht, bool emit, bool contig, const QuantParams& p, hipStream_t s) {
    switch (mode) {
        case MODE_RTN: return launch_r<FMT, GRID, MODE_RTN>(rht, emit, contig, p, s);
        case MODE_SR: return launch_r<FMT, GRID, MODE_SR>(rht, emit, contig, p, s);
        default: return launch_r<FMT, GRID, MODE_GUIDED>(rht, emit, contig, p, s);
    }
}

}  // namespace

hipError_t launch_quantize(int format, int grid, int mode, bool rht, bool emit, bool contig,
                           const QuantParams& p, hipStream_t s) {
    if (format == 0) {
        return grid == 0 ? launch_m<0, 0>(mode, rht, emit, contig, p, s)
                         : launch_m<0, 1>(mode, rht, emit, contig, p, s);
    }
    return grid == 0 ? launch_m<1, 0>(mode, rht, emit, contig, p, s)
                     : launch_m<1, 1>(mode, rht, emit, contig, p, s);
}

}  // namespace fp4q
