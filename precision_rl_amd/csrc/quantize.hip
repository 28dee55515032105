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

// One workgroup's share (kThreads * U groups starting at chunk `wg`) of one tensor.
// OUT = 0 stores codes, scales (and emitted guide bits); OUT = 1 stores the
// dequantized bf16 values instead (fake quantization).
template <int FMT, int GRID, int MODE, bool RHT, bool EMIT, bool CONTIG, int OUT = 0>
__device__ __forceinline__ void quantize_chunk(const QuantParams& p, uint32_t wg) {
    constexpr int U = kGroupsPerLane;
    constexpr float kGmax = GRID == 0 ? 6.0f : 7.0f;
    const uint32_t g0 = wg * (kThreads * U) + threadIdx.x;

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

        if constexpr (OUT == 1) {
            float dv[16];
            const bool ok = dequant16<FMT, GRID>(c0, c1, sc, ts, dv);
            uint32_t o[8];
            to_bf16x16(dv, ok, o);
            const uint32_t row = fastdiv(g, p.gpr);
            uint16_t* dst = p.fq_out + (int64_t)row * p.ld_out + (int64_t)(g - row * p.gpr.d) * 16;
            st_out4(dst, 0, o[0], o[1], o[2], o[3]);
            st_out4(dst, 1, o[4], o[5], o[6], o[7]);
        } else {
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
}

template <int FMT, int GRID, int MODE, bool RHT, bool EMIT, bool CONTIG>
__global__ __launch_bounds__(kThreads) void k_quantize(const QuantParams p) {
    quantize_chunk<FMT, GRID, MODE, RHT, EMIT, CONTIG>(p, blockIdx.x);
}

// Several tensors with one configuration in one launch: workgroup b belongs to
// the tensor t with wg_start[t] <= b < wg_start[t+1] (a uniform scan of at most
// kMaxGroup entries), and processes that tensor's chunk b - wg_start[t].
template <int FMT, int GRID, int MODE, bool RHT, bool EMIT>
__global__ __launch_bounds__(kThreads) void k_quantize_grouped(const GroupedQuantParams gp) {
    const uint32_t b = blockIdx.x;
    uint32_t t = 0;
    while (t + 1 < gp.n && b >= gp.wg_start[t + 1]) ++t;
    const uint32_t wg = b - gp.wg_start[t];
    if ((gp.contig_mask >> t) & 1u)
        quantize_chunk<FMT, GRID, MODE, RHT, EMIT, true>(gp.t[t], wg);
    else
        quantize_chunk<FMT, GRID, MODE, RHT, EMIT, false>(gp.t[t], wg);
}

template <int FMT, int GRID, int MODE, bool RHT, bool EMIT>
hipError_t launch_grouped_t(const GroupedQuantParams& gp, hipStream_t s) {
    const uint32_t blocks = gp.wg_start[gp.n];
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_quantize_grouped<FMT, GRID, MODE, RHT, EMIT>), dim3(blocks), dim3(kThreads), 0, s, gp);
    return hipGetLastError();
}

template <int FMT, int GRID, int MODE, bool RHT, bool CONTIG>
__global__ __launch_bounds__(kThreads) void k_fake_quantize(const QuantParams p) {
    quantize_chunk<FMT, GRID, MODE, RHT, false, CONTIG, 1>(p, blockIdx.x);
}

template <int FMT, int GRID, int MODE>
hipError_t launch_fake_m(bool rht, bool contig, const QuantParams& p, hipStream_t s) {
    const uint32_t per_block = kThreads * kGroupsPerLane;
    const dim3 b((p.ngroups + per_block - 1) / per_block), t(kThreads);
    if (rht) {
        if (contig) hipLaunchKernelGGL((k_fake_quantize<FMT, GRID, MODE, true, true>), b, t, 0, s, p);
        else hipLaunchKernelGGL((k_fake_quantize<FMT, GRID, MODE, true, false>), b, t, 0, s, p);
    } else {
        if (contig) hipLaunchKernelGGL((k_fake_quantize<FMT, GRID, MODE, false, true>), b, t, 0, s, p);
        else hipLaunchKernelGGL((k_fake_quantize<FMT, GRID, MODE, false, false>), b, t, 0, s, p);
    }
    return hipGetLastError();
}

template <int FMT, int GRID>
hipError_t launch_fake_g(int mode, bool rht, bool contig, const QuantParams& p, hipStream_t s) {
    switch (mode) {
        case MODE_RTN: return launch_fake_m<FMT, GRID, MODE_RTN>(rht, contig, p, s);
        case MODE_SR: return launch_fake_m<FMT, GRID, MODE_SR>(rht, contig, p, s);
        default: return launch_fake_m<FMT, GRID, MODE_GUIDED>(rht, contig, p, s);
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

template <int FMT, int GRID, int MODE, bool RHT>
hipError_t launch_grouped_e(bool emit, const GroupedQuantParams& gp, hipStream_t s) {
    if constexpr (MODE == MODE_GUIDED) {
        return launch_grouped_t<FMT, GRID, MODE, RHT, false>(gp, s);
    } else {
        return emit ? launch_grouped_t<FMT, GRID, MODE, RHT, true>(gp, s)
                    : launch_grouped_t<FMT, GRID, MODE, RHT, false>(gp, s);
    }
}

template <int FMT, int GRID>
hipError_t launch_grouped_m(int mode, bool rht, bool emit, const GroupedQuantParams& gp, hipStream_t s) {
    switch (mode) {
        case MODE_RTN:
            return rht ? launch_grouped_e<FMT, GRID, MODE_RTN, true>(emit, gp, s)
                       : launch_grouped_e<FMT, GRID, MODE_RTN, false>(emit, gp, s);
        case MODE_SR:
            return rht ? launch_grouped_e<FMT, GRID, MODE_SR, true>(emit, gp, s)
                       : launch_grouped_e<FMT, GRID, MODE_SR, false>(emit, gp, s);
        default:
            return rht ? launch_grouped_e<FMT, GRID, MODE_GUIDED, true>(emit, gp, s)
                       : launch_grouped_e<FMT, GRID, MODE_GUIDED, false>(emit, gp, s);
    }
}

}  // namespace

uint32_t quantize_chunks(uint32_t ngroups) {
    const uint32_t per = kThreads * kGroupsPerLane;
    return (ngroups + per - 1) / per;
}

hipError_t launch_quantize_grouped(int format, int grid, int mode, bool rht, bool emit,
                                   const GroupedQuantParams& gp, hipStream_t s) {
    if (format == 0) {
        return grid == 0 ? launch_grouped_m<0, 0>(mode, rht, emit, gp, s)
                         : launch_grouped_m<0, 1>(mode, rht, emit, gp, s);
    }
    return grid == 0 ? launch_grouped_m<1, 0>(mode, rht, emit, gp, s)
                     : launch_grouped_m<1, 1>(mode, rht, emit, gp, s);
}

hipError_t launch_fake_quantize(int format, int grid, int mode, bool rht, bool contig,
                                const QuantParams& p, hipStream_t s) {
    if (format == 0) {
        return grid == 0 ? launch_fake_g<0, 0>(mode, rht, contig, p, s)
                         : launch_fake_g<0, 1>(mode, rht, contig, p, s);
    }
    return grid == 0 ? launch_fake_g<1, 0>(mode, rht, contig, p, s)
                     : launch_fake_g<1, 1>(mode, rht, contig, p, s);
}

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
