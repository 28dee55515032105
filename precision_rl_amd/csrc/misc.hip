// misc.hip -- tensor scale, dequantization, guide pack/unpack, standalone RHT16
// and the element-encode entry, for gfx950.
#include <atomic>
#include <mutex>

#include "device.h"
#include "internal.h"

namespace fp4q {

namespace {

__device__ __forceinline__ int64_t row_offset(uint32_t g, FastDiv gpr, int64_t ld) {
    const uint32_t row = fastdiv(g, gpr);
    const uint32_t cg = g - row * gpr.d;
    return (int64_t)row * ld + (int64_t)cg * 16;
}

// ---------------------------------------------------------------- tensor scale
// amax over finite |y| as fp32 bits (order-preserving for non-negative values),
// reduced per wave and merged with one atomic max per wave.

__global__ void k_fill_u32(uint32_t* p, uint32_t v) { *p = v; }

// Each lane keeps U groups (2U half-groups) in flight per iteration of a
// grid-stride loop; the workgroup reduces in LDS and issues one atomic max, so
// a launch of at most kAmaxBlocks workgroups makes at most that many
// same-address atomics.  Those are device-scope, across the XCDs, and cost
// roughly 10-15 ns each: a tensor that fits one pass of 1024 workgroups of
// 4 groups per lane takes 8 groups per lane instead, with half the workgroups
// (4096 x 2048: 10.2 against 12.6 us for the whole tensor scale).  Larger
// tensors keep 4 groups and 1024 workgroups (measured on 512M elements against
// 2 or 8 groups and 256 to 4096 workgroups).
constexpr int kAmaxU = 4;
constexpr int kAmaxUSmall = 8;
constexpr uint32_t kAmaxBlocks = 1024;

// This thread's share of the amax: the largest finite |y| as fp32 bits over the
// groups it loads (0 if none).
template <bool RHT, bool CONTIG, int U>
__device__ __forceinline__ uint32_t amax_thread(const AmaxParams& p) {
    uint32_t m = 0;
    const uint32_t signs = RHT ? rht_sign_mask(p.rht_seed) : 0u;
    const uint32_t lane = threadIdx.x & 63u, q = lane & 1u;
    const uint64_t nhg = 2ull * p.ngroups;
    constexpr int kSlots = 2 * U;                 // half-groups per lane and iteration
    const uint32_t chunk = kThreads * U;          // groups per workgroup and iteration
    for (uint32_t base = blockIdx.x * chunk; base < p.ngroups; base += gridDim.x * chunk) {
        // slot s of a lane reads half-group hg0 + 64 s, so each load instruction
        // of a wave covers 64 consecutive half-groups; past the end a lane reads
        // the last one again
        const uint64_t hg0 = 2ull * base + (threadIdx.x >> 6) * (64u * kSlots) + lane;
        uint32_t w[kSlots][4];
        #pragma unroll
        for (int s = 0; s < kSlots; ++s) {
            const uint64_t hg = min(hg0 + 64u * s, nhg - 1u);
            load16_nt(p.x + half_offset<CONTIG>((uint32_t)hg, p.gpr, p.ld), w[s]);
        }
        #pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (RHT) {
                // whole groups for the transform: after the exchange of slots 2u
                // and 2u+1 this lane holds group (hg0 + 128 u + 64 q) / 2, which
                // counts only if it lies inside the tensor
                uint32_t gw[8];
                pair_exchange(w[2 * u], w[2 * u + 1], q, gw, gw + 4);
                const uint64_t g = (hg0 + 128u * u + 64u * q) >> 1;
                float a[16];   // the transform before its exact factor 1/4
                widen16<true, false>(gw, signs, a);
                uint32_t mg = 0;
                #pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const uint32_t k = __float_as_uint(a[j]) & 0x7FFFFFFFu;
                    mg = k < 0x7F800000u ? max(mg, k) : mg;
                }
                m = g < p.ngroups ? max(m, mg) : m;
            } else {
                // a repeated half-group cannot change the maximum
                #pragma unroll
                for (int s = 2 * u; s < 2 * u + 2; ++s) {
                    #pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t lo = w[s][j] & 0x7FFFu, hi = (w[s][j] >> 16) & 0x7FFFu;
                        m = lo < 0x7F80u ? max(m, lo << 16) : m;
                        m = hi < 0x7F80u ? max(m, hi << 16) : m;
                    }
                }
            }
        }
    }
    if constexpr (RHT) m = __float_as_uint(__uint_as_float(m) * 0.25f);   // exact: max |y| = max |a| / 4
    return m;
}

template <bool RHT, bool CONTIG, int U>
__global__ __launch_bounds__(kThreads) void k_amax(const AmaxParams p) {
    __shared__ uint32_t red[kThreads / 64];
    const uint32_t m = wg_max_t0<kThreads / 64>(amax_thread<RHT, CONTIG, U>(p), red);
    if (threadIdx.x == 0 && m != 0) atomicMax(reinterpret_cast<unsigned int*>(p.acc), m);
}

// ---------------------------------------------------------------- one-launch tensor scale
// Each workgroup stores its maximum, tagged with this call's epoch, in a
// workspace word of its own (device.h, cross-workgroup reduction) and ends;
// workgroup 0 then waits until every word carries the tag, takes their maximum,
// writes s_t and advances the epoch (call_state, end_call: a wait that gives up
// marks the launch, s_t is NaN).  Only workgroup 0 waits, on workgroups that
// never wait themselves, so the grid need not be resident all at once.  Distinct
// words take no atomics: through shared counters, a hundred and more same-
// address atomics per word serialize at about 13 ns each, and agent-scope
// release/acquire fences (an L2 writeback and invalidate per workgroup) cost
// more than the whole pass over a 16 MiB tensor.

template <bool RHT, bool CONTIG>
__global__ __launch_bounds__(kThreads) void k_tensor_scale_1(const AmaxParams p, uint32_t* ws, float gmax448,
                                                             uint32_t polls) {
    __shared__ uint32_t red[kThreads / 64];
    __shared__ CallState cs_sh;
    const uint32_t b = blockIdx.x, nwg = gridDim.x;
    const CallState cs = threadIdx.x == 0 ? call_state(ws + kTsEpoch) : CallState{};
    const uint32_t m = wg_max_t0<kThreads / 64>(amax_thread<RHT, CONTIG, kAmaxU>(p), red);
    uint64_t* const words = reinterpret_cast<uint64_t*>(ws + kTsGather);
    if (threadIdx.x == 0) {
        if (!cs.late) store_agent(words + b, tagged(cs.tag, m));
        cs_sh = cs;
    }
    if (b != 0) return;
    __syncthreads();   // cs_sh; also orders the first use of red before the second
    const CallState c = cs_sh;
    if (c.late) {      // this launch gave up before: s_t is NaN, the state stays
        if (threadIdx.x == 0) *p.acc = __builtin_nanf("");
        return;
    }
    const uint32_t g = wg_max_t0<kThreads / 64>(gather_max<kTsMaxWorkgroups, kThreads>(words, nwg, c.tag, polls), red);
    if (threadIdx.x == 0) {
        *p.acc = g == 0xFFFFFFFFu ? __builtin_nanf("") : ts_from_amax(g, gmax448);
        end_call(ws + kTsEpoch, c.epoch, g == 0xFFFFFFFFu);
    }
}

__global__ void k_ts_finalize(float* acc, float gmax448) {
    *acc = ts_from_amax(__float_as_uint(*acc), gmax448);   // amax bits were accumulated in place
}

template <int U>
void launch_amax(bool rht, bool contig, uint32_t blocks, const AmaxParams& p, hipStream_t s) {
    if (rht) {
        if (contig) hipLaunchKernelGGL((k_amax<true, true, U>), dim3(blocks), dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_amax<true, false, U>), dim3(blocks), dim3(kThreads), 0, s, p);
    } else {
        if (contig) hipLaunchKernelGGL((k_amax<false, true, U>), dim3(blocks), dim3(kThreads), 0, s, p);
        else hipLaunchKernelGGL((k_amax<false, false, U>), dim3(blocks), dim3(kThreads), 0, s, p);
    }
}

// ---------------------------------------------------------------- dequantize
// Work unit: 16 bytes of output, i.e. 8 elements to bf16 (one dword of codes)
// or 4 elements to fp32 (16 bits of codes).  In each of its slots the
// 64 lanes of a wave handle 64 consecutive units, so every store instruction
// of a wave writes 1 KiB contiguously (when ld_out == cols).

// Two slots; bf16 output on four where that still gives kDqWideBlocks
// workgroups (2^27 elements and up).  Back to back, with codes from HBM, four
// are faster (131072 x 8 x 128 NVFP4 to bf16: 110.6 against 115.8 us; 16384 x
// 4096 MXFP4: 29.0 against 29.4), but in the five-kernel step, where the codes
// come from the Infinity Cache just after the guided quantize wrote them, the
// 16384 x 4096 dequantize took 27.6 against 26.9 us; eight slots were slower in
// both (113.5, and 30.5 back to back).
constexpr int kDqSlots = 2;
constexpr int kDqSlotsWide = 4;
constexpr uint64_t kDqWideBlocks = 16384;

template <int FMT, int GRID, bool BF16, int S>
__global__ __launch_bounds__(kThreads) void k_dequantize(const DequantParams p) {
    constexpr uint32_t E = BF16 ? 8u : 4u;                 // elements per unit
    const uint64_t nunits = (uint64_t)p.ngroups * (16u / E);
    const uint64_t u0 = (uint64_t)blockIdx.x * (kThreads * S) + (threadIdx.x >> 6) * (64u * S) + (threadIdx.x & 63u);
    const float ts = FMT == 0 ? *p.ts : 1.0f;
    uint32_t c[S], sc[S];
    #pragma unroll
    for (int s = 0; s < S; ++s) {
        const uint64_t u = u0 + 64u * s;
        c[s] = sc[s] = 0u;
        if (u < nunits) {
            if constexpr (BF16) c[s] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p.codes) + u);
            else c[s] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p.codes) + u);
            sc[s] = p.scales[(u * E) / (FMT == 0 ? 16u : 32u)];   // u*E < 2^35: 64-bit
        }
    }
    #pragma unroll
    for (int s = 0; s < S; ++s) {
        const uint64_t u = u0 + 64u * s;
        if (u >= nunits) continue;
        float v[8];
        const bool ok = dequant8<FMT, GRID>(c[s], sc[s], ts, v);
        const uint32_t g = (uint32_t)(u / (16u / E));        // group of the unit
        const uint32_t row = fastdiv(g, p.gpr);
        const int64_t off = (int64_t)row * p.ld_out + (int64_t)(g - row * p.gpr.d) * 16 +
                            (int64_t)((u * E) & 15u);
        if constexpr (BF16) {
            uint32_t o[4];
            to_bf16x8(v, ok, o);
            st_stream4(reinterpret_cast<uint16_t*>(p.out) + off, 0, o[0], o[1], o[2], o[3]);
        } else {
            uint32_t o[4];
            #pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = ok ? __float_as_uint(v[j]) : 0x7FC00000u;
            st_stream4(reinterpret_cast<float*>(p.out) + off, 0, o[0], o[1], o[2], o[3]);
        }
    }
}

// ---------------------------------------------------------------- guide pack / unpack
// pack: a unit is 32 elements (16 bytes of codes -> 4 bytes of bits, plus the
// unit's scale bytes); unpack: a unit is 16 elements (2 bytes of bits -> 16
// bytes of 0/1).  Slots as in dequantize: loads or stores of a wave are
// contiguous per instruction.

#ifndef FP4Q_GUIDE_SLOTS
#define FP4Q_GUIDE_SLOTS 2
#endif
constexpr int kGuideSlots = FP4Q_GUIDE_SLOTS;   // guide_unpack
// guide_pack: four units per lane for one tensor where that still gives
// kPackWideBlocks workgroups (16384 x 4096 MXFP4: 8.6 against 9.0 us on two,
// 9.2-9.5 on eight), else two (in graphs, 4096 x 1536 NVFP4: 2.9 against 3.15
// us on four, 8192 x 4096 NVFP4 6.1 against 6.35); eight in the grouped launch
// (the nine tensors of an MoE layer: 12.1 against 12.7 us on four, 13.3 on two)
constexpr int kPackSlotsWide = 4;
constexpr uint32_t kPackWideBlocks = 2048;
constexpr int kPackSlotsGrouped = 8;

// Workgroup wg of guide_pack over one tensor.  Every load of the workgroup is
// issued before any of its data is used: lanes past the last whole unit read
// that unit again (in bounds, no branch) and store nothing.  (Loads under a
// branch per slot made the compiler wait for the codes before it issued the
// scale loads, two memory round trips per wave.)  An odd NVFP4 group count
// leaves a last unit of one group (8 bytes of codes), which the lane that owns
// it handles on its own.
template <int FMT, int S>
__device__ __forceinline__ void guide_pack_wg(const GuideParams& p, uint32_t wg) {
    const uint32_t nfull = p.ngroups >> 1;              // units of two groups
    const uint32_t u0 = wg * (kThreads * S) + (threadIdx.x >> 6) * (64u * S) + (threadIdx.x & 63u);
    if (nfull > 0) {
        v4u32 c[S];
        uint32_t sc[S];
        #pragma unroll
        for (int s = 0; s < S; ++s) {
            const uint32_t u = min(u0 + 64u * s, nfull - 1u);
            c[s] = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p.in) + u);
            if constexpr (FMT == 0) sc[s] = p.scales_in[2 * u] | ((uint32_t)p.scales_in[2 * u + 1] << 8);
            else sc[s] = p.scales_in[u];
        }
        #pragma unroll
        for (int s = 0; s < S; ++s) {
            const uint32_t u = u0 + 64u * s;
            if (u >= nfull) continue;
            const uint32_t bits = gather_nibble_lsbs(c[s].x) | (gather_nibble_lsbs(c[s].y) << 8) |
                                  (gather_nibble_lsbs(c[s].z) << 16) | (gather_nibble_lsbs(c[s].w) << 24);
            st_out(reinterpret_cast<uint32_t*>(p.out) + u, bits);
            if constexpr (FMT == 0) {
                st_out(p.scales_out + 2 * u, (uint8_t)sc[s]);
                st_out(p.scales_out + 2 * u + 1, (uint8_t)(sc[s] >> 8));
            } else {
                st_out(p.scales_out + u, (uint8_t)sc[s]);
            }
        }
    }
    if (p.ngroups & 1u) {   // NVFP4 only: the last unit is group 2 nfull alone
        #pragma unroll
        for (int s = 0; s < S; ++s) {
            if (u0 + 64u * s != nfull) continue;
            const v2u32 h = reinterpret_cast<const v2u32*>(p.in)[2 * nfull];
            const uint32_t bits = gather_nibble_lsbs(h.x) | (gather_nibble_lsbs(h.y) << 8);
            st_out(reinterpret_cast<uint16_t*>(p.out) + 2 * nfull, (uint16_t)bits);
            st_out(p.scales_out + 2 * nfull, p.scales_in[2 * nfull]);
        }
    }
}

template <int FMT, int S>
__global__ __launch_bounds__(kThreads) void k_guide_pack(const GuideParams p) {
    guide_pack_wg<FMT, S>(p, blockIdx.x);
}

// Up to kMaxGroup tensors in one launch: tensor t takes workgroups
// wg_start[t] .. wg_start[t + 1] - 1.
template <int FMT>
__global__ __launch_bounds__(kThreads) void k_guide_pack_grouped(const GroupedGuideParams gp) {
    const uint32_t t = group_of<kMaxGroup>(gp.wg_start, gp.n, blockIdx.x);
    guide_pack_wg<FMT, kPackSlotsGrouped>(gp.t[t], blockIdx.x - gp.wg_start[t]);
}

__device__ __forceinline__ uint32_t bits4_to_bytes(uint32_t b) {
    return ((b & 0xFu) * 0x00204081u) & 0x01010101u;
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void k_guide_unpack(const GuideParams p) {
    const uint32_t u0 = blockIdx.x * (kThreads * kGuideSlots) + (threadIdx.x >> 6) * (64u * kGuideSlots) +
                        (threadIdx.x & 63u);
    if (p.ngroups == 0) return;
    // every load issued before any is used: lanes past the end read the last
    // group again (in bounds, no branch) and store nothing
    uint32_t b[kGuideSlots], sc[kGuideSlots];
    #pragma unroll
    for (int s = 0; s < kGuideSlots; ++s) {
        const uint32_t g = min(u0 + 64u * s, p.ngroups - 1u);
        b[s] = reinterpret_cast<const uint16_t*>(p.in)[g];
        sc[s] = p.scales_in[FMT == 0 ? g : (g >> 1)];
    }
    #pragma unroll
    for (int s = 0; s < kGuideSlots; ++s) {
        const uint32_t g = u0 + 64u * s;
        if (g >= p.ngroups) continue;
        st_out4(p.out, g, bits4_to_bytes(b[s]), bits4_to_bytes(b[s] >> 4), bits4_to_bytes(b[s] >> 8),
                bits4_to_bytes(b[s] >> 12));
        if (FMT == 0) st_out(p.scales_out + g, (uint8_t)sc[s]);
        else if ((g & 1u) == 0) st_out(p.scales_out + (g >> 1), (uint8_t)sc[s]);
    }
}

// ---------------------------------------------------------------- RHT16

template <bool INVERSE, bool BF16, bool CONTIG>
__global__ __launch_bounds__(kThreads) void k_rht16(const RhtParams p) {
    const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
    if (g >= p.ngroups) return;
    const uint32_t signs = rht_sign_mask(p.seed);
    const int64_t off = CONTIG ? (int64_t)g * 16 : row_offset(g, p.gpr, p.ld);
    const uint4* src = reinterpret_cast<const uint4*>(p.x + off);
    const uint4 a = src[0], b = src[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float y[16];
    if constexpr (INVERSE) {
        widen16<false>(w, 0u, y);
        butterfly16(y);
        #pragma unroll
        for (int j = 0; j < 16; ++j)
            y[j] = __uint_as_float(__float_as_uint(y[j] * 0.25f) ^ (((signs >> j) & 1u) << 31));
    } else {
        widen16<true>(w, signs, y);
    }
    if constexpr (BF16) {
        uint32_t o[8];
        #pragma unroll
        for (int j = 0; j < 8; ++j)
            o[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){y[2 * j], y[2 * j + 1]}, bf16x2));
        uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.out) + (int64_t)g * 16);
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    } else {
        uint4* dst = reinterpret_cast<uint4*>(reinterpret_cast<float*>(p.out) + (int64_t)g * 16);
        #pragma unroll
        for (int q = 0; q < 4; ++q)
            dst[q] = make_uint4(__float_as_uint(y[4 * q]), __float_as_uint(y[4 * q + 1]),
                                __float_as_uint(y[4 * q + 2]), __float_as_uint(y[4 * q + 3]));
    }
}

// ---------------------------------------------------------------- element encode

template <int GRID, int MODE>
__global__ __launch_bounds__(kThreads) void k_encode_values(const EncodeParams p) {
    const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
    if (t >= p.n8) return;
    const float4* src = reinterpret_cast<const float4*>(p.v) + 2 * (int64_t)t;
    const float4 a = src[0], b = src[1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t r0 = 0, r1 = 0, gbits = 0;
    if (p.aux) {
        const uint2 x = reinterpret_cast<const uint2*>(p.aux)[t];
        r0 = x.x;
        r1 = x.y;
        // the LSB of each of the 8 aux bytes -> bits 0..7
        #pragma unroll
        for (int j = 0; j < 8; ++j) gbits |= (((j < 4 ? x.x : x.y) >> (8 * (j & 3))) & 1u) << j;
    }
    const uint32_t w = encode8<GRID, MODE>(v, r0, r1, gbits);
    const uint32_t lo = (w & 0xFu) | ((w >> 4) & 0xFu) << 8 | ((w >> 8) & 0xFu) << 16 | ((w >> 12) & 0xFu) << 24;
    const uint32_t hi = ((w >> 16) & 0xFu) | ((w >> 20) & 0xFu) << 8 | ((w >> 24) & 0xFu) << 16 | ((w >> 28) & 0xFu) << 24;
    reinterpret_cast<uint2*>(p.out)[t] = make_uint2(lo, hi);
}

// ---------------------------------------------------------------- block-scale encode
// The NVFP4 block-scale rounding on its own (exhaustive verification): the E4M3
// code of each t, four per lane.
__global__ __launch_bounds__(kThreads) void k_encode_scales(const float* t, uint8_t* out, uint32_t n4) {
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= n4) return;
    const float4 v = reinterpret_cast<const float4*>(t)[i];
    const uint32_t c = e4m3_encode_rne(clamp448(v.x)) | e4m3_encode_rne(clamp448(v.y)) << 8 |
                       e4m3_encode_rne(clamp448(v.z)) << 16 | e4m3_encode_rne(clamp448(v.w)) << 24;
    reinterpret_cast<uint32_t*>(out)[i] = c;
}

// ---------------------------------------------------------------- reference copy

__global__ __launch_bounds__(kThreads) void k_stream_copy(const v4u32* __restrict__ src,
                                                          v4u32* __restrict__ dst, uint64_t n16) {
    const uint64_t i = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n16) dst[i] = __builtin_nontemporal_load(src + i);
}

inline uint32_t blocks_for(uint32_t n) { return (n + kThreads - 1) / kThreads; }

}  // namespace

hipError_t launch_tensor_scale(int grid, bool rht, bool contig, const AmaxParams& p, hipStream_t s) {
    hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(1), 0, s, reinterpret_cast<uint32_t*>(p.acc), 0u);
    if (p.ngroups <= kAmaxBlocks * kThreads * kAmaxU) {   // fits one pass: the small-tensor shape
        const uint32_t blocks = (p.ngroups + kThreads * kAmaxUSmall - 1) / (kThreads * kAmaxUSmall);
        if (blocks > 0) launch_amax<kAmaxUSmall>(rht, contig, blocks, p, s);
    } else {
        launch_amax<kAmaxU>(rht, contig, kAmaxBlocks, p, s);
    }
    hipLaunchKernelGGL(k_ts_finalize, dim3(1), dim3(1), 0, s, p.acc, grid == 0 ? 2688.0f : 3136.0f);
    return hipGetLastError();
}

// One launch of at most kTsMaxWorkgroups workgroups of kAmaxU groups per lane
// (a 16 MiB tensor gets 512); an empty tensor still gets one workgroup, which
// writes s_t = 1.
hipError_t launch_tensor_scale_1(int grid, bool rht, bool contig, const AmaxParams& p, uint32_t* ws, hipStream_t s) {
    const float g448 = grid == 0 ? 2688.0f : 3136.0f;
    const uint32_t per_wg = kThreads * kAmaxU;
    uint32_t blocks = (p.ngroups + per_wg - 1) / per_wg;
    blocks = blocks < 1u ? 1u : (blocks > kTsMaxWorkgroups ? kTsMaxWorkgroups : blocks);
    const uint32_t polls = wait_limit();
#define FP4Q_TS1(R, C) \
    hipLaunchKernelGGL((k_tensor_scale_1<R, C>), dim3(blocks), dim3(kThreads), 0, s, p, ws, g448, polls)
    if (rht) { if (contig) FP4Q_TS1(true, true); else FP4Q_TS1(true, false); }
    else { if (contig) FP4Q_TS1(false, true); else FP4Q_TS1(false, false); }
#undef FP4Q_TS1
    return hipGetLastError();
}

namespace {
std::atomic<uint32_t> g_wait_limit{kGatherPolls};
}  // namespace

uint32_t wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }
uint32_t set_wait_limit(uint32_t polls) { return g_wait_limit.exchange(polls, std::memory_order_relaxed); }

// Workspace of fp4_tensor_scale_noalloc, for callers that cannot allocate: one
// array per device, zero when the code object is loaded and left zero by every
// completed call.  It holds the words the one-launch tensor scale uses (the
// epoch and kTsMaxWorkgroups gather words), not those only the fused quantize
// needs.  Host code reaches it
// only through the device address that hipGetSymbolAddress returns for the
// current device (the array's name is a host-side stand-in, not a device
// address).
static __device__ __align__(256) uint32_t scratch[kTsStaticWords];
static_assert(sizeof(scratch) == 16384, "the header states the static workspace size");

namespace {
std::mutex g_scratch_mu;
uint32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

uint32_t* static_ts_workspace(hipError_t* err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {   // set-up, once per device, with that device current
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
    }
    return g_scratch_ptr[dev];
}

hipError_t launch_dequantize(int format, int grid, bool bf16_out, const DequantParams& p, hipStream_t s) {
    const uint64_t units = (uint64_t)p.ngroups * (bf16_out ? 2u : 4u);
    const uint64_t b4 = (units + kThreads * kDqSlotsWide - 1) / (kThreads * kDqSlotsWide);
    const bool wide = bf16_out && b4 >= kDqWideBlocks;
    const dim3 b(wide ? (uint32_t)b4 : (uint32_t)((units + kThreads * kDqSlots - 1) / (kThreads * kDqSlots))),
        t(kThreads);
#define FP4Q_DQ(F, G, B)                                                                   \
    do {                                                                                   \
        if (wide) hipLaunchKernelGGL((k_dequantize<F, G, B, kDqSlotsWide>), b, t, 0, s, p); \
        else hipLaunchKernelGGL((k_dequantize<F, G, B, kDqSlots>), b, t, 0, s, p);          \
    } while (0)
    if (format == 0) {
        if (grid == 0) { if (bf16_out) FP4Q_DQ(0, 0, true); else FP4Q_DQ(0, 0, false); }
        else { if (bf16_out) FP4Q_DQ(0, 1, true); else FP4Q_DQ(0, 1, false); }
    } else {
        if (grid == 0) { if (bf16_out) FP4Q_DQ(1, 0, true); else FP4Q_DQ(1, 0, false); }
        else { if (bf16_out) FP4Q_DQ(1, 1, true); else FP4Q_DQ(1, 1, false); }
    }
#undef FP4Q_DQ
    return hipGetLastError();
}

hipError_t launch_guide_pack(int format, const GuideParams& p, hipStream_t s) {
    const uint32_t units = (p.ngroups + 1u) >> 1;
    const uint32_t b4 = (units + kThreads * kPackSlotsWide - 1) / (kThreads * kPackSlotsWide);
    const dim3 t(kThreads);
    if (b4 >= kPackWideBlocks) {
        if (format == 0) hipLaunchKernelGGL((k_guide_pack<0, kPackSlotsWide>), dim3(b4), t, 0, s, p);
        else hipLaunchKernelGGL((k_guide_pack<1, kPackSlotsWide>), dim3(b4), t, 0, s, p);
    } else {
        const dim3 b((units + kThreads * 2 - 1) / (kThreads * 2));
        if (format == 0) hipLaunchKernelGGL((k_guide_pack<0, 2>), b, t, 0, s, p);
        else hipLaunchKernelGGL((k_guide_pack<1, 2>), b, t, 0, s, p);
    }
    return hipGetLastError();
}

static uint32_t guide_pack_wgs(uint32_t ngroups) {
    const uint32_t units = (ngroups + 1u) >> 1;
    return (units + kThreads * kPackSlotsGrouped - 1) / (kThreads * kPackSlotsGrouped);
}

hipError_t launch_guide_pack_grouped(int format, GroupedGuideParams gp, hipStream_t s) {
    gp.wg_start[0] = 0;
    for (uint32_t t = 0; t < gp.n; ++t) gp.wg_start[t + 1] = gp.wg_start[t] + guide_pack_wgs(gp.t[t].ngroups);
    const dim3 b(gp.wg_start[gp.n]), th(kThreads);
    if (b.x == 0) return hipSuccess;
    if (format == 0) hipLaunchKernelGGL(k_guide_pack_grouped<0>, b, th, 0, s, gp);
    else hipLaunchKernelGGL(k_guide_pack_grouped<1>, b, th, 0, s, gp);
    return hipGetLastError();
}

hipError_t launch_guide_unpack(int format, const GuideParams& p, hipStream_t s) {
    const dim3 b((p.ngroups + kThreads * kGuideSlots - 1) / (kThreads * kGuideSlots)), t(kThreads);
    if (format == 0) hipLaunchKernelGGL(k_guide_unpack<0>, b, t, 0, s, p);
    else hipLaunchKernelGGL(k_guide_unpack<1>, b, t, 0, s, p);
    return hipGetLastError();
}

hipError_t launch_rht16(bool inverse, bool bf16_out, bool contig, const RhtParams& p, hipStream_t s) {
    const dim3 b(blocks_for(p.ngroups)), t(kThreads);
#define FP4Q_RH(I, B, C) hipLaunchKernelGGL((k_rht16<I, B, C>), b, t, 0, s, p)
    if (inverse) {
        if (bf16_out) { if (contig) FP4Q_RH(true, true, true); else FP4Q_RH(true, true, false); }
        else { if (contig) FP4Q_RH(true, false, true); else FP4Q_RH(true, false, false); }
    } else {
        if (bf16_out) { if (contig) FP4Q_RH(false, true, true); else FP4Q_RH(false, true, false); }
        else { if (contig) FP4Q_RH(false, false, true); else FP4Q_RH(false, false, false); }
    }
#undef FP4Q_RH
    return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, uint64_t n16, hipStream_t s) {
    const uint64_t blocks = (n16 + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(k_stream_copy, dim3((uint32_t)blocks), dim3(kThreads), 0, s,
                       static_cast<const v4u32*>(src), static_cast<v4u32*>(dst), n16);
    return hipGetLastError();
}

hipError_t launch_encode_scales(const float* t, uint8_t* out, uint32_t n4, hipStream_t s) {
    hipLaunchKernelGGL(k_encode_scales, dim3(blocks_for(n4)), dim3(kThreads), 0, s, t, out, n4);
    return hipGetLastError();
}

hipError_t launch_encode_values(int grid, int mode, const EncodeParams& p, hipStream_t s) {
    const dim3 b(blocks_for(p.n8)), t(kThreads);
#define FP4Q_EV(G, M) hipLaunchKernelGGL((k_encode_values<G, M>), b, t, 0, s, p)
    if (grid == 0) {
        if (mode == MODE_RTN) FP4Q_EV(0, MODE_RTN);
        else if (mode == MODE_SR) FP4Q_EV(0, MODE_SR);
        else FP4Q_EV(0, MODE_GUIDED);
    } else {
        if (mode == MODE_RTN) FP4Q_EV(1, MODE_RTN);
        else if (mode == MODE_SR) FP4Q_EV(1, MODE_SR);
        else FP4Q_EV(1, MODE_GUIDED);
    }
#undef FP4Q_EV
    return hipGetLastError();
}

}  // namespace fp4q
