// quantize.hip -- block-scaled FP4 quantization kernels for gfx950.
//
// Work mapping.  Loads: in each of its kH load slots a lane reads one
// half-group (8 elements, 16 bytes of bf16), and the 64 lanes of a wave read
// 64 consecutive half-groups, so every load instruction of a wave covers 1 KiB
// contiguously.  (A lane reading a whole 32-byte group needs two loads at a
// 32-byte stride that each touch half of every line: measured about 9% slower.)
// Compute: slots 2k and 2k+1 are then exchanged within each lane pair by DPP
// (4 moves and their selects), after which lane 2m owns group
// G + m and lane 2m+1 owns group G + 32 + m as whole 16-element groups, where
// G is the pair of slots' first group.  Each lane then works on whole groups:
// the NVFP4 block, the Philox block of stochastic rounding and the RHT all
// stay inside the lane, and an MXFP4 block is two lanes apart (quad_perm
// [2,3,0,1]; adjacent lanes after the LDS transpose of the RHT kernels).  Stores: codes are 8 bytes per lane and the guide bits 2 bytes,
// both covering contiguous runs per wave; the bf16 output of fake quantization
// is transposed back and stored per half-group like the loads.  Every lane
// runs every DPP step (only stores are predicated).  Kernels with the RHT are
// bound by arithmetic: they load the same way but transpose through LDS, so
// that lane l owns groups W + l and W + 64 + l of its wave's groups W ...
//
// Per block (scale) [FQT-FP4 §3; TETRAJET §3; TRACE-JA "TRACEの仕組み"]:
//   NVFP4 scale code = E4M3 RNE of amax / RN(Gmax*s_t) (clamped to 448),
//         inv = RN(1/RN(dec(code)*s_t));
//   MXFP4 scale code = max(E(amax) - 2, 0) (E the biased exponent field),
//         inv = 2^-(code-127);
//   guided: the code comes from the guide.
// Per element: v = RN(y*inv), then the grid rounding of device.h.
#include <mutex>

#include "device.h"
#include "internal.h"

namespace fp4q {

namespace {

// Half-groups per lane (load slots); even, since slots are transposed in pairs.
// MXFP4 stochastic rounding without the RHT runs fastest with two (twice the
// workgroups, so more of them in flight); every other kernel is built with four,
// and single-tensor launches take two where that measured faster (launch_t).
template <int FMT, int MODE, bool RHT>
constexpr int halves_per_lane() { return FMT == 1 && MODE == MODE_SR && !RHT ? 2 : 4; }
// Groups per workgroup.
template <int FMT, int MODE, bool RHT>
constexpr uint32_t chunk_groups() { return kThreads * (halves_per_lane<FMT, MODE, RHT>() / 2); }
// Single-tensor launches take two slots instead of four (twice the workgroups,
// so more loads in flight across the chip) for:
//  - RTN and guided rounding without the RHT (16384 x 4096 MXFP4 RTN 29.5
//    against 30.0 us, guided 31.0 against 31.6, NVFP4 RTN 29.7 against 30.1,
//    guided 32.2 against 32.5; on 4096 x 2048 NVFP4 RTN 5.35 against 5.78 us,
//    guided 5.82 against 6.56);
//  - RTN and guided rounding with the RHT, whose slots then go through the DPP
//    pair exchange instead of the LDS transpose (65536 x 8192: MXFP4 RTN 225.5
//    against 233 us, NVFP4 238 against 243.5, uniform 235.5 against 244.5);
//  - uniform SR without the RHT (65536 x 8192: 235 against 245.5 us);
//  - SR without the RHT when four slots would give fewer workgroups than this
//    (8 per compute unit).
// SR with the RHT is bound by VALU issue as much as by memory, and the pair
// exchange and the reciprocal table shared by half as many groups make it
// slower on two slots (C5, uniform + RHT + SR: 259-264 against 240-242 us); it
// takes eight on large tensors instead (below).  NVFP4 E2M1 SR on large tensors
// measured the same either way and the grouped launches are faster with four
// (C4's grouped rollout RTN: 36.3 against 38.1 us).
constexpr uint32_t kSmallLaunchBlocks = 2048;

// Number of nonzero nibbles of w.
__device__ __forceinline__ uint32_t nonzero_nibbles(uint32_t w) {
    return __builtin_popcount((w | (w >> 1) | (w >> 2) | (w >> 3)) & 0x11111111u);
}

// NVFP4: the reciprocals inv = RN(1/RN(dec(c)*s_t)) of all 128 scale magnitudes c
// for one tensor scale, written to LDS by the workgroup (one IEEE division per
// code instead of one per group).  Every thread of the workgroup must call it.
template <int FMT>
__device__ __forceinline__ void build_inv_table(float* tab, const float* ts) {
    if constexpr (FMT == 0) {
        if (threadIdx.x < 128u) tab[threadIdx.x] = nvfp4_inv(threadIdx.x, *ts);
        __syncthreads();
    }
}

// LDS for the RHT kernels' slot transpose: 4 KiB per wave, one array per kernel
// however many times quantize_chunk is instantiated in it.
__device__ __forceinline__ v4u32* rht_transpose_lds() {
    __shared__ v4u32 xt[kThreads / 64 * 256];
    return xt;
}

// One workgroup's share (kChunkGroups groups starting at chunk `wg`) of one tensor.
// OUT = 0 stores codes, scales (and emitted guide bits); OUT = 1 stores the
// dequantized bf16 values instead (fake quantization); OUT = 2 (guided only)
// takes the guide bits from the rollout's full codes and counts, instead of
// storing anything, how often the guided result differs from those codes.
// tab: LDS space for the NVFP4 reciprocal table, which the chunk builds once its
// loads are in flight (OUT = 2: the caller has built it).  PRE: the caller has
// loaded the lane's half-groups (the same ones, in slot order) into pre.
template <int FMT, int GRID, int MODE, bool RHT, bool EMIT, bool CONTIG, int OUT = 0,
          int KH = halves_per_lane<FMT, MODE, RHT>(), bool PRE = false>
__device__ __forceinline__ void quantize_chunk(const QuantParams& p, uint32_t wg, float* tab,
                                               uint32_t* acc = nullptr, const uint32_t (*pre)[4] = nullptr) {
    constexpr float kGmax = GRID == 0 ? 6.0f : 7.0f;
    constexpr int kH = KH;
    constexpr int kG = kH / 2;                                      // whole groups per lane
    constexpr uint32_t kChunkGroups = kThreads * kG;
    static_assert(kH >= 2 && kH % 2 == 0, "half-groups per lane must be even");
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t q = lane & 1u;
    // half-group of slot s: hg0 + 64 s; group owned after transposing slots 2k, 2k+1: gk(k)
    const uint32_t hg0 = wg * (2u * kChunkGroups) + (threadIdx.x >> 6) * (64u * kH) + lane;
    const uint32_t nhg = 2u * p.ngroups;
    // With the RHT on four or eight slots the slots go through LDS (see below)
    // and lane l then owns groups W + l + 64 k of its wave's groups W ..;
    // otherwise (no RHT, or two slots) the DPP pair exchange gives lane 2m groups
    // G + m and lane 2m+1 groups G + 32 + m for each pair of slots.
    constexpr bool kLdsT = RHT && kH % 4 == 0;
    auto gk = [&](int k) {
        return kLdsT ? ((hg0 - lane) >> 1) + 64u * k + lane : (hg0 + 128u * k + 64u * q) >> 1;
    };

    // Lanes past the end load the last half-group instead (in bounds, no
    // branch); their results are never stored.
    uint32_t w[kH][4];
    #pragma unroll
    for (int s = 0; s < kH; ++s) {
        if constexpr (PRE) {
            #pragma unroll
            for (int j = 0; j < 4; ++j) w[s][j] = pre[s][j];
        } else {
            const uint32_t hg = min(hg0 + 64u * s, nhg - 1u);
            load16_nt(p.x + half_offset<CONTIG>(hg, p.gpr, p.ld), w[s]);
        }
    }
    uint32_t gb[kG], gs[kG];
    v2u32 rc[kG];
    #pragma unroll
    for (int k = 0; k < kG; ++k) {
        gb[k] = gs[k] = 0u;
        rc[k] = (v2u32){0u, 0u};
        if constexpr (MODE == MODE_GUIDED) {
            const uint32_t g = min(gk(k), p.ngroups - 1u);
            if constexpr (OUT == 2) {
                rc[k] = reinterpret_cast<const v2u32*>(p.rcodes)[g];
                gb[k] = gather_nibble_lsbs(rc[k].x) | (gather_nibble_lsbs(rc[k].y) << 8);
            } else {
                gb[k] = reinterpret_cast<const uint16_t*>(p.gbits)[g];
            }
            gs[k] = p.gscales[FMT == 0 ? g : (g >> 1)];
        }
    }
    // Every load of the chunk is issued before any of its data is used: left to
    // itself the compiler issues the second group's guide loads after the wait
    // for the first x loads, and their whole latency then ends the wave's life
    // (C2 guided quantize, guides from HBM: 32.6 against 30.2 us without them).
    if constexpr (MODE == MODE_GUIDED) __builtin_amdgcn_sched_barrier(0);
    uint32_t n_skip = 0, n_nonadj = 0, n_mism = 0;   // OUT == 2
    const bool nt = p.stream_out != 0;               // uniform: a scalar branch per store

    const uint32_t signs = RHT ? rht_sign_mask(p.rht_seed) : 0u;   // uniform: scalar unit
    float ts = 1.0f, denom = 1.0f, rden = 0.0f;
    bool rden_ok = false;
    if constexpr (FMT == 0) {
        if constexpr (OUT != 2) build_inv_table<FMT>(tab, p.ts);
        ts = *p.ts;
        denom = kGmax * ts;
        // t = RN(amax / denom) is first taken as RN(amax * RN(1/denom)), which is
        // within 3 fp32 steps of it whenever 1/denom is a normal number
        rden = 1.0f / denom;
        rden_ok = denom >= 0x1p-125f && denom <= 0x1p125f;
    }
    if constexpr (kLdsT) {
        // The RHT kernels on four or eight slots (SR, and the grouped, fused,
        // fake and diagnostic launches) are bound by arithmetic: the slots go
        // through LDS, which costs no VALU instructions, instead of the DPP
        // exchange, four at a time.  In round r, half-group h of the wave's
        // slots 4 r .. 4 r + 3 goes to (h & 1) * 2048 + (h >> 1) * 16, so lane l
        // then reads groups l and 64 + l of the round as two 16-byte pieces
        // each; the writes and the reads both touch consecutive 16-byte slots.
        // The wave's own LDS operations complete in order, so it needs no
        // workgroup barrier.
        static_assert(kH % 4 == 0, "the LDS transpose takes rounds of four slots");
        char* base = reinterpret_cast<char*>(rht_transpose_lds() + (threadIdx.x >> 6) * 256);
        char* wp = base + (lane & 1u) * 2048u + (lane >> 1) * 16u;
        char* rp = base + lane * 16u;
        #pragma unroll
        for (int r = 0; r < kH / 4; ++r) {
            // the previous round's reads (and, in the diagnostic kernel, which calls
            // this once per chunk, the previous chunk's) come before these writes
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            #pragma unroll
            for (int s = 0; s < 4; ++s)
                *reinterpret_cast<v4u32*>(wp + 512 * s) =
                    (v4u32){w[4 * r + s][0], w[4 * r + s][1], w[4 * r + s][2], w[4 * r + s][3]};
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            #pragma unroll
            for (int k = 0; k < 2; ++k) {
                const v4u32 a = *reinterpret_cast<const v4u32*>(rp + 1024 * k);
                const v4u32 b = *reinterpret_cast<const v4u32*>(rp + 2048 + 1024 * k);
                const int s0 = 4 * r + 2 * k;   // group 2 r + k of the lane
                w[s0][0] = a.x; w[s0][1] = a.y; w[s0][2] = a.z; w[s0][3] = a.w;
                w[s0 + 1][0] = b.x; w[s0 + 1][1] = b.y; w[s0 + 1][2] = b.z; w[s0 + 1][3] = b.w;
            }
        }
    }
    // MXFP4 RTN and guided without the RHT convert straight from the bf16 bits;
    // every other path widens the values, and then takes the amax in fp32
    constexpr bool kWidened = RHT || FMT == 0 || GRID == 1 || MODE == MODE_SR;

    #pragma unroll
    for (int k = 0; k < kG; ++k) {
        const uint32_t g = gk(k);
        uint32_t gw[8];
        if constexpr (kLdsT) {
            #pragma unroll
            for (int j = 0; j < 4; ++j) { gw[j] = w[2 * k][j]; gw[4 + j] = w[2 * k + 1][j]; }
        } else {
            pair_exchange(w[2 * k], w[2 * k + 1], q, gw, gw + 4);   // -> this lane's whole group
        }

        // With the RHT, y holds the transform before its exact factor 1/4
        // (a = 4 y); the 1/4 is applied to the block amax and folded into inv.
        float y[16];
        widen16<RHT, false>(gw, signs, y);

        // block amax key: monotone in the amax (bf16 bits, or fp32 bits with the
        // RHT); NaN and Inf give keys >= 0x7F800000
        uint32_t amax_key;
        if constexpr (kWidened) {
            // NaN-propagating maximum of the magnitudes: equal to the widened
            // bf16 maximum when all are finite
            float m = 0.0f;
            #pragma unroll
            for (int j = 0; j < 16; ++j) m = __builtin_elementwise_maximum(m, fabsf(y[j]));
            amax_key = __float_as_uint(RHT ? m * 0.25f : m);
        } else {
            amax_key = amax_bits16(gw) << 16;
        }
        // an MXFP4 block is groups 2b and 2b+1: in lanes l and l ^ 1 after the LDS
        // transpose, in lanes l and l ^ 2 after the pair exchange
        if constexpr (FMT == 1) amax_key = max(amax_key, kLdsT ? dpp_swap1(amax_key) : dpp_swap2(amax_key));
        bool finite = amax_key < 0x7F800000u;

        uint32_t sc;
        float inv;
        if constexpr (MODE == MODE_GUIDED) {
            sc = gs[k];
            if constexpr (FMT == 0) {
                finite = finite && ((sc & 0x7Fu) != 0x7Fu);
                inv = tab[sc & 0x7Fu];
            } else {
                finite = finite && (sc != 0xFFu);
                inv = mx_inv(sc);
            }
        } else if constexpr (FMT == 0) {
            // The E4M3 code of t changes only at the midpoints between E4M3
            // values: fp32 patterns whose low 20 bits are 0x80000 (2^-6 and
            // above; every E4M3 step there is 2^20 patterns).  Where the product
            // is 4 or more steps from a midpoint and at or above 2^-6 + 4 steps
            // (or 0), the exact quotient lies on the same side, so both give the
            // same code; elsewhere the quotient is computed.
            float t = __uint_as_float(amax_key) * rden;
            const uint32_t tb = __float_as_uint(t);
            const bool exact = !rden_ok || tb - 1u < 0x3C800003u || (tb & 0xFFFFFu) - 0x7FFFCu <= 8u;
            if (__builtin_expect(exact, 0)) t = __uint_as_float(amax_key) / denom;
            sc = e4m3_encode_rne(clamp448(t));   // t >= 0; NaN only for a non-finite block
            inv = tab[sc];
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

        // MXFP4 without the RHT: v = bf16 * 2^-e exactly, at most 8 significant
        // bits.  Its E2M1 converts take the inputs and divide by 2^e themselves.
        constexpr bool kShort = FMT == 1 && !RHT;
        constexpr bool kInCvt = kShort && GRID == 0;
        // E2M1 SR of values with up to 24 significant bits takes w = 2^23 v,
        // uniform SR takes w = 256 v
        constexpr bool kSrW = GRID == 0 && MODE == MODE_SR && !kShort;
        constexpr bool kUniSr = GRID == 1 && MODE == MODE_SR;
        float v[16];
        float cscale = 1.0f;
        if constexpr (kInCvt) {
            cscale = mx_scale(sc);
            #pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = y[j];
        } else if constexpr (kSrW) {
            // RN(y * inv * 2^23), or RN(a * inv * 2^21) with the RHT, equals 2^23 v
            // wherever v is normal (smaller v round to 0 with their sign either
            // way); one product where inv times the power of two is exact and finite
            if (inv < 0x1p100f) {
                const float m = inv * (RHT ? 0x1p21f : 0x1p23f);
                #pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = y[j] * m;
            } else {
                const float m = RHT ? inv * 0.25f : inv;   // exact: inv >= 2^100
                #pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = (y[j] * m) * 0x1p23f;
            }
        } else if constexpr (kUniSr) {
            // RN(y * inv * 256), or RN(a * inv * 64) with the RHT, equals 256 v
            // wherever v is normal (smaller v give k = 0 and keep their sign either
            // way); one product where inv times the power of two is exact and
            // finite (for NVFP4 with the RHT also inv >= 2^-124, as below)
            if (inv < 0x1p120f && (FMT == 1 || !RHT || inv >= 0x1p-124f)) {
                const float m = inv * (RHT ? 64.0f : 256.0f);
                #pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = y[j] * m;
            } else {
                #pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = (RHT ? (y[j] * 0.25f) * inv : y[j] * inv) * 256.0f;
            }
        } else if constexpr (RHT) {
            // v = RN((a/4) * inv) = RN(a * (inv/4)) when inv/4 is exact: always
            // for MXFP4 (a power of two >= 2^-129), and for NVFP4 unless inv < 2^-124
            const float inv4 = inv * 0.25f;
            if (FMT == 1 || inv >= 0x1p-124f) {
                #pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = y[j] * inv4;
            } else {
                #pragma unroll
                for (int j = 0; j < 16; ++j) v[j] = (y[j] * 0.25f) * inv;
            }
        } else {
            #pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = y[j] * inv;
        }
        uint32_t c0, c1;
        if constexpr (kInCvt && MODE == MODE_RTN) {   // straight from the bf16 bits
            c0 = pack_rne8_bf16(gw, cscale);
            c1 = pack_rne8_bf16(gw + 4, cscale);
        } else if constexpr (kInCvt && MODE == MODE_GUIDED) {
            c0 = encode8_guided_e2m1_bf16(gw, gb[k] & 0xFFu, cscale);
            c1 = encode8_guided_e2m1_bf16(gw + 4, gb[k] >> 8, cscale);
        } else if constexpr (kSrW) {
            c0 = encode8_sr_e2m1_w(v, r0, r1);
            c1 = encode8_sr_e2m1_w(v + 8, r2, r3);
        } else if constexpr (kUniSr) {
            c0 = encode8_sr_uniform_w(v, r0, r1);
            c1 = encode8_sr_uniform_w(v + 8, r2, r3);
        } else {
            c0 = encode8<GRID, MODE, kShort>(v, r0, r1, gb[k] & 0xFFu, cscale);
            c1 = encode8<GRID, MODE, kShort>(v + 8, r2, r3, gb[k] >> 8, cscale);
        }
        if (!finite) { c0 = 0; c1 = 0; }

        if constexpr (OUT == 2) {
            if (g < p.ngroups) {
                if (finite) {   // blocks guided rounding encodes
                    const uint32_t d0 = c0 ^ rc[k].x, d1 = c1 ^ rc[k].y;
                    n_nonadj += nonzero_nibbles(d0 & 0x77777777u) + nonzero_nibbles(d1 & 0x77777777u);
                    n_mism += nonzero_nibbles(d0) + nonzero_nibbles(d1);
                } else {
                    n_skip += 16u;
                }
            }
        } else if constexpr (OUT == 1) {
            float dv[16];
            const bool ok = dequant16<FMT, GRID>(c0, c1, sc, ts, dv);
            uint32_t o[8];
            to_bf16x16(dv, ok, o);
            if constexpr (RHT) {   // this lane's own group, as loaded
                if (g < p.ngroups) {
                    st_out4(p.fq_out + half_offset<false>(2u * g, p.gpr, p.ld_out), 0, o[0], o[1], o[2], o[3], nt);
                    st_out4(p.fq_out + half_offset<false>(2u * g + 1u, p.gpr, p.ld_out), 0, o[4], o[5], o[6], o[7],
                            nt);
                }
            } else {
                // back to half-groups (the same exchange, inverted): slot 2k takes this
                // lane's first half (q = 0) or the partner's second half (q = 1), slot
                // 2k+1 the partner's first half (q = 0) or this lane's second half
                uint32_t oa[4], ob[4];
                pair_exchange(o, o + 4, q, oa, ob);
                const uint32_t ha = hg0 + 128u * k, hb = ha + 64u;
                if (ha < nhg)
                    st_out4(p.fq_out + half_offset<false>(ha, p.gpr, p.ld_out), 0, oa[0], oa[1], oa[2], oa[3], nt);
                if (hb < nhg)
                    st_out4(p.fq_out + half_offset<false>(hb, p.gpr, p.ld_out), 0, ob[0], ob[1], ob[2], ob[3], nt);
            }
        } else if (g < p.ngroups) {
            st_out2(p.codes, g, c0, c1, nt);
            if constexpr (FMT == 0) {
                st_out(p.scales + g, (uint8_t)sc, nt);
            } else {
                if ((g & 1u) == 0) st_out(p.scales + (g >> 1), (uint8_t)sc, nt);
            }
            if constexpr (EMIT) {
                st_out(reinterpret_cast<uint16_t*>(p.bits_out) + g,
                       (uint16_t)(gather_nibble_lsbs(c0) | (gather_nibble_lsbs(c1) << 8)), nt);
            }
        }
    }

    if constexpr (OUT == 2) {
        acc[0] += n_skip;
        acc[1] += n_nonadj;
        acc[2] += n_mism;
    }
}

template <int FMT, int GRID, int MODE, bool RHT, bool EMIT, bool CONTIG, int KH>
__global__ __launch_bounds__(kThreads) void k_quantize(const QuantParams p) {
    __shared__ float tab[128];
    quantize_chunk<FMT, GRID, MODE, RHT, EMIT, CONTIG, 0, KH>(p, blockIdx.x, tab);
}

// Several tensors with one configuration in one launch: workgroup b belongs to
// the tensor t with wg_start[t] <= b < wg_start[t+1] (group_of), and processes
// that tensor's chunk b - wg_start[t].
template <int FMT, int GRID, int MODE, bool RHT, bool EMIT>
__global__ __launch_bounds__(kThreads) void k_quantize_grouped(const GroupedQuantParams gp) {
    const uint32_t b = blockIdx.x;
    const uint32_t t = group_of<kMaxGroup>(gp.wg_start, gp.n, b);
    const uint32_t wg = b - gp.wg_start[t];
    __shared__ float tab[128];
    if ((gp.contig_mask >> t) & 1u)
        quantize_chunk<FMT, GRID, MODE, RHT, EMIT, true>(gp.t[t], wg, tab);
    else
        quantize_chunk<FMT, GRID, MODE, RHT, EMIT, false>(gp.t[t], wg, tab);
}

template <int FMT, int GRID, int MODE, bool RHT, bool EMIT>
hipError_t launch_grouped_t(const GroupedQuantParams& gp, hipStream_t s) {
    const uint32_t blocks = gp.wg_start[gp.n];
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((k_quantize_grouped<FMT, GRID, MODE, RHT, EMIT>), dim3(blocks), dim3(kThreads), 0, s, gp);
    return hipGetLastError();
}

// At most kMismatchBlocks workgroups, each looping over chunks with its counts
// in registers, then at most one atomic per counter and workgroup: thousands
// of same-address atomics (one per chunk) would serialize and dominate.  The
// element count starts at the whole tensor and workgroups subtract the
// elements of blocks guided rounding does not encode, so, like the other two
// counts, it takes an atomic only where something is counted.
constexpr uint32_t kMismatchBlocks = 1024;

template <int FMT, int GRID, bool RHT, bool CONTIG>
__global__ __launch_bounds__(kThreads) void k_guide_mismatch(const QuantParams p, uint32_t nchunks) {
    uint32_t acc[3] = {0u, 0u, 0u};
    __shared__ float tab[128];
    build_inv_table<FMT>(tab, p.ts);
    for (uint32_t wg = blockIdx.x; wg < nchunks; wg += gridDim.x)   // the same trip count in a workgroup
        quantize_chunk<FMT, GRID, MODE_GUIDED, RHT, false, CONTIG, 2>(p, wg, tab, acc);
    __shared__ uint32_t red[3][kThreads / 64];
    #pragma unroll
    for (int c = 0; c < 3; ++c) {
        #pragma unroll
        for (int o = 32; o >= 1; o >>= 1) acc[c] += (uint32_t)__shfl_xor((int)acc[c], o);
    }
    if ((threadIdx.x & 63u) == 0) {
        #pragma unroll
        for (int c = 0; c < 3; ++c) red[c][threadIdx.x >> 6] = acc[c];
    }
    __syncthreads();
    if (threadIdx.x < 3) {
        unsigned long long t = 0;
        #pragma unroll
        for (int wv = 0; wv < kThreads / 64; ++wv) t += red[threadIdx.x][wv];
        if (t) atomicAdd(p.counts + threadIdx.x, threadIdx.x == 0 ? 0ull - t : t);   // count 0: subtract
    }
}

// Sets the three diagnostic counters to (all elements, 0, 0) (vector stores, one lane each).
__global__ void k_zero_counts(unsigned long long* c, unsigned long long elements) {
    if (threadIdx.x < 3) c[threadIdx.x] = threadIdx.x == 0 ? elements : 0ull;
}

template <int FMT, int GRID>
hipError_t launch_mismatch_g(bool rht, bool contig, const QuantParams& p, hipStream_t s) {
    const uint32_t cg = rht ? chunk_groups<FMT, MODE_GUIDED, true>() : chunk_groups<FMT, MODE_GUIDED, false>();
    const uint32_t chunks = (p.ngroups + cg - 1) / cg;
    const dim3 b(chunks < kMismatchBlocks ? chunks : kMismatchBlocks), t(kThreads);
    if (rht) {
        if (contig) hipLaunchKernelGGL((k_guide_mismatch<FMT, GRID, true, true>), b, t, 0, s, p, chunks);
        else hipLaunchKernelGGL((k_guide_mismatch<FMT, GRID, true, false>), b, t, 0, s, p, chunks);
    } else {
        if (contig) hipLaunchKernelGGL((k_guide_mismatch<FMT, GRID, false, true>), b, t, 0, s, p, chunks);
        else hipLaunchKernelGGL((k_guide_mismatch<FMT, GRID, false, false>), b, t, 0, s, p, chunks);
    }
    return hipGetLastError();
}

// Fake quantization takes two slots for RTN and guided rounding without the RHT,
// as the single-tensor quantize does (16384 x 4096 MXFP4 guided, bf16 out: 44.3
// against 46.9 us on four, 50.2 on eight); the others keep the quantizer's count.
template <int FMT, int MODE, bool RHT>
constexpr int fake_halves() { return !RHT && MODE != MODE_SR ? 2 : halves_per_lane<FMT, MODE, RHT>(); }

template <int FMT, int GRID, int MODE, bool RHT, bool CONTIG>
__global__ __launch_bounds__(kThreads) void k_fake_quantize(const QuantParams p) {
    __shared__ float tab[128];
    quantize_chunk<FMT, GRID, MODE, RHT, false, CONTIG, 1, fake_halves<FMT, MODE, RHT>()>(p, blockIdx.x, tab);
}

template <int FMT, int GRID, int MODE>
hipError_t launch_fake_m(bool rht, bool contig, const QuantParams& p, hipStream_t s) {
    const dim3 t(kThreads);
    if (rht) {
        const dim3 b((p.ngroups + chunk_groups<FMT, MODE, true>() - 1) / chunk_groups<FMT, MODE, true>());
        if (contig) hipLaunchKernelGGL((k_fake_quantize<FMT, GRID, MODE, true, true>), b, t, 0, s, p);
        else hipLaunchKernelGGL((k_fake_quantize<FMT, GRID, MODE, true, false>), b, t, 0, s, p);
    } else {
        constexpr uint32_t cg = kThreads * (fake_halves<FMT, MODE, false>() / 2);
        const dim3 b((p.ngroups + cg - 1) / cg);
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
    constexpr int kH = halves_per_lane<FMT, MODE, RHT>();
    constexpr uint32_t kChunkGroups = chunk_groups<FMT, MODE, RHT>();
    const uint32_t blocks = (p.ngroups + kChunkGroups - 1) / kChunkGroups;
    if constexpr (RHT && MODE == MODE_SR) {
        // eight slots: four groups per lane share the wave's fixed work (load
        // addresses, the reciprocal table), where that still gives this many
        // workgroups (C5: 237.0 against 240.5 us)
        const uint32_t b8 = (p.ngroups + 4 * kThreads - 1) / (4 * kThreads);
        if (b8 >= kSmallLaunchBlocks) {
            hipLaunchKernelGGL((k_quantize<FMT, GRID, MODE, RHT, EMIT, CONTIG, 8>), dim3(b8), dim3(kThreads), 0, s,
                               p);
            return hipGetLastError();
        }
    }
    if constexpr (kH == 4) {
        const bool two = MODE != MODE_SR || (!RHT && (GRID == 1 || blocks < kSmallLaunchBlocks));
        if (two) {
            const uint32_t b2 = (p.ngroups + kThreads - 1) / kThreads;
            hipLaunchKernelGGL((k_quantize<FMT, GRID, MODE, RHT, EMIT, CONTIG, 2>), dim3(b2), dim3(kThreads),
                               0, s, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_quantize<FMT, GRID, MODE, RHT, EMIT, CONTIG, kH>), dim3(blocks), dim3(kThreads),
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


// ---------------------------------------------------------------- tensor scale and quantize in one launch
// NVFP4 (either grid), RTN or SR, no RHT.  Each workgroup loads exactly the
// chunk it will quantize, keeps it in registers, and stores the chunk's largest
// finite |x|, tagged with this call's epoch, in a workspace word of its own;
// workgroup 0 gathers those words as the one-launch tensor scale does and
// publishes s_t in tagged words (copies on several lines, so that the waiting
// workgroups' loads spread), which the others wait for; then each quantizes its
// chunk from its registers.  This needs every workgroup resident at once: the
// host launches it only when the device holds the whole grid, and each wait is
// bounded (wait_limit() polls, by default about a second) so that a workgroup kept from
// seeing s_t gives up with a NaN scale instead of spinning forever.
template <int GRID, int MODE, bool EMIT, bool CONTIG>
__global__ __launch_bounds__(kThreads) void k_quantize_with_scale(const QuantParams p, float* ts_out, uint32_t* ws,
                                                                  float gmax448, uint32_t polls) {
    constexpr int kH = 4;
    constexpr uint32_t kChunkGroups = kThreads * (kH / 2);
    __shared__ float tab[128];
    __shared__ uint32_t red[kThreads / 64];
    __shared__ CallState cs_sh;
    __shared__ float ts_sh;
    const uint32_t b = blockIdx.x, nwg = gridDim.x;
    const uint32_t lane = threadIdx.x & 63u;
    // the workspace's state word, read while the chunk loads (any time before
    // this workgroup's own word is stored will do)
    const CallState cs = threadIdx.x == 0 ? call_state(ws + kTsEpoch) : CallState{};
    // the half-groups quantize_chunk would read for chunk b (past the end, the
    // last one again), kept in registers for it
    const uint32_t hg0 = b * (2u * kChunkGroups) + (threadIdx.x >> 6) * (64u * kH) + lane;
    const uint32_t nhg = 2u * p.ngroups;
    uint32_t w[kH][4];
    #pragma unroll
    for (int s = 0; s < kH; ++s) {
        const uint32_t hg = min(hg0 + 64u * s, nhg - 1u);
        load16_nt(p.x + half_offset<CONTIG>(hg, p.gpr, p.ld), w[s]);
    }
    uint32_t m = 0;
    #pragma unroll
    for (int s = 0; s < kH; ++s) {
        #pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t lo = w[s][j] & 0x7FFFu, hi = (w[s][j] >> 16) & 0x7FFFu;
            m = lo < 0x7F80u ? max(m, lo << 16) : m;
            m = hi < 0x7F80u ? max(m, hi << 16) : m;
        }
    }
    m = wg_max_t0<kThreads / 64>(m, red);
    uint64_t* const words = reinterpret_cast<uint64_t*>(ws + kTsGather);
    if (threadIdx.x == 0) {
        if (!cs.late) store_agent(words + b, tagged(cs.tag, m));
        cs_sh = cs;
    }
    if (b == 0) {
        __syncthreads();   // cs_sh; also orders the first use of red before the second
        const CallState c = cs_sh;
        if (c.late) {      // this launch gave up before: s_t is NaN, the state stays
            if (threadIdx.x == 0) *ts_out = ts_sh = __builtin_nanf("");
        } else {
            const uint32_t g =
                wg_max_t0<kThreads / 64>(gather_max<kTsGatherMax, kThreads>(words, nwg, c.tag, polls), red);
            if (threadIdx.x == 0) {
                const float ts = g == 0xFFFFFFFFu ? __builtin_nanf("") : ts_from_amax(g, gmax448);
                *ts_out = ts;
                #pragma unroll
                for (uint32_t k = 0; k < kTsPubCopies; ++k)
                    store_agent(reinterpret_cast<uint64_t*>(ws + kTsPub + kTsLine * k),
                                tagged(c.tag, __float_as_uint(ts)));
                end_call(ws + kTsEpoch, c.epoch, g == 0xFFFFFFFFu);
                ts_sh = ts;
            }
        }
    } else if (threadIdx.x == 0) {
        const uint64_t* pub = reinterpret_cast<const uint64_t*>(ws + kTsPub + kTsLine * (b % kTsPubCopies));
        uint64_t v = 0;
        for (uint32_t n = 0; !cs.late && n < polls; ++n) {
            v = load_agent(pub);
            if ((uint32_t)(v >> 32) == cs.tag) break;
            __builtin_amdgcn_s_sleep(4);
        }
        ts_sh = !cs.late && (uint32_t)(v >> 32) == cs.tag ? __uint_as_float((uint32_t)v) : __builtin_nanf("");
    }
    __syncthreads();
    QuantParams q = p;
    q.ts = &ts_sh;
    quantize_chunk<0, GRID, MODE, false, EMIT, CONTIG, 0, kH, true>(q, b, tab, nullptr, w);
}

template <int GRID, int MODE, bool EMIT, bool CONTIG>
hipError_t launch_with_scale_t(const QuantParams& p, float* ts_out, uint32_t* ws, bool* fused, hipStream_t s) {
    constexpr uint32_t kChunkGroups = kThreads * 2;
    const uint32_t blocks = (p.ngroups + kChunkGroups - 1) / kChunkGroups;
    // workgroups the device holds at once, per device (the same on every call)
    static std::mutex mu;
    static int resident[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cap = 0;
    if (dev >= 0 && dev < kMaxDevices) {
        std::lock_guard<std::mutex> lock(mu);
        if (resident[dev] == 0) {
            int per_cu = 0, cus = 0;
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(&k_quantize_with_scale<GRID, MODE, EMIT, CONTIG>), kThreads, 0);
            if (e != hipSuccess) return e;
            e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
            if (e != hipSuccess) return e;
            resident[dev] = per_cu * cus > 0 ? per_cu * cus : -1;
        }
        cap = resident[dev];
    }
    const float g448 = GRID == 0 ? 2688.0f : 3136.0f;
    if (blocks > 0 && (int64_t)blocks <= cap && blocks <= kTsGatherMax) {
        *fused = true;
        hipLaunchKernelGGL((k_quantize_with_scale<GRID, MODE, EMIT, CONTIG>), dim3(blocks), dim3(kThreads), 0, s, p,
                           ts_out, ws, g448, wait_limit());
        return hipGetLastError();
    }
    *fused = false;
    return hipErrorNotSupported;   // the caller takes the two-launch path
}

template <int GRID, int MODE, bool EMIT>
hipError_t launch_with_scale_c(bool contig, const QuantParams& p, float* ts_out, uint32_t* ws, bool* fused,
                               hipStream_t s) {
    return contig ? launch_with_scale_t<GRID, MODE, EMIT, true>(p, ts_out, ws, fused, s)
                  : launch_with_scale_t<GRID, MODE, EMIT, false>(p, ts_out, ws, fused, s);
}

template <int GRID, int MODE>
hipError_t launch_with_scale_e(bool emit, bool contig, const QuantParams& p, float* ts_out, uint32_t* ws,
                               bool* fused, hipStream_t s) {
    return emit ? launch_with_scale_c<GRID, MODE, true>(contig, p, ts_out, ws, fused, s)
                : launch_with_scale_c<GRID, MODE, false>(contig, p, ts_out, ws, fused, s);
}

template <int GRID>
hipError_t launch_with_scale_m(int mode, bool emit, bool contig, const QuantParams& p, float* ts_out, uint32_t* ws,
                               bool* fused, hipStream_t s) {
    return mode == MODE_SR ? launch_with_scale_e<GRID, MODE_SR>(emit, contig, p, ts_out, ws, fused, s)
                           : launch_with_scale_e<GRID, MODE_RTN>(emit, contig, p, ts_out, ws, fused, s);
}

}  // namespace

uint32_t quantize_chunks(int format, int mode, bool rht, uint32_t ngroups) {
    const uint32_t c = format == 1 && mode == MODE_SR && !rht ? chunk_groups<1, MODE_SR, false>()
                                                              : chunk_groups<0, MODE_RTN, false>();
    return (ngroups + c - 1) / c;
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

hipError_t launch_guide_mismatch(int format, int grid, bool rht, bool contig, const QuantParams& p, hipStream_t s) {
    hipLaunchKernelGGL(k_zero_counts, dim3(1), dim3(64), 0, s, p.counts, 16ull * p.ngroups);
    if (p.ngroups == 0) return hipGetLastError();
    if (format == 0) {
        return grid == 0 ? launch_mismatch_g<0, 0>(rht, contig, p, s) : launch_mismatch_g<0, 1>(rht, contig, p, s);
    }
    return grid == 0 ? launch_mismatch_g<1, 0>(rht, contig, p, s) : launch_mismatch_g<1, 1>(rht, contig, p, s);
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

hipError_t launch_quantize_with_scale(int grid, int mode, bool rht, bool emit, bool contig, const QuantParams& p,
                                      float* ts_out, uint32_t* ws, bool* fused, hipStream_t s) {
    *fused = false;
    if (p.ngroups > 0 && !rht) {
        const hipError_t e = grid == 0 ? launch_with_scale_m<0>(mode, emit, contig, p, ts_out, ws, fused, s)
                                       : launch_with_scale_m<1>(mode, emit, contig, p, ts_out, ws, fused, s);
        if (*fused || e != hipErrorNotSupported) return e;
    }
    // with the RHT, too large to hold at once, or empty: the one-launch tensor scale, then quantize
    AmaxParams a{};
    a.x = p.x;
    a.ld = p.ld;
    a.ngroups = p.ngroups;
    a.gpr = p.gpr;
    a.rht_seed = p.rht_seed;
    a.acc = ts_out;
    hipError_t e = launch_tensor_scale_1(grid, rht, contig, a, ws, s);
    if (e != hipSuccess || p.ngroups == 0) return e;
    QuantParams q = p;
    q.ts = ts_out;
    return launch_quantize(0, grid, mode, rht, emit, contig, q, s);
}

}  // namespace fp4q
