// gemm.hip -- MXFP4 matrix product on the gfx950 scaled matrix cores.
//
// C[M, N] = A[M, K] * B[N, K]^T with A and B in MXFP4 exactly as the quantizer
// writes them for row-major [M, K] and [N, K] tensors: E2M1 codes two per byte
// along K and one E8M0 scale per 32-element block along K.  This is the
// contraction the FP4 operands of a linear layer feed [TETRAJET section 3:
// per-group scales; section 4: every linear layer's weights, activations and
// gradients in MXFP4].
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in E2M1 (format code 4)
// reads, in lane l, row (l mod 32) and K block (l / 32) of the 64-wide K slice:
// 32 values, which are 16 bytes of our codes in our nibble order, plus that
// block's E8M0 scale in byte 0 of the lane's scale operand.  Result element j
// of lane l is C[8 (j / 4) + 4 (l / 32) + j % 4][l mod 32].  (Layout checked
// on the GPU against a host product of random codes and scales.)
//
// Tiling: a workgroup of 4 waves computes a 128 x 128 tile of C, each wave a
// 64 x 64 quarter as 2 x 2 MFMA tiles.  K advances 128 values (4 scale blocks)
// per stage: the A and B tiles (128 rows x 64 bytes each) are staged in LDS
// with an 80-byte row pitch -- the 16 bytes of padding put the 16-byte
// operand reads of 8 consecutive rows on distinct banks -- and each row's
// four scale bytes in one dword.  The next stage is loaded into registers
// while the MFMAs run and written to the other LDS buffer afterwards, so one
// barrier per stage suffices.  Rows past M or N are clamped on load (their
// results are not stored); K blocks past K load as zero codes.
#include "device.h"
#include "internal.h"

namespace fp4q {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kTile = 128;   // rows of A and of B per workgroup tile
constexpr int kPitch = 80;   // LDS bytes per staged row of 64 code bytes

// Per-thread view of one stage: two 16-byte pieces of A and two of B (piece c
// = thread + 256 h covers row c / 4, scale block c % 4 of the stage) and one
// row's four scale bytes (threads 0..127: A rows, 128..255: B rows).
struct Stage {
    v4u32 a[2], b[2];
    uint32_t s;
};

struct Rows {
    const uint8_t* a[2];
    const uint8_t* b[2];
    const uint8_t* s;
};

template <bool SCALE4>
__device__ __forceinline__ void load_stage(const Rows& r, int64_t step, int valid, Stage& st) {
    const int part = threadIdx.x & 3;
    const int64_t off = step * 64;
    if (part < valid) {
        #pragma unroll
        for (int h = 0; h < 2; ++h) {
            st.a[h] = *reinterpret_cast<const v4u32*>(r.a[h] + off);
            st.b[h] = *reinterpret_cast<const v4u32*>(r.b[h] + off);
        }
    } else {
        #pragma unroll
        for (int h = 0; h < 2; ++h) st.a[h] = st.b[h] = (v4u32){0u, 0u, 0u, 0u};
    }
    const uint8_t* sp = r.s + step * 4;
    if (SCALE4 && valid == 4) {
        st.s = *reinterpret_cast<const uint32_t*>(sp);
    } else {
        uint32_t s = 0;
        #pragma unroll
        for (int j = 0; j < 4; ++j) s |= (j < valid ? (uint32_t)sp[j] : 127u) << (8 * j);
        st.s = s;
    }
}

__device__ __forceinline__ void store_stage(const Stage& st, uint8_t* sA, uint8_t* sB, uint32_t* sS) {
    const int t = threadIdx.x;
    #pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = t + 256 * h;
        const int o = (c >> 2) * kPitch + (c & 3) * 16;
        *reinterpret_cast<v4u32*>(sA + o) = st.a[h];
        *reinterpret_cast<v4u32*>(sB + o) = st.b[h];
    }
    sS[t] = st.s;
}

template <bool BF16, bool SCALE4>
__global__ __launch_bounds__(256) void k_gemm_mx_any(const GemmParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][kTile * kPitch];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][kTile * kPitch];
    __shared__ uint32_t sS[2][2 * kTile];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, kc = lane >> 5;
    const uint32_t tm = blockIdx.x / p.tiles_n, tn = blockIdx.x - tm * p.tiles_n;
    const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTile;
    const int64_t rowb = p.K / 2, srow = p.K / 32;

    Rows rows;
    #pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = t + 256 * h, rr = c >> 2, part = c & 3;
        rows.a[h] = p.a + min(m0 + rr, p.M - 1) * rowb + part * 16;
        rows.b[h] = p.b + min(n0 + rr, p.N - 1) * rowb + part * 16;
    }
    rows.s = t < kTile ? p.as + min(m0 + t, p.M - 1) * srow : p.bs + min(n0 + t - kTile, p.N - 1) * srow;

    v16f acc[2][2];
    #pragma unroll
    for (int i = 0; i < 2; ++i)
        #pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = (v16f){};

    const int64_t kblocks = srow, steps = (kblocks + 3) / 4;
    Stage st;
    if (steps > 0) {
        load_stage<SCALE4>(rows, 0, (int)min<int64_t>(4, kblocks), st);
        store_stage(st, sA[0], sB[0], sS[0]);
    }
    __syncthreads();
    for (int64_t s = 0; s < steps; ++s) {
        const int buf = (int)(s & 1);
        if (s + 1 < steps) load_stage<SCALE4>(rows, s + 1, (int)min<int64_t>(4, kblocks - 4 * (s + 1)), st);
        #pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int blk = 2 * ks + kc;   // this lane's scale block within the stage
            v8i a[2], b[2];
            int sa[2], sb[2];
            #pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ra = wm * 64 + i * 32 + r32, rb = wn * 64 + i * 32 + r32;
                const v4u32 va = *reinterpret_cast<const v4u32*>(&sA[buf][ra * kPitch + blk * 16]);
                const v4u32 vb = *reinterpret_cast<const v4u32*>(&sB[buf][rb * kPitch + blk * 16]);
                a[i] = (v8i){(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
                b[i] = (v8i){(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
                sa[i] = (int)(sS[buf][ra] >> (8 * blk));
                sb[i] = (int)(sS[buf][kTile + rb] >> (8 * blk));
            }
            #pragma unroll
            for (int i = 0; i < 2; ++i)
                #pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0, sa[i],
                                                                              0, sb[j]);
        }
        if (s + 1 < steps) store_stage(st, sA[buf ^ 1], sB[buf ^ 1], sS[buf ^ 1]);
        __syncthreads();
    }

    #pragma unroll
    for (int i = 0; i < 2; ++i)
        #pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = n0 + wn * 64 + j * 32 + r32;
            #pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * kc + (r & 3);
                if (row < p.M && col < p.N) {
                    if constexpr (BF16) {
                        const bf16x2 h = __builtin_convertvector((v2f){acc[i][j][r], 0.0f}, bf16x2);
                        reinterpret_cast<uint16_t*>(p.c)[row * p.ldc + col] =
                            (uint16_t)(__builtin_bit_cast(uint32_t, h) & 0xFFFFu);
                    } else {
                        reinterpret_cast<float*>(p.c)[row * p.ldc + col] = acc[i][j][r];
                    }
                }
            }
        }
}

}  // namespace

// ---------------------------------------------------------------- main path
// K % 128 == 0: operands stream into LDS by direct buffer-to-LDS loads, three
// stages deep, so no registers hold data in flight and two stages of loads
// overlap each stage's MFMAs.  A wave instruction writes 64 lanes x 16 bytes
// contiguously, so the tile cannot be padded; instead a row's four 16-byte
// pieces (one per scale block) sit in the order blk ^ swz(row), which puts
// the 16 rows that 16 consecutive lanes read at one block on 16 distinct
// 16-byte bank groups (and any 8 consecutive rows on 8).  Loads of rows past
// M or N fall outside the buffer range and return zeros.

// Piece order of a staged row: bits 1-2 of the row xor bits 3-4.
static __device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int WM, int WN>
struct LdsTile {
    static constexpr int RA = 64 * WM, RB = 64 * WN;      // rows of A and B per tile
    static constexpr int CODE_BYTES = (RA + RB) * 64;     // one stage of codes
    static constexpr int STAGE_BYTES = CODE_BYTES + (RA + RB) * 4;
    static constexpr int NCODE = (RA + RB) / 16;          // wave loads of codes per stage
    static constexpr int NSCALE = (RA + RB) / 64;         // wave loads of scales per stage
};

constexpr int kStages = 3;

// s_waitcnt immediate: at most n vector-memory operations of this wave outstanding.
#define FP4Q_VMCNT(n) (0x0F70 | ((n) & 0xF) | (((n) >> 4) << 14))

// Workgroup barrier without a memory fence: the waits before it are explicit,
// and the empty asm statements keep the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void barrier_only() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 1: 256 x 192 tiles, when there are enough of them to give every compute
// unit one; 0: 128 x 128 tiles.
static int gemm_config(int64_t M, int64_t N) {
    return ((M + 255) / 256) * ((N + 191) / 192) >= 256 ? 1 : 0;
}

// This wave's share of the direct-to-LDS loads of one stage (wave loads
// i = wave, wave + 4, ...; see the kernel) into LDS stage buffer buf.
__device__ __forceinline__ int clamp31(int64_t v) { return (int)(v > 0x7FFFFFFF ? 0x7FFFFFFF : v); }

struct Bases {
    const uint8_t *a, *b, *as, *bs;   // first row of this tile in each operand
    int na, nb, nas, nbs;             // bytes from there to the end of each operand (clamped)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}

template <int WM, int WN, int PER>
__device__ __forceinline__ void issue_stage(uint8_t* smem, const Bases& bs, const int* voff, int wave,
                                            int64_t step, int buf) {
    using T = LdsTile<WM, WN>;
    constexpr int NL = T::NCODE + T::NSCALE;
    uint8_t* st = smem + buf * T::STAGE_BYTES;
    #pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int i = wave + 4 * q;
        if (i < T::NCODE) {
            const bool isa = i < T::RA / 16;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isa ? rsrc(bs.a, bs.na) : rsrc(bs.b, bs.nb),
                                                     (lds_ptr_t)(st + i * 1024), 16, voff[q], (int)(step * 64), 0, 0);
        } else if (i < NL) {
            const int j = i - T::NCODE;
            const bool isa = j < T::RA / 64;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isa ? rsrc(bs.as, bs.nas) : rsrc(bs.bs, bs.nbs),
                                                     (lds_ptr_t)(st + T::CODE_BYTES + j * 256), 4, voff[q],
                                                     (int)(step * 4), 0, 0);
        }
    }
}

template <int WM, int WN, bool BF16>
__global__ __launch_bounds__(256) void k_gemm_mx_lds(const GemmParams p) {
    using T = LdsTile<WM, WN>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, kc = lane >> 5;

    // tile of this workgroup; consecutive workgroups go to different XCDs, so
    // tiles are handed out XCD by XCD when the grid divides evenly
    uint32_t bid = blockIdx.x;
    if (p.xcd_remap) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
    const uint32_t tm = bid / p.tiles_n, tn = bid - tm * p.tiles_n;
    const int64_t m0 = (int64_t)tm * T::RA, n0 = (int64_t)tn * T::RB;
    const int64_t rowb = p.K / 2, srow = p.K / 32;

    Bases bs;
    bs.a = p.a + m0 * rowb;
    bs.b = p.b + n0 * rowb;
    bs.as = p.as + m0 * srow;
    bs.bs = p.bs + n0 * srow;
    bs.na = clamp31((p.M - m0) * rowb);
    bs.nb = clamp31((p.N - n0) * rowb);
    bs.nas = clamp31((p.M - m0) * srow);
    bs.nbs = clamp31((p.N - n0) * srow);

    // wave load i of a stage: codes i < NCODE (rows 16 i' .. 16 i' + 15 of A, then of B),
    // then scales (rows 64 j .. 64 j + 63 of A, then of B); this wave takes i = wave, wave + 4, ...
    constexpr int NL = T::NCODE + T::NSCALE;
    constexpr int PER = (NL + 3) / 4;
    static_assert(PER <= 63, "vmcnt range");
    const int cnt = (NL - wave + 3) / 4;   // loads this wave issues per stage: PER or PER - 1
    int voff[PER];
    #pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int i = wave + 4 * q;
        if (i < T::NCODE) {
            const int ia = i < T::RA / 16 ? i : i - T::RA / 16;
            const int row = 16 * ia + (lane >> 2);
            voff[q] = (int)(row * rowb) + 16 * ((lane & 3) ^ swz(row));
        } else {
            const int j = i - T::NCODE;
            const int ja = j < T::RA / 64 ? j : j - T::RA / 64;
            voff[q] = (int)((64 * ja + lane) * srow);
        }
    }

    v16f acc[WM][WN];
    #pragma unroll
    for (int i = 0; i < WM; ++i)
        #pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = (v16f){};

    const int64_t steps = p.K / 128;
    #pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
        if (s < steps) issue_stage<WM, WN, PER>(smem, bs, voff, wave, s, s);
    for (int64_t s = 0; s < steps; ++s) {
        const int buf = (int)(s % kStages);
        // this wave's loads of stage s are done once at most those of stage s + 1 remain
        // (loads complete in order); the barrier then covers every wave's loads
        if (s + 1 < steps) {
            if (cnt == PER) __builtin_amdgcn_s_waitcnt(FP4Q_VMCNT(PER));
            else __builtin_amdgcn_s_waitcnt(FP4Q_VMCNT(PER - 1));
        } else {
            __builtin_amdgcn_s_waitcnt(FP4Q_VMCNT(0));
        }
        barrier_only();
        if (s + kStages - 1 < steps)
            issue_stage<WM, WN, PER>(smem, bs, voff, wave, s + kStages - 1,
                                     (int)((s + kStages - 1) % kStages));
        const uint8_t* sa_codes = smem + buf * T::STAGE_BYTES;
        const uint8_t* sb_codes = sa_codes + T::RA * 64;
        const uint32_t* sa_sc = reinterpret_cast<const uint32_t*>(sa_codes + T::CODE_BYTES);
        const uint32_t* sb_sc = sa_sc + T::RA;
        uint32_t sca[WM], scb[WN];
        #pragma unroll
        for (int i = 0; i < WM; ++i) sca[i] = sa_sc[wm * 32 * WM + i * 32 + r32];
        #pragma unroll
        for (int j = 0; j < WN; ++j) scb[j] = sb_sc[wn * 32 * WN + j * 32 + r32];
        #pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int blk = 2 * ks + kc;
            v8i a[WM], b[WN];
            #pragma unroll
            for (int i = 0; i < WM; ++i) {
                const int row = wm * 32 * WM + i * 32 + r32;
                const v4u32 v = *reinterpret_cast<const v4u32*>(sa_codes + row * 64 + 16 * (blk ^ swz(row)));
                a[i] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            }
            #pragma unroll
            for (int j = 0; j < WN; ++j) {
                const int row = wn * 32 * WN + j * 32 + r32;
                const v4u32 v = *reinterpret_cast<const v4u32*>(sb_codes + row * 64 + 16 * (blk ^ swz(row)));
                b[j] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            }
            #pragma unroll
            for (int i = 0; i < WM; ++i)
                #pragma unroll
                for (int j = 0; j < WN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        a[i], b[j], acc[i][j], 4, 4, 0, (int)(sca[i] >> (8 * blk)), 0, (int)(scb[j] >> (8 * blk)));
        }
    }

    #pragma unroll
    for (int i = 0; i < WM; ++i)
        #pragma unroll
        for (int j = 0; j < WN; ++j) {
            const int64_t col = n0 + wn * 32 * WN + j * 32 + r32;
            #pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = m0 + wm * 32 * WM + i * 32 + 8 * (r >> 2) + 4 * kc + (r & 3);
                if (row < p.M && col < p.N) {
                    if constexpr (BF16) {
                        const bf16x2 h = __builtin_convertvector((v2f){acc[i][j][r], 0.0f}, bf16x2);
                        reinterpret_cast<uint16_t*>(p.c)[row * p.ldc + col] =
                            (uint16_t)(__builtin_bit_cast(uint32_t, h) & 0xFFFFu);
                    } else {
                        reinterpret_cast<float*>(p.c)[row * p.ldc + col] = acc[i][j][r];
                    }
                }
            }
        }
}

template <int WM, int WN>
static hipError_t launch_lds(bool bf16_out, GemmParams p, hipStream_t s) {
    using T = LdsTile<WM, WN>;
    const uint32_t tiles_m = (uint32_t)((p.M + T::RA - 1) / T::RA);
    p.tiles_n = (uint32_t)((p.N + T::RB - 1) / T::RB);
    const uint32_t g = tiles_m * p.tiles_n;
    p.xcd_remap = g % 8 == 0 ? 1u : 0u;
    const size_t lds = (size_t)kStages * T::STAGE_BYTES;
    if (bf16_out) hipLaunchKernelGGL((k_gemm_mx_lds<WM, WN, true>), dim3(g), dim3(256), lds, s, p);
    else hipLaunchKernelGGL((k_gemm_mx_lds<WM, WN, false>), dim3(g), dim3(256), lds, s, p);
    return hipGetLastError();
}

hipError_t launch_gemm_mx(bool bf16_out, const GemmParams& p, hipStream_t s) {
    const bool scale4 = p.K % 128 == 0 && ((uintptr_t)p.as & 3) == 0 && ((uintptr_t)p.bs & 3) == 0;
    if (scale4 && p.K > 0 && p.K < (1ll << 24)) {
        const int cfg = gemm_config(p.M, p.N);
        if (cfg == 1) return launch_lds<4, 3>(bf16_out, p, s);
        return launch_lds<2, 2>(bf16_out, p, s);
    }
    GemmParams q = p;
    q.tiles_n = (uint32_t)((p.N + kTile - 1) / kTile);
    const dim3 grid((uint32_t)(((p.M + kTile - 1) / kTile) * q.tiles_n)), block(256);
    if (bf16_out) {
        if (scale4) hipLaunchKernelGGL((k_gemm_mx_any<true, true>), grid, block, 0, s, q);
        else hipLaunchKernelGGL((k_gemm_mx_any<true, false>), grid, block, 0, s, q);
    } else {
        if (scale4) hipLaunchKernelGGL((k_gemm_mx_any<false, true>), grid, block, 0, s, q);
        else hipLaunchKernelGGL((k_gemm_mx_any<false, false>), grid, block, 0, s, q);
    }
    return hipGetLastError();
}

}  // namespace fp4q
