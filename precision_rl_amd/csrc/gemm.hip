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
__global__ __launch_bounds__(256) void k_gemm_mx(const GemmParams p) {
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

uint32_t gemm_tiles(int64_t M, int64_t N) {
    return (uint32_t)(((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile));
}

hipError_t launch_gemm_mx(bool bf16_out, const GemmParams& p, hipStream_t s) {
    const dim3 grid(gemm_tiles(p.M, p.N)), block(256);
    const bool scale4 = p.K % 128 == 0 && ((uintptr_t)p.as & 3) == 0 && ((uintptr_t)p.bs & 3) == 0;
    if (bf16_out) {
        if (scale4) hipLaunchKernelGGL((k_gemm_mx<true, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((k_gemm_mx<true, false>), grid, block, 0, s, p);
    } else {
        if (scale4) hipLaunchKernelGGL((k_gemm_mx<false, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((k_gemm_mx<false, false>), grid, block, 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace fp4q
