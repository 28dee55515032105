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
// block's E8M0 scale in the byte of the lane's scale operand that op_sel picks.
// Result element j of lane l is C[8 (j / 4) + 4 (l / 32) + j % 4][l mod 32].
// (Layout checked on the GPU against a host product of random codes and scales.)
//
// Main path (K % 512 == 0, scales 16-byte aligned), gemm_tile below: a
// workgroup of 4 waves (2 x 2) computes a 256 x 256 or 256 x 192 tile of C,
// whichever finishes the product in fewer tile-times counting whole rounds of
// one tile per compute unit, or 128 x 128 when there are too few 256 x 192
// tiles to give every compute unit one.  Tiles go out in groups of four row
// tiles, XCD by XCD, so that the tiles one XCD runs together share operand
// rows in its L2.  K advances 256 values per stage (128 bytes of codes per
// row, one whole cache line); both operands stream from memory straight into
// LDS by buffer-to-LDS loads, double buffered, with the pieces of each staged
// row permuted so that the rows lanes read together sit on distinct bank
// groups.  Each stage is four MFMA K slices whose operands are read from LDS
// two slices ahead (one for 256 x 256 tiles, whose accumulators fill the
// accumulation registers); the reads and loads are spread between the MFMAs.
// Whole tiles of C are turned around in LDS and written as 16-byte row pieces;
// edge tiles store element by element through a buffer range that drops what
// lies outside C.
// The same K loop can instead end in the MXFP4 quantization of the
// bf16-rounded product, or its NVFP4 quantization under a given tensor scale
// (the producer-side epilogue): C is then not written, only its codes, scales
// and guide bits.
//
// Other K (multiples of 32), k_gemm_mx_any: 128 x 128 tiles, K advancing 128
// values per stage through registers into LDS rows padded to 80 bytes.
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
// K % 512 == 0.  A workgroup of 4 waves (2 x 2) computes a (64 WM) x (64 WN)
// tile of C.  K advances 256 values per stage: 128 bytes of codes per row,
// one whole cache line -- the memory system's cost is per line touched, and
// 64-byte half lines would halve the load rate.  Both operands stream into LDS
// by direct buffer-to-LDS loads (no registers hold data in flight), double
// buffered.  A wave instruction writes 64 lanes x 16 bytes contiguously, so
// the tile cannot be padded; instead the eight 16-byte pieces of a staged row
// (one per scale block) sit in the order blk ^ swz(row), which puts the 16
// rows that 16 consecutive lanes read at one block on 16 distinct 16-byte
// bank groups (and any 8 consecutive rows on 8).  The scales of four stages
// (32 bytes of a row; of two stages for 256 x 256 tiles, whose LDS has no room
// for more) come in with one load per row.  Loads of rows past M or
// N fall outside the buffer range and return zeros.

// Piece order of a staged row of 8 pieces: low 3 bits of row ^ (row >> 3).
static __device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int WM, int WN>
struct LdsTile {
    static constexpr int RA = 64 * WM, RB = 64 * WN;      // rows of A and B per tile
    static constexpr int ROWS = RA + RB;                  // stacked: A rows, then B rows
    static constexpr int CODE_BYTES = ROWS * 128;         // one stage of codes
    // scale loads with nothing to load (not the first stage of a chunk, or
    // past the last row block) still issue, with an empty range, into a sink
    // that every such load of every wave shares
    static constexpr int SINK_BYTES = 1024;
    // Stages whose scales one load per row brings: 4 (32 bytes of a row), or 2
    // where double-buffered chunks of 4 would not fit in LDS beside the codes.
    static constexpr int CHUNK = 2 * CODE_BYTES + 2 * ROWS * 32 + SINK_BYTES <= 160 * 1024 ? 4 : 2;
    static constexpr int SPITCH = 8 * CHUNK;              // bytes of a row's scales in one chunk
    static constexpr int SROWS = 1024 / SPITCH;           // rows per wave load of scales (64 lanes x 16 bytes)
    static constexpr int SCALE_BYTES = ROWS * SPITCH;     // one chunk of scales
    static constexpr int NCODE = ROWS / 8;                // wave loads of codes per stage (8 rows each)
    static constexpr int NCW = NCODE / 4;                 // ... per wave: 2 (WM + WN)
    static constexpr int NSCALE = ROWS / SROWS;           // wave loads of scales per chunk
    static constexpr int NSQ = (NSCALE + 3) / 4;          // scale loads every wave issues per stage
    static constexpr int BATCH = NCW + NSQ;               // loads every wave issues per stage
    // The scale loads issued with the code loads of stage t are those of stage
    // t + LEAD.  Chunks of 2 stages (LEAD 1): one stage ahead of the codes.
    // Their chunk buffer is free by then, the codes' buffer is not.
    static constexpr int LEAD = CHUNK == 2 ? 1 : 0;
    // Loads of this wave that may still be in flight once stage s + 1 is in:
    // those issued after its codes and scales.
    static constexpr int WAIT = LEAD * NSQ;
    // ... once stage 0 is in, after the loads of stages 0 and 1
    static constexpr int WAIT0 = BATCH + LEAD * NSQ;
    static constexpr int LDS_BYTES = 2 * CODE_BYTES + 2 * SCALE_BYTES + SINK_BYTES;
    static_assert(NCODE % 4 == 0, "code loads split evenly over the 4 waves");
    static_assert(RA % SROWS == 0, "a wave load of scales lies within A or within B");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS of one workgroup");
};

// s_waitcnt immediate: at most n vector-memory operations of this wave outstanding.
#define FP4Q_VMCNT(n) (0x0F70 | ((n) & 0xF) | (((n) >> 4) << 14))
// s_waitcnt immediate: no LDS operation of this wave outstanding.
#define FP4Q_LGKMCNT0 0xC07F

// Workgroup barrier without a memory fence: the waits before it are explicit,
// and the empty asm statements keep the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void barrier_only() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 0: 128 x 128 tiles, when there are too few 256 x 192 tiles to give every
// compute unit one; else 1: 256 x 192 or 2: 256 x 256 tiles, whichever
// finishes first counting whole rounds of 256 tiles (one per compute unit) and
// a 256 x 256 tile's time as (256 x 256) / (256 x 192) / kSpeed44 that of a
// 256 x 192 tile (it loads 64 KiB per 64 MFMAs of each wave and stage, where
// the 256 x 192 tile loads 56 KiB per 48).
constexpr double kSpeed44 = 1.1;
static int gemm_config(int64_t M, int64_t N) {
    const int64_t t43 = ((M + 255) / 256) * ((N + 191) / 192), t44 = ((M + 255) / 256) * ((N + 255) / 256);
    if (t43 < 256) return 0;
    const double r43 = (double)((t43 + 255) / 256), r44 = (double)((t44 + 255) / 256);
    return r44 * (256.0 / 192.0) / kSpeed44 < r43 ? 2 : 1;
}

__device__ __forceinline__ int clamp31(int64_t v) { return (int)(v > 0x7FFFFFFF ? 0x7FFFFFFF : v); }

struct Bases {
    const uint8_t *a, *b, *as, *bs;   // first row of this tile in each operand
    int na, nb, nas, nbs;             // bytes from there to the end of each operand (clamped)
    int rowb;                         // bytes per row of codes
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
}

// This wave's code loads of stage t, then its scale loads for stage t + LEAD,
// all issued whatever t, so that the K loop has no branches: code load q
// (stacked rows 8 i .. 8 i + 7, i = wave + 4 q) into code buffer t % 2, and
// scale load q (stacked rows 32 j .. 32 j + 31, j = wave + 4 q) into scale
// buffer (u / CHUNK) % 2, u = t + LEAD, when u starts a chunk.  Loads with
// nothing to load (a stage past the last, a scale load off a chunk start, j
// past the last row block) get an empty range: they move no data and write
// zeros into LDS the kernel no longer reads (scale loads into the sink).  The
// scale loads go last in their batch.  With chunks of 2 stages they go out one
// stage ahead, and the barrier before which the next stage must be in lets
// them still be in flight, so they have two stages to land.  Each touches one
// cache line per row for 16 bytes of it: loaded with the codes of their own
// stage, they made every other stage of 256 x 256 tiles about 30% longer.
// (With chunks of 4 the same lead measured 2% slower on 256 x 192 tiles.)
// PART selects which loads to issue: 0 all, 1 the first half of the code
// loads, 2 the second half and the scale loads.
template <int WM, int WN>
__device__ __forceinline__ void issue_scales(uint8_t* smem, const Bases& bs, const int* soff, int wave, int t,
                                             int steps) {
    using T = LdsTile<WM, WN>;
    const bool chunk = t < steps && (t & (T::CHUNK - 1)) == 0;
    uint8_t* sb = smem + 2 * T::CODE_BYTES + ((t / T::CHUNK) & 1) * T::SCALE_BYTES;
    uint8_t* sink = smem + 2 * T::CODE_BYTES + 2 * T::SCALE_BYTES;
    #pragma unroll
    for (int q = 0; q < T::NSQ; ++q) {
        const int j = wave + 4 * q;
        const bool real = chunk && j < T::NSCALE;
        const __amdgpu_buffer_rsrc_t r =
            j * T::SROWS < T::RA ? rsrc(bs.as, real ? bs.nas : 0) : rsrc(bs.bs, real ? bs.nbs : 0);
        const int so = soff[q];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(real ? sb + j * 1024 : sink), 16, so, t * 8, 0, 0);
    }
}

template <int WM, int WN, int PART = 0>
__device__ __forceinline__ void issue_stage(uint8_t* smem, const Bases& bs, const int* voff, const int* soff,
                                            int wave, int t, int steps) {
    using T = LdsTile<WM, WN>;
    const bool live = t < steps;
    uint8_t* cb = smem + (t & 1) * T::CODE_BYTES;
    const __amdgpu_buffer_rsrc_t ra = rsrc(bs.a, live ? bs.na : 0);
    const __amdgpu_buffer_rsrc_t rb = rsrc(bs.b, live ? bs.nb : 0);
    constexpr int Q0 = PART == 2 ? T::NCW / 2 : 0, Q1 = PART == 1 ? T::NCW / 2 : T::NCW;
    #pragma unroll
    for (int q = Q0; q < Q1; ++q) {
        // stacked row 32 q + (8 wave + lane / 8): its piece order depends on q only through q & 1
        const int vo = voff[q & 1] + (int)((32 * q - (q < 2 * WM ? 0 : T::RA)) * bs.rowb);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(q < 2 * WM ? ra : rb, (lds_ptr_t)(cb + (wave + 4 * q) * 1024), 16,
                                                 vo, t * 128, 0, 0);
    }
    if constexpr (PART == 1) return;
    issue_scales<WM, WN>(smem, bs, soff, wave, t + T::LEAD, steps);
}

// Operands of K slice KS of stage st for this wave: A rows of 32-row blocks
// rowA0 .. rowA0 + WM - 1 and B rows of blocks rowB0 .. rowB0 + WN - 1 of the
// stacked tile, 16 bytes per lane (block 2 KS + kc of the lane's row).
template <int WM, int WN, int KS>
__device__ __forceinline__ void read_ops(const uint8_t* smem, int st, const int (&roff)[4][2], int rowA0, int rowB0,
                                         v4u32 (&a)[WM], v4u32 (&b)[WN]) {
    const uint8_t* ca = smem + (st & 1) * LdsTile<WM, WN>::CODE_BYTES;
    #pragma unroll
    for (int i = 0; i < WM; ++i) {
        const int m = rowA0 + i;
        a[i] = *reinterpret_cast<const v4u32*>(ca + roff[KS][m & 1] + m * 32 * 128);
    }
    #pragma unroll
    for (int j = 0; j < WN; ++j) {
        const int m = rowB0 + j;
        b[j] = *reinterpret_cast<const v4u32*>(ca + roff[KS][m & 1] + m * 32 * 128);
    }
}

// Both scale words of stage st for this wave's rows (word w: blocks 4 w ..
// 4 w + 3).  One 8-byte read per row: rows lie 16 or 32 bytes apart, so
// narrower reads would cost the same bank conflicts twice.
template <int WM, int WN>
__device__ __forceinline__ void read_scales(const uint8_t* sbase, int st, int scA, int scB,
                                            v2u32 (&sa)[WM], v2u32 (&sb)[WN]) {
    using T = LdsTile<WM, WN>;
    const uint8_t* sc = sbase + ((st / T::CHUNK) & 1) * T::SCALE_BYTES + 8 * (st & (T::CHUNK - 1));
    #pragma unroll
    for (int i = 0; i < WM; ++i) sa[i] = *reinterpret_cast<const v2u32*>(sc + scA + i * 32 * T::SPITCH);
    #pragma unroll
    for (int j = 0; j < WN; ++j) sb[j] = *reinterpret_cast<const v2u32*>(sc + scB + j * 32 * T::SPITCH);
}

// The WM x WN MFMAs of K slice KS with the stage's scale words ua, ub, each
// moved down by 8 kc bits here, at its use, so that byte 2 (KS & 1) of word
// KS / 2 is the lane's block 2 KS + kc.  (Shifted where they are read, the
// words of the next stage would make the MFMAs that follow the read wait for
// it.)
template <int WM, int WN, int KS>
__device__ __forceinline__ void mfmas(v16f (&acc)[WM][WN], const v4u32 (&a)[WM], const v4u32 (&b)[WN],
                                      const v2u32 (&ua)[WM], const v2u32 (&ub)[WN], int kc) {
    #pragma unroll
    for (int i = 0; i < WM; ++i) {
        const v8i av = (v8i){(int)a[i].x, (int)a[i].y, (int)a[i].z, (int)a[i].w, 0, 0, 0, 0};
        const int sa = (int)((KS < 2 ? ua[i].x : ua[i].y) >> (8 * kc));
        #pragma unroll
        for (int j = 0; j < WN; ++j) {
            const v8i bv = (v8i){(int)b[j].x, (int)b[j].y, (int)b[j].z, (int)b[j].w, 0, 0, 0, 0};
            const int sb = (int)((KS < 2 ? ub[j].x : ub[j].y) >> (8 * kc));
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 4, 4, 2 * (KS & 1), sa,
                                                                      2 * (KS & 1), sb);
        }
    }
}

// One element of C: fp32, or bf16 by round-to-nearest-even.
template <bool BF16>
__device__ __forceinline__ void store_c(__amdgpu_buffer_rsrc_t rc, int voff, float v) {
    if constexpr (BF16) {
        const bf16x2 h = __builtin_convertvector((v2f){v, 0.0f}, bf16x2);
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(__builtin_bit_cast(uint32_t, h) & 0xFFFFu), rc, voff, 0,
                                              0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rc, voff, 0, 0);
    }
}

// MXFP4 round-to-nearest quantization of one 32-element block of bf16 values
// (16 dwords, element 2j in the low half of w[j]), as the MXFP4 quantizer does
// it without the RHT: scale code max(E(amax) - 2, 0) from the largest bf16
// magnitude, codes by the scaled RNE convert of the bf16 words; a block holding
// a non-finite value gets scale 0xFF and zero codes.  Returns the scale code;
// c receives the 16 bytes of codes.
__device__ __forceinline__ uint32_t quantize_block32_bf16(const uint32_t w[16], uint32_t c[4]) {
    const uint32_t key = max(amax_bits16(w), amax_bits16(w + 8)) << 16;
    const uint32_t e = key >> 23;
    uint32_t sc = e > 2u ? e - 2u : 0u;
    const float cs = mx_scale(sc);
    #pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = pack_rne8_bf16(w + 4 * k, cs);
    if (key >= 0x7F800000u) {
        sc = 0xFFu;
        #pragma unroll
        for (int k = 0; k < 4; ++k) c[k] = 0u;
    }
    return sc;
}

// The NVFP4 tensor scale's per-launch terms: the block divisor RN(6 s_t), its
// reciprocal, and whether that reciprocal is a normal number.
struct NvScale {
    float ts, denom, rden;
    bool rden_ok;
};

__device__ __forceinline__ NvScale nv_scale(float ts) {
    NvScale n;
    n.ts = ts;
    n.denom = 6.0f * ts;
    n.rden = 1.0f / n.denom;
    n.rden_ok = n.denom >= 0x1p-125f && n.denom <= 0x1p125f;
    return n;
}

// NVFP4 round-to-nearest quantization of two 16-element groups of bf16 values
// (w[0..7] the first, w[8..15] the second, element 2j in the low half of a
// dword), as the NVFP4 quantizer does it without the RHT: per group the scale
// code is the E4M3 RNE of amax / RN(6 s_t), saturating at 448 (the quotient taken
// as a product with the reciprocal wherever that gives the same code, else
// divided), the elements are multiplied by RN(1 / RN(dec(code) s_t)) and rounded
// to E2M1 ties to even; a group holding a non-finite value gets scale 0x7F and
// zero codes.  Returns the two scale codes, the first in the low byte; c
// receives the 16 bytes of codes.
__device__ __forceinline__ uint32_t quantize_2x16_nvfp4_bf16(const uint32_t w[16], const NvScale& ns,
                                                             uint32_t c[4]) {
    uint32_t scs = 0;
    #pragma unroll
    for (int g = 0; g < 2; ++g) {
        const uint32_t* gw = w + 8 * g;
        const uint32_t key = amax_bits16(gw) << 16;
        float t = __uint_as_float(key) * ns.rden;
        const uint32_t tb = __float_as_uint(t);
        // the product gives the quotient's E4M3 code unless it lies within 4 fp32
        // steps of a code midpoint, or below 2^-6 + 4 steps (and is not 0)
        if (!ns.rden_ok || tb - 1u < 0x3C800003u || (tb & 0xFFFFFu) - 0x7FFFCu <= 8u)
            t = __uint_as_float(key) / ns.denom;
        uint32_t sc = e4m3_encode_rne(clamp448(t));
        const float inv = nvfp4_inv(sc, ns.ts);
        float y[16];
        widen16<false>(gw, 0u, y);
        #pragma unroll
        for (int j = 0; j < 16; ++j) y[j] = y[j] * inv;
        uint32_t c0 = encode8<0, MODE_RTN>(y, 0u, 0u, 0u), c1 = encode8<0, MODE_RTN>(y + 8, 0u, 0u, 0u);
        if (key >= 0x7F800000u) {
            sc = 0x7Fu;
            c0 = c1 = 0u;
        }
        c[2 * g] = c0;
        c[2 * g + 1] = c1;
        scs |= sc << (8 * g);
    }
    return scs;
}

// Producer-side epilogue: the wave's quarter of C, rounded to bf16, goes through
// LDS half its rows at a time (as the staged store does); then each lane takes
// 32 consecutive elements of a row (one MXFP4 block, or two NVFP4 groups under
// the tensor scale *p.qts when NV), quantizes them with round to nearest and
// writes their 16 bytes of codes, their scale byte(s) and, when asked for, their
// 32 guide bits.  N % 32 == 0, so the 32 elements lie wholly inside or outside C.
template <int WM, int WN, bool NV>
__device__ __forceinline__ void quantize_epilogue(const GemmParams& p, const v16f (&acc)[WM][WN], uint8_t* smem,
                                                  int wave, int lane, int kc, int r32, int64_t row0, int64_t col0) {
    constexpr int HR = 16 * WM;              // rows per half
    constexpr int PITCH = 32 * WN * 2;       // bytes per staged row of bf16
    constexpr int NB = HR * WN;              // 32-element blocks per half
    static_assert(NB % 64 == 0, "whole wave instructions per half");
    uint8_t* st = smem + wave * HR * PITCH;
    const int64_t cb = p.N / 2, sb = p.N / (NV ? 16 : 32), bb = p.N / 8;   // bytes per row of codes, scales, bits
    NvScale ns{};
    if constexpr (NV) ns = nv_scale(*p.qts);
    barrier_only();   // every wave is done with the K loop's LDS
    #pragma unroll
    for (int h = 0; h < 2; ++h) {
        #pragma unroll
        for (int i = 0; i < WM / 2; ++i)
            #pragma unroll
            for (int j = 0; j < WN; ++j)
                #pragma unroll
                for (int r = 0; r < 16; ++r) {
                    uint8_t* d = st + (32 * i + 8 * (r >> 2) + 4 * kc + (r & 3)) * PITCH + (32 * j + r32) * 2;
                    const bf16x2 b = __builtin_convertvector((v2f){acc[h * (WM / 2) + i][j][r], 0.0f}, bf16x2);
                    *reinterpret_cast<uint16_t*>(d) = (uint16_t)(__builtin_bit_cast(uint32_t, b) & 0xFFFFu);
                }
        // this wave's LDS writes complete before its reads (LDS operations of a wave run in order)
        #pragma unroll
        for (int q = 0; q < NB / 64; ++q) {
            const int c = q * 64 + lane, r = c / WN, blk = c - r * WN;
            uint32_t w[16];
            #pragma unroll
            for (int k = 0; k < 4; ++k) {
                const v4u32 v = *reinterpret_cast<const v4u32*>(st + r * PITCH + blk * 64 + 16 * k);
                w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
            }
            uint32_t codes[4];
            const uint32_t sc = NV ? quantize_2x16_nvfp4_bf16(w, ns, codes) : quantize_block32_bf16(w, codes);
            const int64_t row = row0 + h * HR + r, col = col0 + 32 * blk;
            if (row < p.M && col < p.N) {
                *reinterpret_cast<v4u32*>(p.qcodes + row * cb + col / 2) = (v4u32){codes[0], codes[1], codes[2], codes[3]};
                if constexpr (NV) *reinterpret_cast<uint16_t*>(p.qscales + row * sb + col / 16) = (uint16_t)sc;
                else p.qscales[row * sb + col / 32] = (uint8_t)sc;
                if (p.qbits) {
                    const uint32_t bits = gather_nibble_lsbs(codes[0]) | (gather_nibble_lsbs(codes[1]) << 8) |
                                          (gather_nibble_lsbs(codes[2]) << 16) | (gather_nibble_lsbs(codes[3]) << 24);
                    *reinterpret_cast<uint32_t*>(p.qbits + row * bb + col / 8) = bits;
                }
            }
        }
    }
}

// Instruction order of a K-loop region: its NM MFMAs spread out, the first ND
// of them each followed by one LDS read and the first NV by one memory load
// (PER > 0: the LDS reads go with the first ND of every PER MFMAs instead), so
// that the wave issues its reads and loads while the matrix core works, not
// in batches that leave it idle.
template <int NM, int ND, int NV, int PER = 0>
__device__ __forceinline__ void interleave() {
    #pragma unroll
    for (int k = 0; k < NM; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (PER ? (k % PER) < ND : k < ND) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (k < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    if (NV > NM) __builtin_amdgcn_sched_group_barrier(0x020, NV > NM ? NV - NM : 1, 0);
}

// Tile (tm, tn) of the product p, computed by the calling workgroup.  QUANT 1
// (MXFP4) or 2 (NVFP4): the epilogue quantizes the bf16-rounded tile (p.qcodes,
// p.qscales, p.qbits)
// instead of storing C.
template <int WM, int WN, bool BF16, int QUANT = 0>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, uint32_t tm, uint32_t tn, uint8_t* smem) {
    using T = LdsTile<WM, WN>;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, kc = lane >> 5;
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

    // per-lane offsets of this wave's loads (the stage enters as a scalar offset)
    bs.rowb = (int)rowb;
    int voff[2], soff[T::NSQ];
    #pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int row = 8 * (wave + 4 * q) + (lane >> 3);              // stacked row of code load q
        voff[q] = (int)((8 * wave + (lane >> 3)) * rowb) + 16 * ((lane & 7) ^ swz(row));
    }
    #pragma unroll
    for (int q = 0; q < T::NSQ; ++q) {
        const int j = wave + 4 * q;
        constexpr int LPR = T::SPITCH / 16;                            // lanes per row of a scale load
        const int row = T::SROWS * j + lane / LPR;
        soff[q] = (int)((row < T::RA ? row : row - T::RA) * srow) + 16 * (lane % LPR);
    }

    v16f acc[WM][WN];
    #pragma unroll
    for (int i = 0; i < WM; ++i)
        #pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = (v16f){};

    // Each stage is four MFMA K slices (ks = 0..3; lane block 2 ks + kc).  The
    // operands of slice ks + 2 are read from LDS while the MFMAs of slice ks
    // run, so that every wave keeps many LDS reads in flight; between the
    // second and third slices' MFMAs the workgroup meets at the barrier that
    // certifies the next stage's loads, starts the loads of the stage after it
    // into the buffers just read, and reads the next stage's scales and first
    // two slices.
    const int steps = (int)(p.K / 256);   // >= 2, even
    // A stacked row 32 m + r32 holds block blk at piece blk ^ swz(row) =
    // blk ^ lsw ^ 4 (m & 1), lsw = (r32 ^ r32 / 8) & 7: one lane offset per K
    // slice and parity of m, the rest an immediate
    int roff[4][2];
    #pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        #pragma unroll
        for (int par = 0; par < 2; ++par)
            roff[ks][par] = r32 * 128 + 16 * ((2 * ks + kc) ^ ((r32 ^ (r32 >> 3)) & 7) ^ (4 * par));
    const int rowA0 = wm * WM, rowB0 = T::RA / 32 + wn * WN;   // first 32-row blocks of this wave
    const int scA = (wm * 32 * WM + r32) * T::SPITCH, scB = (T::RA + wn * 32 * WN + r32) * T::SPITCH;

    v2u32 sa[WM], sb[WN], na[WM], nb[WN];   // scale words of this stage and the next
    const uint8_t* sbase = smem + 2 * T::CODE_BYTES;

    if constexpr (T::LEAD) issue_scales<WM, WN>(smem, bs, soff, wave, 0, steps);
    issue_stage<WM, WN>(smem, bs, voff, soff, wave, 0, steps);
    issue_stage<WM, WN>(smem, bs, voff, soff, wave, 1, steps);
    // stage 0 is in once only the loads issued after its codes and scales remain
    // (loads complete in order)
    __builtin_amdgcn_s_waitcnt(FP4Q_VMCNT(T::WAIT0));
    barrier_only();
    read_scales<WM, WN>(sbase, 0, scA, scB, sa, sb);
    if constexpr (WM * WN >= 16) {
        // 256 x 256 tiles: the accumulators fill the 256 accumulation registers,
        // so operands are read one slice ahead of their MFMAs into two sets (a
        // slice is 16 MFMAs per wave, 512 cycles, ample for the LDS reads); the
        // barrier comes after the third slice's MFMAs.
        v4u32 xa[WM], xb[WN], ya[WM], yb[WN];
        read_ops<WM, WN, 0>(smem, 0, roff, rowA0, rowB0, xa, xb);
        // stage s with scale words (ca, cb), reading stage s + 1's into (xa_, xb_): the two sets
        // alternate between stages, so that no copy waits for a read
        auto stage = [&](int s, v2u32 (&ca)[WM], v2u32 (&cb)[WN], v2u32 (&na_)[WM], v2u32 (&nb_)[WN]) {
            read_ops<WM, WN, 1>(smem, s, roff, rowA0, rowB0, ya, yb);
            mfmas<WM, WN, 0>(acc, xa, xb, ca, cb, kc);
            read_ops<WM, WN, 2>(smem, s, roff, rowA0, rowB0, xa, xb);
            mfmas<WM, WN, 1>(acc, ya, yb, ca, cb, kc);
            read_ops<WM, WN, 3>(smem, s, roff, rowA0, rowB0, ya, yb);
            mfmas<WM, WN, 2>(acc, xa, xb, ca, cb, kc);
            interleave<3 * WM * WN, WM + WN, 0, WM * WN>();
            // as below: stage s read and stage s + 1 in, for every wave after the barrier
            __builtin_amdgcn_s_waitcnt(FP4Q_LGKMCNT0);
            __builtin_amdgcn_s_waitcnt(FP4Q_VMCNT(T::WAIT));
            barrier_only();
            read_scales<WM, WN>(sbase, s + 1, scA, scB, na_, nb_);
            read_ops<WM, WN, 0>(smem, s + 1, roff, rowA0, rowB0, xa, xb);
            issue_stage<WM, WN, 1>(smem, bs, voff, soff, wave, s + 2, steps);
            mfmas<WM, WN, 3>(acc, ya, yb, ca, cb, kc);
            issue_stage<WM, WN, 2>(smem, bs, voff, soff, wave, s + 2, steps);
            interleave<WM * WN, WM + WN + (WM + WN + 1) / 2, LdsTile<WM, WN>::BATCH>();
        };
        int s = 0;
        for (; s + 2 < steps; s += 2) {
            stage(s, sa, sb, na, nb);
            stage(s + 1, na, nb, sa, sb);
        }
        stage(s, sa, sb, na, nb);   // s = steps - 2: stage steps - 1 has its scales in (na, nb)
        s = steps - 1;
        read_ops<WM, WN, 1>(smem, s, roff, rowA0, rowB0, ya, yb);
        mfmas<WM, WN, 0>(acc, xa, xb, na, nb, kc);
        read_ops<WM, WN, 2>(smem, s, roff, rowA0, rowB0, xa, xb);
        mfmas<WM, WN, 1>(acc, ya, yb, na, nb, kc);
        read_ops<WM, WN, 3>(smem, s, roff, rowA0, rowB0, ya, yb);
        mfmas<WM, WN, 2>(acc, xa, xb, na, nb, kc);
        mfmas<WM, WN, 3>(acc, ya, yb, na, nb, kc);
    } else {
        // operand sets for K slices 0..3 of a stage (read two slices ahead of their MFMAs)
        v4u32 a0[WM], b0[WN], a1[WM], b1[WN], a2[WM], b2[WN], a3[WM], b3[WN];
        read_ops<WM, WN, 0>(smem, 0, roff, rowA0, rowB0, a0, b0);
        read_ops<WM, WN, 1>(smem, 0, roff, rowA0, rowB0, a1, b1);
        auto stage = [&](int s, v2u32 (&ca)[WM], v2u32 (&cb)[WN], v2u32 (&na_)[WM], v2u32 (&nb_)[WN]) {
            read_ops<WM, WN, 2>(smem, s, roff, rowA0, rowB0, a2, b2);
            mfmas<WM, WN, 0>(acc, a0, b0, ca, cb, kc);
            read_ops<WM, WN, 3>(smem, s, roff, rowA0, rowB0, a3, b3);
            mfmas<WM, WN, 1>(acc, a1, b1, ca, cb, kc);
            interleave<2 * WM * WN, 2 * (WM + WN), 0>();
            // this wave's reads of stage s and its loads of stage s + 1 are done; after the
            // barrier every wave's are, so stage s + 2 may load into stage s's buffers
            __builtin_amdgcn_s_waitcnt(FP4Q_LGKMCNT0);
            __builtin_amdgcn_s_waitcnt(FP4Q_VMCNT(T::WAIT));
            barrier_only();
            read_scales<WM, WN>(sbase, s + 1, scA, scB, na_, nb_);
            read_ops<WM, WN, 0>(smem, s + 1, roff, rowA0, rowB0, a0, b0);
            issue_stage<WM, WN, 1>(smem, bs, voff, soff, wave, s + 2, steps);
            mfmas<WM, WN, 2>(acc, a2, b2, ca, cb, kc);
            read_ops<WM, WN, 1>(smem, s + 1, roff, rowA0, rowB0, a1, b1);
            issue_stage<WM, WN, 2>(smem, bs, voff, soff, wave, s + 2, steps);
            mfmas<WM, WN, 3>(acc, a3, b3, ca, cb, kc);
            interleave<2 * WM * WN, 2 * (WM + WN) + (WM + WN + 1) / 2, LdsTile<WM, WN>::BATCH>();
        };
        int s = 0;
        for (; s + 2 < steps; s += 2) {
            stage(s, sa, sb, na, nb);
            stage(s + 1, na, nb, sa, sb);
        }
        stage(s, sa, sb, na, nb);   // s = steps - 2: stage steps - 1 has its scales in (na, nb)
        s = steps - 1;
        read_ops<WM, WN, 2>(smem, s, roff, rowA0, rowB0, a2, b2);
        read_ops<WM, WN, 3>(smem, s, roff, rowA0, rowB0, a3, b3);
        mfmas<WM, WN, 0>(acc, a0, b0, na, nb, kc);
        mfmas<WM, WN, 1>(acc, a1, b1, na, nb, kc);
        mfmas<WM, WN, 2>(acc, a2, b2, na, nb, kc);
        mfmas<WM, WN, 3>(acc, a3, b3, na, nb, kc);
    }
    // the loads issued past the last stage must land before the workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(FP4Q_VMCNT(0));
    if constexpr (QUANT != 0) {
        quantize_epilogue<WM, WN, QUANT == 2>(p, acc, smem, wave, lane, kc, r32, m0 + wm * 32 * WM,
                                              n0 + wn * 32 * WN);
        return;
    }

    // C: result r of MFMA tile (i, j) in this lane is row 32 i + 8 (r / 4) + 4 kc + r % 4, column
    // 32 j + r32 of the wave's quarter.  Stores go through a buffer resource whose range ends at
    // row M, and where a lane's column in tile j is at or past N, all of that tile's stores from
    // the lane are offset past the range, so the hardware drops every element outside C without
    // a test per element.
    constexpr int ESZ = BF16 ? 2 : 4;
    // the row stride passes through an opaque copy here, so that none of the
    // offsets below is computed ahead of the K loop and held in registers through it
    int ldcb = (int)(p.ldc * ESZ);
    asm volatile("" : "+s"(ldcb));
    const int64_t row0 = m0 + wm * 32 * WM, col0 = n0 + wn * 32 * WN;
    uint8_t* cw = reinterpret_cast<uint8_t*>(p.c) + (row0 * p.ldc + col0) * ESZ;
    const int64_t crange = p.M > row0 ? (p.M - row0) * p.ldc * ESZ : 0;
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(cw, (short)0, clamp31(crange), 0x00020000);
    if (p.staged && m0 + T::RA <= p.M && n0 + T::RB <= p.N) {
        // whole tile inside C, rows 16-byte aligned: each wave turns its quarter around in LDS,
        // half its rows at a time, and writes whole 16-byte pieces of rows
        constexpr int HR = 16 * WM;              // rows per half
        constexpr int PITCH = 32 * WN * ESZ;     // bytes per staged row
        constexpr int PIECES = HR * PITCH / 16;  // 16-byte pieces per half
        static_assert(PIECES % 64 == 0, "whole wave instructions per half");
        uint8_t* st = smem + wave * HR * PITCH;
        barrier_only();   // every wave is done with the K loop's LDS
        #pragma unroll
        for (int h = 0; h < 2; ++h) {
            #pragma unroll
            for (int i = 0; i < WM / 2; ++i)
                #pragma unroll
                for (int j = 0; j < WN; ++j)
                    #pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        uint8_t* d = st + (32 * i + 8 * (r >> 2) + 4 * kc + (r & 3)) * PITCH + (32 * j + r32) * ESZ;
                        const float v = acc[h * (WM / 2) + i][j][r];
                        if constexpr (BF16) {
                            const bf16x2 b = __builtin_convertvector((v2f){v, 0.0f}, bf16x2);
                            *reinterpret_cast<uint16_t*>(d) = (uint16_t)(__builtin_bit_cast(uint32_t, b) & 0xFFFFu);
                        } else {
                            *reinterpret_cast<float*>(d) = v;
                        }
                    }
            #pragma unroll
            for (int q = 0; q < PIECES / 64; ++q) {
                const int c = q * 64 + lane, row = c / (PITCH / 16), piece = c % (PITCH / 16);
                const v4u32 v = *reinterpret_cast<const v4u32*>(st + c * 16);
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, v), rc,
                                                       (h * HR + row) * ldcb + piece * 16, 0, 0);
            }
        }
        return;
    }
    int vlane[WN];
    #pragma unroll
    for (int j = 0; j < WN; ++j)
        vlane[j] = col0 + 32 * j + r32 < p.N ? 4 * kc * ldcb + (32 * j + r32) * ESZ : (int)0x80000000u;
    #pragma unroll
    for (int i = 0; i < WM; ++i)
        #pragma unroll
        for (int j = 0; j < WN; ++j)
            #pragma unroll
            for (int r = 0; r < 16; ++r)
                store_c<BF16>(rc, vlane[j] + (32 * i + 8 * (r >> 2) + (r & 3)) * ldcb, acc[i][j][r]);
}

// Consecutive workgroups go to different XCDs, so when the grid divides
// evenly, tiles are handed out XCD by XCD: the workgroups of one XCD then
// share operand rows in its L2.
__device__ __forceinline__ uint32_t xcd_tile(uint32_t remap) {
    uint32_t bid = blockIdx.x;
    if (remap) bid = (bid & 7) * (gridDim.x >> 3) + (bid >> 3);
    return bid;
}

constexpr uint32_t kGroupM = 4;   // row tiles per group of the tile order

// Tile (tm, tn) of the bid-th tile in the order that hands tiles out in groups
// of kGroupM row tiles, column by column within a group: the 8 kGroupM
// consecutive tiles an XCD runs at a time (4 x 8 of them for 256 x 192
// tiles) then read 4 row blocks of A and 8 of B, where a row-major order would
// read one or two of A and 32 of B, three times the bytes that reach its L2
// from memory per stage.
__device__ __forceinline__ void grouped_tile(uint32_t bid, uint32_t tiles_m, uint32_t tiles_n, uint32_t& tm,
                                             uint32_t& tn) {
    const uint32_t per = kGroupM * tiles_n;
    const uint32_t grp = bid / per, first = grp * kGroupM;
    const uint32_t rows = min(tiles_m - first, kGroupM);
    const uint32_t r = bid - grp * per;
    tm = first + r % rows;
    tn = r / rows;
}

template <int WM, int WN, bool BF16, int QUANT = 0>
__global__ __launch_bounds__(256) void k_gemm_mx_lds(const GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const uint32_t bid = xcd_tile(p.xcd_remap);
    uint32_t tm, tn;
    grouped_tile(bid, gridDim.x / p.tiles_n, p.tiles_n, tm, tn);
    gemm_tile<WM, WN, BF16, QUANT>(p, tm, tn, smem);
}

// Several products in one launch: the tiles of product i are workgroups
// tile_start[i] .. tile_start[i + 1] - 1.
template <int WM, int WN, bool BF16>
__global__ __launch_bounds__(256) void k_gemm_mx_lds_grouped(const GroupedGemmParams gp) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const uint32_t bid = xcd_tile(gp.xcd_remap);
    const uint32_t i = group_of<kMaxGemmGroup>(gp.tile_start, gp.n, bid);
    const GemmParams& p = gp.g[i];
    const uint32_t local = bid - gp.tile_start[i];
    const uint32_t tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
    gemm_tile<WM, WN, BF16>(p, tm, tn, smem);
}

template <int WM, int WN>
static hipError_t launch_lds(bool bf16_out, GemmParams p, hipStream_t s, int quant = 0) {
    using T = LdsTile<WM, WN>;
    const uint32_t tiles_m = (uint32_t)((p.M + T::RA - 1) / T::RA);
    p.tiles_n = (uint32_t)((p.N + T::RB - 1) / T::RB);
    const uint32_t g = tiles_m * p.tiles_n;
    p.xcd_remap = g % 8 == 0 ? 1u : 0u;
    const int esz = bf16_out ? 2 : 4;
    p.staged = ((uintptr_t)p.c & 15) == 0 && (p.ldc * esz) % 16 == 0 ? 1u : 0u;
    if (quant == 2) hipLaunchKernelGGL((k_gemm_mx_lds<WM, WN, true, 2>), dim3(g), dim3(256), T::LDS_BYTES, s, p);
    else if (quant) hipLaunchKernelGGL((k_gemm_mx_lds<WM, WN, true, 1>), dim3(g), dim3(256), T::LDS_BYTES, s, p);
    else if (bf16_out) hipLaunchKernelGGL((k_gemm_mx_lds<WM, WN, true>), dim3(g), dim3(256), T::LDS_BYTES, s, p);
    else hipLaunchKernelGGL((k_gemm_mx_lds<WM, WN, false>), dim3(g), dim3(256), T::LDS_BYTES, s, p);
    return hipGetLastError();
}

template <int WM, int WN>
static hipError_t launch_lds_grouped(bool bf16_out, GroupedGemmParams gp, hipStream_t s) {
    using T = LdsTile<WM, WN>;
    const int esz = bf16_out ? 2 : 4;
    gp.tile_start[0] = 0;
    for (uint32_t i = 0; i < gp.n; ++i) {
        GemmParams& p = gp.g[i];
        const uint32_t tiles_m = (uint32_t)((p.M + T::RA - 1) / T::RA);
        p.tiles_n = (uint32_t)((p.N + T::RB - 1) / T::RB);
        p.xcd_remap = 0;
        p.staged = ((uintptr_t)p.c & 15) == 0 && (p.ldc * esz) % 16 == 0 ? 1u : 0u;
        gp.tile_start[i + 1] = gp.tile_start[i] + tiles_m * p.tiles_n;
    }
    const uint32_t g = gp.tile_start[gp.n];
    if (g == 0) return hipSuccess;
    gp.xcd_remap = g % 8 == 0 ? 1u : 0u;
    if (bf16_out)
        hipLaunchKernelGGL((k_gemm_mx_lds_grouped<WM, WN, true>), dim3(g), dim3(256), T::LDS_BYTES, s, gp);
    else
        hipLaunchKernelGGL((k_gemm_mx_lds_grouped<WM, WN, false>), dim3(g), dim3(256), T::LDS_BYTES, s, gp);
    return hipGetLastError();
}

static bool main_path_ok(const GemmParams& p) {
    return p.K % 512 == 0 && p.K > 0 && p.K < (1ll << 24) && ((uintptr_t)p.as & 15) == 0 &&
           ((uintptr_t)p.bs & 15) == 0;
}

hipError_t launch_gemm_mx_grouped(bool bf16_out, const GroupedGemmParams& gp, hipStream_t s) {
    bool all_main = true;
    int64_t big = 0;
    for (uint32_t i = 0; i < gp.n; ++i) {
        all_main = all_main && main_path_ok(gp.g[i]);
        big += ((gp.g[i].M + 255) / 256) * ((gp.g[i].N + 191) / 192);
    }
    if (!all_main) {   // one launch per product
        for (uint32_t i = 0; i < gp.n; ++i) {
            const hipError_t e = launch_gemm_mx(bf16_out, gp.g[i], s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if (big >= 256) return launch_lds_grouped<4, 3>(bf16_out, gp, s);
    return launch_lds_grouped<2, 2>(bf16_out, gp, s);
}

bool gemm_quant_supported(const GemmParams& p) { return main_path_ok(p); }

hipError_t launch_gemm_mx_quant(const GemmParams& p, hipStream_t s) {
    const int q = p.qts ? 2 : 1;
    switch (gemm_config(p.M, p.N)) {
        case 2: return launch_lds<4, 4>(true, p, s, q);
        case 1: return launch_lds<4, 3>(true, p, s, q);
        default: return launch_lds<2, 2>(true, p, s, q);
    }
}

hipError_t launch_gemm_mx(bool bf16_out, const GemmParams& p, hipStream_t s) {
    // main path: K a multiple of 512 (whole stages and 16-byte aligned scale loads)
    if (main_path_ok(p)) {
        switch (gemm_config(p.M, p.N)) {
            case 2: return launch_lds<4, 4>(bf16_out, p, s);
            case 1: return launch_lds<4, 3>(bf16_out, p, s);
            default: return launch_lds<2, 2>(bf16_out, p, s);
        }
    }
    const bool scale4 = p.K % 128 == 0 && ((uintptr_t)p.as & 3) == 0 && ((uintptr_t)p.bs & 3) == 0;
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
