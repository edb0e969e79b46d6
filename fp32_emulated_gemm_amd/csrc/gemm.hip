// gemm.hip -- BF16x9 emulated SGEMM on gfx950 BF16 MFMA.
//
// Method (NVIDIA Technical Blog, "Unlocking Tensor Core Performance for
// Machine Learning Interatomic Potentials", Fig. 1 and its caption;
// discuss.pytorch.kr summary, section "Blackwell의 BF16x9"): each FP32 operand
// is split into x0 + 2^-8 x1 + 2^-16 x2; the nine products A_p B_q run on the
// BF16 matrix cores with FP32 accumulation; products of equal significance
// p + q share one of five band accumulators; the bands are recombined with
// weights 2^-8s, smallest band first.
//
// Two kernels share the tile, band and epilogue code:
//
// gemm_bf16x9_dma_kernel -- the main kernel, for B given as BF16 planes N x K
// (a linear layer's [out][in] weight, or FP32 B split once into a workspace)
// with K a multiple of 2 BK:
//   * persistent: one workgroup of 8 waves per CU walks 128 x 128 output
//     tiles (small grids: gemm_bf16x9_streamk_kernel, the same pipeline over
//     equal runs of (tile, K pair) units);
//   * each wave owns 64 x 32 of the tile: two 32 x 32 MFMA blocks, each with
//     NB band accumulators of 16 FP32 registers per lane
//     (v_mfma_f32_32x32x16_bf16);
//   * K advances in steps of BK = 32; the B planes of a step are copied
//     global -> LDS by buffer loads with LDS destination, two steps ahead,
//     into a ring of three buffers; A is loaded into registers two steps
//     ahead and split one step ahead, interleaved with the MFMAs;
//   * one LDS-only barrier per step; the next step's first fragments are read
//     right after it while the step's last MFMAs run;
//   * a tile's last two steps already load the next tile's first two.
//
// gemm_bf16x9_kernel -- the general kernel (FP32 B split in the kernel, K x N
// planes, N x K planes with any K or layout): one workgroup per tile, A and B
// staged through registers and split there, double-buffered LDS with one
// barrier per step, the K tail masked.
//
// Common to both:
//   * LDS A rows are 32 BF16 plus 8 BF16 of padding (80 bytes): the 128-bit
//     fragment reads of 16 consecutive rows then touch 64 distinct banks
//     (the DMA kernel's B rows are unpadded and XOR-swizzled instead);
//   * tile order: workgroups are dealt round-robin to the 8 XCDs, so the
//     tile index is remapped to give each XCD a contiguous run of tiles, in
//     groups of tile-rows so that concurrent tiles share A and B panels in the
//     XCD's L2;
//   * epilogue: per output, acc = 2^-32 S4; acc = fma(S3, 2^-24, acc);
//     acc = fma(S2, 2^-16, acc); acc = fma(S1, 2^-8, acc); C = acc + S0
//     (then the bias and the activation of the linear entry point).
// Edges: rows of A beyond M and columns of B beyond N are clamped to valid
// memory (their results are never stored); k beyond K is zero-filled.
#include <hip/hip_ext.h>

#include "split_device.hpp"
#include "launch.hpp"

namespace sgemm_emu_dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Launch the last kernel of a call.  With g.done set (a call that used the
// stream's workspace block), the event is tied to that kernel's completion, so
// the next user of the block can wait for it without a separate marker on the
// stream.
template <typename K>
static void launch_last(K kernel, dim3 grid, dim3 block, hipStream_t stream, const GemmArgs &g)
{
    if (g.done != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, nullptr, (hipEvent_t)g.done, 0, g);
    else
        hipLaunchKernelGGL(kernel, grid, block, 0, stream, g);
}

constexpr int BK = 32;
constexpr int KP = BK + 8;          // LDS row pitch in BF16 elements (80 bytes)
constexpr int KG = BK / 8;          // 8-wide k groups per row

template <int WAVES_M_, int WAVES_N_, int WTM_, int WTN_, bool SCHED_ = false, int VALU_PER_MFMA_ = 4,
          int DMA_TAIL_ = 6>
struct Cfg {
    static constexpr bool SCHED = SCHED_;     // explicit MFMA / LDS / VALU interleaving
    static constexpr int VALU_PER_MFMA = VALU_PER_MFMA_;
    static constexpr int DMA_TAIL = DMA_TAIL_; // MFMAs of a DMA step left to cover the next fragment reads
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int NT = 64 * WAVES;
    static constexpr int WTM = WTM_, WTN = WTN_;
    static constexpr int MI = WTM / 32, NI = WTN / 32;
    static constexpr int BM = WAVES_M * WTM, BN = WAVES_N * WTN;
    static constexpr int TILE = (BM + BN) * KP;                 // one component plane, A then B
    static constexpr int A_CHUNKS = BM * KG / NT;               // 8-element chunks of A per thread
    static constexpr int B_CHUNKS = BN * KG / NT;               // 8-element chunks of B per thread
    // 2-column x 4-k chunks of K x N planes (one dword = two columns per row).
    static constexpr int B_PAIRS = (BN / 2) * (BK / 4) / NT;
    static constexpr int B_SLOTS = (B_CHUNKS > 2 * B_PAIRS) ? B_CHUNKS : 2 * B_PAIRS;
    static_assert((BN / 2) * (BK / 4) % NT == 0, "K x N plane chunks not divisible among threads");
    static_assert(BM * KG % NT == 0 && BN * KG % NT == 0, "tile not divisible among threads");
    static_assert(NT % 16 == 0 && (BM % 16) == 0 && (BN % 16) == 0, "loader mapping");
};

using Cfg8 = Cfg<2, 4, 64, 32>;              // 8 waves, 2 per SIMD, 128 x 128 tile
using Cfg8S = Cfg<2, 4, 64, 32, true, 4, 4>; // same, staging interleaved with the MFMAs
using Cfg64S = Cfg<2, 2, 32, 32, true, 4, 4>; // 4 waves, 64 x 64 tile, two workgroups per CU (FP32 B, small grids)
using Cfg64S1 = Cfg<2, 2, 32, 32, true, 2, 4>; // same, for grids of at most one 64 x 64 tile per CU

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t lmin(int64_t a, int64_t b) { return a < b ? a : b; }

// Tile index v in [0, T) -> (tile_m, tile_n).  Consecutive v are dealt
// round-robin to the 8 XCDs, so v is remapped to give each XCD a contiguous
// run of tiles, and tiles run in groups of group_m tile-rows (column-major
// inside a group) so the tiles an XCD runs at once share A and B panels in
// its L2.
__device__ __forceinline__ void tile_of_index(int v, int T, int tiles_m, int tiles_n, int group_m, int &tm,
                                              int &tn)
{
    const int per = T >> 3, extra = T & 7, xcd = v & 7, idx = v >> 3;
    const int t = xcd * per + imin(xcd, extra) + idx;
    const int group_size = group_m * tiles_n;
    const int group = t / group_size;
    const int first_m = group * group_m;
    const int gm = imin(tiles_m - first_m, group_m);
    const int in = t - group * group_size;
    tm = first_m + in % gm;
    tn = in / gm;
}

// One tile per workgroup: the block index is the tile index.
__device__ __forceinline__ void tile_of_block(int tiles_m, int tiles_n, int group_m, int &tm, int &tn)
{
    tile_of_index((int)blockIdx.x, (int)gridDim.x, tiles_m, tiles_n, group_m, tm, tn);
}

// Chunk q of a tile side with `rows` rows (A: rows of A, B: columns of B) ->
// (row, k group).  Within each 64-lane wave, 16 consecutive lanes take 16
// consecutive rows of one k group, so both the global loads (4 lanes per
// 128-byte row segment) and the 128-bit LDS writes (16 rows x 80 bytes) are
// conflict-free.
__device__ __forceinline__ void chunk_rc(int q, int &row, int &kg)
{
    const int lane = q & 63, blk = q >> 6;
    row = blk * 16 + (lane & 15);
    kg = lane >> 4;
}

// ---------------------------------------------------------------- global loads
//
// All global loads are raw buffer loads.  Each K step gets fresh buffer
// descriptors (wave-uniform, so they live in scalar registers and are rebased
// with scalar adds) whose base sits at the step's first row / column, so the
// per-thread offsets are small 32-bit values shared across the three B planes.
// Descriptor sizes end at the last element the step may touch, so a stray
// offset reads zero instead of leaving the operand; the K tail is still masked
// explicitly (the scalar offset is not part of the hardware range check).

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_WORD3 = 0x00020000;   // raw, untyped buffer on gfx9-family GPUs

// Descriptor of `bytes` bytes at `base`.  Callers pass wave-uniform values;
// readfirstlane states that to the compiler, which otherwise may keep a
// value in vector registers and wrap every load in a loop over lanes.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes);
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    void *ub = (void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(n), RSRC_WORD3);
}

__device__ __forceinline__ float bload_f32(rsrc_t r, uint32_t off, uint32_t soff)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, (int)soff, 0));
}

__device__ __forceinline__ uint32_t bload_u32(rsrc_t r, uint32_t off, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, (int)soff, 0);
}

__device__ __forceinline__ uint32_t bload_u16(rsrc_t r, uint32_t off, uint32_t soff)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, (int)soff, 0);
}

__device__ __forceinline__ u32x4_t bload_u32x4(rsrc_t r, uint32_t off, uint32_t soff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, 0);
}

__device__ __forceinline__ void st_lds16(uint16_t *p, const uint32_t (&v)[4])
{
    *reinterpret_cast<u32x4_t *>(p) = u32x4_t{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ void st_lds8(uint16_t *p, const uint32_t (&v)[2])
{
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    *reinterpret_cast<u32x2_t *>(p) = u32x2_t{v[0], v[1]};
}

__device__ __forceinline__ bf16x8_t ld_frag(const uint16_t *p)
{
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(p));
}

// ---------------------------------------------------------------- staging

// One thread's share of one K step, held in registers between load and store.
template <class C, int BSRC>
struct Stage {
    float a[C::A_CHUNKS][8];
    float b[BSRC == B_FP32 ? C::B_CHUNKS : 1][8];
    uint32_t bn[BSRC == B_PLANES_NK ? C::B_CHUNKS : 1][3][4];
    uint32_t bk[BSRC == B_PLANES_KN ? C::B_PAIRS : 1][3][2][2];
};

// Per-thread byte offsets (relative to the step's descriptor bases) and LDS
// offsets, fixed for the whole tile.
template <class C, int BSRC>
struct Roles {
    uint32_t a_off[C::A_CHUNKS];
    int a_lds[C::A_CHUNKS], a_kg[C::A_CHUNKS];
    uint32_t b_off[C::B_SLOTS];
    int b_lds[C::B_SLOTS], b_kg[C::B_SLOTS];
    bool b_second_ok[C::B_PAIRS];
};

template <class C, int BSRC, int BVEC>
__device__ __forceinline__ void make_roles(Roles<C, BSRC> &R, const GemmArgs &g, int64_t m0, int64_t n0)
{
    const int tid = threadIdx.x;
#pragma unroll
    for (int c = 0; c < C::A_CHUNKS; ++c) {
        int row, kg;
        chunk_rc(c * C::NT + tid, row, kg);
        // rows past M re-read row M-1 (valid memory); their results are not stored
        const int64_t r = lmin(m0 + row, g.M - 1) - m0;
        R.a_off[c] = (uint32_t)((r * g.lda + kg * 8) * 4);
        R.a_lds[c] = row * KP + kg * 8;
        R.a_kg[c] = kg;
    }
    if constexpr (BSRC == B_FP32) {
        // thread -> (column, 8-wide k group): lanes run along n for coalesced loads.
#pragma unroll
        for (int c = 0; c < C::B_CHUNKS; ++c) {
            const int q = c * C::NT + tid, col = q % C::BN, kg = q / C::BN;
            const int64_t n = lmin(n0 + col, g.N - 1);
            R.b_off[c] = (uint32_t)(((int64_t)kg * 8 * g.ldb + n) * 4);
            R.b_lds[c] = (C::BM + col) * KP + kg * 8;
            R.b_kg[c] = kg;
        }
    } else if constexpr (BSRC == B_PLANES_NK) {
#pragma unroll
        for (int c = 0; c < C::B_CHUNKS; ++c) {
            int col, kg;
            chunk_rc(c * C::NT + tid, col, kg);
            const int64_t n = lmin(n0 + col, g.N - 1) - n0;
            R.b_off[c] = (uint32_t)((n * g.ldb + kg * 8) * 2);
            R.b_lds[c] = (C::BM + col) * KP + kg * 8;
            R.b_kg[c] = kg;
        }
    } else {
        // thread -> (column pair, 4-wide k group): lanes run along n.
#pragma unroll
        for (int c = 0; c < C::B_PAIRS; ++c) {
            const int q = c * C::NT + tid, pair = q % (C::BN / 2), kq = q / (C::BN / 2);
            const int64_t n = n0 + 2 * pair;
            // Clamp to valid memory; columns past N are discarded at the store.
            // With dword loads (N even) the pair must start on an even column.
            const int64_t nc = BVEC ? lmin(n, (g.N - 1) & ~(int64_t)1) : lmin(n, g.N - 1);
            R.b_off[c] = (uint32_t)(((int64_t)kq * 4 * g.ldb + nc) * 2);
            R.b_second_ok[c] = nc + 1 < g.N;
            R.b_lds[2 * c] = (C::BM + 2 * pair) * KP + kq * 4;
            R.b_lds[2 * c + 1] = (C::BM + 2 * pair + 1) * KP + kq * 4;
            R.b_kg[2 * c] = kq;
            R.b_kg[2 * c + 1] = kq;
        }
    }
}

// Load the K step starting at k0 into registers.  Every load is in bounds of
// its descriptor; elements with k >= K are fixed up by mask_stage:
//   * A and N x K planes run along k inside a row: past K they read the rest
//     of the row (or zero past the descriptor's end), so they are masked;
//   * FP32 B and K x N planes run along k across rows: the row offset is part
//     of the range-checked vector offset, so rows past K read as zero.
template <class C, int BSRC, bool AVEC, int BVEC>
__device__ __forceinline__ void load_stage(Stage<C, BSRC> &st, const Roles<C, BSRC> &R, const GemmArgs &g,
                                           int64_t m0, int64_t n0, int64_t k0)
{
    // A: base at (m0, k0); the descriptor ends at element (last row, K-1).
    {
        const int64_t rows = lmin((int64_t)C::BM, g.M - m0);
        const rsrc_t ra = make_rsrc(g.A + m0 * g.lda + k0, ((rows - 1) * g.lda + (g.K - k0)) * 4);
#pragma unroll
        for (int c = 0; c < C::A_CHUNKS; ++c) {
            float(&x)[8] = st.a[c];
            if (AVEC) {
                const u32x4_t v0 = bload_u32x4(ra, R.a_off[c], 0);
                const u32x4_t v1 = bload_u32x4(ra, R.a_off[c] + 16, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) { x[e] = __uint_as_float(v0[e]); x[4 + e] = __uint_as_float(v1[e]); }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = bload_f32(ra, R.a_off[c] + 4 * e, 0);
            }
        }
    }
    if constexpr (BSRC == B_FP32) {
        // base at row k0; the descriptor ends at element (K-1, N-1)
        const rsrc_t rb = make_rsrc(g.B + k0 * g.ldb, ((g.K - 1 - k0) * g.ldb + g.N) * 4);
        const uint32_t row_bytes = (uint32_t)(g.ldb * 4);
#pragma unroll
        for (int c = 0; c < C::B_CHUNKS; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) st.b[c][e] = bload_f32(rb, R.b_off[c] + e * row_bytes, 0);
    } else if constexpr (BSRC == B_PLANES_NK) {
        // base at (n0, k0); the descriptor ends at element (last column, K-1)
        const int64_t cols = lmin((int64_t)C::BN, g.N - n0);
        const int64_t bytes = ((cols - 1) * g.ldb + (g.K - k0)) * 2;
        const int64_t base = n0 * g.ldb + k0;
        const rsrc_t rr[3] = {make_rsrc(g.B0 + base, bytes), make_rsrc(g.B1 + base, bytes),
                              make_rsrc(g.B2 + base, bytes)};
#pragma unroll
        for (int c = 0; c < C::B_CHUNKS; ++c)
#pragma unroll
            for (int p = 0; p < 3; ++p) {
                if constexpr (BVEC == 1) {
                    const u32x4_t v = bload_u32x4(rr[p], R.b_off[c], 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) st.bn[c][p][i] = v[i];
                } else if constexpr (BVEC == 2) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) st.bn[c][p][i] = bload_u32(rr[p], R.b_off[c] + 4 * i, 0);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        st.bn[c][p][i] = bload_u16(rr[p], R.b_off[c] + 4 * i, 0) |
                                         (bload_u16(rr[p], R.b_off[c] + 4 * i + 2, 0) << 16);
                }
            }
    } else {
        // base at row k0; the descriptor ends at element (K-1, N-1)
        const int64_t bytes = ((g.K - 1 - k0) * g.ldb + g.N) * 2;
        const rsrc_t rr[3] = {make_rsrc(g.B0 + k0 * g.ldb, bytes), make_rsrc(g.B1 + k0 * g.ldb, bytes),
                              make_rsrc(g.B2 + k0 * g.ldb, bytes)};
        const uint32_t row_bytes = (uint32_t)(g.ldb * 2);
#pragma unroll
        for (int c = 0; c < C::B_PAIRS; ++c) {
#pragma unroll
            for (int p = 0; p < 3; ++p) {
                uint32_t r[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t off = R.b_off[c] + e * row_bytes;
                    if (BVEC) {
                        r[e] = bload_u32(rr[p], off, 0);
                    } else {
                        const uint32_t lo = bload_u16(rr[p], off, 0);
                        const uint32_t hi = R.b_second_ok[c] ? bload_u16(rr[p], off + 2, 0) : 0u;
                        r[e] = lo | (hi << 16);
                    }
                }
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    st.bk[c][p][0][i] = __builtin_amdgcn_perm(r[2 * i + 1], r[2 * i], 0x05040100u);  // column n
                    st.bk[c][p][1][i] = __builtin_amdgcn_perm(r[2 * i + 1], r[2 * i], 0x07060302u);  // column n+1
                }
            }
        }
    }
}

// Zero the staged elements whose k is >= K (only the last K step can have any).
template <class C, int BSRC>
__device__ __forceinline__ void mask_stage(Stage<C, BSRC> &st, const Roles<C, BSRC> &R, int64_t k0, int64_t K)
{
#pragma unroll
    for (int c = 0; c < C::A_CHUNKS; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (k0 + R.a_kg[c] * 8 + e >= K) st.a[c][e] = 0.0f;
    if constexpr (BSRC == B_PLANES_NK) {
#pragma unroll
        for (int c = 0; c < C::B_CHUNKS; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t k = k0 + R.b_kg[c] * 8 + 2 * i;
                const uint32_t keep = (k >= K) ? 0u : (k + 1 >= K) ? 0x0000FFFFu : 0xFFFFFFFFu;
#pragma unroll
                for (int p = 0; p < 3; ++p) st.bn[c][p][i] &= keep;
            }
    }
}

// Split the staged FP32 values and write the component tiles to LDS.  The
// split assumes finite inputs; the return value tells the caller whether this
// lane met an Inf or NaN and must run restage_special afterwards.
template <class C, int BSRC, bool RNE>
__device__ __forceinline__ bool store_stage(const Stage<C, BSRC> &st, const Roles<C, BSRC> &R, uint16_t *buf)
{
    uint32_t p0[4], p1[4], p2[4];
    bool special = false;
#pragma unroll
    for (int c = 0; c < C::A_CHUNKS; ++c) {
        special |= split8_packed_finite<RNE>(st.a[c], p0, p1, p2);
        st_lds16(buf + 0 * C::TILE + R.a_lds[c], p0);
        st_lds16(buf + 1 * C::TILE + R.a_lds[c], p1);
        st_lds16(buf + 2 * C::TILE + R.a_lds[c], p2);
    }
    if constexpr (BSRC == B_FP32) {
#pragma unroll
        for (int c = 0; c < C::B_CHUNKS; ++c) {
            special |= split8_packed_finite<RNE>(st.b[c], p0, p1, p2);
            st_lds16(buf + 0 * C::TILE + R.b_lds[c], p0);
            st_lds16(buf + 1 * C::TILE + R.b_lds[c], p1);
            st_lds16(buf + 2 * C::TILE + R.b_lds[c], p2);
        }
    } else if constexpr (BSRC == B_PLANES_NK) {
#pragma unroll
        for (int c = 0; c < C::B_CHUNKS; ++c)
#pragma unroll
            for (int p = 0; p < 3; ++p) st_lds16(buf + p * C::TILE + R.b_lds[c], st.bn[c][p]);
    } else {
#pragma unroll
        for (int c = 0; c < C::B_PAIRS; ++c)
#pragma unroll
            for (int p = 0; p < 3; ++p) {
                st_lds8(buf + p * C::TILE + R.b_lds[2 * c], st.bk[c][p][0]);
                st_lds8(buf + p * C::TILE + R.b_lds[2 * c + 1], st.bk[c][p][1]);
            }
    }
    return special;
}

// Rare path for a lane whose staged values included Inf or NaN: reload the
// same K step and rewrite its FP32-sourced component tiles with the full
// special-value split.  Runs before the barrier that publishes the tile.
template <class C, int BSRC, bool AVEC, int BVEC, bool RNE>
__device__ __forceinline__ void restage_special(const Roles<C, BSRC> &R, const GemmArgs &g, int64_t m0, int64_t n0,
                                             int64_t k0, uint16_t *buf)
{
    Stage<C, BSRC> st;
    load_stage<C, BSRC, AVEC, BVEC>(st, R, g, m0, n0, k0);
    if (k0 + BK > g.K) mask_stage<C, BSRC>(st, R, k0, g.K);
    uint32_t p0[4], p1[4], p2[4];
#pragma unroll
    for (int c = 0; c < C::A_CHUNKS; ++c) {
        split8_packed<RNE>(st.a[c], p0, p1, p2);
        st_lds16(buf + 0 * C::TILE + R.a_lds[c], p0);
        st_lds16(buf + 1 * C::TILE + R.a_lds[c], p1);
        st_lds16(buf + 2 * C::TILE + R.a_lds[c], p2);
    }
    if constexpr (BSRC == B_FP32) {
#pragma unroll
        for (int c = 0; c < C::B_CHUNKS; ++c) {
            split8_packed<RNE>(st.b[c], p0, p1, p2);
            st_lds16(buf + 0 * C::TILE + R.b_lds[c], p0);
            st_lds16(buf + 1 * C::TILE + R.b_lds[c], p1);
            st_lds16(buf + 2 * C::TILE + R.b_lds[c], p2);
        }
    }
}

// ---------------------------------------------------------------- kernel

template <class C, int NB>
struct Acc {
    f32x16_t v[C::MI][C::NI][NB];
};

template <class C>
struct Frags {
    bf16x8_t a[C::MI][3], b[C::NI][3];
};

template <class C>
__device__ __forceinline__ void read_frags(Frags<C> &f, const uint16_t *cur, int kk, int wm, int wn, int lane)
{
    const int frag_row = lane & 31, frag_k = kk + (lane >> 5) * 8;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
            f.a[i][c] = ld_frag(cur + c * C::TILE + (wm * C::WTM + i * 32 + frag_row) * KP + frag_k);
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
            f.b[j][c] = ld_frag(cur + c * C::TILE + (C::BM + wn * C::WTN + j * 32 + frag_row) * KP + frag_k);
    }
}

// The nine (or fewer) band products of one 16-wide k slice.
template <class C, int NB>
__device__ __forceinline__ void mfma_slice(Acc<C, NB> &acc, const Frags<C> &f)
{
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            if (p + q < NB) {
#pragma unroll
                for (int i = 0; i < C::MI; ++i)
#pragma unroll
                    for (int j = 0; j < C::NI; ++j)
                        acc.v[i][j][p + q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i][p], f.b[j][q],
                                                                                     acc.v[i][j][p + q], 0, 0, 0);
            }
        }
}

constexpr int products(int nb) { return nb >= 5 ? 9 : nb == 4 ? 8 : nb == 3 ? 6 : nb == 2 ? 3 : 1; }

// Global load instructions one thread issues per K step (see load_stage).
template <class C, int BSRC, bool AVEC, int BVEC>
constexpr int global_loads_per_stage()
{
    const int a = C::A_CHUNKS * (AVEC ? 2 : 8);
    const int b = BSRC == B_FP32 ? C::B_CHUNKS * 8
                : BSRC == B_PLANES_NK ? C::B_CHUNKS * 3 * (BVEC == 1 ? 1 : BVEC == 2 ? 4 : 8)
                : C::B_PAIRS * 3 * 4 * (BVEC ? 1 : 2);
    return a + b;
}

// One K step that also stages the next one.  Source order keeps the live
// ranges short (loads, slice 0, slice 1, split + LDS writes); with C::SCHED
// the scheduling groups below then pull the fragment reads of slice 1 under
// the MFMAs of slice 0, and the split arithmetic and LDS writes of the next
// step under the MFMAs of slice 1, so the matrix cores keep running while the
// next tile is staged.  The body is a single basic block.
template <class C, int NB, bool AVEC, int BSRC, int BVEC, bool RAGGED, bool RNE>
__device__ __forceinline__ void step_staging_next(Acc<C, NB> &acc, Stage<C, BSRC> &st, const Roles<C, BSRC> &R,
                                                  const GemmArgs &g, int64_t m0, int64_t n0, int64_t k_next,
                                                  const uint16_t *cur, uint16_t *nxt, int wm, int wn, int lane)
{
    load_stage<C, BSRC, AVEC, BVEC>(st, R, g, m0, n0, k_next);
    if constexpr (RAGGED) mask_stage<C, BSRC>(st, R, k_next, g.K);
    Frags<C> f;
    read_frags<C>(f, cur, 0, wm, wn, lane);
    mfma_slice<C, NB>(acc, f);
    read_frags<C>(f, cur, 16, wm, wn, lane);
    mfma_slice<C, NB>(acc, f);
    const bool special = store_stage<C, BSRC, RNE>(st, R, nxt);
    if constexpr (C::SCHED) {
        constexpr int NM = products(NB) * C::MI * C::NI;      // MFMAs per slice
        constexpr int NR = 3 * (C::MI + C::NI);                // fragment reads per slice
        constexpr int NLOAD = global_loads_per_stage<C, BSRC, AVEC, BVEC>();
        constexpr int NVALU = (BSRC == B_FP32) ? 2 * C::VALU_PER_MFMA : C::VALU_PER_MFMA;
        __builtin_amdgcn_sched_group_barrier(0x020, NLOAD, 0);  // next step's global loads first
        (void)NR;
#pragma unroll
        for (int i = 0; i < 2 * NM; ++i) {                      // MFMAs with the split in between
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i >= NM / 2) __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);
        }
    }
    if (__builtin_expect(special, 0)) restage_special<C, BSRC, AVEC, BVEC, RNE>(R, g, m0, n0, k_next, nxt);
}

// GELU in its exact form, 0.5 z (1 + erf(z / sqrt(2))), evaluated as
// 0.5 z erfc(-z / sqrt(2)): the same function, without the cancellation of
// 1 + erf(.) for negative z, so the relative error stays a few ulp.
__device__ __forceinline__ float gelu_erf(float z)
{
    return (0.5f * z) * erfcf(z * -0.70710678118654752f);
}

// Cache policy of the C stores: non-temporal (streamed past L2), so the
// output does not evict the A and B panels other tiles still read.
constexpr int kStreamingStore = 2;

// Recombine the bands smallest first, add the bias (if any), apply the
// activation (if any) and store the tile.  The stores are
// raw buffer stores through a descriptor that starts at the tile's first row
// and ends at element (last row of C inside the tile, N-1): rows past M fall
// outside it and are dropped by the hardware range check, so only the
// column test (fixed per lane) needs a branch.
// Bias of each of this lane's output columns, -0 where there is none (x + (-0)
// is x for every x, including -0 and NaN).  Loaded well before the epilogue
// so its latency never stalls the stores.
template <class C>
__device__ __forceinline__ void load_bias(float (&bv)[C::NI], const GemmArgs &g, int64_t n0, int wn, int lane)
{
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
        const int64_t col = n0 + wn * C::WTN + j * 32 + (lane & 31);
        bv[j] = (g.bias && col < g.N) ? g.bias[col] : -0.0f;
    }
}

// ACT: 0 none, 1 GELU; ACT = -1 writes the recombined K-slice result `slice`
// to the split-K partial buffer instead (no bias, no activation).
template <class C, int NB, int ACT>
__device__ __forceinline__ void store_c_act(const Acc<C, NB> &acc, const float (&bv)[C::NI], const GemmArgs &g,
                                            int64_t m0, int64_t n0, int wm, int wn, int lane, int slice = 0)
{
    const int64_t rows = lmin((int64_t)C::BM, g.M - m0);
    float *const dst = ACT < 0 ? g.partials + (int64_t)slice * g.M * g.ldp : g.C;
    const int64_t ld = ACT < 0 ? g.ldp : g.ldc;
    const rsrc_t rc = make_rsrc(dst + m0 * ld, ((rows - 1) * ld + g.N) * 4);
    // 128 rows of C fit 32-bit byte offsets (leading dimensions are limited)
    const uint32_t ldc4 = (uint32_t)ld * 4u;
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
        const int64_t col = n0 + wn * C::WTN + j * 32 + (lane & 31);
        if (col < g.N) {
            const float bval = bv[j];
            uint32_t lane_off = (uint32_t)col * 4u + (uint32_t)(wm * C::WTM + 4 * (lane >> 5)) * ldc4;
            // Opaque to the optimiser: otherwise it reassociates the 32 row
            // offsets below into tile-invariant values and keeps them all live.
            asm volatile("" : "+v"(lane_off));
#pragma unroll
            for (int i = 0; i < C::MI; ++i) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float v = 0.0f;
                    if constexpr (NB >= 5) v = 0x1p-32f * acc.v[i][j][4][r];
                    if constexpr (NB >= 4) v = __builtin_fmaf(acc.v[i][j][3][r], 0x1p-24f, v);
                    if constexpr (NB >= 3) v = __builtin_fmaf(acc.v[i][j][2][r], 0x1p-16f, v);
                    if constexpr (NB >= 2) v = __builtin_fmaf(acc.v[i][j][1][r], 0x1p-8f, v);
                    v = v + acc.v[i][j][0][r];
                    if constexpr (ACT >= 0) v = v + bval;
                    if constexpr (ACT == 1) v = gelu_erf(v);
                    const uint32_t row = (uint32_t)(i * 32 + 8 * (r >> 2) + (r & 3));
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rc, (int)(lane_off + row * ldc4), 0,
                                                          kStreamingStore);
                }
            }
        }
    }
}

// The epilogue with the activation chosen once per tile (a straight-line body
// per activation, rather than a test per element).
template <class C, int NB>
__device__ __forceinline__ void store_c(const Acc<C, NB> &acc, const float (&bv)[C::NI], const GemmArgs &g,
                                        int64_t m0, int64_t n0, int wm, int wn, int lane)
{
    if (g.act == 1) store_c_act<C, NB, 1>(acc, bv, g, m0, n0, wm, wn, lane);
    else store_c_act<C, NB, 0>(acc, bv, g, m0, n0, wm, wn, lane);
}

template <class C, int NB, bool AVEC, int BSRC, int BVEC, bool RNE>
__global__ __launch_bounds__(C::NT, 1) void gemm_bf16x9_kernel(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 3 * C::TILE];

    int tm, tn;
    tile_of_block(g.tiles_m, g.tiles_n, g.group_m, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

    Roles<C, BSRC> R;
    make_roles<C, BSRC, BVEC>(R, g, m0, n0);
    float bias[C::NI];
    load_bias<C>(bias, g, n0, wn, lane);

    Acc<C, NB> acc;
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
#pragma unroll
            for (int s = 0; s < NB; ++s) acc.v[i][j][s] = f32x16_t{};

    const int64_t nk = (g.K + BK - 1) / BK;

    Stage<C, BSRC> st;
    load_stage<C, BSRC, AVEC, BVEC>(st, R, g, m0, n0, 0);
    if (BK > g.K) mask_stage<C, BSRC>(st, R, 0, g.K);
    if (store_stage<C, BSRC, RNE>(st, R, lds)) restage_special<C, BSRC, AVEC, BVEC, RNE>(R, g, m0, n0, 0, lds);
    __syncthreads();

    // Steady state: every step but the last stages its successor.  Inside the
    // loop the successor is a full K step; a ragged last step is staged by
    // the one step after the loop, which masks k >= K.
    const int64_t nfull = g.K / BK;
    int64_t kt = 0;
    for (; kt + 2 <= nfull; ++kt) {
        const uint16_t *cur = lds + (kt & 1) * 3 * C::TILE;
        uint16_t *nxt = lds + ((kt + 1) & 1) * 3 * C::TILE;
        step_staging_next<C, NB, AVEC, BSRC, BVEC, false, RNE>(acc, st, R, g, m0, n0, (kt + 1) * BK, cur, nxt, wm, wn,
                                                         lane);
        __syncthreads();
    }
    if (kt + 1 < nk) {
        const uint16_t *cur = lds + (kt & 1) * 3 * C::TILE;
        uint16_t *nxt = lds + ((kt + 1) & 1) * 3 * C::TILE;
        step_staging_next<C, NB, AVEC, BSRC, BVEC, true, RNE>(acc, st, R, g, m0, n0, (kt + 1) * BK, cur, nxt, wm, wn,
                                                        lane);
        __syncthreads();
    }
    {
        const uint16_t *cur = lds + ((nk - 1) & 1) * 3 * C::TILE;
        Frags<C> f;
        read_frags<C>(f, cur, 0, wm, wn, lane);
        mfma_slice<C, NB>(acc, f);
        read_frags<C>(f, cur, 16, wm, wn, lane);
        mfma_slice<C, NB>(acc, f);
    }

    store_c<C, NB>(acc, bias, g, m0, n0, wm, wn, lane);
}

// ---------------------------------------------------------------- N x K planes through LDS DMA
//
// Specialisation for pre-split B in the N x K layout with K a multiple of
// 2 BK and 16-byte aligned planes (the layout of a linear layer's [out][in]
// weight).  B never passes through registers: each K step's three plane
// tiles are copied global -> LDS by 16-byte buffer loads with LDS
// destination (lane l lands at base + 16 l), two steps ahead, into a ring of
// three LDS buffers.  B tiles are unpadded (64-byte rows) with the 16-byte
// slot of k group kg of row r stored at slot kg ^ ((r >> 2) & 3), which keeps
// the fragment reads of 16 consecutive rows on 16 distinct bank groups.
// A keeps the register path but with two register sets, also two steps
// ahead, so the split of step kt+1 (interleaved with the MFMAs of step kt)
// never waits for a load issued in the same step.

constexpr int B_DMA_TILE = 128 * BK;   // BF16 elements of one plane tile (BN = 128 rows x 32 k)

template <class C>
struct DmaLayout {
    static constexpr int A_TILE = C::BM * KP;                    // one padded A component tile
    static constexpr int A_BYTES = 2 * 3 * A_TILE * 2;           // two buffers
    static constexpr int B_BYTES = 3 * 3 * B_DMA_TILE * 2;       // three buffers
    static constexpr int TOTAL = A_BYTES + B_BYTES;
    static constexpr int B_ROWS_PER_WAVE = 128 / C::WAVES;       // plane-tile rows one wave copies
    static constexpr int B_COPIES = B_ROWS_PER_WAVE / 16;        // 1 KB copies per plane and wave
    static_assert(C::BN == 128 && B_ROWS_PER_WAVE % 16 == 0, "plane tile rows split into 16-row copies");
};

// Vector-memory operations one thread issues per K step of the DMA pipeline.
template <class C, bool AVEC>
constexpr int dma_vmem_per_step()
{
    return 3 * DmaLayout<C>::B_COPIES + C::A_CHUNKS * (AVEC ? 2 : 8);
}

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations,
// then for the other waves.  Unlike __syncthreads() it does not wait for the
// wave's outstanding LDS-DMA copies (the step that follows issued them for
// later use); callers wait for the copies they need with wait_vmem_at_most.
// The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int bslot(int row, int kg) { return kg ^ ((row >> 2) & 3); }

// Copy one K step (BK columns) of a 128-row tile of three BF16 planes with k
// contiguous (N x K planes of B, or M x K planes of A), rows r0.. of
// `nrows`, global -> LDS: wave w copies tile rows RPW w .. RPW w + RPW - 1,
// 16 rows per copy, lane -> (row, 16-byte slot); rows past the operand
// re-read its last row (never used).  `buf` receives the three plane tiles,
// unpadded 64-byte rows with swizzled slots (bslot).
template <class C>
__device__ __forceinline__ void dma_plane_stage(const uint16_t *P0, const uint16_t *P1, const uint16_t *P2,
                                                int64_t ld, int64_t nrows, int64_t r0, int64_t k0, int64_t K,
                                                uint16_t *buf, int wave, int lane)
{
    typedef __attribute__((address_space(3))) void lds_void_t;
    constexpr int RPW = DmaLayout<C>::B_ROWS_PER_WAVE;
    const int64_t rows = lmin((int64_t)128, nrows - r0);
    const int64_t bytes = ((rows - 1) * ld + (K - k0)) * 2;
    const int64_t base = r0 * ld + k0;
    uint32_t off[DmaLayout<C>::B_COPIES];
#pragma unroll
    for (int d = 0; d < DmaLayout<C>::B_COPIES; ++d) {
        const int row = wave * RPW + d * 16 + (lane >> 2), kg = bslot(row, lane & 3);
        const int64_t n = lmin((int64_t)row, rows - 1);
        off[d] = (uint32_t)((n * ld + kg * 8) * 2);
    }
    const uint16_t *planes[3] = {P0, P1, P2};
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const rsrc_t r = make_rsrc(planes[p] + base, bytes);
#pragma unroll
        for (int d = 0; d < DmaLayout<C>::B_COPIES; ++d) {
            uint16_t *dst = buf + p * B_DMA_TILE + (wave * RPW + d * 16) * BK;   // wave-uniform 1 KB block
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, (int)off[d], 0, 0, 0);
        }
    }
}

template <class C>
__device__ __forceinline__ void dma_b_stage(const GemmArgs &g, int64_t n0, int64_t k0, uint16_t *bbuf, int wave,
                                            int lane)
{
    static_assert(C::BN == 128, "128-row plane tiles");
    dma_plane_stage<C>(g.B0, g.B1, g.B2, g.ldb, g.N, n0, k0, g.K, bbuf, wave, lane);
}

template <class C>
__device__ __forceinline__ void read_frags_dma(Frags<C> &f, const uint16_t *abuf, const uint16_t *bbuf, int kk,
                                               int wm, int wn, int lane)
{
    const int frag_row = lane & 31, kg = (kk >> 3) + (lane >> 5);
#pragma unroll
    for (int c = 0; c < 3; ++c) {
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
            f.a[i][c] = ld_frag(abuf + c * DmaLayout<C>::A_TILE + (wm * C::WTM + i * 32 + frag_row) * KP + kg * 8);
#pragma unroll
        for (int j = 0; j < C::NI; ++j) {
            const int row = wn * C::WTN + j * 32 + frag_row;
            f.b[j][c] = ld_frag(bbuf + c * B_DMA_TILE + row * BK + bslot(row, kg) * 8);
        }
    }
}

template <class C, bool AVEC>
__device__ __forceinline__ void load_a_stage(float (&a)[C::A_CHUNKS][8], const uint32_t (&a_off)[C::A_CHUNKS],
                                             const GemmArgs &g, int64_t m0, int64_t k0)
{
    const int64_t rows = lmin((int64_t)C::BM, g.M - m0);
    // A's own K (g.ka) bounds the descriptor; g.K may be the padded K of the B planes
    const rsrc_t ra = make_rsrc(g.A + m0 * g.lda + k0, ((rows - 1) * g.lda + (g.ka - k0)) * 4);
#pragma unroll
    for (int c = 0; c < C::A_CHUNKS; ++c) {
        if (AVEC) {
            const u32x4_t v0 = bload_u32x4(ra, a_off[c], 0);
            const u32x4_t v1 = bload_u32x4(ra, a_off[c] + 16, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e) { a[c][e] = __uint_as_float(v0[e]); a[c][4 + e] = __uint_as_float(v1[e]); }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) a[c][e] = bload_f32(ra, a_off[c] + 4 * e, 0);
        }
    }
}

// Elements of the staged A at k >= K (the last K step of an operand whose K
// is not a multiple of 2 BK, against zero-padded B planes) must be zero:
// their loads read the next row's values.  kvalid = K - (the step's first k).
template <class C, bool KTAIL>
__device__ __forceinline__ void mask_a_tail(float (&x)[8], const float (&a)[8], int c, int64_t kvalid)
{
    if constexpr (KTAIL) {
        int row, kg;
        chunk_rc(c * C::NT + threadIdx.x, row, kg);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (kg * 8 + e < kvalid) ? a[e] : 0.0f;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = a[e];
    }
}

template <class C, bool RNE, bool KTAIL>
__device__ __forceinline__ bool store_a_stage(const float (&a)[C::A_CHUNKS][8], const int (&a_lds)[C::A_CHUNKS],
                                              uint16_t *abuf, int64_t kvalid)
{
    uint32_t p0[4], p1[4], p2[4];
    bool special = false;
#pragma unroll
    for (int c = 0; c < C::A_CHUNKS; ++c) {
        float x[8];
        mask_a_tail<C, KTAIL>(x, a[c], c, kvalid);
        special |= split8_packed_finite<RNE>(x, p0, p1, p2);
        st_lds16(abuf + 0 * DmaLayout<C>::A_TILE + a_lds[c], p0);
        st_lds16(abuf + 1 * DmaLayout<C>::A_TILE + a_lds[c], p1);
        st_lds16(abuf + 2 * DmaLayout<C>::A_TILE + a_lds[c], p2);
    }
    return special;
}

template <class C, bool AVEC, bool RNE, bool KTAIL>
__device__ __forceinline__ void restage_a_special(const uint32_t (&a_off)[C::A_CHUNKS], const int (&a_lds)[C::A_CHUNKS],
                                                  const GemmArgs &g, int64_t m0, int64_t k0, uint16_t *abuf)
{
    float a[C::A_CHUNKS][8];
    load_a_stage<C, AVEC>(a, a_off, g, m0, k0);
    uint32_t p0[4], p1[4], p2[4];
#pragma unroll
    for (int c = 0; c < C::A_CHUNKS; ++c) {
        float x[8];
        mask_a_tail<C, KTAIL>(x, a[c], c, g.ka - k0);
        split8_packed<RNE>(x, p0, p1, p2);
        st_lds16(abuf + 0 * DmaLayout<C>::A_TILE + a_lds[c], p0);
        st_lds16(abuf + 1 * DmaLayout<C>::A_TILE + a_lds[c], p1);
        st_lds16(abuf + 2 * DmaLayout<C>::A_TILE + a_lds[c], p2);
    }
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (they complete in issue order), leaving the other counters unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmem_at_most()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Per-thread byte offsets of the A chunks of the tile starting at row m0
// (rows past M re-read row M-1; their results are not stored).
template <class C>
__device__ __forceinline__ void a_offsets(uint32_t (&a_off)[C::A_CHUNKS], const GemmArgs &g, int64_t m0)
{
#pragma unroll
    for (int c = 0; c < C::A_CHUNKS; ++c) {
        int row, kg;
        chunk_rc(c * C::NT + threadIdx.x, row, kg);
        const int64_t r = lmin(m0 + row, g.M - 1) - m0;
        a_off[c] = (uint32_t)((r * g.lda + kg * 8) * 4);
    }
}

// Where a K step's operands come from: tile origin, first k, and this
// thread's A offsets for that tile.
template <class C>
struct StepSrc {
    int64_t m0, n0, k0;
    int64_t kb;                  // first k of the work unit (its K range)
    uint32_t a_off[C::A_CHUNKS];
};

// MFMAs [FIRST, LAST) of one k slice, in the order of mfma_slice.
template <class C, int NB, int FIRST, int LAST>
__device__ __forceinline__ void mfma_slice_part(Acc<C, NB> &acc, const Frags<C> &f)
{
    int n = 0;
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            if (p + q < NB) {
#pragma unroll
                for (int i = 0; i < C::MI; ++i)
#pragma unroll
                    for (int j = 0; j < C::NI; ++j) {
                        if (n >= FIRST && n < LAST)
                            acc.v[i][j][p + q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                f.a[i][p], f.b[j][q], acc.v[i][j][p + q], 0, 0, 0);
                        ++n;
                    }
            }
        }
}

// One K step of the DMA pipeline.  On entry f0 holds the fragments of the
// step's first k slice (read after the previous barrier).  The step issues
// the B copy and the A loads of the step two ahead (`ld`, possibly the next
// tile's), reads the second slice's fragments into f1, runs the first slice,
// splits the A of the next step (`a_split`, loaded one step earlier; `sp`
// says where it came from, for the rare special-value path) into `abuf_next`,
// runs most of the second slice, waits for the next step's B copy, passes the
// barrier, reads the next step's first-slice fragments into f0, and finishes
// the second slice while those reads are in flight.  Steps past the end of K
// are harmless: their descriptors end at the operands' last elements, so they
// read zeros or data nobody consumes.
template <class C, int NB, bool AVEC, bool RNE, bool KTAIL>
__device__ __forceinline__ void dma_step(Acc<C, NB> &acc, Frags<C> &f0, Frags<C> &f1,
                                         float (&a_load)[C::A_CHUNKS][8], const float (&a_split)[C::A_CHUNKS][8],
                                         const StepSrc<C> &ld, const StepSrc<C> &sp, const int (&a_lds)[C::A_CHUNKS],
                                         const GemmArgs &g, const uint16_t *abuf, const uint16_t *bbuf,
                                         uint16_t *abuf_next, const uint16_t *bbuf_next, uint16_t *bbuf_ld, int wave,
                                         int wm, int wn, int lane)
{
    constexpr int NM = products(NB) * C::MI * C::NI;     // MFMAs per k slice
    constexpr int TAIL = C::DMA_TAIL < NM ? C::DMA_TAIL : NM;
    dma_b_stage<C>(g, ld.n0, ld.k0, bbuf_ld, wave, lane);
    load_a_stage<C, AVEC>(a_load, ld.a_off, g, ld.m0, ld.k0);
    read_frags_dma<C>(f1, abuf, bbuf, 16, wm, wn, lane);
    mfma_slice<C, NB>(acc, f0);
    const bool special = store_a_stage<C, RNE, KTAIL>(a_split, a_lds, abuf_next, g.ka - sp.k0);
    mfma_slice_part<C, NB, 0, NM - TAIL>(acc, f1);
    if constexpr (C::SCHED) {
        // a_split arrived during the previous step, so its split and LDS
        // writes can run under the MFMAs; the copies and loads go first.
#pragma unroll
        for (int i = 0; i < 2 * NM - TAIL; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
    }
    if (__builtin_expect(special, 0))
        restage_a_special<C, AVEC, RNE, KTAIL>(sp.a_off, a_lds, g, sp.m0, sp.k0, abuf_next);
    // The next step's B tile must have landed before the barrier; only the
    // copies and A loads issued at the top of this step may still be in
    // flight (vector-memory operations complete in order).
    wait_vmem_at_most<dma_vmem_per_step<C, AVEC>()>();
    lds_barrier();
    read_frags_dma<C>(f0, abuf_next, bbuf_next, 0, wm, wn, lane);
    mfma_slice_part<C, NB, NM - TAIL, NM>(acc, f1);
}

// Clear the accumulators with MFMAs of zero operands: one instruction per 16
// registers, on the matrix pipe that idles while the epilogue stores.
template <class C, int NB>
__device__ __forceinline__ void clear_acc(Acc<C, NB> &acc)
{
    const bf16x8_t z = {};
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
#pragma unroll
            for (int s = 0; s < NB; ++s)
                acc.v[i][j][s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(z, z, f32x16_t{}, 0, 0, 0);
}

// Work unit v (a tile) -> its origin; its K range starts at 0.
template <class C>
__device__ __forceinline__ void unit_src(StepSrc<C> &u, int v, int T, const GemmArgs &g)
{
    int tm, tn;
    tile_of_index(v, T, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
    u.m0 = (int64_t)tm * C::BM;
    u.n0 = (int64_t)tn * C::BN;
    u.kb = 0;
    u.k0 = 0;
    a_offsets<C>(u.a_off, g, u.m0);
}

// Persistent: one workgroup per CU walks tiles v = blockIdx.x, + gridDim.x, ...
// The last two K steps of a tile already load the next tile's first two, and
// the last one splits the next tile's first A step and reads its first
// fragments, so a tile's start costs no load latency and its C stores drain
// while the next tile computes.
template <class C, int NB, bool AVEC, bool RNE, bool KTAIL>
__global__ __launch_bounds__(C::NT, 1) void gemm_bf16x9_dma_kernel(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[DmaLayout<C>::TOTAL / 2];
    uint16_t *const a_base = lds;
    uint16_t *const b_base = lds + DmaLayout<C>::A_BYTES / 2;
    constexpr int A_BUF = 3 * DmaLayout<C>::A_TILE, B_BUF = 3 * B_DMA_TILE;

    const int T = g.tiles_m * g.tiles_n, G = (int)gridDim.x;
    const int units = T;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    // K is a multiple of 2 BK on this path: an even number of steps per tile
    const int64_t nk = g.K / BK;

    int a_lds[C::A_CHUNKS];
#pragma unroll
    for (int c = 0; c < C::A_CHUNKS; ++c) {
        int row, kg;
        chunk_rc(c * C::NT + threadIdx.x, row, kg);
        a_lds[c] = row * KP + kg * 8;
    }

    int v = (int)blockIdx.x;
    StepSrc<C> cur;                              // the work unit being computed
    unit_src<C>(cur, v, T, g);

    Acc<C, NB> acc;
    clear_acc<C, NB>(acc);

    float a_next[C::A_CHUNKS][8], a_cur[C::A_CHUNKS][8];
    Frags<C> f0, f1;

    // Prologue: steps 0 and 1 of the first tile in flight, step 0 staged and
    // its first-slice fragments read.
    dma_b_stage<C>(g, cur.n0, cur.kb, b_base, wave, lane);
    load_a_stage<C, AVEC>(a_cur, cur.a_off, g, cur.m0, cur.kb);
    dma_b_stage<C>(g, cur.n0, cur.kb + BK, b_base + B_BUF, wave, lane);
    load_a_stage<C, AVEC>(a_next, cur.a_off, g, cur.m0, cur.kb + BK);
    if (store_a_stage<C, RNE, KTAIL>(a_cur, a_lds, a_base, g.ka - cur.kb))
        restage_a_special<C, AVEC, RNE, KTAIL>(cur.a_off, a_lds, g, cur.m0, cur.kb, a_base);
    wait_vmem_at_most<dma_vmem_per_step<C, AVEC>()>();
    lds_barrier();
    read_frags_dma<C>(f0, a_base, b_base, 0, wm, wn, lane);

    int bs = 0;                                  // B ring slot of the current step
    for (;;) {
        float bias[C::NI];                       // issued now, needed by the tile's epilogue
        load_bias<C>(bias, g, cur.n0, wn, lane);
        // The next unit, or (none left) the current one again, whose steps
        // past its K slice then serve as harmless dummy loads.
        const int64_t vn = (int64_t)v + G;
        const bool has_next = vn < units;
        StepSrc<C> nxt = cur;
        if (has_next) unit_src<C>(nxt, (int)vn, T, g);

        // Two steps per trip keep the register sets static: an even step
        // splits a_next (its successor) and loads a_cur (two ahead); an odd
        // step the reverse.  The step count is even on this path, so A
        // buffer parity follows kt.
        for (int64_t kt = 0; kt < nk; kt += 2) {
            const bool last = kt + 2 >= nk;
            const bool roll = last && has_next;
            StepSrc<C> ld = roll ? nxt : cur;
            ld.k0 = roll ? nxt.kb : cur.kb + (kt + 2) * BK;
            StepSrc<C> sp = cur;
            sp.k0 = cur.kb + (kt + 1) * BK;
            const int b1 = bs == 2 ? 0 : bs + 1, b2 = b1 == 2 ? 0 : b1 + 1;
            dma_step<C, NB, AVEC, RNE, KTAIL>(acc, f0, f1, a_cur, a_next, ld, sp, a_lds, g, a_base, b_base + bs * B_BUF,
                                  a_base + A_BUF, b_base + b1 * B_BUF, b_base + b2 * B_BUF, wave, wm, wn, lane);

            ld.k0 += BK;
            if (last) {
                sp = nxt;
                sp.k0 = has_next ? nxt.kb : cur.kb + nk * BK;
            } else {
                sp.k0 += BK;
            }
            dma_step<C, NB, AVEC, RNE, KTAIL>(acc, f0, f1, a_next, a_cur, ld, sp, a_lds, g, a_base + A_BUF,
                                  b_base + b1 * B_BUF, a_base, b_base + b2 * B_BUF, b_base + bs * B_BUF, wave, wm,
                                  wn, lane);
            bs = b2;
        }

        store_c<C, NB>(acc, bias, g, cur.m0, cur.n0, wm, wn, lane);
        if (!has_next) break;
        clear_acc<C, NB>(acc);
        v = (int)vn;
        cur = nxt;
    }
    wait_vmem_at_most<0>();      // drain the copies issued past the end of K
}

#ifdef SGEMM_EMU_SERIAL_LDS
// Debug build only (SGEMM_EMU_SERIAL_LDS): the N x K plane GEMM with one LDS
// buffer per operand and a barrier on each side of every K step -- no copies in
// flight across a barrier, no ring, no fragment prefetch.  Same tiles, split,
// B copies, fragment reads and MFMA order as gemm_bf16x9_dma_kernel (k slice 0
// then k slice 1 of each step, products in mfma_slice order), so its results
// must equal the pipelined kernel's bit for bit.  One tile per workgroup.
template <class C, int NB, bool AVEC, bool RNE, bool KTAIL>
__global__ __launch_bounds__(C::NT, 1) void gemm_bf16x9_serial_kernel(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[3 * DmaLayout<C>::A_TILE + 3 * B_DMA_TILE];
    uint16_t *const abuf = lds;
    uint16_t *const bbuf = lds + 3 * DmaLayout<C>::A_TILE;
    const int T = g.tiles_m * g.tiles_n;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    int a_lds[C::A_CHUNKS];
#pragma unroll
    for (int c = 0; c < C::A_CHUNKS; ++c) {
        int row, kg;
        chunk_rc(c * C::NT + threadIdx.x, row, kg);
        a_lds[c] = row * KP + kg * 8;
    }
    StepSrc<C> cur;
    unit_src<C>(cur, (int)blockIdx.x, T, g);
    Acc<C, NB> acc;
    clear_acc<C, NB>(acc);
    Frags<C> f;
    for (int64_t k0 = 0; k0 < g.K; k0 += BK) {
        dma_b_stage<C>(g, cur.n0, k0, bbuf, wave, lane);
        float a[C::A_CHUNKS][8];
        load_a_stage<C, AVEC>(a, cur.a_off, g, cur.m0, k0);
        wait_vmem_at_most<0>();
        if (store_a_stage<C, RNE, KTAIL>(a, a_lds, abuf, g.ka - k0))
            restage_a_special<C, AVEC, RNE, KTAIL>(cur.a_off, a_lds, g, cur.m0, k0, abuf);
        __syncthreads();
        read_frags_dma<C>(f, abuf, bbuf, 0, wm, wn, lane);
        mfma_slice<C, NB>(acc, f);
        read_frags_dma<C>(f, abuf, bbuf, 16, wm, wn, lane);
        mfma_slice<C, NB>(acc, f);
        __syncthreads();
    }
    float bias[C::NI];
    load_bias<C>(bias, g, cur.n0, wn, lane);
    store_c<C, NB>(acc, bias, g, cur.m0, cur.n0, wm, wn, lane);
}
#endif

// ---------------------------------------------------------------- stream-K (partly filled grids)
//
// A grid whose 128 x 128 tiles leave CUs idle (fewer tiles than CUs, or a last
// wave of tiles that fills only part of the chip) can cut the work along K
// instead, where a cost model expects that to pay (gemm_streamk_grid): the T tiles x (K / 64)
// pairs of K steps form one sequence of P units (tile-major, K ascending
// inside a tile), and workgroup w of G takes units [w P / G, (w + 1) P / G):
// every CU gets the same number of MFMAs.  A workgroup's run covers the end of
// one tile, whole tiles, and the start of another; it walks its run from the
// end, so the pieces it shares with lower-numbered workgroups come last.
//   * a tile inside one run is stored as usual;
//   * a piece that does not hold the tile's last K pair (at most one per
//     workgroup: the first it computes) recombines its bands, writes the FP32
//     result to its own partial slot (128 x 128 floats at slot w) and
//     publishes it by setting flags[w] to this launch's epoch;
//   * the workgroup holding the tile's last K pair recombines its own piece,
//     waits for the flags of the lower workgroups that hold the tile's earlier
//     pieces (already done: they computed those pieces first), adds their
//     partials in K order and then its own, then the bias and activation, and
//     stores the tile.
// Each piece runs the method on its K range (five band sums, recombined
// smallest first); the pieces' FP32 results are added in K order: a fixed
// order for a given shape and CU count.  Waits point only at lower-numbered
// workgroups, which the dispatcher starts first, and every wait is bounded: a
// piece that never arrives turns its tile into NaN instead of hanging.
//
// Where the tiles divide evenly enough, the sequence is cut into 8 domains,
// one per XCD: the dispatcher deals workgroups to the XCDs in turn, so the
// workgroups w = d (mod 8) share XCD d's L2, and domain d gives them its own
// block of tiles (groups of tile-rows, column-major inside a group); the
// same rules then hold inside each domain.  The partial slots and flags are
// written and read with system-coherent cache policy, because the L2 caches
// of the XCDs are not coherent with each other.

constexpr int SK_TILE = 128 * 128;                 // floats of one partial slot
constexpr int kStreamkGroupRows = 4;               // tile-rows per group of the stream-K order
constexpr uint32_t SK_SPIN_LIMIT = 1u << 24;       // bounded wait (about a second)

// One piece of a workgroup's run: where its steps load from (StepSrc) and
// what it is within its tile.
template <class C>
struct SkPiece {
    StepSrc<C> s;
    int64_t nk;          // K steps of the piece (an even number)
    uint32_t t;          // tile index inside the domain
    bool full;           // the whole tile
    bool last;           // holds the tile's last K pair
};

// The stream-K index arithmetic is 32-bit: the launcher keeps units x
// workgroups below 2^32, so every product below fits.
__device__ __forceinline__ uint32_t sk_owner_of(uint32_t p, uint32_t P, uint32_t G) { return ((p + 1) * G - 1) / P; }

// Tile index v of the stream-K order -> (tile_m, tile_n): groups of group_m
// tile-rows, column-major inside a group, so a domain's consecutive tiles form
// a block that shares A and B panels.
__device__ __forceinline__ void sk_tile(uint32_t v, const GemmArgs &g, uint32_t &tm, uint32_t &tn)
{
    const uint32_t group_size = (uint32_t)g.group_m * (uint32_t)g.tiles_n;
    const uint32_t group = v / group_size, in = v - group * group_size;
    const uint32_t first_m = group * (uint32_t)g.group_m;
    const uint32_t gm = (uint32_t)imin(g.tiles_m - (int)first_m, g.group_m);
    tn = in / gm;
    tm = first_m + (in - tn * gm);
}

// Piece i of this workgroup's run, counted from the run's end; t_first is the
// domain's first tile.
template <class C>
__device__ __forceinline__ void sk_piece(SkPiece<C> &q, uint32_t i, uint32_t pb, uint32_t pe, uint32_t ppt,
                                         uint32_t t_first, const GemmArgs &g)
{
    const uint32_t t = (pe - 1) / ppt - i;
    const uint32_t pa = t * ppt > pb ? t * ppt : pb;
    const uint32_t pz = (t + 1) * ppt < pe ? (t + 1) * ppt : pe;
    q.t = t;
    uint32_t tm, tn;
    sk_tile(t_first + t, g, tm, tn);
    q.s.m0 = (int64_t)tm * C::BM;
    q.s.n0 = (int64_t)tn * C::BN;
    q.s.kb = (int64_t)(pa - t * ppt) * 2 * BK;
    q.s.k0 = q.s.kb;
    q.nk = (int64_t)(pz - pa) * 2;
    q.full = pa == t * ppt && pz == (t + 1) * ppt;
    q.last = pz == (t + 1) * ppt;
    a_offsets<C>(q.s.a_off, g, q.s.m0);
}

// The five-band recombination of one output (smallest band first).
template <class C, int NB>
__device__ __forceinline__ float recombine(const Acc<C, NB> &acc, int i, int j, int r)
{
    float v = 0.0f;
    if constexpr (NB >= 5) v = 0x1p-32f * acc.v[i][j][4][r];
    if constexpr (NB >= 4) v = __builtin_fmaf(acc.v[i][j][3][r], 0x1p-24f, v);
    if constexpr (NB >= 3) v = __builtin_fmaf(acc.v[i][j][2][r], 0x1p-16f, v);
    if constexpr (NB >= 2) v = __builtin_fmaf(acc.v[i][j][1][r], 0x1p-8f, v);
    return v + acc.v[i][j][0][r];
}

// Byte offset of this lane's first output inside a 128 x 128 partial slot;
// output (i, j, r) lies sk_slot_step(i, j, r) bytes further.  The base is made
// opaque to the optimiser, which would otherwise keep all 32 offsets live
// through the whole kernel.
template <class C>
__device__ __forceinline__ uint32_t sk_slot_base(int wm, int wn, int lane)
{
    uint32_t b = (uint32_t)(((wm * C::WTM + 4 * (lane >> 5)) * 128 + wn * C::WTN + (lane & 31)) * 4);
    asm volatile("" : "+v"(b));
    return b;
}

__device__ __forceinline__ constexpr uint32_t sk_slot_step(int i, int j, int r)
{
    return (uint32_t)(((i * 32 + 8 * (r >> 2) + (r & 3)) * 128 + j * 32) * 4);
}

// Cache policy of the partial slots and flags: system-coherent (SC0 | SC1),
// so the stores write through and the loads bypass the caches of the XCD
// that issues them (the L2 caches of the eight XCDs are not coherent with
// each other).  This replaces release/acquire fences at device scope, which
// would write back or invalidate a whole L2 cache.
constexpr int kCoherent = 1 | 16;

// A piece without the tile's last pair: write the recombined result to slot w,
// then publish it: every wave waits until its stores are acknowledged, then
// thread 0 sets the flag.
template <class C, int NB>
__device__ __forceinline__ void sk_publish(const Acc<C, NB> &acc, const GemmArgs &g, int w, int wm, int wn, int lane)
{
    const rsrc_t rs = make_rsrc(g.partials + (int64_t)w * SK_TILE, (int64_t)SK_TILE * 4);
    const uint32_t base = sk_slot_base<C>(wm, wn, lane);
#pragma unroll
    for (int j = 0; j < C::NI; ++j)
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(recombine<C, NB>(acc, i, j, r)), rs,
                                                      (int)(base + sk_slot_step(i, j, r)), 0, kCoherent);
    wait_vmem_at_most<0>();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(g.sk_flags + w, g.sk_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// The piece with the tile's last pair: wait for the workgroups [w0, w) that
// hold the tile's earlier pieces, add their partials in K order, then this
// piece's own result, the bias and the activation; store the tile.
template <class C, int NB, int ACT>
__device__ __forceinline__ void sk_finish(const Acc<C, NB> &acc, const float (&bv)[C::NI], const GemmArgs &g,
                                          int64_t m0, int64_t n0, int64_t w0, int w, int D, int wm, int wn, int lane)
{
    // This piece's own result first, pinned so that it is not recomputed
    // later: the band accumulators die here, which leaves the registers for
    // whole batches of partial loads.
    float own[C::MI][C::NI][16];
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                own[i][j][r] = recombine<C, NB>(acc, i, j, r);
                asm volatile("" : "+v"(own[i][j][r]));
            }
    __shared__ int sk_ok;
    if (threadIdx.x == 0) {
        int ok = 1;
        for (int64_t u = w0; u < w && ok; u += D) {
            uint32_t n = 0;
            while (__hip_atomic_load(g.sk_flags + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != g.sk_epoch) {
                if (++n == SK_SPIN_LIMIT) { ok = 0; break; }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        sk_ok = ok;
    }
    __syncthreads();
    const bool ok = sk_ok != 0;
    // The earlier pieces' sum, in K order (this runs at the very end of the
    // kernel, when no later piece's data is held in registers).
    float sum[C::MI][C::NI][16];
    for (int64_t u = w0; u < w; u += D) {
        const rsrc_t rs = make_rsrc(g.partials + u * SK_TILE, (int64_t)SK_TILE * 4);
        const uint32_t base = sk_slot_base<C>(wm, wn, lane);
        float p[C::MI][C::NI][16];
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
            for (int j = 0; j < C::NI; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    p[i][j][r] = __uint_as_float(
                        __builtin_amdgcn_raw_buffer_load_b32(rs, (int)(base + sk_slot_step(i, j, r)), 0, kCoherent));
        // the whole slot's loads in flight before the first add
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < C::MI; ++i)
#pragma unroll
            for (int j = 0; j < C::NI; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) sum[i][j][r] = u == w0 ? p[i][j][r] : sum[i][j][r] + p[i][j][r];
    }
    const int64_t rows = lmin((int64_t)C::BM, g.M - m0);
    const rsrc_t rc = make_rsrc(g.C + m0 * g.ldc, ((rows - 1) * g.ldc + g.N) * 4);
    const uint32_t ldc4 = (uint32_t)g.ldc * 4u;
#pragma unroll
    for (int j = 0; j < C::NI; ++j) {
        const int64_t col = n0 + wn * C::WTN + j * 32 + (lane & 31);
        if (col < g.N) {
            uint32_t lane_off = (uint32_t)col * 4u + (uint32_t)(wm * C::WTM + 4 * (lane >> 5)) * ldc4;
            asm volatile("" : "+v"(lane_off));
#pragma unroll
            for (int i = 0; i < C::MI; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = w0 < w ? sum[i][j][r] + own[i][j][r] : own[i][j][r];
                    x = x + bv[j];
                    if constexpr (ACT == 1) x = gelu_erf(x);
                    if (!ok) x = __builtin_nanf("");
                    const uint32_t row = (uint32_t)(i * 32 + 8 * (r >> 2) + (r & 3));
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rc, (int)(lane_off + row * ldc4), 0,
                                                          kStreamingStore);
                }
        }
    }
}

// The DMA kernel's pipeline over a stream-K run: the same steps, B copies,
// A split, MFMA order and per-piece band recombination.
template <class C, int NB, bool AVEC, bool RNE, bool KTAIL>
__global__ __launch_bounds__(C::NT, 1) void gemm_bf16x9_streamk_kernel(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[DmaLayout<C>::TOTAL / 2];
    uint16_t *const a_base = lds;
    uint16_t *const b_base = lds + DmaLayout<C>::A_BYTES / 2;
    constexpr int A_BUF = 3 * DmaLayout<C>::A_TILE, B_BUF = 3 * B_DMA_TILE;

    // workgroup w is number j of the Gd workgroups of domain d, which owns
    // tiles [t_first, t_first + Td) of the stream-K order
    const uint32_t T = (uint32_t)g.tiles_m * (uint32_t)g.tiles_n, G = gridDim.x, w = blockIdx.x;
    const bool xcd = g.sk_domains == 8;
    const uint32_t D = xcd ? 8 : 1, d = xcd ? w & 7 : 0, j = xcd ? w >> 3 : w, Gd = xcd ? G >> 3 : G;
    const uint32_t t_first = xcd ? d * T >> 3 : 0, Td = xcd ? ((d + 1) * T >> 3) - t_first : T;
    const uint32_t ppt = (uint32_t)(g.K / (2 * BK));     // K pairs per tile
    const uint32_t P = Td * ppt;
    const uint32_t pb = j * P / Gd, pe = (j + 1) * P / Gd;  // this workgroup's units (at least two)
    const uint32_t npieces = (pe - 1) / ppt - pb / ppt + 1;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

    int a_lds[C::A_CHUNKS];
#pragma unroll
    for (int c = 0; c < C::A_CHUNKS; ++c) {
        int row, kg;
        chunk_rc(c * C::NT + threadIdx.x, row, kg);
        a_lds[c] = row * KP + kg * 8;
    }

    SkPiece<C> cur;
    sk_piece<C>(cur, 0, pb, pe, ppt, t_first, g);

    Acc<C, NB> acc;
    clear_acc<C, NB>(acc);
    float a_next[C::A_CHUNKS][8], a_cur[C::A_CHUNKS][8];
    Frags<C> f0, f1;

    dma_b_stage<C>(g, cur.s.n0, cur.s.kb, b_base, wave, lane);
    load_a_stage<C, AVEC>(a_cur, cur.s.a_off, g, cur.s.m0, cur.s.kb);
    dma_b_stage<C>(g, cur.s.n0, cur.s.kb + BK, b_base + B_BUF, wave, lane);
    load_a_stage<C, AVEC>(a_next, cur.s.a_off, g, cur.s.m0, cur.s.kb + BK);
    if (store_a_stage<C, RNE, KTAIL>(a_cur, a_lds, a_base, g.ka - cur.s.kb))
        restage_a_special<C, AVEC, RNE, KTAIL>(cur.s.a_off, a_lds, g, cur.s.m0, cur.s.kb, a_base);
    wait_vmem_at_most<dma_vmem_per_step<C, AVEC>()>();
    lds_barrier();
    read_frags_dma<C>(f0, a_base, b_base, 0, wm, wn, lane);

    int bs = 0;
    for (uint32_t i = 0;; ++i) {
        float bias[C::NI];
        load_bias<C>(bias, g, cur.s.n0, wn, lane);
        const bool has_next = i + 1 < npieces;
        SkPiece<C> nxt = cur;
        if (has_next) sk_piece<C>(nxt, i + 1, pb, pe, ppt, t_first, g);
        for (int64_t kt = 0; kt < cur.nk; kt += 2) {
            const bool last = kt + 2 >= cur.nk;
            const bool roll = last && has_next;
            StepSrc<C> ld = roll ? nxt.s : cur.s;
            ld.k0 = roll ? nxt.s.kb : cur.s.kb + (kt + 2) * BK;
            StepSrc<C> sp = cur.s;
            sp.k0 = cur.s.kb + (kt + 1) * BK;
            const int b1 = bs == 2 ? 0 : bs + 1, b2 = b1 == 2 ? 0 : b1 + 1;
            dma_step<C, NB, AVEC, RNE, KTAIL>(acc, f0, f1, a_cur, a_next, ld, sp, a_lds, g, a_base, b_base + bs * B_BUF,
                                              a_base + A_BUF, b_base + b1 * B_BUF, b_base + b2 * B_BUF, wave, wm, wn,
                                              lane);
            ld.k0 += BK;
            if (last) {
                sp = nxt.s;
                sp.k0 = has_next ? nxt.s.kb : cur.s.kb + cur.nk * BK;
            } else {
                sp.k0 += BK;
            }
            dma_step<C, NB, AVEC, RNE, KTAIL>(acc, f0, f1, a_next, a_cur, ld, sp, a_lds, g, a_base + A_BUF,
                                              b_base + b1 * B_BUF, a_base, b_base + b2 * B_BUF, b_base + bs * B_BUF,
                                              wave, wm, wn, lane);
            bs = b2;
        }
        if (!has_next) break;
        // an earlier piece: a whole tile, or the first piece of the run (the
        // start of a tile whose last pair a higher workgroup holds)
        if (cur.full) store_c<C, NB>(acc, bias, g, cur.s.m0, cur.s.n0, wm, wn, lane);
        else sk_publish<C, NB>(acc, g, (int)w, wm, wn, lane);
        clear_acc<C, NB>(acc);
        cur = nxt;
    }
    // The run's last piece.  Only it can hold the last pair of a tile shared
    // with lower workgroups (runs are walked from their end), so the wait and
    // the sum happen here, with no later piece's data left in registers.
    wait_vmem_at_most<0>();      // drain the copies issued past the end of the run
    float bias[C::NI];
    load_bias<C>(bias, g, cur.s.n0, wn, lane);
    if (cur.full) {
        store_c<C, NB>(acc, bias, g, cur.s.m0, cur.s.n0, wm, wn, lane);
    } else if (!cur.last) {
        sk_publish<C, NB>(acc, g, (int)w, wm, wn, lane);
    } else {
        const int64_t w0 = (int64_t)(sk_owner_of(cur.t * ppt, P, Gd) * D + d);
        if (g.act == 1) sk_finish<C, NB, 1>(acc, bias, g, cur.s.m0, cur.s.n0, w0, (int)w, (int)D, wm, wn, lane);
        else sk_finish<C, NB, 0>(acc, bias, g, cur.s.m0, cur.s.n0, w0, (int)w, (int)D, wm, wn, lane);
    }
}

// ---------------------------------------------------------------- both operands as planes
//
// A given as three BF16 planes M x K (lda) like B's N x K planes (ldb), K a
// multiple of 2 BK, 16-byte aligned planes.  Nothing is split in the kernel:
// both operands' tiles are copied global -> LDS by buffer loads with LDS
// destination, two steps ahead, into two rings of three buffers (144 KB), in
// the swizzled layout of dma_plane_stage.  One K step: copy the step two
// ahead, read the second slice's fragments, run the first slice, most of the
// second, wait for the next step's copies, pass the barrier, read the next
// step's first fragments and finish the second slice.  Same tiles, persistent
// order, MFMA order and epilogue as gemm_bf16x9_dma_kernel, so the result is
// bitwise that of the kernels that split A themselves.
template <class C>
__device__ __forceinline__ void read_frags_planes(Frags<C> &f, const uint16_t *abuf, const uint16_t *bbuf, int kk,
                                                  int wm, int wn, int lane)
{
    const int frag_row = lane & 31, kg = (kk >> 3) + (lane >> 5);
#pragma unroll
    for (int c = 0; c < 3; ++c) {
#pragma unroll
        for (int i = 0; i < C::MI; ++i) {
            const int row = wm * C::WTM + i * 32 + frag_row;
            f.a[i][c] = ld_frag(abuf + c * B_DMA_TILE + row * BK + bslot(row, kg) * 8);
        }
#pragma unroll
        for (int j = 0; j < C::NI; ++j) {
            const int row = wn * C::WTN + j * 32 + frag_row;
            f.b[j][c] = ld_frag(bbuf + c * B_DMA_TILE + row * BK + bslot(row, kg) * 8);
        }
    }
}

template <class C, int NB>
__global__ __launch_bounds__(C::NT, 1) void gemm_bf16x9_planes_kernel(GemmArgs g)
{
    static_assert(C::BM == 128 && C::BN == 128, "128-row plane tiles");
    constexpr int BUF = 3 * B_DMA_TILE;                      // one ring buffer: three plane tiles
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 3 * BUF];
    uint16_t *const a_base = lds;
    uint16_t *const b_base = lds + 3 * BUF;
    constexpr int NV = 2 * 3 * DmaLayout<C>::B_COPIES;       // copies one thread issues per K step
    constexpr int NM = products(NB) * C::MI * C::NI;          // MFMAs per k slice
    constexpr int TAIL = C::DMA_TAIL < NM ? C::DMA_TAIL : NM;

    const int T = g.tiles_m * g.tiles_n, G = (int)gridDim.x;
    const int units = T;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const int64_t nk = g.K / BK;

    int v = (int)blockIdx.x;
    StepSrc<C> cur;                              // the work unit being computed
    unit_src<C>(cur, v, T, g);
    auto copy = [&](const StepSrc<C> &u, int64_t k0, int slot) {
        dma_plane_stage<C>(g.A0, g.A1, g.A2, g.lda, g.M, u.m0, k0, g.K, a_base + slot * BUF, wave, lane);
        dma_plane_stage<C>(g.B0, g.B1, g.B2, g.ldb, g.N, u.n0, k0, g.K, b_base + slot * BUF, wave, lane);
    };

    Acc<C, NB> acc;
    clear_acc<C, NB>(acc);
    Frags<C> f0, f1;

    // Prologue: steps 0 and 1 in flight, step 0 landed, its first fragments read.
    copy(cur, cur.kb, 0);
    copy(cur, cur.kb + BK, 1);
    wait_vmem_at_most<NV>();
    lds_barrier();
    read_frags_planes<C>(f0, a_base, b_base, 0, wm, wn, lane);

    int bs = 0;                                  // ring slot of the current step
    for (;;) {
        float bias[C::NI];                       // issued now, needed by the unit's epilogue
        load_bias<C>(bias, g, cur.n0, wn, lane);
        // The next unit, or (none left) the current one again, whose steps
        // past its K slice then serve as harmless dummy copies.
        const int64_t vn = (int64_t)v + G;
        const bool has_next = vn < units;
        StepSrc<C> nxt = cur;
        if (has_next) unit_src<C>(nxt, (int)vn, T, g);
        for (int64_t kt = 0; kt < nk; ++kt) {
            const int b1 = bs == 2 ? 0 : bs + 1, b2 = b1 == 2 ? 0 : b1 + 1;
            if (kt + 2 < nk || !has_next) copy(cur, cur.kb + (kt + 2) * BK, b2);
            else copy(nxt, nxt.kb + (kt + 2 - nk) * BK, b2);
            read_frags_planes<C>(f1, a_base + bs * BUF, b_base + bs * BUF, 16, wm, wn, lane);
            mfma_slice<C, NB>(acc, f0);
            mfma_slice_part<C, NB, 0, NM - TAIL>(acc, f1);
            // the next step's tiles must have landed; only this step's copies may be in flight
            wait_vmem_at_most<NV>();
            lds_barrier();
            read_frags_planes<C>(f0, a_base + b1 * BUF, b_base + b1 * BUF, 0, wm, wn, lane);
            mfma_slice_part<C, NB, NM - TAIL, NM>(acc, f1);
            bs = b1;
        }
        store_c<C, NB>(acc, bias, g, cur.m0, cur.n0, wm, wn, lane);
        if (!has_next) break;
        clear_acc<C, NB>(acc);
        v = (int)vn;
        cur = nxt;
    }
    wait_vmem_at_most<0>();      // drain the copies issued past the end of K
}

// ---------------------------------------------------------------- split-K reduction

// C = act(sum over K slices of the slices' recombined results + bias), per
// element, adding the slices in slice order.
// Workgroups walk rows, threads walk a row's columns (no per-element division).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g)
{
    const int64_t plane = g.M * g.ldp;
    for (int64_t r = blockIdx.x; r < g.M; r += gridDim.x) {
        for (int64_t c = threadIdx.x; c < g.N; c += blockDim.x) {
            const float *p = g.partials + r * g.ldp + c;
            float v = p[0];
            for (int sl = 1; sl < g.splits; ++sl) v += p[(int64_t)sl * plane];
            v = v + (g.bias ? g.bias[c] : -0.0f);
            if (g.act == 1) v = gelu_erf(v);
            g.C[r * g.ldc + c] = v;
        }
    }
}

// Domains of a stream-K grid of G workgroups over T tiles of ppt K pairs.
// Workgroup w runs on XCD w % 8 (the dispatcher deals workgroups to the XCDs
// in turn), so 8 domains, domain d holding workgroups w = d (mod 8) and tile
// block d of the stream-K order, keep each block's A and B panels in one L2.
// Taken when every workgroup still gets two K pairs and the largest block is
// within 10 % of an even share of the tiles; otherwise one domain.
static int64_t streamk_domains(int64_t T, int64_t ppt, int64_t G)
{
    if (G % 8 != 0 || T < 8) return 1;
    if (T / 8 * ppt < 2 * (G / 8)) return 1;
    if ((T + 7) / 8 * 80 > T * 11) return 1;
    return 8;
}

// Stream-K against the persistent kernel, in K-pair times per CU: the
// persistent kernel needs ceil(T / G) whole tiles of ppt pairs; stream-K needs
// ceil(T ppt / G) pairs plus the publication, wait and sum of the cut tiles,
// which measured about kStreamkFixPairs pair times (6144 x 256 x 1024,
// 3072 x 1536 x 1024, 8192 x 640 x 1024, 6144 x 768 x 512, 2560^2 x 1024 and
// 4096 x 2048 x 512 on 256 CUs: stream-K 21-24 % faster on grids of 1.1-1.3
// waves of tiles with K = 1024, even at 1.56 waves, 11 % slower at 2 full
// waves).  Stream-K is taken where the model expects it 10 % faster.
constexpr int64_t kStreamkFixPairs = 6;
constexpr int64_t kStreamkMaxPieces = 8;               // per tile: the last piece adds the others' slots one by one

int gemm_streamk_grid(int64_t M, int64_t N, int64_t K, int num_cus)
{
#ifdef SGEMM_EMU_SERIAL_LDS
    (void)M; (void)N; (void)K; (void)num_cus;
    return 0;                                          // the debug build has no stream-K
#endif
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    if (K % (2 * BK) != 0 || tiles == 0) return 0;
    const int64_t ppt = K / (2 * BK), units = tiles * ppt;
    const int64_t G0 = num_cus > 8 ? num_cus & ~7 : 8;
    int64_t G = G0;
    if (units < 2 * G) G = units / 2;                  // at least two K pairs per workgroup
    if (G > kStreamkMaxPieces * tiles) G = kStreamkMaxPieces * tiles;
    if (G < 2) return 0;
    const int64_t t_persistent = (tiles + G0 - 1) / G0 * ppt;
    const int64_t t_streamk = (units + G - 1) / G + kStreamkFixPairs;
    if (t_streamk * 10 >= t_persistent * 9) return 0;
    if (units * G >= ((int64_t)1 << 32)) return 0;     // the kernel's index arithmetic is 32-bit
    return (int)G;
}

int gemm_streamk_pieces(int64_t M, int64_t N, int64_t K, int grid)
{
    if (grid <= 0) return 1;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128), ppt = K / (2 * BK);
    const int64_t D = streamk_domains(tiles, ppt, grid), G = grid / D;
    int64_t most = 1;
    for (int64_t d = 0; d < D; ++d) {
        const int64_t Td = (d + 1) * tiles / D - d * tiles / D, P = Td * ppt;
        for (int64_t t = 0; t < Td; ++t) {
            const int64_t first = ((t * ppt + 1) * G - 1) / P, last = (((t + 1) * ppt) * G - 1) / P;
            if (last - first + 1 > most) most = last - first + 1;
        }
    }
    return (int)most;
}

// FP32 B on a partly filled grid: the one-pass kernel on 64 x 64 tiles (B
// split inside each tile, nothing in a workspace, LDS for two workgroups per
// CU) against what 128 x 128 tiles would run -- one pass per tile (the kernel
// that splits B itself, or the N x K plane kernel after a split of B), or,
// where `streamk` allows it, stream-K on split planes.  Costs in K-pair times
// of a 128 x 128 tile on one CU, in twentieths: a 64 x 64 tile's K pair
// measured half of that on a CU of its own and 0.65 beside a second one
// (512^3, 768^3, 1024^3, 1024 x 1024 x 512, 2048 x 512 x 512,
// 1280 / 1536 / 2048 x 1024 x 1024, 4096 x 512 x 1024, 6144 x 256 x 1024 and
// 512 x 512 x 4096 on 256 CUs); stream-K as in gemm_streamk_grid.  Taken where
// the model expects the 64 x 64 tiles 10 % faster: measured 7-90 % faster
// there, and where it declines (256^2 x 1024, 512^2 x 2048 and x 4096,
// 1024^2 x 2048, 2560 x 1024 x 512, 3072 x 1024 x 1024, 3072 x 1536 x 1024)
// the other path was 3-150 % faster.  Four 64 x 64 tiles cost 1.3 times one
// 128 x 128 tile once the grid fills the CUs, so full grids never take them.
bool gemm_tile64_pays(int64_t M, int64_t N, int64_t K, int num_cus, bool streamk)
{
    const int64_t kpad = (K + 2 * BK - 1) / (2 * BK) * (2 * BK), ppt = kpad / (2 * BK);
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    const int64_t G0 = num_cus > 8 ? num_cus & ~7 : 8;
    int64_t t_other = (tiles + G0 - 1) / G0 * ppt;
    const int G = streamk ? gemm_streamk_grid(M, N, kpad, num_cus) : 0;
    if (G > 0) t_other = (tiles * ppt + G - 1) / G + kStreamkFixPairs;
    const int64_t tiles64 = ((M + 63) / 64) * ((N + 63) / 64);
    const int64_t t_tile64 = ppt * (tiles64 <= G0 ? 10 : 13 * ((tiles64 + 2 * G0 - 1) / (2 * G0)));
    return t_tile64 * 10 <= 20 * t_other * 9;
}

static int group_rows(int tiles_n, int num_cus);

// ---------------------------------------------------------------- native FP32 (performant strategy)
//
// The pages' "performant" strategy uses the emulation only where it expects
// a speed-up over the platform's native FP32 GEMM (NVIDIA blog, section
// "BF16x9 on NVIDIA Blackwell GPUs", Fig. 4; discuss.pytorch.kr summary,
// "PyTorch에서 직접 써 보려면").  This is the library's own native path: the
// FP32 matrix instruction v_mfma_f32_32x32x2_f32, one FP32 accumulator per
// output, no split.
//
// One workgroup per (tile, K slice); waves as in Cfg, each (MI x 32) x (NI x 32)
// of accumulators.  K advances in steps of NBK k (32, or 16 with element
// loads), double-buffered in LDS and loaded NLA steps ahead into registers:
//   * A rows hold NBK k values plus 4 of padding (144 or 80 bytes): 16
//     consecutive rows read with 128-bit loads touch 64 distinct banks;
//   * B rows (one k each) hold the tile's BN columns plus 4 of padding, so
//     the two half-waves reading k and k + 8 land on disjoint banks.
// Within each 16 k of a step, half-wave h (lanes 32h..32h+31) feeds
// k = 8h + kk to the kk-th MFMA: the instruction's two k rows come from k and
// k + 8, so each lane reads its eight A values of the 16 with two 128-bit
// loads.  Every k < K is multiplied in exactly once, in an order the bound
// allows.

// K per step and register stages: with 128-bit loads 32 k and two stages
// ahead (against 16 k and four: 768^3 37.4 -> 43.0 TFLOP/s, 1024^3 68.0 ->
// 77.3, 1024 x 1024 x 512 59.4 -> 66.9, 6144 x 256 x 1024 71.9 -> 76.6, the
// larger grids unchanged); with element loads 16 k and four stages (32 k
// measured 10.2 -> 8.0 TFLOP/s on 333 x 444 x 555).
template <bool VEC>
struct NativeSteps {
    static constexpr int NBK = VEC ? 32 : 16;   // k per step
    static constexpr int NLA = VEC ? 2 : 4;     // steps loaded ahead (register stages)
};

template <class C, int NBK>
struct NativeLayout {
    static constexpr int NAP = NBK + 4;                   // A row pitch in LDS (floats)
    static constexpr int BNP = C::BN + 4;                 // B row pitch in LDS (floats)
    static constexpr int A_FLOATS = C::BM * NAP;
    static constexpr int B_FLOATS = NBK * BNP;
    static constexpr int STAGE = A_FLOATS + B_FLOATS;
    static constexpr int A_VECS = C::BM * (NBK / 4) / C::NT;   // 16-byte A chunks per thread and step
    static constexpr int B_VECS = NBK * (C::BN / 4) / C::NT;   // 16-byte B chunks per thread and step
    static_assert(C::BM * (NBK / 4) % C::NT == 0 && NBK * (C::BN / 4) % C::NT == 0, "loader mapping");
};

template <class C, int NBK>
struct NativeStage {
    float a[NativeLayout<C, NBK>::A_VECS][4];
    float b[NativeLayout<C, NBK>::B_VECS][4];
};

// Thread -> A chunk (row, 4-wide k group): 16 consecutive lanes take 16 rows of
// one k group (conflict-free 128-bit LDS writes at the 80-byte pitch); a wave
// covers 16 rows x 4 k groups, the waves run through the tile's row blocks.
template <class C>
__device__ __forceinline__ void native_a_chunk(int q, int &row, int &kg)
{
    constexpr int ROW_BLOCKS = C::BM / 16;
    const int lane = q & 63, blk = q >> 6;
    row = (blk % ROW_BLOCKS) * 16 + (lane & 15);
    kg = (lane >> 4) + 4 * (blk / ROW_BLOCKS);
}

// Load one step (k0 .. k0 + 15) of A and B into registers.  VEC: 128-bit
// loads (16-byte aligned operands, leading dimensions and K / N multiples of
// 4), else one dword at a time.  A past K reads the next row's values and is
// masked by the caller; B rows past K and A, B beyond the operands read zero
// or values whose outputs are never stored.
template <class C, bool VEC, int NBK>
__device__ __forceinline__ void native_load(NativeStage<C, NBK> &st, const GemmArgs &g, int64_t m0, int64_t n0,
                                            int64_t k0)
{
    using L = NativeLayout<C, NBK>;
    const int tid = threadIdx.x;
    {
        const int64_t rows = lmin((int64_t)C::BM, g.M - m0);
        const rsrc_t ra = make_rsrc(g.A + m0 * g.lda + k0, ((rows - 1) * g.lda + (g.K - k0)) * 4);
#pragma unroll
        for (int c = 0; c < L::A_VECS; ++c) {
            int row, kg;
            native_a_chunk<C>(c * C::NT + tid, row, kg);
            const int64_t r = lmin((int64_t)row, rows - 1);
            const uint32_t off = (uint32_t)((r * g.lda + kg * 4) * 4);
            if (VEC) {
                const u32x4_t v = bload_u32x4(ra, off, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) st.a[c][e] = __uint_as_float(v[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) st.a[c][e] = bload_f32(ra, off + 4 * e, 0);
            }
        }
    }
    {
        // base at row k0; the descriptor ends at element (K-1, N-1)
        const rsrc_t rb = make_rsrc(g.B + k0 * g.ldb, ((g.K - 1 - k0) * g.ldb + g.N) * 4);
#pragma unroll
        for (int c = 0; c < L::B_VECS; ++c) {
            const int q = c * C::NT + tid, col = (q % (C::BN / 4)) * 4, k = q / (C::BN / 4);
            const int64_t n = lmin(n0 + col, (g.N - 1) & ~(int64_t)3);
            const uint32_t off = (uint32_t)(((int64_t)k * g.ldb + (VEC ? n : n0 + col)) * 4);
            if (VEC) {
                const u32x4_t v = bload_u32x4(rb, off, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) st.b[c][e] = __uint_as_float(v[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) st.b[c][e] = bload_f32(rb, off + 4 * e, 0);
            }
        }
    }
}

template <class C, int NBK>
__device__ __forceinline__ void native_store(const NativeStage<C, NBK> &st, float *buf, int64_t kvalid)
{
    using L = NativeLayout<C, NBK>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int c = 0; c < L::A_VECS; ++c) {
        int row, kg;
        native_a_chunk<C>(c * C::NT + tid, row, kg);
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (kg * 4 + e < kvalid) ? st.a[c][e] : 0.0f;
        *reinterpret_cast<u32x4_t *>(buf + row * L::NAP + kg * 4) =
            u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
    }
#pragma unroll
    for (int c = 0; c < L::B_VECS; ++c) {
        const int q = c * C::NT + tid, col = (q % (C::BN / 4)) * 4, k = q / (C::BN / 4);
        *reinterpret_cast<u32x4_t *>(buf + L::A_FLOATS + k * L::BNP + col) =
            u32x4_t{__float_as_uint(st.b[c][0]), __float_as_uint(st.b[c][1]), __float_as_uint(st.b[c][2]),
                    __float_as_uint(st.b[c][3])};
    }
}

template <class C, int NBK>
__device__ __forceinline__ void native_step(Acc<C, 1> &acc, const float *buf, int wm, int wn, int lane)
{
    using L = NativeLayout<C, NBK>;
    const int h = lane >> 5, r = lane & 31;
#pragma unroll
    for (int kb = 0; kb < NBK; kb += 16) {
        float a[C::MI][8];
#pragma unroll
        for (int i = 0; i < C::MI; ++i) {
            const float *p = buf + (wm * C::WTM + i * 32 + r) * L::NAP + kb + 8 * h;
            const u32x4_t v0 = *reinterpret_cast<const u32x4_t *>(p);
            const u32x4_t v1 = *reinterpret_cast<const u32x4_t *>(p + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { a[i][e] = __uint_as_float(v0[e]); a[i][4 + e] = __uint_as_float(v1[e]); }
        }
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            float b[C::NI];
#pragma unroll
            for (int j = 0; j < C::NI; ++j)
                b[j] = buf[L::A_FLOATS + (kb + 8 * h + kk) * L::BNP + wn * C::WTN + j * 32 + r];
#pragma unroll
            for (int i = 0; i < C::MI; ++i)
#pragma unroll
                for (int j = 0; j < C::NI; ++j)
                    acc.v[i][j][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][kk], b[j], acc.v[i][j][0], 0, 0, 0);
        }
    }
}

template <class C, bool VEC>
__global__ __launch_bounds__(C::NT, 2) void gemm_f32_native_kernel(GemmArgs g)
{
    constexpr int NBK = NativeSteps<VEC>::NBK, NLA = NativeSteps<VEC>::NLA;
    using L = NativeLayout<C, NBK>;
    __shared__ __attribute__((aligned(16))) float lds[2 * L::STAGE];
    int tm, tn;
    tile_of_index((int)blockIdx.x, (int)gridDim.x, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    // K slice of this workgroup (split-K): steps [s0, s1)
    const int64_t nsteps = (g.K + NBK - 1) / NBK;
    const int64_t per = (nsteps + g.splits - 1) / g.splits;
    const int64_t s0 = (int64_t)blockIdx.y * per, s1 = lmin(nsteps, s0 + per);

    Acc<C, 1> acc;
#pragma unroll
    for (int i = 0; i < C::MI; ++i)
#pragma unroll
        for (int j = 0; j < C::NI; ++j) acc.v[i][j][0] = f32x16_t{};

    if (s0 < s1) {
        // A ring of NLA register stages: the loads of step t + NLA go out while
        // step t is computed, so each step's loads have NLA - 1 steps of MFMA
        // work to arrive before they are written to LDS (one step of lead
        // leaves these short K steps waiting on memory latency).
        // The loads and LDS writes are unconditional, so every wait for a
        // stage counts only the NLA - 1 stages loaded after it: a load past
        // the slice re-reads its last step and is never stored for use, and
        // the LDS write after the last step goes to a buffer no step reads.
        NativeStage<C, NBK> st[NLA];
#pragma unroll
        for (int r = 0; r < NLA; ++r)
            native_load<C, VEC, NBK>(st[r], g, m0, n0, lmin(s0 + r, s1 - 1) * NBK);
        native_store<C, NBK>(st[0], lds, g.K - s0 * NBK);
        __syncthreads();
        for (int64_t s = s0; s < s1; s += NLA) {
#pragma unroll
            for (int r = 0; r < NLA; ++r) {
                const int64_t t = s + r;          // the step computed now; its data is in LDS
                if (t >= s1) break;
                const float *cur = lds + ((t - s0) & 1) * L::STAGE;
                float *nxt = lds + ((t - s0 + 1) & 1) * L::STAGE;
                native_load<C, VEC, NBK>(st[r], g, m0, n0, lmin(t + NLA, s1 - 1) * NBK);
                native_step<C, NBK>(acc, cur, wm, wn, lane);
                native_store<C, NBK>(st[(r + 1) % NLA], nxt, g.K - (t + 1) * NBK);
                __syncthreads();
            }
        }
    }
    float bias[C::NI];
    load_bias<C>(bias, g, n0, wn, lane);
    if (g.splits > 1) store_c_act<C, 1, -1>(acc, bias, g, m0, n0, wm, wn, lane, (int)blockIdx.y);
    else store_c<C, 1>(acc, bias, g, m0, n0, wm, wn, lane);
}

using CfgN128 = Cfg<2, 2, 64, 64>;    // 4 waves, 128 x 128 tile
using CfgN64 = Cfg<2, 2, 32, 32>;     // 4 waves, 64 x 64 tile

bool native_vec(const float *A, int64_t lda, const float *B, int64_t ldb, int64_t K, int64_t N)
{
    return aligned(A, 16) && aligned(B, 16) && lda % 4 == 0 && ldb % 4 == 0 && K % 4 == 0 && N % 4 == 0;
}

template <class C>
static hipError_t launch_native_cfg(const GemmArgs &args, int splits, hipStream_t stream)
{
    GemmArgs g = args;
    g.tiles_m = (int)((g.M + C::BM - 1) / C::BM);
    g.tiles_n = (int)((g.N + C::BN - 1) / C::BN);
    g.group_m = group_rows(g.tiles_n, g.num_cus);
    g.splits = splits;
    const bool vec = native_vec(g.A, g.lda, g.B, g.ldb, g.K, g.N);
    const dim3 grid((unsigned)((int64_t)g.tiles_m * g.tiles_n), (unsigned)splits), block(C::NT);
    GemmArgs gk = g;
    if (splits > 1) gk.done = nullptr;          // the reduction is the last kernel
    if (vec) launch_last(gemm_f32_native_kernel<C, true>, grid, block, stream, gk);
    else launch_last(gemm_f32_native_kernel<C, false>, grid, block, stream, gk);
    if (splits > 1) {
        const int64_t blocks = g.M < (int64_t)g.num_cus * 8 ? g.M : (int64_t)g.num_cus * 8;   // rows
        launch_last(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), stream, g);
    }
    return hipGetLastError();
}

NativePlan native_plan(int64_t M, int64_t N, int64_t K, int num_cus, bool vec)
{
    const int NBK = vec ? NativeSteps<true>::NBK : NativeSteps<false>::NBK;
    NativePlan p{};
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    if (t128 >= num_cus) {
        p.tile = 128;
        p.splits = 1;
        return p;
    }
    const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64);
    p.tile = 64;
    p.splits = 1;
    // small grids: K slices of at least 8 steps until about one workgroup per
    // CU (the slices' sum costs a second launch), and on to two per CU where a
    // slice would still be longer than 64 steps.  Measured against two per CU
    // throughout: 1024 x 1024 x 512 45.7 -> 62.2 TFLOP/s, 2048 x 512 x 512
    // 45.2 -> 63.5, 1024^3 65.3 -> 71.0, 1024 x 512 x 4096 unchanged at 82.6
    // (it keeps four slices), with 16-k steps; the same counts of the 32-k
    // steps are what the figures above NativeSteps were measured with.
    const int64_t nsteps = (K + NBK - 1) / NBK;
    auto grow = [&](int64_t per_cu) {
        while (p.splits < 16 && t64 * (p.splits + 1) <= per_cu * (int64_t)num_cus && nsteps / (p.splits + 1) >= 8)
            ++p.splits;
    };
    grow(1);
    if (nsteps / p.splits > 64) grow(2);
    return p;
}

hipError_t launch_native(const GemmArgs &args, const NativePlan &plan, hipStream_t stream)
{
    if (plan.splits > 1 && args.partials == nullptr) return hipErrorInvalidValue;
    if (plan.tile == 128) return launch_native_cfg<CfgN128>(args, plan.splits, stream);
    return launch_native_cfg<CfgN64>(args, plan.splits, stream);
}

// ---------------------------------------------------------------- K == 0

__global__ __launch_bounds__(256) void zero_kernel(float *__restrict__ C, int64_t ldc, int64_t M, int64_t N,
                                                   const float *__restrict__ bias, int act)
{
    for (int64_t r = blockIdx.x; r < M; r += gridDim.x) {
        for (int64_t c = threadIdx.x; c < N; c += blockDim.x) {
            float v = bias ? 0.0f + bias[c] : 0.0f;
            if (act == 1) v = gelu_erf(v);
            C[r * ldc + c] = v;
        }
    }
}

hipError_t launch_zero(int64_t M, int64_t N, float *C, int64_t ldc, const float *bias, int act, int num_cus,
                       hipStream_t stream)
{
    const int64_t blocks = M < (int64_t)num_cus * 8 ? M : (int64_t)num_cus * 8;   // rows
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, C, ldc, M, N, bias, act);
    return hipGetLastError();
}

// ---------------------------------------------------------------- dispatch

// Tile-rows per group.  An XCD runs about num_cus / 8 consecutive tiles at
// once.  A narrow tile grid (at least 4 whole tile-rows in that window) runs
// row by row (groups of one row), so the column tiles that read an A row
// panel are neighbours and run together; wider grids use groups of 8 rows,
// which share both A and B panels.
static int group_rows(int tiles_n, int num_cus)
{
    const int per_xcd = num_cus >= 8 ? num_cus / 8 : 1;
    return tiles_n * 4 <= per_xcd ? 1 : 8;
}

template <class C, int NB, bool AVEC, int BSRC, bool RNE>
static void launch_cfg_b(const GemmArgs &g, int bvec, hipStream_t stream)
{
    const dim3 grid((unsigned)((int64_t)g.tiles_m * g.tiles_n)), block(C::NT);
    if constexpr (BSRC == B_FP32) {
        // FP32 B loads element by element; only A has a vector path
        hipLaunchKernelGGL((gemm_bf16x9_kernel<C, NB, AVEC, BSRC, 0, RNE>), grid, block, 0, stream, g);
    } else {
        if (bvec == 1) hipLaunchKernelGGL((gemm_bf16x9_kernel<C, NB, AVEC, BSRC, 1, RNE>), grid, block, 0, stream, g);
        else if (BSRC == B_PLANES_NK && bvec == 2)
            hipLaunchKernelGGL((gemm_bf16x9_kernel<C, NB, AVEC, BSRC, BSRC == B_PLANES_NK ? 2 : 0, RNE>), grid, block, 0,
                               stream, g);
        else hipLaunchKernelGGL((gemm_bf16x9_kernel<C, NB, AVEC, BSRC, 0, RNE>), grid, block, 0, stream, g);
    }
}

// bvec: B's load width -- 1: 128-bit (N x K planes) or 32-bit (K x N planes);
// 2: 32-bit for N x K planes; 0: element loads.
template <class C, int NB, int BSRC, bool RNE>
static void launch_cfg(const GemmArgs &g, bool avec, int bvec, hipStream_t stream)
{
    if (avec) launch_cfg_b<C, NB, true, BSRC, RNE>(g, bvec, stream);
    else launch_cfg_b<C, NB, false, BSRC, RNE>(g, bvec, stream);
}

template <class C, int BSRC, bool RNE = false>
static void launch_nb(const GemmArgs &g, int nbands, bool avec, int bvec, hipStream_t stream)
{
    switch (nbands) {
    case 1: launch_cfg<C, 1, BSRC, RNE>(g, avec, bvec, stream); break;
    case 2: launch_cfg<C, 2, BSRC, RNE>(g, avec, bvec, stream); break;
    case 3: launch_cfg<C, 3, BSRC, RNE>(g, avec, bvec, stream); break;
    case 4: launch_cfg<C, 4, BSRC, RNE>(g, avec, bvec, stream); break;
    default: launch_cfg<C, 5, BSRC, RNE>(g, avec, bvec, stream); break;
    }
}

template <class C, int NB, bool RNE, bool KTAIL>
static void launch_dma_nb(const GemmArgs &g, bool avec, hipStream_t stream)
{
    // One resident workgroup per CU (LDS-limited); a multiple of 8 keeps each
    // workgroup on one XCD for all of its tiles.
    const dim3 block(C::NT);
#ifdef SGEMM_EMU_SERIAL_LDS
    {
        const dim3 grid((unsigned)((int64_t)g.tiles_m * g.tiles_n));
        if (avec) launch_last(gemm_bf16x9_serial_kernel<C, NB, true, RNE, KTAIL>, grid, block, stream, g);
        else launch_last(gemm_bf16x9_serial_kernel<C, NB, false, RNE, KTAIL>, grid, block, stream, g);
        return;
    }
#endif
    if (g.sk_grid > 0) {
        // small tile grid: stream-K over sk_grid workgroups
        GemmArgs s = g;
        s.sk_domains = streamk_domains((int64_t)g.tiles_m * g.tiles_n, g.K / (2 * BK), g.sk_grid);
        s.group_m = kStreamkGroupRows;
        const dim3 grid((unsigned)g.sk_grid);
        if (avec) launch_last(gemm_bf16x9_streamk_kernel<C, NB, true, RNE, KTAIL>, grid, block, stream, s);
        else launch_last(gemm_bf16x9_streamk_kernel<C, NB, false, RNE, KTAIL>, grid, block, stream, s);
        return;
    }
    const int64_t units = (int64_t)g.tiles_m * g.tiles_n;
    int64_t slots = (int64_t)(g.num_cus > 8 ? g.num_cus & ~7 : 8);
    const dim3 grid((unsigned)(units < slots ? units : slots));
    if (avec) launch_last(gemm_bf16x9_dma_kernel<C, NB, true, RNE, KTAIL>, grid, block, stream, g);
    else launch_last(gemm_bf16x9_dma_kernel<C, NB, false, RNE, KTAIL>, grid, block, stream, g);
}

template <class C, bool RNE, bool KTAIL>
static hipError_t launch_dma(const GemmArgs &args, int nbands, hipStream_t stream)
{
    GemmArgs g = args;
    g.tiles_m = (int)((g.M + C::BM - 1) / C::BM);
    g.tiles_n = (int)((g.N + C::BN - 1) / C::BN);
    g.group_m = group_rows(g.tiles_n, g.num_cus);
    // no 128-bit A load may straddle the end of A's rows (see launch_with)
    const bool avec = aligned(g.A, 16) && (g.lda % 4 == 0) && (g.ka % 4 == 0);
    switch (nbands) {
    case 1: launch_dma_nb<C, 1, RNE, KTAIL>(g, avec, stream); break;
    case 2: launch_dma_nb<C, 2, RNE, KTAIL>(g, avec, stream); break;
    case 3: launch_dma_nb<C, 3, RNE, KTAIL>(g, avec, stream); break;
    case 4: launch_dma_nb<C, 4, RNE, KTAIL>(g, avec, stream); break;
    default: launch_dma_nb<C, 5, RNE, KTAIL>(g, avec, stream); break;
    }
    return hipGetLastError();
}

template <class C, int NB>
static void launch_planes_nb(const GemmArgs &g, hipStream_t stream)
{
    const int64_t units = (int64_t)g.tiles_m * g.tiles_n;
    int64_t slots = (int64_t)(g.num_cus > 8 ? g.num_cus & ~7 : 8);
    const dim3 grid((unsigned)(units < slots ? units : slots)), block(C::NT);
    launch_last(gemm_bf16x9_planes_kernel<C, NB>, grid, block, stream, g);
}

hipError_t launch_gemm_planes(const GemmArgs &args, int nbands, hipStream_t stream)
{
    using C = Cfg8S;
    if (args.K % (2 * BK) != 0 || args.lda % 8 != 0 || args.ldb % 8 != 0 || !aligned(args.A0, 16) ||
        !aligned(args.A1, 16) || !aligned(args.A2, 16) || !aligned(args.B0, 16) || !aligned(args.B1, 16) ||
        !aligned(args.B2, 16))
        return hipErrorInvalidValue;
    GemmArgs g = args;
    g.tiles_m = (int)((g.M + C::BM - 1) / C::BM);
    g.tiles_n = (int)((g.N + C::BN - 1) / C::BN);
    g.group_m = group_rows(g.tiles_n, g.num_cus);
    switch (nbands) {
    case 1: launch_planes_nb<C, 1>(g, stream); break;
    case 2: launch_planes_nb<C, 2>(g, stream); break;
    case 3: launch_planes_nb<C, 3>(g, stream); break;
    case 4: launch_planes_nb<C, 4>(g, stream); break;
    default: launch_planes_nb<C, 5>(g, stream); break;
    }
    return hipGetLastError();
}

template <class C>
static GemmArgs tiled(const GemmArgs &args)
{
    GemmArgs g = args;
    g.tiles_m = (int)((g.M + C::BM - 1) / C::BM);
    g.tiles_n = (int)((g.N + C::BN - 1) / C::BN);
    g.group_m = group_rows(g.tiles_n, g.num_cus);
    return g;
}

// 128-bit loads along k need every 4 (A) or 8 (N x K planes) elements to lie
// entirely below or entirely above K, so that no vector load straddles the
// end of its descriptor's range.
static bool a_vec(const GemmArgs &g)
{
    return aligned(g.A, 16) && (g.lda % 4 == 0) && (g.K % 4 == 0);
}

// Load width of N x K planes: 128-bit loads need every 8 elements of a row to
// lie entirely below or above K (16-byte aligned planes, ldb and K multiples of
// 8); 32-bit loads need pairs (4-byte aligned planes, ldb and K even); else
// element loads.
static int nk_bvec(const GemmArgs &g)
{
    if (aligned(g.B0, 16) && aligned(g.B1, 16) && aligned(g.B2, 16) && g.ldb % 8 == 0 && g.K % 8 == 0) return 1;
    if (aligned(g.B0, 4) && aligned(g.B1, 4) && aligned(g.B2, 4) && g.ldb % 2 == 0 && g.K % 2 == 0) return 2;
    return 0;
}

// Load width of K x N planes: 32-bit loads (a column pair) need 4-byte
// aligned planes and ldb, N even; else element loads.
static int kn_bvec(const GemmArgs &g)
{
    return aligned(g.B0, 4) && aligned(g.B1, 4) && aligned(g.B2, 4) && g.ldb % 2 == 0 && g.N % 2 == 0 ? 1 : 0;
}

template <class C>
static hipError_t launch_with(const GemmArgs &args, int nbands, BSource bsrc, hipStream_t stream, bool rne)
{
    const GemmArgs g = tiled<C>(args);
    const bool avec = a_vec(g);
    int bvec = 0;
    if (bsrc == B_PLANES_NK)
        bvec = nk_bvec(g);
    else if (bsrc == B_PLANES_KN)
        bvec = kn_bvec(g);
    if (rne) {
        if (bsrc != B_FP32) return hipErrorInvalidValue;
        launch_nb<C, B_FP32, true>(g, nbands, avec, false, stream);
        return hipGetLastError();
    }
    switch (bsrc) {
    case B_FP32: launch_nb<C, B_FP32>(g, nbands, avec, false, stream); break;
    case B_PLANES_NK: launch_nb<C, B_PLANES_NK>(g, nbands, avec, bvec, stream); break;
    default: launch_nb<C, B_PLANES_KN>(g, nbands, avec, bvec, stream); break;
    }
    return hipGetLastError();
}

template <class C>
static hipError_t launch_tile64_cfg(const GemmArgs &args, int nbands, BSource bsrc, hipStream_t stream, bool rne)
{
    const GemmArgs g = tiled<C>(args);
    if (bsrc == B_PLANES_NK) {
        if (rne) return hipErrorInvalidValue;
        launch_nb<C, B_PLANES_NK>(g, nbands, a_vec(g), nk_bvec(g), stream);
    } else if (bsrc == B_PLANES_KN) {
        if (rne) return hipErrorInvalidValue;
        launch_nb<C, B_PLANES_KN>(g, nbands, a_vec(g), kn_bvec(g), stream);
    } else if (bsrc == B_FP32) {
        if (rne) launch_nb<C, B_FP32, true>(g, nbands, a_vec(g), false, stream);
        else launch_nb<C, B_FP32>(g, nbands, a_vec(g), false, stream);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Where every CU holds at most one 64 x 64 tile, the split's arithmetic spread
// two VALU instructions per MFMA measured faster than four (1024^3 67.7 -> 72.1
// TFLOP/s on FP32 B, 1024 x 1024 x 512 64.2 -> 68.1, 768^3 37.1 -> 39.2; N x K
// and K x N planes up to 4 % faster); with two tiles per CU four stay faster
// (6144 x 256 x 1024 88.1 against 86.5, 1200 x 1300 x 900 80.5 against 77.3).
// Scheduling only: the same bits.
hipError_t launch_gemm_tile64(const GemmArgs &args, int nbands, BSource bsrc, hipStream_t stream, bool rne)
{
    const int64_t tiles64 = ((args.M + 63) / 64) * ((args.N + 63) / 64);
    const int64_t G0 = args.num_cus > 8 ? args.num_cus & ~7 : 8;
    if (tiles64 <= G0) return launch_tile64_cfg<Cfg64S1>(args, nbands, bsrc, stream, rne);
    return launch_tile64_cfg<Cfg64S>(args, nbands, bsrc, stream, rne);
}

bool gemm_uses_dma(int64_t K, int64_t ldb, const void *B0, const void *B1, const void *B2)
{
    return K % (2 * BK) == 0 && ldb % 8 == 0 && aligned(B0, 16) && aligned(B1, 16) && aligned(B2, 16);
}

// Configuration per B source, chosen by measurement on MI355X: the explicit
// MFMA / split interleaving pays off where the kernel splits FP32 B or copies
// N x K planes; with K x N planes the compiler's own schedule is faster.
bool launch_done_attached(const GemmArgs &args, BSource bsrc)
{
    return bsrc == B_PLANES_NK && gemm_uses_dma(args.K, args.ldb, args.B0, args.B1, args.B2);
}

hipError_t launch_gemm(const GemmArgs &args, int nbands, BSource bsrc, hipStream_t stream, bool rne)
{
    if (bsrc == B_PLANES_KN) return launch_with<Cfg8>(args, nbands, bsrc, stream, rne);
    if (bsrc == B_PLANES_NK && gemm_uses_dma(args.K, args.ldb, args.B0, args.B1, args.B2)) {
        // A K tail (only with B planes zero-padded to the kernel's K) masks A past its K
        if (args.ka != args.K) {
            if (rne) return hipErrorInvalidValue;
            return launch_dma<Cfg8S, false, true>(args, nbands, stream);
        }
        return rne ? launch_dma<Cfg8S, true, false>(args, nbands, stream)
                   : launch_dma<Cfg8S, false, false>(args, nbands, stream);
    }
    return launch_with<Cfg8S>(args, nbands, bsrc, stream, rne);
}

}  // namespace sgemm_emu_dev
