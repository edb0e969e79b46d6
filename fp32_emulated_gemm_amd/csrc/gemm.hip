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
// Kernel structure (one workgroup per 128 x 128 tile of C, 512 threads):
//   * 8 waves in a 2 (M) x 4 (N) grid; each wave owns a 64 x 32 sub-tile,
//     i.e. two 32 x 32 MFMA blocks, each with NB band accumulators of 16
//     FP32 registers per lane (v_mfma_f32_32x32x16_bf16).
//   * K advances in steps of 32.  Each thread loads 8 FP32 values of A (one
//     row, 8 consecutive k) and 8 of B (one column, 8 consecutive k) into
//     registers one step ahead, splits them in registers and writes the three
//     BF16 component tiles into LDS, k-contiguous for both operands (B is
//     transposed on the way in).  LDS is double-buffered, so one barrier per
//     step separates producers from consumers.
//   * LDS rows are 32 BF16 plus 8 BF16 of padding (80 bytes): the 128-bit
//     fragment reads of 16 consecutive rows then touch 64 distinct banks.
//   * Tile order: workgroups are dealt round-robin to the 8 XCDs, so the
//     block index is remapped to give each XCD a contiguous run of tiles, and
//     tiles run in groups of 8 tile-rows so concurrent tiles share A panels
//     and B panels in the XCD's L2.
//   * Epilogue: per output, acc = 2^-32 S4; acc = fma(S3, 2^-24, acc);
//     acc = fma(S2, 2^-16, acc); acc = fma(S1, 2^-8, acc); C = acc + S0.
// Edges: rows of A beyond M and columns of B beyond N are clamped to valid
// memory (their results are never stored); k beyond K is zero-filled.
#include "split_device.hpp"
#include "launch.hpp"

namespace sgemm_emu_dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int KP = BK + 8;                      // LDS row pitch in BF16 elements (80 bytes)
constexpr int NTHREADS = 512;
constexpr int WAVES_N = 4;
constexpr int WTM = 64, WTN = 32;               // wave tile
constexpr int MI = WTM / 32, NI = WTN / 32;     // MFMA blocks per wave
constexpr int TILE_ELEMS = (BM + BN) * KP;      // one component plane of A and B
constexpr int GROUP_M = 8;

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t lmin(int64_t a, int64_t b) { return a < b ? a : b; }

// Block index -> (tile_m, tile_n), XCD-contiguous and grouped by tile-rows.
__device__ __forceinline__ void tile_of_block(int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int G = (int)gridDim.x, b = (int)blockIdx.x;
    const int per = G >> 3, extra = G & 7, xcd = b & 7, idx = b >> 3;
    const int t = xcd * per + imin(xcd, extra) + idx;
    const int group_size = GROUP_M * tiles_n;
    const int group = t / group_size;
    const int first_m = group * GROUP_M;
    const int gm = imin(tiles_m - first_m, GROUP_M);
    const int in = t - group * group_size;
    tm = first_m + in % gm;
    tn = in / gm;
}

// ---------------------------------------------------------------- operand staging

// 8 FP32 values of A's row `arow`, starting at column k (k is a multiple of 8).
template <bool AVEC, bool TAIL>
__device__ __forceinline__ void load_a8(const float *__restrict__ arow, int64_t k, int64_t K, float (&x)[8])
{
    if (AVEC && (!TAIL || k + 8 <= K)) {
        const float4 *p = reinterpret_cast<const float4 *>(arow + k);
        float4 v0 = p[0], v1 = p[1];
        x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
        x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (!TAIL || k + e < K) ? arow[k + e] : 0.0f;
    }
}

// 8 FP32 values of B's column: rows k .. k+7 (bcol points at row 0 of the column).
template <bool TAIL>
__device__ __forceinline__ void load_b8(const float *__restrict__ bcol, int64_t ldb, int64_t k, int64_t K,
                                        float (&x)[8])
{
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (!TAIL || k + e < K) ? bcol[(k + e) * ldb] : 0.0f;
}

// 8 BF16 values of one column of each B plane, packed two per dword along k.
template <bool TAIL>
__device__ __forceinline__ void load_b8_planes(const uint16_t *__restrict__ b0, const uint16_t *__restrict__ b1,
                                               const uint16_t *__restrict__ b2, int64_t ldb, int64_t k, int64_t K,
                                               uint32_t (&p0)[4], uint32_t (&p1)[4], uint32_t (&p2)[4])
{
    uint32_t h0[8], h1[8], h2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bool ok = !TAIL || k + e < K;
        const int64_t o = (k + e) * ldb;
        h0[e] = ok ? b0[o] : 0u;
        h1[e] = ok ? b1[o] : 0u;
        h2[e] = ok ? b2[o] : 0u;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p0[i] = h0[2 * i] | (h0[2 * i + 1] << 16);
        p1[i] = h1[2 * i] | (h1[2 * i + 1] << 16);
        p2[i] = h2[2 * i] | (h2[2 * i + 1] << 16);
    }
}

__device__ __forceinline__ void st_lds16(uint16_t *p, const uint32_t (&v)[4])
{
    *reinterpret_cast<u32x4_t *>(p) = u32x4_t{v[0], v[1], v[2], v[3]};
}

// Registers holding one thread's share of the next K step.
template <int BSRC>
struct Stage {
    float a[8];
    float b[8];                 // B_FP32
    uint32_t bp[3][4];          // B_PLANES
};

template <bool AVEC, int BSRC, bool TAIL>
__device__ __forceinline__ void load_stage(Stage<BSRC> &st, const GemmArgs &g, const float *arow,
                                           const float *bcol, const uint16_t *bc0, const uint16_t *bc1,
                                           const uint16_t *bc2, int64_t ka, int64_t kb)
{
    load_a8<AVEC, TAIL>(arow, ka, g.K, st.a);
    if constexpr (BSRC == B_FP32) load_b8<TAIL>(bcol, g.ldb, kb, g.K, st.b);
    else load_b8_planes<TAIL>(bc0, bc1, bc2, g.ldb, kb, g.K, st.bp[0], st.bp[1], st.bp[2]);
}

template <int BSRC>
__device__ __forceinline__ void store_stage(const Stage<BSRC> &st, uint16_t *buf, int a_off, int b_off)
{
    uint32_t p0[4], p1[4], p2[4];
    split8_packed(st.a, p0, p1, p2);
    st_lds16(buf + 0 * TILE_ELEMS + a_off, p0);
    st_lds16(buf + 1 * TILE_ELEMS + a_off, p1);
    st_lds16(buf + 2 * TILE_ELEMS + a_off, p2);
    if constexpr (BSRC == B_FP32) {
        split8_packed(st.b, p0, p1, p2);
        st_lds16(buf + 0 * TILE_ELEMS + b_off, p0);
        st_lds16(buf + 1 * TILE_ELEMS + b_off, p1);
        st_lds16(buf + 2 * TILE_ELEMS + b_off, p2);
    } else {
        st_lds16(buf + 0 * TILE_ELEMS + b_off, st.bp[0]);
        st_lds16(buf + 1 * TILE_ELEMS + b_off, st.bp[1]);
        st_lds16(buf + 2 * TILE_ELEMS + b_off, st.bp[2]);
    }
}

__device__ __forceinline__ bf16x8_t ld_frag(const uint16_t *p)
{
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(p));
}

// ---------------------------------------------------------------- kernel

template <int NB, bool AVEC, int BSRC>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16x9_kernel(GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 3 * TILE_ELEMS];

    int tm, tn;
    tile_of_block(g.tiles_m, g.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

    // Loader roles.  A: wave w stages rows 16w..16w+15; lane -> (row, 8-wide k group).
    const int a_row = wave * 16 + (lane & 15), a_kg = lane >> 4;
    // B: thread -> (column, 8-wide k group).
    const int b_col = tid & (BN - 1), b_kg = tid >> 7;
    const int a_off = a_row * KP + a_kg * 8;
    const int b_off = (BM + b_col) * KP + b_kg * 8;

    const float *arow = g.A + lmin(m0 + a_row, g.M - 1) * g.lda;
    const int64_t bj = lmin(n0 + b_col, g.N - 1);
    const float *bcol = (BSRC == B_FP32) ? g.B + bj : nullptr;
    const uint16_t *bc0 = (BSRC == B_PLANES) ? g.B0 + bj : nullptr;
    const uint16_t *bc1 = (BSRC == B_PLANES) ? g.B1 + bj : nullptr;
    const uint16_t *bc2 = (BSRC == B_PLANES) ? g.B2 + bj : nullptr;

    // Compute roles: wave (wm, wn) owns rows wm*64.., columns wn*32..
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int frag_row = lane & 31, frag_k = (lane >> 5) * 8;

    f32x16_t acc[MI][NB];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int s = 0; s < NB; ++s) acc[i][s] = f32x16_t{};

    const int64_t nk = (g.K + BK - 1) / BK;
    const bool k_ragged = (g.K % BK) != 0;

    Stage<BSRC> st;
    if (nk == 1 && k_ragged)
        load_stage<AVEC, BSRC, true>(st, g, arow, bcol, bc0, bc1, bc2, a_kg * 8, b_kg * 8);
    else
        load_stage<AVEC, BSRC, false>(st, g, arow, bcol, bc0, bc1, bc2, a_kg * 8, b_kg * 8);
    store_stage<BSRC>(st, lds, a_off, b_off);
    __syncthreads();

    for (int64_t kt = 0; kt < nk; ++kt) {
        uint16_t *cur = lds + (kt & 1) * 3 * TILE_ELEMS;
        uint16_t *nxt = lds + ((kt + 1) & 1) * 3 * TILE_ELEMS;
        const bool have_next = kt + 1 < nk;
        if (have_next) {
            const int64_t k0 = (kt + 1) * BK;
            if (kt + 2 == nk && k_ragged)
                load_stage<AVEC, BSRC, true>(st, g, arow, bcol, bc0, bc1, bc2, k0 + a_kg * 8, k0 + b_kg * 8);
            else
                load_stage<AVEC, BSRC, false>(st, g, arow, bcol, bc0, bc1, bc2, k0 + a_kg * 8, k0 + b_kg * 8);
        }

#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8_t af[MI][3], bfr[NI][3];
#pragma unroll
            for (int c = 0; c < 3; ++c) {
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    af[i][c] = ld_frag(cur + c * TILE_ELEMS + (wm * WTM + i * 32 + frag_row) * KP + kk + frag_k);
#pragma unroll
                for (int j = 0; j < NI; ++j)
                    bfr[j][c] = ld_frag(cur + c * TILE_ELEMS + (BM + wn * WTN + j * 32 + frag_row) * KP + kk + frag_k);
            }
#pragma unroll
            for (int p = 0; p < 3; ++p)
#pragma unroll
                for (int q = 0; q < 3; ++q) {
                    if (p + q < NB) {
#pragma unroll
                        for (int i = 0; i < MI; ++i)
                            acc[i][p + q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i][p], bfr[0][q],
                                                                                     acc[i][p + q], 0, 0, 0);
                    }
                }
        }

        if (have_next) store_stage<BSRC>(st, nxt, a_off, b_off);
        __syncthreads();
    }

    // Epilogue: recombine the bands smallest first and store.
    const int col = (int)(n0 + wn * WTN + (lane & 31));
    const bool col_ok = col < g.N;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            float v = 0.0f;
            if constexpr (NB >= 5) v = 0x1p-32f * acc[i][4][r];
            if constexpr (NB >= 4) v = __builtin_fmaf(acc[i][3][r], 0x1p-24f, v);
            if constexpr (NB >= 3) v = __builtin_fmaf(acc[i][2][r], 0x1p-16f, v);
            if constexpr (NB >= 2) v = __builtin_fmaf(acc[i][1][r], 0x1p-8f, v);
            v = v + acc[i][0][r];
            if (col_ok && row < g.M) g.C[row * g.ldc + col] = v;
        }
    }
}

// ---------------------------------------------------------------- K == 0

__global__ __launch_bounds__(256) void zero_kernel(float *__restrict__ C, int64_t ldc, int64_t M, int64_t N)
{
    const int64_t total = M * N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t r = e / N;
        C[r * ldc + (e - r * N)] = 0.0f;
    }
}

hipError_t launch_zero(int64_t M, int64_t N, float *C, int64_t ldc, int num_cus, hipStream_t stream)
{
    int64_t blocks = (M * N + 255) / 256;
    if (blocks > (int64_t)num_cus * 8) blocks = (int64_t)num_cus * 8;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, C, ldc, M, N);
    return hipGetLastError();
}

// ---------------------------------------------------------------- dispatch

template <int NB, int BSRC>
static void launch_nb(const GemmArgs &g, bool avec, dim3 grid, hipStream_t stream)
{
    if (avec)
        hipLaunchKernelGGL((gemm_bf16x9_kernel<NB, true, BSRC>), grid, dim3(NTHREADS), 0, stream, g);
    else
        hipLaunchKernelGGL((gemm_bf16x9_kernel<NB, false, BSRC>), grid, dim3(NTHREADS), 0, stream, g);
}

template <int BSRC>
static void launch_bsrc(const GemmArgs &g, int nbands, bool avec, dim3 grid, hipStream_t stream)
{
    switch (nbands) {
    case 1: launch_nb<1, BSRC>(g, avec, grid, stream); break;
    case 2: launch_nb<2, BSRC>(g, avec, grid, stream); break;
    case 3: launch_nb<3, BSRC>(g, avec, grid, stream); break;
    case 4: launch_nb<4, BSRC>(g, avec, grid, stream); break;
    default: launch_nb<5, BSRC>(g, avec, grid, stream); break;
    }
}

hipError_t launch_gemm(const GemmArgs &args, int nbands, BSource bsrc, hipStream_t stream)
{
    GemmArgs g = args;
    g.tiles_m = (int)((g.M + BM - 1) / BM);
    g.tiles_n = (int)((g.N + BN - 1) / BN);
    const dim3 grid((unsigned)((int64_t)g.tiles_m * g.tiles_n));
    const bool avec = aligned(g.A, 16) && (g.lda % 4 == 0);
    if (bsrc == B_FP32) launch_bsrc<B_FP32>(g, nbands, avec, grid, stream);
    else launch_bsrc<B_PLANES>(g, nbands, avec, grid, stream);
    return hipGetLastError();
}

}  // namespace sgemm_emu_dev
