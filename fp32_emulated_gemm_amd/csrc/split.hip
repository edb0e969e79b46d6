// split.hip -- standalone split kernel: FP32 matrix -> three BF16 planes.
//
// HBM-bound: 4 bytes read and 6 bytes written per element.  The fast kernel
// handles 8 consecutive elements per thread with two 128-bit loads and three
// 128-bit stores; rows are walked with a grid-stride loop over 8-element
// chunks so any grid size covers the matrix.  The scalar kernel covers every
// other layout (odd leading dimensions, unaligned pointers, ragged rows).
#include "split_device.hpp"
#include "launch.hpp"

namespace sgemm_emu_dev {

// Flat chunk index -> (row, chunk-in-row).  chunks_per_row = cols / 8.  FLAT:
// one contiguous row, so no division is needed.
template <bool FLAT, bool RNE>
__global__ __launch_bounds__(256) void split_vec8_kernel(
    const float *__restrict__ X, int64_t ldx, uint16_t *__restrict__ X0, uint16_t *__restrict__ X1,
    uint16_t *__restrict__ X2, int64_t ldo, int64_t chunks_per_row, int64_t total_chunks)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total_chunks; c += stride) {
        const int64_t row = FLAT ? 0 : c / chunks_per_row;
        const int64_t col = (c - row * chunks_per_row) * 8;
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        const f32x4_t *src = reinterpret_cast<const f32x4_t *>(X + row * ldx + col);
        f32x4_t v0 = __builtin_nontemporal_load(src);
        f32x4_t v1 = __builtin_nontemporal_load(src + 1);
        float x[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        uint32_t p0[4], p1[4], p2[4];
        if (split8_packed_finite<RNE>(x, p0, p1, p2)) split8_packed<RNE>(x, p0, p1, p2);
        const int64_t o = row * ldo + col;
        *reinterpret_cast<uint4 *>(X0 + o) = make_uint4(p0[0], p0[1], p0[2], p0[3]);
        *reinterpret_cast<uint4 *>(X1 + o) = make_uint4(p1[0], p1[1], p1[2], p1[3]);
        *reinterpret_cast<uint4 *>(X2 + o) = make_uint4(p2[0], p2[1], p2[2], p2[3]);
    }
}

// One element per thread (any layout).  TRANSPOSE writes the planes of X^T:
// element (row, col) lands at col * ldo + row.
template <bool TRANSPOSE, bool RNE>
__global__ __launch_bounds__(256) void split_scalar_kernel(
    const float *__restrict__ X, int64_t ldx, uint16_t *__restrict__ X0, uint16_t *__restrict__ X1,
    uint16_t *__restrict__ X2, int64_t ldo, int64_t rows, int64_t cols)
{
    const int64_t total = rows * cols;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int64_t row = e / cols;
        const int64_t col = e - row * cols;
        float x = X[row * ldx + col];
        uint32_t c0, c1, c2;
        float t = split_finite<RNE>(x, c0, c1, c2);
        if (t != t) split_fix_special(x, c0, c1, c2);
        const int64_t o = TRANSPOSE ? col * ldo + row : row * ldo + col;
        X0[o] = (uint16_t)(c0 >> 16);
        X1[o] = (uint16_t)(c1 >> 16);
        X2[o] = (uint16_t)(c2 >> 16);
    }
}

// Split with transposition: X is rows x cols (ldx), the planes are cols x rows
// (leading dimension ldo); turns an FP32 K x N operand into N x K planes.
// One workgroup per TT x TT tile of X: TT = 32 up to 4 64 x 64 tiles per CU
// (a weight of up to 2048 x 2048 on 256 CUs), where the split is bound by the
// latency of its one round of loads and four times the workgroups keep more
// of them in flight (1024 x 1024: 5.8 -> 4.1 us alone, 10.2 -> 7.4 us right
// after a GEMM kernel); TT = 64 above, where the larger tiles move the bytes
// faster (4096 x 4096: 26.4 against 27.8 us).  The tile goes through LDS: read along X's
// rows (each wave reads TT contiguous floats per row), then each thread takes
// 8 consecutive rows of one column, splits them, and writes one 16-byte run of
// each plane row; eight neighbouring lanes cover 128 contiguous bytes.  The
// LDS row pitch of TT + 1 floats makes both the row-wise writes and the
// column-wise reads free of bank conflicts.
// Requires rows % 8 == 0, ldo % 8 == 0 and 16-byte aligned planes; other
// layouts take split_scalar_kernel<true>.
template <bool RNE, int TT>
__global__ __launch_bounds__(256) void split_transpose_kernel(
    const float *__restrict__ X, int64_t ldx, uint16_t *__restrict__ X0, uint16_t *__restrict__ X1,
    uint16_t *__restrict__ X2, int64_t ldo, int64_t rows_in, int64_t rows, int64_t cols, int64_t tiles_c)
{
    // rows_in <= rows: X rows past rows_in read as zero (a zero-padded K extent)
    __shared__ float tile[TT][TT + 1];
    constexpr int RPP = 256 / TT;                       // rows read per pass
    // 32-bit block arithmetic: the launcher keeps the tile count below 2^31
    const uint32_t tc = (uint32_t)tiles_c, br = blockIdx.x / tc;
    const int64_t r0 = (int64_t)br * TT;
    const int64_t c0 = (int64_t)(blockIdx.x - br * tc) * TT;
    const int tid = threadIdx.x;
    const int c = tid & (TT - 1);
    const bool col_in = c0 + c < cols;
#pragma unroll
    for (int i = 0; i < TT / RPP; ++i) {
        const int r = tid / TT + RPP * i;
        float v = 0.0f;
        if (col_in && r0 + r < rows_in) v = X[(r0 + r) * ldx + c0 + c];
        tile[r][c] = v;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < (TT * TT / 8 + 255) / 256; ++j) {
        const int u = tid + 256 * j;
        const int kg = u % (TT / 8), n = u / (TT / 8);
        if (n >= TT || c0 + n >= cols || r0 + 8 * kg >= rows) continue;  // rows % 8 == 0: groups are whole
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = tile[8 * kg + e][n];
        uint32_t p0[4], p1[4], p2[4];
        if (split8_packed_finite<RNE>(x, p0, p1, p2)) split8_packed<RNE>(x, p0, p1, p2);
        const int64_t o = (c0 + n) * ldo + r0 + 8 * kg;
        *reinterpret_cast<uint4 *>(X0 + o) = make_uint4(p0[0], p0[1], p0[2], p0[3]);
        *reinterpret_cast<uint4 *>(X1 + o) = make_uint4(p1[0], p1[1], p1[2], p1[3]);
        *reinterpret_cast<uint4 *>(X2 + o) = make_uint4(p2[0], p2[1], p2[2], p2[3]);
    }
}

template <bool RNE>
static hipError_t split_transpose_with(int64_t rows, int64_t cols, const float *X, int64_t ldx, uint16_t *X0,
                                       uint16_t *X1, uint16_t *X2, int64_t ldo, int num_cus, hipStream_t stream,
                                       int64_t rows_out)
{
    const int64_t rows_in = rows;
    if (rows_out > rows) rows = rows_out;
    if (rows == 0 || cols == 0) return hipSuccess;
    if (rows % 8 != 0 || ldo % 8 != 0 || !aligned(X0, 16) || !aligned(X1, 16) || !aligned(X2, 16)) {
        if (rows != rows_in) return hipErrorInvalidValue;   // zero padding needs the tiled kernel
        const int threads = 256;
        int64_t blocks = (rows * cols + threads - 1) / threads;
        if (blocks > (int64_t)num_cus * 8) blocks = (int64_t)num_cus * 8;
        hipLaunchKernelGGL((split_scalar_kernel<true, RNE>), dim3((unsigned)blocks), dim3(threads), 0, stream, X, ldx,
                           X0, X1, X2, ldo, rows, cols);
        return hipGetLastError();
    }
    const int64_t tiles64 = ((cols + 63) / 64) * ((rows + 63) / 64);
    if (tiles64 > 4 * (int64_t)num_cus) {
        const int64_t tiles_c = (cols + 63) / 64, tiles_r = (rows + 63) / 64;
        if (tiles_r > (int64_t)0x7FFFFFFF / tiles_c) return hipErrorInvalidValue;
        hipLaunchKernelGGL((split_transpose_kernel<RNE, 64>), dim3((unsigned)(tiles_r * tiles_c)), dim3(256), 0,
                           stream, X, ldx, X0, X1, X2, ldo, rows_in, rows, cols, tiles_c);
    } else {
        const int64_t tiles_c = (cols + 31) / 32, tiles_r = (rows + 31) / 32;
        hipLaunchKernelGGL((split_transpose_kernel<RNE, 32>), dim3((unsigned)(tiles_r * tiles_c)), dim3(256), 0,
                           stream, X, ldx, X0, X1, X2, ldo, rows_in, rows, cols, tiles_c);
    }
    return hipGetLastError();
}

// Transpose three BF16 planes: P (rows x cols, leading dimension ldp) -> Q
// (cols x rows_out, leading dimension ldq), Q[c][r] = P[r][c] for r < rows and
// zero for rows <= r < rows_out (K x N planes of B into the N x K' layout of
// the DMA kernel).  One workgroup per 64 x 64 tile of Q's index space: each
// wave reads 128-byte runs of P's rows, the tile goes through LDS, and four
// neighbouring lanes write one 128-byte run of a row of Q.
constexpr int kPT = 64;

__global__ __launch_bounds__(256) void transpose_planes_kernel(
    const uint16_t *__restrict__ P0, const uint16_t *__restrict__ P1, const uint16_t *__restrict__ P2, int64_t ldp,
    uint16_t *__restrict__ Q0, uint16_t *__restrict__ Q1, uint16_t *__restrict__ Q2, int64_t ldq, int64_t rows,
    int64_t rows_out, int64_t cols, int64_t tiles_c)
{
    __shared__ uint16_t tile[3][kPT][kPT + 2];
    const uint32_t tc = (uint32_t)tiles_c, br = blockIdx.x / tc;   // fewer than 2^31 tiles
    const int64_t r0 = (int64_t)br * kPT;
    const int64_t c0 = (int64_t)(blockIdx.x - br * tc) * kPT;
    const int tid = threadIdx.x;
    const uint16_t *P[3] = {P0, P1, P2};
    {
        const int c = tid & (kPT - 1);
        const bool col_in = c0 + c < cols;
#pragma unroll
        for (int i = 0; i < kPT / 4; ++i) {
            const int r = (tid >> 6) + 4 * i;
            const bool in = col_in && r0 + r < rows;
#pragma unroll
            for (int p = 0; p < 3; ++p) tile[p][r][c] = in ? P[p][(r0 + r) * ldp + c0 + c] : (uint16_t)0;
        }
    }
    __syncthreads();
    uint16_t *Q[3] = {Q0, Q1, Q2};
    const int n = tid >> 2, q = tid & 3;         // row of Q in the tile, quarter of its 64 elements
    if (c0 + n >= cols) return;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int rb = 16 * q + 8 * h;       // first of 8 consecutive elements of Q's row
            if (r0 + rb >= rows_out) continue;   // rows_out % 8 == 0: groups are whole
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = (uint32_t)tile[p][rb + 2 * e][n] | ((uint32_t)tile[p][rb + 2 * e + 1][n] << 16);
            *reinterpret_cast<uint4 *>(Q[p] + (c0 + n) * ldq + r0 + rb) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

hipError_t launch_transpose_planes(int64_t rows, int64_t cols, const uint16_t *P0, const uint16_t *P1,
                                   const uint16_t *P2, int64_t ldp, uint16_t *Q0, uint16_t *Q1, uint16_t *Q2,
                                   int64_t ldq, int64_t rows_out, hipStream_t stream)
{
    if (rows_out < rows || rows_out % 8 != 0 || ldq % 8 != 0 || ldq < rows_out || !aligned(Q0, 16) ||
        !aligned(Q1, 16) || !aligned(Q2, 16))
        return hipErrorInvalidValue;
    if (rows_out == 0 || cols == 0) return hipSuccess;
    const int64_t tiles_c = (cols + kPT - 1) / kPT, tiles_r = (rows_out + kPT - 1) / kPT;
    if (tiles_r > (int64_t)0x7FFFFFFF / tiles_c) return hipErrorInvalidValue;
    hipLaunchKernelGGL(transpose_planes_kernel, dim3((unsigned)(tiles_r * tiles_c)), dim3(256), 0, stream, P0, P1,
                       P2, ldp, Q0, Q1, Q2, ldq, rows, rows_out, cols, tiles_c);
    return hipGetLastError();
}

hipError_t launch_split_transpose(int64_t rows, int64_t cols, const float *X, int64_t ldx, uint16_t *X0,
                                  uint16_t *X1, uint16_t *X2, int64_t ldo, int num_cus, hipStream_t stream, bool rne,
                                  int64_t rows_out)
{
    return rne ? split_transpose_with<true>(rows, cols, X, ldx, X0, X1, X2, ldo, num_cus, stream, rows_out)
               : split_transpose_with<false>(rows, cols, X, ldx, X0, X1, X2, ldo, num_cus, stream, rows_out);
}

template <bool RNE>
static hipError_t split_with(int64_t rows, int64_t cols, const float *X, int64_t ldx, uint16_t *X0,
                             uint16_t *X1, uint16_t *X2, int64_t ldo, int num_cus, hipStream_t stream)
{
    const bool vec = (cols % 8 == 0) && (ldx % 4 == 0) && (ldo % 8 == 0) &&
                     aligned(X, 16) && aligned(X0, 16) && aligned(X1, 16) && aligned(X2, 16);
    const int threads = 256;
    // Enough resident waves to cover HBM latency; the loops stride over the rest.
    const int64_t max_blocks = (int64_t)num_cus * 8;
    if (vec) {
        // Contiguous rows fold into one long row, which keeps chunk indexing cheap.
        int64_t r = rows, c = cols, lx = ldx, lo = ldo;
        if (ldx == cols && ldo == cols) { c = rows * cols; r = 1; lx = c; lo = c; }
        const int64_t chunks_per_row = c / 8;
        const int64_t total = r * chunks_per_row;
        int64_t blocks = (total + threads - 1) / threads;
        if (blocks > max_blocks) blocks = max_blocks;
        if (r == 1)
            hipLaunchKernelGGL((split_vec8_kernel<true, RNE>), dim3((unsigned)blocks), dim3(threads), 0, stream,
                               X, lx, X0, X1, X2, lo, chunks_per_row, total);
        else
            hipLaunchKernelGGL((split_vec8_kernel<false, RNE>), dim3((unsigned)blocks), dim3(threads), 0, stream,
                               X, lx, X0, X1, X2, lo, chunks_per_row, total);
    } else {
        const int64_t total = rows * cols;
        int64_t blocks = (total + threads - 1) / threads;
        if (blocks > max_blocks) blocks = max_blocks;
        hipLaunchKernelGGL((split_scalar_kernel<false, RNE>), dim3((unsigned)blocks), dim3(threads), 0, stream, X,
                           ldx, X0, X1, X2, ldo, rows, cols);
    }
    return hipGetLastError();
}

hipError_t launch_split(int64_t rows, int64_t cols, const float *X, int64_t ldx, uint16_t *X0,
                        uint16_t *X1, uint16_t *X2, int64_t ldo, int num_cus, hipStream_t stream, bool rne)
{
    return rne ? split_with<true>(rows, cols, X, ldx, X0, X1, X2, ldo, num_cus, stream)
               : split_with<false>(rows, cols, X, ldx, X0, X1, X2, ldo, num_cus, stream);
}

}  // namespace sgemm_emu_dev
