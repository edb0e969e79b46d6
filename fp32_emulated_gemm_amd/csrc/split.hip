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
template <bool FLAT>
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
        if (split8_packed_finite(x, p0, p1, p2)) split8_packed(x, p0, p1, p2);
        const int64_t o = row * ldo + col;
        *reinterpret_cast<uint4 *>(X0 + o) = make_uint4(p0[0], p0[1], p0[2], p0[3]);
        *reinterpret_cast<uint4 *>(X1 + o) = make_uint4(p1[0], p1[1], p1[2], p1[3]);
        *reinterpret_cast<uint4 *>(X2 + o) = make_uint4(p2[0], p2[1], p2[2], p2[3]);
    }
}

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
        float t = split_finite(x, c0, c1, c2);
        if (t != t) split_fix_special(x, c0, c1, c2);
        const int64_t o = row * ldo + col;
        X0[o] = (uint16_t)(c0 >> 16);
        X1[o] = (uint16_t)(c1 >> 16);
        X2[o] = (uint16_t)(c2 >> 16);
    }
}

hipError_t launch_split(int64_t rows, int64_t cols, const float *X, int64_t ldx, uint16_t *X0,
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
            hipLaunchKernelGGL(split_vec8_kernel<true>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                               X, lx, X0, X1, X2, lo, chunks_per_row, total);
        else
            hipLaunchKernelGGL(split_vec8_kernel<false>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                               X, lx, X0, X1, X2, lo, chunks_per_row, total);
    } else {
        const int64_t total = rows * cols;
        int64_t blocks = (total + threads - 1) / threads;
        if (blocks > max_blocks) blocks = max_blocks;
        hipLaunchKernelGGL(split_scalar_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, X, ldx,
                           X0, X1, X2, ldo, rows, cols);
    }
    return hipGetLastError();
}

}  // namespace sgemm_emu_dev
