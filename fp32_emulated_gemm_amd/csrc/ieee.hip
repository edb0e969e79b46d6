// ieee.hip -- optional IEEE fix-up of outputs touched by non-finite inputs.
//
// The emulation multiplies components: an Inf operand meets the zero
// components of its partner (Inf x 0 = NaN), so an output that IEEE FP32
// would give as +-Inf can come out NaN (the pages note that the BF16x9 mode
// is not IEEE-754 compliant; discuss.pytorch.kr summary, section
// "PyTorch에서 직접 써 보려면").  With SGEMM_EMU_IEEE_SPECIALS the library
// recomputes every output whose row of A or column of B holds an Inf or NaN
// as a plain FP32 dot product (k ascending, product and sum rounded
// separately), which carries IEEE's special-value rules; all other outputs
// keep the emulated value.  Such outputs are always Inf or NaN.
//
// Three passes: flag the rows of A and the columns of B that hold a
// non-finite value, compact the flagged columns into a list, then recompute
// the flagged rows in full and the flagged columns of the other rows.
#include "launch.hpp"

namespace sgemm_emu_dev {

__device__ __forceinline__ bool nonfinite(float x) { return (__float_as_uint(x) & 0x7F800000u) == 0x7F800000u; }

// One wave per row of A: any non-finite among its K values.
__global__ __launch_bounds__(256) void flag_rows_kernel(const float *__restrict__ A, int64_t lda, int64_t M,
                                                        int64_t K, int *__restrict__ row_flag)
{
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
    for (int64_t i = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64; i < M; i += waves) {
        bool bad = false;
        for (int64_t k = lane; k < K; k += 64) bad |= nonfinite(A[i * lda + k]);
        const bool any = __any(bad);
        if (lane == 0) row_flag[i] = any ? 1 : 0;
    }
}

// One thread per column of B (lanes along N, so every load is coalesced).
__global__ __launch_bounds__(256) void flag_cols_kernel(const float *__restrict__ B, int64_t ldb, int64_t K,
                                                        int64_t N, int *__restrict__ col_flag)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < N; j += stride) {
        bool bad = false;
        for (int64_t k = 0; k < K; ++k) bad |= nonfinite(B[k * ldb + j]);
        col_flag[j] = bad ? 1 : 0;
    }
}

// Single workgroup: the flagged columns in ascending order, and their count.
__global__ __launch_bounds__(256) void list_cols_kernel(const int *__restrict__ col_flag, int64_t N,
                                                        int *__restrict__ cols, int *__restrict__ count)
{
    __shared__ int base;
    if (threadIdx.x == 0) base = 0;
    __syncthreads();
    for (int64_t j0 = 0; j0 < N; j0 += blockDim.x) {
        const int64_t j = j0 + threadIdx.x;
        const bool f = j < N && col_flag[j];
        // order-preserving compaction of this chunk through a ballot per wave
        __shared__ int wave_total[4];
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        const unsigned long long ball = __ballot(f);
        const int before = __popcll(ball & ((1ull << lane) - 1ull));
        if (lane == 0) wave_total[w] = __popcll(ball);
        __syncthreads();
        int offset = base;
        for (int v = 0; v < w; ++v) offset += wave_total[v];
        if (f) cols[offset + before] = (int)j;
        __syncthreads();
        if (threadIdx.x == 0) base += wave_total[0] + wave_total[1] + wave_total[2] + wave_total[3];
        __syncthreads();
    }
    if (threadIdx.x == 0) *count = base;
}

// Plain FP32 dot product, k ascending, product and sum rounded separately.
__device__ __forceinline__ float ieee_dot(const float *__restrict__ a, const float *__restrict__ B, int64_t ldb,
                                          int64_t K, int64_t j)
{
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        const float p = __fmul_rn(a[k], B[k * ldb + j]);
        acc = __fadd_rn(acc, p);
    }
    return acc;
}

// One workgroup per row (grid-stride): a flagged row is recomputed in full,
// any other row only at the flagged columns.
__global__ __launch_bounds__(256) void ieee_fixup_kernel(const float *__restrict__ A, int64_t lda,
                                                         const float *__restrict__ B, int64_t ldb,
                                                         float *__restrict__ C, int64_t ldc, int64_t M, int64_t N,
                                                         int64_t K, const int *__restrict__ row_flag,
                                                         const int *__restrict__ cols,
                                                         const int *__restrict__ ncols)
{
    const int nc = *ncols;
    for (int64_t i = blockIdx.x; i < M; i += gridDim.x) {
        const float *a = A + i * lda;
        if (row_flag[i]) {
            for (int64_t j = threadIdx.x; j < N; j += blockDim.x) C[i * ldc + j] = ieee_dot(a, B, ldb, K, j);
        } else {
            for (int c = threadIdx.x; c < nc; c += blockDim.x) {
                const int64_t j = cols[c];
                C[i * ldc + j] = ieee_dot(a, B, ldb, K, j);
            }
        }
    }
}

hipError_t launch_ieee_fixup(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                             int64_t ldb, float *C, int64_t ldc, int *work, int num_cus, hipStream_t stream)
{
    int *row_flag = work, *col_flag = work + M, *cols = col_flag + N, *count = cols + N;
    const int64_t max_blocks = (int64_t)num_cus * 8;
    int64_t rb = (M + 3) / 4;
    if (rb > max_blocks) rb = max_blocks;
    hipLaunchKernelGGL(flag_rows_kernel, dim3((unsigned)rb), dim3(256), 0, stream, A, lda, M, K, row_flag);
    int64_t cb = (N + 255) / 256;
    if (cb > max_blocks) cb = max_blocks;
    hipLaunchKernelGGL(flag_cols_kernel, dim3((unsigned)cb), dim3(256), 0, stream, B, ldb, K, N, col_flag);
    hipLaunchKernelGGL(list_cols_kernel, dim3(1), dim3(256), 0, stream, col_flag, N, cols, count);
    const int64_t fb = M < max_blocks ? M : max_blocks;
    hipLaunchKernelGGL(ieee_fixup_kernel, dim3((unsigned)fb), dim3(256), 0, stream, A, lda, B, ldb, C, ldc, M, N, K,
                       row_flag, cols, count);
    return hipGetLastError();
}

}  // namespace sgemm_emu_dev
