// probe.hip -- a measurement aid, separate from the GEMM library: how fast the
// matrix pipes of gfx950 retire v_mfma_f32_32x32x16_bf16 when they do nothing
// else, on operands with random bits or with constant bits.
//
// Under a dense MFMA load the chip lowers its shader clock with the power it
// draws, and operands whose bits toggle draw more than constant ones.  This
// kernel measures that practical ceiling of the instruction the GEMM kernels
// are built on, to set beside the nominal peak (256 CUs x 2.4 GHz).  It is
// built into its own library (libsgemm_probe.so), which only the benchmark
// loads.
//
// Launch shape: one workgroup of 8 waves per CU (2 waves per SIMD, like the
// GEMM), pinned by a static LDS array larger than half the CU's LDS.  Each
// wave keeps four independent accumulators and rotates through four operand
// sets, so consecutive MFMAs see different bits and no MFMA waits for the
// previous result.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int kThreads = 512;       // 8 waves
constexpr int kSets = 4;            // operand sets per operand
constexpr int kAcc = 4;             // independent accumulators
constexpr int kMfmaPerIter = kSets * kAcc;
constexpr int kPinFloats = 96 * 1024 / 4;   // 96 KB of the CU's 160 KB: one workgroup per CU

// 32-bit integer hash (the "lowbias32" mixer published by C. Wellons): the
// random operand bits of lane `x`.
__device__ __forceinline__ uint32_t mix32(uint32_t x)
{
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

// BF16 bit pattern with a random sign and 7-bit mantissa and an exponent in
// [2^-4, 2^3], the magnitudes of split components of unit-scale data.
__device__ __forceinline__ uint16_t rand_bf16(uint32_t h)
{
    const uint32_t sign = (h >> 31) << 15;
    const uint32_t expo = 123u + ((h >> 7) & 7u);
    return (uint16_t)(sign | (expo << 7) | (h & 0x7Fu));
}

__device__ __forceinline__ bf16x8_t operand(uint32_t base, bool random)
{
    bf16x8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint16_t bits = random ? rand_bf16(mix32(base + (uint32_t)e)) : (uint16_t)0x3F80;   // 1.0
        v[e] = __builtin_bit_cast(__bf16, bits);
    }
    return v;
}

__global__ __launch_bounds__(kThreads, 1) void mfma_probe_kernel(int iters, int random, float *out)
{
    __shared__ float pin_lds[kPinFloats];
    const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
    const bool rnd = random != 0;
    bf16x8_t a[kSets], b[kSets];
#pragma unroll
    for (int s = 0; s < kSets; ++s) {
        a[s] = operand(tid * 128u + (uint32_t)s * 16u, rnd);
        b[s] = operand(tid * 128u + 64u + (uint32_t)s * 16u, rnd);
    }
    f32x16_t acc[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j) acc[j] = f32x16_t{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < kSets; ++i)
#pragma unroll
            for (int j = 0; j < kAcc; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + j) % kSets], acc[j], 0, 0, 0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += acc[j][e];
    out[tid] = sum;
    if (iters == -7) ((volatile float *)pin_lds)[threadIdx.x] = sum;   // never taken; keeps the LDS reserved
}

}  // namespace

extern "C" {

// Runs the probe: `blocks` workgroups of 512 threads, each wave issuing
// iters x 16 MFMAs (32x32x16 BF16, 32768 flops each).  random != 0 draws the
// operands from a hash of the lane index; 0 makes every operand 1.0.  `out`
// is a device buffer of blocks x 512 floats (one sum per lane, so the work
// cannot be dropped).  Returns 0, -1 for invalid arguments, -4 if the launch
// failed.  Asynchronous on `stream` (a hipStream_t).
int sgemm_probe_mfma(int blocks, int iters, int random, float *out, void *stream)
{
    if (blocks <= 0 || iters <= 0 || out == nullptr) return -1;
    hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, iters,
                       random, out);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Flops one call performs.
double sgemm_probe_mfma_flops(int blocks, int iters)
{
    return (double)blocks * (kThreads / 64) * (double)iters * kMfmaPerIter * 32.0 * 32.0 * 16.0 * 2.0;
}

}  // extern "C"
