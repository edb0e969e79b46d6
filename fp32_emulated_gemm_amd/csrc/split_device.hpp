// split_device.hpp -- device-side split of FP32 values into three scaled BF16
// components, shared by the standalone split kernel and the GEMM's staging.
//
// Definition (NVIDIA Technical Blog, "Unlocking Tensor Core Performance for
// Machine Learning Interatomic Potentials", Fig. 1 caption; discuss.pytorch.kr
// summary, section "Blackwell의 BF16x9"): x = x0 + 2^-8 x1 + 2^-16 x2, each
// piece carrying 8 significant bits.  Each stage rounds toward zero (RNE
// template argument: to nearest even instead, the rounding ablation):
//   x0 = high half of x's bit pattern,
//   t  = 2^8 (x - x0)            exact (at most 16 significant bits),
//   x1 = high half of t,
//   x2 = 2^8 (t - x1)            exact, at most 8 significant bits, so its
//                                 bit pattern already has a zero low half.
// The subtractions are exact provided FP32 subnormals are not flushed; the
// library is compiled with FP32 denormals enabled.
// Inf and NaN: t is NaN exactly when x is not finite (Inf - Inf, NaN - ...),
// which the callers use to take the rare fix-up path:
//   +-Inf -> (+-Inf, +0, +0);  NaN -> (high half with the quiet bit set, +0, +0).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm_emu_dev {

__device__ __forceinline__ uint32_t f2u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __uint_as_float(u); }

// Round an FP32 pattern to its high half (BF16) to nearest, ties to even, for
// the rounding ablation: adding 0x7FFF plus the kept half's last bit carries
// into the high half exactly when the dropped half lies above the midpoint
// (or on it with an odd kept half).  A carry that reaches the Inf exponent is
// undone (truncation), so a finite value never becomes Inf.
__device__ __forceinline__ uint32_t rne_hi(uint32_t u)
{
    const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    return ((r & 0x7F800000u) == 0x7F800000u) ? (u & 0xFFFF0000u) : r;
}

// The stage rounding: truncation (the method's reading), or nearest-even.
template <bool RNE>
__device__ __forceinline__ uint32_t hi_half(uint32_t u)
{
    if constexpr (RNE) return rne_hi(u);
    else return u & 0xFFFF0000u;
}

// Components of a finite x as FP32 bit patterns with zero low halves.
// Returns t = 2^8 (x - x0); t is NaN iff x is Inf or NaN.
template <bool RNE = false>
__device__ __forceinline__ float split_finite(float x, uint32_t &c0, uint32_t &c1, uint32_t &c2)
{
    c0 = hi_half<RNE>(f2u(x));
    float t = (x - u2f(c0)) * 256.0f;
    c1 = hi_half<RNE>(f2u(t));
    c2 = f2u((t - u2f(c1)) * 256.0f);
    return t;
}

// Overwrite the components of a non-finite x with the defined special split.
__device__ __forceinline__ void split_fix_special(float x, uint32_t &c0, uint32_t &c1, uint32_t &c2)
{
    uint32_t u = f2u(x);
    if ((u & 0x7F800000u) == 0x7F800000u) {
        c0 = (u & 0xFFFF0000u) | ((u & 0x007FFFFFu) ? 0x00400000u : 0u);
        c1 = 0u;
        c2 = 0u;
    }
}

// One dword holding two BF16 values: `lo` (high half of an FP32 pattern) in
// bits 0..15 and `hi` in bits 16..31.
__device__ __forceinline__ uint32_t pack_bf16x2(uint32_t lo, uint32_t hi)
{
    return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// Split 8 values assumed finite and pack each component into 4 dwords
// (element e in half e%2 of dword e/2).  Returns true if any input was Inf or
// NaN, in which case the packed words are not the defined split and the
// caller must redo the chunk with split8_packed.  Branch-free, so it can be
// interleaved with other work.
template <bool RNE = false>
__device__ __forceinline__ bool split8_packed_finite(const float (&x)[8], uint32_t (&p0)[4],
                                                     uint32_t (&p1)[4], uint32_t (&p2)[4])
{
    uint32_t c0[8], c1[8], c2[8];
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = split_finite<RNE>(x[e], c0[e], c1[e], c2[e]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p0[i] = pack_bf16x2(c0[2 * i], c0[2 * i + 1]);
        p1[i] = pack_bf16x2(c1[2 * i], c1[2 * i + 1]);
        p2[i] = pack_bf16x2(c2[2 * i], c2[2 * i + 1]);
    }
    // Any non-finite input makes its t NaN, and NaN survives the sum; finite
    // inputs can at worst overflow the sum to Inf (not NaN) or to Inf - Inf =
    // NaN, which only sends a finite chunk down the exact slow path.
    const float probe = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
    return probe != probe;
}

// Split 8 values of any class and pack each component into 4 dwords.
template <bool RNE = false>
__device__ __forceinline__ void split8_packed(const float (&x)[8], uint32_t (&p0)[4],
                                              uint32_t (&p1)[4], uint32_t (&p2)[4])
{
    uint32_t c0[8], c1[8], c2[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float t = split_finite<RNE>(x[e], c0[e], c1[e], c2[e]);
        if (t != t) split_fix_special(x[e], c0[e], c1[e], c2[e]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p0[i] = pack_bf16x2(c0[2 * i], c0[2 * i + 1]);
        p1[i] = pack_bf16x2(c1[2 * i], c1[2 * i + 1]);
        p2[i] = pack_bf16x2(c2[2 * i], c2[2 * i + 1]);
    }
}

}  // namespace sgemm_emu_dev
