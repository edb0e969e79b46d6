// launch.hpp -- internal launch interface between the C-ABI layer (api.hip)
// and the kernel files.  Not part of the public header.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgemm_emu_dev {

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// B operand source of the GEMM kernel.
enum BSource {
    B_FP32 = 0,        // FP32 K x N, split inside the GEMM
    B_PLANES_KN = 1,   // three BF16 planes, K x N row-major
    B_PLANES_NK = 2    // three BF16 planes, N x K row-major (B transposed, k contiguous)
};

struct GemmArgs {
    int64_t M, N, K;
    int64_t ka;              // K of A (== K, or less when the B planes are zero-padded to K)
    const float *A;
    int64_t lda;
    const float *B;          // B_FP32
    const uint16_t *A0;      // A as three BF16 planes M x K (lda), launch_gemm_planes only
    const uint16_t *A1;
    const uint16_t *A2;
    const uint16_t *B0;      // B_PLANES
    const uint16_t *B1;
    const uint16_t *B2;
    int64_t ldb;
    float *C;
    int64_t ldc;
    const float *bias;       // N values added to every row of C, or null
    int act;                 // activation applied last: 0 none, 1 GELU (erf form)
    int tiles_m, tiles_n;
    int group_m;             // tile-rows per group of the tile order
    int num_cus;             // compute units of the device (persistent grids)
    int splits;              // K slices of the native kernel (1 = none)
    float *partials;         // native: splits planes of M x ldp floats, one per K slice;
                             // stream-K: one 128 x 128 slot per workgroup
    int64_t ldp;
    void *done;              // host only: hipEvent_t to tie to the call's last kernel (or null)
    uint32_t *sk_flags;      // stream-K: one flag per workgroup (G words), zero or older epochs on entry
    uint32_t sk_epoch;       // stream-K: this launch's flag value (never 0)
    int sk_grid;             // stream-K: workgroups G (0: no stream-K)
    int sk_domains;          // stream-K: 1, or 8 (one block of tiles per XCD); set by the launcher
};

// rne: round each split stage to nearest even instead of truncating (ablation).
hipError_t launch_split(int64_t rows, int64_t cols, const float *X, int64_t ldx, uint16_t *X0,
                        uint16_t *X1, uint16_t *X2, int64_t ldo, int num_cus, hipStream_t stream,
                        bool rne = false);

// rows_out >= rows (0: rows): output columns rows .. rows_out-1 of the planes
// are written as zeros (a K extent padded for the plane kernel).
hipError_t launch_split_transpose(int64_t rows, int64_t cols, const float *X, int64_t ldx, uint16_t *X0,
                                  uint16_t *X1, uint16_t *X2, int64_t ldo, int num_cus, hipStream_t stream,
                                  bool rne = false, int64_t rows_out = 0);

// Three BF16 planes rows x cols (ldp) -> cols x rows_out (ldq), zero past
// rows; rows_out and ldq multiples of 8, 16-byte aligned outputs.
hipError_t launch_transpose_planes(int64_t rows, int64_t cols, const uint16_t *P0, const uint16_t *P1,
                                   const uint16_t *P2, int64_t ldp, uint16_t *Q0, uint16_t *Q1, uint16_t *Q2,
                                   int64_t ldq, int64_t rows_out, hipStream_t stream);

// rne: the in-kernel split of A (and of FP32 B) rounds to nearest even; only
// B_FP32 and B_PLANES_NK (DMA kernel) support it.  launch_gemm,
// launch_gemm_planes and launch_native tie args.done (if set) to the last
// kernel they launch on the N x K DMA, plane and native paths; the caller
// checks launch_done_attached() for the others.
hipError_t launch_gemm(const GemmArgs &args, int nbands, BSource bsrc, hipStream_t stream, bool rne = false);

// Both operands as BF16 planes with k contiguous: A0..A2 M x K (lda), B0..B2
// N x K (ldb); K a multiple of 64, leading dimensions multiples of 8,
// 16-byte aligned planes (else hipErrorInvalidValue, nothing launched).
hipError_t launch_gemm_planes(const GemmArgs &args, int nbands, hipStream_t stream);

// Stream-K for the N x K DMA kernel: the number of workgroups G sharing the
// shape's (tile, K pair) units, or 0 for the persistent kernel (where the
// persistent schedule's tile waves are not expected to be 10 % slower, K not
// a multiple of 64, too few units).
// A stream-K launch needs args.sk_flags (G words), args.partials (G x 128 x 128
// floats) and a nonzero args.sk_epoch that differs from the flags' values.
int gemm_streamk_grid(int64_t M, int64_t N, int64_t K, int num_cus);

// Most K pieces any tile is cut into by a stream-K grid of `grid` workgroups.
int gemm_streamk_pieces(int64_t M, int64_t N, int64_t K, int grid);

// True where the cost model expects the one-pass kernel on 64 x 64 tiles to
// be faster on FP32 B of this shape than 128 x 128 tiles: one pass per tile,
// or, if `streamk`, stream-K on planes split with K rounded up to a multiple
// of 64 where gemm_streamk_grid takes it.
bool gemm_tile64_pays(int64_t M, int64_t N, int64_t K, int num_cus, bool streamk);

// FP32 B (args.B, ldb) or N x K or K x N planes (args.B0..B2, ldb) on 64 x 64 tiles,
// one pass over K per tile: the same split, products and MFMA order as
// launch_gemm's one-pass kernels, so bitwise the same result.  Needs no
// workspace; leaves args.done unused.  RNE with planes (split already done)
// or another B source: hipErrorInvalidValue, nothing launched.
hipError_t launch_gemm_tile64(const GemmArgs &args, int nbands, BSource bsrc, hipStream_t stream,
                              bool rne = false);

// True when launch_gemm ties args.done to its last kernel for this call (the
// N x K DMA path).
bool launch_done_attached(const GemmArgs &args, BSource bsrc);

// True when launch_gemm takes the LDS-DMA kernel for N x K planes of this shape.
bool gemm_uses_dma(int64_t K, int64_t ldb, const void *B0, const void *B1, const void *B2);

// The library's native FP32 GEMM (v_mfma_f32_32x32x2_f32, no split): output
// tile 128 or 64, and the K slices it uses (> 1 needs args.partials with
// splits x M x N floats, ldp = N; the slices are added in order).
struct NativePlan {
    int tile;
    int splits;
};
// vec: native_vec() of the call's operands (the kernel's K step depends on it).
NativePlan native_plan(int64_t M, int64_t N, int64_t K, int num_cus, bool vec);
// True when the native kernel loads A and B 128 bits at a time.
bool native_vec(const float *A, int64_t lda, const float *B, int64_t ldb, int64_t K, int64_t N);
hipError_t launch_native(const GemmArgs &args, const NativePlan &plan, hipStream_t stream);

// C := act(0 + bias[j]) (K == 0); without bias and activation C := 0.
// Recompute, as plain FP32 dot products, every output of C = A B whose row of
// A or column of B holds an Inf or NaN.  work: 2 (M + N) + 1 ints.
hipError_t launch_ieee_fixup(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                             int64_t ldb, float *C, int64_t ldc, int *work, int num_cus, hipStream_t stream);

hipError_t launch_zero(int64_t M, int64_t N, float *C, int64_t ldc, const float *bias, int act, int num_cus,
                       hipStream_t stream);

}  // namespace sgemm_emu_dev
