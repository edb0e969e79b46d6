/*
 * sgemm_emu.h -- C ABI of libsgemm_emu: FP32 matrix multiplication emulated on
 * the BF16 matrix cores (MFMA) of AMD Instinct MI355X (gfx950).
 *
 * Method (NVIDIA Technical Blog, "Unlocking Tensor Core Performance for Machine
 * Learning Interatomic Potentials", section "How Tensor Core FP32 closes the
 * hardware gap", Fig. 1 and its caption; discuss.pytorch.kr summary of the same
 * post, section "Blackwell의 BF16x9: 세 조각, 아홉 번의 곱"):
 *   each FP32 operand x is split into three scaled BF16 components,
 *   x = x0 + 2^-8 x1 + 2^-16 x2, each carrying 8 significant bits;
 *   the nine pairwise products A_p * B_q run on BF16 matrix units with FP32
 *   accumulation, grouped into five anti-diagonal bands s = p + q;
 *   the bands are recombined with their weights 2^-8s, smallest band first.
 * Inputs and outputs stay FP32 (same section: "inputs and outputs remain FP32").
 *
 * Readings where the pages are silent (this library's definitions):
 *   - the split rounds toward zero at each stage: x0 = RZ_bf16(x),
 *     x1 = RZ_bf16(2^8 (x - x0)), x2 = 2^16 (x - x0 - 2^-8 x1) exactly;
 *   - +-Inf splits into (+-Inf, +0, +0); NaN into (quiet NaN with the sign and
 *     the high payload bits kept, +0, +0);
 *   - one FP32 accumulator per band over the whole K range; the epilogue forms
 *     acc = 2^-32 S4, acc = fma(S3, 2^-24, acc), acc = fma(S2, 2^-16, acc),
 *     acc = fma(S1, 2^-8, acc), C = acc + S0;
 *   - the order of additions inside a band is the matrix unit's; results are
 *     deterministic for a given shape, entry point and device (no atomics) but
 *     not bitwise equal to a sequential sum.  Partly filled tile grids share
 *     their (tile, K range) work among all CUs (stream-K, see sgemm_emu_split_k):
 *     each piece of a tile runs the method on its K range and the pieces' FP32
 *     results are added in K order; if the device memory for those partial
 *     results cannot be had, the call returns SGEMM_EMU_ENOMEM rather than
 *     round another way.  With FP32 B, some of those grids run one pass over K
 *     per 64 x 64 tile instead (see sgemm_emu_split_k_fp32_b).
 *   - non-finite inputs follow IEEE rules on the components (Inf times a zero
 *     component is NaN), so results are not IEEE-754 SGEMM results for them.
 *
 * Conventions shared by every entry point:
 *   Matrices are row-major.  A is M x K with A[i*lda + k]; B is K x N with
 *   B[k*ldb + j]; C is M x N with C[i*ldc + j].  C := A * B (no alpha, beta).
 *   All matrix pointers are DEVICE pointers on the current HIP device.  The
 *   caller owns every buffer; the library keeps no per-call state beyond the
 *   stream-ordered workspace described below.
 *   `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *   asynchronously; faults inside kernels surface at the caller's next
 *   synchronisation, as in BLAS libraries.
 *   Arguments are validated before any HIP call; on an error status nothing
 *   has been enqueued.
 *   Device memory: sgemm_bf16x9 and sgemm_emu with K' * N <= 2^28 (K' = K
 *   rounded up to a multiple of 64) split B once into an N x K' set of BF16
 *   planes, zero past K (6 K' N bytes), where that is faster than splitting
 *   B inside the GEMM kernel: when the tile grid takes stream-K (see
 *   sgemm_emu_split_k_fp32_b; any M), or when M >= 1024 and 2 M N K >= 1.2e10 (sgemm_emu_ex's
 *   SGEMM_EMU_PRESPLIT_B asks for it whenever M >= 1024 and K' N allow).
 *   sgemm_emu_presplit_b with K x N planes follows the same rule, with the
 *   planes transposed into the workspace instead of split.  Where B is
 *   split so and N >= 4096 (each A element would be split again in each of
 *   the N / 128 tile columns), with K % 64 == 0 and M K <= 2^28, A is split
 *   into workspace planes too (6 M K more bytes) and a kernel that copies
 *   both operands' planes runs (SGEMM_EMU_PRESPLIT_A asks for it whenever
 *   those allow).  All ways give bitwise the same result.  GEMMs on small
 *   tile grids also need stream-K partial slots (see sgemm_emu_split_k).  All of
 *   it lives in one grow-only
 *   workspace block per stream, which the stream's later calls reuse (stream
 *   order keeps them apart; an event recorded after each use orders the next
 *   user of the block, and calls from several host threads on one stream
 *   enqueue one after the other).  A device keeps such blocks for up to 8
 *   streams; a ninth stream takes over the least recently used block.  The
 *   blocks come from a memory pool the library creates per device
 *   (hipMallocFromPoolAsync on the calling stream) and stay allocated until
 *   sgemm_emu_release_workspace gives them back (or the process ends).  On a
 *   stream being captured into a graph the library allocates nothing.  If
 *   no workspace can be had (or the stream is capturing) the GEMM splits B
 *   inside its kernel (bitwise the same result); a small-grid shape whose
 *   stream-K partial slots cannot be had returns SGEMM_EMU_ENOMEM (while
 *   capturing: SGEMM_EMU_ECAPTURE) with nothing enqueued, so the bits of a
 *   shape never depend on the memory available.  Small grids that run on
 *   64 x 64 tiles (sgemm_emu_split_k_fp32_b returns 1 for FP32 B) use no
 *   workspace and capture like any other call.  Callers that must capture
 *   such shapes, or cannot let the library allocate, use
 *   sgemm_emu_presplit_b_noalloc.  No other device memory is allocated
 *   (sgemm_emu_ex's IEEE fix-up aside, documented there).  The
 *   pool, the blocks and their events belong to the device's primary
 *   context: after hipDeviceReset the library must not be called again in
 *   that process.
 *   Float pointers must be 4-byte aligned, BF16 plane pointers 2-byte aligned.
 *   16-byte aligned A with lda % 4 == 0 takes the vector-load path; any other
 *   layout takes a scalar-load path with the same arithmetic.
 *   Leading dimensions are limited to 8,388,544 elements (32-bit offsets
 *   inside a 128-row tile); larger ones give SGEMM_EMU_EINVAL.
 *   M == 0 or N == 0: nothing is done.  K == 0: C is set to zero (plus the
 *   bias, for sgemm_emu_linear).
 *   C must not overlap A or B (not checked).
 *   Column-major callers compute C^T = B^T A^T by swapping the operands.
 */
#ifndef SGEMM_EMU_H
#define SGEMM_EMU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *sgemm_emu_stream_t;

enum sgemm_emu_status {
    SGEMM_EMU_OK = 0,
    SGEMM_EMU_EINVAL = -1,  /* negative size, leading dimension too small, bad nbands,
                               misaligned pointer, or a size whose byte offsets overflow */
    SGEMM_EMU_ENULL = -2,   /* null pointer for an operand with a nonzero extent */
    SGEMM_EMU_EARCH = -3,   /* no HIP device, or the current device is not gfx950 */
    SGEMM_EMU_ELAUNCH = -4, /* the kernel launch itself failed (hipGetLastError), or a HIP call of
                               sgemm_emu_release_workspace failed */
    SGEMM_EMU_ENOMEM = -5,  /* a GEMM on a small tile grid could not get device memory for its
                               stream-K partial results (see sgemm_emu_split_k); nothing was enqueued */
    SGEMM_EMU_ECAPTURE = -6 /* the call needs workspace (stream-K partial results, the IEEE fix-up's
                               flags) and its stream is being captured into a graph, where the
                               library allocates nothing; nothing was enqueued */
};

/*
 * sgemm_bf16x9 -- C = A * B with all nine products (five bands).
 * Defined by the pages' BF16x9 scheme (see the top of this file).
 * A: M x K FP32 (lda >= max(1, K)); B: K x N FP32 (ldb >= max(1, N));
 * C: M x N FP32 (ldc >= max(1, N)), written, never read.
 * Returns SGEMM_EMU_OK or an error status.
 */
int sgemm_bf16x9(int64_t M, int64_t N, int64_t K,
                 const float *A, int64_t lda,
                 const float *B, int64_t ldb,
                 float *C, int64_t ldc,
                 sgemm_emu_stream_t stream);

/*
 * sgemm_emu -- band-drop / product-count variant: keeps only the bands
 * s = p + q < nbands.  nbands = 5, 4, 3, 2, 1 evaluates 9, 8, 6, 3, 1 products.
 * nbands = 2 is the TF32x3 form a_hi b_hi + a_hi b_lo + a_lo b_hi (NVIDIA blog,
 * same section, the equation under Fig. 2) built from BF16 components with
 * hi = x0 and lo = 2^-8 x1.  nbands = 5 is identical to sgemm_bf16x9.
 * Other arguments as sgemm_bf16x9; nbands outside 1..5 gives SGEMM_EMU_EINVAL.
 */
int sgemm_emu(int64_t M, int64_t N, int64_t K,
              const float *A, int64_t lda,
              const float *B, int64_t ldb,
              float *C, int64_t ldc,
              int nbands, sgemm_emu_stream_t stream);

/* Flags of sgemm_emu_ex and split_f32_bf16x3_ex. */
enum sgemm_emu_flags {
    SGEMM_EMU_SPLIT_RNE = 1,        /* rounding ablation: each split stage rounds to the nearest BF16,
                                       ties to even, never to Inf (a finite value that would round to
                                       Inf keeps its truncation), instead of truncating */
    SGEMM_EMU_SPLIT_TRANSPOSE = 2,  /* split_f32_bf16x3_ex only: write the planes of X^T */
    SGEMM_EMU_IEEE_SPECIALS = 4,    /* sgemm_emu_ex only: outputs whose row of A or column of B holds
                                       an Inf or NaN are recomputed as plain FP32 dot products (k
                                       ascending, product and sum rounded separately), so they follow
                                       IEEE-754 FP32 (+-Inf where the emulation's Inf x 0 component
                                       gives NaN); other outputs are unchanged.  Costs one more read
                                       of A and B and a pooled (2 (M + N) + 1)-int buffer. */
    SGEMM_EMU_PRESPLIT_B = 8,       /* sgemm_emu_ex only: split FP32 B once into workspace planes
                                       whenever M >= 1024 and K' N <= 2^28, not only where the default
                                       expects it to be faster (same result, bitwise) */
    SGEMM_EMU_PRESPLIT_A = 16,      /* sgemm_emu_ex only: as SGEMM_EMU_PRESPLIT_B, and split FP32 A
                                       into workspace planes too whenever K % 64 == 0 and M K <= 2^28,
                                       not only for N >= 4096 (same result, bitwise) */
    SGEMM_EMU_PERFORMANT = 32,      /* sgemm_emu_ex only, nbands 5, truncating split: the "performant"
                                       strategy -- all nine BF16 products only where the library expects
                                       them to be faster than its native FP32 kernel on this shape, the
                                       native FP32 kernel elsewhere (see sgemm_emu_ex) */
    SGEMM_EMU_NATIVE_FP32 = 64,     /* sgemm_emu_ex only, nbands 5, truncating split: always the native
                                       FP32 kernel (the strategy's other branch, on its own) */
    SGEMM_EMU_NO_WORKSPACE = 128    /* sgemm_emu_ex only, alone or with SGEMM_EMU_SPLIT_RNE: never use
                                       the stream's workspace -- B (and A) are split inside the GEMM
                                       kernel and every tile runs its whole K in one workgroup (no
                                       stream-K), so nothing is allocated, also while the stream is
                                       being captured; small grids then run slower, and their bits can
                                       differ from the default's (both within the same bound) */
};

/*
 * sgemm_emu_ex -- sgemm_emu with flags (SGEMM_EMU_SPLIT_RNE,
 * SGEMM_EMU_IEEE_SPECIALS, SGEMM_EMU_PRESPLIT_B, SGEMM_EMU_PRESPLIT_A,
 * SGEMM_EMU_PERFORMANT, SGEMM_EMU_NATIVE_FP32, SGEMM_EMU_NO_WORKSPACE; other
 * bits give SGEMM_EMU_EINVAL, and so does SGEMM_EMU_NO_WORKSPACE beside any
 * flag but SGEMM_EMU_SPLIT_RNE).
 * Strategy flags: the pages' cuBLAS integration offers an "eager" strategy
 * (emulate whenever the operation allows) and a "performant" one (emulate only
 * where a speed-up over native FP32 is expected) (NVIDIA blog, section "BF16x9
 * on NVIDIA Blackwell GPUs", Fig. 4; discuss.pytorch.kr summary, section
 * "PyTorch에서 직접 써 보려면").  Without a strategy flag every entry point is
 * eager.  With SGEMM_EMU_PERFORMANT the library runs its native FP32 kernel
 * (v_mfma_f32_32x32x2_f32: FP32 products, FP32 accumulation, one pass over K
 * per output, or K slices added in order on small tile grids) for GEMMs of
 * fewer than 2.5e9 flops (2 M N K), where it measured faster, and the
 * nine-product emulation otherwise; SGEMM_EMU_NATIVE_FP32 always runs the
 * native kernel.  The native kernel's results are IEEE FP32 dot products in
 * the matrix unit's order of additions (within the same elementwise bound as
 * the emulation); they differ in rounding from the emulation's.  Both flags
 * need nbands = 5 and no SGEMM_EMU_SPLIT_RNE (else SGEMM_EMU_EINVAL).  With SGEMM_EMU_SPLIT_RNE both A and B are split
 * with the round-to-nearest rule: with all nine products the result is the
 * same emulated product up to FP32 rounding (both splits are exact); with
 * fewer bands the dropped terms are about half as large and unsigned-biased
 * errors disappear.  The pages leave the rounding of the split open; the
 * library's default is truncation.
 */
int sgemm_emu_ex(int64_t M, int64_t N, int64_t K,
                 const float *A, int64_t lda,
                 const float *B, int64_t ldb,
                 float *C, int64_t ldc,
                 int nbands, int flags, sgemm_emu_stream_t stream);

/* Layouts of pre-split B planes (sgemm_emu_presplit_b). */
enum sgemm_emu_b_layout {
    SGEMM_EMU_B_KN = 0,  /* planes are K x N row-major: B0[k*ldb + j], as split_f32_bf16x3(B) gives */
    SGEMM_EMU_B_NK = 1   /* planes are N x K row-major: B0[j*ldb + k], as split_f32_bf16x3(B^T) gives,
                            e.g. from a linear layer's weight stored [out_features][in_features] */
};

/*
 * sgemm_emu_presplit_b -- as sgemm_emu, with B already split into its three
 * BF16 component planes by split_f32_bf16x3 (for weights split once and reused,
 * as the linear layers of an interatomic potential do).  B0, B1, B2 are uint16
 * BF16 bit patterns in the layout given by b_layout, with leading dimension
 * ldb >= max(1, N) for SGEMM_EMU_B_KN and ldb >= max(1, K) for SGEMM_EMU_B_NK.
 * A is split inside the kernel, or, with M >= 1024, N >= 4096, K % 64 == 0
 * and M K <= 2^28 (and planes the LDS-DMA kernel takes: N x K, or K x N
 * copied as below), once into M x K workspace planes as for sgemm_bf16x9
 * (6 M K bytes).  SGEMM_EMU_B_KN planes are copied once, transposed, into
 * N x K' workspace planes (6 K' N bytes; zero past K) where sgemm_bf16x9
 * would pre-split an FP32 B of this shape, since the kernel for N x K planes
 * copies them into LDS without passing through registers.  The result equals
 * sgemm_emu on the FP32 B bit for bit either way.  SGEMM_EMU_B_NK planes on a
 * partly filled tile grid that does not take stream-K (see sgemm_emu_split_k)
 * run one pass over K per 64 x 64 tile, through registers, where the cost model
 * of sgemm_emu_split_k_fp32_b expects that to be faster (the same bits as one
 * pass per 128 x 128 tile); SGEMM_EMU_B_KN planes with N and ldb even and
 * 4-byte aligned planes take 64 x 64 tiles wherever sgemm_bf16x9 does for
 * FP32 B of the shape (sgemm_emu_split_k_fp32_b returns their K pieces too),
 * other K x N planes only where they would not be copied into the workspace.
 * An unknown b_layout gives SGEMM_EMU_EINVAL.
 */
int sgemm_emu_presplit_b(int64_t M, int64_t N, int64_t K,
                         const float *A, int64_t lda,
                         const uint16_t *B0, const uint16_t *B1, const uint16_t *B2, int64_t ldb,
                         int b_layout,
                         float *C, int64_t ldc,
                         int nbands, sgemm_emu_stream_t stream);

/*
 * sgemm_emu_presplit_b_noalloc -- sgemm_emu_presplit_b with N x K planes
 * (SGEMM_EMU_B_NK layout, ldb >= max(1, K)) that allocates no device memory,
 * for callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same kernels and K
 * partition as sgemm_emu_presplit_b, so the same bits (the separate split of
 * A into workspace planes that sgemm_emu_presplit_b makes for N >= 4096 is
 * skipped; the kernel that splits A itself gives the same result).  The
 * stream-K partial results and flags of small tile grids go to a fixed array
 * in device memory, 16 MiB + 1 KiB per device (one 128 x 128 FP32 slot and one
 * flag word for each of at most 256 workgroups), held from the library's load
 * on the device until the process ends; a device whose stream-K grid would
 * have more workgroups (more than 256 CUs) gets SGEMM_EMU_ENOMEM for such
 * shapes.  All calls on one device share that array: calls that overlap in
 * time on one device (two streams, or two host threads) race on it and must
 * be ordered by the caller.  Each call marks its flags with a new value and
 * reads only slots whose flags carry it, so nothing needs clearing.  Other
 * arguments and errors as sgemm_emu_presplit_b.
 */
int sgemm_emu_presplit_b_noalloc(int64_t M, int64_t N, int64_t K,
                                 const float *A, int64_t lda,
                                 const uint16_t *B0, const uint16_t *B1, const uint16_t *B2, int64_t ldb,
                                 float *C, int64_t ldc,
                                 int nbands, sgemm_emu_stream_t stream);

/* Activation applied by sgemm_emu_linear after the bias. */
enum sgemm_emu_activation {
    SGEMM_EMU_ACT_NONE = 0,
    SGEMM_EMU_ACT_GELU = 1   /* GELU, exact (erf) form: 0.5 z (1 + erf(z / sqrt(2))) */
};

/*
 * sgemm_emu_linear -- the forward pass of a linear layer, Y = act(X W^T + bias), with
 * the weight held as a linear layer stores it, W[out_features][in_features],
 * and given as its three BF16 planes (split_f32_bf16x3 of W, split once and
 * reused).  The pages use the emulation as a drop-in for the FP32 matrix
 * multiplication inside such layers with the trained weights and shapes kept
 * (NVIDIA blog, section "TF32x3 on NVIDIA Ampere GPUs"; discuss.pytorch.kr
 * summary, section "PyTorch에서 직접 써 보려면").
 *   X: M x K FP32 (ldx >= max(1, K)); W0, W1, W2: N x K planes (ldw >= max(1, K));
 *   bias: N FP32 values or NULL; activation: SGEMM_EMU_ACT_NONE or
 *   SGEMM_EMU_ACT_GELU (anything else gives SGEMM_EMU_EINVAL);
 *   Y: M x N FP32 (ldy >= max(1, N)), written.
 * Z[i][j] = fl32(C[i][j] + bias[j]) where C is sgemm_emu_presplit_b(...,
 * SGEMM_EMU_B_NK, ...) on the same arguments: one FP32 rounding after the band
 * recombination.  With bias == NULL, Z equals C bit for bit.  Y = Z without an
 * activation; with SGEMM_EMU_ACT_GELU, Y = GELU(Z) in FP32 (erfc-based, a few
 * ulp from the correctly rounded value, fused into the GEMM's epilogue).  The input
 * gradient dX = dY W of the same layer is sgemm_emu_presplit_b(M, K, N, dY, ldy,
 * W0, W1, W2, ldw, SGEMM_EMU_B_KN, dX, ldx, nbands): the N x K planes of W are
 * the K x N planes of the backward product.  Faster, with the same bits: the
 * planes of W^T (split_f32_bf16x3_transposed of W) with SGEMM_EMU_B_NK.
 */
int sgemm_emu_linear(int64_t M, int64_t N, int64_t K,
                     const float *X, int64_t ldx,
                     const uint16_t *W0, const uint16_t *W1, const uint16_t *W2, int64_t ldw,
                     const float *bias, int activation,
                     float *Y, int64_t ldy,
                     int nbands, sgemm_emu_stream_t stream);

/*
 * split_f32_bf16x3 -- the split alone, as its own kernel: for every element of
 * the rows x cols FP32 matrix X (leading dimension ldx >= max(1, cols)) writes
 * its components to X0, X1, X2 (uint16 BF16 bit patterns, leading dimension
 * ldo >= max(1, cols)).  Bit-exact with the definition at the top of this file.
 */
int split_f32_bf16x3(int64_t rows, int64_t cols,
                     const float *X, int64_t ldx,
                     uint16_t *X0, uint16_t *X1, uint16_t *X2, int64_t ldo,
                     sgemm_emu_stream_t stream);

/*
 * split_f32_bf16x3_ex -- split_f32_bf16x3 with flags: SGEMM_EMU_SPLIT_RNE
 * (round-to-nearest split, see sgemm_emu_ex) and/or SGEMM_EMU_SPLIT_TRANSPOSE
 * (planes of X^T, cols x rows with ldo >= max(1, rows), as
 * split_f32_bf16x3_transposed).  Other flag bits give SGEMM_EMU_EINVAL.
 */
int split_f32_bf16x3_ex(int64_t rows, int64_t cols,
                        const float *X, int64_t ldx,
                        uint16_t *X0, uint16_t *X1, uint16_t *X2, int64_t ldo,
                        int flags, sgemm_emu_stream_t stream);

/*
 * split_f32_bf16x3_transposed -- the same split, written transposed: for the
 * rows x cols FP32 matrix X (ldx >= max(1, cols)), X0, X1, X2 receive the
 * components of X^T, a cols x rows matrix (leading dimension ldo >= max(1, rows)):
 * element X[r][c] lands at X0[c*ldo + r].  Turns a K x N operand into N x K
 * planes (SGEMM_EMU_B_NK), e.g. a linear layer's weight W [out][in] into the
 * planes the input gradient dX = dY W reads fastest.  Bit-exact with
 * split_f32_bf16x3 of the transposed matrix.
 */
int split_f32_bf16x3_transposed(int64_t rows, int64_t cols,
                                const float *X, int64_t ldx,
                                uint16_t *X0, uint16_t *X1, uint16_t *X2, int64_t ldo,
                                sgemm_emu_stream_t stream);

/*
 * sgemm_emu_split_k -- the largest number of pieces along K that any output
 * tile of an M x N x K product is cut into on the current device when the
 * GEMM runs the N x K plane kernel (sgemm_emu_presplit_b with SGEMM_EMU_B_NK
 * and sgemm_emu_linear, which need K % 64 == 0 and 16-byte aligned planes with
 * ldb % 8 == 0; sgemm_bf16x9 / sgemm_emu when they pre-split B, with K rounded
 * up to a multiple of 64).  1 means one pass over K per 128 x 128 output tile.
 * Grids whose tiles leave CUs idle (fewer tiles than CUs, or a last wave of
 * tiles that fills only part of the chip) are shared out stream-K style where
 * the library's cost model expects it to be at least 10 % faster: the (tile,
 * 64-wide K range) units, tile by tile, are cut into equal runs, one per
 * workgroup (at most one per CU, each run at least two units, at most 8
 * pieces per tile);
 * each piece of a tile runs the method on its K range (five band sums,
 * recombined smallest band first); the workgroup holding a tile's last K range
 * adds the other pieces' FP32 results (from the stream's workspace: a
 * 128 x 128 slot and a flag word per workgroup) in K order, then its own, then
 * the bias and activation.  Results differ in rounding from the one-pass order
 * (still within the same error bound) and are deterministic for a given shape
 * and device.  If that workspace cannot be had the GEMM returns
 * SGEMM_EMU_ENOMEM.  Returns the count >= 1, or a negative status (invalid
 * sizes or nbands, no gfx950 device).
 */
int sgemm_emu_split_k(int64_t M, int64_t N, int64_t K, int nbands);

/*
 * sgemm_emu_split_k_fp32_b -- the same count for sgemm_bf16x9 and sgemm_emu
 * (no flags) on FP32 B on the current device.  Where a tile grid leaves CUs
 * idle, the library weighs, with a cost model measured on MI355X, a kernel on
 * 64 x 64 tiles (four times the workgroups of 128 x 128 tiles; B split inside
 * each tile, one pass over K, no workspace) against 128 x 128 tiles: one pass
 * per tile, or, where sgemm_emu_split_k(M, N, K', nbands) > 1 (K' = K rounded
 * up to a multiple of 64), B split into N x K' workspace planes and stream-K.
 * Returns 1 where the GEMM runs one pass over K per tile (on either tile
 * size): its result is then bitwise that of SGEMM_EMU_NO_WORKSPACE (the same
 * split, products and MFMA order for each output).  Otherwise returns
 * sgemm_emu_split_k(M, N, K', nbands): the result is bitwise that of
 * sgemm_emu_presplit_b on those planes.  Returns a negative status as
 * sgemm_emu_split_k does.  Flags of sgemm_emu_ex can change the path:
 * SGEMM_EMU_PRESPLIT_B / _A with M >= 1024 keep the planes (and their
 * stream-K), SGEMM_EMU_NO_WORKSPACE never cuts K, SGEMM_EMU_SPLIT_RNE cuts K
 * only where K % 64 == 0.  The choice depends on the shape and the device's
 * CU count, never on the values.
 */
int sgemm_emu_split_k_fp32_b(int64_t M, int64_t N, int64_t K, int nbands);

/*
 * sgemm_emu_release_workspace -- gives back the workspace the library keeps on
 * the current device (the per-stream blocks described at the top of this file)
 * and trims the library's memory pool to zero, so the memory returns to the
 * device.  The pages keep the caller in charge of memory ("inputs and outputs
 * remain FP32", only the multiplication changes: NVIDIA blog, section "How
 * Tensor Core FP32 closes the hardware gap"); this call hands the library's
 * retained share back.  Waits on the host until the last call that used each
 * block has finished with it, then frees the blocks; GEMM calls from other
 * host threads wait for it (the table lock) and allocate afresh afterwards.
 * Blocks owned by graphs being captured or replayed are not affected.
 * Returns SGEMM_EMU_OK, SGEMM_EMU_EARCH (no gfx950 device current) or
 * SGEMM_EMU_ELAUNCH (a HIP call failed; the table is cleared regardless).
 */
int sgemm_emu_release_workspace(void);

/* Number of BF16 products evaluated for nbands (1, 3, 6, 8, 9), or -1 if invalid. */
int sgemm_emu_products(int nbands);

/* Static, human-readable text for a status code. */
const char *sgemm_emu_strerror(int status);

/* Library version string. */
const char *sgemm_emu_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_EMU_H */
