// api.hip -- the C ABI declared in include/sgemm_emu.h: argument validation,
// the gfx950 device check, and dispatch to the kernels.
//
// Every argument is checked before the first HIP call, so an invalid call
// returns an error status without touching the GPU (and works on machines
// without one).  The library keeps no state besides a per-device cache of
// "is this a gfx950", its CU count, a memory pool and a per-stream workspace
// table.  The only device memory it allocates is stream-ordered workspace: the
// planes of a pre-split FP32 B and the stream-K partial results of small tile
// grids (one
// grow-only block per stream, kept for the stream's later calls), and the
// flags of the IEEE fix-up (hipMallocFromPoolAsync / hipFreeAsync on the
// caller's stream, from the library's own pool).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/sgemm_emu.h"
#include "launch.hpp"

using namespace sgemm_emu_dev;

namespace {

constexpr int64_t kMaxBytes = INT64_MAX / 8;
// sgemm_bf16x9 / sgemm_emu pre-split FP32 B into a workspace from this many rows of A on
// (B is then split once instead of once per 128-row tile row), up to this B size.
constexpr int64_t kPresplitMinRows = 1024;
constexpr uint64_t kPresplitMaxElems = (uint64_t)1 << 28;
// ... and by default only where it pays: a separate split launch and the
// workspace cost a few microseconds, the in-kernel split of B a few percent of
// the GEMM; the in-kernel path also has no stream-K.  Measured on MI355X: the
// in-kernel split wins at 6144x1024x256 (85 vs 74 TFLOP/s) and
// 16384x256x1024 (125 vs 116), loses at 2048^3 (114 vs 123) and above.
constexpr double kPresplitMinFlops = 1.2e10;
// With B pre-split, FP32 A is split once into workspace planes too where N has
// this many columns: the kernel that splits A itself repeats that for each of
// the N / 128 tile columns, the plane kernel copies both operands by DMA.
// Measured on MI355X (A split included): 4096^3 +6-10 %, 8192^3 +2.5 %; at
// N = 1024 the separate split of A costs more than the kernel gains.
constexpr int64_t kPresplitAMinCols = 4096;
// Stream-K: one 128 x 128 FP32 partial slot per workgroup, and a flag word per
// workgroup at the head of every workspace block (at most 1024 workgroups).
constexpr size_t kSkSlotBytes = (size_t)128 * 128 * sizeof(float);
constexpr size_t kFlagBytes = 4096;
// Largest leading dimension (elements) whose 128-row tile span fits 32-bit byte offsets.
constexpr int64_t kMaxTileLd = ((int64_t)1 << 32) / (128 * 4) - 64;

// Largest element offset touched by a rows x cols matrix with leading dimension ld.
bool extent_ok(int64_t rows, int64_t cols, int64_t ld)
{
    if (rows == 0 || cols == 0) return true;
    if (rows - 1 > (kMaxBytes - cols) / ld) return false;
    return true;
}

int check_matrix(int64_t rows, int64_t cols, const void *p, int64_t ld, uintptr_t align)
{
    if (ld < (cols > 1 ? cols : 1)) return SGEMM_EMU_EINVAL;
    if (!extent_ok(rows, cols, ld)) return SGEMM_EMU_EINVAL;
    if (rows > 0 && cols > 0 && p == nullptr) return SGEMM_EMU_ENULL;
    if (((uintptr_t)p % align) != 0) return SGEMM_EMU_EINVAL;
    return SGEMM_EMU_OK;
}

int check_dims(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0) return SGEMM_EMU_EINVAL;
    // One workgroup per 128 x 128 tile; the grid is a 31-bit count.
    const int64_t tm = (M + 127) / 128, tn = (N + 127) / 128;
    if (tm > 0 && tn > (int64_t)0x7FFFFFFF / tm) return SGEMM_EMU_EINVAL;
    return SGEMM_EMU_OK;
}

struct DeviceInfo {
    int checked = 0;   // 0 unknown, 1 gfx950, -1 other
    int num_cus = 0;
    int pool_state = 0;           // 0 not tried, 1 created, -1 unavailable
    hipMemPool_t pool = nullptr;  // workspace pool, kept until the process ends
};

constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];
std::mutex g_mutex;

// Current device if it is a gfx950, with its CU count; SGEMM_EMU_EARCH otherwise.
int current_device(int *num_cus, int *device = nullptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return SGEMM_EMU_EARCH;
    }
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceInfo &d = g_devices[dev];
    if (d.checked == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return SGEMM_EMU_EARCH;
        }
        d.checked = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
        d.num_cus = prop.multiProcessorCount;
    }
    if (d.checked != 1) return SGEMM_EMU_EARCH;
    *num_cus = d.num_cus;
    if (device) *device = dev;
    return SGEMM_EMU_OK;
}

// The library's own stream-ordered memory pool on device `dev` (created on first
// use), or nullptr if pools are unavailable.  Its release threshold is
// unlimited, so freed workspace stays reserved for the next call instead of
// going back to the driver at each synchronisation.
hipMemPool_t workspace_pool(int dev)
{
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceInfo &d = g_devices[dev];
    if (d.pool_state == 0) {
        d.pool_state = -1;
        int supported = 0;
        if (hipDeviceGetAttribute(&supported, hipDeviceAttributeMemoryPoolsSupported, dev) == hipSuccess &&
            supported) {
            hipMemPoolProps props;
            memset(&props, 0, sizeof(props));
            props.allocType = hipMemAllocationTypePinned;
            props.handleTypes = hipMemHandleTypeNone;
            props.location.type = hipMemLocationTypeDevice;
            props.location.id = dev;
            hipMemPool_t pool = nullptr;
            if (hipMemPoolCreate(&pool, &props) == hipSuccess) {
                uint64_t keep = UINT64_MAX;
                (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
                d.pool = pool;
                d.pool_state = 1;
            }
        }
        (void)hipGetLastError();
    }
    return d.pool;
}

int launched(hipError_t e) { return e == hipSuccess ? SGEMM_EMU_OK : SGEMM_EMU_ELAUNCH; }

// ---------------------------------------------------------------- per-stream workspace
// A pooled allocate / free pair costs the host about as much as a small GEMM
// takes on the GPU.  So each stream keeps one grow-only workspace block that
// every later call on that stream reuses; stream order keeps the uses apart.
// A block is tagged with its stream's handle and with an event recorded after
// its last use.  A call first makes its stream wait for that event: this
// covers a stream destroyed with work pending whose handle comes back, and
// lets a full table hand a slot to a new stream (freeing or reusing the old
// block in stream order).
// The device's table lock is held from the lookup until the call's last
// launch, so calls from several host threads on one stream cannot interleave
// their kernels.  Nothing is allocated on a stream being captured into a
// graph (stream_capturing): the callers fall back to paths without workspace
// or report SGEMM_EMU_ECAPTURE.
struct StreamWs {
    bool used = false;
    uintptr_t key = 0;           // the stream handle
    void *ptr = nullptr;
    size_t bytes = 0;
    hipEvent_t done = nullptr;   // recorded on the stream after the last call that used ptr
    bool recorded = false;
    uint64_t tick = 0;           // last use, for eviction
    uint32_t epoch = 0;          // stream-K flag value of the block's last call (flags start at 0)
};

constexpr int kStreamSlots = 8;

struct DeviceWs {
    std::mutex mutex;
    StreamWs slot[kStreamSlots];
    uint64_t clock = 0;
};

DeviceWs g_ws[kMaxDevices];

// Lease on a workspace for one call; release() after the call's last launch.
struct WsLease {
    std::unique_lock<std::mutex> lock;
    StreamWs *entry = nullptr;
    hipStream_t stream = nullptr;
    uint32_t *flags = nullptr;   // the block's stream-K flags (its first kFlagBytes)
    uint32_t epoch = 0;          // this call's flag value

    // The event of the held block, for the launch helpers to tie to the call's
    // last kernel (a separate event record costs the stream a few microseconds).
    void *event() const { return entry != nullptr ? (void *)entry->done : nullptr; }

    // attached: the call's last kernel already carries the event.
    void release(bool attached = false)
    {
        if (entry != nullptr) entry->recorded = attached || hipEventRecord(entry->done, stream) == hipSuccess;
        entry = nullptr;
        if (lock.owns_lock()) lock.unlock();
    }
    ~WsLease() { release(); }
};

// True if `stream` is being captured into a graph (or its state cannot be
// read, which is treated the same way).
bool stream_capturing(hipStream_t stream)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return cs != hipStreamCaptureStatusNone;
}

// A workspace of at least `bytes` for `stream`, or nullptr if none can be had
// (the caller then runs without one).  Never allocates on a capturing stream.
// Every block starts with kFlagBytes of stream-K flags (zeroed when the block
// is allocated; each call gets the next epoch), then the caller's bytes.
void *acquire_workspace(int dev, hipStream_t stream, size_t bytes, WsLease &L)
{
    bytes += kFlagBytes;
    L.stream = stream;
    if (stream_capturing(stream)) return nullptr;
    hipMemPool_t pool = workspace_pool(dev);
    if (pool == nullptr) return nullptr;
    DeviceWs &D = g_ws[dev];
    L.lock = std::unique_lock<std::mutex>(D.mutex);
    StreamWs *e = nullptr;
    for (StreamWs &x : D.slot)
        if (x.used && x.key == (uintptr_t)stream) { e = &x; break; }
    if (e == nullptr) {
        for (StreamWs &x : D.slot)
            if (!x.used) { e = &x; break; }
        if (e == nullptr) {                       // table full: take the least recently used slot
            e = &D.slot[0];
            for (StreamWs &x : D.slot)
                if (x.tick < e->tick) e = &x;
        }
        if (e->done == nullptr && hipEventCreateWithFlags(&e->done, hipEventDisableTiming) != hipSuccess) {
            (void)hipGetLastError();
            e->done = nullptr;
            L.lock.unlock();
            return nullptr;
        }
        e->used = true;
        e->key = (uintptr_t)stream;
    }
    // after the last use of this block, whichever stream made it
    if (e->recorded && hipStreamWaitEvent(stream, e->done, 0) != hipSuccess) {
        (void)hipGetLastError();
        L.lock.unlock();
        return nullptr;
    }
    if (e->bytes < bytes) {
        if (e->ptr != nullptr) (void)hipFreeAsync(e->ptr, stream);
        e->ptr = nullptr;
        e->bytes = 0;
        const size_t grain = (size_t)2 << 20;
        const size_t want = (bytes + grain - 1) / grain * grain;
        void *p = nullptr;
        if (hipMallocFromPoolAsync(&p, want, pool, stream) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            L.lock.unlock();
            return nullptr;
        }
        if (hipMemsetAsync(p, 0, kFlagBytes, stream) != hipSuccess) {
            (void)hipGetLastError();
            (void)hipFreeAsync(p, stream);
            L.lock.unlock();
            return nullptr;
        }
        e->ptr = p;
        e->bytes = want;
        e->epoch = 0;
    }
    e->tick = ++D.clock;
    e->epoch = e->epoch == UINT32_MAX ? 1 : e->epoch + 1;
    L.entry = e;
    L.flags = (uint32_t *)e->ptr;
    L.epoch = e->epoch;
    return (char *)e->ptr + kFlagBytes;
}


// Every check of a GEMM call's arguments, before any HIP call.
int validate_gemm(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                  const uint16_t *B0, const uint16_t *B1, const uint16_t *B2, int64_t ldb, float *C,
                  int64_t ldc, int nbands, BSource bsrc, const float *bias, int act)
{
    int rc;
    if ((rc = check_dims(M, N, K)) != SGEMM_EMU_OK) return rc;
    if (nbands < 1 || nbands > 5) return SGEMM_EMU_EINVAL;
    // A and B only matter when the product is nonempty.
    const int64_t ma = (N > 0) ? M : 0, nb = (M > 0) ? N : 0;
    if ((rc = check_matrix(ma, K, A, lda, 4)) != SGEMM_EMU_OK) return rc;
    if (bsrc == B_FP32) {
        if ((rc = check_matrix(K, nb, B, ldb, 4)) != SGEMM_EMU_OK) return rc;
    } else {
        // planes are K x N, or N x K for the transposed layout
        const int64_t pr = (bsrc == B_PLANES_NK) ? nb : K, pc = (bsrc == B_PLANES_NK) ? K : nb;
        const int64_t rows = (pr > 0 && pc > 0) ? pr : 0;
        if ((rc = check_matrix(rows, pc, B0, ldb, 2)) != SGEMM_EMU_OK) return rc;
        if ((rc = check_matrix(rows, pc, B1, ldb, 2)) != SGEMM_EMU_OK) return rc;
        if ((rc = check_matrix(rows, pc, B2, ldb, 2)) != SGEMM_EMU_OK) return rc;
    }
    if ((rc = check_matrix(M, N, C, ldc, 4)) != SGEMM_EMU_OK) return rc;
    if (((uintptr_t)bias % 4) != 0) return SGEMM_EMU_EINVAL;
    if (act != SGEMM_EMU_ACT_NONE && act != SGEMM_EMU_ACT_GELU) return SGEMM_EMU_EINVAL;
    // The kernels address one K step of a 128 x 128 tile, and the C stores of a
    // 128-row tile, with 32-bit byte offsets.
    if (lda > kMaxTileLd || ldb > kMaxTileLd || ldc > kMaxTileLd) return SGEMM_EMU_EINVAL;
    return SGEMM_EMU_OK;
}

// True where the caller's N x K planes of this shape run on 64 x 64 tiles:
// where the plane kernel would not take stream-K and the cost model expects
// the 64 x 64 tiles to beat one pass per 128 x 128 tile.
static bool nk_tile64(int64_t M, int64_t N, int64_t K, const uint16_t *B0, const uint16_t *B1,
                      const uint16_t *B2, int64_t ldb, int num_cus)
{
    if (gemm_uses_dma(K, ldb, B0, B1, B2) && gemm_streamk_grid(M, N, K, num_cus) > 0) return false;
    return gemm_tile64_pays(M, N, K, num_cus, false);
}

// True where FP32 B may be split into N x K' planes for stream-K (K' = K
// rounded up to a multiple of 64): a workspace may be used, the planes are
// within the size limit, and the RNE split needs no K padding.
static bool fp32_b_streamk_allowed(int64_t N, int64_t K, bool rne, bool no_workspace)
{
    const int64_t kpad = (K + 63) / 64 * 64;
    return !no_workspace && (uint64_t)kpad * (uint64_t)N <= kPresplitMaxElems && !(rne && kpad != K);
}

// True where the caller's K x N planes of this shape run on 64 x 64 tiles.
static bool kn_tile64(int64_t M, int64_t N, int64_t K, const uint16_t *B0, const uint16_t *B1,
                      const uint16_t *B2, int64_t ldb, int num_cus, bool no_workspace)
{
    const bool pairs = ((uintptr_t)B0 | (uintptr_t)B1 | (uintptr_t)B2) % 4 == 0 && ldb % 2 == 0 && N % 2 == 0;
    const bool streamk = fp32_b_streamk_allowed(N, K, false, no_workspace);
    if (pairs) return gemm_tile64_pays(M, N, K, num_cus, streamk);
    const int64_t kpad = (K + 63) / 64 * 64;
    const bool transposed = streamk && (gemm_streamk_grid(M, N, kpad, num_cus) > 0 ||
                                        (M >= kPresplitMinRows && 2.0 * (double)M * (double)N * (double)K >=
                                                                      kPresplitMinFlops));
    return !transposed && gemm_tile64_pays(M, N, K, num_cus, false);
}

int gemm_common(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                const uint16_t *B0, const uint16_t *B1, const uint16_t *B2, int64_t ldb, float *C,
                int64_t ldc, int nbands, BSource bsrc, hipStream_t stream, const float *bias = nullptr,
                int act = SGEMM_EMU_ACT_NONE, bool rne = false, bool force_presplit = false,
                bool force_presplit_a = false, bool no_workspace = false)
{
    int rc;
    if ((rc = validate_gemm(M, N, K, A, lda, B, B0, B1, B2, ldb, C, ldc, nbands, bsrc, bias, act)) != SGEMM_EMU_OK)
        return rc;
    if (M == 0 || N == 0) return SGEMM_EMU_OK;

    int num_cus = 0, dev = 0;
    if ((rc = current_device(&num_cus, &dev)) != SGEMM_EMU_OK) return rc;
    if (K == 0) return launched(launch_zero(M, N, C, ldc, bias, act, num_cus, stream));

    GemmArgs g{};
    g.M = M; g.N = N; g.K = K; g.ka = K;
    g.A = A; g.lda = lda;
    g.B = B; g.B0 = B0; g.B1 = B1; g.B2 = B2; g.ldb = ldb;
    g.C = C; g.ldc = ldc;
    g.bias = bias;
    g.act = act;
    g.num_cus = num_cus;

    g.splits = 1;

    // FP32 B on a partly filled grid where the cost model expects the
    // one-pass kernel on 64 x 64 tiles (B split inside each tile, four times
    // the workgroups, no workspace) to beat 128 x 128 tiles, with or without
    // a split of B and stream-K: the same split, products and MFMA order as
    // the one-pass kernel on 128 x 128 tiles, so bitwise the result of
    // SGEMM_EMU_NO_WORKSPACE, and nothing allocated.
    const int64_t kpad = (K + 63) / 64 * 64;
    if (bsrc == B_FP32 && !(force_presplit && M >= kPresplitMinRows) &&
        gemm_tile64_pays(M, N, K, num_cus, fp32_b_streamk_allowed(N, K, rne, no_workspace)))
        return launched(launch_gemm_tile64(g, nbands, B_FP32, stream, rne));
    // The caller's N x K planes where stream-K would not run (or cannot: K not
    // a multiple of 64, unaligned planes): 64 x 64 tiles against one pass per
    // 128 x 128 tile, by the same model (bitwise the same result).
    if (bsrc == B_PLANES_NK && nk_tile64(M, N, K, B0, B1, B2, ldb, num_cus))
        return launched(launch_gemm_tile64(g, nbands, B_PLANES_NK, stream));
    // K x N planes read as column pairs follow FP32 B's rule: the alternative
    // is their transposition into N x K planes plus stream-K, as the split is
    // for FP32 B.  Element by element (odd N or ldb) the 64 x 64 tiles lose to
    // the transposition wherever that runs, so only one pass per 128 x 128
    // tile is weighed against them.
    if (bsrc == B_PLANES_KN && kn_tile64(M, N, K, B0, B1, B2, ldb, num_cus, no_workspace))
        return launched(launch_gemm_tile64(g, nbands, B_PLANES_KN, stream));

    // FP32 B with many tile rows: split B once into N x K planes in a
    // stream-ordered workspace and run the LDS-DMA kernel, instead of splitting
    // B again in every tile row.  Same split, same products, same order of
    // MFMA accumulation, so the result is bitwise identical (zero-padded K
    // steps add zero products).  A K that is not a multiple of 64 is padded in
    // the planes (zeros) and the kernel masks A past its K.
    // Where pays: grids small enough for stream-K (which only the DMA kernel
    // runs, whatever M), and from M >= 1024 rows large GEMMs.
    const bool small_grid = !no_workspace && gemm_streamk_grid(M, N, kpad, num_cus) > 0;
    const bool large = !no_workspace && M >= kPresplitMinRows &&
                       2.0 * (double)M * (double)N * (double)K >= kPresplitMinFlops;
    const bool presplit = bsrc == B_FP32 && (uint64_t)kpad * (uint64_t)N <= kPresplitMaxElems &&
                          !(rne && kpad != K) &&
                          ((force_presplit && M >= kPresplitMinRows) || small_grid || large);
    // K x N planes, by the same rule: transposed once into N x K' planes in the
    // workspace, so the LDS-DMA kernel runs instead of the kernel that stages
    // K x N planes through registers (same planes and products, same order:
    // bitwise the same result).
    const bool transpose_kn = bsrc == B_PLANES_KN && (uint64_t)kpad * (uint64_t)N <= kPresplitMaxElems && !rne &&
                              (small_grid || large);
    const size_t plane = (presplit || transpose_kn) ? (size_t)N * (size_t)kpad * sizeof(uint16_t) : 0;
    const size_t plane_pad = (plane + 255) & ~(size_t)255;
    // A as well (K needs no padding; A's planes are M x K, k contiguous), also
    // beside a caller's N x K planes that the DMA kernel reads as they are.
    const bool nk_dma = bsrc == B_PLANES_NK && gemm_uses_dma(K, ldb, B0, B1, B2);
    // Grids that would leave CUs idle on the N x K DMA kernel share the (tile,
    // K pair) units among all CUs (stream-K): partial slots and flags in the
    // workspace.  Stream-K splits A inside the kernel.
    const bool dma = presplit || transpose_kn || nk_dma;
    const int skg = dma && !no_workspace ? gemm_streamk_grid(M, N, (presplit || transpose_kn) ? kpad : K, num_cus) : 0;
#ifdef SGEMM_EMU_SERIAL_LDS
    const bool serial_debug = true;                    // the debug build splits A in its one kernel
#else
    const bool serial_debug = false;
#endif
    const bool presplit_a = !no_workspace && !serial_debug &&
                            (presplit || transpose_kn || (nk_dma && M >= kPresplitMinRows)) &&
                            kpad == K &&
                            (uint64_t)M * (uint64_t)K <= kPresplitMaxElems && skg == 0 &&
                            (force_presplit_a || N >= kPresplitAMinCols);
    const size_t aplane = presplit_a ? (size_t)M * (size_t)K * sizeof(uint16_t) : 0;
    const size_t aplane_pad = (aplane + 255) & ~(size_t)255;

    const size_t part_bytes = skg > 0 ? (size_t)skg * kSkSlotBytes : 0;
    const size_t part_pad = (part_bytes + 255) & ~(size_t)255;   // keeps A's planes 256-byte aligned

    // The stream's workspace block holds the planes and the partials.  Without
    // one the GEMM splits B itself (bitwise the same result); a stream-K shape
    // cannot run without its partial slots (one pass per tile would round
    // differently), so it reports SGEMM_EMU_ENOMEM with nothing enqueued.
    WsLease lease;
    void *ws = nullptr;
    if (plane_pad + part_pad + aplane_pad > 0)
        ws = acquire_workspace(dev, stream, 3 * plane_pad + part_pad + 3 * aplane_pad, lease);
    if (ws == nullptr && skg > 0) return stream_capturing(stream) ? SGEMM_EMU_ECAPTURE : SGEMM_EMU_ENOMEM;
    if (ws != nullptr && presplit) {
        uint16_t *P0 = (uint16_t *)ws, *P1 = (uint16_t *)((char *)ws + plane_pad),
                 *P2 = (uint16_t *)((char *)ws + 2 * plane_pad);
        const hipError_t e = launch_split_transpose(K, N, B, ldb, P0, P1, P2, kpad, num_cus, stream, rne, kpad);
        if (e != hipSuccess) return launched(e);
        g.B0 = P0; g.B1 = P1; g.B2 = P2; g.ldb = kpad;
        g.K = kpad;
        bsrc = B_PLANES_NK;
    }
    if (ws != nullptr && transpose_kn) {
        uint16_t *P0 = (uint16_t *)ws, *P1 = (uint16_t *)((char *)ws + plane_pad),
                 *P2 = (uint16_t *)((char *)ws + 2 * plane_pad);
        const hipError_t e = launch_transpose_planes(K, N, B0, B1, B2, ldb, P0, P1, P2, kpad, kpad, stream);
        if (e != hipSuccess) return launched(e);
        g.B0 = P0; g.B1 = P1; g.B2 = P2; g.ldb = kpad;
        g.K = kpad;
        bsrc = B_PLANES_NK;
    }
    if (ws != nullptr && skg > 0) {
        g.sk_grid = skg;
        g.sk_flags = lease.flags;
        g.sk_epoch = lease.epoch;
        g.partials = (float *)((char *)ws + 3 * plane_pad);
    }
    if (ws != nullptr && presplit_a) {
        char *const a_ws = (char *)ws + 3 * plane_pad + part_pad;
        uint16_t *Q0 = (uint16_t *)a_ws, *Q1 = (uint16_t *)(a_ws + aplane_pad),
                 *Q2 = (uint16_t *)(a_ws + 2 * aplane_pad);
        hipError_t e = launch_split(M, K, A, lda, Q0, Q1, Q2, K, num_cus, stream, rne);
        if (e == hipSuccess) {
            g.A0 = Q0; g.A1 = Q1; g.A2 = Q2; g.lda = K;
            g.done = lease.event();
            e = launch_gemm_planes(g, nbands, stream);
        }
        lease.release(e == hipSuccess && g.done != nullptr);
        return launched(e);
    }

    g.done = lease.event();
    const hipError_t e = launch_gemm(g, nbands, bsrc, stream, rne);
    lease.release(e == hipSuccess && g.done != nullptr && launch_done_attached(g, bsrc));
    return launched(e);
}

// ---------------------------------------------------------------- native FP32
// C = A B with FP32 products and FP32 accumulation on the FP32 matrix
// instruction (the library's native path; sgemm_emu_ex's strategy flags).
int gemm_native(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B, int64_t ldb,
                float *C, int64_t ldc, hipStream_t stream)
{
    int rc;
    if ((rc = validate_gemm(M, N, K, A, lda, B, nullptr, nullptr, nullptr, ldb, C, ldc, 5, B_FP32, nullptr,
                            SGEMM_EMU_ACT_NONE)) != SGEMM_EMU_OK)
        return rc;
    if (M == 0 || N == 0) return SGEMM_EMU_OK;
    int num_cus = 0, dev = 0;
    if ((rc = current_device(&num_cus, &dev)) != SGEMM_EMU_OK) return rc;
    if (K == 0) return launched(launch_zero(M, N, C, ldc, nullptr, SGEMM_EMU_ACT_NONE, num_cus, stream));
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K; g.ka = K;
    g.A = A; g.lda = lda;
    g.B = B; g.ldb = ldb;
    g.C = C; g.ldc = ldc;
    g.act = SGEMM_EMU_ACT_NONE;
    g.num_cus = num_cus;
    g.splits = 1;
    const NativePlan plan = native_plan(M, N, K, num_cus, native_vec(A, lda, B, ldb, K, N));
    WsLease lease;
    if (plan.splits > 1) {
        void *ws = acquire_workspace(dev, stream, (size_t)plan.splits * (size_t)M * (size_t)N * sizeof(float), lease);
        if (ws == nullptr) return stream_capturing(stream) ? SGEMM_EMU_ECAPTURE : SGEMM_EMU_ENOMEM;
        g.partials = (float *)ws;
        g.ldp = N;
    }
    g.done = lease.event();
    const hipError_t e = launch_native(g, plan, stream);
    lease.release(e == hipSuccess && g.done != nullptr);
    return launched(e);
}

// The performant strategy's choice (sgemm_emu_ex with SGEMM_EMU_PERFORMANT):
// true where the native FP32 kernel is expected to be faster than all nine
// BF16 products.  Measured on MI355X (256 CUs): the native kernel wins on every
// shape up to 1024^3 (2.1 GFLOP; 512^3 18.2 against 17.4 TFLOP/s, 768^3 46.1
// against 39.7, 1024^3 85.5 against 75.5), where latency weighs on the nine
// products; from 3.2 GFLOP up the emulation is level or ahead
// (1536 x 1024 x 1024 81.3 against 80.9, 6144 x 256 x 1024 86.4 against 80.7,
// 6144 x 1024 x 256 97.6 against 88.0, 4096^3 154.4 against 132.8), with
// 2048 x 1024 x 1024 the exception (105.5 against 108.5).
constexpr double kPerformantMinFlops = 2.5e9;

bool performant_prefers_native(int64_t M, int64_t N, int64_t K, int num_cus)
{
    (void)num_cus;
    return 2.0 * (double)M * (double)N * (double)K < kPerformantMinFlops;
}

// ---------------------------------------------------------------- fixed scratch
// sgemm_emu_presplit_b_noalloc keeps the stream-K partial slots and flags of
// small tile grids in this array instead of allocated workspace: one 128 x 128
// slot per workgroup (at most one workgroup per CU, 256 on MI355X), then one
// flag word per workgroup: 16 MiB + 1 KiB.  Each device holds its own copy for
// the life of the process (zero-initialised, as the flags need).  In host code
// the array's name is only a stand-in for it; the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kScratchSlots = 256;
constexpr size_t kScratchFloats = kScratchSlots * 128 * 128 + kScratchSlots;
static __device__ __align__(256) float scratch[kScratchFloats];

struct ScratchAddr {
    int state = 0;        // 0 not looked up, 1 known, -1 lookup failed
    float *ptr = nullptr;
    uint32_t epoch = 0;   // stream-K flag value of the last call on this device
};
ScratchAddr g_scratch[kMaxDevices];

// Device address of `scratch` on device `dev` (the current device), or nullptr;
// *epoch receives the next flag value for a call.
float *scratch_address(int dev, uint32_t *epoch)
{
    std::lock_guard<std::mutex> lock(g_mutex);
    ScratchAddr &a = g_scratch[dev];
    if (a.state == 0) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess && p != nullptr) {
            a.ptr = (float *)p;
            a.state = 1;
        } else {
            (void)hipGetLastError();
            a.state = -1;
        }
    }
    a.epoch = a.epoch == UINT32_MAX ? 1 : a.epoch + 1;
    *epoch = a.epoch;
    return a.ptr;
}

// sgemm_emu_presplit_b with N x K planes, no device memory allocated: the
// same kernels and K partition as that entry point (its separate split of A
// into planes is skipped; the kernel that splits A itself gives the same
// bits), with the stream-K partial slots and flags in `scratch`.
int gemm_noalloc(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const uint16_t *B0,
                 const uint16_t *B1, const uint16_t *B2, int64_t ldb, float *C, int64_t ldc, int nbands,
                 hipStream_t stream)
{
    int rc;
    if ((rc = validate_gemm(M, N, K, A, lda, nullptr, B0, B1, B2, ldb, C, ldc, nbands, B_PLANES_NK, nullptr,
                            SGEMM_EMU_ACT_NONE)) != SGEMM_EMU_OK)
        return rc;
    if (M == 0 || N == 0) return SGEMM_EMU_OK;
    int num_cus = 0, dev = 0;
    if ((rc = current_device(&num_cus, &dev)) != SGEMM_EMU_OK) return rc;
    if (K == 0) return launched(launch_zero(M, N, C, ldc, nullptr, SGEMM_EMU_ACT_NONE, num_cus, stream));
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K; g.ka = K;
    g.A = A; g.lda = lda;
    g.B0 = B0; g.B1 = B1; g.B2 = B2; g.ldb = ldb;
    g.C = C; g.ldc = ldc;
    g.act = SGEMM_EMU_ACT_NONE;
    g.num_cus = num_cus;
    g.splits = 1;
    if (nk_tile64(M, N, K, B0, B1, B2, ldb, num_cus))
        return launched(launch_gemm_tile64(g, nbands, B_PLANES_NK, stream));
    const int skg = gemm_uses_dma(K, ldb, B0, B1, B2) ? gemm_streamk_grid(M, N, K, num_cus) : 0;
    if (skg > 0) {
        if ((size_t)skg > kScratchSlots) return SGEMM_EMU_ENOMEM;
        uint32_t epoch = 0;
        float *p = scratch_address(dev, &epoch);
        if (p == nullptr) return SGEMM_EMU_ELAUNCH;
        g.sk_grid = skg;
        g.partials = p;
        g.sk_flags = (uint32_t *)(p + kScratchSlots * 128 * 128);
        g.sk_epoch = epoch;
    }
    return launched(launch_gemm(g, nbands, B_PLANES_NK, stream, false));
}

}  // namespace

extern "C" {

int sgemm_bf16x9(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B,
                 int64_t ldb, float *C, int64_t ldc, sgemm_emu_stream_t stream)
{
    return gemm_common(M, N, K, A, lda, B, nullptr, nullptr, nullptr, ldb, C, ldc, 5, B_FP32,
                       (hipStream_t)stream);
}

int sgemm_emu(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B, int64_t ldb,
              float *C, int64_t ldc, int nbands, sgemm_emu_stream_t stream)
{
    return gemm_common(M, N, K, A, lda, B, nullptr, nullptr, nullptr, ldb, C, ldc, nbands, B_FP32,
                       (hipStream_t)stream);
}

int sgemm_emu_ex(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B, int64_t ldb,
                 float *C, int64_t ldc, int nbands, int flags, sgemm_emu_stream_t stream)
{
    if ((flags & ~(SGEMM_EMU_SPLIT_RNE | SGEMM_EMU_IEEE_SPECIALS | SGEMM_EMU_PRESPLIT_B | SGEMM_EMU_PRESPLIT_A |
                   SGEMM_EMU_PERFORMANT | SGEMM_EMU_NATIVE_FP32 | SGEMM_EMU_NO_WORKSPACE)) != 0)
        return SGEMM_EMU_EINVAL;
    // no workspace: only the split's rounding may be chosen beside it
    if ((flags & SGEMM_EMU_NO_WORKSPACE) && (flags & ~(SGEMM_EMU_NO_WORKSPACE | SGEMM_EMU_SPLIT_RNE)) != 0)
        return SGEMM_EMU_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    int rc;
    // The strategy flags choose between all nine products and native FP32, so
    // they take nbands = 5 and the default (truncating) split only.
    const bool strategy = (flags & (SGEMM_EMU_PERFORMANT | SGEMM_EMU_NATIVE_FP32)) != 0;
    if (strategy && (nbands != 5 || (flags & SGEMM_EMU_SPLIT_RNE))) return SGEMM_EMU_EINVAL;
    if ((flags & SGEMM_EMU_IEEE_SPECIALS) && M > 0 && N > 0 && K > 0) {
        // the fix-up needs a flag buffer: refuse before anything is enqueued
        if ((rc = validate_gemm(M, N, K, A, lda, B, nullptr, nullptr, nullptr, ldb, C, ldc, nbands, B_FP32, nullptr,
                                SGEMM_EMU_ACT_NONE)) != SGEMM_EMU_OK)
            return rc;
        int num_cus = 0;
        if ((rc = current_device(&num_cus)) != SGEMM_EMU_OK) return rc;
        if (stream_capturing(s)) return SGEMM_EMU_ECAPTURE;
    }
    bool native = (flags & SGEMM_EMU_NATIVE_FP32) != 0;
    if ((flags & SGEMM_EMU_PERFORMANT) && !native) {
        if ((rc = validate_gemm(M, N, K, A, lda, B, nullptr, nullptr, nullptr, ldb, C, ldc, 5, B_FP32, nullptr,
                                SGEMM_EMU_ACT_NONE)) != SGEMM_EMU_OK)
            return rc;
        int num_cus = 0;
        if (M > 0 && N > 0 && (rc = current_device(&num_cus)) != SGEMM_EMU_OK) return rc;
        native = M > 0 && N > 0 && performant_prefers_native(M, N, K, num_cus);
    }
    if (native)
        rc = gemm_native(M, N, K, A, lda, B, ldb, C, ldc, s);
    else
        rc = gemm_common(M, N, K, A, lda, B, nullptr, nullptr, nullptr, ldb, C, ldc, nbands, B_FP32, s, nullptr,
                         SGEMM_EMU_ACT_NONE, (flags & SGEMM_EMU_SPLIT_RNE) != 0,
                         (flags & (SGEMM_EMU_PRESPLIT_B | SGEMM_EMU_PRESPLIT_A)) != 0,
                         (flags & SGEMM_EMU_PRESPLIT_A) != 0, (flags & SGEMM_EMU_NO_WORKSPACE) != 0);
    if (rc != SGEMM_EMU_OK || !(flags & SGEMM_EMU_IEEE_SPECIALS) || M == 0 || N == 0 || K == 0) return rc;
    // IEEE fix-up of the outputs touched by non-finite inputs (flags and a
    // column list in a pooled stream-ordered buffer)
    int num_cus = 0, dev = 0;
    if ((rc = current_device(&num_cus, &dev)) != SGEMM_EMU_OK) return rc;
    hipMemPool_t pool = workspace_pool(dev);
    if (pool == nullptr) return SGEMM_EMU_ELAUNCH;
    void *work = nullptr;
    const size_t bytes = (size_t)(2 * (M + N) + 1) * sizeof(int);
    if (hipMallocFromPoolAsync(&work, bytes, pool, s) != hipSuccess || work == nullptr) {
        (void)hipGetLastError();
        return SGEMM_EMU_ELAUNCH;
    }
    hipError_t e = launch_ieee_fixup(M, N, K, A, lda, B, ldb, C, ldc, (int *)work, num_cus, s);
    const hipError_t f = hipFreeAsync(work, s);
    return launched(e == hipSuccess ? f : e);
}

int sgemm_emu_presplit_b(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const uint16_t *B0,
                         const uint16_t *B1, const uint16_t *B2, int64_t ldb, int b_layout, float *C,
                         int64_t ldc, int nbands, sgemm_emu_stream_t stream)
{
    if (b_layout != SGEMM_EMU_B_KN && b_layout != SGEMM_EMU_B_NK) return SGEMM_EMU_EINVAL;
    return gemm_common(M, N, K, A, lda, nullptr, B0, B1, B2, ldb, C, ldc, nbands,
                       b_layout == SGEMM_EMU_B_NK ? B_PLANES_NK : B_PLANES_KN, (hipStream_t)stream);
}

int sgemm_emu_linear(int64_t M, int64_t N, int64_t K, const float *X, int64_t ldx, const uint16_t *W0,
                     const uint16_t *W1, const uint16_t *W2, int64_t ldw, const float *bias, int activation,
                     float *Y, int64_t ldy, int nbands, sgemm_emu_stream_t stream)
{
    return gemm_common(M, N, K, X, ldx, nullptr, W0, W1, W2, ldw, Y, ldy, nbands, B_PLANES_NK,
                       (hipStream_t)stream, bias, activation);
}

int sgemm_emu_presplit_b_noalloc(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const uint16_t *B0,
                                 const uint16_t *B1, const uint16_t *B2, int64_t ldb, float *C, int64_t ldc,
                                 int nbands, sgemm_emu_stream_t stream)
{
    return gemm_noalloc(M, N, K, A, lda, B0, B1, B2, ldb, C, ldc, nbands, (hipStream_t)stream);
}

int split_f32_bf16x3(int64_t rows, int64_t cols, const float *X, int64_t ldx, uint16_t *X0, uint16_t *X1,
                     uint16_t *X2, int64_t ldo, sgemm_emu_stream_t stream)
{
    int rc;
    if (rows < 0 || cols < 0) return SGEMM_EMU_EINVAL;
    if ((rc = check_matrix(rows, cols, X, ldx, 4)) != SGEMM_EMU_OK) return rc;
    if ((rc = check_matrix(rows, cols, X0, ldo, 2)) != SGEMM_EMU_OK) return rc;
    if ((rc = check_matrix(rows, cols, X1, ldo, 2)) != SGEMM_EMU_OK) return rc;
    if ((rc = check_matrix(rows, cols, X2, ldo, 2)) != SGEMM_EMU_OK) return rc;
    if (rows == 0 || cols == 0) return SGEMM_EMU_OK;
    int num_cus = 0;
    if ((rc = current_device(&num_cus)) != SGEMM_EMU_OK) return rc;
    return launched(launch_split(rows, cols, X, ldx, X0, X1, X2, ldo, num_cus, (hipStream_t)stream));
}

int split_f32_bf16x3_ex(int64_t rows, int64_t cols, const float *X, int64_t ldx, uint16_t *X0, uint16_t *X1,
                        uint16_t *X2, int64_t ldo, int flags, sgemm_emu_stream_t stream)
{
    int rc;
    if ((flags & ~(SGEMM_EMU_SPLIT_RNE | SGEMM_EMU_SPLIT_TRANSPOSE)) != 0) return SGEMM_EMU_EINVAL;
    const bool rne = (flags & SGEMM_EMU_SPLIT_RNE) != 0, tr = (flags & SGEMM_EMU_SPLIT_TRANSPOSE) != 0;
    // planes are rows x cols, or cols x rows when transposed
    const int64_t pr = tr ? cols : rows, pc = tr ? rows : cols;
    if (rows < 0 || cols < 0) return SGEMM_EMU_EINVAL;
    if ((rc = check_matrix(rows, cols, X, ldx, 4)) != SGEMM_EMU_OK) return rc;
    if ((rc = check_matrix(pr, pc, X0, ldo, 2)) != SGEMM_EMU_OK) return rc;
    if ((rc = check_matrix(pr, pc, X1, ldo, 2)) != SGEMM_EMU_OK) return rc;
    if ((rc = check_matrix(pr, pc, X2, ldo, 2)) != SGEMM_EMU_OK) return rc;
    if (rows == 0 || cols == 0) return SGEMM_EMU_OK;
    int num_cus = 0;
    if ((rc = current_device(&num_cus)) != SGEMM_EMU_OK) return rc;
    hipStream_t s = (hipStream_t)stream;
    return launched(tr ? launch_split_transpose(rows, cols, X, ldx, X0, X1, X2, ldo, num_cus, s, rne)
                       : launch_split(rows, cols, X, ldx, X0, X1, X2, ldo, num_cus, s, rne));
}

int split_f32_bf16x3_transposed(int64_t rows, int64_t cols, const float *X, int64_t ldx, uint16_t *X0,
                                uint16_t *X1, uint16_t *X2, int64_t ldo, sgemm_emu_stream_t stream)
{
    return split_f32_bf16x3_ex(rows, cols, X, ldx, X0, X1, X2, ldo, SGEMM_EMU_SPLIT_TRANSPOSE, stream);
}

int sgemm_emu_split_k(int64_t M, int64_t N, int64_t K, int nbands)
{
    int rc;
    if ((rc = check_dims(M, N, K)) != SGEMM_EMU_OK) return rc;
    if (nbands < 1 || nbands > 5) return SGEMM_EMU_EINVAL;
    int num_cus = 0;
    if ((rc = current_device(&num_cus)) != SGEMM_EMU_OK) return rc;
    if (M == 0 || N == 0 || K == 0) return 1;
    return gemm_streamk_pieces(M, N, K, gemm_streamk_grid(M, N, K, num_cus));
}

int sgemm_emu_split_k_fp32_b(int64_t M, int64_t N, int64_t K, int nbands)
{
    int rc;
    if ((rc = check_dims(M, N, K)) != SGEMM_EMU_OK) return rc;
    if (nbands < 1 || nbands > 5) return SGEMM_EMU_EINVAL;
    int num_cus = 0;
    if ((rc = current_device(&num_cus)) != SGEMM_EMU_OK) return rc;
    if (M == 0 || N == 0 || K == 0) return 1;
    const int64_t kpad = (K + 63) / 64 * 64;
    if (!fp32_b_streamk_allowed(N, K, false, false) || gemm_tile64_pays(M, N, K, num_cus, true)) return 1;
    return gemm_streamk_pieces(M, N, kpad, gemm_streamk_grid(M, N, kpad, num_cus));
}

int sgemm_emu_products(int nbands)
{
    static const int products[6] = {-1, 1, 3, 6, 8, 9};
    return (nbands >= 1 && nbands <= 5) ? products[nbands] : -1;
}

const char *sgemm_emu_strerror(int status)
{
    switch (status) {
    case SGEMM_EMU_OK: return "success";
    case SGEMM_EMU_EINVAL: return "invalid argument (size, leading dimension, nbands or alignment)";
    case SGEMM_EMU_ENULL: return "null pointer for a nonempty operand";
    case SGEMM_EMU_EARCH: return "no HIP device, or the current device is not gfx950";
    case SGEMM_EMU_ELAUNCH: return "kernel launch failed";
    case SGEMM_EMU_ENOMEM: return "no device memory for the stream-K partial results";
    case SGEMM_EMU_ECAPTURE: return "the call needs workspace and the stream is being captured into a graph";
    default: return "unknown status";
    }
}

int sgemm_emu_release_workspace(void)
{
    int num_cus = 0, dev = 0;
    int rc;
    if ((rc = current_device(&num_cus, &dev)) != SGEMM_EMU_OK) return rc;
    hipError_t err = hipSuccess;
    {
        DeviceWs &D = g_ws[dev];
        std::lock_guard<std::mutex> lock(D.mutex);
        for (StreamWs &x : D.slot) {
            if (!x.used) continue;
            // the block's last user has finished with it before it is freed
            if (x.recorded) {
                const hipError_t e = hipEventSynchronize(x.done);
                if (e != hipSuccess && err == hipSuccess) err = e;
            }
            if (x.ptr != nullptr) {
                const hipError_t e = hipFreeAsync(x.ptr, nullptr);
                if (e != hipSuccess && err == hipSuccess) err = e;
            }
            if (x.done != nullptr) (void)hipEventDestroy(x.done);
            x = StreamWs{};
        }
        D.clock = 0;
    }
    const hipError_t e = hipStreamSynchronize(nullptr);
    if (e != hipSuccess && err == hipSuccess) err = e;
    hipMemPool_t pool = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        if (g_devices[dev].pool_state == 1) pool = g_devices[dev].pool;
    }
    if (pool != nullptr) {
        const hipError_t t = hipMemPoolTrimTo(pool, 0);
        if (t != hipSuccess && err == hipSuccess) err = t;
    }
    (void)hipGetLastError();
    return err == hipSuccess ? SGEMM_EMU_OK : SGEMM_EMU_ELAUNCH;
}

#ifdef SGEMM_EMU_SERIAL_LDS
const char *sgemm_emu_version(void) { return "libsgemm_emu 0.2.0 (gfx950, BF16x9, serial-LDS debug build)"; }
#else
const char *sgemm_emu_version(void) { return "libsgemm_emu 0.2.0 (gfx950, BF16x9)"; }
#endif

}  // extern "C"
