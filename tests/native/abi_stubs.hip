// abi_stubs.hip -- stand-ins for the kernel launchers of libsgemm_emu, for a
// host-only build of the C-ABI layer (api.hip) under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU.  There, argument
// validation returns before any launch (an invalid call returns its error, a
// valid one SGEMM_EMU_EARCH), so these are never reached; each reports an
// error if it is.  Test infrastructure only.
#include "../../fp32_emulated_gemm_amd/csrc/launch.hpp"

namespace sgemm_emu_dev {

hipError_t launch_split(int64_t, int64_t, const float *, int64_t, uint16_t *, uint16_t *, uint16_t *, int64_t, int,
                        hipStream_t, bool)
{
    return hipErrorNotSupported;
}

hipError_t launch_split_transpose(int64_t, int64_t, const float *, int64_t, uint16_t *, uint16_t *, uint16_t *,
                                  int64_t, int, hipStream_t, bool, int64_t)
{
    return hipErrorNotSupported;
}

hipError_t launch_transpose_planes(int64_t, int64_t, const uint16_t *, const uint16_t *, const uint16_t *, int64_t,
                                   uint16_t *, uint16_t *, uint16_t *, int64_t, int64_t, hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t launch_gemm(const GemmArgs &, int, BSource, hipStream_t, bool) { return hipErrorNotSupported; }

hipError_t launch_gemm_planes(const GemmArgs &, int, hipStream_t) { return hipErrorNotSupported; }

int gemm_streamk_grid(int64_t, int64_t, int64_t, int) { return 0; }

int gemm_streamk_pieces(int64_t, int64_t, int64_t, int) { return 1; }

bool gemm_tile64_pays(int64_t, int64_t, int64_t, int, bool) { return false; }

hipError_t launch_gemm_tile64(const GemmArgs &, int, BSource, hipStream_t, bool) { return hipErrorNotSupported; }

bool launch_done_attached(const GemmArgs &, BSource) { return false; }

bool gemm_uses_dma(int64_t, int64_t, const void *, const void *, const void *) { return false; }

NativePlan native_plan(int64_t, int64_t, int64_t, int, bool) { return NativePlan{128, 1}; }

bool native_vec(const float *, int64_t, const float *, int64_t, int64_t, int64_t) { return false; }

hipError_t launch_native(const GemmArgs &, const NativePlan &, hipStream_t) { return hipErrorNotSupported; }

hipError_t launch_ieee_fixup(int64_t, int64_t, int64_t, const float *, int64_t, const float *, int64_t, float *,
                             int64_t, int *, int, hipStream_t)
{
    return hipErrorNotSupported;
}

hipError_t launch_zero(int64_t, int64_t, float *, int64_t, const float *, int, int, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace sgemm_emu_dev
