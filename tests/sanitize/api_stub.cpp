// Host-only stand-ins for the kernel launchers and the one HIP call of the C ABI, so that
// api.cpp (argument validation, dispatch, the slot allocator) can be built with the address
// and undefined-behaviour sanitizers on a machine without a GPU. Every launcher records
// that it was reached and returns success without touching the pointers it was given.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/mamba2.h"
#include "../../state_space_model_ssm_amd/csrc/kernels.hpp"

int g_launches = 0;

extern "C" const char *hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub error"; }

namespace m2 {

namespace {
unsigned g_word[4];
hipError_t reached() {
    ++g_launches;
    return hipSuccess;
}
}  // namespace

hipError_t slot_error_word(unsigned **out) {
    *out = g_word;
    return hipSuccess;
}
hipError_t launch_read_slot_errors(unsigned *, int, hipStream_t) { return reached(); }
hipError_t static_scratch(void **ptr, size_t *bytes) {
    alignas(256) static unsigned char fake[256];  // never dereferenced by the stubs
    *ptr = fake;
    *bytes = MAMBA2_STATIC_SCRATCH_BYTES;
    return hipSuccess;
}
hipError_t launch_check_slots(const int32_t *, int, int, unsigned *, hipStream_t) { return reached(); }

bool state_update_supported(const LayerShape &s) { return s.N == 16 || s.N == 64 || s.N == 128; }
hipError_t launch_state_update(const LayerShape &, const StateUpdateArgs &, hipStream_t) { return reached(); }
hipError_t launch_state_update_multi(const LayerShape &, const MultiStepArgs &, hipStream_t) { return reached(); }
hipError_t launch_conv_update_multi(const LayerShape &, const ConvMultiArgs &, hipStream_t) { return reached(); }
bool conv_supported(const LayerShape &s) { return s.W >= 2 && s.W <= 4 && s.cdim() % 8 == 0; }
hipError_t launch_conv_update(const LayerShape &, const ConvUpdateArgs &, hipStream_t) { return reached(); }
hipError_t launch_conv_fwd(const LayerShape &, const ConvFwdArgs &, hipStream_t) { return reached(); }
hipError_t launch_conv_state(const LayerShape &, const ConvFwdArgs &, hipStream_t) { return reached(); }
bool prefill_fused_supported(const LayerShape &s) { return s.P == 64 && s.N == 128 && s.out_dt == 1; }
int64_t fused_workspace_bytes(const LayerShape &s, int64_t T) { return T * (3LL * s.G * s.N * 2 + s.G * 32 * 4); }
hipError_t launch_fused_prefill(const LayerShape &, FusedArgs, void *, hipStream_t) { return reached(); }
bool chunk_scan_blocks_supported(const LayerShape &s) { return prefill_fused_supported(s) && s.act_dt == 1; }
hipError_t launch_block_scan(const LayerShape &, FusedArgs, void *, hipStream_t) { return reached(); }
bool gated_norm_supported(int64_t width, int gs) { return gs > 0 && gs % 4 == 0 && gs <= 4096 && width % gs == 0; }
hipError_t launch_gated_norm(const NormArgs &, int, int, int64_t, int, hipStream_t) { return reached(); }
bool selective_scan_supported(const SelShape &s) { return s.N == 4 || s.N == 8 || s.N == 16; }
hipError_t launch_selective_scan(const SelShape &, const SelScanArgs &, hipStream_t) { return reached(); }
hipError_t launch_selective_update(const SelShape &, const SelUpdateArgs &, hipStream_t) { return reached(); }
bool scan_supported(const LayerShape &s) { return (s.P == 64 && s.N == 128) || (s.P == 16 && s.N == 16); }
hipError_t launch_chunk_scan(const LayerShape &, const ScanArgs &, hipStream_t) { return reached(); }

}  // namespace m2
