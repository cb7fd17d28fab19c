// launch_stubs.hip -- test support for the AddressSanitizer build of the C ABI's host code
// (tests/test_host_asan.py): the kernel launchers of libgdn.so replaced by functions that launch
// nothing.  The tests run against that build reach no launch (every case fails argument checks, asks
// for a workspace size or is an empty no-op), so these only complete the link.
#include "../../linear_attention_sequence_rule_amd/csrc/kernels.hpp"

namespace gdn {

hipError_t launch_step(const StepArgs&) { return hipErrorNotSupported; }
hipError_t launch_chunk_f32(const ChunkArgs&) { return hipErrorNotSupported; }
hipError_t launch_chunk_bf16(const ChunkArgs&) { return hipErrorNotSupported; }
hipError_t launch_conv_prepass(const ChunkArgs&, void*, ChunkArgs&) { return hipErrorNotSupported; }
hipError_t launch_conv_state_update(const ChunkArgs&) { return hipErrorNotSupported; }
hipError_t launch_gated_norm(void*, const void*, const float*, long, int, float, bool, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace gdn
