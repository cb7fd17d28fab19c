// chunk_bf16.hip -- bf16 chunked prefill (placeholder: the exact-fp32 VALU algebra on bf16 I/O).
#include "kernels.hpp"

namespace gdn {

size_t chunk_bf16_workspace(int, int, int, int, int, bool) { return 0; }

hipError_t launch_chunk_bf16(const ChunkArgs& a) { return launch_chunk_valu_bf16(a); }

}  // namespace gdn
