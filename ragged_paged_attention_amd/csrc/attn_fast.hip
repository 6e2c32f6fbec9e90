// MFMA fast paths (bf16/f16, head_dim 128, block_size % 16 == 0).
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

bool fast_path_supported(const AttnArgs&) { return false; }

size_t fast_workspace_bytes(int32_t, int32_t, int32_t, int32_t, int32_t, int32_t) { return 0; }

hipError_t launch_attn_fast(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
