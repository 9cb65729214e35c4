// SageAttention-style quantised prefill (placeholder until the kernels land).
#include "attn_internal.hpp"

namespace attn {

size_t sage_workspace_bytes(int B, int H, int Hkv, int N, int d)
{
    (void)B; (void)H; (void)Hkv; (void)N; (void)d;
    return 0;
}

hipError_t launch_sage(const SageArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace attn
