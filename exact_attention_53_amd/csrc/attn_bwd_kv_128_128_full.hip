// Key/value kernel instances for d_qk = 128, d_v = 128, no mask
// (one file per configuration so that the configurations compile in parallel).
#include "attn_bwd_kernels.hpp"

namespace attn53 {
template hipError_t bwd_main_t<128, 128, false>(const BwdParams&, bool, hipStream_t);
}  // namespace attn53
