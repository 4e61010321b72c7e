// Deterministic dQ kernel instance for d_qk = 128, d_v = 128, no mask
// (one file per configuration so that the configurations compile in parallel).
#include "attn_bwd_kernels.hpp"

namespace attn53 {
template hipError_t bwd_dq_t<128, 128, false>(const BwdParams&, hipStream_t);
}  // namespace attn53
