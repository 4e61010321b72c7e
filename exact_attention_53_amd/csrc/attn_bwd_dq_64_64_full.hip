// Deterministic dQ kernel instance for d_qk = 64, d_v = 64, no mask
// (one file per configuration so that the configurations compile in parallel).
#include "attn_bwd_kernels.hpp"

namespace attn53 {
template hipError_t bwd_dq_t<64, 64, false>(const BwdParams&, hipStream_t);
}  // namespace attn53
