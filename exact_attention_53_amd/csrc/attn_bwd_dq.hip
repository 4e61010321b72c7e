// Deterministic dQ kernel instances for every supported configuration.
#include "attn_bwd_kernels.hpp"

namespace attn53 {
#define ATTN_INSTANTIATE_DQ(DQK, DV, CAUSAL) template hipError_t bwd_dq_t<DQK, DV, CAUSAL>(const BwdParams&, hipStream_t);
ATTN_BWD_CONFIGS(ATTN_INSTANTIATE_DQ)
}  // namespace attn53
