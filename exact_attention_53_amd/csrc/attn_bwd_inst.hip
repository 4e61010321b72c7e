// One configuration of the backward launchers per compilation, so that the
// configurations compile in parallel.  The build defines
//   ATTN_INST_DQ     0: key/value kernel (bwd_main_t), 1: dQ kernel (bwd_dq_t), 2: both in
//                    one launch (bwd_kvdq64_t; d = 64, masks 0 and 1)
//   ATTN_INST_ELEM   bf16 or f16
//   ATTN_INST_DQK, ATTN_INST_DV, ATTN_INST_MASK (0 none, 1 causal, 2 causal + sliding window,
//                    3 causal + ALiBi bias, 4 block-sparse map, 5 block-sparse map + causal)
#include "attn_bwd_kernels.hpp"

namespace attn53 {
#if ATTN_INST_DQ == 2
template hipError_t bwd_kvdq64_t<ATTN_INST_ELEM, ATTN_INST_MASK>(const BwdParams&, hipStream_t);
#elif ATTN_INST_DQ == 1
template hipError_t bwd_dq_t<ATTN_INST_ELEM, ATTN_INST_DQK, ATTN_INST_DV, ATTN_INST_MASK>(const BwdParams&,
                                                                                          hipStream_t);
#else
template hipError_t bwd_main_t<ATTN_INST_ELEM, ATTN_INST_DQK, ATTN_INST_DV, ATTN_INST_MASK>(const BwdParams&, bool,
                                                                                            hipStream_t);
#endif
}  // namespace attn53
