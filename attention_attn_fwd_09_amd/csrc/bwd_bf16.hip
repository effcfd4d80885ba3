// TEMPORARY placeholder, replaced by the real backward kernels before commit.
#include "common.h"
#include "kernels.h"
namespace attn {
int bwd_block_q(int) { return 64; }
int bwd_block_k(int) { return 64; }
hipError_t launch_bwd_preprocess(const BwdParams&, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_dkdv(const BwdParams&, int, int, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_dq(const BwdParams&, int, int, int, hipStream_t) { return hipErrorNotSupported; }
}
