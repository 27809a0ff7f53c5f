// fwd_bf16.hip -- matrix-core (bf16 MFMA, fp32 accumulate) PaTH forward.
#include "common.hpp"
#include "kernels.hpp"

namespace pa {

bool fwd_bf16_supported(int d, int block) { (void)d; (void)block; return false; }

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st) {
    (void)a; (void)st;
    return hipErrorNotSupported;
}

hipError_t launch_causal(const FwdArgs& a, hipStream_t st) {
    (void)a; (void)st;
    return hipErrorNotSupported;
}

}  // namespace pa
