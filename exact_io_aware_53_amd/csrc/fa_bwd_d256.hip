// Backward attention at head size 256, always in the two-pass form. A file of
// its own because its kernels need more than 256 registers per lane: the build
// compiles *_d256.hip files with matrix-core accumulators allowed in the AGPR
// half of the register file.
#include "fa_bwd_kernels.hpp"

namespace fa {

hipError_t launch_bwd_mfma_d256(const BwdArgs& a, hipStream_t st) {
    return a.fp16 ? launch_bwd_td<_Float16, 256, 256>(a, st) : launch_bwd_td<__bf16, 256, 256>(a, st);
}

}  // namespace fa
