// Forward attention at head size 256. A file of its own because its kernels
// need more than 256 registers per lane: the build compiles *_d256.hip files
// with matrix-core accumulators allowed in the AGPR half of the register file.
#include "fa_fwd_kernel.hpp"

namespace fa {

hipError_t launch_fwd_mfma_d256(const FwdArgs& a, hipStream_t st) {
    return a.fp16 ? launch_d<_Float16, 256>(a, st) : launch_d<__bf16, 256>(a, st);
}

}  // namespace fa
