// Backward attention for bf16 tensors.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {

hipError_t launch_bwd_bf16_simple(const BwdArgs& a, hipStream_t st);

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) { return launch_bwd_bf16_simple(a, st); }

}  // namespace fa
