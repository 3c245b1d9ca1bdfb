// Backward attention, bf16/fp16: dispatch over head sizes 32 .. 128 (d = 256 is
// built in fa_bwd_d256.hip). Kernels: fa_bwd_kernels.hpp, fa_bwd_dq.hpp.
#include "fa_bwd_kernels.hpp"

namespace fa {
namespace {

template <typename T>
hipError_t launch_t(const BwdArgs& a, hipStream_t st) {
    switch (a.s.d) {
        case 32: return launch_bwd_td<T, 64, 32>(a, st);     // rows padded to 64
        case 64: return launch_bwd_td<T, 64, 64>(a, st);
        case 96: return launch_bwd_td<T, 128, 96>(a, st);    // rows padded to 128
        case 128: return launch_bwd_td<T, 128, 128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t st) {
    if (a.s.d == 256) return launch_bwd_mfma_d256(a, st);
    return a.fp16 ? launch_t<_Float16>(a, st) : launch_t<__bf16>(a, st);
}

}  // namespace fa
