// Forward attention, bf16/fp16: dispatch over head sizes 32 .. 128 (d = 256 is
// built in fa_fwd_d256.hip). The kernel is in fa_fwd_kernel.hpp.
#include "fa_fwd_kernel.hpp"

namespace fa {
namespace {

template <typename T>
hipError_t launch_t(const FwdArgs& a, hipStream_t st) {
    switch (a.s.d) {
        case 32: return launch_d<T, 32>(a, st);
        case 64: return launch_d<T, 64>(a, st);
        case 96: return launch_d<T, 96>(a, st);
        case 128: return launch_d<T, 128>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t st) {
    if (a.s.d == 256) return launch_fwd_mfma_d256(a, st);
    return a.fp16 ? launch_t<_Float16>(a, st) : launch_t<__bf16>(a, st);
}

}  // namespace fa
