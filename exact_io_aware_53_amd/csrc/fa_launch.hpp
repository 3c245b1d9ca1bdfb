// Host-side interface between the C ABI (fa_api.cpp) and the kernel launchers.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct AttnShape {
    int B, H, N, d;
    float scale;
    bool causal;
    float dropout_p;
    uint64_t seed;
};

struct FwdArgs {
    AttnShape s;
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
};

struct BwdArgs {
    AttnShape s;
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* dq_accum;   // workspace: fp32 [B,H,N,d]
    float* dsum;       // workspace: fp32 [B,H,N], D_i = <dO_i, O_i>
    float* lse2;       // workspace: fp32 [B,H,N], LSE_i * log2(e)
};

// Dropout threshold: an element is dropped iff Philox word 0 < thr, thr = ceil(p * 2^32).
uint32_t dropout_threshold(float p);

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t stream);
hipError_t launch_dropout_mask(uint8_t* mask, int B, int H, int N, int b, int h, float p,
                               uint64_t seed, hipStream_t stream);

}  // namespace fa
