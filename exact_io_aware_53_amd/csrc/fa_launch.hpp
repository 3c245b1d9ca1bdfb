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
    bool deterministic = false;   // dQ from its own pass instead of atomics (bf16 only)
};

struct DecodeArgs {
    const void* q;     // [B, H, Nq, d]
    const void* k;     // [B, H, Nk, d]
    const void* v;     // [B, H, Nk, d]
    void* o;           // [B, H, Nq, d]
    float* lse;        // [B, H, Nq]
    float* o_part;     // workspace: fp32 [B*H, S, Nq, d] (S > 1)
    float* lse_part;   // workspace: fp32 [B*H, S, Nq] (S > 1)
    int B, H, Nq, Nk, d;
    float scale;
    bool causal;
    // Paged key/value (block_table != nullptr): k and v are page pools
    // [num_pages, H, page, d]; sequence b's key row j lives in page
    // block_table[b * max_blocks + j / page], row j % page; seq_lens[b] keys.
    const int* block_table = nullptr;
    const int* seq_lens = nullptr;
    int max_blocks = 0, page = 0, num_pages = 0;
};

// How the decode forward splits its work: nrb 32-row query blocks, S key
// chunks of `chunk` keys. Shared by the workspace size and the launch.
struct DecodeSplit {
    int nrb, S, chunk;
};
DecodeSplit decode_split(int B, int H, int Nq, int Nk);

// Dropout threshold: an element is dropped iff Philox word 0 < thr, thr = ceil(p * 2^32).
uint32_t dropout_threshold(float p);

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
// The query-side pass of the deterministic backward: dQ only (bf16 path).
hipError_t launch_bwd_dq_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_decode_bf16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_dropout_mask(uint8_t* mask, int B, int H, int N, int b, int h, float p,
                               uint64_t seed, hipStream_t stream);

}  // namespace fa
