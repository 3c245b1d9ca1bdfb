// Host-side interface between the C ABI (fa_api.cpp) and the kernel launchers.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Element strides of a [B, H, N, d] view whose d elements are contiguous
// (batch stride unused for packed sequences).
struct Strides {
    int64_t sb, sh;
    int sn;
    // Element offset of row `start` of head (b, h).
    __host__ __device__ size_t base(int b, int h, int start) const {
        return (size_t)((int64_t)b * sb + (int64_t)h * sh + (int64_t)start * sn);
    }
};

// Layouts of every tensor of a call, and the packed-sequence offsets.
struct TensorLayouts {
    Strides q, k, v, o, lse, dout, dq, dk, dv;
    const int* cu_seqlens = nullptr;   // device [B + 1], or null
    int total = 0;                     // rows of the packed token dimension
};

// Contiguous [B, H, N, d] strides.
inline Strides contiguous(int H, int N, int d) {
    return Strides{(int64_t)H * N * d, (int64_t)N * d, d};
}
inline TensorLayouts contiguous_layouts(int H, int N, int d) {
    TensorLayouts L;
    L.q = L.k = L.v = L.o = L.dout = L.dq = L.dk = L.dv = contiguous(H, N, d);
    L.lse = contiguous(H, N, 1);
    return L;
}

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
    // Matrix-core path only: strided views, fp16, packed sequences.
    TensorLayouts L;
    bool fp16 = false;
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
    bool deterministic = false;   // dQ from its own pass instead of atomics
    // Matrix-core path only: strided views, fp16, packed sequences.
    TensorLayouts L;
    bool fp16 = false;
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

// bf16/fp16 matrix-core forward (any layout in a.L, d in {32, 64, 96, 128, 256}).
hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t stream);
// bf16/fp16 matrix-core backward (any layout in a.L, d in {32, 64, 96, 128, 256}).
hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_mfma_d256(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_mfma_d256(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_decode_bf16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_dropout_mask(uint8_t* mask, int B, int H, int N, int b, int h, float p,
                               uint64_t seed, hipStream_t stream);

}  // namespace fa
