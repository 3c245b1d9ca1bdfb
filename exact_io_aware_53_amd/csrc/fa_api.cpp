// C ABI of libfa.so: host-side argument validation and dispatch to the gfx950
// kernels. Every check happens before the first HIP call, so a rejected call
// touches neither the device nor the stream. See include/fa.h for the contract.
#include "../../include/fa.h"

#include <math.h>

#include <mutex>

#include "fa_launch.hpp"

namespace fa {

uint32_t dropout_threshold(float p) {
    // ceil(p * 2^32) of the float value, exact in double; p < 1 keeps it below 2^32.
    return (uint32_t)ceil((double)p * 4294967296.0);
}

}  // namespace fa

namespace {

constexpr long long kMaxElems = 2147483647LL;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(int B, int H, int N, int d, float scale, float dropout_p) {
    if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;   // also rejects NaN
    if (!(dropout_p >= 0.0f && dropout_p < 1.0f)) return FA_ERR_INVALID_ARG;   // also rejects NaN
    if ((long long)B * H * N * d > kMaxElems) return FA_ERR_INVALID_ARG;
    // a head's rows, ragged tail tiles included, within 32-bit offsets below the
    // out-of-range offset of zero-filled chunks (0xf0000000)
    if ((long long)(N + 256) * d * 4 >= 0xf0000000LL) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t workspace_bytes(int B, int H, int N, int d) {
    const size_t rows = (size_t)B * H * N;
    return round256(rows * d * sizeof(float)) + 2 * round256(rows * sizeof(float));
}

int map_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

bool decode_shape_ok(int B, int H, int Nq, int Nk, int d) {
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 || Nq > Nk) return false;
    return (long long)B * H * Nk * d <= kMaxElems;
}

size_t decode_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
    const fa::DecodeSplit sp = fa::decode_split(B, H, Nq, Nk);
    if (sp.S == 1) return 0;
    const size_t rows = (size_t)B * H * sp.S * Nq;
    return round256(rows * d * sizeof(float)) + round256(rows * sizeof(float));
}

fa::AttnShape shape(int B, int H, int N, int d, float scale, int causal, float p, uint64_t seed) {
    return fa::AttnShape{B, H, N, d, scale, causal != 0, p, seed};
}

int fwd_common(bool bf16, const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, float dropout_p,
               uint64_t seed, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    const int st = check_shape(B, H, N, d, scale, dropout_p);
    if (st != FA_OK) return st;
    fa::FwdArgs a{shape(B, H, N, d, scale, causal, dropout_p, seed), q, k, v, o, lse};
    a.L = fa::contiguous_layouts(H, N, d);
    hipStream_t s = (hipStream_t)stream;
    return map_hip(bf16 ? fa::launch_fwd_mfma(a, s) : fa::launch_fwd_f32(a, s));
}

bool head_size_ok(int d) { return d == 32 || d == 64 || d == 96 || d == 128 || d == 256; }

// Bytes a head's rows may span: below the out-of-range offset (0xf0000000)
// the kernels use for zero-filled chunks.
constexpr long long kHeadBytes = 0xf0000000LL;

// One 16-bit tensor's strides: non-negative, 16-byte aligned rows, rows not
// overlapping, and rows 0 .. N+255 of a head within kHeadBytes.
bool strides16_ok(const fa_layout& l, int N, int d, fa::Strides& out) {
    if (l.batch < 0 || l.head < 0 || l.row < d) return false;
    if (l.batch % 8 != 0 || l.head % 8 != 0 || l.row % 8 != 0) return false;
    if ((long long)(N + 256) * l.row * 2 >= kHeadBytes) return false;
    out = fa::Strides{l.batch, l.head, (int)l.row};
    return true;
}

bool strides32_ok(const fa_layout& l, int N, fa::Strides& out) {
    if (l.batch < 0 || l.head < 0 || l.row < 1) return false;
    if ((long long)(N + 256) * l.row * 4 >= kHeadBytes) return false;
    out = fa::Strides{l.batch, l.head, (int)l.row};
    return true;
}

// Validates a problem description and turns it into kernel layouts.
int problem_layouts(const fa_problem* pb, bool backward, fa::TensorLayouts& L) {
    if (!pb) return FA_ERR_INVALID_ARG;
    if (pb->B < 1 || pb->H < 1 || pb->N < 1 || pb->d < 1) return FA_ERR_INVALID_ARG;
    if (!head_size_ok(pb->d)) return FA_ERR_UNSUPPORTED;
    if (pb->dtype != FA_DTYPE_BF16 && pb->dtype != FA_DTYPE_FP16) return FA_ERR_UNSUPPORTED;
    const int N = pb->N, d = pb->d;
    if (!strides16_ok(pb->q, N, d, L.q) || !strides16_ok(pb->k, N, d, L.k) ||
        !strides16_ok(pb->v, N, d, L.v) || !strides16_ok(pb->o, N, d, L.o) ||
        !strides32_ok(pb->lse, N, L.lse))
        return FA_ERR_INVALID_ARG;
    if (backward && (!strides16_ok(pb->dout, N, d, L.dout) || !strides16_ok(pb->dq, N, d, L.dq) ||
                     !strides16_ok(pb->dk, N, d, L.dk) || !strides16_ok(pb->dv, N, d, L.dv)))
        return FA_ERR_INVALID_ARG;
    if ((long long)pb->B * pb->H * ((N + 255) / 256) > (1LL << 30)) return FA_ERR_INVALID_ARG;
    L.cu_seqlens = pb->cu_seqlens;
    L.total = 0;
    if (pb->cu_seqlens) {
        if (((uintptr_t)pb->cu_seqlens & 3u) != 0 || pb->total_tokens < 1) return FA_ERR_INVALID_ARG;
        L.total = pb->total_tokens;
    }
    return FA_OK;
}

// Checks of the tensor arguments of fa_bwd and its variants (everything but the workspace).
int bwd_check(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
              float scale, float dropout_p) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    return check_shape(B, H, N, d, scale, dropout_p);
}

int bwd_common(bool bf16, const void* q, const void* k, const void* v, const void* o,
               const void* dout, const float* lse, void* dq, void* dk, void* dv,
               int B, int H, int N, int d, float scale, int causal, float dropout_p,
               uint64_t seed, void* workspace, size_t ws_bytes, void* stream,
               bool deterministic = false) {
    const int st = bwd_check(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, dropout_p);
    if (st != FA_OK) return st;
    if (!workspace || ((uintptr_t)workspace & 255u) != 0) return FA_ERR_INVALID_ARG;
    if (ws_bytes < workspace_bytes(B, H, N, d)) return FA_ERR_INVALID_ARG;
    const size_t rows = (size_t)B * H * N;
    float* dq_acc = (float*)workspace;
    float* dsum = (float*)((char*)workspace + round256(rows * d * sizeof(float)));
    float* lse2 = (float*)((char*)dsum + round256(rows * sizeof(float)));
    fa::BwdArgs a{shape(B, H, N, d, scale, causal, dropout_p, seed), q, k, v, o, dout, lse,
                  dq, dk, dv, dq_acc, dsum, lse2, deterministic};
    a.L = fa::contiguous_layouts(H, N, d);
    hipStream_t s = (hipStream_t)stream;
    return map_hip(bf16 ? fa::launch_bwd_mfma(a, s) : fa::launch_bwd_f32(a, s));
}

// ---- device scratch of fa_bwd_noalloc ------------------------------------
// The workspace of fa_bwd_noalloc lives in this array, one copy on every GPU the
// library runs on, held until the process ends. In host code its name is only a
// host-side stand-in: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device with that device current, and only
// that address is ever handed to a kernel.
static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void* scratch_ptr[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

int scratch_for_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_HIP;
    if (dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
    std::call_once(scratch_once[dev], [dev] {
        void* p = nullptr;
        scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (scratch_err[dev] != hipSuccess || !scratch_ptr[dev]) return FA_ERR_HIP;
    *out = scratch_ptr[dev];
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal,
           float dropout_p, uint64_t seed, void* stream) {
    return fwd_common(true, q, k, v, o, lse, B, H, N, d, scale, causal, dropout_p, seed, stream);
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               float dropout_p, uint64_t seed, void* stream) {
    return fwd_common(false, q, k, v, o, lse, B, H, N, d, scale, causal, dropout_p, seed, stream);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal,
           float dropout_p, uint64_t seed, void* workspace, size_t workspace_bytes_,
           void* stream) {
    return bwd_common(true, q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal,
                      dropout_p, seed, workspace, workspace_bytes_, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal,
                   float dropout_p, uint64_t seed, void* stream) {
    const int st = bwd_check(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, dropout_p);
    if (st != FA_OK) return st;
    if (workspace_bytes(B, H, N, d) > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_INVALID_ARG;
    void* ws = nullptr;
    const int sst = scratch_for_current_device(&ws);
    if (sst != FA_OK) return sst;
    return bwd_common(true, q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal,
                      dropout_p, seed, ws, FA_NOALLOC_SCRATCH_BYTES, stream);
}

int fa_bwd_deterministic(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int B, int H, int N, int d, float scale, int causal,
                         float dropout_p, uint64_t seed, void* workspace,
                         size_t workspace_bytes_, void* stream) {
    return bwd_common(true, q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal,
                      dropout_p, seed, workspace, workspace_bytes_, stream, true);
}

int fa_bwd_f32(const float* q, const float* k, const float* v, const float* o,
               const float* dout, const float* lse, float* dq, float* dk, float* dv,
               int B, int H, int N, int d, float scale, int causal,
               float dropout_p, uint64_t seed, void* workspace, size_t workspace_bytes_,
               void* stream) {
    return bwd_common(false, q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal,
                      dropout_p, seed, workspace, workspace_bytes_, stream);
}

int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Nq, int Nk, int d, float scale, int causal,
                  void* workspace, size_t workspace_bytes_, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    if (!decode_shape_ok(B, H, Nq, Nk, d)) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    const size_t need = decode_workspace_bytes(B, H, Nq, Nk, d);
    if (need > 0) {
        if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes_ < need)
            return FA_ERR_INVALID_ARG;
    }
    const fa::DecodeSplit sp = fa::decode_split(B, H, Nq, Nk);
    const size_t rows = (size_t)B * H * sp.S * Nq;
    float* o_part = need > 0 ? (float*)workspace : nullptr;
    float* lse_part = need > 0 ? (float*)((char*)workspace + round256(rows * d * sizeof(float))) : nullptr;
    fa::DecodeArgs a{q, k, v, o, lse, o_part, lse_part, B, H, Nq, Nk, d, scale, causal != 0};
    return map_hip(fa::launch_fwd_decode_bf16(a, (hipStream_t)stream));
}

int fa_fwd_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                        const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                        int B, int H, int Nq, int max_blocks, int page_size, int num_pages, int d,
                        float scale, int causal, void* workspace, size_t workspace_bytes_, void* stream) {
    if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) || !aligned16(lse) ||
        ((uintptr_t)block_table & 3u) != 0 || ((uintptr_t)seq_lens & 3u) != 0)
        return FA_ERR_INVALID_ARG;
    if (page_size < 32 || page_size % 32 != 0 || max_blocks < 1 || num_pages < 1)
        return FA_ERR_INVALID_ARG;
    if ((long long)max_blocks * page_size > kMaxElems) return FA_ERR_INVALID_ARG;
    const int max_keys = max_blocks * page_size;
    if (!decode_shape_ok(B, H, Nq, max_keys, 1)) return FA_ERR_INVALID_ARG;
    if ((long long)B * H * Nq * d > kMaxElems) return FA_ERR_INVALID_ARG;
    if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    const size_t need = decode_workspace_bytes(B, H, Nq, max_keys, d);
    if (need > 0) {
        if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes_ < need)
            return FA_ERR_INVALID_ARG;
    }
    const fa::DecodeSplit sp = fa::decode_split(B, H, Nq, max_keys);
    const size_t rows = (size_t)B * H * sp.S * Nq;
    float* o_part = need > 0 ? (float*)workspace : nullptr;
    float* lse_part = need > 0 ? (float*)((char*)workspace + round256(rows * d * sizeof(float))) : nullptr;
    fa::DecodeArgs a{q, k_pages, v_pages, o, lse, o_part, lse_part, B, H, Nq, max_keys, d, scale, causal != 0};
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.max_blocks = max_blocks;
    a.page = page_size;
    a.num_pages = num_pages;
    return map_hip(fa::launch_fwd_decode_bf16(a, (hipStream_t)stream));
}

size_t fa_fwd_decode_paged_workspace_size(int B, int H, int Nq, int max_blocks, int page_size, int d) {
    if (page_size < 32 || page_size % 32 != 0 || max_blocks < 1) return 0;
    if ((long long)max_blocks * page_size > kMaxElems) return 0;
    const int max_keys = max_blocks * page_size;
    if (!decode_shape_ok(B, H, Nq, max_keys, 1) || d < 1) return 0;
    return decode_workspace_bytes(B, H, Nq, max_keys, d);
}

size_t fa_fwd_decode_workspace_size(int B, int H, int Nq, int Nk, int d) {
    if (!decode_shape_ok(B, H, Nq, Nk, d)) return 0;
    return decode_workspace_bytes(B, H, Nq, Nk, d);
}

int fa_fwd_ex(const fa_problem* pb, const void* q, const void* k, const void* v, void* o,
              float* lse, float scale, int causal, float dropout_p, uint64_t seed, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3u) != 0)
        return FA_ERR_INVALID_ARG;
    fa::TensorLayouts L;
    const int st = problem_layouts(pb, false, L);
    if (st != FA_OK) return st;
    if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (!(dropout_p >= 0.0f && dropout_p < 1.0f)) return FA_ERR_INVALID_ARG;
    fa::FwdArgs a{shape(pb->B, pb->H, pb->N, pb->d, scale, causal, dropout_p, seed), q, k, v, o, lse};
    a.L = L;
    a.fp16 = pb->dtype == FA_DTYPE_FP16;
    return map_hip(fa::launch_fwd_mfma(a, (hipStream_t)stream));
}

// Width the backward computes at: head sizes 32 and 96 run on rows padded to 64 and 128.
int compute_width(int d) { return d == 32 ? 64 : d == 96 ? 128 : d; }

// One head's fp32 dQ accumulator rows (ragged tail tiles included) must stay
// within the 32-bit byte range of the buffer resource that addresses them, as
// check_shape requires of fa_bwd: past it the range would wrap and the dQ
// atomics would be dropped.
bool dq_acc_head_ok(int N, int dc) { return (long long)(N + 256) * dc * 4 < kHeadBytes; }

size_t fa_bwd_ex_workspace_size(const fa_problem* pb) {
    fa::TensorLayouts L;
    if (problem_layouts(pb, true, L) != FA_OK) return 0;
    if (!dq_acc_head_ok(pb->N, compute_width(pb->d))) return 0;
    return workspace_bytes(pb->B, pb->H, pb->N, compute_width(pb->d));
}

int fa_bwd_ex(const fa_problem* pb, const void* q, const void* k, const void* v, const void* o,
              const void* dout, const float* lse, void* dq, void* dk, void* dv, float scale,
              int causal, float dropout_p, uint64_t seed, int deterministic, void* workspace,
              size_t ws_bytes, void* stream) {
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
        return FA_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
    for (const void* p : ptrs)
        if (!aligned16(p)) return FA_ERR_INVALID_ARG;
    if (((uintptr_t)lse & 3u) != 0 || ((uintptr_t)workspace & 255u) != 0) return FA_ERR_INVALID_ARG;
    fa::TensorLayouts L;
    const int st = problem_layouts(pb, true, L);
    if (st != FA_OK) return st;
    if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (!(dropout_p >= 0.0f && dropout_p < 1.0f)) return FA_ERR_INVALID_ARG;
    const int B = pb->B, H = pb->H, N = pb->N, dc = compute_width(pb->d);
    if ((long long)B * H * N * dc > kMaxElems) return FA_ERR_INVALID_ARG;   // workspace indexing
    if (!dq_acc_head_ok(N, dc)) return FA_ERR_INVALID_ARG;
    if (ws_bytes < workspace_bytes(B, H, N, dc)) return FA_ERR_INVALID_ARG;
    const size_t rows = (size_t)B * H * N;
    float* dq_acc = (float*)workspace;
    float* dsum = (float*)((char*)workspace + round256(rows * dc * sizeof(float)));
    float* lse2 = (float*)((char*)dsum + round256(rows * sizeof(float)));
    fa::BwdArgs a{shape(B, H, N, pb->d, scale, causal, dropout_p, seed), q, k, v, o, dout, lse,
                  dq, dk, dv, dq_acc, dsum, lse2, deterministic != 0};
    a.L = L;
    a.fp16 = pb->dtype == FA_DTYPE_FP16;
    return map_hip(fa::launch_bwd_mfma(a, (hipStream_t)stream));
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
    if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
    if ((long long)B * H * N * d > kMaxElems) return 0;
    return workspace_bytes(B, H, N, d);
}

int fa_dropout_mask(uint8_t* mask, int B, int H, int N, int b, int h,
                    float dropout_p, uint64_t seed, void* stream) {
    if (!mask) return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1 || b < 0 || b >= B || h < 0 || h >= H) return FA_ERR_INVALID_ARG;
    if (!(dropout_p >= 0.0f && dropout_p < 1.0f)) return FA_ERR_INVALID_ARG;
    if ((long long)N * N > kMaxElems) return FA_ERR_INVALID_ARG;
    return map_hip(fa::launch_dropout_mask(mask, B, H, N, b, h, dropout_p, seed,
                                           (hipStream_t)stream));
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported head size or dtype";
        case FA_ERR_HIP: return "FA_ERR_HIP: HIP launch error";
        default: return "unknown fa_status";
    }
}

}  // extern "C"
