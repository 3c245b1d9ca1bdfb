/*
 * fa.h - C ABI of libfa.so: exact, IO-aware scaled dot-product attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation
 * -------------
 * For every batch index b and head h, with Q, K, V the [N, d] matrices of that
 * head and s = `scale` (the pages fix s = 1/sqrt(d)):
 *
 *   S_ij  = s * <Q_i, K_j>                       scaled scores
 *   A_i   = { j : j <= i } if causal, else all j  (query i never sees later keys)
 *   LSE_i = log( sum_{j in A_i} exp(S_ij) )       natural log, fp32
 *   P_ij  = exp(S_ij - LSE_i) for j in A_i, else 0
 *   O_i   = sum_j P_ij * Z_ij * V_j / (1 - p)     Z = dropout keep mask, all ones if p = 0
 *
 * Sources: the scaled score and the online-softmax statistics are those of
 * "DL0056 FlashAttention" (intvml), section "Mathematical Formulation"; the
 * result is exact standard attention (same page, answer and point (3); emergent.sh
 * glossary "Flash Attention", section "Flash Attention vs. Regular Attention").
 * Causal masking and dropout inside the fused kernel: inferensys glossary
 * "FlashAttention", paragraph on causal masking and dropout. The forward pass
 * writes only O and the per-row statistic; the N x N score and probability
 * matrices never reach device memory (inferensys, paragraph on tiling). The
 * backward pass recomputes them from the stored statistic instead of storing
 * them (inferensys, paragraph on recomputation; emergent.sh, "How Flash
 * Attention Works", step 6) and regenerates the same dropout pattern
 * (emergent.sh, "Key Components of Flash Attention").
 *
 * Dropout mask (the pages name no generator): Z_ij = 1 iff word 0 of
 * Philox-4x32-10 (Salmon et al., SC'11) at counter (b, h, i, j) under key
 * (seed & 0xffffffff, seed >> 32) is >= ceil(p * 2^32), p being the float
 * argument. i and j are absolute row indices inside the head.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Layout: Q, K, V, O, dO, dQ, dK, dV are contiguous [B, H, N, d] arrays, d
 *   fastest (row-major), element type given by the symbol (bf16 or fp32);
 *   fa_fwd_ex and fa_bwd_ex take strided views, fp16 and packed batches.
 *   LSE is a contiguous [B, H, N] fp32 array. Every tensor pointer must be
 *   16-byte aligned.
 * - Memory: every pointer is device memory owned by the caller. The library
 *   never allocates or frees; the backward pass takes its fp32 scratch in
 *   `workspace`. Inputs must not alias outputs (undefined result, not checked).
 * - Streams: `stream` is a hipStream_t (NULL = the default stream). Calls are
 *   asynchronous: a return of FA_OK means the work is enqueued; outputs are
 *   valid once the stream has been synchronised.
 * - Errors: arguments are validated on the host before any HIP call.
 *   FA_ERR_INVALID_ARG  null pointer, B/H/N < 1, dropout_p outside [0, 1),
 *                       scale not a positive finite number, misaligned
 *                       pointer, too small a workspace, B*H*N*d above
 *                       2^31 - 1, or one head's rows past 32-bit offsets
 *                       ((N + 256) * d * 4 >= 0xf0000000).
 *   FA_ERR_UNSUPPORTED  head size d other than 64 or 128 (fa_fwd_ex and fa_bwd_ex
 *                       also take 32, 96 and 256; the caller keeps its
 *                       own fallback, as emergent.sh "How to Enable Flash
 *                       Attention Safely", step 7, advises).
 *   FA_ERR_HIP          a HIP launch error; the stream state is unspecified.
 *   No exception or abort crosses the ABI.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,
    FA_ERR_UNSUPPORTED = 2,
    FA_ERR_HIP = 3
} fa_status;

/*
 * Forward pass, bf16 tensors (fp32 accumulation and softmax).
 *   q, k, v   in : [B, H, N, d] bf16
 *   o         out: [B, H, N, d] bf16 (round-to-nearest-even from fp32)
 *   lse       out: [B, H, N] fp32, natural-log log-sum-exp of the scaled,
 *                  masked scores, excluding dropout
 *   scale     score scale s (1/sqrt(d) for standard attention)
 *   causal    nonzero: query i attends to keys j <= i (top-left aligned)
 *   dropout_p probability of dropping an attention weight, in [0, 1)
 *   seed      64-bit dropout seed (ignored when dropout_p == 0)
 *   stream    hipStream_t to enqueue on
 * Returns an fa_status. The result is bitwise deterministic run to run.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal,
           float dropout_p, uint64_t seed, void* stream);

/*
 * Backward pass, bf16 tensors. Given the forward inputs, its outputs O and LSE
 * (as fa_fwd wrote them, same scale/causal/dropout_p/seed) and the output
 * gradient dO, writes dQ, dK, dV ([B, H, N, d] bf16).
 *   workspace        device scratch of at least fa_bwd_workspace_size(B,H,N,d)
 *                    bytes, 256-byte aligned; contents on entry are ignored.
 * With dropout_p > 0, dQ is accumulated with fp32 atomics, so its last bits
 * may vary run to run. With dropout_p == 0 the call takes the two-pass form of
 * fa_bwd_deterministic (faster there) and the result is bitwise deterministic.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, float scale, int causal,
           float dropout_p, uint64_t seed, void* workspace, size_t workspace_bytes,
           void* stream);

/*
 * Backward pass, bf16, bitwise deterministic run to run: the same arguments,
 * workspace contract and result definition as fa_bwd, but dQ comes from a
 * second pass over the query blocks that recomputes P and dS (the dropout mask
 * is regenerated a second time from the same Philox counters) and sums each
 * dQ row's key tiles in a fixed order, instead of fp32 atomics. dK and dV are
 * the same bits fa_bwd writes; without dropout so is dQ (fa_bwd takes this
 * path then). The gradients are those of the forward, computed in fused
 * kernels ("DL0056 FlashAttention", point (3)) from score and probability
 * blocks recomputed rather than stored (inferensys glossary "FlashAttention",
 * paragraph on recomputation); that dQ may come from a pass of its own over
 * the same recomputed dS is this library's reading of those passages.
 */
int fa_bwd_deterministic(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int B, int H, int N, int d, float scale, int causal,
                         float dropout_p, uint64_t seed, void* workspace,
                         size_t workspace_bytes, void* stream);

/* The same two passes for fp32 tensors (fp32 arithmetic throughout). */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               float dropout_p, uint64_t seed, void* stream);
int fa_bwd_f32(const float* q, const float* k, const float* v, const float* o,
               const float* dout, const float* lse, float* dq, float* dk, float* dv,
               int B, int H, int N, int d, float scale, int causal,
               float dropout_p, uint64_t seed, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * Bytes of device scratch that fa_bwd / fa_bwd_f32 need: an fp32 [B,H,N,d]
 * dQ accumulator, the fp32 [B,H,N] row terms D_i = <dO_i, O_i>, and the
 * fp32 [B,H,N] log-sum-exp in log2 units, each rounded up to 256 bytes.
 * Returns 0 if an argument is out of range.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): fa_bwd with
 * the same arguments, result and validation, but no workspace argument. Its
 * scratch (the same fp32 dQ accumulator, D and log2-unit LSE as fa_bwd's
 * workspace) is a device array of FA_NOALLOC_SCRATCH_BYTES inside the library,
 * one per GPU it runs on, held until the process ends; the call itself
 * allocates nothing. Problems whose fa_bwd_workspace_size exceeds
 * FA_NOALLOC_SCRATCH_BYTES return FA_ERR_INVALID_ARG (for d = 64 that is
 * B*H*N up to 508 000 rows, for d = 128 up to 258 000). Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and give undefined results; calls ordered on
 * one stream, or synchronised, are safe. The first call on a device looks up
 * the array's device address (FA_ERR_HIP if that fails).
 */
#define FA_NOALLOC_SCRATCH_BYTES (128u << 20)
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal,
                   float dropout_p, uint64_t seed, void* stream);

/*
 * General layouts, element types, head sizes and variable-length batches.
 * The pages list tensor layouts, head sizes, numeric precision, padding and
 * uneven sequence lengths among what decides whether an attention kernel
 * applies (emergent.sh glossary "Flash Attention", "Practical Limits and
 * Common Pitfalls" and "How to Enable Flash Attention Safely", step 3). The
 * _ex entry points compute the same operation as fa_fwd / fa_bwd on:
 *   - bf16 or fp16 tensors (fp32 accumulation and softmax either way);
 *   - head size d in {32, 64, 96, 128, 256};
 *   - any strided [B, H, N, d] view with d contiguous: each tensor has its own
 *     batch, head and row strides in elements, for example [B, N, H, d]
 *     storage (row stride H*d, head stride d) or views into a packed QKV
 *     projection (row stride 3*H*d);
 *   - packed variable-length batches: with cu_seqlens non-NULL, sequence b is
 *     rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of the token dimension of every
 *     tensor (row stride as given, batch stride ignored); its element (h, i)
 *     lives at base + h * head + (cu_seqlens[b] + i) * row. Causal masking,
 *     the dropout counter (b, h, i, j) and LSE are per sequence, i and j
 *     counted from the sequence's first token.
 */
typedef enum { FA_DTYPE_BF16 = 0, FA_DTYPE_FP16 = 1 } fa_dtype;

/* Element strides of one tensor seen as [B, H, N, d] (d contiguous). */
typedef struct {
    int64_t batch;
    int64_t head;
    int64_t row;
} fa_layout;

typedef struct {
    int B, H;
    int N;                  /* sequence length; with cu_seqlens, an upper bound on every length */
    int d;                  /* 32, 64, 96, 128 or 256 */
    int dtype;              /* fa_dtype of q, k, v, o, dout, dq, dk, dv */
    const int32_t* cu_seqlens;  /* device int32 [B + 1], or NULL */
    int total_tokens;       /* with cu_seqlens: rows of the packed token dimension */
    fa_layout q, k, v, o;   /* 16-bit tensors */
    fa_layout lse;          /* fp32 LSE as a [B, H, N] view (d = 1) */
    fa_layout dout, dq, dk, dv;   /* backward only */
} fa_problem;

/*
 * Checks on the host (FA_ERR_INVALID_ARG otherwise): B, H, N >= 1; row
 * strides >= d and, like head and batch strides, non-negative multiples of 8
 * elements for the 16-bit tensors (16-byte aligned rows); LSE strides
 * non-negative, its row stride >= 1; every head's rows 0 .. N+255 within
 * 0xf0000000 bytes ((N + 256) * row * element size); total_tokens >= 1
 * with cu_seqlens. FA_ERR_UNSUPPORTED: d or dtype outside the lists above.
 * cu_seqlens is read on the device: each sequence is clamped to
 * [0, total_tokens) rows and to at most N rows, so out-of-order or oversized
 * entries cannot make a kernel touch memory outside the tensors; its contents
 * are otherwise the caller's contract (non-decreasing, cu_seqlens[0] = 0).
 * Outputs of padded rows (those no sequence covers) are not written.
 */
int fa_fwd_ex(const fa_problem* problem, const void* q, const void* k, const void* v, void* o,
              float* lse, float scale, int causal, float dropout_p, uint64_t seed, void* stream);

/*
 * Backward of fa_fwd_ex on the same problem (O and LSE as fa_fwd_ex wrote
 * them). deterministic != 0 asks for the two-pass form of fa_bwd_deterministic
 * (always taken without dropout, and for d in {32, 96, 256}); otherwise dQ is
 * summed with fp32 atomics when dropout is on. Head sizes 32 and 96 compute
 * on rows padded with zeros to 64 and 128 (exact; the products take the
 * padded width). workspace: fa_bwd_ex_workspace_size(problem) bytes, 256-byte
 * aligned.
 */
int fa_bwd_ex(const fa_problem* problem, const void* q, const void* k, const void* v,
              const void* o, const void* dout, const float* lse, void* dq, void* dk, void* dv,
              float scale, int causal, float dropout_p, uint64_t seed, int deterministic,
              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device scratch fa_bwd_ex needs for this problem (0 if invalid). */
size_t fa_bwd_ex_workspace_size(const fa_problem* problem);

/*
 * Decode-shaped forward, bf16: Nq query rows against Nk key/value rows of the
 * same head, 1 <= Nq <= Nk, for example the newest tokens against the key/value
 * cache that inference servers keep (inferensys glossary "FlashAttention",
 * paragraph on integration with inference servers). Same result as fa_fwd on
 * that problem (same definition of O and LSE; no dropout). The key range is
 * split over workgroups and the partial results are merged with the rescaling
 * of the online softmax.
 *   q         in : [B, H, Nq, d] bf16
 *   k, v      in : [B, H, Nk, d] bf16
 *   o         out: [B, H, Nq, d] bf16
 *   lse       out: [B, H, Nq] fp32
 *   causal    nonzero: query row i sits at key position Nk - Nq + i and sees
 *             keys j <= Nk - Nq + i (bottom-right aligned); zero: every key
 *   workspace device scratch of fa_fwd_decode_workspace_size(...) bytes,
 *             256-byte aligned; may be NULL when that size is 0
 * Errors as for fa_fwd; also FA_ERR_INVALID_ARG when Nq > Nk or the workspace
 * is missing or too small. The result is bitwise deterministic run to run.
 */
int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Nq, int Nk, int d, float scale, int causal,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device scratch fa_fwd_decode needs: fp32 partial outputs and
 * log-sum-exps of the key chunks, each region rounded up to 256 bytes. 0 when
 * the problem is not split, or when an argument is out of range.
 */
size_t fa_fwd_decode_workspace_size(int B, int H, int Nq, int Nk, int d);

/*
 * Decode-shaped forward over a paged key/value cache, bf16: the kernel side of
 * paged KV-cache management (inferensys glossary "FlashAttention", related term
 * PagedAttention: the cache lives in non-contiguous fixed-size blocks). Sequence
 * b has seq_lens[b] keys; its key row j is row (j % page_size) of page
 * block_table[b * max_blocks + j / page_size]. Otherwise as fa_fwd_decode, with
 * Nk = seq_lens[b] per sequence (bottom-right causal alignment per sequence).
 *   k_pages, v_pages in : [num_pages, H, page_size, d] bf16 page pools
 *   block_table      in : [B, max_blocks] int32, device memory
 *   seq_lens         in : [B] int32, device memory; values are clamped to
 *                         [0, max_blocks * page_size]
 *   page_size           : a multiple of 32 (32-key tiles never straddle pages)
 * The tables are read on the device and not validated there beyond this: a
 * table entry outside [0, num_pages) reads as zeros (no memory access). A
 * query row that sees no key (a sequence shorter than Nq, causal; or empty)
 * gets O = 0 and LSE = -inf.
 */
int fa_fwd_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                        const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                        int B, int H, int Nq, int max_blocks, int page_size, int num_pages, int d,
                        float scale, int causal, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Workspace bytes fa_fwd_decode_paged needs (0 when not split or invalid). */
size_t fa_fwd_decode_paged_workspace_size(int B, int H, int Nq, int max_blocks, int page_size, int d);

/*
 * Test aid: writes the dropout keep mask Z of head (b, h) as an [N, N] array
 * of bytes (1 = kept, 0 = dropped) into device memory `mask`, using the same
 * device generator as the attention kernels. Causal masking is not applied.
 */
int fa_dropout_mask(uint8_t* mask, int B, int H, int N, int b, int h,
                    float dropout_p, uint64_t seed, void* stream);

/* Static, human-readable name of a status code. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
