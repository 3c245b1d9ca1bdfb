// Backward attention for bf16 and fp16 tensors on gfx950 matrix cores.
//
// Recomputation instead of storage (inferensys glossary "FlashAttention",
// paragraph on recomputation; emergent.sh glossary "Flash Attention", "How
// Flash Attention Works", step 6): the score and probability tiles are rebuilt
// from Q, K and the stored row log-sum-exp, P = exp(S - LSE), tile by tile,
// and the dropout pattern is regenerated from the same Philox counters
// (emergent.sh, "Key Components of Flash Attention"). The gradients are those
// of exact attention, fused into one kernel per key block (DL0056
// FlashAttention, point (3)):
//
//   D_i  = <dO_i, O_i>                   (pre-pass, fp32)
//   dV_j += sum_i P_ij Z'_ij dO_i         Z' = Z / (1 - p)
//   dP_ij = <dO_i, V_j> Z'_ij
//   dS_ij = P_ij (dP_ij - D_i)
//   dK_j += s sum_i dS_ij Q_i,   dQ_i += s sum_j dS_ij K_j   (fp32 atomics)
//
// gfx950 mapping
// --------------
// * A workgroup of 4 waves owns 128 keys (32 per wave). K and V rows of the
//   wave's keys stay in registers as matrix-core operands; dK and dV
//   accumulate in registers over every query tile, transposed (d x keys).
// * Query tiles of 64 rows (Q, dO, LSE, D) stream HBM -> LDS through
//   buffer_load ... lds; the next tile is fetched while the current one's dQ
//   products run.
// * S = Q K^T and dP = dO V^T leave a lane holding one key and 16 query rows,
//   which is exactly the B-operand layout that dV^T = dO^T (P Z') and
//   dK^T = Q^T dS need; dO^T and Q^T come from LDS through ds_read_b64_tr_b16.
// * dS goes to LDS (transposed, bf16) once per tile; the four waves then form
//   dQ_tile = dS K for all 128 keys and add it to an fp32 accumulator in HBM
//   with global atomics. A last pass converts that accumulator to bf16.
// * LDS rows are XOR-swizzled in 16-byte chunks (chunk_swizzle) so that both
//   access shapes, row operands and transposed reads, are conflict-free.
// * Two-pass form (DQ = false): the same kernel without the dQ products, then
//   bwd_dq_kernel for dQ. No atomics, so bitwise deterministic; without
//   dropout it is also the faster form and the default. At d = 128 its key
//   side is bwd_kv_split_kernel: the work of each 32 keys split between two
//   waves of one SIMD.
// * Layouts as in the forward: per-tensor batch/head/row strides, packed
//   variable-length sequences. Head sizes 32 and 96 run the kernels of 64 and
//   128 on rows padded with zeros (DH = the stored width, D = the computed
//   one): padded columns load as zeros and are never stored.
#pragma once

#include "fa_bwd_dq.hpp"
#include "fa_device.hpp"
#include "fa_launch.hpp"

#include <type_traits>

namespace fa {
namespace {

#ifndef FA_KV_PF
#define FA_KV_PF 2
#endif
#ifndef FA_KV_TF
#define FA_KV_TF 2
#endif
// Operand reads in flight ahead of the products of the split key side (d = 128).
#ifndef FA_KVS_PF
#define FA_KVS_PF 2
#endif
#ifndef FA_KVS_TF
#define FA_KVS_TF 2
#endif

constexpr int kBKV = 128;     // keys per workgroup
constexpr int kNW = 4;        // waves per workgroup (32 keys each)

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse2;     // LSE_i * log2(e), written by the pre-pass ([B*H, N] rows)
    const float* dsum;
    float* dq_acc;         // [B*H, N, D] fp32
    void* dk;
    void* dv;
    Strides lq, lk, lv, ldo, ldk, ldv;
    const int* cu;         // packed sequences, or null
    int total;
    int H, N, nkb, heads;
    float scale, sl2, inv_keep;
    uint32_t thr;
    PhiloxKey key;
};

// Source offset (bytes) of 16-byte chunk `ch` of row `row` in a tensor with
// row stride ld whose stored rows are DH elements wide; chunks past DH come
// from an out-of-range offset and load as zeros.
template <int DH>
__device__ __forceinline__ uint32_t chunk_src(int row, int ch, int ld) {
    return ch * 8 < DH ? (uint32_t)(row * ld + ch * 8) * 2 : 0xf0000000u;
}

// Transposed matrix-core operand: two ds_read_b64_tr_b16 at per-lane byte
// offsets off0/off1 (the first and second 8 rows of a 16-row block).
template <typename V8>
__device__ __forceinline__ V8 tr_read(const FA_LDS char* base, int off0, int off1) {
    const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(base + off0));
    const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(base + off1));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    return __builtin_bit_cast(V8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// DQ = false: the key/value side only (dK, dV); dQ then comes from its own
// pass (bwd_dq_kernel). Without the dQ products the Q/dO tiles are
// double-buffered and one barrier per tile remains.
template <typename T, int D, int DH, int BQ, bool CAUSAL, bool DROPOUT, bool DQ>
__global__ __launch_bounds__(kNW * 64) void bwd_kv_kernel(BwdParams p) {
    using V8 = typename Vec<T>::x8;
    using V4 = typename Vec<T>::x4;
    constexpr int CH = D / 8;
    constexpr int QB = BQ / 32;        // 32-row query blocks per tile
    constexpr int DB = D / 32;
    constexpr int NCD = D / 16;        // 16-wide d chunks (contraction of S and dP)
    constexpr int TILE = BQ * D * 2;
    constexpr int QLOADS = BQ * CH / (64 * kNW);
    constexpr int KLOADS = kBKV * CH / (64 * kNW);
    static_assert(QLOADS * 64 * kNW == BQ * CH, "query tile must split over the waves");
    static_assert(!DQ || BQ == 64, "dS^T rows need 8 chunks for the swizzle");
    static_assert(BQ == 32 || BQ == 64, "query tiles of 32 or 64 rows");
    static_assert((QB * DB) % kNW == 0, "dQ blocks must split evenly over the waves");
    constexpr int DQ_ATOMICS = (QB * DB / kNW) * 16;   // dQ atomics per lane per tile
    static_assert(!DQ || DQ_ATOMICS <= 63, "vmcnt holds at most 63");

    constexpr int NBUF = DQ ? 1 : 2;   // Q/dO tile buffers
    // LDS operand pairs in flight ahead of their products (S/dP, then dV/dK).
    constexpr int kPf = D == 256 ? 1 : FA_KV_PF, kTf = D == 256 ? 1 : FA_KV_TF;
    __shared__ __attribute__((aligned(1024))) char q_s[NBUF * TILE];
    __shared__ __attribute__((aligned(1024))) char do_s[NBUF * TILE];
    __shared__ __attribute__((aligned(1024))) char k_s[DQ ? kBKV * D * 2 : 16];
    __shared__ __attribute__((aligned(1024))) char dst_s[DQ ? kBKV * BQ * 2 : 16];
    // Row terms: 64 per buffer slot whatever BQ (one per lane of the copying wave).
    __shared__ float lse_s[NBUF * 64];
    __shared__ float dsum_s[NBUF * 64];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    FA_LDS char* const qL = (FA_LDS char*)q_s;
    FA_LDS char* const doL = (FA_LDS char*)do_s;
    FA_LDS char* const kL = (FA_LDS char*)k_s;
    FA_LDS char* const dsL = (FA_LDS char*)dst_s;

    int bh, kb;
    const int bid = blockIdx.x;
    if ((p.heads & 7) == 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        bh = (slot / p.nkb) * 8 + xcd;
        kb = slot % p.nkb;
    } else {
        bh = bid % p.heads;
        kb = bid / p.heads;
    }
    // Workgroup-uniform by construction; stated explicitly so that the buffer
    // descriptors below live in SGPRs.
    bh = __builtin_amdgcn_readfirstlane(bh);
    kb = __builtin_amdgcn_readfirstlane(kb);
    const int b = bh / p.H, h = bh - b * p.H;
    int start, N;
    sequence(p.cu, p.total, p.N, b, start, N);
    const int j0 = kb * kBKV;
    if (j0 >= N) return;                          // past this sequence's keys
    const int ldq = p.lq.sn, ldk = p.lk.sn, ldv = p.lv.sn, ldo = p.ldo.sn;
    const T* const qh = (const T*)p.q + p.lq.base(b, h, start);
    const T* const kh = (const T*)p.k + p.lk.base(b, h, start);
    const T* const vh = (const T*)p.v + p.lv.base(b, h, start);
    const T* const doh = (const T*)p.dout + p.ldo.base(b, h, start);
    const auto rs_q = make_rsrc(qh, (uint32_t)(((size_t)(N - 1) * ldq + DH) * 2));
    const auto rs_k = make_rsrc(kh, (uint32_t)(((size_t)(N - 1) * ldk + DH) * 2));
    const auto rs_v = make_rsrc(vh, (uint32_t)(((size_t)(N - 1) * ldv + DH) * 2));
    const auto rs_do = make_rsrc(doh, (uint32_t)(((size_t)(N - 1) * ldo + DH) * 2));
    // Row terms and the dQ accumulator: [B*H, p.N] rows in the workspace.
    const size_t wrow = (size_t)bh * p.N;
    const auto rs_lse = make_rsrc(p.lse2 + wrow, (uint32_t)N * 4);
    const auto rs_ds = make_rsrc(p.dsum + wrow, (uint32_t)N * 4);
    // dQ accumulator of the head; atomics at rows >= N fall outside and are dropped.
    const auto rs_dq = make_rsrc(p.dq_acc + wrow * D, (uint32_t)N * D * 4);

    const int kw = j0 + wave * 32;     // first key of this wave
    const int my_key = kw + l32;
    // Dropout generator of this lane's key column (counter b, h, row, key).
    const PhiloxCol philox_col((uint32_t)b, (uint32_t)h, (uint32_t)my_key, p.key);

    // Per-lane LDS byte offsets of the operand reads. The chunk swizzle depends
    // only on the low four row bits, so the 16-row and 32-row block terms added
    // to these are immediates.
    //  * row operand (Q, dO as A of S and dP): row l32, d = 16c + 8hi .. +7;
    //  * transposed operand (Q^T, dO^T, K as the contraction-over-rows side):
    //    within a 16-lane group, lane s reads row s/4 (+4 for the upper groups,
    //    +8 for the second read) and 4 columns at 4(s%4) of a 32-wide block;
    //  * dS^T tile (128-byte rows): the same pattern over query columns.
    const int grp = lane >> 4, sl = lane & 15;
    const int tr_row = 4 * (grp >> 1) + (sl >> 2), tr_col = 16 * (grp & 1) + 4 * (sl & 3);
    int roff[NCD], troff[DB][2], tsoff[QB][2];
#pragma unroll
    for (int c = 0; c < NCD; ++c) roff[c] = tile_offset<CH>(l32, 16 * c + 8 * hi);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int db = 0; db < DB; ++db) troff[db][half] = tile_offset<CH>(tr_row + 8 * half, 32 * db + tr_col);
        if constexpr (DQ) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) tsoff[qb][half] = tile_offset<BQ / 8>(tr_row + 8 * half, 32 * qb + tr_col);
        }
    }
    constexpr int ROW = D * 2, SROW = BQ * 2;     // LDS row bytes: Q/dO/K tiles, dS^T tile

    // K and V rows of this wave's keys as B operands (d chunk c: d = 16c + 8hi .. +7)
    V8 kt[NCD], vt[NCD];
#pragma unroll
    for (int c = 0; c < NCD; ++c) {
        kt[c] = __builtin_bit_cast(V8, buffer_load16(rs_k, chunk_src<DH>(my_key, 2 * c + hi, ldk)));
        vt[c] = __builtin_bit_cast(V8, buffer_load16(rs_v, chunk_src<DH>(my_key, 2 * c + hi, ldv)));
    }
    // All 128 keys of the block into LDS for the dQ products.
    if (DQ) {
#pragma unroll
        for (int i = 0; i < KLOADS; ++i) {
            const int blk = i * kNW + wave, pos = blk * 64 + lane;
            const int row = pos / CH, sw = pos % CH;
            buffer_to_lds16_async(rs_k, (FA_LDS void*)(kL + blk * 1024),
                            chunk_src<DH>(j0 + row, sw ^ chunk_swizzle<CH>(row), ldk));
        }
    }

    f32x16 dva[DB], dka[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) dva[i][r] = dka[i][r] = 0.0f;

    auto issue_tile = [&](int i0, int buf) {
#pragma unroll
        for (int i = 0; i < QLOADS; ++i) {
            const int blk = i * kNW + wave, pos = blk * 64 + lane;
            const int row = pos / CH, sw = pos % CH;
            const int ch = sw ^ chunk_swizzle<CH>(row);
            buffer_to_lds16_async(rs_q, (FA_LDS void*)(qL + buf * TILE + blk * 1024), chunk_src<DH>(i0 + row, ch, ldq));
            buffer_to_lds16_async(rs_do, (FA_LDS void*)(doL + buf * TILE + blk * 1024), chunk_src<DH>(i0 + row, ch, ldo));
        }
        if (wave == 0) buffer_to_lds4_async(rs_lse, (FA_LDS void*)(lse_s + buf * 64), (uint32_t)(i0 + lane) * 4);
        if (wave == 1) buffer_to_lds4_async(rs_ds, (FA_LDS void*)(dsum_s + buf * 64), (uint32_t)(i0 + lane) * 4);
    };

    // Query tiles run from the last one down to the first one this key block
    // sees. Every key block of a head then starts on the same tile, so the
    // workgroups of one head that run side by side on an XCD read the same Q
    // and dO tiles and add into the same dQ rows at about the same time, and
    // those stay in that XCD's L2.
    const int i_first = CAUSAL ? j0 : 0;         // j0 < N, so i_first <= i_last
    const int i_last = (N - 1) / BQ * BQ;
    issue_tile(i_last, 0);

    for (int i0 = i_last; i0 >= i_first; i0 -= BQ) {
        const int buf = DQ ? 0 : ((i_last - i0) / BQ) & 1;
        // Vector-memory operations retire in issue order, and the previous tile
        // issued this tile's loads before exactly DQ_ATOMICS atomics per lane:
        // waiting until at most that many remain waits for the loads only.
        if (!DQ || i0 == i_last)
            wait_vmem();
        else
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DQ_ATOMICS) : "memory");
        __syncthreads();
        if (!DQ && i0 > i_first) issue_tile(i0 - BQ, buf ^ 1);   // the other buffer: read last tile
        const FA_LDS char* const qT = qL + buf * TILE;
        const FA_LDS char* const doT = doL + buf * TILE;
        const float* const lse_t = lse_s + buf * 64;
        const float* const dsum_t = dsum_s + buf * 64;

        // Every query of the tile precedes our keys. (d = 256 runs such tiles
        // fully masked instead: their zero contributions cost less than the
        // register copies a second path through the loop costs.)
        const bool skip = CAUSAL && D != 256 && kw > i0 + BQ - 1;
        if (skip) {
            // this wave's rows of dS^T are zero for this tile
            if constexpr (DQ)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *(FA_LDS u32x2*)(dsL + tile_offset<BQ / 8>(wave * 32 + l32, qb * 32 + 8 * g + 4 * hi)) =
                        u32x2{0u, 0u};
        } else {
            // LDS operand reads run kPf steps ahead of their products; the
            // scheduling fences keep them there (one wave per SIMD here, so
            // nothing else hides their latency).
            f32x16 s[QB], dp[QB];
            if constexpr (DQ) {
                // the fused form: the compiler's own order measured faster here
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
                    for (int c = 0; c < NCD; ++c) {
                        const int o = roff[c] + qb * 32 * ROW;
                        s[qb] = mfma32(*(const FA_LDS V8*)(qT + o), kt[c], c == 0 ? f32x16{} : s[qb]);
                        dp[qb] = mfma32(*(const FA_LDS V8*)(doT + o), vt[c], c == 0 ? f32x16{} : dp[qb]);
                    }
                }
            } else {
                constexpr int SI = QB * NCD;
                auto so = [&](int i) { return roff[i % NCD] + (i / NCD) * 32 * ROW; };
                V8 qa[kPf], da[kPf];
#pragma unroll
                for (int j = 0; j < kPf; ++j) {
                    qa[j] = *(const FA_LDS V8*)(qT + so(j));
                    da[j] = *(const FA_LDS V8*)(doT + so(j));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < SI; ++i) {
                    const int qb = i / NCD, c = i % NCD;
                    s[qb] = mfma32(qa[i % kPf], kt[c], c == 0 ? f32x16{} : s[qb]);
                    dp[qb] = mfma32(da[i % kPf], vt[c], c == 0 ? f32x16{} : dp[qb]);
                    if (i + kPf < SI) {
                        qa[i % kPf] = *(const FA_LDS V8*)(qT + so(i + kPf));
                        da[i % kPf] = *(const FA_LDS V8*)(doT + so(i + kPf));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // P and dS of 16-row chunk qc + 1 between the dV/dK products of chunk qc
            // (the two-pass form at d = 64: one wave per SIMD, so no other wave fills
            // the matrix core while this one does vector work; measured 4% faster).
            // At d = 128 it measured 7% slower, and the padded d = 32 kernel would
            // lose a wave per SIMD, so every other kernel keeps the order below.
            constexpr bool kChunked = !DQ && D == 64 && DH == 64;
            if constexpr (kChunked) {
                if ((CAUSAL && i0 < kw + 31) || kw + 32 > N || i0 + BQ > N) {
                    const int e_lo = CAUSAL ? my_key - i0 - 4 * hi : -1;   // causal: e >= e_lo
                    const int e_hi = my_key < N ? N - i0 - 4 * hi : 0;       // e < e_hi (none past N)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int e = qb * 32 + 8 * (r >> 2) + (r & 3);
                            if (e < e_lo || e >= e_hi) s[qb][r] = -INFINITY;   // -inf stays -inf below
                        }
                }
                // P = exp2(s scale log2(e) - LSE_i log2(e)) and dS = P (dP Z' - D_i) of
                // element (qb, r), rounded to the element type into the product
                // operands bp_out[idx] (P Z', for dV) and bs_out[idx] (dS, for dK)
                auto p_ds = [&](int qb, int r, V8& bp_out, V8& bs_out, int idx) {
                    const int qrow = qb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    const float pr = fast_exp2(fmaf(s[qb][r], p.sl2, -lse_t[qrow]));   // exp2(-inf) = 0
                    float z = 1.0f;
                    if (DROPOUT) {
                        const uint32_t w = philox_col.word0((uint32_t)(i0 + qrow));
                        z = w >= p.thr ? p.inv_keep : 0.0f;
                    }
                    const float ds = pr * fmaf(dp[qb][r], z, -dsum_t[qrow]);
                    bp_out[idx] = (T)(pr * z);
                    bs_out[idx] = (T)ds;
                };
                constexpr int TI = (BQ / 16) * DB;     // steps j = qc * DB + db
                auto to = [&](int j, int half) { return troff[j % DB][half] + 16 * (j / DB) * ROW; };
                V8 oa[kTf], ta[kTf];
#pragma unroll
                for (int j = 0; j < kTf; ++j) {
                    oa[j] = tr_read<V8>(doT, to(j, 0), to(j, 1));
                    ta[j] = tr_read<V8>(qT, to(j, 0), to(j, 1));
                }
                V8 bp[2], bs[2];
#pragma unroll
                for (int i = 0; i < 8; ++i) p_ds(0, i, bp[0], bs[0], i);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < TI; ++j) {
                    const int qc = j / DB, db = j % DB;
                    dva[db] = mfma32(oa[j % kTf], bp[qc & 1], dva[db]);
                    dka[db] = mfma32(ta[j % kTf], bs[qc & 1], dka[db]);
                    if (j + kTf < TI) {
                        oa[j % kTf] = tr_read<V8>(doT, to(j + kTf, 0), to(j + kTf, 1));
                        ta[j % kTf] = tr_read<V8>(qT, to(j + kTf, 0), to(j + kTf, 1));
                    }
                    // the elements of chunk qc + 1 that ride behind these products
                    if (qc + 1 < BQ / 16) {
                        const int nq = qc + 1;
#pragma unroll
                        for (int i = db * 8 / DB; i < (db + 1) * 8 / DB; ++i)
                            p_ds(nq >> 1, 8 * (nq & 1) + i, bp[nq & 1], bs[nq & 1], i);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // log2 of P: s * scale * log2(e) - LSE_i * log2(e)
    #pragma unroll
                for (int qb = 0; qb < QB; ++qb)
    #pragma unroll
                    for (int r = 0; r < 16; ++r)
                        s[qb][r] = fmaf(s[qb][r], p.sl2, -lse_t[qb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3)]);
                // Only tiles that cross the diagonal or a ragged end hold masked elements.
                // Element (qb, r) is query row i0 + 4hi + e with e = 32qb + 8(r/4) + r%4, a
                // compile-time offset; the bounds are moved to the lane's side.
                if ((CAUSAL && i0 < kw + 31) || kw + 32 > N || i0 + BQ > N) {
                    const int e_lo = CAUSAL ? my_key - i0 - 4 * hi : -1;   // causal: e >= e_lo
                    const int e_hi = my_key < N ? N - i0 - 4 * hi : 0;       // e < e_hi (none past N)
    #pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
    #pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int e = qb * 32 + 8 * (r >> 2) + (r & 3);
                            if (e < e_lo || e >= e_hi) s[qb][r] = -INFINITY;
                        }
                }
    #pragma unroll
                for (int qb = 0; qb < QB; ++qb)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int qrow = qb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                        const int qi = i0 + qrow;
                        const float pr = fast_exp2(s[qb][r]);     // exp2(-inf) = 0
                        float z = 1.0f;
                        if (DROPOUT) {
                            const uint32_t w = philox_col.word0((uint32_t)qi);
                            z = w >= p.thr ? p.inv_keep : 0.0f;
                        }
                        const float ds = pr * fmaf(dp[qb][r], z, -dsum_t[qrow]);
                        s[qb][r] = pr * z;      // P Z' for dV
                        dp[qb][r] = ds;         // dS
                    }
                // dV^T += dO^T (P Z'),  dK^T += Q^T dS  (contraction over the tile's query rows)
                if constexpr (DQ) {
    #pragma unroll
                    for (int qc = 0; qc < BQ / 16; ++qc) {
                        V8 bp, bs;
    #pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            bp[i] = (T)s[qc >> 1][8 * (qc & 1) + i];
                            bs[i] = (T)dp[qc >> 1][8 * (qc & 1) + i];
                        }
    #pragma unroll
                        for (int db = 0; db < DB; ++db) {
                            const int o0 = troff[db][0] + 16 * qc * ROW, o1 = troff[db][1] + 16 * qc * ROW;
                            dva[db] = mfma32(tr_read<V8>(doT, o0, o1), bp, dva[db]);
                            dka[db] = mfma32(tr_read<V8>(qT, o0, o1), bs, dka[db]);
                        }
                    }
                } else {
                    constexpr int TI = (BQ / 16) * DB;     // steps j = qc * DB + db
                    auto to = [&](int j, int half) { return troff[j % DB][half] + 16 * (j / DB) * ROW; };
                    V8 oa[kTf], ta[kTf];
    #pragma unroll
                    for (int j = 0; j < kTf; ++j) {
                        oa[j] = tr_read<V8>(doT, to(j, 0), to(j, 1));
                        ta[j] = tr_read<V8>(qT, to(j, 0), to(j, 1));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    V8 bp, bs;
    #pragma unroll
                    for (int j = 0; j < TI; ++j) {
                        const int qc = j / DB, db = j % DB;
                        if (db == 0) {
    #pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                bp[i] = (T)s[qc >> 1][8 * (qc & 1) + i];
                                bs[i] = (T)dp[qc >> 1][8 * (qc & 1) + i];
                            }
                        }
                        dva[db] = mfma32(oa[j % kTf], bp, dva[db]);
                        dka[db] = mfma32(ta[j % kTf], bs, dka[db]);
                        if (j + kTf < TI) {
                            oa[j % kTf] = tr_read<V8>(doT, to(j + kTf, 0), to(j + kTf, 1));
                            ta[j % kTf] = tr_read<V8>(qT, to(j + kTf, 0), to(j + kTf, 1));
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            // dS^T (bf16) to LDS: row = key within the block, columns = query rows
            if constexpr (DQ)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w;
                    w[0] = pack2<T>(dp[qb][4 * g + 0], dp[qb][4 * g + 1]);
                    w[1] = pack2<T>(dp[qb][4 * g + 2], dp[qb][4 * g + 3]);
                    *(FA_LDS u32x2*)(dsL + tile_offset<BQ / 8>(wave * 32 + l32, qb * 32 + 8 * g + 4 * hi)) = w;
                }
        }
        if (!DQ) continue;
        __syncthreads();
        if (i0 > i_first) issue_tile(i0 - BQ, 0);   // Q/dO/LSE/D are not read again this tile

        // dQ_tile = dS K over the block's 128 keys, 32x32 blocks dealt to the waves
#pragma unroll
        for (int blk = wave; blk < QB * DB; blk += kNW) {
            const int qb = blk / DB, db = blk % DB;
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
            for (int kc = 0; kc < kBKV / 16; ++kc)
                acc = mfma32(tr_read<V8>(dsL, tsoff[qb][0] + 16 * kc * SROW, tsoff[qb][1] + 16 * kc * SROW),
                             tr_read<V8>(kL, troff[db][0] + 16 * kc * ROW, troff[db][1] + 16 * kc * ROW), acc);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qi = i0 + qb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                    acc[r] * p.scale, rs_dq, (uint32_t)(qi * D + 32 * db + l32) * 4, 0, 0);
            }
        }
    }

    // dK = s dK^T, dV = dV^T, transposed on the way out (lane = key, registers = d)
    if (my_key < N) {
        T* dkr = (T*)p.dk + p.ldk.base(b, h, start) + (size_t)my_key * p.ldk.sn;
        T* dvr = (T*)p.dv + p.ldv.base(b, h, start) + (size_t)my_key * p.ldv.sn;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            if (32 * db >= DH) break;          // padded columns are not stored
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                V4 wk, wv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    wk[i] = (T)(dka[db][4 * g + i] * p.scale);
                    wv[i] = (T)dva[db][4 * g + i];
                }
                *(V4*)(dkr + 32 * db + 8 * g + 4 * hi) = wk;
                *(V4*)(dvr + 32 * db + 8 * g + 4 * hi) = wv;
            }
        }
    }
}

// Key-side pass of the two-pass form at d = 128 with the work of 32 keys
// split between two waves on one SIMD (8 waves, 128 keys per workgroup). (It
// also builds for d = 64, where the one-wave kernel above measured faster.)
// Wave p (p < 4) takes the P side: S = Q K^T, P = exp(S - LSE), and
// dV^T += dO^T (P Z'). Wave p + 4, on the same SIMD, takes the dS side:
// dP = dO V^T, dS = P (dP Z' - D), and dK^T += Q^T dS. Each wave then holds one
// operand block and one accumulator pair (K or V, dV^T or dK^T), which fits the
// 256 registers of a lane at two waves per SIMD, and each SIMD always has a
// second wave whose products run while the first does vector work or waits for
// LDS. P crosses from the P side to the dS side through LDS in fp32 (its sign
// bit carries the dropout decision Z = 0), one tile late: in iteration t the dS
// side forms dS and the dK products of tile t - 1 while both sides run the
// products of tile t, so one barrier per tile orders everything. Q tiles are
// kept three deep (t - 1 for dK, t, t + 1 arriving), dO tiles two deep. The
// arithmetic of every element and the order of every accumulation are those of
// bwd_kv_kernel, so dK and dV are bit-identical to it.
template <typename T, int D, int DH, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(2 * kNW * 64) void bwd_kv_split_kernel(BwdParams p) {
    using V8 = typename Vec<T>::x8;
    constexpr int NW = 2 * kNW;                      // waves per workgroup
    constexpr int BQ = 64, QB = 2, CH = D / 8, DB = D / 32, NCD = D / 16;
    constexpr int TILE = BQ * D * 2, ROW = D * 2;
    constexpr int QLOADS = BQ * CH / (64 * kNW);     // copies per P-side wave and tensor
    constexpr int NQ = 3, NO = 2;                    // Q and dO tile buffers
    constexpr int XF = kNW * QB * 16 * 64;           // floats of P per exchange buffer
    constexpr int kPf = FA_KVS_PF, kTf = FA_KVS_TF;
    constexpr int kXa = 2;                           // dS side: P and D groups read ahead
    constexpr int SI = QB * NCD;                     // score products per wave and tile
    constexpr int TI = (BQ / 16) * DB;               // dV or dK products per wave and tile
    static_assert(D == 64 || D == 128, "d = 64 or 128");
    static_assert(QB * 4 <= SI, "the P side reads its LSE groups during the score products");
    static_assert(QLOADS >= 1 && QLOADS * 64 * kNW == BQ * CH, "copies split over the P-side waves");
    __shared__ __attribute__((aligned(1024))) char q_s[NQ * TILE];
    __shared__ __attribute__((aligned(1024))) char do_s[NO * TILE];
    __shared__ __attribute__((aligned(16))) float x_s[2 * XF];
    __shared__ __attribute__((aligned(16))) float lse_s[NQ * 64];
    __shared__ __attribute__((aligned(16))) float dsum_s[NQ * 64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = wave & 3;                       // key slice; waves pair and pair + 4 share a SIMD
    const bool dside = wave >= kNW;
    const int l32 = lane & 31, hi = lane >> 5;
    FA_LDS char* const qL = (FA_LDS char*)q_s;
    FA_LDS char* const doL = (FA_LDS char*)do_s;

    int bh, kb;
    const int bid = blockIdx.x;
    if ((p.heads & 7) == 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        bh = (slot / p.nkb) * 8 + xcd;
        kb = slot % p.nkb;
    } else {
        bh = bid % p.heads;
        kb = bid / p.heads;
    }
    bh = __builtin_amdgcn_readfirstlane(bh);
    kb = __builtin_amdgcn_readfirstlane(kb);
    const int b = bh / p.H, h = bh - b * p.H;
    int start, N;
    sequence(p.cu, p.total, p.N, b, start, N);
    const int j0 = kb * kBKV;
    if (j0 >= N) return;
    const int ldq = p.lq.sn, ldk = p.lk.sn, ldv = p.lv.sn, ldo = p.ldo.sn;
    const T* const qh = (const T*)p.q + p.lq.base(b, h, start);
    const T* const kh = (const T*)p.k + p.lk.base(b, h, start);
    const T* const vh = (const T*)p.v + p.lv.base(b, h, start);
    const T* const doh = (const T*)p.dout + p.ldo.base(b, h, start);
    const auto rs_q = make_rsrc(qh, (uint32_t)(((size_t)(N - 1) * ldq + DH) * 2));
    const auto rs_k = make_rsrc(kh, (uint32_t)(((size_t)(N - 1) * ldk + DH) * 2));
    const auto rs_v = make_rsrc(vh, (uint32_t)(((size_t)(N - 1) * ldv + DH) * 2));
    const auto rs_do = make_rsrc(doh, (uint32_t)(((size_t)(N - 1) * ldo + DH) * 2));
    const size_t wrow = (size_t)bh * p.N;
    const auto rs_lse = make_rsrc(p.lse2 + wrow, (uint32_t)N * 4);
    const auto rs_ds = make_rsrc(p.dsum + wrow, (uint32_t)N * 4);

    const int kw = j0 + pair * 32;
    const int my_key = kw + l32;
    const PhiloxCol philox_col((uint32_t)b, (uint32_t)h, (uint32_t)my_key, p.key);

    // Operand offsets as in bwd_kv_kernel.
    const int grp = lane >> 4, sl = lane & 15;
    const int tr_row = 4 * (grp >> 1) + (sl >> 2), tr_col = 16 * (grp & 1) + 4 * (sl & 3);
    int roff[NCD], troff[DB][2];
#pragma unroll
    for (int c = 0; c < NCD; ++c) roff[c] = tile_offset<CH>(l32, 16 * c + 8 * hi);
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int db = 0; db < DB; ++db) troff[db][half] = tile_offset<CH>(tr_row + 8 * half, 32 * db + tr_col);
    auto so = [&](int i) { return roff[i / QB] + (i % QB) * 32 * ROW; };       // score step i: chunk i/QB, block i%QB
    auto to = [&](int j, int half) { return troff[j % DB][half] + 16 * (j / DB) * ROW; };

    // K rows (P side) or V rows (dS side) of this pair's keys as B operands.
    V8 kv[NCD];
    {
        const auto rs = dside ? rs_v : rs_k;
        const int ld = dside ? ldv : ldk;
#pragma unroll
        for (int c = 0; c < NCD; ++c) kv[c] = __builtin_bit_cast(V8, buffer_load16(rs, chunk_src<DH>(my_key, 2 * c + hi, ld)));
    }
    f32x16 acc[DB];                 // dV^T (P side) or dK^T (dS side)
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    f32x16 sc[QB];                  // S (P side) or dP of the previous tile (dS side)
    V8 bop[BQ / 16];                // P Z' (P side) or dS (dS side), bf16 B operands

    // Copies of tile i0: QLOADS Q chunks and QLOADS dO chunks per P-side wave,
    // and one row-term copy (LSE by even pairs, D by odd ones). A wave that
    // issues copies stalls until the CU's memory path has taken them (about
    // 700 cycles for a tile's 36 KB). The P side issues every copy, after its
    // score products: its waves wait at each barrier for the dS side, so the
    // stall comes out of that wait. Issued by the dS side, the copies delayed
    // its dS elements, which lie on the tile's critical path.
    auto issue_tile = [&](int i0, int t) __attribute__((always_inline)) {
        const int qbuf = t % NQ, obuf = t % NO;
#pragma unroll
        for (int i = 0; i < QLOADS; ++i) {
            const int blk = i * kNW + pair, pos = blk * 64 + lane;
            const int row = pos / CH, ch = (pos % CH) ^ chunk_swizzle<CH>(row);
            buffer_to_lds16_async(rs_q, (FA_LDS void*)(qL + qbuf * TILE + blk * 1024), chunk_src<DH>(i0 + row, ch, ldq));
            buffer_to_lds16_async(rs_do, (FA_LDS void*)(doL + obuf * TILE + blk * 1024),
                                  chunk_src<DH>(i0 + row, ch, ldo));
        }
        if (pair & 1)
            buffer_to_lds4_async(rs_ds, (FA_LDS void*)(dsum_s + qbuf * 64), (uint32_t)(i0 + lane) * 4);
        else
            buffer_to_lds4_async(rs_lse, (FA_LDS void*)(lse_s + qbuf * 64), (uint32_t)(i0 + lane) * 4);
    };

    // LSE or D of tile t, group n = 4qb + g: rows 32qb + 8g + 4hi .. +3, the
    // elements r = 4g .. 4g + 3 of score block qb.
    auto row_terms = [&](const float* base, int t, int n) {
        return *(const f32x4*)(base + (t % NQ) * 64 + (n >> 2) * 32 + 8 * (n & 3) + 4 * hi);
    };
    // dS of tile t (from dP in sc, P from exchange buffer t % 2, D from slot
    // t % NQ) into bop, then dK^T += Q^T dS over Q buffer t % NQ. The dP
    // products of the next tile, if any (NEXT), are interleaved with the dK
    // products.
    auto ds_side = [&](int t, auto next, int tn) __attribute__((always_inline)) {
        constexpr bool NEXT = decltype(next)::value;
        const float* const xp = x_s + (t & 1) * XF + pair * QB * 16 * 64;
        // group n: its P and D are read kXa groups ahead
        auto xo = [&](int n) { return xp + (n * 64 + lane) * 4; };
        f32x4 xr[kXa], dr[kXa];
#pragma unroll
        for (int a = 0; a < kXa; ++a) {
            xr[a] = *(const f32x4*)xo(a);
            dr[a] = row_terms(dsum_s, t, a);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int n = 0; n < QB * 4; ++n) {
            const int qb = n >> 2, g = n & 3;
            const f32x4 x = xr[n % kXa], dd = dr[n % kXa];
            if (n + kXa < QB * 4) {
                xr[n % kXa] = *(const f32x4*)xo(n + kXa);
                dr[n % kXa] = row_terms(dsum_s, t, n + kXa);
            }
            float ds[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float pr = x[u], z = 1.0f;
                if (DROPOUT) {
                    const uint32_t bits = __float_as_uint(x[u]);
                    z = (bits >> 31) ? 0.0f : p.inv_keep;
                    pr = __uint_as_float(bits & 0x7fffffffu);
                }
                ds[u] = pr * fmaf(sc[qb][4 * g + u], z, -dd[u]);
            }
            // element r = 4g + u of block qb is element 8(qc & 1) + i of chunk qc = 2qb + g/2
            const int qc = 2 * qb + (g >> 1), i = 4 * (g & 1);
#pragma unroll
            for (int u = 0; u < 4; ++u) bop[qc][i + u] = (T)ds[u];
            __builtin_amdgcn_sched_barrier(0);
        }
        const FA_LDS char* const qT = qL + (t % NQ) * TILE;
        const FA_LDS char* const doN = doL + (tn % NO) * TILE;
        V8 ta[kTf], da[kPf];
#pragma unroll
        for (int j = 0; j < kTf; ++j) ta[j] = tr_read<V8>(qT, to(j, 0), to(j, 1));
        if constexpr (NEXT) {
#pragma unroll
            for (int j = 0; j < kPf; ++j) da[j] = *(const FA_LDS V8*)(doN + so(j));
        }
        __builtin_amdgcn_sched_barrier(0);
        static_assert(TI == SI, "one dP product per dK product");
#pragma unroll
        for (int j = 0; j < TI; ++j) {
            const int qc = j / DB, db = j % DB;
            acc[db] = mfma32(ta[j % kTf], bop[qc], acc[db]);
            if (j + kTf < TI) ta[j % kTf] = tr_read<V8>(qT, to(j + kTf, 0), to(j + kTf, 1));
            if constexpr (NEXT) {
                const int qb = j % QB, c = j / QB;
                sc[qb] = mfma32(da[j % kPf], kv[c], c == 0 ? f32x16{} : sc[qb]);
                if (j + kPf < SI) da[j % kPf] = *(const FA_LDS V8*)(doN + so(j + kPf));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    const int i_first = CAUSAL ? j0 : 0;
    const int i_last = (N - 1) / BQ * BQ;
    const int ntiles = (i_last - i_first) / BQ + 1;   // tile t starts at row i_last - t BQ
    if (!dside) issue_tile(i_last, 0);

    // Each side runs a loop of its own (their loop-invariant values would
    // otherwise all be live in one loop); both take the same barriers.
    if (!dside) {
        for (int t = 0; t < ntiles; ++t) {
            const int i0 = i_last - t * BQ;
            wait_vmem();
            __syncthreads();
            // ---- P side: S = Q K^T of tile t (its LSE read meanwhile)
            const FA_LDS char* const qT = qL + (t % NQ) * TILE;
            f32x4 lreg[QB * 4];
            V8 qa[kPf];
#pragma unroll
            for (int j = 0; j < kPf; ++j) qa[j] = *(const FA_LDS V8*)(qT + so(j));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < SI; ++i) {
                const int qb = i % QB, c = i / QB;
                sc[qb] = mfma32(qa[i % kPf], kv[c], c == 0 ? f32x16{} : sc[qb]);
                if (i + kPf < SI) qa[i % kPf] = *(const FA_LDS V8*)(qT + so(i + kPf));
                if (i < QB * 4) lreg[i] = row_terms(lse_s, t, i);
                __builtin_amdgcn_sched_barrier(0);
            }
            // the next tile's copies (see issue_tile)
            if (t + 1 < ntiles) issue_tile(i0 - BQ, t + 1);
            if ((CAUSAL && i0 < kw + 31) || kw + 32 > N || i0 + BQ > N) {
                const int e_lo = CAUSAL ? my_key - i0 - 4 * hi : -1;   // causal: e >= e_lo
                const int e_hi = my_key < N ? N - i0 - 4 * hi : 0;       // e < e_hi (none past N)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int e = qb * 32 + 8 * (r >> 2) + (r & 3);
                        if (e < e_lo || e >= e_hi) sc[qb][r] = -INFINITY;
                    }
            }
            // P = exp2(s scale log2(e) - LSE_i log2(e)); P Z' into the dV operands,
            // P (sign = dropped) to the dS side
            float* const xp = x_s + (t & 1) * XF + pair * QB * 16 * 64;
#pragma unroll
            for (int n = 0; n < QB * 4; ++n) {
                const int qb = n >> 2, g = n & 3;
                const f32x4 lv = lreg[n];
                f32x4 x;
                const int qc = 2 * qb + (g >> 1), i = 4 * (g & 1);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float pr = fast_exp2(fmaf(sc[qb][4 * g + u], p.sl2, -lv[u]));   // exp2(-inf) = 0
                    float z = 1.0f;
                    x[u] = pr;
                    if (DROPOUT) {
                        const int qrow = qb * 32 + 8 * g + 4 * hi + u;
                        const bool keep = philox_col.word0((uint32_t)(i0 + qrow)) >= p.thr;
                        z = keep ? p.inv_keep : 0.0f;
                        x[u] = __uint_as_float(__float_as_uint(pr) | (keep ? 0u : 0x80000000u));
                    }
                    bop[qc][i + u] = (T)(pr * z);
                }
                *(f32x4*)(xp + (n * 64 + lane) * 4) = x;
                __builtin_amdgcn_sched_barrier(0);
            }
            // dV^T += dO^T (P Z') over tile t
            const FA_LDS char* const doT = doL + (t % NO) * TILE;
            V8 oa[kTf];
#pragma unroll
            for (int j = 0; j < kTf; ++j) oa[j] = tr_read<V8>(doT, to(j, 0), to(j, 1));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < TI; ++j) {
                const int qc = j / DB, db = j % DB;
                acc[db] = mfma32(oa[j % kTf], bop[qc], acc[db]);
                if (j + kTf < TI) oa[j % kTf] = tr_read<V8>(doT, to(j + kTf, 0), to(j + kTf, 1));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();
    } else {
        for (int t = 0; t < ntiles; ++t) {
            const int i0 = i_last - t * BQ;
            wait_vmem();
            __syncthreads();
            // ---- dS side: dS and dK of tile t - 1, with the dP products of tile t
            if (t == 0) {
                const FA_LDS char* const doT = doL;
                V8 da[kPf];
#pragma unroll
                for (int j = 0; j < kPf; ++j) da[j] = *(const FA_LDS V8*)(doT + so(j));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < SI; ++i) {
                    const int qb = i % QB, c = i / QB;
                    sc[qb] = mfma32(da[i % kPf], kv[c], c == 0 ? f32x16{} : sc[qb]);
                    if (i + kPf < SI) da[i % kPf] = *(const FA_LDS V8*)(doT + so(i + kPf));
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                ds_side(t - 1, std::true_type{}, t);
            }
        }
        // the last tile's dS and dK (its P was written in the last iteration)
        __syncthreads();
        ds_side(ntiles - 1, std::false_type{}, 0);
    }

    {
        // dV (P side) or dK (dS side) through LDS, stored four whole rows per
        // instruction (a lane of the product layout holds 4-element runs of one
        // key's row, so its direct stores touch 32 rows each). The P side stages
        // in the dO buffers (past the final barrier nothing reads them), the dS
        // side in the exchange buffer its last dS did not read; 8 KB per wave,
        // rows unpadded with 16-byte chunk c of row r at c ^ (r % RCH).
        using V4 = typename Vec<T>::x4;
        constexpr int RCH = D / 8, SROWB = D * 2;
        static_assert(kNW * 32 * SROWB <= NO * TILE && kNW * 32 * SROWB <= XF * 4, "staging fits");
        FA_LDS char* const stg = (dside ? (FA_LDS char*)(x_s + (ntiles & 1) * XF) : doL) + pair * (32 * SROWB);
        const float mul = dside ? p.scale : 1.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                V4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (T)(dside ? acc[db][4 * g + i] * mul : acc[db][4 * g + i]);
                const int c = 4 * db + g;   // 16-byte chunk of the row (8 elements)
                *(FA_LDS V4*)(stg + l32 * SROWB + ((c ^ (l32 % RCH)) * 16) + hi * 8) = w;
            }
        asm volatile("" ::: "memory");
        const Strides& lo = dside ? p.ldk : p.ldv;
        T* const base = (T*)(dside ? p.dk : p.dv) + lo.base(b, h, start);
#pragma unroll
        for (int i = 0; i < 32 * RCH / 64; ++i) {
            const int pos = i * 64 + lane, r = pos / RCH, c = pos % RCH;
            const typename Vec<T>::x8 w = *(const FA_LDS typename Vec<T>::x8*)(stg + r * SROWB + ((c ^ (r % RCH)) * 16));
            if (kw + r < N && c * 8 < DH) *(typename Vec<T>::x8*)(base + (size_t)(kw + r) * lo.sn + c * 8) = w;
        }
    }
}

// Row terms of the backward, one workspace row r = (b*H + h)*N + i per query
// row: D_i = <dO_i, O_i> in fp32 and LSE_i in log2 units; ZERO also clears the
// row's dQ accumulator (DZ floats). 8 lanes per row.
struct PreParams {
    const void* o;
    const void* dout;
    const float* lse;
    float* dsum;
    float* lse2;
    float* dq_acc;
    Strides lo, ldo, ll;
    const int* cu;
    int total, H, N, rows;
};

template <typename T, int DH, int DZ, bool ZERO>
__global__ __launch_bounds__(256) void bwd_pre_kernel(PreParams p) {
    using V8 = typename Vec<T>::x8;
    constexpr int CH = DH / 8;
    const int r = blockIdx.x * 32 + (threadIdx.x >> 3);
    const int part = threadIdx.x & 7;
    if (r >= p.rows) return;
    if (ZERO) {
        float* z = p.dq_acc + (size_t)r * DZ;
#pragma unroll
        for (int c = part * 4; c < DZ; c += 32) *(f32x4*)(z + c) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int bh = r / p.N, i = r - bh * p.N;
    const int b = bh / p.H, h = bh - b * p.H;
    int start, n;
    sequence(p.cu, p.total, p.N, b, start, n);
    float acc = 0.0f;
    if (i < n) {
        const T* orow = (const T*)p.o + p.lo.base(b, h, start) + (size_t)i * p.lo.sn;
        const T* grow = (const T*)p.dout + p.ldo.base(b, h, start) + (size_t)i * p.ldo.sn;
#pragma unroll
        for (int c = part; c < CH; c += 8) {
            const V8 a = *(const V8*)(orow + 8 * c);
            const V8 g = *(const V8*)(grow + 8 * c);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)g[e], acc);
        }
    }
    // The 8 lanes of a row are consecutive and every lane of the group is live
    // (rows are whole 8-lane groups), so the exchanges stay inside the row.
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (i < n && part == 0) {
        p.dsum[r] = acc;
        p.lse2[r] = p.lse[p.ll.base(b, h, start) + (size_t)i * p.ll.sn] * kLog2e;
    }
}

// dQ = element type of the fp32 accumulator (D-wide rows), DH columns stored
// through the dQ layout; one thread per 8 elements.
struct ConvertParams {
    const float* acc;
    void* dq;
    Strides ldq;
    const int* cu;
    int total, H, N;
    size_t n8;
};

template <typename T, int D, int DH>
__global__ __launch_bounds__(256) void dq_convert_kernel(ConvertParams p) {
    using V8 = typename Vec<T>::x8;
    constexpr int CH = DH / 8;
    const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= p.n8) return;
    const size_t r = t / CH;
    const int c = (int)(t - r * CH);
    const int bh = (int)(r / p.N), i = (int)(r - (size_t)bh * p.N);
    const int b = bh / p.H, h = bh - b * p.H;
    int start, n;
    sequence(p.cu, p.total, p.N, b, start, n);
    if (i >= n) return;
    const float* a = p.acc + r * D + 8 * c;
    const f32x4 x = *(const f32x4*)a;
    const f32x4 y = *(const f32x4*)(a + 4);
    V8 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        w[e] = (T)x[e];
        w[4 + e] = (T)y[e];
    }
    *(V8*)((T*)p.dq + p.ldq.base(b, h, start) + (size_t)i * p.ldq.sn + 8 * c) = w;
}

template <typename T, int D, int DH, bool CAUSAL, bool DROPOUT, bool DQ>
hipError_t launch_kv_cfg(const BwdArgs& a, hipStream_t st) {
    BwdParams p{};
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.dout = a.dout;
    p.lse2 = a.lse2;
    p.dsum = a.dsum;
    p.dq_acc = a.dq_accum;
    p.dk = a.dk;
    p.dv = a.dv;
    p.lq = a.L.q;
    p.lk = a.L.k;
    p.lv = a.L.v;
    p.ldo = a.L.dout;
    p.ldk = a.L.dk;
    p.ldv = a.L.dv;
    p.cu = a.L.cu_seqlens;
    p.total = a.L.total;
    p.H = a.s.H;
    p.N = a.s.N;
    p.nkb = (a.s.N + kBKV - 1) / kBKV;
    p.heads = a.s.B * a.s.H;
    p.scale = a.s.scale;
    p.sl2 = a.s.scale * kLog2e;
    p.inv_keep = 1.0f / (1.0f - a.s.dropout_p);
    p.thr = dropout_threshold(a.s.dropout_p);
    p.key = PhiloxKey{(uint32_t)(a.s.seed & 0xffffffffu), (uint32_t)(a.s.seed >> 32)};
    // d = 256: 32-row query tiles, so that K, V, dK, dV of a wave's 32 keys and
    // the score tile fit in the 512 registers of a lane.
    constexpr int BQ = D == 256 ? 32 : 64;
    // d = 128, two-pass form: the key side split over two waves per SIMD.
    if constexpr (!DQ && D == 128)
        hipLaunchKernelGGL((bwd_kv_split_kernel<T, D, DH, CAUSAL, DROPOUT>), dim3(p.heads * p.nkb),
                           dim3(2 * kNW * 64), 0, st, p);
    else
        hipLaunchKernelGGL((bwd_kv_kernel<T, D, DH, BQ, CAUSAL, DROPOUT, DQ>), dim3(p.heads * p.nkb),
                           dim3(kNW * 64), 0, st, p);
    return hipGetLastError();
}

template <typename T, int D, int DH, bool DQ>
hipError_t launch_kv(const BwdArgs& a, hipStream_t st) {
    const bool drop = dropout_threshold(a.s.dropout_p) != 0;
    if (a.s.causal)
        return drop ? launch_kv_cfg<T, D, DH, true, true, DQ>(a, st) : launch_kv_cfg<T, D, DH, true, false, DQ>(a, st);
    return drop ? launch_kv_cfg<T, D, DH, false, true, DQ>(a, st) : launch_kv_cfg<T, D, DH, false, false, DQ>(a, st);
}

template <typename T, int DH, int DZ, bool ZERO>
void launch_pre(const BwdArgs& a, hipStream_t st) {
    PreParams p{};
    p.o = a.o;
    p.dout = a.dout;
    p.lse = a.lse;
    p.dsum = a.dsum;
    p.lse2 = a.lse2;
    p.dq_acc = a.dq_accum;
    p.lo = a.L.o;
    p.ldo = a.L.dout;
    p.ll = a.L.lse;
    p.cu = a.L.cu_seqlens;
    p.total = a.L.total;
    p.H = a.s.H;
    p.N = a.s.N;
    p.rows = a.s.B * a.s.H * a.s.N;
    hipLaunchKernelGGL((bwd_pre_kernel<T, DH, DZ, ZERO>), dim3((p.rows + 31) / 32), dim3(256), 0, st, p);
}

// The two-pass backward (key side, then dQ), or with dropout the fused one with
// dQ atomics. D: computed width; DH: stored head size.
template <typename T, int D, int DH>
hipError_t launch_bwd_td(const BwdArgs& a, hipStream_t st) {
    const bool drop = dropout_threshold(a.s.dropout_p) != 0;
    // The fused form exists for unpadded d = 64 and 128 (its dQ atomics of d = 256
    // would overflow the wait counter it relies on).
    constexpr bool kFused = D == DH && D <= 128;
    if (a.deterministic || !drop || !kFused) {
        launch_pre<T, DH, D, false>(a, st);
        const hipError_t e = launch_kv<T, D, DH, false>(a, st);
        if (e != hipSuccess) return e;
        return launch_bwd_dq<T, D, DH>(a, st);
    }
    if constexpr (kFused) {
        launch_pre<T, DH, D, true>(a, st);
        const hipError_t e = launch_kv<T, D, DH, true>(a, st);
        if (e != hipSuccess) return e;
        ConvertParams c{};
        c.acc = a.dq_accum;
        c.dq = a.dq;
        c.ldq = a.L.dq;
        c.cu = a.L.cu_seqlens;
        c.total = a.L.total;
        c.H = a.s.H;
        c.N = a.s.N;
        c.n8 = (size_t)a.s.B * a.s.H * a.s.N * (DH / 8);
        hipLaunchKernelGGL((dq_convert_kernel<T, D, DH>), dim3((unsigned)((c.n8 + 255) / 256)), dim3(256), 0,
                           st, c);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace
}  // namespace fa
