// Forward attention for bf16 tensors on gfx950 matrix cores.
//
// The method: "DL0056 FlashAttention" (intvml), "Mathematical Formulation" and
// points (1)-(3); emergent.sh glossary "Flash Attention", "How Flash Attention
// Works", steps 1-5. Each workgroup owns a block of query rows held in
// registers, streams key/value tiles through LDS, keeps the running row maximum
// m and the rescaled running denominator l of the page's recurrence, rescales
// its output accumulator by the same factor, and writes only O and the row
// log-sum-exp. Scores and probabilities live in registers only.
//
// gfx950 mapping
// --------------
// * One wave owns 32 query rows. It computes the transposed score tile
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = 32 keys of K, B = the
//   wave's Q rows), so a lane holds 16 keys of ONE query row and its partner
//   lane (lane ^ 32) holds the other 16: row max and row sum are in-lane
//   reductions plus one v_permlane32_swap.
// * The accumulator layout of S^T is exactly the B-operand layout of the
//   second product O^T = V^T P^T, so P (unnormalised, rounded to bf16) feeds
//   the matrix core straight from registers. V^T is read from LDS with
//   ds_read_b64_tr_b16, which transposes 4x16 blocks of V on the fly.
// * K/V tiles travel HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//   staging), double-buffered, with out-of-range rows of a ragged tail
//   returned as zeros by the buffer range check. Chunks of 16 bytes are
//   XOR-swizzled per row (chunk_swizzle) so that both the K reads (16 rows,
//   same columns) and the transposed V reads hit distinct LDS banks.
// * The scale is applied in fp32 after the product and folded with log2(e)
//   into the exp2 argument: p = exp2(s * c - m2) with c = scale * log2(e) and
//   m2 the running maximum of s * c. The division by l (and by 1 - p_drop)
//   is deferred to the epilogue.
// * Causal: key tiles past the workgroup's last query row are never loaded;
//   a wave skips tiles that are fully masked for its own 32 rows; only tiles
//   that cross the diagonal (or the ragged end) evaluate the element mask.
//   Workgroups are ordered longest-first, and when B*H is a multiple of 8 the
//   query blocks of one head are dispatched to one XCD (workgroup IDs are
//   dealt round-robin over the 8 XCDs) so the head's K/V stays in that L2.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

// Slack, in log2 units, by which a tile maximum may exceed the reference
// maximum before the accumulators are rescaled. Zero keeps the reference equal
// to the true running maximum (the recurrence as printed), so the key that
// attains a row's maximum gets P~ = 1 exactly, with no bf16 rounding on the
// dominant term of a peaked row; a positive slack lets that term round.
constexpr float RESCALE_SLACK = 0.0f;

struct FwdParamsB {
    const __bf16* q;
    const __bf16* k;
    const __bf16* v;
    __bf16* o;
    float* lse;
    int H, N, nqb, heads;
    float sl2;        // scale * log2(e)
    float inv_keep;   // 1 / (1 - p)
    uint32_t thr;
    PhiloxKey key;
};

// LDS operand reads kept in flight ahead of the matrix-core product that uses them.
#ifndef FA_FWD_PREFETCH
#define FA_FWD_PREFETCH 2
#endif
constexpr int kPrefetch = FA_FWD_PREFETCH;

template <int D, int BC, int NW, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void fwd_bf16_kernel(FwdParamsB p) {
    constexpr int BR = NW * 32;            // query rows per workgroup
    constexpr int CH = D / 8;              // 16-byte chunks per row
    constexpr int KB = BC / 32;            // 32-key blocks per tile
    constexpr int NC = BC / 16;            // 16-key chunks per tile (PV k-steps)
    constexpr int DB = D / 32;             // 32-wide d blocks of O^T
    constexpr int TILE_BYTES = BC * D * 2;
    constexpr int LOADS = BC * CH / (64 * NW);   // 16-byte loads per lane per tensor per tile
    static_assert(LOADS * 64 * NW == BC * CH, "tile must split evenly over the waves");
    constexpr int S_MFMA = KB * (D / 16);  // products of one score tile
    constexpr int PV_MFMA = NC * DB;       // products of one PV update
    constexpr int E = KB * 16;             // score elements per lane
    // Slots of the interleaved score/softmax sequence: the row maximum is
    // spread over the first MAX_SLOTS products, one slot exchanges it across
    // the half-waves, and the exponentials fill the remaining EXP_SLOTS.
    constexpr int MAX_SLOTS = S_MFMA >= 8 ? S_MFMA / 4 : 1;
    constexpr int EXP_SLOTS = S_MFMA - MAX_SLOTS - 1;
    static_assert(EXP_SLOTS >= 1, "too few products to interleave the softmax");

    __shared__ __attribute__((aligned(1024))) char kbuf[2 * TILE_BYTES];   // two K tiles
    __shared__ __attribute__((aligned(1024))) char vbuf[2 * TILE_BYTES];   // two V tiles

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // ---- workgroup -> (head, query block)
    int bh, qb;
    const int bid = blockIdx.x;
    if ((p.heads & 7) == 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        bh = (slot / p.nqb) * 8 + xcd;
        qb = slot % p.nqb;
    } else {
        bh = bid % p.heads;
        qb = bid / p.heads;
    }
    if (CAUSAL) qb = p.nqb - 1 - qb;
    const int b = bh / p.H, h = bh - b * p.H;
    const int N = p.N;
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const auto rs_q = make_rsrc(p.q + head, head_bytes);
    const auto rs_k = make_rsrc(p.k + head, head_bytes);
    const auto rs_v = make_rsrc(p.v + head, head_bytes);

    const int q0 = qb * BR;
    const int qw = q0 + wave * 32;         // first query row of this wave
    const int my_q = qw + l32;             // this lane's query row

    // ---- Q rows as B operands: chunk c holds d = 16c + 8*hi .. +7 of row my_q
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        const u32x4 raw = buffer_load16(rs_q, (uint32_t)(my_q * D + 16 * c + 8 * hi) * 2);
        qreg[c] = __builtin_bit_cast(bf16x8, raw);
    }

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
    float m2 = -INFINITY;   // reference maximum of s * c for row my_q (same in both half-waves)
    float lsum = 0.0f;      // this lane's share of the running denominator

    const int last_q = min(N, q0 + BR) - 1;
    const int ntiles = CAUSAL ? (last_q / BC + 1) : (N + BC - 1) / BC;
    // Tiles this wave needs: causal rows stop at their diagonal; rows past N need none.
    const int ntiles_w = qw >= N ? 0 : CAUSAL ? min(ntiles, min(qw + 31, N - 1) / BC + 1) : ntiles;

    auto kl = [&](int i) { return (FA_LDS char*)kbuf + i * TILE_BYTES; };
    auto vl = [&](int i) { return (FA_LDS char*)vbuf + i * TILE_BYTES; };

    // HBM -> LDS copy of rows [t*BC, t*BC + BC) of K or V, chunks swizzled per row.
    auto issue = [&](const __amdgpu_buffer_rsrc_t& rs, int t, FA_LDS char* dst) {
        const int k0 = t * BC;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int blk = i * NW + wave;             // 1 KB block of the tile written by this wave
            const int pos = blk * 64 + lane;           // 16-byte slot in the tile
            const int row = pos / CH, sw = pos % CH;
            const uint32_t off = ((uint32_t)(k0 + row) * D + (uint32_t)((sw ^ chunk_swizzle<CH>(row)) * 8)) * 2;
            buffer_to_lds16(rs, (FA_LDS void*)(dst + blk * 1024), off);
        }
    };

    // S^T = K Q^T for KB blocks of 32 keys. Element (kb, r) of a lane is key
    // row 32kb + 8(r/4) + 4hi + r%4 of the tile against query row my_q.
    auto score_tile = [&](f32x16 (&s)[KB], const FA_LDS char* kt) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const bf16x8 a = *(const FA_LDS bf16x8*)(kt + tile_offset<CH>(kb * 32 + l32, 16 * c + 8 * hi));
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[c], s[kb], 0, 0, 0);
            }
    };

    // K operand of score product i (i = c * KB + kb): key row 32kb + l32, d = 16c + 8hi .. +7.
    auto k_operand = [&](const FA_LDS char* kt, int i) {
        const int kb = i % KB, c = i / KB;
        return *(const FA_LDS bf16x8*)(kt + tile_offset<CH>(kb * 32 + l32, 16 * c + 8 * hi));
    };

    // V^T operand of PV product j (j = c * DB + db): lane holds d = 32db + l32
    // and keys 16c + 4hi + {0..3} (first read) and 16c + 8 + 4hi + {0..3}
    // (second read). Within a 16-lane group, lane s of the transposed read
    // addresses key (s / 4) and columns 4 (s % 4) .. +3 of its 4x16 block.
    const int grp = lane >> 4, sl = lane & 15;
    const int vd = 16 * (grp & 1) + 4 * (sl & 3);      // column inside the 32-wide d block
    auto v_operand = [&](const FA_LDS char* vt, int j) {
        const int c = j / DB, db = j % DB;
        bf16x8 a;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int key = 16 * c + 8 * half + 4 * (grp >> 1) + (sl >> 2);
            const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (FA_LDS s16x4*)(vt + tile_offset<CH>(key, 32 * db + vd)));
            const bf16x4 xb = __builtin_bit_cast(bf16x4, x);
#pragma unroll
            for (int i = 0; i < 4; ++i) a[4 * half + i] = xb[i];
        }
        return a;
    };

    // Next score tile on the matrix cores interleaved, product by product,
    // with this tile's softmax on the vector ALUs (no dropout). The order is
    // fixed with scheduling fences; K operands are read kPrefetch products
    // ahead so the LDS latency stays hidden.
    auto score_and_softmax = [&](f32x16 (&sn)[KB], const FA_LDS char* kt, f32x16 (&s)[KB],
                                 bf16x8 (&pb)[NC], float& m_new, float& tsum) {
        bf16x8 kop[kPrefetch];
#pragma unroll
        for (int j = 0; j < kPrefetch; ++j) kop[j] = k_operand(kt, j);
        float mx = -INFINITY, neg = 0.0f;
        tsum = 0.0f;
#pragma unroll
        for (int i = 0; i < S_MFMA; ++i) {
            const int kb = i % KB, c = i / KB;
            if (c == 0)
                sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[i % kPrefetch], qreg[0], f32x16{}, 0, 0, 0);
            else
                sn[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[i % kPrefetch], qreg[c], sn[kb], 0, 0, 0);
            if (i + kPrefetch < S_MFMA) kop[i % kPrefetch] = k_operand(kt, i + kPrefetch);
            if (i < MAX_SLOTS) {
#pragma unroll
                for (int e = i * E / MAX_SLOTS; e < (i + 1) * E / MAX_SLOTS; ++e)
                    mx = fmaxf(mx, s[e / 16][e % 16]);
            } else if (i == MAX_SLOTS) {
                mx = max_with_partner32(mx) * p.sl2;
                m_new = fmaxf(m2, mx);
                neg = -m_new;
            } else {
                const int j = i - MAX_SLOTS - 1;
                const int e0 = ((j * E) / EXP_SLOTS) & ~1, e1 = (((j + 1) * E) / EXP_SLOTS) & ~1;
#pragma unroll
                for (int e = e0; e < e1; e += 2) {
                    const float x0 = fast_exp2(fmaf(s[e / 16][e % 16], p.sl2, neg));
                    const float x1 = fast_exp2(fmaf(s[e / 16][e % 16 + 1], p.sl2, neg));
                    tsum += x0;
                    tsum += x1;
                    const int pc = (e / 16) * 2 + (e % 16) / 8, pi = e % 8;
                    pb[pc][pi] = (__bf16)x0;
                    pb[pc][pi + 1] = (__bf16)x1;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Online softmax of one score tile (log2 domain): row maximum against the
    // reference m2, P~ = exp2(s*c - m_new) with its row sum, dropout, and the
    // bf16 B operands of the PV product. O~ and l are rescaled afterwards.
    auto softmax = [&](f32x16 (&s)[KB], bf16x8 (&pb)[NC], float& m_new, float& tsum, int k0) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = max_with_partner32(mx) * p.sl2;
        m_new = fmaxf(m2, mx);
        // dropout keep bits, bit r of word kb for element (kb, r)
        uint32_t keep[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            keep[kb] = 0xffffu;
            if (DROPOUT) {
                uint32_t bits = 0;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    const uint32_t w = philox_word0((uint32_t)b, (uint32_t)h, (uint32_t)my_q,
                                                    (uint32_t)key, p.key);
                    bits |= (uint32_t)(w >= p.thr) << r;
                }
                keep[kb] = bits;
            }
        }
        const float neg = -m_new;
        tsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = fast_exp2(fmaf(s[kb][r], p.sl2, neg));
                tsum += e;
                s[kb][r] = DROPOUT ? ((keep[kb] >> r) & 1u ? e : 0.0f) : e;
            }
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) pb[c][i] = (__bf16)s[c >> 1][8 * (c & 1) + i];
    };

    // One key/value tile: wait for K_{t+1} and V_t, refill the buffers freed
    // by the previous step (V_{t+1}, K_{t+2}), then overlap the next score
    // tile on the matrix cores with this tile's softmax on the vector ALUs,
    // and finish with O~ += V_t^T P_t^T.
    auto step = [&](f32x16 (&sc)[KB], f32x16 (&sn)[KB], int t) {
        wait_vmem();
        __syncthreads();
        if (t + 1 < ntiles) issue(rs_v, t + 1, vl((t + 1) & 1));
        if (t + 2 < ntiles) issue(rs_k, t + 2, kl(t & 1));
        if (t >= ntiles_w) return;

        const int k0 = t * BC;
        // mask: only tiles that cross the diagonal or the ragged end
        if ((CAUSAL && k0 + BC - 1 > qw) || (k0 + BC > N)) {
            const int lim = CAUSAL ? min(my_q, N - 1) : N - 1;   // last visible key
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    sc[kb][r] = key > lim ? -INFINITY : sc[kb][r];
                }
        }

        bf16x8 pb[NC];
        float m_new, tsum;
        if (t + 1 < ntiles_w) {
            if (DROPOUT) {
                // the dropout generator's long integer chains dominate; the
                // default schedule overlaps them with the products
                score_tile(sn, kl((t + 1) & 1));
                softmax(sc, pb, m_new, tsum, k0);
            } else {
                score_and_softmax(sn, kl((t + 1) & 1), sc, pb, m_new, tsum);
            }
        } else {
            softmax(sc, pb, m_new, tsum, k0);
        }

        // Rescale only when some row of the wave raised its maximum (by more
        // than RESCALE_SLACK); otherwise every factor would be exactly 1.
        if (__builtin_amdgcn_ballot_w64(m_new > m2 + RESCALE_SLACK)) {
            const float alpha = fast_exp2(m2 - m_new);   // exp2(-inf) = 0 on the first tile
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        m2 = m_new;
        lsum += tsum;

        // O~^T += V^T P^T, V^T operands read kPrefetch products ahead
        const FA_LDS char* vt = vl(t & 1);
        bf16x8 vop[kPrefetch];
#pragma unroll
        for (int j = 0; j < kPrefetch; ++j) vop[j] = v_operand(vt, j);
#pragma unroll
        for (int j = 0; j < PV_MFMA; ++j) {
            const int c = j / DB, db = j % DB;
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[j % kPrefetch], pb[c], oacc[db], 0, 0, 0);
            if (j + kPrefetch < PV_MFMA) vop[j % kPrefetch] = v_operand(vt, j + kPrefetch);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- prologue: K_0, V_0, K_1 resident, first score tile
    issue(rs_k, 0, kl(0));
    issue(rs_v, 0, vl(0));
    if (ntiles > 1) issue(rs_k, 1, kl(1));
    wait_vmem();
    __syncthreads();
    f32x16 sa[KB], sb[KB];
    if (ntiles_w > 0) score_tile(sa, kl(0));

    // Two steps per trip so the current and next score tiles swap roles
    // without register copies.
    for (int t = 0; t < ntiles; t += 2) {
        step(sa, sb, t);
        if (t + 1 < ntiles) step(sb, sa, t + 1);
    }

    // ---- epilogue: O = O~ / (l (1 - p)), LSE = (m2 + log2 l) ln 2
    const float ltot = add_with_partner32(lsum);
    const float inv = p.inv_keep / ltot;
    if (my_q < N) {
        __bf16* orow = p.o + head + (size_t)my_q * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (__bf16)(oacc[db][4 * g + i] * inv);
                *(bf16x4*)(orow + 32 * db + 8 * g + 4 * hi) = w;
            }
        if (hi == 0) p.lse[(size_t)bh * N + my_q] = (m2 + fast_log2(ltot)) * kLn2;
    }
}

// Two-group ("ping-pong") form of the same forward pass. Eight waves share
// each K/V tile: waves 0-3 (group A) own query rows [q0, q0+128) and waves
// 4-7 (group B) rows [q0+128, q0+256); wave w and wave w+4 share one SIMD.
// A group alternates a matrix-core phase M(t) = {O~ += V_{t-1}^T P_{t-1}^T,
// S_t = K_t Q^T} with a vector-ALU phase V(t) = softmax of S_t. Group B runs
// one phase behind group A and a workgroup barrier closes every phase, so on
// each SIMD one wave feeds the matrix core while the other runs its softmax.
//
//   interval:   0      1      2      3      4    ...
//   group A:   M(0)   V(0)   M(1)   V(1)   M(2)
//   group B:    -     M(0)   V(0)   M(1)   V(1)
//
// K_t and V_{t-1} are read in intervals 2t and 2t+1. K_{t+1} and V_t are
// fetched at the start of interval 2t into the buffers last read in interval
// 2t-1, and waited for at the end of interval 2t+1.
template <int D, int BC, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_pingpong_kernel(FwdParamsB p) {
    constexpr int NW = 8, BR = 256;
    constexpr int CH = D / 8, KB = BC / 32, NC = BC / 16, DB = D / 32;
    constexpr int TILE_BYTES = BC * D * 2;
    constexpr int LOADS = BC * CH / (64 * NW);
    static_assert(LOADS * 64 * NW == BC * CH, "tile must split evenly over the waves");
    constexpr int S_MFMA = KB * (D / 16), PV_MFMA = NC * DB;

    __shared__ __attribute__((aligned(1024))) char kbuf[2 * TILE_BYTES];
    __shared__ __attribute__((aligned(1024))) char vbuf[2 * TILE_BYTES];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const bool group_b = wave >= 4;

    int bh, qb;
    const int bid = blockIdx.x;
    if ((p.heads & 7) == 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        bh = (slot / p.nqb) * 8 + xcd;
        qb = slot % p.nqb;
    } else {
        bh = bid % p.heads;
        qb = bid / p.heads;
    }
    if (CAUSAL) qb = p.nqb - 1 - qb;
    const int b = bh / p.H, h = bh - b * p.H;
    const int N = p.N;
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const auto rs_q = make_rsrc(p.q + head, head_bytes);
    const auto rs_k = make_rsrc(p.k + head, head_bytes);
    const auto rs_v = make_rsrc(p.v + head, head_bytes);

    const int q0 = qb * BR;
    const int qw = q0 + wave * 32;
    const int my_q = qw + l32;

    bf16x8 qreg[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
        qreg[c] = __builtin_bit_cast(bf16x8, buffer_load16(rs_q, (uint32_t)(my_q * D + 16 * c + 8 * hi) * 2));

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
    float m2 = -INFINITY, lsum = 0.0f;

    const int last_q = min(N, q0 + BR) - 1;
    const int ntiles = CAUSAL ? (last_q / BC + 1) : (N + BC - 1) / BC;
    const int ntiles_w = qw >= N ? 0 : CAUSAL ? min(ntiles, min(qw + 31, N - 1) / BC + 1) : ntiles;

    auto kl = [&](int i) { return (FA_LDS char*)kbuf + i * TILE_BYTES; };
    auto vl = [&](int i) { return (FA_LDS char*)vbuf + i * TILE_BYTES; };
    auto issue = [&](const __amdgpu_buffer_rsrc_t& rs, int t, FA_LDS char* dst) {
        const int k0 = t * BC;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int blk = i * NW + wave, pos = blk * 64 + lane;
            const int row = pos / CH, sw = pos % CH;
            const uint32_t off = ((uint32_t)(k0 + row) * D + (uint32_t)((sw ^ chunk_swizzle<CH>(row)) * 8)) * 2;
            buffer_to_lds16(rs, (FA_LDS void*)(dst + blk * 1024), off);
        }
    };
    // Per-lane LDS byte offsets of the operand reads. A K read (product i =
    // c*KB + kb) is koff[c] + kb*32 rows; a V^T read (product j = c*DB + db,
    // half) is voff[db][half] + 16c rows: the swizzle depends only on the low
    // row bits, so the row-block terms are plain immediate offsets.
    constexpr int ROW_BYTES = CH * 16;
    int koff[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) koff[c] = tile_offset<CH>(l32, 16 * c + 8 * hi);
    const int grp = lane >> 4, sl = lane & 15;
    const int vd = 16 * (grp & 1) + 4 * (sl & 3);
    int voff[DB][2];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half)
            voff[db][half] = tile_offset<CH>(8 * half + 4 * (grp >> 1) + (sl >> 2), 32 * db + vd);
    auto k_operand = [&](const FA_LDS char* kt, int i) {
        const int kb = i % KB, c = i / KB;
        return *(const FA_LDS bf16x8*)(kt + koff[c] + kb * 32 * ROW_BYTES);
    };
    auto v_operand = [&](const FA_LDS char* vt, int j) {
        const int c = j / DB, db = j % DB;
        bf16x8 a;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (FA_LDS s16x4*)(vt + voff[db][half] + 16 * c * ROW_BYTES));
            const bf16x4 xb = __builtin_bit_cast(bf16x4, x);
#pragma unroll
            for (int i = 0; i < 4; ++i) a[4 * half + i] = xb[i];
        }
        return a;
    };

    f32x16 s[KB];
    bf16x8 pb[NC];

    // M(t): O~ += V_{t-1}^T P_{t-1}^T and S_t = K_t Q^T, operands read kPrefetch ahead.
    auto matrix_phase = [&](int t) {
        const bool do_pv = t >= 1 && t - 1 < ntiles_w;
        const bool do_s = t < ntiles_w;
        if (do_pv) {
            const FA_LDS char* vt = vl((t - 1) & 1);
            bf16x8 vop[kPrefetch];
#pragma unroll
            for (int j = 0; j < kPrefetch; ++j) vop[j] = v_operand(vt, j);
#pragma unroll
            for (int j = 0; j < PV_MFMA; ++j) {
                oacc[j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[j % kPrefetch], pb[j / DB], oacc[j % DB], 0, 0, 0);
                if (j + kPrefetch < PV_MFMA) vop[j % kPrefetch] = v_operand(vt, j + kPrefetch);
            }
        }
        if (do_s) {
            const FA_LDS char* kt = kl(t & 1);
            bf16x8 kop[kPrefetch];
#pragma unroll
            for (int j = 0; j < kPrefetch; ++j) kop[j] = k_operand(kt, j);
#pragma unroll
            for (int i = 0; i < S_MFMA; ++i) {
                const int kb = i % KB, c = i / KB;
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[i % kPrefetch], qreg[c],
                                                                c == 0 ? f32x16{} : s[kb], 0, 0, 0);
                if (i + kPrefetch < S_MFMA) kop[i % kPrefetch] = k_operand(kt, i + kPrefetch);
            }
        }
    };

    // V(t): mask, online softmax of S_t (log2 domain), dropout, P_t as bf16
    // B operands, and the rescale of O~ and l when a row maximum grew.
    auto vector_phase = [&](int t) {
        if (t >= ntiles_w) return;
        const int k0 = t * BC;
        if ((CAUSAL && k0 + BC - 1 > qw) || (k0 + BC > N)) {
            const int lim = CAUSAL ? min(my_q, N - 1) : N - 1;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    s[kb][r] = key > lim ? -INFINITY : s[kb][r];
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = max_with_partner32(mx) * p.sl2;
        const float m_new = fmaxf(m2, mx);
        uint32_t keep[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            keep[kb] = 0xffffu;
            if (DROPOUT) {
                uint32_t bits = 0;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    const uint32_t w = philox_word0((uint32_t)b, (uint32_t)h, (uint32_t)my_q,
                                                    (uint32_t)key, p.key);
                    bits |= (uint32_t)(w >= p.thr) << r;
                }
                keep[kb] = bits;
            }
        }
        const float neg = -m_new;
        float tsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float x0 = fast_exp2(fmaf(s[kb][r], p.sl2, neg));
                const float x1 = fast_exp2(fmaf(s[kb][r + 1], p.sl2, neg));
                tsum += x0;
                tsum += x1;
                const int pc = kb * 2 + r / 8, pi = r % 8;
                pb[pc][pi] = (__bf16)(DROPOUT ? ((keep[kb] >> r) & 1u ? x0 : 0.0f) : x0);
                pb[pc][pi + 1] = (__bf16)(DROPOUT ? ((keep[kb] >> (r + 1)) & 1u ? x1 : 0.0f) : x1);
            }
        if (__builtin_amdgcn_ballot_w64(m_new > m2 + RESCALE_SLACK)) {
            const float alpha = fast_exp2(m2 - m_new);
            lsum *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        m2 = m_new;
        lsum += tsum;
    };

    // prologue: K_0 resident before interval 0
    issue(rs_k, 0, kl(0));
    wait_vmem();
    __syncthreads();

    // Interval 2t starts by fetching K_{t+1} and V_t; interval 2t+1 ends by
    // waiting for them. Each group runs its own loop with the same barriers.
    auto fetch = [&](int t) {
        if (t + 1 < ntiles) issue(rs_k, t + 1, kl((t + 1) & 1));
        if (t < ntiles) issue(rs_v, t, vl(t & 1));
    };
    if (!group_b) {
        for (int t = 0; t <= ntiles; ++t) {
            fetch(t);
            matrix_phase(t);
            __syncthreads();
            vector_phase(t);
            wait_vmem();
            __syncthreads();
        }
    } else {
        for (int t = 0; t <= ntiles; ++t) {
            fetch(t);
            if (t >= 1) vector_phase(t - 1);
            __syncthreads();
            matrix_phase(t);
            wait_vmem();
            __syncthreads();
        }
    }

    const float ltot = add_with_partner32(lsum);
    const float inv = p.inv_keep / ltot;
    if (my_q < N) {
        __bf16* orow = p.o + head + (size_t)my_q * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (__bf16)(oacc[db][4 * g + i] * inv);
                *(bf16x4*)(orow + 32 * db + 8 * g + 4 * hi) = w;
            }
        if (hi == 0) p.lse[(size_t)bh * N + my_q] = (m2 + fast_log2(ltot)) * kLn2;
    }
}

// Keys per K/V tile and waves (32 query rows each) per workgroup.
#ifndef FA_FWD_BC
#define FA_FWD_BC 64
#endif
#ifndef FA_FWD_NW
#define FA_FWD_NW 4
#endif

// The two-group form is kept for measurement; on gfx950 the matrix cores and
// the vector ALUs of a SIMD do not run concurrently (measured: their cycle
// counts add), so it does not beat the single-group form.
#ifndef FA_FWD_PINGPONG
#define FA_FWD_PINGPONG 0
#endif

template <int D, bool CAUSAL, bool DROPOUT>
hipError_t launch_cfg(const FwdArgs& a, hipStream_t st) {
    constexpr bool PP = FA_FWD_PINGPONG;
    constexpr int BC = FA_FWD_BC, NW = PP ? 8 : FA_FWD_NW, BR = NW * 32;
    FwdParamsB p{};
    p.q = (const __bf16*)a.q;
    p.k = (const __bf16*)a.k;
    p.v = (const __bf16*)a.v;
    p.o = (__bf16*)a.o;
    p.lse = a.lse;
    p.H = a.s.H;
    p.N = a.s.N;
    p.nqb = (a.s.N + BR - 1) / BR;
    p.heads = a.s.B * a.s.H;
    p.sl2 = a.s.scale * kLog2e;
    p.inv_keep = 1.0f / (1.0f - a.s.dropout_p);
    p.thr = dropout_threshold(a.s.dropout_p);
    p.key = PhiloxKey{(uint32_t)(a.s.seed & 0xffffffffu), (uint32_t)(a.s.seed >> 32)};
    if (PP)
        hipLaunchKernelGGL((fwd_pingpong_kernel<D, BC, CAUSAL, DROPOUT>), dim3(p.heads * p.nqb),
                           dim3(NW * 64), 0, st, p);
    else
        hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, NW, CAUSAL, DROPOUT>), dim3(p.heads * p.nqb),
                           dim3(NW * 64), 0, st, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t st) {
    const bool drop = dropout_threshold(a.s.dropout_p) != 0;
    if (a.s.causal) return drop ? launch_cfg<D, true, true>(a, st) : launch_cfg<D, true, false>(a, st);
    return drop ? launch_cfg<D, false, true>(a, st) : launch_cfg<D, false, false>(a, st);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t st) {
    return a.s.d == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace fa
