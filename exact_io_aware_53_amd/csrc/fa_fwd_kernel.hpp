// Forward attention for bf16 and fp16 tensors on gfx950 matrix cores.
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
//   S^T = K Q^T with v_mfma_f32_32x32x16_{bf16,f16} (A = 32 keys of K, B = the
//   wave's Q rows), so a lane holds 16 keys of ONE query row and its partner
//   lane (lane ^ 32) holds the other 16: row max and row sum are in-lane
//   reductions plus one v_permlane32_swap.
// * The accumulator layout of S^T is exactly the B-operand layout of the
//   second product O^T = V^T P^T, so P (unnormalised, rounded to bf16) feeds
//   the matrix core straight from registers. V^T is read from LDS with
//   ds_read_b64_tr_b16, which transposes 4x16 blocks of V on the fly.
// * K/V tiles travel HBM -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//   staging), double-buffered, with out-of-range rows of a ragged tail
//   returned as zeros by the buffer range check. LDS rows are padded (K by 16
//   bytes, V by 64) so that both the K reads (16 rows, same columns) and the
//   transposed V reads hit distinct LDS banks, and every operand read is one
//   base register plus an immediate offset.
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
// * Layouts: every tensor is addressed as a [B, H, N, d] view with its own
//   batch, head and row strides (d contiguous), so [B, N, H, d] storage and
//   views into packed projections need no copy. Variable-length batches pack
//   their sequences along the token dimension (cu_seqlens offsets); a
//   workgroup whose block lies past its sequence's end returns at once.
// * Head sizes 32, 64, 96, 128 and 256 (the last with 64-key tiles).
// * At d = 128 without dropout the 8-wave grid runs fwd_pp_kernel, in which
//   the two waves of a SIMD alternate: one issues a tile's products while the
//   other runs its softmax (same arithmetic, same bits).
#pragma once

#include "fa_device.hpp"
#include "fa_launch.hpp"
#include "fa_tiles.hpp"

namespace fa {
namespace {

// Without dropout the softmax keeps the exact running maximum: each tile's row
// maximum is found first (in-lane max3 and one v_permlane32_swap) and moves the
// reference, rescaling O~ and l, whenever it grows. The largest weight of a
// row is then exactly 1 in bf16, so the dominant term of a peaked row carries
// no rounding of its weight, and O~ is divided by the fp32 row sum l itself
// (the same l that gives the log-sum-exp). With dropout the scores cannot stay
// live for a second look without spilling (the generator needs the registers),
// so those kernels move the reference only once it is exceeded by
// DROPOUT_SLACK, and divide O~ by the sum of the same bf16-rounded weights it
// accumulated (lb), which keeps a dominant weight's rounding out of O.
constexpr float DROPOUT_SLACK = 8.0f;     // log2 units

// LDS operand reads kept in flight ahead of the matrix-core product that uses them.
// d = 128 without dropout on the 8-wave grid: the two-group kernel (0: fwd_kernel).
#ifndef FA_FWD_PP
#define FA_FWD_PP 1
#endif
#ifndef FA_FWD_PREFETCH
#define FA_FWD_PREFETCH 4
#endif
constexpr int kPrefetch = FA_FWD_PREFETCH;

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    Strides lq, lk, lv, lo, ll;
    const int* cu;    // [B + 1] token offsets of packed sequences, or null
    int total;        // rows of the packed token dimension
    int H, N, nqb, heads;
    float sl2;        // scale * log2(e)
    float inv_keep;   // 1 / (1 - p)
    uint32_t thr;
    PhiloxKey key;
};

// Workgroup -> (head, block index). When B*H is a multiple of 8 the heads are
// split over the 8 XCDs (workgroup IDs are dealt round-robin over the XCDs),
// so each head's K/V is read through one XCD's L2. An XCD takes its heads
// kHeadGroup at a time, the blocks of a group interleaved over its heads;
// `reverse` deals the blocks last-first.
#ifndef FA_HEAD_GROUP
#define FA_HEAD_GROUP 2
#endif
constexpr int kHeadGroup = FA_HEAD_GROUP;

__device__ __forceinline__ void decode_block(int bid, int heads, int nqb, bool reverse, int& bh, int& qb) {
    if ((heads & 7) == 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        const int hpx = heads >> 3;
        const int g = hpx % kHeadGroup == 0 ? kHeadGroup : 1;
        const int grp = slot / (g * nqb), in = slot - grp * (g * nqb);
        bh = (grp * g + in % g) * 8 + xcd;
        qb = in / g;
    } else {
        bh = bid % heads;
        qb = bid / heads;
    }
    if (reverse) qb = nqb - 1 - qb;
}

template <typename T, int D, int BC, int NW, int RB, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(RB == 1 && D == 64 && BC == 64 ? 4 : RB == 1 && D <= 128 ? 2 : 1)))
void fwd_kernel(FwdParams p) {
    using V8 = typename Vec<T>::x8;
    using V4 = typename Vec<T>::x4;
    using V2 = typename Vec<T>::x2;
    constexpr int WR = 32 * RB;            // query rows per wave (RB blocks of 32)
    constexpr int BR = NW * WR;            // query rows per workgroup
    constexpr int CH = D / 8;              // 16-byte chunks per row
    constexpr int ROW_BYTES = CH * 16;
    constexpr int KB = BC / 32;            // 32-key blocks per tile
    constexpr int NC = BC / 16;            // 16-key chunks per tile (PV k-steps)
    constexpr int DB = D / 32;             // 32-wide d blocks of O^T
    using PT = PaddedTiles<D, BC>;
    constexpr int K_TILE = PT::K_TILE, V_TILE = PT::V_TILE;
    constexpr int S_MFMA = KB * (D / 16);  // K operands of one score tile
    constexpr int PV_MFMA = NC * DB;       // V^T operands of one PV update

    __shared__ __attribute__((aligned(1024))) char kbuf[2 * K_TILE];   // two K tiles
    __shared__ __attribute__((aligned(1024))) char vbuf[2 * V_TILE];   // two V tiles

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    // ---- workgroup -> (head, query blocks). Causal: a workgroup takes the
    // query blocks nqb-1-k and k of its head, one after the other, so every
    // workgroup has the same number of key tiles (nqb + 1 when nqb is even)
    // and no long block is left to run alone at the end of the grid.
    int bh, slot;
    decode_block(blockIdx.x, p.heads, CAUSAL ? (p.nqb + 1) / 2 : p.nqb, false, bh, slot);
    bh = __builtin_amdgcn_readfirstlane(bh);
    slot = __builtin_amdgcn_readfirstlane(slot);
    const int b = bh / p.H, h = bh - b * p.H;
    // This sequence: its first token and length (the whole N without
    // cu_seqlens), clamped to the packed rows and to N.
    int start, N;
    sequence(p.cu, p.total, p.N, b, start, N);
    const int nqb = (N + BR - 1) / BR;
    if (slot >= (CAUSAL ? (nqb + 1) / 2 : nqb)) return;    // past this sequence's blocks
    const T* const qh = (const T*)p.q + p.lq.base(b, h, start);
    const T* const kh = (const T*)p.k + p.lk.base(b, h, start);
    const T* const vh = (const T*)p.v + p.lv.base(b, h, start);
    T* const oh = (T*)p.o + p.lo.base(b, h, start);
    float* const lh = p.lse + p.ll.base(b, h, start);
    // Bytes of the head's rows 0 .. N-1 (row strides >= d): every row at or past
    // N lies beyond the range and loads as zeros.
    const auto rs_q = make_rsrc(qh, (uint32_t)(((size_t)(N - 1) * p.lq.sn + D) * 2));
    const auto rs_k = make_rsrc(kh, (uint32_t)(((size_t)(N - 1) * p.lk.sn + D) * 2));
    const auto rs_v = make_rsrc(vh, (uint32_t)(((size_t)(N - 1) * p.lv.sn + D) * 2));
    const int ldq = p.lq.sn, ldo = p.lo.sn, ldl = p.ll.sn;

    const TileCopy<D, BC, PT::KCH, NW> kcopy(wave, lane, p.lk.sn);
    const TileCopy<D, BC, PT::VCH, NW> vcopy(wave, lane, p.lv.sn);
    const int kbase = k_base<D, BC>(lane), vbase = v_base<D, BC>(lane);

    auto run_block = [&](int qb) {
        const int q0 = qb * BR;
        const int qw = q0 + wave * WR;         // first query row of this wave
        // Row block rb of this wave holds query rows qw + 32rb .. +31; lane's row: qw + 32rb + l32.

        // ---- Q rows as B operands: chunk c holds d = 16c + 8*hi .. +7
        V8 qreg[RB][D / 16];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int c = 0; c < D / 16; ++c)
                qreg[rb][c] = __builtin_bit_cast(
                    V8, buffer_load16(rs_q, (uint32_t)((qw + 32 * rb + l32) * ldq + 16 * c + 8 * hi) * 2));

        f32x16 oacc[RB][DB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int i = 0; i < DB; ++i)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[rb][i][r] = 0.0f;
        float m2[RB], lsum[RB], lbf[RB];   // reference max of s*c; shares of sum P~ (fp32) and sum bf16(P~)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            m2[rb] = -INFINITY;
            lsum[rb] = 0.0f;
            lbf[rb] = 0.0f;
        }

        // Dropout generator state of each row block's row (counter b, h, row, key).
        PhiloxRow philox[RB] = {PhiloxRow((uint32_t)b, (uint32_t)h, (uint32_t)(qw + l32), p.key)};
#pragma unroll
        for (int rb = 1; rb < RB; ++rb)
            philox[rb] = PhiloxRow((uint32_t)b, (uint32_t)h, (uint32_t)(qw + 32 * rb + l32), p.key);

        const int last_q = min(N, q0 + BR) - 1;
        const int ntiles = CAUSAL ? (last_q / BC + 1) : (N + BC - 1) / BC;
        // Tiles this wave needs: causal rows stop at their diagonal; rows past N need none.
        const int ntiles_w = qw >= N ? 0 : CAUSAL ? min(ntiles, min(qw + WR - 1, N - 1) / BC + 1) : ntiles;

        // HBM -> LDS copy of K and V tile t into buffer buf.
        auto issue = [&](int t, int buf) {
            kcopy.issue(rs_k, (FA_LDS char*)kbuf + buf * K_TILE, t, wave);
            vcopy.issue(rs_v, (FA_LDS char*)vbuf + buf * V_TILE, t, wave);
        };
        issue(0, 0);

        for (int t = 0; t < ntiles; ++t) {
            const int buf = t & 1;
            wait_vmem();
            __syncthreads();
            if (t >= ntiles_w) {                       // whole tile above this wave's diagonal
                if (t + 1 < ntiles) issue(t + 1, buf ^ 1);
                continue;
            }

            const FA_LDS char* kt = (const FA_LDS char*)kbuf + buf * K_TILE;
            const FA_LDS char* vt = (const FA_LDS char*)vbuf + buf * V_TILE;
            const int k0 = t * BC;

            // ---- S^T = K Q^T. Element (kb, r) of a lane in row block rb: key row
            // 32kb + 8(r/4) + 4hi + r%4 of the tile against query row qw + 32rb + l32.
            // Each K operand read feeds the RB row blocks.
            // The scheduling fences keep kPrefetch operand reads in flight; without
            // them the compiler sinks each read to just before its product.
            f32x16 s[RB][KB];
            {
                V8 kop[kPrefetch];
#pragma unroll
                for (int j = 0; j < kPrefetch; ++j) kop[j] = k_operand<D, BC, V8>(kt, kbase, j);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < S_MFMA; ++i) {
                    const int kb = i % KB, c = i / KB;
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        s[rb][kb] = mfma32(kop[i % kPrefetch], qreg[rb][c], c == 0 ? f32x16{} : s[rb][kb]);
                    if (i + kPrefetch < S_MFMA) kop[i % kPrefetch] = k_operand<D, BC, V8>(kt, kbase, i + kPrefetch);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }

            // The next tile's copies go out after this tile's score products: the
            // issuing wave stalls on its vector-memory instructions, and here that
            // stall delays only vector work instead of the products' operand reads.
            if (t + 1 < ntiles) issue(t + 1, buf ^ 1);
            V8 pb[RB][NC];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const int row0 = qw + 32 * rb;     // first row of the block
                const int my_q = row0 + l32;
                // ---- mask: only tiles that cross the diagonal or the ragged end
                if ((CAUSAL && k0 + BC - 1 > row0) || (k0 + BC > N)) {
                    // last visible key, relative to the lane's first key of the tile;
                    // element offsets are then compile-time constants
                    const int rel = (CAUSAL ? min(my_q, N - 1) : N - 1) - k0 - 4 * hi;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            s[rb][kb][r] = kb * 32 + 8 * (r >> 2) + (r & 3) > rel ? -INFINITY : s[rb][kb][r];
                }

                // ---- online softmax (log2 domain): P~ = exp2(s c - m2) into pb,
                // adding to this lane's shares of l and lb
                const V2 ones = {(T)1.0f, (T)1.0f};
                auto weights = [&](const uint32_t* keep) {
                    const float neg = -m2[rb];
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; r += 2) {
                            const float x0 = fast_exp2(fmaf(s[rb][kb][r], p.sl2, neg));
                            const float x1 = fast_exp2(fmaf(s[rb][kb][r + 1], p.sl2, neg));
                            lsum[rb] += x0;
                            lsum[rb] += x1;
                            V2 w;
                            w[0] = (T)x0;
                            w[1] = (T)x1;
                            if constexpr (DROPOUT) lbf[rb] = dot2(w, ones, lbf[rb]);
                            if (DROPOUT) {
                                w[0] = (T)((keep[kb] >> r) & 1u ? x0 : 0.0f);
                                w[1] = (T)((keep[kb] >> (r + 1)) & 1u ? x1 : 0.0f);
                            }
                            const int pc = kb * 2 + r / 8, pi = r % 8;
                            pb[rb][pc][pi] = w[0];
                            pb[rb][pc][pi + 1] = w[1];
                        }
                };
                // move the reference to the running maximum, rescaling l, lb and O~
                auto to_max = [&](float l0, float lb0) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rb][kb][r]);
                    mx = max_with_partner32(mx) * p.sl2;
                    const float m_new = fmaxf(m2[rb], mx);
                    // exp2(-inf) = 0 when the row had no reference yet; a row with no
                    // visible key so far keeps factor 1
                    const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m2[rb] - m_new);
                    lsum[rb] = l0 * alpha;
                    lbf[rb] = lb0 * alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[rb][db][r] *= alpha;
                    m2[rb] = m_new;
                };
                if constexpr (DROPOUT) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rb][kb][r]);
                    if (__builtin_amdgcn_ballot_w64(max_with_partner32(mx) * p.sl2 > m2[rb] + DROPOUT_SLACK))
                        to_max(lsum[rb], lbf[rb]);
                    uint32_t keep[KB];
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        uint32_t bits = 0;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                            bits |= (uint32_t)(philox[rb].word0((uint32_t)key) >= p.thr) << r;
                        }
                        keep[kb] = bits;
                    }
                    weights(keep);
                } else {
                    // exact running maximum: move the reference whenever a row's maximum grows
                    float mx = -INFINITY;
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[rb][kb][r]);
                    const float mxc = max_with_partner32(mx) * p.sl2;
                    if (__builtin_amdgcn_ballot_w64(mxc > m2[rb])) {
                        const float m_new = fmaxf(m2[rb], mxc);
                        // exp2(-inf) = 0 on a row's first tile; a row with no visible key keeps 1
                        const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m2[rb] - m_new);
                        lsum[rb] *= alpha;
#pragma unroll
                        for (int db = 0; db < DB; ++db)
#pragma unroll
                            for (int r = 0; r < 16; ++r) oacc[rb][db][r] *= alpha;
                        m2[rb] = m_new;
                    }
                    weights(nullptr);
                }
            }

            // ---- O~^T += V^T P^T; each V^T operand read feeds the RB row blocks
            {
                V8 vop[kPrefetch];
#pragma unroll
                for (int j = 0; j < kPrefetch; ++j) vop[j] = v_operand<D, BC, V8>(vt, vbase, j);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < PV_MFMA; ++j) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        oacc[rb][j % DB] = mfma32(vop[j % kPrefetch], pb[rb][j / DB], oacc[rb][j % DB]);
                    if (j + kPrefetch < PV_MFMA) vop[j % kPrefetch] = v_operand<D, BC, V8>(vt, vbase, j + kPrefetch);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }

        // ---- epilogue: O = O~ / (l (1 - p)) (lb with dropout), LSE = (m2 + log2 l) ln 2
        // Where the buffers allow, the wave's rows of O go through LDS so that
        // each store writes four whole rows (a lane of the product layout holds
        // 4-element runs of one row: its stores would touch 32 rows each). The
        // K and V buffers not used by the last tile are free for every wave
        // since that tile's barrier: the first half of the waves stages in the
        // K one, the second half in the V one, 32 rows of 2d + 16 bytes each
        // (the pad keeps the row writes of the 32 lanes on distinct bank pairs).
        constexpr int SROW = D * 2 + 16, STG = 32 * SROW;
        constexpr bool STAGE = RB == 1 && D % 64 == 0 && (NW / 2) * STG <= K_TILE && (NW / 2) * STG <= V_TILE;
        if constexpr (STAGE) {
            const int fb = ntiles & 1;                 // the buffer of tile ntiles - 2
            FA_LDS char* const stg = (wave < NW / 2 ? (FA_LDS char*)kbuf + fb * K_TILE
                                                    : (FA_LDS char*)vbuf + fb * V_TILE) + (wave % (NW / 2)) * STG;
            const float ltot = add_with_partner32(lsum[0]);
            const float lbtot = DROPOUT ? add_with_partner32(lbf[0]) : ltot;
            const float inv = p.inv_keep / lbtot;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    V4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = (T)(oacc[0][db][4 * g + i] * inv);
                    *(FA_LDS V4*)(stg + l32 * SROW + (32 * db + 8 * g + 4 * hi) * 2) = w;
                }
            asm volatile("" ::: "memory");
            constexpr int RCH = D / 8;               // 16-byte chunks per row
#pragma unroll
            for (int i = 0; i < 32 * RCH / 64; ++i) {
                const int pos = i * 64 + lane, r = pos / RCH, c = pos % RCH;
                const V8 w = *(const FA_LDS V8*)(stg + r * SROW + c * 16);
                if (qw + r < N) *(V8*)(oh + (size_t)(qw + r) * ldo + c * 8) = w;
            }
            const int my_q = qw + l32;
            if (hi == 0 && my_q < N) lh[(size_t)my_q * ldl] = (m2[0] + fast_log2(ltot)) * kLn2;
        } else
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            const int my_q = qw + 32 * rb + l32;
            const float ltot = add_with_partner32(lsum[rb]);
            const float lbtot = DROPOUT ? add_with_partner32(lbf[rb]) : ltot;
            const float inv = p.inv_keep / lbtot;
            if (my_q < N) {
                T* orow = oh + (size_t)my_q * ldo;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        V4 w;
#pragma unroll
                        for (int i = 0; i < 4; ++i) w[i] = (T)(oacc[rb][db][4 * g + i] * inv);
                        *(V4*)(orow + 32 * db + 8 * g + 4 * hi) = w;
                    }
                if (hi == 0) lh[(size_t)my_q * ldl] = (m2[rb] + fast_log2(ltot)) * kLn2;
            }
        }
    };

    if (CAUSAL) {
        const int longer = nqb - 1 - slot;
        run_block(longer);
        if (slot != longer) {
            __syncthreads();     // every wave is done with the buffers the next block refills
            run_block(slot);
        }
    } else {
        run_block(slot);
    }
}

// Two-group form of the forward for d = 128 without dropout (same tiles, rows
// per wave and arithmetic as fwd_kernel, so the same bits): the waves of a
// SIMD take turns. Waves 0-3 (group 0) issue the products of their rows while
// waves 4-7 (group 1) compute the softmax of theirs, and the other way round in
// the next half step; a workgroup barrier separates the half steps. In half
// step 2k group 0 runs O~ += P(k-1) V(k-1) and S(k) = Q K(k)^T and group 1 the
// softmax of tile k-1; in half step 2k+1 group 0 runs the softmax of tile k and
// group 1 the products. One wave then owns the SIMD's matrix core for a whole
// run of 64 products, and the other wave's exponentials run beside it, where in
// fwd_kernel both waves' softmax phases overlap for most of their length.
// Tile copies go out from the group in its softmax half: K(k+1) by group 1 in
// half step 2k (needed from 2k+2), V(k) by group 0 in half step 2k+1 (needed
// from 2k+2). Each group waits for its own copies at the start of its next
// products half.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_pp_kernel(FwdParams p) {
    using V8 = typename Vec<T>::x8;
    using V4 = typename Vec<T>::x4;
    using V2 = typename Vec<T>::x2;
    constexpr int BC = 128, NW = 8, WR = 32, BR = NW * WR;
    constexpr int KB = BC / 32, NC = BC / 16, DB = D / 32;
    using PT = PaddedTiles<D, BC>;
    // K rows padded as in fwd_kernel. V rows unpadded: the 64-byte segment s of
    // tile row r sits at segment s ^ (r & 3), so the four rows of a transposed
    // read pass still fall on four distinct 64-byte bank groups, a tile is 32
    // copy blocks instead of 40, and a lane's copy offset is one register.
    constexpr int VROW = D * 2;
    constexpr int K_TILE = PT::K_TILE, V_TILE = BC * VROW;
    constexpr int S_MFMA = KB * (D / 16), PV_MFMA = NC * DB;
    static_assert(D == 128, "the swizzle assumes four 64-byte segments per row");

    __shared__ __attribute__((aligned(1024))) char kbuf[2 * K_TILE];
    __shared__ __attribute__((aligned(1024))) char vbuf[2 * V_TILE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    int bh, slot;
    decode_block(blockIdx.x, p.heads, CAUSAL ? (p.nqb + 1) / 2 : p.nqb, false, bh, slot);
    bh = __builtin_amdgcn_readfirstlane(bh);
    slot = __builtin_amdgcn_readfirstlane(slot);
    const int b = bh / p.H, h = bh - b * p.H;
    int start, N;
    sequence(p.cu, p.total, p.N, b, start, N);
    const int nqb = (N + BR - 1) / BR;
    if (slot >= (CAUSAL ? (nqb + 1) / 2 : nqb)) return;
    const T* const qh = (const T*)p.q + p.lq.base(b, h, start);
    const T* const kh = (const T*)p.k + p.lk.base(b, h, start);
    const T* const vh = (const T*)p.v + p.lv.base(b, h, start);
    T* const oh = (T*)p.o + p.lo.base(b, h, start);
    float* const lh = p.lse + p.ll.base(b, h, start);
    const auto rs_q = make_rsrc(qh, (uint32_t)(((size_t)(N - 1) * p.lq.sn + D) * 2));
    const auto rs_k = make_rsrc(kh, (uint32_t)(((size_t)(N - 1) * p.lk.sn + D) * 2));
    const auto rs_v = make_rsrc(vh, (uint32_t)(((size_t)(N - 1) * p.lv.sn + D) * 2));
    const int ldq = p.lq.sn, ldo = p.lo.sn, ldl = p.ll.sn;

    // each group's four waves share the copy blocks of the tensor it copies
    const TileCopy<D, BC, PT::KCH, 4> kcopy(wave & 3, lane, p.lk.sn);
    const int kbase = k_base<D, BC>(lane);
    // swizzled V: the lane's read base for d block 0 (d block db is at base ^
    // 64 db: the segment bits 6-7 are the only ones the swizzle touches), and
    // its source offset in a 1 KB copy block (4 rows; lane -> row lane/16,
    // chunk lane%16)
    const int vsw0 = (4 * (lane >> 5) + ((lane & 15) >> 2)) * VROW + 64 * ((lane >> 2) & 3) +
                     2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    const uint32_t vcopy_lane =
        (uint32_t)((lane >> 4) * p.lv.sn + (((lane & 15) ^ (((lane >> 4) & 3) << 2)) * 8)) * 2;
    constexpr int VBLKS = V_TILE / 1024 / 4;   // copy blocks per group-0 wave and tile

    auto run_block = [&](int qb) {
        const int q0 = qb * BR;
        const int qw = q0 + wave * WR;
        const int my_q = qw + l32;
        V8 qreg[D / 16];
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
            qreg[c] = __builtin_bit_cast(V8, buffer_load16(rs_q, (uint32_t)(my_q * ldq + 16 * c + 8 * hi) * 2));
        f32x16 oacc[DB];
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
        float m2 = -INFINITY, lsum = 0.0f;

        const int last_q = min(N, q0 + BR) - 1;
        const int ntiles = CAUSAL ? (last_q / BC + 1) : (N + BC - 1) / BC;
        const int ntiles_w = qw >= N ? 0 : CAUSAL ? min(ntiles, min(qw + WR - 1, N - 1) / BC + 1) : ntiles;

        f32x16 s[KB];
        V8 pb[NC];
        // block i of group 0's share of V tile t (rows 4 blk .. 4 blk + 3)
        auto copy_v_blk = [&](int t, int i) __attribute__((always_inline)) {
            const int blk = i * 4 + (wave & 3);
            const uint32_t base = (uint32_t)((t * BC + blk * 4) * p.lv.sn) * 2;
            buffer_to_lds16_async(rs_v, (FA_LDS void*)((FA_LDS char*)vbuf + (t & 1) * V_TILE + blk * 1024),
                                  vcopy_lane + (uint32_t)__builtin_amdgcn_readfirstlane(base));
        };
        // S^T = K Q^T over K tile t
        auto s_products = [&](int t) __attribute__((always_inline)) {
            const FA_LDS char* kt = (const FA_LDS char*)kbuf + (t & 1) * K_TILE;
            V8 kop[kPrefetch];
#pragma unroll
            for (int j = 0; j < kPrefetch; ++j) kop[j] = k_operand<D, BC, V8>(kt, kbase, j);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < S_MFMA; ++i) {
                const int kb = i % KB, c = i / KB;
                s[kb] = mfma32(kop[i % kPrefetch], qreg[c], c == 0 ? f32x16{} : s[kb]);
                if (i + kPrefetch < S_MFMA) kop[i % kPrefetch] = k_operand<D, BC, V8>(kt, kbase, i + kPrefetch);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // V^T operand j = c * DB + db (16-key chunk c, d block db) from the
        // swizzled tile, read base vb
        auto v_op = [&](const FA_LDS char* vt, int vb, int j) __attribute__((always_inline)) {
            s16x4 x[2];
#pragma unroll
            for (int half = 0; half < 2; ++half)
                x[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (FA_LDS s16x4*)(vt + (vb ^ (64 * (j % DB))) + (16 * (j / DB) + 8 * half) * VROW));
            typedef short s16x8 __attribute__((ext_vector_type(8)));
            return __builtin_bit_cast(V8, __builtin_shufflevector(x[0], x[1], 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // O~^T += V^T P^T over V tile t
        auto pv_products = [&](int t) __attribute__((always_inline)) {
            const FA_LDS char* vt = (const FA_LDS char*)vbuf + (t & 1) * V_TILE;
            // an opaque copy of the read base: its four d-block variants are then
            // formed here, not kept live across the whole loop
            int vb = vsw0;
            asm volatile("" : "+v"(vb));
            V8 vop[kPrefetch];
#pragma unroll
            for (int j = 0; j < kPrefetch; ++j) vop[j] = v_op(vt, vb, j);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < PV_MFMA; ++j) {
                oacc[j % DB] = mfma32(vop[j % kPrefetch], pb[j / DB], oacc[j % DB]);
                if (j + kPrefetch < PV_MFMA) vop[j % kPrefetch] = v_op(vt, vb, j + kPrefetch);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // mask, exact running maximum (rescaling l and O~ when it grows), and
        // P~ = exp2(s c - m2) into pb, as in fwd_kernel without dropout
        auto softmax = [&](int t) __attribute__((always_inline)) {
            const int k0 = t * BC;
            if ((CAUSAL && k0 + BC - 1 > qw) || (k0 + BC > N)) {
                const int rel = (CAUSAL ? min(my_q, N - 1) : N - 1) - k0 - 4 * hi;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        s[kb][r] = kb * 32 + 8 * (r >> 2) + (r & 3) > rel ? -INFINITY : s[kb][r];
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            const float mxc = max_with_partner32(mx) * p.sl2;
            if (__builtin_amdgcn_ballot_w64(mxc > m2)) {
                const float m_new = fmaxf(m2, mxc);
                const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m2 - m_new);
                lsum *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
                m2 = m_new;
            }
            const float neg = -m2;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float x0 = fast_exp2(fmaf(s[kb][r], p.sl2, neg));
                    const float x1 = fast_exp2(fmaf(s[kb][r + 1], p.sl2, neg));
                    lsum += x0;
                    lsum += x1;
                    const int pc = kb * 2 + r / 8, pi = r % 8;
                    pb[pc][pi] = (T)x0;
                    pb[pc][pi + 1] = (T)x1;
                }
        };
        auto copy_k = [&](int t) __attribute__((always_inline)) {
            kcopy.issue(rs_k, (FA_LDS char*)kbuf + (t & 1) * K_TILE, t, wave & 3);
        };

        // Half steps 0 .. 2 ntiles + 1; each group runs a loop of its own with
        // the same barriers.
        if (grp == 0) {
            for (int k = 0; k <= ntiles; ++k) {
                wait_vmem();                  // V(k-1), issued in half step 2k-1
                __syncthreads();              // half step 2k: products
                if (k >= 1 && k - 1 < ntiles_w) pv_products(k - 1);
                if (k < ntiles_w) s_products(k);
                __syncthreads();              // half step 2k+1: softmax, after the copies of V(k)
                if (k < ntiles) {
#pragma unroll
                    for (int i = 0; i < VBLKS; ++i) copy_v_blk(k, i);
                }
                if (k < ntiles_w) softmax(k);
            }
        } else {
            copy_k(0);
            for (int k = 0; k <= ntiles; ++k) {
                wait_vmem();                  // K(k), issued in half step 2k-2
                __syncthreads();              // half step 2k: softmax
                if (k + 1 < ntiles) copy_k(k + 1);
                if (k >= 1 && k - 1 < ntiles_w) softmax(k - 1);
                __syncthreads();              // half step 2k+1: products
                if (k >= 1 && k - 1 < ntiles_w) pv_products(k - 1);
                if (k < ntiles_w) s_products(k);
            }
        }

        // epilogue: O = O~ / l, LSE = (m2 + log2 l) ln 2
        const float ltot = add_with_partner32(lsum);
        const float inv = 1.0f / ltot;
        // The wave's 32 rows of O go through LDS so that each store writes
        // four whole rows (a lane of the product layout holds 4-element runs
        // of one row: its stores would touch 32 rows each). No K tile is
        // read any more: group g stages in the g-th half of the K buffers,
        // wave w in its own 32 rows of 272 bytes (16 bytes of pad keep the
        // row writes of the 32 lanes on distinct bank pairs).
        constexpr int SROW = D * 2 + 16;
        static_assert(8 * 32 * SROW <= 2 * K_TILE, "staging fits in the K buffers");
        FA_LDS char* const stg = (FA_LDS char*)kbuf + (grp * 4 + (wave & 3)) * (32 * SROW);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                V4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = (T)(oacc[db][4 * g + i] * inv);
                *(FA_LDS V4*)(stg + l32 * SROW + (32 * db + 8 * g + 4 * hi) * 2) = w;
            }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < 32 * D * 2 / 1024; ++i) {
            const int r = 4 * i + (lane >> 4), c = lane & 15;
            const V8 w = *(const FA_LDS V8*)(stg + r * SROW + c * 16);
            if (qw + r < N) *(V8*)(oh + (size_t)(qw + r) * ldo + c * 8) = w;
        }
        if (hi == 0 && my_q < N) lh[(size_t)my_q * ldl] = (m2 + fast_log2(ltot)) * kLn2;
    };

    if (CAUSAL) {
        const int longer = nqb - 1 - slot;
        run_block(longer);
        if (slot != longer) {
            wait_vmem();
            __syncthreads();     // every wave is done with the buffers the next block refills
            run_block(slot);
        }
    } else {
        run_block(slot);
    }
}

// Keys per K/V tile and waves (32 query rows each) per workgroup: 128-key tiles
// and 8 waves, one workgroup per CU (two waves per SIMD) sharing each K/V copy.
// d = 256 takes 64-key tiles (two 128-key K/V tiles would not fit in LDS) and
// 4 waves with up to 512 registers each: the Q rows (64 registers) and the
// output accumulator (128) leave too little of 256 for the score tile.
// At d = 64 without dropout a second kernel takes 64-key tiles: 43 KB of LDS
// and at most 128 registers per lane let two workgroups (four waves per SIMD)
// share a CU, which pays once the grid gives every CU two workgroups (measured:
// +11% non-causal at B4 H16 N2048, +4.5% causal at B1 H16 N16384) and costs
// 2-4% on a grid of one workgroup per CU, where the 128-key kernel stays.
#ifndef FA_FWD_BC
#define FA_FWD_BC 128
#endif
constexpr int kFwdOnePerCu = 256;                // MI355X's compute units
constexpr int kFwdTwoPerCu = 2 * kFwdOnePerCu;   // workgroups that fill them twice
#ifndef FA_FWD_NW
#define FA_FWD_NW 8
#endif
// 32-row query blocks per wave: each K/V operand read from LDS feeds this many products.
#ifndef FA_FWD_RB
#define FA_FWD_RB 1
#endif

// Workgroups of the forward grid with NW waves (32 * RB query rows each) per
// workgroup: one per pair of query blocks of a head when causal (a short and a
// long one), one per query block otherwise.
template <int NW>
long long fwd_workgroups(const FwdArgs& a) {
    constexpr int BR = NW * 32 * FA_FWD_RB;
    const long long nqb = (a.s.N + BR - 1) / BR;
    return (long long)a.s.B * a.s.H * (a.s.causal ? (nqb + 1) / 2 : nqb);
}

template <typename T, int D, int BC, int NW, bool CAUSAL, bool DROPOUT>
hipError_t launch_cfg(const FwdArgs& a, hipStream_t st) {
    constexpr int RB = FA_FWD_RB;
    constexpr int BR = NW * 32 * RB;
    FwdParams p{};
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.o = a.o;
    p.lse = a.lse;
    p.lq = a.L.q;
    p.lk = a.L.k;
    p.lv = a.L.v;
    p.lo = a.L.o;
    p.ll = a.L.lse;
    p.cu = a.L.cu_seqlens;
    p.total = a.L.total;
    p.H = a.s.H;
    p.N = a.s.N;
    p.nqb = (a.s.N + BR - 1) / BR;
    p.heads = a.s.B * a.s.H;
    p.sl2 = a.s.scale * kLog2e;
    p.inv_keep = 1.0f / (1.0f - a.s.dropout_p);
    p.thr = dropout_threshold(a.s.dropout_p);
    p.key = PhiloxKey{(uint32_t)(a.s.seed & 0xffffffffu), (uint32_t)(a.s.seed >> 32)};
    const int blocks = CAUSAL ? (p.nqb + 1) / 2 : p.nqb;
    if constexpr (FA_FWD_PP && D == 128 && BC == 128 && NW == 8 && RB == 1 && !DROPOUT)
        hipLaunchKernelGGL((fwd_pp_kernel<T, D, CAUSAL>), dim3(p.heads * blocks), dim3(NW * 64), 0, st, p);
    else
        hipLaunchKernelGGL((fwd_kernel<T, D, BC, NW, RB, CAUSAL, DROPOUT>), dim3(p.heads * blocks),
                           dim3(NW * 64), 0, st, p);
    return hipGetLastError();
}

template <typename T, int D, bool CAUSAL, bool DROPOUT>
hipError_t launch_tiles(const FwdArgs& a, hipStream_t st) {
    if constexpr (D == 256) {
        return launch_cfg<T, D, 64, 4, CAUSAL, DROPOUT>(a, st);
    } else {
        constexpr int NW = FA_FWD_NW;
        if constexpr (D == 64 && !DROPOUT) {
            if (fwd_workgroups<NW>(a) >= kFwdTwoPerCu) return launch_cfg<T, D, 64, NW, CAUSAL, false>(a, st);
        }
        if constexpr (NW == 8) {
            // A grid that leaves CUs idle: halving the rows per workgroup doubles
            // the workgroups. As long as they still fit one round (one per CU),
            // the chip finishes in about half the time, though a wave per SIMD
            // hides less latency than two. Where halving adds no workgroups (a
            // causal head of 129-256 rows: one pair of short blocks instead of
            // one block) it only lengthens each workgroup's walk.
            const long long w4 = fwd_workgroups<4>(a);
            if (w4 <= kFwdOnePerCu && w4 > fwd_workgroups<NW>(a))
                return launch_cfg<T, D, FA_FWD_BC, 4, CAUSAL, DROPOUT>(a, st);
        }
        return launch_cfg<T, D, FA_FWD_BC, NW, CAUSAL, DROPOUT>(a, st);
    }
}

template <typename T, int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t st) {
    const bool drop = dropout_threshold(a.s.dropout_p) != 0;
    if (a.s.causal) return drop ? launch_tiles<T, D, true, true>(a, st) : launch_tiles<T, D, true, false>(a, st);
    return drop ? launch_tiles<T, D, false, true>(a, st) : launch_tiles<T, D, false, false>(a, st);
}


}  // namespace
}  // namespace fa
