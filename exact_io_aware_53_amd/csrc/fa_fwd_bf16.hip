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
//   XOR-swizzled per row so that both the K reads (8 rows, same columns) and
//   the transposed V reads (4 rows x 32 bytes) hit distinct LDS banks.
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

// 16-byte chunk swizzles inside one row of a K or V tile.
__device__ __forceinline__ int swz_k(int row) { return row & 7; }
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 1; }

template <int D, int BC, int NW, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdParamsB p) {
    constexpr int BR = NW * 32;            // query rows per workgroup
    constexpr int CH = D / 8;              // 16-byte chunks per row
    constexpr int KB = BC / 32;            // 32-key blocks per tile
    constexpr int NC = BC / 16;            // 16-key chunks per tile (PV k-steps)
    constexpr int DB = D / 32;             // 32-wide d blocks of O^T
    constexpr int TILE_BYTES = BC * D * 2;
    constexpr int LOADS = BC * CH / (64 * NW);   // 16-byte loads per lane per tensor per tile
    static_assert(LOADS * 64 * NW == BC * CH, "tile must split evenly over the waves");

    __shared__ __attribute__((aligned(1024))) char smem[2][2][TILE_BYTES];   // [buffer][K, V]

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
    float m2 = -INFINITY;   // running max of s * c for row my_q (same in both half-waves)
    float lsum = 0.0f;      // this lane's share of the running denominator

    const int last_q = min(N, q0 + BR) - 1;
    const int ntiles = CAUSAL ? (last_q / BC + 1) : (N + BC - 1) / BC;

    auto issue_tile = [&](int t, int buf) {
        const int k0 = t * BC;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int blk = i * NW + wave;             // 1 KB block of the tile written by this wave
            const int pos = blk * 64 + lane;           // 16-byte slot in the tile
            const int row = pos / CH, sw = pos % CH;
            const uint32_t base = (uint32_t)(k0 + row) * D;
            buffer_to_lds16(rs_k, (FA_LDS void*)(&smem[buf][0][blk * 1024]),
                            (base + (uint32_t)((sw ^ swz_k(row)) * 8)) * 2);
            buffer_to_lds16(rs_v, (FA_LDS void*)(&smem[buf][1][blk * 1024]),
                            (base + (uint32_t)((sw ^ swz_v(row)) * 8)) * 2);
        }
    };

    issue_tile(0, 0);

    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        wait_vmem();
        __syncthreads();
        if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);

        const int k0 = t * BC;
        if (CAUSAL && k0 > qw + 31) continue;      // whole tile above the diagonal for this wave

        const FA_LDS char* kt = (const FA_LDS char*)smem[buf][0];
        const FA_LDS char* vt = (const FA_LDS char*)smem[buf][1];

        // ---- S^T = K Q^T for KB blocks of 32 keys
        f32x16 s[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
            const int row = kb * 32 + l32;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const int chunk = (2 * c + hi) ^ swz_k(row);
                const bf16x8 a = *(const FA_LDS bf16x8*)(kt + row * D * 2 + chunk * 16);
                s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[c], s[kb], 0, 0, 0);
            }
        }

        // ---- mask (diagonal / ragged tiles only). Element (kb, r): key row
        // 32kb + 8(r/4) + 4hi + r%4 of the tile, query row my_q.
        const bool need_mask = (CAUSAL && k0 + BC - 1 > qw) || (k0 + BC > N);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    const bool dead = (CAUSAL && key > my_q) || key >= N;
                    if (dead) s[kb][r] = -INFINITY;
                }
        }

        // ---- online softmax (log2 domain)
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        mx = max_with_partner32(mx);
        const float m_new = fmaxf(m2, mx * p.sl2);
        const float alpha = fast_exp2(m2 - m_new);   // exp2(-inf) = 0 on the first tile
        const float neg = -m_new;
        float tsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = fast_exp2(fmaf(s[kb][r], p.sl2, neg));
                s[kb][r] = e;
                tsum += e;
            }
        lsum = fmaf(lsum, alpha, tsum);
        m2 = m_new;

        if (DROPOUT) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
                    const uint32_t w = philox_word0((uint32_t)b, (uint32_t)h, (uint32_t)my_q,
                                                    (uint32_t)key, p.key);
                    if (w < p.thr) s[kb][r] = 0.0f;
                }
        }

        // ---- P^T chunks as bf16 B operands: chunk c = 16 keys, regs 8*(c%2) .. +7 of block c/2
        bf16x8 pb[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) pb[c][i] = (__bf16)s[c >> 1][8 * (c & 1) + i];

#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

        // ---- O^T += V^T P^T. A operand for (db, c): lane holds d = 32db + l32
        // and keys 16c + 4hi + {0..3} (first read) and 16c + 8 + 4hi + {0..3}
        // (second read). Within a 16-lane group, lane s of the transposed read
        // addresses key (s / 4) and columns 4 (s % 4) .. +3 of its 4x16 block.
        const int grp = lane >> 4, sl = lane & 15;
        const int vd = 16 * (grp & 1) + 4 * (sl & 3);      // column inside the 32-wide d block
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                bf16x8 a;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int key = 16 * c + 8 * half + 4 * (grp >> 1) + (sl >> 2);
                    const int d = 32 * db + vd;
                    const int chunk = (d >> 3) ^ swz_v(key);
                    const FA_LDS s16x4* src =
                        (const FA_LDS s16x4*)(vt + key * D * 2 + chunk * 16 + (d & 7) * 2);
                    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)src);
                    const bf16x4 xb = __builtin_bit_cast(bf16x4, x);
#pragma unroll
                    for (int i = 0; i < 4; ++i) a[4 * half + i] = xb[i];
                }
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c], oacc[db], 0, 0, 0);
            }
        }
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

template <int D, bool CAUSAL, bool DROPOUT>
hipError_t launch_cfg(const FwdArgs& a, hipStream_t st) {
    constexpr int BC = 64, NW = 4, BR = NW * 32;
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
