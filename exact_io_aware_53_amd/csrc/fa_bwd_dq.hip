// dQ of the backward pass as a pass of its own, without atomics: the
// deterministic variant (no fp32 accumulator in HBM, dQ written once).
//
// Same gradient as the fused backward ("DL0056 FlashAttention", point (3);
// inferensys glossary "FlashAttention", paragraph on recomputation): for each
// query block, over the key tiles it sees,
//
//   P_ij  = exp2(S_ij * scale * log2(e) - LSE_i * log2(e))      recomputed
//   dP_ij = <dO_i, V_j> Z'_ij                                    Z' = Z / (1 - p)
//   dS_ij = P_ij (dP_ij - D_i)
//   dQ_i  = scale * sum_j dS_ij K_j
//
// where the dropout mask Z is regenerated from the same Philox counters. The
// key/value side (dK, dV) comes from the fused kernel run without its dQ part.
//
// gfx950 mapping: the forward's shape. One wave owns 32 query rows; Q and dO
// rows sit in registers as the B operands of S^T = K Q^T and dP^T = V dO^T,
// so a lane holds one query row and its LSE and D are per-lane constants. K
// and V tiles stream through double-buffered LDS (16-byte chunks XOR-swizzled
// per row); K is read both as rows (for S^T) and transposed with
// ds_read_b64_tr_b16 (the A operand of dQ^T = K^T dS^T); dS^T, rounded to
// bf16, is the B operand straight from registers. Causal query blocks are
// paired long-with-short per workgroup, as in the forward.
#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

struct DqParams {
    const __bf16* q;
    const __bf16* k;
    const __bf16* v;
    const __bf16* dout;
    const float* lse2;     // LSE * log2(e), [B,H,N]
    const float* dsum;     // D_i, [B,H,N]
    __bf16* dq;
    int H, N, nqb, heads;
    float scale, sl2, inv_keep;
    uint32_t thr;
    PhiloxKey key;
};

// HBM -> LDS copy of a swizzled [BC x D] tile: 1 KB blocks shared by NW waves,
// per-lane source offsets computed once; a tile adds t * BC rows.
template <int D, int BC, int NW>
struct SwizzledCopy {
    static constexpr int CH = D / 8, BLKS = BC * CH / 64, PER = (BLKS + NW - 1) / NW;
    static_assert(BLKS * 64 == BC * CH, "a tile is whole 1 KB copy blocks");
    uint32_t off[PER];

    __device__ __forceinline__ SwizzledCopy(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int pos = (i * NW + wave) * 64 + lane;
            const int row = pos / CH, sw = pos % CH;
            off[i] = (uint32_t)(row * D + ((sw ^ chunk_swizzle<CH>(row)) << 3)) * 2;
        }
    }
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, FA_LDS char* base, int t, int wave) const {
        const uint32_t toff = __builtin_amdgcn_readfirstlane((uint32_t)t * (BC * D * 2));
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int blk = i * NW + wave;
            if (blk < BLKS) buffer_to_lds16(rs, (FA_LDS void*)(base + blk * 1024), off[i] + toff);
        }
    }
};

template <int D, int BC, int NW, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(DqParams p) {
    constexpr int BR = NW * 32;
    constexpr int CH = D / 8, ROW = D * 2;
    constexpr int KB = BC / 32, NC = BC / 16, DB = D / 32, NCD = D / 16;
    constexpr int TILE = BC * D * 2;

    __shared__ __attribute__((aligned(1024))) char kbuf[2 * TILE];
    __shared__ __attribute__((aligned(1024))) char vbuf[2 * TILE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hi = lane >> 5;

    // workgroup -> (head, query blocks); causal: blocks nqb-1-k and k
    const int nslot = CAUSAL ? (p.nqb + 1) / 2 : p.nqb;
    int bh, slot;
    if ((p.heads & 7) == 0) {
        const int xcd = blockIdx.x & 7, s = blockIdx.x >> 3;
        bh = (s / nslot) * 8 + xcd;
        slot = s % nslot;
    } else {
        bh = blockIdx.x % p.heads;
        slot = blockIdx.x / p.heads;
    }
    const int b = bh / p.H, h = bh - b * p.H;
    const int N = p.N;
    const size_t head = (size_t)bh * N * D;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const auto rs_q = make_rsrc(p.q + head, head_bytes);
    const auto rs_k = make_rsrc(p.k + head, head_bytes);
    const auto rs_v = make_rsrc(p.v + head, head_bytes);
    const auto rs_do = make_rsrc(p.dout + head, head_bytes);
    const auto rs_l = make_rsrc(p.lse2 + (size_t)bh * N, (uint32_t)N * 4);
    const auto rs_d = make_rsrc(p.dsum + (size_t)bh * N, (uint32_t)N * 4);

    const SwizzledCopy<D, BC, NW> copy(wave, lane);
    // Row operand (K for S^T, V for dP^T): key row 32kb + l32, d = 16c + 8hi .. +7.
    int roff[NCD];
#pragma unroll
    for (int c = 0; c < NCD; ++c) roff[c] = tile_offset<CH>(l32, 16 * c + 8 * hi);
    // Transposed K operand (A of dQ^T = K^T dS^T): d = 32db + column, keys
    // 16c + 4(lane/32) + {0..3} and +8; within a 16-lane group, lane s reads key
    // row s/4 and 4 columns at 4(s%4).
    int troff[DB][2];
    {
        const int g = lane >> 4, sl = lane & 15;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int half = 0; half < 2; ++half)
                troff[db][half] = tile_offset<CH>(8 * half + 4 * (g >> 1) + (sl >> 2), 32 * db + 16 * (g & 1) + 4 * (sl & 3));
    }

    auto run_block = [&](int qb) {
        const int q0 = qb * BR;
        const int qw = q0 + wave * 32;
        const int my_q = qw + l32;

        bf16x8 qreg[NCD], doreg[NCD];
#pragma unroll
        for (int c = 0; c < NCD; ++c) {
            const uint32_t o = (uint32_t)(my_q * D + 16 * c + 8 * hi) * 2;
            qreg[c] = __builtin_bit_cast(bf16x8, buffer_load16(rs_q, o));
            doreg[c] = __builtin_bit_cast(bf16x8, buffer_load16(rs_do, o));
        }
        const float lse2 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_l, (uint32_t)my_q * 4, 0, 0));
        const float dsum = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs_d, (uint32_t)my_q * 4, 0, 0));
        const PhiloxRow philox((uint32_t)b, (uint32_t)h, (uint32_t)my_q, p.key);

        f32x16 dqa[DB];
#pragma unroll
        for (int i = 0; i < DB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) dqa[i][r] = 0.0f;

        const int last_q = min(N, q0 + BR) - 1;
        const int T = CAUSAL ? last_q / BC + 1 : (N + BC - 1) / BC;
        const int Tw = qw >= N ? 0 : CAUSAL ? min(T, min(qw + 31, N - 1) / BC + 1) : T;

        auto issue = [&](int t, int buf) {
            copy.issue(rs_k, (FA_LDS char*)kbuf + buf * TILE, t, wave);
            copy.issue(rs_v, (FA_LDS char*)vbuf + buf * TILE, t, wave);
        };
        issue(0, 0);
        for (int t = 0; t < T; ++t) {
            const int buf = t & 1;
            wait_vmem();
            __syncthreads();
            if (t + 1 < T) issue(t + 1, buf ^ 1);
            if (t >= Tw) continue;
            const FA_LDS char* kt = (const FA_LDS char*)kbuf + buf * TILE;
            const FA_LDS char* vt = (const FA_LDS char*)vbuf + buf * TILE;
            const int k0 = t * BC;

            // S^T = K Q^T and dP^T = V dO^T; element (kb, r): key 32kb + 8(r/4) + 4hi + r%4, row my_q
            f32x16 s[KB], dp[KB];
#pragma unroll
            for (int c = 0; c < NCD; ++c)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb) {
                    const int o = roff[c] + kb * 32 * ROW;
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const FA_LDS bf16x8*)(kt + o), qreg[c],
                                                                    c == 0 ? f32x16{} : s[kb], 0, 0, 0);
                    dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const FA_LDS bf16x8*)(vt + o), doreg[c],
                                                                     c == 0 ? f32x16{} : dp[kb], 0, 0, 0);
                }
            // log2 P = s * scale * log2(e) - LSE_i * log2(e); masked elements -> -inf
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(s[kb][r], p.sl2, -lse2);
            if ((CAUSAL && k0 + BC - 1 > qw) || k0 + BC > N) {
                const int rel = (CAUSAL ? min(my_q, N - 1) : N - 1) - k0 - 4 * hi;
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        s[kb][r] = kb * 32 + 8 * (r >> 2) + (r & 3) > rel ? -INFINITY : s[kb][r];
            }
            bf16x8 dsb[NC];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    float ds[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const float pr = fast_exp2(s[kb][r + e]);
                        float z = 1.0f;
                        if (DROPOUT) {
                            const int key = k0 + kb * 32 + 8 * ((r + e) >> 2) + 4 * hi + ((r + e) & 3);
                            z = philox.word0((uint32_t)key) >= p.thr ? p.inv_keep : 0.0f;
                        }
                        ds[e] = pr * fmaf(dp[kb][r + e], z, -dsum);
                    }
                    const int pc = kb * 2 + r / 8, pi = r % 8;
                    dsb[pc][pi] = (__bf16)ds[0];
                    dsb[pc][pi + 1] = (__bf16)ds[1];
                }
            // dQ^T += K^T dS^T over the tile's 16-key chunks
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x4 x0 = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (FA_LDS s16x4*)(kt + troff[db][0] + 16 * c * ROW)));
                    const bf16x4 x1 = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (FA_LDS s16x4*)(kt + troff[db][1] + 16 * c * ROW)));
                    bf16x8 a;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a[e] = x0[e];
                        a[4 + e] = x1[e];
                    }
                    dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[c], dqa[db], 0, 0, 0);
                }
        }

        if (my_q < N) {
            __bf16* row = p.dq + head + (size_t)my_q * D;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    bf16x4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = (__bf16)(dqa[db][4 * g + i] * p.scale);
                    *(bf16x4*)(row + 32 * db + 8 * g + 4 * hi) = w;
                }
        }
    };

    if (CAUSAL) {
        const int longer = p.nqb - 1 - slot;
        run_block(longer);
        if (slot != longer) {
            __syncthreads();     // every wave is done with the buffers the next block refills
            run_block(slot);
        }
    } else {
        run_block(slot);
    }
}

template <int D, bool CAUSAL, bool DROPOUT>
hipError_t launch(const BwdArgs& a, hipStream_t st) {
    constexpr int BC = 64, NW = 4, BR = NW * 32;
    DqParams p{};
    p.q = (const __bf16*)a.q;
    p.k = (const __bf16*)a.k;
    p.v = (const __bf16*)a.v;
    p.dout = (const __bf16*)a.dout;
    p.lse2 = a.lse2;
    p.dsum = a.dsum;
    p.dq = (__bf16*)a.dq;
    p.H = a.s.H;
    p.N = a.s.N;
    p.nqb = (a.s.N + BR - 1) / BR;
    p.heads = a.s.B * a.s.H;
    p.scale = a.s.scale;
    p.sl2 = a.s.scale * kLog2e;
    p.inv_keep = 1.0f / (1.0f - a.s.dropout_p);
    p.thr = dropout_threshold(a.s.dropout_p);
    p.key = PhiloxKey{(uint32_t)(a.s.seed & 0xffffffffu), (uint32_t)(a.s.seed >> 32)};
    const int blocks = CAUSAL ? (p.nqb + 1) / 2 : p.nqb;
    hipLaunchKernelGGL((bwd_dq_kernel<D, BC, NW, CAUSAL, DROPOUT>), dim3(p.heads * blocks), dim3(NW * 64), 0, st,
                       p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_dq_bf16(const BwdArgs& a, hipStream_t st) {
    const bool drop = dropout_threshold(a.s.dropout_p) != 0;
    if (a.s.d == 64) {
        if (a.s.causal) return drop ? launch<64, true, true>(a, st) : launch<64, true, false>(a, st);
        return drop ? launch<64, false, true>(a, st) : launch<64, false, false>(a, st);
    }
    if (a.s.causal) return drop ? launch<128, true, true>(a, st) : launch<128, true, false>(a, st);
    return drop ? launch<128, false, true>(a, st) : launch<128, false, false>(a, st);
}

}  // namespace fa
