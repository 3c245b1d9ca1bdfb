// dQ of the backward pass as a pass of its own, without atomics: the
// deterministic variant (no fp32 accumulator in HBM, dQ written once).
// Element types, layouts, packed sequences and padded head sizes as in the
// key-side kernel (fa_bwd_kernels.hpp).
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
#pragma once

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

#ifndef FA_DQ_PF
#define FA_DQ_PF 2
#endif
#ifndef FA_DQ_TF
#define FA_DQ_TF 4
#endif


struct DqParams {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* lse2;     // LSE * log2(e), [B*H, N] workspace rows
    const float* dsum;     // D_i, [B*H, N] workspace rows
    void* dq;
    Strides lq, lk, lv, ldo, ldq;
    const int* cu;
    int total;
    int H, N, nqb, heads;
    float scale, sl2, inv_keep;
    uint32_t thr;
    PhiloxKey key;
};

// HBM -> LDS copy of a swizzled [BC x D] tile of a tensor with row stride ld
// whose rows hold DH <= D elements (chunks past DH load as zeros): 1 KB blocks
// shared by NW waves, per-lane source offsets computed once; a tile adds t * BC
// rows.
template <int D, int DH, int BC, int NW>
struct SwizzledCopy {
    static constexpr int CH = D / 8, BLKS = BC * CH / 64, PER = (BLKS + NW - 1) / NW;
    static_assert(BLKS * 64 == BC * CH, "a tile is whole 1 KB copy blocks");
    uint32_t off[PER];
    uint32_t step;

    __device__ __forceinline__ SwizzledCopy(int wave, int lane, int ld) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int pos = (i * NW + wave) * 64 + lane;
            const int row = pos / CH, sw = pos % CH;
            const int ch = sw ^ chunk_swizzle<CH>(row);
            off[i] = ch * 8 < DH ? (uint32_t)(row * ld + ch * 8) * 2 : 0xf0000000u;
        }
        step = (uint32_t)(BC * ld * 2);
    }
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, FA_LDS char* base, int t, int wave) const {
        const uint32_t toff = __builtin_amdgcn_readfirstlane((uint32_t)t * step);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int blk = i * NW + wave;
            // Padded chunks keep their out-of-range offset (no tile offset added,
            // so it cannot wrap back into range).
            const uint32_t o = DH == D || off[i] != 0xf0000000u ? off[i] + toff : off[i];
            // blocks i * NW + wave with i < PER - 1 are below BLKS for every wave
            if (i < PER - 1 || blk < BLKS) buffer_to_lds16_async(rs, (FA_LDS void*)(base + blk * 1024), o);
        }
    }
};

template <typename T, int D, int DH, int BC, int NW, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D <= 128 ? 2 : 1)))
void bwd_dq_kernel(DqParams p) {
    using V8 = typename Vec<T>::x8;
    using V4 = typename Vec<T>::x4;
    constexpr int BR = NW * 32;
    constexpr int CH = D / 8, ROW = D * 2;
    constexpr int KB = BC / 32, NC = BC / 16, DB = D / 32, NCD = D / 16;
    constexpr int TILE = BC * D * 2;
    // LDS operand reads in flight ahead of their products (score and dP
    // products: pairs of K and V reads; dQ products: K^T reads).
    constexpr int kPf = FA_DQ_PF, kTf = FA_DQ_TF;

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
    bh = __builtin_amdgcn_readfirstlane(bh);
    slot = __builtin_amdgcn_readfirstlane(slot);
    const int b = bh / p.H, h = bh - b * p.H;
    int start, N;
    sequence(p.cu, p.total, p.N, b, start, N);
    const int nqb = (N + BR - 1) / BR;
    if (slot >= (CAUSAL ? (nqb + 1) / 2 : nqb)) return;    // past this sequence's blocks
    const int ldq = p.lq.sn, ldo = p.ldo.sn;
    const auto rs_q = make_rsrc((const T*)p.q + p.lq.base(b, h, start), (uint32_t)(((size_t)(N - 1) * ldq + DH) * 2));
    const auto rs_k = make_rsrc((const T*)p.k + p.lk.base(b, h, start),
                                (uint32_t)(((size_t)(N - 1) * p.lk.sn + DH) * 2));
    const auto rs_v = make_rsrc((const T*)p.v + p.lv.base(b, h, start),
                                (uint32_t)(((size_t)(N - 1) * p.lv.sn + DH) * 2));
    const auto rs_do = make_rsrc((const T*)p.dout + p.ldo.base(b, h, start),
                                 (uint32_t)(((size_t)(N - 1) * ldo + DH) * 2));
    const size_t wrow = (size_t)bh * p.N;
    const auto rs_l = make_rsrc(p.lse2 + wrow, (uint32_t)N * 4);
    const auto rs_d = make_rsrc(p.dsum + wrow, (uint32_t)N * 4);

    const SwizzledCopy<D, DH, BC, NW> kcopy(wave, lane, p.lk.sn);
    const SwizzledCopy<D, DH, BC, NW> vcopy(wave, lane, p.lv.sn);
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

        V8 qreg[NCD], doreg[NCD];
#pragma unroll
        for (int c = 0; c < NCD; ++c) {
            const bool live = 16 * c + 8 * hi < DH;    // padded columns load as zeros
            qreg[c] = __builtin_bit_cast(V8, buffer_load16(rs_q, live ? (uint32_t)(my_q * ldq + 16 * c + 8 * hi) * 2
                                                                    : 0xf0000000u));
            doreg[c] = __builtin_bit_cast(V8, buffer_load16(rs_do, live ? (uint32_t)(my_q * ldo + 16 * c + 8 * hi) * 2
                                                                      : 0xf0000000u));
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
        const int nt = CAUSAL ? last_q / BC + 1 : (N + BC - 1) / BC;
        const int Tw = qw >= N ? 0 : CAUSAL ? min(nt, min(qw + 31, N - 1) / BC + 1) : nt;

        auto issue = [&](int t, int buf) {
            kcopy.issue(rs_k, (FA_LDS char*)kbuf + buf * TILE, t, wave);
            vcopy.issue(rs_v, (FA_LDS char*)vbuf + buf * TILE, t, wave);
        };
        issue(0, 0);
        for (int t = 0; t < nt; ++t) {
            const int buf = t & 1;
            wait_vmem();
            __syncthreads();
            if (t >= Tw) {
                if (t + 1 < nt) issue(t + 1, buf ^ 1);
                continue;
            }
            const FA_LDS char* kt = (const FA_LDS char*)kbuf + buf * TILE;
            const FA_LDS char* vt = (const FA_LDS char*)vbuf + buf * TILE;
            const int k0 = t * BC;

            // S^T = K Q^T and dP^T = V dO^T; element (kb, r): key 32kb + 8(r/4) + 4hi + r%4, row my_q
            // Operand reads run kPf steps ahead of their products; the scheduling
            // fences keep them there (the compiler would sink each read to its use).
            f32x16 s[KB], dp[KB];
            {
                constexpr int SI = NCD * KB;
                auto ldo = [&](int i) { return roff[i / KB] + (i % KB) * 32 * ROW; };
                V8 ka[kPf], va[kPf];
#pragma unroll
                for (int j = 0; j < kPf; ++j) {
                    ka[j] = *(const FA_LDS V8*)(kt + ldo(j));
                    va[j] = *(const FA_LDS V8*)(vt + ldo(j));
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < SI; ++i) {
                    const int c = i / KB, kb = i % KB;
                    s[kb] = mfma32(ka[i % kPf], qreg[c], c == 0 ? f32x16{} : s[kb]);
                    dp[kb] = mfma32(va[i % kPf], doreg[c], c == 0 ? f32x16{} : dp[kb]);
                    if (i + kPf < SI) {
                        ka[i % kPf] = *(const FA_LDS V8*)(kt + ldo(i + kPf));
                        va[i % kPf] = *(const FA_LDS V8*)(vt + ldo(i + kPf));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // The next tile's copies go out once this tile's score products are
            // issued: issuing copies stalls the wave, and here that stall overlaps
            // the products instead of delaying their first operand reads.
            if (t + 1 < nt) issue(t + 1, buf ^ 1);
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
            V8 dsb[NC];
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
                    dsb[pc][pi] = (T)ds[0];
                    dsb[pc][pi + 1] = (T)ds[1];
                }
            // dQ^T += K^T dS^T over the tile's 16-key chunks
            {
                constexpr int QI = NC * DB;
                auto ldt = [&](int j) {    // K^T operand of step j = c * DB + db
                    const int c = j / DB, db = j % DB;
                    const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (FA_LDS s16x4*)(kt + troff[db][0] + 16 * c * ROW));
                    const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (FA_LDS s16x4*)(kt + troff[db][1] + 16 * c * ROW));
                    typedef short s16x8 __attribute__((ext_vector_type(8)));
                    return __builtin_bit_cast(V8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
                };
                V8 ta[kTf];
#pragma unroll
                for (int j = 0; j < kTf; ++j) ta[j] = ldt(j);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < QI; ++j) {
                    dqa[j % DB] = mfma32(ta[j % kTf], dsb[j / DB], dqa[j % DB]);
                    if (j + kTf < QI) ta[j % kTf] = ldt(j + kTf);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }

        if (my_q < N) {
            T* row = (T*)p.dq + p.ldq.base(b, h, start) + (size_t)my_q * p.ldq.sn;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                if (32 * db >= DH) break;          // padded columns are not stored
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    V4 w;
#pragma unroll
                    for (int i = 0; i < 4; ++i) w[i] = (T)(dqa[db][4 * g + i] * p.scale);
                    *(V4*)(row + 32 * db + 8 * g + 4 * hi) = w;
                }
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

template <typename T, int D, int DH, int NW, bool CAUSAL, bool DROPOUT>
hipError_t launch_dq_nw(const BwdArgs& a, hipStream_t st) {
    constexpr int BC = 64, BR = NW * 32;
    DqParams p{};
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.dout = a.dout;
    p.lse2 = a.lse2;
    p.dsum = a.dsum;
    p.dq = a.dq;
    p.lq = a.L.q;
    p.lk = a.L.k;
    p.lv = a.L.v;
    p.ldo = a.L.dout;
    p.ldq = a.L.dq;
    p.cu = a.L.cu_seqlens;
    p.total = a.L.total;
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
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, DH, BC, NW, CAUSAL, DROPOUT>), dim3(p.heads * blocks), dim3(NW * 64),
                       0, st, p);
    return hipGetLastError();
}

// Up to d = 128, eight waves (256 query rows) share each K/V tile when that
// grid still has two workgroups per CU of the 256-CU device; otherwise four
// (128 rows), which doubles the workgroups of small grids. Each row's
// arithmetic is the same either way, so dQ is bit-identical. (d = 256 needs a
// SIMD's whole register file per wave: four waves.)
template <typename T, int D, int DH, bool CAUSAL, bool DROPOUT>
hipError_t launch_dq_cfg(const BwdArgs& a, hipStream_t st) {
    if constexpr (D <= 128) {
        const int nqb8 = (a.s.N + 255) / 256;
        const long long wg8 = (long long)a.s.B * a.s.H * (CAUSAL ? (nqb8 + 1) / 2 : nqb8);
        if (wg8 >= 512) return launch_dq_nw<T, D, DH, 8, CAUSAL, DROPOUT>(a, st);
    }
    return launch_dq_nw<T, D, DH, 4, CAUSAL, DROPOUT>(a, st);
}

// The query-side pass of the two-pass backward: dQ only.
template <typename T, int D, int DH>
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t st) {
    const bool drop = dropout_threshold(a.s.dropout_p) != 0;
    if (a.s.causal) return drop ? launch_dq_cfg<T, D, DH, true, true>(a, st) : launch_dq_cfg<T, D, DH, true, false>(a, st);
    return drop ? launch_dq_cfg<T, D, DH, false, true>(a, st) : launch_dq_cfg<T, D, DH, false, false>(a, st);
}

}  // namespace
}  // namespace fa
