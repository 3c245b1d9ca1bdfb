// Padded K/V tiles in LDS for the gfx950 attention kernels: layout, the
// HBM -> LDS copy through the buffer unit's LDS path, and the per-lane operand
// reads of the matrix-core products.
#pragma once

#include "fa_device.hpp"

namespace fa {

// K/V tiles in LDS use padded rows instead of a swizzle, so that every
// operand read of a lane is one base register plus an immediate offset:
//  * K rows are read 16 rows x 16 bytes per pass (row operands); a row stride
//    of 2D + 16 bytes puts 16 consecutive rows on 16 distinct 16-byte bank
//    groups.
//  * V is read transposed, 4 rows x 64 bytes per pass; a row stride of 64 or
//    192 bytes modulo 256 (2D + 64 bytes for d = 64 and 128, no pad for d = 32
//    and 96) puts 4 consecutive rows on 4 distinct 64-byte bank groups.
// The copy engine writes 64 x 16 contiguous bytes per wave instruction, so the
// pad chunks are copied too, from an out-of-range offset (zeros, no memory
// access).
template <int D, int BC>
struct PaddedTiles {
    static constexpr int CH = D / 8;                 // 16-byte chunks of data per row
    static constexpr int vch() {
        int v = CH;
        while (v % 16 != 4 && v % 16 != 12) ++v;
        return v;
    }
    static_assert(CH % 2 == 0, "an odd K row stride in chunks needs an even chunk count");
    static constexpr int KCH = CH + 1, VCH = vch();
    static constexpr int KS = KCH * 16, VS = VCH * 16;
    static constexpr int K_TILE = BC * KS, V_TILE = BC * VS;
};

// Copy of rows [t*BC, t*BC + BC) of one head (row stride ld elements) into a
// padded tile with RCH chunks per row; the NW waves of the workgroup share the
// 1 KB copy blocks.
// The per-lane source offsets within a tile are computed once; a tile adds
// t * BC rows. Pad chunks read from far past the head (zeros, no memory
// access; should the sum wrap for a huge head they load real bytes, which is
// harmless: pad chunks are never read).
template <int D, int BC, int RCH, int NW>
struct TileCopy {
    static constexpr int CH = D / 8, BLKS = BC * RCH / 64, PER = (BLKS + NW - 1) / NW;
    static_assert(BLKS * 64 == BC * RCH, "a tile is whole 1 KB copy blocks");
    static constexpr uint32_t kPad = 0xf0000000u;
    uint32_t off[PER];
    uint32_t step;      // bytes per tile of rows

    __device__ __forceinline__ TileCopy(int wave, int lane, int ld = D) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int pos = (i * NW + wave) * 64 + lane;
            const int row = pos / RCH, ch = pos % RCH;
            off[i] = ch < CH ? (uint32_t)(row * ld + ch * 8) * 2 : kPad;
        }
        step = (uint32_t)(BC * ld * 2);
    }
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, FA_LDS char* base, int t, int wave) const {
        // Tile offset as an opaque scalar: otherwise loop strength reduction
        // turns every off[i] into a vector induction variable of its own.
        const uint32_t toff = __builtin_amdgcn_readfirstlane((uint32_t)t * step);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            // blocks i * NW + wave with i < PER - 1 are below BLKS for every wave
            const int blk = i * NW + wave;
            if (i < PER - 1 || blk < BLKS) buffer_to_lds16_async(rs, (FA_LDS void*)(base + blk * 1024), off[i] + toff);
        }
    }
};

// Per-lane base offsets of the operand reads in padded tiles.
//  K operand (S^T = K Q^T, A side): key row l32 (+32 per key block), d = 16c + 8hi .. +7.
//  V^T operand (O^T = V^T P^T, A side): d = 32db + column, keys 16c + 4(lane/32) + {0..3}
//  and +8; within a 16-lane group, lane s reads key row s/4 and 4 columns at 4(s%4).
template <int D, int BC>
__device__ __forceinline__ int k_base(int lane) {
    return (lane & 31) * PaddedTiles<D, BC>::KS + (lane >> 5) * 16;
}
template <int D, int BC>
__device__ __forceinline__ int v_base(int lane) {
    return (4 * (lane >> 5) + ((lane & 15) >> 2)) * PaddedTiles<D, BC>::VS +
           2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));
}
// K operand i = c * KB + kb of a tile (KB = BC / 32 key blocks).
template <int D, int BC, typename V8 = bf16x8>
__device__ __forceinline__ V8 k_operand(const FA_LDS char* kt, int kbase, int i) {
    constexpr int KB = BC / 32;
    return *(const FA_LDS V8*)(kt + kbase + (i / KB) * 32 + (i % KB) * 32 * PaddedTiles<D, BC>::KS);
}
// V^T operand j = c * DB + db of a tile (DB = D / 32 d blocks, c = 16-key chunk).
template <int D, int BC, typename V8 = bf16x8>
__device__ __forceinline__ V8 v_operand(const FA_LDS char* vt, int vbase, int j) {
    constexpr int DB = D / 32, VS = PaddedTiles<D, BC>::VS;
    s16x4 x[2];
#pragma unroll
    for (int half = 0; half < 2; ++half)
        x[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (FA_LDS s16x4*)(vt + vbase + (16 * (j / DB) + 8 * half) * VS + 64 * (j % DB)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 a = __builtin_shufflevector(x[0], x[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(V8, a);
}

}  // namespace fa
