// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, bf16 packing, buffer resources (hardware range checks that
// return zeros past the end of a head), cross-half wave exchange, and the
// Philox-4x32-10 dropout generator.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- buffers
// Raw buffer resource over `bytes` bytes at `base`. Loads at or past `bytes`
// return zero instead of touching memory, which covers ragged sequence tails.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16 bytes per lane from the buffer into LDS at lds_wave_base + lane * 16.
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t rs, FA_LDS void* lds_wave_base,
                                                uint32_t voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_wave_base, 16, voffset, 0, 0, 0);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voffset) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, voffset, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------------- LDS swizzle
// gfx950 LDS serves 256 bytes per pass: 16 lanes of a 16-byte read, or 32
// lanes of an 8-byte transposed read. Tiles are stored row-major with their
// 16-byte chunks XOR-permuted per row so that both access shapes used by the
// matrix-core operands hit 16 distinct 16-byte bank groups:
//   * 16 consecutive rows, same chunk (row operands, ds_read_b128);
//   * 4 aligned rows x 64 contiguous bytes (ds_read_b64_tr_b16 of a 32-wide
//     column block by lanes 0-31).
// CPR = 16-byte chunks per row (8 for 128-byte rows, 16 for 256-byte rows).
template <int CPR>
__device__ __forceinline__ int chunk_swizzle(int row) {
    static_assert(CPR == 8 || CPR == 16, "rows of 128 or 256 bytes");
    if (CPR == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Byte offset of element (row, col) of a bf16 tile with CPR chunks per row.
template <int CPR>
__device__ __forceinline__ int tile_offset(int row, int col) {
    return row * CPR * 16 + (((col >> 3) ^ chunk_swizzle<CPR>(row)) << 4) + ((col & 7) << 1);
}

// --------------------------------------------------------------- exchange
// Value held by lane (l ^ 32): v_permlane32_swap exchanges the upper half of
// the first operand with the lower half of the second, so swapping x with
// itself leaves the partner's value in one of the two results.
__device__ __forceinline__ float max_with_partner32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_with_partner32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ------------------------------------------------------------------- bf16
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 r;
    r[0] = (__bf16)a;   // v_cvt_pk_bf16_f32: round to nearest even
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// ------------------------------------------------------------------ Philox
// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds; each round
// takes the 64-bit products of words 0 and 2 with the two round multipliers
// and mixes their high halves with words 1 and 3 and the round key; the key
// advances by the two Weyl increments between rounds.
constexpr uint32_t kPhiloxM0 = 0xD2511F53u;
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u;
constexpr uint32_t kPhiloxW1 = 0xBB67AE85u;

struct PhiloxKey {
    uint32_t k0, k1;
};

// Output word 0 of the block function at counter (c0, c1, c2, c3).
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 PhiloxKey key) {
    uint32_t k0 = key.k0, k1 = key.k1;
#pragma unroll
    for (int r = 0; r < 9; ++r) {
        const uint32_t hi0 = __umulhi(kPhiloxM0, c0), lo0 = kPhiloxM0 * c0;
        const uint32_t hi1 = __umulhi(kPhiloxM1, c2), lo1 = kPhiloxM1 * c2;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += kPhiloxW0;
        k1 += kPhiloxW1;
    }
    return __umulhi(kPhiloxM1, c2) ^ c1 ^ k0;   // round 10, word 0 only
}

}  // namespace fa
