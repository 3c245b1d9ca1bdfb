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
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Element types of the matrix-core path: bf16 and fp16 share every layout
// (16-bit elements); they differ in the product instruction, the dot product
// of the weight sums and the float -> element rounding (both round to nearest
// even).
template <typename T> struct Vec;
template <> struct Vec<__bf16> {
    using x8 = bf16x8;
    using x4 = bf16x4;
    using x2 = bf16x2;
};
template <> struct Vec<_Float16> {
    using x8 = f16x8;
    using x4 = f16x4;
    using x2 = f16x2;
};

// 32x32 output, 16-deep contraction, fp32 accumulate.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// a0 b0 + a1 b1 + c in fp32.
__device__ __forceinline__ float dot2(bf16x2 a, bf16x2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}
__device__ __forceinline__ float dot2(f16x2 a, f16x2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Sequence of batch entry b: first token and length, clamped to the packed
// rows and to N (the whole N without packed sequences).
__device__ __forceinline__ void sequence(const int* cu, int total, int Nmax, int b, int& start, int& n) {
    start = 0;
    n = Nmax;
    if (cu) {
        start = min(max(cu[b], 0), total);
        n = min(min(max(cu[b + 1], start), total) - start, Nmax);
    }
}

// ---------------------------------------------------------------- buffers
// Raw buffer resource over `bytes` bytes at `base`. Loads at or past `bytes`
// return zero instead of touching memory, which covers ragged sequence tails.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16 bytes per lane from the buffer into LDS at lds_wave_base + lane * 16,
// issued as inline assembly, outside the compiler's wait-count tracking. With
// the compiler's own LDS-copy builtin the compiler cannot tell which LDS
// buffer a copy writes, so it makes every later LDS read wait for every copy
// still in flight, and a double-buffered loop that issues the next tile's
// copy before reading the current tile would wait for that copy first.
// Callers order it themselves: s_waitcnt vmcnt(0) (wait_vmem) and a workgroup
// barrier before any read of the destination, and no write of the
// destination's LDS by other code while it may be in flight. It has no register outputs; M0 carries the wave's
// LDS base, written by the compiler. The compiler's hazard checks do not see
// into the asm, so it leads with the five wait states a vector-memory
// instruction needs after a vector instruction wrote one of the SGPRs it reads
// (v_readlane / v_readfirstlane into the resource words or M0, as SGPR spills
// and reloads produce); that also covers the one wait state after an M0 write.
__device__ __forceinline__ void buffer_to_lds16_async(__amdgpu_buffer_rsrc_t rs, FA_LDS void* lds_wave_base,
                                                      uint32_t voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "{m0}"(m0), "v"(voffset), "s"(rs)
                 : "memory");
}

// 4 bytes per lane into LDS at lds_wave_base + lane * 4, ordered the same way.
__device__ __forceinline__ void buffer_to_lds4_async(__amdgpu_buffer_rsrc_t rs, FA_LDS void* lds_wave_base,
                                                     uint32_t voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
    asm volatile("s_nop 4\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :
                 : "{m0}"(m0), "v"(voffset), "s"(rs)
                 : "memory");
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voffset) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, voffset, 0, 0);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima), as a builtin
// so that the compiler's own wait tracking sees its loads complete here; an
// asm form would leave the compiler waiting for them again later, by counts
// that the untracked copies above would then stretch.
__device__ __forceinline__ void wait_vmem() {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------------------- LDS swizzle
// gfx950 LDS serves 256 bytes per pass: 16 lanes of a 16-byte read, or 32
// lanes of an 8-byte transposed read. Tiles are stored row-major with their
// 16-byte chunks XOR-permuted per row so that both access shapes used by the
// matrix-core operands hit 16 distinct 16-byte bank groups:
//   * 16 consecutive rows, same chunk (row operands, ds_read_b128);
//   * 4 aligned rows x 64 contiguous bytes (ds_read_b64_tr_b16 of a 32-wide
//     column block by lanes 0-31).
// CPR = 16-byte chunks per row (8, 16 or 32 for 128-, 256- or 512-byte rows).
template <int CPR>
__device__ __forceinline__ int chunk_swizzle(int row) {
    static_assert(CPR == 8 || CPR == 16 || CPR == 32, "rows of 128, 256 or 512 bytes");
    if (CPR >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);   // 512-byte rows: same banks as 256
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
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    typename Vec<T>::x2 r;
    r[0] = (T)a;
    r[1] = (T)b;
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

// a ^ b ^ k in one v_bitop3_b32 (truth table 0x96); k is wave-uniform.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t k) {
    uint32_t r;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
    return r;
}

// One round on counter (c0, c1, c2, c3) with round key (k0, k1). The 32x32->64
// products are plain 64-bit multiplies (one v_mad_u64_u32 each on gfx950).
__device__ __forceinline__ void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                             uint32_t k0, uint32_t k1) {
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c0;
    const uint64_t p1 = (uint64_t)kPhiloxM1 * c2;
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
}

// Output word 0 of the block function at counter (c0, c1, c2, c3).
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 PhiloxKey key) {
    uint32_t k0 = key.k0, k1 = key.k1;
#pragma unroll
    for (int r = 0; r < 9; ++r) {
        philox_round(c0, c1, c2, c3, k0, k1);
        k0 += kPhiloxW0;
        k1 += kPhiloxW1;
    }
    return xor3((uint32_t)(((uint64_t)kPhiloxM1 * c2) >> 32), c1, k0);   // round 10, word 0 only
}

// Word 0 at counter (c0, c1, c2, j) for a fixed (c0, c1, c2) and varying j:
// the parts of rounds 1-3 that do not depend on j are computed once.
//   round 1: x0, x1, x3 fixed; x2 = A ^ j
//   round 2: y0 = hi(M1 x2) ^ B, y1 = lo(M1 x2); y2, y3 fixed
//   round 3: z0 = D0 ^ y1, z1 = E1 fixed, z2 = hi(M0 y0) ^ F, z3 = lo(M0 y0)
struct PhiloxRow {
    uint32_t A, B, D0, E1, F;
    uint32_t k0_3, k1_3;   // key of round 4

    PhiloxRow() = default;
    __device__ __forceinline__ PhiloxRow(uint32_t c0, uint32_t c1, uint32_t c2, PhiloxKey key) {
        uint32_t k0 = key.k0, k1 = key.k1;
        const uint64_t p0 = (uint64_t)kPhiloxM0 * c0;   // round 1
        const uint64_t p1 = (uint64_t)kPhiloxM1 * c2;
        const uint32_t x0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t x1 = (uint32_t)p1;
        const uint32_t x3 = (uint32_t)p0;
        A = (uint32_t)(p0 >> 32) ^ k1;
        k0 += kPhiloxW0;
        k1 += kPhiloxW1;
        const uint64_t q0 = (uint64_t)kPhiloxM0 * x0;   // round 2, fixed half
        B = x1 ^ k0;
        const uint32_t y2 = (uint32_t)(q0 >> 32) ^ x3 ^ k1;
        const uint32_t y3 = (uint32_t)q0;
        k0 += kPhiloxW0;
        k1 += kPhiloxW1;
        const uint64_t r1 = (uint64_t)kPhiloxM1 * y2;   // round 3, fixed half
        D0 = (uint32_t)(r1 >> 32) ^ k0;
        E1 = (uint32_t)r1;
        F = y3 ^ k1;
        k0_3 = k0 + kPhiloxW0;
        k1_3 = k1 + kPhiloxW1;
    }

    __device__ __forceinline__ uint32_t word0(uint32_t j) const {
        const uint64_t q1 = (uint64_t)kPhiloxM1 * (A ^ j);   // round 2, varying half
        const uint32_t y0 = (uint32_t)(q1 >> 32) ^ B;
        const uint32_t y1 = (uint32_t)q1;
        const uint64_t r0 = (uint64_t)kPhiloxM0 * y0;       // round 3, varying half
        uint32_t c0 = D0 ^ y1, c1 = E1, c2 = (uint32_t)(r0 >> 32) ^ F, c3 = (uint32_t)r0;
        uint32_t k0 = k0_3, k1 = k1_3;
#pragma unroll
        for (int r = 3; r < 9; ++r) {
            philox_round(c0, c1, c2, c3, k0, k1);
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        return xor3((uint32_t)(((uint64_t)kPhiloxM1 * c2) >> 32), c1, k0);
    }
};

// Word 0 at counter (c0, c1, i, c3) for a fixed (c0, c1, c3) and varying row
// i (the key-side backward: a lane holds one key j = c3 against many rows):
//   round 1: x2 = hi(M0 c0) ^ c3 ^ k1 and x3 = lo(M0 c0) fixed; x0, x1 from M1 i
//   round 2: y1 = lo(M1 x2) and hi(M1 x2) ^ k0 fixed; y0, y2, y3 vary
struct PhiloxCol {
    uint32_t c1k0, G, y1, X3K;   // c1 ^ k0 (round 1); hi(M1 x2) ^ k0 and lo(M1 x2), x3 ^ k1 (round 2)
    uint32_t k0_2, k1_2;          // key of round 3

    PhiloxCol() = default;
    __device__ __forceinline__ PhiloxCol(uint32_t c0, uint32_t c1, uint32_t c3, PhiloxKey key) {
        uint32_t k0 = key.k0, k1 = key.k1;
        const uint64_t p0 = (uint64_t)kPhiloxM0 * c0;   // round 1, fixed half
        const uint32_t x2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        const uint32_t x3 = (uint32_t)p0;
        c1k0 = c1 ^ k0;
        k0 += kPhiloxW0;
        k1 += kPhiloxW1;
        const uint64_t q1 = (uint64_t)kPhiloxM1 * x2;   // round 2, fixed half
        G = (uint32_t)(q1 >> 32) ^ k0;
        y1 = (uint32_t)q1;
        X3K = x3 ^ k1;
        k0_2 = k0 + kPhiloxW0;
        k1_2 = k1 + kPhiloxW1;
    }

    __device__ __forceinline__ uint32_t word0(uint32_t i) const {
        const uint64_t p1 = (uint64_t)kPhiloxM1 * i;          // round 1, varying half
        const uint32_t x0 = (uint32_t)(p1 >> 32) ^ c1k0;
        const uint32_t x1 = (uint32_t)p1;
        const uint64_t q0 = (uint64_t)kPhiloxM0 * x0;         // round 2, varying half
        uint32_t c0 = G ^ x1, c1 = y1, c2 = (uint32_t)(q0 >> 32) ^ X3K, c3 = (uint32_t)q0;
        uint32_t k0 = k0_2, k1 = k1_2;
#pragma unroll
        for (int r = 2; r < 9; ++r) {
            philox_round(c0, c1, c2, c3, k0, k1);
            k0 += kPhiloxW0;
            k1 += kPhiloxW1;
        }
        return xor3((uint32_t)(((uint64_t)kPhiloxM1 * c2) >> 32), c1, k0);
    }
};

}  // namespace fa
