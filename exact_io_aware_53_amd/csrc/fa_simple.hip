// Vector-ALU attention kernels in fp32 arithmetic, templated on the storage
// type. They serve the fp32 entry points (fa_fwd_f32 / fa_bwd_f32), where the
// matrix cores' bf16 path does not apply.
//
// Forward: the tile-by-tile method of "DL0056 FlashAttention" (intvml),
// "Mathematical Formulation": each workgroup owns 16 query rows, streams K/V
// tiles of 32 keys through LDS, keeps the running row maximum m and the
// rescaled running denominator l, and rescales its output accumulator by the
// same factor exp(m_old - m_new) (the output update the page describes in
// point (2) without printing it). Only O and LSE = m + ln l are written.
//
// Backward: recomputation (inferensys glossary "FlashAttention", paragraph on
// recomputation): P = exp(S - LSE) is rebuilt from the stored LSE, never read
// from memory. One kernel forms D_i = <dO_i, O_i>; one accumulates dK, dV per
// key block over the query rows; one accumulates dQ per query block over the
// key rows (no atomics). Dropout regenerates the forward's Philox mask.
#include <math.h>

#include "fa_device.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kRows = 64;      // backward: query (dQ) or key (dK/dV) rows per workgroup
constexpr int kTile = 32;      // streamed rows per LDS tile
constexpr int kThreads = 256;  // backward: 4 threads per row, each owning d/4 columns

template <typename T> __device__ __forceinline__ float ld(const T* p) { return (float)*p; }
template <typename T> __device__ __forceinline__ void st(T* p, float x) { *p = (T)x; }

struct SimpleParams {
    const void* q; const void* k; const void* v; const void* o; const void* dout;
    const float* lse; void* out0; void* out1; void* out2; float* lse_out; float* dsum;
    int H, N;
    float scale, inv_keep;   // inv_keep = 1 / (1 - p)
    uint32_t thr;            // dropout iff thr > 0
    PhiloxKey key;
    bool causal;
};

__device__ __forceinline__ float keep_scale(const SimpleParams& p, int b, int h, int i, int j) {
    if (p.thr == 0) return 1.0f;
    return philox_word0((uint32_t)b, (uint32_t)h, (uint32_t)i, (uint32_t)j, p.key) >= p.thr ? p.inv_keep : 0.0f;
}

// Sum over the 4 consecutive lanes that share one row.
__device__ __forceinline__ float quad_sum(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    return x;
}

// Stage rows [r0, r0 + kTile) of a [N, D] head into LDS as fp32 (zeros past N).
template <typename T, int D>
__device__ __forceinline__ void stage_rows(float (*dst)[D], const T* src, int r0, int N) {
    for (int e = threadIdx.x; e < kTile * D; e += kThreads) {
        const int r = e / D, c = e % D;
        dst[r][c] = (r0 + r < N) ? ld(src + (size_t)(r0 + r) * D + c) : 0.0f;
    }
}

// Forward: 16 query rows per workgroup, 16 consecutive lanes per row, each
// lane owning D/16 columns. For a 32-key tile a lane first forms its partial
// dot products with all 32 keys (independent chains), then each is summed over
// the row's 16 lanes.
constexpr int kFRows = 16;
constexpr int kFLanes = kThreads / kFRows;

__device__ __forceinline__ float row_sum16(float x) {
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    return x;
}

// Rows [r0, r0 + kTile) of a [N, D] fp32 head, 16 bytes per load, into
// registers (zeros past N); each thread holds kTile * D / (4 kThreads) of them.
template <int D>
struct TileRegs {
    static constexpr int NV = kTile * D / (4 * kThreads);
    static_assert(NV * 4 * kThreads == kTile * D, "a tile is whole 16-byte groups per thread");
    float4 x[NV];
    __device__ __forceinline__ void load(const float* src, int r0, int N) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = (i * kThreads + threadIdx.x) * 4, r = e / D, c = e % D;
            x[i] = r0 + r < N ? *(const float4*)(src + (size_t)(r0 + r) * D + c) : float4{0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
    __device__ __forceinline__ void store(float (*dst)[D]) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = (i * kThreads + threadIdx.x) * 4, r = e / D, c = e % D;
            *(float4*)&dst[r][c] = x[i];
        }
    }
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void fwd_simple_kernel(SimpleParams p) {
    static_assert(sizeof(T) == 4, "the forward stages fp32 rows");
    constexpr int DC = D / kFLanes;
    __shared__ __attribute__((aligned(16))) float ks[kTile][D];
    __shared__ __attribute__((aligned(16))) float vs[kTile][D];
    const int nblk = (p.N + kFRows - 1) / kFRows;
    const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
    const int b = bh / p.H, h = bh % p.H;
    const int row = blk * kFRows + threadIdx.x / kFLanes, c0 = (threadIdx.x % kFLanes) * DC;
    const size_t head = (size_t)bh * p.N * D;
    const T* q = (const T*)p.q + head;
    const T* k = (const T*)p.k + head;
    const T* v = (const T*)p.v + head;

    float qr[DC], acc[DC];
    for (int t = 0; t < DC; ++t) {
        qr[t] = row < p.N ? ld(q + (size_t)row * D + c0 + t) : 0.0f;
        acc[t] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    const int last_row = min(p.N, (blk + 1) * kFRows) - 1;
    const int key_end = p.causal ? last_row + 1 : p.N;
    // K/V tiles double-buffered through registers: the loads of tile t + 1 are in
    // flight while tile t is computed from LDS.
    TileRegs<D> kr, vr;
    kr.load((const float*)k, 0, p.N);
    vr.load((const float*)v, 0, p.N);
    for (int k0 = 0; k0 < key_end; k0 += kTile) {
        __syncthreads();
        kr.store(ks);
        vr.store(vs);
        __syncthreads();
        if (k0 + kTile < key_end) {
            kr.load((const float*)k, k0 + kTile, p.N);
            vr.load((const float*)v, k0 + kTile, p.N);
        }
        float s[kTile];
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            float part = 0.0f;
#pragma unroll
            for (int t = 0; t < DC; ++t) part = fmaf(qr[t], ks[j][c0 + t], part);
            s[j] = part;
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const float sc = row_sum16(s[j]) * p.scale;
            const int key = k0 + j;
            const bool live = key < p.N && (!p.causal || key <= row);
            s[j] = live ? sc : -INFINITY;
            tmax = fmaxf(tmax, s[j]);
        }
        const float m_new = fmaxf(m, tmax);
        if (m_new == -INFINITY) continue;          // nothing visible yet for this row
        const float alpha = expf(m - m_new);       // 0 on the first live tile
        float psum = 0.0f;
#pragma unroll
        for (int t = 0; t < DC; ++t) acc[t] *= alpha;
        for (int j = 0; j < kTile; ++j) {
            const float pj = expf(s[j] - m_new);   // exp(-inf) = 0 for masked keys
            psum += pj;
            const float w = pj * keep_scale(p, b, h, row, k0 + j);
#pragma unroll
            for (int t = 0; t < DC; ++t) acc[t] = fmaf(w, vs[j][c0 + t], acc[t]);
        }
        l = alpha * l + psum;
        m = m_new;
    }
    if (row < p.N) {
        const float inv = 1.0f / l;
        T* o = (T*)p.out0 + head + (size_t)row * D + c0;
        for (int t = 0; t < DC; ++t) st(o + t, acc[t] * inv);
        if (threadIdx.x % kFLanes == 0) p.lse_out[(size_t)bh * p.N + row] = m + logf(l);
    }
}

// D_i = <dO_i, O_i>, one thread per row.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dsum_kernel(SimpleParams p, int rows) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const T* o = (const T*)p.o + (size_t)r * D;
    const T* g = (const T*)p.dout + (size_t)r * D;
    float acc = 0.0f;
    for (int t = 0; t < D; ++t) acc = fmaf(ld(o + t), ld(g + t), acc);
    p.dsum[r] = acc;
}

// dK, dV for 64 key rows; streams query tiles (Q, dO) through LDS.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_dkdv_simple_kernel(SimpleParams p) {
    constexpr int DQ = D / 4;
    __shared__ float qs[kTile][D];
    __shared__ float gs[kTile][D];
    __shared__ float lse_s[kTile], dsum_s[kTile];
    const int nblk = (p.N + kRows - 1) / kRows;
    const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
    const int b = bh / p.H, h = bh % p.H;
    const int key = blk * kRows + threadIdx.x / 4, c0 = (threadIdx.x % 4) * DQ;
    const size_t head = (size_t)bh * p.N * D;
    const T* q = (const T*)p.q + head;
    const T* k = (const T*)p.k + head;
    const T* v = (const T*)p.v + head;
    const T* g = (const T*)p.dout + head;

    float kr[DQ], vr[DQ], dk[DQ], dv[DQ];
    for (int t = 0; t < DQ; ++t) {
        kr[t] = key < p.N ? ld(k + (size_t)key * D + c0 + t) : 0.0f;
        vr[t] = key < p.N ? ld(v + (size_t)key * D + c0 + t) : 0.0f;
        dk[t] = dv[t] = 0.0f;
    }
    const int q_begin = p.causal ? (blk * kRows) / kTile * kTile : 0;
    for (int i0 = q_begin; i0 < p.N; i0 += kTile) {
        __syncthreads();
        stage_rows<T, D>(qs, q, i0, p.N);
        stage_rows<T, D>(gs, g, i0, p.N);
        if (threadIdx.x < kTile) {
            const int i = i0 + threadIdx.x;
            lse_s[threadIdx.x] = i < p.N ? p.lse[(size_t)bh * p.N + i] : 0.0f;
            dsum_s[threadIdx.x] = i < p.N ? p.dsum[(size_t)bh * p.N + i] : 0.0f;
        }
        __syncthreads();
        for (int r = 0; r < kTile; ++r) {
            const int i = i0 + r;
            float sp = 0.0f, dpp = 0.0f;
            for (int t = 0; t < DQ; ++t) {
                sp = fmaf(kr[t], qs[r][c0 + t], sp);
                dpp = fmaf(vr[t], gs[r][c0 + t], dpp);
            }
            sp = quad_sum(sp);
            dpp = quad_sum(dpp);
            const bool live = i < p.N && key < p.N && (!p.causal || key <= i);
            if (!live) continue;
            const float pij = expf(sp * p.scale - lse_s[r]);
            const float z = keep_scale(p, b, h, i, key);
            const float ds = pij * (dpp * z - dsum_s[r]);
            for (int t = 0; t < DQ; ++t) {
                dv[t] = fmaf(pij * z, gs[r][c0 + t], dv[t]);
                dk[t] = fmaf(ds, qs[r][c0 + t], dk[t]);
            }
        }
    }
    if (key < p.N) {
        T* dko = (T*)p.out1 + head + (size_t)key * D + c0;
        T* dvo = (T*)p.out2 + head + (size_t)key * D + c0;
        for (int t = 0; t < DQ; ++t) {
            st(dko + t, dk[t] * p.scale);
            st(dvo + t, dv[t]);
        }
    }
}

// dQ for 64 query rows; streams key tiles (K, V) through LDS.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_simple_kernel(SimpleParams p) {
    constexpr int DQ = D / 4;
    __shared__ float ks[kTile][D];
    __shared__ float vs[kTile][D];
    const int nblk = (p.N + kRows - 1) / kRows;
    const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
    const int b = bh / p.H, h = bh % p.H;
    const int row = blk * kRows + threadIdx.x / 4, c0 = (threadIdx.x % 4) * DQ;
    const size_t head = (size_t)bh * p.N * D;
    const T* q = (const T*)p.q + head;
    const T* k = (const T*)p.k + head;
    const T* v = (const T*)p.v + head;
    const T* g = (const T*)p.dout + head;

    float qr[DQ], gr[DQ], dq[DQ];
    for (int t = 0; t < DQ; ++t) {
        qr[t] = row < p.N ? ld(q + (size_t)row * D + c0 + t) : 0.0f;
        gr[t] = row < p.N ? ld(g + (size_t)row * D + c0 + t) : 0.0f;
        dq[t] = 0.0f;
    }
    const float lse_i = row < p.N ? p.lse[(size_t)bh * p.N + row] : 0.0f;
    const float dsum_i = row < p.N ? p.dsum[(size_t)bh * p.N + row] : 0.0f;
    const int last_row = min(p.N, (blk + 1) * kRows) - 1;
    const int key_end = p.causal ? last_row + 1 : p.N;
    for (int k0 = 0; k0 < key_end; k0 += kTile) {
        __syncthreads();
        stage_rows<T, D>(ks, k, k0, p.N);
        stage_rows<T, D>(vs, v, k0, p.N);
        __syncthreads();
        for (int j = 0; j < kTile; ++j) {
            const int key = k0 + j;
            float sp = 0.0f, dpp = 0.0f;
            for (int t = 0; t < DQ; ++t) {
                sp = fmaf(qr[t], ks[j][c0 + t], sp);
                dpp = fmaf(gr[t], vs[j][c0 + t], dpp);
            }
            sp = quad_sum(sp);
            dpp = quad_sum(dpp);
            const bool live = row < p.N && key < p.N && (!p.causal || key <= row);
            if (!live) continue;
            const float pij = expf(sp * p.scale - lse_i);
            const float z = keep_scale(p, b, h, row, key);
            const float ds = pij * (dpp * z - dsum_i);
            for (int t = 0; t < DQ; ++t) dq[t] = fmaf(ds, ks[j][c0 + t], dq[t]);
        }
    }
    if (row < p.N) {
        T* dqo = (T*)p.out0 + head + (size_t)row * D + c0;
        for (int t = 0; t < DQ; ++t) st(dqo + t, dq[t] * p.scale);
    }
}

SimpleParams make_params(const AttnShape& s) {
    SimpleParams p{};
    p.H = s.H;
    p.N = s.N;
    p.scale = s.scale;
    p.inv_keep = 1.0f / (1.0f - s.dropout_p);
    p.thr = dropout_threshold(s.dropout_p);
    p.key = PhiloxKey{(uint32_t)(s.seed & 0xffffffffu), (uint32_t)(s.seed >> 32)};
    p.causal = s.causal;
    return p;
}

template <typename T, int D>
hipError_t fwd_simple(const FwdArgs& a, hipStream_t st) {
    SimpleParams p = make_params(a.s);
    p.q = a.q; p.k = a.k; p.v = a.v; p.out0 = a.o; p.lse_out = a.lse;
    const int nblk = (a.s.N + kFRows - 1) / kFRows;
    hipLaunchKernelGGL((fwd_simple_kernel<T, D>), dim3(a.s.B * a.s.H * nblk), dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_simple(const BwdArgs& a, hipStream_t st) {
    SimpleParams p = make_params(a.s);
    p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o; p.dout = a.dout; p.lse = a.lse;
    p.out0 = a.dq; p.out1 = a.dk; p.out2 = a.dv; p.dsum = a.dsum;
    const int rows = a.s.B * a.s.H * a.s.N;
    hipLaunchKernelGGL((bwd_dsum_kernel<T, D>), dim3((rows + 255) / 256), dim3(256), 0, st, p, rows);
    const int nblk = (a.s.N + kRows - 1) / kRows;
    const dim3 grid(a.s.B * a.s.H * nblk);
    hipLaunchKernelGGL((bwd_dkdv_simple_kernel<T, D>), grid, dim3(kThreads), 0, st, p);
    hipLaunchKernelGGL((bwd_dq_simple_kernel<T, D>), grid, dim3(kThreads), 0, st, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t st) {
    return a.s.d == 64 ? fwd_simple<float, 64>(a, st) : fwd_simple<float, 128>(a, st);
}

hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t st) {
    return a.s.d == 64 ? bwd_simple<float, 64>(a, st) : bwd_simple<float, 128>(a, st);
}

}  // namespace fa
