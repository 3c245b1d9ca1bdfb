// Decode-shaped forward for bf16 tensors on gfx950: a few query rows (the
// newest tokens) against a long key/value sequence (the cache that inference
// servers keep; inferensys glossary "FlashAttention", paragraph on
// integration with inference servers). The computation is the same attention
// as the forward ("DL0056 FlashAttention", "Mathematical Formulation"); only
// the work split differs. A short query block gives too few query blocks to
// fill the chip, so the key range is split instead:
//
//   split kernel  one workgroup per (head, 32-row query block, key chunk).
//                 Its four waves take interleaved 32-key tiles of the chunk,
//                 each with its own running max, denominator and output, and
//                 merge them at the end through LDS. The chunk's partial
//                 output O_s (normalised) and log-sum-exp LSE_s go to the
//                 workspace, or straight to O and LSE when there is one chunk.
//   merge kernel  LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s:
//                 the rescaling of the online softmax applied to whole chunks.
//
// Causal: query row i sits at key position Nk - Nq + i and sees keys up to it.
//
// gfx950 mapping. The work is bound by reading K and V once from HBM. Each
// wave loads the K rows of its tile straight into registers as matrix-core A
// operands (S^T = K Q^T, as in the forward), and copies the V tile into its
// own double-buffered LDS region (padded rows) for the transposed reads of
// O^T = V^T P^T. The waves never wait for each other inside the loop.
#include "fa_device.hpp"
#include "fa_launch.hpp"
#include "fa_tiles.hpp"

namespace fa {
namespace {

constexpr float DEC_SLACK = 8.0f;   // lazy rescale slack (log2 units), as in the forward with dropout
constexpr int kDecNW = 4;           // waves per workgroup
constexpr int kDecTile = 32;        // keys per wave tile
constexpr int kDecChunk = kDecNW * kDecTile;   // key chunks are multiples of this

struct DecodeParams {
    const __bf16* q;
    const __bf16* k;          // contiguous: [heads, Nk, D]; paged: the page pool [num_pages, H, page, D]
    const __bf16* v;
    __bf16* o;
    float* lse;
    float* o_part;     // [heads, S, Nq, D] fp32 partial outputs (S > 1)
    float* lse_part;   // [heads, S, Nq] fp32 partial log-sum-exp (S > 1)
    const int* block_table;   // paged: [B, max_blocks] page of each logical block
    const int* seq_lens;      // paged: [B] key count of each sequence
    int Nq, Nk, nrb, S, chunk;
    int H, max_blocks, page, num_pages;
    float sl2;         // scale * log2(e)
};

template <int D, bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(kDecNW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_split_kernel(DecodeParams p) {
    constexpr int DB = D / 32, NCD = D / 16;
    using PT = PaddedTiles<D, kDecTile>;
    constexpr int VT = PT::V_TILE;                                  // one padded 32-key V tile
    constexpr int MERGE_BYTES = kDecNW * 32 * D * 4 + kDecNW * 32 * 3 * 4;
    constexpr int LDS_BYTES = kDecNW * 2 * VT > MERGE_BYTES ? kDecNW * 2 * VT : MERGE_BYTES;
    __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, hi = lane >> 5;

    const int bid = blockIdx.x;
    const int s = bid % p.S, rest = bid / p.S;
    const int rb = rest % p.nrb, bh = rest / p.nrb;
    const int Nq = p.Nq;
    const int b = bh / p.H, h = bh - b * p.H;
    // Keys of this sequence (paged: its own length, clamped to the block table's reach).
    const int Nk = PAGED ? min(max(p.seq_lens[b], 0), p.max_blocks * p.page) : p.Nk;
    const int r0 = rb * 32, my_q = r0 + l32;
    const auto rs_q = make_rsrc(p.q + (size_t)bh * Nq * D, (uint32_t)Nq * D * 2);
    const auto rs_k = make_rsrc(p.k + (size_t)bh * Nk * D, (uint32_t)Nk * D * 2);
    const auto rs_v = make_rsrc(p.v + (size_t)bh * Nk * D, (uint32_t)Nk * D * 2);
    // Paged: the 32-key tile at key0 lies in one page (pages are whole tiles).
    // A block-table entry outside [0, num_pages) reads as zeros.
    struct TileSrc {
        __amdgpu_buffer_rsrc_t k, v;
        int row;                       // first row of the tile inside the resource
    };
    auto tile_src = [&](int key0) {
        if (!PAGED) return TileSrc{rs_k, rs_v, key0};
        const int lb = key0 / p.page;
        const int pid = p.block_table[(size_t)b * p.max_blocks + lb];
        const bool ok = pid >= 0 && pid < p.num_pages;
        const size_t base = ((size_t)(ok ? pid : 0) * p.H + h) * p.page * D;
        const uint32_t bytes = ok ? (uint32_t)p.page * D * 2 : 0u;
        return TileSrc{make_rsrc(p.k + base, bytes), make_rsrc(p.v + base, bytes), key0 - lb * p.page};
    };

    // Keys of this chunk that any row of the block may see.
    const int off = Nk - Nq;                                        // key position of query row 0
    const int k_lo = s * p.chunk;
    int k_hi = min(Nk, k_lo + p.chunk);
    if (CAUSAL) k_hi = min(k_hi, off + min(r0 + 31, Nq - 1) + 1);
    const int ntiles = k_hi > k_lo ? (k_hi - k_lo + kDecTile - 1) / kDecTile : 0;
    // Last key row my_q may see; rows past Nq are never stored.
    const int lim = CAUSAL ? min(off + my_q, k_hi - 1) : k_hi - 1;

    bf16x8 qreg[NCD];
#pragma unroll
    for (int c = 0; c < NCD; ++c)
        qreg[c] = __builtin_bit_cast(bf16x8, buffer_load16(rs_q, (uint32_t)(my_q * D + 16 * c + 8 * hi) * 2));

    f32x16 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] = 0.0f;
    float m2 = -INFINITY, lsum = 0.0f, lbf = 0.0f;

    FA_LDS char* const vw = (FA_LDS char*)lds + wave * 2 * VT;     // this wave's two V buffers
    const TileCopy<D, kDecTile, PT::VCH, 1> vcopy(0, lane);
    const int vbase = v_base<D, kDecTile>(lane);
    // Tile t of this wave covers keys k_lo + 32 (wave + 4t) ...
    auto key0 = [&](int t) { return k_lo + kDecTile * (wave + kDecNW * t); };
    auto load_kv = [&](int t, bf16x8 (&kr)[NCD]) {
        const TileSrc src = tile_src(key0(t));
        const int row = src.row + l32;
#pragma unroll
        for (int c = 0; c < NCD; ++c)
            kr[c] = __builtin_bit_cast(bf16x8, buffer_load16(src.k, (uint32_t)(row * D + 16 * c + 8 * hi) * 2));
        vcopy.issue(src.v, vw + (t & 1) * VT, src.row / kDecTile, 0);
    };

    const int nt_w = ntiles > wave ? (ntiles - wave + kDecNW - 1) / kDecNW : 0;   // this wave's tiles
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    // Tile t with its K operands in kc; the next tile's K goes to kn (the two
    // register sets swap roles from tile to tile, so no copy waits on a load).
    auto tile = [&](int t, bf16x8 (&kc)[NCD], bf16x8 (&kn)[NCD]) {
        wait_vmem();                      // K registers and V tile t have landed
        if (t + 1 < nt_w) load_kv(t + 1, kn);
        // S^T = K Q^T: element r is key key0(t) + 8(r/4) + 4hi + r%4 against row my_q.
        f32x16 sc;
#pragma unroll
        for (int c = 0; c < NCD; ++c)
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc[c], qreg[c], c == 0 ? f32x16{} : sc, 0, 0, 0);
        const int k0 = key0(t);
        if (k0 + kDecTile - 1 > (CAUSAL ? off + r0 : k_hi - 1) || k0 + kDecTile > k_hi) {
            const int rel = lim - k0 - 4 * hi;
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[r] = 8 * (r >> 2) + (r & 3) > rel ? -INFINITY : sc[r];
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(mx, __builtin_fmaxf(sc[r], sc[r + 1]));
        mx = max_with_partner32(mx) * p.sl2;
        if (__builtin_amdgcn_ballot_w64(mx > m2 + DEC_SLACK)) {
            const float m_new = fmaxf(m2, mx);
            const float alpha = m_new == -INFINITY ? 1.0f : fast_exp2(m2 - m_new);
            lsum *= alpha;
            lbf *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            m2 = m_new;
        }
        // A row that has seen no key yet keeps m2 = -inf; its scores are all -inf here.
        const float neg = m2 == -INFINITY ? 0.0f : -m2;
        bf16x8 pb[2];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float x0 = fast_exp2(fmaf(sc[r], p.sl2, neg));
            const float x1 = fast_exp2(fmaf(sc[r + 1], p.sl2, neg));
            lsum += x0;
            lsum += x1;
            bf16x2 w;
            w[0] = (__bf16)x0;
            w[1] = (__bf16)x1;
            lbf = __builtin_amdgcn_fdot2_f32_bf16(w, ones, lbf, false);
            pb[r / 8][r % 8] = w[0];
            pb[r / 8][r % 8 + 1] = w[1];
        }
        // O~^T += V^T P^T over the tile's two 16-key chunks
        const FA_LDS char* vt = vw + (t & 1) * VT;
#pragma unroll
        for (int j = 0; j < 2 * DB; ++j)
            oacc[j % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand<D, kDecTile>(vt, vbase, j),
                                                                  pb[j / DB], oacc[j % DB], 0, 0, 0);
    };
    bf16x8 ka[NCD], kb[NCD];
    if (nt_w > 0) load_kv(0, ka);
    for (int t = 0; t < nt_w; t += 2) {
        tile(t, ka, kb);
        if (t + 1 < nt_w) tile(t + 1, kb, ka);
    }

    // ---- merge the four waves through LDS (reusing the V buffers)
    __syncthreads();
    float* const om = (float*)lds;                                  // [wave][row][D]
    float* const sm = om + kDecNW * 32 * D;                         // [wave][row][m2, l, lb]
    const float ltot = add_with_partner32(lsum);
    const float lbtot = add_with_partner32(lbf);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *(f32x4*)(om + (wave * 32 + l32) * D + 32 * db + 8 * g + 4 * hi) =
                f32x4{oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
    if (hi == 0) {
        sm[(wave * 32 + l32) * 3 + 0] = m2;
        sm[(wave * 32 + l32) * 3 + 1] = ltot;
        sm[(wave * 32 + l32) * 3 + 2] = lbtot;
    }
    __syncthreads();

    // thread -> (row, D/8 columns)
    constexpr int COLS = D / 8;
    const int row = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * COLS;
    const int qi = r0 + row;
    float mrow = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecNW; ++w) mrow = fmaxf(mrow, sm[(w * 32 + row) * 3]);
    float lrow = 0.0f, lbrow = 0.0f, a[kDecNW];
#pragma unroll
    for (int w = 0; w < kDecNW; ++w) {
        const float mw = sm[(w * 32 + row) * 3];
        a[w] = mw == -INFINITY ? 0.0f : fast_exp2(mw - mrow);
        lrow += a[w] * sm[(w * 32 + row) * 3 + 1];
        lbrow += a[w] * sm[(w * 32 + row) * 3 + 2];
    }
    const bool empty = mrow == -INFINITY;                           // no visible key in this chunk
    const float inv = empty ? 0.0f : 1.0f / lbrow;
    const float lse_row = empty ? -INFINITY : (mrow + fast_log2(lrow)) * kLn2;
    if (qi < Nq) {
        float acc[COLS];
#pragma unroll
        for (int c = 0; c < COLS; ++c) acc[c] = 0.0f;
#pragma unroll
        for (int w = 0; w < kDecNW; ++w)
#pragma unroll
            for (int c = 0; c < COLS; c += 4) {
                const f32x4 x = *(const f32x4*)(om + (w * 32 + row) * D + c0 + c);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[c + e] = fmaf(a[w], x[e], acc[c + e]);
            }
        if (p.S == 1) {
            __bf16* orow = p.o + ((size_t)bh * Nq + qi) * D + c0;
#pragma unroll
            for (int c = 0; c < COLS; c += 8) {
                bf16x8 w;
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e] = (__bf16)(acc[c + e] * inv);
                *(bf16x8*)(orow + c) = w;
            }
            if ((threadIdx.x & 7) == 0) p.lse[(size_t)bh * Nq + qi] = lse_row;
        } else {
            float* orow = p.o_part + (((size_t)bh * p.S + s) * Nq + qi) * D + c0;
#pragma unroll
            for (int c = 0; c < COLS; c += 4)
                *(f32x4*)(orow + c) = f32x4{acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
            if ((threadIdx.x & 7) == 0) p.lse_part[((size_t)bh * p.S + s) * Nq + qi] = lse_row;
        }
    }
}

// One wave per query row: combine the S chunk results of that row.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p, int rows) {
    constexpr int PER = D / 64;       // columns per lane
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);          // bh * Nq + i
    if (row >= rows) return;
    const int bh = row / p.Nq, qi = row - bh * p.Nq;
    const float* lp = p.lse_part + (size_t)bh * p.S * p.Nq + qi;
    float m = -INFINITY;
    for (int s = 0; s < p.S; ++s) m = fmaxf(m, lp[(size_t)s * p.Nq]);
    float l = 0.0f, acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
    for (int s = 0; s < p.S; ++s) {
        const float ls = lp[(size_t)s * p.Nq];
        if (ls == -INFINITY) continue;                               // chunk with no visible key
        const float w = fast_exp2((ls - m) * kLog2e);
        l += w;
        const float* op = p.o_part + (((size_t)bh * p.S + s) * p.Nq + qi) * D + lane * PER;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, op[e], acc[e]);
    }
    // A row that sees no key at all (paged, causal, sequence shorter than Nq)
    // gets O = 0 and LSE = -inf.
    const float inv = m == -INFINITY ? 0.0f : 1.0f / l;
    __bf16* orow = p.o + (size_t)row * D + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) orow[e] = (__bf16)(acc[e] * inv);
    if (lane == 0) p.lse[row] = m == -INFINITY ? -INFINITY : m + fast_log2(l) * kLn2;
}

template <int D, bool CAUSAL, bool PAGED>
hipError_t launch(const DecodeArgs& a, hipStream_t st) {
    const DecodeSplit sp = decode_split(a.B, a.H, a.Nq, PAGED ? a.max_blocks * a.page : a.Nk);
    DecodeParams p{};
    p.q = (const __bf16*)a.q;
    p.k = (const __bf16*)a.k;
    p.v = (const __bf16*)a.v;
    p.o = (__bf16*)a.o;
    p.lse = a.lse;
    p.o_part = a.o_part;
    p.lse_part = a.lse_part;
    p.block_table = a.block_table;
    p.seq_lens = a.seq_lens;
    p.Nq = a.Nq;
    p.Nk = a.Nk;
    p.H = a.H;
    p.max_blocks = a.max_blocks;
    p.page = a.page;
    p.num_pages = a.num_pages;
    p.nrb = sp.nrb;
    p.S = sp.S;
    p.chunk = sp.chunk;
    p.sl2 = a.scale * kLog2e;
    const int heads = a.B * a.H;
    hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL, PAGED>), dim3(heads * sp.nrb * sp.S), dim3(kDecNW * 64),
                       0, st, p);
    if (sp.S > 1) {
        const int rows = heads * a.Nq;
        hipLaunchKernelGGL(decode_merge_kernel<D>, dim3((rows + 3) / 4), dim3(256), 0, st, p, rows);
    }
    return hipGetLastError();
}

}  // namespace

// Workgroups the key split aims at: two per CU, all resident at once (one
// round). Measured on the decode workloads: 256 and 512 stream at 70-74% of
// 8 TB/s, 1024 at 64-70%, 4096 at 48-64% (more partial results, more merge).
#ifndef FA_DEC_TARGET
#define FA_DEC_TARGET 512
#endif

DecodeSplit decode_split(int B, int H, int Nq, int Nk) {
    // Chunks of whole 128-key steps.
    constexpr long long kTargetWorkgroups = FA_DEC_TARGET;
    DecodeSplit sp;
    sp.nrb = (Nq + 31) / 32;
    const long long base = (long long)B * H * sp.nrb;
    const int max_s = (Nk + kDecChunk - 1) / kDecChunk;
    long long want = (kTargetWorkgroups + base - 1) / base;
    if (want < 1) want = 1;
    if (want > max_s) want = max_s;
    const int per = (int)((Nk + want - 1) / want);
    sp.chunk = (per + kDecChunk - 1) / kDecChunk * kDecChunk;
    sp.S = (Nk + sp.chunk - 1) / sp.chunk;
    return sp;
}

hipError_t launch_fwd_decode_bf16(const DecodeArgs& a, hipStream_t st) {
    if (a.block_table) {
        if (a.d == 64) return a.causal ? launch<64, true, true>(a, st) : launch<64, false, true>(a, st);
        return a.causal ? launch<128, true, true>(a, st) : launch<128, false, true>(a, st);
    }
    if (a.d == 64) return a.causal ? launch<64, true, false>(a, st) : launch<64, false, false>(a, st);
    return a.causal ? launch<128, true, false>(a, st) : launch<128, false, false>(a, st);
}

}  // namespace fa
