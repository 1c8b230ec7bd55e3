// Split-K paged decode on the matrix cores (gfx950 MFMA) for query tiles of
// 16 rows or more: speculative verification, where each sequence brings Tq
// new query tokens (8 target tokens per verification step on the
// vllm-sm12x-nvfp4-dflash2 page, "What makes this stack different") and the
// G query heads of a kv head times the Tq tokens form G*Tq rows that share
// every key and value row. The vllm-sm70 page ("Why", Attention bullet) runs
// such speculative positions as a virtual batch of one-token decodes; here
// all rows of a kv head are MFMA operands, so the KV is read once.
//
// Workgroup = 4 waves for one split-K partition of one kv head g of one
// sequence b and up to 16*NT rows r = t*G + h' (query token t, head g*G + h');
// row r sees keys 0 .. L_b - Tq + t (causal inside the Tq new tokens).
// Per 16-token KV block:
//  - each wave moves 4 rows of the block's K and V tiles (16-byte loads of
//    whole-row runs) through a 3-block register ring into row-major LDS tiles
//    (double-buffered, rows padded against bank conflicts);
//  - wave w < NT owns row tile w: its queries stay in registers as the B
//    operands of S^T = K Q^T (v_mfma_f32_16x16x32 bf16 / f16, K operands read
//    from LDS), it runs the softmax and writes 16-bit weights to LDS. The S^T
//    result layout (lane l: tokens 4*(l/16)+i of row l%16) is exactly the
//    A-operand layout of the PV product, so no shuffle is needed;
//  - every wave accumulates O[row][d] += P[row][token] V[token][d]
//    (v_mfma_f32_16x16x32 bf16 / f16 over a block pair's 32 tokens) for its
//    quarter of the output dims; the V operand (8 tokens of one dim per lane)
//    comes from the transposing LDS reads of gfx950: the 16-bit one (bf16,
//    NVFP4 widened to f16) or the 8-bit one (int8 / FP8 codes, both blocks'
//    tokens in one read).
// The scores of block j+1 and the PV of block j share one iteration, so one
// workgroup barrier per block covers the staged tiles and the weights.
// int8 caches: codes become f16 (1024 + code + 128) by a byte permute, queries
// are scaled into f16 by a power of two, probabilities times the value scale
// are f16; the code bias is removed once per row. FP8 (OCP E4M3) caches: keys
// are widened to bf16 (exact) against bf16 queries, values to f16 (exact)
// against f16 probabilities times the value scale. Softmax: log2 units against a
// per-row reference raised only when beaten by 2^8.
#include <type_traits>
#include <utility>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kW = 4;  // waves per workgroup
constexpr uint32_t kMagic = 0x64646464u;
constexpr float kCodeBias = 1152.0f;  // 1024 + 128

__device__ __forceinline__ uint32_t f16pair_lo(uint32_t u) { return __builtin_amdgcn_perm(kMagic, u, 0x04010400u); }
__device__ __forceinline__ uint32_t f16pair_hi(uint32_t u) { return __builtin_amdgcn_perm(kMagic, u, 0x04030402u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

__device__ __forceinline__ float f16lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// 4 x bf16 in LDS, the operand type of the transposing LDS read
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_gcc;
typedef __attribute__((address_space(3))) bf16x4_gcc lds_bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2_gcc;
typedef __attribute__((address_space(3))) i32x2_gcc lds_i32x2;

template <int I>
using ic = std::integral_constant<int, I>;

// f(ic<0>{}), f(ic<1>{}), ..., f(ic<N-1>{})
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(ic<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace

// Two workgroups per CU (two waves per SIMD) need at most 256 registers per
// lane of the unified VGPR/AGPR file. At D = 256 the instances with four row
// tiles, or three with fp32 queries, exceed that unless bounded, and fit
// without spills when bounded; the bf16, int8 and fp8 ones with four tiles
// and fp32 queries would spill and keep one workgroup per CU.
template <int KVT, int D, int NT, int QS>
constexpr int mfma_min_waves() {
    return (D == 256 && NT + QS >= 5 && !(NT == 4 && QS == 2 && KVT != KV_NVFP4)) ? 2 : 1;
}

template <int KVT, int D, int NT, int QS>
__global__ __launch_bounds__(64 * kW, (mfma_min_waves<KVT, D, NT, QS>())) void decode_mfma_kernel(DecodeParams p) {
    static_assert(KVT == KV_BF16 || KVT == KV_I8 || KVT == KV_FP8 || KVT == KV_NVFP4, "bf16, int8, fp8 or nvfp4");
    static_assert(NT >= 1 && NT <= kW, "one row tile per wave");
    constexpr bool I8 = KVT == KV_I8;
    constexpr bool F8 = KVT == KV_FP8;
    constexpr bool F4 = KVT == KV_NVFP4;
    constexpr bool QNT = I8 || F8 || F4;  // codes with a per-(token, kv head) scale; f16 PV
    constexpr int E = Elt<KVT>::bytes;
    constexpr int KS = D / 32;                 // k-steps of the score product
    constexpr int DW = D / kW;                 // output dims per wave
    constexpr int NDT = DW / 16;               // 16-wide output tiles per wave
    constexpr int NQ = QS == 2 ? 2 : 1;        // query parts (hi, lo) for fp32 queries
    // block pairs in flight per wave (register ring depth); at least 2, as the
    // keys of pair i + 1 are staged while pair i's values are
    constexpr int S2 = 2;
    static_assert(S2 == 2, "the unmasked-pair argument of the block loop assumes two pairs per check");
    // Global loads: wave w moves rows 4w .. 4w+3 of a block's K and V tiles,
    // as runs of whole rows (RB bytes each), GB bytes per lane and load
    constexpr int RB = F4 ? D / 2 : D * E;           // code bytes of one cache row
    constexpr int RBQ = kv_code_row_bytes<KVT>(D);   // row stride within a block (code bytes)
    constexpr int GB = RB / 16 >= 16 ? 16 : RB / 16;  // bytes per lane per load
    constexpr int NL = RB / 16 / GB;                 // loads per lane per tile
    // LDS tiles, row-major; keys as 16-bit elements (int8 codes widened to
    // f16), values as stored; the row pads spread the operand reads over banks
    constexpr int KRS = 2 * D + 16;  // bytes per staged key row
    constexpr int VRS = (F4 ? 2 * D : RB) + 32;  // bytes per staged value row (nvfp4: f16)
    // int8 / FP8: 16 bytes between the pair's two value blocks, so that the
    // 8-bit transposing reads of PV (4 rows of each block per 16 lanes) meet
    // no bank twice
    constexpr int VBP = (I8 || F8) ? 16 : 0;

    // [stage][block of the pair] ...
    __shared__ __align__(16) unsigned char kst[2][2][kBlockSize][KRS];  // staged keys
    __shared__ __align__(16) unsigned char vst[2][2][kBlockSize * VRS + VBP];  // staged values, rows of VRS bytes
    __shared__ __align__(16) u32x4 pst[2][NT][64];  // weights of a pair's 32 tokens (A operands of PV)
    __shared__ __align__(16) float sst[2][2][32];   // int8: key then value scales of a block's tokens
    __shared__ __align__(16) float ast[2][NT][16];  // per-row rescale factors
    __shared__ int araise[2][NT];                   // whether a tile's rows were rescaled
    __shared__ float fin[2][NT][16];                // epilogue: 1/l and code bias per row
    __shared__ float red[kW];

    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, lg = lane >> 4;
    const bool owner = wv < NT;  // computes the scores of row tile wv
    auto vrow = [&](int stage, int h, int row) { return &vst[stage][h][row * VRS]; };

    int wg = blockIdx.x;
    const int part = wg % p.NP;
    wg /= p.NP;
    const int rc = wg % p.nchunk;
    wg /= p.nchunk;
    const int g = wg % p.Hkv;
    const int b = wg / p.Hkv;

    // Row r of the row set: sequence b + r / (Tq G) (stacked rows span the
    // batch, whose grid coordinate b is then 0), token (r / G) % Tq, head
    // g G + r % G.
    const int G = p.G, Tq = p.Tq, TG = G * Tq;
    const int R = p.stacked ? p.B * TG : TG;
    const int row0 = rc * 16 * NT;
    const int rlast = min(R, row0 + 16 * NT) - 1;  // one sequence: largest t is in the last row
    // keys of the row set: a sequence's own from kv_begin on (causal end
    // L - Tq + t), or the shared list's first prefix_len, visible to all rows
    // per-head tables: row b Hkv + g of the table and lengths
    const int hrow = p.head_tables ? b * p.Hkv + g : b;
    const int L = p.stacked ? p.prefix_len : p.seq_lens[hrow] - p.kv_begin;
    const int n_chunk = p.stacked ? L : L - Tq + rlast / G + 1;
    const int start = part * p.P;
    const int64_t wpart = p.part_base + part;  // workspace partition

    // flat (b, t, h) row id of row r: with u = r / G, b Tq + u is the
    // sequence times Tq plus the token, also for stacked rows (b = 0 there,
    // u = sequence * Tq + token)
    auto row_out = [&](int r) -> int64_t {
        const int u = r / G, hh = r % G;
        return ((int64_t)b * Tq + u) * p.Hq + g * G + hh;
    };

    if (start >= n_chunk) {
        if (p.np_stride == 1) {
            for (int r = row0; r <= rlast; ++r) {
                const int64_t rid = row_out(r);
                for (int d = threadIdx.x; d < D; d += 64 * kW) {
                    if (p.out_bf16)
                        reinterpret_cast<uint16_t*>(p.out)[rid * D + d] = 0;
                    else
                        reinterpret_cast<float*>(p.out)[rid * D + d] = 0.0f;
                }
                if (p.lse != nullptr && threadIdx.x == 0) p.lse[rid] = -INFINITY;
            }
        } else if (p.fill_empty) {
            for (int r = row0 + (int)threadIdx.x; r <= rlast; r += 64 * kW)
                p.ws_lse[row_out(r) * p.np_stride + wpart] = -INFINITY;
        }
        return;
    }
    const int end = min(start + p.P, n_chunk);

    // ---------------------------------------------------------------- queries
    // owner wave: B operand (row 16*wv + l16, dims 32 ks + 8 lg .. +7) per k-step
    const int myrow = row0 + 16 * wv + l16;
    const bool row_ok = owner && myrow < R;
    float qx[KS][8];
    float qmax = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (row_ok) {
            const int64_t off = row_out(myrow) * D + 32 * ks + 8 * lg;
            if constexpr (QS == 1) {
                Raw<16> raw;
                load_raw<16>(raw, reinterpret_cast<const uint16_t*>(p.q) + off);
#pragma unroll
                for (int k = 0; k < 8; ++k) qx[ks][k] = elem_f32<KV_BF16>(raw, k);
            } else {
                Raw<32> raw;
                load_raw<32>(raw, reinterpret_cast<const float*>(p.q) + off);
#pragma unroll
                for (int k = 0; k < 8; ++k) qx[ks][k] = elem_f32<KV_F32>(raw, k);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) qx[ks][k] = 0.0f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) qmax = fmaxf(qmax, fabsf(qx[ks][k]));
    }
    float qscale = 1.0f, qpost = p.qk_scale_log2;
    if constexpr (I8) {
        // one power of two for the workgroup puts max|q| in [2^14, 2^15)
        qmax = wave_max(qmax);
        if (lane == 0) red[wv] = qmax;
        __syncthreads();
        qmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        const int e2 = qmax > 0.0f ? 14 - ilogbf(qmax) : 0;
        qscale = ldexpf(1.0f, e2);
        qpost = ldexpf(p.qk_scale_log2, -e2);
    }
    u32x4 qreg[NQ][KS];
    float corr = 0.0f;  // int8: 1152 * sum_d q'[row] of the lane's row (after the reduction below)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float x0 = qx[ks][2 * k] * qscale, x1 = qx[ks][2 * k + 1] * qscale;
            if constexpr (I8) {
                hi[k] = pack_f16x2(x0, x1);
                lo[k] = pack_f16x2(x0 - f16lo(hi[k]), x1 - f16hi(hi[k]));
                corr += f16lo(hi[k]) + f16hi(hi[k]);
                if constexpr (QS == 2) corr += f16lo(lo[k]) + f16hi(lo[k]);
            } else {
                hi[k] = pack_bf16x2(x0, x1);
                lo[k] = pack_bf16x2(x0 - bf16_to_f32((uint16_t)hi[k]), x1 - bf16_to_f32((uint16_t)(hi[k] >> 16)));
            }
        }
        qreg[0][ks] = u32x4{hi[0], hi[1], hi[2], hi[3]};
        if constexpr (QS == 2) qreg[NQ - 1][ks] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    }
    if constexpr (I8) {
        corr += __shfl_xor(corr, 16);
        corr += __shfl_xor(corr, 32);
        corr *= kCodeBias;
    }

    // ------------------------------------------------------- softmax state
    // owner, score layout: lane holds row myrow, tokens 4*lg + i of a block
    const int nvis = !row_ok ? 0 : p.stacked ? end : min(end, L - Tq + myrow / G + 1);
    float mref = -INFINITY, lpart = 0.0f, spart = 0.0f;
    // output layout: lane holds rows 16*t + 4*lg + i, dim wv*DW + 16*nd + l16
    f32x4 o[NT][NDT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int nd = 0; nd < NDT; ++nd) o[t][nd] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int32_t* table =
        p.stacked ? p.block_table : p.block_table + (int64_t)hrow * p.max_blocks + p.kv_begin / kBlockSize;
    const int64_t tok_stride = (int64_t)p.Hkv * RBQ;
    const int64_t blk_bytes = kBlockSize * (int64_t)p.Hkv * kv_row_bytes<KVT>(D);  // nvfp4: + scale planes
    const char* kbase = reinterpret_cast<const char*>(p.k_cache) + (int64_t)g * RBQ;
    const char* vbase = reinterpret_cast<const char*>(p.v_cache) + (int64_t)g * RBQ;
    // nvfp4: this head's scale plane in a block; byte 16 k + 4 r + q holds the
    // scale of elements 16 k .. 16 k + 15 of token 4 q + r
    const int64_t plane = kBlockSize * tok_stride + (int64_t)g * D - (int64_t)g * RBQ;  // from kbase
    const int j0 = start / kBlockSize, jend = (end + kBlockSize - 1) / kBlockSize;
    // physical block of logical block j (clamped to the partition)
    auto phys_of = [&](int j) -> int64_t { return (int64_t)table[j < jend ? j : jend - 1]; };
    // Inside the block loop the table entries go through the vector memory
    // path (the workgroup barrier's fences keep the compiler from scalar
    // loads there), and loads complete in issue order: an entry is therefore
    // requested one iteration before it is used, ahead of that iteration's
    // K/V prefetches, so waiting for it never drains them.

    // int8 / fp8: probabilities times value scales are kept below 2^15 (f16) by 2^vsh
    float vsh = 1.0f, vsh_inv = 1.0f;
    if constexpr (QNT) {
        float vmax = 0.0f;
        for (int j = j0 + (threadIdx.x >> 4); j < jend; j += 4 * kW) {
            const int pos = j * kBlockSize + l16;
            if (pos < end) vmax = fmaxf(vmax, p.v_scale[((int64_t)table[j] * p.Hkv + g) * kBlockSize + l16]);
        }
        vmax = wave_max(vmax);
        __syncthreads();
        if (lane == 0) red[wv] = vmax;
        __syncthreads();
        vmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        const int e2 = vmax > 0.0f ? 6 - ilogbf(vmax) : 0;
        vsh = ldexpf(1.0f, e2);
        vsh_inv = ldexpf(1.0f, -e2);
    }

    // ---------------------------------------------------------- pipeline
    // Blocks go in pairs: iteration i takes the 32 tokens of blocks
    // jp = j0 + 2 i and jp + 1 (the PV contracts 32 tokens per MFMA). Register
    // ring of S2 pairs: pair i (this wave's rows of both blocks' K and V tiles,
    // plus (int8) their scales, all requested together: a load issued later
    // would make its wait drain the prefetches) lives in slot i % S2.
    // Iteration i stages K(pair i + 1) (wave 0 also its scales) and V(pair i)
    // in LDS and then requests pair i + S2 into V(pair i)'s slot.
    const int npair = (jend - j0 + 1) / 2;
    struct Blk {
        Raw<GB> k[NL], v[NL];
        // nvfp4: the scales of the lane's row (4 q + r, r = lane / 16) for
        // q = 0..3 in the 16-element block of its 2 GB elements; q is the wave
        Raw<4> ksw, vsw;
        float sc;  // int8: lane l < 16 the key scale, 16 <= l < 32 the value scale of token l % 16
    };
    Blk ring[S2][2];
    // lane's share of a tile: load i covers bytes x = (i * 64 + lane) * GB of
    // the wave's four rows, i.e. row 4 * wv + x / RB, byte x % RB
    auto row_of = [&](int i) { return 4 * wv + ((i * 64 + lane) * GB) / RB; };
    auto col_of = [&](int i) { return ((i * 64 + lane) * GB) % RB; };
    auto load_blk = [&](Blk& dst, int64_t ph) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int64_t off = ph * blk_bytes + row_of(i) * tok_stride + col_of(i);
            load_raw<GB, true>(dst.k[i], kbase + off);
            load_raw<GB, true>(dst.v[i], vbase + off);
        }
        if constexpr (F4) {
            static_assert(NL == 1, "nvfp4: one load per lane per tile");
            const int64_t sb = ph * blk_bytes + plane + 16 * (col_of(0) / 8) + 4 * (row_of(0) & 3);
            load_raw<4, true>(dst.ksw, kbase + sb);
            load_raw<4, true>(dst.vsw, vbase + sb);
        }
        dst.sc = 1.0f;
        if constexpr (QNT) {
            // one load for the block's 32 scales (lanes 32..63 repeat 0..31)
            const float* src = (lane & 16) ? p.v_scale : p.k_scale;
            dst.sc = src[(ph * p.Hkv + g) * kBlockSize + l16];
        }
    };
    auto store_k = [&](const Blk& src, int stage, int h) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            unsigned char* dst = &kst[stage][h][row_of(i)][col_of(i) * (2 / E)];
            if constexpr (I8) {
                // codes c -> f16 (1024 + c + 128), two output bytes per code
                uint32_t f[GB / 2];
#pragma unroll
                for (int w = 0; w < GB / 4; ++w) {
                    const uint32_t u = src.k[i].w[w] ^ 0x80808080u;
                    f[2 * w] = f16pair_lo(u);
                    f[2 * w + 1] = f16pair_hi(u);
                }
                if constexpr (GB == 16) {
                    reinterpret_cast<u32x4*>(dst)[0] = u32x4{f[0], f[1], f[2], f[3]};
                    reinterpret_cast<u32x4*>(dst)[1] = u32x4{f[4], f[5], f[6], f[7]};
                } else if constexpr (GB == 8) {
                    *reinterpret_cast<u32x4*>(dst) = u32x4{f[0], f[1], f[2], f[3]};
                } else {
                    *reinterpret_cast<u32x2*>(dst) = u32x2{f[0], f[1]};
                }
            } else if constexpr (F4) {
                // E2M1 code pairs times the block scale -> bf16 (exact: at most
                // 6 significant bits), four output bytes per code byte
                const float sc = fp8_value(src.ksw.w[0] >> (8 * wv));
                uint32_t f[GB];
#pragma unroll
                for (int b2 = 0; b2 < GB; ++b2) {
                    const uint32_t wd = src.k[i].w[b2 / 4];
                    const pa_f32x2 e = (b2 & 3) == 0 ? fp4x2_to_f32<0>(wd) : (b2 & 3) == 1 ? fp4x2_to_f32<1>(wd)
                                       : (b2 & 3) == 2 ? fp4x2_to_f32<2>(wd) : fp4x2_to_f32<3>(wd);
                    f[b2] = pack_bf16_rne(e.x * sc, e.y * sc);
                }
                unsigned char* d4 = &kst[stage][h][row_of(i)][col_of(i) * 4];
                if constexpr (GB == 8) {
                    reinterpret_cast<u32x4*>(d4)[0] = u32x4{f[0], f[1], f[2], f[3]};
                    reinterpret_cast<u32x4*>(d4)[1] = u32x4{f[4], f[5], f[6], f[7]};
                } else if constexpr (GB == 4) {
                    *reinterpret_cast<u32x4*>(d4) = u32x4{f[0], f[1], f[2], f[3]};
                } else {
                    *reinterpret_cast<u32x2*>(d4) = u32x2{f[0], f[1]};
                }
            } else if constexpr (F8) {
                // E4M3 codes -> bf16 (exact), two output bytes per code
                uint32_t f[GB / 2];
#pragma unroll
                for (int w = 0; w < GB / 4; ++w) {
                    const pa_f32x2 lo = fp8x2_to_f32<false>(src.k[i].w[w]);
                    const pa_f32x2 hi = fp8x2_to_f32<true>(src.k[i].w[w]);
                    f[2 * w] = pack_bf16_rne(lo.x, lo.y);
                    f[2 * w + 1] = pack_bf16_rne(hi.x, hi.y);
                }
                if constexpr (GB == 16) {
                    reinterpret_cast<u32x4*>(dst)[0] = u32x4{f[0], f[1], f[2], f[3]};
                    reinterpret_cast<u32x4*>(dst)[1] = u32x4{f[4], f[5], f[6], f[7]};
                } else if constexpr (GB == 8) {
                    *reinterpret_cast<u32x4*>(dst) = u32x4{f[0], f[1], f[2], f[3]};
                } else {
                    *reinterpret_cast<u32x2*>(dst) = u32x2{f[0], f[1]};
                }
            } else {
                if constexpr (GB == 16)
                    *reinterpret_cast<u32x4*>(dst) = u32x4{src.k[i].w[0], src.k[i].w[1], src.k[i].w[2], src.k[i].w[3]};
                else if constexpr (GB == 8)
                    *reinterpret_cast<u32x2*>(dst) = u32x2{src.k[i].w[0], src.k[i].w[1]};
                else
                    *reinterpret_cast<uint32_t*>(dst) = src.k[i].w[0];
            }
        }
        if (QNT && wv == 0 && lane < 32) sst[stage][h][lane] = src.sc;
    };
    auto store_v = [&](const Blk& src, int stage, int h) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            if constexpr (F4) {
                // E2M1 code pairs times the block scale -> f16 (exact), read
                // back by the 16-bit transposing LDS read as bf16 tiles are
                const float sc = fp8_value(src.vsw.w[0] >> (8 * wv));
                uint32_t f[GB];
#pragma unroll
                for (int b2 = 0; b2 < GB; ++b2) {
                    const uint32_t wd = src.v[i].w[b2 / 4];
                    const pa_f32x2 e = (b2 & 3) == 0 ? fp4x2_to_f32<0>(wd) : (b2 & 3) == 1 ? fp4x2_to_f32<1>(wd)
                                       : (b2 & 3) == 2 ? fp4x2_to_f32<2>(wd) : fp4x2_to_f32<3>(wd);
                    f[b2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(e.x * sc, e.y * sc));
                }
                unsigned char* d4 = vrow(stage, h, row_of(i)) + col_of(i) * 4;
                if constexpr (GB == 8) {
                    reinterpret_cast<u32x4*>(d4)[0] = u32x4{f[0], f[1], f[2], f[3]};
                    reinterpret_cast<u32x4*>(d4)[1] = u32x4{f[4], f[5], f[6], f[7]};
                } else if constexpr (GB == 4) {
                    *reinterpret_cast<u32x4*>(d4) = u32x4{f[0], f[1], f[2], f[3]};
                } else {
                    *reinterpret_cast<u32x2*>(d4) = u32x2{f[0], f[1]};
                }
                continue;
            }
            unsigned char* dst = vrow(stage, h, row_of(i)) + col_of(i);
            if constexpr (GB == 16)
                *reinterpret_cast<u32x4*>(dst) = u32x4{src.v[i].w[0], src.v[i].w[1], src.v[i].w[2], src.v[i].w[3]};
            else if constexpr (GB == 8)
                *reinterpret_cast<u32x2*>(dst) = u32x2{src.v[i].w[0], src.v[i].w[1]};
            else
                *reinterpret_cast<uint32_t*>(dst) = src.v[i].w[0];
        }
    };
    // int8 / FP8 V operands: lane 2 r8 + c8 of a 16-lane group names row r8 of
    // the 8-bit transposing read
    const int r8 = l16 >> 1, c8 = l16 & 1;

    // scores, softmax and weights of pair i into LDS stage i % 2 (owners only).
    // Lane l ends with row l16's tokens 4 lg + 0..3 of both blocks, which is
    // the A-operand layout of a 16x16x32 PV product whose k index 8 lg + e
    // means token 4 lg + e % 4 of block e / 4 of the pair.
    // INNER: the pair lies wholly before the partition's end and before every
    // valid row's causal limit, so only invalid rows need masking
    auto scores = [&](int i, auto inner) {
        // bf16: the scheduler's MFMA / exp interleaving for the scores (measured)
        if constexpr (KVT == KV_BF16) __builtin_amdgcn_iglp_opt(3);
        constexpr bool INNER = decltype(inner)::value;
        const int stage = i & 1;
        const int jp = j0 + 2 * i;
        // int8: key and value scales of the lane's 4 tokens in each block
        f32x4 kraw[2], vraw[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            kraw[h] = f32x4{1.0f, 1.0f, 1.0f, 1.0f};
            vraw[h] = kraw[h];
            if constexpr (QNT) {
                kraw[h] = *reinterpret_cast<const f32x4*>(&sst[stage][h][4 * lg]);
                vraw[h] = *reinterpret_cast<const f32x4*>(&sst[stage][h][16 + 4 * lg]);
            }
        }
        // all K operands requested at once (token l16, 16-bit elements
        // 32 ks + 8 lg .. + 7), then four independent accumulation chains
        u32x4 a[2][KS];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                a[h][ks] = *reinterpret_cast<const u32x4*>(&kst[stage][h][l16][(32 * ks + 8 * lg) * 2]);
        f32x4 acc[2][2];
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[h][0] = acc[h][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int q2 = 0; q2 < NQ; ++q2) {
                    f32x4& c = acc[h][ks & 1];
                    if constexpr (I8)
                        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[h][ks]),
                                                                   __builtin_bit_cast(f16x8, qreg[q2][ks]), c, 0, 0, 0);
                    else
                        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[h][ks]),
                                                                    __builtin_bit_cast(bf16x8, qreg[q2][ks]), c, 0, 0, 0);
                }
            }
        }
        float sc[2][4];
        bool raise = false;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f32x4 s = acc[h][0] + acc[h][1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = INNER ? row_ok : (jp + h) * kBlockSize + 4 * lg + e < nvis;
                float ksc = qpost;
                if constexpr (QNT) ksc *= kraw[h][e];
                sc[h][e] = ok ? (s[e] - corr) * ksc : -INFINITY;
                raise |= sc[h][e] > mref + 8.0f;
            }
        }
        const bool any = __builtin_amdgcn_ballot_w64(raise) != 0;
        if (any) {
            float bm = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                             fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
            bm = fmaxf(bm, __shfl_xor(bm, 16));
            bm = fmaxf(bm, __shfl_xor(bm, 32));
            const float mn = fmaxf(mref, bm);
            const float base = mn == -INFINITY ? 0.0f : mn;
            const float alpha = exp2_guarded(mref - base);
            mref = mn;
            lpart *= alpha;
            spart *= alpha;
            if (lg == 0) ast[stage][wv][l16] = alpha;
        }
        if (lane == 0) araise[stage][wv] = any ? 1 : 0;
        const float base = mref == -INFINITY ? 0.0f : mref;
        float pr[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                pr[h][e] = exp2_weight(sc[h][e] - base);  // sc = -inf gives 0
                lpart += pr[h][e];
            }
        u32x4 pa;
        if constexpr (QNT) {
            float ph2[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = INNER || (jp + h) * kBlockSize + 4 * lg + e < end;
                    ph2[h][e] = (float)(_Float16)(ok ? pr[h][e] * vraw[h][e] * vsh : 0.0f);
                    spart += ph2[h][e];
                }
            pa = u32x4{pack_f16x2(ph2[0][0], ph2[0][1]), pack_f16x2(ph2[0][2], ph2[0][3]),
                       pack_f16x2(ph2[1][0], ph2[1][1]), pack_f16x2(ph2[1][2], ph2[1][3])};
        } else {
            pa = u32x4{pack_bf16_rne(pr[0][0], pr[0][1]), pack_bf16_rne(pr[0][2], pr[0][3]),
                       pack_bf16_rne(pr[1][0], pr[1][1]), pack_bf16_rne(pr[1][2], pr[1][3])};
            // sum of the rounded weights: the output is normalised by it, so it
            // stays a convex combination of value rows (l keeps the exact ones)
#pragma unroll
            for (int w = 0; w < 4; ++w) spart += bf16_to_f32((uint16_t)pa[w]) + bf16_to_f32((uint16_t)(pa[w] >> 16));
        }
        pst[stage][wv][lane] = pa;
    };

    // PV of pair i (all waves): weights and values from LDS stage i % 2
    auto values = [&](int i, auto inner) {
        // quantised caches: the scheduler's LDS-read / MFMA interleaving for the PV (measured)
        if constexpr (QNT) __builtin_amdgcn_iglp_opt(0);
        constexpr bool INNER = decltype(inner)::value;
        const int stage = i & 1;
        const int jp = j0 + 2 * i;
        u32x4 bop[NDT];
#pragma unroll
        for (int nd = 0; nd < NDT; ++nd) {
            if constexpr (I8 || F8) {
                // 8-bit transposing LDS read: lane 2 r8 + c8 of a 16-lane
                // group names token 4 lg + r8 % 4 of block r8 / 4 of the pair,
                // dims wv DW + 16 nd + 8 c8 .. + 7; lane i receives dim
                // wv DW + 16 nd + i of the group's 4 tokens of the first block
                // (bytes 0..3) and of the second (bytes 4..7): k index 8 lg + e
                // of the PV product
                const unsigned char* src = vrow(stage, r8 >> 2, 4 * lg + (r8 & 3)) + wv * DW + 16 * nd + 8 * c8;
                const u32x2 raw = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)src));
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    u32x2 w;
                    if constexpr (I8) {
                        const uint32_t tw = raw[h] ^ 0x80808080u;
                        w = u32x2{f16pair_lo(tw), f16pair_hi(tw)};
                    } else {
                        // the 4 tokens' codes of one dim as two exact f16 pairs
                        const pa_f32x2 lo = fp8x2_to_f32<false>(raw[h]), hi = fp8x2_to_f32<true>(raw[h]);
                        w = u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo.x, lo.y)),
                                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(hi.x, hi.y))};
                        const int pos0 = (jp + h) * kBlockSize;
                        if (!INNER && pos0 + kBlockSize > end) {  // tokens past the end may hold NaN codes
                            const int t0 = pos0 + 4 * lg;  // element k is token 4*lg + k
                            w.x = (t0 + 0 < end ? w.x & 0x0000FFFFu : 0u) | (t0 + 1 < end ? w.x & 0xFFFF0000u : 0u);
                            w.y = (t0 + 2 < end ? w.y & 0x0000FFFFu : 0u) | (t0 + 3 < end ? w.y & 0xFFFF0000u : 0u);
                        }
                    }
                    bop[nd][2 * h] = w.x;
                    bop[nd][2 * h + 1] = w.y;
                }
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int pos0 = (jp + h) * kBlockSize;
                    // transposing LDS read: lane 4r + c of a 16-lane group names
                    // row (token) 4 lg + r, dims 4c .. 4c + 3 of the 16-dim tile;
                    // lane i receives dim i of the group's 4 tokens
                    const unsigned char* src =
                        vrow(stage, h, 4 * lg + (l16 >> 2)) + (wv * DW + 16 * nd + 4 * (l16 & 3)) * 2;
                    u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)src));
                    if (!INNER && pos0 + kBlockSize > end) {  // tokens past the end may hold anything
                        const int t0 = pos0 + 4 * lg;  // element k is token 4*lg + k
                        w.x = (t0 + 0 < end ? w.x & 0x0000FFFFu : 0u) | (t0 + 1 < end ? w.x & 0xFFFF0000u : 0u);
                        w.y = (t0 + 2 < end ? w.y & 0x0000FFFFu : 0u) | (t0 + 3 < end ? w.y & 0xFFFF0000u : 0u);
                    }
                    bop[nd][2 * h] = w.x;
                    bop[nd][2 * h + 1] = w.y;
                }
            }
        }
        // every tile's flag, factors and weights requested at once
        int rz[NT];
        f32x4 a4[NT];
        u32x4 pw[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            rz[t] = araise[stage][t];
            a4[t] = *reinterpret_cast<const f32x4*>(&ast[stage][t][4 * lg]);
            pw[t] = pst[stage][t][lane];
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (rz[t]) {
#pragma unroll
                for (int nd = 0; nd < NDT; ++nd) o[t][nd] *= a4[t];
            }
#pragma unroll
            for (int nd = 0; nd < NDT; ++nd) {
                if constexpr (QNT)
                    o[t][nd] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(f16x8, pw[t]), __builtin_bit_cast(f16x8, bop[nd]), o[t][nd], 0, 0, 0);
                else
                    o[t][nd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, pw[t]), __builtin_bit_cast(bf16x8, bop[nd]), o[t][nd], 0, 0, 0);
            }
        }
    };

    // prologue: pairs 0 .. S2 - 1 requested, K(pair 0) staged, scores of pair
    // 0 done. Unconditional (blocks past the partition re-read its last one,
    // masked by position): the loop's wait counts assume all S2 in flight.
    {
#pragma unroll
        for (int x = 0; x < S2; ++x)
#pragma unroll
            for (int h = 0; h < 2; ++h) load_blk(ring[x][h], phys_of(j0 + 2 * x + h));
        store_k(ring[0][0], 0, 0);
        store_k(ring[0][1], 0, 1);
        __syncthreads();
        if (owner) scores(0, std::false_type{});
    }
    // physical blocks of pair i + S2 at iteration i, not yet uniform
    int tp0 = (int)phys_of(j0 + 2 * S2), tp1 = (int)phys_of(j0 + 2 * S2 + 1);
    // iteration i: stage K(pair i+1) and V(pair i), barrier, scores of pair
    // i+1, PV of pair i. FULL: the pair this iteration requests starts inside
    // the partition. The main loop runs S2 = 2 iterations per check of
    // i + 2 S2 <= npair, so in both of them pair i ends at least 3 blocks
    // before the partition's last block (its values need no mask), and in the
    // first (X = 0) so does pair i + 1, which then also lies inside every
    // valid row's causal range (at most Tq - 1 <= 15 tokens short of the end):
    // its scores need no mask either. In the second, pair i + 1 may reach the
    // block before the last, within that causal margin.
    // issue priorities of the other phases per cache type (measured): bf16
    // stores its staged tiles and requests the next ones ahead of the other
    // workgroup's waves, the quantised caches run their PV ahead
    constexpr int kStagePrio = KVT == KV_BF16 ? 2 : 0;
    constexpr int kPvPrio = QNT ? 1 : 0;
    auto iter = [&](int i, auto xc, auto full) __attribute__((always_inline)) {
        constexpr int X = decltype(xc)::value;  // slot of pair i: i % S2
        constexpr int Y = (X + 1) % S2;         // slot of pair i + 1
        constexpr bool FULL = decltype(full)::value;
        const int jn = j0 + 2 * (i + 1 + S2);
        const int tn0 = table[jn < jend ? jn : jend - 1], tn1 = table[jn + 1 < jend ? jn + 1 : jend - 1];
        if constexpr (kStagePrio != 0) __builtin_amdgcn_s_setprio(kStagePrio);
        if (FULL || i + 1 < npair) {
            store_k(ring[Y][0], (i + 1) & 1, 0);
            store_k(ring[Y][1], (i + 1) & 1, 1);
        }
        store_v(ring[X][0], i & 1, 0);
        store_v(ring[X][1], i & 1, 1);
        const int64_t ph0 = __builtin_amdgcn_readfirstlane(tp0), ph1 = __builtin_amdgcn_readfirstlane(tp1);
        if (FULL || i + S2 < npair) {
            load_blk(ring[X][0], ph0);
            load_blk(ring[X][1], ph1);
        }
        if constexpr (kStagePrio != 0) __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        // the owners' scores and softmax are the per-pair chain that every
        // wave's next barrier waits on: they issue ahead of the other
        // workgroup's waves on the same SIMD
        if (owner && (FULL || i + 1 < npair)) {
            __builtin_amdgcn_s_setprio(3);
            scores(i + 1, std::integral_constant<bool, FULL && X == 0>{});
            __builtin_amdgcn_s_setprio(0);
        }
        if constexpr (kPvPrio != 0) __builtin_amdgcn_s_setprio(kPvPrio);
        values(i, full);
        if constexpr (kPvPrio != 0) __builtin_amdgcn_s_setprio(0);
        tp0 = tn0;
        tp1 = tn1;
        // keep the next iteration's table wait behind this iteration's work
        __builtin_amdgcn_sched_barrier(0);
    };
    int i = 0;
    for (; i + 2 * S2 <= npair; i += S2)
        static_for<S2>([&](auto xc) __attribute__((always_inline)) { iter(i + decltype(xc)::value, xc, std::true_type{}); });
    for (; i < npair; i += S2)
        static_for<S2>([&](auto xc) __attribute__((always_inline)) {
            if (i + decltype(xc)::value < npair) iter(i + decltype(xc)::value, xc, std::false_type{});
        });

    // ------------------------------------------------------------ epilogue
    if (owner) {
        float l = lpart;
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        float sp = spart;
        sp += __shfl_xor(sp, 16);
        sp += __shfl_xor(sp, 32);
        if (lg == 0) {
            const float lnorm = QNT ? l : sp;  // bf16: the sum of the weights the values were multiplied by
            fin[0][wv][l16] = lnorm > 0.0f ? 1.0f / lnorm : 0.0f;
            fin[1][wv][l16] = kCodeBias * sp;
            if (myrow < R) {
                const float lse2 = l > 0.0f ? (mref + log2f(l)) * kLn2 : -INFINITY;
                const int64_t rid = row_out(myrow);
                if (p.np_stride == 1) {
                    if (p.lse != nullptr) p.lse[rid] = lse2;
                } else {
                    p.ws_lse[rid * p.np_stride + wpart] = lse2;
                }
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = row0 + 16 * t + 4 * lg + i;
            if (r >= R) continue;
            const float inv = fin[0][t][4 * lg + i];
            const float bias = fin[1][t][4 * lg + i];
            const int64_t rid = row_out(r);
#pragma unroll
            for (int nd = 0; nd < NDT; ++nd) {
                float v = o[t][nd][i];
                if constexpr (I8) v = (v - bias) * vsh_inv;
                if constexpr (F8 || F4) v *= vsh_inv;
                v *= inv;
                const int d = wv * DW + 16 * nd + l16;
                if (p.np_stride == 1) {
                    if (p.out_bf16)
                        reinterpret_cast<uint16_t*>(p.out)[rid * D + d] = f32_to_bf16(v);
                    else
                        reinterpret_cast<float*>(p.out)[rid * D + d] = v;
                } else {
                    p.ws_o[(rid * p.np_stride + wpart) * D + d] = v;
                }
            }
        }
    }
}

namespace {
template <int KVT, int D, int NT, int QS>
hipError_t launch_one(const DecodeParams& p, hipStream_t s) {
    const int64_t grid = (int64_t)p.NP * p.nchunk * p.Hkv * (p.stacked ? 1 : p.B);
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_mfma_kernel<KVT, D, NT, QS>), dim3((unsigned)grid), dim3(64 * kW), 0, s, p);
    return hipGetLastError();
}

template <int KVT, int D, int QS>
hipError_t by_nt(int NT, const DecodeParams& p, hipStream_t s) {
    switch (NT) {
    case 1: return launch_one<KVT, D, 1, QS>(p, s);
    case 2: return launch_one<KVT, D, 2, QS>(p, s);
    case 3: return launch_one<KVT, D, 3, QS>(p, s);
    case 4: return launch_one<KVT, D, 4, QS>(p, s);
    default: return hipErrorInvalidValue;
    }
}

template <int KVT, int QS>
hipError_t by_d(int D, int NT, const DecodeParams& p, hipStream_t s) {
    switch (D) {
    case 64: return by_nt<KVT, 64, QS>(NT, p, s);
    case 128: return by_nt<KVT, 128, QS>(NT, p, s);
    case 256: return by_nt<KVT, 256, QS>(NT, p, s);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_decode_mfma(int kv_type, int D, int NT, const DecodeParams& p, hipStream_t stream) {
    const int qs = p.q_bf16 ? 1 : 2;
    if (kv_type == KV_BF16) return qs == 1 ? by_d<KV_BF16, 1>(D, NT, p, stream) : by_d<KV_BF16, 2>(D, NT, p, stream);
    if (kv_type == KV_I8) return qs == 1 ? by_d<KV_I8, 1>(D, NT, p, stream) : by_d<KV_I8, 2>(D, NT, p, stream);
    if (kv_type == KV_FP8) return qs == 1 ? by_d<KV_FP8, 1>(D, NT, p, stream) : by_d<KV_FP8, 2>(D, NT, p, stream);
    if (kv_type == KV_NVFP4)
        return qs == 1 ? by_d<KV_NVFP4, 1>(D, NT, p, stream) : by_d<KV_NVFP4, 2>(D, NT, p, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa
