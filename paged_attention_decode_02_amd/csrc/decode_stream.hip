// Split-K paged decode on the matrix cores for one tile of query rows
// (G * Tq <= 16 rows of a kv head), with every wave streaming its own blocks.
//
// The long int8, FP8 and NVFP4 decodes (the split-K paged decode with an
// int8 KV cache of the vllm-sm70 page, "Why", Attention bullet; FP8 KV
// dequantised inline, nvllm page, "Acknowledgments", b12x; the all-NVFP4
// stack of the vllm-sm12x-nvfp4-dflash2 page, "What makes this stack
// different") have one 16-row tile per kv head: 6 query heads at one query
// token. A workgroup of four waves takes one
// split-K partition of one kv head; wave w takes blocks w, w + 4, ... of the
// partition and runs the whole block itself, so the waves never wait for
// each other inside the loop:
//  - the block's K and V tiles are copied from HBM straight into the wave's
//    own LDS (buffer loads with the LDS flag: whole 16-byte runs of a row per
//    lane, no register staging), double-buffered: block i + 1 is in flight
//    while block i is computed;
//  - S^T = K Q^T on v_mfma_f32_16x16x32 (keys read from LDS in the A-operand
//    layout, int8 codes widened to f16 as 1024 + code + 128, FP8 codes to
//    bf16, NVFP4 code pairs to f16 times their E4M3 block scale (exact); the
//    queries stay in registers as B operands); lane l holds row
//    l % 16 and tokens 4 (l / 16) + 0..3, which is the A-operand layout of
//    the PV product, so the weights never leave the registers;
//  - online softmax in log2 units with a per-row reference raised only when a
//    score beats it by 2^8;
//  - O += P V on v_mfma_f32_16x16x16 over all D output columns, the V operand
//    (4 tokens of one column per lane) from LDS: a 4x4 byte transpose inside
//    each lane quad (int8), the 8-bit transposing LDS read of gfx950 (FP8, one
//    read for two column tiles) or its 16-bit one (bf16; NVFP4 after the
//    block's values are widened with their block scales into a per-wave f16
//    tile).
// Quantised values: weight times value scale in f16, against a per-wave
// power-of-two reference of the value scales that is raised (O rescaled
// exactly) when a block's scale passes it, so no pass over the scales is
// needed before the loop. The four waves' states are merged through LDS at
// the end (log-sum-exp weights, fixed order).
#include <type_traits>
#include <utility>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_gcc;
typedef __attribute__((address_space(3))) bf16x4_gcc lds_bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2_gcc;
typedef __attribute__((address_space(3))) i32x2_gcc lds_i32x2;

constexpr uint32_t kMagic = 0x64646464u;
constexpr float kCodeBias = 1152.0f;  // 1024 + 128
constexpr float kVScaleRoom = 64.0f;  // weight (<= 2^8) x value scale / reference (<= 1) x 2^6 < 2^15 (f16)

__device__ __forceinline__ uint32_t f16pair_lo(uint32_t u) { return __builtin_amdgcn_perm(kMagic, u, 0x04010400u); }
__device__ __forceinline__ uint32_t f16pair_hi(uint32_t u) { return __builtin_amdgcn_perm(kMagic, u, 0x04030402u); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}

// 4x4 transpose of bytes inside a lane quad: lane i (= lane & 3) holds
// elements (i, 0..3) in one dword, afterwards lane j holds (0..3, j).
__device__ __forceinline__ uint32_t quad_transpose8(uint32_t w, int i) {
    const int b1 = (i >> 1) & 1, b0 = i & 1;
    const uint32_t recv = dpp_u32<kDppQuadXor2>(w);
    const uint32_t u = __builtin_amdgcn_perm(recv, w, b1 ? 0x03020706u : 0x05040100u);
    const uint32_t pu = dpp_u32<kDppQuadXor1>(u);
    return __builtin_amdgcn_perm(pu, u, b0 ? 0x03070105u : 0x06020400u);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}
__device__ __forceinline__ float f16lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)w); }
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// Wait until at most N vector-memory operations of this wave are in flight
// (the LDS-destined loads count there too). The memory clobber keeps LDS
// reads of the block after the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Order this wave's LDS accesses across lanes (its LDS operations execute in
// issue order; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// NVFP4: a byte of two E2M1 codes times an f16 block-scale pair, as an f16
// pair (exact: at most 6 significant bits, 2^-10 to 2688).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_scaled_f16x2(uint32_t w, f16x2 sc) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, fp4x2_to_f16x2<SEL>(w)) * sc);
}
__device__ __forceinline__ f16x2 e4m3_f16x2(uint32_t code) {
    const _Float16 h = (_Float16)fp8_value(code);
    return f16x2{h, h};
}

// Buffer loads whose data goes straight to LDS: lane l's 16 (or 4) bytes at
// rsrc + voff land at lds + 16 l (4 l); nontemporal. (Plain functions: the
// builtin is device-only, and a template kernel that names it directly gets
// no host-side launch stub.)
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, unsigned char* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, 0, 0, 2);
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t rs, float* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 4, voff, 0, 0, 2);
}

template <int I>
using ic = std::integral_constant<int, I>;

// Position (in 16-byte chunks) of global chunk c of row r inside the staged
// tiles: K and V rows use different swizzles so that the MFMA-layout reads
// (16 rows, one chunk column: K; 4 rows, 4 columns: V) hit distinct banks.
template <int CPR>
__device__ __forceinline__ int swz_k(int r) { return r % CPR; }
template <int CPR>
__device__ __forceinline__ int swz_v(int r) { return CPR >= 16 ? 4 * (r & 3) : CPR == 8 ? 4 * ((r >> 1) & 1) : 0; }
// FP8 value tiles, read by the 8-bit transposing LDS read: a 16-lane group
// reads tokens 4 lg + 0..3 at chunks t and t + 1 (t even), 8 bytes a lane;
// the swizzle puts the group's 16 pieces in distinct banks, and those of the
// groups lg and lg + 1 apart (whether the LDS serves 16 or 32 lanes of the
// read at a time)
template <int CPR>
__device__ __forceinline__ int swz_v8(int r) {
    return CPR >= 16 ? (2 * (r & 3)) ^ (8 * ((r >> 2) & 1))
           : CPR == 8 ? (2 * (r & 3)) ^ (2 * ((r >> 2) & 1))
                      : (2 * ((r >> 1) & 1)) ^ (2 * ((r >> 2) & 1));
}

}  // namespace

template <int KVT, int D, int QS, int HPG>
__global__ __launch_bounds__(64 * stream_waves(KVT, D), 1) void decode_stream_kernel(DecodeParams p) {
    static_assert(KVT == KV_BF16 || KVT == KV_I8 || KVT == KV_FP8 || KVT == KV_NVFP4, "bf16, int8, fp8 or nvfp4");
    constexpr bool I8 = KVT == KV_I8;
    constexpr bool F8 = KVT == KV_FP8;
    constexpr bool F4 = KVT == KV_NVFP4;
    constexpr bool QNT = I8 || F8 || F4;  // codes with a per-(token, kv head) scale
    constexpr bool H16 = I8 || F4;        // f16 products: queries scaled into f16
    // FP8 values by the 8-bit transposing read. (For int8 the quad transpose
    // is kept: with one wave per SIMD the transposing reads made the 250K
    // decode slower, 85.5 -> 91-101 us, where FP8 gained 91.0 -> 88.5.)
    constexpr bool VT8 = F8;
    constexpr int E = Elt<KVT>::bytes;
    constexpr int RB = kv_code_row_bytes<KVT>(D);  // code bytes of one cache row
    constexpr int CPR = RB / 16;       // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;      // rows per LDS-destined load instruction (16 CPR lanes active if > 16)
    constexpr int NI = RPI > 16 ? 1 : 16 / RPI;  // such instructions per 16-row tile
    constexpr int TILE = 16 * RB;      // bytes of a staged tile
    // nvfp4: the values of the block being computed, widened to f16 (times
    // their block scales) in a per-wave row-major tile laid out like a bf16
    // tile (rows of 2 D bytes, 16-byte chunks swizzled by swz_v), so the PV
    // takes its operands with the transposing LDS read
    constexpr int RB16 = 2 * D, CPR16 = RB16 / 16;
    constexpr int KS = D / 32;         // k-steps of the score product
    constexpr int NDT = D / 16;        // 16-column output tiles
    constexpr int NQ = QS == 2 ? 2 : 1;
    constexpr int NVM = 2 * NI + (QNT ? 2 : 0) + (F4 ? 2 : 0);  // vector-memory operations per block
    constexpr int NST = stream_stages(KVT, D);    // LDS stages per wave
    constexpr int kW = stream_waves(KVT, D);      // waves per workgroup
    constexpr int WPH = kW / HPG;                 // waves per kv head
    static_assert(RPI >= 1 && (NI * RPI == 16 || (NI == 1 && RPI > 16)), "tile split");
    static_assert(HPG == 1 || HPG == 2 || HPG == 4, "kv heads per workgroup");
    static_assert((NST - 1) * NVM < 64, "vmcnt range");

    // per wave: [stage][K, V][16 rows x RB], rows swizzled by 16-byte chunk,
    // then (nvfp4) the widened value tile [16 rows x RB16]; after the block
    // loop the same bytes hold the merge's partial outputs ([16 rows][D]
    // floats: the region is at least that large when waves merge)
    constexpr int WAVE_TILES = NST * 2 * TILE + (F4 ? 16 * RB16 : 0);
    constexpr int WAVE_STG = (WPH > 1 && 16 * D * 4 > WAVE_TILES) ? 16 * D * 4 : WAVE_TILES;
    __shared__ __align__(16) unsigned char stg[kW][WAVE_STG];
    // nvfp4: [wave][stage][K, V] the block's E4M3 scale plane of the wave's
    // head (D bytes)
    __shared__ __align__(16) unsigned char spl[F4 ? kW : 1][NST][2][F4 ? D : 16];
    // quantised: [wave][stage][K, V] the block's 16 scales (dword loads of all
    // 64 lanes land here; lanes past the 64-byte run write zeros)
    __shared__ __align__(16) float sst[kW][NST][2][QNT ? 64 : 1];
    __shared__ float mst[kW][3][16];  // per wave and row: reference m (log2), sum l, sum of rounded weights

    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int l16 = lane & 15, lg = lane >> 4;

    // workgroup: partition part of kv heads gg HPG .. gg HPG + HPG - 1 of
    // sequence b; wave wv serves head g = gg HPG + wv / WPH and takes every
    // WPH-th block of the partition from block sub = wv % WPH on
    int wg = blockIdx.x;
    const int part = wg % p.NP;
    wg /= p.NP;
    const int ngrp = p.Hkv / HPG;
    const int gg = wg % ngrp;
    const int b = wg / ngrp;
    const int gi = wv / WPH, sub = wv % WPH;
    const int g = gg * HPG + gi;

    const int G = p.G, Tq = p.Tq, R = G * Tq;  // rows r = t G + h'
    // row of the block table and length (per-head tables: one head per workgroup)
    const int hrow = p.head_tables ? b * p.Hkv + g : b;
    const int L = p.seq_lens[hrow] - p.kv_begin;
    const int n_last = L - Tq + (R - 1) / G + 1;   // keys of the last row (largest t)
    const int start = part * p.P;
    const int64_t wpart = p.part_base + part;

    // flat output row of row r of kv head gh
    auto row_out_h = [&](int gh, int r) -> int64_t {
        return ((int64_t)b * Tq + r / G) * p.Hq + gh * G + r % G;
    };
    auto row_out = [&](int r) -> int64_t { return row_out_h(g, r); };

    if (start >= n_last) {
        // the lengths are the same for every head of the workgroup here
        for (int x = threadIdx.x; x < HPG * R * D; x += 64 * kW) {
            const int gh = gg * HPG + x / (R * D), r = (x / D) % R, d = x % D;
            const int64_t rid = row_out_h(gh, r);
            if (p.np_stride == 1) {
                if (p.out_bf16)
                    reinterpret_cast<uint16_t*>(p.out)[rid * D + d] = 0;
                else
                    reinterpret_cast<float*>(p.out)[rid * D + d] = 0.0f;
                if (p.lse != nullptr && d == 0) p.lse[rid] = -INFINITY;
            } else if (p.fill_empty && d == 0) {
                p.ws_lse[rid * p.np_stride + wpart] = -INFINITY;
            }
        }
        return;
    }
    const int end = min(start + p.P, n_last);
    // every valid row sees tokens below lim_all (the first query token's limit)
    const int lim_all = min(end, L - Tq + 1);

    // ---------------------------------------------------------------- queries
    // B operand of k-step ks: row l16, k slots 8 lg .. 8 lg + 7 = dims qdim(ks, e)
    auto qdim = [&](int ks, int e) {
        return E == 1 ? 64 * (ks >> 1) + 16 * lg + 8 * (ks & 1) + e : 32 * ks + 8 * lg + e;
    };
    const bool row_ok = l16 < R;
    const int myt = l16 / (G > 0 ? G : 1);
    float qx[KS][8];
    float qmax = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if (row_ok) {
            const int64_t off = row_out(l16) * D + qdim(ks, 0);
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
    float qpost = p.qk_scale_log2;
    float qscale = 1.0f;
    if constexpr (H16) {
        // one power of two for all rows puts max|q| in [2^14, 2^15) (f16)
        qmax = wave_max(qmax);
        const int e2 = qmax > 0.0f ? 14 - ilogbf(qmax) : 0;
        qscale = ldexpf(1.0f, e2);
        qpost = ldexpf(p.qk_scale_log2, -e2);
    }
    u32x4 qreg[NQ][KS];
    float corr = 0.0f;  // int8: 1152 * sum_d q'[row] (the code bias of the widened keys)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float x0 = qx[ks][2 * k] * qscale, x1 = qx[ks][2 * k + 1] * qscale;
            if constexpr (H16) {
                hi[k] = pack_f16x2(x0, x1);
                lo[k] = pack_f16x2(x0 - f16lo(hi[k]), x1 - f16hi(hi[k]));
                if constexpr (I8) {
                    corr += f16lo(hi[k]) + f16hi(hi[k]);
                    if constexpr (QS == 2) corr += f16lo(lo[k]) + f16hi(lo[k]);
                }
            } else {
                hi[k] = pack_bf16_rne(x0, x1);
                lo[k] = pack_bf16_rne(x0 - bf16_to_f32((uint16_t)hi[k]), x1 - bf16_to_f32((uint16_t)(hi[k] >> 16)));
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

    // ------------------------------------------------------------- state
    const int nvis = row_ok ? min(end, L - Tq + myt + 1) : 0;  // keys of the lane's row in this partition
    float mref = -INFINITY, lpart = 0.0f, spart = 0.0f;
    float vref = 0.0f;  // quantised: power-of-two bound of the value scales seen so far (0: none yet)
    f32x4 o[NDT];
#pragma unroll
    for (int t = 0; t < NDT; ++t) o[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int32_t* table = p.block_table + (int64_t)hrow * p.max_blocks + p.kv_begin / kBlockSize;
    const int tok_stride = p.Hkv * RB;                 // bytes between tokens of a block
    const int blk_bytes = kBlockSize * p.Hkv * kv_row_bytes<KVT>(D);  // bytes of a KV block (all heads)
    const int plane_off = kBlockSize * tok_stride + g * D;  // nvfp4: this head's scale plane in a block
    const char* kcache = reinterpret_cast<const char*>(p.k_cache);
    const char* vcache = reinterpret_cast<const char*>(p.v_cache);
    const int j0 = start / kBlockSize, jend = (end + kBlockSize - 1) / kBlockSize;
    const int jw = j0 + sub;                                    // this wave's first block
    const int nbw = jw < jend ? (jend - jw + WPH - 1) / WPH : 0;  // its block count (<= 256)

    // LDS-destined loads: instruction c moves rows RPI c .. RPI c + RPI - 1;
    // lane l takes row RPI c + l / CPR and the global chunk whose swizzled
    // position is l % CPR
    const int ldrow = lane / CPR, ldpos = lane % CPR;
    int voff_k[NI], voff_v[NI];
#pragma unroll
    for (int c = 0; c < NI; ++c) {
        const int r = RPI * c + ldrow;
        voff_k[c] = r * tok_stride + g * RB + 16 * (ldpos ^ swz_k<CPR>(r));
        voff_v[c] = r * tok_stride + g * RB + 16 * (ldpos ^ (VT8 ? swz_v8<CPR>(r) : swz_v<CPR>(r)));
    }
    unsigned char* my_stage = &stg[wv][0];

    // physical blocks of this wave's blocks: register k, lane l holds block
    // 64 k + l's (the launcher keeps a wave at 256 blocks or fewer); read per
    // block with readlane, so the loop never waits on a scalar load
    int tb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        tb[k] = 64 * k + lane < nbw ? table[jw + WPH * (64 * k + lane)] : 0;
        // the values pass through an empty asm once loaded: later reads of
        // them wait for nothing (otherwise every block would wait for all
        // loads in flight before reading its table entry)
        asm volatile("" : "+v"(tb[k]));
    }

    auto issue = [&](int i, int stage) {
        const int k = i >> 6;
        const int tv = k == 0 ? tb[0] : k == 1 ? tb[1] : k == 2 ? tb[2] : tb[3];
        const int64_t ph = (int64_t)__builtin_amdgcn_readlane(tv, i & 63);
        const auto rk = range_rsrc(kcache + ph * blk_bytes, blk_bytes);
        const auto rv = range_rsrc(vcache + ph * blk_bytes, blk_bytes);
        unsigned char* kst = my_stage + (stage * 2 + 0) * TILE;
        unsigned char* vst = my_stage + (stage * 2 + 1) * TILE;
        if (RPI <= 16 || lane < 16 * CPR) {  // a tile of fewer than 1024 bytes: its lanes only
#pragma unroll
            for (int c = 0; c < NI; ++c) lds_load16(rk, kst + 1024 * c, voff_k[c]);
#pragma unroll
            for (int c = 0; c < NI; ++c) lds_load16(rv, vst + 1024 * c, voff_v[c]);
        }
        if constexpr (F4) {
            if (lane < D / 16) {  // the D-byte scale planes, 16 bytes a lane
                lds_load16(rk, &spl[wv][stage][0][0], plane_off + 16 * lane);
                lds_load16(rv, &spl[wv][stage][1][0], plane_off + 16 * lane);
            }
        }
        if constexpr (QNT) {
            const int64_t s0 = (ph * p.Hkv + g) * kBlockSize;
            const auto rks = range_rsrc(p.k_scale + s0, 4 * kBlockSize);
            const auto rvs = range_rsrc(p.v_scale + s0, 4 * kBlockSize);
            lds_load4(rks, &sst[wv][stage][0][0], 4 * lane);
            lds_load4(rvs, &sst[wv][stage][1][0], 4 * lane);
        }
    };

    // one block: scores, softmax, PV. MASK: some token of the block is past
    // the partition's end or a row's causal limit.
    auto compute = [&](int jblk, int stage, auto mask) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask)::value;
        const unsigned char* kst = my_stage + (stage * 2 + 0) * TILE;
        const unsigned char* vst = my_stage + (stage * 2 + 1) * TILE;
        const int pos0 = jblk * kBlockSize;

        // -------------------------------------------------------------- QK
        f32x4 acc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
        if constexpr (F4) {
            // 16 codes per read (8 bytes): dims 64 m + 16 lg .. + 15 of token
            // l16 = k-steps 2m and 2m + 1, one 16-element block of one scale
            const unsigned char* sk = &spl[wv][stage][0][0];
#pragma unroll
            for (int m = 0; m < KS / 2; ++m) {
                const int cb = 32 * m + 8 * lg;  // code byte of the first dim
                const u32x2 raw = *reinterpret_cast<const u32x2*>(kst + l16 * RB + 16 * ((cb >> 4) ^ swz_k<CPR>(l16)) +
                                                                   (cb & 15));
                const f16x2 sc2 = e4m3_f16x2(sk[nvfp4_scale_byte(l16, 4 * m + lg)]);
                u32x4 a[2];
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    a[h] = u32x4{fp4x2_scaled_f16x2<0>(raw[h], sc2), fp4x2_scaled_f16x2<1>(raw[h], sc2),
                                 fp4x2_scaled_f16x2<2>(raw[h], sc2), fp4x2_scaled_f16x2<3>(raw[h], sc2)};
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int q2 = 0; q2 < NQ; ++q2)
                        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[h]),
                                                                        __builtin_bit_cast(f16x8, qreg[q2][2 * m + h]),
                                                                        acc[h], 0, 0, 0);
            }
        } else if constexpr (E == 1) {
            // 16 codes per read: k-steps 2m and 2m + 1 of token l16
#pragma unroll
            for (int m = 0; m < KS / 2; ++m) {
                const int c = 4 * m + lg;
                const u32x4 raw = *reinterpret_cast<const u32x4*>(kst + l16 * RB + 16 * (c ^ swz_k<CPR>(l16)));
                u32x4 a[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if constexpr (I8) {
                        const uint32_t u0 = raw[2 * h] ^ 0x80808080u, u1 = raw[2 * h + 1] ^ 0x80808080u;
                        a[h] = u32x4{f16pair_lo(u0), f16pair_hi(u0), f16pair_lo(u1), f16pair_hi(u1)};
                    } else {
                        const pa_f32x2 x0 = fp8x2_to_f32<false>(raw[2 * h]), x1 = fp8x2_to_f32<true>(raw[2 * h]);
                        const pa_f32x2 x2 = fp8x2_to_f32<false>(raw[2 * h + 1]), x3 = fp8x2_to_f32<true>(raw[2 * h + 1]);
                        a[h] = u32x4{pack_bf16_rne(x0.x, x0.y), pack_bf16_rne(x1.x, x1.y), pack_bf16_rne(x2.x, x2.y),
                                     pack_bf16_rne(x3.x, x3.y)};
                    }
                }
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int q2 = 0; q2 < NQ; ++q2) {
                        if constexpr (I8)
                            acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[h]),
                                                                            __builtin_bit_cast(f16x8, qreg[q2][2 * m + h]),
                                                                            acc[h], 0, 0, 0);
                        else
                            acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[h]),
                                                                             __builtin_bit_cast(bf16x8, qreg[q2][2 * m + h]),
                                                                             acc[h], 0, 0, 0);
                    }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c = 4 * ks + lg;
                const u32x4 a = *reinterpret_cast<const u32x4*>(kst + l16 * RB + 16 * (c ^ swz_k<CPR>(l16)));
#pragma unroll
                for (int q2 = 0; q2 < NQ; ++q2)
                    acc[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, qreg[q2][ks]), acc[ks & 1], 0, 0, 0);
            }
        }
        const f32x4 s4 = acc[0] + acc[1];

        // ----------------------------------------------------------- softmax
        // lane: row l16, tokens 4 lg + e of the block
        float kf[4] = {1.0f, 1.0f, 1.0f, 1.0f}, vf[4] = {1.0f, 1.0f, 1.0f, 1.0f};
        if constexpr (QNT) {
            const f32x4 k4 = *reinterpret_cast<const f32x4*>(&sst[wv][stage][0][4 * lg]);
            const f32x4 v4 = *reinterpret_cast<const f32x4*>(&sst[wv][stage][1][4 * lg]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kf[e] = k4[e];
                vf[e] = v4[e];
            }
        }
        float sc[4];
        bool raise = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool ok = MASK ? pos0 + 4 * lg + e < nvis : row_ok;
            sc[e] = ok ? (s4[e] - corr) * (qpost * kf[e]) : -INFINITY;
            raise |= sc[e] > mref + 8.0f;
        }
        // value-scale reference (quantised): raised to the next power of two
        // at or above the block's largest scale of a visible token
        float vr_new = vref;
        if constexpr (QNT) {
            bool vraise = false;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = MASK ? pos0 + 4 * lg + e < end : true;
                vraise |= ok && vf[e] > vref;
            }
            if (__builtin_amdgcn_ballot_w64(vraise) != 0) {
                float vm = 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = MASK ? pos0 + 4 * lg + e < end : true;
                    vm = fmaxf(vm, ok ? vf[e] : 0.0f);
                }
                vm = wave_max(vm);
                vr_new = ldexpf(1.0f, ilogbf(vm) + 1);  // > vm, a power of two
            }
        }
        const bool any_m = __builtin_amdgcn_ballot_w64(raise) != 0;
        if (any_m || vr_new != vref) {
            // rescale o (rows 4 lg + e) and the row sums by the factors of the
            // rows' references and the value reference
            float alpha = 1.0f;
            if (any_m) {
                float bm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
                bm = fmaxf(bm, __shfl_xor(bm, 16));
                bm = fmaxf(bm, __shfl_xor(bm, 32));
                const float mn = fmaxf(mref, bm);
                const float base = mn == -INFINITY ? 0.0f : mn;
                alpha = exp2_guarded(mref - base);
                mref = mn;
                lpart *= alpha;
                spart *= alpha;
            }
            float vfac = 1.0f;
            if constexpr (QNT) {
                if (vr_new != vref) {
                    vfac = vref == 0.0f ? 0.0f : vref / vr_new;  // exact: powers of two (o is 0 while vref is 0)
                    spart *= vfac;
                    vref = vr_new;
                }
            }
            f32x4 a4;
#pragma unroll
            for (int e = 0; e < 4; ++e) a4[e] = __shfl(alpha, 4 * lg + e) * vfac;
#pragma unroll
            for (int t = 0; t < NDT; ++t) o[t] *= a4;
        }
        const float base = mref == -INFINITY ? 0.0f : mref;
        float pr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pr[e] = exp2_weight(sc[e] - base);  // sc = -inf gives 0
            lpart += pr[e];
        }
        u32x2 pa;
        if constexpr (QNT) {
            const float vmul = vref > 0.0f ? kVScaleRoom / vref : 0.0f;
            float ph[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = MASK ? pos0 + 4 * lg + e < end : true;
                ph[e] = (float)(_Float16)(ok ? pr[e] * vf[e] * vmul : 0.0f);
                spart += ph[e];
            }
            pa = u32x2{pack_f16x2(ph[0], ph[1]), pack_f16x2(ph[2], ph[3])};
        } else {
            pa = u32x2{pack_bf16_rne(pr[0], pr[1]), pack_bf16_rne(pr[2], pr[3])};
#pragma unroll
            for (int w = 0; w < 2; ++w) spart += bf16_to_f32((uint16_t)pa[w]) + bf16_to_f32((uint16_t)(pa[w] >> 16));
        }

        // ---------------------------------------------------------------- PV
        if constexpr (F4) {
            // widen the block's values into the wave's f16 tile: lane (token
            // vt, quarter vq) takes dims DQ vq .. DQ vq + DQ - 1, block scale
            // by block (16 dims, 8 code bytes)
            constexpr int DQ = D / 4, NB16 = DQ / 16;
            const int vt = lane >> 2, vq = lane & 3;
            const unsigned char* sv = &spl[wv][stage][1][0];
            unsigned char* wt = my_stage + NST * 2 * TILE;
            wave_lds_order();  // the previous block's reads of the tile are done
#pragma unroll
            for (int j = 0; j < NB16; ++j) {
                const int blk16 = vq * NB16 + j;  // 16-element block of the row
                const int cb = 8 * blk16;         // its first code byte
                const u32x2 raw = *reinterpret_cast<const u32x2*>(vst + vt * RB + 16 * ((cb >> 4) ^ swz_v<CPR>(vt)) +
                                                                   (cb & 15));
                const f16x2 sc2 = e4m3_f16x2(sv[nvfp4_scale_byte(vt, blk16)]);
                const u32x4 w0 = u32x4{fp4x2_scaled_f16x2<0>(raw[0], sc2), fp4x2_scaled_f16x2<1>(raw[0], sc2),
                                       fp4x2_scaled_f16x2<2>(raw[0], sc2), fp4x2_scaled_f16x2<3>(raw[0], sc2)};
                const u32x4 w1 = u32x4{fp4x2_scaled_f16x2<0>(raw[1], sc2), fp4x2_scaled_f16x2<1>(raw[1], sc2),
                                       fp4x2_scaled_f16x2<2>(raw[1], sc2), fp4x2_scaled_f16x2<3>(raw[1], sc2)};
                // dims 16 blk16 .. + 7 and + 8 .. + 15: 16-byte chunks 2 blk16 and 2 blk16 + 1 of the f16 row
                *reinterpret_cast<u32x4*>(wt + vt * RB16 + 16 * ((2 * blk16) ^ swz_v<CPR16>(vt))) = w0;
                *reinterpret_cast<u32x4*>(wt + vt * RB16 + 16 * ((2 * blk16 + 1) ^ swz_v<CPR16>(vt))) = w1;
            }
            wave_lds_order();  // every lane's widened values are in the tile
            // transposing LDS read, as for bf16 values: lane 4 r' + c' of a
            // 16-lane group names token 4 lg + r', dims 16 t + 4 c' .. + 3;
            // lane i receives dim 16 t + i of the group's 4 tokens
            const int vr = 4 * lg + (l16 >> 2), cq = l16 & 3;
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                const int c = 2 * t + (cq >> 1);
                const unsigned char* src = wt + vr * RB16 + 16 * (c ^ swz_v<CPR16>(vr)) + 8 * (cq & 1);
                u32x2 bop = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)src));
                if (MASK) {  // tokens past the end may hold NaN block scales
                    const int t0 = pos0 + 4 * lg;
                    bop.x = (t0 + 0 < end ? bop.x & 0x0000FFFFu : 0u) | (t0 + 1 < end ? bop.x & 0xFFFF0000u : 0u);
                    bop.y = (t0 + 2 < end ? bop.y & 0x0000FFFFu : 0u) | (t0 + 3 < end ? bop.y & 0xFFFF0000u : 0u);
                }
                o[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, pa), __builtin_bit_cast(f16x4, bop),
                                                             o[t], 0, 0, 0);
            }
        } else if constexpr (VT8) {
            // 8-bit transposing LDS read, two 16-column tiles per read: lane
            // 2 r8 + c8 of a 16-lane group names token 4 lg + r8 % 4 and dims
            // 16 (t + r8 / 4) + 8 c8 .. + 7; lane i receives dim 16 t + i of
            // the group's 4 tokens in bytes 0..3 and dim 16 (t + 1) + i in
            // bytes 4..7
            const int r8 = l16 >> 1, c8 = l16 & 1, vr = 4 * lg + (r8 & 3);
#pragma unroll
            for (int t = 0; t < NDT; t += 2) {
                const unsigned char* src = vst + vr * RB + 16 * ((t + (r8 >> 2)) ^ swz_v8<CPR>(vr)) + 8 * c8;
                const u32x2 raw = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)src));
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const pa_f32x2 x0 = fp8x2_to_f32<false>(raw[h]), x1 = fp8x2_to_f32<true>(raw[h]);
                    u32x2 bop = u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x0.x, x0.y)),
                                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x1.x, x1.y))};
                    if (MASK) {  // tokens past the end may hold NaN codes
                        const int t0 = pos0 + 4 * lg;  // element k is token 4 lg + k
                        bop.x = (t0 + 0 < end ? bop.x & 0x0000FFFFu : 0u) | (t0 + 1 < end ? bop.x & 0xFFFF0000u : 0u);
                        bop.y = (t0 + 2 < end ? bop.y & 0x0000FFFFu : 0u) | (t0 + 3 < end ? bop.y & 0xFFFF0000u : 0u);
                    }
                    o[t + h] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, pa),
                                                                     __builtin_bit_cast(f16x4, bop), o[t + h], 0, 0, 0);
                }
            }
        } else if constexpr (E == 1) {
            // int8: lane (quad q, position i): token 4 lg + i, chunks 4 m + q; after
            // the quad transpose of dword w, dim 16 (4 m + q) + 4 w + i of
            // tokens 4 lg .. 4 lg + 3 = column 4 q + i of tile 4 m + w
            const int i4 = l16 & 3, qd = l16 >> 2, vr = 4 * lg + i4;
#pragma unroll
            for (int m = 0; m < NDT / 4; ++m) {
                const u32x4 raw = *reinterpret_cast<const u32x4*>(vst + vr * RB + 16 * ((4 * m + qd) ^ swz_v<CPR>(vr)));
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t tw = quad_transpose8(raw[w], i4) ^ 0x80808080u;
                    const u32x2 bop = u32x2{f16pair_lo(tw), f16pair_hi(tw)};
                    o[4 * m + w] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, pa),
                                                                         __builtin_bit_cast(f16x4, bop), o[4 * m + w],
                                                                         0, 0, 0);
                }
            }
        } else {
            // transposing LDS read: lane 4 r' + c' of a 16-lane group names
            // token 4 lg + r', dims 16 t + 4 c' .. + 3; lane i receives dim
            // 16 t + i of the group's 4 tokens
            const int vr = 4 * lg + (l16 >> 2), cq = l16 & 3;
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                const int c = 2 * t + (cq >> 1);
                const unsigned char* src = vst + vr * RB + 16 * (c ^ swz_v<CPR>(vr)) + 8 * (cq & 1);
                u32x2 bop = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)src));
                if (MASK) {  // tokens past the end may hold anything
                    const int t0 = pos0 + 4 * lg;
                    bop.x = (t0 + 0 < end ? bop.x & 0x0000FFFFu : 0u) | (t0 + 1 < end ? bop.x & 0xFFFF0000u : 0u);
                    bop.y = (t0 + 2 < end ? bop.y & 0x0000FFFFu : 0u) | (t0 + 3 < end ? bop.y & 0xFFFF0000u : 0u);
                }
                o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, pa),
                                                                 __builtin_bit_cast(s16x4, bop), o[t], 0, 0, 0);
            }
        }
    };

    // ---------------------------------------------------------- block loop
    // block i of this wave is jw + WPH i, staged in stage i % NST; the loads
    // of blocks i + 1 .. i + NST - 1 stay in flight while block i is
    // computed (each block's NVM vector-memory operations issued in order).
    // Blocks wholly below lim_all need no mask; they come first.
    auto wait_block = [&](int after) __attribute__((always_inline)) {
        // wait until block i has landed while `after` later blocks may still fly
        if constexpr (NST > 3) {
            if (after >= 3) {
                wait_vm<3 * NVM>();
                return;
            }
        }
        if constexpr (NST > 2) {
            if (after == 2) {
                wait_vm<2 * NVM>();
                return;
            }
        }
        if (after >= 1)
            wait_vm<NVM>();
        else
            wait_vm<0>();
    };
    auto step = [&](int i, auto mask) __attribute__((always_inline)) {
        const int ahead = i + NST - 1;
        if (ahead < nbw) {
            wait_lds();  // this wave's reads of the stage block `ahead` reuses are complete
            issue(ahead, ahead % NST);
        }
        wait_block(min(nbw - 1 - i, NST - 1));
        compute(jw + WPH * i, i % NST, mask);
    };
#pragma unroll
    for (int x = 0; x < NST - 1; ++x)
        if (x < nbw) issue(x, x);
    // blocks jw + WPH i with (jw + WPH i + 1) * 16 <= lim_all are unmasked
    const int nfull = lim_all >= (jw + 1) * kBlockSize ? min(nbw, (lim_all / kBlockSize - jw - 1) / WPH + 1) : 0;
    int i = 0;
    for (; i < nfull; ++i) step(i, std::false_type{});
    for (; i < nbw; ++i) step(i, std::true_type{});

    // ------------------------------------------------------------ epilogue
    // row sums of this wave (lanes 0..15 hold rows 0..15 after the butterfly)
    float l = lpart;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    float sp = spart;
    sp += __shfl_xor(sp, 16);
    sp += __shfl_xor(sp, 32);
    // output column of tile t for this lane
    auto dim_of = [&](int t) {
        return I8 ? 64 * (t >> 2) + 16 * (l16 >> 2) + 4 * (t & 3) + (l16 & 3) : 16 * t + l16;
    };
    const float vfin = QNT ? vref * (1.0f / kVScaleRoom) : 1.0f;  // undoes the value-scale reference
    if constexpr (WPH == 1) {
        // the wave ran its head's whole partition: normalise and write
        float bias[4], inv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lr = __shfl(l, 4 * lg + e), sr = __shfl(sp, 4 * lg + e);
            const float lnorm = QNT ? lr : sr;  // bf16: the sum of the weights the values were multiplied by
            inv[e] = lnorm > 0.0f ? vfin / lnorm : 0.0f;
            bias[e] = I8 ? kCodeBias * sr : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 4 * lg + e;
            if (row >= R) continue;
            const int64_t rid = row_out(row);
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
                const float val = (o[t][e] - bias[e]) * inv[e];
                const int d = dim_of(t);
                if (p.np_stride == 1) {
                    if (p.out_bf16)
                        reinterpret_cast<uint16_t*>(p.out)[rid * D + d] = f32_to_bf16(val);
                    else
                        reinterpret_cast<float*>(p.out)[rid * D + d] = val;
                } else {
                    p.ws_o[(rid * p.np_stride + wpart) * D + d] = val;
                }
            }
        }
        if (lg == 0 && l16 < R) {
            const float lse2 = l > 0.0f ? (mref + log2f(l)) * kLn2 : -INFINITY;
            const int64_t rid = row_out(l16);
            if (p.np_stride == 1) {
                if (p.lse != nullptr) p.lse[rid] = lse2;
            } else {
                p.ws_lse[rid * p.np_stride + wpart] = lse2;
            }
        }
    } else {
        // the WPH waves of each head merge through LDS
        __syncthreads();  // every wave is done with its staged tiles: reuse them
        float* ow = reinterpret_cast<float*>(&stg[wv][0]);  // [16 rows][D], unnormalised
        if (lg == 0) {
            mst[wv][0][l16] = mref;
            mst[wv][1][l16] = l;
            mst[wv][2][l16] = sp;
        }
        float bias[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) bias[e] = I8 ? kCodeBias * __shfl(sp, 4 * lg + e) : 0.0f;
#pragma unroll
        for (int t = 0; t < NDT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) ow[(4 * lg + e) * D + dim_of(t)] = (o[t][e] - bias[e]) * vfin;
        __syncthreads();
        // output element (head, row, d) per thread, the head's waves in a fixed order
        for (int idx = threadIdx.x; idx < HPG * R * D; idx += 64 * kW) {
            const int hg = idx / (R * D), row = (idx / D) % R, d = idx % D;
            const int w0 = hg * WPH;
            float M = -INFINITY;
#pragma unroll
            for (int k = 0; k < WPH; ++k) M = fmaxf(M, mst[w0 + k][0][row]);
            const float mb = M == -INFINITY ? 0.0f : M;
            float acc = 0.0f, lsum = 0.0f, lrs = 0.0f;
#pragma unroll
            for (int k = 0; k < WPH; ++k) {
                const float wt = exp2_guarded(mst[w0 + k][0][row] - mb);
                lsum += wt * mst[w0 + k][1][row];
                lrs += wt * mst[w0 + k][2][row];
                acc += wt * reinterpret_cast<const float*>(&stg[w0 + k][0])[row * D + d];
            }
            const float lnorm = QNT ? lsum : lrs;
            const float val = lnorm > 0.0f ? acc / lnorm : 0.0f;
            const int64_t rid = row_out_h(gg * HPG + hg, row);
            if (p.np_stride == 1) {
                if (p.out_bf16)
                    reinterpret_cast<uint16_t*>(p.out)[rid * D + d] = f32_to_bf16(val);
                else
                    reinterpret_cast<float*>(p.out)[rid * D + d] = val;
            } else {
                p.ws_o[(rid * p.np_stride + wpart) * D + d] = val;
            }
            if (d == 0) {
                const float lse2 = lsum > 0.0f ? (M + log2f(lsum)) * kLn2 : -INFINITY;
                if (p.np_stride == 1) {
                    if (p.lse != nullptr) p.lse[rid] = lse2;
                } else {
                    p.ws_lse[rid * p.np_stride + wpart] = lse2;
                }
            }
        }
    }
}

namespace {
template <int KVT, int D, int QS, int HPG>
hipError_t launch_one(const DecodeParams& p, hipStream_t s) {
    const int64_t grid = (int64_t)p.NP * (p.Hkv / HPG) * p.B;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    // one row tile; at most 256 blocks per wave (the per-wave table window);
    // per-head tables take one head per workgroup
    if (p.G * p.Tq > 16 || p.stacked || p.Hkv % HPG || (p.head_tables && HPG != 1) ||
        p.P > kStreamMaxPartition * (stream_waves(KVT, D) / HPG))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_stream_kernel<KVT, D, QS, HPG>), dim3((unsigned)grid), dim3(64 * stream_waves(KVT, D)),
                       0, s, p);
    return hipGetLastError();
}

template <int KVT, int D, int QS>
hipError_t by_hpg(const DecodeParams& p, hipStream_t s) {
    switch (p.hpg) {
    case 1: return launch_one<KVT, D, QS, 1>(p, s);
    case 2: return launch_one<KVT, D, QS, 2>(p, s);
    case 4: return launch_one<KVT, D, QS, 4>(p, s);
    default: return hipErrorInvalidValue;
    }
}

template <int KVT, int QS>
hipError_t by_d(int D, const DecodeParams& p, hipStream_t s) {
    switch (D) {
    case 64: return by_hpg<KVT, 64, QS>(p, s);
    case 128: return by_hpg<KVT, 128, QS>(p, s);
    case 256: return by_hpg<KVT, 256, QS>(p, s);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_decode_stream(int kv_type, int D, const DecodeParams& p, hipStream_t stream) {
    const int qs = p.q_bf16 ? 1 : 2;
    if (kv_type == KV_BF16) return qs == 1 ? by_d<KV_BF16, 1>(D, p, stream) : by_d<KV_BF16, 2>(D, p, stream);
    if (kv_type == KV_I8) return qs == 1 ? by_d<KV_I8, 1>(D, p, stream) : by_d<KV_I8, 2>(D, p, stream);
    if (kv_type == KV_FP8) return qs == 1 ? by_d<KV_FP8, 1>(D, p, stream) : by_d<KV_FP8, 2>(D, p, stream);
    if (kv_type == KV_NVFP4) return qs == 1 ? by_d<KV_NVFP4, 1>(D, p, stream) : by_d<KV_NVFP4, 2>(D, p, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa
