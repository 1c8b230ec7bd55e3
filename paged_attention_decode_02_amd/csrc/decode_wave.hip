// Split-K paged decode on the vector ALUs for bf16, int8 and FP8 (OCP E4M3)
// KV caches (query groups below an MFMA tile).
//
// A workgroup of four 64-lane waves handles one split-K partition of P tokens
// of hpg kv heads (1, 2 or 4), one query token t of one sequence b, and GT
// query heads of each kv head's group, so every K/V byte is read once for all
// GT heads (grouped-query attention). The 4 / hpg waves of a kv head take
// every (4 / hpg)-th block of the partition, each with its own softmax state,
// merged through LDS at the end. With hpg = 4 a workgroup reads whole token
// rows (all kv heads) of each block, and workgroups of every kv head do the
// same work (the heads' byte offsets in a row map to memory channels
// differently; one head per workgroup made some workgroups 15% slower). The
// split-K decode keeps per-partition softmax statistics (vllm-sm70 page,
// "Why", Attention bullet: split-K paged decode with an int8 KV cache); the
// log-sum-exp reduce merges partitions. Per 16-token KV block:
//
// QK. Row r (16 lanes) of the wave takes tokens r, r+4, r+8, r+12 ("slots");
// lane c of a row holds D/16 consecutive elements of a key row, so a row
// reads whole contiguous key rows. Partial dot products use v_dot2 (bf16
// pairs against bf16 queries; for int8, codes turned into f16 by a byte
// permute against f16 queries scaled by a power of two; for FP8, codes
// widened to fp32 pairs by the hardware conversion and packed to bf16, exact,
// against bf16 queries). The 4 slots x GT
// heads partial sums are then reduced across the row by a *transposed*
// butterfly: four DPP steps (row_mirror, row_half_mirror, quad xor 2, quad
// xor 1) each add a partner lane's half of the items, so that afterwards each
// lane owns whole scores of distinct (token, head) items instead of every
// lane holding every score. This works because the lanes' registers are laid
// out with the halves swapped between partners: which token a K register holds
// (load address) and which head a q register holds (query load) depend on
// the lane's coordinates in the basis {15, 7, 2, 1} of the four DPP pairings.
//
// Softmax. Scores are in log2 units against a per-head reference m that is
// raised only when some score exceeds it by more than 2^8 (then o and l are
// rescaled); otherwise p = exp2(s - m) <= 256 and the result is exact anyway
// because o and l share the reference. Each exp is computed once.
//
// PV. The probabilities go through a small per-wave LDS buffer, as 16-bit
// pairs of consecutive tokens, to the PV layout, in which a group of lanes
// takes one whole value row (16-byte loads for 512-byte rows, else one row
// per wave) and each lane owns its row slice's output elements for all GT
// heads. Both cache types use v_dot2 over pairs of tokens: bf16 values
// against bf16 weights (the output is normalised by the sum of the same
// rounded weights, so it stays a convex combination of value rows; the LSE
// uses the exact sum); int8 codes as (1024 + code + 128) f16 pairs against
// f16 weights times the value scale, with 1152 * sum(p) subtracted once at
// the end; FP8 values as exact f16 pairs against f16 weights times the value
// scale.
//
// Loads are ping-ponged: the V block is requested before the QK of the same
// block, the next K block before the PV, so one half-block is always in
// flight per wave.
#include <type_traits>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

typedef __attribute__((ext_vector_type(2))) _Float16 half2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf162_t;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a), __builtin_bit_cast(bf162_t, b), c, false);
}

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c, false);
}

// First product of a dot-product chain. The VOP3P encoding takes the zero
// accumulator as an inline constant; written as dot2(a, b, 0.0f) the compiler
// zeroes a register and uses the accumulate-in-place encoding, one more
// instruction per chain.
__device__ __forceinline__ float dot2_bf16_first(uint32_t a, uint32_t b) {
    float r;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ float dot2_f16_first(uint32_t a, uint32_t b) {
    float r;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Two floats as an f16 pair, rounded toward zero (exact for the values
// packed here).
__device__ __forceinline__ half2_t pkrtz_h2(float a, float b) {
    return __builtin_bit_cast(half2_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

constexpr uint32_t kMagic = 0x64646464u;  // f16 0x64xx = 1024 + xx
constexpr float kCodeBias = 1152.0f;      // 1024 + 128

// Bytes 0,1 (lo) or 2,3 (hi) of biased codes u (= code ^ 0x80) as f16 (1024 + u).
__device__ __forceinline__ uint32_t f16pair_lo(uint32_t u) { return __builtin_amdgcn_perm(kMagic, u, 0x04010400u); }
__device__ __forceinline__ uint32_t f16pair_hi(uint32_t u) { return __builtin_amdgcn_perm(kMagic, u, 0x04030402u); }

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
    return (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

template <int CTRL>
__device__ __forceinline__ float add_dpp(float own, float partner_src) {
    return own + dpp_f32<CTRL>(partner_src);
}

// Number of (token, head) items a lane owns after the transposed reduction,
// and how the heads were split at the two quad levels.
template <int GT>
struct Split {
    static constexpr bool kC = GT % 2 == 0;  // level C halves the heads
    static constexpr int kAfterC = kC ? GT / 2 : GT;
    static constexpr bool kD = kAfterC % 2 == 0;  // level D halves them again
    static constexpr int kItems = kD ? kAfterC / 2 : kAfterC;
};

// Head held in q register h by a lane with quad coordinates (cc, dd).
template <int GT>
__device__ __forceinline__ int head_of(int h, int cc, int dd) {
    if constexpr (Split<GT>::kC) {
        constexpr int H2 = GT / 2;
        int half = (h / H2) ^ cc;
        int hh = h % H2;
        if constexpr (Split<GT>::kD) hh = (hh + (H2 / 2) * dd) % H2;
        return half * H2 + hh;
    } else {
        return h;
    }
}

}  // namespace

constexpr int kWaves = 4;  // waves per workgroup

// Wave-local ordering of LDS accesses (the wave's LDS operations execute in
// order; this only keeps the compiler from moving them across).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int KVT, int D, int GT, int QS>
__global__ __launch_bounds__(64 * kWaves) void decode_wave_kernel(DecodeParams p) {
    static_assert(KVT == KV_BF16 || KVT == KV_I8 || KVT == KV_FP8 || KVT == KV_NVFP4, "bf16, int8, fp8 or nvfp4");
    constexpr bool I8 = KVT == KV_I8;
    constexpr bool F8 = KVT == KV_FP8;
    constexpr bool F4 = KVT == KV_NVFP4;
    constexpr bool QNT = I8 || F8 || F4;  // codes with a per-(token, kv head) scale
    constexpr int E = Elt<KVT>::bytes;
    constexpr int RBC = F4 ? D / 2 : D * E;      // code bytes of a row
    constexpr int RBQ = kv_code_row_bytes<KVT>(D);  // row stride within a block (code bytes)
    constexpr int KB = RBC / 16;    // key bytes per lane per token (QK layout)
    constexpr int KW = KB / 4;      // ... in dwords
    constexpr int QW = D / 32;      // q dwords (element pairs) per head per lane
    constexpr int NI = Split<GT>::kItems;
    constexpr int GP = (GT + 3) / 4 * 4;  // padded heads per token in the LDS p buffer
    // PV layout: a lane takes VB bytes of a value row per token, LPT lanes per
    // row, TPW rows per wave step. 512-byte rows with up to 6 heads use 16-byte
    // loads (measured faster there; more heads would not fit their outputs in
    // registers), everything else one row per wave (at least 4 bytes a lane).
    constexpr int RB = RBC;  // code bytes of a row
    constexpr int VB = (RB >= 512 && GT <= 6) ? 16 : (RB / 64 > 4 ? RB / 64 : 4);  // value bytes per lane per token
    constexpr int LPT = RB / VB;
    constexpr int TPW = 64 / LPT;
    constexpr int EV = F4 ? 2 * VB : VB / E;  // value elements per lane per token
    constexpr int STEPS = kBlockSize / TPW;
    static_assert((F4 ? KB >= 2 : KB >= 4) && VB >= 4, "layout");
    static_assert(!F4 || VB == 4, "nvfp4: a lane's value codes lie in one 16-element block");
    static_assert(STEPS % 2 == 0, "PV pairs tokens");

    __shared__ __align__(16) uint32_t pbuf_all[kWaves][kBlockSize / 2 * GP];
    __shared__ __align__(16) float merge_o[kWaves][GT][D];
    __shared__ float merge_ml[kWaves][3][GT];  // m, l, sum of the 16-bit weights

    // the wave index is uniform across the wave: saying so keeps the block
    // loop, the table reads and the base addresses on the scalar unit
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    // 16-bit weight pairs [token / 2][head] (bf16, or f16 for int8 values)
    uint32_t* pbuf_u = reinterpret_cast<uint32_t*>(pbuf_all[wv]);
    const int r = lane >> 4, c16 = lane & 15;
    // coordinates of the lane in the basis of the DPP pairings {15, 7, 2, 1}
    const int b0 = c16 & 1, b1 = (c16 >> 1) & 1, b2 = (c16 >> 2) & 1, b3 = (c16 >> 3) & 1;
    const int ca = b3, cb = b2 ^ b3, cc = b1 ^ b2, cd = b0 ^ b2;
    const int sx = 2 * ca + cb;      // slot swap pattern of this lane
    const int my_tok = 4 * sx + r;   // token (within a block) of the items this lane owns
    const int vgrp = lane / LPT, vl = lane % LPT;  // PV layout
    // token of wave step st for this lane: steps 2k and 2k + 1 take adjacent
    // tokens (one 16-bit weight pair in LDS), the TPW lane groups interleave
    auto tok_of = [&](int st) { return 2 * TPW * (st >> 1) + 2 * vgrp + (st & 1); };

    // kv head of this wave and its place among the head's WPH waves
    const int WPH = kWaves / p.hpg;
    const int sub = wv % WPH;
    int wg = blockIdx.x;
    const int part = wg % p.NP;
    wg /= p.NP;
    const int chunk = wg % p.nchunk;
    wg /= p.nchunk;
    const int ngrp = p.Hkv / p.hpg;
    const int g = (wg % ngrp) * p.hpg + wv / WPH;
    wg /= ngrp;
    const int t = wg % p.Tq;
    const int b = wg / p.Tq;

    // keys visible to query token t, counted from the sequence's token kv_begin
    // (per-head tables: row b Hkv + g of the table and lengths; one kv head
    // per workgroup then)
    const int hrow = p.head_tables ? b * p.Hkv + g : b;
    const int n = p.seq_lens[hrow] - p.kv_begin - p.Tq + t + 1;
    const int start = part * p.P;
    const int64_t wpart = p.part_base + part;  // workspace partition
    const int hbase = g * p.G + chunk * GT;
    const int nh = min(GT, p.G - chunk * GT);
    const int64_t rowbase = ((int64_t)b * p.Tq + t) * p.Hq + hbase;  // flat row id of head hbase
    if (start >= n) {
        if (p.np_stride == 1) {
            for (int r2 = 0; r2 < nh; ++r2) {
                for (int d = sub * 64 + lane; d < D; d += 64 * WPH) {
                    if (p.out_bf16)
                        reinterpret_cast<uint16_t*>(p.out)[(rowbase + r2) * D + d] = 0;
                    else
                        reinterpret_cast<float*>(p.out)[(rowbase + r2) * D + d] = 0.0f;
                }
                if (p.lse != nullptr && sub == 0 && lane == 0) p.lse[rowbase + r2] = -INFINITY;
            }
        } else if (p.fill_empty && sub == 0 && lane < nh) {
            p.ws_lse[(rowbase + lane) * p.np_stride + wpart] = -INFINITY;
        }
        return;
    }
    const int end = min(start + p.P, n);

    // ---------------------------------------------------------------- queries
    // q register h holds head head_of(h) for the lane's D/16 elements.
    uint32_t qv[GT][QW];
    uint32_t ql[QS == 2 ? GT : 1][QW];
    float qpost;  // factor turning a reduced dot product into log2 units
    float corr[NI];  // int8: 1152 * sum_d q'[head], in the item layout
    {
        // raw loads of the lane's D/16 query elements of each head (16-byte or
        // smaller vector loads); heads past the group are loaded from head 0
        // of the chunk and zeroed
        constexpr int QB = (D / 16) * (QS == 1 ? 2 : 4);
        float qf[GT][2 * QW];
        float qmax = 0.0f;
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            const int hh = head_of<GT>(h, cc, cd);
            const bool valid = hh < nh;
            const int64_t off = (rowbase + (valid ? hh : 0)) * D + c16 * (D / 16);
            Raw<QB> raw;
            if constexpr (QS == 1)
                load_raw<QB>(raw, reinterpret_cast<const uint16_t*>(p.q) + off);
            else
                load_raw<QB>(raw, reinterpret_cast<const float*>(p.q) + off);
#pragma unroll
            for (int e = 0; e < 2 * QW; ++e) {
                const float v = QS == 1 ? elem_f32<KV_BF16>(raw, e) : elem_f32<KV_F32>(raw, e);
                qf[h][e] = valid ? v : 0.0f;
                qmax = fmaxf(qmax, fabsf(qf[h][e]));
            }
            if constexpr (!I8 && QS == 1) {
#pragma unroll
                for (int i = 0; i < QW; ++i) qv[h][i] = valid ? raw.w[i] : 0u;  // already bf16 pairs
            }
        }
        if constexpr (I8) {
            // one power-of-two scale for all heads puts max|q| in [2^14, 2^15)
            qmax = wave_max(qmax);
            const int e2 = qmax > 0.0f ? 14 - ilogbf(qmax) : 0;
            const float sc = ldexpf(1.0f, e2);
            qpost = ldexpf(p.qk_scale_log2, -e2);
            float qs[GT];
#pragma unroll
            for (int h = 0; h < GT; ++h) {
                qs[h] = 0.0f;
#pragma unroll
                for (int i = 0; i < QW; ++i) {
                    const float x0 = qf[h][2 * i] * sc, x1 = qf[h][2 * i + 1] * sc;
                    const uint32_t hi = pack_f16(x0, x1);
                    qv[h][i] = hi;
                    const half2_t hh = __builtin_bit_cast(half2_t, hi);
                    float s = (float)hh.x + (float)hh.y;
                    if constexpr (QS == 2) {
                        const uint32_t lo = pack_f16(x0 - (float)hh.x, x1 - (float)hh.y);
                        ql[h][i] = lo;
                        const half2_t ll = __builtin_bit_cast(half2_t, lo);
                        s += (float)ll.x + (float)ll.y;
                    }
                    qs[h] += s;
                }
                // plain sums over the slot levels (heads do not change there)
                qs[h] += dpp_f32<kDppRowMirror>(qs[h]);
                qs[h] += dpp_f32<kDppRowHalfMirror>(qs[h]);
            }
            // head levels exactly as for the scores
            float c2[GT];
#pragma unroll
            for (int h = 0; h < GT; ++h) c2[h] = qs[h];
            if constexpr (Split<GT>::kC) {
#pragma unroll
                for (int h = 0; h < GT / 2; ++h) c2[h] = add_dpp<kDppQuadXor2>(c2[h], c2[h + GT / 2]);
            } else {
#pragma unroll
                for (int h = 0; h < GT; ++h) c2[h] = add_dpp<kDppQuadXor2>(c2[h], c2[h]);
            }
            constexpr int AC = Split<GT>::kAfterC;
            if constexpr (Split<GT>::kD) {
#pragma unroll
                for (int h = 0; h < AC / 2; ++h) c2[h] = add_dpp<kDppQuadXor1>(c2[h], c2[h + AC / 2]);
            } else {
#pragma unroll
                for (int h = 0; h < AC; ++h) c2[h] = add_dpp<kDppQuadXor1>(c2[h], c2[h]);
            }
#pragma unroll
            for (int j = 0; j < NI; ++j) corr[j] = kCodeBias * c2[j];
        } else {
            qpost = p.qk_scale_log2;
            if constexpr (QS == 2) {
#pragma unroll
                for (int h = 0; h < GT; ++h) {
#pragma unroll
                    for (int i = 0; i < QW; ++i) {
                        const float x0 = qf[h][2 * i], x1 = qf[h][2 * i + 1];
                        const uint32_t hi = pack_bf16(x0, x1);
                        qv[h][i] = hi;
                        ql[h][i] = pack_bf16(x0 - bf16_to_f32((uint16_t)hi), x1 - bf16_to_f32((uint16_t)(hi >> 16)));
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < NI; ++j) corr[j] = 0.0f;
        }
    }

    // heads of the lane's items
    int ihead[NI];
#pragma unroll
    for (int j = 0; j < NI; ++j) ihead[j] = head_of<GT>(j, cc, cd);

    // ------------------------------------------------------- partition state
    float mref[GT];  // per-head reference (log2 units), uniform across the wave
    float mloc[NI];  // mref of the lane's item heads
    float lloc[NI];  // partial sums of p over the lane's items
    float sloc[NI];  // partial sums of the 16-bit weights (int8: times the value scales)
    float o[GT][EV];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        mref[h] = -INFINITY;
#pragma unroll
        for (int e = 0; e < EV; ++e) o[h][e] = 0.0f;
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        mloc[j] = -INFINITY;
        lloc[j] = 0.0f;
        sloc[j] = 0.0f;
    }

    const int32_t* table = p.block_table + (int64_t)hrow * p.max_blocks + p.kv_begin / kBlockSize;
    // KV addressing: a buffer resource per block (scalar) plus per-lane
    // offsets that do not change from block to block; the host keeps a
    // block's bytes below 2^31
    const int tok_stride = p.Hkv * RBQ;  // bytes between consecutive tokens of a block
    const int blk_bytes = kBlockSize * p.Hkv * kv_row_bytes<KVT>(D);  // nvfp4: + the scale planes
    const char* kcache = reinterpret_cast<const char*>(p.k_cache);
    const char* vcache = reinterpret_cast<const char*>(p.v_cache);
    const int j0 = start / kBlockSize, jend = (end + kBlockSize - 1) / kBlockSize;

    // int8 / fp8: value probabilities are scaled by 2^vsh so that
    // p * v_scale * 2^vsh stays below 2^15 (f16) for every token of the
    // partition (p <= 2^8)
    float vsh = 1.0f, vsh_inv = 1.0f;
    if constexpr (QNT) {
        float vmax = 0.0f;
        for (int j = j0 + sub + WPH * (lane >> 4); j < jend; j += 4 * WPH) {
            const int64_t ph = table[j];
            const float sv = p.v_scale[(ph * p.Hkv + g) * kBlockSize + c16];
            const int pos = j * kBlockSize + c16;
            if (pos < end) vmax = fmaxf(vmax, sv);
        }
        vmax = wave_max(vmax);
        const int e2 = vmax > 0.0f ? 6 - ilogbf(vmax) : 0;
        vsh = ldexpf(1.0f, e2);
        vsh_inv = ldexpf(1.0f, -e2);
    }

    // K registers: register s holds slot s ^ sx (token 4 * (s ^ sx) + r)
    Raw<KB> kr[4];
    Raw<VB> vr[STEPS];
    // nvfp4 block scales (E4M3 codes). A lane's D/16 key elements and 2 VB
    // value elements each lie in one 16-element block k; in the head's scale
    // plane of a block, byte 16 k + 4 r' + q' is token 4 q' + r', so the
    // lane's keys (tokens 4 q' + r, q' = slot ^ sx) are the dword at 16 k + 4 r
    // and its values (tokens 2 TPW (st >> 1) + 2 vgrp + (st & 1)) the bytes
    // TPW/2 (st >> 1) + (vgrp >> 1) of the two dwords at 16 k + 8 (vgrp & 1)
    Raw<4> ksw;
    Raw<8> vsw;
    int koff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) koff[s] = (4 * (s ^ sx) + r) * tok_stride + g * RBQ + c16 * KB;
    const int voff = 2 * vgrp * tok_stride + g * RBQ + vl * VB;  // + the step's uniform token offset
    const int plane = kBlockSize * tok_stride + g * D;  // this head's block scales
    const int ksw_off = plane + 16 * (c16 * KB / 8) + 4 * r;
    const int vsw_off = plane + 16 * (vl * VB / 8) + 8 * (vgrp & 1);
    // byte s of perm(ksw, ksw, ksel) is byte s ^ sx of ksw (slot s's scale)
    const uint32_t ksel = 0x03020100u ^ (0x01010101u * (uint32_t)sx);
    const int soff = (g * kBlockSize + my_tok) * 4;  // scale of the lane's token within a block's scales
    const int jw = j0 + sub;  // this wave's first block; it takes every WPH-th block
    int64_t phys = jw < jend ? (int64_t)table[jw] : 0;
    auto load_k = [&](int64_t ph) {
        const auto rs = range_rsrc(kcache + ph * blk_bytes, blk_bytes);
#pragma unroll
        for (int s = 0; s < 4; ++s) load_buf<KB>(kr[s], rs, koff[s], 0);
        if constexpr (F4) load_buf<4>(ksw, rs, ksw_off, 0);
    };
    auto load_v = [&](int64_t ph) {
        const auto rs = range_rsrc(vcache + ph * blk_bytes, blk_bytes);
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
            load_buf<VB>(vr[st], rs, voff, (2 * TPW * (st >> 1) + (st & 1)) * tok_stride);
        if constexpr (F4) load_buf<8>(vsw, rs, vsw_off, 0);
    };
    if (jw < jend) load_k(phys);

    // one block of the wave; MORE: a later block follows, whose keys are
    // requested during this one (the last block is peeled off, so no load is
    // ever issued under a branch and none reads past the partition)
    auto block = [&](int j, auto more) {
        constexpr bool MORE = decltype(more)::value;
        const int pos0 = j * kBlockSize;
        // int8 / fp8 scales of the lane's token first: a load issued after
        // the prefetches would make its wait drain them (in-order counting)
        float kscale_raw = 1.0f, vscale_raw = 1.0f;
        if constexpr (QNT) {
            const int64_t first = phys * kBlockSize * p.Hkv;  // the block's first scale
            const int sbytes = kBlockSize * p.Hkv * 4;
            Raw<4> ks, vs;
            load_buf<4>(ks, range_rsrc(p.k_scale + first, sbytes), soff, 0);
            load_buf<4>(vs, range_rsrc(p.v_scale + first, sbytes), soff, 0);
            kscale_raw = __uint_as_float(ks.w[0]);
            vscale_raw = __uint_as_float(vs.w[0]);
        }
        load_v(phys);
        int64_t phys_next = phys;
        if constexpr (MORE) phys_next = (int64_t)table[j + WPH];

        // ---------------------------------------------------------------- QK
        float kscl[4] = {1.0f, 1.0f, 1.0f, 1.0f};  // nvfp4: block scale of the lane's keys per slot
        if constexpr (F4) {
            const uint32_t kp = __builtin_amdgcn_perm(ksw.w[0], ksw.w[0], ksel);
            const pa_f32x2 lo = fp8x2_to_f32<false>(kp), hi = fp8x2_to_f32<true>(kp);
            kscl[0] = lo.x;
            kscl[1] = lo.y;
            kscl[2] = hi.x;
            kscl[3] = hi.y;
        }
        float ps[4][GT];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int h = 0; h < GT; ++h) {
                float acc;
                if constexpr (I8) {
#pragma unroll
                    for (int w = 0; w < KW; ++w) {
                        const uint32_t u = kr[s].w[w] ^ 0x80808080u;
                        acc = w == 0 ? dot2_f16_first(qv[h][0], f16pair_lo(u)) : dot2_f16(qv[h][2 * w], f16pair_lo(u), acc);
                        acc = dot2_f16(qv[h][2 * w + 1], f16pair_hi(u), acc);
                        if constexpr (QS == 2) {
                            acc = dot2_f16(ql[h][2 * w], f16pair_lo(u), acc);
                            acc = dot2_f16(ql[h][2 * w + 1], f16pair_hi(u), acc);
                        }
                    }
                } else if constexpr (F4) {
                    // code byte b -> elements 2b, 2b + 1 as an exact bf16 pair;
                    // the block scale multiplies the lane's partial sum
#pragma unroll
                    for (int b2 = 0; b2 < KB; ++b2) {
                        const uint32_t wd = kr[s].w[b2 / 4];
                        const uint32_t kp = (b2 & 3) == 0 ? fp4x2_to_bf16x2<0>(wd)
                                            : (b2 & 3) == 1 ? fp4x2_to_bf16x2<1>(wd)
                                            : (b2 & 3) == 2 ? fp4x2_to_bf16x2<2>(wd)
                                                            : fp4x2_to_bf16x2<3>(wd);
                        acc = b2 == 0 ? dot2_bf16_first(qv[h][0], kp) : dot2_bf16(qv[h][b2], kp, acc);
                        if constexpr (QS == 2) acc = dot2_bf16(ql[h][b2], kp, acc);
                    }
                    acc *= kscl[s];
                } else if constexpr (F8) {
#pragma unroll
                    for (int w = 0; w < KW; ++w) {
                        // four codes -> two exact bf16 pairs (elements 4w .. 4w + 3)
                        const pa_f32x2 lo = fp8x2_to_f32<false>(kr[s].w[w]);
                        const pa_f32x2 hi = fp8x2_to_f32<true>(kr[s].w[w]);
                        const uint32_t k01 = pack_bf16_rne(lo.x, lo.y), k23 = pack_bf16_rne(hi.x, hi.y);
                        acc = w == 0 ? dot2_bf16_first(qv[h][0], k01) : dot2_bf16(qv[h][2 * w], k01, acc);
                        acc = dot2_bf16(qv[h][2 * w + 1], k23, acc);
                        if constexpr (QS == 2) {
                            acc = dot2_bf16(ql[h][2 * w], k01, acc);
                            acc = dot2_bf16(ql[h][2 * w + 1], k23, acc);
                        }
                    }
                } else {
#pragma unroll
                    for (int w = 0; w < KW; ++w) {
                        acc = w == 0 ? dot2_bf16_first(qv[h][0], kr[s].w[0]) : dot2_bf16(qv[h][w], kr[s].w[w], acc);
                        if constexpr (QS == 2) acc = dot2_bf16(ql[h][w], kr[s].w[w], acc);
                    }
                }
                ps[s][h] = acc;
            }
        }
        // next block's keys go out now; they are not needed before the next QK
        if constexpr (MORE) load_k(phys_next);

        // transposed reduction across the row
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int h = 0; h < GT; ++h) ps[s][h] = add_dpp<kDppRowMirror>(ps[s][h], ps[s + 2][h]);
#pragma unroll
        for (int h = 0; h < GT; ++h) ps[0][h] = add_dpp<kDppRowHalfMirror>(ps[0][h], ps[1][h]);
        float x[GT];
#pragma unroll
        for (int h = 0; h < GT; ++h) x[h] = ps[0][h];
        if constexpr (Split<GT>::kC) {
#pragma unroll
            for (int h = 0; h < GT / 2; ++h) x[h] = add_dpp<kDppQuadXor2>(x[h], x[h + GT / 2]);
        } else {
#pragma unroll
            for (int h = 0; h < GT; ++h) x[h] = add_dpp<kDppQuadXor2>(x[h], x[h]);
        }
        constexpr int AC = Split<GT>::kAfterC;
        if constexpr (Split<GT>::kD) {
#pragma unroll
            for (int h = 0; h < AC / 2; ++h) x[h] = add_dpp<kDppQuadXor1>(x[h], x[h + AC / 2]);
        } else {
#pragma unroll
            for (int h = 0; h < AC; ++h) x[h] = add_dpp<kDppQuadXor1>(x[h], x[h]);
        }

        // scores of the lane's items, log2 units; masked past the end
        // a block followed by another of this wave (MORE) is not the
        // partition's last and lies wholly before its end, which for this
        // workgroup's one query token is also the causal limit
        const bool tok_ok = MORE || pos0 + my_tok < end;
        float ksc = qpost;
        if constexpr (QNT) ksc *= kscale_raw;
        float sc[NI];
        bool raise = false;
#pragma unroll
        for (int j2 = 0; j2 < NI; ++j2) {
            const bool ok = tok_ok && ihead[j2] < nh;
            sc[j2] = ok ? (x[j2] - corr[j2]) * ksc : -INFINITY;
            raise |= sc[j2] > mloc[j2] + 8.0f;
        }

        // ------------------------------------------- raise the references (rare)
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
            for (int h = 0; h < GT; ++h) {
                float v = -INFINITY;
#pragma unroll
                for (int j2 = 0; j2 < NI; ++j2) v = ihead[j2] == h ? fmaxf(v, sc[j2]) : v;
                const float bm = wave_max(v);
                const float mn = fmaxf(mref[h], bm);
                const float base = mn == -INFINITY ? 0.0f : mn;
                const float alpha = exp2_guarded(mref[h] - base);
                mref[h] = mn;
#pragma unroll
                for (int e = 0; e < EV; ++e) o[h][e] *= alpha;
#pragma unroll
                for (int j2 = 0; j2 < NI; ++j2) {
                    if (ihead[j2] == h) {
                        lloc[j2] *= alpha;
                        sloc[j2] *= alpha;
                        mloc[j2] = mn;
                    }
                }
            }
        }

        // ------------------------------------------------- probabilities -> LDS
        float sv = 1.0f;
        if constexpr (QNT) sv = vscale_raw * vsh;
#pragma unroll
        for (int j2 = 0; j2 < NI; ++j2) {
            const float base = mloc[j2] == -INFINITY ? 0.0f : mloc[j2];
            const float pr = exp2_weight(sc[j2] - base);  // sc = -inf gives 0
            uint16_t* slot16 = reinterpret_cast<uint16_t*>(pbuf_u) + ((my_tok >> 1) * GP + ihead[j2]) * 2 + (my_tok & 1);
            if constexpr (QNT) {
                lloc[j2] += pr;
                const _Float16 ph = (_Float16)(tok_ok ? pr * sv : 0.0f);
                sloc[j2] += (float)ph;
                *slot16 = __builtin_bit_cast(uint16_t, ph);
            } else {
                // bf16 weight (round to nearest even). l keeps the exact
                // weights (for the LSE); the output is normalised by the sum
                // of the rounded ones, so it stays a convex combination of
                // value rows
                const uint32_t pb = pack_bf16_rne(pr, 0.0f) & 0xFFFFu;
                lloc[j2] += pr;
                sloc[j2] += __uint_as_float(pb << 16);
                *slot16 = (uint16_t)pb;
            }
        }
        wave_lds_sync();

        // ---------------------------------------------------------------- PV
        // tokens past the end may hold anything (bf16: NaN or Inf times a zero
        // weight; fp8: NaN codes); int8 codes are always finite
        // nvfp4: step st's value scale in byte TPW/2 (st >> 1) of vs[st & 1]
        uint32_t vs[2] = {0u, 0u};
        if constexpr (F4) {
            const int sh = TPW > 2 ? 8 * (vgrp >> 1) : 0;
            vs[0] = vsw.w[0] >> sh;
            vs[1] = vsw.w[1] >> sh;
        }
        if constexpr (!I8) {
            if (!MORE && pos0 + kBlockSize > end) {
#pragma unroll
                for (int st = 0; st < STEPS; ++st) {
                    const bool ok = pos0 + tok_of(st) < end;
#pragma unroll
                    for (int w = 0; w < VB / 4; ++w) vr[st].w[w] = ok ? vr[st].w[w] : 0u;
                    if constexpr (F4) vs[st & 1] &= ok ? 0xFFFFFFFFu : ~(0xFFu << (8 * (TPW / 2) * (st >> 1)));
                }
            }
        }
        // nvfp4: the scales of step pair (2 i, 2 i + 1) as an f16 pair (exact)
        half2_t sabs[F4 ? STEPS / 2 : 1];
        if constexpr (F4) {
#pragma unroll
            for (int i = 0; i < STEPS / 2; i += 2) {
                constexpr int T2 = TPW / 2;
                const uint32_t b0 = T2 * i, b1 = i + 1 < STEPS / 2 ? T2 * (i + 1) : 0;
                // bytes (vs[0].b0, vs[1].b0, vs[0].b1, vs[1].b1)
                const uint32_t x = __builtin_amdgcn_perm(vs[1], vs[0], b0 | (4 + b0) << 8 | b1 << 16 | (4 + b1) << 24);
                const pa_f32x2 lo = fp8x2_to_f32<false>(x);
                sabs[i] = pkrtz_h2(lo.x, lo.y);
                if (i + 1 < STEPS / 2) {
                    const pa_f32x2 hi = fp8x2_to_f32<true>(x);
                    sabs[i + 1] = pkrtz_h2(hi.x, hi.y);
                }
            }
        }
#pragma unroll
        for (int st = 0; st < STEPS; st += 2) {
            // token pair (tk, tk + 1) against a 16-bit weight pair from LDS
            const int tk = tok_of(st);
            uint32_t pp[GT];
#pragma unroll
            for (int h = 0; h < GT; ++h) pp[h] = pbuf_u[(tk >> 1) * GP + h];
#pragma unroll
            for (int w = 0; w < VB / 4; ++w) {
                const uint32_t A = vr[st].w[w];
                const uint32_t B = vr[st + 1].w[w];
                if constexpr (I8) {
                    // codes as (1024 + code + 128) f16 pairs of the two tokens
                    const uint32_t x0 = __builtin_amdgcn_perm(B, A, 0x05010400u) ^ 0x80808080u;  // a0 b0 a1 b1
                    const uint32_t x1 = __builtin_amdgcn_perm(B, A, 0x07030602u) ^ 0x80808080u;  // a2 b2 a3 b3
                    const uint32_t f0 = f16pair_lo(x0), f1 = f16pair_hi(x0);
                    const uint32_t f2 = f16pair_lo(x1), f3 = f16pair_hi(x1);
#pragma unroll
                    for (int h = 0; h < GT; ++h) {
                        o[h][4 * w + 0] = dot2_f16(pp[h], f0, o[h][4 * w + 0]);
                        o[h][4 * w + 1] = dot2_f16(pp[h], f1, o[h][4 * w + 1]);
                        o[h][4 * w + 2] = dot2_f16(pp[h], f2, o[h][4 * w + 2]);
                        o[h][4 * w + 3] = dot2_f16(pp[h], f3, o[h][4 * w + 3]);
                    }
                } else if constexpr (F4) {
                    // element e of tokens tk and tk + 1 times their block
                    // scales as an f16 pair (exact: at most 6 significant
                    // bits): the two tokens' nibbles of each element are
                    // paired in one byte (even elements in xe, odd in xo),
                    // converted as an f16 pair and multiplied by the scales
                    const half2_t sab = sabs[st >> 1];
                    const uint32_t xe = (A & 0x0F0F0F0Fu) | ((B << 4) & 0xF0F0F0F0u);
                    const uint32_t xo = ((A >> 4) & 0x0F0F0F0Fu) | (B & 0xF0F0F0F0u);
#pragma unroll
                    for (int b2 = 0; b2 < 4; ++b2) {
                        const uint32_t pe = b2 == 0 ? fp4x2_to_f16x2<0>(xe) : b2 == 1 ? fp4x2_to_f16x2<1>(xe)
                                            : b2 == 2 ? fp4x2_to_f16x2<2>(xe) : fp4x2_to_f16x2<3>(xe);
                        const uint32_t po = b2 == 0 ? fp4x2_to_f16x2<0>(xo) : b2 == 1 ? fp4x2_to_f16x2<1>(xo)
                                            : b2 == 2 ? fp4x2_to_f16x2<2>(xo) : fp4x2_to_f16x2<3>(xo);
                        const uint32_t f0 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, pe) * sab);
                        const uint32_t f1 = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, po) * sab);
#pragma unroll
                        for (int h = 0; h < GT; ++h) {
                            o[h][2 * b2 + 0] = dot2_f16(pp[h], f0, o[h][2 * b2 + 0]);
                            o[h][2 * b2 + 1] = dot2_f16(pp[h], f1, o[h][2 * b2 + 1]);
                        }
                    }
                } else if constexpr (F8) {
                    // element e of tokens tk and tk + 1 as an f16 pair (exact:
                    // every finite E4M3 value is an f16; round-toward-zero packing)
                    const pa_f32x2 a01 = fp8x2_to_f32<false>(A), a23 = fp8x2_to_f32<true>(A);
                    const pa_f32x2 b01 = fp8x2_to_f32<false>(B), b23 = fp8x2_to_f32<true>(B);
                    const uint32_t f0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a01.x, b01.x));
                    const uint32_t f1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a01.y, b01.y));
                    const uint32_t f2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a23.x, b23.x));
                    const uint32_t f3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a23.y, b23.y));
#pragma unroll
                    for (int h = 0; h < GT; ++h) {
                        o[h][4 * w + 0] = dot2_f16(pp[h], f0, o[h][4 * w + 0]);
                        o[h][4 * w + 1] = dot2_f16(pp[h], f1, o[h][4 * w + 1]);
                        o[h][4 * w + 2] = dot2_f16(pp[h], f2, o[h][4 * w + 2]);
                        o[h][4 * w + 3] = dot2_f16(pp[h], f3, o[h][4 * w + 3]);
                    }
                } else {
                    // bf16 pairs (element e of token tk, element e of token tk + 1)
                    const uint32_t e0 = __builtin_amdgcn_perm(B, A, 0x05040100u);
                    const uint32_t e1 = __builtin_amdgcn_perm(B, A, 0x07060302u);
#pragma unroll
                    for (int h = 0; h < GT; ++h) {
                        o[h][2 * w + 0] = dot2_bf16(pp[h], e0, o[h][2 * w + 0]);
                        o[h][2 * w + 1] = dot2_bf16(pp[h], e1, o[h][2 * w + 1]);
                    }
                }
            }
        }
        wave_lds_sync();
        phys = phys_next;
    };
    int j = jw;
    for (; j + WPH < jend; j += WPH) block(j, std::true_type{});
    if (j < jend) block(j, std::false_type{});

    // ------------------------------------------------------------ epilogue
    // lane groups of the PV layout hold disjoint token subsets: add them
    if constexpr (TPW > 1) {
#pragma unroll
        for (int h = 0; h < GT; ++h)
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                float v = o[h][e];
                for (int off = LPT; off < 64; off <<= 1) v += __shfl_xor(v, off);
                o[h][e] = v;
            }
    }
    float lh[GT], sh[GT];
#pragma unroll
    for (int h = 0; h < GT; ++h) {
        float v = 0.0f, w2 = 0.0f;
#pragma unroll
        for (int j2 = 0; j2 < NI; ++j2) {
            v += ihead[j2] == h ? lloc[j2] : 0.0f;
            w2 += ihead[j2] == h ? sloc[j2] : 0.0f;
        }
        // lanes that duplicate an item (plain butterfly levels) count it more than once
        lh[h] = wave_sum(v);
        sh[h] = wave_sum(w2);
    }
    // duplication factor of the plain levels
    constexpr int DUP = (Split<GT>::kC ? 1 : 2) * (Split<GT>::kD ? 1 : 2);
    // this wave's unnormalised state (values relative to 2^mref) -> LDS
    if (vgrp == 0) {
#pragma unroll
        for (int h = 0; h < GT; ++h) {
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                float acc = o[h][e];
                if constexpr (I8) acc = (acc - kCodeBias * sh[h] * (1.0f / DUP)) * vsh_inv;
                if constexpr (F8 || F4) acc *= vsh_inv;
                merge_o[wv][h][vl * EV + e] = acc;
            }
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < GT; ++h) {
            merge_ml[wv][0][h] = mref[h];
            merge_ml[wv][1][h] = lh[h] * (1.0f / DUP);
            merge_ml[wv][2][h] = sh[h] * (1.0f / DUP);
        }
    }
    __syncthreads();
    // wave sub of a kv head merges its heads sub, sub + WPH, ... over the
    // head's waves w0 .. w0 + WPH - 1: weights 2^(m_w - M) in a fixed order
    const int w0 = wv - sub;
    for (int h = sub; h < nh; h += WPH) {
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < kWaves; ++k)
            if (k < WPH) M = fmaxf(M, merge_ml[w0 + k][0][h]);
        const float base = M == -INFINITY ? 0.0f : M;
        float wt[kWaves], l = 0.0f, lr = 0.0f;
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
            wt[k] = 0.0f;
            if (k < WPH) {
                wt[k] = exp2_guarded(merge_ml[w0 + k][0][h] - base);
                l += merge_ml[w0 + k][1][h] * wt[k];
                lr += merge_ml[w0 + k][2][h] * wt[k];
            }
        }
        const float lnorm = QNT ? l : lr;  // bf16: the sum of the weights the values were multiplied by
        const float inv = lnorm > 0.0f ? 1.0f / lnorm : 0.0f;
        const float lse2 = l > 0.0f ? (M + log2f(l)) * kLn2 : -INFINITY;
        const int64_t rowid = rowbase + h;
        for (int d = lane; d < D; d += 64) {
            // merge_o[w][h] holds element d at index d (lane vl owns elements vl*EV ..)
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < kWaves; ++k)
                if (k < WPH) acc += wt[k] * merge_o[w0 + k][h][d];
            const float val = acc * inv;
            if (p.np_stride == 1) {
                if (p.out_bf16)
                    reinterpret_cast<uint16_t*>(p.out)[rowid * D + d] = f32_to_bf16(val);
                else
                    reinterpret_cast<float*>(p.out)[rowid * D + d] = val;
            } else {
                p.ws_o[(rowid * p.np_stride + wpart) * D + d] = val;
            }
        }
        if (lane == 0) {
            if (p.np_stride == 1) {
                if (p.lse != nullptr) p.lse[rowid] = lse2;
            } else {
                p.ws_lse[rowid * p.np_stride + wpart] = lse2;
            }
        }
    }
}

namespace {
template <int KVT, int D, int GT, int QS>
hipError_t launch_one(const DecodeParams& p, hipStream_t s) {
    if (p.hpg < 1 || p.hpg > kWaves || kWaves % p.hpg || p.Hkv % p.hpg) return hipErrorInvalidValue;
    const int64_t grid = (int64_t)p.NP * p.nchunk * (p.Hkv / p.hpg) * p.Tq * p.B;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_wave_kernel<KVT, D, GT, QS>), dim3((unsigned)grid), dim3(64 * kWaves), 0, s, p);
    return hipGetLastError();
}

template <int KVT, int D, int QS>
hipError_t by_gt(int GT, const DecodeParams& p, hipStream_t s) {
    switch (GT) {
    case 1: return launch_one<KVT, D, 1, QS>(p, s);
    case 2: return launch_one<KVT, D, 2, QS>(p, s);
    case 4: return launch_one<KVT, D, 4, QS>(p, s);
    case 6: return launch_one<KVT, D, 6, QS>(p, s);
    case 8: return launch_one<KVT, D, 8, QS>(p, s);
    default: return hipErrorInvalidValue;
    }
}

template <int KVT, int QS>
hipError_t by_d(int D, int GT, const DecodeParams& p, hipStream_t s) {
    switch (D) {
    case 64: return by_gt<KVT, 64, QS>(GT, p, s);
    case 128: return by_gt<KVT, 128, QS>(GT, p, s);
    case 256: return by_gt<KVT, 256, QS>(GT, p, s);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_decode_wave(int kv_type, int D, int GT, const DecodeParams& p, hipStream_t stream) {
    const int qs = p.q_bf16 ? 1 : 2;
    if (kv_type == KV_BF16) return qs == 1 ? by_d<KV_BF16, 1>(D, GT, p, stream) : by_d<KV_BF16, 2>(D, GT, p, stream);
    if (kv_type == KV_I8) return qs == 1 ? by_d<KV_I8, 1>(D, GT, p, stream) : by_d<KV_I8, 2>(D, GT, p, stream);
    if (kv_type == KV_FP8) return qs == 1 ? by_d<KV_FP8, 1>(D, GT, p, stream) : by_d<KV_FP8, 2>(D, GT, p, stream);
    if (kv_type == KV_NVFP4)
        return qs == 1 ? by_d<KV_NVFP4, 1>(D, GT, p, stream) : by_d<KV_NVFP4, 2>(D, GT, p, stream);
    return hipErrorInvalidValue;
}

}  // namespace pa
