// Device-side helpers shared by the gfx950 paged-attention kernels:
// element types of the KV cache, raw vector loads, element conversion, and
// wavefront reductions built on DPP lane permutes (64-lane waves, rows of 16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// KV_FP8: OCP E4M3 codes; KV_NVFP4: E2M1 code pairs + E4M3 scale per 16 elements
enum KvType : int { KV_F32 = 0, KV_BF16 = 1, KV_I8 = 2, KV_FP8 = 3, KV_NVFP4 = 4 };

constexpr int kBlockSize = 16;  // tokens per KV block
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int KVT>
struct Elt {
    static constexpr int bytes = KVT == KV_F32 ? 4 : (KVT == KV_BF16 ? 2 : 1);  // NVFP4: see nvfp4_row_bytes
};

// NVFP4 block of 16 tokens and Hkv heads (9 Hkv D bytes): the code rows of
// its 16 Hkv (token, head) pairs, D/2 bytes each in (token, head) order with
// element 2i in the low nibble of byte i, then one plane of D bytes per head
// holding that head's E4M3 block scales, the scale of elements 16k .. 16k+15
// of token t = 4q + r at byte 16k + 4r + q. Rows are 64-byte aligned for
// D >= 128 and each head's scales of a block are one contiguous run, so no
// 64-byte fetch is split between rows or between codes and scales; the
// (r, q) order gives each lane of the decode its scales in one load.
__host__ __device__ constexpr int nvfp4_row_bytes(int D) { return D / 2 + D / 16; }  // per (token, head)
__host__ __device__ constexpr int nvfp4_scale_byte(int t, int k) { return 16 * k + 4 * (t & 3) + (t >> 2); }

// Code bytes of one cache row of D elements (the row stride within a block).
template <int KVT>
__host__ __device__ constexpr int kv_code_row_bytes(int D) {
    return KVT == KV_NVFP4 ? D / 2 : D * Elt<KVT>::bytes;
}

// Storage bytes per (token, kv head); a block is 16 Hkv times this.
template <int KVT>
__host__ __device__ constexpr int kv_row_bytes(int D) {
    return KVT == KV_NVFP4 ? nvfp4_row_bytes(D) : D * Elt<KVT>::bytes;
}

// ---------------------------------------------------------------- raw loads
// Load NB bytes (NB in {2, 4, 8, 16, 32, 64}) from a 16-byte-aligned (NB>=16)
// or NB-aligned address into dwords; a 2-byte load fills the low half.
template <int NB>
struct Raw {
    static constexpr int kDwords = NB >= 4 ? NB / 4 : 1;
    uint32_t w[kDwords];
};

template <typename T, bool NT>
__device__ __forceinline__ T ld(const T* p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

// NT: nontemporal (streaming) loads, for data read exactly once; they keep
// the caches free for everything else and reach a higher HBM read rate.
template <int NB, bool NT = false>
__device__ __forceinline__ void load_raw(Raw<NB>& r, const void* p) {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
    if constexpr (NB >= 16) {
        const u32x4* s = reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < NB / 16; ++i) {
            const u32x4 v = ld<u32x4, NT>(s + i);
            r.w[4 * i + 0] = v.x;
            r.w[4 * i + 1] = v.y;
            r.w[4 * i + 2] = v.z;
            r.w[4 * i + 3] = v.w;
        }
    } else if constexpr (NB == 8) {
        const u32x2 v = ld<u32x2, NT>(reinterpret_cast<const u32x2*>(p));
        r.w[0] = v.x;
        r.w[1] = v.y;
    } else if constexpr (NB == 4) {
        r.w[0] = ld<uint32_t, NT>(reinterpret_cast<const uint32_t*>(p));
    } else if constexpr (NB == 2) {
        r.w[0] = ld<uint16_t, NT>(reinterpret_cast<const uint16_t*>(p));
    } else {
        static_assert(NB == 1, "unsupported load width");
        r.w[0] = ld<uint8_t, NT>(reinterpret_cast<const uint8_t*>(p));
    }
}

// Buffer resource over one contiguous byte range (a KV block, a block's
// scales): loads then take a 32-bit per-lane offset plus a uniform offset, so
// the 64-bit address arithmetic is done once per block on the scalar unit
// instead of per load on the vector ALU. Word 3 is the gfx9 raw-buffer format
// (32-bit data, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Nontemporal load of NB bytes at rsrc + voff + soff (voff per lane, soff uniform).
template <int NB>
__device__ __forceinline__ void load_buf(Raw<NB>& r, __amdgpu_buffer_rsrc_t rs, int voff, int soff) {
    typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
    typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
    constexpr int kNT = 2;  // cache policy: nontemporal
    if constexpr (NB >= 16) {
#pragma unroll
        for (int i = 0; i < NB / 16; ++i) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16 * i, soff, kNT);
            r.w[4 * i + 0] = v.x;
            r.w[4 * i + 1] = v.y;
            r.w[4 * i + 2] = v.z;
            r.w[4 * i + 3] = v.w;
        }
    } else if constexpr (NB == 8) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, kNT);
        r.w[0] = v.x;
        r.w[1] = v.y;
    } else if constexpr (NB == 4) {
        r.w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, kNT);
    } else if constexpr (NB == 2) {
        r.w[0] = __builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, kNT);
    } else {
        static_assert(NB == 1, "unsupported load width");
        r.w[0] = __builtin_amdgcn_raw_buffer_load_b8(rs, voff, soff, kNT);
    }
}

// Element e of a raw vector as fp32 (int8: the code itself, exact).
template <int KVT, int NB>
__device__ __forceinline__ float elem_f32(const Raw<NB>& r, int e) {
    if constexpr (KVT == KV_F32) {
        return __uint_as_float(r.w[e]);
    } else if constexpr (KVT == KV_BF16) {
        uint32_t w = r.w[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    } else {
        return (float)(int8_t)(r.w[e >> 2] >> (8 * (e & 3)));
    }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// ------------------------------------------------------------ FP8 (E4M3)
typedef __attribute__((ext_vector_type(2))) float pa_f32x2;

// Two OCP E4M3 codes of w as fp32 (bytes 0, 1, or with HI bytes 2, 3);
// exact for every finite code. (gfx950's fp8 -> 16-bit conversions are not
// used: a probe of all 256 codes found their second element wrong.)
template <bool HI>
__device__ __forceinline__ pa_f32x2 fp8x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

// Two FP4 E2M1 codes of w (byte SEL: element 2 SEL in the low nibble, 2 SEL + 1
// in the high nibble) as fp32, exact. The conversion's scale operand takes
// only a power of two (probed), so block scales are applied separately.
template <int SEL>
__device__ __forceinline__ pa_f32x2 fp4x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Two FP4 E2M1 codes of w (byte SEL, as above) as a bf16 or an f16 pair (low
// half from the low nibble), exact for every code byte except that a negative
// zero comes out positive (probed over all 256 bytes); no sum of products can
// tell the two zeros apart.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_f16x2(uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL));
}

// The value of one E4M3 code (the low byte of b), exact.
__device__ __forceinline__ float fp8_value(uint32_t b) { return fp8x2_to_f32<false>(b).x; }

// fp32 -> FP4 E2M1 code (0..15): nearest magnitude of {0, 0.5, 1, 1.5, 2, 3,
// 4, 6}, ties to the even code, sign from y, saturating at 6. The magnitude
// code counts the decision points |y| has passed; at the tie points (0.25,
// 0.75, ...) the comparison is strict or not so that the even code wins.
__device__ __forceinline__ uint32_t f32_to_e2m1(float y) {
    const float a = fabsf(y);
    const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
                       (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
    return m | (__float_as_uint(y) >> 31 << 3);
}

// Four fp32 values -> four OCP E4M3 codes (byte i = code of v[i]), nearest
// even, saturating at +-448: the hardware pack rounds to nearest even but
// sends magnitudes from 464 up to NaN, so the inputs are clamped first.
__device__ __forceinline__ uint32_t f32x4_to_fp8x4(float a, float b, float c, float d) {
    a = fminf(fmaxf(a, -448.0f), 448.0f);
    b = fminf(fmaxf(b, -448.0f), 448.0f);
    c = fminf(fmaxf(c, -448.0f), 448.0f);
    d = fminf(fmaxf(d, -448.0f), 448.0f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ------------------------------------------------------------ lane permutes
// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i inside each half row
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i inside each row

// Every control used here names a source lane inside the lane's own row, so
// no lane keeps an old value: a plain DPP move (no zero-initialised
// destination needed), which also fuses into a following add.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over the 16 lanes of a row; every lane of the row gets the same bits
// (each step adds two partial sums whose order does not change the result).
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp_f32<kDppQuadXor1>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppRowHalfMirror>(x);
    x += dpp_f32<kDppRowMirror>(x);
    return x;
}

__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp_f32<kDppQuadXor1>(x));
    x = fmaxf(x, dpp_f32<kDppQuadXor2>(x));
    x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
    x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
    return x;
}

__device__ __forceinline__ float wave_max(float x) {
    x = row_max16(x);
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
    x = row_sum16(x);
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ float exp2_guarded(float x) {  // exp2 with exp2(-inf) = 0
    return x == -INFINITY ? 0.0f : exp2f(x);
}

// Softmax weight 2^x for x <= 8 (log2 units against the running reference):
// the hardware v_exp_f32 (1 ulp; 2^-inf = 0; results below 2^-126 are
// negligible against the reference's weight 1).
__device__ __forceinline__ float exp2_weight(float x) { return __builtin_amdgcn_exp2f(x); }

// Two finite floats -> packed bf16 pair (round to nearest even), one
// v_cvt_pk_bf16_f32 on gfx950; a in the low half.
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
    typedef __attribute__((ext_vector_type(2))) float f2;
    typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){a, b}, bf2));
}

}  // namespace pa
