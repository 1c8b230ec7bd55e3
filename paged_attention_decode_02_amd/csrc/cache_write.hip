// Store new tokens' key/value rows into the paged caches.
//
// The cache is the block pool of PagedAttention; the int8 variant is the
// vllm-sm70 page's int8 KV cache ("Why", Attention bullet), here symmetric
// with one fp32 scale per (token, kv head):
//   s = fp32(max|x| / 127),  code = clamp(rint_even(fp32(x / s)), -127, 127),
// and s = 0, codes 0 for an all-zero row. The FP8 variant (FP8 KV: nvllm
// page, "Acknowledgments", b12x) stores OCP E4M3 codes the same way against
// 448, the largest finite E4M3 magnitude: s = fp32(max|x| / 448), code = the
// E4M3 value nearest to fp32(x / s), ties to even, saturating. The NVFP4
// variant (the KV format of the vllm-sm12x-nvfp4-dflash2 page, "What makes
// this stack different") stores E2M1 codes with an E4M3 scale per 16
// elements and an fp32 row scale: S = fp32(max|x| / 2688), per block
// u = fp32(fp32(max|x_b| / 6) / S), s_b = E4M3(u), d_b = fp32(value(s_b) * S),
// code = the E2M1 value nearest to fp32(x / d_b), ties to even. Every
// division is correctly rounded binary32, so the codes are bit-exact.
// A negative slot skips the token (padded rows must not write into other
// requests' slots: vllm-sm70 page, "Known limitations").
//
// One wave per (token, kv head); lane c handles D/64 consecutive elements.
// The source rows are requested before the slot, so both loads are in flight
// together.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

template <int CT, int D, bool SRC_BF16>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p) {
    constexpr int EPL = D / 64;               // elements per lane
    constexpr int SB = EPL * (SRC_BF16 ? 2 : 4);  // source bytes per lane
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t pair = (int64_t)blockIdx.x * 4 + wv;  // (token, kv head)
    if (pair >= p.num_tokens * p.Hkv) return;
    const int64_t i = pair / p.Hkv;
    const int g = (int)(pair % p.Hkv);
    const int64_t src_off = (i * p.Hkv + g) * D + lane * EPL;
    Raw<SB> raw[2];
    load_raw<SB>(raw[0], reinterpret_cast<const char*>(p.k_src) + src_off * (SRC_BF16 ? 2 : 4));
    load_raw<SB>(raw[1], reinterpret_cast<const char*>(p.v_src) + src_off * (SRC_BF16 ? 2 : 4));
    const int64_t slot = p.slots[i];
    if (slot < 0) return;  // wave-uniform
    const int64_t dst_row = slot * p.Hkv + g;  // (block * 16 + offset) * Hkv + g
    // scales [num_blocks, Hkv, 16]: a kv head's scales of a block together
    const int64_t srow = ((slot / kBlockSize) * p.Hkv + g) * kBlockSize + slot % kBlockSize;
    const int64_t dst_off = dst_row * D + lane * EPL;

#pragma unroll
    for (int which = 0; which < 2; ++which) {
        void* cache = which ? p.v_cache : p.k_cache;
        float x[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) x[e] = elem_f32<SRC_BF16 ? KV_BF16 : KV_F32>(raw[which], e);
        if constexpr (CT == KV_NVFP4) {
            constexpr int LPB = 16 / EPL;  // lanes per 16-element block
            const int64_t blk = slot / kBlockSize;
            const int t = (int)(slot % kBlockSize);
            unsigned char* base = reinterpret_cast<unsigned char*>(cache) + blk * 9 * p.Hkv * D;
            unsigned char* row = base + ((int64_t)t * p.Hkv + g) * (D / 2);
            unsigned char* plane = base + (int64_t)kBlockSize * p.Hkv * (D / 2) + (int64_t)g * D;
            float la = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) la = fmaxf(la, fabsf(x[e]));
            const float amax = wave_max(la);
            float bmax = la;
#pragma unroll
            for (int off = 1; off < LPB; off <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, off));
            const float S = __fdiv_rn(amax, 2688.0f);
            uint32_t sb = 0;  // E4M3 code of the block scale
            float d = 0.0f;   // the block's effective scale
            if (amax != 0.0f) {
                sb = f32x4_to_fp8x4(__fdiv_rn(__fdiv_rn(bmax, 6.0f), S), 0.0f, 0.0f, 0.0f) & 0xFFu;
                d = __fmul_rn(fp8_value(sb), S);
            }
            uint32_t nib = 0;  // the lane's codes, element e in bits 4e .. 4e + 3
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const uint32_t c = d != 0.0f ? f32_to_e2m1(__fdiv_rn(x[e], d)) : 0u;
                nib |= c << (4 * e);
            }
            if constexpr (EPL == 4) {
                *reinterpret_cast<uint16_t*>(row + 2 * lane) = (uint16_t)nib;
            } else if constexpr (EPL == 2) {
                row[lane] = (unsigned char)nib;
            } else {  // one element per lane: lane pairs share a byte
                const uint32_t hi = __shfl_xor(nib, 1);
                if ((lane & 1) == 0) row[lane / 2] = (unsigned char)(nib | (hi << 4));
            }
            if (lane % LPB == 0) plane[nvfp4_scale_byte(t, lane / LPB)] = (unsigned char)sb;
            if (lane == 0) (which ? p.v_scale : p.k_scale)[srow] = S;
        } else if constexpr (CT == KV_F32) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) reinterpret_cast<float*>(cache)[dst_off + e] = x[e];
        } else if constexpr (CT == KV_BF16) {
            uint16_t* dst = reinterpret_cast<uint16_t*>(cache) + dst_off;
            uint32_t w[(EPL + 1) / 2];
            if constexpr (SRC_BF16) {  // bit copy
#pragma unroll
                for (int k = 0; k < (EPL + 1) / 2; ++k) w[k] = raw[which].w[k];
            } else {
#pragma unroll
                for (int k = 0; k < EPL / 2; ++k)
                    w[k] = (uint32_t)f32_to_bf16(x[2 * k]) | ((uint32_t)f32_to_bf16(x[2 * k + 1]) << 16);
                if constexpr (EPL == 1) w[0] = f32_to_bf16(x[0]);
            }
            if constexpr (EPL == 4)
                *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
            else if constexpr (EPL == 2)
                *reinterpret_cast<uint32_t*>(dst) = w[0];
            else
                *dst = (uint16_t)w[0];
        } else {
            constexpr bool F8 = CT == KV_FP8;
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
            amax = wave_max(amax);
            const float s = __fdiv_rn(amax, F8 ? 448.0f : 127.0f);
            uint32_t packed = 0;
            if constexpr (F8) {
                if (amax != 0.0f) {
                    float y[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int e = 0; e < EPL; ++e) y[e] = __fdiv_rn(x[e], s);
                    packed = f32x4_to_fp8x4(y[0], y[1], y[2], y[3]);
                    if constexpr (EPL < 4) packed &= (1u << (8 * EPL)) - 1u;
                }
            } else {
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    int c = 0;
                    if (amax != 0.0f) {
                        float r = rintf(__fdiv_rn(x[e], s));
                        r = fminf(fmaxf(r, -127.0f), 127.0f);
                        c = (int)r;
                    }
                    packed |= ((uint32_t)c & 0xFFu) << (8 * e);
                }
            }
            int8_t* dst = reinterpret_cast<int8_t*>(cache) + dst_off;
            if constexpr (EPL == 4)
                *reinterpret_cast<uint32_t*>(dst) = packed;
            else if constexpr (EPL == 2)
                *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
            else
                *dst = (int8_t)packed;
            if (lane == 0) (which ? p.v_scale : p.k_scale)[srow] = s;
        }
    }
}

namespace {
template <int CT, bool SB>
hipError_t launch_src(int D, const CacheWriteParams& p, hipStream_t s) {
    const int64_t pairs = p.num_tokens * p.Hkv;
    const int64_t grid = (pairs + 3) / 4;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    switch (D) {
    case 64: hipLaunchKernelGGL((cache_write_kernel<CT, 64, SB>), dim3((unsigned)grid), dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL((cache_write_kernel<CT, 128, SB>), dim3((unsigned)grid), dim3(256), 0, s, p); break;
    case 256: hipLaunchKernelGGL((cache_write_kernel<CT, 256, SB>), dim3((unsigned)grid), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int CT>
hipError_t launch_ct(int D, const CacheWriteParams& p, hipStream_t s) {
    return p.src_bf16 ? launch_src<CT, true>(D, p, s) : launch_src<CT, false>(D, p, s);
}
}  // namespace

hipError_t launch_cache_write(int cache_type, const CacheWriteParams& p, hipStream_t stream) {
    switch (cache_type) {
    case KV_F32: return launch_ct<KV_F32>(p.D, p, stream);
    case KV_BF16: return launch_ct<KV_BF16>(p.D, p, stream);
    case KV_I8: return launch_ct<KV_I8>(p.D, p, stream);
    case KV_FP8: return launch_ct<KV_FP8>(p.D, p, stream);
    case KV_NVFP4: return launch_ct<KV_NVFP4>(p.D, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
