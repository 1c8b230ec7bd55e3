// Store new tokens' key/value rows into the paged caches.
//
// The cache is the block pool of PagedAttention; the int8 variant is the
// vllm-sm70 page's int8 KV cache ("Why", Attention bullet), here symmetric
// with one fp32 scale per (token, kv head):
//   s = fp32(max|x| / 127),  code = clamp(rint_even(fp32(x / s)), -127, 127),
// and s = 0, codes 0 for an all-zero row. Both divisions are correctly
// rounded binary32 divisions, so the codes are bit-exact.
// A negative slot skips the token (padded rows must not write into other
// requests' slots: vllm-sm70 page, "Known limitations").
//
// One wave per (token, kv head); lane c handles D/64 consecutive elements.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

template <int CT, int D>
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p) {
    constexpr int EPL = D / 64;  // elements per lane
    const int lane = threadIdx.x & 63;
    const int64_t pair = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (token, kv head)
    if (pair >= p.num_tokens * p.Hkv) return;
    const int64_t i = pair / p.Hkv;
    const int g = (int)(pair % p.Hkv);
    const int64_t slot = p.slots[i];
    if (slot < 0) return;  // wave-uniform
    const int64_t src_off = (i * p.Hkv + g) * D + lane * EPL;
    const int64_t dst_row = slot * p.Hkv + g;  // (block * 16 + offset) * Hkv + g
    const int64_t dst_off = dst_row * D + lane * EPL;

#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const void* src = which ? p.v_src : p.k_src;
        void* cache = which ? p.v_cache : p.k_cache;
        float x[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            x[e] = p.src_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(src)[src_off + e])
                              : reinterpret_cast<const float*>(src)[src_off + e];
        }
        if constexpr (CT == KV_F32) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) reinterpret_cast<float*>(cache)[dst_off + e] = x[e];
        } else if constexpr (CT == KV_BF16) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                reinterpret_cast<uint16_t*>(cache)[dst_off + e] =
                    p.src_bf16 ? reinterpret_cast<const uint16_t*>(src)[src_off + e]  // bit copy
                               : f32_to_bf16(x[e]);
            }
        } else {
            float amax = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
            amax = wave_max(amax);
            const float s = __fdiv_rn(amax, 127.0f);
            uint32_t packed = 0;
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
            int8_t* dst = reinterpret_cast<int8_t*>(cache) + dst_off;
            if constexpr (EPL == 4)
                *reinterpret_cast<uint32_t*>(dst) = packed;
            else if constexpr (EPL == 2)
                *reinterpret_cast<uint16_t*>(dst) = (uint16_t)packed;
            else
                *dst = (int8_t)packed;
            if (lane == 0) (which ? p.v_scale : p.k_scale)[dst_row] = s;
        }
    }
}

namespace {
template <int CT>
hipError_t launch_ct(int D, const CacheWriteParams& p, hipStream_t s) {
    const int64_t pairs = p.num_tokens * p.Hkv;
    const int64_t grid = (pairs + 3) / 4;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    switch (D) {
    case 64: hipLaunchKernelGGL((cache_write_kernel<CT, 64>), dim3((unsigned)grid), dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL((cache_write_kernel<CT, 128>), dim3((unsigned)grid), dim3(256), 0, s, p); break;
    case 256: hipLaunchKernelGGL((cache_write_kernel<CT, 256>), dim3((unsigned)grid), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}
}  // namespace

hipError_t launch_cache_write(int cache_type, const CacheWriteParams& p, hipStream_t stream) {
    switch (cache_type) {
    case KV_F32: return launch_ct<KV_F32>(p.D, p, stream);
    case KV_BF16: return launch_ct<KV_BF16>(p.D, p, stream);
    case KV_I8: return launch_ct<KV_I8>(p.D, p, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace pa
