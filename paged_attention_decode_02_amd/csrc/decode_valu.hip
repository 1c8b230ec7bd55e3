// Split-K paged decode on the vector ALUs (gfx950) for fp32 caches.
//
// One 64-lane wave (= one workgroup) handles one split-K partition of P
// tokens for one kv head g, one query token t of one sequence b, and GT query
// heads of g's group (grouped-query attention: the K/V rows are read once for
// all GT heads). The split-K decode with per-partition softmax statistics is
// the vllm-sm70 page's "split-K paged decode" ("Why", Attention bullet); the
// partition results are merged by the log-sum-exp reduce kernel.
//
// Lane layouts per 16-token KV block:
//  - QK: each row of 16 lanes takes one token at a time; lane c of the row
//    holds D/16 consecutive elements of that token's key, so a row reads one
//    whole contiguous key row (D * elt bytes) and the wave reads 4 tokens per
//    load. Row r takes tokens r, r+4, r+8, r+12. The partial dot products are
//    summed across the row with DPP permutes.
//  - PV: each half-wave (32 lanes) takes one token at a time, lane c holding
//    D/32 consecutive value elements. Half 0 takes the tokens of rows 0 and 1,
//    half 1 those of rows 2 and 3, so the scores only cross between the two
//    rows of a half (one lane swap).
// Each half keeps its own running max and sum (online softmax in log2 units);
// the two halves are merged at the end of the partition. Block j + 1's keys
// and values are requested before block j is computed.
#include <type_traits>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

template <int KVT, int D, int GT>
__global__ __launch_bounds__(64) void decode_valu_kernel(DecodeParams p) {
    constexpr int E = Elt<KVT>::bytes;
    constexpr int EK = D / 16;  // key elements per lane per token (QK layout)
    constexpr int KB = EK * E;
    constexpr int EV = D / 32;  // value elements per lane per token (PV layout)
    constexpr int VB = EV * E;

    const int lane = threadIdx.x;
    const int row = lane >> 4, c16 = lane & 15;
    const int half = lane >> 5, c32 = lane & 31;

    int wg = blockIdx.x;
    const int part = wg % p.NP;
    wg /= p.NP;
    const int chunk = wg % p.nchunk;
    wg /= p.nchunk;
    const int g = wg % p.Hkv;
    wg /= p.Hkv;
    const int t = wg % p.Tq;
    const int b = wg / p.Tq;

    const int n = p.seq_lens[b] - p.Tq + t + 1;  // keys visible to query token t
    const int start = part * p.P;
    const int hbase = g * p.G + chunk * GT;
    const int nh = min(GT, p.G - chunk * GT);
    if (start >= n) {
        // No visible key in this partition. With one partition the row has no
        // key at all: out = 0, lse = -inf. With several, the reduce never
        // reads this partition.
        if (p.NP == 1 && lane < 32) {
            for (int r = 0; r < nh; ++r) {
                const int64_t rowid = ((int64_t)b * p.Tq + t) * p.Hq + hbase + r;
                for (int d = lane; d < D; d += 32) {
                    if (p.out_bf16)
                        reinterpret_cast<uint16_t*>(p.out)[rowid * D + d] = 0;
                    else
                        reinterpret_cast<float*>(p.out)[rowid * D + d] = 0.0f;
                }
                if (p.lse != nullptr && lane == 0) p.lse[rowid] = -INFINITY;
            }
        }
        return;
    }
    const int end = min(start + p.P, n);

    // queries of the GT heads, pre-multiplied by softmax_scale * log2(e)
    float qf[GT][EK];
#pragma unroll
    for (int r = 0; r < GT; ++r) {
        const int64_t qoff = (((int64_t)b * p.Tq + t) * p.Hq + hbase + r) * D + c16 * EK;
#pragma unroll
        for (int e = 0; e < EK; ++e) {
            float v = 0.0f;
            if (r < nh) {
                v = p.q_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(p.q)[qoff + e])
                             : reinterpret_cast<const float*>(p.q)[qoff + e];
            }
            qf[r][e] = v * p.qk_scale_log2;
        }
    }

    float o[GT][EV];
    float m[GT], l[GT];
#pragma unroll
    for (int r = 0; r < GT; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.0f;
#pragma unroll
        for (int e = 0; e < EV; ++e) o[r][e] = 0.0f;
    }

    const int32_t* table = p.block_table + (int64_t)b * p.max_blocks;
    const int64_t tok_stride = (int64_t)p.Hkv * D * E;  // bytes between consecutive tokens
    const char* kbase = reinterpret_cast<const char*>(p.k_cache) + (int64_t)g * D * E;
    const char* vbase = reinterpret_cast<const char*>(p.v_cache) + (int64_t)g * D * E;

    const int j0 = start / kBlockSize, jend = (end + kBlockSize - 1) / kBlockSize;

    // two register buffers of a block's keys (QK layout) and values (PV
    // layout): block j + 1 is requested before block j is computed
    Raw<KB> kr[2][4];
    Raw<VB> vr[2][8];
    auto load_blk = [&](int x, int j) {  // past the partition: its last block again
        const int64_t blk_off = (int64_t)table[j < jend ? j : jend - 1] * kBlockSize * tok_stride;
#pragma unroll
        for (int s = 0; s < 4; ++s) load_raw<KB>(kr[x][s], kbase + blk_off + (4 * s + row) * tok_stride + c16 * KB);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int tok = 4 * (k >> 1) + 2 * half + (k & 1);
            load_raw<VB>(vr[x][k], vbase + blk_off + tok * tok_stride + c32 * VB);
        }
    };
    auto block = [&](int j, auto xc) {
        constexpr int X = decltype(xc)::value;
        const int pos0 = j * kBlockSize;

        // ---- QK: scores of tokens 4s + row, in log2 units
        float srow[4][GT];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int tok = 4 * s + row;
#pragma unroll
            for (int r = 0; r < GT; ++r) {
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < EK; ++e) acc = fmaf(qf[r][e], elem_f32<KVT>(kr[X][s], e), acc);
                acc = row_sum16(acc);
                srow[s][r] = (pos0 + tok < end) ? acc : -INFINITY;
            }
        }

        // ---- the half's 8 tokens: k -> token 4 * (k >> 1) + 2 * half + (k & 1)
        float sc[8][GT];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int r = 0; r < GT; ++r) {
                const float other = __shfl_xor(srow[s][r], 16);
                sc[2 * s + 0][r] = (row & 1) ? other : srow[s][r];
                sc[2 * s + 1][r] = (row & 1) ? srow[s][r] : other;
            }
        }

        // ---- online softmax update of this half
#pragma unroll
        for (int r = 0; r < GT; ++r) {
            float bm = sc[0][r];
#pragma unroll
            for (int k = 1; k < 8; ++k) bm = fmaxf(bm, sc[k][r]);
            const float mn = fmaxf(m[r], bm);
            const float mref = mn == -INFINITY ? 0.0f : mn;
            const float alpha = exp2_guarded(m[r] - mref);
            m[r] = mn;
            l[r] *= alpha;
#pragma unroll
            for (int e = 0; e < EV; ++e) o[r][e] *= alpha;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                sc[k][r] = exp2_guarded(sc[k][r] - mref);
                l[r] += sc[k][r];
            }
        }

        // ---- PV
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int tok = 4 * (k >> 1) + 2 * half + (k & 1);
            // Slots past the end may hold anything (NaN included): select, never
            // multiply by a zero weight.
            const bool ok = pos0 + tok < end;
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const float v = ok ? elem_f32<KVT>(vr[X][k], e) : 0.0f;
#pragma unroll
                for (int r = 0; r < GT; ++r) o[r][e] = fmaf(ok ? sc[k][r] : 0.0f, v, o[r][e]);
            }
        }
    };
    load_blk(0, j0);
    int j = j0;
    for (; j + 1 < jend; j += 2) {
        load_blk(1, j + 1);
        block(j, std::integral_constant<int, 0>{});
        load_blk(0, j + 2);
        block(j + 1, std::integral_constant<int, 1>{});
    }
    if (j < jend) block(j, std::integral_constant<int, 0>{});

    // ---- merge the two halves, normalise, write
#pragma unroll
    for (int r = 0; r < GT; ++r) {
        const float mo = __shfl_xor(m[r], 32);
        const float lo = __shfl_xor(l[r], 32);
        const float M = fmaxf(m[r], mo);
        const float mref = M == -INFINITY ? 0.0f : M;
        const float a = exp2_guarded(m[r] - mref), c = exp2_guarded(mo - mref);
        const float lt = l[r] * a + lo * c;
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            const float oo = __shfl_xor(o[r][e], 32);
            o[r][e] = (o[r][e] * a + oo * c) * inv;
        }
        l[r] = lt;
        m[r] = lt > 0.0f ? (M + log2f(lt)) * kLn2 : -INFINITY;  // natural-log LSE
    }
    if (half != 0) return;
#pragma unroll
    for (int r = 0; r < GT; ++r) {
        if (r >= nh) break;
        const int h = hbase + r;
        const int64_t rowid = ((int64_t)b * p.Tq + t) * p.Hq + h;
        const int d0 = c32 * EV;
        if (p.NP == 1) {
            if (p.out_bf16) {
                uint16_t* dst = reinterpret_cast<uint16_t*>(p.out) + rowid * D + d0;
#pragma unroll
                for (int e = 0; e < EV; ++e) dst[e] = f32_to_bf16(o[r][e]);
            } else {
                float* dst = reinterpret_cast<float*>(p.out) + rowid * D + d0;
#pragma unroll
                for (int e = 0; e < EV; ++e) dst[e] = o[r][e];
            }
            if (p.lse != nullptr && c32 == 0) p.lse[rowid] = m[r];
        } else {
            float* dst = p.ws_o + (rowid * p.NP + part) * D + d0;
#pragma unroll
            for (int e = 0; e < EV; ++e) dst[e] = o[r][e];
            if (c32 == 0) p.ws_lse[rowid * p.NP + part] = m[r];
        }
    }
}

namespace {
template <int KVT, int D, int GT>
hipError_t launch_one(const DecodeParams& p, hipStream_t s) {
    const int64_t grid = (int64_t)p.NP * p.nchunk * p.Hkv * p.Tq * p.B;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_valu_kernel<KVT, D, GT>), dim3((unsigned)grid), dim3(64), 0, s, p);
    return hipGetLastError();
}

template <int KVT, int D>
hipError_t by_gt(int GT, const DecodeParams& p, hipStream_t s) {
    switch (GT) {
    case 1: return launch_one<KVT, D, 1>(p, s);
    case 2: return launch_one<KVT, D, 2>(p, s);
    case 4: return launch_one<KVT, D, 4>(p, s);
    case 6: return launch_one<KVT, D, 6>(p, s);
    case 8: return launch_one<KVT, D, 8>(p, s);
    default: return hipErrorInvalidValue;
    }
}

template <int KVT>
hipError_t by_d(int D, int GT, const DecodeParams& p, hipStream_t s) {
    switch (D) {
    case 64: return by_gt<KVT, 64>(GT, p, s);
    case 128: return by_gt<KVT, 128>(GT, p, s);
    case 256: return by_gt<KVT, 256>(GT, p, s);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

bool decode_valu_has_gt(int GT) { return GT == 1 || GT == 2 || GT == 4 || GT == 6 || GT == 8; }

hipError_t launch_decode_valu(int kv_type, int D, int GT, const DecodeParams& p, hipStream_t stream) {
    if (kv_type != KV_F32) return hipErrorInvalidValue;  // bf16 / int8 caches have their own kernels
    return by_d<KV_F32>(D, GT, p, stream);
}

}  // namespace pa
