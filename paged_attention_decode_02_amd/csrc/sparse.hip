// Sparse block-selection decode: per-block mean keys, block scores, top-N
// selection, and the compacted block tables the decode kernels then read.
//
// The vllm-sm70 page names the parts ("Changes relative to 1Cat-vLLM", item
// 8: sparse-decode mean keys refreshed for every request of a decode batch;
// "Known limitations": the sparse decode selection supports at most 4096 key
// blocks, a 262,144-token table at 64-token blocks), not the rule. The rule
// taken here: a sequence's positions form sparse blocks of SB tokens (a
// multiple of the 16-token cache block); a block's mean key is the plain
// mean of its keys below the sequence length; the blocks holding the query
// tokens are always selected; every other block scores the largest, over the
// kv head's query rows, of softmax_scale * q . mean key, and the top ones
// (ties to the lower index) fill top_blocks; the decode then attends to the
// selected blocks' keys with the plain causal rule.
//
// Kernels:
//  - sparse_mean_kernel: one workgroup per (sequence, refreshed block, kv
//    head); thread d sums element d over the block's tokens in position
//    order (fp32) and divides by their count;
//  - sparse_score_kernel: one workgroup per (sequence and kv head, 32
//    candidate blocks): the candidates' mean keys and 16 query rows at a
//    time are staged in LDS (padded rows, coalesced loads), each thread takes
//    one candidate and two rows, dot products in fp32 in dimension order;
//  - sparse_select_kernel: one workgroup per (sequence, kv head): a radix
//    select over the candidates' scores (4 passes of 8 bits on the
//    order-preserving integer image of the fp32 score) finds the threshold,
//    ties at the threshold go to the lower block index (a prefix count in
//    block order), the selected blocks are compacted in increasing order with
//    the kept blocks last, and their cache blocks written as one block table
//    row with the compacted length.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

// Element d of the key row of (physical block ph, token off, kv head g).
template <int KVT>
__device__ __forceinline__ float key_elem(const void* cache, const float* scale, int64_t ph, int off, int g, int Hkv,
                                          int D, int d) {
    if constexpr (KVT == KV_NVFP4) {
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(cache) + ph * kBlockSize * Hkv * nvfp4_row_bytes(D);
        const uint32_t code = blk[(int64_t)(off * Hkv + g) * (D / 2) + d / 2];
        const pa_f32x2 e = fp4x2_to_f32<0>(code);
        const uint32_t sb = blk[(int64_t)kBlockSize * Hkv * (D / 2) + (int64_t)g * D + nvfp4_scale_byte(off, d / 16)];
        return ((d & 1) ? e.y : e.x) * fp8_value(sb) * scale[(ph * Hkv + g) * kBlockSize + off];
    } else {
        const int64_t row = (ph * kBlockSize + off) * Hkv + g;
        if constexpr (KVT == KV_F32) {
            return reinterpret_cast<const float*>(cache)[row * D + d];
        } else if constexpr (KVT == KV_BF16) {
            return bf16_to_f32(reinterpret_cast<const uint16_t*>(cache)[row * D + d]);
        } else {
            const uint32_t code = reinterpret_cast<const uint8_t*>(cache)[row * D + d];
            const float s = scale[(ph * Hkv + g) * kBlockSize + off];
            if constexpr (KVT == KV_I8)
                return (float)(int8_t)code * s;
            else
                return fp8_value(code) * s;
        }
    }
}

// Order-preserving unsigned image of a float (larger float, larger key).
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// First sparse block holding a query token of a sequence of L tokens.
__device__ __forceinline__ int first_kept(int L, int Tq, int SB) { return (L - Tq > 0 ? L - Tq : 0) / SB; }

constexpr int kScoreTile = 32;   // candidate blocks per score workgroup
constexpr int kScoreRows = 16;   // query rows staged at a time
constexpr int kSelThreads = 1024;
constexpr int kSelPer = 4;       // candidates per select thread (4096 in all)

}  // namespace

template <int KVT>
__global__ __launch_bounds__(256) void sparse_mean_kernel(SparseParams p) {
    const int b = blockIdx.x, k = blockIdx.y, g = blockIdx.z;
    const int L = p.seq_lens[b];
    if (L <= 0) return;
    const int SB = p.sparse_block;
    const int nsb = (L + SB - 1) / SB;
    const int j = (L - p.num_new > 0 ? L - p.num_new : 0) / SB + k;  // blocks holding the newest tokens
    if (j >= nsb) return;
    const int p0 = j * SB, p1 = min(p0 + SB, L);
    const int32_t* table = p.block_table + (int64_t)b * p.max_blocks;
    float* dst = p.mean_k + (((int64_t)b * p.max_sblocks + j) * p.Hkv + g) * p.D;
    for (int d = threadIdx.x; d < p.D; d += blockDim.x) {
        float sum = 0.0f;
        for (int pos = p0; pos < p1; ++pos)
            sum += key_elem<KVT>(p.k_cache, p.k_scale, (int64_t)table[pos / kBlockSize], pos % kBlockSize, g, p.Hkv,
                                 p.D, d);
        dst[d] = sum / (float)(p1 - p0);
    }
}

__global__ __launch_bounds__(256) void sparse_score_kernel(SparseParams p) {
    // mean keys of the tile's candidates, rows padded by 4 floats (the
    // threads of a wave read 32 different rows at one column)
    __shared__ __align__(16) float mk[kScoreTile][256 + 4];
    __shared__ __align__(16) float qs[kScoreRows][256];
    __shared__ float red[256 / kScoreTile][kScoreTile];
    const int bg = blockIdx.x, b = bg / p.Hkv, g = bg % p.Hkv;
    const int L = p.seq_lens[b];
    const int kept0 = L > 0 ? first_kept(L, p.Tq, p.sparse_block) : 0;
    const int j0 = blockIdx.y * kScoreTile;
    if (j0 >= kept0) return;
    const int D = p.D, G = p.Hq / p.Hkv, R = p.Tq * G;
    const int tid = threadIdx.x;
    for (int x = tid; x < kScoreTile * D; x += 256) {
        const int c = x / D, d = x % D;
        mk[c][d] = j0 + c < kept0 ? p.mean_k[(((int64_t)b * p.max_sblocks + j0 + c) * p.Hkv + g) * D + d] : 0.0f;
    }
    const int c = tid % kScoreTile, rg = tid / kScoreTile;  // candidate, row group (8)
    float best = -INFINITY;
    for (int r0 = 0; r0 < R; r0 += kScoreRows) {
        __syncthreads();
        for (int x = tid; x < kScoreRows * D; x += 256) {
            const int r = r0 + x / D, d = x % D;
            float v = 0.0f;
            if (r < R) {
                const int64_t qoff = (((int64_t)b * p.Tq + r / G) * p.Hq + g * G + r % G) * D + d;
                v = p.q_bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(p.q)[qoff])
                             : reinterpret_cast<const float*>(p.q)[qoff];
            }
            qs[x / D][d] = v;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kScoreRows / 8; ++k) {
            const int rr = rg + 8 * k;
            if (r0 + rr >= R) continue;
            float dot = 0.0f;
            for (int d = 0; d < D; d += 4) {
                const float4 a = *reinterpret_cast<const float4*>(&qs[rr][d]);
                const float4 m = *reinterpret_cast<const float4*>(&mk[c][d]);
                dot = fmaf(a.x, m.x, dot);
                dot = fmaf(a.y, m.y, dot);
                dot = fmaf(a.z, m.z, dot);
                dot = fmaf(a.w, m.w, dot);
            }
            best = fmaxf(best, p.softmax_scale * dot);
        }
    }
    red[rg][c] = best;
    __syncthreads();
    if (rg == 0 && j0 + c < kept0) {
        float m = red[0][c];
        for (int k = 1; k < 256 / kScoreTile; ++k) m = fmaxf(m, red[k][c]);
        p.scores[(int64_t)bg * p.nsb_max + j0 + c] = m;
    }
}

namespace {
// exclusive prefix sum over the workgroup (kSelThreads threads), in thread order
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int acc = 0;
        for (int i = 0; i < kSelThreads / 64; ++i) {
            const int t = wsum[i];
            wsum[i] = acc;
            acc += t;
        }
        *total = acc;
    }
    __syncthreads();
    const int r = x - v + wsum[w];
    __syncthreads();
    return r;
}
}  // namespace

__global__ __launch_bounds__(kSelThreads) void sparse_select_kernel(SparseParams p) {
    __shared__ int hist[256];
    __shared__ int lsel[kSelThreads * kSelPer];  // the selected blocks in increasing order
    __shared__ int wsum[kSelThreads / 64];
    __shared__ int total;
    __shared__ uint32_t s_prefix;
    __shared__ int s_remaining;
    const int bg = blockIdx.x, b = bg / p.Hkv;
    const int tid = threadIdx.x;
    const int SB = p.sparse_block, SBB = SB / kBlockSize;
    const int L = p.seq_lens[b];
    const int nsb = L > 0 ? (L + SB - 1) / SB : 0;
    const int kept0 = L > 0 ? first_kept(L, p.Tq, SB) : 0;
    const int nkept = nsb - kept0;
    int want = p.top_blocks - nkept;
    want = want < 0 ? 0 : want > kept0 ? kept0 : want;

    // this thread's candidates: blocks kSelPer tid .. kSelPer tid + kSelPer - 1
    uint32_t key[kSelPer];
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
        const int j = kSelPer * tid + i;
        key[i] = j < kept0 ? order_key(p.scores[(int64_t)bg * p.nsb_max + j]) : 0u;
    }
    // threshold T: the want-th largest key (want candidates have key >= T and
    // fewer than want have key > T), by 8-bit digits from the top
    if (tid == 0) {
        s_prefix = 0u;
        s_remaining = want;
    }
    uint32_t mask = 0u;
    if (want > 0 && want < kept0) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
            __syncthreads();
            const uint32_t prefix = s_prefix;
#pragma unroll
            for (int i = 0; i < kSelPer; ++i) {
                const int j = kSelPer * tid + i;
                if (j < kept0 && (key[i] & mask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 0xFF], 1);
            }
            __syncthreads();
            if (tid == 0) {
                int rem = s_remaining, dgt = 255;
                for (; dgt > 0; --dgt) {
                    if (hist[dgt] >= rem) break;
                    rem -= hist[dgt];
                }
                s_prefix = prefix | ((uint32_t)dgt << shift);
                s_remaining = rem;  // keys equal to the final prefix still to take
            }
            mask |= 0xFFu << shift;
            __syncthreads();
        }
    }
    const uint32_t T = s_prefix;
    const int need_eq = s_remaining;  // with want in (0, kept0): keys == T to take, in block order
    // selection flags in block order: all candidates (want == kept0), none
    // (want == 0), or key > T and the first need_eq keys == T
    int eq_cnt = 0;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
        const int j = kSelPer * tid + i;
        eq_cnt += (want > 0 && want < kept0 && j < kept0 && key[i] == T) ? 1 : 0;
    }
    int eq_before = block_exclusive_scan(eq_cnt, wsum, &total);
    bool flag[kSelPer];
    int nflag = 0;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
        const int j = kSelPer * tid + i;
        bool f = false;
        if (j < kept0) {
            if (want >= kept0)
                f = true;
            else if (want > 0) {
                if (key[i] > T)
                    f = true;
                else if (key[i] == T) {
                    f = eq_before < need_eq;
                    ++eq_before;
                }
            }
        }
        flag[i] = f;
        nflag += f ? 1 : 0;
    }
    const int pos0 = block_exclusive_scan(nflag, wsum, &total);
    const int nsel = total;  // == want
    const int count = nsel + nkept;
    int pos = pos0;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i)
        if (flag[i]) lsel[pos++] = kSelPer * tid + i;
    for (int k = tid; k < nkept; k += kSelThreads) lsel[nsel + k] = kept0 + k;
    __syncthreads();
    // compacted table row: the cache blocks of the selected blocks in order
    const int32_t* table = p.block_table + (int64_t)b * p.max_blocks;
    int32_t* ct = p.ctab + (int64_t)bg * p.ctab_width;
    for (int x = tid; x < count * SBB; x += kSelThreads) {
        const int jb = lsel[x / SBB] * SBB + x % SBB;  // logical cache block
        ct[x] = jb < p.max_blocks ? table[jb] : 0;     // past the table: never read (beyond the length)
    }
    if (tid == 0) p.clen[bg] = count > 0 ? (count - 1) * SB + (L - (nsb - 1) * SB) : 0;
    if (p.sel_out != nullptr)
        for (int k = tid; k < p.max_sel; k += kSelThreads)
            p.sel_out[(int64_t)bg * p.max_sel + k] = k < count ? lsel[k] : -1;
}

hipError_t launch_sparse_mean(int kv_type, const SparseParams& p, int nref, hipStream_t s) {
    if (p.B <= 0 || nref <= 0) return hipSuccess;
    const dim3 grid((unsigned)p.B, (unsigned)nref, (unsigned)p.Hkv);
    switch (kv_type) {
    case KV_F32: hipLaunchKernelGGL(sparse_mean_kernel<KV_F32>, grid, dim3(256), 0, s, p); break;
    case KV_BF16: hipLaunchKernelGGL(sparse_mean_kernel<KV_BF16>, grid, dim3(256), 0, s, p); break;
    case KV_I8: hipLaunchKernelGGL(sparse_mean_kernel<KV_I8>, grid, dim3(256), 0, s, p); break;
    case KV_FP8: hipLaunchKernelGGL(sparse_mean_kernel<KV_FP8>, grid, dim3(256), 0, s, p); break;
    case KV_NVFP4: hipLaunchKernelGGL(sparse_mean_kernel<KV_NVFP4>, grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_sparse_select(const SparseParams& p, hipStream_t s) {
    if (p.B <= 0) return hipSuccess;
    if (p.D > 256 || p.nsb_max > kSelThreads * kSelPer) return hipErrorInvalidValue;
    const unsigned bgs = (unsigned)(p.B * p.Hkv);
    const unsigned tiles = (unsigned)((p.nsb_max + kScoreTile - 1) / kScoreTile);
    if (tiles > 0) {
        hipLaunchKernelGGL(sparse_score_kernel, dim3(bgs, tiles), dim3(256), 0, s, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sparse_select_kernel, dim3(bgs), dim3(kSelThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace pa
