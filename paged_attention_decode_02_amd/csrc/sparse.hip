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
//    head); a thread takes 4 consecutive elements of every (256 / (D / 4))-th
//    token of the block, all its loads issued before the sums (the block's
//    table entries staged in LDS first); the per-thread sums (fp32, token
//    order) are combined in thread order, so the result is deterministic;
//  - sparse_score_kernel: one workgroup per (sequence and kv head, 64
//    candidate blocks), 16 candidates per wave; a lane quad holds one
//    candidate's mean key in registers (interleaved 16-byte pieces, loaded at
//    once), the query rows are staged 16 at a time in LDS, and each row's dot
//    product is summed over the quad by two DPP lane moves;
//  - sparse_select_kernel: one workgroup per (sequence, kv head): a radix
//    select over the candidates' scores finds the threshold: on the
//    order-preserving integer image of the fp32 score less the smallest one
//    (which spreads scores of one sign and exponent over the bins), 11-bit
//    digits from the highest bit that varies, each digit found by a
//    wave-parallel suffix count over the 2048 bins; ties at the threshold go
//    to the lower block index (a prefix count in block order), the selected
//    blocks are compacted in increasing order with the kept blocks last, and
//    their cache blocks written as one block table row with the compacted
//    length.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

// Elements d0 .. d0 + 3 (d0 a multiple of 4) of the key row of (physical
// block ph, token off, kv head g), dequantised.
template <int KVT>
__device__ __forceinline__ float4 key4(const void* cache, const float* scale, int64_t ph, int off, int g, int Hkv,
                                       int D, int d0) {
    if constexpr (KVT == KV_NVFP4) {
        const uint8_t* blk = reinterpret_cast<const uint8_t*>(cache) + ph * kBlockSize * Hkv * nvfp4_row_bytes(D);
        const uint32_t codes =
            *reinterpret_cast<const uint16_t*>(blk + (int64_t)(off * Hkv + g) * (D / 2) + d0 / 2);
        const uint32_t sb = blk[(int64_t)kBlockSize * Hkv * (D / 2) + (int64_t)g * D + nvfp4_scale_byte(off, d0 / 16)];
        const float f = fp8_value(sb) * scale[(ph * Hkv + g) * kBlockSize + off];
        const pa_f32x2 lo = fp4x2_to_f32<0>(codes), hi = fp4x2_to_f32<1>(codes);
        return make_float4(lo.x * f, lo.y * f, hi.x * f, hi.y * f);
    } else {
        const int64_t row = (ph * kBlockSize + off) * Hkv + g;
        if constexpr (KVT == KV_F32) {
            return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(cache) + row * D + d0);
        } else if constexpr (KVT == KV_BF16) {
            const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(cache) + row * D + d0);
            return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                               __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
        } else {
            const uint32_t c = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(cache) + row * D + d0);
            const float sc = scale[(ph * Hkv + g) * kBlockSize + off];
            if constexpr (KVT == KV_I8) {
                return make_float4((float)(int8_t)c * sc, (float)(int8_t)(c >> 8) * sc, (float)(int8_t)(c >> 16) * sc,
                                   (float)(int8_t)(c >> 24) * sc);
            } else {
                const pa_f32x2 lo = fp8x2_to_f32<false>(c), hi = fp8x2_to_f32<true>(c);
                return make_float4(lo.x * sc, lo.y * sc, hi.x * sc, hi.y * sc);
            }
        }
    }
}

// Order-preserving unsigned image of a float (larger float, larger key; the
// two zeros map to one key, as they compare equal).
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// First sparse block holding a query token of a sequence of L tokens.
__device__ __forceinline__ int first_kept(int L, int Tq, int SB) { return (L - Tq > 0 ? L - Tq : 0) / SB; }

constexpr int kScoreCands = 64;  // candidate blocks per score workgroup (16 per wave)
constexpr int kScoreRows = 16;   // query rows staged at a time
constexpr int kSelThreads = 1024;
constexpr int kSelPer = 4;       // candidates per select thread (4096 in all)
constexpr int kSelBits = 11;     // radix digit of the select
constexpr int kSelBins = 1 << kSelBits;
constexpr int kMeanUnroll = 8;   // token loads a mean-key thread keeps in flight
}  // namespace

template <int KVT>
__global__ __launch_bounds__(256) void sparse_mean_kernel(SparseParams p) {
    __shared__ int32_t tab[kSparseMaxBlockTokens / kBlockSize];
    __shared__ __align__(16) float part[256 * 4];  // [token lane][D]: 256 / (D / 4) lanes of D floats
    const int b = blockIdx.x, k = blockIdx.y, g = blockIdx.z;
    const int L = p.seq_lens[b];
    if (L <= 0) return;
    const int SB = p.sparse_block;
    const int nsb = (L + SB - 1) / SB;
    const int j = (L - p.num_new > 0 ? L - p.num_new : 0) / SB + k;  // blocks holding the newest tokens
    if (j >= nsb) return;
    const int p0 = j * SB, p1 = min(p0 + SB, L), n = p1 - p0;
    const int D = p.D, DG = D / 4, lanes = 256 / DG;
    const int tid = threadIdx.x, tl = tid / DG, d0 = (tid % DG) * 4;
    const int32_t* table = p.block_table + (int64_t)b * p.max_blocks;
    for (int x = tid; x < (n + kBlockSize - 1) / kBlockSize; x += 256) tab[x] = table[p0 / kBlockSize + x];
    __syncthreads();
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int t0 = tl; t0 < n; t0 += lanes * kMeanUnroll) {
        float4 v[kMeanUnroll];
#pragma unroll
        for (int u = 0; u < kMeanUnroll; ++u) {  // tokens past n reread token n - 1, not summed
            const int t = min(t0 + u * lanes, n - 1);
            v[u] = key4<KVT>(p.k_cache, p.k_scale, (int64_t)tab[t / kBlockSize], t % kBlockSize, g, p.Hkv, D, d0);
        }
#pragma unroll
        for (int u = 0; u < kMeanUnroll; ++u) {
            if (t0 + u * lanes < n) {
                s.x += v[u].x;
                s.y += v[u].y;
                s.z += v[u].z;
                s.w += v[u].w;
            }
        }
    }
    *reinterpret_cast<float4*>(&part[tl * D + d0]) = s;
    __syncthreads();
    float* dst = p.mean_k + (((int64_t)b * p.max_sblocks + j) * p.Hkv + g) * D;
    if (tid < D) {
        float sum = 0.0f;
        for (int l = 0; l < lanes; ++l) sum += part[l * D + tid];
        dst[tid] = sum / (float)n;
    }
}

template <int D>
__global__ __launch_bounds__(256) void sparse_score_kernel(SparseParams p) {
    __shared__ __align__(16) float qs[kScoreRows][D];
    constexpr int NI = D / 16;  // 16-byte pieces of a candidate's mean key per lane
    const int bg = blockIdx.x, b = bg / p.Hkv, g = bg % p.Hkv;
    const int L = p.seq_lens[b];
    const int kept0 = L > 0 ? first_kept(L, p.Tq, p.sparse_block) : 0;
    const int j0 = blockIdx.y * kScoreCands;
    if (j0 >= kept0) return;
    const int G = p.Hq / p.Hkv, R = p.Tq * G;
    const int tid = threadIdx.x, lane = tid & 63;
    const int c = j0 + (tid >> 6) * 16 + (lane >> 2), kq = lane & 3;  // candidate, quarter
    const bool valid = c < kept0;
    // this lane's part of the candidate's mean key: elements 16 i + 4 kq .. + 3
    // (an invalid candidate reads candidate 0's row and discards it)
    const float* src = p.mean_k + (((int64_t)b * p.max_sblocks + (valid ? c : 0)) * p.Hkv + g) * D + 4 * kq;
    float4 m[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) m[i] = *reinterpret_cast<const float4*>(src + 16 * i);
    float best = -INFINITY;
    for (int r0 = 0; r0 < R; r0 += kScoreRows) {
        // stage rows r0 .. r0 + 15 (rows past R as zeros): every load issued
        // before the first store
        constexpr int NU = kScoreRows * D / 256;
        float v[NU];
        if (p.q_bf16) {
            const uint16_t* q = reinterpret_cast<const uint16_t*>(p.q);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int x = tid + 256 * u, r = r0 + x / D, rc = r < R ? r : R - 1;
                v[u] = bf16_to_f32(q[(((int64_t)b * p.Tq + rc / G) * p.Hq + g * G + rc % G) * D + x % D]);
            }
        } else {
            const float* q = reinterpret_cast<const float*>(p.q);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int x = tid + 256 * u, r = r0 + x / D, rc = r < R ? r : R - 1;
                v[u] = q[(((int64_t)b * p.Tq + rc / G) * p.Hq + g * G + rc % G) * D + x % D];
            }
        }
        __syncthreads();  // the previous rows' reads are done
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int x = tid + 256 * u;
            qs[x / D][x % D] = r0 + x / D < R ? v[u] : 0.0f;
        }
        __syncthreads();
        const int nr = min(kScoreRows, R - r0);
        for (int rr = 0; rr < nr; ++rr) {
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const float4 a = *reinterpret_cast<const float4*>(&qs[rr][16 * i + 4 * kq]);
                acc = fmaf(a.x, m[i].x, acc);
                acc = fmaf(a.y, m[i].y, acc);
                acc = fmaf(a.z, m[i].z, acc);
                acc = fmaf(a.w, m[i].w, acc);
            }
            acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0xB1, 0xF, 0xF, true));  // quad [1,0,3,2]
            acc += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(acc), 0x4E, 0xF, 0xF, true));  // quad [2,3,0,1]
            best = fmaxf(best, p.softmax_scale * acc);
        }
    }
    if (kq == 0 && valid) p.scores[(int64_t)bg * p.nsb_max + c] = best;
}

namespace {
constexpr int kSelWaves = kSelThreads / 64;

// Wave-level scans and reductions on DPP (vector-ALU lane moves), not on LDS
// permutes. dpp<CTRL, ROWS>(x, id): lane l receives the lane CTRL names, or
// id where the source is outside the row or the row is not in ROWS.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp(int x, int id) {
    return __builtin_amdgcn_update_dpp(id, x, CTRL, ROWS, 0xF, false);
}

// inclusive prefix sum over the 64 lanes (within rows of 16 by shifts, then
// the row totals broadcast to the rows above)
__device__ __forceinline__ int wave_incl_sum(int x) {
    x += dpp<0x111>(x, 0);  // row_shr:1
    x += dpp<0x112>(x, 0);  // row_shr:2
    x += dpp<0x114>(x, 0);  // row_shr:4
    x += dpp<0x118>(x, 0);  // row_shr:8
    x += dpp<0x142, 0xA>(x, 0);  // row_bcast:15 into rows 1 and 3
    x += dpp<0x143, 0xC>(x, 0);  // row_bcast:31 into rows 2 and 3
    return x;
}

// unsigned minimum / maximum over the 64 lanes, in every lane (each row
// reduced by quad and mirror moves, the four row results read as scalars)
template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax(uint32_t x) {
    auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
    x = op(x, (uint32_t)dpp<0xB1>((int)x, 0));   // quad_perm [1, 0, 3, 2]
    x = op(x, (uint32_t)dpp<0x4E>((int)x, 0));   // quad_perm [2, 3, 0, 1]
    x = op(x, (uint32_t)dpp<0x141>((int)x, 0));  // row_half_mirror
    x = op(x, (uint32_t)dpp<0x140>((int)x, 0));  // row_mirror
    const uint32_t r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
    return op(op(r0, r1), op(r2, r3));
}

// Exclusive prefix sum of v over the workgroup in thread order, with one
// barrier: a shuffle scan inside each wave, the wave totals through LDS
// (wsum: kSelWaves ints, free for reuse only after the caller's next
// barrier). *total receives the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int x = wave_incl_sum(v);
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
        const int t = wsum[i];
        before += i < w ? t : 0;
        all += t;
    }
    *total = all;
    return before + x - v;
}
}  // namespace

__global__ __launch_bounds__(kSelThreads) void sparse_select_kernel(SparseParams p) {
    __shared__ __align__(16) int hist[2][kSelBins];     // double-buffered digit counts
    __shared__ int lsel[kSelThreads * kSelPer];         // the selected blocks in increasing order
    __shared__ int wsum[2][kSelWaves];                  // scan totals (two scans in flight)
    __shared__ uint32_t wmin[kSelWaves], wmax[kSelWaves];
    __shared__ uint32_t s_prefix;
    __shared__ int s_remaining, s_eq;
    const int bg = blockIdx.x, b = bg / p.Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int SB = p.sparse_block, SBB = SB / kBlockSize;
    const int L = p.seq_lens[b];
    const int nsb = L > 0 ? (L + SB - 1) / SB : 0;
    const int kept0 = L > 0 ? first_kept(L, p.Tq, SB) : 0;
    const int nkept = nsb - kept0;
    int want = p.top_blocks - nkept;
    want = want < 0 ? 0 : want > kept0 ? kept0 : want;
    const bool partial = want > 0 && want < kept0;  // uniform over the workgroup

    // this thread's candidates: blocks kSelPer tid .. kSelPer tid + kSelPer - 1
    // (every load issued unconditionally, from a clamped index, before any use)
    const int jmax = p.nsb_max > 0 ? p.nsb_max - 1 : 0;
    float sc[kSelPer];
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) sc[i] = p.scores[(int64_t)bg * p.nsb_max + min(kSelPer * tid + i, jmax)];
    uint32_t key[kSelPer];
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) key[i] = kSelPer * tid + i < kept0 ? order_key(sc[i]) : 0u;
    // threshold T: the want-th largest key (want candidates have key >= T and
    // fewer than want have key > T), found on rel = key - (smallest key) by
    // kSelBits-bit digits from the highest bit in which the keys differ
    uint32_t T = 0u;
    int need_eq = 0;       // keys == T to take, in block order
    bool all_eq = true;    // every key == T is taken (no tie to break)
    if (partial) {
        uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
        for (int i = 0; i < kSelPer; ++i)
            if (kSelPer * tid + i < kept0) {
                lo = min(lo, key[i]);
                hi = max(hi, key[i]);
            }
        lo = wave_minmax<false>(lo);
        hi = wave_minmax<true>(hi);
        if (lane == 0) {
            wmin[wv] = lo;
            wmax[wv] = hi;
        }
        for (int i = tid; i < kSelBins; i += kSelThreads) hist[0][i] = 0;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kSelWaves; ++i) {
            lo = min(lo, wmin[i]);
            hi = max(hi, wmax[i]);
        }
        const uint32_t kmin = lo, span = hi - lo;
        const int nbits = span ? 32 - __clz(span) : 0;
        uint32_t rel[kSelPer];
#pragma unroll
        for (int i = 0; i < kSelPer; ++i) rel[i] = key[i] - kmin;
        uint32_t prefix = 0u, mask = 0u;
        int rem = want, eq = -1, buf = 0;
        for (int top = nbits; top > 0; top -= kSelBits, buf ^= 1) {
            const int shift = top > kSelBits ? top - kSelBits : 0;
            const uint32_t dmask = (1u << (top - shift)) - 1u;
            int* h = hist[buf];
#pragma unroll
            for (int i = 0; i < kSelPer; ++i)
                if (kSelPer * tid + i < kept0 && (rel[i] & mask) == prefix) atomicAdd(&h[(rel[i] >> shift) & dmask], 1);
            // the other buffer, last read by the previous pass's search, for the next pass
            for (int i = tid; i < kSelBins; i += kSelThreads) hist[buf ^ 1][i] = 0;
            __syncthreads();
            if (tid < 64) {
                // lane owns bins 32 lane .. 32 lane + 31; suffix(d) = keys
                // with digit >= d, non-increasing in d; the digit is the
                // highest d with suffix(d) >= rem
                int c[32], tot = 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int4 v = *reinterpret_cast<const int4*>(&h[32 * lane + 4 * k]);
                    c[4 * k] = v.x;
                    c[4 * k + 1] = v.y;
                    c[4 * k + 2] = v.z;
                    c[4 * k + 3] = v.w;
                    tot += v.x + v.y + v.z + v.w;
                }
                const int incl = wave_incl_sum(tot);
                int run = __builtin_amdgcn_readlane(incl, 63) - incl;  // keys in the bins of the lanes above
                int sfx[32];
#pragma unroll
                for (int k = 31; k >= 0; --k) {
                    run += c[k];
                    sfx[k] = run;
                }
                int best = -1, rem_at = rem, cnt = 0;
#pragma unroll
                for (int k = 0; k < 32; ++k) {  // the last k that qualifies is the highest
                    const bool ok = sfx[k] >= rem;
                    best = ok ? 32 * lane + k : best;
                    rem_at = ok ? rem - (sfx[k] - c[k]) : rem_at;
                    cnt = ok ? c[k] : cnt;
                }
                // the qualifying bins are a prefix: the highest lane holding one has the digit
                const uint64_t any = __ballot(best >= 0);
                const int hl = any ? 63 - __clzll((long long)any) : -1;
                if (lane == hl) {
                    s_prefix = prefix | ((uint32_t)best << shift);
                    s_remaining = rem_at;
                    s_eq = cnt;
                } else if (hl < 0 && lane == 0) {  // unreachable: suffix(0) counts every key left
                    s_prefix = prefix;
                    s_remaining = rem;
                    s_eq = -1;
                }
            }
            __syncthreads();
            prefix = s_prefix;
            rem = s_remaining;
            eq = s_eq;
            mask |= dmask << shift;
        }
        T = kmin + prefix;
        need_eq = rem;
        // keys == T: the last pass's bin count (every key when all are equal)
        all_eq = (nbits == 0 ? want == kept0 : eq == rem);
    }
    // selection flags in block order: all candidates (want == kept0), none
    // (want == 0), or key > T and the first need_eq keys == T (a prefix count
    // in block order, only when some keys == T are left out)
    int eq_before = 0, eq_total;
    if (partial && !all_eq) {
        int eq_cnt = 0;
#pragma unroll
        for (int i = 0; i < kSelPer; ++i) eq_cnt += (kSelPer * tid + i < kept0 && key[i] == T) ? 1 : 0;
        eq_before = block_exclusive_scan(eq_cnt, wsum[0], &eq_total);
    }
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
                    f = all_eq || eq_before < need_eq;
                    ++eq_before;
                }
            }
        }
        flag[i] = f;
        nflag += f ? 1 : 0;
    }
    int nsel;
    const int pos0 = block_exclusive_scan(nflag, wsum[1], &nsel);  // nsel == want
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
    const int nct = count * SBB;
    for (int x0 = tid; x0 < nct; x0 += 4 * kSelThreads) {
        int32_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int x = x0 + u * kSelThreads;
            const int jb = x < nct ? lsel[x / SBB] * SBB + x % SBB : 0;  // logical cache block
            v[u] = x < nct && jb < p.max_blocks ? table[jb] : 0;        // past the table: never read
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (x0 + u * kSelThreads < nct) ct[x0 + u * kSelThreads] = v[u];
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
    if (p.nsb_max > kSelThreads * kSelPer) return hipErrorInvalidValue;
    const unsigned bgs = (unsigned)(p.B * p.Hkv);
    const unsigned tiles = (unsigned)((p.nsb_max + kScoreCands - 1) / kScoreCands);
    if (tiles > 0) {
        switch (p.D) {
        case 64: hipLaunchKernelGGL(sparse_score_kernel<64>, dim3(bgs, tiles), dim3(256), 0, s, p); break;
        case 128: hipLaunchKernelGGL(sparse_score_kernel<128>, dim3(bgs, tiles), dim3(256), 0, s, p); break;
        case 256: hipLaunchKernelGGL(sparse_score_kernel<256>, dim3(bgs, tiles), dim3(256), 0, s, p); break;
        default: return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sparse_select_kernel, dim3(bgs), dim3(kSelThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace pa
