// Log-sum-exp merge of split-K partials (the "split-KV merge" of the b12x
// kernel credited on the nvllm page, "Acknowledgments").
//
// Partition i of a row carries o_i (normalised within the partition) and its
// natural-log LSE lse_i. With M = max_i lse_i and w_i = exp(lse_i - M):
//   out = sum_i w_i o_i / sum_i w_i,   lse = M + log(sum_i w_i).
// Two merges. Rows with few partitions: a workgroup of T threads per row
// (T = 256, or 1024 when a row has more partitions than 256 threads
// preload) in S = T / (D/4) slices; thread (slice, q) owns output elements
// 4q..4q+3 and takes partitions slice, slice + S, ...; the slices meet in
// LDS in a fixed order. Rows with many partitions:
// one wave per (row, column slice), four waves per workgroup, no LDS and no
// barrier: the row's D/4 float4 columns are split over cs waves of CW
// columns each, and lane (s, c) of a wave (column c < CW, slice s < SL =
// 64 / CW) takes partitions s, s + SL, ... . Each lane accumulates its
// partitions in increasing order and the slices are combined by a fixed
// butterfly, so the result is deterministic. The first kPre partitions of
// every lane, with their LSEs, are requested before the row's length is
// known, and the row's maximum is taken from them, so a row of up to kPre
// SL partitions costs one memory round trip; partitions past the row's
// visible length are masked afterwards.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {
constexpr int kPreRow = 8;                // partitions per thread loaded up front (workgroup-per-row merge)

template <int kThreads>
__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

template <int kThreads>
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r += red[i];
    __syncthreads();
    return r;
}
}  // namespace

template <int kThreads>
__global__ __launch_bounds__(kThreads) void splitk_reduce_rows_kernel(ReduceParams p) {
    __shared__ float red[kThreads / 64];
    __shared__ float4 part[kThreads];
    const int tid = threadIdx.x;
    const int64_t rowid = blockIdx.x / p.cs;
    const int csi = blockIdx.x % p.cs;
    const int t = (int)((rowid / p.Hq) % p.Tq);
    const int b = (int)(rowid / ((int64_t)p.Hq * p.Tq));
    // per-head lengths: entry b Hkv + kv head of the row's query head
    const int hl = p.head_lens ? b * p.Hkv + (int)(rowid % p.Hq) / (p.Hq / p.Hkv) : b;
    const float* lse_row = p.ws_lse + rowid * p.NP;
    const float4* o_row = reinterpret_cast<const float4*>(p.ws_o + rowid * p.NP * p.D);
    const int DQ = p.D / 4;     // float4 columns of the row
    const int DQc = DQ / p.cs;  // ... of this workgroup
    const int S = kThreads / DQc;
    const int slice = tid / DQc, qc = tid % DQc;
    const int q = csi * DQc + qc;

    float4 ov[kPreRow];
    float lv[kPreRow];
#pragma unroll
    for (int k = 0; k < kPreRow; ++k) {
        const int i = slice + k * S;
        ov[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        lv[k] = -INFINITY;
        if (i < p.NP) {
            ov[k] = o_row[(int64_t)i * DQ + q];
            lv[k] = lse_row[i];
        }
    }
    // partitions that hold keys of the row (all of them when every partition
    // was written, which the shared-prefix decode's two passes do)
    const int n = p.seq_lens[hl] - p.Tq + t + 1;
    const int np = p.all_parts ? p.NP : n > 0 ? min((n + p.P - 1) / p.P, p.NP) : 0;

    // the slices' preloaded partitions are 0 .. kPreRow * S - 1; the rest is read here
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kPreRow; ++k)
        if (slice + k * S < np) mx = fmaxf(mx, lv[k]);
    for (int i = kPreRow * S + tid; i < np; i += kThreads) mx = fmaxf(mx, lse_row[i]);
    const float M = block_max<kThreads>(mx, red);
    const float mref = M == -INFINITY ? 0.0f : M;

    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float wsum = 0.0f;
    auto add = [&](int i, float li, float4 v) {
        const bool ok = i < np && li != -INFINITY;  // partials past the row's length are stale
        const float w = ok ? __expf(li - mref) : 0.0f;
        if (!ok) v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        acc.x = fmaf(w, v.x, acc.x);
        acc.y = fmaf(w, v.y, acc.y);
        acc.z = fmaf(w, v.z, acc.z);
        acc.w = fmaf(w, v.w, acc.w);
        wsum += w;
    };
#pragma unroll
    for (int k = 0; k < kPreRow; ++k) add(slice + k * S, lv[k], ov[k]);
    for (int i = slice + kPreRow * S; i < np; i += S) add(i, lse_row[i], o_row[(int64_t)i * DQ + q]);
    // every thread of a slice holds the slice's weight sum: count it once
    const float W = block_sum<kThreads>(qc == 0 ? wsum : 0.0f, red);
    part[tid] = acc;
    __syncthreads();
    if (slice == 0) {
        for (int s = 1; s < S; ++s) {
            const float4 v = part[s * DQc + qc];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        const float inv = W > 0.0f ? 1.0f / W : 0.0f;
        const float r[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
        const int64_t o0 = rowid * p.D + 4 * q;
        if (p.out_bf16) {
            uint2 packed;
            packed.x = (uint32_t)f32_to_bf16(r[0]) | ((uint32_t)f32_to_bf16(r[1]) << 16);
            packed.y = (uint32_t)f32_to_bf16(r[2]) | ((uint32_t)f32_to_bf16(r[3]) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + o0) = packed;
        } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + o0) = make_float4(r[0], r[1], r[2], r[3]);
        }
        // the row's first workgroup writes the lse
        if (q == 0 && p.lse != nullptr) p.lse[rowid] = W > 0.0f ? M + __logf(W) : -INFINITY;
    }
}

namespace {
constexpr int kPre = 16;  // partitions per lane requested up front
// Rows with this many partitions merge one wave per column slice; fewer,
// one workgroup per row (measured: 64 partitions of 96 rows 8.1 -> 7.1 us,
// 32 of 768 rows 9.0 -> 9.5 us with the wave merge)
constexpr int kWaveMergeMinPartitions = 48;
}  // namespace

template <int CW>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(ReduceParams p) {
    constexpr int SL = 64 / CW;  // partition slices of a wave
    const int lane = threadIdx.x & 63;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= (int64_t)p.B * p.Tq * p.Hq * p.cs) return;  // whole waves; nothing below synchronises
    const int64_t rowid = wid / p.cs;
    const int csi = (int)(wid % p.cs);
    const int t = (int)((rowid / p.Hq) % p.Tq);
    const int b = (int)(rowid / ((int64_t)p.Hq * p.Tq));
    const int hl = p.head_lens ? b * p.Hkv + (int)(rowid % p.Hq) / (p.Hq / p.Hkv) : b;
    const int c = lane % CW, s = lane / CW;
    const int DQ = p.D / 4;       // float4 columns of the row
    const int q = csi * CW + c;   // this lane's column
    const float* lse_row = p.ws_lse + rowid * p.NP;
    const float4* o_row = reinterpret_cast<const float4*>(p.ws_o + rowid * p.NP * p.D);

    float4 ov[kPre];
    float lv[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
        const int i = s + k * SL;
        ov[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        lv[k] = -INFINITY;
        if (i < p.NP) {
            ov[k] = o_row[(int64_t)i * DQ + q];
            lv[k] = lse_row[i];
        }
    }
    // partitions that hold keys of the row (all of them when every partition
    // was written, which the shared-prefix decode's two passes do)
    const int n = p.seq_lens[hl] - p.Tq + t + 1;
    const int np = p.all_parts ? p.NP : n > 0 ? min((n + p.P - 1) / p.P, p.NP) : 0;

    // the row's largest LSE: the preloaded partitions (kPre SL of them, every
    // partition of most rows) from registers, any later ones loaded here
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kPre; ++k)
        if (s + k * SL < np) mx = fmaxf(mx, lv[k]);
    for (int i = kPre * SL + lane; i < np; i += 64) mx = fmaxf(mx, lse_row[i]);
    const float M = wave_max(mx);
    const float mref = M == -INFINITY ? 0.0f : M;

    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float wsum = 0.0f;
    auto add = [&](int i, float li, float4 v) {
        const bool ok = i < np && li != -INFINITY;  // partials past the row's length are stale
        const float w = ok ? __expf(li - mref) : 0.0f;
        if (!ok) v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        acc.x = fmaf(w, v.x, acc.x);
        acc.y = fmaf(w, v.y, acc.y);
        acc.z = fmaf(w, v.z, acc.z);
        acc.w = fmaf(w, v.w, acc.w);
        wsum += w;
    };
#pragma unroll
    for (int k = 0; k < kPre; ++k) add(s + k * SL, lv[k], ov[k]);
    for (int i = s + kPre * SL; i < np; i += SL) add(i, lse_row[i], o_row[(int64_t)i * DQ + q]);
    // the CW lanes of a slice share its partitions: count its weights once
    const float W = wave_sum(c == 0 ? wsum : 0.0f);
#pragma unroll
    for (int m = CW; m < 64; m *= 2) {
        acc.x += __shfl_xor(acc.x, m);
        acc.y += __shfl_xor(acc.y, m);
        acc.z += __shfl_xor(acc.z, m);
        acc.w += __shfl_xor(acc.w, m);
    }
    if (s == 0) {
        const float inv = W > 0.0f ? 1.0f / W : 0.0f;
        const float r[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
        const int64_t o0 = rowid * p.D + 4 * q;
        if (p.out_bf16) {
            uint2 packed;
            packed.x = (uint32_t)f32_to_bf16(r[0]) | ((uint32_t)f32_to_bf16(r[1]) << 16);
            packed.y = (uint32_t)f32_to_bf16(r[2]) | ((uint32_t)f32_to_bf16(r[3]) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + o0) = packed;
        } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out) + o0) = make_float4(r[0], r[1], r[2], r[3]);
        }
        // the row's first wave writes the lse
        if (q == 0 && p.lse != nullptr) p.lse[rowid] = W > 0.0f ? M + __logf(W) : -INFINITY;
    }
}

hipError_t launch_splitk_reduce(const ReduceParams& p0, hipStream_t stream) {
    const int64_t rows = (int64_t)p0.B * p0.Tq * p0.Hq;
    if (rows <= 0) return hipSuccess;
    ReduceParams p = p0;
    const int DQ = p.D / 4;
    if (p.NP < kWaveMergeMinPartitions) {
        // a workgroup per row, its threads in partition slices of D/4 columns
        if (rows > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
        p.cs = 1;
        if ((int64_t)p.NP * DQ <= (int64_t)256 * kPreRow)
            hipLaunchKernelGGL(splitk_reduce_rows_kernel<256>, dim3((unsigned)rows), dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL(splitk_reduce_rows_kernel<1024>, dim3((unsigned)rows), dim3(1024), 0, stream, p);
        return hipGetLastError();
    }
    // split the columns until there are 2048 waves (eight per CU), keeping
    // at least 4 columns per wave and no more slices than partitions
    p.cs = DQ > 64 ? DQ / 64 : 1;
    auto cw = [&](int cs) { return DQ / cs; };
    while (rows * p.cs < 2048 && cw(2 * p.cs) >= 4 && 64 / cw(2 * p.cs) <= p.NP) p.cs *= 2;
    const int64_t waves = rows * p.cs;
    const int64_t grid = (waves + 3) / 4;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    switch (cw(p.cs)) {
    case 64: hipLaunchKernelGGL(splitk_reduce_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, p); break;
    case 32: hipLaunchKernelGGL(splitk_reduce_kernel<32>, dim3((unsigned)grid), dim3(256), 0, stream, p); break;
    case 16: hipLaunchKernelGGL(splitk_reduce_kernel<16>, dim3((unsigned)grid), dim3(256), 0, stream, p); break;
    case 8: hipLaunchKernelGGL(splitk_reduce_kernel<8>, dim3((unsigned)grid), dim3(256), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(splitk_reduce_kernel<4>, dim3((unsigned)grid), dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pa
