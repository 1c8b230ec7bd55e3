// Log-sum-exp merge of split-K partials (the "split-KV merge" of the b12x
// kernel credited on the nvllm page, "Acknowledgments").
//
// Partition i of a row carries o_i (normalised within the partition) and its
// natural-log LSE lse_i. With M = max_i lse_i and w_i = exp(lse_i - M):
//   out = sum_i w_i o_i / sum_i w_i,   lse = M + log(sum_i w_i).
// cs workgroups of T threads per (b, t, h) row, each taking C = D/(4 cs)
// float4 columns (T = 256, or 1024 when a row has more partitions than 256
// threads preload). The column split keeps a batch of few rows from putting
// all of a row's partials through one CU. A workgroup's threads form
// S = T / C slices of C threads; thread (slice, q) owns output elements
// 4q..4q+3 (one 16-byte load per partition) and takes partitions slice,
// slice + S, ... . Slices are combined in a fixed order, so the result is
// deterministic, and every workgroup of a row computes the same M and W. Every load of the first kPre partitions of a thread is
// issued before the row's length is known (addresses depend only on the
// partition count), so the row costs one memory round trip; partitions past
// the row's visible length are masked afterwards.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {
constexpr int kPre = 8;                   // partitions per thread loaded up front
constexpr int kSplitMinPartitions = 160;  // column-split the rows above this many partitions

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
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(ReduceParams p) {
    __shared__ float red[kThreads / 64];
    __shared__ float4 part[kThreads];
    const int tid = threadIdx.x;
    const int64_t rowid = blockIdx.x / p.cs;
    const int csi = blockIdx.x % p.cs;
    const int t = (int)((rowid / p.Hq) % p.Tq);
    const int b = (int)(rowid / ((int64_t)p.Hq * p.Tq));
    const float* lse_row = p.ws_lse + rowid * p.NP;
    const float4* o_row = reinterpret_cast<const float4*>(p.ws_o + rowid * p.NP * p.D);
    const int DQ = p.D / 4;     // float4 columns of the row
    const int DQc = DQ / p.cs;  // ... of this workgroup
    const int S = kThreads / DQc;
    const int slice = tid / DQc, qc = tid % DQc;
    const int q = csi * DQc + qc;

    float4 ov[kPre];
    float lv[kPre];
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
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
    const int n = p.seq_lens[b] - p.Tq + t + 1;
    const int np = p.all_parts ? p.NP : n > 0 ? min((n + p.P - 1) / p.P, p.NP) : 0;

    // the slices' preloaded partitions are 0 .. kPre * S - 1; the rest is read here
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kPre; ++k)
        if (slice + k * S < np) mx = fmaxf(mx, lv[k]);
    for (int i = kPre * S + tid; i < np; i += kThreads) mx = fmaxf(mx, lse_row[i]);
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
    for (int k = 0; k < kPre; ++k) add(slice + k * S, lv[k], ov[k]);
    for (int i = slice + kPre * S; i < np; i += S) add(i, lse_row[i], o_row[(int64_t)i * DQ + q]);
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

hipError_t launch_splitk_reduce(const ReduceParams& p0, hipStream_t stream) {
    const int64_t rows = (int64_t)p0.B * p0.Tq * p0.Hq;
    if (rows <= 0) return hipSuccess;
    ReduceParams p = p0;
    // many partitions per row: split the columns until the grid has 512
    // workgroups or each takes 4 float4 columns (measured: at 250K tokens and
    // 24 rows, 252 partitions merge in 9.1 us split, 10.9 unsplit; at 128 or
    // fewer partitions the split is slower)
    const int DQ = p.D / 4;
    p.cs = 1;
    if (p.NP > kSplitMinPartitions)
        while (rows * p.cs < 512 && DQ / (2 * p.cs) >= 4) p.cs *= 2;
    const int64_t grid = rows * p.cs;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if ((int64_t)p.NP * (DQ / p.cs) <= (int64_t)256 * kPre)
        hipLaunchKernelGGL(splitk_reduce_kernel<256>, dim3((unsigned)grid), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<1024>, dim3((unsigned)grid), dim3(1024), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa
