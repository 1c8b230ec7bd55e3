// Log-sum-exp merge of split-K partials (the "split-KV merge" of the b12x
// kernel credited on the nvllm page, "Acknowledgments").
//
// Partition i of a row carries o_i (normalised within the partition) and its
// natural-log LSE lse_i. With M = max_i lse_i and w_i = exp(lse_i - M):
//   out = sum_i w_i o_i / sum_i w_i,   lse = M + log(sum_i w_i).
// One 256-thread workgroup per (b, t, h) row. Threads are split into
// 256 / D slices over the partitions; thread (slice, d) owns output element d,
// so each slice reads a whole D-vector of a partition per step (coalesced).
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

__global__ __launch_bounds__(256) void splitk_reduce_kernel(ReduceParams p) {
    __shared__ float red[256];
    __shared__ float red_w[256];
    const int tid = threadIdx.x;
    const int64_t rowid = blockIdx.x;
    const int h = (int)(rowid % p.Hq);
    const int t = (int)((rowid / p.Hq) % p.Tq);
    const int b = (int)(rowid / ((int64_t)p.Hq * p.Tq));
    (void)h;
    const int n = p.seq_lens[b] - p.Tq + t + 1;
    const int np = n > 0 ? min((n + p.P - 1) / p.P, p.NP) : 0;
    const float* lse_row = p.ws_lse + rowid * p.NP;
    const float* o_row = p.ws_o + rowid * p.NP * p.D;

    // M = max_i lse_i
    float mx = -INFINITY;
    for (int i = tid; i < np; i += 256) mx = fmaxf(mx, lse_row[i]);
    red[tid] = mx;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
        __syncthreads();
    }
    const float M = red[0];
    __syncthreads();
    const float mref = M == -INFINITY ? 0.0f : M;

    const int slices = 256 / p.D;  // D in {64, 128, 256}
    const int slice = tid / p.D, d = tid % p.D;
    float acc = 0.0f, wsum = 0.0f;
    if (slice < slices) {
#pragma unroll 4
        for (int i = slice; i < np; i += slices) {
            const float li = lse_row[i];
            const float w = li == -INFINITY ? 0.0f : __expf(li - mref);
            wsum += w;
            acc = fmaf(w, o_row[(int64_t)i * p.D + d], acc);
        }
    }
    red[tid] = acc;
    red_w[tid] = wsum;
    __syncthreads();
    if (slice == 0) {
        for (int s2 = 1; s2 < slices; ++s2) {
            acc += red[s2 * p.D + d];
            wsum += red_w[s2 * p.D + d];
        }
        const float val = wsum > 0.0f ? acc / wsum : 0.0f;
        if (p.out_bf16)
            reinterpret_cast<uint16_t*>(p.out)[rowid * p.D + d] = f32_to_bf16(val);
        else
            reinterpret_cast<float*>(p.out)[rowid * p.D + d] = val;
        if (d == 0 && p.lse != nullptr) p.lse[rowid] = wsum > 0.0f ? M + __logf(wsum) : -INFINITY;
    }
}

hipError_t launch_splitk_reduce(const ReduceParams& p, hipStream_t stream) {
    const int64_t rows = (int64_t)p.B * p.Tq * p.Hq;
    if (rows <= 0) return hipSuccess;
    if (rows > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)rows), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa
