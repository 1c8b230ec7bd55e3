// Debug-time validation of the device-side inputs the decode and the cache
// writer trust (block ids, sequence lengths, slots). The vllm-sm70 page
// ("Changes relative to 1Cat-vLLM" and "Known limitations") reports block
// and slot ids that went out of range or pointed into other requests' slots;
// these kernels find such entries without touching the caches.
//
// One workgroup of 256 threads scans everything (a debug aid, not a hot
// path), so no cross-workgroup atomics or pre-zeroed status are needed: the
// workgroup reduces its counts and first offending index in LDS and writes
// the two status words at the end. Every read is in bounds whatever the
// values: a table row is never read past max_blocks, whatever seq_lens says.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {
constexpr int kT = 256;

// count and the smallest flagged index over the workgroup -> status[0..1]
__device__ void finish(int64_t count, int64_t first, int32_t* status) {
    __shared__ int64_t cnt[kT / 64], fst[kT / 64];
    for (int off = 32; off > 0; off >>= 1) {
        count += __shfl_xor(count, off);
        const int64_t o = __shfl_xor(first, off);
        first = o < first ? o : first;
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        cnt[w] = count;
        fst[w] = first;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int64_t c = 0, f = INT64_MAX;
        for (int i = 0; i < kT / 64; ++i) {
            c += cnt[i];
            f = fst[i] < f ? fst[i] : f;
        }
        status[0] = (int32_t)(c > 0x7FFFFFFF ? 0x7FFFFFFF : c);
        status[1] = f == INT64_MAX ? -1 : (int32_t)(f > 0x7FFFFFFF ? 0x7FFFFFFF : f);
    }
}
}  // namespace

// Flat index of a violation: b * (max_blocks + 1) + j for table entry j of
// sequence b, b * (max_blocks + 1) + max_blocks for sequence b's length.
__global__ __launch_bounds__(kT) void decode_check_kernel(DecodeCheckParams p) {
    int64_t count = 0, first = INT64_MAX;
    const int64_t stride = (int64_t)p.max_blocks + 1;
    for (int b = 0; b < p.B; ++b) {
        const int L = p.seq_lens[b];
        const bool bad_len = L < 0 || L > p.max_seq_len;
        if (bad_len && threadIdx.x == 0) {
            ++count;
            first = b * stride + p.max_blocks < first ? b * stride + p.max_blocks : first;
        }
        const int64_t nb_used = L > 0 ? ((int64_t)L + kBlockSize - 1) / kBlockSize : 0;
        const int64_t n = nb_used < p.max_blocks ? nb_used : p.max_blocks;
        for (int64_t j = threadIdx.x; j < n; j += kT) {
            const int32_t id = p.block_table[(int64_t)b * p.max_blocks + j];
            if (id < 0 || id >= p.num_blocks) {
                ++count;
                first = b * stride + j < first ? b * stride + j : first;
            }
        }
    }
    finish(count, first, p.status);
}

// Flat index of a violation: the token index i of a slot >= num_slots (a
// negative slot means "skip" and is valid).
__global__ __launch_bounds__(kT) void slots_check_kernel(SlotsCheckParams p) {
    int64_t count = 0, first = INT64_MAX;
    for (int64_t i = threadIdx.x; i < p.num_tokens; i += kT) {
        const int64_t s = p.slots[i];
        if (s >= p.num_slots) {
            ++count;
            first = i < first ? i : first;
        }
    }
    finish(count, first, p.status);
}

hipError_t launch_decode_check(const DecodeCheckParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(decode_check_kernel, dim3(1), dim3(kT), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_slots_check(const SlotsCheckParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(slots_check_kernel, dim3(1), dim3(kT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pa
