// Read-bandwidth probe: the streaming-read ceiling that the decode's read
// rate is set against (a plain read of a large buffer, every byte once, with
// the decode kernels' nontemporal 16-byte buffer loads). The loaded words are
// summed (32-bit, wrapping) per workgroup so that no load is dropped and the
// caller can check that every word was read exactly once.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;                                     // loads in flight per thread
constexpr int kProbeSeg = kProbeThreads * kProbeUnroll * 16;       // bytes per workgroup and iteration
}  // namespace

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const unsigned char* buf, int64_t bytes,
                                                                    uint32_t* sink) {
    __shared__ uint32_t red[kProbeThreads / 64];
    uint32_t acc = 0u;
    const int64_t nseg = (bytes + kProbeSeg - 1) / kProbeSeg;
    for (int64_t s = blockIdx.x; s < nseg; s += gridDim.x) {
        const int64_t base = s * kProbeSeg;
        const int64_t left = bytes - base;
        // the segment's resource ends at the buffer's end: loads past it read 0
        const auto rs = range_rsrc(buf + base, (uint32_t)(left < kProbeSeg ? left : kProbeSeg));
        Raw<16> r[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) load_buf<16>(r[u], rs, 16 * ((int)threadIdx.x + kProbeThreads * u), 0);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc += r[u].w[0] + r[u].w[1] + r[u].w[2] + r[u].w[3];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += (uint32_t)__shfl_xor((int)acc, m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0u;
#pragma unroll
        for (int w = 0; w < kProbeThreads / 64; ++w) t += red[w];
        sink[blockIdx.x] = t;
    }
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int workgroups, hipStream_t stream) {
    if (workgroups < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream,
                       reinterpret_cast<const unsigned char*>(buf), bytes, sink);
    return hipGetLastError();
}

}  // namespace pa
