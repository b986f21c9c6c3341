// Platform probe: the streaming-read rate this part delivers to a plain
// kernel ("GEMM Kernel 性能优化十问", Q10, step 0: measure the new
// platform's memory bandwidth before deciding whether a kernel is
// compute- or memory-bound).  Each workgroup reads one 64 KB slice of the
// buffer with 16-byte loads, every load issued before any is consumed, and
// folds the words into one value that is stored only if it equals a
// constant no real buffer sums to by accident (so the loads stay live).
#include "gmm_launch.hpp"

namespace gmm {

namespace {

constexpr int kProbeSlice16 = 4096;   // 16-byte words per workgroup (64 KB)

__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ buf,
                                                          uint32_t* __restrict__ sink) {
    const uint4* q = buf + (size_t)blockIdx.x * kProbeSlice16;
    uint32_t acc = 0;
#pragma unroll
    for (int i = threadIdx.x; i < kProbeSlice16; i += 256) {
        const uint4 v = q[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

hipError_t launch_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink,
                                    hipStream_t stream) {
    const int64_t slices = bytes / (kProbeSlice16 * 16);
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)slices), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(buf), sink);
    return hipGetLastError();
}

}  // namespace gmm
