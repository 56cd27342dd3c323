// probe.hip -- streaming-read probe: the achievable HBM read rate of this GPU,
// against which the decode's bandwidth is reported.
#include "device.hpp"
#include "kernels.hpp"

namespace mpa {

// Grid-stride 16-byte loads, four in flight per thread, no reuse.  The XOR of
// everything read is compared with a constant so the loads stay live; sink is
// written only on that (practically impossible) match.
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, size_t n16,
                                                         uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    hipLaunchKernelGGL(read_probe_kernel, dim3(cus * 8), dim3(256), 0, st, (const uint4*)buf, bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace mpa
