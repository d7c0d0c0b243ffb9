// Plain streaming read of a device buffer: the achievable HBM read rate of
// this GPU, measured beside the paged decode (whose only significant traffic
// is reading each needed page once), so that the decode's rate can be read
// against what a trivial kernel reaches as well as against the spec peak.
// Every lane loads 16-byte pieces grid-stride, eight in flight, and folds them
// with XOR; one atomic XOR per wave into *sink keeps the loads alive.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeGrid = 2048;   // 8 workgroups per CU

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4 *__restrict__ src, size_t n16,
                                                                   uint32_t *__restrict__ sink)
{
    const size_t stride = (size_t)gridDim.x * kProbeThreads;
    size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        u32x4 a[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= a[u][0] ^ a[u][1] ^ a[u][2] ^ a[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 a = src[i];
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

}  // namespace

hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    const size_t n16 = bytes / 16;
    const size_t need = (n16 + kProbeThreads - 1) / kProbeThreads;
    const unsigned grid = (unsigned)(need < (size_t)kProbeGrid ? (need ? need : 1) : (size_t)kProbeGrid);
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4 *>(src), n16, sink);
    return hipGetLastError();
}

}  // namespace fa
