// Plain streaming read of a device buffer: the achievable HBM read rate of
// this GPU, measured beside the paged decode (whose only significant traffic
// is reading each needed page once), so that the decode's rate can be read
// against what a trivial kernel reaches as well as against the spec peak.
// Each workgroup streams one contiguous slab of the buffer, every lane eight
// 16-byte pieces in flight (non-temporal), folded with XOR; one atomic XOR
// per wave into *sink keeps the loads alive (so *sink ends as the XOR of every
// 32-bit word read). Measured on MI355X over 8 GiB: 512 slabs reach about
// 7.1 TB/s, 1024 slabs 6.9, 2048 slabs 6.5; a grid-stride sweep over the same
// buffer by 2048 workgroups 6.2; and workgroups reading random 4 KiB blocks
// (the decode's unit, one (page, head) of the cache) 6.3-6.5.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeGrid = 512;   // 2 workgroups per CU
constexpr int kProbeInFlight = 8;

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4 *__restrict__ src, size_t n16,
                                                                   uint32_t *__restrict__ sink)
{
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = min(n16, (size_t)blockIdx.x * per), b1 = min(n16, b0 + per);
    uint32_t acc = 0;
    size_t i = b0 + threadIdx.x;
    for (; i + (kProbeInFlight - 1) * kProbeThreads < b1; i += kProbeInFlight * kProbeThreads) {
        u32x4 a[kProbeInFlight];
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) a[u] = __builtin_nontemporal_load(src + i + u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) acc ^= a[u][0] ^ a[u][1] ^ a[u][2] ^ a[u][3];
    }
    for (; i < b1; i += kProbeThreads) {
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
