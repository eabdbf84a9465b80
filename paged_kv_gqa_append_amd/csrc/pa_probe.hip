// pa_probe.hip -- contiguous-read probe: the bandwidth a plain read stream
// reaches on this GPU, the ceiling the paged kernels' figures are compared
// with.  Workgroup w reads one contiguous chunk of the buffer, 16 bytes per
// lane and kProbeLoads loads in flight per lane (each load instruction covers
// 4 KiB), with the non-temporal hint; of the forms measured on MI355X
// (grid-stride or one chunk per workgroup, with or without the hint, 4 to 16
// loads in flight, 256 to 4096 workgroups of 256 or 512 lanes) this one was
// at or within 1 % of the fastest at 136 MiB, 256 MiB and 1 GiB.  Each lane
// XORs what it reads and stores one word only if that XOR equals a fixed
// constant, so the loads cannot be removed and nothing of size is written.
#include <algorithm>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 8;           // 16-byte loads in flight per lane
constexpr int64_t kProbeMaxBlocks = 2048;  // 8 workgroups per CU
constexpr uint32_t kProbeMagic = 0x9E3779B9u;

__global__ __launch_bounds__(kProbeThreads) void k_stream_read(const u32x4 *__restrict__ buf, int64_t n_vec,
                                                               int64_t per, uint32_t *__restrict__ sink) {
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * per;
    const int64_t hi = min(n_vec, lo + per);
    int64_t i = lo + threadIdx.x;
    uint32_t acc = 0;
    // whole groups of kProbeLoads vectors: the loads are unconditional, so
    // they are all in flight before the first is consumed
    for (; i + (kProbeLoads - 1) * kProbeThreads < hi; i += kProbeLoads * kProbeThreads) {
        u32x4 v[kProbeLoads];
#pragma unroll
        for (int u = 0; u < kProbeLoads; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kProbeLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < hi; i += kProbeThreads) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == kProbeMagic) sink[0] = acc;
}

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream) {
    const int64_t n_vec = static_cast<int64_t>(bytes / 16);
    if (n_vec == 0) return hipSuccess;
    // chunk per workgroup: a whole number of unrolled groups, at most
    // kProbeMaxBlocks chunks; every workgroup's chunk starts inside the buffer
    const int64_t unit = static_cast<int64_t>(kProbeThreads) * kProbeLoads;
    const int64_t per = ((n_vec + kProbeMaxBlocks - 1) / kProbeMaxBlocks + unit - 1) / unit * unit;
    const int64_t blocks = (n_vec + per - 1) / per;
    hipLaunchKernelGGL(k_stream_read, dim3(static_cast<unsigned>(blocks)), dim3(kProbeThreads), 0, stream,
                       static_cast<const u32x4 *>(buf), n_vec, per, sink);
    return hipGetLastError();
}

}  // namespace pa
