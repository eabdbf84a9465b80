// pa_order.hip -- a longest-first dispatch order computed on the device.
//
// Continuous batching admits a request as soon as its page budget is free
// (samir-vllm, "Gestion de la KV cache et strategies de batching"), so one
// decode batch mixes contexts of very different lengths.  A decode launch
// dealt in slot order can then start its longest sequences last, and they run
// on alone, as the launch's tail.  This kernel ranks the sequences by their
// lengths where the lengths live, in device memory, so that a caller can
// order every layer's decode of a step with one small launch and without
// reading the lengths back.  The order changes only when each (sequence, KV
// head) is served, never the arithmetic that serves it.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kOrderThreads = kMaxDispatchOrder;  // one sequence per thread, one workgroup
constexpr int kOrderWaves = kOrderThreads / 64;
constexpr int kOrderClasses = 64;
static_assert(kOrderClasses * kOrderWaves == kOrderThreads, "one (class, wave) count per thread");

// number of set bits of m in the lanes below this one
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// Rank = (longer classes first) + (same class, lower index first).  A class
// spans cw = ceil(max_blocks / 64) pages: sequence s with 1 <= L <= 16 *
// max_blocks has class (ceil(L / 16) - 1) / cw; a length outside that range
// (which the decode rejects) has class 0, the last.  The ranks are then dealt
// in runs: long_run from the long end, short_run from the short end, and so
// on until the two meet; order[position] = s.
__device__ __forceinline__ int mixed_position(int r, int n, int k, int m) {
    const int G = n / (k + m), R = n % (k + m);
    const int from_long = G * k + min(R, k);  // ranks dealt from the long end
    if (r < from_long) return (r / k) * (k + m) + r % k;
    const int t = n - 1 - r;  // 0 = the shortest
    return (t / m) * (k + m) + k + t % m;
}

__global__ __launch_bounds__(kOrderThreads) void k_order_by_length(const int32_t *lens, int n, int max_blocks,
                                                                   int long_run, int short_run, int32_t *order) {
    __shared__ int s_cnt[kOrderClasses][kOrderWaves];   // members of class v among wave w's sequences
    __shared__ int s_base[kOrderClasses][kOrderWaves];  // rank of the first of them
    __shared__ int s_scan_total[kOrderWaves];
    const int t = threadIdx.x;
    const int lane = t & 63;
    const int w = t >> 6;
    const int cw = (max_blocks + kOrderClasses - 1) / kOrderClasses;
    int cls = kOrderClasses;  // past the last class: no sequence
    if (t < n) {
        const int64_t L = lens[t];
        cls = (L >= 1 && L <= static_cast<int64_t>(max_blocks) * kPage)
                  ? static_cast<int>(((L + kPage - 1) / kPage - 1) / cw) : 0;
    }
    s_cnt[t / kOrderWaves][t % kOrderWaves] = 0;
    // The lanes of this wave in the same class as this lane, bit-sliced: one
    // ballot per bit of the class (7 bits: 64 classes and "none"), and this
    // lane keeps the lanes that agree with it on every bit.
    uint64_t same = ~0ull;
#pragma unroll
    for (int k = 0; k < 7; ++k) {
        const uint64_t bk = __ballot((cls >> k) & 1);
        same &= ((cls >> k) & 1) ? bk : ~bk;
    }
    const int within = lanes_below(same);  // members of its class in this wave, below this lane
    __syncthreads();
    if (cls < kOrderClasses && within == 0) s_cnt[cls][w] = __popcll(same);
    __syncthreads();
    // Exclusive scan of the counts in rank order (class descending, wave
    // ascending): thread k holds entry k of that order.  Within a wave the
    // prefix is formed bit by bit (a count is at most 64, 7 bits); the waves'
    // totals are then added in.
    const int v = kOrderClasses - 1 - t / kOrderWaves;
    const int ww = t % kOrderWaves;
    const int c = s_cnt[v][ww];
    int pre = 0;
#pragma unroll
    for (int k = 0; k < 7; ++k) pre += lanes_below(__ballot((c >> k) & 1)) << k;
    if (lane == 63) s_scan_total[w] = pre + c;
    __syncthreads();
    for (int x = 0; x < w; ++x) pre += s_scan_total[x];
    s_base[v][ww] = pre;
    __syncthreads();
    if (t < n) order[mixed_position(s_base[cls][w] + within, n, long_run, short_run)] = t;
}

}  // namespace

hipError_t launch_order_by_length(const int32_t *lens, int n, int max_blocks, int long_run, int short_run,
                                  int32_t *order, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_order_by_length, dim3(1), dim3(kOrderThreads), 0, stream, lens, n, max_blocks, long_run,
                       short_run, order);
    return hipGetLastError();
}

}  // namespace pa
