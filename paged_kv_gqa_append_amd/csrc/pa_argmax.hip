// pa_argmax.hip -- greedy next-token choice on the GPU: the index of the
// largest logit of each row.
//
// samir-vllm article, section "Architecture et flux d'inference": the engine
// takes the argmax on the GPU.  tiny-vllm ch.2, section "Preallocating the 16
// compute buffers": the CPU argmax it replaces scans the row with a strict
// greater-than from element 0, so the first maximum wins.  Here NaN entries
// are never chosen (the pages are silent on them), -0.0 equals +0.0, and a row
// of NaN only gives 0.
//
// The work is a read of rows x vocab logits with one compare per element:
// HBM-bound.  A workgroup of 256 threads scans one chunk of one row, every
// thread issuing all of its 16-byte loads before it compares anything; within
// a thread indices only grow, so a strict > keeps the first maximum.  Threads,
// waves and chunks then combine (value, index) pairs through a 64-bit key
// that orders by value first and by lower index second.  Rows longer than
// one chunk fold each chunk's key into the row's word of the workspace with an
// atomic max; the chunk that arrives last (an arrival count beside the key)
// writes the index and sets both words back to zero, so one launch does the
// whole call and the workspace is left as it was found.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kArgThreads = 256;
constexpr int kArgLoads = 8;  // 16-byte loads per thread per chunk

// Monotone unsigned key of a float's bits: a larger value has a larger key,
// -0.0 and +0.0 share one, and NaN gets 0 (below -inf, whose key is 0x007FFFFF).
__device__ __forceinline__ uint32_t order_key(uint32_t u) {
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// (key, index) packed so that unsigned max picks the larger key, then the
// smaller index; "nothing seen" (index 0xFFFFFFFF with key 0) packs to 0.
__device__ __forceinline__ uint64_t pack_key(uint32_t key, uint32_t idx) {
    return (static_cast<uint64_t>(key) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ int32_t unpack_index(uint64_t k) {
    return k == 0 ? 0 : static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(k));
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
        const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), k, 64);
        const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), k, 64);
        v = max_u64(v, (static_cast<uint64_t>(hi) << 32) | lo);
    }
    return v;
}

// Strict-greater update of a thread's running best; the first element it sees
// is taken whatever its value (unless NaN), so -inf rows still name an index.
__device__ __forceinline__ void take(float v, uint32_t i, float &best, uint32_t &bi) {
    const bool first = bi == 0xFFFFFFFFu && !isnan(v);
    if (v > best || first) {
        best = v;
        bi = i;
    }
}

template <bool kBF16>
__device__ __forceinline__ float load_scalar(const void *p, int64_t k) {
    if (kBF16) return bf16_to_f32(static_cast<const uint16_t *>(p)[k]);
    return static_cast<const float *>(p)[k];
}

// grid (splits, rows).  kVec: every row starts 16-byte aligned and holds a
// whole number of 16-byte vectors, and chunk is a multiple of 256 vectors.
// ws (splits > 1): per row a running key and an arrival count, both zero on
// entry and zero again once the row's last chunk has finished.
template <bool kBF16, bool kVec>
__global__ __launch_bounds__(kArgThreads) void k_argmax(const void *__restrict__ logits, int vocab, int chunk,
                                                       int splits, uint64_t *__restrict__ ws,
                                                       int32_t *__restrict__ out) {
    constexpr int E = kBF16 ? 8 : 4;  // elements per 16-byte vector
    const int split = blockIdx.x;
    const int row = blockIdx.y;
    const int tid = threadIdx.x;
    const int64_t rbase = static_cast<int64_t>(row) * vocab;
    const int c0 = split * chunk;
    const int c1 = min(vocab, c0 + chunk);
    float best = -INFINITY;
    uint32_t bi = 0xFFFFFFFFu;
    if (kVec) {
        u32x4 buf[kArgLoads];
#pragma unroll
        for (int u = 0; u < kArgLoads; ++u) {
            const int i0 = c0 + (u * kArgThreads + tid) * E;
            if (i0 < c1) {
                const char *p = static_cast<const char *>(logits) + (rbase + i0) * (kBF16 ? 2 : 4);
                buf[u] = *reinterpret_cast<const u32x4 *>(p);
            }
        }
#pragma unroll
        for (int u = 0; u < kArgLoads; ++u) {
            const int i0 = c0 + (u * kArgThreads + tid) * E;
            if (i0 < c1) {
                const uint32_t w[4] = {buf[u].x, buf[u].y, buf[u].z, buf[u].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if (kBF16) {
                        take(bf16_lo(w[k]), i0 + 2 * k, best, bi);
                        take(bf16_hi(w[k]), i0 + 2 * k + 1, best, bi);
                    } else {
                        take(__builtin_bit_cast(float, w[k]), i0 + k, best, bi);
                    }
                }
            }
        }
    } else {
        for (int i = c0 + tid; i < c1; i += kArgThreads) take(load_scalar<kBF16>(logits, rbase + i), i, best, bi);
    }
    uint64_t key = bi == 0xFFFFFFFFu ? 0 : pack_key(order_key(__builtin_bit_cast(uint32_t, best)), bi);
    key = wave_max_u64(key);
    __shared__ uint64_t s_key[kArgThreads / 64];
    if ((tid & 63) == 0) s_key[tid >> 6] = key;
    __syncthreads();
    if (tid != 0) return;
#pragma unroll
    for (int w = 1; w < kArgThreads / 64; ++w) key = max_u64(key, s_key[w]);
    if (splits == 1) {
        out[row] = unpack_index(key);
        return;
    }
    uint64_t *row_key = ws + 2 * static_cast<int64_t>(row);
    uint64_t *row_count = row_key + 1;
    // Ordering without cache maintenance.  Every access to the row's two
    // words is an agent-scope atomic read-modify-write, so each is performed at
    // the one point where that address is kept coherent for all XCDs.  The
    // arrival is not issued until the max has returned its old value (the
    // increment is computed from it; no key is all ones), so the max has been
    // performed first.  The last arrival sees every other arrival performed,
    // hence every maximum, before it reads and clears the key.  An agent-scope
    // release/acquire pair would say the same to the compiler, but it writes
    // back and invalidates the whole L2 in every workgroup (a third slower).
    const uint64_t prev = __hip_atomic_fetch_max(row_key, key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t before =
        __hip_atomic_fetch_add(row_count, prev == ~0ull ? 2ull : 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (before == static_cast<uint64_t>(splits - 1)) {
        const uint64_t row_best = __hip_atomic_exchange(row_key, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_exchange(row_count, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        out[row] = unpack_index(row_best);
    }
}

int argmax_chunk_elems(bool bf16) { return kArgThreads * kArgLoads * (bf16 ? 8 : 4); }

hipError_t launch_argmax(int32_t *out, const void *logits, int rows, int vocab, bool bf16, bool vec, void *workspace,
                         hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    const int chunk = argmax_chunk_elems(bf16);
    const int splits = (vocab + chunk - 1) / chunk;
    uint64_t *ws = static_cast<uint64_t *>(workspace);
    const dim3 grid(static_cast<unsigned>(splits), static_cast<unsigned>(rows));
    if (bf16) {
        if (vec) hipLaunchKernelGGL((k_argmax<true, true>), grid, dim3(kArgThreads), 0, stream, logits, vocab, chunk, splits, ws, out);
        else hipLaunchKernelGGL((k_argmax<true, false>), grid, dim3(kArgThreads), 0, stream, logits, vocab, chunk, splits, ws, out);
    } else {
        if (vec) hipLaunchKernelGGL((k_argmax<false, true>), grid, dim3(kArgThreads), 0, stream, logits, vocab, chunk, splits, ws, out);
        else hipLaunchKernelGGL((k_argmax<false, false>), grid, dim3(kArgThreads), 0, stream, logits, vocab, chunk, splits, ws, out);
    }
    return hipGetLastError();
}

}  // namespace pa
