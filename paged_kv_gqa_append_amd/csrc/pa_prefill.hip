// pa_prefill.hip -- causal chunked-prefill attention over the paged pool, on
// bf16 MFMA tiles (gfx950 v_mfma_f32_32x32x16_bf16), fp32 accumulation.
//
// What is computed (TinyLoop, section "prefill_chunk and scratch residency":
// the prompt is processed in row chunks; samir-vllm, "Gestion de la KV cache
// ...": the prompt's pages are filled during prefill): after the chunk's K/V
// rows have been appended and its q rows rotated (k_append_rope, prefix mode),
// every chunk query at absolute position p = prefix + i attends to keys
// 0..p of its sequence, read through the block table:
//     out[s][i][h] = sum_t softmax_t(scale <q[s][i][h], K_t>) V_t,  t <= p.
// No score matrix is stored (contrast tiny-vllm's prefill, which keeps a
// 512 x 512 x 32 score buffer, ch.2 buffer table).
//
// Work decomposition
//   One workgroup per (sequence, KV head j, tile of 32 chunk positions); its 4
//   waves are the 4 query heads of that KV head, so every K/V block serves 4 x
//   32 query rows.  Keys are taken 32 at a time (two pages).
//   Scores are computed transposed, S^T = K Q^T (32 keys x 32 queries per
//   wave): in the MFMA result layout each lane then holds 16 keys of ONE query
//   (lane l: query l%32, keys 8i + 4(l/32) + r for register 4i+r), so the
//   online softmax is lane-local plus one exchange with lane l^32.
//   The output is accumulated transposed too, O^T = V^T P^T (64 d x 32
//   queries): same lane-per-query layout, so rescaling is lane-local.  P^T is
//   the MFMA B operand straight from the score registers; the key slots of
//   the MFMA are permuted to match, and V^T is staged in LDS in that order.
//   P is fed as a bf16 hi/lo pair (two MFMAs), so the weights keep ~16
//   significant bits; V and q, K are bf16 as stored.
//   Online softmax in log2 units with a lazy running max (rescale only when
//   a score exceeds it by more than 2^8), as in the decode kernel.
#include <math.h>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kQT = 32;           // chunk positions per workgroup
constexpr int kKB = 32;           // keys per block
constexpr int kVtStride = 36;     // bf16 per V^T row in LDS (32 keys + 4 pad: spreads banks)
constexpr float kNegBig = -1.0e30f;
constexpr float kRescaleLog2 = 8.0f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value of lane l^32 (permlane32 swap; the second operand is hidden from the
// compiler, which would otherwise fold a swap of equal operands).
__device__ __forceinline__ float partner32(float v) {
    const unsigned a = __builtin_bit_cast(unsigned, v);
    unsigned b = a;
    asm volatile("" : "+v"(b));
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    // lanes < 32 keep their own value in r0 and get the partner's in r1
    return __lane_id() < 32 ? __builtin_bit_cast(float, r1) : __builtin_bit_cast(float, r0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace

struct PrefillParams {
    void *out;
    const uint16_t *q;
    const uint16_t *k_pool;
    const uint16_t *v_pool;
    const int32_t *bt;
    const int32_t *prefix_lens;
    int chunk_len;
    int max_blocks;
    int num_pages;
    int max_pos;
    int n_tiles;
    float scale_log2;
    int out_fp32;
    uint32_t *flags;
};

__global__ __launch_bounds__(256) void k_prefill_attn(PrefillParams P) {
    const int tile = P.n_tiles - 1 - (blockIdx.x % P.n_tiles);  // longest tiles are dispatched first
    const int sj = blockIdx.x / P.n_tiles;
    const int j = sj & (kHKV - 1);
    const int s = sj >> 3;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int h = j * kGroup + w;
    const int C = P.chunk_len;
    const int i0 = tile * kQT;

    __shared__ int s_pages[kMaxBlocksPrefill];
    __shared__ __align__(16) uint16_t s_vt[kD * kVtStride];  // V^T of one key block: [d][key]

    // ---- validation: the whole sequence's pages, as the append saw them -----
    const int prefix = P.prefix_lens[s];
    const int total = prefix + C;
    const bool len_ok = prefix >= 0 && total <= P.max_blocks * kPage && total <= P.max_pos &&
                        P.max_blocks <= kMaxBlocksPrefill;
    const int n_pages = len_ok ? (total + kPage - 1) / kPage : 0;
    const int32_t *bt_row = P.bt + static_cast<int64_t>(s) * P.max_blocks;
    int bad = 0;
    for (int b = tid; b < n_pages; b += 256) {
        const int pid = bt_row[b];
        s_pages[b] = pid;
        bad |= (pid < 0) | (pid >= P.num_pages);
    }
    const bool ok = len_ok && __syncthreads_or(bad) == 0;
    const int qcol = lane & 31;   // this lane's query within the tile
    const int half = lane >> 5;   // which 4-key run of every 8 this lane holds
    const int iq = i0 + qcol;
    const bool q_valid = iq < C;
    if (!ok) {  // zero-fill this tile's rows of this head, flag once
        if (q_valid && half == 0) {
            const int64_t o = ((static_cast<int64_t>(s) * C + iq) * kHQ + h) * kD;
            for (int d = 0; d < kD; ++d) {
                if (P.out_fp32) static_cast<float *>(P.out)[o + d] = 0.0f;
                else static_cast<uint16_t *>(P.out)[o + d] = 0;
            }
        }
        if (tid == 0 && tile == P.n_tiles - 1 && P.flags) atomicOr(P.flags, len_ok ? kDevErrPageId : kDevErrContextLen);
        return;
    }

    // ---- q^T fragments (MFMA B operand): query qcol, d = 16kk + 8*half .. +7 --
    const int iq_c = min(iq, C - 1);
    const int pq = prefix + iq_c;  // absolute position of this lane's query
    const uint16_t *qrow = P.q + ((static_cast<int64_t>(s) * C + iq_c) * kHQ + h) * kD;
    bf16x8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4 *>(qrow + 16 * kk + 8 * half));

    // keys needed by this tile: 0 .. prefix + last valid query position
    const int last_key = prefix + min(i0 + kQT, C) - 1;
    const int n_kb = last_key / kKB + 1;
    const int64_t tile_j = static_cast<int64_t>(j) * kTile;

    float m_run = kNegBig;
    float l_run = 0.0f;
    f32x16 o0 = {}, o1 = {};  // O^T for d 0..31 and 32..63 (lane: query qcol)

    for (int kb = 0; kb < n_kb; ++kb) {
        // -- stage V^T of this block in LDS: thread t moves key t>>3, d 8(t&7)..+7
        {
            const int kr = tid >> 3, c8 = tid & 7;
            const int key = kb * kKB + kr;
            u32x4 v = {0, 0, 0, 0};
            if (key < total) {
                const int64_t row = static_cast<int64_t>(s_pages[key >> 4]) * kPageElems + tile_j + (key & 15) * kD;
                v = *reinterpret_cast<const u32x4 *>(P.v_pool + row + 8 * c8);
            }
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s_vt[(8 * c8 + 2 * e) * kVtStride + kr] = static_cast<uint16_t>(wv[e] & 0xFFFFu);
                s_vt[(8 * c8 + 2 * e + 1) * kVtStride + kr] = static_cast<uint16_t>(wv[e] >> 16);
            }
        }
        // -- K fragments (MFMA A operand): key kb*32 + qcol, d = 16kk + 8*half .. +7
        bf16x8 kf[4];
        {
            const int key = kb * kKB + qcol;
            const int kc = key < total ? key : 0;  // a dead key reads key 0 and is masked below
            const uint16_t *krow = P.k_pool + static_cast<int64_t>(s_pages[kc >> 4]) * kPageElems + tile_j + (kc & 15) * kD;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) kf[kk] = as_bf16x8(*reinterpret_cast<const u32x4 *>(krow + 16 * kk + 8 * half));
        }
        // -- S^T = K Q^T (32 keys x 32 queries)
        f32x16 st = {};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) st = mfma32(kf[kk], qf[kk], st);
        float x[16];
        const int kbase = kb * kKB + 4 * half;
        const bool diag = kb * kKB + kKB - 1 > prefix + i0;  // some key of this block may be > some query
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            x[v] = st[v] * P.scale_log2;
            if (diag) {
                const int key = kbase + 8 * (v >> 2) + (v & 3);
                if (key > pq || key >= total) x[v] = -INFINITY;
            }
        }
        // -- online softmax per query (lane-local + partner lane l^32)
        float mx = x[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, x[v]);
        mx = fmaxf(mx, partner32(mx));
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleLog2)) {
            const float mn = mx > m_run + kRescaleLog2 ? mx : m_run;
            const float f = fast_exp2(m_run - mn);
            m_run = mn;
            l_run *= f;
            o0 *= f;
            o1 *= f;
        }
        float pv[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            pv[v] = fast_exp2(x[v] - m_run);
            l_run += pv[v];
        }
        // -- P^T as bf16 hi + lo (B operand), registers 8sb .. 8sb+7 per key half sb
        bf16x8 phi[2], plo[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const __bf16 hi = static_cast<__bf16>(pv[8 * sb + e]);
                phi[sb][e] = hi;
                plo[sb][e] = static_cast<__bf16>(pv[8 * sb + e] - static_cast<float>(hi));
            }
        }
        __syncthreads();  // V^T staged
        // -- O^T += V^T P^T: A = V^T rows d, key slots (16sb + 4*half + 0..3, +8 + 0..3)
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const int d = 32 * db + qcol;
                const uint16_t *r = &s_vt[d * kVtStride + 16 * sb + 4 * half];
                const uint2 lo4 = *reinterpret_cast<const uint2 *>(r);
                const uint2 hi4 = *reinterpret_cast<const uint2 *>(r + 8);
                const bf16x8 va = as_bf16x8(u32x4{lo4.x, lo4.y, hi4.x, hi4.y});
                if (db == 0) {
                    o0 = mfma32(va, phi[sb], o0);
                    o0 = mfma32(va, plo[sb], o0);
                } else {
                    o1 = mfma32(va, phi[sb], o1);
                    o1 = mfma32(va, plo[sb], o1);
                }
            }
        }
        __syncthreads();  // V^T consumed before the next block overwrites it
    }

    // ---- out[s][iq][h][d] = O^T[d][query] / l, d = 32db + 8i + 4*half + r ------
    const float l_tot = l_run + partner32(l_run);
    if (!q_valid) return;
    const float inv = 1.0f / l_tot;
    const int64_t orow = ((static_cast<int64_t>(s) * C + iq) * kHQ + h) * kD;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int d = 32 * db + 8 * i + 4 * half;
            float r4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) r4[r] = (db == 0 ? o0[4 * i + r] : o1[4 * i + r]) * inv;
            if (P.out_fp32) {
                *reinterpret_cast<f32x4 *>(static_cast<float *>(P.out) + orow + d) = f32x4{r4[0], r4[1], r4[2], r4[3]};
            } else {
                const uint2 pk = {pack_bf16x2(r4[0], r4[1]), pack_bf16x2(r4[2], r4[3])};
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(P.out) + orow + d) = pk;
            }
        }
    }
}

hipError_t launch_prefill_attention(const PrefillLaunch &p, hipStream_t stream) {
    if (p.num_seqs == 0 || p.chunk_len == 0) return hipSuccess;
    if (p.max_blocks > kMaxBlocksPrefill) return hipErrorInvalidValue;
    PrefillParams P{};
    P.out = p.out;
    P.q = static_cast<const uint16_t *>(p.q);
    P.k_pool = static_cast<const uint16_t *>(p.k_pool);
    P.v_pool = static_cast<const uint16_t *>(p.v_pool);
    P.bt = p.block_tables;
    P.prefix_lens = p.prefix_lens;
    P.chunk_len = p.chunk_len;
    P.max_blocks = p.max_blocks;
    P.num_pages = p.num_pages;
    P.max_pos = p.max_pos;
    P.n_tiles = (p.chunk_len + kQT - 1) / kQT;
    P.scale_log2 = p.scale * 1.4426950408889634f;
    P.out_fp32 = p.out_fp32;
    P.flags = p.flags;
    const int64_t blocks = static_cast<int64_t>(p.num_seqs) * kHKV * P.n_tiles;
    hipLaunchKernelGGL(k_prefill_attn, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, P);
    return hipGetLastError();
}

}  // namespace pa
