// Row helpers shared by the verify kernels (materialised draft logits) and the verify pass
// that rebuilds the draft logits from the Markov factors (gfx950): the per-request row
// layout, the chunk tiling of a vocabulary row, and the merge of chunk partials into lse.
#pragma once

#include "common.h"
#include "kernels.h"

namespace dspark {
namespace rows {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kPer = 32;                      // logits per thread per chunk
constexpr int kChunk = kThreads * kPer;       // 8192 logits (32 KB) per workgroup

struct ReqRows {
    int ell;
    long long off;
    bool ok;
};

__device__ __forceinline__ ReqRows request_rows(const RowSet& rs, int b) {
    ReqRows q;
    q.ell = rs.len ? rs.len[b] : rs.gamma;
    q.off = rs.t_off ? static_cast<long long>(rs.t_off[b])
                     : static_cast<long long>(b) * (rs.gamma + 1);
    q.ok = q.ell >= 0 && q.ell <= rs.gamma && q.off >= 0 && q.off + q.ell < rs.Lt_rows;
    return q;
}

__device__ __forceinline__ float qnan() { return __int_as_float(0x7fc00000); }

// Chunk c in the rescan layout: thread t owns the kPer consecutive logits starting at
// c*kChunk + kPer*t, so a block scan runs in token-id order.
template <bool VEC4>
__device__ __forceinline__ void load_chunk_contig(const float* __restrict__ row, int c, int V,
                                                  float (&x)[kPer]) {
    const long long base =
        static_cast<long long>(c) * kChunk + static_cast<long long>(kPer) * threadIdx.x;
    if (VEC4) {
        const float4* r4 = reinterpret_cast<const float4*>(row + base);
#pragma unroll
        for (int g = 0; g < kPer / 4; ++g) {
            float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            if (base + 4 * g < V) v = r4[g];
            x[4 * g] = v.x; x[4 * g + 1] = v.y; x[4 * g + 2] = v.z; x[4 * g + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kPer; ++e) x[e] = (base + e < V) ? row[base + e] : -INFINITY;
    }
}

// lse of one row from its chunk partials, merged by one wave with all lanes active (max
// first, then the scaled sums in lane-strided order and a fixed-order wave sum); the same
// value in every lane.
__device__ __forceinline__ float merge_lse_wave(const float2* __restrict__ P, int nch) {
#pragma clang fp contract(off)          // each product and sum rounds on its own at every call site
    const int lane = threadIdx.x & (kWave - 1);
    float mm = -INFINITY;
    float2 p0 = make_float2(-INFINITY, 0.0f);
    if (lane < nch) p0 = P[lane];
    for (int i = lane + kWave; i < nch; i += kWave) mm = fmaxf(mm, P[i].x);
    mm = wave_max_dpp(fmaxf(mm, p0.x));
    if (mm == -INFINITY) return -INFINITY;
    float ss = (p0.x == -INFINITY) ? 0.0f : p0.y * __expf(p0.x - mm);
    for (int i = lane + kWave; i < nch; i += kWave)
        ss += (P[i].x == -INFINITY) ? 0.0f : P[i].y * __expf(P[i].x - mm);
    ss = wave_sum_dpp(ss);
    return mm + __logf(ss);
}

// Row slots of a request: slot s <= gamma is target row s, slot gamma+1+k is draft row k.
__device__ __forceinline__ const float2* slot_part(const float2* part, int b, int slot, int G,
                                                   int nch) {
    return part + (static_cast<long long>(b) * (2 * G + 1) + slot) * nch;
}

}  // namespace rows
}  // namespace dspark
