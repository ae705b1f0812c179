// Vocabulary-slab machinery shared by the slab draft step and the verify pass that rebuilds
// the draft logits from the Markov factors (gfx950).
//
// A slab workgroup (8 waves) owns 128 * NT vocabulary columns; wave w owns the 16 * NT
// columns of its "wave tile" and holds W2 for them, all ranks, in registers as A fragments
// of v_mfma_f32_16x16x32_bf16 (W2^T: 16 columns x 32 ranks per fragment). Rows of the batch
// stream through the slab; the logits of a row are the MFMA of these fragments with the W1
// row of its previous token (B operand), accumulated onto the row's base logits U (C
// operand). Column j of an MFMA result depends only on column j of the B and C operands, so
// recomputing one row's tile with the same fragments and U in the same rank order
// reproduces the step's logits bit for bit.
#pragma once

#include "common.h"

namespace dspark {
namespace slab {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSlabWaves = 8;
constexpr int kSlabThreads = kSlabWaves * kWave;
constexpr int kKS = 8;                   // rank chunks of 32 (r <= 256)
constexpr int kMaxRank = kKS * 32;
constexpr int kMaxNT = 5;                // 16-column MFMA tiles per wave
constexpr int kHRow = kMaxRank * 2;      // bytes of one gathered W1 row in LDS
constexpr int kLdsBytes = 160 * 1024;
constexpr int kSelRegs = 32;             // tile partials per lane a draw holds (2048 tiles)

template <int NT> struct Slab {
    static constexpr int WC = 16 * NT;                // columns of a wave tile
    static constexpr int SW = kSlabWaves * WC;        // columns of a slab
    static constexpr int Pitch = 32 * NT + 8;         // staged W2 rank row, bytes
    static constexpr int Stage = 32 * Pitch;          // one wave's staging area, bytes
};

// Global memory straight into LDS, 16 or 4 bytes per lane: lane l's bytes land at
// base + 16 l (base + 4 l); the LDS base must be wave-uniform. Every lane of the wave must
// be active, so that each call issues exactly one instruction (the vmcnt waits count them).
// The instruction is written as inline assembly on purpose: the compiler then does not
// treat it as an LDS write, and so does not put a wait for every outstanding direct load in
// front of each later LDS read (which would serialise the prefetch). The kernels order these
// loads themselves with explicit vmcnt waits and barriers. M0, which holds the LDS base, is
// used by nothing else in these kernels (no LDS-DMA builtins, no indexed register moves).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"     // m0 in the clobber lists below
__device__ __forceinline__ uint32_t lds_addr(const void* l) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) char*)(l)));
}
// The LDS address is a 32-bit byte offset (lds_addr of a __shared__ pointer plus an offset):
// computing it as an integer keeps the compiler from materialising 64-bit generic pointers
// into LDS, which it would otherwise hoist out of loops, one register pair per address.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t l) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(l)) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t l) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(l)) : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) lgkmcnt(0), expcnt not waited on (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without a memory fence: the direct-to-LDS loads are ordered by the
// explicit vmcnt waits, and the empty asm statements keep the compiler from moving memory
// accesses across the barrier.
// The lane index made opaque to the optimiser: per-lane addresses derived from it are then
// computed where they are used instead of being hoisted out of the loops around that use,
// where each would hold a register for the whole loop.
__device__ __forceinline__ int opaque_lane() {
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    return lane;
}

__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// W2 fragments of one wave tile (columns cw .. cw + 16 NT): fragment [t][s] holds, in lane
// l, ranks 32 s + 8 (l / 16) .. + 8 of column cw + 16 t + l % 16. Ranks >= r and columns
// >= V are zero, and so are the chunks s >= ks = ceil(r / 32), which are not loaded: every
// caller then runs all kKS rank chunks whatever r is (a zero fragment adds exact zeros), so
// the step kernels and the tile recomputations perform the same MFMA sequence. Rank rows are
// loaded as 16-byte pieces, PF chunks of 32 ranks in flight, and transposed through the
// wave-private LDS area `stg` (NSTG slots of Slab<NT>::Stage bytes; chunk s uses slot
// s % NSTG).
template <int NT, int PF, int NSTG>
__device__ __forceinline__ void load_w2_frags(bf16x8 (&w2f)[NT][kKS], const uint16_t* __restrict__ W2,
                                              int V, int r, long long cw, char* stg) {
    const int ks = (r + 31) / 32;
    constexpr int CH = 2 * NT;                      // 16-byte pieces per rank row
    constexpr int P = Slab<NT>::Pitch;
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t V32 = static_cast<uint32_t>(V);
    uint4 g[PF][NT];
    auto issue = [&](int s, uint4 (&dst)[NT]) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int q = j * kWave + lane, rho = q / CH, cc = q - rho * CH;
            const int rank = 32 * s + rho;
            const long long col = cw + 8 * cc;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (rank < r && col < V)
                v = *reinterpret_cast<const uint4*>(W2 + (static_cast<uint32_t>(rank) * V32 + static_cast<uint32_t>(col)));
            dst[j] = v;
        }
    };
#pragma unroll
    for (int d = 0; d < PF; ++d)
        if (d < ks) issue(d, g[d]);
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
        if (s >= ks) {
#pragma unroll
            for (int t = 0; t < NT; ++t) w2f[t][s] = __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
            continue;
        }
        char* slot = stg + (s % NSTG) * Slab<NT>::Stage;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int q = j * kWave + lane, rho = q / CH, cc = q - rho * CH;
            uint2* dst = reinterpret_cast<uint2*>(slot + rho * P + 16 * cc);
            dst[0] = make_uint2(g[s % PF][j].x, g[s % PF][j].y);
            dst[1] = make_uint2(g[s % PF][j].z, g[s % PF][j].w);
        }
        if (s + PF < ks) issue(s + PF, g[s % PF]);
        asm volatile("" ::: "memory");                // keeps later chunks' loads below
        const uint16_t* src = reinterpret_cast<const uint16_t*>(slot + (8 * (lane >> 4)) * P) + (lane & 15);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            uint32_t bv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bv[e] = static_cast<uint32_t>(src[(2 * e) * (P / 2) + 16 * t]) |
                        (static_cast<uint32_t>(src[(2 * e + 1) * (P / 2) + 16 * t]) << 16);
            w2f[t][s] = __builtin_bit_cast(bf16x8, make_uint4(bv[0], bv[1], bv[2], bv[3]));
        }
    }
}

__device__ __forceinline__ float swz_xor16(float v) {   // lane ^ 16 within each 32 lanes
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}

// Wave tiles per slab-tiled row: slabs of 128 NT columns, NT = ceil(V / 32768) clamped to
// [1, kMaxNT], so that V <= 163840 needs at most 256 slabs (one per compute unit).
__host__ __device__ inline int slab_nt(int V) {
    const int nt = (V + 32767) / 32768;
    return nt < 1 ? 1 : (nt > kMaxNT ? kMaxNT : nt);
}
__host__ __device__ inline int slab_count(int V) {
    const int sw = kSlabWaves * 16 * slab_nt(V);
    return (V + sw - 1) / sw;
}

}  // namespace slab
}  // namespace dspark
