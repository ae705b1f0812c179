// Inverse-CDF draw from vocabulary-tile partials, shared by the draft kernels.
//
// [P3] "DSpark Speculative Decoding", section "Semi-Autoregressive Generation": x_k is a sample
// of softmax(U_k + B_k). With one host uniform u per draw the sample is the inverse CDF taken
// in token order, x = min { v : F(v) > u }. A step kernel leaves, per request and vocabulary
// tile of TC columns, the tile's (max, sum exp(l - max)) and the logits row itself; a draw
// merges the partials in tile order into (m, Z), lse = m + log Z, finds the first tile whose
// running mass exceeds u * Z and rescans that tile's logits in token order. Rounding that
// leaves the point past the end takes the last column with positive mass.
// ([P3] = the concept note "DSpark Speculative Decoding".)
#pragma once

#include "common.h"

namespace dspark {

constexpr int kSelThreads = 256;      // draw kernels: 4 requests per workgroup, one per wave

// Tile partials per lane a draw keeps in registers: enough for a 2^18-token vocabulary at
// either tile width (512 tiles of 512 columns, 1024 tiles of 256 columns).
template <int TC>
struct RegTiles {
    static constexpr int value = TC >= 512 ? 8 : 16;
};

// Loads of partials and logits. COHERENT = device-scope loads that bypass the per-XCD L2
// copies, for data another workgroup wrote earlier in the same launch.
template <bool COHERENT>
__device__ __forceinline__ float2 load_part(const float2* p) {
    if (!COHERENT) return *p;
    const unsigned long long v = __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p),
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return __builtin_bit_cast(float2, v);
}

template <bool COHERENT>
__device__ __forceinline__ float load_logit(const float* p) {
    if (!COHERENT) return *p;
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float tile_mass(float2 p, float m) {
    return (p.x == -INFINITY) ? 0.0f : p.y * __expf(p.x - m);
}

// Where a draw writes its results (nothing when `write` is false).
struct DrawOut {
    int32_t* x;
    float* q;
    float* lse;
    bool write;
};

__device__ __forceinline__ void put(const DrawOut& o, int tok, float q, float lse) {
    *o.x = tok;
    if (o.q) *o.q = q;
    if (o.lse) *o.lse = lse;
}

// In-tile search over weights already in registers: lane owns CPL consecutive columns
// starting at c0, in token order across lanes. Returns the first column whose running weight
// exceeds tprime, or (rounding left the point past the end; tprime = INFINITY asks for it)
// the last column with positive weight; -1 when no column has weight. Runs with all 64
// lanes of the wave active (the wave-level steps are DPP forms).
template <int CPL>
__device__ __forceinline__ int scan_pick(const float (&e)[CPL], long long c0, float tprime) {
    float local = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) local += e[j];
    const float incl = wave_incl_scan_dpp(local);
    float run = wave_shr1_dpp(incl);
    // bit j of pos: column c0 + j has weight; of past: it has weight and the running weight up
    // to it exceeds tprime (bit masks rather than branches)
    static_assert(CPL <= 32, "one bit per column of a lane");
    unsigned pos = 0u, past = 0u;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        run += e[j];
        pos |= (e[j] > 0.0f) ? (1u << j) : 0u;
        past |= (run > tprime) ? (1u << j) : 0u;
    }
    past &= pos;
    const int hit = past ? static_cast<int>(c0) + __builtin_ctz(past) : INT32_MAX;
    const int lastpos = pos ? static_cast<int>(c0) + 31 - __builtin_clz(pos) : -1;
    const int tok = wave_min_int_dpp(hit);
    return tok == INT32_MAX ? wave_max_int_dpp(lastpos) : tok;
}

// In-tile rescan over logits already in registers (same lane layout, absent columns as
// -inf): weights exp(l - m), then scan_pick; writes the token, p(token) and lse.
template <int CPL>
__device__ __forceinline__ int rescan_values(const float (&lv)[CPL], long long c0, int tile_c0,
                                             float m, float lse, float tprime,
                                             const DrawOut& o) {
    const int lane = threadIdx.x & (kWave - 1);
    float e[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) e[j] = (lv[j] == -INFINITY) ? 0.0f : __expf(lv[j] - m);
    const int tok = scan_pick<CPL>(e, c0, tprime);
    const int rel = tok - tile_c0;
    const int owner = rel / CPL, jj = rel - owner * CPL;
    float mine = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
        if (j == jj) mine = lv[j];
    const float lx = wave_bcast(mine, owner);
    if (o.write && lane == 0) put(o, tok, __expf(lx - lse), lse);
    return tok;
}

// In-tile rescan of logits in memory: lane owns TC/64 consecutive columns of `tile`.
template <int TC, bool COHERENT = false>
__device__ __forceinline__ int rescan_tile_wave(int V, const float* __restrict__ row, int tile,
                                                float m, float lse, float tprime,
                                                const DrawOut& o) {
    constexpr int CPL = TC / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const long long c0 = static_cast<long long>(tile) * TC + lane * CPL;
    float lv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) lv[j] = (c0 + j < V) ? load_logit<COHERENT>(row + c0 + j) : -INFINITY;
    return rescan_values<CPL>(lv, c0, tile * TC, m, lse, tprime, o);
}

// Result of merging one request's tile partials: the normaliser and the tile that holds
// the inverse-CDF point. tile < 0: the request has no mass.
struct TilePick {
    int tile;
    float m, lse, tprime;
};

// Search of NREG tile masses per lane (lane l holds tiles [l * NREG, (l + 1) * NREG)) in
// tile order for the first tile whose running mass exceeds `target`; `local` is the lane's
// own sum. tprime is the mass still to cover inside the found tile; INFINITY when rounding
// left the target past the end and the last tile with mass is taken. tile = -1: no mass.
struct MassPick {
    int tile;
    float tprime;
};

template <int NREG>
__device__ __forceinline__ MassPick search_mass(const float (&mass)[NREG], float local, float target) {
    const int lane = threadIdx.x & (kWave - 1);
    const float incl = wave_incl_scan_dpp(local);
    float run = wave_shr1_dpp(incl);
    int hit = INT32_MAX, last = -1;
    float before = 0.0f;
#pragma unroll
    for (int t = 0; t < NREG; ++t) {
        const float nr = run + mass[t];
        if (mass[t] > 0.0f) {
            last = lane * NREG + t;
            if (hit == INT32_MAX && nr > target) {
                hit = lane * NREG + t;
                before = run;
            }
        }
        run = nr;
    }
    MassPick r;
    const int found = wave_min_int_dpp(hit);
    if (found == INT32_MAX) {
        r.tile = wave_max_int_dpp(last);
        r.tprime = INFINITY;
    } else {
        r.tile = found;
        r.tprime = target - wave_bcast(before, found / NREG);
    }
    return r;
}

// Merge of NREG tile partials per lane (lane l holds tiles [l * NREG, (l + 1) * NREG),
// absent tiles as (-inf, 0)) in tile order, and the search for the first tile whose running
// mass exceeds u * Z.
template <int NREG>
__device__ __forceinline__ TilePick pick_tile(const float2 (&p)[NREG], float u) {
    TilePick r;
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < NREG; ++t) m = fmaxf(m, p[t].x);
    m = wave_max_dpp(m);
    r.m = m;
    if (m == -INFINITY) {
        r.tile = -1;
        r.lse = -INFINITY;
        r.tprime = INFINITY;
        return r;
    }
    float mass[NREG];
    float local = 0.0f;
#pragma unroll
    for (int t = 0; t < NREG; ++t) {
        mass[t] = tile_mass(p[t], m);
        local += mass[t];
    }
    const float Z = wave_sum_dpp(local);
    r.lse = m + __logf(Z);
    const MassPick mp = search_mass<NREG>(mass, local, clamp_uniform(u) * Z);
    r.tile = mp.tile;
    r.tprime = mp.tprime;
    return r;
}

// Two-level pick over vocabulary slabs of 8 consecutive tiles. merge_slab8 merges a slab's 8
// tile partials in tile order into the slab partial (max, sum exp(l - max)); walk_slab8
// searches the 8 tile masses (relative to the request's max m) for the first whose running
// mass exceeds `tprime`, the mass still to cover inside the slab. Without a hit (rounding, or
// tprime = INFINITY) the last tile with mass is taken and the in-tile search runs to its last
// column. Used identically by every form of the slab draw, so their picks agree bit for bit.
__device__ __forceinline__ float2 merge_slab8(const float2 (&p)[8]) {
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < 8; ++w) m = fmaxf(m, p[w].x);
    float z = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) z += tile_mass(p[w], m);
    return make_float2(m, z);
}

struct SlabWalk {
    int w;          // tile of the slab, -1 when no tile has mass
    float tprime;
};

__device__ __forceinline__ SlabWalk walk_slab8(const float2 (&p)[8], float m, float tprime) {
    SlabWalk r{-1, INFINITY};
    int last = -1;
    float run = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const float mt = tile_mass(p[w], m);
        const float nr = run + mt;
        if (mt > 0.0f) {
            last = w;
            if (r.w < 0 && nr > tprime) {
                r.w = w;
                r.tprime = tprime - run;
            }
        }
        run = nr;
    }
    if (r.w < 0) r.w = last;
    return r;
}

// The draw from tile partials already in registers: lane l holds tiles
// [l * RegTiles, (l + 1) * RegTiles), absent tiles as (-inf, 0). Returns the token (-1 for a
// request with no mass) in every lane; `row` is read only for the in-tile rescan.
template <int TC, bool COHERENT = false>
__device__ int draw_regs(int V, const float2 (&p)[RegTiles<TC>::value],
                         const float* __restrict__ row, float u, const DrawOut& o) {
    const int lane = threadIdx.x & (kWave - 1);
    const TilePick tp = pick_tile<RegTiles<TC>::value>(p, u);
    if (tp.tile < 0) {
        if (o.write && lane == 0) put(o, -1, 0.0f, -INFINITY);
        return -1;
    }
    return rescan_tile_wave<TC, COHERENT>(V, row, tp.tile, tp.m, tp.lse, tp.tprime, o);
}

// One wave draws one request's token; returns it (-1 for a dead request) in every lane.
template <int TC, bool COHERENT = false>
__device__ int draw_wave(int V, const float2* __restrict__ P, int nblk,
                         const float* __restrict__ row, float u, const DrawOut& o) {
    constexpr int kSelRegTiles = RegTiles<TC>::value;
    const int lane = threadIdx.x & (kWave - 1);
    if (nblk <= kWave * kSelRegTiles) {
        // register form: lane l holds tiles [l * kSelRegTiles, (l + 1) * kSelRegTiles)
        float2 p[kSelRegTiles];
#pragma unroll
        for (int t = 0; t < kSelRegTiles; ++t) {
            const int i = lane * kSelRegTiles + t;
            p[t] = (i < nblk) ? load_part<COHERENT>(P + i) : make_float2(-INFINITY, 0.0f);
        }
        return draw_regs<TC, COHERENT>(V, p, row, u, o);
    }
    // loop form for vocabularies with more tiles than the registers hold
    float m = -INFINITY;
    for (int i = lane; i < nblk; i += kWave) m = fmaxf(m, load_part<COHERENT>(P + i).x);
    m = wave_max(m);
    if (m == -INFINITY) {
        if (o.write && lane == 0) put(o, -1, 0.0f, -INFINITY);
        return -1;
    }
    float z = 0.0f;
    for (int i = lane; i < nblk; i += kWave) z += tile_mass(load_part<COHERENT>(P + i), m);
    const float Z = wave_sum(z);
    const float lse = m + __logf(Z);
    const float target = clamp_uniform(u) * Z;
    int found = -1;
    float tprime = INFINITY;
    float run = 0.0f;
    for (int base = 0; base < nblk; base += kWave) {
        const int i = base + lane;
        const float v = (i < nblk) ? tile_mass(load_part<COHERENT>(P + i), m) : 0.0f;
        const float incl = wave_incl_scan(v);
        float excl = __shfl_up(incl, 1, kWave);
        if (lane == 0) excl = 0.0f;
        const unsigned long long hit = __ballot((i < nblk) && (v > 0.0f) && (run + incl > target));
        if (hit) {
            const int f = __ffsll(static_cast<long long>(hit)) - 1;
            found = base + f;
            tprime = target - (run + __shfl(excl, f, kWave));
            break;
        }
        run += __shfl(incl, kWave - 1, kWave);
    }
    if (found < 0) {
        int last = -1;
        for (int i = lane; i < nblk; i += kWave)
            if (tile_mass(load_part<COHERENT>(P + i), m) > 0.0f) last = i;
        found = wave_max_int(last);
    }
    return rescan_tile_wave<TC, COHERENT>(V, row, found, m, lse, tprime, o);
}

// Draw of position k for every request, one wave per request; partials of TC-column tiles.
template <int TC>
__global__ __launch_bounds__(kSelThreads)
void draft_select(int B, int V, int gamma, int k, const float2* __restrict__ part, int nblk,
                  const float* __restrict__ L, long long L_bstride, const float* __restrict__ u,
                  int32_t* __restrict__ x_out, float* __restrict__ q_out,
                  float* __restrict__ lse_out) {
    const int b = blockIdx.x * (kSelThreads / kWave) + threadIdx.x / kWave;
    if (b >= B) return;
    const long long o = static_cast<long long>(b) * gamma + k;
    const DrawOut out{x_out + o, q_out ? q_out + o : nullptr, lse_out ? lse_out + o : nullptr,
                      true};
    draw_wave<TC>(V, part + static_cast<long long>(b) * nblk, nblk, L + b * L_bstride, u[o], out);
}

}  // namespace dspark
