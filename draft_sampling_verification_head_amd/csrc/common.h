// Device helpers shared by the DSpark kernels (gfx950, wave64).
//
// Every reduction and scan here has a fixed combination order, so results are bitwise
// reproducible run to run: butterfly reductions give the same value in every lane
// (fp add / max are commutative) and block-level steps combine wave results in wave order.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace dspark {

constexpr int kWave = 64;
constexpr float kUMax = 0.99999994039535522461f;   // 1 - 2^-24

__device__ __forceinline__ float clamp_uniform(float u) {
    // NaN compares false and is mapped to 0 by fmaxf
    return fminf(fmaxf(u, 0.0f), kUMax);
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t bits) {
    return __uint_as_float(static_cast<uint32_t>(bits) << 16);
}

// ---------------------------------------------------------------- wave level
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
    return v;
}

// Inclusive prefix sum across the wave (Hillis-Steele, fixed order).
__device__ __forceinline__ float wave_incl_scan(float v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        float t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

__device__ __forceinline__ double wave_incl_scan(double v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        double t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        int t = __shfl_up(v, o, kWave);
        if (lane >= o) v += t;
    }
    return v;
}

// ---------------------------------------------------------------- wave level, DPP forms
// For code in which all 64 lanes are active. Reductions run a butterfly inside each row of
// 16 lanes on DPP (quad xor 1, quad xor 2, half-row mirror, row mirror), which leaves the
// row result in every lane of the row, then read the four row results out with v_readlane
// and combine them in row order, so every lane returns the same value. The scan is the
// Hillis-Steele prefix inside each row (row_shr 1, 2, 4, 8) followed by the row_bcast 15 and
// 31 steps that carry row totals forward. All orders are fixed, so results are reproducible.
template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}

template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<CTRL, ROW_MASK, BOUND_ZERO>(__float_as_int(v)));
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

template <class Op>
__device__ __forceinline__ float wave_reduce_dpp(float v, Op op) {
    v = op(v, dpp_f<0xB1>(v));     // quad_perm [1,0,3,2]
    v = op(v, dpp_f<0x4E>(v));     // quad_perm [2,3,0,1]
    v = op(v, dpp_f<0x141>(v));    // row_half_mirror
    v = op(v, dpp_f<0x140>(v));    // row_mirror
    return op(op(readlane_f(v, 0), readlane_f(v, 16)), op(readlane_f(v, 32), readlane_f(v, 48)));
}

template <class Op>
__device__ __forceinline__ int wave_reduce_dpp(int v, Op op) {
    v = op(v, dpp_i<0xB1>(v));
    v = op(v, dpp_i<0x4E>(v));
    v = op(v, dpp_i<0x141>(v));
    v = op(v, dpp_i<0x140>(v));
    return op(op(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
              op(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

struct OpMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct OpSum { __device__ float operator()(float a, float b) const { return a + b; } };
struct OpMinI { __device__ int operator()(int a, int b) const { return min(a, b); } };
struct OpMaxI { __device__ int operator()(int a, int b) const { return max(a, b); } };

__device__ __forceinline__ float wave_max_dpp(float v) { return wave_reduce_dpp(v, OpMax{}); }
__device__ __forceinline__ float wave_sum_dpp(float v) { return wave_reduce_dpp(v, OpSum{}); }
__device__ __forceinline__ int wave_min_int_dpp(int v) { return wave_reduce_dpp(v, OpMinI{}); }
__device__ __forceinline__ int wave_max_int_dpp(int v) { return wave_reduce_dpp(v, OpMaxI{}); }

// Inclusive prefix sum across the wave.
__device__ __forceinline__ float wave_incl_scan_dpp(float v) {
    v += dpp_f<0x111, 0xF, true>(v);   // row_shr 1, zero at the row start
    v += dpp_f<0x112, 0xF, true>(v);   // row_shr 2
    v += dpp_f<0x114, 0xF, true>(v);   // row_shr 4
    v += dpp_f<0x118, 0xF, true>(v);   // row_shr 8
    v += dpp_f<0x142, 0xA>(v);         // row_bcast 15 into rows 1 and 3
    v += dpp_f<0x143, 0xC>(v);         // row_bcast 31 into rows 2 and 3
    return v;
}

// Value of the previous lane (0 in lane 0): turns an inclusive scan into an exclusive one.
__device__ __forceinline__ float wave_shr1_dpp(float v) { return dpp_f<0x138, 0xF, true>(v); }

// v from a lane index that is the same in every lane.
__device__ __forceinline__ float wave_bcast(float v, int lane) {
    return readlane_f(v, __builtin_amdgcn_readfirstlane(lane));
}

// ---------------------------------------------------------------- block level
// `scratch` must hold at least NT/64 + 1 elements; callers may reuse it right after.
template <int NT>
__device__ __forceinline__ float block_max(float v, float* scratch) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    v = wave_max(v);
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    if (wave == 0) {
        float t = lane < NW ? scratch[lane] : -INFINITY;
        t = wave_max(t);
        if (lane == 0) scratch[NW] = t;
    }
    __syncthreads();
    float r = scratch[NW];
    __syncthreads();
    return r;
}

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* scratch) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    v = wave_sum(v);
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    if (wave == 0) {
        float t = lane < NW ? scratch[lane] : 0.0f;
        t = wave_sum(t);
        if (lane == 0) scratch[NW] = t;
    }
    __syncthreads();
    float r = scratch[NW];
    __syncthreads();
    return r;
}

template <int NT>
__device__ __forceinline__ int block_min_int(int v, int* scratch) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    v = wave_min_int(v);
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int t = lane < NW ? scratch[lane] : INT32_MAX;
        t = wave_min_int(t);
        if (lane == 0) scratch[NW] = t;
    }
    __syncthreads();
    int r = scratch[NW];
    __syncthreads();
    return r;
}

template <int NT>
__device__ __forceinline__ int block_max_int(int v, int* scratch) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    v = wave_max_int(v);
    if (lane == 0) scratch[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int t = lane < NW ? scratch[lane] : INT32_MIN;
        t = wave_max_int(t);
        if (lane == 0) scratch[NW] = t;
    }
    __syncthreads();
    int r = scratch[NW];
    __syncthreads();
    return r;
}

// Block exclusive prefix sum. Returns this thread's exclusive prefix; *total receives the
// block total. Inside a wave the exclusive value of lane i is the inclusive value of lane
// i-1 taken from that lane (never formed by subtraction); waves add their offset in order.
template <int NT, typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* scratch, T* total) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    T incl = wave_incl_scan(v);
    T prev = __shfl_up(incl, 1, kWave);
    if (lane == 0) prev = T(0);
    if (lane == kWave - 1) scratch[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        T t = lane < NW ? scratch[lane] : T(0);
        T ti = wave_incl_scan(t);
        T te = __shfl_up(ti, 1, kWave);
        if (lane == 0) te = T(0);
        if (lane < NW) scratch[lane] = te;           // exclusive offset of wave `lane`
        if (lane == NW - 1) scratch[NW] = ti;        // block total
    }
    __syncthreads();
    T off = scratch[wave];
    *total = scratch[NW];
    __syncthreads();
    return off + prev;
}

}  // namespace dspark
