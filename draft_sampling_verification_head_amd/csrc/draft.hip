// Markov-head sequential draft kernels (gfx950).
//
// [P3] "DSpark Speculative Decoding", section "Semi-Autoregressive Generation": position k
// samples x_k from softmax(U_k + B_k), B_k = W1[x_{k-1}] W2 with rank-r factors. [P1]
// section "DSpark 架构设计：半自回归生成与马尔可夫修正": only the previous token feeds the head.
// ([P1] = the Best Partners TV article "大模型推理加速的系统级工程：DeepSeek V4-Pro DSpark
// 推测解码方案深度解析与开源工具链 DeepSpec"; [P3] = the concept note "DSpark Speculative
// Decoding".)
//
// One draft step:
//   sweep  - grid (vocabulary tiles of 512 columns, request groups of up to 8). Gathers
//            W1[x_{k-1}] into LDS, streams the tile's W2 columns once for the whole group
//            (each lane 8 consecutive columns, waves split the rank), adds U_k, writes the
//            logits row segment and the tile's (max, sum exp(l - max)) partial.
//   select - one wave per request. Merges the partials in tile order into (m, Z),
//            lse = m + log Z, finds the tile holding the inverse-CDF point u * Z and rescans
//            that tile's stored logits for x_k = min { v : F(v) > u }.
// Up to 8 requests the select runs inside the sweep's last workgroup (one launch per step);
// larger batches launch it separately. Step k+1 reads x_k from device memory, so the gamma
// steps are enqueued back to back with no host round trip.
#include "common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kSweepThreads = 512;                 // 8 waves
constexpr int kSweepWaves = kSweepThreads / kWave;
constexpr int kColsPerLane = 8;
constexpr int kTileCols = kWave * kColsPerLane;    // 512 vocabulary columns per tile
static_assert(kTileCols == kSweepThreads, "one output column per thread in the epilogue");

constexpr int kSelThreads = 256;                 // 4 requests per workgroup, one per wave

// Eight consecutive factor elements as fp32. VEC: the eight are in bounds and 16-byte
// aligned (V % 8 == 0); otherwise each element is guarded by `avail` (elements left).
template <bool VEC>
__device__ __forceinline__ void load8(const float* p, long long avail, float (&o)[8]) {
    if (VEC) {
        float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = *reinterpret_cast<const float4*>(p + 4);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (e < avail) ? p[e] : 0.0f;
    }
}

template <bool VEC>
__device__ __forceinline__ void load8(const uint16_t* p, long long avail, float (&o)[8]) {
    if (VEC) {
        uint4 a = *reinterpret_cast<const uint4*>(p);
        o[0] = __uint_as_float(a.x << 16); o[1] = __uint_as_float(a.x & 0xffff0000u);
        o[2] = __uint_as_float(a.y << 16); o[3] = __uint_as_float(a.y & 0xffff0000u);
        o[4] = __uint_as_float(a.z << 16); o[5] = __uint_as_float(a.z & 0xffff0000u);
        o[6] = __uint_as_float(a.w << 16); o[7] = __uint_as_float(a.w & 0xffff0000u);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (e < avail) ? to_f32(p[e]) : 0.0f;
    }
}

__device__ __forceinline__ float tile_mass(float2 p, float m) {
    return (p.x == -INFINITY) ? 0.0f : p.y * __expf(p.x - m);
}

// ----------------------------------------------------------------------------- select
// One wave draws one request's token from its tile partials and stored logits row:
// (m, Z) merged in tile order, lse = m + log Z, the first tile whose running mass exceeds
// u * Z, then the first column of that tile whose running mass exceeds the remainder.
// Rounding that leaves the point past the end falls back to the last positive column.
__device__ void select_wave(int V, const float2* __restrict__ P, int nblk,
                            const float* __restrict__ row, float u, int32_t* x_o, float* q_o,
                            float* lse_o) {
    const int lane = threadIdx.x & (kWave - 1);
    float m = -INFINITY;
    for (int i = lane; i < nblk; i += kWave) m = fmaxf(m, P[i].x);
    m = wave_max(m);
    if (m == -INFINITY) {                 // invalid previous token or an all -inf row
        if (lane == 0) {
            *x_o = -1;
            if (q_o) *q_o = 0.0f;
            if (lse_o) *lse_o = -INFINITY;
        }
        return;
    }
    float z = 0.0f;
    for (int i = lane; i < nblk; i += kWave) z += tile_mass(P[i], m);
    const float Z = wave_sum(z);
    const float lse = m + __logf(Z);
    const float target = clamp_uniform(u) * Z;

    int found = -1;
    float tprime = INFINITY, run = 0.0f;
    for (int base = 0; base < nblk; base += kWave) {
        const int i = base + lane;
        const float v = (i < nblk) ? tile_mass(P[i], m) : 0.0f;
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
            if (tile_mass(P[i], m) > 0.0f) last = i;
        found = wave_max_int(last);
        tprime = INFINITY;
    }

    const long long c0 = static_cast<long long>(found) * kTileCols + lane * kColsPerLane;
    float e[kColsPerLane];
    float local = 0.0f;
#pragma unroll
    for (int j = 0; j < kColsPerLane; ++j) {
        const long long c = c0 + j;
        const float l = (c < V) ? row[c] : -INFINITY;
        e[j] = (l == -INFINITY) ? 0.0f : __expf(l - m);
        local += e[j];
    }
    const float incl = wave_incl_scan(local);
    float run2 = __shfl_up(incl, 1, kWave);
    if (lane == 0) run2 = 0.0f;
    int hitc = INT32_MAX, lastpos = -1;
#pragma unroll
    for (int j = 0; j < kColsPerLane; ++j) {
        run2 += e[j];
        if (e[j] > 0.0f) {
            lastpos = static_cast<int>(c0 + j);
            if (hitc == INT32_MAX && run2 > tprime) hitc = static_cast<int>(c0 + j);
        }
    }
    int tok = wave_min_int(hitc);
    if (tok == INT32_MAX) tok = wave_max_int(lastpos);
    if (lane == 0) {
        *x_o = tok;
        if (q_o) *q_o = (tok >= 0) ? __expf(row[tok] - lse) : 0.0f;
        if (lse_o) *lse_o = lse;
    }
}

// ----------------------------------------------------------------------------- sweep
// FUSED: the last workgroup of a request group to finish (counted with a device-scope
// atomic after a release fence) also runs the select, one wave per request, so a step is a
// single launch. Its counter is reset before it returns, so counters stay zero between
// launches.
template <typename WT, int BT, bool VEC, bool FUSED>
__global__ __launch_bounds__(kSweepThreads)
void draft_sweep_gemv(int B, int V, int r, int gamma, int k,
                      const float* __restrict__ U, const WT* __restrict__ W1,
                      const WT* __restrict__ W2, const int32_t* __restrict__ prev,
                      int prev_stride, float* __restrict__ L, long long L_bstride,
                      float2* __restrict__ part, int nblk, unsigned int* __restrict__ counters,
                      const float* __restrict__ u, int32_t* __restrict__ x_out,
                      float* __restrict__ q_out, float* __restrict__ lse_out) {
    extern __shared__ float smem[];
    float* h = smem;                       // [BT][r] gathered W1 rows
    float* red = smem + BT * r;            // [kSweepWaves][kTileCols] cross-wave partials
    __shared__ float scratch[kSweepWaves + 1];
    __shared__ int tok[BT];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int blk = static_cast<int>(blockIdx.x % static_cast<unsigned>(nblk));   // vocab tile
    const int grp = static_cast<int>(blockIdx.x / static_cast<unsigned>(nblk));   // request group
    const int b0 = grp * BT;

    if (tid < BT) {
        const int b = b0 + tid;
        int t = -1;
        if (b < B) {
            t = prev[static_cast<long long>(b) * prev_stride];
            if (t < 0 || t >= V) t = -1;   // out-of-range previous token: sentinel request
        }
        tok[tid] = t;
    }
    __syncthreads();
    for (int i = tid; i < BT * r; i += kSweepThreads) {
        const int bi = i / r, j = i - bi * r;
        const int t = tok[bi];
        h[i] = (t >= 0) ? to_f32(W1[static_cast<long long>(t) * r + j]) : 0.0f;
    }
    __syncthreads();

    // projection: lane owns 8 consecutive columns, waves split the rank dimension
    const long long col0 = static_cast<long long>(blk) * kTileCols + lane * kColsPerLane;
    const long long avail = static_cast<long long>(V) - col0;
    float acc[BT][kColsPerLane];
#pragma unroll
    for (int bi = 0; bi < BT; ++bi)
#pragma unroll
        for (int e = 0; e < kColsPerLane; ++e) acc[bi][e] = 0.0f;
    if (avail > 0) {
        const WT* wp = W2 + col0;
#pragma unroll 4
        for (int j = wave; j < r; j += kSweepWaves) {
            float w[kColsPerLane];
            load8<VEC>(wp + static_cast<long long>(j) * V, avail, w);
#pragma unroll
            for (int bi = 0; bi < BT; ++bi) {
                const float hv = h[bi * r + j];
#pragma unroll
                for (int e = 0; e < kColsPerLane; ++e) acc[bi][e] = fmaf(hv, w[e], acc[bi][e]);
            }
        }
    }

    // epilogue per request: fixed-order cross-wave sum, + U_k, logits store, tile partial
    const long long col = static_cast<long long>(blk) * kTileCols + tid;
#pragma unroll
    for (int bi = 0; bi < BT; ++bi) {
        const int b = b0 + bi;
#pragma unroll
        for (int e = 0; e < kColsPerLane; ++e)
            red[wave * kTileCols + lane * kColsPerLane + e] = acc[bi][e];
        __syncthreads();
        const bool live = (b < B) && (tok[bi] >= 0);
        float l = -INFINITY;
        if (live && col < V) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < kSweepWaves; ++w) s += red[w * kTileCols + tid];
            l = U[(static_cast<long long>(b) * gamma + k) * V + col] + s;
        }
        if (b < B && col < V) L[b * L_bstride + col] = l;
        const float m = block_max<kSweepThreads>(l, scratch);   // also fences `red` reuse
        const float ex = (l == -INFINITY) ? 0.0f : __expf(l - m);
        const float s = block_sum<kSweepThreads>(ex, scratch);
        if (tid == 0 && b < B) part[static_cast<long long>(b) * nblk + blk] = make_float2(m, s);
    }

    if (FUSED) {
        __threadfence();                   // release this workgroup's logits and partials
        __syncthreads();
        if (tid == 0) {
            const unsigned int done = atomicAdd(&counters[grp], 1u);
            s_last = (done == static_cast<unsigned int>(nblk) - 1u);
        }
        __syncthreads();
        if (!s_last) return;
        __threadfence();                   // acquire the other workgroups' results
        if (tid == 0) counters[grp] = 0u;
        if (wave < BT) {
            const int b = b0 + wave;
            if (b < B) {
                const long long o = static_cast<long long>(b) * gamma + k;
                select_wave(V, part + static_cast<long long>(b) * nblk, nblk, L + b * L_bstride,
                            u[o], x_out + o, q_out ? q_out + o : nullptr,
                            lse_out ? lse_out + o : nullptr);
            }
        }
    }
}

__global__ __launch_bounds__(kSelThreads)
void draft_select(int B, int V, int gamma, int k, const float2* __restrict__ part, int nblk,
                  const float* __restrict__ L, long long L_bstride, const float* __restrict__ u,
                  int32_t* __restrict__ x_out, float* __restrict__ q_out,
                  float* __restrict__ lse_out) {
    const int b = blockIdx.x * (kSelThreads / kWave) + threadIdx.x / kWave;
    if (b >= B) return;
    const long long o = static_cast<long long>(b) * gamma + k;
    select_wave(V, part + static_cast<long long>(b) * nblk, nblk, L + b * L_bstride, u[o],
                x_out + o, q_out ? q_out + o : nullptr, lse_out ? lse_out + o : nullptr);
}

template <typename WT, int BT, bool FUSED>
hipError_t launch_sweep_bt(const DraftStep& s, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(s.nblk) * ((s.B + BT - 1) / BT));   // 1-D: tile fastest
    const size_t smem = (static_cast<size_t>(BT) * s.r + kSweepWaves * kTileCols) * sizeof(float);
    const bool vec = (s.V % kColsPerLane) == 0 &&
                     (reinterpret_cast<uintptr_t>(s.W2) % 16) == 0;
#define DSPARK_SWEEP_ARGS                                                                     \
    s.B, s.V, s.r, s.gamma, s.k, s.U, static_cast<const WT*>(s.W1),                             \
        static_cast<const WT*>(s.W2), s.prev, s.prev_stride, s.L, s.L_bstride, s.part, s.nblk,  \
        s.counters, s.u, s.x_out, s.q_out, s.lse_out
    if (vec)
        hipLaunchKernelGGL((draft_sweep_gemv<WT, BT, true, FUSED>), grid, dim3(kSweepThreads),
                           smem, st, DSPARK_SWEEP_ARGS);
    else
        hipLaunchKernelGGL((draft_sweep_gemv<WT, BT, false, FUSED>), grid, dim3(kSweepThreads),
                           smem, st, DSPARK_SWEEP_ARGS);
#undef DSPARK_SWEEP_ARGS
    return hipGetLastError();
}

template <typename WT>
hipError_t launch_step_w(const DraftStep& s, hipStream_t st) {
    // small batches: one fused launch per step, all requests of the batch in one group
    if (s.B == 1) return launch_sweep_bt<WT, 1, true>(s, st);
    if (s.B == 2) return launch_sweep_bt<WT, 2, true>(s, st);
    if (s.B <= 4) return launch_sweep_bt<WT, 4, true>(s, st);
    if (s.B <= 8) return launch_sweep_bt<WT, 8, true>(s, st);
    hipError_t e = launch_sweep_bt<WT, 8, false>(s, st);
    if (e != hipSuccess) return e;
    const int waves = kSelThreads / kWave;
    hipLaunchKernelGGL(draft_select, dim3((s.B + waves - 1) / waves), dim3(kSelThreads), 0, st,
                       s.B, s.V, s.gamma, s.k, s.part, s.nblk, s.L, s.L_bstride, s.u, s.x_out,
                       s.q_out, s.lse_out);
    return hipGetLastError();
}

}  // namespace

int draft_tile_cols() { return kTileCols; }

int draft_counter_count(int B) { return (B + 7) / 8; }

hipError_t launch_draft_step(const DraftStep& s, hipStream_t st) {
    return (s.w_dtype == 1) ? launch_step_w<uint16_t>(s, st) : launch_step_w<float>(s, st);
}

}  // namespace dspark
