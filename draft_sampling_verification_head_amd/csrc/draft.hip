// Markov-head sequential draft kernels (gfx950).
//
// [P3] "DSpark Speculative Decoding", section "Semi-Autoregressive Generation": position k
// samples x_k from softmax(U_k + B_k), B_k = W1[x_{k-1}] W2 with rank-r factors. [P1]
// section "DSpark 架构设计：半自回归生成与马尔可夫修正": only the previous token feeds the head.
// ([P1] = the Best Partners TV article "大模型推理加速的系统级工程：DeepSeek V4-Pro DSpark
// 推测解码方案深度解析与开源工具链 DeepSpec"; [P3] = the concept note "DSpark Speculative
// Decoding".)
//
// A draft of gamma positions is gamma + 1 launches, all on one stream:
//   step k  - 1-D grid over (request group of up to 8, vocabulary tile of 512 columns), tile
//             fastest. Each workgroup first draws x_{k-1} itself from step k-1's tile
//             partials and stored logits (every workgroup of the step computes the same
//             token; workgroup 0 also writes it out), gathers W1[x_{k-1}] into LDS, streams
//             the tile's W2 columns once for the whole group, adds U_k and writes the logits
//             row segment and the tile's (max, sum exp(l - max)) partial. Each lane owns 8
//             consecutive columns (one 16-byte bf16 load per W2 row); the 16 waves split the
//             rank with 4 rows of loads in flight each, and waves that do not draw start their
//             first rows before the draw. Step 0 takes x_0 from the caller.
//   select  - draws x_{gamma-1} from the last step's partials, one wave per request.
// The draw: (m, Z) merged from the partials in tile order, lse = m + log Z, the first tile
// whose running mass exceeds u * Z, then the first column of that tile whose running mass
// exceeds the remainder: x = min { v : F(v) > u } (inverse CDF in token order). Rounding
// that leaves the point past the end falls back to the last positive column. Results cross
// workgroups only at kernel boundaries, so no workgroup needs a device-scope fence.
#include "common.h"
#include "draw.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kSweepThreads = 1024;                // 16 waves
constexpr int kSweepWaves = kSweepThreads / kWave;
constexpr int kColsPerLane = 8;
constexpr int kTileCols = kWave * kColsPerLane;    // 512 vocabulary columns per tile
static_assert(kTileCols * 2 == kSweepThreads, "epilogue: one column per thread of the first half");


// Eight consecutive factor elements of one W2 row.
template <typename WT>
struct Seg;

template <>
struct Seg<uint16_t> {
    uint4 v;
    __device__ __forceinline__ void load(const uint16_t* p) {
        v = *reinterpret_cast<const uint4*>(p);
    }
    __device__ __forceinline__ void load_guarded(const uint16_t* p, long long avail) {
        uint32_t t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (e < avail) ? static_cast<uint32_t>(p[e]) : 0u;
        v = make_uint4(t[0] | (t[1] << 16), t[2] | (t[3] << 16), t[4] | (t[5] << 16),
                       t[6] | (t[7] << 16));
    }
    __device__ __forceinline__ void to_f32(float (&o)[8]) const {
        o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
        o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
        o[4] = __uint_as_float(v.z << 16); o[5] = __uint_as_float(v.z & 0xffff0000u);
        o[6] = __uint_as_float(v.w << 16); o[7] = __uint_as_float(v.w & 0xffff0000u);
    }
};

template <>
struct Seg<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ void load_guarded(const float* p, long long avail) {
        float t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (e < avail) ? p[e] : 0.0f;
        a = make_float4(t[0], t[1], t[2], t[3]);
        b = make_float4(t[4], t[5], t[6], t[7]);
    }
    __device__ __forceinline__ void to_f32(float (&o)[8]) const {
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
};

// ----------------------------------------------------------------------------- step kernel
struct StepArgs {
    int B, V, r, gamma, k, nblk;
    const float* U;
    const void* W1;
    const void* W2;
    const int32_t* x0;
    const float* u;
    int32_t* x_out;
    float* q_out;
    float* lse_out;
    float* L;                 // this step's logits: L + b * L_bstride
    const float* Lprev;       // the previous step's logits, same stride
    long long L_bstride;
    float2* part;             // this step's partials [B][nblk]
    const float2* part_prev;  // the previous step's partials
};

template <typename WT, int BT, bool VEC>
__global__ __launch_bounds__(kSweepThreads, (BT == 1 ? 8 : (BT == 2 ? 6 : 4)))
void draft_step_gemv(StepArgs a) {
    // 16 bytes per lane and 4 bf16 rows in flight per wave keep a single request's kernel at
    // 64 VGPRs, so two 16-wave workgroups fit per CU and every tile is resident at once.
    constexpr int RB = (!VEC || sizeof(WT) == 4) ? 2 : 4;
    extern __shared__ float smem[];
    float* h = smem;                       // [BT][r] gathered W1 rows
    float* red = smem + BT * a.r;          // [kSweepWaves][kTileCols] cross-wave partials
    __shared__ float scratch[kSweepWaves + 1];
    __shared__ int tok[BT];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int blk = static_cast<int>(blockIdx.x % static_cast<unsigned>(a.nblk));   // vocab tile
    const int grp = static_cast<int>(blockIdx.x / static_cast<unsigned>(a.nblk));   // req group
    const int b0 = grp * BT;
    const int V = a.V, r = a.r;
    const WT* W1 = static_cast<const WT*>(a.W1);
    const WT* W2 = static_cast<const WT*>(a.W2);

    // lane owns 8 consecutive columns; wave w owns rank rows [jb, je)
    const long long col0 = static_cast<long long>(blk) * kTileCols + lane * kColsPerLane;
    const long long avail = static_cast<long long>(V) - col0;
    const int rpw = (r + kSweepWaves - 1) / kSweepWaves;
    const int jb = wave * rpw, je = min(r, jb + rpw);
    const WT* wp = W2 + col0;
    Seg<WT> seg[RB];
    const bool streams = avail > 0 && jb < je;

    // 1. previous token of every request in the group. Waves that do not draw issue their
    //    first W2 rows meanwhile (W2 does not depend on the token).
    const bool drawing = a.k > 0 && wave < BT;
    const bool preloaded = !drawing && streams;
    if (preloaded) {
#pragma unroll
        for (int t = 0; t < RB; ++t) {
            const long long j = min(jb + t, je - 1);
            if (VEC) seg[t].load(wp + j * V); else seg[t].load_guarded(wp + j * V, avail);
        }
    }
    if (a.k == 0) {
        if (tid < BT) {
            const int b = b0 + tid;
            int t = -1;
            if (b < a.B) {
                t = a.x0[b];
                if (t < 0 || t >= V) t = -1;   // out-of-range context token: dead request
            }
            tok[tid] = t;
        }
    } else if (drawing) {
        const int b = b0 + wave;
        int t = -1;
        if (b < a.B) {
            const long long o = static_cast<long long>(b) * a.gamma + (a.k - 1);
            const DrawOut out{a.x_out + o, a.q_out ? a.q_out + o : nullptr,
                              a.lse_out ? a.lse_out + o : nullptr, blk == 0};
            t = draw_wave<kTileCols>(V, a.part_prev + static_cast<long long>(b) * a.nblk, a.nblk,
                          a.Lprev + b * a.L_bstride, a.u[o], out);
        }
        if (lane == 0) tok[wave] = t;
    }
    __syncthreads();
    for (int i = tid; i < BT * r; i += kSweepThreads) {
        const int bi = i / r, j = i - bi * r;
        const int t = tok[bi];
        h[i] = (t >= 0) ? to_f32(W1[static_cast<long long>(t) * r + j]) : 0.0f;
    }
    // U_k of this thread's epilogue column, fetched before the sweep
    const bool owner = tid < kTileCols;
    const long long col = static_cast<long long>(blk) * kTileCols + tid;
    float uk[BT];
#pragma unroll
    for (int bi = 0; bi < BT; ++bi) {
        const int b = b0 + bi;
        uk[bi] = (owner && b < a.B && col < V)
                     ? a.U[(static_cast<long long>(b) * a.gamma + a.k) * V + col] : 0.0f;
    }
    __syncthreads();

    // 2. projection, fp32 accumulation in row order
    float acc[BT][kColsPerLane];
#pragma unroll
    for (int bi = 0; bi < BT; ++bi)
#pragma unroll
        for (int e = 0; e < kColsPerLane; ++e) acc[bi][e] = 0.0f;
    if (streams) {
        for (int j0 = jb; j0 < je; j0 += RB) {
            if (!(preloaded && j0 == jb)) {
#pragma unroll
                for (int t = 0; t < RB; ++t) {
                    const long long j = min(j0 + t, je - 1);     // clamped: always a valid row
                    if (VEC) seg[t].load(wp + j * V); else seg[t].load_guarded(wp + j * V, avail);
                }
            }
#pragma unroll
            for (int t = 0; t < RB; ++t) {
                const int j = j0 + t;
                const float on = (j < je) ? 1.0f : 0.0f;     // rows past je add nothing
                float w[kColsPerLane];
                seg[t].to_f32(w);
#pragma unroll
                for (int bi = 0; bi < BT; ++bi) {
                    const float hv = on * h[bi * r + min(j, je - 1)];
#pragma unroll
                    for (int e = 0; e < kColsPerLane; ++e) acc[bi][e] = fmaf(hv, w[e], acc[bi][e]);
                }
            }
        }
    }

    // 3. epilogue per request: fixed-order cross-wave sum, + U_k, logits store, tile partial
#pragma unroll
    for (int bi = 0; bi < BT; ++bi) {
        const int b = b0 + bi;
        float4* dst = reinterpret_cast<float4*>(red + wave * kTileCols + lane * kColsPerLane);
        dst[0] = make_float4(acc[bi][0], acc[bi][1], acc[bi][2], acc[bi][3]);
        dst[1] = make_float4(acc[bi][4], acc[bi][5], acc[bi][6], acc[bi][7]);
        __syncthreads();
        const bool live = (b < a.B) && (tok[bi] >= 0);
        float l = -INFINITY;
        if (owner && live && col < V) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < kSweepWaves; ++w) s += red[w * kTileCols + tid];
            l = uk[bi] + s;
        }
        if (owner && b < a.B && col < V) a.L[b * a.L_bstride + col] = l;
        const float m = block_max<kSweepThreads>(l, scratch);   // also fences `red` reuse
        const float ex = (l == -INFINITY) ? 0.0f : __expf(l - m);
        const float s = block_sum<kSweepThreads>(ex, scratch);
        if (tid == 0 && b < a.B) a.part[static_cast<long long>(b) * a.nblk + blk] = make_float2(m, s);
    }
}

template <typename WT, int BT>
hipError_t launch_step_bt(const StepArgs& a, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(a.nblk) * ((a.B + BT - 1) / BT));   // 1-D: tile fastest
    const size_t smem = (static_cast<size_t>(BT) * a.r + kSweepWaves * kTileCols) * sizeof(float);
    const bool vec = (a.V % kColsPerLane) == 0 && (reinterpret_cast<uintptr_t>(a.W2) % 16) == 0;
    if (vec)
        hipLaunchKernelGGL((draft_step_gemv<WT, BT, true>), grid, dim3(kSweepThreads), smem, st, a);
    else
        hipLaunchKernelGGL((draft_step_gemv<WT, BT, false>), grid, dim3(kSweepThreads), smem, st, a);
    return hipGetLastError();
}

template <typename WT>
hipError_t launch_step_w(const StepArgs& a, hipStream_t st) {
    if (a.B == 1) return launch_step_bt<WT, 1>(a, st);
    if (a.B == 2) return launch_step_bt<WT, 2>(a, st);
    if (a.B <= 4) return launch_step_bt<WT, 4>(a, st);
    return launch_step_bt<WT, 8>(a, st);
}

}  // namespace

int draft_part_tiles(int V) {
    const int t = kTileCols < draft_mfma_tile_cols() ? kTileCols : draft_mfma_tile_cols();
    const int n = (V + t - 1) / t;
    const int ns = draft_slab_tiles(V);
    return n > ns ? n : ns;
}

int draft_path_of(const DraftCall& c, bool* one_launch) {
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) % 16) == 0; };
    bool one = false;
    int path = 0;                                       // DSPARK_PATH_SWEEP
    if (!c.per_position && draft_resident_ok(c.B, c.V, c.r, c.w_dtype, c.W1, c.W2)) {
        path = 2;                                       // DSPARK_PATH_RESIDENT
        one = true;
    } else if (draft_slab_ok(c.B, c.V, c.r, c.w_dtype, c.W1, c.W2) && al16(c.U) &&
               (!c.L_out || al16(c.L[0]))) {
        path = 3;                                       // DSPARK_PATH_SLAB
        one = !c.per_position && draft_slab_one_launch(c.B, c.V, c.L_out);
    } else if (draft_mfma_ok(c.B, c.V, c.r, c.w_dtype, c.W1, c.W2)) {
        path = 1;                                       // DSPARK_PATH_MFMA
    }
    if (one_launch) *one_launch = one;
    return path;
}

hipError_t launch_draft(const DraftCall& c, hipStream_t st) {
    const int path = draft_path_of(c, nullptr);
    if (path == 2) return launch_draft_resident(c, st);
    if (path == 3) return launch_draft_slab(c, st);
    if (path == 1) return launch_draft_mfma(c, st);
    StepArgs a;
    a.B = c.B; a.V = c.V; a.r = c.r; a.gamma = c.gamma; a.nblk = (c.V + kTileCols - 1) / kTileCols;
    a.U = c.U; a.W1 = c.W1; a.W2 = c.W2; a.x0 = c.x0; a.u = c.u;
    a.x_out = c.x_out; a.q_out = c.q_out; a.lse_out = c.lse_out;
    a.L_bstride = c.L_bstride;
    for (int k = 0; k < c.gamma; ++k) {
        a.k = k;
        a.L = c.L[k];
        a.Lprev = k ? c.L[k - 1] : nullptr;
        a.part = c.part[k & 1];
        a.part_prev = c.part[(k + 1) & 1];
        const hipError_t e = (c.w_dtype == 1) ? launch_step_w<uint16_t>(a, st)
                                              : launch_step_w<float>(a, st);
        if (e != hipSuccess) return e;
    }
    const int k = c.gamma - 1;
    const int waves = kSelThreads / kWave;
    hipLaunchKernelGGL(draft_select<kTileCols>, dim3((c.B + waves - 1) / waves), dim3(kSelThreads), 0, st,
                       c.B, c.V, c.gamma, k, static_cast<const float2*>(c.part[k & 1]), a.nblk,
                       c.L[k], c.L_bstride, c.u, c.x_out, c.q_out, c.lse_out);
    return hipGetLastError();
}

}  // namespace dspark
