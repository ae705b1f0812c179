// Batched Markov-head draft step on bf16 MFMA (gfx950).
//
// [P3] "DSpark Speculative Decoding", section "Semi-Autoregressive Generation": the bias of
// position k is B_k = W1[x_{k-1}] W2 for every request, i.e. one [B x r] * [r x V] product
// per step (rank r = 256) added to the backbone logits U_k. ([P3] = the concept note
// "DSpark Speculative Decoding".)
//
// Used when a batch is large enough for the product to be a dense GEMM (B > 8 requests,
// bf16 factors). Workgroup = 64 requests x 256 vocabulary columns, 8 waves that run
// independently after the W1 rows of the 64 requests (the A operand, rank-contiguous) are
// gathered into LDS:
//   - Wave w owns columns [32w, 32w + 32) and both 32-request halves, accumulating
//     v_mfma_f32_32x32x16_bf16 in fp32.
//   - Its B operand streams from HBM as one 16-byte load per lane per 16-rank chunk (W2's
//     natural [r][V] layout). Each chunk passes through a wave-private LDS area that turns
//     it into the fragment layout, so no workgroup barrier is needed. Two chunks stay in
//     flight per wave.
//   - U_k for the wave's 64 x 32 tile is loaded first, together with the first chunks.
// The epilogue adds U_k, stores the logits, and reduces each request row to (max, sum exp):
//   - a 31-step reduce-scatter butterfly across the 32 lanes of a half-wave (ds_swizzle for
//     lane distance 16, then DPP row rotate, half-row mirror and quad swaps), after which
//     lane l32 holds one row;
//   - the 8 waves' row results are then merged in wave order through LDS.
// Workgroups are mapped so that the request groups of one vocabulary tile run on the same
// XCD (shared L2).
#include "common.h"
#include "draw.h"
#include "kernels.h"

namespace dspark {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMT = 64;                 // requests per workgroup
constexpr int kNT = 256;                // vocabulary columns per workgroup
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kKC = 16;                 // rank rows per W2 chunk (one MFMA k-step)
constexpr int kHPad = 8;                // H row padding (bf16)
constexpr int kWS = 40;                 // row stride (bf16) of a wave's W2 chunk in LDS
constexpr int kXcds = 8;
constexpr int kPF = 2;                  // W2 chunks in flight per wave
constexpr int kMaxRank = 256;           // rank the A operand staging covers
constexpr int kHSeg = kMT * kMaxRank / 8 / kThreads;   // 16-byte W1 segments per thread
static_assert(kHSeg * kThreads * 8 == kMT * kMaxRank, "W1 gather covers 64 rows of rank kMaxRank");
static_assert(kWaves * 32 == kNT, "one 32-column MFMA tile per wave");

struct MfmaArgs {
    int B, V, r, rp, gamma, k, ntiles, mgroups;
    const float* U;
    const uint16_t* W1;
    const uint16_t* W2;
    const uint16_t* Hrows;    // RNN head: the state of request b as bf16 rows hi, lo at
                              // Hrows + 2 b rp (zero beyond r); the A operand instead of W1[x]
    const int32_t* tok;       // x_{k-1}: tok[b * tok_stride]
    int tok_stride;
    float* L;                 // logits rows L + b * L_bstride
    long long L_bstride;
    float2* part;             // [B][ntiles] (max, sum exp) per request and tile
    // RNN head: workgroups from mv0 on (one per request) form A h_k while the tiles run
    const uint16_t* A;        // [r][r] bf16
    const float* hcur;        // [B][r] fp32 state h_k
    float* Ah;                // [B][r] fp32 A h_k, for the draw launch to finish h_{k+1}
    unsigned mv0;             // first matvec workgroup (the grid's end when there is none)
};

// Row of accumulator element v of half-tile h, for the lane half hf = lane / 32.
__device__ __forceinline__ int acc_row(int h, int v, int hf) {
    return 32 * h + 8 * (v / 4) + 4 * hf + (v % 4);
}

__device__ __forceinline__ float swz_xor16(float v) {   // lane ^ 16 within each 32 lanes
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}

// Reduce-scatter across the 32 lanes of a half-wave: x[rho] is this lane's value of row
// index rho; the result is row index (lane & 31) reduced over the 32 lanes. Each step keeps
// the upper half of the values when the lane's bit is set and receives the partner's copy
// of the kept half; the partner of every step agrees with the lane on all bits handled
// before and differs on the current one.
template <class Op>
__device__ __forceinline__ float reduce_scatter32(const float (&x)[32], Op op) {
    const int l = threadIdx.x & 31;
    float a16[16], a8[8], a4[4], a2[2];
    const bool b4 = l & 16, b3 = l & 8, b2 = l & 4, b1 = l & 2, b0 = l & 1;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        a16[i] = op(b4 ? x[i + 16] : x[i], swz_xor16(b4 ? x[i] : x[i + 16]));
#pragma unroll
    for (int i = 0; i < 8; ++i)                                     // row_ror 8: lane ^ 8
        a8[i] = op(b3 ? a16[i + 8] : a16[i], dpp_f<0x128>(b3 ? a16[i] : a16[i + 8]));
#pragma unroll
    for (int i = 0; i < 4; ++i)                                     // half-row mirror
        a4[i] = op(b2 ? a8[i + 4] : a8[i], dpp_f<0x141>(b2 ? a8[i] : a8[i + 4]));
#pragma unroll
    for (int i = 0; i < 2; ++i)                                     // quad lane ^ 2
        a2[i] = op(b1 ? a4[i + 2] : a4[i], dpp_f<0x4E>(b1 ? a4[i] : a4[i + 2]));
    return op(b0 ? a2[1] : a2[0], dpp_f<0xB1>(b0 ? a2[0] : a2[1]));  // quad lane ^ 1
}

// RNN = false: the Markov head (A operand = the gathered W1 rows of the previous tokens).
// RNN = true: the RNN head's state rows, split into bf16 hi + lo parts (h = hi + lo to about
// 2^-17 relative), each multiplied with the same W2 fragment into the same accumulators.
// A h_k of request b in fp32, row i summed over j in ascending order from 0 (the sum
// rnn_state_kernel forms before adding the W1 row). hp: r floats of LDS.
__device__ void rnn_matvec(const MfmaArgs& a, int b, float* hp) {
    const int i = threadIdx.x, r = a.r;
    if (i < r) hp[i] = a.hcur[static_cast<long long>(b) * r + i];
    __syncthreads();
    if (i >= r) return;
    const uint16_t* Ar = a.A + static_cast<long long>(i) * r;
    float h = 0.0f;
    for (int j = 0; j < r; j += 8) {
        const uint4 w = *reinterpret_cast<const uint4*>(Ar + j);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            h = fmaf(__uint_as_float(ww[e] << 16), hp[j + 2 * e], h);
            h = fmaf(__uint_as_float(ww[e] & 0xffff0000u), hp[j + 2 * e + 1], h);
        }
    }
    a.Ah[static_cast<long long>(b) * r + i] = h;
}

template <bool RNN>
__global__ __launch_bounds__(kThreads, 4)      // 4 waves per SIMD: two workgroups per CU
void draft_step_mfma(MfmaArgs a) {
    extern __shared__ uint16_t sm16[];
    if constexpr (RNN) {
        if (blockIdx.x >= a.mv0) {
            rnn_matvec(a, static_cast<int>(blockIdx.x - a.mv0), reinterpret_cast<float*>(sm16));
            return;
        }
    }
    const int HS = a.rp + kHPad;
    uint16_t* Hs = sm16;                              // [kMT][HS] gathered W1 rows (RNN: hi)
    uint16_t* Hl = sm16 + kMT * HS;                   // RNN: [kMT][HS] lo parts
    uint16_t* Ws = sm16 + (RNN ? 2 : 1) * kMT * HS;   // [kWaves][kKC][kWS] W2 chunk per wave
    __shared__ float red[kWaves][kMT];
    __shared__ float rowmax[kMT];
    __shared__ int stok[kMT];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const unsigned xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int mg = static_cast<int>(slot % static_cast<unsigned>(a.mgroups));
    const int tile = static_cast<int>(slot / static_cast<unsigned>(a.mgroups)) * kXcds + static_cast<int>(xcd);
    if (tile >= a.ntiles) return;
    const int m0 = mg * kMT;
    const long long n0 = static_cast<long long>(tile) * kNT;
    const int hf = lane >> 5, l32 = lane & 31;
    const long long col = n0 + wave * 32 + l32;
    const bool colok = col < a.V;

    // 1. loads that do not depend on the tokens: U_k of the wave's tile, first W2 chunks.
    //    B fragment of chunk c: ranks 16c + 8hf .. +8 of column `col`, two per register.
    // 32-bit element offsets from workgroup-uniform bases (the host checks they fit)
    const float* Ub = a.U + (static_cast<long long>(m0) * a.gamma + a.k) * a.V;
    const uint32_t urow = static_cast<uint32_t>(a.gamma) * static_cast<uint32_t>(a.V);
    const uint32_t c32 = static_cast<uint32_t>(col);
    float lv[32];                                      // U_k, then the logits
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = acc_row(h, v, hf);
            lv[16 * h + v] = (colok && m0 + i < a.B) ? Ub[static_cast<uint32_t>(i) * urow + c32] : 0.0f;
        }
    // W2 chunk c as one 16-byte load per lane: rank 16c + lane / 4, 8 columns starting at
    // 32w + 8 (lane % 4)
    const uint32_t V32 = static_cast<uint32_t>(a.V);
    const int wq = lane >> 2, wcol = (lane & 3) * 8;
    const long long gcol = n0 + wave * 32 + wcol;
    auto load_w = [&](int c) {
        const int kk = kKC * c + wq;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (kk < a.r && gcol < a.V)
            v = *reinterpret_cast<const uint4*>(a.W2 + (static_cast<uint32_t>(kk) * V32 + static_cast<uint32_t>(gcol)));
        return v;
    };
    const int nkc = a.rp / kKC;
    uint4 gq[kPF];
#pragma unroll
    for (int d = 0; d < kPF; ++d) gq[d] = (d < nkc) ? load_w(d) : make_uint4(0u, 0u, 0u, 0u);

    // 2. tokens and the gathered W1 rows (A operand: zero beyond r and for dead / absent requests)
    if (tid < kMT) {
        const int b = m0 + tid;
        int t = -1;
        if (b < a.B) {
            t = a.tok[static_cast<long long>(b) * a.tok_stride];
            if (t < 0 || t >= a.V) t = -1;             // dead request: no bias, -inf logits
        }
        stok[tid] = t;
    }
    __syncthreads();
    const int segs = a.rp / 8;                         // rp <= 256: at most kHSeg per thread
#pragma unroll
    for (int q = 0; q < kHSeg; ++q) {
        const int s = tid + q * kThreads;
        if (s < kMT * segs) {
            const int i = s / segs, c = (s % segs) * 8;
            const int t = stok[i];
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (RNN) {
                uint4 vl = make_uint4(0u, 0u, 0u, 0u);
                if (t >= 0) {
                    const uint16_t* hr = a.Hrows + static_cast<long long>(m0 + i) * 2 * a.rp + c;
                    v = *reinterpret_cast<const uint4*>(hr);
                    vl = *reinterpret_cast<const uint4*>(hr + a.rp);
                }
                *reinterpret_cast<uint4*>(Hl + i * HS + c) = vl;
            } else if (t >= 0 && c < a.r) {
                v = *reinterpret_cast<const uint4*>(a.W1 + static_cast<long long>(t) * a.r + c);
            }
            *reinterpret_cast<uint4*>(Hs + i * HS + c) = v;
        }
    }
    __syncthreads();

    // 3. K loop, wave-local: kPF chunks in flight in a statically indexed register ring; each
    //    chunk passes through the wave's own LDS area (row-major, 16 ranks x 32 columns) to
    //    become the B fragment (ranks 8hf .. 8hf+7 of column l32). LDS accesses of one wave
    //    execute in order, so no barrier is needed.
    uint16_t* ws = Ws + wave * (kKC * kWS);
    f32x16 acc0 = {}, acc1 = {};
    for (int kc0 = 0; kc0 < nkc; kc0 += kPF) {
#pragma unroll
        for (int d = 0; d < kPF; ++d) {
            const int kc = kc0 + d;
            if (kc < nkc) {
                const uint4 g = gq[d];
                if (kc + kPF < nkc) gq[d] = load_w(kc + kPF);
                uint2* dst = reinterpret_cast<uint2*>(ws + wq * kWS + wcol);
                dst[0] = make_uint2(g.x, g.y);
                dst[1] = make_uint2(g.z, g.w);
                const uint16_t* src = ws + (8 * hf) * kWS + l32;
                uint32_t bv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    bv[e] = static_cast<uint32_t>(src[(2 * e) * kWS]) |
                            (static_cast<uint32_t>(src[(2 * e + 1) * kWS]) << 16);
                const bf16x8 bfrag = __builtin_bit_cast(bf16x8, make_uint4(bv[0], bv[1], bv[2], bv[3]));
                const int kofs = kc * kKC + 8 * hf;
                const bf16x8 a0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Hs + l32 * HS + kofs));
                const bf16x8 a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Hs + (32 + l32) * HS + kofs));
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bfrag, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bfrag, acc1, 0, 0, 0);
                if (RNN) {
                    const bf16x8 l0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Hl + l32 * HS + kofs));
                    const bf16x8 l1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Hl + (32 + l32) * HS + kofs));
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l0, bfrag, acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(l1, bfrag, acc1, 0, 0, 0);
                }
            }
        }
    }

    // 4. epilogue: logits, stores, per-row (max, sum exp) over the workgroup's 256 columns
    float* Lb = a.L + static_cast<long long>(m0) * a.L_bstride;
    const uint32_t lrow = static_cast<uint32_t>(a.L_bstride);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = acc_row(h, v, hf);
            const int b = m0 + i;
            const bool live = colok && b < a.B && stok[i] >= 0;
            const float accv = h ? acc1[v] : acc0[v];
            lv[16 * h + v] = live ? lv[16 * h + v] + accv : -INFINITY;
            if (colok && b < a.B) Lb[static_cast<uint32_t>(i) * lrow + c32] = lv[16 * h + v];
        }
    const int myrow = acc_row(l32 >> 4, l32 & 15, hf);  // row index l32 of this lane's half
    float m = reduce_scatter32(lv, OpMax{});
    red[wave][myrow] = m;
    __syncthreads();
    if (tid < kMT) {
        float mm = red[0][tid];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, red[w][tid]);
        rowmax[tid] = mm;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float x = lv[16 * h + v];
            lv[16 * h + v] = (x == -INFINITY) ? 0.0f : __expf(x - rowmax[acc_row(h, v, hf)]);
        }
    const float s = reduce_scatter32(lv, OpSum{});
    red[wave][myrow] = s;
    __syncthreads();
    if (tid < kMT) {
        const int b = m0 + tid;
        if (b < a.B) {
            float ss = red[0][tid];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) ss += red[w][tid];
            a.part[static_cast<long long>(b) * a.ntiles + tile] = make_float2(rowmax[tid], ss);
        }
    }
}

}  // namespace

int draft_mfma_tile_cols() { return kNT; }

bool draft_mfma_ok(int B, int V, int r, int w_dtype, const void* W1, const void* W2) {
    // element offsets inside W2 and inside 64 requests' rows of U / L_d stay below 2^32
    const long long span = static_cast<long long>(kMT) * 64 * V;   // gamma <= 64
    return w_dtype == 1 && B > 8 && r <= kMaxRank && (r % 8) == 0 && (V % 8) == 0 &&
           static_cast<long long>(kMaxRank) * V < (1LL << 32) && span < (1LL << 32) &&
           (reinterpret_cast<uintptr_t>(W1) % 16) == 0 && (reinterpret_cast<uintptr_t>(W2) % 16) == 0;
}

hipError_t launch_draft_mfma(const DraftCall& c, hipStream_t st) {
    MfmaArgs a;
    a.B = c.B; a.V = c.V; a.r = c.r; a.rp = (c.r + kKC - 1) / kKC * kKC;
    if (a.rp % 8) a.rp += 8 - a.rp % 8;
    a.gamma = c.gamma;
    a.ntiles = (c.V + kNT - 1) / kNT;
    a.mgroups = (c.B + kMT - 1) / kMT;
    a.U = c.U;
    a.W1 = static_cast<const uint16_t*>(c.W1);
    a.W2 = static_cast<const uint16_t*>(c.W2);
    a.L_bstride = c.L_bstride;
    const unsigned grid_tiles = static_cast<unsigned>((a.ntiles + kXcds - 1) / kXcds * kXcds);
    const dim3 grid(grid_tiles * a.mgroups);
    const size_t smem = (static_cast<size_t>(kMT) * (a.rp + kHPad) + kWaves * kKC * kWS) * sizeof(uint16_t);
    const int waves = kSelThreads / kWave;
    for (int k = 0; k < c.gamma; ++k) {
        if (k > 0) {
            hipLaunchKernelGGL(draft_select<kNT>, dim3((c.B + waves - 1) / waves), dim3(kSelThreads),
                               0, st, c.B, c.V, c.gamma, k - 1,
                               static_cast<const float2*>(c.part[(k - 1) & 1]), a.ntiles, c.L[k - 1],
                               c.L_bstride, c.u, c.x_out, c.q_out, c.lse_out);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        a.k = k;
        a.tok = k ? c.x_out + (k - 1) : c.x0;
        a.tok_stride = k ? c.gamma : 1;
        a.L = c.L[k];
        a.part = c.part[k & 1];
        a.Hrows = nullptr;
        a.A = nullptr;
        a.hcur = nullptr;
        a.Ah = nullptr;
        a.mv0 = grid.x;
        hipLaunchKernelGGL(draft_step_mfma<false>, grid, dim3(kThreads), smem, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int k = c.gamma - 1;
    hipLaunchKernelGGL(draft_select<kNT>, dim3((c.B + waves - 1) / waves), dim3(kSelThreads), 0, st,
                       c.B, c.V, c.gamma, k, static_cast<const float2*>(c.part[k & 1]), a.ntiles,
                       c.L[k], c.L_bstride, c.u, c.x_out, c.q_out, c.lse_out);
    return hipGetLastError();
}

// ---------------------------------------------------------------- RNN head, batched
// [P3] "Semi-Autoregressive Generation" (the RNN head: a recurrent state inside the block),
// with the recurrence h_1 = W1[x_0], h_k = A h_{k-1} + W1[x_{k-1}], B_k = h_k W2.

namespace {

constexpr int kStateThreads = 256;      // one thread per state element (r <= 256)

// One workgroup per request: h_next = (k > 0 ? A h_prev : 0) + W1[x_{k-1}] in fp32, summed
// over j in ascending order; written as fp32 (h_next, and h_out when asked) and as the bf16
// hi / lo rows the projection multiplies (hi = bf16(h), lo = bf16(h - hi), zero beyond r).
// A request whose previous token is invalid is dead: its state is 0 (its logits are -inf).
__global__ __launch_bounds__(kStateThreads)
void rnn_state_kernel(int B, int r, int rp, int k, int gamma, const uint16_t* __restrict__ A,
                      const uint16_t* __restrict__ W1, int V, const int32_t* __restrict__ tok,
                      int tok_stride, const float* __restrict__ h_prev, float* __restrict__ h_next,
                      uint16_t* __restrict__ hrows, float* __restrict__ h_out) {
    __shared__ float hp[kMaxRank];
    const int b = blockIdx.x, i = threadIdx.x;
    int t = tok[static_cast<long long>(b) * tok_stride];
    if (t < 0 || t >= V) t = -1;
    if (k > 0 && i < r) hp[i] = h_prev[static_cast<long long>(b) * r + i];
    __syncthreads();
    float h = 0.0f;
    if (i < r && t >= 0) {
        if (k > 0) {
            const uint16_t* Ar = A + static_cast<long long>(i) * r;
            for (int j = 0; j < r; j += 8) {
                const uint4 w = *reinterpret_cast<const uint4*>(Ar + j);
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h = fmaf(__uint_as_float(ww[e] << 16), hp[j + 2 * e], h);
                    h = fmaf(__uint_as_float(ww[e] & 0xffff0000u), hp[j + 2 * e + 1], h);
                }
            }
        }
        h += to_f32(W1[static_cast<long long>(t) * r + i]);
    }
    if (i < r) {
        h_next[static_cast<long long>(b) * r + i] = h;
        if (h_out) h_out[(static_cast<long long>(b) * gamma + k) * r + i] = h;
    }
    if (i < rp) {
        const __bf16 hi = static_cast<__bf16>(h);
        const __bf16 lo = static_cast<__bf16>(h - static_cast<float>(hi));
        uint16_t* row = hrows + static_cast<long long>(b) * 2 * rp;
        row[i] = __builtin_bit_cast(uint16_t, hi);
        row[rp + i] = __builtin_bit_cast(uint16_t, lo);
    }
}

// Draw of position k for every request (one wave per request, as draft_select), then, when
// a later position follows, the request's next state h_{k+1} = A h_k + W1[x_k]: A h_k comes
// from the matvec workgroups of position k's projection launch, and the W1 row of the token
// just drawn is added to it, so the state equals rnn_state_kernel's bit for bit. It is
// written as rnn_state_kernel writes it (fp32, h_out, bf16 hi / lo rows); a dead request's
// state is 0.
__global__ __launch_bounds__(kSelThreads)
void rnn_select_kernel(int B, int V, int r, int rp, int gamma, int k,
                       const float2* __restrict__ part, int nblk, const float* __restrict__ L,
                       long long L_bstride, const float* __restrict__ u, int32_t* __restrict__ x_out,
                       float* __restrict__ q_out, float* __restrict__ lse_out,
                       const float* __restrict__ Ah, const uint16_t* __restrict__ W1,
                       float* __restrict__ h_next, uint16_t* __restrict__ hrows,
                       float* __restrict__ h_out) {
    const int b = blockIdx.x * (kSelThreads / kWave) + threadIdx.x / kWave;
    if (b >= B) return;
    const int lane = threadIdx.x & (kWave - 1);
    const long long o = static_cast<long long>(b) * gamma + k;
    const DrawOut out{x_out + o, q_out ? q_out + o : nullptr, lse_out ? lse_out + o : nullptr,
                      true};
    int t = draw_wave<kNT>(V, part + static_cast<long long>(b) * nblk, nblk, L + b * L_bstride,
                           u[o], out);
    if (k + 1 >= gamma) return;
    if (t < 0 || t >= V) t = -1;
    uint16_t* row = hrows + static_cast<long long>(b) * 2 * rp;
    for (int i = lane; i < rp; i += kWave) {
        float h = 0.0f;
        if (i < r && t >= 0) {
            h = Ah[static_cast<long long>(b) * r + i];
            h += to_f32(W1[static_cast<long long>(t) * r + i]);
        }
        if (i < r) {
            h_next[static_cast<long long>(b) * r + i] = h;
            if (h_out) h_out[(static_cast<long long>(b) * gamma + k + 1) * r + i] = h;
        }
        const __bf16 hi = static_cast<__bf16>(h);
        const __bf16 lo = static_cast<__bf16>(h - static_cast<float>(hi));
        row[i] = __builtin_bit_cast(uint16_t, hi);
        row[rp + i] = __builtin_bit_cast(uint16_t, lo);
    }
}

}  // namespace

int rnn_rank_pad(int r) {
    int rp = (r + kKC - 1) / kKC * kKC;
    if (rp % 8) rp += 8 - rp % 8;
    return rp;
}

bool rnn_mfma_ok(int V, int r, const void* W1, const void* W2, const void* A) {
    return r <= kMaxRank && (r % 8) == 0 && (V % 8) == 0 &&
           static_cast<long long>(kMaxRank) * V < (1LL << 32) &&
           static_cast<long long>(kMT) * 64 * V < (1LL << 32) &&
           (reinterpret_cast<uintptr_t>(W1) % 16) == 0 && (reinterpret_cast<uintptr_t>(W2) % 16) == 0 &&
           (reinterpret_cast<uintptr_t>(A) % 16) == 0;
}

hipError_t launch_rnn_mfma(const RnnCall& rc, hipStream_t st) {
    const DraftCall& c = rc.d;
    MfmaArgs a;
    a.B = c.B; a.V = c.V; a.r = c.r; a.rp = rnn_rank_pad(c.r);
    a.gamma = c.gamma;
    a.ntiles = (c.V + kNT - 1) / kNT;
    a.mgroups = (c.B + kMT - 1) / kMT;
    a.U = c.U;
    a.W1 = static_cast<const uint16_t*>(c.W1);
    a.W2 = static_cast<const uint16_t*>(c.W2);
    a.Hrows = rc.hrows;
    a.L_bstride = c.L_bstride;
    const unsigned grid_tiles = static_cast<unsigned>((a.ntiles + kXcds - 1) / kXcds * kXcds);
    const dim3 grid(grid_tiles * a.mgroups);
    const size_t smem = (2 * static_cast<size_t>(kMT) * (a.rp + kHPad) + kWaves * kKC * kWS) * sizeof(uint16_t);
    {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(draft_step_mfma<true>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 static_cast<int>(smem));
        if (e != hipSuccess) return e;
    }
    a.A = static_cast<const uint16_t*>(rc.A);
    a.Ah = rc.ah;
    // h_1 = W1[x_0]; afterwards each draw launch finishes the next state (rnn_select_kernel)
    hipLaunchKernelGGL(rnn_state_kernel, dim3(c.B), dim3(kStateThreads), 0, st, c.B, c.r, a.rp, 0,
                       c.gamma, static_cast<const uint16_t*>(rc.A), a.W1, c.V, c.x0, 1,
                       rc.hstate[1], rc.hstate[0], rc.hrows, rc.h_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int waves = kSelThreads / kWave;
    for (int k = 0; k < c.gamma; ++k) {
        a.k = k;
        a.tok = k ? c.x_out + (k - 1) : c.x0;
        a.tok_stride = k ? c.gamma : 1;
        a.L = c.L[k];
        a.part = c.part[k & 1];
        a.hcur = rc.hstate[k & 1];
        a.mv0 = grid.x;
        const dim3 g(grid.x + (k + 1 < c.gamma ? static_cast<unsigned>(c.B) : 0u));
        hipLaunchKernelGGL(draft_step_mfma<true>, g, dim3(kThreads), smem, st, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(rnn_select_kernel, dim3((c.B + waves - 1) / waves), dim3(kSelThreads), 0, st,
                           c.B, c.V, c.r, a.rp, c.gamma, k, static_cast<const float2*>(c.part[k & 1]),
                           a.ntiles, c.L[k], c.L_bstride, c.u, c.x_out, c.q_out, c.lse_out, rc.ah,
                           a.W1, rc.hstate[(k + 1) & 1], rc.hrows, rc.h_out);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dspark
