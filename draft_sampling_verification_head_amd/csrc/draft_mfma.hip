// Batched Markov-head draft step on bf16 MFMA (gfx950).
//
// [P3] "DSpark Speculative Decoding", section "Semi-Autoregressive Generation": the bias of
// position k is B_k = W1[x_{k-1}] W2 for every request, i.e. one [B x r] * [r x V] product
// per step (rank r = 256) added to the backbone logits U_k. ([P3] = the concept note
// "DSpark Speculative Decoding".)
//
// Used when a batch is large enough for the product to be a dense GEMM (B > 8 requests,
// bf16 factors). Workgroup = 64 requests x 256 vocabulary columns, 8 waves; wave w owns
// columns [32w, 32w + 32) and both 32-request halves, accumulating with
// v_mfma_f32_32x32x16_bf16 in fp32. The gathered W1 rows (A operand, rank-contiguous) sit in
// LDS for the whole workgroup; W2 (B operand) streams through LDS in 16-row chunks, double
// buffered, in its natural [r][V] layout, and each lane picks its 8 rank values of one
// column with 2-byte LDS reads. The epilogue adds U_k, stores the logits and reduces each
// request row of the tile to a (max, sum exp) partial for the draw. Workgroups are mapped so
// that the request groups of one vocabulary tile run on the same XCD (shared L2).
#include "common.h"
#include "draw.h"
#include "kernels.h"

namespace dspark {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMT = 64;                 // requests per workgroup
constexpr int kNT = 256;                // vocabulary columns per workgroup
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kKC = 16;                 // rank rows per W2 chunk (one MFMA k-step)
constexpr int kWS = kNT + 4;            // W2 chunk row stride (bf16), padded against bank conflicts
constexpr int kHPad = 8;                // H row padding (bf16)
constexpr int kXcds = 8;
static_assert(kWaves * 32 == kNT, "one 32-column MFMA tile per wave");

struct MfmaArgs {
    int B, V, r, rp, gamma, k, ntiles, mgroups;
    const float* U;
    const uint16_t* W1;
    const uint16_t* W2;
    const int32_t* tok;       // x_{k-1}: tok[b * tok_stride]
    int tok_stride;
    float* L;                 // logits rows L + b * L_bstride
    long long L_bstride;
    float2* part;             // [B][ntiles] (max, sum exp) per request and tile
};

__global__ __launch_bounds__(kThreads, 2)
void draft_step_mfma(MfmaArgs a) {
    extern __shared__ uint16_t sm16[];
    const int HS = a.rp + kHPad;
    uint16_t* Hs = sm16;                              // [kMT][HS] gathered W1 rows
    uint16_t* Ws = sm16 + kMT * HS;                   // [2][kKC][kWS] W2 chunks
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
    // A operand: the gathered W1 rows, zero beyond r and for dead / absent requests
    const int segs = a.rp / 8;
    for (int s = tid; s < kMT * segs; s += kThreads) {
        const int i = s / segs, c = (s % segs) * 8;
        const int t = stok[i];
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (t >= 0 && c < a.r) v = *reinterpret_cast<const uint4*>(a.W1 + static_cast<long long>(t) * a.r + c);
        *reinterpret_cast<uint4*>(Hs + i * HS + c) = v;
    }
    // W2 chunk kc -> registers: thread t holds row t/32, columns 8*(t%32) .. +8
    const int wrow = tid >> 5, wcol = (tid & 31) * 8;
    auto load_chunk = [&](int kc) {
        const int kk = kc * kKC + wrow;
        const long long col = n0 + wcol;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (kk < a.r && col < a.V) v = *reinterpret_cast<const uint4*>(a.W2 + static_cast<long long>(kk) * a.V + col);
        return v;
    };
    auto store_chunk = [&](int buf, uint4 v) {
        uint16_t* dst = Ws + (buf * kKC + wrow) * kWS + wcol;
        reinterpret_cast<uint2*>(dst)[0] = make_uint2(v.x, v.y);
        reinterpret_cast<uint2*>(dst)[1] = make_uint2(v.z, v.w);
    };
    store_chunk(0, load_chunk(0));
    __syncthreads();

    f32x16 acc0 = {}, acc1 = {};
    const int nkc = a.rp / kKC;
    const int half = lane >> 5, l32 = lane & 31;
    for (int kc = 0; kc < nkc; ++kc) {
        const int cur = kc & 1;
        uint4 nxt = make_uint4(0u, 0u, 0u, 0u);
        if (kc + 1 < nkc) nxt = load_chunk(kc + 1);   // in flight during the MFMAs
        // B fragment: column 32*wave + l32, rank rows 8*half .. +8 of the chunk
        const uint16_t* wc = Ws + (cur * kKC + 8 * half) * kWS + wave * 32 + l32;
        s16x8 bv;
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = static_cast<short>(wc[e * kWS]);
        const bf16x8 bfrag = __builtin_bit_cast(bf16x8, bv);
        // A fragments: request rows l32 and 32 + l32, the same 8 rank values
        const int kofs = kc * kKC + 8 * half;
        const bf16x8 a0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Hs + l32 * HS + kofs));
        const bf16x8 a1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(Hs + (32 + l32) * HS + kofs));
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bfrag, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bfrag, acc1, 0, 0, 0);
        if (kc + 1 < nkc) store_chunk(cur ^ 1, nxt);
        __syncthreads();
    }

    // epilogue: element v of the accumulator of half-tile h is request row
    // 32h + 8(v/4) + 4*half + v%4, column 32*wave + l32
    const long long col = n0 + wave * 32 + l32;
    const bool colok = col < a.V;
    float lv[32];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = 32 * h + 8 * (v / 4) + 4 * half + (v % 4);
            const int b = m0 + i;
            const bool live = colok && b < a.B && stok[i] >= 0;
            const float accv = h ? acc1[v] : acc0[v];
            lv[16 * h + v] = live ? a.U[(static_cast<long long>(b) * a.gamma + a.k) * a.V + col] + accv
                                  : -INFINITY;
        }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = 32 * h + 8 * (v / 4) + 4 * half + (v % 4);
            const int b = m0 + i;
            if (colok && b < a.B) a.L[b * a.L_bstride + col] = lv[16 * h + v];
        }
    // per request row: max over the tile (lanes of a half, then waves in order)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            float m = lv[16 * h + v];
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
            if (l32 == 0) red[wave][32 * h + 8 * (v / 4) + 4 * half + (v % 4)] = m;
        }
    __syncthreads();
    if (tid < kMT) {
        float m = red[0][tid];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) m = fmaxf(m, red[w][tid]);
        rowmax[tid] = m;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int i = 32 * h + 8 * (v / 4) + 4 * half + (v % 4);
            const float m = rowmax[i];
            const float x = lv[16 * h + v];
            float e = (x == -INFINITY) ? 0.0f : __expf(x - m);
#pragma unroll
            for (int o = 16; o > 0; o >>= 1) e += __shfl_xor(e, o, kWave);
            if (l32 == 0) red[wave][i] = e;
        }
    __syncthreads();
    if (tid < kMT) {
        const int b = m0 + tid;
        if (b < a.B) {
            float s = red[0][tid];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) s += red[w][tid];
            a.part[static_cast<long long>(b) * a.ntiles + tile] = make_float2(rowmax[tid], s);
        }
    }
}

}  // namespace

int draft_mfma_tile_cols() { return kNT; }

bool draft_mfma_ok(int B, int V, int r, int w_dtype, const void* W1, const void* W2) {
    return w_dtype == 1 && B > 8 && r <= 256 && (r % 8) == 0 && (V % 8) == 0 &&
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
    const size_t smem = (static_cast<size_t>(kMT) * (a.rp + kHPad) + 2 * kKC * kWS) * sizeof(uint16_t);
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
        hipLaunchKernelGGL(draft_step_mfma, grid, dim3(kThreads), smem, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int k = c.gamma - 1;
    hipLaunchKernelGGL(draft_select<kNT>, dim3((c.B + waves - 1) / waves), dim3(kSelThreads), 0, st,
                       c.B, c.V, c.gamma, k, static_cast<const float2*>(c.part[k & 1]), a.ntiles,
                       c.L[k], c.L_bstride, c.u, c.x_out, c.q_out, c.lse_out);
    return hipGetLastError();
}

}  // namespace dspark
