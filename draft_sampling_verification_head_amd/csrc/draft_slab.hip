// Batched Markov-head draft with each vocabulary slab of W2 held in registers (gfx950).
//
// [P3] "DSpark Speculative Decoding", section "Semi-Autoregressive Generation": the bias of
// position k is B_k = W1[x_{k-1}] W2 for every request, one [B x r] * [r x V] product per step
// (rank r = 256), added to the backbone logits U_k; x_k is drawn from softmax(U_k + B_k).
// ([P3] = the concept note "DSpark Speculative Decoding".)
//
// Step kernel (draft_slab_step), one launch per draft position:
//   - One workgroup of 8 waves per vocabulary slab of 128 * NT columns. Wave w owns the
//     16 * NT columns of its "wave tile" and keeps W2 for those columns, all ranks, in
//     registers as MFMA A fragments of W2^T (v_mfma_f32_16x16x32_bf16: 16 columns x 32 ranks
//     per fragment, NT * 8 fragments). W2 is read from HBM once per launch, staged through a
//     wave-private LDS area that turns rank-major rows into rank-contiguous fragments.
//   - The batch then streams through the slab in groups of 16 requests. A group's U_k rows
//     (16 x 128 NT floats) and gathered W1 rows (16 x 256 bf16) arrive in LDS by direct
//     global-to-LDS loads, issued two groups ahead into one of three buffers, so HBM keeps
//     two groups in flight while the current one is multiplied.
//   - Per group and wave: NT * r/32 MFMAs give the bias for 16 requests x 16 * NT columns;
//     the epilogue adds U_k, optionally stores the logits, and reduces each request's
//     columns of the wave tile to (max, sum exp(l - max)), the tile partial the draw uses.
// Draw kernel (draft_slab_select), one wave per request: merges the request's tile partials
// in tile order, picks the tile that holds the inverse-CDF point, and recomputes that tile's
// logits with the same MFMA sequence on the same operands. A fragment column of the MFMA
// result depends only on that column's operands, so the recomputed logits are bit-identical
// to the step's and the logits never need to be written to memory.
#include "common.h"
#include "draw.h"
#include "kernels.h"
#include "slab.h"

namespace dspark {

namespace {
using namespace slab;

constexpr int kGrp = 16;                 // requests per group (MFMA N)
constexpr int kHBuf = kGrp * kHRow;      // 8 KB of gathered W1 rows per group

struct SlabArgs {
    int B, V, r, gamma, k, ntw;
    const float* U;           // [B][gamma][V]
    const uint16_t* W1;       // [V][r] bf16
    const uint16_t* W2;       // [r][V] bf16
    const int32_t* tok;       // x_{k-1}: tok[b * tok_stride]
    int tok_stride;
    float* L;                 // logits rows L + b * L_bstride, or null (not stored)
    long long L_bstride;
    float2* part;             // [B][ntw] (max, sum exp) per request and wave tile
};

// LDS: [U0][U1][H0][H1][U2][H2][H3][tokens]. U slot i holds group g = i (mod 3), every wave's
// own tiles (wave-private); H slot j holds group g = j (mod 4), shared by the waves. The W2
// staging areas overlay U2 + H2 + H3, which are first written after the staging.
template <int NT>
constexpr int ubuf_bytes() { return kGrp * Slab<NT>::SW * 4; }   // one group's U_k slice
template <int NT>
__device__ __forceinline__ int ubuf_off(int i) {
    constexpr int UB = ubuf_bytes<NT>();
    return i == 0 ? 0 : (i == 1 ? UB : 2 * UB + 2 * kHBuf);
}
template <int NT>
__device__ __forceinline__ int hbuf_off(int j) {
    constexpr int UB = ubuf_bytes<NT>();
    return j < 2 ? 2 * UB + j * kHBuf : 3 * UB + j * kHBuf;
}
template <int NT>
constexpr int tok_off() { return 3 * ubuf_bytes<NT>() + 4 * kHBuf; }

// Pipeline (per wave, three groups of loads in flight while a group is computed):
//   wait for group g's loads; store group g - 1's results; copy this wave's U_k tiles of
//   group g into registers (the wave's U slot is then free); barrier (group g's W1 rows are
//   visible, every wave is done with group g - 1's W1 slot); issue group g + 3's loads into
//   the freed slots; MFMA and epilogue of group g.
// The stores of group g - 1 are issued before group g + 3's loads, so that the loads issued
// after group g's are always the 2 (NT + 1) of groups g + 1 and g + 2 (plus stores that
// precede them): vector memory loads complete in order, so once at most 2 (NT + 1)
// operations are outstanding, group g's loads have landed.
template <int NT, bool LOUT>
__global__ __launch_bounds__(kSlabThreads)
void draft_slab_step(SlabArgs a) {
    using S = Slab<NT>;
    constexpr int UB = ubuf_bytes<NT>();
    constexpr int NL = NT + 1;                        // direct loads per wave and group
    static_assert(kSlabWaves * S::Stage <= UB + 2 * kHBuf, "W2 staging fits in U2 + H2 + H3");
    extern __shared__ __align__(16) char sm[];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int slab = blockIdx.x;
    const long long cw = static_cast<long long>(slab) * S::SW + wave * S::WC;
    const int ng = (a.B + kGrp - 1) / kGrp;
    int* stok = reinterpret_cast<int*>(sm + tok_off<NT>());

    for (int b = tid; b < a.B; b += kSlabThreads) {
        const int t = a.tok[static_cast<long long>(b) * a.tok_stride];
        stok[b] = (t >= 0 && t < a.V) ? t : -1;       // dead request: no bias, -inf logits
    }
    __syncthreads();

    // Loads of group g, NT + 1 direct-to-LDS instructions per wave, every lane active
    // (addresses of absent requests / columns / ranks are clamped to valid memory; the
    // epilogue masks those values), so each wave issues exactly NT + 1 of them.
    //  U: wave w fills its tiles w NT .. w NT + NT - 1 of the slab, 1 KB each ([16 req][16 col]);
    //     lane l loads request l / 4, 4-column chunk (l % 4) ^ ((l / 16) % 4), an XOR swizzle
    //     that makes the register copy's reads bank-conflict free.
    //  H: wave w fills rows 2w, 2w + 1 (512 bytes each); lane l loads 16-byte piece
    //     (l % 32) ^ (row % 16) of the row, again a swizzle for the fragment reads.
    const int u_rq = lane >> 2, u_ch = (lane & 3) ^ ((lane >> 4) & 3);
    const int h_row = 2 * wave + (lane >> 5), h_piece = (lane & 31) ^ (h_row & 15);
    auto issue = [&](int g) {
        const int m0 = g * kGrp;
        const int b = min(m0 + u_rq, a.B - 1);
        const float* urow = a.U + (static_cast<long long>(b) * a.gamma + a.k) * a.V;
        char* ub = sm + ubuf_off<NT>(g % 3) + wave * NT * 1024;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            long long col = cw + 16 * t + 4 * u_ch;
            if (col >= a.V) col = 0;
            lds_dma16(urow + col, ub + t * 1024);
        }
        int tk = (m0 + h_row < a.B) ? stok[m0 + h_row] : -1;
        if (tk < 0) tk = 0;
        const int piece = (8 * h_piece < a.r) ? h_piece : 0;
        lds_dma16(a.W1 + static_cast<long long>(tk) * a.r + 8 * piece, sm + hbuf_off<NT>(g & 3) + wave * 1024);
    };

    issue(0);
    if (ng > 1) issue(1);
    bf16x8 w2f[NT][kKS];
    load_w2_frags<NT, 4, 1>(w2f, a.W2, a.V, a.r, cw, sm + 2 * UB + 2 * kHBuf + wave * S::Stage);
    wait_lgkm0();
    __syncthreads();                                  // every wave is done with the staging area
    if (ng > 2) issue(2);

    const int rq = lane & 15, cg = lane >> 4;
    const int upos = 4 * rq + (cg ^ ((rq >> 2) & 3));  // this lane's 16 bytes of a U tile
    int pend_b = -1;                                   // request of the pending results
    float2 pend_part = make_float2(0.0f, 0.0f);
    float4 pend_l[LOUT ? NT : 1];
    auto flush = [&]() {
        if (pend_b < 0) return;
        if (LOUT) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const long long col = cw + 16 * t + 4 * cg;
                if (col < a.V) *reinterpret_cast<float4*>(a.L + pend_b * a.L_bstride + col) = pend_l[LOUT ? t : 0];
            }
        }
        if (lane < kGrp)
            a.part[static_cast<long long>(pend_b) * a.ntw + slab * kSlabWaves + wave] = pend_part;
    };
    for (int g = 0; g < ng; ++g) {
        if (g + 2 < ng) wait_vm_lgkm<2 * NL>();
        else if (g + 1 < ng) wait_vm_lgkm<NL>();
        else wait_vm_lgkm<0>();
        flush();
        float4 u4[NT];
        const char* Ub = sm + ubuf_off<NT>(g % 3) + wave * NT * 1024;
#pragma unroll
        for (int t = 0; t < NT; ++t) u4[t] = *reinterpret_cast<const float4*>(Ub + t * 1024 + 16 * upos);
        wait_lgkm0();                                 // the U slot may be refilled
        bare_barrier();
        if (g + 3 < ng) issue(g + 3);

        const char* H = sm + hbuf_off<NT>(g & 3);
        f32x4 acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        // B fragments one rank chunk ahead; the empty asm keeps the compiler from hoisting
        // every chunk's fragment at once, which would not fit beside the W2 fragments
        auto hfrag = [&](int s) {
            const int piece = (4 * s + cg) ^ rq;
            return *reinterpret_cast<const bf16x8*>(H + rq * kHRow + 16 * piece);
        };
        bf16x8 hf = hfrag(0);
#pragma unroll
        for (int s = 0; s < kKS; ++s) {
            const bf16x8 hn = (s + 1 < kKS) ? hfrag(s + 1) : hf;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2f[t][s], hf, acc[t], 0, 0, 0);
            asm volatile("" ::: "memory");
            hf = hn;
        }

        // epilogue: lane holds request rq, columns 4 cg .. 4 cg + 3 of each of its NT tiles.
        // Dead or absent requests and columns past V get -inf; when the whole wave is live
        // and its tile lies inside the vocabulary (all but the last slab), no per-element
        // masking is needed. exp(-inf - max) is 0, so only an all -inf row needs care.
        const int b = g * kGrp + rq;
        const bool live = b < a.B && stok[b] >= 0;
        const bool fast = cw + S::WC <= a.V && __builtin_amdgcn_read_exec() == ~0ull &&
                          __ballot(live) == ~0ull;
        float lv[NT][4];
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            lv[t][0] = u4[t].x + acc[t][0];
            lv[t][1] = u4[t].y + acc[t][1];
            lv[t][2] = u4[t].z + acc[t][2];
            lv[t][3] = u4[t].w + acc[t][3];
            if (!fast) {
                const bool ok = live && cw + 16 * t + 4 * cg < a.V;
#pragma unroll
                for (int v = 0; v < 4; ++v) lv[t][v] = ok ? lv[t][v] : -INFINITY;
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) mx = fmaxf(mx, lv[t][v]);
            if (LOUT) pend_l[LOUT ? t : 0] = make_float4(lv[t][0], lv[t][1], lv[t][2], lv[t][3]);
        }
        mx = fmaxf(mx, swz_xor16(mx));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        float sum = 0.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) sum += __expf(lv[t][v] - mx);
        sum += swz_xor16(sum);
        sum += __shfl_xor(sum, 32, kWave);
        if (mx == -INFINITY) sum = 0.0f;
        pend_b = b < a.B ? b : -1;
        pend_part = make_float2(mx, sum);
    }
    flush();
}

struct SlabSelArgs {
    int B, V, r, gamma, k, ntw;
    const float* U;
    const uint16_t* W1;
    const uint16_t* W2;
    const int32_t* tok;       // x_{k-1}
    int tok_stride;
    const float2* part;
    const float* u;           // [B][gamma]
    int32_t* x_out;
    float* q_out;
    float* lse_out;
};

// One wave (one workgroup) per request: tile pick from the partials, MFMA recompute of that
// tile's logits, in-tile rescan. Every W2 load of the tile is in flight at once (one LDS
// staging slot per rank chunk), and the W1 row is fetched before the merge.
template <int NT>
__global__ __launch_bounds__(kWave)
void draft_slab_select(SlabSelArgs a) {
    using S = Slab<NT>;
    constexpr int CPL = (S::WC + kWave - 1) / kWave;
    __shared__ __align__(16) char stg[kKS * S::Stage];
    __shared__ float rowv[S::WC];
    const int lane = threadIdx.x;
    const int b = blockIdx.x;
    const long long o = static_cast<long long>(b) * a.gamma + a.k;
    const DrawOut out{a.x_out + o, a.q_out ? a.q_out + o : nullptr,
                      a.lse_out ? a.lse_out + o : nullptr, true};
    const int rq = lane & 15, cg = lane >> 4;

    // the W1 row of the previous token in every one of the 16 request columns of the B
    // operand (only used when the request has mass, which implies a valid token)
    int tk = a.tok[static_cast<long long>(b) * a.tok_stride];
    if (tk < 0 || tk >= a.V) tk = 0;
    uint4 hv[kKS];
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
        const int rank = 32 * s + 8 * cg;
        hv[s] = make_uint4(0u, 0u, 0u, 0u);
        if (rank < a.r) hv[s] = *reinterpret_cast<const uint4*>(a.W1 + static_cast<long long>(tk) * a.r + rank);
    }
    // lane l holds tiles [32 l, 32 l + 32): 16 loads of two partials each
    float2 p[kSelRegs];
    const float4* P4 = reinterpret_cast<const float4*>(a.part + static_cast<long long>(b) * a.ntw);
#pragma unroll
    for (int t = 0; t < kSelRegs / 2; ++t) {
        const int i = lane * kSelRegs + 2 * t;        // ntw is a multiple of 8: pairs are whole
        float4 v = make_float4(-INFINITY, 0.0f, -INFINITY, 0.0f);
        if (i < a.ntw) v = P4[i / 2];
        p[2 * t] = make_float2(v.x, v.y);
        p[2 * t + 1] = make_float2(v.z, v.w);
    }
    const TilePick tp = pick_tile<kSelRegs>(p, a.u[o]);
    if (tp.tile < 0) {
        if (lane == 0) put(out, -1, 0.0f, -INFINITY);
        return;
    }
    const long long cw = static_cast<long long>(tp.tile) * S::WC;
    const float* urow = a.U + (static_cast<long long>(b) * a.gamma + a.k) * a.V;
    float4 u4[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const long long col = cw + 16 * t + 4 * cg;
        u4[t] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (rq == 0 && col < a.V) u4[t] = *reinterpret_cast<const float4*>(urow + col);
    }
    bf16x8 w2f[NT][kKS];
    load_w2_frags<NT, kKS, kKS>(w2f, a.W2, a.V, a.r, cw, stg);
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
        {
            const bf16x8 hf = __builtin_bit_cast(bf16x8, hv[s]);
#pragma unroll
            for (int t = 0; t < NT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2f[t][s], hf, acc[t], 0, 0, 0);
        }
    }
    if (rq == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bool ok = cw + 16 * t + 4 * cg < a.V;
            float* rv = &rowv[16 * t + 4 * cg];
            rv[0] = ok ? u4[t].x + acc[t][0] : -INFINITY;
            rv[1] = ok ? u4[t].y + acc[t][1] : -INFINITY;
            rv[2] = ok ? u4[t].z + acc[t][2] : -INFINITY;
            rv[3] = ok ? u4[t].w + acc[t][3] : -INFINITY;
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0): the row is in LDS
    __builtin_amdgcn_wave_barrier();
    float lv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane * CPL + j;
        lv[j] = (c < S::WC) ? rowv[c] : -INFINITY;
    }
    rescan_values<CPL>(lv, cw + lane * CPL, static_cast<int>(cw), tp.m, tp.lse, tp.tprime, out);
}

size_t slab_lds_bytes(int nt, int B) {
    return 3 * static_cast<size_t>(kGrp) * kSlabWaves * 16 * nt * 4 + 4 * kHBuf + 4 * static_cast<size_t>(B);
}

template <int NT>
hipError_t launch_nt(const DraftCall& c, hipStream_t st) {
    SlabArgs a;
    a.B = c.B; a.V = c.V; a.r = c.r; a.gamma = c.gamma;
    a.ntw = draft_slab_tiles(c.V);
    a.U = c.U;
    a.W1 = static_cast<const uint16_t*>(c.W1);
    a.W2 = static_cast<const uint16_t*>(c.W2);
    a.L_bstride = c.L_bstride;
    SlabSelArgs s;
    s.B = c.B; s.V = c.V; s.r = c.r; s.gamma = c.gamma; s.ntw = a.ntw;
    s.U = c.U; s.W1 = a.W1; s.W2 = a.W2; s.u = c.u;
    s.x_out = c.x_out; s.q_out = c.q_out; s.lse_out = c.lse_out;
    const size_t smem = slab_lds_bytes(NT, c.B);
    const dim3 grid(static_cast<unsigned>(slab_count(c.V)));
    const dim3 sgrid(static_cast<unsigned>(c.B));
    for (int k = 0; k < c.gamma; ++k) {
        a.k = k;
        a.tok = k ? c.x_out + (k - 1) : c.x0;
        a.tok_stride = k ? c.gamma : 1;
        a.L = c.L_out ? c.L[k] : nullptr;
        a.part = c.part[k & 1];
        if (c.L_out)
            hipLaunchKernelGGL((draft_slab_step<NT, true>), grid, dim3(kSlabThreads), smem, st, a);
        else
            hipLaunchKernelGGL((draft_slab_step<NT, false>), grid, dim3(kSlabThreads), smem, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        s.k = k;
        s.tok = a.tok;
        s.tok_stride = a.tok_stride;
        s.part = a.part;
        hipLaunchKernelGGL(draft_slab_select<NT>, sgrid, dim3(kWave), 0, st, s);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

int draft_slab_tiles(int V) { return slab_count(V) * kSlabWaves; }

bool draft_slab_ok(int B, int V, int r, int w_dtype, const void* W1, const void* W2) {
    if (w_dtype != 1 || B <= 8 || r > kMaxRank || (r % 8) != 0 || (V % 8) != 0) return false;
    if (draft_slab_tiles(V) > kWave * kSelRegs) return false;     // the draw keeps every partial in registers
    if (slab_lds_bytes(slab_nt(V), B) > static_cast<size_t>(kLdsBytes)) return false;
    if (static_cast<long long>(kMaxRank) * V >= (1LL << 32)) return false;
    return (reinterpret_cast<uintptr_t>(W1) % 16) == 0 && (reinterpret_cast<uintptr_t>(W2) % 16) == 0;
}

hipError_t launch_draft_slab(const DraftCall& c, hipStream_t st) {
    switch (slab_nt(c.V)) {
        case 1: return launch_nt<1>(c, st);
        case 2: return launch_nt<2>(c, st);
        case 3: return launch_nt<3>(c, st);
        case 4: return launch_nt<4>(c, st);
        default: return launch_nt<5>(c, st);
    }
}

}  // namespace dspark
