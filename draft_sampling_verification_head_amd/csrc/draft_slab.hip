// Batched Markov-head draft with each vocabulary slab of W2 held in registers (gfx950).
//
// [P3] "DSpark Speculative Decoding", section "Semi-Autoregressive Generation": the bias of
// position k is B_k = W1[x_{k-1}] W2 for every request, one [B x r] * [r x V] product per step
// (rank r = 256), added to the backbone logits U_k; x_k is drawn from softmax(U_k + B_k).
// ([P3] = the concept note "DSpark Speculative Decoding".)
//
// Stream (one position): one workgroup of 8 waves per vocabulary slab of 128 * NT columns.
// Wave w owns the 16 * NT columns of its "wave tile" and keeps W2 for those columns, all
// ranks, in registers as MFMA A fragments of W2^T (v_mfma_f32_16x16x32_bf16: 16 columns x 32
// ranks per fragment, NT * 8 fragments), staged once through a wave-private LDS area that
// turns rank-major rows into rank-contiguous fragments. The batch streams through the slab in
// groups of 16 requests: U_k tiles and gathered W1 rows arrive in LDS by direct loads three
// groups ahead, the MFMAs, their accumulators started at U_k, give the logits U_k + bias of
// 16 requests x 16 NT columns per wave, and the epilogue optionally stores the logits and
// reduces each request's columns of the wave tile to (max, sum exp(l - max)), the tile
// partial the draw uses.
//
// Draw (one request): a two-level pick. The 8 wave-tile partials of each slab are merged in
// tile order into a slab partial; the request's slab partials give the slab that holds the
// inverse-CDF point, and that slab's 8 tile partials the tile. The chosen tile's logits are
// then recomputed with the same MFMA sequence on the same operands. A column of an MFMA
// result depends only on that column's operands, so the recomputed logits are bit-identical
// to the stream's and the logits never need to be written to memory.
//
// Two launch shapes, which draw the same tokens bit for bit and store the same logits:
//   - per position, a stream launch (draft_slab_step) and a draw launch (draft_slab_select,
//     one wave per request, which merges the slab partials from the tile partials itself and
//     loads the chosen tile's W2 fragments);
//   - one persistent launch for all positions (draft_slab_resident) when every slab
//     workgroup fits on the device at once and the caller did not ask for per-position
//     launches. W2 is loaded once per call;
//     each position runs in three phases separated by flag barriers (as in the single-request
//     resident draft): the stream, which also merges each group's slab partials through LDS
//     and publishes them; the slab picks, each workgroup for its share of the requests; the
//     draws, each by the wave that holds the chosen tile's W2 fragments in registers. Polling
//     is bounded; a workgroup that gives up writes -1 tokens for its requests' remaining
//     positions and stops, so the launch drains.
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
    int B, V, r, gamma, ntw, G;
    const float* U;           // [B][gamma][V]
    const uint16_t* W1;       // [V][r] bf16
    const uint16_t* W2;       // [r][V] bf16
    const int32_t* x0;        // [B]
    const float* u;           // [B][gamma]
    int32_t* x_out;           // [B][gamma]
    float* q_out;
    float* lse_out;
    float* L;                 // step: logits rows of the position, L + b * L_bstride;
                              // resident: those of position 0, position k at L + k * V
    long long L_bstride;
    float2* part;             // [B][ntw] (max, sum exp) per request and wave tile
    float2* spart;            // resident: [B][G] the same per request and slab (8 wave tiles)
    unsigned long long* flags;   // resident: [3][gamma][G], kEmpty until published
    unsigned long long* epoch;   // resident: [2] the call counter E and the ready word F
    unsigned* status;         // resident: number of workgroups that gave up (reset with the flags)
    unsigned spin;            // resident: polls before a flag wait gives up
    float4* picks;            // resident: [B] (slab, max, lse, mass left in the slab)
};

constexpr unsigned long long kEmpty = ~0ull;

// Ready word of a resident call with counter e (the single-request draft uses the same word
// in draft_resident.hip): the finaliser of the splitmix64 generator
// (Steele, Lea and Flood, "Fast splittable pseudorandom number generators", 2014) applied to
// e xor a constant, so that counters of all-zero or all-one bytes do not map to those bytes.
__device__ __forceinline__ unsigned long long ready_word(unsigned long long e) {
    unsigned long long z = e ^ 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

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


// Device-scope accesses for data that other workgroups of the same launch read or wrote.
__device__ __forceinline__ void store_coherent(float2* p, float2 v) {
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), __builtin_bit_cast(unsigned long long, v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(int32_t* p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_coherent(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long load_coherent(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Loads of group g of position k, NT + 1 direct-to-LDS instructions per wave, every lane
// active (addresses of absent requests / columns / ranks are clamped to valid memory; the
// epilogue masks those values), so each wave issues exactly NT + 1 of them.
//  U: wave w fills its tiles w NT .. w NT + NT - 1 of the slab, 1 KB each ([16 req][16 col]);
//     lane l loads request l / 4, 4-column chunk (l % 4) ^ ((l / 16) % 4), an XOR swizzle that
//     makes the register copy's reads bank-conflict free.
//  H: wave w fills rows 2w, 2w + 1 (512 bytes each); lane l loads 16-byte piece
//     (l % 32) ^ (row % 16) of the row, again a swizzle for the fragment reads.
// PARTS: 1 = the U loads only, 2 = the H load only, 3 = both.
template <int NT, int PARTS = 3>
__device__ __forceinline__ void issue_group(const SlabArgs& a, int k, int g, char* sm, const int* stok) {
    using S = Slab<NT>;
    const int lane = opaque_lane(), wave = threadIdx.x / kWave;
    const long long cw = static_cast<long long>(blockIdx.x) * S::SW + wave * S::WC;
    const int u_rq = lane >> 2, u_ch = (lane & 3) ^ ((lane >> 4) & 3);
    const int h_row = 2 * wave + (lane >> 5), h_piece = (lane & 31) ^ (h_row & 15);
    const int m0 = g * kGrp;
    const int b = min(m0 + u_rq, a.B - 1);
    const float* urow = a.U + (static_cast<long long>(b) * a.gamma + k) * a.V;
    const uint32_t ub = lds_addr(sm) + ubuf_off<NT>(g % 3) + wave * NT * 1024;
    if (PARTS & 1) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            long long col = cw + 16 * t + 4 * u_ch;
            if (col >= a.V) col = 0;
            lds_dma16(urow + col, ub + t * 1024);
        }
    }
    if (!(PARTS & 2)) return;
    int tk = (m0 + h_row < a.B) ? stok[m0 + h_row] : -1;
    if (tk < 0) tk = 0;
    const int piece = (8 * h_piece < a.r) ? h_piece : 0;
    lds_dma16(a.W1 + static_cast<long long>(tk) * a.r + 8 * piece,
              lds_addr(sm) + hbuf_off<NT>(g & 3) + wave * 1024);
}

// One position of the stream for this workgroup (slab): the tokens x_{k-1} of every request
// are in stok (-1: dead request). The caller has issued the loads of the first groups:
// `issued` whole groups (0 or 2), or with PRE the U loads of groups 0 .. min(ng, 3) - 1 (U
// does not depend on the tokens), whose H loads are then issued here first.
// Pipeline per wave, three groups of loads in flight while a group is computed: wait for
// group g's loads; store group g - 1's results; copy this wave's U_k tiles of group g into
// registers (the wave's U slot is then free); barrier (group g's W1 rows are visible, every
// wave is done with group g - 1's W1 slot); issue group g + 3's loads; MFMA and epilogue of
// group g. The stores of group g - 1 are issued before group g + 3's loads. Vector memory
// operations complete in order, so group g's loads have landed once no more operations are
// outstanding than were issued after group g's last load (the loads of later groups counted;
// stores between them only make the wait longer): 2 (NT + 1) in the steady state, fewer in
// the first groups and at the tail (after_group).
template <int NT, bool LOUT, bool PRE>
__device__ __forceinline__ void slab_stream(const SlabArgs& a, int k, float* L, const bf16x8 (&w2f)[NT][kKS],
                                            char* sm, const int* stok, int issued) {
    using S = Slab<NT>;
    constexpr int NL = NT + 1;                        // direct loads per wave and group
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int slab = blockIdx.x;
    const long long cw = static_cast<long long>(slab) * S::SW + wave * S::WC;
    const int ng = (a.B + kGrp - 1) / kGrp;

    auto issue = [&](int g) { issue_group<NT>(a, k, g, sm, stok); };
    const int npre = ng < 3 ? ng : 3;                 // groups issued before the loop
    if (PRE) {
        for (int g = 0; g < npre; ++g) issue_group<NT, 2>(a, k, g, sm, stok);
    } else {
        for (int g = issued; g < npre; ++g) issue(g);
    }
    // loads issued after group g's last load when group g is waited for
    auto after_group = [&](int g) {
        int n = 0;
        if (g < 3) n += (npre - 1 - g) * (PRE ? 1 : NL);   // later groups of the prologue
        for (int j = (g < 3 ? 0 : g - 2); j < g; ++j)       // groups j + 3 issued in loop j
            if (j + 3 < ng) n += NL;
        return n;
    };

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
                if (col < a.V) *reinterpret_cast<float4*>(L + pend_b * a.L_bstride + col) = pend_l[LOUT ? t : 0];
            }
        }
        if (lane < kGrp) a.part[static_cast<long long>(pend_b) * a.ntw + slab * kSlabWaves + wave] = pend_part;
    };

    for (int g = 0; g < ng; ++g) {
        const int n = after_group(g);                 // wait-uniform: a scalar branch
        if (n >= 2 * NL) wait_vm_lgkm<2 * NL>();
        else if (n >= NL + 1) wait_vm_lgkm<NL + 1>();
        else if (n >= NL) wait_vm_lgkm<NL>();
        else if (n >= 2) wait_vm_lgkm<2>();
        else if (n >= 1) wait_vm_lgkm<1>();
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
        // the accumulators start at U_k, so the MFMAs leave the logits U_k + bias
        f32x4 acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4{u4[t].x, u4[t].y, u4[t].z, u4[t].w};
        // B fragments one rank chunk ahead; the empty asm keeps the compiler from hoisting
        // every chunk's fragment at once, which would not fit beside the W2 fragments
        const int hl = opaque_lane(), hrq = hl & 15, hcg = hl >> 4;
        auto hfrag = [&](int s) {
            const int piece = (4 * s + hcg) ^ hrq;
            return *reinterpret_cast<const bf16x8*>(H + hrq * kHRow + 16 * piece);
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
            lv[t][0] = acc[t][0];
            lv[t][1] = acc[t][1];
            lv[t][2] = acc[t][2];
            lv[t][3] = acc[t][3];
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

// Draw of request b at position k, by one wave (all 64 lanes active), in three parts.
//  slab pick:      the slab (8 wave tiles) holding the inverse-CDF point, from the request's
//                  slab partials, and the mass still to cover inside it: merged from the tile
//                  partials in registers (slab_pick_regs, lane l holds tiles [32 l, 32 l + 32),
//                  that is slabs [4 l, 4 l + 4)), or the slab partials the persistent stream
//                  merged with the same arithmetic (slab_pick_coherent, device scope).
//  walk:           the tile of that slab, from its 8 tile partials (walk_pick, walk_slab8).
//  recompute:      that tile's logits rebuilt with the MFMA sequence of the stream, from the
//                  tile's W2 fragments, the W1 row of x_{k-1} and U_k, then the in-tile
//                  rescan: slab_recompute (the draw launch, operands from recompute_loads;
//                  `rowv` holds the tile's logits) or batch_recompute (the persistent form).
// slab_finish writes the token (COH: at device scope), p(token) and lse.
constexpr int kSlabRegs = kSelRegs / kSlabWaves;     // slabs per lane (256 slabs at most)

// The slab pick from tile partials in registers (lane l holds tiles [32 l, 32 l + 32)): the
// slab partials merged per lane, then the pick over slabs.
__device__ __forceinline__ TilePick slab_pick_regs(const float2 (&p)[kSelRegs], float u) {
    float2 sp[kSlabRegs];
#pragma unroll
    for (int j = 0; j < kSlabRegs; ++j) {
        float2 q[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) q[w] = p[8 * j + w];
        sp[j] = merge_slab8(q);
    }
    return pick_tile<kSlabRegs>(sp, u);
}

// The slab pick from the slab partials the persistent stream published (device scope).
__device__ __forceinline__ TilePick slab_pick_coherent(const SlabArgs& a, int b, int k) {
    const int lane = threadIdx.x & (kWave - 1);
    const float2* P = a.spart + static_cast<long long>(b) * a.G;
    float2 sp[kSlabRegs];
#pragma unroll
    for (int j = 0; j < kSlabRegs; ++j) {
        const int i = lane * kSlabRegs + j;
        sp[j] = (i < a.G) ? load_part<true>(P + i) : make_float2(-INFINITY, 0.0f);
    }
    return pick_tile<kSlabRegs>(sp, a.u[static_cast<long long>(b) * a.gamma + k]);
}

// The tile of the picked slab sp.tile from its 8 tile partials p8 (walk_slab8): the global
// tile index and the mass left inside it.
__device__ __forceinline__ TilePick walk_pick(const TilePick& sp, const float2 (&p8)[8]) {
    const SlabWalk w = walk_slab8(p8, sp.m, sp.tprime);
    TilePick r = sp;
    r.tile = w.w < 0 ? -1 : sp.tile * kSlabWaves + w.w;
    r.tprime = w.tprime;
    return r;
}

// The same, with the 8 partials read from the tile partials in memory.
__device__ __forceinline__ TilePick slab_walk(const SlabArgs& a, int b, const TilePick& sp) {
    const float4* P4 = reinterpret_cast<const float4*>(a.part + static_cast<long long>(b) * a.ntw +
                                                       sp.tile * kSlabWaves);
    float2 p8[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float4 v = P4[t];
        p8[2 * t] = make_float2(v.x, v.y);
        p8[2 * t + 1] = make_float2(v.z, v.w);
    }
    return walk_pick(sp, p8);
}

template <bool COH>
__device__ __forceinline__ void slab_finish(const SlabArgs& a, int b, int k, int tok, float q, float lse) {
    if ((threadIdx.x & (kWave - 1)) != 0) return;
    const long long o = static_cast<long long>(b) * a.gamma + k;
    if (COH) store_coherent(a.x_out + o, tok);
    else a.x_out[o] = tok;
    if (a.q_out) a.q_out[o] = q;
    if (a.lse_out) a.lse_out[o] = lse;
}

// The global operands of a tile's recompute, loaded before the MFMAs: U_k at the lane's
// columns (lanes of request column 0) and the W1 row of the previous token (every column).
template <int NT>
struct RecomputeIn {
    float4 u4[NT];
    uint4 hv[kKS];
};

template <int NT>
__device__ __forceinline__ void recompute_loads(const SlabArgs& a, int b, int k, int tk, int tile,
                                                RecomputeIn<NT>& in) {
    using S = Slab<NT>;
    const int lane = threadIdx.x & (kWave - 1);
    const int rq = lane & 15, cg = lane >> 4;
    if (tk < 0 || tk >= a.V) tk = 0;
    const long long cw = static_cast<long long>(tile) * S::WC;
    const float* urow = a.U + (static_cast<long long>(b) * a.gamma + k) * a.V;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const long long col = cw + 16 * t + 4 * cg;
        in.u4[t] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (rq == 0 && col < a.V) in.u4[t] = *reinterpret_cast<const float4*>(urow + col);
    }
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
        const int rank = 32 * s + 8 * cg;
        in.hv[s] = make_uint4(0u, 0u, 0u, 0u);
        if (rank < a.r) in.hv[s] = *reinterpret_cast<const uint4*>(a.W1 + static_cast<long long>(tk) * a.r + rank);
    }
}

template <int NT>
__device__ __forceinline__ void slab_recompute(const SlabArgs& a, int b, int k, const TilePick& tp,
                                               const bf16x8 (&w2f)[NT][kKS],
                                               const RecomputeIn<NT>& in, float* rowv) {
    using S = Slab<NT>;
    constexpr int CPL = (S::WC + kWave - 1) / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int rq = lane & 15, cg = lane >> 4;
    const long long cw = static_cast<long long>(tp.tile) * S::WC;
    f32x4 acc[NT];                                   // from U_k, as in the stream
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{in.u4[t].x, in.u4[t].y, in.u4[t].z, in.u4[t].w};
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
        // the W1 row of the previous token in every one of the 16 request columns
        const bf16x8 hf = __builtin_bit_cast(bf16x8, in.hv[s]);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2f[t][s], hf, acc[t], 0, 0, 0);
    }
    if (rq == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bool ok = cw + 16 * t + 4 * cg < a.V;
            float* rv = rowv + 16 * t + 4 * cg;
            rv[0] = ok ? acc[t][0] : -INFINITY;
            rv[1] = ok ? acc[t][1] : -INFINITY;
            rv[2] = ok ? acc[t][2] : -INFINITY;
            rv[3] = ok ? acc[t][3] : -INFINITY;
        }
    }
    wait_lgkm0();                                     // the row is in LDS
    __builtin_amdgcn_wave_barrier();
    float lv[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane * CPL + j;
        lv[j] = (c < S::WC) ? rowv[c] : -INFINITY;
    }
    const DrawOut none{nullptr, nullptr, nullptr, false};
    const int tok = rescan_values<CPL>(lv, cw + lane * CPL, static_cast<int>(cw), tp.m, tp.lse,
                                       tp.tprime, none);
    const int rel = tok - static_cast<int>(cw), owner = rel / CPL, jj = rel - owner * CPL;
    float mine = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
        if (j == jj) mine = lv[j];
    const float lx = wave_bcast(mine, owner);
    slab_finish<false>(a, b, k, tok, __expf(lx - tp.lse), tp.lse);
}

// Draws of up to kBatch requests whose chosen tile is this wave's (the persistent form): one
// MFMA pass rebuilds the tile for all of them, request j in B column j (a column of the
// result depends only on its own operands, so each is bit-identical to the single-request
// recompute), and the in-tile rescans follow one request at a time from `rowb`
// ([kBatch][WC] floats of this wave's LDS). bb, pk: the requests and their picks (uniform);
// `breq` (kBatch ints of this wave's LDS) hands each lane its column's request.
constexpr int kBatch = 4;

template <int NT>
__device__ __forceinline__ void batch_recompute(const SlabArgs& a, int k, int n, const int (&bb)[kBatch],
                                                const TilePick (&pk)[kBatch], const int* stok,
                                                const bf16x8 (&w2f)[NT][kKS], float* rowb, int* breq) {
    using S = Slab<NT>;
    constexpr int CPL = (S::WC + kWave - 1) / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int rq = lane & 15, cg = lane >> 4;
    const int i = rq < n ? rq : 0;                    // request of this lane's B / C column
    if (lane < kBatch) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            if (lane == j) breq[j] = bb[j];
    }
    wait_lgkm0();
    __builtin_amdgcn_wave_barrier();
    const int rb = breq[i];
    int tk = stok[rb];
    if (tk < 0 || tk >= a.V) tk = 0;
    const long long cw = static_cast<long long>(pk[0].tile) * S::WC;
    const float* urow = a.U + (static_cast<long long>(rb) * a.gamma + k) * a.V;
    float4 u4[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const long long col = cw + 16 * t + 4 * cg;
        u4[t] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (rq < n && col < a.V) u4[t] = *reinterpret_cast<const float4*>(urow + col);
    }
    f32x4 acc[NT];                                   // from U_k, as in the stream
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{u4[t].x, u4[t].y, u4[t].z, u4[t].w};
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
        // the W1 row of request i's previous token in column i
        const int rank = 32 * s + 8 * cg;
        uint4 hv = make_uint4(0u, 0u, 0u, 0u);
        if (rank < a.r) hv = *reinterpret_cast<const uint4*>(a.W1 + static_cast<long long>(tk) * a.r + rank);
        const bf16x8 hf = __builtin_bit_cast(bf16x8, hv);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2f[t][s], hf, acc[t], 0, 0, 0);
    }
    if (rq < n) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bool ok = cw + 16 * t + 4 * cg < a.V;
            float* rv = rowb + rq * S::WC + 16 * t + 4 * cg;
            rv[0] = ok ? acc[t][0] : -INFINITY;
            rv[1] = ok ? acc[t][1] : -INFINITY;
            rv[2] = ok ? acc[t][2] : -INFINITY;
            rv[3] = ok ? acc[t][3] : -INFINITY;
        }
    }
    wait_lgkm0();                                     // the rows are in LDS
    __builtin_amdgcn_wave_barrier();
    const DrawOut none{nullptr, nullptr, nullptr, false};
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {                // static indices keep bb, pk in registers
        if (j >= n) break;
        float lv[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
            const int c = lane * CPL + q;
            lv[q] = (c < S::WC) ? rowb[j * S::WC + c] : -INFINITY;
        }
        const TilePick tp = pk[j];
        const int tok = rescan_values<CPL>(lv, cw + lane * CPL, static_cast<int>(cw), tp.m, tp.lse,
                                           tp.tprime, none);
        const int rel = tok - static_cast<int>(cw), owner = rel / CPL, jj = rel - owner * CPL;
        float mine = 0.0f;
#pragma unroll
        for (int q = 0; q < CPL; ++q)
            if (q == jj) mine = lv[q];
        const float lx = wave_bcast(mine, owner);
        slab_finish<true>(a, bb[j], k, tok, __expf(lx - tp.lse), tp.lse);
    }
    __builtin_amdgcn_wave_barrier();                  // rowb may be rewritten by the next batch
}

// One position: stream launch (W2 staged once per launch; the logits stored when LOUT).
template <int NT, bool LOUT>
__global__ __launch_bounds__(kSlabThreads)
void draft_slab_step(SlabArgs a, int k) {
    using S = Slab<NT>;
    constexpr int UB = ubuf_bytes<NT>();
    static_assert(kSlabWaves * S::Stage <= UB + 2 * kHBuf, "W2 staging fits in U2 + H2 + H3");
    extern __shared__ __align__(16) char sm[];
    const int tid = threadIdx.x, wave = tid / kWave;
    const long long cw = static_cast<long long>(blockIdx.x) * S::SW + wave * S::WC;
    int* stok = reinterpret_cast<int*>(sm + tok_off<NT>());
    const int32_t* tok = k ? a.x_out + (k - 1) : a.x0;
    const long long stride = k ? a.gamma : 1;
    for (int b = tid; b < a.B; b += kSlabThreads) {
        const int t = tok[b * stride];
        stok[b] = (t >= 0 && t < a.V) ? t : -1;       // dead request: no bias, -inf logits
    }
    __syncthreads();
    // the first two groups' loads go out before the W2 staging (whose area they do not use)
    const int ng = (a.B + kGrp - 1) / kGrp;
    for (int g = 0; g < 2 && g < ng; ++g) issue_group<NT>(a, k, g, sm, stok);
    bf16x8 w2f[NT][kKS];
    load_w2_frags<NT, 4, 1>(w2f, a.W2, a.V, a.r, cw, sm + 2 * UB + 2 * kHBuf + wave * S::Stage);
    wait_lgkm0();
    __syncthreads();                                  // every wave is done with the staging area
    slab_stream<NT, LOUT, false>(a, k, a.L, w2f, sm, stok, ng < 2 ? ng : 2);
}

// One position: draw launch, one workgroup (one wave) per request; every W2 load of the
// chosen tile is in flight at once (one LDS staging slot per rank chunk).
template <int NT>
__global__ __launch_bounds__(kWave)
void draft_slab_select(SlabArgs a, int k) {
    using S = Slab<NT>;
    __shared__ __align__(16) char stg[kKS * S::Stage];
    __shared__ float rowv[S::WC];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int tk = k ? a.x_out[static_cast<long long>(b) * a.gamma + k - 1] : a.x0[b];
    // the request's tile partials, lane l holding tiles [32 l, 32 l + 32) = slabs [4 l, 4 l + 4)
    float2 p[kSelRegs];
    const float4* P4 = reinterpret_cast<const float4*>(a.part + static_cast<long long>(b) * a.ntw);
#pragma unroll
    for (int t = 0; t < kSelRegs / 2; ++t) {
        const int i = lane * kSelRegs + 2 * t;        // ntw is a multiple of 8: slabs are whole
        float4 v = make_float4(-INFINITY, 0.0f, -INFINITY, 0.0f);
        if (i < a.ntw) v = P4[i / 2];
        p[2 * t] = make_float2(v.x, v.y);
        p[2 * t + 1] = make_float2(v.z, v.w);
    }
    const TilePick sp = slab_pick_regs(p, a.u[static_cast<long long>(b) * a.gamma + k]);
    if (sp.tile < 0) {
        slab_finish<false>(a, b, k, -1, 0.0f, -INFINITY);
        return;
    }
    // the picked slab's 8 tile partials, from the lane that holds them
    const int owner = sp.tile / kSlabRegs, jj = sp.tile - owner * kSlabRegs;
    float2 p8[8];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        float2 mine = p[w];
#pragma unroll
        for (int j = 1; j < kSlabRegs; ++j)
            if (j == jj) mine = p[8 * j + w];
        p8[w] = make_float2(wave_bcast(mine.x, owner), wave_bcast(mine.y, owner));
    }
    const TilePick tp = walk_pick(sp, p8);
    if (tp.tile < 0) {
        slab_finish<false>(a, b, k, -1, 0.0f, -INFINITY);
        return;
    }
    // the recompute's U and W1 loads go out before the W2 fragments', so both are in flight
    RecomputeIn<NT> in;
    recompute_loads<NT>(a, b, k, tk, tp.tile, in);
    bf16x8 w2f[NT][kKS];
    load_w2_frags<NT, kKS, kKS>(w2f, a.W2, a.V, a.r, static_cast<long long>(tp.tile) * S::WC, stg);
    slab_recompute<NT>(a, b, k, tp, w2f, in, rowv);
}

// All positions in one launch (see the file comment). Per position k three flag rows,
// [f][k][g] for f = 0, 1, 2: workgroup g's slab partials, its slab picks, its tokens
// published. The draw is split so that no workgroup needs a second copy of W2: workgroup g
// picks the slab of its share of the requests (b = g, g + G, ...); the workgroup of a
// picked slab walks its 8 tile partials, and the wave that holds the chosen tile in
// registers recomputes that tile's logits and draws the token.
template <int NT, bool LOUT>
__global__ __launch_bounds__(kSlabThreads)
void draft_slab_resident(SlabArgs a) {
    using S = Slab<NT>;
    constexpr int UB = ubuf_bytes<NT>();
    static_assert(kSlabWaves * S::Stage <= UB + 2 * kHBuf, "W2 staging fits in U2 + H2 + H3");
    extern __shared__ __align__(16) char sm[];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int slab = blockIdx.x, G = a.G;
    // set by a wave whose flag wait ran out; after the tokens (the launch adds kResidentExtra)
    volatile int& gave_up = *reinterpret_cast<int*>(sm + tok_off<NT>() + 4 * a.B);
    const long long cw = static_cast<long long>(slab) * S::SW + wave * S::WC;
    const int my_tile = slab * kSlabWaves + wave;
    const int ng = (a.B + kGrp - 1) / kGrp, npre = ng < 3 ? ng : 3;
    int* stok = reinterpret_cast<int*>(sm + tok_off<NT>());
    // the draw's LDS lies in the W1 row slots, idle between streams (the U slots then hold the
    // next position's first groups): the picked slabs in H0 + H1, each wave's batch of logit
    // rows in H2 + H3
    static_assert(kSlabWaves * (kBatch * (S::WC + 1) + kWave) * 4 <= 2 * kHBuf, "draw LDS fits in H2 + H3");
    int* pslab = reinterpret_cast<int*>(sm + hbuf_off<NT>(0));
    float* rowb = reinterpret_cast<float*>(sm + hbuf_off<NT>(2)) + wave * kBatch * S::WC;
    int* breq = reinterpret_cast<int*>(sm + hbuf_off<NT>(2) + kSlabWaves * kBatch * S::WC * 4) +
                wave * kBatch;
    int* dlist = reinterpret_cast<int*>(sm + hbuf_off<NT>(2) + kSlabWaves * kBatch * (S::WC + 1) * 4) +
                 wave * kWave;
    if (tid == 0) gave_up = 0;
    // The launch resets its own position flags (see the single-request draft): tid 0 of every
    // workgroup reads the call counter E; workgroup 0 fills the flags with the sentinel while
    // W2 loads and then stores the ready word F = ready_word(E); no workgroup publishes its
    // first flag before it has seen that F; workgroup 0 advances E at the end, once every
    // workgroup has published all its flags of the last position.
    unsigned long long e0 = 0, key = 0;
    if (tid == 0) {
        e0 = load_coherent(a.epoch);
        key = ready_word(e0);
    }
    if (slab == 0) {
        for (long long i = tid; i < 3ll * a.gamma * G; i += kSlabThreads) store_coherent(a.flags + i, kEmpty);
        if (tid == 0) __hip_atomic_store(a.status, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    bf16x8 w2f[NT][kKS];
    load_w2_frags<NT, 4, 1>(w2f, a.W2, a.V, a.r, cw, sm + 2 * UB + 2 * kHBuf + wave * S::Stage);
    wait_lgkm0();
    __syncthreads();                                  // every wave is done with the staging area
    if (slab == 0) {                                  // the flags are reset: publish F
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) store_coherent(a.epoch + 1, key);
    }
    // U loads of the first groups of a position (they do not depend on the tokens)
    auto prefetch_u = [&](int kk) {
        for (int g = 0; g < npre; ++g) issue_group<NT, 1>(a, kk, g, sm, stok);
    };
    prefetch_u(0);

    auto flag_row = [&](int f, int k) { return a.flags + (static_cast<long long>(f) * a.gamma + k) * G; };
    // wave 0 waits until all G flags of `row` are set (false after the spin bound); the other
    // waves wait at the workgroup barrier that follows, so each workgroup polls with one wave
    auto wait_flags = [&](const unsigned long long* row) {
        if (gave_up) return false;                    // this workgroup could not publish
        for (unsigned n = 0;; ++n) {
            bool missing = false;
            for (int i = lane; i < G; i += kWave) missing |= load_coherent(row + i) == kEmpty;
            if (!__any(missing)) return true;
            if (n > a.spin) return false;
            __builtin_amdgcn_s_sleep(1);
        }
    };
    // publishes flag (f, k) of this workgroup once every thread's stores are visible
    auto publish = [&](int f, int k) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            if (f == 0 && k == 0) {                   // the flags must be reset first
                for (unsigned n = 0; load_coherent(a.epoch + 1) != key; ++n) {
                    if (n > a.spin) {
                        gave_up = 1;
                        return;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            store_coherent(flag_row(f, k) + slab, 0ull);
        }
    };
    int k = 0;
    int kfail = a.gamma;              // first position whose draws may be missing after a give-up
    for (; k < a.gamma; ++k) {
        // tokens x_{k-1} of every request: x0, or the previous position's draws
        if (k > 0 && wave == 0 && !wait_flags(flag_row(2, k - 1)) && lane == 0) gave_up = 1;
        __syncthreads();                              // also: every wave is done with the draw LDS
        if (gave_up) {
            // a drawer of position k - 1 may have given up before drawing it
            kfail = k > 0 ? k - 1 : 0;
            break;
        }
        for (int b = tid; b < a.B; b += kSlabThreads) {
            const int t = k ? load_coherent(a.x_out + static_cast<long long>(b) * a.gamma + k - 1) : a.x0[b];
            stok[b] = (t >= 0 && t < a.V) ? t : -1;
        }
        __syncthreads();
        slab_stream<NT, LOUT, true>(a, k, LOUT ? a.L + static_cast<long long>(k) * a.V : nullptr, w2f, sm,
                                    stok, 0);
        // slab partials of every request for this slab, merged from the tile partials this
        // workgroup's waves stored (visible within the workgroup after the barrier)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int b = tid; b < a.B; b += kSlabThreads) {
            const float4* P4 = reinterpret_cast<const float4*>(a.part + static_cast<long long>(b) * a.ntw +
                                                               slab * kSlabWaves);
            float2 p[8];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float4 v = P4[t];
                p[2 * t] = make_float2(v.x, v.y);
                p[2 * t + 1] = make_float2(v.z, v.w);
            }
            store_coherent(a.spart + static_cast<long long>(b) * G + slab, merge_slab8(p));
        }
        publish(0, k);

        // slab picks of this workgroup's requests, one wave per request
        if (wave == 0 && !wait_flags(flag_row(0, k)) && lane == 0) gave_up = 1;
        __syncthreads();
        if (gave_up) break;
        for (int b = slab + G * wave; b < a.B; b += G * kSlabWaves) {
            const TilePick tp = slab_pick_coherent(a, b, k);
            if (lane == 0) {
                unsigned long long* rec = reinterpret_cast<unsigned long long*>(a.picks + b);
                store_coherent(rec, __builtin_bit_cast(unsigned long long, make_float2(__int_as_float(tp.tile), tp.m)));
                store_coherent(rec + 1, __builtin_bit_cast(unsigned long long, make_float2(tp.lse, tp.tprime)));
            }
            if (tp.tile < 0) slab_finish<true>(a, b, k, -1, 0.0f, -INFINITY);
        }
        publish(1, k);

        // requests picked in this slab: every wave walks the slab's 8 tile partials (written
        // by this workgroup), and the wave holding the chosen tile in registers draws. The
        // picked slabs of all requests are staged in LDS after the waves' logit rows.
        if (wave == 0 && !wait_flags(flag_row(1, k)) && lane == 0) gave_up = 1;
        __syncthreads();
        if (gave_up) break;
        for (int b = tid; b < a.B; b += kSlabThreads)
            pslab[b] = static_cast<int>(load_coherent(reinterpret_cast<const unsigned long long*>(a.picks + b)));
        __syncthreads();
        // the requests picked in this slab, compacted into this wave's list (up to 64 at a
        // time); lane j walks list entry j (its record and the slab's 8 tile partials, all
        // lanes' loads in flight together), then this wave draws those whose tile it holds,
        // kBatch at a time
        auto process = [&](int m) {
            const bool here = lane < m;
            const int b = here ? dlist[lane] : 0;
            TilePick tp;
            tp.tile = -1;
            if (here) {
                const unsigned long long* rec = reinterpret_cast<const unsigned long long*>(a.picks + b);
                const float2 r0 = __builtin_bit_cast(float2, load_coherent(rec));
                const float2 r1 = __builtin_bit_cast(float2, load_coherent(rec + 1));
                TilePick sp;
                sp.tile = slab;
                sp.m = r0.y;
                sp.lse = r1.x;
                sp.tprime = r1.y;
                tp = slab_walk(a, b, sp);
                if (tp.tile < 0 && wave == 0) {       // no tile with mass: the request is dead
                    const long long o = static_cast<long long>(b) * a.gamma + k;
                    store_coherent(a.x_out + o, -1);
                    if (a.q_out) a.q_out[o] = 0.0f;
                    if (a.lse_out) a.lse_out[o] = -INFINITY;
                }
            }
            unsigned long long hit = __ballot(here && tp.tile == my_tile);
            while (hit) {
                int bb[kBatch];
                TilePick pk[kBatch];
                int n = 0;
#pragma unroll
                for (int j = 0; j < kBatch; ++j) {
                    bb[j] = dlist[0];
                    pk[j] = TilePick{my_tile, 0.0f, 0.0f, 0.0f};
                    if (hit) {
                        const int f = __ffsll(static_cast<long long>(hit)) - 1;
                        hit &= hit - 1;
                        bb[j] = __builtin_amdgcn_readlane(b, f);
                        pk[j].m = wave_bcast(tp.m, f);
                        pk[j].lse = wave_bcast(tp.lse, f);
                        pk[j].tprime = wave_bcast(tp.tprime, f);
                        n = j + 1;
                    }
                }
                batch_recompute<NT>(a, k, n, bb, pk, stok, w2f, rowb, breq);
            }
            __builtin_amdgcn_wave_barrier();          // dlist may be refilled
        };
        int m = 0;                                    // wave-uniform length of dlist
        for (int base = 0; base < a.B; base += kWave) {
            const int b = base + lane;
            const unsigned long long hit = __ballot(b < a.B && pslab[min(b, a.B - 1)] == slab);
            const int cnt = __popcll(hit);
            if (m + cnt > kWave) {
                process(m);
                m = 0;
            }
            if ((hit >> lane) & 1ull) dlist[m + __popcll(hit & ((1ull << lane) - 1ull))] = b;
            m += cnt;
            wait_lgkm0();
            __builtin_amdgcn_wave_barrier();
        }
        if (m > 0) process(m);
        publish(2, k);
        if (k + 1 < a.gamma) prefetch_u(k + 1);
    }
    __builtin_amdgcn_s_waitcnt(0);                    // no load in flight at exit
    // every workgroup has read E (each published the flags workgroup 0 waited for), or the
    // launch gave up; E moves on either way
    if (slab == 0 && tid == 0) store_coherent(a.epoch, e0 + 1);
    if (gave_up && tid == 0) __hip_atomic_fetch_add(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (gave_up) {                                    // this workgroup's requests: -1 from kfail on
        if (kfail > k) kfail = k;
        for (long long i = tid; i < static_cast<long long>(a.B) * a.gamma; i += kSlabThreads) {
            const int b = static_cast<int>(i / a.gamma), kk = static_cast<int>(i % a.gamma);
            if (b % G != slab || kk < kfail) continue;
            a.x_out[i] = -1;
            if (a.q_out) a.q_out[i] = 0.0f;
            if (a.lse_out) a.lse_out[i] = -INFINITY;
        }
    }
}

size_t slab_lds_bytes(int nt, int B) {
    return 3 * static_cast<size_t>(kGrp) * kSlabWaves * 16 * nt * 4 + 4 * kHBuf + 4 * static_cast<size_t>(B);
}
constexpr size_t kResidentExtra = 16;     // the resident launch's give-up word, after the tokens

struct SlabFit {
    int cus = -1;
    int occupancy[2][kMaxNT + 1] = {{-1, -1, -1, -1, -1, -1}, {-1, -1, -1, -1, -1, -1}};
};

template <int NT, bool LOUT>
int resident_occupancy(size_t smem) {
    int occ = 0;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&draft_slab_resident<NT, LOUT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem)) != hipSuccess)
        return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, draft_slab_resident<NT, LOUT>, kSlabThreads, smem) !=
        hipSuccess)
        return 0;
    return occ;
}

template <bool LOUT>
int resident_occupancy_nt(int nt, size_t smem) {
    switch (nt) {
        case 1: return resident_occupancy<1, LOUT>(smem);
        case 2: return resident_occupancy<2, LOUT>(smem);
        case 3: return resident_occupancy<3, LOUT>(smem);
        case 4: return resident_occupancy<4, LOUT>(smem);
        default: return resident_occupancy<5, LOUT>(smem);
    }
}

// Whether every slab workgroup of the resident launch (with or without the logits output)
// can be on the device at once (queried with the largest LDS the path uses, so smaller
// batches fit as well).
bool resident_fits(int V, bool L_out) {
    thread_local SlabFit cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    SlabFit& f = cache[dev];
    if (f.cus < 0 && hipDeviceGetAttribute(&f.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    const int nt = slab_nt(V);
    int& occ = f.occupancy[L_out ? 1 : 0][nt];
    if (occ < 0) {
        const size_t smem = static_cast<size_t>(kLdsBytes);
        occ = L_out ? resident_occupancy_nt<true>(nt, smem) : resident_occupancy_nt<false>(nt, smem);
    }
    return f.cus > 0 && occ >= 1 && slab_count(V) <= f.cus * occ;
}

}  // namespace

// The persistent form: its LDS (with the B picked slabs in H0 + H1) fits, and every slab
// workgroup can be on the device at once. It writes the logits too when they are wanted.
bool draft_slab_one_launch(int B, int V, bool L_out) {
    const int nt = slab_nt(V);
    const bool lds_ok = slab_lds_bytes(nt, B) + kResidentExtra <= static_cast<size_t>(kLdsBytes) &&
                        4 * static_cast<size_t>(B) <= 2 * static_cast<size_t>(kHBuf);
    return lds_ok && resident_fits(V, L_out);
}

namespace {

template <int NT>
hipError_t launch_nt(const DraftCall& c, hipStream_t st) {
    SlabArgs a;
    a.B = c.B; a.V = c.V; a.r = c.r; a.gamma = c.gamma;
    a.ntw = draft_slab_tiles(c.V);
    a.G = slab_count(c.V);
    a.U = c.U;
    a.W1 = static_cast<const uint16_t*>(c.W1);
    a.W2 = static_cast<const uint16_t*>(c.W2);
    a.x0 = c.x0; a.u = c.u;
    a.x_out = c.x_out; a.q_out = c.q_out; a.lse_out = c.lse_out;
    a.L = nullptr;
    a.L_bstride = c.L_bstride;
    a.flags = reinterpret_cast<unsigned long long*>(c.slots);
    a.epoch = nullptr;
    a.status = c.status;
    a.spin = c.spin;
    // resident: the second partial buffer holds the picks [B] and the slab partials [B][G]
    a.picks = reinterpret_cast<float4*>(c.part[1]);
    a.spart = c.part[1] + 2 * static_cast<long long>(c.B);
    const size_t smem = slab_lds_bytes(NT, c.B);
    const dim3 grid(static_cast<unsigned>(a.G));
    if (!c.per_position && draft_slab_one_launch(c.B, c.V, c.L_out)) {
        a.epoch = a.flags + 3ll * c.gamma * a.G;      // after the flags
        a.part = c.part[0];
        if (c.L_out) {
            a.L = c.L[0];                             // the caller's [B][gamma][V]: L[k] = L[0] + k V
            hipLaunchKernelGGL((draft_slab_resident<NT, true>), grid, dim3(kSlabThreads), smem + kResidentExtra,
                               st, a);
        } else {
            hipLaunchKernelGGL((draft_slab_resident<NT, false>), grid, dim3(kSlabThreads), smem + kResidentExtra,
                               st, a);
        }
        return hipGetLastError();
    }
    for (int k = 0; k < c.gamma; ++k) {
        a.L = c.L_out ? c.L[k] : nullptr;
        a.part = c.part[k & 1];
        if (c.L_out)
            hipLaunchKernelGGL((draft_slab_step<NT, true>), grid, dim3(kSlabThreads), smem, st, a, k);
        else
            hipLaunchKernelGGL((draft_slab_step<NT, false>), grid, dim3(kSlabThreads), smem, st, a, k);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(draft_slab_select<NT>, dim3(static_cast<unsigned>(c.B)), dim3(kWave), 0, st, a, k);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

int draft_slab_tiles(int V) { return slab_count(V) * kSlabWaves; }

// position flags [3][gamma][G], then the call counter and the ready word
size_t draft_slab_flag_bytes(int V, int gamma) {
    return (3 * static_cast<size_t>(gamma) * slab_count(V) + 2) * sizeof(unsigned long long);
}

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
