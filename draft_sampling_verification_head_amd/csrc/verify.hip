// Rejection-sampling verification and TV-label kernels (gfx950).
//
// [P1] = "大模型推理加速的系统级工程：DeepSeek V4-Pro DSpark 推测解码方案深度解析与开源工具链
// DeepSpec" (Best Partners TV); [P3] = "DSpark Speculative Decoding" (concept note).
//
// Every vocabulary row is cut into chunks of 8192 logits, one workgroup per chunk, so even a
// single request spreads over the whole chip and every pass is one HBM sweep. Per-row
// results are combined by the next kernel on the stream (kernel boundaries order the
// writes; no workgroup needs a device-scope fence).
//
// row_stats      - [P1] section "大模型推理的显存瓶颈与推测解码的演进逻辑": the acceptance test needs
//                  normalised probabilities; every verified row gets chunk (max, sum exp)
//                  partials.
// verify_chunks  - per request and chunk: merges the row partials into lse (chunk order),
//                  runs the acceptance test of every verified position
//                  (log u < log p_t(x) - log p_d(x); first rejection from a ballot) and sums the
//                  chunk's mass under the final law: the residual max(0, p_t - p_d) at the first
//                  rejection, or the bonus row p_t when all are kept ([P3] intro). Chunk 0 also
//                  publishes n and the normalisers.
// verify_select  - per request: finds the chunk holding u * total in chunk order and rescans
//                  it in token order for the emitted token.
// tv_chunks / tv_merge - [P3] "Confidence-Scheduled Verification": c* = sum_v min(p_d, p_t),
//                  summed per chunk as exp(min(l_d - lse_d, l_t - lse_t)), then in chunk order.
// Target rows are flattened with per-request offsets ([P1] section "极致的工程实现与内核优化").
#include "common.h"
#include "kernels.h"
#include "rows.h"

// Every product and sum below rounds on its own (fused only where written as fmaf), so the
// verify's forms (one launch, sweep, chunked kernels) form each probability, mass and running
// sum with the same roundings whatever the contraction choices at each site: they agree bit
// for bit by construction.
#pragma clang fp contract(off)

namespace dspark {

namespace {

using namespace rows;


// Chunk c of a row in the sweep layout: thread t holds float4 granules t + kThreads*g. The
// chunk's base is wave-uniform and the lane offsets are 32-bit, so each load takes a scalar base
// and one offset register.
template <bool VEC4>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int c, int V,
                                           float (&x)[kPer]) {
    const long long base = static_cast<long long>(c) * kChunk;
    const unsigned t = threadIdx.x;
    const long long left = static_cast<long long>(V) - base;
    const unsigned lim = static_cast<unsigned>(left < kChunk ? left : kChunk);   // logits in the chunk
    if (VEC4) {
        const float4* r4 = reinterpret_cast<const float4*>(row + base);
#pragma unroll
        for (int g = 0; g < kPer / 4; ++g) {
            const unsigned i = t + kThreads * g;
            float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
            if (4 * i < lim) v = r4[i];             // V % 4 == 0: a granule is in or out
            x[4 * g] = v.x; x[4 * g + 1] = v.y; x[4 * g + 2] = v.z; x[4 * g + 3] = v.w;
        }
    } else {
        const float* r = row + base;
#pragma unroll
        for (int g = 0; g < kPer / 4; ++g)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const unsigned v = 4 * (t + kThreads * g) + w;
                x[4 * g + w] = (v < lim) ? r[v] : -INFINITY;
            }
    }
}

// Within a chunk every probability is formed from the chunk's own maximum M: the term
// e = exp(x - M) gives both the chunk's (max, sum exp) partial and, once the row's lse is known,
// the probability p = e * exp(M - lse). So one exponential per logit serves the normalisers, the
// TV sums and the final-draw masses, and every kernel that forms a probability of a chunk forms
// the same value.

// The maximum of a chunk held kPer values per thread (the same in every thread): within each
// wave by DPP, then over the waves. red holds kWaves floats, not written again before a later
// barrier.
__device__ __forceinline__ float chunk_max(const float (&x)[kPer], float* red) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    float ml = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPer; ++e) ml = fmaxf(ml, x[e]);
    ml = wave_max_dpp(ml);
    if (lane == 0) red[wave] = ml;
    __syncthreads();
    float mm = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mm = fmaxf(mm, red[w]);
    return mm;
}

// Two chunks' maxima at once (one barrier); red holds [2][kWaves] floats.
__device__ __forceinline__ void chunk_max2(const float (&x)[kPer], const float (&y)[kPer],
                                           float& mx, float& my, float (*red)[kWaves]) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    float ax = -INFINITY, ay = -INFINITY;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        ax = fmaxf(ax, x[e]);
        ay = fmaxf(ay, y[e]);
    }
    ax = wave_max_dpp(ax);
    ay = wave_max_dpp(ay);
    if (lane == 0) {
        red[0][wave] = ax;
        red[1][wave] = ay;
    }
    __syncthreads();
    mx = red[0][0];
    my = red[1][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        mx = fmaxf(mx, red[0][w]);
        my = fmaxf(my, red[1][w]);
    }
}

// e = exp(x - m) of a logit x of a chunk whose max is m, as 2^(x log2(e) - m log2(e)) with
// one fused multiply-add. A chunk whose max is -inf holds only -inf logits: there m log2(e)
// is taken as 0, and every term is 2^-inf = 0.
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ float chunk_ml2(float m) { return (m == -INFINITY) ? 0.0f : m * kLog2e; }
__device__ __forceinline__ float chunk_e2(float x, float ml2) {
    return __builtin_amdgcn_exp2f(fmaf(x, kLog2e, -ml2));
}
__device__ __forceinline__ float chunk_e(float x, float m) { return chunk_e2(x, chunk_ml2(m)); }

// The factor exp(M - lse) that turns a chunk's terms into probabilities; 0 for a row (or chunk)
// with no mass.
__device__ __forceinline__ float chunk_scale(float m, float lse) {
    return (m == -INFINITY || lse == -INFINITY) ? 0.0f : __expf(m - lse);
}

// (max, sum exp(x - max)) of one chunk: the chunk's max, then its terms, summed within each
// wave by DPP and over the waves in wave order. With KEEP the terms replace x. red holds
// [2][kWaves] floats, not written again before a later barrier.
template <bool KEEP>
__device__ __forceinline__ void chunk_ms(float (&x)[kPer], float& m, float& s,
                                         float (*red)[kWaves]) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const float mm = chunk_max(x, red[0]);
    const float ml2 = chunk_ml2(mm);
    float sl = 0.0f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const float v = chunk_e2(x[e], ml2);
        sl += v;
        if (KEEP) x[e] = v;
    }
    sl = wave_sum_dpp(sl);
    if (lane == 0) red[1][wave] = sl;
    __syncthreads();
    float ss = red[1][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) ss += red[1][w];
    m = mm;
    s = ss;
}

// chunk_ms of two rows at once (per row the same arithmetic), one pair of barriers for both;
// red holds [4][kWaves] floats.
template <bool KEEP>
__device__ __forceinline__ void chunk_ms2(float (&x)[kPer], float (&y)[kPer], float& mx,
                                          float& sx, float& my, float& sy, float (*red)[kWaves]) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    float mmx, mmy;
    chunk_max2(x, y, mmx, mmy, red);
    const float lx2 = chunk_ml2(mmx), ly2 = chunk_ml2(mmy);
    float lx = 0.0f, ly = 0.0f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const float vx = chunk_e2(x[e], lx2), vy = chunk_e2(y[e], ly2);
        lx += vx;
        ly += vy;
        if (KEEP) {
            x[e] = vx;
            y[e] = vy;
        }
    }
    lx = wave_sum_dpp(lx);
    ly = wave_sum_dpp(ly);
    if (lane == 0) {
        red[2][wave] = lx;
        red[3][wave] = ly;
    }
    __syncthreads();
    float ssx = red[2][0], ssy = red[3][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        ssx += red[2][w];
        ssy += red[3][w];
    }
    mx = mmx;
    sx = ssx;
    my = mmy;
    sy = ssy;
}

// Workgroup sums of N per-thread values at once: within each wave by DPP, then over the waves
// in wave order, one barrier for all N. scratch holds N kWaves floats, not written again before
// a later barrier. Every chunk-level sum of a probability (TV sums, final-draw masses) goes
// through here, so each kernel that forms such a sum forms the same value.
template <int N>
__device__ __forceinline__ void chunk_sums(float (&v)[N], float* scratch) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = wave_sum_dpp(v[j]);
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < N; ++j) scratch[j * kWaves + wave] = v[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < N; ++j) {
        float t = scratch[j * kWaves];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) t += scratch[j * kWaves + w];
        v[j] = t;
    }
}

__device__ __forceinline__ float chunk_sum(float x, float* scratch) {
    float v[1] = {x};
    chunk_sums<1>(v, scratch);
    return v[0];
}

// ----------------------------------------------------------------------------- row_stats
template <bool VEC4>
__global__ __launch_bounds__(kThreads)
void row_stats_kernel(RowSet rs, int nch, const float* __restrict__ lse_d_in,
                      float2* __restrict__ part) {
    __shared__ float sm[2][kWaves];
    const int G = rs.gamma, S = 2 * G + 1;
    const int c = static_cast<int>(blockIdx.x % static_cast<unsigned>(nch));
    const long long rowid = blockIdx.x / static_cast<unsigned>(nch);        // b * S + slot
    const int slot = static_cast<int>(rowid % S);
    const int b = static_cast<int>(rowid / S);
    const ReqRows q = request_rows(rs, b);
    const float* row;
    bool valid;
    if (slot <= G) {
        valid = q.ok && slot <= q.ell;
        row = rs.Lt + (q.off + slot) * rs.V;
    } else {
        const int k = slot - G - 1;
        valid = q.ok && k < q.ell && !lse_d_in;
        row = rs.Ld + (static_cast<long long>(b) * G + k) * rs.V;
    }
    if (!valid) return;
    float x[kPer];
    load_chunk<VEC4>(row, c, rs.V, x);
    float m, s;
    chunk_ms<false>(x, m, s, sm);
    if (threadIdx.x == 0) part[rowid * nch + c] = make_float2(m, s);
}

// ----------------------------------------------------------------------------- verify
// The final draw's row: its weights are p_t (bonus, or residual with zero mass) or
// max(0, p_t - p_d), formed per chunk from the chunk's terms (see chunk_ms).
struct FinalRow {
    const float* lt;
    const float* ld;
    float lse_t, lse_d;
    int residual;
    float sct, scd;                 // this chunk's exp(M - lse) of the target and draft rows

    // the scales of a chunk whose target and draft maxima are mt and md
    __device__ __forceinline__ void at_chunk(float mt, float md) {
        sct = chunk_scale(mt, lse_t);
        scd = residual ? chunk_scale(md, lse_d) : 0.0f;
    }
    // the weight of a logit pair from its chunk terms e_t, e_d
    __device__ __forceinline__ float weight(float et, float ed) const {
        const float pt = et * sct;
        if (!residual) return pt;
        return fmaxf(pt - ed * scd, 0.0f);
    }
};

// A chunk's terms in place and the scales of fr at that chunk (the chunk's maxima by block
// reductions). red holds [2][kWaves] floats.
__device__ __forceinline__ void chunk_terms(FinalRow& fr, float (&t)[kPer], float (&d)[kPer],
                                            float (*red)[kWaves]) {
    float mt, md = -INFINITY;
    if (fr.residual)
        chunk_max2(t, d, mt, md, red);
    else
        mt = chunk_max(t, red[0]);
    const float t2 = chunk_ml2(mt), d2 = chunk_ml2(md);
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        t[e] = chunk_e2(t[e], t2);
        d[e] = fr.residual ? chunk_e2(d[e], d2) : 0.0f;
    }
    fr.at_chunk(mt, md);
}

// The draw inside one chunk. Thread i holds the weights w of the kPer tokens v0, v0 + 1, ...
// (the threads' runs follow token order). Returns the first token whose running sum exceeds
// tprime or, when rounding leaves tprime at or past the chunk's sum, the last token of positive
// weight (-1 if there is none). The running sum adds a thread's own weights in order to the sum
// of the runs before it: the runs' sums are scanned across the wave by DPP and the wave totals
// added in wave order. fscr holds kWaves floats and iscr 2 * kWaves ints; a caller syncs before
// it reuses them. Called by the whole workgroup.
__device__ __forceinline__ int chunk_pick(const float (&w)[kPer], float tprime, int v0, float* fscr,
                                          int* iscr) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    float local = 0.0f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) local += w[e];
    const float incl = wave_incl_scan_dpp(local);
    const float excl = wave_shr1_dpp(incl);
    if (lane == kWave - 1) fscr[wave] = incl;
    __syncthreads();
    float run = 0.0f;
#pragma unroll
    for (int j = 0; j < kWaves - 1; ++j)
        if (j < wave) run += fscr[j];
    run += excl;
    // bit e of pos: token v0 + e has weight; of past: it has weight and the running sum up to
    // it exceeds tprime (bit masks rather than branches)
    unsigned pos = 0u, past = 0u;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        run += w[e];
        const unsigned bit = 1u << e;
        pos |= (w[e] > 0.0f) ? bit : 0u;
        past |= (run > tprime) ? bit : 0u;
    }
    past &= pos;
    int hit = past ? v0 + __builtin_ctz(past) : INT32_MAX;
    int last = pos ? v0 + 31 - __builtin_clz(pos) : -1;
    static_assert(kPer == 32, "one bit per token of a thread's run");
    hit = wave_min_int_dpp(hit);
    last = wave_max_int_dpp(last);
    if (lane == 0) {
        iscr[wave] = hit;
        iscr[kWaves + wave] = last;
    }
    __syncthreads();
    int h = iscr[0], l = iscr[kWaves];
#pragma unroll
    for (int j = 1; j < kWaves; ++j) {
        h = min(h, iscr[j]);
        l = max(l, iscr[kWaves + j]);
    }
    return h != INT32_MAX ? h : l;
}

template <bool VEC4>
__device__ __forceinline__ float chunk_mass(FinalRow fr, int c, int V, float (*red)[kWaves]) {
    float t[kPer], d[kPer];
    load_chunk<VEC4>(fr.lt, c, V, t);
    if (fr.residual) load_chunk<VEC4>(fr.ld, c, V, d);
    chunk_terms(fr, t, d, red);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) s += fr.weight(t[e], d[e]);
    return s;
}

// Per-request state handed from verify_chunks (chunk 0) to verify_select.
struct ReqState {
    int n;          // accepted count, -1 for a faulty request
    int residual;   // 1: residual draw at position n+1, 0: p_t draw
    float lse_t, lse_d;
};

template <bool VEC4>
__device__ __forceinline__ void verify_chunks_body(const RowSet& rs, int nch, const int32_t* __restrict__ x,
                                   const float2* __restrict__ part, const float* __restrict__ lse_d_in,
                                   const float* __restrict__ u_acc, float* __restrict__ lse_d_out,
                                   float* __restrict__ lse_t_out, float* __restrict__ csum,
                                   ReqState* __restrict__ state, unsigned blk) {
    __shared__ float fscr[kWaves + 1];
    __shared__ float red[2][kWaves];
    __shared__ float s_lt[65], s_ld[64];
    __shared__ int s_n, s_bad;

    const int c = static_cast<int>(blk % static_cast<unsigned>(nch));
    const int b = static_cast<int>(blk / static_cast<unsigned>(nch));
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int G = rs.gamma, V = rs.V;
    const ReqRows q = request_rows(rs, b);
    if (!q.ok) {
        if (c == 0 && tid == 0) state[b] = ReqState{-1, 0, 0.0f, 0.0f};
        if (c == 0) {
            for (int i = tid; i <= G; i += kThreads) {
                if (lse_t_out) lse_t_out[static_cast<long long>(b) * (G + 1) + i] = qnan();
                if (lse_d_out && i < G) lse_d_out[static_cast<long long>(b) * G + i] = qnan();
            }
        }
        return;
    }
    // the acceptance test's inputs do not depend on the normalisers: wave 0 loads the drafted
    // tokens, their uniforms and the two logits at each token before the merges below
    int xk = 0;
    float ltx = 0.0f, ldx = 0.0f, ua = 0.0f;
    if (wave == 0 && lane < q.ell) {
        xk = x[static_cast<long long>(b) * G + lane];
        ua = u_acc[static_cast<long long>(b) * G + lane];
        if (xk >= 0 && xk < V) {
            ltx = rs.Lt[(q.off + lane) * V + xk];
            ldx = rs.Ld[(static_cast<long long>(b) * G + lane) * V + xk];
        }
    }
    // normalisers of the verified rows: each wave merges the partials of some rows
    for (int slot = wave; slot <= q.ell; slot += kWaves) {
        const float v = merge_lse_wave(slot_part(part, b, slot, G, nch), nch);
        if (lane == 0) s_lt[slot] = v;
    }
    for (int k = wave; k < q.ell; k += kWaves) {
        float v;
        if (lse_d_in)
            v = lse_d_in[static_cast<long long>(b) * G + k];
        else
            v = merge_lse_wave(slot_part(part, b, G + 1 + k, G, nch), nch);
        if (lane == 0) s_ld[k] = v;
    }
    __syncthreads();

    // acceptance test for every verified position in one wave (gamma <= 64)
    if (wave == 0) {
        bool bad = false, rej = false;
        const int k = lane;
        if (k < q.ell) {
            if (xk < 0 || xk >= V) {
                bad = true;
            } else {
                const float lst = s_lt[k], lsd = s_ld[k];
                const float lpt = (lst == -INFINITY) ? -INFINITY : ltx - lst;
                const float lpd = (lsd == -INFINITY) ? -INFINITY : ldx - lsd;
                bool acc;
                if (lpd == -INFINITY)
                    acc = lpt > -INFINITY;
                else
                    acc = logf(clamp_uniform(ua)) < lpt - lpd;
                rej = !acc;
            }
        }
        const unsigned long long badm = __ballot(bad);
        const unsigned long long rejm = __ballot(rej);
        if (lane == 0) {
            s_bad = badm != 0ull;
            s_n = rejm ? (__ffsll(static_cast<long long>(rejm)) - 1) : q.ell;
        }
    }
    __syncthreads();
    const int n = s_n;
    if (c == 0) {
        for (int i = tid; i <= G; i += kThreads) {
            if (lse_t_out)
                lse_t_out[static_cast<long long>(b) * (G + 1) + i] = (i <= q.ell) ? s_lt[i] : qnan();
            if (lse_d_out && i < G)
                lse_d_out[static_cast<long long>(b) * G + i] = (i < q.ell) ? s_ld[i] : qnan();
        }
        if (tid == 0)
            state[b] = s_bad ? ReqState{-1, 0, 0.0f, 0.0f}
                             : ReqState{n, n < q.ell ? 1 : 0, s_lt[n], n < q.ell ? s_ld[n] : 0.0f};
    }
    if (s_bad) return;
    FinalRow fr;
    fr.lt = rs.Lt + (q.off + n) * V;
    fr.lse_t = s_lt[n];
    fr.residual = n < q.ell;
    fr.ld = fr.residual ? rs.Ld + (static_cast<long long>(b) * G + n) * V : nullptr;
    fr.lse_d = fr.residual ? s_ld[n] : 0.0f;
    const float s = chunk_sum(chunk_mass<VEC4>(fr, c, V, red), fscr);
    if (tid == 0) csum[static_cast<long long>(b) * nch + c] = s;
}

template <bool VEC4>
__global__ __launch_bounds__(kThreads)
void verify_chunks_kernel(RowSet rs, int nch, const int32_t* __restrict__ x,
                          const float2* __restrict__ part, const float* __restrict__ lse_d_in,
                          const float* __restrict__ u_acc, float* __restrict__ lse_d_out,
                          float* __restrict__ lse_t_out, float* __restrict__ csum,
                          ReqState* __restrict__ state) {
    verify_chunks_body<VEC4>(rs, nch, x, part, lse_d_in, u_acc, lse_d_out, lse_t_out, csum, state,
                             blockIdx.x);
}

// The final draw of a request from its row's chunk masses `cs` (nch of them, in chunk order):
// the chunk that holds u * total, then a rescan of that chunk in token order. When a residual
// rounded to zero mass, the p_t masses of the same row are formed into `cs` and drawn from
// instead. Returns the token (-1 when the row has no mass). Called by a whole workgroup.
template <bool VEC4>
__device__ __forceinline__ int final_draw(int V, int nch, FinalRow fr, float* cs, float uf) {
    __shared__ float fscr[kWaves + 1];
    __shared__ float red[2][kWaves];
    __shared__ int iscr[2 * kWaves];
    __shared__ int s_found;
    __shared__ float s_tprime, s_total;
    const int tid = threadIdx.x;
    for (int pass = 0; pass < 2; ++pass) {
        // chunk totals in chunk order by one wave: lane-strided sums then a butterfly give the
        // total; the search walks the chunks in order with per-lane running sums
        if (tid < kWave) {
            float tot = 0.0f;
            for (int i = tid; i < nch; i += kWave) tot += cs[i];
            tot = wave_sum_dpp(tot);
            const float target = uf * tot;
            int found = -1;
            float tprime = INFINITY, run = 0.0f;
            for (int base = 0; base < nch && found < 0; base += kWave) {
                const int i = base + tid;
                const float v = (i < nch) ? cs[i] : 0.0f;
                const float incl = wave_incl_scan_dpp(v);
                const float excl = wave_shr1_dpp(incl);
                const unsigned long long hit =
                    __ballot((i < nch) && (v > 0.0f) && (run + incl > target));
                if (hit) {
                    const int f = __ffsll(static_cast<long long>(hit)) - 1;
                    found = base + f;
                    tprime = target - (run + wave_bcast(excl, f));
                }
                run += wave_bcast(incl, kWave - 1);
            }
            if (found < 0 && tot > 0.0f) {      // rounding left the target past the end
                int last = -1;
                for (int i = tid; i < nch; i += kWave)
                    if (cs[i] > 0.0f) last = i;
                found = wave_max_int_dpp(last);
                tprime = INFINITY;
            }
            if (tid == 0) {
                s_found = found;
                s_tprime = tprime;
                s_total = tot;
            }
        }
        __syncthreads();
        if (s_total > 0.0f || !fr.residual) break;
        // residual mass rounded to zero: draw from p_t of the same target row instead
        fr.residual = 0;
        for (int i = 0; i < nch; ++i) {
            const float s = chunk_sum(chunk_mass<VEC4>(fr, i, V, red), fscr);
            if (tid == 0) cs[i] = s;
        }
        __syncthreads();
    }

    int z = -1;
    const int found = s_found;
    if (found >= 0) {
        float t[kPer], d[kPer];
        load_chunk_contig<VEC4>(fr.lt, found, V, t);
        if (fr.residual) load_chunk_contig<VEC4>(fr.ld, found, V, d);
        chunk_terms(fr, t, d, red);
        float w[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) w[e] = fr.weight(t[e], d[e]);
        z = chunk_pick(w, s_tprime, found * kChunk + kPer * tid, fscr, iscr);
    }
    return z;
}

template <bool VEC4>
__device__ __forceinline__ void verify_select_body(const RowSet& rs, int nch, const int32_t* __restrict__ x,
                                   const float* __restrict__ u_fin, float* __restrict__ csum,
                                   const ReqState* __restrict__ state, int32_t* __restrict__ n_out,
                                   int32_t* __restrict__ y_out, int b) {
    const int tid = threadIdx.x;
    const int G = rs.gamma, V = rs.V;
    int32_t* y = y_out + static_cast<long long>(b) * (G + 1);
    const ReqState st = state[b];
    if (st.n < 0) {
        for (int i = tid; i <= G; i += kThreads) y[i] = -1;
        if (tid == 0) n_out[b] = -1;
        return;
    }
    const ReqRows q = request_rows(rs, b);
    const int n = st.n;
    FinalRow fr;
    fr.lt = rs.Lt + (q.off + n) * V;
    fr.lse_t = st.lse_t;
    fr.residual = st.residual;
    fr.ld = fr.residual ? rs.Ld + (static_cast<long long>(b) * G + n) * V : nullptr;
    fr.lse_d = st.lse_d;
    const int z = final_draw<VEC4>(V, nch, fr, csum + static_cast<long long>(b) * nch,
                                   clamp_uniform(u_fin[b]));
    for (int i = tid; i <= G; i += kThreads)
        y[i] = (i < n) ? x[static_cast<long long>(b) * G + i] : (i == n ? z : -1);
    if (tid == 0) n_out[b] = n;
}

template <bool VEC4>
__global__ __launch_bounds__(kThreads)
void verify_select_kernel(RowSet rs, int nch, const int32_t* __restrict__ x,
                          const float* __restrict__ u_fin, float* __restrict__ csum,
                          const ReqState* __restrict__ state, int32_t* __restrict__ n_out,
                          int32_t* __restrict__ y_out) {
    verify_select_body<VEC4>(rs, nch, x, u_fin, csum, state, n_out, y_out, blockIdx.x);
}

// ----------------------------------------------------------------------------- TV labels
// lse_d / lse_t given, or merged here from row partials.
template <bool VEC4>
__device__ __forceinline__ void tv_chunks_body(const RowSet& rs, int nch, const float* __restrict__ lse_d,
                               const float* __restrict__ lse_t, const float2* __restrict__ part,
                               float* __restrict__ psum, unsigned blk) {
    __shared__ float fscr[kWaves + 1];
    __shared__ float red[2][kWaves];
    __shared__ float s_lse[2];
    const int G = rs.gamma, V = rs.V, tid = threadIdx.x;
    const int c = static_cast<int>(blk % static_cast<unsigned>(nch));
    const long long pair = blk / static_cast<unsigned>(nch);                 // b * G + k
    const int k = static_cast<int>(pair % G);
    const int b = static_cast<int>(pair / G);
    const ReqRows q = request_rows(rs, b);
    if (!q.ok || k >= q.ell) return;
    if (tid < 2 * kWave) {
        const int w = tid / kWave;   // 0: draft row k, 1: target row k
        float v;
        if (w == 0)
            v = lse_d ? lse_d[pair] : merge_lse_wave(slot_part(part, b, G + 1 + k, G, nch), nch);
        else
            v = lse_t ? lse_t[static_cast<long long>(b) * (G + 1) + k]
                      : merge_lse_wave(slot_part(part, b, k, G, nch), nch);
        if ((tid & (kWave - 1)) == 0) s_lse[w] = v;
    }
    __syncthreads();
    const float a = s_lse[0], cc = s_lse[1];
    float s = 0.0f;
    if (a != -INFINITY && cc != -INFINITY) {     // a zero distribution shares no mass
        float ld[kPer], lt[kPer];
        load_chunk<VEC4>(rs.Ld + pair * V, c, V, ld);
        load_chunk<VEC4>(rs.Lt + (q.off + k) * V, c, V, lt);
        float md, mt;
        chunk_max2(ld, lt, md, mt, red);
        const float scd = chunk_scale(md, a), sct = chunk_scale(mt, cc);
        const float d2 = chunk_ml2(md), t2 = chunk_ml2(mt);
#pragma unroll
        for (int e = 0; e < kPer; ++e) s += fminf(chunk_e2(ld[e], d2) * scd, chunk_e2(lt[e], t2) * sct);
    }
    s = chunk_sum(s, fscr);
    if (tid == 0) psum[pair * nch + c] = s;
}

template <bool VEC4>
__global__ __launch_bounds__(kThreads)
void tv_chunks_kernel(RowSet rs, int nch, const float* __restrict__ lse_d,
                      const float* __restrict__ lse_t, const float2* __restrict__ part,
                      float* __restrict__ psum) {
    tv_chunks_body<VEC4>(rs, nch, lse_d, lse_t, part, psum, blockIdx.x);
}

__device__ __forceinline__ void tv_merge_body(const RowSet& rs, int nch, const float* __restrict__ psum,
                              float* __restrict__ cstar, unsigned blk) {
    const int G = rs.gamma;
    const long long pair = static_cast<long long>(blk) * kWaves + threadIdx.x / kWave;
    if (pair >= static_cast<long long>(rs.B) * G) return;
    const int k = static_cast<int>(pair % G);
    const int b = static_cast<int>(pair / G);
    const ReqRows q = request_rows(rs, b);
    const int lane = threadIdx.x & (kWave - 1);
    float s = 0.0f;
    const bool live = q.ok && k < q.ell;
    if (live)
        for (int i = lane; i < nch; i += kWave) s += psum[pair * nch + i];
    s = wave_sum_dpp(s);
    if (lane == 0) cstar[pair] = live ? s : qnan();
}

__global__ __launch_bounds__(kThreads)
void tv_merge_kernel(RowSet rs, int nch, const float* __restrict__ psum,
                     float* __restrict__ cstar) {
    tv_merge_body(rs, nch, psum, cstar, blockIdx.x);
}

// ----------------------------------------------------------------------------- verify + TV
// One launch for the verify chunk pass and the TV chunk pass (first nch*B workgroups verify,
// the rest sum min(p_d, p_t) per row pair and chunk), one for the final draws and the TV
// merges (first B workgroups draw, the rest merge four row pairs each).
template <bool VEC4>
__global__ __launch_bounds__(kThreads)
void verify_tv_chunks_kernel(RowSet rs, int nch, const int32_t* __restrict__ x,
                             const float2* __restrict__ part, const float* __restrict__ lse_d_in,
                             const float* __restrict__ u_acc, float* __restrict__ lse_d_out,
                             float* __restrict__ lse_t_out, float* __restrict__ csum,
                             ReqState* __restrict__ state, float* __restrict__ psum,
                             unsigned nverify) {
    if (blockIdx.x < nverify)
        verify_chunks_body<VEC4>(rs, nch, x, part, lse_d_in, u_acc, lse_d_out, lse_t_out, csum,
                                 state, blockIdx.x);
    else
        tv_chunks_body<VEC4>(rs, nch, lse_d_in, nullptr, part, psum, blockIdx.x - nverify);
}

template <bool VEC4>
__global__ __launch_bounds__(kThreads)
void verify_tv_select_kernel(RowSet rs, int nch, const int32_t* __restrict__ x,
                             const float* __restrict__ u_fin, float* __restrict__ csum,
                             const ReqState* __restrict__ state, int32_t* __restrict__ n_out,
                             int32_t* __restrict__ y_out, const float* __restrict__ psum,
                             float* __restrict__ cstar) {
    if (blockIdx.x < static_cast<unsigned>(rs.B))
        verify_select_body<VEC4>(rs, nch, x, u_fin, csum, state, n_out, y_out, blockIdx.x);
    else
        tv_merge_body(rs, nch, psum, cstar, blockIdx.x - rs.B);
}

// ----------------------------------------------------------------------------- one sweep
// Verify and TV labels in one pass over the rows. A unit is one verified position of a request
// (its draft row and target row) or its bonus target row; each unit is cut into the same
// 8192-logit chunks as above, and task (unit, chunk) keeps its chunk of both rows in registers:
//   1. the chunk's (max, sum exp) of both rows, formed exactly as row_stats forms them, go into
//      the unit's slot for that chunk as four words tagged with this call's tag;
//   2. wave 0 waits until all chunks of the unit carry the tag (one round loads every word of
//      the unit, polled every few hundred cycles so the polls do not crowd the rows' loads) and
//      merges them in chunk order (the same merge as verify_chunks), giving lse_d and lse_t;
//   3. from the registers: the chunk's sum of min(p_d, p_t) (as tv_chunks forms it) and its
//      mass under the unit's final-draw law (the residual max(0, p_t - p_d) of a verified
//      position, p_t of the bonus row; as chunk_mass forms them).
// So every row is read once, and all partial results equal those of the three-kernel path bit
// for bit. vt_select then runs the acceptance test and the final draw per request from these
// results (reading only the drafted tokens' logits and the one chunk it rescans) and merges c*.
//
// The grid is persistent: every workgroup is resident at once (checked by the host). It is
// split into groups of N >= nch workgroups, each group sweeping a contiguous range of units
// (the verified rows only, when the lengths are given and B <= kLiveMax), and workgroup w of
// a group takes the group's tasks w, w + N, w + 2N, ... A unit's nch chunks
// are consecutive tasks, so they belong to nch different workgroups, each of which reaches them
// after finishing tasks of earlier units only; by induction over units every wait ends. Polling is bounded all the
// same: a workgroup that gives up writes the call's key into the give-up word, and vt_select
// then reports every request as faulty.
//
// The key is the splitmix64 finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014) of a call counter E in the workspace, xor a constant, and the tag
// is call_tag(E): slots left by earlier calls carry earlier tags. Every sweep workgroup reads E
// at its start; vt_select (which runs after the whole sweep) advances it.

__device__ __forceinline__ unsigned long long call_key(unsigned long long e) {
    unsigned long long z = e ^ 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ unsigned long long ld_agent(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void st_agent(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Hand-over words between workgroups: 32 bits of this call's tag beside a 32-bit value,
// stored and loaded as one 64-bit word, so a word is valid on its own and no store needs to
// wait for another. The tag is the low half of the call counter xor a constant: consecutive
// calls differ, and all-zero or all-one words carry no call's tag.
__device__ __forceinline__ unsigned call_tag(unsigned long long e) {
    return static_cast<unsigned>(e) ^ 0x9e3779b9u;
}
__device__ __forceinline__ unsigned long long tagged(unsigned tag, float v) {
    return (static_cast<unsigned long long>(tag) << 32) | __float_as_uint(v);
}
__device__ __forceinline__ unsigned long long tagged(unsigned tag, unsigned v) {
    return (static_cast<unsigned long long>(tag) << 32) | v;
}
__device__ __forceinline__ bool has_tag(unsigned long long w, unsigned tag) {
    return static_cast<unsigned>(w >> 32) == tag;
}
__device__ __forceinline__ float tagged_f(unsigned long long w) {
    return __uint_as_float(static_cast<unsigned>(w));
}

struct SweepArgs {
    RowSet rs;
    int nch;
    long long ntasks;                 // B (gamma + 1) nch
    const float* lse_d_in;            // nullable
    unsigned long long* slots;        // [unit][nch][4] tagged: draft max, sum; target max, sum
    float2* ulse;                     // [unit] (lse_d, lse_t)
    float* rmass;                     // [unit][nch] mass under the unit's final-draw law
    float* psum;                      // [b gamma + k][nch] sum of min(p_d, p_t)
    unsigned long long* hdr;          // [0] call counter E, [1] give-up key, [2] this sweep's key
    unsigned spin;
    long long units;                  // B (gamma + 1)
    int groups;                       // workgroup groups, each sweeping its own range of units
    int compact;                      // 1: the tasks cover the verified rows only (B <= kLiveMax)
};

// Requests whose verified rows the sweep can index through LDS: with per-request lengths, the
// tasks then cover only the rows that exist (len + 1 target and len draft rows per valid
// request), so a workgroup never meets runs of absent rows that others do not.
constexpr int kLiveMax = 4096;

// lse of a unit's row from the lanes' chunk partials (lane i holds chunk i < nch <= 64; the
// other lanes hold (-inf, 0)): merge_lse_wave's arithmetic on the same values.
__device__ __forceinline__ float merge_lanes(float2 p0) {
    const float mm = wave_max_dpp(fmaxf(-INFINITY, p0.x));
    if (mm == -INFINITY) return -INFINITY;
    float ss = (p0.x == -INFINITY) ? 0.0f : p0.y * __expf(p0.x - mm);
    ss = wave_sum_dpp(ss);
    return mm + __logf(ss);
}

template <bool VEC4>
__global__ __launch_bounds__(kThreads, 4)      // four workgroups per CU
void vt_sweep_kernel(SweepArgs a) {
    __shared__ float sm[4][kWaves];
    __shared__ float fscr[2 * (kWaves + 1)];
    __shared__ float s_lse[2];
    __shared__ int s_gave;
    __shared__ unsigned long long s_key;
    __shared__ unsigned s_tag;
    __shared__ int s_cum[kLiveMax];                  // compact: verified rows of requests <= b
    __shared__ int s_wsum[kWaves];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const RowSet& rs = a.rs;
    const int G = rs.gamma, V = rs.V, nch = a.nch, G1 = G + 1;
    if (tid == 0) {
        const unsigned long long e = ld_agent(a.hdr);
        s_key = call_key(e);
        s_tag = call_tag(e);
        s_gave = 0;
        if (blockIdx.x == 0) st_agent(a.hdr + 2, s_key);
    }
    // compact: inclusive scan over the requests of their verified rows (0 for a faulty one)
    long long units = a.units;
    if (a.compact) {
        int carry = 0;
        for (int b0 = 0; b0 < rs.B; b0 += kThreads) {
            const int b = b0 + tid;
            int v = 0;
            if (b < rs.B) {
                const ReqRows q = request_rows(rs, b);
                v = q.ok ? q.ell + 1 : 0;
            }
#pragma unroll
            for (int o = 1; o < kWave; o <<= 1) {
                const int w = __shfl_up(v, o, kWave);
                if (lane >= o) v += w;
            }
            if (lane == kWave - 1) s_wsum[wave] = v;
            __syncthreads();
            int before = carry;
            for (int w = 0; w < wave; ++w) before += s_wsum[w];
            if (b < rs.B) s_cum[b] = before + v;
            for (int w = 0; w < kWaves; ++w) carry += s_wsum[w];
            __syncthreads();
        }
        units = carry;
    }
    __syncthreads();
    const unsigned long long key = s_key;
    const unsigned tag = s_tag;
    // group grp of the workgroups sweeps units [u0, u1), its workgroups taking its tasks
    // round-robin; a unit's waits then involve the workgroups of one group only
    const unsigned per = gridDim.x / static_cast<unsigned>(a.groups);
    const unsigned grp = blockIdx.x / per;
    const long long u0 = units * grp / a.groups, u1 = units * (grp + 1) / a.groups;
    int bcur = 0;                                    // compact: request of the current task
    for (long long lt = blockIdx.x - grp * per; lt < (u1 - u0) * nch; lt += per) {
        const long long task = u0 * nch + lt;
        const long long lu = task / nch;
        const int c = static_cast<int>(task - lu * nch);
        int b, s;
        if (a.compact) {
            // tasks of a workgroup come in increasing order, so the request only moves forward
            while (s_cum[bcur] <= lu) ++bcur;
            b = bcur;
            s = static_cast<int>(lu - (b ? s_cum[b - 1] : 0));
        } else {
            b = static_cast<int>(lu / G1);
            s = static_cast<int>(lu - static_cast<long long>(b) * G1);
        }
        const long long unit = static_cast<long long>(b) * G1 + s;
        const ReqRows q = request_rows(rs, b);
        if (!q.ok || s > q.ell) continue;               // no such row: nobody waits for it
        const bool pair = s < q.ell;
        // the draft's given normaliser, loaded ahead of the chunk (it is needed right after the wait)
        const float lsdi = (pair && a.lse_d_in) ? a.lse_d_in[static_cast<long long>(b) * G + s] : 0.0f;
        float t[kPer], d[kPer];
        load_chunk<VEC4>(rs.Lt + (q.off + s) * V, c, V, t);
        if (pair) load_chunk<VEC4>(rs.Ld + (static_cast<long long>(b) * G + s) * V, c, V, d);
        // 1. chunk partials (row_stats' arithmetic), published as tagged words
        // (the registers then hold the chunk's terms exp(x - M); a pair forms both rows'
        // terms, also when the draft's lse is given)
        float mt, st, md = -INFINITY, sd = 0.0f;
        if (pair)
            chunk_ms2<true>(t, d, mt, st, md, sd, sm);
        else
            chunk_ms<true>(t, mt, st, sm);
        unsigned long long* us = a.slots + unit * nch * 4;
        if (tid < 4) {
            const float v = tid == 0 ? md : tid == 1 ? sd : tid == 2 ? mt : st;
            st_agent(us + 4 * c + tid, tagged(tag, v));
        }
        // 2. the unit's normalisers, once every chunk's words carry the tag
        if (wave == 0) {
            float2 pd = make_float2(-INFINITY, 0.0f), pt = make_float2(-INFINITY, 0.0f);
            bool ok = true;
            if (lane < nch) {
                unsigned long long w[4];
                for (unsigned n = 0;;) {
                    bool all = true;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        w[j] = ld_agent(us + 4 * lane + j);
                        all &= has_tag(w[j], tag);
                    }
                    if (all) break;
                    if (++n > a.spin) {
                        ok = false;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(16);
                }
                if (ok) {
                    pd = make_float2(tagged_f(w[0]), tagged_f(w[1]));
                    pt = make_float2(tagged_f(w[2]), tagged_f(w[3]));
                }
            }
            if (__any(!ok)) {
                if (lane == 0) {
                    s_gave = 1;
                    st_agent(a.hdr + 1, key);
                }
            }
            const float lt = merge_lanes(pt);
            float ld = 0.0f;
            if (pair) ld = a.lse_d_in ? lsdi : merge_lanes(pd);
            if (lane == 0) {
                s_lse[0] = ld;
                s_lse[1] = lt;
            }
        }
        __syncthreads();
        if (s_gave) break;
        const float lsd = s_lse[0], lst = s_lse[1];
        if (c == 0 && tid == 0) a.ulse[unit] = make_float2(lsd, lst);
        // 3. sum of min(p_d, p_t) (tv_chunks' arithmetic) and the final-draw mass
        //    (chunk_mass' arithmetic) from the chunk's terms in the registers
        const float sct = chunk_scale(mt, lst);
        float sv = 0.0f, mass = 0.0f;
        if (pair) {
            // (a row with no mass has scale 0, so the sum is 0 as tv_chunks leaves it)
            const float scd = chunk_scale(md, lsd);
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                const float pt = t[e] * sct, pd = d[e] * scd;
                sv += fminf(pd, pt);
                mass += fmaxf(pt - pd, 0.0f);
            }
            float v2[2] = {sv, mass};
            chunk_sums<2>(v2, fscr);
            sv = v2[0];
            mass = v2[1];
            if (tid == 0) a.psum[(static_cast<long long>(b) * G + s) * nch + c] = sv;
        } else {
#pragma unroll
            for (int e = 0; e < kPer; ++e) mass += t[e] * sct;
            mass = chunk_sum(mass, fscr);
        }
        if (tid == 0) a.rmass[unit * nch + c] = mass;
    }
    __builtin_amdgcn_s_waitcnt(0);
}

// Per request (first B workgroups): the acceptance test on the unit normalisers (the same
// test as verify_chunks on the same values), the final draw from the unit's chunk masses, the
// outputs; the remaining workgroups merge c* as tv_merge does. A call whose sweep gave up
// reports every request as faulty. Workgroup 0 advances the call counter last.
template <bool VEC4>
__global__ __launch_bounds__(kThreads)
void vt_select_kernel(SweepArgs a, const int32_t* __restrict__ x, const float* __restrict__ u_acc,
                      const float* __restrict__ u_fin, float* __restrict__ lse_d_out,
                      float* __restrict__ lse_t_out, int32_t* __restrict__ n_out,
                      int32_t* __restrict__ y_out, float* __restrict__ cstar) {
    __shared__ float s_lt[65], s_ld[64];
    __shared__ int s_n, s_bad, s_gave;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const RowSet& rs = a.rs;
    const int G = rs.gamma, V = rs.V, nch = a.nch, G1 = G + 1;
    if (tid == 0) s_gave = ld_agent(a.hdr + 1) == ld_agent(a.hdr + 2);
    __syncthreads();
    const bool gave = s_gave;
    if (blockIdx.x >= static_cast<unsigned>(rs.B)) {
        const unsigned blk = blockIdx.x - rs.B;
        if (!gave) {
            tv_merge_body(rs, nch, a.psum, cstar, blk);
        } else {
            const long long pair = static_cast<long long>(blk) * kWaves + wave;
            if (pair < static_cast<long long>(rs.B) * G && lane == 0) cstar[pair] = qnan();
        }
        return;
    }
    const int b = blockIdx.x;
    int32_t* y = y_out + static_cast<long long>(b) * G1;
    const ReqRows q = request_rows(rs, b);
    if (!q.ok || gave) {
        for (int i = tid; i <= G; i += kThreads) {
            y[i] = -1;
            if (lse_t_out) lse_t_out[static_cast<long long>(b) * G1 + i] = qnan();
            if (lse_d_out && i < G) lse_d_out[static_cast<long long>(b) * G + i] = qnan();
        }
        if (tid == 0) n_out[b] = -1;
    } else {
        int xk = 0;
        float ltx = 0.0f, ldx = 0.0f, ua = 0.0f;
        if (wave == 0 && lane < q.ell) {
            xk = x[static_cast<long long>(b) * G + lane];
            ua = u_acc[static_cast<long long>(b) * G + lane];
            if (xk >= 0 && xk < V) {
                ltx = rs.Lt[(q.off + lane) * V + xk];
                ldx = rs.Ld[(static_cast<long long>(b) * G + lane) * V + xk];
            }
        }
        const float2* ul = a.ulse + static_cast<long long>(b) * G1;
        for (int i = tid; i <= q.ell; i += kThreads) {
            s_lt[i] = ul[i].y;
            if (i < q.ell) s_ld[i] = a.lse_d_in ? a.lse_d_in[static_cast<long long>(b) * G + i] : ul[i].x;
        }
        __syncthreads();
        if (wave == 0) {
            bool bad = false, rej = false;
            const int k = lane;
            if (k < q.ell) {
                if (xk < 0 || xk >= V) {
                    bad = true;
                } else {
                    const float lst = s_lt[k], lsd = s_ld[k];
                    const float lpt = (lst == -INFINITY) ? -INFINITY : ltx - lst;
                    const float lpd = (lsd == -INFINITY) ? -INFINITY : ldx - lsd;
                    bool acc;
                    if (lpd == -INFINITY)
                        acc = lpt > -INFINITY;
                    else
                        acc = logf(clamp_uniform(ua)) < lpt - lpd;
                    rej = !acc;
                }
            }
            const unsigned long long badm = __ballot(bad);
            const unsigned long long rejm = __ballot(rej);
            if (lane == 0) {
                s_bad = badm != 0ull;
                s_n = rejm ? (__ffsll(static_cast<long long>(rejm)) - 1) : q.ell;
            }
        }
        __syncthreads();
        const int n = s_n;
        for (int i = tid; i <= G; i += kThreads) {
            if (lse_t_out) lse_t_out[static_cast<long long>(b) * G1 + i] = (i <= q.ell) ? s_lt[i] : qnan();
            if (lse_d_out && i < G) lse_d_out[static_cast<long long>(b) * G + i] = (i < q.ell) ? s_ld[i] : qnan();
        }
        if (s_bad) {
            for (int i = tid; i <= G; i += kThreads) y[i] = -1;
            if (tid == 0) n_out[b] = -1;
        } else {
            FinalRow fr;
            fr.lt = rs.Lt + (q.off + n) * V;
            fr.lse_t = s_lt[n];
            fr.residual = n < q.ell;
            fr.ld = fr.residual ? rs.Ld + (static_cast<long long>(b) * G + n) * V : nullptr;
            fr.lse_d = fr.residual ? s_ld[n] : 0.0f;
            const int z = final_draw<VEC4>(V, nch, fr, a.rmass + (static_cast<long long>(b) * G1 + n) * nch,
                                           clamp_uniform(u_fin[b]));
            for (int i = tid; i <= G; i += kThreads)
                y[i] = (i < n) ? x[static_cast<long long>(b) * G + i] : (i == n ? z : -1);
            if (tid == 0) n_out[b] = n;
        }
    }
    if (b == 0 && tid == 0) st_agent(a.hdr, ld_agent(a.hdr) + 1);   // the next call's key
}

// ----------------------------------------------------------------------------- one launch
// Verify and TV labels of a small batch in one launch: one workgroup per task (unit, chunk),
// every workgroup resident at once (the host checks), and every hand-over between workgroups
// a key-tagged slot instead of a kernel boundary. A task
//   1. forms its chunk's partials and waits for its unit's normalisers, as vt_sweep does;
//   2. publishes its chunk's sum of min(p_d, p_t), its mass under the unit's final-draw law and
//      its p_t mass (for a residual that rounds to zero), and, if its chunk holds the drafted
//      token, the acceptance decision (as verify_chunks forms it; chunk 0 flags a token outside
//      [0, V));
//   3. chunk 0 of a verified position merges c* (as tv_merge); every task of the unit that the
//      decisions make the final one waits for that unit's masses, finds the chunk that holds
//      u * total (as final_draw), and that chunk's task rescans its own registers in token order
//      (through LDS, in final_draw's layout and order) and writes n and y.
// Every result equals the chunked kernels' bit for bit. Chunk 0 of request 0's first unit
// waits at the end until every live task has published, then advances the call counter.
// Polling is bounded: a workgroup that gives up writes the call's key into the give-up word
// (the outputs of such a call are not defined).


constexpr int kSmallMaxTasks = 768;                 // one-launch form: tasks per call at most

struct SmallArgs {
    RowSet rs;
    int nch;
    long long ntasks;
    const float* lse_d_in;
    const int32_t* x;
    const float* u_acc;
    const float* u_fin;
    float* lse_d_out;
    float* lse_t_out;
    int32_t* n_out;
    int32_t* y_out;
    float* cstar;
    unsigned long long* slots;        // [unit][nch][4] tagged: draft max, sum; target max, sum
    unsigned long long* mslots;       // [unit][nch][4] tagged: sum min, final mass, p_t mass, -
    unsigned long long* flags;        // [B][gamma] tagged acceptance codes: 1 keep, 2 reject, 3 bad token
    unsigned long long* hdr;          // [0] call counter E, [1] give-up key
    unsigned spin;
};

// Polls until each of every lane's N words carries the tag (a null pointer counts as ready);
// false after the spin bound. Every round loads the lane's untagged words together, so the
// wait costs the round trips of the slowest word. The whole wave calls it.
template <int N>
__device__ __forceinline__ bool poll_tagged_n(const unsigned long long* const (&p)[N],
                                              unsigned long long (&v)[N], unsigned tag, unsigned spin) {
    bool done[N];
#pragma unroll
    for (int j = 0; j < N; ++j) done[j] = p[j] == nullptr;
    for (unsigned n = 0;;) {
#pragma unroll
        for (int j = 0; j < N; ++j)
            if (!done[j]) v[j] = ld_agent(p[j]);
        bool all = true;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            done[j] = done[j] || has_tag(v[j], tag);
            all = all && done[j];
        }
        if (__all(all)) return true;
        if (++n > spin) return false;
        __builtin_amdgcn_s_sleep(1);
    }
}

template <bool VEC4>
__global__ __launch_bounds__(kThreads, 2)
void vt_small_kernel(SmallArgs a) {
    __shared__ float sm[4][kWaves];
    __shared__ float fscr[3 * kWaves + 1];
    __shared__ int iscr[2 * kWaves];
    __shared__ float s_lse[2];
    __shared__ int s_gave, s_n, s_bad, s_found, s_residual;
    __shared__ float s_tprime;
    __shared__ unsigned s_tag;
    // the rescan's weights in token order, 4 words of padding after every 32 (one thread's
    // run), so the row-wise writes and the run-wise reads both spread over the banks
    __shared__ float4 wl[(kChunk + kChunk / 8) / 4];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const RowSet& rs = a.rs;
    const int G = rs.gamma, V = rs.V, nch = a.nch, G1 = G + 1;
    const long long task = blockIdx.x;
    const long long unit = task / nch;
    const int c = static_cast<int>(task - unit * nch);
    const int b = static_cast<int>(unit / G1), s = static_cast<int>(unit - static_cast<long long>(b) * G1);
    const ReqRows q = request_rows(rs, b);
    const bool anchor = b == 0 && s == 0 && c == 0;
    int32_t* y = a.y_out + static_cast<long long>(b) * G1;
    if (!q.ok) {                                     // a faulty request: its first task reports it
        if (s == 0 && c == 0) {
            for (int i = tid; i <= G; i += kThreads) {
                y[i] = -1;
                if (a.lse_t_out) a.lse_t_out[static_cast<long long>(b) * G1 + i] = qnan();
                if (i < G) {
                    if (a.lse_d_out) a.lse_d_out[static_cast<long long>(b) * G + i] = qnan();
                    a.cstar[static_cast<long long>(b) * G + i] = qnan();
                }
            }
            if (tid == 0) a.n_out[b] = -1;
        }
        if (!anchor) return;
    }
    const bool live = q.ok && s <= q.ell;
    const bool pair = live && s < q.ell;
    float t[kPer], d[kPer];
    float lsd = 0.0f, lst = 0.0f;
    unsigned long long* us = a.slots + unit * nch * 4;
    unsigned long long* ms = a.mslots + unit * nch * 4;
    // the later steps' inputs, loaded ahead of the chunk: the drafted token, its uniform and the
    // draft's given normaliser; the final draw's uniform and the request's drafted tokens
    int xk = -1, xr = -1;
    float ua = 0.0f, lsdi = 0.0f, uf = 0.0f;
    if (live) {
        if (pair) {
            xk = a.x[static_cast<long long>(b) * G + s];
            ua = a.u_acc[static_cast<long long>(b) * G + s];
            if (a.lse_d_in) lsdi = a.lse_d_in[static_cast<long long>(b) * G + s];
        }
        uf = a.u_fin[b];
        if (tid < G) xr = a.x[static_cast<long long>(b) * G + tid];
    }
    const long long base = static_cast<long long>(c) * kChunk;
    const bool owner = pair && xk >= 0 && xk < V && xk >= base && xk < base + kChunk;
    float ltx = 0.0f, ldx = 0.0f;                    // the two logits at the drafted token
    if (live) {
        load_chunk<VEC4>(rs.Lt + (q.off + s) * V, c, V, t);
        if (pair) load_chunk<VEC4>(rs.Ld + (static_cast<long long>(b) * G + s) * V, c, V, d);
        if (owner && tid == 0) {
            ltx = rs.Lt[(q.off + s) * V + xk];
            ldx = rs.Ld[(static_cast<long long>(b) * G + s) * V + xk];
        }
    }
    // the call's tag, read while the chunk is on its way (the anchor counts on every task
    // having read it before it publishes)
    if (tid == 0) {
        s_tag = call_tag(ld_agent(a.hdr));
        s_gave = 0;
    }
    __syncthreads();
    const unsigned tag = s_tag;
    float cmt = -INFINITY, cmd = -INFINITY;          // the chunk's maxima (target, draft)
    if (live) {
        // 1. partials, published as tagged words; the unit's normalisers (a pair forms both
        //    rows' partials, also when the draft's lse is given: its terms need the max). The
        //    chunk's terms replace its logits.
        float mt, st, md = -INFINITY, sd = 0.0f;
        if (pair)
            chunk_ms2<true>(t, d, mt, st, md, sd, sm);
        else
            chunk_ms<true>(t, mt, st, sm);
        cmt = mt;
        cmd = md;
        if (tid < 4) {
            const float v = tid == 0 ? md : tid == 1 ? sd : tid == 2 ? mt : st;
            st_agent(us + 4 * c + tid, tagged(tag, v));
        }
        if (wave == 0) {
            // lane i reads chunk i's four words
            float2 pd = make_float2(-INFINITY, 0.0f), pt = make_float2(-INFINITY, 0.0f);
            bool ok = true;
            if (lane < nch) {
                unsigned long long w[4];
                for (unsigned n = 0;;) {
                    bool all = true;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        w[j] = ld_agent(us + 4 * lane + j);
                        all &= has_tag(w[j], tag);
                    }
                    if (all) break;
                    if (++n > a.spin) {
                        ok = false;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (ok) {
                    pd = make_float2(tagged_f(w[0]), tagged_f(w[1]));
                    pt = make_float2(tagged_f(w[2]), tagged_f(w[3]));
                }
            }
            if (__any(!ok) && lane == 0) {
                s_gave = 1;
                st_agent(a.hdr + 1, static_cast<unsigned long long>(tag));
            }
            const float lt = merge_lanes(pt);
            float ld = 0.0f;
            if (pair) ld = a.lse_d_in ? lsdi : merge_lanes(pd);
            if (lane == 0) {
                s_lse[0] = ld;
                s_lse[1] = lt;
            }
        }
        __syncthreads();
        lsd = s_lse[0];
        lst = s_lse[1];
    }
    if (live && !s_gave) {
        // 2. the chunk's sums, published; the acceptance decision of its drafted token
        // (from the chunk's terms: sum of min(p_d, p_t), the final-draw mass, p_t's mass)
        const float sct = chunk_scale(cmt, lst);
        float sv = 0.0f, mass = 0.0f, ptm = 0.0f;
        if (pair) {
            const float scd = chunk_scale(cmd, lsd);
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                const float pt = t[e] * sct, pd = d[e] * scd;
                sv += fminf(pd, pt);
                mass += fmaxf(pt - pd, 0.0f);
                ptm += pt;
            }
        } else {
#pragma unroll
            for (int e = 0; e < kPer; ++e) mass += t[e] * sct;
        }
        float v3[3] = {sv, mass, ptm};
        chunk_sums<3>(v3, fscr);
        sv = v3[0];
        mass = v3[1];
        ptm = v3[2];
        if (tid < 3) st_agent(ms + 4 * c + tid, tagged(tag, tid == 0 ? sv : tid == 1 ? mass : ptm));
        if (pair) {
            unsigned long long* fl = a.flags + static_cast<long long>(b) * G + s;
            if (xk < 0 || xk >= V) {
                if (c == 0 && tid == 0) st_agent(fl, tagged(tag, 3u));
            } else if (owner && tid == 0) {
                const float lpt = (lst == -INFINITY) ? -INFINITY : ltx - lst;
                const float lpd = (lsd == -INFINITY) ? -INFINITY : ldx - lsd;
                bool acc;
                if (lpd == -INFINITY)
                    acc = lpt > -INFINITY;
                else
                    acc = logf(clamp_uniform(ua)) < lpt - lpd;
                st_agent(fl, tagged(tag, acc ? 1u : 2u));
            }
        }
        // normalisers out (chunk 0 of each unit; the bonus unit also fills what lies beyond)
        if (c == 0) {
            if (tid == 0) {
                if (a.lse_t_out) a.lse_t_out[static_cast<long long>(b) * G1 + s] = lst;
                if (pair && a.lse_d_out) a.lse_d_out[static_cast<long long>(b) * G + s] = lsd;
            }
            if (!pair) {
                for (int i = s + 1 + tid; i <= G; i += kThreads)
                    if (a.lse_t_out) a.lse_t_out[static_cast<long long>(b) * G1 + i] = qnan();
                for (int i = s + tid; i < G; i += kThreads) {
                    if (a.lse_d_out) a.lse_d_out[static_cast<long long>(b) * G + i] = qnan();
                    a.cstar[static_cast<long long>(b) * G + i] = qnan();
                }
            }
        }
        // 3. one poll for the request's acceptance codes and the unit's chunk sums
        if (wave == 0) {
            const unsigned long long* const pw[4] = {
                lane < q.ell ? a.flags + static_cast<long long>(b) * G + lane : nullptr,
                lane < nch ? ms + 4 * lane : nullptr, lane < nch ? ms + 4 * lane + 1 : nullptr,
                lane < nch ? ms + 4 * lane + 2 : nullptr};
            unsigned long long wv4[4] = {0, 0, 0, 0};
            const bool ok = poll_tagged_n<4>(pw, wv4, tag, a.spin);
            const unsigned long long fv = wv4[0], w0 = wv4[1], w1 = wv4[2], w2 = wv4[3];
            const unsigned code = static_cast<unsigned>(fv) & 3u;
            const bool bad = ok && lane < q.ell && code == 3u;
            const bool rej = ok && lane < q.ell && code == 2u;
            const unsigned long long badm = __ballot(bad), rejm = __ballot(rej);
            const int n = rejm ? (__ffsll(static_cast<long long>(rejm)) - 1) : q.ell;
            // c* of a verified position (chunk 0): tv_merge's sum over the chunks
            float ps = (ok && lane < nch) ? tagged_f(w0) : 0.0f;
            ps = wave_sum_dpp(ps);
            if (pair && c == 0 && ok && lane == 0) a.cstar[static_cast<long long>(b) * G + s] = ps;
            // the final draw's search when this unit is the final one (final_draw's search)
            int found = -1;
            float tprime = INFINITY;
            bool residual = pair;
            if (ok && badm == 0ull && s == n) {
                float mv = (lane < nch) ? tagged_f(w1) : 0.0f;
                const float pv = (lane < nch) ? tagged_f(w2) : 0.0f;
                const float ufc = clamp_uniform(uf);
                for (int pass = 0; pass < 2; ++pass) {
                    const float v = (lane < nch) ? mv : 0.0f;
                    const float tot = wave_sum_dpp(v);
                    const float target = ufc * tot;
                    found = -1;
                    tprime = INFINITY;
                    const float incl = wave_incl_scan_dpp(v);
                    const float excl = wave_shr1_dpp(incl);
                    const unsigned long long hit = __ballot((lane < nch) && (v > 0.0f) && (incl > target));
                    if (hit) {
                        const int f = __ffsll(static_cast<long long>(hit)) - 1;
                        found = f;
                        tprime = target - (0.0f + wave_bcast(excl, f));
                    }
                    if (found < 0 && tot > 0.0f) {
                        const int last = (lane < nch && v > 0.0f) ? lane : -1;
                        found = wave_max_int_dpp(last);
                        tprime = INFINITY;
                    }
                    if (tot > 0.0f || !residual) break;
                    residual = false;                 // residual rounded to zero: p_t instead
                    mv = pv;
                }
            }
            if (lane == 0) {
                if (!ok) {
                    s_gave = 1;
                    st_agent(a.hdr + 1, static_cast<unsigned long long>(tag));
                }
                s_bad = badm != 0ull;
                s_n = n;
                s_found = found;
                s_tprime = tprime;
                s_residual = residual ? 1 : 0;
            }
        }
        __syncthreads();
        const int n = s_n;
        if (!s_gave && s_bad && !pair && c == 0) {    // a drafted token outside [0, V)
            for (int i = tid; i <= G; i += kThreads) y[i] = -1;
            if (tid == 0) a.n_out[b] = -1;
        }
        const int found = s_found;
        if (!s_gave && !s_bad && s == n && (found == c || (found < 0 && c == 0))) {
            int z = -1;
            if (found == c) {
                // the rescan: weights into LDS in token order, then final_draw's layout and order
                FinalRow fw;
                fw.lt = nullptr;
                fw.ld = nullptr;
                fw.lse_t = lst;
                fw.lse_d = pair ? lsd : 0.0f;
                fw.residual = s_residual;
                fw.at_chunk(cmt, cmd);
                // token row r (tokens 4 r .. 4 r + 3) goes to padded vector r + r / 8; the run
                // of thread i starts at vector 9 i
                const bool rd = fw.residual;
#pragma unroll
                for (int g = 0; g < kPer / 4; ++g) {
                    const int e = 4 * g, r = tid + kThreads * g;
                    wl[r + (r >> 3)] = make_float4(fw.weight(t[e], rd ? d[e] : 0.0f),
                                                   fw.weight(t[e + 1], rd ? d[e + 1] : 0.0f),
                                                   fw.weight(t[e + 2], rd ? d[e + 2] : 0.0f),
                                                   fw.weight(t[e + 3], rd ? d[e + 3] : 0.0f));
                }
                __syncthreads();
                float wv[kPer];
#pragma unroll
                for (int g = 0; g < kPer / 4; ++g) {
                    const float4 v = wl[(kPer / 4 + 1) * tid + g];
                    wv[4 * g] = v.x;
                    wv[4 * g + 1] = v.y;
                    wv[4 * g + 2] = v.z;
                    wv[4 * g + 3] = v.w;
                }
                z = chunk_pick(wv, s_tprime, c * kChunk + kPer * tid, fscr, iscr);
            }
            // gamma <= 64 < kThreads: thread i writes y[i] (its drafted token was loaded above)
            for (int i = tid; i <= G; i += kThreads)
                y[i] = (i < n) ? (i == tid ? xr : a.x[static_cast<long long>(b) * G + i]) : (i == n ? z : -1);
            if (tid == 0) a.n_out[b] = n;
        }
    }
    // the anchor: once every live task has published its partials, the next call's counter
    if (anchor) {
        if (wave == 0) {
            // lane l watches tasks l, l + 64, ...: all of its words are loaded together per round
            constexpr int kPerLane = kSmallMaxTasks / kWave;
            bool watch[kPerLane];
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) {
                const long long tk = lane + static_cast<long long>(kWave) * j;
                watch[j] = false;
                if (tk < a.ntasks) {
                    const long long u2 = tk / nch;
                    const int b2 = static_cast<int>(u2 / G1), s2 = static_cast<int>(u2 - static_cast<long long>(b2) * G1);
                    const ReqRows q2 = request_rows(rs, b2);
                    watch[j] = q2.ok && s2 <= q2.ell;
                }
            }
            for (unsigned n2 = 0;; ++n2) {
                unsigned long long w[kPerLane];
#pragma unroll
                for (int j = 0; j < kPerLane; ++j)
                    w[j] = watch[j] ? ld_agent(a.slots + (lane + static_cast<long long>(kWave) * j) * 4 + 3) : 0ull;
                bool miss = false;
#pragma unroll
                for (int j = 0; j < kPerLane; ++j) {
                    if (watch[j] && has_tag(w[j], tag)) watch[j] = false;
                    miss |= watch[j];
                }
                if (!__any(miss) || n2 > a.spin) break;
                __builtin_amdgcn_s_sleep(1);
            }
        }
        __syncthreads();
        if (tid == 0) st_agent(a.hdr, ld_agent(a.hdr) + 1);
    }
}

}  // namespace

int verify_chunk_elems() { return kChunk; }
size_t verify_state_bytes() { return sizeof(ReqState); }

static bool rows_vec4(const RowSet& rs) {
    return (rs.V % 4) == 0 && (reinterpret_cast<uintptr_t>(rs.Ld) % 16) == 0 &&
           (reinterpret_cast<uintptr_t>(rs.Lt) % 16) == 0;
}

static int nchunks(int V) { return (V + kChunk - 1) / kChunk; }

#define DSPARK_LAUNCH_VEC4(kernel, grid, ...)                                              \
    do {                                                                                    \
        if (rows_vec4(rs))                                                                  \
            hipLaunchKernelGGL(kernel<true>, grid, dim3(kThreads), 0, st, __VA_ARGS__);     \
        else                                                                                \
            hipLaunchKernelGGL(kernel<false>, grid, dim3(kThreads), 0, st, __VA_ARGS__);    \
    } while (0)

hipError_t launch_row_stats(const RowSet& rs, const float* lse_d_in, float2* part,
                            hipStream_t st) {
    const int nch = nchunks(rs.V);
    const dim3 grid(static_cast<unsigned>(nch) * (2 * rs.gamma + 1) * rs.B);
    DSPARK_LAUNCH_VEC4(row_stats_kernel, grid, rs, nch, lse_d_in, part);
    return hipGetLastError();
}

hipError_t launch_verify(const RowSet& rs, const int32_t* x, const float2* part,
                         const float* lse_d_in, const float* u_acc, const float* u_fin,
                         float* lse_d_out, float* lse_t_out, float* csum, void* state,
                         int32_t* n_out, int32_t* y_out, hipStream_t st) {
    const int nch = nchunks(rs.V);
    ReqState* rstate = static_cast<ReqState*>(state);
    DSPARK_LAUNCH_VEC4(verify_chunks_kernel, dim3(static_cast<unsigned>(nch) * rs.B), rs, nch, x,
                       part, lse_d_in, u_acc, lse_d_out, lse_t_out, csum, rstate);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    DSPARK_LAUNCH_VEC4(verify_select_kernel, dim3(rs.B), rs, nch, x, u_fin, csum, rstate, n_out,
                       y_out);
    return hipGetLastError();
}

hipError_t launch_verify_tv(const RowSet& rs, const int32_t* x, const float2* part,
                            const float* lse_d_in, const float* u_acc, const float* u_fin,
                            float* lse_d_out, float* lse_t_out, float* csum, void* state,
                            float* psum, int32_t* n_out, int32_t* y_out, float* cstar,
                            hipStream_t st) {
    const int nch = nchunks(rs.V);
    ReqState* rstate = static_cast<ReqState*>(state);
    const unsigned nverify = static_cast<unsigned>(nch) * rs.B;
    const unsigned ntv = static_cast<unsigned>(nch) * rs.gamma * rs.B;
    DSPARK_LAUNCH_VEC4(verify_tv_chunks_kernel, dim3(nverify + ntv), rs, nch, x, part, lse_d_in,
                       u_acc, lse_d_out, lse_t_out, csum, rstate, psum, nverify);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long pairs = static_cast<long long>(rs.B) * rs.gamma;
    const unsigned nmerge = static_cast<unsigned>((pairs + kWaves - 1) / kWaves);
    DSPARK_LAUNCH_VEC4(verify_tv_select_kernel, dim3(static_cast<unsigned>(rs.B) + nmerge), rs, nch,
                       x, u_fin, csum, rstate, n_out, y_out, psum, cstar);
    return hipGetLastError();
}

// ---- one-sweep verify + TV
namespace {

struct SweepFit {
    int cus = -1;
    int occ[2] = {-1, -1};
};

// Resident workgroups of vt_sweep_kernel on the current device (0 if unknown).
int sweep_capacity(bool vec4) {
    thread_local SweepFit cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    SweepFit& f = cache[dev];
    if (f.cus < 0 && hipDeviceGetAttribute(&f.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    int& occ = f.occ[vec4 ? 1 : 0];
    if (occ < 0) {
        int o = 0;
        const hipError_t e = vec4 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, vt_sweep_kernel<true>, kThreads, 0)
                                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, vt_sweep_kernel<false>, kThreads, 0);
        occ = (e == hipSuccess) ? o : 0;
    }
    return f.cus > 0 ? f.cus * occ : 0;
}

}  // namespace

size_t verify_sweep_bytes(int B, int V, int gamma) {
    const size_t nch = static_cast<size_t>(nchunks(V));
    const size_t units = static_cast<size_t>(B) * (gamma + 1);
    auto al = [](size_t n) { return (n + 255) / 256 * 256; };
    const size_t sweep = 256 + al(units * nch * 4 * sizeof(unsigned long long)) + al(units * sizeof(float2)) +
                         al(units * nch * sizeof(float)) + al(static_cast<size_t>(B) * gamma * nch * sizeof(float));
    const size_t small = 256 + 2 * al(units * nch * 4 * sizeof(unsigned long long)) +
                         al(static_cast<size_t>(B) * gamma * sizeof(unsigned long long));
    return sweep > small ? sweep : small;
}

// Resident workgroups of vt_small_kernel on the current device (0 if unknown).
int small_capacity(bool vec4) {
    thread_local SweepFit cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    SweepFit& f = cache[dev];
    if (f.cus < 0 && hipDeviceGetAttribute(&f.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    int& occ = f.occ[vec4 ? 1 : 0];
    if (occ < 0) {
        int o = 0;
        const hipError_t e = vec4 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, vt_small_kernel<true>, kThreads, 0)
                                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, vt_small_kernel<false>, kThreads, 0);
        occ = (e == hipSuccess) ? o : 0;
    }
    return f.cus > 0 ? f.cus * occ : 0;
}

bool verify_sweep_ok(int V) {
    return nchunks(V) <= kWave && sweep_capacity(true) >= nchunks(V) && sweep_capacity(false) >= nchunks(V);
}

bool verify_small_ok(const RowSet& rs) {
    const int nch = nchunks(rs.V);
    const long long ntasks = static_cast<long long>(rs.B) * (rs.gamma + 1) * nch;
    return nch <= kWave && ntasks <= kSmallMaxTasks && ntasks <= small_capacity(rows_vec4(rs));
}

hipError_t launch_verify_small(const RowSet& rs, const int32_t* x, const float* lse_d_in,
                               const float* u_acc, const float* u_fin, float* lse_d_out,
                               float* lse_t_out, int32_t* n_out, int32_t* y_out, float* cstar,
                               void* ws, unsigned spin, hipStream_t st) {
    SmallArgs a;
    a.rs = rs;
    a.nch = nchunks(rs.V);
    a.ntasks = static_cast<long long>(rs.B) * (rs.gamma + 1) * a.nch;
    a.lse_d_in = lse_d_in;
    a.x = x; a.u_acc = u_acc; a.u_fin = u_fin;
    a.lse_d_out = lse_d_out; a.lse_t_out = lse_t_out; a.n_out = n_out; a.y_out = y_out;
    a.cstar = cstar;
    a.spin = spin;
    char* p = static_cast<char*>(ws);
    auto al = [](size_t n) { return (n + 255) / 256 * 256; };
    const size_t units = static_cast<size_t>(rs.B) * (rs.gamma + 1);
    a.hdr = reinterpret_cast<unsigned long long*>(p);
    p += 256;
    a.slots = reinterpret_cast<unsigned long long*>(p);
    p += al(units * a.nch * 4 * sizeof(unsigned long long));
    a.mslots = reinterpret_cast<unsigned long long*>(p);
    p += al(units * a.nch * 4 * sizeof(unsigned long long));
    a.flags = reinterpret_cast<unsigned long long*>(p);
    const bool v4 = rows_vec4(rs);
    if (v4)
        hipLaunchKernelGGL(vt_small_kernel<true>, dim3(static_cast<unsigned>(a.ntasks)), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(vt_small_kernel<false>, dim3(static_cast<unsigned>(a.ntasks)), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_verify_sweep(const RowSet& rs, const int32_t* x, const float* lse_d_in,
                               const float* u_acc, const float* u_fin, float* lse_d_out,
                               float* lse_t_out, int32_t* n_out, int32_t* y_out, float* cstar,
                               void* ws, unsigned spin, hipStream_t st) {
    SweepArgs a;
    a.rs = rs;
    a.nch = nchunks(rs.V);
    a.ntasks = static_cast<long long>(rs.B) * (rs.gamma + 1) * a.nch;
    a.lse_d_in = lse_d_in;
    a.spin = spin;
    char* p = static_cast<char*>(ws);
    auto al = [](size_t n) { return (n + 255) / 256 * 256; };
    const size_t units = static_cast<size_t>(rs.B) * (rs.gamma + 1);
    a.hdr = reinterpret_cast<unsigned long long*>(p);
    p += 256;
    a.slots = reinterpret_cast<unsigned long long*>(p);
    p += al(units * a.nch * 4 * sizeof(unsigned long long));
    a.ulse = reinterpret_cast<float2*>(p);
    p += al(units * sizeof(float2));
    a.rmass = reinterpret_cast<float*>(p);
    p += al(units * a.nch * sizeof(float));
    a.psum = reinterpret_cast<float*>(p);
    const bool v4 = rows_vec4(rs);
    const long long cap = sweep_capacity(v4);
    a.units = static_cast<long long>(units);
    // two groups when each still has a workgroup per chunk of a row and the sweep takes
    // several rounds of tasks
    a.groups = (cap / 2 >= a.nch && a.ntasks >= 2 * cap) ? 2 : 1;
    a.compact = (rs.len != nullptr && rs.B <= kLiveMax) ? 1 : 0;
    unsigned grid = static_cast<unsigned>(a.ntasks < cap ? a.ntasks : cap);
    grid = grid / a.groups * a.groups;
    if (v4)
        hipLaunchKernelGGL(vt_sweep_kernel<true>, dim3(grid), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(vt_sweep_kernel<false>, dim3(grid), dim3(kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long pairs = static_cast<long long>(rs.B) * rs.gamma;
    const dim3 g2(static_cast<unsigned>(rs.B + (pairs + kWaves - 1) / kWaves));
    if (v4)
        hipLaunchKernelGGL(vt_select_kernel<true>, g2, dim3(kThreads), 0, st, a, x, u_acc, u_fin, lse_d_out,
                           lse_t_out, n_out, y_out, cstar);
    else
        hipLaunchKernelGGL(vt_select_kernel<false>, g2, dim3(kThreads), 0, st, a, x, u_acc, u_fin, lse_d_out,
                           lse_t_out, n_out, y_out, cstar);
    return hipGetLastError();
}

hipError_t launch_tv(const RowSet& rs, const float* lse_d, const float* lse_t,
                     const float2* part, float* psum, float* cstar, hipStream_t st) {
    const int nch = nchunks(rs.V);
    DSPARK_LAUNCH_VEC4(tv_chunks_kernel, dim3(static_cast<unsigned>(nch) * rs.gamma * rs.B), rs,
                       nch, lse_d, lse_t, part, psum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long pairs = static_cast<long long>(rs.B) * rs.gamma;
    hipLaunchKernelGGL(tv_merge_kernel, dim3(static_cast<unsigned>((pairs + kWaves - 1) / kWaves)),
                       dim3(kThreads), 0, st, rs, nch, psum, cstar);
    return hipGetLastError();
}

#undef DSPARK_LAUNCH_VEC4

}  // namespace dspark
