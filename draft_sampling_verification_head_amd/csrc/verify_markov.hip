// Verification and TV labels with the draft logits rebuilt from the Markov factors (gfx950).
//
// [P1] = "大模型推理加速的系统级工程：DeepSeek V4-Pro DSpark 推测解码方案深度解析与开源工具链
// DeepSpec" (Best Partners TV); [P3] = "DSpark Speculative Decoding" (concept note).
//
// The draft logits of position k are L_d[b, k] = U_k + W1[x_{k-1}] W2 ([P3] section
// "Semi-Autoregressive Generation"; x_{-1} is the context token x0). Verification ([P1]
// section "大模型推理的显存瓶颈与推测解码的演进逻辑", [P3] intro) needs, per verified position,
// p_d(x_k) for the acceptance test, the residual max(0, p_t - p_d) at the first rejection and,
// for the TV labels ([P3] "Confidence-Scheduled Verification"), sum_v min(p_d, p_t). Instead
// of reading a materialised [B][gamma][V] L_d, this path recomputes the rows it needs with the
// slab MFMA machinery of the draft (bit-identical to the slab draft's logits), so the draft
// never has to write them and verify reads U once instead of L_d twice. Launches:
//   row_stats - chunk (max, sum exp) of the target rows (the draft normalisers come from the
//               draft call);
//   vm_scan   - offsets of each request's verified draft rows in a compact row list;
//   vm_rows   - lse of the target rows, and one record per verified draft row (U row, target
//               row, W1 row of the previous token, drafted token, both normalisers);
//   vm_tv     - slab pass over the compact rows: U, L_t and W1 rows arrive in LDS by direct
//               loads ahead of the group being computed; per row and wave tile it leaves
//               sum min(p_d, p_t) and sum max(0, p_t - p_d), and the draft logit of the
//               drafted token. Up to four 16-column tiles per wave (vm_tv16): groups of 16
//               rows, the MFMA's full width, one group ahead; five tiles (vm_tv): groups of
//               8 rows, two groups ahead, as five tiles of 16 rows do not fit in LDS twice;
//   vm_select - per request: acceptance scan (same test as the materialised verify), TV labels
//               (wave-tile sums in tile order), and the final draw: the residual from its
//               wave-tile masses with the chosen tile recomputed by MFMA, or p_t (bonus, or a
//               residual that rounded to zero) from the target row's chunk partials.
#include "common.h"
#include "draw.h"
#include "kernels.h"
#include "rows.h"
#include "slab.h"

namespace dspark {

namespace {

using namespace slab;
using namespace rows;

constexpr int kRows = 8;                  // verified draft rows per vm_tv group
constexpr int kFields = 8;                // record fields (see VmRec)
enum VmRec { kUrow = 0, kTrow, kHrow, kXk, kLsd, kLst, kRb, kRk };

template <int NT>
struct VmLds {
    static constexpr int NTP = (NT + 1) / 2;                // 1 KB blocks per wave: 2 tiles x 8 rows
    static constexpr int UT = kSlabWaves * NTP * 1024;      // one group's U (or L_t) slice
    static constexpr int HB = kRows * kHRow;                // the group's W1 rows, 4 KB
    static constexpr int Buf = 2 * UT + HB;
    static constexpr int Meta = 4 * kFields * kRows * 4;    // record ring, 4 groups
    static constexpr int Total = 3 * Buf + Meta;
};

// ----------------------------------------------------------------------------- vm_scan
// d_off[b] = sum of the verified lengths of requests before b (0 for a faulty request);
// d_off[B] = number of verified draft rows.
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads)
void vm_scan(RowSet rs, int32_t* __restrict__ d_off) {
    __shared__ int scr[kScanThreads / kWave + 1];
    const int B = rs.B, tid = threadIdx.x;
    const int per = (B + kScanThreads - 1) / kScanThreads;
    const int b0 = tid * per, b1 = min(b0 + per, B);
    int local = 0;
    for (int b = b0; b < b1; ++b) {
        const ReqRows q = request_rows(rs, b);
        local += q.ok ? q.ell : 0;
    }
    int tot;
    int run = block_excl_scan<kScanThreads>(local, scr, &tot);
    for (int b = b0; b < b1; ++b) {
        d_off[b] = run;
        const ReqRows q = request_rows(rs, b);
        run += q.ok ? q.ell : 0;
    }
    if (tid == 0) d_off[B] = tot;
}

// ----------------------------------------------------------------------------- vm_rows
// One wave per request: lse of target slots s <= ell (NaN beyond), and the records of its
// verified draft rows at d_off[b] + k, structure of arrays rec[field * cap + row].
__global__ __launch_bounds__(kThreads)
void vm_rows(RowSet rs, int nch, const int32_t* __restrict__ x0, const int32_t* __restrict__ x,
             const float* __restrict__ ld_lse, const float2* __restrict__ part_t,
             const int32_t* __restrict__ d_off, int32_t* __restrict__ rec, long long cap,
             float* __restrict__ lse_t) {
    __shared__ float s_lt[kWaves][65];
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int b = blockIdx.x * kWaves + wave;
    if (b >= rs.B) return;
    const int G = rs.gamma, V = rs.V;
    const ReqRows q = request_rows(rs, b);
    for (int s = 0; s <= G; ++s) {
        float v = qnan();
        if (q.ok && s <= q.ell) v = merge_lse_wave(slot_part(part_t, b, s, G, nch), nch);
        if (lane == 0) {
            s_lt[wave][s] = v;
            lse_t[static_cast<long long>(b) * (G + 1) + s] = v;
        }
    }
    if (!q.ok) return;
    __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0): s_lt is written
    __builtin_amdgcn_wave_barrier();
    const long long d0 = d_off[b];
    for (int k = lane; k < q.ell; k += kWave) {
        const long long j = d0 + k;
        int h = k ? x[static_cast<long long>(b) * G + k - 1] : x0[b];
        if (h < 0 || h >= V) h = 0;                   // faulty request: vm_select reports it
        rec[kUrow * cap + j] = b * G + k;
        rec[kTrow * cap + j] = static_cast<int>(q.off + k);
        rec[kHrow * cap + j] = h;
        rec[kXk * cap + j] = x[static_cast<long long>(b) * G + k];
        rec[kLsd * cap + j] = __float_as_int(ld_lse[static_cast<long long>(b) * G + k]);
        rec[kLst * cap + j] = __float_as_int(s_lt[wave][k]);
        rec[kRb * cap + j] = b;
        rec[kRk * cap + j] = k;
    }
}

// ----------------------------------------------------------------------------- vm_tv
struct VmArgs {
    int V, r, ntw;
    long long cap;
    const float* U;
    const uint16_t* W1;
    const uint16_t* W2;
    const float* Lt;
    const int32_t* rec;       // [kFields][cap]
    const int32_t* nd;        // number of verified draft rows (d_off[B])
    float2* part;             // [cap][ntw] (sum min(p_d, p_t), sum max(0, p_t - p_d))
    float* ldx;               // [cap] draft logit at the drafted token
};

// Weights of one column: p_d, p_t from the logits and the row normalisers (a row without
// mass contributes nothing). vm_tv and vm_select evaluate them the same way.
__device__ __forceinline__ float pexp(float l, float lse) {
    return (lse == -INFINITY) ? 0.0f : __expf(l - lse);
}

template <int NT>
__global__ __launch_bounds__(kSlabThreads)
void vm_tv(VmArgs a) {
    using S = Slab<NT>;
    using Ly = VmLds<NT>;
    static_assert(kSlabWaves * S::Stage <= Ly::Buf, "W2 staging fits in buffer 2");
    constexpr int NL = 2 * Ly::NTP + 2;               // direct loads per wave and group
    extern __shared__ __align__(16) char sm[];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int slab = blockIdx.x;
    const long long cw = static_cast<long long>(slab) * S::SW + wave * S::WC;
    const int nd = *a.nd;
    const int ng = (nd + kRows - 1) / kRows;
    if (ng == 0) return;
    int* meta = reinterpret_cast<int*>(sm + 3 * Ly::Buf);

    // records of group g into ring slot g % 4 (wave 0 only): lane l loads field l / 8 of
    // row g * 8 + l % 8 (rows past the end repeat the last row; the epilogue masks them)
    auto meta_issue = [&](int g) {
        const int row = min(g * kRows + (lane & 7), nd - 1);
        lds_dma4(a.rec + static_cast<long long>(lane >> 3) * a.cap + row,
                 lds_addr(meta) + 4 * (g & 3) * (kFields * kRows));
    };
    // U and L_t slices of group g: per pair of tiles one 16-byte direct load each, into a
    // 1 KB block of 64 slots; slot l holds row l / 8, 4-column chunk (l % 8) ^ (l / 8) of the
    // pair's 32 columns (a swizzle for conflict-free epilogue reads). Chunks past V load
    // column 0 (the epilogue masks them). W1 rows: wave w loads row w of the group, 16-byte
    // piece p of the row at position p ^ w. Every lane issues every load.
    auto issue = [&](int g, int i) {
        const int* mt = meta + (g & 3) * (kFields * kRows);
        const uint32_t ub = lds_addr(sm) + i * Ly::Buf + wave * Ly::NTP * 1024;
        const uint32_t lb = ub + Ly::UT;
        const uint32_t hb = lds_addr(sm) + i * Ly::Buf + 2 * Ly::UT;
        const int l = opaque_lane(), lr = l >> 3;
        const int cbase = static_cast<int>(cw) + 4 * ((l & 7) ^ lr);
        const float* up = a.U + static_cast<long long>(mt[kUrow * kRows + lr]) * a.V;
        const float* tp = a.Lt + static_cast<long long>(mt[kTrow * kRows + lr]) * a.V;
#pragma unroll
        for (int q = 0; q < Ly::NTP; ++q) {
            int col = cbase + 32 * q;
            if (col > a.V - 4) col = 0;
            lds_dma16(up + col, ub + q * 1024);
            lds_dma16(tp + col, lb + q * 1024);
        }
        const int hrow = mt[kHrow * kRows + wave];
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
            const int p = 16 * i2 + (lane >> 2);
            int c = p ^ wave;
            if (8 * c >= a.r) c = 0;
            lds_dma4(a.W1 + static_cast<long long>(hrow) * a.r + 8 * c + 2 * (lane & 3),
                     hb + wave * kHRow + i2 * 256);
        }
    };

    if (wave == 0) {
        meta_issue(0);
        if (ng > 1) meta_issue(1);
    }
    wait_vm_lgkm<0>();
    __syncthreads();
    issue(0, 0);
    if (ng > 1) {
        if (wave == 0 && ng > 2) meta_issue(2);       // before group 1's loads (see the wait)
        issue(1, 1);
    }
    bf16x8 w2f[NT][kKS];
    load_w2_frags<NT, (NT > 4 ? 2 : 4), 1>(w2f, a.W2, a.V, a.r, cw, sm + 2 * Ly::Buf + wave * S::Stage);

    const int rq = lane & 15, cg = lane >> 4, rr = rq & 7;
    // A group's results are stored at the top of the next group, before its loads, so that
    // the wait below covers loads only (see draft_slab_step).
    long long pend_j = -1;
    float2 pend_part = make_float2(0.0f, 0.0f);
    float pend_ldx = 0.0f;
    bool pend_has_ldx = false;
    auto flush = [&]() {
        if (pend_j < 0) return;
        if (cg == 0) a.part[pend_j * a.ntw + slab * kSlabWaves + wave] = pend_part;
        if (pend_has_ldx) a.ldx[pend_j] = pend_ldx;
    };
    for (int g = 0; g < ng; ++g) {
        const int i = g % 3;
        // group g's loads (and the records of group g + 2, issued before group g + 1's
        // loads) have landed once at most the NL loads of group g + 1 are outstanding
        if (g + 1 < ng) wait_vm_lgkm<NL>();
        else wait_vm_lgkm<0>();
        bare_barrier();
        flush();
        if (wave == 0 && g + 3 < ng) meta_issue(g + 3);   // slot of group g - 1, now free
        if (g + 2 < ng) issue(g + 2, (g + 2) % 3);

        const char* ub = sm + i * Ly::Buf;
        const char* lb = ub + Ly::UT;
        const char* H = ub + 2 * Ly::UT;
        // this lane's chunk of tile t: the accumulators start at U, as in the slab draft
        auto toff = [&](int t) {
            const int c = ((t & 1) << 2) + cg;        // chunk of the tile pair t / 2
            return (wave * Ly::NTP + (t >> 1)) * 1024 + 16 * (rr * 8 + (c ^ rr));
        };
        f32x4 acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float4 u4 = *reinterpret_cast<const float4*>(ub + toff(t));
            acc[t] = f32x4{u4.x, u4.y, u4.z, u4.w};
        }
        // B fragments one rank chunk ahead (request columns 8..15 repeat rows 0..7); the
        // empty asm keeps the compiler from hoisting every chunk's fragment at once, which
        // would not fit beside the W2 fragments
        auto hfrag = [&](int s) {
            const int p = (4 * s + cg) ^ rr;
            return *reinterpret_cast<const bf16x8*>(H + rr * kHRow + 16 * p);
        };
        bf16x8 hf = hfrag(0);
#pragma unroll
        for (int s = 0; s < kKS; ++s) {
            {
                const bf16x8 hn = (s + 1 < kKS) ? hfrag(s + 1) : hf;
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2f[t][s], hf, acc[t], 0, 0, 0);
                asm volatile("" ::: "memory");
                hf = hn;
            }
        }

        const int* mt = meta + (g & 3) * (kFields * kRows);
        const long long j = static_cast<long long>(g) * kRows + rr;
        const bool valid = rq < kRows && j < nd;
        const float lsd = __int_as_float(mt[kLsd * kRows + rr]);
        const float lst = __int_as_float(mt[kLst * kRows + rr]);
        const int xk = mt[kXk * kRows + rr];
        float smin = 0.0f, sres = 0.0f;
        bool has_ldx = false;
        float ldx_v = 0.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float4 t4 = *reinterpret_cast<const float4*>(lb + toff(t));
            const long long col = cw + 16 * t + 4 * cg;
            const bool ok = col < a.V;
            const float ld[4] = {ok ? acc[t][0] : -INFINITY, ok ? acc[t][1] : -INFINITY,
                                 ok ? acc[t][2] : -INFINITY, ok ? acc[t][3] : -INFINITY};
            const float lt[4] = {ok ? t4.x : -INFINITY, ok ? t4.y : -INFINITY,
                                 ok ? t4.z : -INFINITY, ok ? t4.w : -INFINITY};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float pd = pexp(ld[v], lsd), pt = pexp(lt[v], lst);
                smin += fminf(pd, pt);
                sres += fmaxf(pt - pd, 0.0f);
                if (valid && ok && xk == col + v) {
                    has_ldx = true;
                    ldx_v = ld[v];
                }
            }
        }
        smin += swz_xor16(smin);
        smin += __shfl_xor(smin, 32, kWave);
        sres += swz_xor16(sres);
        sres += __shfl_xor(sres, 32, kWave);
        pend_j = valid ? j : -1;
        pend_part = make_float2(smin, sres);
        pend_ldx = ldx_v;
        pend_has_ldx = has_ldx;
    }
    flush();
}

// vm_tv for NT <= 4 with groups of 16 rows (the MFMA's N): lane (rq, cg) of the epilogue owns
// row rq, columns 4 cg .. 4 cg + 3 of each tile, as in vm_tv, so the per-lane sums and their
// reductions run in the same order and the outputs are bit-identical. Two LDS buffers: the
// loads of group g + 1 are issued after the barrier of group g and land while it is computed.
constexpr int kRows16 = 16;

template <int NT>
struct VmLds16 {
    static constexpr int UT = kSlabWaves * NT * 1024;      // [wave][tile][16 rows][16 cols] fp32
    static constexpr int HB = kRows16 * kHRow;             // the group's W1 rows, 8 KB
    static constexpr int Buf = 2 * UT + HB;
    static constexpr int Meta = 4 * kFields * kRows16 * 4; // record ring, 4 groups
    static constexpr int Total = 2 * Buf + Meta;
};

template <int NT>
__global__ __launch_bounds__(kSlabThreads)
void vm_tv16(VmArgs a) {
    using S = Slab<NT>;
    using Ly = VmLds16<NT>;
    static_assert(NT <= 4 && Ly::Total <= kLdsBytes, "two buffers of 16-row groups fit in LDS");
    static_assert(kSlabWaves * S::Stage <= Ly::Buf, "W2 staging fits in buffer 1");
    extern __shared__ __align__(16) char sm[];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int slab = blockIdx.x;
    const long long cw = static_cast<long long>(slab) * S::SW + wave * S::WC;
    const int nd = *a.nd;
    const int ng = (nd + kRows16 - 1) / kRows16;
    if (ng == 0) return;
    int* meta = reinterpret_cast<int*>(sm + 2 * Ly::Buf);
    // record ring slot: field f of row i of the group at [(i / 8) * 64 + f * 8 + i % 8]
    auto fld = [](const int* mt, int f, int i) { return mt[(i >> 3) * 64 + f * 8 + (i & 7)]; };

    // records of group g into ring slot g % 4 (wave 0 only), two 4-byte direct loads: lane l
    // of load h takes field l / 8 of row 16 g + 8 h + l % 8 (rows past the end repeat the last)
    auto meta_issue = [&](int g) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = min(g * kRows16 + 8 * h + (lane & 7), nd - 1);
            lds_dma4(a.rec + static_cast<long long>(lane >> 3) * a.cap + row,
                     lds_addr(meta) + 4 * ((g & 3) * (kFields * kRows16) + 64 * h));
        }
    };
    // U and L_t tiles of group g as in the slab draft ([16 rows][16 cols] per tile, lane l
    // loads row l / 4, 4-column chunk (l % 4) ^ ((l / 16) % 4)); W1 rows: wave w fills rows
    // 2w, 2w + 1, lane l loads 16-byte piece (l % 32) ^ (row % 16). Every lane issues every
    // load; chunks past V load column 0 (the epilogue masks them).
    auto issue = [&](int g, int i) {
        const int* mt = meta + (g & 3) * (kFields * kRows16);
        const uint32_t ub = lds_addr(sm) + i * Ly::Buf + wave * NT * 1024;
        const uint32_t lb = ub + Ly::UT;
        const uint32_t hb = lds_addr(sm) + i * Ly::Buf + 2 * Ly::UT;
        const int l = opaque_lane();
        const int u_rq = l >> 2, u_ch = (l & 3) ^ ((l >> 4) & 3);
        const float* up = a.U + static_cast<long long>(fld(mt, kUrow, u_rq)) * a.V;
        const float* tp = a.Lt + static_cast<long long>(fld(mt, kTrow, u_rq)) * a.V;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            int col = static_cast<int>(cw) + 16 * t + 4 * u_ch;
            if (col > a.V - 4) col = 0;
            lds_dma16(up + col, ub + t * 1024);
            lds_dma16(tp + col, lb + t * 1024);
        }
        const int h_row = 2 * wave + (l >> 5), h_piece = (l & 31) ^ (h_row & 15);
        const int piece = (8 * h_piece < a.r) ? h_piece : 0;
        lds_dma16(a.W1 + static_cast<long long>(fld(mt, kHrow, h_row)) * a.r + 8 * piece,
                  hb + wave * 1024);
    };

    if (wave == 0) {
        meta_issue(0);
        if (ng > 1) meta_issue(1);
    }
    wait_vm_lgkm<0>();
    __syncthreads();
    issue(0, 0);
    bf16x8 w2f[NT][kKS];
    load_w2_frags<NT, 4, 1>(w2f, a.W2, a.V, a.r, cw, sm + Ly::Buf + wave * S::Stage);
    wait_lgkm0();
    __syncthreads();                                  // buffer 1 (the staging area) is free

    const int rq = lane & 15, cg = lane >> 4;
    const int upos = 4 * rq + (cg ^ ((rq >> 2) & 3));  // this lane's 16 bytes of a tile
    long long pend_j = -1;
    float2 pend_part = make_float2(0.0f, 0.0f);
    float pend_ldx = 0.0f;
    bool pend_has_ldx = false;
    auto flush = [&]() {
        if (pend_j < 0) return;
        if (cg == 0) a.part[pend_j * a.ntw + slab * kSlabWaves + wave] = pend_part;
        if (pend_has_ldx) a.ldx[pend_j] = pend_ldx;
    };
    for (int g = 0; g < ng; ++g) {
        const int i = g & 1;
        // group g's loads and the records of group g + 1 were issued in the previous
        // iteration; nothing issued since is needed later than them
        wait_vm_lgkm<0>();
        bare_barrier();
        flush();
        if (wave == 0 && g + 2 < ng) meta_issue(g + 2);   // slot of group g - 2, now free
        if (g + 1 < ng) issue(g + 1, i ^ 1);

        const char* ub = sm + i * Ly::Buf + wave * NT * 1024;
        const char* lb = ub + Ly::UT;
        const char* H = sm + i * Ly::Buf + 2 * Ly::UT;
        f32x4 acc[NT];                                // from U, as in the slab draft
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float4 u4 = *reinterpret_cast<const float4*>(ub + t * 1024 + 16 * upos);
            acc[t] = f32x4{u4.x, u4.y, u4.z, u4.w};
        }
        const int hl = opaque_lane(), hrq = hl & 15, hcg = hl >> 4;
        auto hfrag = [&](int s) {
            const int p = (4 * s + hcg) ^ hrq;
            return *reinterpret_cast<const bf16x8*>(H + hrq * kHRow + 16 * p);
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

        const int* mt = meta + (g & 3) * (kFields * kRows16);
        const long long j = static_cast<long long>(g) * kRows16 + rq;
        const bool valid = j < nd;
        const float lsd = __int_as_float(fld(mt, kLsd, rq));
        const float lst = __int_as_float(fld(mt, kLst, rq));
        const int xk = fld(mt, kXk, rq);
        float smin = 0.0f, sres = 0.0f;
        bool has_ldx = false;
        float ldx_v = 0.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float4 t4 = *reinterpret_cast<const float4*>(lb + t * 1024 + 16 * upos);
            const long long col = cw + 16 * t + 4 * cg;
            const bool ok = col < a.V;
            const float ld[4] = {ok ? acc[t][0] : -INFINITY, ok ? acc[t][1] : -INFINITY,
                                 ok ? acc[t][2] : -INFINITY, ok ? acc[t][3] : -INFINITY};
            const float lt[4] = {ok ? t4.x : -INFINITY, ok ? t4.y : -INFINITY,
                                 ok ? t4.z : -INFINITY, ok ? t4.w : -INFINITY};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float pd = pexp(ld[v], lsd), pt = pexp(lt[v], lst);
                smin += fminf(pd, pt);
                sres += fmaxf(pt - pd, 0.0f);
                if (valid && ok && xk == col + v) {
                    has_ldx = true;
                    ldx_v = ld[v];
                }
            }
        }
        smin += swz_xor16(smin);
        smin += __shfl_xor(smin, 32, kWave);
        sres += swz_xor16(sres);
        sres += __shfl_xor(sres, 32, kWave);
        pend_j = valid ? j : -1;
        pend_part = make_float2(smin, sres);
        pend_ldx = ldx_v;
        pend_has_ldx = has_ldx;
    }
    flush();
}

// ----------------------------------------------------------------------------- vm_select
struct SelArgs {
    RowSet rs;
    int nch, r, ntw;
    const float* U;
    const uint16_t* W1;
    const uint16_t* W2;
    const int32_t* x0;
    const int32_t* x;
    const float* ld_lse;
    const float* u_acc;
    const float* u_fin;
    const float2* part_t;     // chunk partials of the target rows (row_stats layout)
    const int32_t* d_off;
    const float* lse_t;       // [B][gamma + 1]
    const float2* part;       // [cap][ntw] from vm_tv
    const float* ldx;
    int32_t* n_out;
    int32_t* y_out;
    float* lse_t_out;
    float* cstar;
};

template <int NT>
__global__ __launch_bounds__(kThreads)
void vm_select(SelArgs a) {
    using S = Slab<NT>;
    constexpr int CPL = (S::WC + kWave - 1) / kWave;
    __shared__ __align__(16) char stg[kKS * S::Stage];
    __shared__ float rowv[S::WC];
    __shared__ float s_lt[65];
    __shared__ float fscr[kWaves + 1];
    __shared__ int iscr[kWaves + 1];
    __shared__ int s_n, s_bad, s_z, s_resid, s_found;
    __shared__ float s_tprime;
    const RowSet& rs = a.rs;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int G = rs.gamma, V = rs.V;
    int32_t* y = a.y_out + static_cast<long long>(b) * (G + 1);
    const ReqRows q = request_rows(rs, b);
    for (int s = tid; s <= G; s += kThreads) {
        const float v = a.lse_t[static_cast<long long>(b) * (G + 1) + s];
        s_lt[s] = v;
        if (a.lse_t_out) a.lse_t_out[static_cast<long long>(b) * (G + 1) + s] = v;
    }
    __syncthreads();
    const long long d0 = q.ok ? a.d_off[b] : 0;

    // acceptance scan, one wave (gamma <= 64): log u < log p_t(x) - log p_d(x)
    if (wave == 0) {
        bool bad = !q.ok, rej = false;
        const int k = lane;
        if (q.ok && k < q.ell) {
            const int xk = a.x[static_cast<long long>(b) * G + k];
            if (xk < 0 || xk >= V) {
                bad = true;
            } else {
                const float ltx = rs.Lt[(q.off + k) * V + xk];
                const float ldx = a.ldx[d0 + k];
                const float lst = s_lt[k], lsd = a.ld_lse[static_cast<long long>(b) * G + k];
                const float lpt = (lst == -INFINITY) ? -INFINITY : ltx - lst;
                const float lpd = (lsd == -INFINITY) ? -INFINITY : ldx - lsd;
                bool acc;
                if (lpd == -INFINITY)
                    acc = lpt > -INFINITY;
                else
                    acc = logf(clamp_uniform(a.u_acc[static_cast<long long>(b) * G + k])) < lpt - lpd;
                rej = !acc;
            }
        }
        if (q.ok && k == 0 && q.ell > 0 && (a.x0[b] < 0 || a.x0[b] >= V)) bad = true;
        const unsigned long long badm = __ballot(bad);
        const unsigned long long rejm = __ballot(rej);
        if (lane == 0) {
            s_bad = badm != 0ull;
            s_n = rejm ? (__ffsll(static_cast<long long>(rejm)) - 1) : q.ell;
        }
    }
    __syncthreads();
    const bool bad = s_bad;
    const int n = s_n;

    // TV labels: sums of the row's wave-tile partials in tile order (lane-strided, then a
    // fixed-order wave sum); NaN past the verified length and for a faulty request
    for (int k = wave; k < G; k += kWaves) {
        float cs = qnan();
        if (!bad && k < q.ell) {
            const float2* P = a.part + (d0 + k) * a.ntw;
            float s = 0.0f;
            for (int i = lane; i < a.ntw; i += kWave) s += P[i].x;
            cs = wave_sum_dpp(s);
        }
        if (lane == 0 && a.cstar) a.cstar[static_cast<long long>(b) * G + k] = cs;
    }
    if (bad) {
        for (int i = tid; i <= G; i += kThreads) y[i] = -1;
        if (tid == 0) a.n_out[b] = -1;
        return;
    }

    // residual at the first rejection: wave 0 picks the wave tile from the masses and
    // recomputes that tile's draft logits (same MFMA sequence as vm_tv)
    if (tid == 0) s_resid = 0;
    __syncthreads();
    if (n < q.ell && wave == 0) {
        const long long j = d0 + n;
        float mass[kSelRegs];
        const float4* P4 = reinterpret_cast<const float4*>(a.part + j * a.ntw);
        float local = 0.0f;
#pragma unroll
        for (int t = 0; t < kSelRegs / 2; ++t) {
            const int i = lane * kSelRegs + 2 * t;    // ntw is a multiple of 8: pairs are whole
            float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (i < a.ntw) v = P4[i / 2];
            mass[2 * t] = v.y;
            mass[2 * t + 1] = v.w;
            local += v.y + v.w;
        }
        const float R = wave_sum_dpp(local);
        if (R > 0.0f) {
            const MassPick mp = search_mass<kSelRegs>(mass, local, clamp_uniform(a.u_fin[b]) * R);
            const long long cw = static_cast<long long>(mp.tile) * S::WC;
            const int rq = lane & 15, cg = lane >> 4;
            const int hrow = n ? a.x[static_cast<long long>(b) * G + n - 1] : a.x0[b];
            uint4 hv[kKS];
#pragma unroll
            for (int s = 0; s < kKS; ++s) {
                const int rank = 32 * s + 8 * cg;
                hv[s] = make_uint4(0u, 0u, 0u, 0u);
                if (rank < a.r)
                    hv[s] = *reinterpret_cast<const uint4*>(a.W1 + static_cast<long long>(hrow) * a.r + rank);
            }
            const float* urow = a.U + (static_cast<long long>(b) * G + n) * V;
            const float* trow = rs.Lt + (q.off + n) * V;
            float4 u4[NT], t4[NT];
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const long long col = cw + 16 * t + 4 * cg;
                u4[t] = t4[t] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (rq == 0 && col < V) {
                    u4[t] = *reinterpret_cast<const float4*>(urow + col);
                    t4[t] = *reinterpret_cast<const float4*>(trow + col);
                }
            }
            bf16x8 w2f[NT][kKS];
            load_w2_frags<NT, kKS, kKS>(w2f, a.W2, V, a.r, cw, stg);
            f32x4 acc[NT];                            // from U, as in the slab draft
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = f32x4{u4[t].x, u4[t].y, u4[t].z, u4[t].w};
#pragma unroll
            for (int s = 0; s < kKS; ++s) {
                {
                    const bf16x8 hf = __builtin_bit_cast(bf16x8, hv[s]);
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w2f[t][s], hf, acc[t], 0, 0, 0);
                }
            }
            const float lsd = a.ld_lse[static_cast<long long>(b) * G + n], lst = s_lt[n];
            if (rq == 0) {
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const bool ok = cw + 16 * t + 4 * cg < V;
                    const float ld[4] = {acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
                    const float lt[4] = {t4[t].x, t4[t].y, t4[t].z, t4[t].w};
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        rowv[16 * t + 4 * cg + v] =
                            ok ? fmaxf(pexp(lt[v], lst) - pexp(ld[v], lsd), 0.0f) : 0.0f;
                }
            }
            __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): the row is in LDS
            __builtin_amdgcn_wave_barrier();
            float e[CPL];
#pragma unroll
            for (int jj = 0; jj < CPL; ++jj) {
                const int c = lane * CPL + jj;
                e[jj] = (c < S::WC) ? rowv[c] : 0.0f;
            }
            const int z = scan_pick<CPL>(e, cw + lane * CPL, mp.tprime);
            if (lane == 0) {
                s_z = z;
                s_resid = 1;
            }
        }
    }
    __syncthreads();
    const bool resid_done = s_resid;
    int z = resid_done ? s_z : -1;
    if (!resid_done) {
        // p_t of target row n (the bonus row when n = ell, or a residual that rounded to
        // zero): chunk masses from the row's chunk partials, then a block rescan of the chunk
        const float lst = s_lt[n];
        const float* trow = rs.Lt + (q.off + n) * V;
        const float2* P = slot_part(a.part_t, b, n, G, a.nch);
        if (wave == 0) {
            float tot = 0.0f;
            for (int i = lane; i < a.nch; i += kWave)
                tot += (P[i].x == -INFINITY || lst == -INFINITY) ? 0.0f : P[i].y * __expf(P[i].x - lst);
            tot = wave_sum_dpp(tot);
            const float target = clamp_uniform(a.u_fin[b]) * tot;
            int found = -1;
            float tprime = INFINITY, run = 0.0f;
            for (int base = 0; base < a.nch && found < 0; base += kWave) {
                const int i = base + lane;
                const float v = (i < a.nch && P[i].x != -INFINITY && lst != -INFINITY)
                                    ? P[i].y * __expf(P[i].x - lst) : 0.0f;
                const float incl = wave_incl_scan_dpp(v);
                const float excl = wave_shr1_dpp(incl);
                const unsigned long long hit = __ballot((i < a.nch) && (v > 0.0f) && (run + incl > target));
                if (hit) {
                    const int f = __ffsll(static_cast<long long>(hit)) - 1;
                    found = base + f;
                    tprime = target - (run + wave_bcast(excl, f));
                }
                run += wave_bcast(incl, kWave - 1);
            }
            if (found < 0 && tot > 0.0f) {            // rounding left the target past the end
                int last = -1;
                for (int i = lane; i < a.nch; i += kWave)
                    if (P[i].x != -INFINITY && P[i].y > 0.0f) last = i;
                found = wave_max_int_dpp(last);
                tprime = INFINITY;
            }
            if (lane == 0) {
                s_found = found;
                s_tprime = tprime;
            }
        }
        __syncthreads();
        const int found = s_found;
        z = -1;
        if (found >= 0) {
            float t[kPer];
            load_chunk_contig<true>(trow, found, V, t);
            float w[kPer];
            float local = 0.0f;
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                w[e] = pexp(t[e], lst);
                local += w[e];
            }
            float tot;
            const float ex = block_excl_scan<kThreads>(local, fscr, &tot);
            const long long v0 = static_cast<long long>(found) * kChunk + static_cast<long long>(kPer) * tid;
            int hit = INT32_MAX, lastpos = -1;
            float run = ex;
            const float tprime = s_tprime;
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                run += w[e];
                if (w[e] > 0.0f) {
                    lastpos = static_cast<int>(v0 + e);
                    if (hit == INT32_MAX && run > tprime) hit = static_cast<int>(v0 + e);
                }
            }
            z = block_min_int<kThreads>(hit, iscr);
            if (z == INT32_MAX) z = block_max_int<kThreads>(lastpos, iscr);
        }
    }
    for (int i = tid; i <= G; i += kThreads)
        y[i] = (i < n) ? a.x[static_cast<long long>(b) * G + i] : (i == n ? z : -1);
    if (tid == 0) a.n_out[b] = n;
}

template <int NT>
hipError_t launch_nt(const VerifyMarkovCall& c, hipStream_t st) {
    const RowSet& rs = c.rs;
    const int nch = (rs.V + kChunk - 1) / kChunk;
    hipError_t e = launch_row_stats(rs, c.ld_lse, c.part_t, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(vm_scan, dim3(1), dim3(kScanThreads), 0, st, rs, c.d_off);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const long long cap = static_cast<long long>(rs.B) * rs.gamma;
    hipLaunchKernelGGL(vm_rows, dim3(static_cast<unsigned>((rs.B + kWaves - 1) / kWaves)), dim3(kThreads),
                       0, st, rs, nch, c.x0, c.x, c.ld_lse, c.part_t, c.d_off, c.rec, cap, c.lse_t);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    VmArgs v;
    v.V = rs.V; v.r = c.r; v.ntw = verify_markov_tiles(rs.V); v.cap = cap;
    v.U = c.U; v.W1 = static_cast<const uint16_t*>(c.W1); v.W2 = static_cast<const uint16_t*>(c.W2);
    v.Lt = rs.Lt; v.rec = c.rec; v.nd = c.d_off + rs.B; v.part = c.tvpart; v.ldx = c.ldx;
    if constexpr (NT <= 4)
        hipLaunchKernelGGL(vm_tv16<NT>, dim3(static_cast<unsigned>(slab_count(rs.V))),
                           dim3(kSlabThreads), VmLds16<NT>::Total, st, v);
    else
        hipLaunchKernelGGL(vm_tv<NT>, dim3(static_cast<unsigned>(slab_count(rs.V))), dim3(kSlabThreads),
                           VmLds<NT>::Total, st, v);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    SelArgs s;
    s.rs = rs; s.nch = nch; s.r = c.r; s.ntw = v.ntw;
    s.U = c.U; s.W1 = v.W1; s.W2 = v.W2; s.x0 = c.x0; s.x = c.x; s.ld_lse = c.ld_lse;
    s.u_acc = c.u_acc; s.u_fin = c.u_fin; s.part_t = c.part_t; s.d_off = c.d_off; s.lse_t = c.lse_t;
    s.part = c.tvpart; s.ldx = c.ldx; s.n_out = c.n_out; s.y_out = c.y_out;
    s.lse_t_out = c.lse_t_out; s.cstar = c.cstar;
    hipLaunchKernelGGL(vm_select<NT>, dim3(static_cast<unsigned>(rs.B)), dim3(kThreads), 0, st, s);
    return hipGetLastError();
}

}  // namespace

int verify_markov_tiles(int V) { return slab_count(V) * kSlabWaves; }

bool verify_markov_ok(int V, int r) {
    return r >= 1 && r <= kMaxRank && (r % 8) == 0 && (V % 8) == 0 &&
           verify_markov_tiles(V) <= kWave * kSelRegs && static_cast<long long>(kMaxRank) * V < (1LL << 32);
}

hipError_t launch_verify_markov(const VerifyMarkovCall& c, hipStream_t st) {
    switch (slab_nt(c.rs.V)) {
        case 1: return launch_nt<1>(c, st);
        case 2: return launch_nt<2>(c, st);
        case 3: return launch_nt<3>(c, st);
        case 4: return launch_nt<4>(c, st);
        default: return launch_nt<5>(c, st);
    }
}

}  // namespace dspark
