// Single-request Markov-head draft with W2 held in registers across all positions (gfx950).
//
// [P3] "DSpark Speculative Decoding", section "Semi-Autoregressive Generation": position k
// samples x_k from softmax(U_k + B_k) with B_k = W1[x_{k-1}] W2 (rank r), one position after
// the other. For a single request each position is a GEMV whose only large operand, W2
// (r x V bf16, 77.8 MB at r = 256, V = 151936), is the same at every position. The chip's
// vector register files hold 128 MB, so one persistent launch reads W2 from HBM once and
// keeps it in registers for all gamma positions. Each position then moves only U_k, the
// logits row and one W1 row. ([P3] = the concept note "DSpark Speculative Decoding".)
//
// Layout. One workgroup of 8 waves per CU, G = ceil(V / 640) workgroups (238 at
// V = 151936), all resident at once. Workgroup g owns the 640 columns starting at 640g.
//   - Wave w owns the rank group [32w, 32w + 32).
//   - Lane l owns the 10 consecutive columns starting at 640g + 10l.
// Each register holds two consecutive ranks of one column as bf16, 160 registers per
// lane. The load phase reads each 1280-byte W2 row segment with 16-byte coalesced loads
// into LDS, and each lane then picks its columns out of it. The products use v_dot2
// (bf16 x bf16 pairs into fp32). The 8 rank-group partial sums of a column meet in LDS and
// are added in wave order.
//
// Positions meet through their tile partials and one token slot, with no separate barrier:
//   - The slots are reset inside the launch. Two words follow them in the workspace: a call
//     counter E and a ready word F. Every workgroup reads E at the start; workgroup 0 fills
//     the partial and token slots with the sentinel while the W2 load is under way, then
//     stores F = mix(E) (a 64-bit mixing function); no workgroup publishes a partial before it
//     has seen that F, and workgroup 0 advances E when the launch is done, once every
//     workgroup is known to have started (each has published its last partial). A previous
//     call left F = mix(E - 1), so stale slots are never taken for this call's; a workspace
//     of arbitrary bytes matches only if F happens to equal mix(E).
//   - At position k every workgroup keeps its 640 logits in LDS (and stores them to the
//     logits output when the caller wants it), then publishes its tile's (max, sum exp) into
//     slot [k][g] with one 8-byte device-scope store.
//   - Wave 0 of workgroup 0 polls the G slots of position k until none holds the sentinel,
//     picks the tile that holds the inverse-CDF point from those partials (in tile order),
//     and publishes the pick (tile, global max, remaining mass) in two pick words. Wave 0 of
//     every other workgroup polls the pick words and token slot [k] together. The workgroup
//     that owns the picked tile rescans its logits from LDS in token order and publishes
//     (logit, token) in token slot [k]; the others take the token from there.
//   A single poller of the partials keeps the polling light: when every workgroup polled the
//   G partial slots, the loads queued and each of the two round trips took several times the
//   latency of one store seen by one poller; the pick costs one light hop more.
// No workgroup ever reads another's logits, so nothing waits for the logits stores, and the
// draw costs one published token instead of a read of the chosen tile. No L2 write-back
// fence is used, because that costs tens of microseconds per position on this part. Polling
// is bounded: a workgroup that gives up stops, so the launch always drains, and workgroup 0
// then writes the -1 sentinel into the positions it could not draw.
#include "common.h"
#include "draw.h"
#include "kernels.h"
#include "schedule_small.h"

namespace dspark {

namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kRThreads = 512;                            // 8 waves
constexpr int kRWaves = kRThreads / kWave;
constexpr int kGroupRanks = 32;                           // ranks per wave
constexpr int kResMaxRank = kRWaves * kGroupRanks;        // 256
constexpr int kLaneCols = 10;                             // consecutive columns per lane
constexpr int kResTileCols = kWave * kLaneCols;           // 640 columns per workgroup
constexpr int kStageRows = 8;                             // W2 rows per wave per staging round
constexpr int kChunks = kResTileCols / 8;                 // 16-byte chunks per row segment
constexpr int kStageLoads = kStageRows * kChunks / kWave; // uint4 loads per lane per round
constexpr size_t kResLds = static_cast<size_t>(kRWaves) * kStageRows * kResTileCols * 2;
constexpr int kPartRegs = RegTiles<kResTileCols>::value;  // partials per lane in the draw
constexpr int kMaxTiles = kWave * kPartRegs;              // 512 workgroups at most
constexpr unsigned long long kEmpty = ~0ull;              // sentinel: both halves NaN
// RNN head: the recurrence A, transposed into bf16 pairs (A[2p][j], A[2p+1][j]) at [j][p], sits
// in LDS after the rank-group sums, where the W2 staging was
constexpr size_t kRedBytes = sizeof(float) * kRWaves * kResTileCols;
constexpr size_t kAtBytes = static_cast<size_t>(kResMaxRank) * (kResMaxRank / 2) * 4;
constexpr size_t kResLdsRnn = kRedBytes + kAtBytes;
static_assert(kResLdsRnn >= kResLds, "the RNN layout covers the staging area");
static_assert(kStageLoads * kWave == kStageRows * kChunks, "staging rounds cover whole rows");
static_assert(kResLds >= sizeof(float) * kRWaves * kResTileCols, "sums fit in the staging area");
static_assert(kResTileCols == 640 && kRThreads + 128 == kResTileCols, "epilogue ownership");

struct ResArgs {
    int V, r, gamma, G;
    const float* U;           // [gamma][V]
    const uint16_t* W1;       // [V][r] bf16 bits
    const uint16_t* W2;       // [r][V] bf16 bits
    const int32_t* x0;
    const float* u;           // [gamma]
    int32_t* x_out;
    float* q_out;
    float* lse_out;
    float* L[64];             // logits row of position k (written when L_out)
    int L_out;
    float2* slots;            // [gamma][G] tile partials, kEmpty until published
    unsigned long long* toks; // [gamma] (logit bits << 32 | token) of each draw, kEmpty until published
    unsigned long long* picks;   // [gamma][2] (max bits << 32 | tile + 1), (remaining mass bits << 32 |
                                 // tile + 1) of each pick (tile + 1 = 0: no mass), kEmpty until published
    unsigned long long* epoch;   // [2]: the call counter E and the ready word F (after the picks)
    unsigned* status;         // number of workgroups that gave up (reset with the slots)
    unsigned spin;            // polls before a wait gives up
    const uint16_t* A;        // RNN head: [r][r] bf16 recurrence
    float* h_out;             // RNN head: [gamma][r] fp32 state of each position (nullable)
    sched::SmallJob job;      // with_job: the schedule run by workgroup G, beside the draft
    int with_job;
};

// Ready word of a call with counter e: the finaliser of the splitmix64 generator (Steele, Lea
// and Flood, "Fast splittable pseudorandom number generators", 2014) applied to e xor a
// constant, so that counters of all-zero or all-one bytes do not map to those bytes.
__device__ __forceinline__ unsigned long long ready_word(unsigned long long e) {
    unsigned long long z = e ^ 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ float dot2(uint32_t w, uint32_t h, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                           __builtin_bit_cast(bf16x2, h), acc, false);
}

__device__ __forceinline__ void store_coherent(float2* p, float2 v) {
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                       __builtin_bit_cast(unsigned long long, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long load_slot(const float2* p) {
    return __hip_atomic_load(reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_token(unsigned long long* p, unsigned long long v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long load_token(const unsigned long long* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// RNN = false: the Markov head, B_k = W1[x_{k-1}] W2.
// RNN = true: the RNN head, B_k = h_k W2 with h_1 = W1[x_0], h_k = A h_{k-1} + W1[x_{k-1}]
// ([P3] "Semi-Autoregressive Generation": a recurrent state inside the block). Every
// workgroup keeps h in fp32 in LDS and A (128 KB in bf16) in the LDS that the W2 staging
// used. A h_k does not depend on the token drawn at position k, so waves 4..7 form it while
// wave 0 waits for the position's partials; once the token is known, h_{k+1} = A h_k +
// W1[x_k]. The products take h as bf16 hi + lo parts (h = hi + lo to about 2^-17 relative)
// against the same W2 registers.
template <bool RNN>
__global__ __launch_bounds__(kRThreads, 1)
void draft_resident(ResArgs a) {
    __shared__ uint4 lds[(RNN ? kResLdsRnn : kResLds) / sizeof(uint4)];   // W2 staging, then sums (+ A)
    __shared__ float2 wpart[kRWaves];
    __shared__ float tl[kResTileCols];                     // this position's logits of the tile
    __shared__ uint32_t hs[kResMaxRank / 2];               // W1[x] as bf16 pairs
    __shared__ float hst[RNN ? kResMaxRank : 1];           // RNN: the state h_k in fp32
    __shared__ float ah[RNN ? 2 : 1][RNN ? kResMaxRank : 1];   // RNN: A h_k, two halves of j
    __shared__ uint32_t hhi[RNN ? kResMaxRank / 2 : 1];    // RNN: h_k as bf16 pairs, hi parts
    __shared__ uint32_t hlo[RNN ? kResMaxRank / 2 : 1];    //                        lo parts
    __shared__ unsigned long long ptile[kMaxTiles];       // workgroup 0: the position's tile partials
    __shared__ int stok;
    __shared__ int gave_up;
    __shared__ unsigned long long s_e0;                    // the call counter read at the start
    if (a.with_job && blockIdx.x == static_cast<unsigned>(a.G)) {
        // the extra workgroup: the schedule, by its first wave, on LDS the draft leaves alone
        // (this workgroup drafts nothing and takes no part in the position slots)
        if (threadIdx.x < kWave)
            sched::schedule_small<false>(a.job, reinterpret_cast<double*>(lds),
                                         reinterpret_cast<double*>(lds) + sched::kSmallCand);
        return;
    }
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int V = a.V, r = a.r;
    if (tid == 0) s_e0 = load_token(a.epoch);             // seen by every thread after a barrier
    if (blockIdx.x == 0) {                                // reset this call's slots
        unsigned long long* sl = reinterpret_cast<unsigned long long*>(a.slots);
        const int n = a.gamma * a.G + 3 * a.gamma;         // partial slots, token slots, pick words
        for (int i = tid; i < n; i += kRThreads) store_token(sl + i, kEmpty);
        if (tid == 0) __hip_atomic_store(a.status, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const long long c0 = static_cast<long long>(blockIdx.x) * kResTileCols;
    // epilogue columns of this thread: c0 + tid, and c0 + 512 + tid for tid < 128
    const long long e1 = c0 + tid, e2 = c0 + kRThreads + tid;
    const bool own2 = tid < kResTileCols - kRThreads;

    // 0. what position 0 needs besides W2, issued first: U_0 and the W1 row of x_0
    int tok0 = a.x0[0];
    if (tok0 < 0 || tok0 >= V) tok0 = -1;                  // dead request: -inf logits
    float u1 = (e1 < V) ? a.U[e1] : 0.0f;
    float u2 = (own2 && e2 < V) ? a.U[e2] : 0.0f;
    uint4 h0 = make_uint4(0u, 0u, 0u, 0u);
    if (tid < kResMaxRank / 8 && tok0 >= 0 && 8 * tid < r)
        h0 = *reinterpret_cast<const uint4*>(a.W1 + static_cast<long long>(tok0) * r + 8 * tid);

    // 1. W2 slice: w[i][m] = (W2[32w + 2m][c + i], W2[32w + 2m + 1][c + i]), c = 640g + 10l.
    //    Each wave issues all of its 32 rows at once as 16-byte coalesced loads of the
    //    workgroup's 1280-byte row segments (V % 8 == 0), then passes them through LDS in 4
    //    rounds of 8 rows, and every lane picks its 10 columns out of each row as 5 aligned
    //    4-byte words.
    uint16_t* stage = reinterpret_cast<uint16_t*>(lds) + wave * (kStageRows * kResTileCols);
    uint32_t w[kLaneCols][kGroupRanks / 2];
    constexpr int kRounds = kGroupRanks / kStageRows;
    uint4 v[kRounds][kStageLoads];                         // all of the lane's loads in flight
#pragma unroll
    for (int rho = 0; rho < kRounds; ++rho)
#pragma unroll
        for (int n = 0; n < kStageLoads; ++n) {
            const int i = lane + kWave * n, t = i / kChunks, ch = i - t * kChunks;
            const int row = kGroupRanks * wave + kStageRows * rho + t;
            const long long col = c0 + 8 * ch;
            v[rho][n] = make_uint4(0u, 0u, 0u, 0u);
            if (row < r && col < V)
                v[rho][n] = *reinterpret_cast<const uint4*>(a.W2 + static_cast<long long>(row) * V + col);
        }
    if (tid < kResMaxRank / 8) {
        reinterpret_cast<uint4*>(hs)[tid] = h0;
        if (RNN) {                                         // h_1 = W1[x_0]: hi exact, lo zero
            reinterpret_cast<uint4*>(hhi)[tid] = h0;
            reinterpret_cast<uint4*>(hlo)[tid] = make_uint4(0u, 0u, 0u, 0u);
            const uint32_t hw[4] = {h0.x, h0.y, h0.z, h0.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                hst[8 * tid + 2 * e] = __uint_as_float(hw[e] << 16);
                hst[8 * tid + 2 * e + 1] = __uint_as_float(hw[e] & 0xffff0000u);
            }
        }
    }
#pragma unroll
    for (int rho = 0; rho < kRounds; ++rho) {
#pragma unroll
        for (int n = 0; n < kStageLoads; ++n) {
            const int i = lane + kWave * n, t = i / kChunks, ch = i - t * kChunks;
            *reinterpret_cast<uint4*>(stage + t * kResTileCols + 8 * ch) = v[rho][n];
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < kStageRows; t += 2) {
            const uint32_t* r0p = reinterpret_cast<const uint32_t*>(stage + t * kResTileCols + kLaneCols * lane);
            const uint32_t* r1p = reinterpret_cast<const uint32_t*>(stage + (t + 1) * kResTileCols + kLaneCols * lane);
            const int m = (kStageRows / 2) * rho + t / 2;
#pragma unroll
            for (int i = 0; i < kLaneCols / 2; ++i) {
                const uint32_t r0 = r0p[i], r1 = r1p[i];
                w[2 * i][m] = (r0 & 0xffffu) | (r1 << 16);
                w[2 * i + 1][m] = (r0 >> 16) | (r1 & 0xffff0000u);
            }
        }
        __syncthreads();
    }
    float (*red)[kResTileCols] = reinterpret_cast<float (*)[kResTileCols]>(lds);   // reuses the staging area
    uint32_t* at2 = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(lds) + kRedBytes);   // RNN: A^T pairs
    if (RNN) {
        // A^T as bf16 pairs: at2[j * 128 + p] = (A[2p][j], A[2p+1][j]); zero beyond r. Task
        // (p, jc) reads 8 columns of rows 2p and 2p+1; a wave's lanes take consecutive p.
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            uint4 ra[4], rb[4];
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int task = tid + kRThreads * (4 * half + n);
                const int pp = task & (kResMaxRank / 2 - 1), jc = task >> 7;
                ra[n] = rb[n] = make_uint4(0u, 0u, 0u, 0u);
                if (2 * pp < r && 8 * jc < r) {
                    ra[n] = *reinterpret_cast<const uint4*>(a.A + static_cast<long long>(2 * pp) * r + 8 * jc);
                    rb[n] = *reinterpret_cast<const uint4*>(a.A + static_cast<long long>(2 * pp + 1) * r + 8 * jc);
                }
            }
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int task = tid + kRThreads * (4 * half + n);
                const int pp = task & (kResMaxRank / 2 - 1), jc = task >> 7;
                const uint32_t wa[4] = {ra[n].x, ra[n].y, ra[n].z, ra[n].w};
                const uint32_t wb[4] = {rb[n].x, rb[n].y, rb[n].z, rb[n].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    at2[(8 * jc + 2 * e) * (kResMaxRank / 2) + pp] = (wa[e] & 0xffffu) | (wb[e] << 16);
                    at2[(8 * jc + 2 * e + 1) * (kResMaxRank / 2) + pp] = (wa[e] >> 16) | (wb[e] & 0xffff0000u);
                }
            }
        }
    }

    if (tid == 0) gave_up = 0;
    const unsigned long long key = ready_word(s_e0);
    if (blockIdx.x == 0) {                                // the slots are reset: publish F
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) store_token(a.epoch + 1, key);
    }
    int tok = tok0;
    int k = 0;
    for (; k < a.gamma; ++k) {
        // 2. projection from registers: this wave's 32 ranks of the lane's 10 columns, with
        //    h = W1[x_{k-1}] from LDS (staged before the last workgroup barrier)
        if (RNN && a.h_out && blockIdx.x == 0 && tid < r) a.h_out[static_cast<long long>(k) * r + tid] = hst[tid];
        uint32_t hv[kGroupRanks / 2], hvl[RNN ? kGroupRanks / 2 : 1];
#pragma unroll
        for (int m = 0; m < kGroupRanks / 2; ++m) hv[m] = (RNN ? hhi : hs)[(kGroupRanks / 2) * wave + m];
        if (RNN) {
#pragma unroll
            for (int m = 0; m < kGroupRanks / 2; ++m) hvl[m] = hlo[(kGroupRanks / 2) * wave + m];
        }
        float acc[kLaneCols];
#pragma unroll
        for (int i = 0; i < kLaneCols; ++i) {
            float s = 0.0f;
#pragma unroll
            for (int m = 0; m < kGroupRanks / 2; ++m) {
                s = dot2(w[i][m], hv[m], s);
                if (RNN) s = dot2(w[i][m], hvl[m], s);
            }
            acc[i] = s;
        }
#pragma unroll
        for (int i = 0; i < kLaneCols / 2; ++i)
            reinterpret_cast<float2*>(&red[wave][kLaneCols * lane])[i] = make_float2(acc[2 * i], acc[2 * i + 1]);
        __syncthreads();
        // 3. logits (rank groups added in wave order), logits row, tile partial
        const bool live = tok >= 0;
        float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
        for (int g = 0; g < kRWaves; ++g) s1 += red[g][tid];
        if (own2) {
#pragma unroll
            for (int g = 0; g < kRWaves; ++g) s2 += red[g][kRThreads + tid];
        }
        const float l1 = (live && e1 < V) ? u1 + s1 : -INFINITY;
        const float l2 = (live && own2 && e2 < V) ? u2 + s2 : -INFINITY;
        tl[tid] = l1;
        if (own2) tl[kRThreads + tid] = l2;
        if (a.L_out) {
            float* Lk = a.L[k];
            if (e1 < V) Lk[e1] = l1;
            if (own2 && e2 < V) Lk[e2] = l2;
        }
        const float mw = wave_max_dpp(fmaxf(l1, l2));
        const float ew = (mw == -INFINITY) ? 0.0f
                         : ((l1 == -INFINITY ? 0.0f : __expf(l1 - mw)) +
                            (l2 == -INFINITY ? 0.0f : __expf(l2 - mw)));
        const float sw = wave_sum_dpp(ew);
        if (lane == 0) wpart[wave] = make_float2(mw, sw);
        __syncthreads();
        float2* slot = a.slots + static_cast<long long>(k) * a.G;
        if (tid == 0) {
            float m = -INFINITY;
#pragma unroll
            for (int i = 0; i < kRWaves; ++i) m = fmaxf(m, wpart[i].x);
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < kRWaves; ++i) s += tile_mass(wpart[i], m);
            if (k == 0) {                                 // the slots must be reset first
                for (unsigned n = 0; load_token(a.epoch + 1) != key; ++n) {
                    if (n > a.spin) {
                        gave_up = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            if (!gave_up) store_coherent(slot + blockIdx.x, make_float2(m, s));   // publishes the tile
        }
        // U_{k+1} goes out now, so it is in flight while the partials arrive
        if (k + 1 < a.gamma) {
            const long long o = static_cast<long long>(k + 1) * V;
            u1 = (e1 < V) ? a.U[o + e1] : 0.0f;
            u2 = (own2 && e2 < V) ? a.U[o + e2] : 0.0f;
        }
        // 4. wave 0: draw x_k (workgroup 0 picks the tile, its owner rescans it), stage W1[x_k]
        if (wave == 0) {
            int t = -1;
            float lx = 0.0f;
            TilePick tp;
            tp.tile = -1;
            tp.m = tp.lse = -INFINITY;
            tp.tprime = INFINITY;
            bool known = false;                           // the pick is known here
            unsigned long long* pk = a.picks + 2 * k;
            if (blockIdx.x == 0) {
                // load j of lane l reads tile 64 j + l, so each load covers 512 contiguous
                // bytes (a round costs one request per line, and their count sets its latency);
                // LDS then hands lane l the tiles [4 l, 4 l + 4) that the pick takes
                unsigned long long q[kPartRegs];
                unsigned n = 0;
                while (!gave_up) {
                    bool missing = false;
#pragma unroll
                    for (int j = 0; j < kPartRegs; ++j) {
                        const int i = kWave * j + lane;
                        q[j] = (i < a.G) ? load_slot(slot + i) : 0ull;
                        missing |= (i < a.G) && q[j] == kEmpty;
                    }
                    if (!__any(missing)) break;
                    if (++n > a.spin) {
                        if (lane == 0) gave_up = 1;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
#pragma unroll
                for (int j = 0; j < kPartRegs; ++j) ptile[kWave * j + lane] = q[j];
                __builtin_amdgcn_wave_barrier();          // the wave's LDS writes before its reads
                float2 p[kPartRegs];
#pragma unroll
                for (int t = 0; t < kPartRegs; ++t) {
                    const int i = lane * kPartRegs + t;
                    p[t] = (i < a.G) ? __builtin_bit_cast(float2, ptile[i]) : make_float2(-INFINITY, 0.0f);
                }
                if (!gave_up) {
                    tp = pick_tile<kPartRegs>(p, a.u[k]);
                    known = true;
                    if (lane == 0) {
                        const unsigned long long id = static_cast<uint32_t>(tp.tile + 1);
                        store_token(pk, (static_cast<unsigned long long>(__float_as_uint(tp.m)) << 32) | id);
                        store_token(pk + 1, (static_cast<unsigned long long>(__float_as_uint(tp.tprime)) << 32) | id);
                    }
                }
            }
            // every workgroup: the token from its slot, or, in the owner of the picked tile, from a
            // rescan of its logits in LDS in token order (lane l owns the 10 columns from 10 l)
            bool have = known && tp.tile < 0;             // no mass: no token
            for (unsigned n2 = 0; !gave_up && !have;) {
                if (known && tp.tile == static_cast<int>(blockIdx.x)) {
                    float lv[kLaneCols], e[kLaneCols];
#pragma unroll
                    for (int j = 0; j < kLaneCols; ++j) {
                        lv[j] = tl[lane * kLaneCols + j];
                        e[j] = (lv[j] == -INFINITY) ? 0.0f : __expf(lv[j] - tp.m);
                    }
                    t = scan_pick<kLaneCols>(e, c0 + lane * kLaneCols, tp.tprime);
                    const int rel = t - static_cast<int>(c0);
                    const int owner = rel / kLaneCols, jj = rel - owner * kLaneCols;
                    float mine = 0.0f;
#pragma unroll
                    for (int j = 0; j < kLaneCols; ++j)
                        if (j == jj) mine = lv[j];
                    lx = wave_bcast(mine, owner);
                    if (lane == 0)
                        store_token(a.toks + k, (static_cast<unsigned long long>(__float_as_uint(lx)) << 32) |
                                                    static_cast<uint32_t>(t));
                    have = true;
                    break;
                }
                // one round: the pick words (until known) and the token slot, loaded together
                unsigned long long w0 = 0ull, w1 = 0ull;
                if (!known) {
                    w0 = load_token(pk);
                    w1 = load_token(pk + 1);
                }
                const unsigned long long v = load_token(a.toks + k);
                if (v != kEmpty) {
                    t = static_cast<int>(static_cast<uint32_t>(v));
                    lx = __uint_as_float(static_cast<uint32_t>(v >> 32));
                    have = true;
                    break;
                }
                if (!known && w0 != kEmpty && w1 != kEmpty) {
                    tp.tile = static_cast<int>(static_cast<uint32_t>(w0)) - 1;
                    tp.m = __uint_as_float(static_cast<uint32_t>(w0 >> 32));
                    tp.tprime = __uint_as_float(static_cast<uint32_t>(w1 >> 32));
                    known = true;
                    have = tp.tile < 0;
                    continue;                             // the owner rescans at once
                }
                if (++n2 > a.spin) {
                    if (lane == 0) gave_up = 1;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            if (!gave_up) {
                if (blockIdx.x == 0 && lane == 0) {          // workgroup 0 writes the outputs
                    const DrawOut out{a.x_out + k, a.q_out ? a.q_out + k : nullptr,
                                      a.lse_out ? a.lse_out + k : nullptr, true};
                    if (tp.tile < 0) put(out, -1, 0.0f, -INFINITY);
                    else put(out, t, __expf(lx - tp.lse), tp.lse);
                }
                if (lane == 0) stok = t;
                if (k + 1 < a.gamma && lane < kResMaxRank / 8) {
                    uint4 hn = make_uint4(0u, 0u, 0u, 0u);
                    if (t >= 0 && 8 * lane < r)
                        hn = *reinterpret_cast<const uint4*>(a.W1 + static_cast<long long>(t) * r + 8 * lane);
                    reinterpret_cast<uint4*>(hs)[lane] = hn;
                }
            }
        }
        else if (RNN && wave >= kRWaves / 2 && k + 1 < a.gamma) {
            // A h_k: thread (p, half) forms rows 2p, 2p+1 over j in [128 half, 128 half + 128)
            const int t2 = tid - kRThreads / 2;
            const int pp = t2 & (kResMaxRank / 2 - 1), jh = t2 >> 7;
            const int j0 = jh * (kResMaxRank / 2), j1 = min(j0 + kResMaxRank / 2, r);
            float s0 = 0.0f, s1 = 0.0f;
            for (int j = j0; j < j1; ++j) {
                const uint32_t wv = at2[j * (kResMaxRank / 2) + pp];
                const float hj = hst[j];
                s0 = fmaf(__uint_as_float(wv << 16), hj, s0);
                s1 = fmaf(__uint_as_float(wv & 0xffff0000u), hj, s1);
            }
            ah[jh][2 * pp] = s0;
            ah[jh][2 * pp + 1] = s1;
        }
        __syncthreads();
        if (gave_up) break;
        tok = stok;
        if (RNN && k + 1 < a.gamma) {
            // h_{k+1} = A h_k + W1[x_k] (hs holds W1[x_k] as bf16 pairs, zero for no token)
            if (tid < kResMaxRank) {
                const uint32_t pr = hs[tid >> 1];
                const float w1v = __uint_as_float((tid & 1) ? (pr & 0xffff0000u) : (pr << 16));
                const float h = (tid < r) ? (ah[0][tid] + ah[1][tid]) + w1v : 0.0f;
                hst[tid] = h;
                const __bf16 hi = static_cast<__bf16>(h);
                const __bf16 lo = static_cast<__bf16>(h - static_cast<float>(hi));
                reinterpret_cast<uint16_t*>(hhi)[tid] = __builtin_bit_cast(uint16_t, hi);
                reinterpret_cast<uint16_t*>(hlo)[tid] = __builtin_bit_cast(uint16_t, lo);
            }
            __syncthreads();
        }
    }
    // every workgroup has read E: each published its last partial, which workgroup 0 saw
    // (or the launch gave up, and E moves on all the same)
    if (blockIdx.x == 0 && tid == 0) store_token(a.epoch, s_e0 + 1);
    if (gave_up && tid == 0) __hip_atomic_fetch_add(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (gave_up && blockIdx.x == 0 && tid == 0) {
        for (int i = k; i < a.gamma; ++i) {
            a.x_out[i] = -1;
            if (a.q_out) a.q_out[i] = 0.0f;
            if (a.lse_out) a.lse_out[i] = -INFINITY;
        }
    }
}

struct DeviceFit {
    int cus = -1;
    int occupancy = -1;
};

template <bool RNN>
DeviceFit device_fit() {
    thread_local DeviceFit cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DeviceFit{};
    DeviceFit& f = cache[dev];
    if (f.cus < 0) {
        int cus = 0, occ = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, draft_resident<RNN>, kRThreads, 0) !=
                hipSuccess)
            return DeviceFit{};
        f.cus = cus;
        f.occupancy = occ;
    }
    return f;
}

int tiles_of(int V) { return (V + kResTileCols - 1) / kResTileCols; }

template <bool RNN>
bool fits(int V, int r, const void* W1, const void* W2) {
    if (r > kResMaxRank || (r % 8) != 0 || (V % 8) != 0) return false;
    if ((reinterpret_cast<uintptr_t>(W1) % 16) != 0 || (reinterpret_cast<uintptr_t>(W2) % 16) != 0)
        return false;
    const DeviceFit f = device_fit<RNN>();
    const int G = tiles_of(V);
    return f.cus > 0 && f.occupancy >= 1 && G <= f.cus && G <= kMaxTiles;
}

template <bool RNN>
hipError_t launch(const DraftCall& c, const void* A, float* h_out, hipStream_t st) {
    ResArgs a;
    a.V = c.V; a.r = c.r; a.gamma = c.gamma;
    a.G = tiles_of(c.V);
    a.U = c.U;
    a.W1 = static_cast<const uint16_t*>(c.W1);
    a.W2 = static_cast<const uint16_t*>(c.W2);
    a.x0 = c.x0; a.u = c.u;
    a.x_out = c.x_out; a.q_out = c.q_out; a.lse_out = c.lse_out;
    for (int k = 0; k < c.gamma; ++k) a.L[k] = c.L[k];
    a.L_out = c.L_out ? 1 : 0;
    a.slots = c.slots;
    a.toks = reinterpret_cast<unsigned long long*>(c.slots + static_cast<long long>(c.gamma) * a.G);
    a.picks = a.toks + c.gamma;
    a.epoch = a.picks + 2 * c.gamma;
    a.status = c.status;
    a.spin = c.spin;
    a.A = static_cast<const uint16_t*>(A);
    a.h_out = h_out;
    a.with_job = (!RNN && c.job) ? 1 : 0;
    if (a.with_job) a.job = *c.job;
    hipLaunchKernelGGL(draft_resident<RNN>, dim3(a.G + a.with_job), dim3(kRThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

// tile partials [gamma][G], the token slots [gamma], the pick words [gamma][2], then the call
// counter and ready word
size_t draft_resident_slot_bytes(int V, int gamma) {
    return static_cast<size_t>(gamma) * tiles_of(V) * sizeof(float2) +
           (3 * static_cast<size_t>(gamma) + 2) * sizeof(unsigned long long);
}

bool draft_resident_ok(int B, int V, int r, int w_dtype, const void* W1, const void* W2) {
    return B == 1 && w_dtype == 1 && fits<false>(V, r, W1, W2);
}

bool draft_resident_takes_job(int V) {
    const DeviceFit f = device_fit<false>();
    return f.cus > 0 && f.occupancy >= 1 &&
           static_cast<long long>(tiles_of(V)) + 1 <= static_cast<long long>(f.cus) * f.occupancy;
}

hipError_t launch_draft_resident(const DraftCall& c, hipStream_t st) {
    return launch<false>(c, nullptr, nullptr, st);
}

bool rnn_resident_ok(int B, int V, int r, const void* W1, const void* W2, const void* A) {
    return B == 1 && (reinterpret_cast<uintptr_t>(A) % 16) == 0 && fits<true>(V, r, W1, W2);
}

hipError_t launch_rnn_resident(const RnnCall& c, hipStream_t st) {
    return launch<true>(c.d, c.A, c.h_out, st);
}

}  // namespace dspark
