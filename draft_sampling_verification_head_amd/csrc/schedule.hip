// Hardware-aware prefix scheduler kernel (gfx950), one workgroup.
//
// [P1] "大模型推理加速的系统级工程：DeepSeek V4-Pro DSpark 推测解码方案深度解析与开源工具链
// DeepSpec" (Best Partners TV), section "硬件感知与置信度自适应调度机制", and [P3] "DSpark
// Speculative Decoding", section "Confidence-Scheduled Verification":
//   c'_{r,j} = 1 / (1 + ((1 - c)/c)^(1/T_j))      per-position temperature (order preserving)
//   a_{r,j}  = prod_{i<=j} c'_{r,i}                 prefix survival
//   rank all candidates by a (descending), add them one by one and keep the batch size n
//   that maximises Theta(n) = (R + sum of the top-n a) * SPS(R + n) (global search), or stop
//   at the first n where Theta stops rising (early stopping).
//
// Ranking: one 64-bit key per candidate, key = (~a_bits[63:20]) << 20 | j << 14 | r, so that
// ascending keys mean descending a, then position ascending, then request ascending. The kept
// 44 bits of the fp64 a (sign, exponent, 32 mantissa bits) carry the sums. Lengths come from
// one cut key: request r keeps its candidates whose key is below the key at rank n*; since
// a is non-increasing along a block and ties rank earlier positions first, that set is a
// prefix of every block. Up to 64 candidates run in one wave (schedule_small_kernel); more
// run as a rank pass over many workgroups followed by one pick workgroup.
//
// Two-step-lag confidences ([P1] same section, the asynchronous adaptation; [P3] same
// section, the batch capacity predicted from confidences two steps old): a ring of three
// [R][gamma] slots and a round counter n in device memory. A push stores the round's
// confidences in slot n mod 3 and advances n; the lagged schedule reads slot (n - 2) mod 3,
// the confidences pushed two rounds before the next push (all 1.0 until two pushes exist).
// The slot is resolved on the device, so a captured round needs no host round trip.
#include "common.h"
#include "kernels.h"
#include "schedule_small.h"

namespace dspark {

namespace {

using namespace sched;

constexpr int kMaxCand = 16384;            // 128 KB of keys in LDS
__global__ __launch_bounds__(kWave)
void schedule_small_kernel(SmallJob job) {
    __shared__ double cs[kSmallCand];
    __shared__ double sorted[kSmallCand];
    schedule_small<true>(job, cs, sorted);
}

// ---------------------------------------------------------------- many candidates
// Along a request's block the keys increase strictly (a is non-increasing in j and ties
// rank the earlier position first), so a candidate's rank is the sum over requests of a
// binary search in that request's row of keys. schedule_rank_kernel: every workgroup loads
// all keys into LDS and ranks 16 candidates, 16 threads per candidate splitting the
// requests; the ranked keys are scattered into sorted order (the keys themselves come from a
// one-thread-per-request kernel before). schedule_pick_kernel: one
// workgroup scans the ranked values into S(n), evaluates Theta, finds n* and counts each
// request's candidates ranked before n*.
constexpr int kRankThreads = 256;
constexpr int kRankSplit = 16;                              // threads per candidate
constexpr int kRankPerBlock = kRankThreads / kRankSplit;

// keys of every candidate: the temperature-scaled confidences in parallel (one thread per
// candidate), then the prefix products of each request in position order (one thread per
// request, as the oracle multiplies). A workgroup covers whole requests.
__global__ __launch_bounds__(kRankThreads)
void schedule_keys_kernel(int R, int G, const float* __restrict__ conf_in,
                          const long long* __restrict__ ring_n,
                          const float* __restrict__ temp, float* __restrict__ a_out,
                          unsigned long long* __restrict__ row_keys) {
    const float* conf = lagged(conf_in, ring_n, R, G);
    __shared__ double cs[kRankThreads];
    const int per = kRankThreads / G;                        // requests per workgroup
    const int rb = blockIdx.x * per;
    const int tid = threadIdx.x;
    const int i = rb * G + tid;
    if (tid < per * G && i < R * G) cs[tid] = scaled_conf(conf[i], temp, tid % G);
    __syncthreads();
    const int r = rb + tid;
    if (tid < per && r < R) {
        double a = 1.0;
        for (int j = 0; j < G; ++j) {
            a *= cs[tid * G + j];
            const int k = r * G + j;
            row_keys[k] = make_key(a, j, r);
            if (a_out) a_out[k] = static_cast<float>(a);
        }
    }
}

// number of keys of one row (strictly increasing, length G <= 64) below `key`
__device__ __forceinline__ int count_below(const unsigned long long* row, int G,
                                           unsigned long long key) {
    int lo = 0;
#pragma unroll
    for (int step = 64; step > 0; step >>= 1) {           // branch-free: always an in-row read
        const unsigned long long v = row[min(lo + step, G) - 1];
        lo += (lo + step <= G && v < key) ? step : 0;
    }
    return lo;
}

__host__ __device__ inline int rank_stride(int R, int G) {
    return (static_cast<long long>(R) * (G + 1) <= kMaxCand) ? G + 1 : G;
}

// Rows sit in LDS at a stride of G + 1 keys when that fits, and the 16 threads of a
// candidate take interleaved requests, so their reads fall on different banks.
__global__ __launch_bounds__(kRankThreads)
void schedule_rank_kernel(int R, int G, const unsigned long long* __restrict__ row_keys,
                          unsigned long long* __restrict__ sorted_keys,
                          int32_t* __restrict__ ranks) {
    extern __shared__ unsigned long long keys[];             // R rows at stride S
    const int tid = threadIdx.x;
    const int N = R * G;
    const int S = rank_stride(R, G);
    constexpr int kBatch = 8;                                 // loads in flight per thread
    for (int i0 = tid; i0 < N; i0 += kBatch * kRankThreads) {
        unsigned long long v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int i = i0 + q * kRankThreads;
            v[q] = (i < N) ? row_keys[i] : 0ull;
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int i = i0 + q * kRankThreads;
            if (i < N) {
                const int r = i / G;
                keys[static_cast<long long>(r) * S + (i - r * G)] = v[q];
            }
        }
    }
    __syncthreads();
    const int cand = blockIdx.x * kRankPerBlock + tid / kRankSplit, part = tid % kRankSplit;
    if (cand >= N) return;                                   // whole groups leave together
    const unsigned long long key = row_keys[cand];
    int cnt = 0;
    int r = part;
    for (; r + 3 * kRankSplit < R; r += 4 * kRankSplit) {    // four independent searches
        const int c0 = count_below(keys + static_cast<long long>(r) * S, G, key);
        const int c1 = count_below(keys + static_cast<long long>(r + kRankSplit) * S, G, key);
        const int c2 = count_below(keys + static_cast<long long>(r + 2 * kRankSplit) * S, G, key);
        const int c3 = count_below(keys + static_cast<long long>(r + 3 * kRankSplit) * S, G, key);
        cnt += (c0 + c1) + (c2 + c3);
    }
    for (; r < R; r += kRankSplit) cnt += count_below(keys + static_cast<long long>(r) * S, G, key);
#pragma unroll
    for (int o = 1; o < kRankSplit; o <<= 1) cnt += __shfl_xor(cnt, o, kWave);
    if (part == 0) {
        sorted_keys[cnt] = key;
        ranks[cand] = cnt;
    }
}

constexpr int kPickThreads = 1024;
constexpr int kPickMaxE = kMaxCand / kPickThreads;            // ranks per thread at the cap

__global__ __launch_bounds__(kPickThreads)
void schedule_pick_kernel(int R, int G, const float* __restrict__ sps, int Bmax, int mode,
                          const int32_t* __restrict__ ranks,
                          const unsigned long long* __restrict__ sorted_keys,
                          int32_t* __restrict__ len_out, int32_t* __restrict__ t_off_out,
                          int32_t* __restrict__ K_out, float* __restrict__ theta_out) {
    __shared__ double dscr[kPickThreads / kWave + 1];
    __shared__ int iscr[kPickThreads / kWave + 1];
    __shared__ double bth[kPickThreads / kWave];
    __shared__ int bn[kPickThreads / kWave];
    __shared__ int s_nstar;
    __shared__ double s_theta;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int N = R * G;
    const int nmax = min(N, Bmax - R);
    const int E = (N + kPickThreads - 1) / kPickThreads;     // ranks per thread (<= 16)
    const int p0 = tid * E;
    double val[kPickMaxE], spv[kPickMaxE + 1];                // loads issued together
#pragma unroll
    for (int e = 0; e < kPickMaxE; ++e) {
        const int p = p0 + e;
        val[e] = (e < E && p < N) ? key_value(sorted_keys[p]) : 0.0;
    }
#pragma unroll
    for (int e = 0; e <= kPickMaxE; ++e) {
        const int n = p0 + e;
        spv[e] = (e <= E && n <= nmax) ? static_cast<double>(sps[R + n]) : 0.0;
    }
    double local = 0.0;
#pragma unroll
    for (int e = 0; e < kPickMaxE; ++e) local += val[e];
    double tot;
    const double S0 = block_excl_scan<kPickThreads>(local, dscr, &tot);   // S(p0)
    Best best{-INFINITY, INT32_MAX};
    int first_drop = INT32_MAX;
    {
        double S = S0, th_prev = 0.0;
        bool have_prev = false;
        if (p0 <= nmax) {
            th_prev = (static_cast<double>(R) + S) * spv[0];
            have_prev = true;
            best = better(best, Best{th_prev, p0});
        }
#pragma unroll
        for (int e = 0; e < kPickMaxE; ++e) {
            const int n = p0 + e + 1;
            if (e < E && n <= nmax) {
                S += val[e];
                const double th = (static_cast<double>(R) + S) * spv[e + 1];
                if (have_prev && th <= th_prev && first_drop == INT32_MAX) first_drop = n - 1;
                best = better(best, Best{th, n});
                th_prev = th;
                have_prev = true;
            }
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        Best other{__shfl_xor(best.theta, o, kWave), __shfl_xor(best.n, o, kWave)};
        best = better(best, other);
    }
    if (lane == 0) {
        bth[wave] = best.theta;
        bn[wave] = best.n;
    }
    const int drop = block_min_int<kPickThreads>(first_drop, iscr);   // contains a barrier
    if (tid == 0) {
        Best bb{bth[0], bn[0]};
        for (int w = 1; w < kPickThreads / kWave; ++w) bb = better(bb, Best{bth[w], bn[w]});
        s_nstar = (mode == 1) ? ((drop == INT32_MAX) ? nmax : drop)
                              : ((bb.n == INT32_MAX) ? 0 : bb.n);
    }
    __syncthreads();
    const int nstar = s_nstar;
    {
        const bool mine = (nstar == 0) ? (tid == 0) : (nstar > p0 && nstar <= p0 + E);
        if (mine) {
            double S = S0;
#pragma unroll
            for (int e = 0; e < kPickMaxE; ++e)
                if (p0 + e + 1 <= nstar) S += val[e];
            if (nstar == 0) S = 0.0;
            s_theta = (static_cast<double>(R) + S) * static_cast<double>(sps[R + nstar]);
        }
    }
    __syncthreads();
    // lengths: candidates of request r below the cut (a prefix of its row)
    int run = 0;
    for (int base = 0; base < R; base += kPickThreads) {
        const int r = base + tid;
        int cnt = 0;
        if (r < R) {                                          // ranks of the block, loaded together
            const int32_t* rk = ranks + static_cast<long long>(r) * G;
            for (int j0 = 0; j0 < G; j0 += 16) {
                int rv[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) rv[q] = (j0 + q < G) ? rk[j0 + q] : INT32_MAX;
#pragma unroll
                for (int q = 0; q < 16; ++q) cnt += rv[q] < nstar;
            }
            len_out[r] = cnt;
        }
        if (t_off_out) {
            int total;
            const int ex = block_excl_scan<kPickThreads>((r < R) ? cnt + 1 : 0, iscr, &total);
            if (r < R) t_off_out[r] = run + ex;
            run += total;
        }
    }
    if (tid == 0) {
        if (t_off_out) t_off_out[R] = run;
        if (K_out) *K_out = R + nstar;
        if (theta_out) *theta_out = static_cast<float>(s_theta);
    }
}

// Ring set-up: counter 0, every slot 1.0 (no history yet: every position survives). One
// workgroup; a fill kernel rather than a memset, so that it can sit in a captured graph.
__global__ __launch_bounds__(1024)
void conf_ring_init_kernel(long long* __restrict__ ring_n, float* __restrict__ slots, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) slots[i] = 1.0f;
    if (threadIdx.x == 0) *ring_n = 0;
}

// Push: slot n mod 3 <- conf, then n <- n + 1 once every thread has read n.
__global__ __launch_bounds__(1024)
void conf_ring_push_kernel(long long* __restrict__ ring_n, float* __restrict__ slots,
                           const float* __restrict__ conf, int per_slot) {
    const long long n = *ring_n;
    float* dst = slots + (n % 3) * static_cast<long long>(per_slot);
    for (int i = threadIdx.x; i < per_slot; i += blockDim.x) dst[i] = conf[i];
    __syncthreads();
    if (threadIdx.x == 0) *ring_n = n + 1;
}

}  // namespace

int schedule_max_candidates() { return kMaxCand; }

hipError_t launch_conf_ring_init(long long* ring_n, float* slots, int R, int gamma, hipStream_t st) {
    hipLaunchKernelGGL(conf_ring_init_kernel, dim3(1), dim3(1024), 0, st, ring_n, slots, 3 * R * gamma);
    return hipGetLastError();
}

hipError_t launch_conf_ring_push(long long* ring_n, float* slots, const float* conf, int R, int gamma,
                                 hipStream_t st) {
    hipLaunchKernelGGL(conf_ring_push_kernel, dim3(1), dim3(1024), 0, st, ring_n, slots, conf, R * gamma);
    return hipGetLastError();
}

hipError_t launch_schedule(int R, int gamma, const float* conf, const long long* ring_n,
                           const float* temp, const float* sps, int Bmax, int mode,
                           int32_t* len_out, int32_t* t_off_out, int32_t* K_out, float* theta_out,
                           float* a_out, double* a_ws, hipStream_t st) {
    if (R * gamma <= kSmallCand) {
        const SmallJob job{R, gamma, conf, ring_n, temp, sps, Bmax, mode, len_out, t_off_out, K_out,
                           theta_out, a_out};
        hipLaunchKernelGGL(schedule_small_kernel, dim3(1), dim3(kWave), 0, st, job);
        return hipGetLastError();
    }
    const int N = R * gamma;
    unsigned long long* row_keys = reinterpret_cast<unsigned long long*>(a_ws);
    unsigned long long* sorted_keys = row_keys + N;
    int32_t* ranks = reinterpret_cast<int32_t*>(sorted_keys + N);
    const int per = kRankThreads / gamma;
    hipLaunchKernelGGL(schedule_keys_kernel, dim3((R + per - 1) / per), dim3(kRankThreads), 0, st, R,
                       gamma, conf, ring_n, temp, a_out, row_keys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t lds = static_cast<size_t>(R) * rank_stride(R, gamma) * sizeof(unsigned long long);
    hipLaunchKernelGGL(schedule_rank_kernel, dim3((N + kRankPerBlock - 1) / kRankPerBlock),
                       dim3(kRankThreads), lds, st, R, gamma, row_keys, sorted_keys, ranks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(schedule_pick_kernel, dim3(1), dim3(kPickThreads), 0, st, R, gamma, sps, Bmax,
                       mode, ranks, sorted_keys, len_out, t_off_out, K_out, theta_out);
    return hipGetLastError();
}

}  // namespace dspark
