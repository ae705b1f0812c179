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
// Layout: one 64-bit key per candidate in LDS, key = (~a_bits[63:20]) << 20 | j << 14 | r,
// so an ascending sort gives a descending, then position ascending, then request ascending.
// The kept 44 bits of the fp64 a (sign, exponent, 32 mantissa bits) carry the sums.
// Lengths come from one cut key: request r keeps its candidates whose key is below the key
// at rank n*. Because a is non-increasing along a block and ties rank earlier positions
// first, that set is a prefix of every block. The fp64 prefix products are kept in the
// caller's workspace between the ranking and the counting.
#include "common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kMaxCand = 16384;            // 128 KB of keys in LDS
constexpr unsigned long long kMask44 = (1ull << 44) - 1ull;

__device__ __forceinline__ double scaled_conf(float c, const float* temp, int j) {
    const double cd = static_cast<double>(c);
    if (!(cd > 0.0)) return 0.0;          // also NaN
    if (cd >= 1.0) return 1.0;
    if (!temp) return cd;
    double T = static_cast<double>(temp[j]);
    if (!(T > 0.0)) T = 1.0;
    return 1.0 / (1.0 + pow((1.0 - cd) / cd, 1.0 / T));
}

__device__ __forceinline__ unsigned long long make_key(double a, int j, int r) {
    const unsigned long long q = static_cast<unsigned long long>(__double_as_longlong(a)) >> 20;
    return (((~q) & kMask44) << 20) | (static_cast<unsigned long long>(j) << 14) |
           static_cast<unsigned long long>(r);
}

__device__ __forceinline__ double key_value(unsigned long long key) {
    const unsigned long long q = (~(key >> 20)) & kMask44;
    return __longlong_as_double(static_cast<long long>(q << 20));
}

struct Best {
    double theta;
    int n;
};

__device__ __forceinline__ Best better(Best a, Best b) {
    // larger Theta wins; equal Theta -> smaller n. NaN Theta never wins.
    if (b.theta > a.theta || (b.theta == a.theta && b.n < a.n) || (a.theta != a.theta)) return b;
    return a;
}

template <int kThreads>
__global__ __launch_bounds__(kThreads)
void schedule_kernel(int R, int G, const float* __restrict__ conf, const float* __restrict__ temp,
                     const float* __restrict__ sps, int Bmax, int mode, int npad,
                     int32_t* __restrict__ len_out, int32_t* __restrict__ t_off_out,
                     int32_t* __restrict__ K_out, float* __restrict__ theta_out,
                     float* __restrict__ a_out, double* __restrict__ a_ws) {
    __shared__ unsigned long long keys[kMaxCand];
    __shared__ double dscr[kThreads / kWave + 1];
    __shared__ int iscr[kThreads / kWave + 1];
    __shared__ double bth[kThreads / kWave];
    __shared__ int bn[kThreads / kWave];
    __shared__ int s_nstar;
    __shared__ double s_theta;

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int N = R * G;

    // 1. temperature-scaled confidences, one candidate per thread (fp64 bits parked in keys)
    for (int i = tid; i < N; i += kThreads)
        keys[i] = static_cast<unsigned long long>(__double_as_longlong(scaled_conf(conf[i], temp, i % G)));
    for (int i = N + tid; i < npad; i += kThreads) keys[i] = ~0ull;
    __syncthreads();
    // 2. prefix products along each block, then the ranking keys
    for (int r = tid; r < R; r += kThreads) {
        double a = 1.0;
        for (int j = 0; j < G; ++j) {
            const int i = r * G + j;
            a *= __longlong_as_double(static_cast<long long>(keys[i]));
            a_ws[i] = a;
            keys[i] = make_key(a, j, r);
            if (a_out) a_out[i] = static_cast<float>(a);
        }
    }
    __syncthreads();

    // 3. bitonic sort, ascending
    for (int kk = 2; kk <= npad; kk <<= 1) {
        for (int jj = kk >> 1; jj > 0; jj >>= 1) {
            for (int i = tid; i < npad; i += kThreads) {
                const int ixj = i ^ jj;
                if (ixj > i) {
                    const unsigned long long x = keys[i], y = keys[ixj];
                    const bool up = (i & kk) == 0;
                    if ((x > y) == up) {
                        keys[i] = y;
                        keys[ixj] = x;
                    }
                }
            }
            __syncthreads();
        }
    }

    // 4. prefix sums of the ranked a, Theta(n) for n = 0..nmax
    const int nmax = min(N, Bmax - R);
    const int E = (npad + kThreads - 1) / kThreads;     // ranks per thread
    const int p0 = tid * E;
    double local = 0.0;
    for (int e = 0; e < E; ++e) {
        const int p = p0 + e;
        if (p < N) local += key_value(keys[p]);
    }
    double tot;
    const double S0 = block_excl_scan<kThreads>(local, dscr, &tot);   // S(p0)

    Best best{-INFINITY, INT32_MAX};
    int first_drop = INT32_MAX;
    {
        double S = S0;
        double th_prev = 0.0;
        bool have_prev = false;
        if (p0 <= nmax) {
            th_prev = (static_cast<double>(R) + S) * static_cast<double>(sps[R + p0]);
            have_prev = true;
            best = better(best, Best{th_prev, p0});
        }
        for (int e = 0; e < E; ++e) {
            const int n = p0 + e + 1;
            if (n > nmax) break;
            S += key_value(keys[n - 1]);
            const double th = (static_cast<double>(R) + S) * static_cast<double>(sps[R + n]);
            if (have_prev && th <= th_prev && first_drop == INT32_MAX) first_drop = n - 1;
            best = better(best, Best{th, n});
            th_prev = th;
            have_prev = true;
        }
    }
    // block reductions
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        Best other{__shfl_xor(best.theta, o, kWave), __shfl_xor(best.n, o, kWave)};
        best = better(best, other);
    }
    if (lane == 0) {
        bth[wave] = best.theta;
        bn[wave] = best.n;
    }
    const int drop = block_min_int<kThreads>(first_drop, iscr);   // contains a barrier
    if (tid == 0) {
        Best bb{bth[0], bn[0]};
        for (int w = 1; w < kThreads / kWave; ++w) bb = better(bb, Best{bth[w], bn[w]});
        int nstar;
        if (mode == 1)
            nstar = (drop == INT32_MAX) ? nmax : drop;
        else
            nstar = (bb.n == INT32_MAX) ? 0 : bb.n;
        s_nstar = nstar;
    }
    __syncthreads();
    const int nstar = s_nstar;

    // Theta(n*) from the thread whose range ends at n*
    {
        const bool mine = (nstar == 0) ? (tid == 0) : (nstar > p0 && nstar <= p0 + E);
        if (mine) {
            double S = S0;
            for (int n = p0 + 1; n <= nstar; ++n) S += key_value(keys[n - 1]);
            if (nstar == 0) S = 0.0;
            s_theta = (static_cast<double>(R) + S) * static_cast<double>(sps[R + nstar]);
        }
    }
    const unsigned long long cut = (nstar < npad) ? keys[nstar] : ~0ull;
    __syncthreads();

    // 5. lengths: candidates ranked above the cut (a_ws rows were written by this thread)
    for (int r = tid; r < R; r += kThreads) {
        int cnt = 0;
        for (int j = 0; j < G; ++j) cnt += make_key(a_ws[r * G + j], j, r) < cut;
        len_out[r] = cnt;
    }

    // 6. offsets: exclusive scan of len + 1
    if (t_off_out) {
        int run = 0;
        for (int base = 0; base < R; base += kThreads) {
            const int r = base + tid;
            const int v = (r < R) ? len_out[r] + 1 : 0;   // written by this same thread above
            int total;
            const int ex = block_excl_scan<kThreads>(v, iscr, &total);
            if (r < R) t_off_out[r] = run + ex;
            run += total;
        }
        if (tid == 0) t_off_out[R] = run;
    }
    if (tid == 0) {
        if (K_out) *K_out = R + nstar;
        if (theta_out) *theta_out = static_cast<float>(s_theta);
    }
}

// One wave for up to 64 candidates (a few short requests): every candidate sits in a lane,
// ranks come from comparing against all keys (read out with v_readlane), and everything
// else is a wave-level scan or reduction. The SPS entries the search reads do not depend on
// the data, so they are loaded together with the confidences.
constexpr int kSmallCand = kWave;

__global__ __launch_bounds__(kWave)
void schedule_small_kernel(int R, int G, const float* __restrict__ conf,
                           const float* __restrict__ temp, const float* __restrict__ sps,
                           int Bmax, int mode, int32_t* __restrict__ len_out,
                           int32_t* __restrict__ t_off_out, int32_t* __restrict__ K_out,
                           float* __restrict__ theta_out, float* __restrict__ a_out) {
    __shared__ double cs[kSmallCand];
    __shared__ double sorted[kSmallCand];
    const int lane = threadIdx.x;
    const int N = R * G;
    const int nmax = min(N, Bmax - R);
    // loads: the candidate's confidence and SPS(R + lane + 1), SPS(R) for n = 0
    const float c = (lane < N) ? conf[lane] : 0.0f;
    const double sps_next = (lane < nmax) ? static_cast<double>(sps[R + lane + 1]) : 0.0;
    const double sps0 = static_cast<double>(sps[R]);
    cs[lane] = (lane < N) ? scaled_conf(c, temp, lane % G) : 0.0;
    __syncthreads();
    // prefix products in position order, one lane per request (same order as the oracle)
    if (lane < R) {
        double a = 1.0;
        for (int j = 0; j < G; ++j) {
            a *= cs[lane * G + j];
            cs[lane * G + j] = a;
        }
    }
    __syncthreads();
    const double a = (lane < N) ? cs[lane] : 0.0;
    if (a_out && lane < N) a_out[lane] = static_cast<float>(a);
    const int r = lane / G, j = lane - r * G;
    const unsigned long long key = (lane < N) ? make_key(a, j, r) : ~0ull;
    // rank = number of smaller keys (keys are distinct: they carry j and r)
    int rank = 0;
    for (int i = 0; i < N; ++i) {
        const unsigned lo = __builtin_amdgcn_readlane(static_cast<unsigned>(key), i);
        const unsigned hi = __builtin_amdgcn_readlane(static_cast<unsigned>(key >> 32), i);
        rank += ((static_cast<unsigned long long>(hi) << 32 | lo) < key) ? 1 : 0;
    }
    if (lane < N) sorted[rank] = key_value(key);
    __syncthreads();
    // S(n) for n = lane + 1: inclusive sum of the ranked values (lane-order fp64 scan)
    double S = (lane < N) ? sorted[lane] : 0.0;
    S = wave_incl_scan(S);
    // Theta(0) and Theta(lane + 1); GLOBAL = smallest argmax, EARLY_STOP = first drop
    const double th0 = static_cast<double>(R) * sps0;
    const bool valid = lane < nmax;
    const double th = valid ? (static_cast<double>(R) + S) * sps_next : -INFINITY;
    double th_prev = __shfl_up(th, 1, kWave);
    if (lane == 0) th_prev = th0;
    const unsigned long long drop = __ballot(valid && th <= th_prev);
    Best best{th0, 0};
    Best mine{th, lane + 1};
    if (valid) best = better(best, mine);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        Best other{__shfl_xor(best.theta, o, kWave), __shfl_xor(best.n, o, kWave)};
        best = better(best, other);
    }
    int nstar;
    if (mode == 1)
        nstar = drop ? (__ffsll(static_cast<long long>(drop)) - 1) : nmax;
    else
        nstar = best.n;
    const double S_star = (nstar == 0) ? 0.0 : __shfl(S, nstar - 1, kWave);
    const double sps_star = (nstar == 0) ? sps0 : __shfl(sps_next, nstar - 1, kWave);
    // lengths: candidates ranked before n*, counted per request
    const bool kept = lane < N && rank < nstar;
    const unsigned long long keptm = __ballot(kept);
    int len = 0;
    if (lane < R) {
        const unsigned long long blockm = ((G == 64) ? ~0ull : ((1ull << G) - 1ull)) << (lane * G);
        len = __popcll(keptm & blockm);
        len_out[lane] = len;
    }
    if (t_off_out) {
        const int v = (lane < R) ? len + 1 : 0;
        const int incl = wave_incl_scan(v);
        if (lane < R) t_off_out[lane] = incl - v;
        if (lane == R - 1) t_off_out[R] = incl;
    }
    if (lane == 0) {
        if (K_out) *K_out = R + nstar;
        if (theta_out) *theta_out = static_cast<float>((static_cast<double>(R) + S_star) * sps_star);
    }
}

}  // namespace

int schedule_max_candidates() { return kMaxCand; }

hipError_t launch_schedule(int R, int gamma, const float* conf, const float* temp,
                           const float* sps, int Bmax, int mode, int32_t* len_out,
                           int32_t* t_off_out, int32_t* K_out, float* theta_out, float* a_out,
                           double* a_ws, hipStream_t st) {
    if (R * gamma <= kSmallCand) {
        hipLaunchKernelGGL(schedule_small_kernel, dim3(1), dim3(kWave), 0, st, R, gamma, conf, temp,
                           sps, Bmax, mode, len_out, t_off_out, K_out, theta_out, a_out);
        return hipGetLastError();
    }
    int npad = 1;
    while (npad < R * gamma) npad <<= 1;
    if (npad <= 2048 && R <= 2048)
        hipLaunchKernelGGL(schedule_kernel<256>, dim3(1), dim3(256), 0, st, R, gamma, conf, temp,
                           sps, Bmax, mode, npad, len_out, t_off_out, K_out, theta_out, a_out,
                           a_ws);
    else
        hipLaunchKernelGGL(schedule_kernel<1024>, dim3(1), dim3(1024), 0, st, R, gamma, conf,
                           temp, sps, Bmax, mode, npad, len_out, t_off_out, K_out, theta_out,
                           a_out, a_ws);
    return hipGetLastError();
}

}  // namespace dspark
