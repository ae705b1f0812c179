// The one-wave prefix scheduler (up to 64 candidates) and the helpers every scheduler kernel
// shares: the schedule launch runs it in a workgroup of one wave; the single-request draft
// launch can run it in one extra workgroup beside the draft (see schedule.hip for the method:
// [P1] section "硬件感知与置信度自适应调度机制", [P3] "Confidence-Scheduled Verification").
#pragma once

#include "common.h"

namespace dspark {
namespace sched {

constexpr unsigned long long kMask44 = (1ull << 44) - 1ull;

// The confidences a schedule reads: `conf`, or with a ring counter the lagged ring slot.
__device__ __forceinline__ const float* lagged(const float* conf, const long long* ring_n, int R, int G) {
    if (!ring_n) return conf;
    const long long n = *ring_n;
    return conf + ((n + 1) % 3) * static_cast<long long>(R) * G;   // (n - 2) mod 3 for n >= 0
}

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

// The arguments of one schedule call (the outputs as in dspark_schedule).
struct SmallJob {
    int R, G;
    const float* conf;
    const long long* ring_n;     // non-null: the lagged ring slot replaces conf
    const float* temp;
    const float* sps;
    int Bmax, mode;
    int32_t* len_out;
    int32_t* t_off_out;
    int32_t* K_out;
    float* theta_out;
    float* a_out;
};

// One wave for up to 64 candidates (a few short requests): every candidate sits in a lane,
// ranks come from comparing against all keys (read out with v_readlane), and everything
// else is a wave-level scan or reduction. The SPS entries the search reads do not depend on
// the data, so they are loaded together with the confidences. Run by the first wave of a
// workgroup: WG = true in a one-wave workgroup (the exchanges through cs and sorted use
// workgroup barriers); WG = false when the other waves of the workgroup do not take part
// (the exchanges stay inside the wave, whose LDS operations complete in order). cs and
// sorted: 64 doubles of LDS each.
constexpr int kSmallCand = kWave;

template <bool WG>
__device__ __forceinline__ void schedule_small(const SmallJob& job, double* cs, double* sorted) {
    auto sync = [] {
        if (WG) {
            __syncthreads();
        } else {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_s_waitcnt(0xc07f);        // lgkmcnt(0): this wave's LDS writes done
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    };
    const int R = job.R, G = job.G, Bmax = job.Bmax, mode = job.mode;
    const float* __restrict__ conf_in = job.conf;
    const long long* __restrict__ ring_n = job.ring_n;
    const float* __restrict__ temp = job.temp;
    const float* __restrict__ sps = job.sps;
    int32_t* __restrict__ len_out = job.len_out;
    int32_t* __restrict__ t_off_out = job.t_off_out;
    int32_t* __restrict__ K_out = job.K_out;
    float* __restrict__ theta_out = job.theta_out;
    float* __restrict__ a_out = job.a_out;
    const float* conf = lagged(conf_in, ring_n, R, G);
    const int lane = threadIdx.x;
    const int N = R * G;
    const int nmax = min(N, Bmax - R);
    // loads: the candidate's confidence and SPS(R + lane + 1), SPS(R) for n = 0
    const float c = (lane < N) ? conf[lane] : 0.0f;
    const double sps_next = (lane < nmax) ? static_cast<double>(sps[R + lane + 1]) : 0.0;
    const double sps0 = static_cast<double>(sps[R]);
    cs[lane] = (lane < N) ? scaled_conf(c, temp, lane % G) : 0.0;
    sync();
    // prefix products in position order, one lane per request (same order as the oracle)
    if (lane < R) {
        double a = 1.0;
        for (int j = 0; j < G; ++j) {
            a *= cs[lane * G + j];
            cs[lane * G + j] = a;
        }
    }
    sync();
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
    sync();
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

}  // namespace sched
}  // namespace dspark
