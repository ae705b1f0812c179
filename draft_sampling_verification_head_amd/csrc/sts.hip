// Sequential temperature scaling (STS) fit and expected calibration error (gfx950).
//
// [P1] "大模型推理加速的系统级工程：DeepSeek V4-Pro DSpark 推测解码方案深度解析与开源工具链
// DeepSpec" (Best Partners TV), section "硬件感知与置信度自适应调度机制": the confidence
// head's raw scores are over-confident; one temperature per candidate position, found by a
// one-dimensional grid search on validation data, calibrates them (the expected calibration
// error falls to about 1 %) and keeps their order. [P3] "DSpark Speculative Decoding",
// section "Confidence-Scheduled Verification": c_k estimates P(position k accepted | prefix
// accepted).
//
// Validation pairs come from verify's results: for request i, positions k < n_i were
// accepted, position n_i was rejected when n_i < len_i, later positions were not observed.
// The calibrated score is sigmoid(logit(c) / T) = 1 / (1 + exp(g / T)) with the log-odds
// complement g = log((1 - c) / c), in fp64. Three launches:
//   sts_prep   - the outcome of every pair and, for the observed ones, g (+inf for c <= 0
//                or NaN, -inf for c >= 1, so that the same expression gives the scores 0
//                and 1 there), one contiguous column per position;
//   sts_stats  - one workgroup per (position, five or four grid temperatures, slice of
//                the samples). Each wave packs the observed samples of its 64-sample chunks
//                into an LDS queue, in sample order, and evaluates full waves of them at the
//                workgroup's temperatures: the NLL summed per lane in queue order, and per ECE bin
//                the sum of (outcome - score), rounded per sample to 2^-30 and added as
//                integers (exact, so the order of the adds does not matter);
//   sts_pick   - one wave per position: the slices' partials summed in slice order, the
//                objective per temperature (NLL, or the ECE: over the bins,
//                |sum(outcome - score)| / observed count, which equals count / N times
//                |mean outcome - mean score|), the first minimum, the ECE before and after.
// Every sum has a fixed order or is exact, so reruns are bitwise identical.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kStsThreads = 256;
constexpr int kStsWaves = kStsThreads / kWave;
constexpr int kStsMaxBins = 16;
constexpr int kStsMinSlice = 2048;             // samples per workgroup, at least
constexpr int kStsTargetGroups = 2048;         // slices are added up to about this grid
constexpr int kPart = 2 + kStsMaxBins;         // words per partial: NLL, count, bin sums
constexpr int kBatch = 4;                      // 64-sample chunks loaded together
constexpr int kQueue = 8 * kWave;              // per-wave queue: < 64 left + kBatch * 64 new
constexpr double kStsEps = 1e-12;
constexpr double kFix = 1073741824.0;          // 2^30: |outcome - score| * 2^30 fits an int32

struct StsShape {
    int temps;         // temperatures per workgroup: 5 when they divide nT + 1, else 4
    int groups;        // temperature groups (the last one may be partial)
    int S;             // slices of the samples
    long long slice;   // samples per slice
};

StsShape sts_shape(int N, int G, int nT) {
    StsShape s;
    s.temps = ((nT + 1) % 5 == 0) ? 5 : 4;
    s.groups = (nT + 1 + s.temps - 1) / s.temps;
    const long long cells = static_cast<long long>(G) * s.groups;
    const long long want = (kStsTargetGroups + cells - 1) / cells;
    const long long most = (static_cast<long long>(N) + kStsMinSlice - 1) / kStsMinSlice;
    s.S = static_cast<int>(std::max(1LL, std::min(want, most)));
    s.slice = (static_cast<long long>(N) + s.S - 1) / s.S;
    return s;
}

// One workgroup per tile of T = 256 / gamma samples (one score per thread): the tile's
// scores and outcomes are read in their [N][gamma] order and transposed through LDS, then
// written as contiguous columns; g is formed in the second pass and only for observed pairs
// (the sweep reads no other), so the late positions, mostly unobserved, skip the logarithm.
__global__ __launch_bounds__(kStsThreads)
void sts_prep(int N, int G, const float* __restrict__ conf, const int32_t* __restrict__ n_acc,
              const int32_t* __restrict__ len, double* __restrict__ gt, int8_t* __restrict__ ot) {
    __shared__ float lc[kStsThreads + 64];                // [position][T + 1], padded rows
    __shared__ int8_t lo[kStsThreads + 64];
    const int T = kStsThreads / G;                         // G <= 64, so T >= 4
    const long long s0 = static_cast<long long>(blockIdx.x) * T;
    const int tid = threadIdx.x;
    if (tid < T * G) {
        const int j = tid / G, k = tid - j * G;
        const long long s = s0 + j;
        if (s < N) {
            const int n = n_acc[s];
            const int ell = len ? len[s] : G;
            int8_t o = -1;
            if (n >= 0 && ell >= 0) {
                if (k < n) o = 1;
                else if (k == n && n < ell) o = 0;
            }
            lc[k * (T + 1) + j] = conf[s * G + k];
            lo[k * (T + 1) + j] = o;
        }
    }
    __syncthreads();
    if (tid < T * G) {
        const int k = tid / T, j = tid - k * T;
        const long long s = s0 + j;
        if (s < N) {
            const int8_t o = lo[k * (T + 1) + j];
            double g = 0.0;                                // unobserved: never read
            if (o >= 0) {
                const double c = static_cast<double>(lc[k * (T + 1) + j]);
                if (!(c > 0.0)) g = INFINITY;             // also NaN: score 0 at every T
                else if (c >= 1.0) g = -INFINITY;         // score 1 at every T
                else g = log((1.0 - c) / c);
            }
            gt[static_cast<long long>(k) * N + s] = g;
            ot[static_cast<long long>(k) * N + s] = o;
        }
    }
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// part[((k * (nT + 1) + t) * S + s) * kPart + j]: j = 0 the NLL (fp64 bits), 1 the observed
// count, 2 + m the fixed-point sum of (outcome - score) over bin m.
template <int TG>
__global__ __launch_bounds__(kStsThreads)
void sts_stats(int N, int nT, const float* __restrict__ grid, int bins, int S, long long slice,
               const double* __restrict__ gt, const int8_t* __restrict__ ot,
               unsigned long long* __restrict__ part) {
    __shared__ long long dsum[TG][kStsMaxBins];
    __shared__ double qg[kStsWaves][kQueue];
    __shared__ int8_t qo[kStsWaves][kQueue];
    __shared__ double wnll[kStsWaves][TG];
    __shared__ int wobs[kStsWaves];
    const int groups = (nT + 1 + TG - 1) / TG;
    unsigned id = blockIdx.x;
    const int s = static_cast<int>(id % static_cast<unsigned>(S));
    id /= static_cast<unsigned>(S);
    const int tg = static_cast<int>(id % static_cast<unsigned>(groups));
    const int k = static_cast<int>(id / static_cast<unsigned>(groups));
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;

    // 1 / T per temperature (T = 1 for the "before" slot nT and the unused tail of the last
    // group; T <= 0 or NaN counts as 1; an infinite T gives a tiny positive factor, so that
    // finite g give exp(0) = 1 and the edge scores stay 0 and 1)
    double inv[TG];
#pragma unroll
    for (int j = 0; j < TG; ++j) {
        const int t = tg * TG + j;
        double T = (t < nT) ? static_cast<double>(grid[t]) : 1.0;
        if (!(T > 0.0)) T = 1.0;
        inv[j] = isinf(T) ? 1e-300 : 1.0 / T;
    }
    if (tid < TG * kStsMaxBins) (&dsum[0][0])[tid] = 0;
    __syncthreads();

    const double* g = gt + static_cast<long long>(k) * N;
    const int8_t* o = ot + static_cast<long long>(k) * N;
    const long long s0 = static_cast<long long>(s) * slice;
    const long long s1 = std::min(static_cast<long long>(N), s0 + slice);
    double nll[TG];
#pragma unroll
    for (int j = 0; j < TG; ++j) nll[j] = 0.0;
    int nobs = 0;
    int head = 0, tail = 0;           // wave-uniform queue positions (entries modulo kQueue)

    auto eval = [&](bool on) {
        const int e = (head + lane) & (kQueue - 1);
        const double gv = qg[wave][e];
        const int ov = qo[wave][e];
        if (on) {
            ++nobs;
#pragma unroll
            for (int j = 0; j < TG; ++j) {
                const double cs = 1.0 / (1.0 + exp(gv * inv[j]));
                const double p = ov ? cs : 1.0 - cs;
                nll[j] -= log(fmax(p, kStsEps));
                const int b = min(static_cast<int>(floor(cs * bins)), bins - 1);
                const int q = static_cast<int>(rint((static_cast<double>(ov) - cs) * kFix));
                __hip_atomic_fetch_add(&dsum[j][b], static_cast<long long>(q), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
    };

    // chunks are taken kBatch at a time: their loads are all in flight before the first is
    // queued, since at the sparse late positions the loop is otherwise one load latency per
    // chunk with little to evaluate
    for (long long c0 = s0 + static_cast<long long>(kWave) * wave; c0 < s1;
         c0 += static_cast<long long>(kWave) * kStsWaves * kBatch) {
        int ov[kBatch];
        double gv[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const long long i = c0 + static_cast<long long>(kWave) * kStsWaves * u + lane;
            ov[u] = -1;
            gv[u] = 0.0;
            if (i < s1) {
                ov[u] = o[i];
                gv[u] = g[i];
            }
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const unsigned long long m = __ballot(ov[u] >= 0);
            if (ov[u] >= 0) {
                const int e = (tail + __popcll(m & ((1ull << lane) - 1ull))) & (kQueue - 1);
                qg[wave][e] = gv[u];
                qo[wave][e] = static_cast<int8_t>(ov[u]);
            }
            tail += __popcll(m);
        }
        while (tail - head >= kWave) {                // full waves of observed samples
            eval(true);
            head += kWave;
        }
    }
    if (tail > head) eval(lane < tail - head);

#pragma unroll
    for (int j = 0; j < TG; ++j) nll[j] = wave_sum_f64(nll[j]);
    nobs = wave_sum_i32(nobs);
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < TG; ++j) wnll[wave][j] = nll[j];
        wobs[wave] = nobs;
    }
    __syncthreads();
    if (tid < TG) {
        const int t = tg * TG + tid;
        if (t <= nT) {
            double v = wnll[0][tid];
            long long n = wobs[0];
#pragma unroll
            for (int w = 1; w < kStsWaves; ++w) {
                v += wnll[w][tid];
                n += wobs[w];
            }
            unsigned long long* pp =
                part + ((static_cast<long long>(k) * (nT + 1) + t) * S + s) * kPart;
            pp[0] = static_cast<unsigned long long>(__double_as_longlong(v));
            pp[1] = static_cast<unsigned long long>(n);
            for (int m = 0; m < bins; ++m) pp[2 + m] = static_cast<unsigned long long>(dsum[tid][m]);
        }
    }
}

// The partials of (position, temperature) p[s * kPart + j], summed over the S slices in order.
__device__ double nll_of(const unsigned long long* p, int S) {
    double v = 0.0;
#pragma unroll 8
    for (int s = 0; s < S; ++s) v += __longlong_as_double(static_cast<long long>(p[s * kPart]));
    return v;
}

// The ECE from the partials, by one wave: lane l adds bin l % 16 (and, in lane 0, the
// observed count) over the slices l / 16, l / 16 + 4, ...; the integer sums are exact, so
// the lanes' order does not matter.
__device__ double ece_wave(const unsigned long long* p, int S, int bins, int lane) {
    const int m = lane & 15;
    long long d = 0, n = 0;
    for (int s = lane >> 4; s < S; s += 4) {
        if (m < bins) d += static_cast<long long>(p[s * kPart + 2 + m]);
        if (m == 0) n += static_cast<long long>(p[s * kPart + 1]);
    }
    d += __shfl_xor(d, 16, kWave);
    d += __shfl_xor(d, 32, kWave);
    n += __shfl_xor(n, 16, kWave);
    n += __shfl_xor(n, 32, kWave);
    long long a = (m < bins) ? (d < 0 ? -d : d) : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) a += __shfl_xor(a, o, kWave);
    const long long nobs = __shfl(n, 0, kWave);
    if (nobs == 0) return 0.0;
    return static_cast<double>(__shfl(a, 0, kWave)) / kFix / static_cast<double>(nobs);
}

// The same ECE by one lane (the objective of one temperature).
__device__ double ece_lane(const unsigned long long* p, int S, int bins) {
    long long nobs = 0;
    for (int s = 0; s < S; ++s) nobs += static_cast<long long>(p[s * kPart + 1]);
    if (nobs == 0) return 0.0;
    long long e = 0;
    for (int m = 0; m < bins; ++m) {
        long long d = 0;
        for (int s = 0; s < S; ++s) d += static_cast<long long>(p[s * kPart + 2 + m]);
        e += d < 0 ? -d : d;
    }
    return static_cast<double>(e) / kFix / static_cast<double>(nobs);
}

// One wave per position; lane-strided objectives, first minimum by (value, index).
__global__ __launch_bounds__(kWave)
void sts_pick(int G, int nT, const float* __restrict__ grid, int bins, int objective, int S,
              const unsigned long long* __restrict__ part, float* __restrict__ T_out,
              float* __restrict__ ece_before, float* __restrict__ ece_after,
              float* __restrict__ obj_out) {
    const int k = blockIdx.x, lane = threadIdx.x;
    const long long per_t = static_cast<long long>(S) * kPart;
    const unsigned long long* pk = part + static_cast<long long>(k) * (nT + 1) * per_t;
    double best = INFINITY;
    int bi = INT32_MAX;
    for (int t = lane; t < nT; t += kWave) {
        const unsigned long long* p = pk + t * per_t;
        const double v = (objective == 0) ? nll_of(p, S) : ece_lane(p, S, bins);
        if (obj_out) obj_out[static_cast<long long>(k) * nT + t] = static_cast<float>(v);
        if (v < best) {                                   // lane-strided: first t wins ties
            best = v;
            bi = t;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const double ov = __shfl_xor(best, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (ov < best || (ov == best && oi < bi)) {
            best = ov;
            bi = oi;
        }
    }
    if (bi == INT32_MAX) bi = 0;                          // every objective NaN: first value
    const double before = ece_wave(pk + nT * per_t, S, bins, lane);
    const double after = ece_wave(pk + bi * per_t, S, bins, lane);
    if (lane == 0) {
        T_out[k] = grid[bi];
        ece_before[k] = static_cast<float>(before);
        ece_after[k] = static_cast<float>(after);
    }
}

}  // namespace

int sts_max_bins() { return kStsMaxBins; }

size_t sts_stats_bytes(int N, int gamma, int n_grid) {
    const StsShape s = sts_shape(N, gamma, n_grid);
    return static_cast<size_t>(gamma) * (n_grid + 1) * s.S * kPart * sizeof(unsigned long long);
}

hipError_t launch_sts_fit(int N, int G, const float* conf, const int32_t* n_acc,
                          const int32_t* len, const float* grid, int nT, int bins, int objective,
                          double* gt, int8_t* ot, unsigned long long* part, float* T_out,
                          float* ece_before, float* ece_after, float* obj_out, hipStream_t st) {
    const int tile = kStsThreads / G;
    hipLaunchKernelGGL(sts_prep, dim3(static_cast<unsigned>((N + tile - 1) / tile)),
                       dim3(kStsThreads), 0, st, N, G, conf, n_acc, len, gt, ot);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const StsShape sh = sts_shape(N, G, nT);
    const dim3 nblk(static_cast<unsigned>(static_cast<long long>(G) * sh.groups * sh.S));
    if (sh.temps == 5)
        hipLaunchKernelGGL(sts_stats<5>, nblk, dim3(kStsThreads), 0, st, N, nT, grid, bins, sh.S,
                           sh.slice, gt, ot, part);
    else
        hipLaunchKernelGGL(sts_stats<4>, nblk, dim3(kStsThreads), 0, st, N, nT, grid, bins, sh.S,
                           sh.slice, gt, ot, part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sts_pick, dim3(G), dim3(kWave), 0, st, G, nT, grid, bins, objective, sh.S,
                       part, T_out, ece_before, ece_after, obj_out);
    return hipGetLastError();
}

}  // namespace dspark
