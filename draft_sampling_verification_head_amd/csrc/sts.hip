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
// The calibrated score is sigmoid(logit(c) / T), evaluated as 1 / (1 + exp(log((1-c)/c) / T))
// in fp64. Three launches:
//   sts_prep   - scores and outcomes transposed to one contiguous column per position;
//   sts_stats  - one workgroup per (position, grid temperature, plus T = 1 for the "before"
//                figure) sweeps every sample: NLL sum, and per equal-width bin the count,
//                the accepted count and the score sum. fp64 throughout, reduced in a fixed
//                order (thread-strided sums, then a wave butterfly, then waves in order);
//   sts_pick   - one wave per position: objective per temperature (NLL, or ECE from the bin
//                sums), first minimum, ECE before and after.
#include "common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kStsThreads = 256;
constexpr int kStsWaves = kStsThreads / kWave;
constexpr int kStsMaxBins = 16;
constexpr int kStatVals = 2 + 3 * kStsMaxBins;      // nll, nobs, then cnt / acc / score per bin
constexpr double kStsEps = 1e-12;

__global__ __launch_bounds__(kStsThreads)
void sts_prep(int N, int G, const float* __restrict__ conf, const int32_t* __restrict__ n_acc,
              const int32_t* __restrict__ len, float* __restrict__ ct, int8_t* __restrict__ ot) {
    const long long i = static_cast<long long>(blockIdx.x) * kStsThreads + threadIdx.x;
    if (i >= static_cast<long long>(N) * G) return;
    const int s = static_cast<int>(i / G), k = static_cast<int>(i - static_cast<long long>(s) * G);
    const int n = n_acc[s];
    const int ell = len ? len[s] : G;
    int8_t o = -1;
    if (n >= 0 && ell >= 0) {
        if (k < n) o = 1;
        else if (k == n && n < ell) o = 0;
    }
    ct[static_cast<long long>(k) * N + s] = conf[i];
    ot[static_cast<long long>(k) * N + s] = o;
}

__device__ __forceinline__ double scaled(float c, double T) {
    const double cd = static_cast<double>(c);
    if (!(cd > 0.0)) return 0.0;                      // also NaN
    if (cd >= 1.0) return 1.0;
    return 1.0 / (1.0 + exp(log((1.0 - cd) / cd) / T));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// stats[(k * (nT + 1) + t) * kStatVals + j]
__global__ __launch_bounds__(kStsThreads)
void sts_stats(int N, int nT, const float* __restrict__ grid, int bins,
               const float* __restrict__ ct, const int8_t* __restrict__ ot,
               double* __restrict__ stats) {
    __shared__ double part[kStsWaves][kStatVals];
    const int t = static_cast<int>(blockIdx.x % static_cast<unsigned>(nT + 1));
    const int k = static_cast<int>(blockIdx.x / static_cast<unsigned>(nT + 1));
    double T = (t < nT) ? static_cast<double>(grid[t]) : 1.0;
    if (!(T > 0.0)) T = 1.0;
    const float* c = ct + static_cast<long long>(k) * N;
    const int8_t* o = ot + static_cast<long long>(k) * N;
    double nll = 0.0, nobs = 0.0;
    double cnt[kStsMaxBins], acc[kStsMaxBins], sc[kStsMaxBins];
#pragma unroll
    for (int m = 0; m < kStsMaxBins; ++m) cnt[m] = acc[m] = sc[m] = 0.0;
    for (int i = threadIdx.x; i < N; i += kStsThreads) {
        const int oi = o[i];
        if (oi < 0) continue;
        const double cs = scaled(c[i], T);
        const double p = oi ? cs : 1.0 - cs;
        nll -= log(fmax(p, kStsEps));
        nobs += 1.0;
        const int b = min(static_cast<int>(floor(cs * bins)), bins - 1);
#pragma unroll
        for (int m = 0; m < kStsMaxBins; ++m)
            if (m == b) {
                cnt[m] += 1.0;
                acc[m] += static_cast<double>(oi);
                sc[m] += cs;
            }
    }
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    auto put = [&](int j, double v) {
        v = wave_sum_f64(v);
        if (lane == 0) part[wave][j] = v;
    };
    put(0, nll);
    put(1, nobs);
#pragma unroll
    for (int m = 0; m < kStsMaxBins; ++m) {
        put(2 + 3 * m, cnt[m]);
        put(3 + 3 * m, acc[m]);
        put(4 + 3 * m, sc[m]);
    }
    __syncthreads();
    if (threadIdx.x < kStatVals) {
        double v = part[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < kStsWaves; ++w) v += part[w][threadIdx.x];
        stats[static_cast<long long>(blockIdx.x) * kStatVals + threadIdx.x] = v;
    }
}

__device__ __forceinline__ double ece_of(const double* s, int bins) {
    const double nobs = s[1];
    if (nobs == 0.0) return 0.0;
    double e = 0.0;
    for (int m = 0; m < bins; ++m) {
        const double cnt = s[2 + 3 * m];
        if (cnt > 0.0) e += cnt / nobs * fabs(s[3 + 3 * m] / cnt - s[4 + 3 * m] / cnt);
    }
    return e;
}

// One wave per position; lane-strided objectives, first minimum by (value, index).
__global__ __launch_bounds__(kWave)
void sts_pick(int G, int nT, const float* __restrict__ grid, int bins, int objective,
              const double* __restrict__ stats, float* __restrict__ T_out,
              float* __restrict__ ece_before, float* __restrict__ ece_after,
              float* __restrict__ obj_out) {
    const int k = blockIdx.x, lane = threadIdx.x;
    const double* sk = stats + static_cast<long long>(k) * (nT + 1) * kStatVals;
    double best = INFINITY;
    int bi = INT32_MAX;
    for (int t = lane; t < nT; t += kWave) {
        const double* s = sk + static_cast<long long>(t) * kStatVals;
        const double v = (objective == 0) ? s[0] : ece_of(s, bins);
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
    if (lane == 0) {
        if (bi == INT32_MAX) bi = 0;                      // every objective NaN: first value
        T_out[k] = grid[bi];
        ece_before[k] = static_cast<float>(ece_of(sk + static_cast<long long>(nT) * kStatVals, bins));
        ece_after[k] = static_cast<float>(ece_of(sk + static_cast<long long>(bi) * kStatVals, bins));
    }
}

}  // namespace

int sts_max_bins() { return kStsMaxBins; }

size_t sts_stats_bytes(int gamma, int n_grid) {
    return static_cast<size_t>(gamma) * (n_grid + 1) * kStatVals * sizeof(double);
}

hipError_t launch_sts_fit(int N, int G, const float* conf, const int32_t* n_acc,
                          const int32_t* len, const float* grid, int nT, int bins, int objective,
                          float* ct, int8_t* ot, double* stats, float* T_out, float* ece_before,
                          float* ece_after, float* obj_out, hipStream_t st) {
    const long long total = static_cast<long long>(N) * G;
    hipLaunchKernelGGL(sts_prep, dim3(static_cast<unsigned>((total + kStsThreads - 1) / kStsThreads)),
                       dim3(kStsThreads), 0, st, N, G, conf, n_acc, len, ct, ot);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sts_stats, dim3(static_cast<unsigned>(G) * (nT + 1)), dim3(kStsThreads), 0,
                       st, N, nT, grid, bins, ct, ot, stats);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sts_pick, dim3(G), dim3(kWave), 0, st, G, nT, grid, bins, objective, stats,
                       T_out, ece_before, ece_after, obj_out);
    return hipGetLastError();
}

}  // namespace dspark
