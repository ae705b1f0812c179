// Rejection-sampling verification and TV-label kernels (gfx950).
//
// [P1] = "大模型推理加速的系统级工程：DeepSeek V4-Pro DSpark 推测解码方案深度解析与开源工具链
// DeepSpec" (Best Partners TV); [P3] = "DSpark Speculative Decoding" (concept note).
//
// row_lse        - [P1] section "大模型推理的显存瓶颈与推测解码的演进逻辑": the accept test needs
//                  normalised probabilities, so every verified row gets its logsumexp in one
//                  HBM pass (online max / sum-exp, float4 loads, one workgroup per row).
// verify_finish  - one workgroup per request: gathers p_d(x_k), p_t(x_k), tests
//                  log u < log p_t - log p_d for all k in one wave, takes the first rejection
//                  from a ballot, then draws the residual max(0, p_t - p_d) (or the bonus
//                  p_t row, [P3] intro) by inverse CDF: chunk sums in id order, chunk search,
//                  in-chunk rescan.
// tv             - [P3] "Confidence-Scheduled Verification": c* = sum_v min(p_d, p_t), computed
//                  as sum_v exp(min(l_d - lse_d, l_t - lse_t)) (one exp per element).
// Target rows are flattened with per-request offsets ([P1] section "极致的工程实现与内核优化").
#include "common.h"
#include "kernels.h"

namespace dspark {

namespace {

constexpr int kLseThreads = 256;
constexpr int kFinThreads = 1024;
constexpr int kFinPerThread = 4;
constexpr int kChunk = kFinThreads * kFinPerThread;
constexpr int kTvThreads = 256;

struct ReqRows {
    int ell;
    long long off;
    bool ok;
};

__device__ __forceinline__ ReqRows request_rows(const RowSet& rs, int b) {
    ReqRows q;
    q.ell = rs.len ? rs.len[b] : rs.gamma;
    q.off = rs.t_off ? static_cast<long long>(rs.t_off[b])
                     : static_cast<long long>(b) * (rs.gamma + 1);
    q.ok = q.ell >= 0 && q.ell <= rs.gamma && q.off >= 0 && q.off + q.ell < rs.Lt_rows;
    return q;
}

// (max, sum exp(x - max)) pairs; combination is symmetric, so butterflies are exact.
__device__ __forceinline__ void ms_combine(float& m, float& s, float m2, float s2) {
    const float mm = fmaxf(m, m2);
    if (mm == -INFINITY) {
        m = -INFINITY;
        s = 0.0f;
        return;
    }
    s = s * __expf(m - mm) + s2 * __expf(m2 - mm);
    m = mm;
}

__device__ __forceinline__ void ms_push4(float& m, float& s, float a, float b, float c, float d) {
    const float cm = fmaxf(fmaxf(a, b), fmaxf(c, d));
    if (cm == -INFINITY) return;
    if (cm > m) {
        s = (m == -INFINITY) ? 0.0f : s * __expf(m - cm);
        m = cm;
    }
    s += (__expf(a - m) + __expf(b - m)) + (__expf(c - m) + __expf(d - m));
}

template <bool VEC4>
__device__ float row_logsumexp(const float* __restrict__ row, int V) {
    __shared__ float ms[2][kLseThreads / kWave];
    float m = -INFINITY, s = 0.0f;
    const int tid = threadIdx.x;
    if (VEC4) {
        const float4* r4 = reinterpret_cast<const float4*>(row);
        const int n4 = V >> 2;
        for (int i = tid; i < n4; i += kLseThreads) {
            const float4 x = r4[i];
            ms_push4(m, s, x.x, x.y, x.z, x.w);
        }
    } else {
        for (long long base = static_cast<long long>(tid) * 4; base < V; base += 4LL * kLseThreads) {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (base + e < V) ? row[base + e] : -INFINITY;
            ms_push4(m, s, x[0], x[1], x[2], x[3]);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o, kWave), s2 = __shfl_xor(s, o, kWave);
        ms_combine(m, s, m2, s2);
    }
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    if (lane == 0) {
        ms[0][wave] = m;
        ms[1][wave] = s;
    }
    __syncthreads();
    m = ms[0][0];
    s = ms[1][0];
#pragma unroll
    for (int w = 1; w < kLseThreads / kWave; ++w) ms_combine(m, s, ms[0][w], ms[1][w]);
    return (m == -INFINITY) ? -INFINITY : m + __logf(s);
}

template <bool VEC4>
__global__ __launch_bounds__(kLseThreads)
void row_lse_kernel(RowSet rs, const float* __restrict__ lse_d_in, float* __restrict__ lse_d,
                    float* __restrict__ lse_t) {
    const int G = rs.gamma;
    const int slot = static_cast<int>(blockIdx.x % static_cast<unsigned>(2 * G + 1));
    const int b = static_cast<int>(blockIdx.x / static_cast<unsigned>(2 * G + 1));
    const ReqRows q = request_rows(rs, b);
    const float* row;
    float* out;
    bool valid;
    if (slot <= G) {
        out = lse_t + static_cast<long long>(b) * (G + 1) + slot;
        valid = q.ok && slot <= q.ell;
        row = rs.Lt + (q.off + slot) * rs.V;
    } else {
        const int k = slot - G - 1;
        out = lse_d + static_cast<long long>(b) * G + k;
        valid = q.ok && k < q.ell;
        row = rs.Ld + (static_cast<long long>(b) * G + k) * rs.V;
        if (valid && lse_d_in) {
            if (threadIdx.x == 0) *out = lse_d_in[static_cast<long long>(b) * G + k];
            return;
        }
    }
    if (!valid) {
        if (threadIdx.x == 0) *out = __int_as_float(0x7fc00000);
        return;
    }
    const float lse = row_logsumexp<VEC4>(row, rs.V);
    if (threadIdx.x == 0) *out = lse;
}

// Weights of the final draw: p_t (bonus, or residual with zero mass) or max(0, p_t - p_d).
struct FinalRow {
    const float* lt;
    const float* ld;
    float lse_t, lse_d;
    int residual;

    __device__ __forceinline__ float weight(float lt_v, float ld_v) const {
        const float pt = (lse_t == -INFINITY) ? 0.0f : __expf(lt_v - lse_t);
        if (!residual) return pt;
        const float pd = (lse_d == -INFINITY) ? 0.0f : __expf(ld_v - lse_d);
        return fmaxf(pt - pd, 0.0f);
    }
};

template <bool VEC4>
__device__ __forceinline__ void weights4(const FinalRow& fr, long long v0, int V, float (&w)[4]) {
    if (VEC4 && v0 + 4 <= V) {
        const float4 t = *reinterpret_cast<const float4*>(fr.lt + v0);
        float4 d = make_float4(0.f, 0.f, 0.f, 0.f);
        if (fr.residual) d = *reinterpret_cast<const float4*>(fr.ld + v0);
        w[0] = fr.weight(t.x, d.x);
        w[1] = fr.weight(t.y, d.y);
        w[2] = fr.weight(t.z, d.z);
        w[3] = fr.weight(t.w, d.w);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const long long v = v0 + e;
            w[e] = (v < V) ? fr.weight(fr.lt[v], fr.residual ? fr.ld[v] : 0.0f) : 0.0f;
        }
    }
}

template <bool VEC4>
__global__ __launch_bounds__(kFinThreads)
void verify_finish_kernel(RowSet rs, const int32_t* __restrict__ x, const float* __restrict__ lse_d,
                          const float* __restrict__ lse_t, const float* __restrict__ u_acc,
                          const float* __restrict__ u_fin, float* __restrict__ chunk_ws,
                          int nchunk, int32_t* __restrict__ n_out, int32_t* __restrict__ y_out) {
    __shared__ float fscr[kFinThreads / kWave + 1];
    __shared__ int iscr[kFinThreads / kWave + 1];
    __shared__ int s_n, s_bad, s_found;
    __shared__ float s_tprime, s_total;

    const int b = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int G = rs.gamma, V = rs.V;
    int32_t* y = y_out + static_cast<long long>(b) * (G + 1);
    const ReqRows q = request_rows(rs, b);
    if (!q.ok) {
        for (int i = tid; i <= G; i += kFinThreads) y[i] = -1;
        if (tid == 0) n_out[b] = -1;
        return;
    }

    // acceptance test for every verified position in one wave (gamma <= 64)
    if (wave == 0) {
        bool bad = false, rej = false;
        const int k = lane;
        if (k < q.ell) {
            const int xk = x[static_cast<long long>(b) * G + k];
            if (xk < 0 || xk >= V) {
                bad = true;
            } else {
                const float ltx = rs.Lt[(q.off + k) * V + xk];
                const float ldx = rs.Ld[(static_cast<long long>(b) * G + k) * V + xk];
                const float lst = lse_t[static_cast<long long>(b) * (G + 1) + k];
                const float lsd = lse_d[static_cast<long long>(b) * G + k];
                const float lpt = (lst == -INFINITY) ? -INFINITY : ltx - lst;
                const float lpd = (lsd == -INFINITY) ? -INFINITY : ldx - lsd;
                bool acc;
                if (lpd == -INFINITY)
                    acc = lpt > -INFINITY;
                else
                    acc = logf(clamp_uniform(u_acc[static_cast<long long>(b) * G + k])) < lpt - lpd;
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
    if (s_bad) {
        for (int i = tid; i <= G; i += kFinThreads) y[i] = -1;
        if (tid == 0) n_out[b] = -1;
        return;
    }
    const int n = s_n;

    FinalRow fr;
    if (n < q.ell) {
        fr.lt = rs.Lt + (q.off + n) * V;
        fr.ld = rs.Ld + (static_cast<long long>(b) * G + n) * V;
        fr.lse_t = lse_t[static_cast<long long>(b) * (G + 1) + n];
        fr.lse_d = lse_d[static_cast<long long>(b) * G + n];
        fr.residual = 1;
    } else {
        fr.lt = rs.Lt + (q.off + q.ell) * V;
        fr.ld = nullptr;
        fr.lse_t = lse_t[static_cast<long long>(b) * (G + 1) + q.ell];
        fr.lse_d = 0.0f;
        fr.residual = 0;
    }
    const float uf = clamp_uniform(u_fin[b]);
    float* cs = chunk_ws + static_cast<long long>(b) * nchunk;

    for (int pass = 0; pass < 2; ++pass) {
        for (int c = 0; c < nchunk; ++c) {
            float w[4];
            weights4<VEC4>(fr, static_cast<long long>(c) * kChunk + tid * kFinPerThread, V, w);
            const float s = block_sum<kFinThreads>((w[0] + w[1]) + (w[2] + w[3]), fscr);
            if (tid == 0) cs[c] = s;
        }
        if (tid == 0) {
            float tot = 0.0f;
            for (int c = 0; c < nchunk; ++c) tot += cs[c];
            const float target = uf * tot;
            int found = -1;
            float tprime = INFINITY;
            if (tot > 0.0f) {
                float run = 0.0f;
                for (int c = 0; c < nchunk; ++c) {
                    const float nr = run + cs[c];
                    if (cs[c] > 0.0f && nr > target) {
                        found = c;
                        tprime = target - run;
                        break;
                    }
                    run = nr;
                }
                if (found < 0)       // rounding left the target past the end
                    for (int c = nchunk - 1; c >= 0; --c)
                        if (cs[c] > 0.0f) { found = c; break; }
            }
            s_found = found;
            s_tprime = tprime;
            s_total = tot;
        }
        __syncthreads();
        if (s_total > 0.0f || !fr.residual) break;
        fr.residual = 0;           // residual mass rounded to zero: draw from p_t instead
        __syncthreads();
    }

    int z = -1;
    const int found = s_found;
    if (found >= 0) {
        const long long v0 = static_cast<long long>(found) * kChunk + tid * kFinPerThread;
        float w[4];
        weights4<VEC4>(fr, v0, V, w);
        float tot;
        const float ex = block_excl_scan<kFinThreads>((w[0] + w[1]) + (w[2] + w[3]), fscr, &tot);
        const float tprime = s_tprime;
        int hit = INT32_MAX, lastpos = -1;
        float run = ex;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            run += w[e];
            if (w[e] > 0.0f) {
                lastpos = static_cast<int>(v0 + e);
                if (hit == INT32_MAX && run > tprime) hit = static_cast<int>(v0 + e);
            }
        }
        z = block_min_int<kFinThreads>(hit, iscr);
        if (z == INT32_MAX) z = block_max_int<kFinThreads>(lastpos, iscr);
    }
    for (int i = tid; i <= G; i += kFinThreads)
        y[i] = (i < n) ? x[static_cast<long long>(b) * G + i] : (i == n ? z : -1);
    if (tid == 0) n_out[b] = n;
}

template <bool VEC4>
__global__ __launch_bounds__(kTvThreads)
void tv_kernel(RowSet rs, const float* __restrict__ lse_d, const float* __restrict__ lse_t,
               float* __restrict__ cstar) {
    __shared__ float fscr[kTvThreads / kWave + 1];
    const int G = rs.gamma, V = rs.V, tid = threadIdx.x;
    const int k = static_cast<int>(blockIdx.x % static_cast<unsigned>(G));
    const int b = static_cast<int>(blockIdx.x / static_cast<unsigned>(G));
    const ReqRows q = request_rows(rs, b);
    float* out = cstar + static_cast<long long>(b) * G + k;
    if (!q.ok || k >= q.ell) {
        if (tid == 0) *out = __int_as_float(0x7fc00000);
        return;
    }
    const float a = lse_d[static_cast<long long>(b) * G + k];
    const float c = lse_t[static_cast<long long>(b) * (G + 1) + k];
    if (a == -INFINITY || c == -INFINITY) {     // a zero distribution shares no mass
        if (tid == 0) *out = 0.0f;
        return;
    }
    const float* ld = rs.Ld + (static_cast<long long>(b) * G + k) * V;
    const float* lt = rs.Lt + (q.off + k) * V;
    float s = 0.0f;
    if (VEC4) {
        const float4* d4 = reinterpret_cast<const float4*>(ld);
        const float4* t4 = reinterpret_cast<const float4*>(lt);
        for (int i = tid; i < (V >> 2); i += kTvThreads) {
            const float4 d = d4[i], t = t4[i];
            s += (__expf(fminf(d.x - a, t.x - c)) + __expf(fminf(d.y - a, t.y - c))) +
                 (__expf(fminf(d.z - a, t.z - c)) + __expf(fminf(d.w - a, t.w - c)));
        }
    } else {
        for (int v = tid; v < V; v += kTvThreads) s += __expf(fminf(ld[v] - a, lt[v] - c));
    }
    s = block_sum<kTvThreads>(s, fscr);
    if (tid == 0) *out = s;
}

}  // namespace

int verify_chunk_elems() { return kChunk; }

static bool rows_vec4(const RowSet& rs) {
    return (rs.V % 4) == 0 && (reinterpret_cast<uintptr_t>(rs.Ld) % 16) == 0 &&
           (reinterpret_cast<uintptr_t>(rs.Lt) % 16) == 0;
}

hipError_t launch_row_lse(const RowSet& rs, const float* lse_d_in, float* lse_d, float* lse_t,
                          hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(2 * rs.gamma + 1) * rs.B);
    if (rows_vec4(rs))
        hipLaunchKernelGGL(row_lse_kernel<true>, grid, dim3(kLseThreads), 0, st, rs, lse_d_in,
                           lse_d, lse_t);
    else
        hipLaunchKernelGGL(row_lse_kernel<false>, grid, dim3(kLseThreads), 0, st, rs, lse_d_in,
                           lse_d, lse_t);
    return hipGetLastError();
}

hipError_t launch_verify_finish(const RowSet& rs, const int32_t* x, const float* lse_d,
                                const float* lse_t, const float* u_acc, const float* u_fin,
                                float* chunk_ws, int nchunk, int32_t* n_out, int32_t* y_out,
                                hipStream_t st) {
    if (rows_vec4(rs))
        hipLaunchKernelGGL(verify_finish_kernel<true>, dim3(rs.B), dim3(kFinThreads), 0, st, rs, x,
                           lse_d, lse_t, u_acc, u_fin, chunk_ws, nchunk, n_out, y_out);
    else
        hipLaunchKernelGGL(verify_finish_kernel<false>, dim3(rs.B), dim3(kFinThreads), 0, st, rs, x,
                           lse_d, lse_t, u_acc, u_fin, chunk_ws, nchunk, n_out, y_out);
    return hipGetLastError();
}

hipError_t launch_tv(const RowSet& rs, const float* lse_d, const float* lse_t, float* cstar,
                     hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(rs.gamma) * rs.B);
    if (rows_vec4(rs))
        hipLaunchKernelGGL(tv_kernel<true>, grid, dim3(kTvThreads), 0, st, rs, lse_d, lse_t, cstar);
    else
        hipLaunchKernelGGL(tv_kernel<false>, grid, dim3(kTvThreads), 0, st, rs, lse_d, lse_t, cstar);
    return hipGetLastError();
}

}  // namespace dspark
