// C-ABI host layer of libdspark: argument validation, workspace carving, kernel launches.
//
// Every check here runs before any HIP call, so a rejected call enqueues nothing and leaves
// the outputs untouched. Launch failures come back as DSPARK_ERR_HIP.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/dspark.h"
#include "kernels.h"
#include "schedule_small.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return DSPARK_OK;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(DSPARK_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

// Carves consecutive aligned regions out of the caller's workspace.
struct Carver {
    char* base;
    size_t used = 0;
    explicit Carver(void* p) : base(static_cast<char*>(p)) {}
    template <typename T>
    T* take(size_t count) {
        T* p = reinterpret_cast<T*>(base + used);
        used += align_up(count * sizeof(T));
        return p;
    }
};

constexpr long long kMaxElems = 1LL << 40;

constexpr int kMaxB = 1 << 24;         // keeps every 1-D grid below 2^31 workgroups

bool common_sizes_ok(int B, int V, int gamma) {
    return B >= 1 && B <= kMaxB && V >= 1 && gamma >= 1 && gamma <= 64 &&
           static_cast<long long>(B) * gamma * V < kMaxElems;
}

int ceil_div(long long a, long long b) { return static_cast<int>((a + b - 1) / b); }

// sizes of the draft workspace regions
size_t draft_part_count(int B, int V) {
    return static_cast<size_t>(B) * dspark::draft_part_tiles(V);
}

// flags / slots of the one-launch draft forms (single request, or slab)
size_t draft_slot_bytes(int V, int gamma) {
    const size_t a = dspark::draft_resident_slot_bytes(V, gamma), b = dspark::draft_slab_flag_bytes(V, gamma);
    return a > b ? a : b;
}

}  // namespace

extern "C" {

const char* dspark_status_string(int status) {
    switch (status) {
        case DSPARK_OK: return "ok";
        case DSPARK_ERR_INVALID_ARG: return "invalid argument";
        case DSPARK_ERR_WORKSPACE: return "workspace too small";
        case DSPARK_ERR_UNSUPPORTED: return "size outside the supported caps";
        case DSPARK_ERR_HIP: return "HIP launch failure";
        default: return "unknown status";
    }
}

const char* dspark_last_error(void) { return g_last_error; }

int dspark_version(void) { return 10000; }

// ----------------------------------------------------------------------------- draft
int dspark_markov_draft_path(int B, int V, int r, int w_dtype, const void* W1, const void* W2) {
    if (dspark::draft_resident_ok(B, V, r, w_dtype, W1, W2)) return DSPARK_PATH_RESIDENT;
    if (dspark::draft_slab_ok(B, V, r, w_dtype, W1, W2)) return DSPARK_PATH_SLAB;
    if (dspark::draft_mfma_ok(B, V, r, w_dtype, W1, W2)) return DSPARK_PATH_MFMA;
    return DSPARK_PATH_SWEEP;
}

int dspark_markov_draft_one_launch(int B, int V, int r, int w_dtype, const void* W1, const void* W2,
                                   int want_logits) {
    const int p = dspark_markov_draft_path(B, V, r, w_dtype, W1, W2);
    if (p == DSPARK_PATH_RESIDENT) return 1;
    return p == DSPARK_PATH_SLAB && dspark::draft_slab_one_launch(B, V, want_logits != 0) ? 1 : 0;
}

}  // extern "C"

// Draft workspace layout: a 256-byte header (bytes 0..3: the give-up count of the last
// one-launch call), the position slots of the one-launch forms, the two tile-partial buffers
// (every path but the single-request one), and two logits rows per request (the sweep and
// MFMA paths, when the caller does not take the logits). A call needs only the regions of
// the path it takes; dspark_markov_draft_workspace_bytes covers every path.
namespace {

constexpr size_t kDraftHeader = 256;

struct DraftNeed {
    size_t slots, parts, rows;
    size_t total() const { return kDraftHeader + slots + parts + rows; }
};

DraftNeed draft_need(int B, int V, int gamma, int path, bool L_out) {
    DraftNeed n{align_up(draft_slot_bytes(V, gamma)), 0, 0};
    if (path != DSPARK_PATH_RESIDENT) n.parts = 2 * align_up(draft_part_count(B, V) * sizeof(float2));
    if ((path == DSPARK_PATH_SWEEP || path == DSPARK_PATH_MFMA) && !L_out)
        n.rows = 2 * align_up(static_cast<size_t>(B) * V * sizeof(float));
    return n;
}

bool draft_sizes_ok(int B, int V, int r, int gamma) {
    return B >= 1 && V >= 1 && gamma >= 1 && r >= 1 && gamma <= 64 && r <= 1024 &&
           common_sizes_ok(B, V, gamma);
}

// The DraftCall of these arguments with every pointer but the workspace's set (the path
// choice depends on the factors' and U's alignment, on Ld_out and on the options).
dspark::DraftCall draft_call(int B, int V, int r, int gamma, const float* U, const void* W1,
                             const void* W2, int w_dtype, const float* Ld_out, int options) {
    dspark::DraftCall dc;
    dc.B = B; dc.V = V; dc.r = r; dc.gamma = gamma; dc.w_dtype = w_dtype;
    dc.U = U; dc.W1 = W1; dc.W2 = W2;
    dc.L_out = Ld_out != nullptr;
    dc.L[0] = const_cast<float*>(Ld_out);
    dc.per_position = (options & DSPARK_DRAFT_PER_POSITION) != 0;
    return dc;
}

}  // namespace

extern "C" {

size_t dspark_markov_draft_workspace_bytes(int B, int V, int r, int gamma) {
    (void)r;
    if (B < 1 || V < 1 || gamma < 1) return 0;
    return draft_need(B, V, gamma, DSPARK_PATH_SWEEP, false).total();
}

int dspark_markov_draft_plan(int B, int V, int r, int gamma, int w_dtype, const void* W1,
                             const void* W2, const float* U, const float* Ld_out, int options,
                             int* path_out, int* one_launch_out, size_t* ws_bytes_out) {
    if (options & ~(DSPARK_DRAFT_PER_POSITION | DSPARK_DRAFT_TEST_SPIN))
        return fail(DSPARK_ERR_INVALID_ARG, "markov_draft_plan: unknown option bits 0x%x", options);
    if (!draft_sizes_ok(B, V, r, gamma))
        return fail(DSPARK_ERR_INVALID_ARG, "markov_draft_plan: B=%d V=%d r=%d gamma=%d outside caps",
                    B, V, r, gamma);
    if (w_dtype != DSPARK_F32 && w_dtype != DSPARK_BF16)
        return fail(DSPARK_ERR_INVALID_ARG, "markov_draft_plan: unknown w_dtype %d", w_dtype);
    const dspark::DraftCall dc = draft_call(B, V, r, gamma, U, W1, W2, w_dtype, Ld_out, options);
    bool one = false;
    const int path = dspark::draft_path_of(dc, &one);
    if (path_out) *path_out = path;
    if (one_launch_out) *one_launch_out = one ? 1 : 0;
    if (ws_bytes_out) *ws_bytes_out = draft_need(B, V, gamma, path, Ld_out != nullptr).total();
    return ok();
}

}  // extern "C"

namespace {

// The draft of dspark_markov_draft_ex; with a one-wave schedule job that the single-request
// launch can take, that launch also runs the job (*job_taken set), else the job is left to
// the caller.
int draft_run(const char* who, int B, int V, int r, int gamma, const float* U, const void* W1,
              const void* W2, int w_dtype, const int32_t* x0, const float* u, int32_t* x_out,
              float* q_out, float* lse_out, float* Ld_out, void* ws, size_t ws_bytes, void* stream,
              int options, const dspark::sched::SmallJob* job, bool* job_taken) {
    if (options & ~(DSPARK_DRAFT_PER_POSITION | DSPARK_DRAFT_TEST_SPIN))
        return fail(DSPARK_ERR_INVALID_ARG, "%s: unknown option bits 0x%x", who, options);
    if (B < 1 || V < 1 || gamma < 1 || r < 1)
        return fail(DSPARK_ERR_INVALID_ARG, "%s: B=%d V=%d r=%d gamma=%d must be >= 1",
                    who, B, V, r, gamma);
    if (!draft_sizes_ok(B, V, r, gamma))
        return fail(DSPARK_ERR_UNSUPPORTED, "%s: gamma=%d r=%d B*gamma*V outside caps",
                    who, gamma, r);
    if (w_dtype != DSPARK_F32 && w_dtype != DSPARK_BF16)
        return fail(DSPARK_ERR_INVALID_ARG, "%s: unknown w_dtype %d", who, w_dtype);
    if (!U || !W1 || !W2 || !x0 || !u || !x_out)
        return fail(DSPARK_ERR_INVALID_ARG, "%s: a required pointer is NULL", who);
    dspark::DraftCall dc = draft_call(B, V, r, gamma, U, W1, W2, w_dtype, Ld_out, options);
    const int path = dspark::draft_path_of(dc, nullptr);
    const DraftNeed need = draft_need(B, V, gamma, path, Ld_out != nullptr);
    if (!ws || ws_bytes < need.total())
        return fail(DSPARK_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", who, ws_bytes,
                    need.total());
    Carver c(ws);
    dc.status = c.take<unsigned>(kDraftHeader / sizeof(unsigned));
    dc.slots = reinterpret_cast<float2*>(c.take<char>(need.slots));
    float* lbuf[2] = {nullptr, nullptr};
    if (need.parts) {
        dc.part[0] = c.take<float2>(draft_part_count(B, V));
        dc.part[1] = c.take<float2>(draft_part_count(B, V));
    } else {
        dc.part[0] = dc.part[1] = nullptr;
    }
    if (need.rows) {
        lbuf[0] = c.take<float>(static_cast<size_t>(B) * V);
        lbuf[1] = c.take<float>(static_cast<size_t>(B) * V);
    }
    dc.x0 = x0; dc.u = u;
    dc.x_out = x_out; dc.q_out = q_out; dc.lse_out = lse_out;
    for (int k = 0; k < gamma; ++k)
        dc.L[k] = Ld_out ? Ld_out + static_cast<long long>(k) * V : lbuf[k & 1];
    dc.L_bstride = Ld_out ? static_cast<long long>(gamma) * V : V;
    if (options & DSPARK_DRAFT_TEST_SPIN) dc.spin = 0;
    if (job && path == DSPARK_PATH_RESIDENT && dspark::draft_resident_takes_job(V)) {
        dc.job = job;
        *job_taken = true;
    }
    const hipError_t e = dspark::launch_draft(dc, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, who);
    return ok();
}

}  // namespace

extern "C" {

int dspark_markov_draft_ex(int B, int V, int r, int gamma, const float* U, const void* W1,
                           const void* W2, int w_dtype, const int32_t* x0, const float* u,
                           int32_t* x_out, float* q_out, float* lse_out, float* Ld_out, void* ws,
                           size_t ws_bytes, void* stream, int options) {
    bool taken = false;
    return draft_run("markov_draft", B, V, r, gamma, U, W1, W2, w_dtype, x0, u, x_out, q_out,
                     lse_out, Ld_out, ws, ws_bytes, stream, options, nullptr, &taken);
}

}  // extern "C"

// Scratch of the allocation-free draft: one static device array per GPU the library runs on
// (held until the process ends). Host code never passes the array's name to a kernel: its
// device address comes from hipGetSymbolAddress, taken once per device with that device
// current, and is kept per device.
constexpr size_t kNoAllocScratch = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratch];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, or nullptr with *err set.
void* scratch_for_current_device(hipError_t* err) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *err = e != hipSuccess ? e : hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    *err = hipSuccess;
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t dspark_noalloc_scratch_bytes(void) { return kNoAllocScratch; }

int dspark_markov_draft_noalloc(int B, int V, int r, int gamma, const float* U, const void* W1,
                                const void* W2, int w_dtype, const int32_t* x0, const float* u,
                                int32_t* x_out, float* q_out, float* lse_out, float* Ld_out,
                                void* stream, int options) {
    size_t need = 0;
    const int st = dspark_markov_draft_plan(B, V, r, gamma, w_dtype, W1, W2, U, Ld_out, options,
                                            nullptr, nullptr, &need);
    if (st != DSPARK_OK) return st;
    if (need > kNoAllocScratch)
        return fail(DSPARK_ERR_UNSUPPORTED,
                    "markov_draft_noalloc: this call needs %zu bytes of scratch, the static "
                    "scratch holds %zu (pass Ld_out, or use dspark_markov_draft with a workspace)",
                    need, kNoAllocScratch);
    hipError_t e = hipSuccess;
    void* ws = scratch_for_current_device(&e);
    if (!ws) return hip_fail(e, "markov_draft_noalloc/scratch");
    return dspark_markov_draft_ex(B, V, r, gamma, U, W1, W2, w_dtype, x0, u, x_out, q_out, lse_out,
                                  Ld_out, ws, kNoAllocScratch, stream, options);
}

int dspark_markov_draft(int B, int V, int r, int gamma, const float* U, const void* W1,
                        const void* W2, int w_dtype, const int32_t* x0, const float* u,
                        int32_t* x_out, float* q_out, float* lse_out, float* Ld_out, void* ws,
                        size_t ws_bytes, void* stream) {
    return dspark_markov_draft_ex(B, V, r, gamma, U, W1, W2, w_dtype, x0, u, x_out, q_out, lse_out,
                                  Ld_out, ws, ws_bytes, stream, 0);
}

// ----------------------------------------------------------------------------- RNN head
namespace {

// header, slots (single-request one-launch form), tile partials, logits rows (when the caller
// does not take them), fp32 state ping-pong and A h_k, bf16 hi / lo state rows (batched form)
size_t rnn_ws_bytes(int B, int V, int r, int gamma) {
    const int rp = dspark::rnn_rank_pad(r);
    return kDraftHeader + align_up(draft_slot_bytes(V, gamma)) +
           2 * align_up(draft_part_count(B, V) * sizeof(float2)) +
           2 * align_up(static_cast<size_t>(B) * V * sizeof(float)) +
           3 * align_up(static_cast<size_t>(B) * r * sizeof(float)) +
           align_up(static_cast<size_t>(B) * 2 * rp * sizeof(uint16_t));
}

}  // namespace

size_t dspark_rnn_draft_workspace_bytes(int B, int V, int r, int gamma) {
    if (B < 1 || V < 1 || gamma < 1 || r < 1) return 0;
    return rnn_ws_bytes(B, V, r, gamma);
}

int dspark_rnn_draft(int B, int V, int r, int gamma, const float* U, const void* W1,
                     const void* W2, const void* A, int w_dtype, const int32_t* x0, const float* u,
                     int32_t* x_out, float* q_out, float* lse_out, float* Ld_out, float* h_out,
                     void* ws, size_t ws_bytes, void* stream) {
    if (B < 1 || V < 1 || gamma < 1 || r < 1)
        return fail(DSPARK_ERR_INVALID_ARG, "rnn_draft: B=%d V=%d r=%d gamma=%d must be >= 1", B, V,
                    r, gamma);
    if (!draft_sizes_ok(B, V, r, gamma))
        return fail(DSPARK_ERR_UNSUPPORTED, "rnn_draft: gamma=%d r=%d B*gamma*V outside caps", gamma, r);
    if (w_dtype != DSPARK_F32 && w_dtype != DSPARK_BF16)
        return fail(DSPARK_ERR_INVALID_ARG, "rnn_draft: unknown w_dtype %d", w_dtype);
    if (!U || !W1 || !W2 || !A || !x0 || !u || !x_out)
        return fail(DSPARK_ERR_INVALID_ARG, "rnn_draft: a required pointer is NULL");
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) % 16) == 0; };
    if (w_dtype != DSPARK_BF16 || !dspark::rnn_mfma_ok(V, r, W1, W2, A) || !al16(U))
        return fail(DSPARK_ERR_UNSUPPORTED,
                    "rnn_draft: needs bf16 factors, r <= 256 with r %% 8 == 0, V %% 8 == 0 and "
                    "16-byte aligned U, W1, W2, A (w_dtype=%d r=%d V=%d)", w_dtype, r, V);
    const size_t need = rnn_ws_bytes(B, V, r, gamma);
    if (!ws || ws_bytes < need)
        return fail(DSPARK_ERR_WORKSPACE, "rnn_draft: workspace %zu bytes, need %zu", ws_bytes, need);
    Carver c(ws);
    dspark::RnnCall rc;
    dspark::DraftCall& dc = rc.d;
    dc.B = B; dc.V = V; dc.r = r; dc.gamma = gamma; dc.w_dtype = w_dtype;
    dc.U = U; dc.W1 = W1; dc.W2 = W2; dc.x0 = x0; dc.u = u;
    dc.x_out = x_out; dc.q_out = q_out; dc.lse_out = lse_out;
    dc.status = c.take<unsigned>(kDraftHeader / sizeof(unsigned));
    dc.slots = reinterpret_cast<float2*>(c.take<char>(draft_slot_bytes(V, gamma)));
    dc.part[0] = c.take<float2>(draft_part_count(B, V));
    dc.part[1] = c.take<float2>(draft_part_count(B, V));
    float* lbuf[2] = {c.take<float>(static_cast<size_t>(B) * V), c.take<float>(static_cast<size_t>(B) * V)};
    for (int k = 0; k < gamma; ++k)
        dc.L[k] = Ld_out ? Ld_out + static_cast<long long>(k) * V : lbuf[k & 1];
    dc.L_bstride = Ld_out ? static_cast<long long>(gamma) * V : V;
    dc.L_out = Ld_out != nullptr;
    rc.A = A;
    rc.h_out = h_out;
    rc.hstate[0] = c.take<float>(static_cast<size_t>(B) * r);
    rc.hstate[1] = c.take<float>(static_cast<size_t>(B) * r);
    rc.hrows = c.take<uint16_t>(static_cast<size_t>(B) * 2 * dspark::rnn_rank_pad(r));
    rc.ah = c.take<float>(static_cast<size_t>(B) * r);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = dspark::rnn_resident_ok(B, V, r, W1, W2, A) ? dspark::launch_rnn_resident(rc, st)
                                                                     : dspark::launch_rnn_mfma(rc, st);
    if (e != hipSuccess) return hip_fail(e, "rnn_draft");
    return ok();
}

int dspark_rnn_draft_path(int B, int V, int r, const void* W1, const void* W2, const void* A) {
    if (dspark::rnn_resident_ok(B, V, r, W1, W2, A)) return DSPARK_PATH_RESIDENT;
    return DSPARK_PATH_MFMA;
}

// ----------------------------------------------------------------------------- verify / TV
namespace {

long long row_chunks(int V) { return ceil_div(V, dspark::verify_chunk_elems()); }

int check_rows(const char* who, int B, int V, int gamma, const float* Ld, const float* Lt,
               int Lt_rows, const int32_t* t_off) {
    if (B < 1 || V < 1 || gamma < 1)
        return fail(DSPARK_ERR_INVALID_ARG, "%s: B=%d V=%d gamma=%d must be >= 1", who, B, V, gamma);
    if (!common_sizes_ok(B, V, gamma) ||
        row_chunks(V) * (2 * gamma + 1) * static_cast<long long>(B) > INT32_MAX)
        return fail(DSPARK_ERR_UNSUPPORTED, "%s: B=%d gamma=%d V=%d outside caps", who, B, gamma, V);
    if (!Ld || !Lt) return fail(DSPARK_ERR_INVALID_ARG, "%s: Ld / Lt is NULL", who);
    if (Lt_rows < 1) return fail(DSPARK_ERR_INVALID_ARG, "%s: Lt_rows=%d", who, Lt_rows);
    if (!t_off && static_cast<long long>(Lt_rows) < static_cast<long long>(B) * (gamma + 1))
        return fail(DSPARK_ERR_INVALID_ARG, "%s: padded layout needs %lld target rows, got %d",
                    who, static_cast<long long>(B) * (gamma + 1), Lt_rows);
    return DSPARK_OK;
}

size_t part_bytes(int B, int V, int gamma) {
    return align_up(static_cast<size_t>(B) * (2 * gamma + 1) * row_chunks(V) * sizeof(float2));
}

}  // namespace

size_t dspark_verify_workspace_bytes(int B, int V, int gamma) {
    if (B < 1 || V < 1 || gamma < 1) return 0;
    return part_bytes(B, V, gamma) +
           align_up(static_cast<size_t>(B) * row_chunks(V) * sizeof(float)) +
           align_up(static_cast<size_t>(B) * dspark::verify_state_bytes());
}

int dspark_verify(int B, int V, int gamma, const float* Ld, const float* Lt, int Lt_rows,
                  const int32_t* t_off, const int32_t* len, const int32_t* x, const float* ld_lse,
                  const float* u_acc, const float* u_fin, int32_t* n_acc_out, int32_t* y_out,
                  float* lse_d_out, float* lse_t_out, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_rows("verify", B, V, gamma, Ld, Lt, Lt_rows, t_off);
    if (rc != DSPARK_OK) return rc;
    if (!x || !u_acc || !u_fin || !n_acc_out || !y_out)
        return fail(DSPARK_ERR_INVALID_ARG, "verify: a required pointer is NULL");
    const size_t need = dspark_verify_workspace_bytes(B, V, gamma);
    if (!ws || ws_bytes < need)
        return fail(DSPARK_ERR_WORKSPACE, "verify: workspace %zu bytes, need %zu", ws_bytes, need);
    Carver c(ws);
    float2* part = c.take<float2>(static_cast<size_t>(B) * (2 * gamma + 1) * row_chunks(V));
    float* csum = c.take<float>(static_cast<size_t>(B) * row_chunks(V));
    char* state = c.take<char>(static_cast<size_t>(B) * dspark::verify_state_bytes());
    dspark::RowSet rs{B, V, gamma, Ld, Lt, Lt_rows, t_off, len};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = dspark::launch_row_stats(rs, ld_lse, part, st);
    if (e != hipSuccess) return hip_fail(e, "verify/row_stats");
    e = dspark::launch_verify(rs, x, part, ld_lse, u_acc, u_fin, lse_d_out, lse_t_out, csum,
                              state, n_acc_out, y_out, st);
    if (e != hipSuccess) return hip_fail(e, "verify");
    return ok();
}

size_t dspark_verify_tv_workspace_bytes(int B, int V, int gamma) {
    if (B < 1 || V < 1 || gamma < 1) return 0;
    const size_t chunked = dspark_verify_workspace_bytes(B, V, gamma) +
                           align_up(static_cast<size_t>(B) * gamma * row_chunks(V) * sizeof(float));
    const size_t sweep = dspark::verify_sweep_bytes(B, V, gamma);
    return chunked > sweep ? chunked : sweep;
}

int dspark_verify_tv(int B, int V, int gamma, const float* Ld, const float* Lt, int Lt_rows,
                     const int32_t* t_off, const int32_t* len, const int32_t* x,
                     const float* ld_lse, const float* u_acc, const float* u_fin,
                     int32_t* n_acc_out, int32_t* y_out, float* lse_d_out, float* lse_t_out,
                     float* cstar_out, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_rows("verify_tv", B, V, gamma, Ld, Lt, Lt_rows, t_off);
    if (rc != DSPARK_OK) return rc;
    if (!x || !u_acc || !u_fin || !n_acc_out || !y_out || !cstar_out)
        return fail(DSPARK_ERR_INVALID_ARG, "verify_tv: a required pointer is NULL");
    const size_t need = dspark_verify_tv_workspace_bytes(B, V, gamma);
    if (!ws || ws_bytes < need)
        return fail(DSPARK_ERR_WORKSPACE, "verify_tv: workspace %zu bytes, need %zu", ws_bytes,
                    need);
    dspark::RowSet rs{B, V, gamma, Ld, Lt, Lt_rows, t_off, len};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (dspark::verify_sweep_ok(V) && dspark::verify_small_ok(rs)) {   // one launch
        const hipError_t e = dspark::launch_verify_small(rs, x, ld_lse, u_acc, u_fin, lse_d_out,
                                                         lse_t_out, n_acc_out, y_out, cstar_out, ws,
                                                         1u << 20, st);
        if (e != hipSuccess) return hip_fail(e, "verify_tv/small");
        return ok();
    }
    if (dspark::verify_sweep_ok(V)) {                 // every row read once
        const hipError_t e = dspark::launch_verify_sweep(rs, x, ld_lse, u_acc, u_fin, lse_d_out,
                                                         lse_t_out, n_acc_out, y_out, cstar_out, ws,
                                                         1u << 20, st);
        if (e != hipSuccess) return hip_fail(e, "verify_tv/sweep");
        return ok();
    }
    Carver c(ws);
    float2* part = c.take<float2>(static_cast<size_t>(B) * (2 * gamma + 1) * row_chunks(V));
    float* csum = c.take<float>(static_cast<size_t>(B) * row_chunks(V));
    char* state = c.take<char>(static_cast<size_t>(B) * dspark::verify_state_bytes());
    float* psum = c.take<float>(static_cast<size_t>(B) * gamma * row_chunks(V));
    hipError_t e = dspark::launch_row_stats(rs, ld_lse, part, st);
    if (e != hipSuccess) return hip_fail(e, "verify_tv/row_stats");
    e = dspark::launch_verify_tv(rs, x, part, ld_lse, u_acc, u_fin, lse_d_out, lse_t_out, csum,
                                 state, psum, n_acc_out, y_out, cstar_out, st);
    if (e != hipSuccess) return hip_fail(e, "verify_tv");
    return ok();
}

size_t dspark_verify_markov_workspace_bytes(int B, int V, int r, int gamma) {
    (void)r;
    if (B < 1 || V < 1 || gamma < 1) return 0;
    const size_t rows = static_cast<size_t>(B) * gamma;
    return part_bytes(B, V, gamma) + align_up((static_cast<size_t>(B) + 1) * sizeof(int32_t)) +
           align_up(8 * rows * sizeof(int32_t)) +
           align_up(static_cast<size_t>(B) * (gamma + 1) * sizeof(float)) +
           align_up(rows * dspark::verify_markov_tiles(V) * sizeof(float2)) +
           align_up(rows * sizeof(float));
}

int dspark_verify_markov(int B, int V, int r, int gamma, const float* U, const void* W1,
                         const void* W2, int w_dtype, const int32_t* x0, const int32_t* x,
                         const float* ld_lse, const float* Lt, int Lt_rows, const int32_t* t_off,
                         const int32_t* len, const float* u_acc, const float* u_fin,
                         int32_t* n_acc_out, int32_t* y_out, float* lse_t_out, float* cstar_out,
                         void* ws, size_t ws_bytes, void* stream) {
    int rc = check_rows("verify_markov", B, V, gamma, Lt, Lt, Lt_rows, t_off);
    if (rc != DSPARK_OK) return rc;
    if (r < 1) return fail(DSPARK_ERR_INVALID_ARG, "verify_markov: r=%d must be >= 1", r);
    if (w_dtype != DSPARK_BF16 || !dspark::verify_markov_ok(V, r))
        return fail(DSPARK_ERR_UNSUPPORTED,
                    "verify_markov: needs bf16 factors, r <= 256 with r %% 8 == 0, V %% 8 == 0 and "
                    "V <= 163840 (w_dtype=%d r=%d V=%d)", w_dtype, r, V);
    if (!U || !W1 || !W2 || !x0 || !x || !ld_lse || !u_acc || !u_fin || !n_acc_out || !y_out)
        return fail(DSPARK_ERR_INVALID_ARG, "verify_markov: a required pointer is NULL");
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) % 16) == 0; };
    if (!al16(U) || !al16(W1) || !al16(W2) || !al16(Lt))
        return fail(DSPARK_ERR_INVALID_ARG, "verify_markov: U, W1, W2 and Lt must be 16-byte aligned");
    const size_t need = dspark_verify_markov_workspace_bytes(B, V, r, gamma);
    if (!ws || ws_bytes < need)
        return fail(DSPARK_ERR_WORKSPACE, "verify_markov: workspace %zu bytes, need %zu", ws_bytes,
                    need);
    Carver c(ws);
    const size_t rows = static_cast<size_t>(B) * gamma;
    dspark::VerifyMarkovCall vc;
    vc.rs = dspark::RowSet{B, V, gamma, Lt, Lt, Lt_rows, t_off, len};
    vc.r = r; vc.U = U; vc.W1 = W1; vc.W2 = W2; vc.x0 = x0; vc.x = x; vc.ld_lse = ld_lse;
    vc.u_acc = u_acc; vc.u_fin = u_fin; vc.n_out = n_acc_out; vc.y_out = y_out;
    vc.lse_t_out = lse_t_out; vc.cstar = cstar_out;
    vc.part_t = c.take<float2>(static_cast<size_t>(B) * (2 * gamma + 1) * row_chunks(V));
    vc.d_off = c.take<int32_t>(static_cast<size_t>(B) + 1);
    vc.rec = c.take<int32_t>(8 * rows);
    vc.lse_t = c.take<float>(static_cast<size_t>(B) * (gamma + 1));
    vc.tvpart = c.take<float2>(rows * dspark::verify_markov_tiles(V));
    vc.ldx = c.take<float>(rows);
    const hipError_t e = dspark::launch_verify_markov(vc, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "verify_markov");
    return ok();
}

size_t dspark_tv_labels_workspace_bytes(int B, int V, int gamma) {
    if (B < 1 || V < 1 || gamma < 1) return 0;
    return part_bytes(B, V, gamma) +
           align_up(static_cast<size_t>(B) * gamma * row_chunks(V) * sizeof(float));
}

int dspark_tv_labels(int B, int V, int gamma, const float* Ld, const float* Lt, int Lt_rows,
                     const int32_t* t_off, const int32_t* len, const float* lse_d,
                     const float* lse_t, float* cstar_out, void* ws, size_t ws_bytes,
                     void* stream) {
    int rc = check_rows("tv_labels", B, V, gamma, Ld, Lt, Lt_rows, t_off);
    if (rc != DSPARK_OK) return rc;
    if (!cstar_out) return fail(DSPARK_ERR_INVALID_ARG, "tv_labels: cstar_out is NULL");
    const size_t need = dspark_tv_labels_workspace_bytes(B, V, gamma);
    if (!ws || ws_bytes < need)
        return fail(DSPARK_ERR_WORKSPACE, "tv_labels: workspace %zu bytes, need %zu", ws_bytes,
                    need);
    Carver c(ws);
    float2* part = c.take<float2>(static_cast<size_t>(B) * (2 * gamma + 1) * row_chunks(V));
    float* psum = c.take<float>(static_cast<size_t>(B) * gamma * row_chunks(V));
    dspark::RowSet rs{B, V, gamma, Ld, Lt, Lt_rows, t_off, len};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (!lse_d || !lse_t) {
        // partials of every row whose lse is missing (draft rows only when lse_d is missing)
        const hipError_t e = dspark::launch_row_stats(rs, lse_d, part, st);
        if (e != hipSuccess) return hip_fail(e, "tv_labels/row_stats");
    }
    const hipError_t e = dspark::launch_tv(rs, lse_d, lse_t, part, psum, cstar_out, st);
    if (e != hipSuccess) return hip_fail(e, "tv_labels");
    return ok();
}

// ----------------------------------------------------------------------------- schedule
size_t dspark_schedule_workspace_bytes(int R, int gamma, int Bmax) {
    (void)Bmax;
    if (R < 1 || gamma < 1) return 0;
    // row keys, ranked keys, ranks
    return align_up(static_cast<size_t>(R) * gamma * (2 * sizeof(double) + sizeof(int32_t)));
}

namespace {

// Shared checks and launch of dspark_schedule / dspark_schedule_lagged (ring_n: the ring's
// counter, conf then the base of its slots).
int schedule_check(const char* who, int R, int gamma, const float* conf, const float* sps,
                   int Bmax, int mode, const int32_t* len_out) {
    if (R < 1 || gamma < 1)
        return fail(DSPARK_ERR_INVALID_ARG, "%s: R=%d gamma=%d must be >= 1", who, R, gamma);
    if (gamma > 64 || static_cast<long long>(R) * gamma > dspark::schedule_max_candidates())
        return fail(DSPARK_ERR_UNSUPPORTED, "%s: R*gamma=%lld exceeds %d (or gamma > 64)", who,
                    static_cast<long long>(R) * gamma, dspark::schedule_max_candidates());
    if (Bmax < R || Bmax > (1 << 20))
        return fail(DSPARK_ERR_INVALID_ARG, "%s: need R <= Bmax <= 2^20 (R=%d Bmax=%d)", who, R,
                    Bmax);
    if (mode != DSPARK_SCHED_GLOBAL && mode != DSPARK_SCHED_EARLY_STOP)
        return fail(DSPARK_ERR_INVALID_ARG, "%s: unknown mode %d", who, mode);
    if (!conf || !sps || !len_out)
        return fail(DSPARK_ERR_INVALID_ARG, "%s: conf / sps / len_out is NULL", who);
    return DSPARK_OK;
}

int schedule_call(const char* who, int R, int gamma, const float* conf, const long long* ring_n,
                  const float* temp, const float* sps, int Bmax, int mode, int32_t* len_out,
                  int32_t* t_off_out, int32_t* K_out, float* theta_out, float* a_out, void* ws,
                  size_t ws_bytes, void* stream) {
    const int st = schedule_check(who, R, gamma, conf, sps, Bmax, mode, len_out);
    if (st != DSPARK_OK) return st;
    const size_t need = dspark_schedule_workspace_bytes(R, gamma, Bmax);
    if (!ws || ws_bytes < need)
        return fail(DSPARK_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", who, ws_bytes, need);
    const hipError_t e = dspark::launch_schedule(R, gamma, conf, ring_n, temp, sps, Bmax, mode,
                                                 len_out, t_off_out, K_out, theta_out, a_out,
                                                 static_cast<double*>(ws),
                                                 static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, who);
    return ok();
}

// Ring layout: the round counter (int64) in the first 256 bytes, then three [R][gamma] slots.
constexpr size_t kRingHeader = 256;

int check_ring(const char* who, int R, int gamma, const void* ring, size_t ring_bytes) {
    if (R < 1 || gamma < 1)
        return fail(DSPARK_ERR_INVALID_ARG, "%s: R=%d gamma=%d must be >= 1", who, R, gamma);
    if (static_cast<long long>(R) * gamma > dspark::schedule_max_candidates())
        return fail(DSPARK_ERR_UNSUPPORTED, "%s: R*gamma=%lld exceeds %d", who,
                    static_cast<long long>(R) * gamma, dspark::schedule_max_candidates());
    if (!ring || (reinterpret_cast<uintptr_t>(ring) % 8) != 0)
        return fail(DSPARK_ERR_INVALID_ARG, "%s: ring is NULL or not 8-byte aligned", who);
    const size_t need = dspark_conf_ring_bytes(R, gamma);
    if (ring_bytes < need)
        return fail(DSPARK_ERR_WORKSPACE, "%s: ring %zu bytes, need %zu", who, ring_bytes, need);
    return DSPARK_OK;
}

long long* ring_counter(const void* ring) {
    return static_cast<long long*>(const_cast<void*>(ring));
}
float* ring_slots(const void* ring) {
    return reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(ring)) + kRingHeader);
}

}  // namespace

int dspark_schedule(int R, int gamma, const float* conf, const float* temp, const float* sps,
                    int Bmax, int mode, int32_t* len_out, int32_t* t_off_out, int32_t* K_out,
                    float* theta_out, float* a_out, void* ws, size_t ws_bytes, void* stream) {
    return schedule_call("schedule", R, gamma, conf, nullptr, temp, sps, Bmax, mode, len_out,
                         t_off_out, K_out, theta_out, a_out, ws, ws_bytes, stream);
}

// ----------------------------------------------------------------------------- lag ring
size_t dspark_conf_ring_bytes(int R, int gamma) {
    if (R < 1 || gamma < 1) return 0;
    return kRingHeader + 3 * static_cast<size_t>(R) * gamma * sizeof(float);
}

int dspark_conf_ring_init(int R, int gamma, void* ring, size_t ring_bytes, void* stream) {
    const int st = check_ring("conf_ring_init", R, gamma, ring, ring_bytes);
    if (st != DSPARK_OK) return st;
    const hipError_t e = dspark::launch_conf_ring_init(ring_counter(ring), ring_slots(ring), R, gamma,
                                                       static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "conf_ring_init");
    return ok();
}

int dspark_conf_ring_push(int R, int gamma, void* ring, size_t ring_bytes, const float* conf,
                          void* stream) {
    const int st = check_ring("conf_ring_push", R, gamma, ring, ring_bytes);
    if (st != DSPARK_OK) return st;
    if (!conf) return fail(DSPARK_ERR_INVALID_ARG, "conf_ring_push: conf is NULL");
    const hipError_t e = dspark::launch_conf_ring_push(ring_counter(ring), ring_slots(ring), conf, R,
                                                       gamma, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "conf_ring_push");
    return ok();
}

int dspark_schedule_lagged(int R, int gamma, const void* ring, size_t ring_bytes, const float* temp,
                           const float* sps, int Bmax, int mode, int32_t* len_out,
                           int32_t* t_off_out, int32_t* K_out, float* theta_out, float* a_out,
                           void* ws, size_t ws_bytes, void* stream) {
    const int st = check_ring("schedule_lagged", R, gamma, ring, ring_bytes);
    if (st != DSPARK_OK) return st;
    return schedule_call("schedule_lagged", R, gamma, ring_slots(ring), ring_counter(ring), temp, sps,
                         Bmax, mode, len_out, t_off_out, K_out, theta_out, a_out, ws, ws_bytes,
                         stream);
}

// ----------------------------------------------------------------------------- draft + schedule
size_t dspark_markov_draft_schedule_workspace_bytes(int B, int V, int r, int gamma, int R, int Bmax) {
    const size_t d = dspark_markov_draft_workspace_bytes(B, V, r, gamma);
    const size_t s = dspark_schedule_workspace_bytes(R, gamma, Bmax);
    if (!d || !s) return 0;
    return align_up(d) + s;
}

int dspark_markov_draft_schedule_fused(int B, int V, int r, int gamma, int w_dtype, const void* W1,
                                       const void* W2, int R) {
    if (R < 1 || gamma < 1 || static_cast<long long>(R) * gamma > dspark::sched::kSmallCand) return 0;
    return dspark_markov_draft_path(B, V, r, w_dtype, W1, W2) == DSPARK_PATH_RESIDENT &&
                   dspark::draft_resident_takes_job(V)
               ? 1
               : 0;
}

int dspark_markov_draft_schedule(int B, int V, int r, int gamma, const float* U, const void* W1,
                                 const void* W2, int w_dtype, const int32_t* x0, const float* u,
                                 int32_t* x_out, float* q_out, float* lse_out, float* Ld_out, int R,
                                 const float* conf, const void* ring, size_t ring_bytes,
                                 const float* temp, const float* sps, int Bmax, int mode,
                                 int32_t* len_out, int32_t* t_off_out, int32_t* K_out,
                                 float* theta_out, float* a_out, void* ws, size_t ws_bytes,
                                 void* stream) {
    const char* who = "markov_draft_schedule";
    const float* cf = conf;
    const long long* ring_n = nullptr;
    if (ring) {
        const int st = check_ring(who, R, gamma, ring, ring_bytes);
        if (st != DSPARK_OK) return st;
        cf = ring_slots(ring);
        ring_n = ring_counter(ring);
    }
    int st = schedule_check(who, R, gamma, cf, sps, Bmax, mode, len_out);
    if (st != DSPARK_OK) return st;
    const size_t need = dspark_markov_draft_schedule_workspace_bytes(B, V, r, gamma, R, Bmax);
    if (!need) return fail(DSPARK_ERR_INVALID_ARG, "%s: B=%d V=%d gamma=%d must be >= 1", who, B, V, gamma);
    if (!ws || ws_bytes < need)
        return fail(DSPARK_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", who, ws_bytes, need);
    const size_t dbytes = align_up(dspark_markov_draft_workspace_bytes(B, V, r, gamma));
    const dspark::sched::SmallJob job{R, gamma, cf, ring_n, temp, sps, Bmax, mode,
                                      len_out, t_off_out, K_out, theta_out, a_out};
    const bool small = static_cast<long long>(R) * gamma <= dspark::sched::kSmallCand;
    bool taken = false;
    st = draft_run(who, B, V, r, gamma, U, W1, W2, w_dtype, x0, u, x_out, q_out, lse_out, Ld_out, ws,
                   dbytes, stream, 0, small ? &job : nullptr, &taken);
    if (st != DSPARK_OK || taken) return st;
    return schedule_call(who, R, gamma, cf, ring_n, temp, sps, Bmax, mode, len_out, t_off_out, K_out,
                         theta_out, a_out, static_cast<char*>(ws) + dbytes, ws_bytes - dbytes, stream);
}

// ----------------------------------------------------------------------------- STS fit
size_t dspark_sts_fit_workspace_bytes(int N, int gamma, int n_grid) {
    if (N < 1 || gamma < 1 || n_grid < 1) return 0;
    const size_t cells = static_cast<size_t>(N) * gamma;
    return align_up(cells * sizeof(double)) + align_up(cells) +
           align_up(dspark::sts_stats_bytes(N, gamma, n_grid));
}

int dspark_sts_fit(int N, int gamma, const float* conf, const int32_t* n_acc, const int32_t* len,
                   const float* grid, int n_grid, int bins, int objective, float* T_out,
                   float* ece_before, float* ece_after, float* obj_out, void* ws, size_t ws_bytes,
                   void* stream) {
    if (N < 1 || gamma < 1 || n_grid < 1 || bins < 1)
        return fail(DSPARK_ERR_INVALID_ARG, "sts_fit: N=%d gamma=%d n_grid=%d bins=%d must be >= 1",
                    N, gamma, n_grid, bins);
    if (gamma > 64 || n_grid > 4096 || bins > dspark::sts_max_bins() ||
        static_cast<long long>(N) * gamma >= (1LL << 31))
        return fail(DSPARK_ERR_UNSUPPORTED, "sts_fit: gamma=%d n_grid=%d bins=%d N*gamma outside caps",
                    gamma, n_grid, bins);
    if (objective != DSPARK_STS_NLL && objective != DSPARK_STS_ECE)
        return fail(DSPARK_ERR_INVALID_ARG, "sts_fit: unknown objective %d", objective);
    if (!conf || !n_acc || !grid || !T_out || !ece_before || !ece_after)
        return fail(DSPARK_ERR_INVALID_ARG, "sts_fit: a required pointer is NULL");
    const size_t need = dspark_sts_fit_workspace_bytes(N, gamma, n_grid);
    if (!ws || ws_bytes < need)
        return fail(DSPARK_ERR_WORKSPACE, "sts_fit: workspace %zu bytes, need %zu", ws_bytes, need);
    Carver c(ws);
    const size_t cells = static_cast<size_t>(N) * gamma;
    double* gt = c.take<double>(cells);
    int8_t* ot = c.take<int8_t>(cells);
    auto* part = c.take<unsigned long long>(dspark::sts_stats_bytes(N, gamma, n_grid) /
                                            sizeof(unsigned long long));
    const hipError_t e = dspark::launch_sts_fit(N, gamma, conf, n_acc, len, grid, n_grid, bins,
                                                objective, gt, ot, part, T_out, ece_before,
                                                ece_after, obj_out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "sts_fit");
    return ok();
}

}  // extern "C"
