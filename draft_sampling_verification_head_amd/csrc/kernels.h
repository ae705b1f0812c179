// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspark {

// ---------------------------------------------------------------- draft
namespace sched { struct SmallJob; }

struct DraftCall {
    int B, V, r, gamma, w_dtype;
    const float* U;
    const void* W1;
    const void* W2;
    const int32_t* x0;
    const float* u;
    int32_t* x_out;
    float* q_out;
    float* lse_out;
    float* L[64];             // logits rows of step k: L[k] + b * L_bstride
    long long L_bstride;
    bool L_out;               // L[k] is the caller's output (else workspace the path may skip)
    bool per_position = false;   // no persistent launch: each position is its own launches
    float2* part[2];          // tile partials [B][draft_part_tiles(V)] of even / odd steps
    float2* slots;            // max(draft_resident_slot_bytes, draft_slab_flag_bytes) of workspace
    unsigned* status;         // one-launch forms: number of workgroups that gave up waiting
    unsigned spin = 1u << 20; // polls before a one-launch form gives up (about a second)
    // a one-wave schedule the single-request launch runs in one extra workgroup (the caller
    // checks draft_resident_takes_job first); null: none
    const sched::SmallJob* job = nullptr;
};

// Which path (DSPARK_PATH_*) launch_draft takes for this call, and whether it runs every
// position in one launch.
int draft_path_of(const DraftCall& c, bool* one_launch);

// Vocabulary tiles per request the partial buffers must hold (the finest tiling in use).
int draft_part_tiles(int V);
hipError_t launch_draft(const DraftCall& c, hipStream_t st);

// Batched path on bf16 MFMA (draft_mfma.hip), chosen by launch_draft when it applies.
bool draft_mfma_ok(int B, int V, int r, int w_dtype, const void* W1, const void* W2);
int draft_mfma_tile_cols();
hipError_t launch_draft_mfma(const DraftCall& c, hipStream_t st);

// Batched path with each vocabulary slab of W2 in registers (draft_slab.hip), chosen by
// launch_draft when it applies and U (and the caller's logits output) are 16-byte aligned.
bool draft_slab_ok(int B, int V, int r, int w_dtype, const void* W1, const void* W2);
int draft_slab_tiles(int V);
size_t draft_slab_flag_bytes(int V, int gamma);   // position flags of the one-launch form
bool draft_slab_one_launch(int B, int V, bool L_out);   // whether a slab call is that form
hipError_t launch_draft_slab(const DraftCall& c, hipStream_t st);

// Single-request path with W2 resident in registers (draft_resident.hip), chosen by
// launch_draft when it applies: one launch covers all gamma positions.
bool draft_resident_ok(int B, int V, int r, int w_dtype, const void* W1, const void* W2);
int draft_resident_tile_cols();
size_t draft_resident_slot_bytes(int V, int gamma);
// Whether the single-request launch at this V can add one workgroup for a schedule job (every
// workgroup of the launch resident at once, the draft's included).
bool draft_resident_takes_job(int V);
hipError_t launch_draft_resident(const DraftCall& c, hipStream_t st);

// RNN-head draft (the recurrence h_1 = W1[x_0], h_k = A h_{k-1} + W1[x_{k-1}], B_k = h_k W2):
// the draft's arguments and workspace plus the recurrence and the state buffers.
struct RnnCall {
    DraftCall d;              // bf16 factors; d.slots / d.status used by the one-launch form
    const void* A;            // [r][r] bf16
    float* h_out;             // [B][gamma][r] fp32 states (nullable)
    float* hstate[2];         // [B][r] fp32, ping-pong (batched form)
    uint16_t* hrows;          // [B][2][rnn_rank_pad(r)] bf16 hi / lo rows (batched form)
    float* ah;                // [B][r] fp32 A h_k (batched form)
};
int rnn_rank_pad(int r);
bool rnn_mfma_ok(int V, int r, const void* W1, const void* W2, const void* A);
hipError_t launch_rnn_mfma(const RnnCall& c, hipStream_t st);
bool rnn_resident_ok(int B, int V, int r, const void* W1, const void* W2, const void* A);
hipError_t launch_rnn_resident(const RnnCall& c, hipStream_t st);

// ---------------------------------------------------------------- verify / TV
struct RowSet {               // the draft and target rows of a verify batch
    int B, V, gamma;
    const float* Ld;
    const float* Lt;
    int Lt_rows;
    const int32_t* t_off;     // nullable
    const int32_t* len;       // nullable
};

int verify_chunk_elems();
size_t verify_state_bytes();

// Chunk (max, sum exp) partials of every verified row: part [B][2gamma+1][nch], slot s <=
// gamma is target row s, slot gamma+1+k is draft row k (skipped when lse_d_in is given).
hipError_t launch_row_stats(const RowSet& rs, const float* lse_d_in, float2* part,
                            hipStream_t st);

// Acceptance scan + residual / bonus draw from the row partials. csum: [B][nch] chunk
// masses; state: [B] per-request records of verify_state_bytes() each.
hipError_t launch_verify(const RowSet& rs, const int32_t* x, const float2* part,
                         const float* lse_d_in, const float* u_acc, const float* u_fin,
                         float* lse_d_out, float* lse_t_out, float* csum, void* state,
                         int32_t* n_out, int32_t* y_out, hipStream_t st);

// Verify and TV labels together, after launch_row_stats: two launches instead of four.
// psum: [B][gamma][nch].
hipError_t launch_verify_tv(const RowSet& rs, const int32_t* x, const float2* part,
                            const float* lse_d_in, const float* u_acc, const float* u_fin,
                            float* lse_d_out, float* lse_t_out, float* csum, void* state,
                            float* psum, int32_t* n_out, int32_t* y_out, float* cstar,
                            hipStream_t st);

// Verify and TV labels in one pass over the rows (two launches: the sweep, then the draws and
// the c* merges), with the same results as launch_row_stats + launch_verify_tv bit for bit.
// Applies when a row has at most 64 chunks and the sweep's persistent grid fits the device.
// `ws` holds verify_sweep_bytes(B, V, gamma) bytes (a call counter in its first word; the
// rest needs no preparation). `spin`: polls before a wait gives up.
size_t verify_sweep_bytes(int B, int V, int gamma);
bool verify_sweep_ok(int V);
// The same in one launch, one workgroup per (row, chunk) task, where every task fits the
// device at once (small batches); the same workspace layout header and results.
bool verify_small_ok(const RowSet& rs);
hipError_t launch_verify_small(const RowSet& rs, const int32_t* x, const float* lse_d_in,
                               const float* u_acc, const float* u_fin, float* lse_d_out,
                               float* lse_t_out, int32_t* n_out, int32_t* y_out, float* cstar,
                               void* ws, unsigned spin, hipStream_t st);
hipError_t launch_verify_sweep(const RowSet& rs, const int32_t* x, const float* lse_d_in,
                               const float* u_acc, const float* u_fin, float* lse_d_out,
                               float* lse_t_out, int32_t* n_out, int32_t* y_out, float* cstar,
                               void* ws, unsigned spin, hipStream_t st);

// TV labels; normalisers from lse_d / lse_t when given, else merged from `part`.
// psum: [B][gamma][nch].
hipError_t launch_tv(const RowSet& rs, const float* lse_d, const float* lse_t,
                     const float2* part, float* psum, float* cstar, hipStream_t st);

// Verify + TV labels with the draft logits rebuilt from the Markov factors
// (verify_markov.hip). Workspace regions are carved by the host layer.
struct VerifyMarkovCall {
    RowSet rs;                // Ld unused (set to Lt)
    int r;
    const float* U;
    const void* W1;
    const void* W2;
    const int32_t* x0;
    const int32_t* x;
    const float* ld_lse;
    const float* u_acc;
    const float* u_fin;
    int32_t* n_out;
    int32_t* y_out;
    float* lse_t_out;
    float* cstar;
    float2* part_t;           // [B][2 gamma + 1][chunks] row partials
    int32_t* d_off;           // [B + 1]
    int32_t* rec;             // [8][B gamma]
    float* lse_t;             // [B][gamma + 1]
    float2* tvpart;           // [B gamma][verify_markov_tiles(V)]
    float* ldx;               // [B gamma]
};
int verify_markov_tiles(int V);
bool verify_markov_ok(int V, int r);
hipError_t launch_verify_markov(const VerifyMarkovCall& c, hipStream_t st);

// ---------------------------------------------------------------- schedule
int schedule_max_candidates();
// conf: the confidences, or with ring_n the base of the three ring slots (the lagged slot is
// resolved on the device from the counter).
hipError_t launch_schedule(int R, int gamma, const float* conf, const long long* ring_n,
                           const float* temp, const float* sps, int Bmax, int mode,
                           int32_t* len_out, int32_t* t_off_out, int32_t* K_out, float* theta_out,
                           float* a_out, double* a_ws, hipStream_t st);
hipError_t launch_conf_ring_init(long long* ring_n, float* slots, int R, int gamma, hipStream_t st);
hipError_t launch_conf_ring_push(long long* ring_n, float* slots, const float* conf, int R, int gamma,
                                 hipStream_t st);

// ---------------------------------------------------------------- STS fit
int sts_max_bins();
size_t sts_stats_bytes(int N, int gamma, int n_grid);
hipError_t launch_sts_fit(int N, int G, const float* conf, const int32_t* n_acc,
                          const int32_t* len, const float* grid, int nT, int bins, int objective,
                          double* gt, int8_t* ot, unsigned long long* part, float* T_out,
                          float* ece_before, float* ece_after, float* obj_out, hipStream_t st);

}  // namespace dspark
