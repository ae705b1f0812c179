// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

// ---------------------------------------------------------------- draft
struct DraftStep {
    int B, V, r, gamma, k, w_dtype;
    const float* U;
    const void* W1;
    const void* W2;
    const int32_t* prev;      // x_{k-1}: prev[b * prev_stride]
    int prev_stride;
    float* L;                 // logits rows: L + b * L_bstride
    long long L_bstride;
    float2* part;             // [B][nblk] tile partials (max, sum exp)
    int nblk;
    unsigned int* counters;   // [draft_counter_count(B)] zero between launches
    const float* u;
    int32_t* x_out;
    float* q_out;
    float* lse_out;
};

int draft_tile_cols();
int draft_counter_count(int B);
hipError_t launch_draft_step(const DraftStep& s, hipStream_t st);

// ---------------------------------------------------------------- verify / TV
struct RowSet {               // the draft and target rows of a verify batch
    int B, V, gamma;
    const float* Ld;
    const float* Lt;
    int Lt_rows;
    const int32_t* t_off;     // nullable
    const int32_t* len;       // nullable
};

// lse of every target row (lse_t [B][gamma+1]) and, unless lse_d_in is given, of every
// draft row (lse_d [B][gamma]); lse_d_in is copied into lse_d otherwise. Slots beyond a
// request's length, and faulty requests, get NaN.
hipError_t launch_row_lse(const RowSet& rs, const float* lse_d_in, float* lse_d, float* lse_t,
                          hipStream_t st);

int verify_chunk_elems();
hipError_t launch_verify_finish(const RowSet& rs, const int32_t* x, const float* lse_d,
                                const float* lse_t, const float* u_acc, const float* u_fin,
                                float* chunk_ws, int nchunk, int32_t* n_out, int32_t* y_out,
                                hipStream_t st);

hipError_t launch_tv(const RowSet& rs, const float* lse_d, const float* lse_t, float* cstar,
                     hipStream_t st);

// ---------------------------------------------------------------- schedule
int schedule_max_candidates();
hipError_t launch_schedule(int R, int gamma, const float* conf, const float* temp,
                           const float* sps, int Bmax, int mode, int32_t* len_out,
                           int32_t* t_off_out, int32_t* K_out, float* theta_out, float* a_out,
                           hipStream_t st);

}  // namespace dspark
