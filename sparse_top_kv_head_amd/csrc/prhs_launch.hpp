// Internal launchers behind the C ABI. Arguments are already validated.
#pragma once

#include <hip/hip_runtime.h>

#include "prhs.h"

namespace prhs {

// Score scan geometry: keys per workgroup.
constexpr int kScoreChunk = 256;
// Sparse decode geometry: selected rows per workgroup (one split).
constexpr int kDecodeRows = 256;

inline int score_nchunks(const prhs_dims& d) { return (d.ctx_len + kScoreChunk - 1) / kScoreChunk; }
inline int decode_nsplit(int cap) { return (cap + kDecodeRows - 1) / kDecodeRows; }

// Writes scores; with ws, also the per-chunk (max, sum) partials of the dense
// softmax; with lse_all (needs ws), also merges them into lse_all.
hipError_t launch_score(const prhs_dims& d, const void* q, const void* k, float* scores,
                        float* lse_all, void* ws, hipStream_t stream);

// score_ws: when non-NULL, the per-chunk partials that launch_score left in
// that workspace; the select kernel then merges them and writes lse_all
// itself. Otherwise lse_all is an input (read in DELTA mode only).
hipError_t launch_select(const prhs_dims& d, const float* scores, float* lse_all,
                         const void* score_ws, int mode, int n_budget, float delta_target,
                         int* idx, int idx_cap, int* count, int* cap_hit, hipStream_t stream);

hipError_t launch_cis(const prhs_dims& d, const int* anchor_idx, int anchor_cap,
                      const int* anchor_count, int radius, const void* q_cur, const void* q_anchor,
                      float sim_tau, int* out_idx, int out_cap, int* out_count, int* reuse_ok,
                      hipStream_t stream);

hipError_t launch_decode(const prhs_dims& d, const void* q, const void* k, const void* v,
                         const int* idx, int idx_cap, const int* count, const float* scores,
                         const float* lse_all, float* out, float* lse_sel, float* delta, float* tau,
                         void* ws, hipStream_t stream);

hipError_t launch_dropped_mass(const prhs_dims& d, const float* lse_sel, const float* lse_all,
                               float* delta, float* tau, hipStream_t stream);

}  // namespace prhs
