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
// Rows the one-workgroup-per-head decode holds (their scores in LDS), and
// whether a decode runs that way: the heads alone fill about half of the 256
// CUs, or the set fits one split anyway.
constexpr int kDecodeHeadRows = 8192;
inline bool decode_per_head(const prhs_dims& d, int cap) {
  return cap <= kDecodeHeadRows && (d.batch * d.n_q_heads >= 128 || cap <= kDecodeRows);
}

// Count marking a (head, chunk) for which no candidates were written.
constexpr uint32_t kNoCand = 0xFFFFFFFFu;

// Candidate output of the scan: keys whose score >= theta[head] (theta not
// finite: none), as (score bits, index) in cand[head][chunk][0:kScoreChunk],
// counts in cand_cnt[head][chunk]. All NULL: no candidate output.
struct ScanCand {
  const float* theta = nullptr;
  uint2* cand = nullptr;
  uint32_t* cand_cnt = nullptr;
  const int* active = nullptr;   // per query head; a KV group with no active head is skipped
  // Matrix-core scan only: no score row for heads with a finite theta (the
  // selection recomputes it when the candidates miss).
  bool skip_hinted = false;
};

// The scan scores on the matrix cores: fp16 rows of 128, and a unit's rows
// addressable with 32-bit byte offsets.
inline bool scan_uses_mfma(const prhs_dims& d) {
  return d.dtype == PRHS_F16 && d.head_dim == 128 &&
         (unsigned long long)d.ctx_len * (unsigned long long)d.kv_stride_t * 2ull < (1ull << 32);
}

// Writes scores; with ws, also the per-chunk (max, sum) partials of the dense
// softmax; with lse_all (needs ws), also merges them into lse_all.
hipError_t launch_score(const prhs_dims& d, const void* q, const void* k, float* scores,
                        float* lse_all, void* ws, hipStream_t stream,
                        const ScanCand* cand = nullptr);

// Arguments of the selection kernel (t, ld and nchunks are filled in by
// launch_select from the dims).
struct SelectArgs {
  const float* scores = nullptr;
  float* lse_all = nullptr;       // read in DELTA mode unless part is given
  const float2* part = nullptr;   // scan partials: merged into lse_all by the kernel
  int mode = PRHS_TOPN;
  int n_budget = 0;
  float delta_target = 0.f;
  int* idx = nullptr;
  int idx_cap = 0;
  int* count = nullptr;
  int* cap_hit = nullptr;
  float* sel_scores = nullptr;    // scores of the selected keys, in idx order
  const uint2* cand = nullptr;    // scan candidates (TOPN)
  const uint32_t* cand_cnt = nullptr;
  float* theta_out = nullptr;     // next-step threshold hint per unit query norm (TOPN)
  const void* hint_q = nullptr;   // the queries [heads, head_dim] whose norms scale theta_out
  int hint_q_f16 = 1;             // hint_q element type: fp16 (else fp32)
  int hint_d = 128;               // hint_q row length (64 or 128)
  // Score rows skipped by a hinted matrix-core scan: when the candidates of
  // such a head miss, its row is recomputed from q and K (strides kv_*,
  // heads hq / hkv) into rescore_row before the full search.
  const void* rescore_q = nullptr;
  const void* rescore_k = nullptr;
  float* rescore_row = nullptr;
  float rescore_scale = 0.f;
  const int* active = nullptr;    // per head; inactive heads are left untouched
  // Fused decode (TOPN or DELTA with scan partials, fp16 rows of 128): when v is given,
  // each head's workgroup attends over its own selection and writes out,
  // lse_sel and, when delta is given, delta (and tau).
  const void* v = nullptr;
  long long kv_sb = 0, kv_sh = 0, kv_st = 0;  // element strides of V
  int hq = 0, hkv = 0;
  float* out = nullptr;
  float* lse_sel = nullptr;
  float* delta = nullptr;
  float* tau = nullptr;
  int t = 0;
  int ld = 0;
  int nchunks = 0;
};

hipError_t launch_select(const prhs_dims& d, const SelectArgs& a, hipStream_t stream);

// Largest budget the fused select-and-decode takes. At any head count it
// beats the select kernel followed by the split decode and its merge: a head's
// V rows (at most 512 KiB) take one CU about as long as the two launches and
// the round trips through the selection's outputs that it saves.
constexpr int kFuseRows = 2048;
inline bool fuse_decode(const prhs_dims& d, int mode, int n_budget) {
  return (mode == PRHS_TOPN || mode == PRHS_DELTA) && d.dtype == PRHS_F16 && d.head_dim == 128 &&
         n_budget <= kFuseRows;
}

hipError_t launch_cis(const prhs_dims& d, const int* anchor_idx, int anchor_cap,
                      const int* anchor_count, int radius, const void* q_cur, const void* q_anchor,
                      float sim_tau, int* out_idx, int out_cap, int* out_count, int* reuse_ok,
                      hipStream_t stream, const int* skip = nullptr);

// Control scores of the random expansion: anchor members score high, every
// other key minus its 23-bit draw (rows of ld floats).
hipError_t launch_expand_scores(const prhs_dims& d, const int* anchor_idx, int anchor_cap,
                                const int* anchor_count, const int* draws, float* out,
                                hipStream_t stream);

// Similarity gate of the adaptive CIS step, per head: refresh = force, or no
// anchor yet, or cos(q, q_anchor) < sim_tau; a refreshing head's q_anchor
// becomes q. sim (nullable) receives the cosine (NaN without an anchor).
hipError_t launch_gate(const prhs_dims& d, const void* q, void* q_anchor, const int* anchor_count,
                       int force, float sim_tau, int* refresh, float* sim, hipStream_t stream);

// Scores of the selected rows come from sel_scores (compact, in idx order) if
// given, else are gathered from scores, else computed from gathered K rows.
hipError_t launch_decode(const prhs_dims& d, const void* q, const void* k, const void* v,
                         const int* idx, int idx_cap, const int* count, const float* sel_scores,
                         const float* scores,
                         const float* lse_all, float* out, float* lse_sel, float* delta, float* tau,
                         void* ws, hipStream_t stream);

// Merge split partials [head][nsplit][d + 2] = (o[d], max, sum) of every head
// into out and lse; delta/tau from lse_all when given.
hipError_t launch_merge(const prhs_dims& d, const float* part, int nsplit, float* out,
                        float* lse, const float* lse_all, float* delta, float* tau,
                        hipStream_t stream, const int* mix = nullptr);

// Decode where head h attends over (idx, count, sel_scores) when mix[h] != 0
// and over (idx2, count2) with scores from gathered K rows otherwise; delta
// and tau are written for the mix[h] != 0 heads only.
// CIS reuse step: dilation of the anchor sets, then the decode over gathered
// K and V rows; in one kernel when the per-head decode applies, out_cap fits
// its LDS and the windows are short, else dilation and decode back to back.
// Results equal those of the two steps in sequence, bit for bit.
hipError_t launch_reuse(const prhs_dims& d, const int* anchor_idx, int anchor_cap,
                        const int* anchor_count, int radius, const void* q, const void* k,
                        const void* v, int* out_idx, int out_cap, int* out_count, float* out,
                        float* lse_sel, void* ws, hipStream_t stream);

// Adaptive step's decode: heads with mix[head] != 0 attend over their fresh
// selection with its scores; the others dilate their anchor set (into
// dil_idx / dil_count, which fresh heads leave untouched) and attend with
// gathered K rows. One kernel when the per-head decode applies and the windows
// are short, else the masked dilation and the mixed decode; the results are the
// same bit for bit.
hipError_t launch_adaptive_decode(const prhs_dims& d, const void* q, const void* k,
                                  const void* v, const int* mix, const int* anchor_idx,
                                  int anchor_cap, const int* anchor_count,
                                  const float* sel_scores, int radius, int* dil_idx, int dil_cap,
                                  int* dil_count, const float* lse_all, float* out,
                                  float* lse_sel, float* delta, float* tau, void* ws,
                                  hipStream_t stream);

hipError_t launch_decode_mixed(const prhs_dims& d, const void* q, const void* k, const void* v,
                               const int* mix, const int* idx, int idx_cap, const int* count,
                               const float* sel_scores, const int* idx2, int idx2_cap,
                               const int* count2, const float* lse_all, float* out,
                               float* lse_sel, float* delta, float* tau, void* ws,
                               hipStream_t stream);

// Dense attention over all ctx_len keys: split partials in ws, then the merge.
// k[b, g, pos, :] = k_new[b, g, :] and v[b, g, pos, :] = v_new[b, g, :].
hipError_t launch_append_kv(const prhs_dims& d, const void* k_new, const void* v_new, void* k,
                            void* v, int pos, hipStream_t stream);

hipError_t launch_dense(const prhs_dims& d, const void* q, const void* k, const void* v,
                        float* out, float* lse, void* ws, hipStream_t stream);

// Read `bytes` (a multiple of 16) of device memory once (HBM ceiling probe).
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

// Bits of the device-check words (builds with PRHS_DEVICE_CHECKS).
enum : uint32_t {
  kCheckIndex = 1u,  // an index of a given set lies outside [0, t)
  kCheckOrder = 2u,  // an anchor set is not strictly ascending
  kCheckList = 4u,   // a candidate list would exceed its LDS capacity
};

// Device-check words of the kernel sources (read and cleared; always 0 unless
// the library is built with PRHS_DEVICE_CHECKS; bit 31 if the read failed).
uint32_t take_checks_select();
uint32_t take_checks_decode();
uint32_t take_checks_cis();

hipError_t launch_dropped_mass(const prhs_dims& d, const float* lse_sel, const float* lse_all,
                               float* delta, float* tau, hipStream_t stream);

}  // namespace prhs
