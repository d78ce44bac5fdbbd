// C ABI of the PrHS decode hot path: host-side validation and dispatch.
//
// Every entry point checks all of its arguments before touching the HIP
// runtime, so an invalid call returns its status with nothing enqueued and no
// output written. Launch errors are reported as PRHS_E_HIP.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "prhs.h"
#include "prhs_probe.h"
#include "prhs_launch.hpp"

namespace {

thread_local char g_last_error[256] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return PRHS_OK;
}

bool debug_sync() {
  static const bool on = [] {
    const char* e = std::getenv("PRHS_DEBUG_SYNC");
    return e != nullptr && e[0] == '1';
  }();
  return on;
}

#ifdef PRHS_DEVICE_CHECKS
constexpr bool kDeviceChecks = true;
#else
constexpr bool kDeviceChecks = false;
#endif

// True while `stream` is being captured into a graph: nothing may wait on it.
bool capturing(hipStream_t stream) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(stream, &st) == hipSuccess && st == hipStreamCaptureStatusActive;
}

int finish(hipError_t err, hipStream_t stream, const char* what) {
  // the debug synchronisation and the device checks are skipped for work
  // being captured into a graph (it has not run yet)
  const bool check = kDeviceChecks && err == hipSuccess && !capturing(stream);
  if (err == hipSuccess && (debug_sync() || check) && !capturing(stream)) {
    err = hipStreamSynchronize(stream);
    if (err == hipSuccess) err = hipGetLastError();
  }
  if (err != hipSuccess) return fail(PRHS_E_HIP, "%s: %s", what, hipGetErrorString(err));
  if (check) {
    // the checked build: every kernel source's check word, read and cleared
    const uint32_t bits =
        prhs::take_checks_select() | prhs::take_checks_decode() | prhs::take_checks_cis();
    if (bits != 0u)
      return fail(PRHS_E_HIP, "%s: device check failed (0x%x):%s%s%s%s", what, bits,
                  (bits & prhs::kCheckIndex) ? " an index outside [0, t)" : "",
                  (bits & prhs::kCheckOrder) ? " an anchor set not strictly ascending" : "",
                  (bits & prhs::kCheckList) ? " a candidate list past its capacity" : "",
                  (bits & 0x80000000u) ? " (check words unreadable)" : "");
  }
  return ok();
}

size_t elem_size(int dtype) { return dtype == PRHS_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by every call that takes dims.
int check_dims(const prhs_dims* d) {
  if (d == nullptr) return fail(PRHS_E_NULL, "dims is NULL");
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
    return fail(PRHS_E_DIMS, "batch and head counts must be >= 1");
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(PRHS_E_DIMS, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", d->n_q_heads,
                d->n_kv_heads);
  if ((long long)d->batch * d->n_q_heads > 65535)
    return fail(PRHS_E_DIMS, "batch * n_q_heads must be <= 65535");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PRHS_E_DIMS, "head_dim must be 64 or 128 (got %d)", d->head_dim);
  if (d->ctx_len < 1) return fail(PRHS_E_DIMS, "ctx_len must be >= 1");
  if (d->dtype != PRHS_F32 && d->dtype != PRHS_F16)
    return fail(PRHS_E_DTYPE, "unknown dtype %d", d->dtype);
  if (d->kv_stride_t < d->head_dim || d->kv_stride_h < 0 || d->kv_stride_b < 0)
    return fail(PRHS_E_DIMS, "kv strides must be non-negative and kv_stride_t >= head_dim");
  const long long es = (long long)elem_size(d->dtype);
  if ((d->kv_stride_t * es) % 16 || (d->kv_stride_h * es) % 16 || (d->kv_stride_b * es) % 16)
    return fail(PRHS_E_ALIGN, "kv strides must keep rows 16-byte aligned");
  if (d->scores_ld < d->ctx_len) return fail(PRHS_E_DIMS, "scores_ld must be >= ctx_len");
  if (d->scores_ld % 4) return fail(PRHS_E_ALIGN, "scores_ld must be a multiple of 4");
  return PRHS_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t score_part_bytes(const prhs_dims* d) {
  return (size_t)d->batch * d->n_q_heads * prhs::score_nchunks(*d) * 2 * sizeof(float);
}

size_t decode_part_bytes(const prhs_dims* d, int cap) {
  return (size_t)d->batch * d->n_q_heads * prhs::decode_nsplit(cap) * (d->head_dim + 2) *
         sizeof(float);
}

size_t score_ws(const prhs_dims* d) { return score_part_bytes(d); }

size_t decode_ws(const prhs_dims* d, int cap) { return decode_part_bytes(d, cap); }

// Random expansion: one control-score row (scores_ld floats) per head.
size_t expand_ws(const prhs_dims* d) {
  return (size_t)d->batch * d->n_q_heads * (size_t)d->scores_ld * sizeof(float);
}

// Dense decode: split partials over all t keys.
size_t dense_ws(const prhs_dims* d) { return decode_part_bytes(d, d->ctx_len); }

// Anchor-step workspace: scan partials | candidate counts | candidates |
// selected scores | decode partials, each part 256-byte aligned.
struct StepWs {
  size_t part, cnt, cand, sel, dec, total;
};

StepWs step_ws_layout(const prhs_dims* d, int cap) {
  const size_t heads = (size_t)d->batch * d->n_q_heads;
  const size_t nch = (size_t)prhs::score_nchunks(*d);
  StepWs w;
  w.part = 0;
  w.cnt = w.part + align256(score_part_bytes(d));
  w.cand = w.cnt + align256(heads * nch * sizeof(uint32_t));
  w.sel = w.cand + align256(heads * nch * prhs::kScoreChunk * sizeof(uint2));
  w.dec = w.sel + align256(heads * (size_t)cap * sizeof(float));
  w.total = w.dec + decode_part_bytes(d, cap);
  return w;
}

size_t step_ws(const prhs_dims* d, int cap) { return step_ws_layout(d, cap).total; }

// Argument checks of prhs_sparse_decode other than its workspace.
int check_decode(const prhs_dims* dims, const void* q, const void* k, const void* v,
                 const int32_t* idx, int32_t idx_cap, const int32_t* count, const float* sel_scores,
                 const float* scores, const float* lse_all, float* out, float* lse_sel,
                 float* delta, float* tau) {
  int st = check_dims(dims);
  if (st) return st;
  if (!v || !idx || !count || !out || !lse_sel)
    return fail(PRHS_E_NULL, "v, idx, count, out and lse_sel are required");
  if (!scores && !sel_scores && (!q || !k))
    return fail(PRHS_E_NULL, "without scores or sel_scores, q and k are required");
  if (delta && !lse_all) return fail(PRHS_E_NULL, "delta needs lse_all");
  if (tau && !delta) return fail(PRHS_E_NULL, "tau needs delta");
  if (!aligned16(v) || (k && !aligned16(k)) || (q && !aligned16(q)))
    return fail(PRHS_E_ALIGN, "q, k and v must be 16-byte aligned");
  if (idx_cap < 1) return fail(PRHS_E_CAPACITY, "idx_cap must be >= 1");
  return PRHS_OK;
}

// The allocation-free decode's scratch: one array per GPU (each device holds
// its own copy of this symbol), reached through the device address that
// hipGetSymbolAddress gives on that device. The symbol's name in host code
// stands for a host-side shadow, never for device memory.
static __device__ __align__(256) unsigned char scratch[PRHS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// This device's scratch address (looked up once per device, with the device
// current).
int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail(PRHS_E_HIP, "hipGetDevice: %s", hipGetErrorString(err));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PRHS_E_HIP, "device %d beyond the %d the scratch table covers", dev, kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || p == nullptr)
      return fail(PRHS_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(err));
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return PRHS_OK;
}

}  // namespace

extern "C" {

const char* prhs_status_string(int status) {
  switch (status) {
    case PRHS_OK: return "ok";
    case PRHS_E_NULL: return "a required pointer is NULL";
    case PRHS_E_DIMS: return "invalid dimensions";
    case PRHS_E_DTYPE: return "unsupported element type";
    case PRHS_E_BUDGET: return "budget, target or radius out of range";
    case PRHS_E_CAPACITY: return "index buffer capacity too small";
    case PRHS_E_WORKSPACE: return "workspace missing or too small";
    case PRHS_E_HIP: return "HIP runtime error";
    case PRHS_E_ALIGN: return "misaligned pointer, stride or leading dimension";
    default: return "unknown status";
  }
}

const char* prhs_last_error(void) { return g_last_error; }

size_t prhs_workspace_bytes(const prhs_dims* dims, int32_t op, int32_t cap) {
  if (check_dims(dims) != PRHS_OK) return 0;
  switch (op) {
    case PRHS_OP_SCORE: return score_ws(dims);
    case PRHS_OP_SELECT: return 0;
    case PRHS_OP_DECODE: return cap >= 1 ? decode_ws(dims, cap) : 0;
    case PRHS_OP_ANCHOR_STEP: return cap >= 1 ? step_ws(dims, cap) : 0;
    case PRHS_OP_DENSE: return dense_ws(dims);
    case PRHS_OP_EXPAND: return expand_ws(dims);
    default: return 0;
  }
}

int prhs_score(const prhs_dims* dims, const void* q, const void* k, float* scores, float* lse_all,
               void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !k || !scores) return fail(PRHS_E_NULL, "q, k and scores are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(scores))
    return fail(PRHS_E_ALIGN, "q, k and scores must be 16-byte aligned");
  if (lse_all) {
    if (!ws) return fail(PRHS_E_WORKSPACE, "workspace is required when lse_all is requested");
    if (ws_bytes < score_ws(dims))
      return fail(PRHS_E_WORKSPACE, "workspace needs %zu bytes, got %zu", score_ws(dims), ws_bytes);
    if (!aligned16(ws)) return fail(PRHS_E_ALIGN, "workspace must be 16-byte aligned");
  }
  return finish(prhs::launch_score(*dims, q, k, scores, lse_all, ws, stream), stream, "prhs_score");
}

int prhs_select_topk(const prhs_dims* dims, const float* scores, const float* lse_all, int32_t mode,
                     int32_t n_budget, float delta_target, int32_t* idx, int32_t idx_cap,
                     int32_t* count, int32_t* cap_hit, float* sel_scores, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->ctx_len > PRHS_MAX_SELECT_CTX)
    return fail(PRHS_E_DIMS, "selection supports ctx_len <= %d", PRHS_MAX_SELECT_CTX);
  if (!scores || !idx || !count) return fail(PRHS_E_NULL, "scores, idx and count are required");
  if (mode != PRHS_TOPN && mode != PRHS_DELTA) return fail(PRHS_E_BUDGET, "unknown mode %d", mode);
  if (mode == PRHS_DELTA && !lse_all) return fail(PRHS_E_NULL, "DELTA mode needs lse_all");
  if (!aligned16(scores)) return fail(PRHS_E_ALIGN, "scores must be 16-byte aligned");
  if (n_budget < 1 || n_budget > dims->ctx_len)
    return fail(PRHS_E_BUDGET, "n_budget %d outside [1, %d]", n_budget, dims->ctx_len);
  if (mode == PRHS_DELTA && !(delta_target >= 0.f && delta_target <= 1.f))
    return fail(PRHS_E_BUDGET, "delta_target must lie in [0, 1]");
  if (idx_cap < n_budget)
    return fail(PRHS_E_CAPACITY, "idx_cap %d < n_budget %d", idx_cap, n_budget);
  prhs::SelectArgs a;
  a.scores = scores;
  a.lse_all = const_cast<float*>(lse_all);  // read only: no partials are given
  a.mode = mode;
  a.n_budget = n_budget;
  a.delta_target = delta_target;
  a.idx = idx;
  a.idx_cap = idx_cap;
  a.count = count;
  a.cap_hit = cap_hit;
  a.sel_scores = sel_scores;
  return finish(prhs::launch_select(*dims, a, stream), stream, "prhs_select_topk");
}

int prhs_cis_reuse(const prhs_dims* dims, const int32_t* anchor_idx, int32_t anchor_cap,
                   const int32_t* anchor_count, int32_t radius, const void* q_cur,
                   const void* q_anchor, float sim_tau, int32_t* out_idx, int32_t out_cap,
                   int32_t* out_count, int32_t* reuse_ok, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!anchor_idx || !anchor_count || !out_idx || !out_count)
    return fail(PRHS_E_NULL, "anchor_idx, anchor_count, out_idx and out_count are required");
  if (reuse_ok && (!q_cur || !q_anchor))
    return fail(PRHS_E_NULL, "the similarity gate needs q_cur and q_anchor");
  if (radius < 0) return fail(PRHS_E_BUDGET, "radius must be >= 0");
  if (reuse_ok && std::isnan(sim_tau)) return fail(PRHS_E_BUDGET, "sim_tau is NaN");
  if (anchor_cap < 1) return fail(PRHS_E_CAPACITY, "anchor_cap must be >= 1");
  const long long need_ll = (2LL * radius + 1) * (long long)anchor_cap;
  const long long need = need_ll < dims->ctx_len ? need_ll : dims->ctx_len;
  if (out_cap < need)
    return fail(PRHS_E_CAPACITY, "out_cap %d < min(t, (2r+1)*anchor_cap) = %lld", out_cap, need);
  return finish(prhs::launch_cis(*dims, anchor_idx, anchor_cap, anchor_count, radius, q_cur,
                                 q_anchor, sim_tau, out_idx, out_cap, out_count, reuse_ok, stream),
                stream, "prhs_cis_reuse");
}

int prhs_sparse_decode(const prhs_dims* dims, const void* q, const void* k, const void* v,
                       const int32_t* idx, int32_t idx_cap, const int32_t* count,
                       const float* sel_scores, const float* scores, const float* lse_all,
                       float* out, float* lse_sel, float* delta, float* tau, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  int st = check_decode(dims, q, k, v, idx, idx_cap, count, sel_scores, scores, lse_all, out,
                        lse_sel, delta, tau);
  if (st) return st;
  if (!ws) return fail(PRHS_E_WORKSPACE, "workspace is required");
  if (ws_bytes < decode_ws(dims, idx_cap))
    return fail(PRHS_E_WORKSPACE, "workspace needs %zu bytes, got %zu", decode_ws(dims, idx_cap),
                ws_bytes);
  if (!aligned16(ws)) return fail(PRHS_E_ALIGN, "workspace must be 16-byte aligned");
  return finish(prhs::launch_decode(*dims, q, k, v, idx, idx_cap, count, sel_scores, scores,
                                    lse_all, out, lse_sel, delta, tau, ws, stream),
                stream, "prhs_sparse_decode");
}

int prhs_sparse_decode_noalloc(const prhs_dims* dims, const void* q, const void* k, const void* v,
                               const int32_t* idx, int32_t idx_cap, const int32_t* count,
                               const float* sel_scores, const float* scores, const float* lse_all,
                               float* out, float* lse_sel, float* delta, float* tau,
                               hipStream_t stream) {
  int st = check_decode(dims, q, k, v, idx, idx_cap, count, sel_scores, scores, lse_all, out,
                        lse_sel, delta, tau);
  if (st) return st;
  // A decode that runs one workgroup per head leaves no partials.
  const size_t need = prhs::decode_per_head(*dims, idx_cap) ? 0 : decode_ws(dims, idx_cap);
  if (need > PRHS_NOALLOC_SCRATCH_BYTES)
    return fail(PRHS_E_WORKSPACE,
                "the decode needs %zu bytes of split partials; the allocation-free call holds %u",
                need, (unsigned)PRHS_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st) return st;
  return finish(prhs::launch_decode(*dims, q, k, v, idx, idx_cap, count, sel_scores, scores,
                                    lse_all, out, lse_sel, delta, tau, ws, stream),
                stream, "prhs_sparse_decode_noalloc");
}

int prhs_reuse_step(const prhs_dims* dims, const int32_t* anchor_idx, int32_t anchor_cap,
                    const int32_t* anchor_count, int32_t radius, const void* q, const void* k,
                    const void* v, int32_t* out_idx, int32_t out_cap, int32_t* out_count,
                    float* out, float* lse_sel, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!anchor_idx || !anchor_count || !out_idx || !out_count)
    return fail(PRHS_E_NULL, "anchor_idx, anchor_count, out_idx and out_count are required");
  if (!q || !k || !v || !out || !lse_sel)
    return fail(PRHS_E_NULL, "q, k, v, out and lse_sel are required");
  if (radius < 0) return fail(PRHS_E_BUDGET, "radius must be >= 0");
  if (anchor_cap < 1) return fail(PRHS_E_CAPACITY, "anchor_cap must be >= 1");
  const long long need_ll = (2LL * radius + 1) * (long long)anchor_cap;
  const long long need = need_ll < dims->ctx_len ? need_ll : dims->ctx_len;
  if (out_cap < need)
    return fail(PRHS_E_CAPACITY, "out_cap %d < min(t, (2r+1)*anchor_cap) = %lld", out_cap, need);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(PRHS_E_ALIGN, "q, k and v must be 16-byte aligned");
  if (!ws) return fail(PRHS_E_WORKSPACE, "workspace is required");
  if (ws_bytes < decode_ws(dims, out_cap))
    return fail(PRHS_E_WORKSPACE, "workspace needs %zu bytes, got %zu", decode_ws(dims, out_cap),
                ws_bytes);
  if (!aligned16(ws)) return fail(PRHS_E_ALIGN, "workspace must be 16-byte aligned");
  return finish(prhs::launch_reuse(*dims, anchor_idx, anchor_cap, anchor_count, radius, q, k, v,
                                   out_idx, out_cap, out_count, out, lse_sel, ws, stream),
                stream, "prhs_reuse_step");
}

int prhs_adaptive_step(const prhs_dims* dims, int32_t n_budget, int32_t radius,
                       int32_t force_refresh, float sim_tau, const void* q, const void* k,
                       const void* v, float* scores, float* lse_all, int32_t* anchor_idx,
                       int32_t* anchor_count, void* anchor_q, int32_t* dil_idx, int32_t dil_cap,
                       int32_t* dil_count, int32_t* refresh, float* sim, float* out,
                       float* lse_sel, float* delta, float* tau, float* theta, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->ctx_len > PRHS_MAX_SELECT_CTX)
    return fail(PRHS_E_DIMS, "selection supports ctx_len <= %d", PRHS_MAX_SELECT_CTX);
  if (!q || !k || !v || !scores || !lse_all || !anchor_idx || !anchor_count || !anchor_q ||
      !dil_idx || !dil_count || !refresh || !out || !lse_sel)
    return fail(PRHS_E_NULL, "q, k, v, scores, lse_all, anchor_idx, anchor_count, anchor_q, "
                             "dil_idx, dil_count, refresh, out and lse_sel are required");
  if (tau && !delta) return fail(PRHS_E_NULL, "tau needs delta");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(scores))
    return fail(PRHS_E_ALIGN, "q, k, v and scores must be 16-byte aligned");
  if (n_budget < 1 || n_budget > dims->ctx_len)
    return fail(PRHS_E_BUDGET, "n_budget %d outside [1, %d]", n_budget, dims->ctx_len);
  if (radius < 0) return fail(PRHS_E_BUDGET, "radius must be >= 0");
  if (std::isnan(sim_tau)) return fail(PRHS_E_BUDGET, "sim_tau is NaN");
  const long long need_ll = (2LL * radius + 1) * (long long)n_budget;
  const long long need = need_ll < dims->ctx_len ? need_ll : dims->ctx_len;
  if (dil_cap < need)
    return fail(PRHS_E_CAPACITY, "dil_cap %d < min(t, (2r+1)*n_budget) = %lld", dil_cap, need);
  if (!ws) return fail(PRHS_E_WORKSPACE, "workspace is required");
  if (ws_bytes < step_ws(dims, dil_cap))
    return fail(PRHS_E_WORKSPACE, "workspace needs %zu bytes, got %zu", step_ws(dims, dil_cap),
                ws_bytes);
  if (!aligned16(ws)) return fail(PRHS_E_ALIGN, "workspace must be 16-byte aligned");
  char* w = static_cast<char*>(ws);
  const StepWs L = step_ws_layout(dims, dil_cap);
  float2* part = reinterpret_cast<float2*>(w + L.part);
  float* sel = reinterpret_cast<float*>(w + L.sel);
  hipError_t err = prhs::launch_gate(*dims, q, anchor_q, anchor_count, force_refresh ? 1 : 0,
                                     sim_tau, refresh, sim, stream);
  prhs::ScanCand cd;
  cd.active = refresh;
  if (theta) {
    cd.theta = theta;
    cd.cand = reinterpret_cast<uint2*>(w + L.cand);
    cd.cand_cnt = reinterpret_cast<uint32_t*>(w + L.cnt);
  }
  if (err == hipSuccess) err = prhs::launch_score(*dims, q, k, scores, nullptr, part, stream, &cd);
  if (err == hipSuccess) {
    prhs::SelectArgs a;
    a.scores = scores;
    a.lse_all = lse_all;
    a.part = part;
    a.mode = PRHS_TOPN;
    a.n_budget = n_budget;
    a.idx = anchor_idx;
    a.idx_cap = n_budget;
    a.count = anchor_count;
    a.sel_scores = sel;
    a.cand = cd.cand;
    a.cand_cnt = cd.cand_cnt;
    a.theta_out = theta;
    a.hint_q = q;
    a.hint_q_f16 = dims->dtype == PRHS_F16;
    a.hint_d = dims->head_dim;
    a.active = refresh;
    err = prhs::launch_select(*dims, a, stream);
  }
  if (err == hipSuccess)
    err = prhs::launch_adaptive_decode(*dims, q, k, v, refresh, anchor_idx, n_budget, anchor_count,
                                       sel, radius, dil_idx, dil_cap, dil_count, lse_all, out,
                                       lse_sel, delta, tau, w + L.dec, stream);
  return finish(err, stream, "prhs_adaptive_step");
}

int prhs_random_expand(const prhs_dims* dims, const int32_t* anchor_idx, int32_t anchor_cap,
                       const int32_t* anchor_count, const int32_t* draws, int32_t m,
                       int32_t* out_idx, int32_t out_cap, int32_t* out_count, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->ctx_len > PRHS_MAX_SELECT_CTX)
    return fail(PRHS_E_DIMS, "selection supports ctx_len <= %d", PRHS_MAX_SELECT_CTX);
  if (!anchor_idx || !anchor_count || !draws || !out_idx || !out_count)
    return fail(PRHS_E_NULL, "anchor_idx, anchor_count, draws, out_idx and out_count are required");
  if (anchor_cap < 1) return fail(PRHS_E_CAPACITY, "anchor_cap must be >= 1");
  if (m < anchor_cap || m > dims->ctx_len)
    return fail(PRHS_E_BUDGET, "m %d outside [anchor_cap %d, t %d]", m, anchor_cap, dims->ctx_len);
  if (out_cap < m) return fail(PRHS_E_CAPACITY, "out_cap %d < m %d", out_cap, m);
  if (!ws) return fail(PRHS_E_WORKSPACE, "workspace is required");
  if (ws_bytes < expand_ws(dims))
    return fail(PRHS_E_WORKSPACE, "workspace needs %zu bytes, got %zu", expand_ws(dims), ws_bytes);
  if (!aligned16(ws)) return fail(PRHS_E_ALIGN, "workspace must be 16-byte aligned");
  float* cs = static_cast<float*>(ws);
  hipError_t err = prhs::launch_expand_scores(*dims, anchor_idx, anchor_cap, anchor_count, draws,
                                              cs, stream);
  if (err == hipSuccess) {
    prhs::SelectArgs a;
    a.scores = cs;
    a.mode = PRHS_TOPN;
    a.n_budget = m;
    a.idx = out_idx;
    a.idx_cap = out_cap;
    a.count = out_count;
    err = prhs::launch_select(*dims, a, stream);
  }
  return finish(err, stream, "prhs_random_expand");
}

int prhs_dense_decode(const prhs_dims* dims, const void* q, const void* k, const void* v,
                      float* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!q || !k || !v || !out || !lse) return fail(PRHS_E_NULL, "q, k, v, out and lse are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(PRHS_E_ALIGN, "q, k and v must be 16-byte aligned");
  if (!ws) return fail(PRHS_E_WORKSPACE, "workspace is required");
  if (ws_bytes < dense_ws(dims))
    return fail(PRHS_E_WORKSPACE, "workspace needs %zu bytes, got %zu", dense_ws(dims), ws_bytes);
  if (!aligned16(ws)) return fail(PRHS_E_ALIGN, "workspace must be 16-byte aligned");
  return finish(prhs::launch_dense(*dims, q, k, v, out, lse, ws, stream), stream,
                "prhs_dense_decode");
}

int prhs_append_kv(const prhs_dims* dims, const void* k_new, const void* v_new, void* k, void* v,
                   int32_t pos, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!k_new || !v_new || !k || !v) return fail(PRHS_E_NULL, "k_new, v_new, k and v are required");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k) || !aligned16(v))
    return fail(PRHS_E_ALIGN, "k_new, v_new, k and v must be 16-byte aligned");
  if (pos < 0 || pos >= dims->ctx_len)
    return fail(PRHS_E_DIMS, "pos %d outside [0, %d)", pos, dims->ctx_len);
  return finish(prhs::launch_append_kv(*dims, k_new, v_new, k, v, pos, stream), stream,
                "prhs_append_kv");
}

int prhs_anchor_step(const prhs_dims* dims, int32_t mode, int32_t n_budget, float delta_target,
                     const void* q, const void* k, const void* v, float* scores, float* lse_all,
                     int32_t* idx, int32_t idx_cap, int32_t* count, int32_t* cap_hit, float* out,
                     float* lse_sel, float* delta, float* tau, float* theta, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->ctx_len > PRHS_MAX_SELECT_CTX)
    return fail(PRHS_E_DIMS, "selection supports ctx_len <= %d", PRHS_MAX_SELECT_CTX);
  if (!q || !k || !v || !scores || !lse_all || !idx || !count || !out || !lse_sel)
    return fail(PRHS_E_NULL, "q, k, v, scores, lse_all, idx, count, out and lse_sel are required");
  if (tau && !delta) return fail(PRHS_E_NULL, "tau needs delta");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(scores))
    return fail(PRHS_E_ALIGN, "q, k, v and scores must be 16-byte aligned");
  if (mode != PRHS_TOPN && mode != PRHS_DELTA) return fail(PRHS_E_BUDGET, "unknown mode %d", mode);
  if (n_budget < 1 || n_budget > dims->ctx_len)
    return fail(PRHS_E_BUDGET, "n_budget %d outside [1, %d]", n_budget, dims->ctx_len);
  if (mode == PRHS_DELTA && !(delta_target >= 0.f && delta_target <= 1.f))
    return fail(PRHS_E_BUDGET, "delta_target must lie in [0, 1]");
  if (idx_cap < n_budget)
    return fail(PRHS_E_CAPACITY, "idx_cap %d < n_budget %d", idx_cap, n_budget);
  if (!ws) return fail(PRHS_E_WORKSPACE, "workspace is required");
  if (ws_bytes < step_ws(dims, idx_cap))
    return fail(PRHS_E_WORKSPACE, "workspace needs %zu bytes, got %zu", step_ws(dims, idx_cap),
                ws_bytes);
  if (!aligned16(ws)) return fail(PRHS_E_ALIGN, "workspace must be 16-byte aligned");
  char* w = static_cast<char*>(ws);
  const StepWs L = step_ws_layout(dims, idx_cap);
  float2* part = reinterpret_cast<float2*>(w + L.part);
  float* sel = reinterpret_cast<float*>(w + L.sel);
  prhs::ScanCand cd;
  const bool hint = theta != nullptr && mode == PRHS_TOPN;
  if (hint) {
    cd.theta = theta;
    cd.cand = reinterpret_cast<uint2*>(w + L.cand);
    cd.cand_cnt = reinterpret_cast<uint32_t*>(w + L.cnt);
    // hinted heads get no score row from a matrix-core scan; the selection
    // recomputes the row of a head whose candidates miss
    cd.skip_hinted = prhs::scan_uses_mfma(*dims);
  }
  // With fp16 rows of 128 and a budget of at most 2048 each head's select
  // workgroup also decodes its head: no split partials and no merge launch.
  const bool fuse = prhs::fuse_decode(*dims, mode, n_budget);
  hipError_t err = prhs::launch_score(*dims, q, k, scores, nullptr, part, stream, &cd);
  if (err == hipSuccess) {
    prhs::SelectArgs a;
    a.scores = scores;
    a.lse_all = lse_all;
    a.part = part;
    a.mode = mode;
    a.n_budget = n_budget;
    a.delta_target = delta_target;
    a.idx = idx;
    a.idx_cap = idx_cap;
    a.count = count;
    a.cap_hit = cap_hit;
    a.sel_scores = fuse ? nullptr : sel;
    a.cand = cd.cand;
    a.cand_cnt = cd.cand_cnt;
    a.theta_out = hint ? theta : nullptr;
    a.hint_q = q;
    a.hint_q_f16 = dims->dtype == PRHS_F16;
    a.hint_d = dims->head_dim;
    a.kv_sb = dims->kv_stride_b;
    a.kv_sh = dims->kv_stride_h;
    a.kv_st = dims->kv_stride_t;
    a.hq = dims->n_q_heads;
    a.hkv = dims->n_kv_heads;
    if (cd.skip_hinted) {
      a.rescore_q = q;
      a.rescore_k = k;
      a.rescore_row = scores;
      a.rescore_scale = (float)(1.0 / std::sqrt((double)dims->head_dim));
    }
    if (fuse) {
      a.v = v;
      a.kv_sb = dims->kv_stride_b;
      a.kv_sh = dims->kv_stride_h;
      a.kv_st = dims->kv_stride_t;
      a.hq = dims->n_q_heads;
      a.hkv = dims->n_kv_heads;
      a.out = out;
      a.lse_sel = lse_sel;
      a.delta = delta;
      a.tau = tau;
    }
    err = prhs::launch_select(*dims, a, stream);
  }
  if (err == hipSuccess && !fuse)
    err = prhs::launch_decode(*dims, q, k, v, idx, idx_cap, count, sel, nullptr, lse_all, out,
                              lse_sel, delta, tau, w + L.dec, stream);
  return finish(err, stream, "prhs_anchor_step");
}

int prhs_dropped_mass(const prhs_dims* dims, const float* lse_sel, const float* lse_all,
                      float* delta, float* tau, hipStream_t stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (!lse_sel || !lse_all || !delta) return fail(PRHS_E_NULL, "lse_sel, lse_all and delta are required");
  return finish(prhs::launch_dropped_mass(*dims, lse_sel, lse_all, delta, tau, stream), stream,
                "prhs_dropped_mass");
}

int prhs_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (buf == nullptr || sink == nullptr) return fail(PRHS_E_NULL, "buf and sink must be non-NULL");
  if (!aligned16(buf)) return fail(PRHS_E_ALIGN, "buf must be 16-byte aligned");
  if (bytes == 0 || bytes % 16) return fail(PRHS_E_DIMS, "bytes must be a positive multiple of 16");
  return finish(prhs::launch_stream_read(buf, bytes, sink, stream), stream, "prhs_probe_stream_read");
}

}  // extern "C"
