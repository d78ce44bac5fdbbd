// Critical-index-set (CIS) reuse with dilation (page "Near-Oracle KV
// Selection via Pre-hoc Sparsity for Long-Context Inference", Fig. 4: one
// query's critical set serves the next adjacent queries, grown around its
// clusters; Table VIII: dilation radius r; Fig. 8 / Fig. 9(c): sharing only
// while the queries stay similar).
//
// One 512-thread workgroup per (b, h). The ascending anchor list is processed
// in tiles of 512 (the next tile's indices are loaded while the current one
// is processed): each index i proposes the window [i - r, i + r] clipped to
// [0, t) and starts it after the largest window end seen so far (a workgroup
// prefix-max), so windows never overlap and the output stays strictly
// ascending. A prefix sum of the window lengths gives each window's output
// offset. Short windows (2r + 1 <= 64) are written by their own thread; longer
// ones cooperatively, each thread finding its source window by binary search
// over the tile's offsets, so the work stays balanced however large r is.
// All positions are below t, so 32-bit arithmetic suffices.
#include "prhs_device.hpp"
#include "prhs_launch.hpp"

namespace prhs {
namespace {

constexpr int kCisThreads = 512;
constexpr int kShortWindow = 64;

template <typename T>
__global__ __launch_bounds__(kCisThreads) void cis_dilate_kernel(
    const int* __restrict__ anchor_idx, int anchor_cap, const int* __restrict__ anchor_count,
    int radius, int t, int* __restrict__ out_idx, int out_cap, int* __restrict__ out_count,
    const T* __restrict__ q_cur, const T* __restrict__ q_anchor, float sim_tau,
    int* __restrict__ reuse_ok, int D, const int* __restrict__ skip) {
  constexpr int NW = kCisThreads / kWave;
  if (skip != nullptr && skip[blockIdx.x] != 0) return;  // head left untouched
  __shared__ int s_end[kCisThreads];   // inclusive end offset of each window in the tile
  __shared__ int s_lo[kCisThreads];
  __shared__ int s_wmax[2][NW];        // double-buffered by tile parity
  __shared__ uint32_t s_wsum[2][NW];
  __shared__ float s_red[3][NW];

  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int n = max(0, min(anchor_count[head], anchor_cap));
  const int* src = anchor_idx + (size_t)head * anchor_cap;
  int* dst = out_idx + (size_t)head * out_cap;
  const int r = radius < t ? radius : t;
  const bool short_windows = 2 * r + 1 <= kShortWindow;

  int base = 0;        // outputs written so far
  int prev_end = -1;   // largest window end so far
  int next = tid < n ? src[tid] : -1;
  for (int tile = 0, par = 0; tile < n; tile += kCisThreads, par ^= 1) {
    const int j = tile + tid;
    const int i = next;
    next = j + kCisThreads < n ? src[j + kCisThreads] : -1;
    PRHS_CHECK(j >= n || (i >= 0 && i < t), kCheckIndex);
    PRHS_CHECK(j >= n || j == 0 || src[j - 1] < i, kCheckOrder);
    int lo = 0, hi = -1;
    if (j < n && i >= 0 && i < t) {
      lo = i - r > 0 ? i - r : 0;
      hi = i < t - 1 - r ? i + r : t - 1;
    }
    // exclusive prefix-max of window ends over the tile, seeded with prev_end
    const int incl_max = wave_inclusive_max(hi);
    if (lane == kWave - 1) s_wmax[par][w] = incl_max;
    __syncthreads();
    int before = prev_end;
    int tile_max = prev_end;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const int v = s_wmax[par][k];
      if (k < w) before = before > v ? before : v;
      tile_max = tile_max > v ? tile_max : v;
    }
    int excl_max = __shfl_up(incl_max, 1);
    if (lane == 0) excl_max = -1;
    if (excl_max > before) before = excl_max;
    if (lo < before + 1) lo = before + 1;
    const uint32_t len = hi >= lo ? (uint32_t)(hi - lo + 1) : 0u;
    // prefix sum of lengths
    const uint32_t incl = wave_scan_u32(len);
    if (lane == kWave - 1) s_wsum[par][w] = incl;
    __syncthreads();
    uint32_t off = 0, tile_total = 0;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const uint32_t v = s_wsum[par][k];
      if (k < w) off += v;
      tile_total += v;
    }
    off += incl - len;
    if (short_windows) {
      for (uint32_t k = 0; k < len; ++k) {
        const uint32_t o = (uint32_t)base + off + k;
        if (o < (uint32_t)out_cap) dst[o] = lo + (int)k;
      }
    } else {
      s_end[tid] = (int)(off + len);
      s_lo[tid] = lo;
      __syncthreads();
      for (int p = tid; p < (int)tile_total; p += kCisThreads) {
        // first window whose inclusive end exceeds p
        int a = 0, b = kCisThreads - 1;
        while (a < b) {
          const int mid = (a + b) >> 1;
          if (s_end[mid] > p) b = mid;
          else a = mid + 1;
        }
        const int start = a ? s_end[a - 1] : 0;
        const long long o = (long long)base + p;
        if (o < out_cap) dst[o] = s_lo[a] + (p - start);
      }
      __syncthreads();
    }
    base += (int)tile_total;
    prev_end = tile_max;
  }
  if (tid == 0) out_count[head] = base < out_cap ? base : out_cap;

  if (reuse_ok != nullptr && q_cur != nullptr && q_anchor != nullptr) {
    float dot = 0.f, n1 = 0.f, n2 = 0.f;
    for (int c = tid; c < D; c += kCisThreads) {
      const float x = (float)q_cur[(size_t)head * D + c];
      const float y = (float)q_anchor[(size_t)head * D + c];
      dot += x * y;
      n1 += x * x;
      n2 += y * y;
    }
    dot = wave_sum(dot);
    n1 = wave_sum(n1);
    n2 = wave_sum(n2);
    if (lane == 0) {
      s_red[0][w] = dot;
      s_red[1][w] = n1;
      s_red[2][w] = n2;
    }
    __syncthreads();
    if (tid == 0) {
      float a = 0.f, b = 0.f, c = 0.f;
      for (int k = 0; k < NW; ++k) {
        a += s_red[0][k];
        b += s_red[1][k];
        c += s_red[2][k];
      }
      const float den = sqrtf(b) * sqrtf(c);
      reuse_ok[head] = (den > 0.f && a >= sim_tau * den) ? 1 : 0;
    }
  }
}

// Similarity gate of the adaptive step: one wave per head. Sharing continues
// while cos(q, q_anchor) >= sim_tau (Fig. 8 / Fig. 9(c)); otherwise, when the
// step is forced, or before the head's first anchor, the head refreshes and
// its anchor query becomes q.
template <typename T>
__global__ __launch_bounds__(256) void cis_gate_kernel(const T* __restrict__ q,
                                                       T* __restrict__ q_anchor,
                                                       const int* __restrict__ anchor_count,
                                                       int force, float sim_tau,
                                                       int* __restrict__ refresh,
                                                       float* __restrict__ sim, int D,
                                                       int nheads) {
  const int head = blockIdx.x * (256 / kWave) + (int)(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  if (head >= nheads) return;
  const T* qc = q + (size_t)head * D;
  T* qa = q_anchor + (size_t)head * D;
  float dot = 0.f, n1 = 0.f, n2 = 0.f;
  for (int c = lane; c < D; c += kWave) {
    const float x = (float)qc[c];
    const float y = (float)qa[c];
    dot += x * y;
    n1 += x * x;
    n2 += y * y;
  }
  dot = wave_sum(dot);
  n1 = wave_sum(n1);
  n2 = wave_sum(n2);
  const bool has_anchor = anchor_count[head] > 0;
  const float den = sqrtf(n1) * sqrtf(n2);
  const bool share = has_anchor && den > 0.f && dot >= sim_tau * den;
  const bool fresh = force != 0 || !share;
  if (fresh)
    for (int c = lane; c < D; c += kWave) qa[c] = qc[c];
  if (lane == 0) {
    refresh[head] = fresh ? 1 : 0;
    if (sim != nullptr) sim[head] = has_anchor && den > 0.f ? dot / den : __builtin_nanf("");
  }
}

// Control scores of the random expansion (Table VI, Panel A: RandomExpansion,
// the budget-matched control of dilation): members of the anchor set score
// kMember, every other key minus its 23-bit draw, so that the exact top-m of
// these scores is the anchor set plus the m - |S_a| outside keys of smallest
// draw (the lower index on equal draws, by the selection's tie rule). One
// workgroup per head marks the set in an LDS bitmap, then writes the row.
constexpr float kMember = 3.0e38f;

__global__ __launch_bounds__(256) void expand_scores_kernel(
    const int* __restrict__ anchor_idx, int anchor_cap, const int* __restrict__ anchor_count,
    const int* __restrict__ draws, int t, float* __restrict__ out, int ld) {
  __shared__ uint32_t member[PRHS_MAX_SELECT_CTX / 32];
  const int head = blockIdx.x;
  const int nwords = (t + 31) >> 5;
  for (int i = threadIdx.x; i < nwords; i += 256) member[i] = 0u;
  __syncthreads();
  const int n = max(0, min(anchor_count[head], anchor_cap));
  const int* src = anchor_idx + (size_t)head * anchor_cap;
  for (int j = threadIdx.x; j < n; j += 256) {
    const int i = src[j];
    PRHS_CHECK(i >= 0 && i < t, kCheckIndex);
    if (i >= 0 && i < t) atomicOr(&member[i >> 5], 1u << (i & 31));
  }
  __syncthreads();
  const int* dr = draws + (size_t)head * t;
  float* row = out + (size_t)head * ld;
  for (int i = threadIdx.x; i < t; i += 256)
    row[i] = (member[i >> 5] >> (i & 31)) & 1u ? kMember : -(float)(dr[i] & 0x7FFFFF);
}

}  // namespace

hipError_t launch_expand_scores(const prhs_dims& d, const int* anchor_idx, int anchor_cap,
                                const int* anchor_count, const int* draws, float* out,
                                hipStream_t stream) {
  const int nheads = d.batch * d.n_q_heads;
  hipLaunchKernelGGL(expand_scores_kernel, dim3(nheads), dim3(256), 0, stream, anchor_idx,
                     anchor_cap, anchor_count, draws, d.ctx_len, out, d.scores_ld);
  return hipGetLastError();
}

hipError_t launch_gate(const prhs_dims& d, const void* q, void* q_anchor, const int* anchor_count,
                       int force, float sim_tau, int* refresh, float* sim, hipStream_t stream) {
  const int nheads = d.batch * d.n_q_heads;
  const dim3 grid((nheads + 3) / 4);
  if (d.dtype == PRHS_F16)
    hipLaunchKernelGGL((cis_gate_kernel<__half>), grid, dim3(256), 0, stream,
                       static_cast<const __half*>(q), static_cast<__half*>(q_anchor), anchor_count,
                       force, sim_tau, refresh, sim, d.head_dim, nheads);
  else
    hipLaunchKernelGGL((cis_gate_kernel<float>), grid, dim3(256), 0, stream,
                       static_cast<const float*>(q), static_cast<float*>(q_anchor), anchor_count,
                       force, sim_tau, refresh, sim, d.head_dim, nheads);
  return hipGetLastError();
}

hipError_t launch_cis(const prhs_dims& d, const int* anchor_idx, int anchor_cap,
                      const int* anchor_count, int radius, const void* q_cur, const void* q_anchor,
                      float sim_tau, int* out_idx, int out_cap, int* out_count, int* reuse_ok,
                      hipStream_t stream, const int* skip) {
  const int nheads = d.batch * d.n_q_heads;
  if (d.dtype == PRHS_F16)
    hipLaunchKernelGGL((cis_dilate_kernel<__half>), dim3(nheads), dim3(kCisThreads), 0, stream,
                       anchor_idx, anchor_cap, anchor_count, radius, d.ctx_len, out_idx, out_cap,
                       out_count, static_cast<const __half*>(q_cur),
                       static_cast<const __half*>(q_anchor), sim_tau, reuse_ok, d.head_dim, skip);
  else
    hipLaunchKernelGGL((cis_dilate_kernel<float>), dim3(nheads), dim3(kCisThreads), 0, stream,
                       anchor_idx, anchor_cap, anchor_count, radius, d.ctx_len, out_idx, out_cap,
                       out_count, static_cast<const float*>(q_cur),
                       static_cast<const float*>(q_anchor), sim_tau, reuse_ok, d.head_dim, skip);
  return hipGetLastError();
}

PRHS_CHECK_READER(take_checks_cis)

}  // namespace prhs
