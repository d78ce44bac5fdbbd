// Critical-index-set (CIS) reuse with dilation (page "Near-Oracle KV
// Selection via Pre-hoc Sparsity for Long-Context Inference", Fig. 4: one
// query's critical set serves the next adjacent queries, grown around its
// clusters; Table VIII: dilation radius r; Fig. 8 / Fig. 9(c): sharing only
// while the queries stay similar).
//
// One 256-thread workgroup per (b, h). The ascending anchor list is processed
// in tiles of 256: each index i proposes the window [i - r, i + r] clipped to
// [0, t) and starts it after the largest window end seen so far (a workgroup
// prefix-max), so windows never overlap and the output stays strictly
// ascending. A prefix sum of the window lengths gives each window's output
// offset; the tile's output is then written cooperatively, each thread finding
// its source window by binary search over the tile's offsets, so the work is
// balanced however large r is.
#include "prhs_device.hpp"
#include "prhs_launch.hpp"

namespace prhs {
namespace {

constexpr int kCisThreads = 256;

__device__ __forceinline__ long long wave_inclusive_max(long long x) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const long long y = __shfl_up(x, o);
    if (lane >= o) x = x > y ? x : y;
  }
  return x;
}

template <typename T>
__global__ __launch_bounds__(kCisThreads) void cis_dilate_kernel(
    const int* __restrict__ anchor_idx, int anchor_cap, const int* __restrict__ anchor_count,
    int radius, int t, int* __restrict__ out_idx, int out_cap, int* __restrict__ out_count,
    const T* __restrict__ q_cur, const T* __restrict__ q_anchor, float sim_tau,
    int* __restrict__ reuse_ok, int D) {
  constexpr int NW = kCisThreads / kWave;
  __shared__ long long s_end[kCisThreads];   // inclusive end offset of each window in the tile
  __shared__ long long s_lo[kCisThreads];
  __shared__ long long s_wmax[NW];
  __shared__ long long s_wsum[NW];
  __shared__ float s_red[3][NW];

  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = tid / kWave;
  const int n = max(0, min(anchor_count[head], anchor_cap));
  const int* src = anchor_idx + (size_t)head * anchor_cap;
  int* dst = out_idx + (size_t)head * out_cap;
  const long long r = radius;

  long long base = 0;        // outputs written so far
  long long prev_end = -1;   // largest window end so far
  for (int tile = 0; tile < n; tile += kCisThreads) {
    const int j = tile + tid;
    long long lo = 0, hi = -1;
    if (j < n) {
      const long long i = src[j];
      if (i >= 0 && i < t) {
        lo = i - r > 0 ? i - r : 0;
        hi = i + r < t - 1 ? i + r : t - 1;
      }
    }
    // exclusive prefix-max of window ends over the tile, seeded with prev_end
    const long long incl_max = wave_inclusive_max(hi);
    if (lane == kWave - 1) s_wmax[w] = incl_max;
    __syncthreads();
    long long before = prev_end;
    long long tile_max = prev_end;
    for (int k = 0; k < NW; ++k) {
      const long long v = s_wmax[k];
      if (k < w) before = before > v ? before : v;
      tile_max = tile_max > v ? tile_max : v;
    }
    long long excl_max = __shfl_up(incl_max, 1);
    if (lane == 0) excl_max = -1;
    if (excl_max > before) before = excl_max;
    if (lo < before + 1) lo = before + 1;
    const long long len = hi >= lo ? hi - lo + 1 : 0;
    // prefix sum of lengths
    const long long incl = wave_inclusive_scan(len);
    if (lane == kWave - 1) s_wsum[w] = incl;
    __syncthreads();
    long long off = 0, tile_total = 0;
    for (int k = 0; k < NW; ++k) {
      const long long v = s_wsum[k];
      if (k < w) off += v;
      tile_total += v;
    }
    s_end[tid] = off + incl;
    s_lo[tid] = lo;
    __syncthreads();
    for (long long p = tid; p < tile_total; p += kCisThreads) {
      // first window whose inclusive end exceeds p
      int a = 0, b = kCisThreads - 1;
      while (a < b) {
        const int mid = (a + b) >> 1;
        if (s_end[mid] > p) b = mid;
        else a = mid + 1;
      }
      const long long start = a ? s_end[a - 1] : 0;
      const long long o = base + p;
      if (o < out_cap) dst[o] = (int)(s_lo[a] + (p - start));
    }
    base += tile_total;
    prev_end = tile_max;
    __syncthreads();
  }
  if (tid == 0) out_count[head] = (int)(base < out_cap ? base : out_cap);

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

}  // namespace

hipError_t launch_cis(const prhs_dims& d, const int* anchor_idx, int anchor_cap,
                      const int* anchor_count, int radius, const void* q_cur, const void* q_anchor,
                      float sim_tau, int* out_idx, int out_cap, int* out_count, int* reuse_ok,
                      hipStream_t stream) {
  const int nheads = d.batch * d.n_q_heads;
  if (d.dtype == PRHS_F16)
    hipLaunchKernelGGL((cis_dilate_kernel<__half>), dim3(nheads), dim3(kCisThreads), 0, stream,
                       anchor_idx, anchor_cap, anchor_count, radius, d.ctx_len, out_idx, out_cap,
                       out_count, static_cast<const __half*>(q_cur),
                       static_cast<const __half*>(q_anchor), sim_tau, reuse_ok, d.head_dim);
  else
    hipLaunchKernelGGL((cis_dilate_kernel<float>), dim3(nheads), dim3(kCisThreads), 0, stream,
                       anchor_idx, anchor_cap, anchor_count, radius, d.ctx_len, out_idx, out_cap,
                       out_count, static_cast<const float*>(q_cur),
                       static_cast<const float*>(q_anchor), sim_tau, reuse_ok, d.head_dim);
  return hipGetLastError();
}

}  // namespace prhs
